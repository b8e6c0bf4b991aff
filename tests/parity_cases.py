"""Discriminating bf16 parity cases: inputs on which an honest bf16 kernel stays
far below the bar while each planted mistake of ``test_oracle_mutants`` lands
far above it.

The standard workloads use fast gates (the memory of the state is a few tokens),
a small initial state and nearly orthogonal unit keys, so several wrong
algorithms (no delta term, a dropped initial state, an erase that skips the
decay) change the outputs by less than the bf16 tolerance of the throughput
configurations.  The two cases here (each with and without the L2 norm, as
the kernel forms the gated Q K^T tiles in different waves for the two) are
built so that they do not:

* slow_recall: slow gates (a ~ N(-5, 1), A_log ~ U(0, ln 4), so |g| is of the
  order of 1e-2 and the state remembers hundreds of tokens), beta near 0.9
  (b ~ N(2.2, 0.25)) and an O(1) initial state (N(0, 1)): the initial state,
  the delta term and beta all stay visible in every output;
* fast_overlap: the gate law of the tiny configuration with beta near 0.9 and
  keys and queries of one key head sharing a direction (k, q = c + N(0, 1)),
  so that neighbouring keys overlap: the erase term e^g S^T k is large, which
  exposes an erase without the decay and a gate applied to the wrong token.

Bars are max-abs errors against the fp64 oracle, per case, about three times
the largest error the bf16 kernel shows on the case and its larger variants
(measured: slow_recall 1.6e-3 on o, 7.0e-3 on S; fast_overlap 1.7e-3 and
3.5e-3; without the norm, slow_recall_nonorm 1.3e-3 and 6.4e-3, and
fast_overlap_nonorm 3.7e-3 and 5.5e-3, whose keys of squared length about 2
give outputs of about twice the size).  ``test_parity_gate_power`` checks on the CPU that every mutant
misses these bars by at least a factor of five on the same inputs.
"""
import math

from workloads import WORKLOADS, scaled

SLOW = dict(a_mean=-5.0, a_log_hi=math.log(4.0), b_mean=2.2, b_std=0.25, init="all", init_std=1.0)
FAST = dict(a_mean=0.0, b_mean=2.2, b_std=0.25, qk_common=1.0, init="all", init_std=1.0)

# (workload, bar on o, bar on the final state)
BASE = {
    "slow_recall": (scaled(WORKLOADS["gva"], "slow_recall", B=2, T=320, H=2, HV=4, **SLOW), 5e-3, 2e-2),
    "fast_overlap": (scaled(WORKLOADS["gva"], "fast_overlap", B=2, T=320, H=2, HV=4, **FAST), 5e-3, 1e-2),
    # the same gates without the L2 norm (keys of length about 1, the
    # stable form of the wide configuration)
    "slow_recall_nonorm": (scaled(WORKLOADS["wide_stable"], "slow_recall_nonorm", B=2, T=320, H=2, HV=4, **SLOW),
                           5e-3, 2e-2),
    "fast_overlap_nonorm": (scaled(WORKLOADS["wide_stable"], "fast_overlap_nonorm", B=2, T=320, H=2, HV=4, **FAST),
                            1.2e-2, 1.5e-2),
}

# the same inputs at the sizes of the kernel's other layouts (whole 128-column
# value heads per workgroup once there are 256 (sequence, value head) pairs),
# packed sequences included; same bars
VARIANTS = {
    "slow_recall_heads": ("slow_recall", scaled(WORKLOADS["gva"], "slow_recall_heads", B=2, T=200, H=8, HV=128,
                                                **SLOW)),
    "fast_overlap_heads": ("fast_overlap", scaled(WORKLOADS["gva"], "fast_overlap_heads", B=2, T=200, H=8, HV=128,
                                                  **FAST)),
    "slow_recall_packed": ("slow_recall", scaled(WORKLOADS["varlen"], "slow_recall_packed", H=16, HV=32,
                                                 lengths=(1, 64, 65, 127, 0, 200, 3, 129), **SLOW)),
    "slow_recall_nonorm_heads": ("slow_recall_nonorm", scaled(WORKLOADS["wide_stable"], "slow_recall_nonorm_heads",
                                                              B=2, T=200, H=8, HV=128, **SLOW)),
    "fast_overlap_nonorm_heads": ("fast_overlap_nonorm", scaled(WORKLOADS["wide_stable"],
                                                                "fast_overlap_nonorm_heads", B=2, T=200, H=8,
                                                                HV=128, **FAST)),
}


def cases():
    """name -> (workload, bar on o, bar on S) for every discriminating case."""
    out = dict(BASE)
    for name, (base, w) in VARIANTS.items():
        out[name] = (w, BASE[base][1], BASE[base][2])
    return out
