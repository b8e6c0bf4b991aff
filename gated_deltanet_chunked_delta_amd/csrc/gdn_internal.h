// Internal interface between the C-ABI host code (gdn_api.cpp) and the HIP
// kernels (gdn_fused.hip, gdn_fused_ws.hip, gdn_recurrent.hip, gdn_gating.hip,
// gdn_split.hip, gdn_backward.hip).  Not part of
// the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace gdn {

constexpr int kChunk = 64;   // chunk length in tokens (the NPU page's tiling section: 64)

// Raw gate inputs: when A_log is non-null the kernels compute
// g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b) per (token,
// value head) themselves, and the g / beta pointers are not read.
struct Gates {
    const float *A_log, *dt_bias;    // [HV]
    const void *a, *b;               // [rows, HV], the element type of q/k/v
};

// Everything a launch needs.  Pointers are device pointers.
struct Params {
    // inputs
    const void *q, *k, *v;           // [T_tot, H, K], [T_tot, H, K], [T_tot, HV, V]
    const float *g, *beta;           // [T_tot, HV]
    const float *initial_state;      // [N, HV, K, V] or null
    const int32_t *cu_seqlens;       // [N+1] or null (equal-length mode)
    // outputs
    void *out;                       // [T_tot, HV, V]
    float *final_state;              // [N, HV, K, V] or null
    // sizes
    int B, T, H, HV, K, V, N;
    float scale;
    int use_l2norm;
    Gates gates;                     // used instead of g, beta when gates.A_log != null
    // State pool: when state_indices is non-null, initial_state and
    // final_state point at one pool [pool_size, HV, K, V] and sequence n uses
    // slot state_indices[n] (a slot outside the pool: zero start, no store).
    // state_bf16: the states (pool or not) are stored as bf16.
    const int32_t *state_indices;
    int pool_size;
    int state_bf16;
    // Sequence split (the transfer-map run): v_zero = v points at one zero row
    // of HV x V elements read for every token; init_shared = initial_state
    // holds one [HV, K, V] state used by every sequence.
    int v_zero;
    int init_shared;
    // Packed batches: when non-null, the sequences in the order the
    // workgroups take them, longest first ([N]; see launch_seq_order).
    const int32_t *seq_order;
};

// The kernels of one forward pass, for the timing hook.
// fused_kernel: single-role prefill kernel (the fp32 check mode);
// fused_ws_kernel: warp-specialized prefill kernel (bf16);
// recurrent_update_kernel: the decode step;
// gating_kernel: the stand-alone gate computation.
// split_setup_kernel, split_combine_kernel, split_final_kernel: the
// sequence split of long sequences (gdn_split.hip);
// seq_order_kernel: the longest-first order of a packed batch's sequences.
// bwd_*_kernel: the backward pass (gdn_backward.hip).
enum KernelKind { kFusedKernel = 0, kFusedWsKernel = 1, kRecurrentKernel = 2, kGatingKernel = 3,
                  kSplitSetupKernel = 4, kSplitCombineKernel = 5, kSplitFinalKernel = 6,
                  kBwdSetupKernel = 7, kBwdPrepKernel = 8, kBwdFwdScanKernel = 9, kBwdDhScanKernel = 10,
                  kBwdGradsKernel = 11, kBwdReduceKernel = 12, kSeqOrderKernel = 13, kNumKernelKinds = 14 };
const char *kernel_name(int kind);

// Timing hook: when given, the launch sequence calls begin/end around each
// kernel it enqueues (on the same stream).
struct Profiler {
    virtual void begin(int kind, hipStream_t stream) = 0;
    virtual void end(int kind, hipStream_t stream) = 0;
    virtual ~Profiler() {}
};

// Enqueues the whole forward pass.  Returns the HIP error of the launches.
// With p.seq_order set (a packed batch of 2..kSeqOrderMax sequences and N
// int32 of workspace), a one-workgroup kernel first writes the longest-first
// order of the sequences there.
hipError_t launch_forward(const Params &p, int dtype, hipStream_t stream, Profiler *prof);
constexpr int kSeqOrderMax = 1024;

// Everything a decode-step launch needs.  Pointers are device pointers.
struct DecodeParams {
    const void *q, *k, *v;           // [N, H, K], [N, H, K], [N, HV, V]
    const float *g, *beta;           // [N, HV]
    Gates gates;                     // used instead of g, beta when gates.A_log != null
    float *state_pool;               // [pool_size, HV, K, V], updated in place (bf16 when state_bf16)
    const int32_t *state_indices;    // [N]
    void *out;                       // [N, HV, V]
    int N, H, HV, K, V, pool_size;
    float scale;
    int use_l2norm;
    int state_bf16;
};

// Enqueues the decode step (gdn_recurrent.hip).
hipError_t launch_recurrent(const DecodeParams &p, int dtype, hipStream_t stream, Profiler *prof);

// Enqueues the stand-alone gate computation (gdn_gating.hip) for rows x HV
// gates into g and beta.
hipError_t launch_gating(const Gates &gt, int64_t rows, int HV, int dtype, float *g, float *beta,
                         hipStream_t stream, Profiler *prof);

// Sequence split (gdn_split.hip).  A batch of few, long, equal-length
// sequences gives too few workgroups to fill the GPU; each sequence is then
// cut into S segments of L tokens that run side by side.  The state is affine
// in a segment's initial state h_s: its end state is F_s + M_s h_s, with F_s
// the end state from a zero start and M_s the segment's K x K transfer map.  So
//   1. every segment runs without outputs from zero (segment 0 from the true
//      initial state) -> end states F;
//   2. every segment runs without outputs with v = 0 from the identity (K
//      state columns) -> transfer maps M;
//   3. h_1 = F_0, h_{s+1} = M_s h_s + F_s in segment order;
//   4. every segment runs from h_s with outputs (the outputs and end states
//      of the unsplit pass, up to rounding); the last segments' end states
//      are the final states.
struct SplitPlan {
    bool active = false;
    int S = 1, L = 0;                 // segments per sequence, tokens per segment (multiple of 64)
    size_t off_cu = 0, off_idx = 0, off_pool = 0, off_map = 0, off_fin = 0, off_id = 0,
           off_zero = 0, bytes = 0;   // workspace carve-up (256-byte aligned)
};
// The split for these sizes (equal-length sequences only); bytes = 0 when none.
SplitPlan plan_split(int B, int T, int H, int HV, int K, int V, int elem_bytes);
// Enqueues the split forward pass of p (cu_seqlens null) with workspace ws.
hipError_t launch_split(const Params &p, int dtype, const SplitPlan &plan, void *ws, hipStream_t stream,
                        Profiler *prof);
// Device address of the library's static scratch (GDN_STATIC_SCRATCH_BYTES
// bytes) on the device of `stream` (the current device for the null stream),
// looked up on the first call for that device.
hipError_t static_scratch(hipStream_t stream, void **ptr);

// Everything the backward pass needs (gdn_backward.hip).  Pointers are device
// pointers; the intermediates point into the caller's workspace.
struct BwdParams {
    // inputs
    const void *q, *k, *v;           // [T_tot, H, K], [T_tot, H, K], [T_tot, HV, V]
    const float *g, *beta;           // [T_tot, HV]
    const void *dout;                // [T_tot, HV, V], gradient of the output
    const float *dht;                // [N, HV, K, V] gradient of the final state, or null
    const float *initial_state;      // [N, HV, K, V] or null
    const int32_t *cu_seqlens;       // [N+1] or null (equal-length mode)
    // outputs
    void *dq, *dk, *dv;              // shapes of q, k, v
    float *dg, *dbeta;               // [T_tot, HV]
    float *dh0;                      // [N, HV, K, V] or null
    // workspace
    int32_t *chunk_offsets;          // [N+1] first chunk of each packed sequence
    float *gam;                      // [T_tot, HV] chunk-local cumsum of g
    float *tm, *ag, *pm;             // [chunks, HV, 64, 64]: (I+A)^-1, A / beta, masked gated Q K^T
    float *hs, *dhs;                 // [chunks, HV, K, V]: state at chunk start, its gradient at chunk end
    float *vn, *db;                  // [T_tot, HV, V]: delta-rule errors and their B-gradient
    float *dqp, *dkp;                // [T_tot, HV, K]: dq, dk per value head
    int32_t *seq_order;              // [N] packed sequences longest first, or null (index order)
    // sizes
    int B, T, H, HV, K, V, N, T_tot;
    float scale;
    int use_l2norm;
};
// Workspace carve-up of the backward pass (256-byte aligned offsets).
struct BwdPlan {
    int nc_max = 0;                   // chunk slots (an upper bound on the chunks of packed sequences)
    size_t off_co = 0, off_gam = 0, off_tm = 0, off_ag = 0, off_pm = 0, off_hs = 0, off_dhs = 0, off_vn = 0,
           off_db = 0, off_dqp = 0, off_dkp = 0, bytes = 0;
    bool ordered = false;             // packed batch of 2..kSeqOrderMax sequences: an order at off_ord
    size_t off_ord = 0;
};
BwdPlan plan_backward(int B, int T, int H, int HV, int K, int V, int N, bool varlen);
hipError_t launch_backward(BwdParams p, int dtype, const BwdPlan &plan, void *ws, hipStream_t stream,
                           Profiler *prof);

// The single-role fused kernel's launch (gdn_fused.hip).
hipError_t launch_fused(const Params &p, int dtype, hipStream_t stream);
// The warp-specialized bf16 kernel's launch (gdn_fused_ws.hip).
hipError_t launch_fused_ws(const Params &p, hipStream_t stream);

}  // namespace gdn
