/*
 * Oracle for the gated delta rule forward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * may load this library.  The GPU library shares no code with it.
 *
 * What it computes (plain, token by token, in double precision):
 *
 *   For every sequence n and value head j, with key head jk = j / (HV/H)
 *   (contiguous groups of value heads share one key head: the LightLLM page
 *   "gdn.py", LinearAttBackend._init_linear_layer_metadata, derives
 *   num_v_heads_per_k_head = HV / H), start from S = S0[n, j] (a K x V
 *   matrix, zero when no initial state is given) and for each token t:
 *
 *     qh = q[t, jk], kh = k[t, jk]
 *     if use_l2norm:  x <- x / sqrt(sum(x^2) + 1e-6)   for x in {qh, kh}
 *     S  <- exp(g[t, j]) * S                          (forget)
 *     d  <- beta[t, j] * (v[t, j] - S^T kh)           (delta-rule error)
 *     S  <- S + kh d^T                                (write)
 *     o[t, j] = scale * S^T qh                        (read after write)
 *
 *   and the final state of (n, j) is S after the last token.
 *
 * Source of the recurrence: the Gated Delta Networks paper (arXiv:2412.06464)
 * that the page "NPU Training Operators - GDN" cites in its section on the
 * operator's semantics (g controls forgetting, beta the strength of the delta
 * update, q/k/v what is read and written).  Tensor layouts follow the page
 * "[Qwen3.5][Feature] support fla triton kernel for qwen3.5" (FastDeploy PR
 * #7024), section "Usage or Command", item 1: q, k [B,T,H,K], v [B,T,HV,V],
 * states [N,HV,K,V]; g and beta are per value head ([B,T,HV]) as the review
 * comments on that page and LightLLM's gating call establish.  The L2-norm
 * epsilon (1e-6, inside the square root) is not given on the pages; it is a
 * stated reading.
 *
 * Inputs are the exact values handed to the GPU, passed as float32 (bf16 and
 * fp32 values convert to float32 exactly) and upcast to double here.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Runs the recurrence for one (sequence, value head) unit.
 *   q, k:   first token row of this unit's key head, row stride qk_stride
 *   v:      first token row of this value head, row stride v_stride
 *   g, beta: first token entry of this value head, stride gb_stride
 *   S:      K x V double, holds the initial state on entry, final on exit
 *   o:      L x V double output rows
 */
static void recurrent_unit(int64_t L, int K, int V,
                           const float *q, const float *k, int64_t qk_stride,
                           const float *v, int64_t v_stride,
                           const float *g, const float *beta, int64_t gb_stride,
                           double scale, int use_l2norm,
                           double *S, double *o, double *work)
{
    double *qh = work;
    double *kh = work + K;
    double *d = work + 2 * K;
    for (int64_t t = 0; t < L; ++t) {
        const float *qt = q + t * qk_stride;
        const float *kt = k + t * qk_stride;
        const float *vt = v + t * v_stride;
        for (int r = 0; r < K; ++r) {
            qh[r] = (double)qt[r];
            kh[r] = (double)kt[r];
        }
        if (use_l2norm) {
            double sq = 0.0, sk = 0.0;
            for (int r = 0; r < K; ++r) {
                sq += qh[r] * qh[r];
                sk += kh[r] * kh[r];
            }
            double iq = 1.0 / sqrt(sq + 1e-6);
            double ik = 1.0 / sqrt(sk + 1e-6);
            for (int r = 0; r < K; ++r) {
                qh[r] *= iq;
                kh[r] *= ik;
            }
        }
        double alpha = exp((double)g[t * gb_stride]);
        double b = (double)beta[t * gb_stride];
        for (int64_t e = 0; e < (int64_t)K * V; ++e) S[e] *= alpha;
        for (int c = 0; c < V; ++c) {
            double acc = 0.0;
            for (int r = 0; r < K; ++r) acc += S[(int64_t)r * V + c] * kh[r];
            d[c] = b * ((double)vt[c] - acc);
        }
        for (int r = 0; r < K; ++r)
            for (int c = 0; c < V; ++c) S[(int64_t)r * V + c] += kh[r] * d[c];
        for (int c = 0; c < V; ++c) {
            double acc = 0.0;
            for (int r = 0; r < K; ++r) acc += S[(int64_t)r * V + c] * qh[r];
            o[t * V + c] = scale * acc;
        }
    }
}

/*
 * Batch driver.
 *   q, k:   [T_tot, H, K] float32 (the [B,T,H,K] tensor with B and T merged)
 *   v:      [T_tot, HV, V] float32
 *   g, beta:[T_tot, HV] float32
 *   initial_state: [N, HV, K, V] float32, or NULL for a zero state
 *   cu_seqlens: [N+1] int64 token offsets of the sequences in T_tot
 *   units:  n_units entries u = n*HV + j selecting (sequence, value head)
 *   out_row: n_units row offsets into `out` (each unit writes len(n) rows)
 *   out:    [sum of unit lengths, V] double
 *   final_state: [n_units, K, V] double
 *   nthreads: OpenMP threads (<= 0: library default)
 * Returns 0, or -1 on an argument error (nothing is written then).
 */
int gdn_oracle_forward(const float *q, const float *k, const float *v,
                       const float *g, const float *beta,
                       const float *initial_state, const int64_t *cu_seqlens,
                       int64_t N, int H, int HV, int K, int V,
                       double scale, int use_l2norm,
                       const int64_t *units, int64_t n_units,
                       const int64_t *out_row, double *out, double *final_state,
                       int nthreads)
{
    if (!q || !k || !v || !g || !beta || !cu_seqlens || !units || !out_row ||
        !out || !final_state)
        return -1;
    if (H <= 0 || HV <= 0 || HV % H != 0 || K <= 0 || V <= 0 || N < 0)
        return -1;
    for (int64_t u = 0; u < n_units; ++u)
        if (units[u] < 0 || units[u] >= N * HV) return -1;
    const int G = HV / H;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *S_work = (double *)malloc(sizeof(double) * (size_t)(2 * K + V));
        if (!S_work) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t u = 0; u < n_units; ++u) {
            if (!S_work) continue;
            int64_t n = units[u] / HV;
            int j = (int)(units[u] % HV);
            int jk = j / G;
            int64_t t0 = cu_seqlens[n];
            int64_t L = cu_seqlens[n + 1] - t0;
            double *S = final_state + u * (int64_t)K * V;
            if (initial_state) {
                const float *s0 = initial_state + (n * HV + j) * (int64_t)K * V;
                for (int64_t e = 0; e < (int64_t)K * V; ++e) S[e] = (double)s0[e];
            } else {
                memset(S, 0, sizeof(double) * (size_t)K * V);
            }
            recurrent_unit(L, K, V,
                           q + (t0 * H + jk) * (int64_t)K,
                           k + (t0 * H + jk) * (int64_t)K, (int64_t)H * K,
                           v + (t0 * HV + j) * (int64_t)V, (int64_t)HV * V,
                           g + t0 * HV + j, beta + t0 * HV + j, HV,
                           scale, use_l2norm, S, out + out_row[u] * (int64_t)V,
                           S_work);
        }
        free(S_work);
    }
    return bad ? -1 : 0;
}
