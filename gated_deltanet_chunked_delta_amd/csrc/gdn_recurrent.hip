// Fused recurrent decode step (one token per sequence) with an in-place,
// pool-indexed fp32 state, for gfx950.
//
// For sequence n, value head j and state slot s = state_indices[n] (a slot
// outside [0, pool_size) marks a padding row), with kh, qh the (optionally
// L2-normalised) key and query rows of key head j / (HV/H):
//
//   a   = S^T kh,  b = S^T qh                      (S = pool[s, j] before the step)
//   u   = v - e^g a                                 (the delta-rule residual)
//   S'  = e^g S + beta kh u^T                       (written back in place)
//   out = scale S'^T qh = scale (e^g b + beta (kh . qh) u)
//
// which is one token of the gated delta rule (the recurrence in include/gdn.h)
// with both inner products taken on the state before the step, so that each
// state column is read once and written once.  This is the decode operation of
// the FastDeploy PR #7024 page ("Usage or Command", item 2: the fused recurrent
// kernel with its ssm_pool / ssm_indices interface).
//
// The step is bound by HBM: every (sequence, value head) reads and writes its
// K x V fp32 state once (2 * 4 K V bytes) and touches only K + K + V other
// elements.  A workgroup of K/32 waves handles 64 state columns of one
// (sequence, value head): lane = column, each wave holds 32 rows of its column
// in registers between the read and the write (the waves' partial inner
// products are combined through LDS), and every state access is a coalesced
// 256-byte row of 64 columns.  Few registers per wave let 8 waves share a
// SIMD, which keeps enough state reads in flight to approach the HBM rate.
#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <typename E, int K, int V>
__global__ void __launch_bounds__(64 * (K / 32)) recurrent_update_kernel(DecodeParams p) {
    constexpr int VB = 64;                     // state columns per workgroup
    constexpr int NW = K / 32;                 // waves per workgroup
    constexpr int KH = 32;                     // state rows per wave
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's 32 rows
    const int vs = blockIdx.x % (V / VB), nj = blockIdx.x / (V / VB);
    const int n = nj / p.HV, j = nj % p.HV, jk = j / (p.HV / p.H);
    const int c = vs * VB + lane;
    E *__restrict__ out = (E *)p.out + ((size_t)n * p.HV + j) * V + c;
    const int slot = p.state_indices[n];
    if (slot < 0 || slot >= p.pool_size) {   // padding row: the pool slot is not touched
        if (wv == 0) *out = to_e<E>(0.f);
        return;
    }
    // the state block of (slot, j) is uniform; lanes add 32-bit column offsets
    float *__restrict__ S = p.state_pool + ((size_t)slot * p.HV + j) * K * V + (size_t)wv * KH * V;

    // key and query rows (raw) in LDS; squared norms and their dot product by
    // a workgroup reduction.  ku is a second copy of the key row for the
    // update: reading it from a separate array keeps the compiler from holding
    // the first reads of ks in registers across the column.
    __shared__ float ks[K], qs[K], ku[K];
    __shared__ float part[NW][3][64];
    const E *kp = (const E *)p.k + ((size_t)n * p.H + jk) * K;
    const E *qp = (const E *)p.q + ((size_t)n * p.H + jk) * K;
    float kk = 0.f, qq = 0.f, kq = 0.f;
    if (tid < K) {   // one key element per thread
        const float kv = to_f(kp[tid]), qv = to_f(qp[tid]);
        ks[tid] = kv;
        ku[tid] = kv;
        qs[tid] = qv;
        kk = kv * kv;
        qq = qv * qv;
        kq = kv * qv;
    }
    kk = wave_sum(kk);
    qq = wave_sum(qq);
    kq = wave_sum(kq);
    if (lane == 0) {
        part[wv][0][0] = kk;
        part[wv][1][0] = qq;
        part[wv][2][0] = kq;
    }
    // this wave's 32 rows of the column, read once
    float s[KH];
#pragma unroll
    for (int r = 0; r < KH; ++r) s[r] = S[r * V + c];
    __syncthreads();
    kk = qq = kq = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        kk += part[w][0][0];
        qq += part[w][1][0];
        kq += part[w][2][0];
    }
    const float rk = p.use_l2norm ? rsqrtf(kk + 1e-6f) : 1.f;
    const float rq = p.use_l2norm ? rsqrtf(qq + 1e-6f) : 1.f;
    const float *kr = ks + wv * KH, *qr = qs + wv * KH;
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int r = 0; r < KH; r += 2) {
        a0 += s[r] * kr[r];
        a1 += s[r + 1] * kr[r + 1];
        b0 += s[r] * qr[r];
        b1 += s[r + 1] * qr[r + 1];
    }
    // partial S^T k and S^T q of these rows, combined across the waves
    __syncthreads();   // the first reads of part are done before it is rewritten
    part[wv][0][lane] = a0 + a1;
    part[wv][1][lane] = b0 + b1;
    __syncthreads();
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        a += part[w][0][lane];
        b += part[w][1][lane];
    }
    a *= rk;
    b *= rq;
    const size_t nh = (size_t)n * p.HV + j;
    const float eg = __expf(p.g[nh]), bt = p.beta[nh];
    const float u = to_f(((const E *)p.v)[nh * V + c]) - eg * a;
    const float bu = bt * u * rk;              // beta u times the key norm factor
    const float *kw = ku + wv * KH;
#pragma unroll
    for (int r = 0; r < KH; ++r) S[r * V + c] = eg * s[r] + bu * kw[r];
    if (wv == 0) *out = to_e<E>(p.scale * (eg * b + bt * (kq * rk * rq) * u));
}

template <typename E, int K, int V>
hipError_t launch_cfg(const DecodeParams &p, hipStream_t st) {
    const unsigned grid = (unsigned)((size_t)p.N * p.HV * (V / 64));
    recurrent_update_kernel<E, K, V><<<grid, 64 * (K / 32), 0, st>>>(p);
    return hipGetLastError();
}

template <typename E>
hipError_t launch_dtype(const DecodeParams &p, hipStream_t st) {
    if (p.K == 64 && p.V == 64) return launch_cfg<E, 64, 64>(p, st);
    if (p.K == 64 && p.V == 128) return launch_cfg<E, 64, 128>(p, st);
    if (p.K == 128 && p.V == 64) return launch_cfg<E, 128, 64>(p, st);
    return launch_cfg<E, 128, 128>(p, st);
}

}  // namespace

hipError_t launch_recurrent(const DecodeParams &p, int dtype, hipStream_t stream, Profiler *prof) {
    if (p.N == 0) return hipSuccess;
    if (prof) prof->begin(kRecurrentKernel, stream);
    const hipError_t err = dtype == 0 ? launch_dtype<bf16>(p, stream) : launch_dtype<float>(p, stream);
    if (prof) prof->end(kRecurrentKernel, stream);
    return err;
}

}  // namespace gdn
