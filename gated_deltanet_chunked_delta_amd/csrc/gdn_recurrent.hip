// Fused recurrent decode step (one token per sequence) with an in-place,
// pool-indexed state (fp32, or bf16 rounded to nearest even), for gfx950.
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
// K x V state once (2 * 4 K V bytes in fp32, half that in a bf16 pool) and
// touches only K + K + V other elements.  One workgroup of K/8 waves owns the
// whole state of one (sequence, value head).  A lane holds four adjacent
// columns (16 bytes in fp32, 8 in bf16) of 8 / (64 / (V/4)) rows, so one
// wave-wide access covers 64 / (V/4) full rows; each wave keeps its 8 rows in
// registers (fp32) between the read and the write.  The inner products over
// rows are summed across the lanes that share columns, then across the waves
// through LDS.  Fewer than 64 registers per lane let 8 waves share a SIMD,
// which keeps enough state reads in flight to approach the HBM rate.  The
// state is touched exactly once each way, so its loads and stores are marked
// non-temporal (streamed past the caches rather than kept in them).
#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Four consecutive state elements of type S (fp32 or bf16) as fp32, and back
// (bf16 rounded to nearest even); non-temporal: each state byte is touched
// once each way.
template <typename S> struct State4;
template <> struct State4<float> {
    typedef f32x4 T;
    static __device__ __forceinline__ f32x4 load(const T *p) { return __builtin_nontemporal_load(p); }
    static __device__ __forceinline__ void store(T *p, f32x4 x) { __builtin_nontemporal_store(x, p); }
};
template <> struct State4<bf16> {
    typedef bf16x4 T;
    static __device__ __forceinline__ f32x4 load(const T *p) {
        const bf16x4 x = __builtin_nontemporal_load(p);
        return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    }
    static __device__ __forceinline__ void store(T *p, f32x4 x) {
        __builtin_nontemporal_store(bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]}, p);
    }
};

template <typename E, typename SE, int K, int V>
__global__ void __launch_bounds__(64 * (K / 8)) recurrent_update_kernel(DecodeParams p) {
    constexpr int NW = K / 8;                  // waves per workgroup (8 rows each)
    constexpr int LPR = V / 4;                 // lanes per state row (4 columns each)
    constexpr int RPI = 64 / LPR;              // state rows per wave-wide access
    constexpr int RW = K / NW;                 // state rows per wave
    constexpr int NI = RW / RPI;               // 16-byte state pieces per lane
    static_assert(NI >= 1 && RW % RPI == 0, "unsupported head size");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c4 = (lane % LPR) * 4;           // this lane's first column
    const int rl = lane / LPR;                 // its row within an access
    const int nj = blockIdx.x, n = nj / p.HV, j = nj % p.HV, jk = j / (p.HV / p.H);
    const size_t nh = (size_t)n * p.HV + j;
    E *__restrict__ out = (E *)p.out + nh * V;
    const int slot = p.state_indices[n];
    if (slot < 0 || slot >= p.pool_size) {   // padding row: the pool slot is not touched
        if (tid < V) out[tid] = to_e<E>(0.f);
        return;
    }
    // the lane's rows are wv*RW + i*RPI + rl, i < NI, at columns c4 .. c4+3
    typedef State4<SE> SIO;
    typename SIO::T *__restrict__ S =
        (typename SIO::T *)((SE *)p.state_pool + (((size_t)slot * p.HV + j) * K + wv * RW + rl) * V + c4);
    f32x4 s[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) s[i] = SIO::load(S + i * RPI * V / 4);

    // key and query rows (raw) in LDS; squared norms and k.q by a workgroup
    // reduction, combined after the barrier that publishes the rows
    __shared__ __attribute__((aligned(16))) float ks[K], qs[K];
    __shared__ float pn[NW][3];
    __shared__ f32x4 pa[NW][V / 4], pb[NW][V / 4];
    float kk = 0.f, qq = 0.f, kq = 0.f;
    if (tid < K) {
        const float kv = to_f(((const E *)p.k)[((size_t)n * p.H + jk) * K + tid]);
        const float qv = to_f(((const E *)p.q)[((size_t)n * p.H + jk) * K + tid]);
        ks[tid] = kv;
        qs[tid] = qv;
        kk = kv * kv;
        qq = qv * qv;
        kq = kv * qv;
    }
    kk = wave_sum(kk);
    qq = wave_sum(qq);
    kq = wave_sum(kq);
    if (lane == 0) {
        pn[wv][0] = kk;
        pn[wv][1] = qq;
        pn[wv][2] = kq;
    }
    __syncthreads();
    // partial S^T k and S^T q over this lane's rows
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = wv * RW + i * RPI + rl;
        a += s[i] * ks[r];
        b += s[i] * qs[r];
    }
    // lanes holding the same columns (different rows) first, then the waves
#pragma unroll
    for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] += __shfl_xor(a[e], o);
            b[e] += __shfl_xor(b[e], o);
        }
    }
    if (rl == 0) {
        pa[wv][lane] = a;
        pb[wv][lane] = b;
    }
    __syncthreads();
    // a few threads finish the sums over the waves (2V column sums, 3 norms)
    __shared__ __attribute__((aligned(16))) float fin[2][V];
    __shared__ float fn[3];
    if (tid < 2 * V) {
        const int col = tid % V;
        const float *src = (const float *)(tid < V ? &pa[0][0] : &pb[0][0]);
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) x += src[w * V + col];
        fin[tid / V][col] = x;
    } else if (tid < 2 * V + 3) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) x += pn[w][tid - 2 * V];
        fn[tid - 2 * V] = x;
    }
    __syncthreads();
    a = *(const f32x4 *)&fin[0][c4];
    b = *(const f32x4 *)&fin[1][c4];
    kk = fn[0];
    qq = fn[1];
    kq = fn[2];
    const float rk = p.use_l2norm ? rsqrtf(kk + 1e-6f) : 1.f;
    const float rq = p.use_l2norm ? rsqrtf(qq + 1e-6f) : 1.f;
    float gv, bt;
    if (p.gates.A_log) {   // gates from the raw inputs
        gv = gate_g(to_f(((const E *)p.gates.a)[nh]), -expf(p.gates.A_log[j]), p.gates.dt_bias[j]);
        bt = gate_beta(to_f(((const E *)p.gates.b)[nh]));
    } else {
        gv = p.g[nh];
        bt = p.beta[nh];
    }
    const float eg = __expf(gv);
    const E *vp = (const E *)p.v + nh * V + c4;
    f32x4 u;
#pragma unroll
    for (int e = 0; e < 4; ++e) u[e] = to_f(vp[e]) - eg * rk * a[e];
    const f32x4 bu = u * (bt * rk);            // beta u times the key norm factor
#pragma unroll
    for (int i = 0; i < NI; ++i) SIO::store(S + i * RPI * V / 4, eg * s[i] + bu * ks[wv * RW + i * RPI + rl]);
    if (wv == 0 && rl == 0) {
        const float cq = bt * kq * rk * rq;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[c4 + e] = to_e<E>(p.scale * (eg * rq * b[e] + cq * u[e]));
    }
}

template <typename E, typename SE, int K, int V>
hipError_t launch_cfg(const DecodeParams &p, hipStream_t st) {
    const unsigned grid = (unsigned)((size_t)p.N * p.HV);
    recurrent_update_kernel<E, SE, K, V><<<grid, 64 * (K / 8), 0, st>>>(p);
    return hipGetLastError();
}

template <typename E, typename SE>
hipError_t launch_kv(const DecodeParams &p, hipStream_t st) {
    if (p.K == 64 && p.V == 64) return launch_cfg<E, SE, 64, 64>(p, st);
    if (p.K == 64 && p.V == 128) return launch_cfg<E, SE, 64, 128>(p, st);
    if (p.K == 128 && p.V == 64) return launch_cfg<E, SE, 128, 64>(p, st);
    return launch_cfg<E, SE, 128, 128>(p, st);
}

template <typename E>
hipError_t launch_dtype(const DecodeParams &p, hipStream_t st) {
    return p.state_bf16 ? launch_kv<E, bf16>(p, st) : launch_kv<E, float>(p, st);
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
