// Sequence split of long sequences for gfx950: the plan, the setup, combine
// and correction kernels, and the launch sequence (the scheme is described
// with SplitPlan in gdn_internal.h).
//
// It rests on the state being affine in a segment's initial state: with
// A_t = e^{g_t} (I - beta_t k_t k_t^T), the recurrence S_t = A_t S_{t-1} +
// beta_t k_t v_t^T of the Gated Delta Networks rule (cited by the page "NPU
// Training Operators - GDN", References) gives S_t = S0_t + M_t h for a
// segment started from h, where S0_t starts from zero and M_t = A_t ... A_a.
// M_t is what the same recurrence computes from the identity with v = 0, and
// its output scale M_t^T q_t turns o_t = scale S_t^T q_t into o0_t + h^T
// (scale M_t^T q_t).
#include <mutex>

#include "gdn.h"
#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct SplitDims {
    int B, T, HV, K, V, S, L;
};

// Segment offsets and slot indices; the state pool (slot (b, 0): the caller's
// initial state of sequence b, or zero; later slots: zero); the identity maps
// [HV, K, K]; the zero v row [HV, K].
template <typename E>
__global__ void __launch_bounds__(256) split_setup_kernel(SplitDims d, const float *__restrict__ init,
                                                          int32_t *__restrict__ cu, int32_t *__restrict__ idx,
                                                          float *__restrict__ pool, float *__restrict__ ident,
                                                          E *__restrict__ zrow) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, nth = (int64_t)gridDim.x * blockDim.x;
    const int64_t nseg = (int64_t)d.B * d.S;
    for (int64_t i = tid; i <= nseg; i += nth) {
        const int b = (int)(i / d.S), s = (int)(i % d.S);
        cu[i] = i == nseg ? d.B * d.T : b * d.T + min(s * d.L, d.T);
        if (i < nseg) idx[i] = (int32_t)i;
    }
    const int64_t st = (int64_t)d.HV * d.K * d.V;
    for (int64_t i = tid; i < nseg * st; i += nth) {
        const int64_t slot = i / st, r = i % st;
        const int64_t b = slot / d.S, s = slot % d.S;
        pool[i] = (s == 0 && init) ? init[b * st + r] : 0.f;
    }
    const int64_t kk = (int64_t)d.K * d.K;
    for (int64_t i = tid; i < (int64_t)d.HV * kk; i += nth) {
        const int64_t r = i % kk;
        ident[i] = (r / d.K == r % d.K) ? 1.f : 0.f;
    }
    for (int64_t i = tid; i < (int64_t)d.HV * d.K; i += nth) zrow[i] = to_e<E>(0.f);
}

// h_1 = h0_0 (segment 0 ran from the true initial state); h_{s+1} = M_s h_s +
// h0_s; h_s (s >= 1) are published for the correction, transposed ([V][K])
// and rounded to the I/O type once, which is how the correction's products
// take them; h_S is the final state.  One workgroup per (sequence, value
// head, 32 state columns): M_s and the workgroup's columns of h_s in LDS,
// each thread a 4 x 4 block of the product, fp32 throughout.
constexpr int kCombineCols = 32;

template <typename E>
__global__ void __launch_bounds__(256) split_combine_kernel(SplitDims d, const float *__restrict__ pool,
                                                            const float *__restrict__ maps, E *__restrict__ hsT,
                                                            float *__restrict__ final_state) {
    constexpr int CW = kCombineCols, CP = CW + 4, MP = 128 + 4;   // padded rows of h and M
    __shared__ __attribute__((aligned(16))) float h[128 * CP], m[128 * MP];
    const int K = d.K, V = d.V, ncb = V / CW;
    const int cb = blockIdx.x % ncb, bj = blockIdx.x / ncb;
    const int b = bj / d.HV, j = bj % d.HV, col0 = cb * CW;
    const int t = threadIdx.x, nb = (K / 4) * (CW / 4);
    const int r0 = 4 * (t / (CW / 4)), c0 = 4 * (t % (CW / 4));
    const float *h0 = pool + ((int64_t)b * d.S * d.HV + j) * K * V;
    for (int i = t; i < K * CW; i += blockDim.x) h[(i / CW) * CP + i % CW] = h0[(i / CW) * V + col0 + i % CW];
    // M_s moves in 16-byte pieces, M_{s+1} loading into registers during step s
    constexpr int NM = 128 * 128 / 4 / 256;
    const int nm4 = K * K / 4;
    f32x4 mr[NM];
    auto fetch_m = [&](int s) {
        const f32x4 *ms = (const f32x4 *)(maps + (((int64_t)b * d.S + s) * d.HV + j) * K * K);
#pragma unroll
        for (int u = 0; u < NM; ++u)
            if (t + 256 * u < nm4) mr[u] = ms[t + 256 * u];
    };
    if (d.S > 1) fetch_m(1);
    for (int s = 1; s < d.S; ++s) {
        const int64_t slot = (int64_t)b * d.S + s;
        E *hsd = hsT + (slot * d.HV + j) * K * V + (int64_t)col0 * K;   // rows col0.. of [V][K]
#pragma unroll
        for (int u = 0; u < NM; ++u) {
            const int i = 4 * (t + 256 * u);
            if (i < K * K) *(f32x4 *)&m[(i / K) * MP + i % K] = mr[u];
        }
        __syncthreads();   // h (step s - 1, or the load above) and M_s are in place
        for (int i = t; i < K * CW; i += blockDim.x) hsd[i] = to_e<E>(h[(i % K) * CP + i / K]);
        if (s + 1 < d.S) fetch_m(s + 1);
        float acc[4][4];
        if (t < nb) {
            const float *h0s = pool + (slot * d.HV + j) * K * V + col0;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[a][c] = h0s[(r0 + a) * V + c0 + c];
#pragma unroll 4
            for (int kk = 0; kk < K; ++kk) {
                float mv[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) mv[a] = m[(r0 + a) * MP + kk];
                const f32x4 hv = *(const f32x4 *)&h[kk * CP + c0];
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[a][c] += mv[a] * hv[c];
            }
        }
        __syncthreads();   // every thread is done reading h and m
        if (t < nb) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *(f32x4 *)&h[(r0 + a) * CP + c0] = f32x4{acc[a][0], acc[a][1], acc[a][2], acc[a][3]};
        }
    }
    __syncthreads();
    if (final_state) {
        float *fd = final_state + ((int64_t)b * d.HV + j) * K * V;
        for (int i = t; i < K * CW; i += blockDim.x) fd[(i / CW) * V + col0 + i % CW] = h[(i / CW) * CP + i % CW];
    }
}

// o_t += h_s^T oM_t for the tokens of segment s >= 1: C[token][v] =
// sum_k oM[token][k] h_s[k][v] on MFMA (bf16 operands, or fp32 in the check
// mode), added to the output in fp32 and rounded once.  One workgroup per
// (sequence, segment, value head, TB x 64 tokens); each wave 16 tokens of a
// 64-token tile.  The product is computed transposed, C^T[v][token], and the
// two 16-row tiles of each 32-column block of v take their rows in the order
// v = 32p + 8 (r / 4) + 4 (tile % 2) + r % 4, so that the eight values a lane
// holds for one token over the pair are consecutive: every output access is
// one 16-byte (bf16) read and write.  The next tile's rows are loaded while
// the current one is computed.
constexpr int kCorrectTiles = 16;

template <typename E, int K, int V>
__global__ void __launch_bounds__(256) split_correct_kernel(SplitDims d, const E *__restrict__ om,
                                                            const E *__restrict__ hsT, E *__restrict__ out) {
    constexpr int TB = kCorrectTiles, KP = K + 8, KS = K / 32, NP = V / 32;   // KP: padded rows of h^T
    __shared__ __attribute__((aligned(16))) E hT[V * KP];
    const int nblk = (d.L + 64 * TB - 1) / (64 * TB);
    int x = blockIdx.x;
    const int blk = x % nblk;
    x /= nblk;
    const int j = x % d.HV;
    x /= d.HV;
    const int s = 1 + x % (d.S - 1), b = x / (d.S - 1);
    const int seg0 = b * d.T + s * d.L, seg1 = b * d.T + min((s + 1) * d.L, d.T);
    const int64_t slot = (int64_t)b * d.S + s;
    const E *hsrc = hsT + (slot * d.HV + j) * K * V;   // [V][K], rounded by the combine kernel
    {
        typedef typename VT<E>::v16b v16b;
        constexpr int PV = VT<E>::kVec;                    // elements per 16 bytes
        for (int i = threadIdx.x; i < V * K / PV; i += blockDim.x) {
            const int v = i / (K / PV), k = (i % (K / PV)) * PV;
            *(v16b *)&hT[v * KP + k] = *(const v16b *)(hsrc + v * K + k);
        }
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, grp = lane >> 4;
    // this wave's tiles: tokens first + 64 t + (0..15) for t < ntile (each tile starts inside the segment)
    const int first = seg0 + blk * TB * 64 + 16 * wave;
    const int ntile = first >= seg1 ? 0 : min(TB, (seg1 - first + 63) / 64);
    typedef typename VT<E>::v8 v8;
    v8 bf[KS], ov[NP];
    auto fetch = [&](int tile, v8 *bo, v8 *oo) {
        const int64_t t = min(first + 64 * tile + l16, seg1 - 1);   // rows past the segment: clamped, not stored
        const E *brow = om + (t * d.HV + j) * K + 8 * grp;
        const E *orow = out + (t * d.HV + j) * V + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bo[ks] = ld8<E>(brow + 32 * ks);
#pragma unroll
        for (int q = 0; q < NP; ++q) oo[q] = ld8<E>(orow + 32 * q);
    };
    if (ntile > 0) fetch(0, bf, ov);
    const int va = 8 * (l16 >> 2) + (l16 & 3);   // A-operand row of this lane inside a 32-column block
    for (int tile = 0; tile < ntile; ++tile) {
        v8 nb[KS], no[NP];
        if (tile + 1 < ntile) fetch(tile + 1, nb, no);
        const int tt = first + 64 * tile + l16;
        E *orow = out + ((int64_t)tt * d.HV + j) * V + 8 * grp;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            f32x4 c0 = f32x4{0.f, 0.f, 0.f, 0.f}, c1 = c0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                c0 = mma(ld8<E>(&hT[(32 * q + va) * KP + 32 * ks + 8 * grp]), bf[ks], c0);
                c1 = mma(ld8<E>(&hT[(32 * q + 4 + va) * KP + 32 * ks + 8 * grp]), bf[ks], c1);
            }
            if (tt < seg1) {
                v8 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    r[e] = to_e<E>(to_f(ov[q][e]) + c0[e]);
                    r[4 + e] = to_e<E>(to_f(ov[q][4 + e]) + c1[e]);
                }
                *(v8 *)(orow + 32 * q) = r;
            }
            __builtin_amdgcn_sched_barrier(0);   // one block's h^T fragments live at a time
        }
        if (tile + 1 < ntile) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) bf[ks] = nb[ks];
#pragma unroll
            for (int q = 0; q < NP; ++q) ov[q] = no[q];
        }
    }
}

template <typename E>
hipError_t launch_correct(const SplitDims &d, const void *om, const void *hs, void *out, hipStream_t st) {
    const int nblk = (d.L + 64 * kCorrectTiles - 1) / (64 * kCorrectTiles);
    const unsigned grid = (unsigned)((int64_t)d.B * (d.S - 1) * d.HV * nblk);
    const E *o = (const E *)om, *hsT = (const E *)hs;
    E *dst = (E *)out;
    if (d.K == 64 && d.V == 64) split_correct_kernel<E, 64, 64><<<grid, 256, 0, st>>>(d, o, hsT, dst);
    else if (d.K == 64 && d.V == 128) split_correct_kernel<E, 64, 128><<<grid, 256, 0, st>>>(d, o, hsT, dst);
    else if (d.K == 128 && d.V == 64) split_correct_kernel<E, 128, 64><<<grid, 256, 0, st>>>(d, o, hsT, dst);
    else split_correct_kernel<E, 128, 128><<<grid, 256, 0, st>>>(d, o, hsT, dst);
    return hipGetLastError();
}

}  // namespace

// The split's workspace for callers that cannot allocate
// (gdn_chunk_fwd_noalloc): one copy of this array on every GPU the library
// runs on, held until the process ends.  In host code `scratch` is a host-side
// stand-in, never the device address: kernels and copies take the address
// static_scratch() looked up for the device.
static __device__ __align__(256) unsigned char scratch[GDN_STATIC_SCRATCH_BYTES];

hipError_t static_scratch(hipStream_t stream, void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int cur = -1, dev = -1;
    hipError_t err = hipGetDevice(&cur);
    if (err != hipSuccess) return err;
    dev = cur;
    if (stream) {   // the stream's device, which need not be the current one
        err = hipStreamGetDevice(stream, &dev);
        if (err != hipSuccess) return err;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        // once per device, with that device current
        if (dev != cur && (err = hipSetDevice(dev)) != hipSuccess) return err;
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t back = hipSetDevice(cur);
            if (err == hipSuccess) err = back;
        }
        if (err != hipSuccess) return err;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

SplitPlan plan_split(int B, int T, int H, int HV, int K, int V, int elem_bytes) {
    (void)H;
    SplitPlan pl;
    // workgroups of the unsplit launch (one per sequence, value head, 64 columns)
    const int64_t units = (int64_t)B * HV * (V / 64);
    if (B < 1 || units > 64 || T < 2048 || elem_bytes == 0) return pl;
    int S = (int)(256 / units);
    S = S < 2 ? 2 : S > 8 ? 8 : S;
    // With V = 128 the forward gives each (sequence, value head) one workgroup
    // of 128 columns once there are 256 such pairs, and runs a column about a
    // third faster that way than in two 64-column workgroups: take the
    // segments that make 256 pairs where at most 8 do.
    const int64_t heads = (int64_t)B * HV;
    if (V == 128 && heads * 8 >= 256) {
        const int S128 = (int)((256 + heads - 1) / heads);
        S = S128 > S ? S128 : S;
    }
    const int L = ((T + S - 1) / S + 63) / 64 * 64;
    S = (T + L - 1) / L;
    if (S < 2) return pl;
    pl.active = true;
    pl.S = S;
    pl.L = L;
    const size_t nseg = (size_t)B * S, st = (size_t)HV * K * V * 4, mt = (size_t)HV * K * K * 4;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    pl.off_cu = take((nseg + 1) * 4);
    pl.off_idx = take(nseg * 4);
    pl.off_pool = take(nseg * st);
    pl.off_map = take(nseg * mt);
    pl.off_hs = take(nseg * st);
    pl.off_om = take((size_t)B * T * HV * K * elem_bytes);
    pl.off_id = take(mt);
    pl.off_zero = take((size_t)HV * K * elem_bytes);
    pl.bytes = o;
    return pl;
}

hipError_t launch_split(const Params &p, int dtype, const SplitPlan &pl, void *ws, hipStream_t stream,
                        Profiler *prof) {
    char *w = (char *)ws;
    int32_t *cu = (int32_t *)(w + pl.off_cu), *idx = (int32_t *)(w + pl.off_idx);
    float *pool = (float *)(w + pl.off_pool), *maps = (float *)(w + pl.off_map), *hs = (float *)(w + pl.off_hs);
    float *ident = (float *)(w + pl.off_id);
    void *om = w + pl.off_om, *zrow = w + pl.off_zero;
    const SplitDims d{p.B, p.T, p.HV, p.K, p.V, pl.S, pl.L};
    const int nseg = p.B * pl.S;
    hipError_t err;

    if (prof) prof->begin(kSplitSetupKernel, stream);
    if (dtype == 0)
        split_setup_kernel<bf16><<<1024, 256, 0, stream>>>(d, p.initial_state, cu, idx, pool, ident, (bf16 *)zrow);
    else
        split_setup_kernel<float><<<1024, 256, 0, stream>>>(d, p.initial_state, cu, idx, pool, ident, (float *)zrow);
    err = hipGetLastError();
    if (prof) prof->end(kSplitSetupKernel, stream);
    if (err != hipSuccess) return err;

    // the segments as packed sequences: states in the pool (segment 0 starts
    // from the caller's state), outputs o0 into the caller's buffer
    Params a = p;
    a.B = 1;
    a.T = p.B * p.T;
    a.N = nseg;
    a.cu_seqlens = cu;
    a.initial_state = pool;
    a.final_state = pool;
    a.state_indices = idx;
    a.pool_size = nseg;
    a.state_bf16 = 0;
    err = launch_forward(a, dtype, stream, prof);
    if (err != hipSuccess) return err;

    // the transfer maps: v = 0, the identity as initial state (K state columns)
    Params m = a;
    m.V = p.K;
    m.v = zrow;
    m.v_zero = 1;
    m.initial_state = ident;
    m.init_shared = 1;
    m.final_state = maps;
    m.state_indices = nullptr;
    m.pool_size = 0;
    m.out = om;
    err = launch_forward(m, dtype, stream, prof);
    if (err != hipSuccess) return err;

    if (prof) prof->begin(kSplitCombineKernel, stream);
    const unsigned ncomb = (unsigned)(p.B * p.HV * (p.V / kCombineCols));
    if (dtype == 0)
        split_combine_kernel<bf16><<<ncomb, 256, 0, stream>>>(d, pool, maps, (bf16 *)hs, p.final_state);
    else
        split_combine_kernel<float><<<ncomb, 256, 0, stream>>>(d, pool, maps, (float *)hs, p.final_state);
    err = hipGetLastError();
    if (prof) prof->end(kSplitCombineKernel, stream);
    if (err != hipSuccess) return err;

    if (prof) prof->begin(kSplitCorrectKernel, stream);
    err = dtype == 0 ? launch_correct<bf16>(d, om, hs, p.out, stream) : launch_correct<float>(d, om, hs, p.out, stream);
    if (prof) prof->end(kSplitCorrectKernel, stream);
    return err;
}

}  // namespace gdn
