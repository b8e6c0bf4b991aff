// Sequence split of long sequences for gfx950: the plan, the setup, combine
// and final-state kernels, and the launch sequence (the scheme is described
// with SplitPlan in gdn_internal.h).
//
// It rests on the state being affine in a segment's initial state: with
// A_t = e^{g_t} (I - beta_t k_t k_t^T), the recurrence S_t = A_t S_{t-1} +
// beta_t k_t v_t^T of the Gated Delta Networks rule (cited by the page "NPU
// Training Operators - GDN", References) gives S_end = F + M h for a segment
// started from h, where F is its end state from a zero start and M = A_last
// ... A_first is what the same recurrence computes from the identity with
// v = 0.  The segments' starting states follow in order from (F, M), and one
// more pass from those starts gives the outputs directly.
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

// The segments' starting states: h_0 is the caller's state (already in slot
// (b, 0) of the start pool), h_1 = F_0 (segment 0 ran from h_0), and
// h_{s+1} = M_s h_s + F_s in segment order; h_s (s >= 1) is written into slot
// (b, s) of the start pool.  One workgroup per (sequence, value head, 32
// state columns): M_s and the workgroup's columns of h_s in LDS, each thread
// a 4 x 4 block of the product, fp32 throughout.
constexpr int kCombineCols = 32;

__global__ void __launch_bounds__(256) split_combine_kernel(SplitDims d, const float *__restrict__ fin,
                                                            const float *__restrict__ maps,
                                                            float *__restrict__ starts) {
    constexpr int CW = kCombineCols, CP = CW + 4, MP = 128 + 4;   // padded rows of h and M
    __shared__ __attribute__((aligned(16))) float h[128 * CP], m[128 * MP];
    const int K = d.K, V = d.V, ncb = V / CW;
    const int cb = blockIdx.x % ncb, bj = blockIdx.x / ncb;
    const int b = bj / d.HV, j = bj % d.HV, col0 = cb * CW;
    const int t = threadIdx.x, nb = (K / 4) * (CW / 4);
    const int r0 = 4 * (t / (CW / 4)), c0 = 4 * (t % (CW / 4));
    const float *f0 = fin + ((int64_t)b * d.S * d.HV + j) * K * V;
    for (int i = t; i < K * CW; i += blockDim.x) h[(i / CW) * CP + i % CW] = f0[(i / CW) * V + col0 + i % CW];
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
    if (d.S > 2) fetch_m(1);
    for (int s = 1; s < d.S; ++s) {
        const int64_t slot = (int64_t)b * d.S + s;
        __syncthreads();   // h_s is in place (the load above, or step s - 1)
        float *hd = starts + (slot * d.HV + j) * K * V + col0;
        for (int i = t; i < K * CW; i += blockDim.x) hd[(i / CW) * V + i % CW] = h[(i / CW) * CP + i % CW];
        if (s + 1 == d.S) break;   // the last segment's start is the last one needed
#pragma unroll
        for (int u = 0; u < NM; ++u) {
            const int i = 4 * (t + 256 * u);
            if (i < K * K) *(f32x4 *)&m[(i / K) * MP + i % K] = mr[u];
        }
        __syncthreads();   // M_s is in place
        if (s + 2 < d.S) fetch_m(s + 1);
        float acc[4][4];
        if (t < nb) {
            const float *fs = fin + (slot * d.HV + j) * K * V + col0;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[a][c] = fs[(r0 + a) * V + c0 + c];
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
}

// final_state[b] = the end state of segment (b, S - 1), 16 bytes per thread.
__global__ void __launch_bounds__(256) split_final_kernel(SplitDims d, const float *__restrict__ fin,
                                                          float *__restrict__ final_state) {
    const int64_t st4 = (int64_t)d.HV * d.K * d.V / 4, n4 = (int64_t)d.B * st4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = i / st4, r = i % st4;
        ((f32x4 *)final_state)[i] = ((const f32x4 *)fin)[(b * d.S + d.S - 1) * st4 + r];
    }
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
    pl.off_fin = take(nseg * st);
    pl.off_id = take(mt);
    pl.off_zero = take((size_t)HV * K * elem_bytes);
    pl.bytes = o;
    return pl;
}

hipError_t launch_split(const Params &p, int dtype, const SplitPlan &pl, void *ws, hipStream_t stream,
                        Profiler *prof) {
    char *w = (char *)ws;
    int32_t *cu = (int32_t *)(w + pl.off_cu), *idx = (int32_t *)(w + pl.off_idx);
    float *pool = (float *)(w + pl.off_pool), *maps = (float *)(w + pl.off_map), *fin = (float *)(w + pl.off_fin);
    float *ident = (float *)(w + pl.off_id);
    void *zrow = w + pl.off_zero;
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

    // 1. the segments as packed sequences, without outputs: segment 0 from the
    //    caller's state (slot (b, 0) of the start pool), the others from zero;
    //    end states F into fin
    Params a = p;
    a.B = 1;
    a.T = p.B * p.T;
    a.N = nseg;
    a.cu_seqlens = cu;
    a.initial_state = pool;
    a.final_state = fin;
    a.state_indices = idx;
    a.pool_size = nseg;
    a.state_bf16 = 0;
    a.out = nullptr;
    err = launch_forward(a, dtype, stream, prof);
    if (err != hipSuccess) return err;

    // 2. the transfer maps, without outputs: v = 0, the identity as the
    //    initial state (K state columns)
    Params m = a;
    m.V = p.K;
    m.v = zrow;
    m.v_zero = 1;
    m.initial_state = ident;
    m.init_shared = 1;
    m.final_state = maps;
    m.state_indices = nullptr;
    m.pool_size = 0;
    err = launch_forward(m, dtype, stream, prof);
    if (err != hipSuccess) return err;

    // 3. the segments' starting states into the start pool
    if (prof) prof->begin(kSplitCombineKernel, stream);
    const unsigned ncomb = (unsigned)(p.B * p.HV * (p.V / kCombineCols));
    split_combine_kernel<<<ncomb, 256, 0, stream>>>(d, fin, maps, pool);
    err = hipGetLastError();
    if (prof) prof->end(kSplitCombineKernel, stream);
    if (err != hipSuccess) return err;

    // 4. the segments again from their starting states, with outputs
    Params o = a;
    o.out = p.out;
    err = launch_forward(o, dtype, stream, prof);
    if (err != hipSuccess) return err;

    // 5. the sequences' final states: the last segments' end states
    if (p.final_state) {
        if (prof) prof->begin(kSplitFinalKernel, stream);
        split_final_kernel<<<256, 256, 0, stream>>>(d, fin, p.final_state);
        err = hipGetLastError();
        if (prof) prof->end(kSplitFinalKernel, stream);
    }
    return err;
}

}  // namespace gdn
