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
    // 16 bytes per store (HV K V and K K are multiples of 4)
    const int64_t st4 = (int64_t)d.HV * d.K * d.V / 4;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i = tid; i < nseg * st4; i += nth) {
        const int64_t slot = i / st4, r = i - slot * st4;
        const int64_t b = slot / d.S, s = slot - b * d.S;
        ((f32x4 *)pool)[i] = (s == 0 && init) ? ((const f32x4 *)init)[b * st4 + r] : z4;
    }
    const int kk4 = d.K * d.K / 4;
    for (int64_t i = tid; i < (int64_t)d.HV * kk4; i += nth) {
        const int r = (int)(i % kk4), row = r / (d.K / 4), c0 = 4 * (r - row * (d.K / 4));
        f32x4 v = z4;
        if (row >= c0 && row < c0 + 4) v[row - c0] = 1.f;
        ((f32x4 *)ident)[i] = v;
    }
    for (int64_t i = tid; i < (int64_t)d.HV * d.K; i += nth) zrow[i] = to_e<E>(0.f);
}

// The segments' starting states: h_0 is the caller's state (already in slot
// (b, 0) of the start pool), h_1 = F_0 (segment 0 ran from h_0), and
// h_{s+1} = M_s h_s + F_s in segment order; h_s (s >= 1) is written into slot
// (b, s) of the start pool.  One workgroup of four waves per (sequence, value
// head, 32 state columns), fp32 throughout: wave w computes rows
// 16 RT w .. 16 RT (w + 1) - 1 of h_{s+1} (both 16-column tiles) with fp32
// matrix-core products (16x16x4); its rows of M_s go from global memory
// straight into registers, a step ahead, and F_s's tiles start the sums; h_s
// sits in LDS transposed (a column's K entries contiguous, padded by four so
// that the sixteen columns of a read fall in different banks), double-buffered
// so that each step needs one barrier.
constexpr int kCombineCols = 32;
template <int K>
__global__ void __launch_bounds__(256) split_combine_kernel(SplitDims d, const float *__restrict__ fin,
                                                            const float *__restrict__ maps,
                                                            float *__restrict__ starts) {
    constexpr int CW = kCombineCols, RT = K / 64, KB = K / 32, HP = K + 4;
    __shared__ __attribute__((aligned(16))) float ht[2][CW * HP];
    const int V = d.V, ncb = V / CW;
    const int cb = blockIdx.x % ncb, bj = blockIdx.x / ncb;
    const int b = bj / d.HV, j = bj % d.HV, col0 = cb * CW;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, l16 = lane & 15, grp = lane >> 4;
    const int row0 = wave * 16 * RT;
    // offset of this workgroup's columns of state (b, s)
    auto soff = [&](int s) { return (((int64_t)b * d.S + s) * d.HV + j) * K * V + col0; };
    // h_1 = F_0
    {
        const float *f0 = fin + soff(0);
        for (int i = t; i < K * CW; i += 256) ht[0][(i % CW) * HP + i / CW] = f0[(int64_t)(i / CW) * V + i % CW];
    }
    // M_s's rows of this wave as A fragments (slot e of lane (l16, grp) in
    // block kb: column 32 kb + 8 grp + e), F_s's tiles in the accumulator layout
    f32x8 mn[RT][KB];
    f32x4 fn[RT][2];
    auto fetch = [&](int s) {
        const float *ms = maps + (((int64_t)b * d.S + s) * d.HV + j) * K * K;
        const float *fs = fin + soff(s);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float *pr = ms + (int64_t)(row0 + 16 * rt + l16) * K + 8 * grp;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const f32x4 lo = *(const f32x4 *)(pr + 32 * kb), hi = *(const f32x4 *)(pr + 32 * kb + 4);
                mn[rt][kb] = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) fn[rt][ct][e] = fs[(int64_t)(row0 + 16 * rt + 4 * grp + e) * V + 16 * ct + l16];
        }
    };
    if (d.S > 2) fetch(1);
    __syncthreads();   // h_1 is in place
    int buf = 0;
    for (int s = 1; s < d.S; ++s) {
        const float *hs = ht[buf];
        float *hd = starts + soff(s);
        for (int i = t; i < K * CW; i += 256) hd[(int64_t)(i / CW) * V + i % CW] = hs[(i % CW) * HP + i / CW];
        if (s + 1 == d.S) break;   // the last segment's start is the last one needed
        f32x8 mc[RT][KB];
        f32x4 acc[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) mc[rt][kb] = mn[rt][kb];
            acc[rt][0] = fn[rt][0];
            acc[rt][1] = fn[rt][1];
        }
        if (s + 2 < d.S) fetch(s + 1);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f32x8 bf[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const float *pc = hs + (16 * ct + l16) * HP + 32 * kb + 8 * grp;
                const f32x4 lo = *(const f32x4 *)pc, hi = *(const f32x4 *)(pc + 4);
                bf[ct] = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = mma(mc[rt][kb], bf[ct], acc[rt][ct]);
        }
        float *hn = ht[buf ^ 1];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) *(f32x4 *)&hn[(16 * ct + l16) * HP + row0 + 16 * rt + 4 * grp] = acc[rt][ct];
        __syncthreads();   // h_{s+1} is in place; h_s is no longer read
        buf ^= 1;
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
    if (p.K == 64) split_combine_kernel<64><<<ncomb, 256, 0, stream>>>(d, fin, maps, pool);
    else split_combine_kernel<128><<<ncomb, 256, 0, stream>>>(d, fin, maps, pool);
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
