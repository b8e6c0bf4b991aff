// Backward pass of the chunked gated delta rule, for gfx950.
//
// The page "NPU Training Operators - GDN" lists, beside the forward operators,
// the backward ones (gradients of q, k, v, the gates g and beta, and of the
// initial state; the gate gradient by a reverse cumulative sum).  The pages
// give no equations for them; the ones below are the chain rule applied to the
// chunked (WY) form of the forward pass.  Per chunk of L <= 64 rows, with
// gamma the chunk-local inclusive cumsum of g, D_i = exp(gamma_i), qh / kh the
// (optionally L2-normalised) rows and h the state at the chunk start:
//
//   A    = strictly lower, A_ij = beta_i exp(gamma_i - gamma_j) kh_i . kh_j
//   Tm   = (I + A)^-1
//   B    = diag(beta) (V - diag(D) Kh h)
//   Vn   = Tm B                                      (the delta-rule errors)
//   h'   = D_L h + Kh^T diag(exp(gamma_L - gamma)) Vn
//   O    = scale (diag(D) Qh h + Pm Vn),  Pm_ij = [j <= i] exp(gamma_i - gamma_j) qh_i . kh_j
//
// Going back through a chunk, given dO and dh' (the gradient of h'):
//
//   dVn  = scale Pm^T dO + diag(exp(gamma_L - gamma)) Kh dh'
//   dB   = Tm^T dVn                                  ((I + A) Vn = B)
//   dh   = D_L dh' + scale Qh^T diag(D) dO - Kh^T diag(beta D) dB
//   dA   = -dB Vn^T (strictly lower part),  dV = diag(beta) dB
//   dQh  = scale diag(D) dO h^T + dSqk Kh,    dSqk = [j <= i] exp(gamma_i - gamma_j) scale (dO Vn^T)_ij
//   dKh  = dSqk^T Qh + F dh'^T - diag(beta) E + Ad Kh + Ad^T Kh
//          with F = diag(exp(gamma_L - gamma)) Vn, E = diag(D) dB h^T, Ad = dA * beta_i exp(gamma_i - gamma_j)
//   dbeta_i  = dB_i . V_i - kh_i . E_i + sum_j dA_ij exp(gamma_i - gamma_j) kh_i . kh_j
//   dgamma_i = qh_i . (scale D_i dO_i h^T) - beta_i kh_i . E_i - kh_i . (F dh'^T)_i
//              + rowsum_i(Z) - colsum_i(Z),   Z = dSqk * (qh_i . kh_j) + dA * A
//              + [i = L] (D_L <dh', h> + sum_j kh_j . (F dh'^T)_j)
//   dg_s     = sum_{i >= s in the chunk} dgamma_i
//
// and the L2 norm's backward dx = f (dxh - xh (xh . dxh)), f = 1/sqrt(|x|^2 + 1e-6).
// The state gradient runs backwards over chunks just as the state runs
// forwards, so the pass is five launches (six with packed sequences, whose
// chunk offsets, and for 2..kSeqOrderMax sequences the longest-first order the
// two scans take them in, bwd_setup_kernel computes first):
//   bwd_prep_kernel      per (chunk, value head): gamma, Tm, A / beta and Pm
//   bwd_fwd_scan_kernel  per (sequence, value head, 64 value columns; 32 for
//                        fp32 rows), forward over chunks: the chunk-start
//                        states h and Vn
//   bwd_dh_scan_kernel   the same grid, backward over chunks: dh' per chunk,
//                        dB, the initial-state gradient
// (with few (sequence, value head) pairs both scans take 32- or 16-column
// tiles; bf16 rows at 64 columns rescan in bwd_fwd_scan_b16_kernel, and at 16
// columns with K = 128 both scans run the 8-wave *_sk_kernel forms)
//   bwd_grads_kernel     per (chunk, value head): dq, dk per value head, dv,
//                        dg, dbeta
//   bwd_reduce_kernel    dq, dk summed over the value heads of each key head
// All arithmetic is fp32-accurate: the products run on the matrix cores with
// fp32 operands (v_mfma_f32_16x16x4f32), except on v_mfma_f32_16x16x32_bf16
// with fp32 accumulation where every operand is exact in bf16: the prep
// kernel's K K^T and Q K^T of raw bf16 rows, and the products of the 64-column
// bf16 rescan and of the gradients kernel over the value columns, which split
// each fp32 operand into bf16 hi + lo parts (hi hi + hi lo + lo hi; a bf16
// input is its own hi part).  The intermediates live in the caller's workspace
// (layout in BwdPlan).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

using namespace dev;

constexpr int kThreads = 256;
constexpr int kVT = 32;          // value columns per tile of the gradients kernel
constexpr int kPadC = kChunk + 1;

// Tm, A / beta and Pm are zero above their diagonal 16 x 16 blocks, so the
// workspace keeps only the ten blocks on and below the diagonal: block
// (bi, bj), bj <= bi, at bi (bi + 1) / 2 + bj, row-major inside the block
// (10 of the 16 blocks of a full 64 x 64 tile).
constexpr int kTriFloats = 10 * 16 * 16;
__device__ __forceinline__ bool tri_in(int r, int c) { return (c >> 4) <= (r >> 4); }
__device__ __forceinline__ int tri_off(int r, int c) {
    const int bi = r >> 4, bj = c >> 4;
    return (bi * (bi + 1) / 2 + bj) * 256 + (r & 15) * 16 + (c & 15);
}

// LDS sizes in floats.
// grads: the value tiles (2 K x 33 + 4 x 64 x 33) come first and the two
// 64 x 65 matrices of the second phase reuse their space.
// grads: the value tiles as bf16 hi / lo pairs, rows of 32 value columns at a
// stride of kVS elements (16-byte aligned MFMA operand reads): h, dh' (K rows
// each), Vn, dB, dO (64 rows each, hi and lo); the two 64 x 65 fp32 matrices of
// the second phase reuse the space.
constexpr int kVS = 40;
template <int K>
constexpr int grads_tile_floats() { return (4 * K + 6 * kChunk) * kVS / 2; }
static_assert(grads_tile_floats<64>() >= 2 * kChunk * kPadC, "phase-2 matrices must fit in the tile region");

// Products on the matrix cores: 16 x 16 fp32 tiles by v_mfma_f32_16x16x4f32
// (fp32 operands, fp32 accumulation, so the pass keeps fp32 accuracy).
// Inside a wave, lane l holds elements (4 (l >> 4) + e, l & 15), e < 4, of
// each tile.  A k-step feeds four contraction indices, one per group of 16
// lanes: group q takes index q KD/4 + s at step s, the same index for both
// operands, so the assignment only fixes the order of the sum.
//   acc[t] += sum_{m < KD} fa(ra(t) + (l & 15), m) * fb(cb(t) + (l & 15), m)
// Operand reads that coincide between tiles (same ra or cb) are shared.  The
// k-steps run in groups whose operands are read from LDS into registers ahead
// of their products: the next group's reads are issued before the current
// group's products, so LDS latency hides behind matrix-core work.  Groups are
// sized to keep at most ~15 reads in flight (what the LDS counter tracks).
template <int NT>
constexpr int wmm_group(int S) {
    return (S % 4 == 0 && NT + 1 <= 4) ? 4 : (S % 2 == 0 ? 2 : 1);
}
template <int NT, int KD, typename RA, typename CB, typename FA, typename FB>
__device__ __forceinline__ void wmm(f32x4 (&acc)[NT], RA ra, CB cb, FA fa, FB fb) {
    constexpr int S = KD / 4;
    constexpr int G = wmm_group<NT>(S);
    static_assert(S % G == 0, "k-steps must split into whole groups");
    const int i = threadIdx.x & 15, q = (threadIdx.x >> 4) & 3;
    float av[2][G][NT], bv[2][G][NT];
    auto load = [&](int buf, int g) {
#pragma unroll
        for (int s = 0; s < G; ++s) {
            const int m = q * S + g + s;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                av[buf][s][t] = fa(ra(t) + i, m);
                bv[buf][s][t] = fb(cb(t) + i, m);
            }
        }
    };
    auto run = [&](int buf) {
#pragma unroll
        for (int s = 0; s < G; ++s)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[buf][s][t], bv[buf][s][t], acc[t], 0, 0, 0);
    };
    load(0, 0);
#pragma unroll 1
    for (int g = 0; g < S; g += 2 * G) {
        if (g + G < S) load(1, g + G);
        run(0);
        if (g + 2 * G < S) load(0, g + 2 * G);
        if (g + G < S) run(1);
    }
}

// Two products that share the second operand:
//   acc1[t] += sum_m fa1(ra(t) + (l & 15), m) fb(cb(t) + (l & 15), m), acc2 likewise with fa2.
template <int NT, int KD, typename RA, typename CB, typename FA1, typename FA2, typename FB>
__device__ __forceinline__ void wmm2(f32x4 (&acc1)[NT], f32x4 (&acc2)[NT], RA ra, CB cb, FA1 fa1, FA2 fa2, FB fb) {
    constexpr int S = KD / 4;
    constexpr int G0 = NT >= 4 ? 4 : 8;
    constexpr int G = S <= G0 ? S : (S % G0 == 0 ? G0 : (S % 4 == 0 ? 4 : 1));
    static_assert(S % G == 0, "k-steps must split into whole groups");
    const int i = threadIdx.x & 15, q = (threadIdx.x >> 4) & 3;
#pragma unroll 1
    for (int g = 0; g < S; g += G) {
        float a1[G][NT], a2[G][NT], bv[G][NT];
#pragma unroll
        for (int s = 0; s < G; ++s) {
            const int m = q * S + g + s;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                a1[s][t] = fa1(ra(t) + i, m);
                a2[s][t] = fa2(ra(t) + i, m);
                bv[s][t] = fb(cb(t) + i, m);
            }
        }
#pragma unroll
        for (int s = 0; s < G; ++s)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                acc1[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[s][t], bv[s][t], acc1[t], 0, 0, 0);
                acc2[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2[s][t], bv[s][t], acc2[t], 0, 0, 0);
            }
    }
}

template <int NT>
__device__ __forceinline__ void zero(f32x4 (&acc)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Row and column of element e of this lane in a tile at (r0, c0).
__device__ __forceinline__ int lrow(int r0, int e) { return r0 + 4 * ((threadIdx.x >> 4) & 3) + e; }
__device__ __forceinline__ int lcol(int c0) { return c0 + (threadIdx.x & 15); }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Sum over the 16 lanes that hold the same tile rows (lanes l & 15 = 0..15).
__device__ __forceinline__ float sum16(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// The chunk of a chunk index: sequence n, first token t0 (packed index),
// rows L, and the chunk index c inside its sequence.  Returns false for
// indices past the last chunk.
struct ChunkRef {
    int n, c, t0, L;
};
__device__ __forceinline__ bool find_chunk(const BwdParams &p, int cid, ChunkRef &r) {
    if (!p.cu_seqlens) {
        const int ncs = (p.T + kChunk - 1) / kChunk;
        if (ncs == 0 || cid >= p.B * ncs) return false;
        r.n = cid / ncs;
        r.c = cid - r.n * ncs;
        r.t0 = r.n * p.T + r.c * kChunk;
        r.L = min(kChunk, p.T - r.c * kChunk);
        return true;
    }
    const int *co = p.chunk_offsets;
    if (cid >= co[p.N]) return false;
    int lo = 0, hi = p.N;   // co[lo] <= cid < co[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (co[mid] <= cid) lo = mid;
        else hi = mid;
    }
    r.n = lo;
    r.c = cid - co[lo];
    const int bos = p.cu_seqlens[lo], eos = p.cu_seqlens[lo + 1];
    r.t0 = bos + r.c * kChunk;
    r.L = min(kChunk, eos - r.t0);
    return true;
}

// Sequence n's first token, length and first chunk index.
__device__ __forceinline__ void seq_of(const BwdParams &p, int n, int &bos, int &len, int &cid0) {
    if (!p.cu_seqlens) {
        bos = n * p.T;
        len = p.T;
        cid0 = n * ((p.T + kChunk - 1) / kChunk);
    } else {
        bos = p.cu_seqlens[n];
        len = p.cu_seqlens[n + 1] - bos;
        cid0 = p.chunk_offsets[n];
    }
}

// ---- register-staged copies for workgroups of NTH threads and value tiles
// of VW columns (the scans), with the key/query rows kept raw in the input
// type in LDS (row stride K + RowPad<E>; the L2 norms are applied as row
// scales inside the products).
template <typename E> struct RowPad;
template <> struct RowPad<bf16> { static constexpr int v = 2; };    // 4-byte rows, odd word stride
template <> struct RowPad<float> { static constexpr int v = 1; };

template <typename E, int K, int NTH, int PAD = RowPad<E>::v>
struct RawRowsReg {
    static constexpr int PER_ROW = K / 8, VPT = kChunk * PER_ROW / NTH, KS = K + PAD;
    static_assert(VPT >= 1 && kChunk * PER_ROW % NTH == 0, "rows must split evenly");
    typename VT<E>::v8 v[VPT];
    __device__ __forceinline__ void load(const E *src, int t0, int L, int H, int jk) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int i = threadIdx.x + NTH * u, r = i / PER_ROW, c = (i % PER_ROW) * 8;
            if (r < L) v[u] = ld8<E>(src + ((int64_t)(t0 + r) * H + jk) * K + c);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) v[u][e] = to_e<E>(0.f);
        }
    }
    __device__ __forceinline__ void commit(E *dst) const {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int i = threadIdx.x + NTH * u, r = i / PER_ROW, c = (i % PER_ROW) * 8;
            if constexpr (sizeof(E) == 2) {   // even offsets: four 32-bit words
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 x = __builtin_bit_cast(u32x4, v[u]);
                unsigned int *d = (unsigned int *)(dst + r * KS + c);
#pragma unroll
                for (int e = 0; e < 4; ++e) d[e] = x[e];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) dst[r * KS + c + e] = v[u][e];
            }
        }
    }
};
// A 64 x 64 fp32 matrix (contiguous) into dst[64][65].
template <int NTH>
struct Mat64RegN {
    static constexpr int N4 = kChunk * kChunk / 4 / NTH;
    f32x4 v[N4];
    // from the lower block-triangular storage (tri_off); the blocks above the
    // diagonal are zero
    __device__ __forceinline__ void load(const float *src) {
#pragma unroll
        for (int u = 0; u < N4; ++u) {
            const int i = threadIdx.x + NTH * u, r = i >> 4, c = (i & 15) * 4;
            v[u] = tri_in(r, c) ? *(const f32x4 *)(src + tri_off(r, c)) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __device__ __forceinline__ void commit(float *dst) const {
#pragma unroll
        for (int u = 0; u < N4; ++u) {
            const int i = threadIdx.x + NTH * u, r = i >> 4, c = (i & 15) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[r * kPadC + c + e] = v[u][e];
        }
    }
};
// Rows t0..t0+L-1 (zero past L), VW columns from c0, of a [T_tot, HV, V]
// tensor at value head j, into dst[64][VW+1] as fp32.
template <typename E, int VW, int NTH>
struct TileRegN {
    static constexpr int EPT = kChunk * VW / NTH;   // consecutive elements per thread
    static_assert(EPT == 8 || EPT == 4, "one run of 8 or 4 elements per thread");
    typedef typename VT<E>::v8 v8t;
    typedef typename VT<E>::v4 v4t;
    typename std::conditional<EPT == 8, v8t, v4t>::type v;
    __device__ __forceinline__ void load(const E *src, int t0, int L, int HV, int j, int V, int c0) {
        const int r = threadIdx.x / (VW / EPT), c = (threadIdx.x % (VW / EPT)) * EPT;
        if (r < L) {
            const E *at = src + ((int64_t)(t0 + r) * HV + j) * V + c0 + c;
            if constexpr (EPT == 8) v = ld8<E>(at);
            else v = *(const v4t *)at;
        } else {
#pragma unroll
            for (int e = 0; e < EPT; ++e) v[e] = to_e<E>(0.f);
        }
    }
    __device__ __forceinline__ void commit(float *dst) const {
        const int r = threadIdx.x / (VW / EPT), c = (threadIdx.x % (VW / EPT)) * EPT;
#pragma unroll
        for (int e = 0; e < EPT; ++e) dst[r * (VW + 1) + c + e] = to_f(v[e]);
    }
};
// K rows x VW columns from c0 of a K x V fp32 state (row stride V), to and from dst[K][VW+1].
template <int K, int VW, int NTH>
struct StateTileN {
    static constexpr int N4 = K * VW / 4 / NTH, Q = VW / 4;
    f32x4 v[N4];
    __device__ __forceinline__ void load(const float *src, int V, int c0) {
#pragma unroll
        for (int u = 0; u < N4; ++u) {
            const int i = threadIdx.x + NTH * u, r = i / Q, c = (i % Q) * 4;
            v[u] = *(const f32x4 *)(src + (int64_t)r * V + c0 + c);
        }
    }
    __device__ __forceinline__ void commit(float *dst) const {
#pragma unroll
        for (int u = 0; u < N4; ++u) {
            const int i = threadIdx.x + NTH * u, r = i / Q, c = (i % Q) * 4;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[r * (VW + 1) + c + e] = v[u][e];
        }
    }
    static __device__ __forceinline__ void store(const float *tile, float *dst, int V, int c0) {
#pragma unroll
        for (int u = 0; u < N4; ++u) {
            const int i = threadIdx.x + NTH * u, r = i / Q, c = (i % Q) * 4;
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = tile[r * (VW + 1) + c + e];
            *(f32x4 *)(dst + (int64_t)r * V + c0 + c) = x;
        }
    }
};
// Sum of squares of row r of a raw row set, over the NTH / 64 lanes that
// share the row (r = threadIdx.x / (NTH / 64)); every such lane gets the sum.
template <typename E, int K, int NTH, int PAD = RowPad<E>::v>
__device__ __forceinline__ float row_sumsq(const E *rows, int r) {
    constexpr int LPR = NTH / kChunk, KS = K + PAD;
    const int part = threadIdx.x % LPR;
    float s = 0.f;
    for (int c = part; c < K; c += LPR) {
        const float x = to_f(rows[r * KS + c]);
        s = fmaf(x, x, s);
    }
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) s += __shfl_xor(s, o);
    return s;
}

// One block row I of Tm = (I + A)^-1 (16-row blocks, diagonal blocks already
// in Tm, blocks above the diagonal zero): wave J < I computes
// T_IJ = -X_I sum_{K<I} A_IK T_KJ, staging the sum in its scratch ysc [16][17].
// Every thread of the workgroup calls it (it holds two barriers).
template <int I>
__device__ __forceinline__ void tm_block_row(const float *A, float *Tm, float *ysc, int w) {
    if (w < I) {
        f32x4 y[1];
        zero(y);
        wmm<1, 16 * I>(y, [&](int) { return 16 * I; }, [&](int) { return 16 * w; },
                       [&](int r, int m) { return A[r * kPadC + m]; },
                       [&](int c, int m) { return Tm[m * kChunk + c]; });
#pragma unroll
        for (int e = 0; e < 4; ++e) ysc[lrow(0, e) * 17 + lcol(0)] = y[0][e];
    }
    lds_barrier();
    if (w < I) {
        f32x4 z[1];
        zero(z);
        wmm<1, 16>(z, [&](int) { return 16 * I; }, [&](int) { return 0; },
                   [&](int r, int m) { return Tm[r * kChunk + 16 * I + m]; },
                   [&](int c, int m) { return ysc[m * 17 + c]; });
#pragma unroll
        for (int e = 0; e < 4; ++e) Tm[lrow(16 * I, e) * kChunk + lcol(16 * w)] = -z[0][e];
    }
    lds_barrier();
}

// ---------------------------------------------------------------------------
// chunk offsets of packed sequences: co[n] = sum_{m < n} ceil(len_m / 64);
// with ord, also the sequences longest first (by chunk count, ties in index
// order: ord[rank] = n), which the two scans take their sequences in, so that
// a long sequence's serial scan never starts last (N <= kSeqOrderMax)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void bwd_setup_kernel(const int32_t *cu, int N, int32_t *co, int32_t *ord) {
    __shared__ int part[kThreads];
    __shared__ int ncs[kSeqOrderMax];
    const int per = (N + kThreads - 1) / kThreads;
    const int a = min(N, (int)threadIdx.x * per), b = min(N, a + per);
    int s = 0;
    for (int n = a; n < b; ++n) s += (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
    part[threadIdx.x] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int i = 0; i < kThreads; ++i) {
            const int x = part[i];
            part[i] = run;
            run += x;
        }
        co[N] = run;
    }
    __syncthreads();
    int run = part[threadIdx.x];
    for (int n = a; n < b; ++n) {
        co[n] = run;
        run += (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
    }
    if (ord) {
        for (int n = threadIdx.x; n < N; n += kThreads) ncs[n] = (cu[n + 1] - cu[n] + kChunk - 1) / kChunk;
        __syncthreads();
        for (int n = threadIdx.x; n < N; n += kThreads) {
            const int c = ncs[n];
            int r = 0;
            for (int m = 0; m < N; ++m) r += ncs[m] > c || (ncs[m] == c && m < n);
            ord[r] = n;
        }
    }
}

// ---------------------------------------------------------------------------
// per (chunk, value head): gamma, Tm = (I + A)^-1, A / beta and Pm
// ---------------------------------------------------------------------------
// Row padding of prep's raw rows: bf16 rows are MFMA operands read 16 bytes at a time.
template <typename E> struct PrepPad { static constexpr int v = sizeof(E) == 2 ? 8 : RowPad<E>::v; };
template <typename E, int K>
constexpr int prep_floats() {   // raw q/k rows, then A [64][65] and Tm [64][64] in the same space
    return ((2 * kChunk * (K + PrepPad<E>::v) * (int)sizeof(E) + 3) / 4 > kChunk * kPadC + kChunk * kChunk
                ? (2 * kChunk * (K + PrepPad<E>::v) * (int)sizeof(E) + 3) / 4
                : kChunk * kPadC + kChunk * kChunk) +
           4 * 16 * 17 + 4 * kChunk;
}
// bf16 rows: four workgroups per CU
static_assert(prep_floats<bf16, 128>() * 4 <= 40 * 1024, "bf16 prep must fit four times per CU");

template <typename E, int K>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(BwdParams p) {
    constexpr int PAD = PrepPad<E>::v, KS = K + PAD;
    __shared__ __attribute__((aligned(16))) float sm[prep_floats<E, K>()];
    E *kr = (E *)sm;                         // [64][KS] raw k rows
    E *qr = kr + kChunk * KS;                // [64][KS] raw q rows
    float *A = sm;                           // [64][65] after the products (the rows are dead then)
    float *Tm = A + kChunk * kPadC;          // [64][64]
    float *ysc = sm + prep_floats<E, K>() - 4 * 16 * 17 - 4 * kChunk;   // [4][16][17] solve scratch
    float *gam = ysc + 4 * 16 * 17;          // [64]
    float *bet = gam + kChunk;               // [64]
    float *fk = bet + kChunk;                // [64] 1 / |k|
    float *fq = fk + kChunk;                 // [64] 1 / |q|

    ChunkRef cr;
    if (!find_chunk(p, blockIdx.x, cr)) return;
    const int j = blockIdx.y, HV = p.HV, jk = j / (HV / p.H);
    const int cid = blockIdx.x, L = cr.L, t0 = cr.t0;

    if (threadIdx.x < kChunk) {   // wave 0: gamma by an inclusive scan over its 64 lanes
        const int r = threadIdx.x;
        float x = r < L ? p.g[(int64_t)(t0 + r) * HV + j] : 0.f;
#pragma unroll
        for (int o = 1; o < kChunk; o <<= 1) {
            const float y = __shfl_up(x, o);
            if (r >= o) x += y;
        }
        gam[r] = x;
        bet[r] = r < L ? p.beta[(int64_t)(t0 + r) * HV + j] : 0.f;
        if (r < L) p.gam[(int64_t)(t0 + r) * HV + j] = x;
    }
    {
        RawRowsReg<E, K, kThreads, PAD> rk, rq;
        rk.load((const E *)p.k, t0, L, p.H, jk);
        rq.load((const E *)p.q, t0, L, p.H, jk);
        rk.commit(kr);
        rq.commit(qr);
    }
    lds_barrier();
    {
        constexpr int LPR = kThreads / kChunk;
        const int r = threadIdx.x / LPR;
        const float sk = row_sumsq<E, K, kThreads, PAD>(kr, r), sq = row_sumsq<E, K, kThreads, PAD>(qr, r);
        if (threadIdx.x % LPR == 0) {
            fk[r] = p.use_l2norm ? 1.f / sqrtf(sk + 1e-6f) : 1.f;
            fq[r] = p.use_l2norm ? 1.f / sqrtf(sq + 1e-6f) : 1.f;
        }
    }

    // K K^T and Q K^T of the raw rows (the norms scale rows and columns below):
    // wave w computes rows 16w..16w+15, all four column tiles.
    const int w = wave_id();
    auto ra = [&](int) { return 16 * w; };
    auto cb = [&](int t) { return 16 * t; };
    f32x4 kk[4], qk[4];
    zero(kk);
    zero(qk);
    if constexpr (sizeof(E) == 2) {
        // bf16 rows are exact bf16 operands: one bf16 product per 32 keys, fp32 accumulation
        const int i = threadIdx.x & 15, q = (threadIdx.x >> 4) & 3;
#pragma unroll
        for (int k0 = 0; k0 < K; k0 += 32) {
            const bf16x8 ak = *(const bf16x8 *)(kr + (16 * w + i) * KS + k0 + 8 * q);
            const bf16x8 aq = *(const bf16x8 *)(qr + (16 * w + i) * KS + k0 + 8 * q);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bf16x8 b = *(const bf16x8 *)(kr + (16 * t + i) * KS + k0 + 8 * q);
                kk[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, b, kk[t], 0, 0, 0);
                qk[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, b, qk[t], 0, 0, 0);
            }
        }
    } else {
        wmm2<4, K>(kk, qk, ra, cb, [&](int r, int m) { return to_f(kr[r * KS + m]); },
                   [&](int r, int m) { return to_f(qr[r * KS + m]); },
                   [&](int c, int m) { return to_f(kr[c * KS + m]); });
    }
    float *ag_out = p.ag + ((int64_t)cid * HV + j) * kTriFloats;
    float *pm_out = p.pm + ((int64_t)cid * HV + j) * kTriFloats;
    lds_barrier();   // A overwrites qh
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = lrow(16 * w, e), c = lcol(16 * t);
            const float d = (c <= r && r < L) ? __expf(gam[r] - gam[c]) * fk[c] : 0.f;
            const float ag = c < r ? d * fk[r] * kk[t][e] : 0.f;
            A[r * kPadC + c] = bet[r] * ag;
            Tm[r * kChunk + c] = 0.f;
            if (tri_in(r, c)) {   // t <= w: the tile is on or below the diagonal
                ag_out[tri_off(r, c)] = ag;
                pm_out[tri_off(r, c)] = d * fq[r] * qk[t][e];
            }
        }
    lds_barrier();

    // Tm = (I + A)^-1, blocked by 16.  Wave w inverts the diagonal block
    // X_w = (I + A_ww)^-1 by forward substitution, X_im = -sum_{j<=m<i} A_im X_mj:
    // lane (column l & 15, part l >> 4) keeps rows part, part + 4, ... of its column.
    {
        const int col = threadIdx.x & 15, part = (threadIdx.x >> 4) & 3, b0 = 16 * w;
        float xr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = 0.f;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (part + 4 * u < i) s = fmaf(A[(b0 + i) * kPadC + b0 + part + 4 * u], xr[u], s);
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            const float x = i == col ? 1.f : (col < i ? -s : 0.f);
            if (part == (i & 3)) xr[i >> 2] = x;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) Tm[(b0 + part + 4 * u) * kChunk + b0 + col] = xr[u];
    }
    lds_barrier();
    // Off-diagonal blocks, one block row at a time.
    tm_block_row<1>(A, Tm, ysc + w * 16 * 17, w);
    tm_block_row<2>(A, Tm, ysc + w * 16 * 17, w);
    tm_block_row<3>(A, Tm, ysc + w * 16 * 17, w);
    float *tm_out = p.tm + ((int64_t)cid * HV + j) * kTriFloats;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = 4 * (threadIdx.x + kThreads * u), r = i >> 6, c = i & 63;
        if (tri_in(r, c)) *(f32x4 *)(tm_out + tri_off(r, c)) = f32x4{Tm[i], Tm[i + 1], Tm[i + 2], Tm[i + 3]};
    }
}

// ---------------------------------------------------------------------------
// forward over chunks per (sequence, value head, VW value columns), NTH
// threads: the chunk-start states h and Vn.  The key rows stay raw in LDS;
// their L2 norms enter as the row scales sD and sFk.
// ---------------------------------------------------------------------------
template <typename E, int K, int VW>
constexpr int fwd_scan_floats() {
    return K * (VW + 1) + kChunk * kPadC + kChunk * (VW + 1) + 5 * kChunk +
           (kChunk * (K + RowPad<E>::v) * (int)sizeof(E) + 3) / 4;
}
// fp32 rows: two workgroups share a CU (160 KB of LDS)
static_assert(fwd_scan_floats<float, 128, 32>() * 4 <= 80 * 1024, "fp32 forward scan must fit twice per CU");
static_assert(fwd_scan_floats<bf16, 128, 64>() * 4 <= 160 * 1024, "bf16 forward scan must fit one CU");

template <typename E, int K, int VW, int NTH>
__global__ __launch_bounds__(NTH) void bwd_fwd_scan_kernel(BwdParams p) {
    constexpr int VP = VW + 1, KS = K + RowPad<E>::v, W = NTH / 64, CT = VW / 16;
    constexpr int NT1 = 4 * CT / W;          // 16 x 16 tiles of a 64 x VW product per wave
    constexpr int NT2 = (K / 16) * CT / W;   // tiles of the K x VW state per wave
    static_assert(NT1 >= 1 && NT2 >= 1, "every wave needs a tile");
    __shared__ float sm[fwd_scan_floats<E, K, VW>()];
    float *h = sm;                           // [K][VP]
    float *Tm = h + K * VP;                  // [64][65]
    float *vv = Tm + kChunk * kPadC;         // [64][VP]: v, then B (in place), then F / |k|
    float *gam = vv + kChunk * VP;           // [64]
    float *bet = gam + kChunk;               // [64]
    float *sD = bet + kChunk;                // [64] exp(gamma) / |k|
    float *sF = sD + kChunk;                 // [64] exp(gamma_L - gamma), 0 past L
    float *sFk = sF + kChunk;                // [64] exp(gamma_L - gamma) / |k|, 0 past L
    E *kr = (E *)(sFk + kChunk);             // [64][KS] raw k rows

    const int HV = p.HV, V = p.V;
    const int seq_rank = blockIdx.x / HV, j = blockIdx.x - seq_rank * HV, jk = j / (HV / p.H);
    const int n = p.seq_order ? p.seq_order[seq_rank] : seq_rank;   // longest first for packed batches
    const int c0 = blockIdx.y * VW;
    int bos, len, cid0;
    seq_of(p, n, bos, len, cid0);
    const int nc = (len + kChunk - 1) / kChunk;

    if (p.initial_state) {
        StateTileN<K, VW, NTH> r0;
        r0.load(p.initial_state + ((int64_t)n * HV + j) * K * V, V, c0);
        r0.commit(h);
    } else {
        for (int e = threadIdx.x; e < K * VW; e += NTH) h[(e / VW) * VP + e % VW] = 0.f;
    }
    RawRowsReg<E, K, NTH> rk;
    Mat64RegN<NTH> rt;
    TileRegN<E, VW, NTH> rv;
    float rg = 0.f, rb = 0.f;
    auto fetch = [&](int ci) {
        const int cid = cid0 + ci, t0 = bos + ci * kChunk, L = min(kChunk, len - ci * kChunk);
        rk.load((const E *)p.k, t0, L, p.H, jk);
        rt.load(p.tm + ((int64_t)cid * HV + j) * kTriFloats);
        rv.load((const E *)p.v, t0, L, HV, j, V, c0);
        if (threadIdx.x < kChunk) {
            const int r = threadIdx.x;
            rg = r < L ? p.gam[(int64_t)(t0 + r) * HV + j] : 0.f;
            rb = r < L ? p.beta[(int64_t)(t0 + r) * HV + j] : 0.f;
        }
    };
    if (nc > 0) fetch(0);
    lds_barrier();
    const int w = wave_id();
    auto ra = [&](int t) { return 16 * ((w * NT1 + t) / CT); };
    auto cb = [&](int t) { return 16 * ((w * NT1 + t) % CT); };
    auto rs = [&](int t) { return 16 * ((w * NT2 + t) / CT); };
    auto cs = [&](int t) { return 16 * ((w * NT2 + t) % CT); };
    for (int ci = 0; ci < nc; ++ci) {
        const int cid = cid0 + ci, t0 = bos + ci * kChunk, L = min(kChunk, len - ci * kChunk);
        StateTileN<K, VW, NTH>::store(h, p.hs + ((int64_t)cid * HV + j) * K * V, V, c0);
        rk.commit(kr);
        rt.commit(Tm);
        rv.commit(vv);
        if (threadIdx.x < kChunk) {
            gam[threadIdx.x] = rg;
            bet[threadIdx.x] = rb;
        }
        lds_barrier();
        {
            constexpr int LPR = NTH / kChunk;   // lanes per row
            const int r = threadIdx.x / LPR;
            const float sk = row_sumsq<E, K, NTH>(kr, r);
            if (threadIdx.x % LPR == 0) {
                const float fk = p.use_l2norm ? 1.f / sqrtf(sk + 1e-6f) : 1.f;
                const float f = r < L ? __expf(gam[L - 1] - gam[r]) : 0.f;
                sD[r] = __expf(gam[r]) * fk;
                sF[r] = f;
                sFk[r] = f * fk;
            }
        }
        lds_barrier();
        if (ci + 1 < nc) fetch(ci + 1);

        // B = diag(beta) (V - diag(D) Kh h), in place over v
        {
            f32x4 x[NT1];
            zero(x);
            wmm<NT1, K>(x, ra, cb, [&](int r, int m) { return to_f(kr[r * KS + m]); },
                        [&](int c, int m) { return h[m * VP + c]; });
#pragma unroll
            for (int t = 0; t < NT1; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = lrow(ra(t), e), c = lcol(cb(t));
                    vv[r * VP + c] = bet[r] * (vv[r * VP + c] - sD[r] * x[t][e]);
                }
        }
        lds_barrier();
        // Vn = Tm B; then, once every wave has read B, diag(exp(gamma_L - gamma) / |k|) Vn into vv
        {
            f32x4 x[NT1];
            zero(x);
            wmm<NT1, kChunk>(x, ra, cb, [&](int r, int m) { return Tm[r * kPadC + m]; },
                             [&](int c, int m) { return vv[m * VP + c]; });
            lds_barrier();
#pragma unroll
            for (int t = 0; t < NT1; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = lrow(ra(t), e), c = lcol(cb(t));
                    if (r < L) p.vn[((int64_t)(t0 + r) * HV + j) * V + c0 + c] = x[t][e];
                    vv[r * VP + c] = sFk[r] * x[t][e];
                }
        }
        lds_barrier();
        // h <- D_L h + Kh^T F
        {
            f32x4 x[NT2];
            zero(x);
            wmm<NT2, kChunk>(x, rs, cs, [&](int r, int m) { return to_f(kr[m * KS + r]); },
                             [&](int c, int m) { return vv[m * VP + c]; });
            const float dl = __expf(gam[L - 1]);
#pragma unroll
            for (int t = 0; t < NT2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float &hv = h[lrow(rs(t), e) * VP + lcol(cs(t))];
                    hv = fmaf(dl, hv, x[t][e]);
                }
        }
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// The forward rescan for bf16 rows with 64 value columns and 8 waves, with its
// two products over 128 keys / 64 tokens on the bf16 matrix cores: K h with
// the raw bf16 key rows (exact) against bf16 hi / lo parts of the state, and
// K^T F with the transposed raw rows against hi / lo parts of F.  The state
// stays in fp32 (hs and the update use it); its hi / lo copy, transposed to
// [value column][key], is refreshed by every update.  Tm B keeps fp32 products.
// ---------------------------------------------------------------------------
template <int K>
constexpr int fwd_scan_b16_floats() {
    return K * 65 + (2 * 64 * (K + 8) * 2) / 4 + (kChunk * (K + 8) * 2) / 4 + (K * 72 * 2) / 4 + 2 * kChunk * kPadC +
           (2 * 64 * 72 * 2) / 4 + 5 * kChunk;
}
static_assert(fwd_scan_b16_floats<128>() * 4 <= 160 * 1024, "bf16 forward rescan must fit one CU");

template <int K>
__global__ __launch_bounds__(512) void bwd_fwd_scan_b16_kernel(BwdParams p) {
    typedef bf16 E;
    constexpr int NTH = 512, VW = 64, VP = VW + 1, KP = K + 8, W = 8, CT = VW / 16;
    constexpr int NT1 = 4 * CT / W;          // 2 tiles of the 64 x 64 products per wave
    constexpr int NT2 = (K / 16) * CT / W;   // tiles of the K x 64 state per wave
    __shared__ __attribute__((aligned(16))) float sm[fwd_scan_b16_floats<K>()];
    float *h = sm;                           // [K][65] fp32 state
    bf16 *hTHi = (bf16 *)(h + K * VP);       // [64][KP] state, transposed, hi part
    bf16 *hTLo = hTHi + 64 * KP;             // [64][KP] lo part
    bf16 *kr = hTLo + 64 * KP;               // [64][KP] raw k rows
    bf16 *kT = kr + kChunk * KP;             // [K][72] raw k rows transposed
    float *Tm = (float *)(kT + K * 72);      // [64][65]
    float *Bm = Tm + kChunk * kPadC;         // [64][65]: v, then B in place
    bf16 *FTHi = (bf16 *)(Bm + kChunk * kPadC);   // [64][72] F transposed, hi
    bf16 *FTLo = FTHi + 64 * 72;                  // lo
    float *gam = (float *)(FTLo + 64 * 72);  // [64]
    float *bet = gam + kChunk;               // [64]
    float *sD = bet + kChunk;                // [64] exp(gamma) / |k|
    float *sF = sD + kChunk;                 // [64] exp(gamma_L - gamma), 0 past L
    float *sFk = sF + kChunk;                // [64] exp(gamma_L - gamma) / |k|, 0 past L

    const int HV = p.HV, V = p.V;
    const int seq_rank = blockIdx.x / HV, j = blockIdx.x - seq_rank * HV, jk = j / (HV / p.H);
    const int n = p.seq_order ? p.seq_order[seq_rank] : seq_rank;   // longest first for packed batches
    const int c0 = blockIdx.y * VW;
    int bos, len, cid0;
    seq_of(p, n, bos, len, cid0);
    const int nc = (len + kChunk - 1) / kChunk;
    const int i16 = threadIdx.x & 15, q = (threadIdx.x >> 4) & 3;

    if (p.initial_state) {
        StateTileN<K, VW, NTH> r0;
        r0.load(p.initial_state + ((int64_t)n * HV + j) * K * V, V, c0);
        r0.commit(h);
    } else {
        for (int e = threadIdx.x; e < K * VW; e += NTH) h[(e / VW) * VP + e % VW] = 0.f;
    }
    lds_barrier();
    for (int e = threadIdx.x; e < K * VW; e += NTH) {   // the transposed hi / lo copy
        const int r = e / VW, c = e % VW;
        const float x = h[r * VP + c];
        const bf16 hi = (bf16)x;
        hTHi[c * KP + r] = hi;
        hTLo[c * KP + r] = (bf16)(x - (float)hi);
    }
    RawRowsReg<E, K, NTH, 8> rk;
    Mat64RegN<NTH> rt;
    TileRegN<E, VW, NTH> rv;
    float rg = 0.f, rb = 0.f;
    auto fetch = [&](int ci) {
        const int cid = cid0 + ci, t0 = bos + ci * kChunk, L = min(kChunk, len - ci * kChunk);
        rk.load((const E *)p.k, t0, L, p.H, jk);
        rt.load(p.tm + ((int64_t)cid * HV + j) * kTriFloats);
        rv.load((const E *)p.v, t0, L, HV, j, V, c0);
        if (threadIdx.x < kChunk) {
            const int r = threadIdx.x;
            rg = r < L ? p.gam[(int64_t)(t0 + r) * HV + j] : 0.f;
            rb = r < L ? p.beta[(int64_t)(t0 + r) * HV + j] : 0.f;
        }
    };
    if (nc > 0) fetch(0);
    const int w = wave_id();
    auto ra = [&](int t) { return 16 * ((w * NT1 + t) / CT); };
    auto cb = [&](int t) { return 16 * ((w * NT1 + t) % CT); };
    auto rs = [&](int t) { return 16 * ((w * NT2 + t) / CT); };
    auto cs = [&](int t) { return 16 * ((w * NT2 + t) % CT); };
    for (int ci = 0; ci < nc; ++ci) {
        const int cid = cid0 + ci, t0 = bos + ci * kChunk, L = min(kChunk, len - ci * kChunk);
        StateTileN<K, VW, NTH>::store(h, p.hs + ((int64_t)cid * HV + j) * K * V, V, c0);
        rk.commit(kr);
#pragma unroll
        for (int u = 0; u < RawRowsReg<E, K, NTH, 8>::VPT; ++u) {
            constexpr int PER_ROW = K / 8;
            const int i = threadIdx.x + NTH * u, r = i / PER_ROW, c = (i % PER_ROW) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) kT[(c + e) * 72 + r] = rk.v[u][e];
        }
        rt.commit(Tm);
        rv.commit(Bm);
        if (threadIdx.x < kChunk) {
            gam[threadIdx.x] = rg;
            bet[threadIdx.x] = rb;
        }
        lds_barrier();
        {
            constexpr int LPR = NTH / kChunk;   // lanes per row
            const int r = threadIdx.x / LPR;
            const float sk = row_sumsq<E, K, NTH, 8>(kr, r);
            if (threadIdx.x % LPR == 0) {
                const float fk = p.use_l2norm ? 1.f / sqrtf(sk + 1e-6f) : 1.f;
                const float f = r < L ? __expf(gam[L - 1] - gam[r]) : 0.f;
                sD[r] = __expf(gam[r]) * fk;
                sF[r] = f;
                sFk[r] = f * fk;
            }
        }
        lds_barrier();
        if (ci + 1 < nc) fetch(ci + 1);

        // B = diag(beta) (V - diag(D) Kh h): K_raw (exact) times the hi and lo parts of h
        {
            f32x4 x[NT1];
            zero(x);
#pragma unroll
            for (int k0 = 0; k0 < K; k0 += 32) {
                const bf16x8 a = *(const bf16x8 *)(kr + (ra(0) + i16) * KP + k0 + 8 * q);
#pragma unroll
                for (int t = 0; t < NT1; ++t) {
                    const int bo = (cb(t) + i16) * KP + k0 + 8 * q;
                    x[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, *(const bf16x8 *)(hTHi + bo), x[t], 0, 0, 0);
                    x[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, *(const bf16x8 *)(hTLo + bo), x[t], 0, 0, 0);
                }
            }
#pragma unroll
            for (int t = 0; t < NT1; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = lrow(ra(t), e), c = lcol(cb(t));
                    Bm[r * VP + c] = bet[r] * (Bm[r * VP + c] - sD[r] * x[t][e]);
                }
        }
        lds_barrier();
        // Vn = Tm B; F = diag(exp(gamma_L - gamma) / |k|) Vn, transposed, as hi / lo parts
        {
            f32x4 x[NT1];
            zero(x);
            wmm<NT1, kChunk>(x, ra, cb, [&](int r, int m) { return Tm[r * kPadC + m]; },
                             [&](int c, int m) { return Bm[m * VP + c]; });
#pragma unroll
            for (int t = 0; t < NT1; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = lrow(ra(t), e), c = lcol(cb(t));
                    if (r < L) p.vn[((int64_t)(t0 + r) * HV + j) * V + c0 + c] = x[t][e];
                    const float f = sFk[r] * x[t][e];
                    const bf16 hi = (bf16)f;
                    FTHi[c * 72 + r] = hi;
                    FTLo[c * 72 + r] = (bf16)(f - (float)hi);
                }
        }
        lds_barrier();
        // h <- D_L h + Kh^T F: K_raw^T (exact) times the hi and lo parts of F
        {
            f32x4 x[NT2];
            zero(x);
#pragma unroll
            for (int m0 = 0; m0 < kChunk; m0 += 32) {
#pragma unroll
                for (int t = 0; t < NT2; ++t) {
                    const bf16x8 a = *(const bf16x8 *)(kT + (rs(t) + i16) * 72 + m0 + 8 * q);
                    const int bo = (cs(t) + i16) * 72 + m0 + 8 * q;
                    x[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, *(const bf16x8 *)(FTHi + bo), x[t], 0, 0, 0);
                    x[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, *(const bf16x8 *)(FTLo + bo), x[t], 0, 0, 0);
                }
            }
            const float dl = __expf(gam[L - 1]);
#pragma unroll
            for (int t = 0; t < NT2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = lrow(rs(t), e), c = lcol(cs(t));
                    float &hv = h[r * VP + c];
                    hv = fmaf(dl, hv, x[t][e]);
                    const bf16 hi = (bf16)hv;
                    hTHi[c * KP + r] = hi;
                    hTLo[c * KP + r] = (bf16)(hv - (float)hi);
                }
        }
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// backward over chunks per (sequence, value head, VW value columns), NTH
// threads: dh' per chunk, dB, and the initial-state gradient.  The key and
// query rows stay raw in LDS; their L2 norms enter as the row scales sFk, sD
// and sB of the three products that use them.
// ---------------------------------------------------------------------------
template <typename E, int K, int VW, int NTH>
constexpr int dh_scan_floats() {
    return K * (VW + 1) + 2 * kChunk * kPadC + 3 * kChunk * (VW + 1) + 5 * kChunk +
           (2 * kChunk * (K + RowPad<E>::v) * (int)sizeof(E) + 3) / 4;
}
static_assert(dh_scan_floats<bf16, 128, 64, 512>() * 4 <= 160 * 1024, "bf16 dh scan must fit one CU");
static_assert(dh_scan_floats<float, 128, 32, 256>() * 4 <= 160 * 1024, "fp32 dh scan must fit one CU");

template <typename E, int K, int VW, int NTH>
__global__ __launch_bounds__(NTH) void bwd_dh_scan_kernel(BwdParams p) {
    constexpr int VP = VW + 1, KS = K + RowPad<E>::v, W = NTH / 64, CT = VW / 16;
    constexpr int NT1 = 4 * CT / W;          // 16 x 16 tiles of a 64 x VW product per wave
    constexpr int NT2 = (K / 16) * CT / W;   // tiles of the K x VW state per wave
    static_assert(NT1 >= 1 && NT2 >= 1, "every wave needs a tile");
    __shared__ float sm[dh_scan_floats<E, K, VW, NTH>()];
    float *dh = sm;                          // [K][VP]
    float *Tm = dh + K * VP;                 // [64][65]
    float *Pm = Tm + kChunk * kPadC;         // [64][65]
    float *dO = Pm + kChunk * kPadC;         // [64][VP]
    float *dVn = dO + kChunk * VP;           // [64][VP]
    float *dB = dVn + kChunk * VP;           // [64][VP]
    float *gam = dB + kChunk * VP;           // [64]
    float *bet = gam + kChunk;               // [64]
    float *sFk = bet + kChunk;               // [64] exp(gamma_L - gamma) / |k|, 0 past L
    float *sD = sFk + kChunk;                // [64] scale exp(gamma) / |q|
    float *sB = sD + kChunk;                 // [64] -beta exp(gamma) / |k|
    E *kr = (E *)(sB + kChunk);              // [64][KS] raw k rows
    E *qr = kr + kChunk * KS;                // [64][KS] raw q rows

    const int HV = p.HV, V = p.V;
    const int seq_rank = blockIdx.x / HV, j = blockIdx.x - seq_rank * HV, jk = j / (HV / p.H);
    const int n = p.seq_order ? p.seq_order[seq_rank] : seq_rank;   // longest first for packed batches
    const int c0 = blockIdx.y * VW;
    int bos, len, cid0;
    seq_of(p, n, bos, len, cid0);
    const int nc = (len + kChunk - 1) / kChunk;
    const float scale = p.scale;

    if (p.dht) {
        StateTileN<K, VW, NTH> r0;
        r0.load(p.dht + ((int64_t)n * HV + j) * K * V, V, c0);
        r0.commit(dh);
    } else {
        for (int e = threadIdx.x; e < K * VW; e += NTH) dh[(e / VW) * VP + e % VW] = 0.f;
    }
    RawRowsReg<E, K, NTH> rk, rq;
    Mat64RegN<NTH> rt, rp;
    TileRegN<E, VW, NTH> ro;
    float rg = 0.f, rb = 0.f;
    auto fetch = [&](int ci) {
        const int cid = cid0 + ci, t0 = bos + ci * kChunk, L = min(kChunk, len - ci * kChunk);
        rk.load((const E *)p.k, t0, L, p.H, jk);
        rq.load((const E *)p.q, t0, L, p.H, jk);
        rt.load(p.tm + ((int64_t)cid * HV + j) * kTriFloats);
        rp.load(p.pm + ((int64_t)cid * HV + j) * kTriFloats);
        ro.load((const E *)p.dout, t0, L, HV, j, V, c0);
        if (threadIdx.x < kChunk) {
            const int r = threadIdx.x;
            rg = r < L ? p.gam[(int64_t)(t0 + r) * HV + j] : 0.f;
            rb = r < L ? p.beta[(int64_t)(t0 + r) * HV + j] : 0.f;
        }
    };
    if (nc > 0) fetch(nc - 1);
    lds_barrier();
    // tile τ = w NT + t of a product with CT column tiles sits at row tile τ / CT, column tile τ % CT
    const int w = wave_id();
    auto ra = [&](int t) { return 16 * ((w * NT1 + t) / CT); };
    auto cb = [&](int t) { return 16 * ((w * NT1 + t) % CT); };
    auto rs = [&](int t) { return 16 * ((w * NT2 + t) / CT); };
    auto cs = [&](int t) { return 16 * ((w * NT2 + t) % CT); };
    for (int ci = nc - 1; ci >= 0; --ci) {
        const int cid = cid0 + ci, t0 = bos + ci * kChunk, L = min(kChunk, len - ci * kChunk);
        StateTileN<K, VW, NTH>::store(dh, p.dhs + ((int64_t)cid * HV + j) * K * V, V, c0);
        rk.commit(kr);
        rq.commit(qr);
        rt.commit(Tm);
        rp.commit(Pm);
        ro.commit(dO);
        if (threadIdx.x < kChunk) {
            gam[threadIdx.x] = rg;
            bet[threadIdx.x] = rb;
        }
        lds_barrier();
        {
            constexpr int LPR = NTH / kChunk;   // lanes per row
            const int r = threadIdx.x / LPR;
            const float sk = row_sumsq<E, K, NTH>(kr, r), sq = row_sumsq<E, K, NTH>(qr, r);
            if (threadIdx.x % LPR == 0) {
                const float fk = p.use_l2norm ? 1.f / sqrtf(sk + 1e-6f) : 1.f;
                const float fq = p.use_l2norm ? 1.f / sqrtf(sq + 1e-6f) : 1.f;
                const float d = __expf(gam[r]);
                sFk[r] = r < L ? __expf(gam[L - 1] - gam[r]) * fk : 0.f;
                sD[r] = scale * d * fq;
                sB[r] = -bet[r] * d * fk;
            }
        }
        lds_barrier();
        if (ci > 0) fetch(ci - 1);
        const float gl = gam[L - 1];

        // dVn = scale Pm^T dO + diag(exp(gamma_L - gamma)) Kh dh'
        {
            f32x4 a[NT1], b[NT1];
            zero(a);
            zero(b);
            wmm<NT1, kChunk>(a, ra, cb, [&](int r, int m) { return Pm[m * kPadC + r]; },
                             [&](int c, int m) { return dO[m * VP + c]; });
            wmm<NT1, K>(b, ra, cb, [&](int r, int m) { return to_f(kr[r * KS + m]); },
                        [&](int c, int m) { return dh[m * VP + c]; });
#pragma unroll
            for (int t = 0; t < NT1; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = lrow(ra(t), e), c = lcol(cb(t));
                    dVn[r * VP + c] = scale * a[t][e] + sFk[r] * b[t][e];
                }
        }
        lds_barrier();
        // dB = Tm^T dVn
        {
            f32x4 a[NT1];
            zero(a);
            wmm<NT1, kChunk>(a, ra, cb, [&](int r, int m) { return Tm[m * kPadC + r]; },
                             [&](int c, int m) { return dVn[m * VP + c]; });
#pragma unroll
            for (int t = 0; t < NT1; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = lrow(ra(t), e), c = lcol(cb(t));
                    dB[r * VP + c] = a[t][e];
                    if (r < L) p.db[((int64_t)(t0 + r) * HV + j) * V + c0 + c] = a[t][e];
                }
        }
        lds_barrier();
        // dh <- D_L dh' + scale Qh^T diag(D) dO - Kh^T diag(beta D) dB
        {
            f32x4 a[NT2];
            zero(a);
            wmm<NT2, kChunk>(a, rs, cs, [&](int r, int m) { return to_f(qr[m * KS + r]); },
                             [&](int c, int m) { return sD[m] * dO[m * VP + c]; });
            wmm<NT2, kChunk>(a, rs, cs, [&](int r, int m) { return to_f(kr[m * KS + r]); },
                             [&](int c, int m) { return sB[m] * dB[m * VP + c]; });
            const float dl = __expf(gl);
#pragma unroll
            for (int t = 0; t < NT2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float &x = dh[lrow(rs(t), e) * VP + lcol(cs(t))];
                    x = fmaf(dl, x, a[t][e]);
                }
        }
        lds_barrier();
    }
    if (p.dh0) StateTileN<K, VW, NTH>::store(dh, p.dh0 + ((int64_t)n * HV + j) * K * V, V, c0);
}

// ---------------------------------------------------------------------------
// The forward rescan with 16 value columns and 8 waves (bf16 rows, K = 128),
// for few (sequence, value head) pairs, in the same form as the 8-wave dh
// scan below: the two 64-row products split their reduction between wave
// pairs (keys, then tokens, in halves; the partial sums added where the next
// stage reads them) and the state update takes one row tile per wave.
// ---------------------------------------------------------------------------
constexpr int fwd_scan_sk_floats() {
    return 128 * 17 + kChunk * kPadC + 5 * kChunk * 17 + 4 * kChunk + (kChunk * (128 + 2) * 2 + 3) / 4;
}

__global__ __launch_bounds__(512) void bwd_fwd_scan_sk_kernel(BwdParams p) {
    typedef bf16 E;
    constexpr int K = 128, VW = 16, VP = VW + 1, KS = K + RowPad<E>::v, NTH = 512;
    __shared__ float sm[fwd_scan_sk_floats()];
    float *h = sm;                           // [K][VP]
    float *Tm = h + K * VP;                  // [64][65]
    float *vv = Tm + kChunk * kPadC;         // [64][VP] v
    float *X0 = vv + kChunk * VP;            // [64][VP] Kh h, keys 0..63
    float *X1 = X0 + kChunk * VP;            // [64][VP]       keys 64..127
    float *Y0 = X1 + kChunk * VP;            // [64][VP] Vn = Tm B, tokens 0..31
    float *Y1 = Y0 + kChunk * VP;            // [64][VP]             tokens 32..63
    float *gam = Y1 + kChunk * VP;           // [64]
    float *bet = gam + kChunk;               // [64]
    float *sD = bet + kChunk;                // [64] exp(gamma) / |k|
    float *sFk = sD + kChunk;                // [64] exp(gamma_L - gamma) / |k|, 0 past L
    E *kr = (E *)(sFk + kChunk);             // [64][KS] raw k rows

    const int HV = p.HV, V = p.V;
    const int seq_rank = blockIdx.x / HV, j = blockIdx.x - seq_rank * HV, jk = j / (HV / p.H);
    const int n = p.seq_order ? p.seq_order[seq_rank] : seq_rank;   // longest first for packed batches
    const int c0 = blockIdx.y * VW;
    int bos, len, cid0;
    seq_of(p, n, bos, len, cid0);
    const int nc = (len + kChunk - 1) / kChunk;
    const bool lo = threadIdx.x < 256;       // the v tile moves through the first four waves

    if (p.initial_state) {
        StateTileN<K, VW, NTH> r0;
        r0.load(p.initial_state + ((int64_t)n * HV + j) * K * V, V, c0);
        r0.commit(h);
    } else {
        for (int e = threadIdx.x; e < K * VW; e += NTH) h[(e / VW) * VP + e % VW] = 0.f;
    }
    RawRowsReg<E, K, NTH> rk;
    Mat64RegN<NTH> rt;
    TileRegN<E, VW, 256> rv;
    float rg = 0.f, rb = 0.f;
    auto fetch = [&](int ci) {
        const int cid = cid0 + ci, t0 = bos + ci * kChunk, L = min(kChunk, len - ci * kChunk);
        rk.load((const E *)p.k, t0, L, p.H, jk);
        rt.load(p.tm + ((int64_t)cid * HV + j) * kTriFloats);
        if (lo) rv.load((const E *)p.v, t0, L, HV, j, V, c0);
        if (threadIdx.x < kChunk) {
            const int r = threadIdx.x;
            rg = r < L ? p.gam[(int64_t)(t0 + r) * HV + j] : 0.f;
            rb = r < L ? p.beta[(int64_t)(t0 + r) * HV + j] : 0.f;
        }
    };
    if (nc > 0) fetch(0);
    lds_barrier();
    const int w = wave_id(), rt4 = 16 * (w & 3), half = w >> 2;
    auto ra = [&](int) { return rt4; };
    auto rs = [&](int) { return 16 * w; };
    auto cb = [&](int) { return 0; };
    for (int ci = 0; ci < nc; ++ci) {
        const int cid = cid0 + ci, t0 = bos + ci * kChunk, L = min(kChunk, len - ci * kChunk);
        StateTileN<K, VW, NTH>::store(h, p.hs + ((int64_t)cid * HV + j) * K * V, V, c0);
        rk.commit(kr);
        rt.commit(Tm);
        if (lo) rv.commit(vv);
        if (threadIdx.x < kChunk) {
            gam[threadIdx.x] = rg;
            bet[threadIdx.x] = rb;
        }
        lds_barrier();
        {
            constexpr int LPR = NTH / kChunk;   // lanes per row
            const int r = threadIdx.x / LPR;
            const float sk = row_sumsq<E, K, NTH>(kr, r);
            if (threadIdx.x % LPR == 0) {
                const float fk = p.use_l2norm ? 1.f / sqrtf(sk + 1e-6f) : 1.f;
                const float f = r < L ? __expf(gam[L - 1] - gam[r]) : 0.f;
                sD[r] = __expf(gam[r]) * fk;
                sFk[r] = f * fk;
            }
        }
        lds_barrier();
        if (ci + 1 < nc) fetch(ci + 1);

        // X = Kh h (raw rows; the norms sit in sD), each half of the keys in one wave
        {
            const int k0 = 64 * half;
            f32x4 x[1];
            zero(x);
            wmm<1, 64>(x, ra, cb, [&](int r, int m) { return to_f(kr[r * KS + k0 + m]); },
                       [&](int c, int m) { return h[(k0 + m) * VP + c]; });
            float *dst = half ? X1 : X0;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[lrow(rt4, e) * VP + lcol(0)] = x[0][e];
        }
        lds_barrier();
        // Vn = Tm B with B = diag(beta) (V - diag(D) X), each half of the tokens in one wave
        {
            const int m0 = 32 * half;
            f32x4 x[1];
            zero(x);
            wmm<1, 32>(x, ra, cb, [&](int r, int m) { return Tm[r * kPadC + m0 + m]; },
                       [&](int c, int m) {
                           const int t = m0 + m;
                           return bet[t] * (vv[t * VP + c] - sD[t] * (X0[t * VP + c] + X1[t * VP + c]));
                       });
            float *dst = half ? Y1 : Y0;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[lrow(rt4, e) * VP + lcol(0)] = x[0][e];
        }
        lds_barrier();
        // h <- D_L h + Kh^T diag(exp(gamma_L - gamma)) Vn: row tile w; Vn to HBM
        {
            f32x4 x[1];
            zero(x);
            wmm<1, kChunk>(x, rs, cb, [&](int r, int m) { return to_f(kr[m * KS + r]); },
                           [&](int c, int m) { return sFk[m] * (Y0[m * VP + c] + Y1[m * VP + c]); });
            const float dl = __expf(gam[L - 1]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float &hv = h[lrow(16 * w, e) * VP + lcol(0)];
                hv = fmaf(dl, hv, x[0][e]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {   // 64 x 16 values, two per thread
                const int i = threadIdx.x + NTH * u, r = i / VW, c = i % VW;
                if (r < L) p.vn[((int64_t)(t0 + r) * HV + j) * V + c0 + c] = Y0[r * VP + c] + Y1[r * VP + c];
            }
        }
        lds_barrier();
    }
}
static_assert(fwd_scan_sk_floats() * 4 <= 160 * 1024, "split forward rescan must fit one CU");

// ---------------------------------------------------------------------------
// The dh scan with 16 value columns and 8 waves (bf16 rows, K = 128): the
// narrowest tiles, for few (sequence, value head) pairs.  Four waves would
// leave one wave per SIMD and nothing to hide the latency of each chunk
// step's chained products; here the two 64-row products split their
// reduction between wave pairs (keys or tokens in halves, the partial sums
// added where they are read) and the 128-row state update takes one row tile
// per wave.
// ---------------------------------------------------------------------------
constexpr int dh_scan_sk_floats() {
    return 128 * 17 + 2 * kChunk * kPadC + 5 * kChunk * 17 + 5 * kChunk + (2 * kChunk * (128 + 2) * 2 + 3) / 4;
}

__global__ __launch_bounds__(512) void bwd_dh_scan_sk_kernel(BwdParams p) {
    typedef bf16 E;
    constexpr int K = 128, VW = 16, VP = VW + 1, KS = K + RowPad<E>::v, NTH = 512;
    __shared__ float sm[dh_scan_sk_floats()];
    float *dh = sm;                          // [K][VP]
    float *Tm = dh + K * VP;                 // [64][65]
    float *Pm = Tm + kChunk * kPadC;         // [64][65]
    float *dO = Pm + kChunk * kPadC;         // [64][VP]
    float *dV0 = dO + kChunk * VP;           // [64][VP] dVn, keys 0..63 / tokens 0..31
    float *dV1 = dV0 + kChunk * VP;          // [64][VP]             keys 64..127 / tokens 32..63
    float *dB0 = dV1 + kChunk * VP;          // [64][VP] dB, tokens 0..31
    float *dB1 = dB0 + kChunk * VP;          // [64][VP]     tokens 32..63
    float *gam = dB1 + kChunk * VP;          // [64]
    float *bet = gam + kChunk;               // [64]
    float *sFk = bet + kChunk;               // [64] exp(gamma_L - gamma) / |k|, 0 past L
    float *sD = sFk + kChunk;                // [64] scale exp(gamma) / |q|
    float *sB = sD + kChunk;                 // [64] -beta exp(gamma) / |k|
    E *kr = (E *)(sB + kChunk);              // [64][KS] raw k rows
    E *qr = kr + kChunk * KS;                // [64][KS] raw q rows

    const int HV = p.HV, V = p.V;
    const int seq_rank = blockIdx.x / HV, j = blockIdx.x - seq_rank * HV, jk = j / (HV / p.H);
    const int n = p.seq_order ? p.seq_order[seq_rank] : seq_rank;   // longest first for packed batches
    const int c0 = blockIdx.y * VW;
    int bos, len, cid0;
    seq_of(p, n, bos, len, cid0);
    const int nc = (len + kChunk - 1) / kChunk;
    const float scale = p.scale;
    const bool lo = threadIdx.x < 256;       // the dO tile moves through the first four waves

    if (p.dht) {
        StateTileN<K, VW, NTH> r0;
        r0.load(p.dht + ((int64_t)n * HV + j) * K * V, V, c0);
        r0.commit(dh);
    } else {
        for (int e = threadIdx.x; e < K * VW; e += NTH) dh[(e / VW) * VP + e % VW] = 0.f;
    }
    RawRowsReg<E, K, NTH> rk, rq;
    Mat64RegN<NTH> rt, rp;
    TileRegN<E, VW, 256> ro;
    float rg = 0.f, rb = 0.f;
    auto fetch = [&](int ci) {
        const int cid = cid0 + ci, t0 = bos + ci * kChunk, L = min(kChunk, len - ci * kChunk);
        rk.load((const E *)p.k, t0, L, p.H, jk);
        rq.load((const E *)p.q, t0, L, p.H, jk);
        rt.load(p.tm + ((int64_t)cid * HV + j) * kTriFloats);
        rp.load(p.pm + ((int64_t)cid * HV + j) * kTriFloats);
        if (lo) ro.load((const E *)p.dout, t0, L, HV, j, V, c0);
        if (threadIdx.x < kChunk) {
            const int r = threadIdx.x;
            rg = r < L ? p.gam[(int64_t)(t0 + r) * HV + j] : 0.f;
            rb = r < L ? p.beta[(int64_t)(t0 + r) * HV + j] : 0.f;
        }
    };
    if (nc > 0) fetch(nc - 1);
    lds_barrier();
    const int w = wave_id(), rt4 = 16 * (w & 3), half = w >> 2;
    auto ra = [&](int) { return rt4; };
    auto rs = [&](int) { return 16 * w; };
    auto cb = [&](int) { return 0; };
    for (int ci = nc - 1; ci >= 0; --ci) {
        const int cid = cid0 + ci, t0 = bos + ci * kChunk, L = min(kChunk, len - ci * kChunk);
        StateTileN<K, VW, NTH>::store(dh, p.dhs + ((int64_t)cid * HV + j) * K * V, V, c0);
        rk.commit(kr);
        rq.commit(qr);
        rt.commit(Tm);
        rp.commit(Pm);
        if (lo) ro.commit(dO);
        if (threadIdx.x < kChunk) {
            gam[threadIdx.x] = rg;
            bet[threadIdx.x] = rb;
        }
        lds_barrier();
        {
            constexpr int LPR = NTH / kChunk;   // lanes per row
            const int r = threadIdx.x / LPR;
            const float sk = row_sumsq<E, K, NTH>(kr, r), sq = row_sumsq<E, K, NTH>(qr, r);
            if (threadIdx.x % LPR == 0) {
                const float fk = p.use_l2norm ? 1.f / sqrtf(sk + 1e-6f) : 1.f;
                const float fq = p.use_l2norm ? 1.f / sqrtf(sq + 1e-6f) : 1.f;
                const float d = __expf(gam[r]);
                sFk[r] = r < L ? __expf(gam[L - 1] - gam[r]) * fk : 0.f;
                sD[r] = scale * d * fq;
                sB[r] = -bet[r] * d * fk;
            }
        }
        lds_barrier();
        if (ci > 0) fetch(ci - 1);
        const float gl = gam[L - 1];

        // dVn = scale Pm^T dO + diag(exp(gamma_L - gamma)) Kh dh', each half of
        // the tokens (first product) and of the keys (second) in one wave
        {
            const int m0 = 32 * half, k0 = 64 * half;
            f32x4 a[1], b[1];
            zero(a);
            zero(b);
            wmm<1, 32>(a, ra, cb, [&](int r, int m) { return Pm[(m0 + m) * kPadC + r]; },
                       [&](int c, int m) { return dO[(m0 + m) * VP + c]; });
            wmm<1, 64>(b, ra, cb, [&](int r, int m) { return to_f(kr[r * KS + k0 + m]); },
                       [&](int c, int m) { return dh[(k0 + m) * VP + c]; });
            float *dst = half ? dV1 : dV0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = lrow(rt4, e), c = lcol(0);
                dst[r * VP + c] = scale * a[0][e] + sFk[r] * b[0][e];
            }
        }
        lds_barrier();
        // dB = Tm^T dVn, each half of the tokens in one wave
        {
            const int m0 = 32 * half;
            f32x4 a[1];
            zero(a);
            wmm<1, 32>(a, ra, cb, [&](int r, int m) { return Tm[(m0 + m) * kPadC + r]; },
                       [&](int c, int m) { return dV0[(m0 + m) * VP + c] + dV1[(m0 + m) * VP + c]; });
            float *dst = half ? dB1 : dB0;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[lrow(rt4, e) * VP + lcol(0)] = a[0][e];
        }
        lds_barrier();
        // dh <- D_L dh' + scale Qh^T diag(D) dO - Kh^T diag(beta D) dB: row tile w
        {
            f32x4 x[1];
            zero(x);
            wmm<1, kChunk>(x, rs, cb, [&](int r, int m) { return to_f(qr[m * KS + r]); },
                           [&](int c, int m) { return sD[m] * dO[m * VP + c]; });
            wmm<1, kChunk>(x, rs, cb, [&](int r, int m) { return to_f(kr[m * KS + r]); },
                           [&](int c, int m) { return sB[m] * (dB0[m * VP + c] + dB1[m * VP + c]); });
            const float dl = __expf(gl);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float &v = dh[lrow(16 * w, e) * VP + lcol(0)];
                v = fmaf(dl, v, x[0][e]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {   // dB to HBM: 64 x 16 values, two per thread
                const int i = threadIdx.x + NTH * u, r = i / VW, c = i % VW;
                if (r < L) p.db[((int64_t)(t0 + r) * HV + j) * V + c0 + c] = dB0[r * VP + c] + dB1[r * VP + c];
            }
        }
        lds_barrier();
    }
    if (p.dh0) StateTileN<K, VW, NTH>::store(dh, p.dh0 + ((int64_t)n * HV + j) * K * V, V, c0);
}
static_assert(dh_scan_sk_floats() * 4 <= 160 * 1024, "split dh scan must fit one CU");

// ---------------------------------------------------------------------------
// per (chunk, value head): dq, dk (per value head), dv, dg, dbeta.  512
// threads: wave w holds rows 16 (w & 3).. and column half w >> 2 of every
// 64 x 64 and 64 x K product; the row sums of the two halves meet in LDS.
// The key and query rows stay raw in LDS and their L2 norms enter as scales.
// ---------------------------------------------------------------------------
constexpr int kGThreads = 512;

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): a product of two split
// values, hi hi + hi lo + lo hi, misses only lo lo (2^-16 of it) and the
// rounding of the lo parts, so it keeps fp32 accuracy on the bf16 matrix cores.
__device__ __forceinline__ void split_store4(const float *x, bf16 *hi, bf16 *lo) {
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = (bf16)x[e];
        l[e] = (bf16)(x[e] - (float)h[e]);
    }
    *(bf16x4 *)hi = h;
    *(bf16x4 *)lo = l;
}
// acc[t] += sum over 32 value columns of X[ra + (l & 15)][.] Y[cb(t) + (l & 15)][.]
// for bf16 rows X, Y at stride kVS (one v_mfma_f32_16x16x32_bf16 per tile).
template <int NT, typename CB>
__device__ __forceinline__ void vmm(f32x4 (&acc)[NT], const bf16 *X, int ra, const bf16 *Y, CB cb) {
    const int i = threadIdx.x & 15, q = (threadIdx.x >> 4) & 3;
    const bf16x8 a = *(const bf16x8 *)(X + (ra + i) * kVS + 8 * q);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const bf16x8 b = *(const bf16x8 *)(Y + (cb(t) + i) * kVS + 8 * q);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[t], 0, 0, 0);
    }
}
// Rows t0..t0+L-1 (zero past L), 32 columns from c0, of a [T_tot, HV, V]
// tensor at value head j, four elements per thread: row threadIdx.x / 8,
// columns 4 (threadIdx.x % 8) .. +3 (staged into LDS by the caller).
template <typename E>
struct Tile4Reg {
    typename VT<E>::v4 v;
    __device__ __forceinline__ void load(const E *src, int t0, int L, int HV, int j, int V, int c0) {
        const int r = threadIdx.x >> 3, c = (threadIdx.x & 7) * 4;
        if (r < L) v = *(const typename VT<E>::v4 *)(src + ((int64_t)(t0 + r) * HV + j) * V + c0 + c);
        else
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = to_e<E>(0.f);
    }
};
// bf16 rows: the second phase's four 64 x 64 operands as bf16 hi / lo pairs
// at a row stride of kMS elements, and the raw q / k rows transposed (exact
// bf16 operands of the same products).
constexpr int kMS = 72;
template <typename E, int K>
constexpr int grads_region_floats() {
    return sizeof(E) == 2 && 8 * kChunk * kMS / 2 > grads_tile_floats<K>() ? 8 * kChunk * kMS / 2
                                                                            : grads_tile_floats<K>();
}
template <typename E, int K>
constexpr int grads_floats() {
    return grads_region_floats<E, K>() + 23 * kChunk + 8 + (2 * kChunk * (K + RowPad<E>::v) * (int)sizeof(E) + 3) / 4 +
           (sizeof(E) == 2 ? 2 * K * kMS / 2 : 0);
}
static_assert(grads_floats<float, 128>() * 4 <= 160 * 1024, "fp32 grads must fit one CU");
static_assert(grads_floats<bf16, 128>() * 4 <= 160 * 1024, "bf16 grads must fit one CU");

template <typename E, int K, int V>
__global__ __launch_bounds__(kGThreads) void bwd_grads_kernel(BwdParams p) {
    constexpr int KS = K + RowPad<E>::v, KR = K / 16, NTK = KR / 2;
    __shared__ __attribute__((aligned(16))) float sm[grads_floats<E, K>()];   // 16-byte operand reads
    float *tile = sm;                        // per value tile, then the 64 x 64 matrices
    bf16 *hHi = (bf16 *)tile, *hLo = hHi + K * kVS;        // [K][kVS] h rows (key index), value columns
    bf16 *dhHi = hLo + K * kVS, *dhLo = dhHi + K * kVS;   // [K][kVS] dh'
    bf16 *vnHi = dhLo + K * kVS, *vnLo = vnHi + kChunk * kVS;   // [64][kVS] Vn
    bf16 *dbHi = vnLo + kChunk * kVS, *dbLo = dbHi + kChunk * kVS;   // [64][kVS] dB
    bf16 *doHi = dbLo + kChunk * kVS, *doLo = doHi + kChunk * kVS;   // [64][kVS] dO (lo only for fp32 I/O)
    float *dS = tile;                        // [64][65] dSqk (after the value tiles)
    float *Ad = dS + kChunk * kPadC;         // [64][65]
    float *rows = tile + grads_region_floats<E, K>();   // scalars per row
    float *gam = rows;                       // [64]
    float *bet = gam + kChunk;               // [64]
    float *fk = bet + kChunk;                // [64] 1 / |k|
    float *fq = fk + kChunk;                 // [64] 1 / |q|
    float *sbvA = fq + kChunk;               // [64] sum_v dB v
    float *pt = sbvA + kChunk;               // [5][2][64] per column half: q.dQ, k.E, k.F, dA.A, k.dK
    float *psq = pt + 10 * kChunk;           // [2][64] q.dQ after the second phase
    float *prs = psq + 2 * kChunk;           // [2][64] row sums of Z per column half
    float *pcs = prs + 2 * kChunk;           // [4][64] column sums of Z per row block
    float *red = pcs + 4 * kChunk;           // [8] <dh', h> per wave
    E *kr = (E *)(red + 8);                  // [64][KS] raw k rows
    static_assert(5 + 10 + 2 + 2 + 4 == 23, "row arrays of grads_floats");
    E *qr = kr + kChunk * KS;                // [64][KS] raw q rows
    constexpr bool kB16 = sizeof(E) == 2;
    // bf16 rows: the raw rows transposed, [K][kMS] (key index, token), and the
    // second phase's operands over the tile region, [64][kMS] hi / lo each
    bf16 *kT = (bf16 *)(qr + kChunk * KS), *qT = kT + K * kMS;
    bf16 *dSkHi = (bf16 *)tile, *dSkLo = dSkHi + kChunk * kMS;       // dSqk[r][m] / |k_m|
    bf16 *dSqHi = dSkLo + kChunk * kMS, *dSqLo = dSqHi + kChunk * kMS;   // dSqk[m][r] / |q_m| at [r][m]
    bf16 *AdkHi = dSqLo + kChunk * kMS, *AdkLo = AdkHi + kChunk * kMS;   // Ad[r][m] / |k_m|
    bf16 *AtkHi = AdkLo + kChunk * kMS, *AtkLo = AtkHi + kChunk * kMS;   // Ad[m][r] / |k_m| at [r][m]

    ChunkRef cr;
    if (!find_chunk(p, blockIdx.x, cr)) return;
    const int j = blockIdx.y, HV = p.HV, jk = j / (HV / p.H);
    const int cid = blockIdx.x, L = cr.L, t0 = cr.t0;
    const float scale = p.scale;
    const int w = wave_id(), rb = w & 3, hf = w >> 2, lane16 = threadIdx.x & 15;
    auto ra = [&](int) { return 16 * rb; };
    auto cbP = [&](int t) { return 16 * (2 * hf + t); };
    auto cbK = [&](int t) { return 16 * (hf * NTK + t); };

    if (threadIdx.x < kChunk) {
        const int r = threadIdx.x;
        gam[r] = r < L ? p.gam[(int64_t)(t0 + r) * HV + j] : 0.f;
        bet[r] = r < L ? p.beta[(int64_t)(t0 + r) * HV + j] : 0.f;
    }
    const float *hs = p.hs + ((int64_t)cid * HV + j) * K * V;
    const float *dhs = p.dhs + ((int64_t)cid * HV + j) * K * V;
    StateTileN<K, kVT, kGThreads> th, tdh;
    Tile4Reg<float> tvn, tdb;
    Tile4Reg<E> tdo, tv;
    auto fetch = [&](int c0) {
        th.load(hs, V, c0);
        tdh.load(dhs, V, c0);
        tvn.load(p.vn, t0, L, HV, j, V, c0);
        tdb.load(p.db, t0, L, HV, j, V, c0);
        tdo.load((const E *)p.dout, t0, L, HV, j, V, c0);
        tv.load((const E *)p.v, t0, L, HV, j, V, c0);
    };
    {
        RawRowsReg<E, K, kGThreads> rk, rq;
        rk.load((const E *)p.k, t0, L, p.H, jk);
        rq.load((const E *)p.q, t0, L, p.H, jk);
        fetch(0);
        rk.commit(kr);
        rq.commit(qr);
        if constexpr (kB16) {
#pragma unroll
            for (int u = 0; u < RawRowsReg<E, K, kGThreads>::VPT; ++u) {
                constexpr int PER_ROW = K / 8;
                const int i = threadIdx.x + kGThreads * u, r = i / PER_ROW, c = (i % PER_ROW) * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    kT[(c + e) * kMS + r] = rk.v[u][e];
                    qT[(c + e) * kMS + r] = rq.v[u][e];
                }
            }
        }
    }
    lds_barrier();
    {
        constexpr int LPR = kGThreads / kChunk;
        const int r = threadIdx.x / LPR;
        const float sk = row_sumsq<E, K, kGThreads>(kr, r), sq = row_sumsq<E, K, kGThreads>(qr, r);
        if (threadIdx.x % LPR == 0) {
            fk[r] = p.use_l2norm ? 1.f / sqrtf(sk + 1e-6f) : 1.f;
            fq[r] = p.use_l2norm ? 1.f / sqrtf(sq + 1e-6f) : 1.f;
        }
    }

    f32x4 aP[2], aA[2], dQ[NTK], aE[NTK], aF[NTK];
    zero(aP);
    zero(aA);
    zero(dQ);
    zero(aE);
    zero(aF);
    float sdh = 0.f;      // this thread's part of <dh', h>
    float sbv = 0.f;      // row (threadIdx.x >> 3): sum_v dB v
    constexpr bool kExactDo = sizeof(E) == 2;   // bf16 dO is its own hi part
    for (int c0 = 0; c0 < V; c0 += kVT) {
        // stage the tiles as hi / lo pairs; <dh', h>, sum_v dB v and dv from the registers
#pragma unroll
        for (int u = 0; u < StateTileN<K, kVT, kGThreads>::N4; ++u) {
            const int i = threadIdx.x + kGThreads * u, r = i >> 3, c = (i & 7) * 4;
            float xh[4], xd[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xh[e] = th.v[u][e];
                xd[e] = tdh.v[u][e];
                sdh = fmaf(xh[e], xd[e], sdh);
            }
            split_store4(xh, hHi + r * kVS + c, hLo + r * kVS + c);
            split_store4(xd, dhHi + r * kVS + c, dhLo + r * kVS + c);
        }
        {
            const int r = threadIdx.x >> 3, c = (threadIdx.x & 7) * 4;
            float xv[4], xb[4], xo[4];
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xv[e] = tvn.v[e];
                xb[e] = tdb.v[e];
                xo[e] = to_f(tdo.v[e]);
                s = fmaf(xb[e], to_f(tv.v[e]), s);
            }
            split_store4(xv, vnHi + r * kVS + c, vnLo + r * kVS + c);
            split_store4(xb, dbHi + r * kVS + c, dbLo + r * kVS + c);
            if constexpr (kExactDo) {
                *(bf16x4 *)(doHi + r * kVS + c) = bf16x4{(bf16)xo[0], (bf16)xo[1], (bf16)xo[2], (bf16)xo[3]};
            } else {
                split_store4(xo, doHi + r * kVS + c, doLo + r * kVS + c);
            }
            s += __shfl_xor(s, 1);
            s += __shfl_xor(s, 2);
            s += __shfl_xor(s, 4);
            sbv += s;
            if (r < L) {
                typename VT<E>::v4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = to_e<E>(bet[r] * xb[e]);
                *(typename VT<E>::v4 *)((E *)p.dv + ((int64_t)(t0 + r) * HV + j) * V + c0 + c) = o;
            }
        }
        lds_barrier();
        if (c0 + kVT < V) fetch(c0 + kVT);
        const int r0 = 16 * rb;
        // aP += dO Vn^T, aA += dB Vn^T, dQ += dO h^T, aE += dB h^T, aF += Vn dh'^T
        vmm(aP, doHi, r0, vnHi, cbP);
        vmm(aP, doHi, r0, vnLo, cbP);
        vmm(aA, dbHi, r0, vnHi, cbP);
        vmm(aA, dbHi, r0, vnLo, cbP);
        vmm(aA, dbLo, r0, vnHi, cbP);
        vmm(dQ, doHi, r0, hHi, cbK);
        vmm(dQ, doHi, r0, hLo, cbK);
        vmm(aE, dbHi, r0, hHi, cbK);
        vmm(aE, dbHi, r0, hLo, cbK);
        vmm(aE, dbLo, r0, hHi, cbK);
        vmm(aF, vnHi, r0, dhHi, cbK);
        vmm(aF, vnHi, r0, dhLo, cbK);
        vmm(aF, vnLo, r0, dhHi, cbK);
        if constexpr (!kExactDo) {
            vmm(aP, doLo, r0, vnHi, cbP);
            vmm(dQ, doLo, r0, hHi, cbK);
        }
        lds_barrier();
    }

    // <dh', h> per wave; sum_v dB v per row
    {
        float s = sdh;
        for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
        if ((threadIdx.x & 63) == 0) red[w] = s;
        if ((threadIdx.x & 7) == 0) sbvA[threadIdx.x >> 3] = sbv;
    }
    const float gl = gam[L - 1];
    // row scalings and this half's row dot products with the raw q / k rows
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = lrow(16 * rb, e);
        const float d = __expf(gam[r]);
        const float f = r < L ? __expf(gl - gam[r]) : 0.f;
        float t1 = 0.f, t2 = 0.f, t3 = 0.f;
#pragma unroll
        for (int t = 0; t < NTK; ++t) {
            const int col = lcol(cbK(t));
            dQ[t][e] *= scale * d;
            aE[t][e] *= d;
            aF[t][e] *= f;
            t1 = fmaf(to_f(qr[r * KS + col]), dQ[t][e], t1);
            t2 = fmaf(to_f(kr[r * KS + col]), aE[t][e], t2);
            t3 = fmaf(to_f(kr[r * KS + col]), aF[t][e], t3);
        }
        t1 = sum16(t1);
        t2 = sum16(t2);
        t3 = sum16(t3);
        if (lane16 == 0) {
            pt[(0 * 2 + hf) * kChunk + r] = t1;
            pt[(1 * 2 + hf) * kChunk + r] = t2;
            pt[(2 * 2 + hf) * kChunk + r] = t3;
        }
    }
    // dK so far: F dh'^T - diag(beta) E
    f32x4 dK[NTK];
#pragma unroll
    for (int t = 0; t < NTK; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) dK[t][e] = aF[t][e] - bet[lrow(16 * rb, e)] * aE[t][e];

    // the 64 x 64 matrices dSqk and Ad; Z = dSqk * (qh . kh) + dA * A only
    // through its row and column sums, reduced here in registers
    const float *pm = p.pm + ((int64_t)cid * HV + j) * kTriFloats;
    const float *ag = p.ag + ((int64_t)cid * HV + j) * kTriFloats;
    float dbA[4] = {0.f, 0.f, 0.f, 0.f}, zr[4] = {0.f, 0.f, 0.f, 0.f}, zc[2] = {0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = lrow(16 * rb, e), c = lcol(cbP(t));
            const bool low = c <= r && r < L;
            const float d = low ? __expf(gam[r] - gam[c]) : 0.f;
            const float dpm = scale * aP[t][e];
            const float dsq = d * dpm;                   // dSqk
            // zero above the diagonal blocks; the reads stay unconditional (a
            // block above the diagonal reads element 0 and discards it)
            const bool tin = tri_in(r, c);
            const int to = tin ? tri_off(r, c) : 0;
            const float pmv = pm[to], agr = ag[to];
            const float z1 = tin ? dpm * pmv : 0.f;      // dPm * Pm
            const float dA = c < r && r < L ? -aA[t][e] : 0.f;
            const float agv = tin ? agr : 0.f;
            const float adv = dA * bet[r] * d;
            if constexpr (kB16) {
                const float x4[4] = {dsq * fk[c], dsq * fq[r], adv * fk[c], adv * fk[r]};
                bf16 h4[4], l4[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    h4[u] = (bf16)x4[u];
                    l4[u] = (bf16)(x4[u] - (float)h4[u]);
                }
                dSkHi[r * kMS + c] = h4[0];
                dSkLo[r * kMS + c] = l4[0];
                dSqHi[c * kMS + r] = h4[1];
                dSqLo[c * kMS + r] = l4[1];
                AdkHi[r * kMS + c] = h4[2];
                AdkLo[r * kMS + c] = l4[2];
                AtkHi[c * kMS + r] = h4[3];
                AtkLo[c * kMS + r] = l4[3];
            } else {
                dS[r * kPadC + c] = dsq;
                Ad[r * kPadC + c] = adv;
            }
            const float z = z1 + dA * bet[r] * agv;
            zr[e] += z;
            zc[t] += z;
            dbA[e] = fmaf(dA, agv, dbA[e]);
        }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float s = sum16(dbA[e]);
        const float z = sum16(zr[e]);
        if (lane16 == 0) {
            pt[(3 * 2 + hf) * kChunk + lrow(16 * rb, e)] = s;
            prs[hf * kChunk + lrow(16 * rb, e)] = z;
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {   // the 16 rows of this block: the four lane groups
        float z = zc[t];
        z += __shfl_xor(z, 16);
        z += __shfl_xor(z, 32);
        if ((threadIdx.x & 48) == 0) pcs[rb * kChunk + lcol(cbP(t))] = z;
    }
    lds_barrier();
    // wave 0: dgamma, dbeta per row (lane = row), then dg by a reverse cumsum over the lanes
    if (threadIdx.x < kChunk) {
        const int r = threadIdx.x;
        const float t1 = fq[r] * (pt[0 * kChunk + r] + pt[1 * kChunk + r]);
        const float t2 = fk[r] * (pt[2 * kChunk + r] + pt[3 * kChunk + r]);
        const float t3 = fk[r] * (pt[4 * kChunk + r] + pt[5 * kChunk + r]);
        const float rs = prs[r] + prs[kChunk + r];
        const float cs = (pcs[r] + pcs[kChunk + r]) + (pcs[2 * kChunk + r] + pcs[3 * kChunk + r]);
        float t3all = t3;
        for (int o = 32; o >= 1; o >>= 1) t3all += __shfl_xor(t3all, o);
        float sdh_all = 0.f;
#pragma unroll
        for (int u = 0; u < kGThreads / 64; ++u) sdh_all += red[u];
        float dgr = t1 - bet[r] * t2 - t3 + rs - cs;
        if (r == L - 1) dgr += __expf(gl) * sdh_all + t3all;
        const float dbr = -t2 + pt[6 * kChunk + r] + pt[7 * kChunk + r] + sbvA[r];
        float x = r < L ? dgr : 0.f;
#pragma unroll
        for (int o = 1; o < kChunk; o <<= 1) {
            const float y = __shfl_down(x, o);
            if (r + o < kChunk) x += y;
        }
        if (r < L) {
            p.dg[(int64_t)(t0 + r) * HV + j] = x;
            p.dbeta[(int64_t)(t0 + r) * HV + j] = dbr;
        }
    }

    // dQ += dSqk Kh;  dK += dSqk^T Qh + (Ad + Ad^T) Kh   (Kh = diag(fk) K, Qh = diag(fq) Q)
    if constexpr (kB16) {
        // the norms sit in the split operands; the transposed raw rows are exact
        const int i = threadIdx.x & 15, q = (threadIdx.x >> 4) & 3;
#pragma unroll
        for (int m0 = 0; m0 < kChunk; m0 += 32) {
            const int ao = (16 * rb + i) * kMS + m0 + 8 * q;
            const bf16x8 s1 = *(const bf16x8 *)(dSkHi + ao), s2 = *(const bf16x8 *)(dSkLo + ao);
            const bf16x8 s3 = *(const bf16x8 *)(dSqHi + ao), s4 = *(const bf16x8 *)(dSqLo + ao);
            const bf16x8 s5 = *(const bf16x8 *)(AdkHi + ao), s6 = *(const bf16x8 *)(AdkLo + ao);
            const bf16x8 s7 = *(const bf16x8 *)(AtkHi + ao), s8 = *(const bf16x8 *)(AtkLo + ao);
#pragma unroll
            for (int t = 0; t < NTK; ++t) {
                const int bo = (cbK(t) + i) * kMS + m0 + 8 * q;
                const bf16x8 bk = *(const bf16x8 *)(kT + bo), bq = *(const bf16x8 *)(qT + bo);
                dQ[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s1, bk, dQ[t], 0, 0, 0);
                dQ[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s2, bk, dQ[t], 0, 0, 0);
                dK[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s3, bq, dK[t], 0, 0, 0);
                dK[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s4, bq, dK[t], 0, 0, 0);
                dK[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s5, bk, dK[t], 0, 0, 0);
                dK[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s6, bk, dK[t], 0, 0, 0);
                dK[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s7, bk, dK[t], 0, 0, 0);
                dK[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(s8, bk, dK[t], 0, 0, 0);
            }
        }
    } else {
        wmm<NTK, kChunk>(dQ, ra, cbK, [&](int r, int m) { return dS[r * kPadC + m]; },
                         [&](int c, int m) { return fk[m] * to_f(kr[m * KS + c]); });
        wmm<NTK, kChunk>(dK, ra, cbK, [&](int r, int m) { return dS[m * kPadC + r]; },
                         [&](int c, int m) { return fq[m] * to_f(qr[m * KS + c]); });
        wmm<NTK, kChunk>(dK, ra, cbK, [&](int r, int m) { return Ad[r * kPadC + m] + Ad[m * kPadC + r]; },
                         [&](int c, int m) { return fk[m] * to_f(kr[m * KS + c]); });
    }

    // L2-norm backward and the per-value-head partial dq, dk: the row dot
    // products qh . dQ and kh . dK meet across the two column halves
    if (p.use_l2norm) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = lrow(16 * rb, e);
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int t = 0; t < NTK; ++t) {
                sq = fmaf(to_f(qr[r * KS + lcol(cbK(t))]), dQ[t][e], sq);
                sk = fmaf(to_f(kr[r * KS + lcol(cbK(t))]), dK[t][e], sk);
            }
            sq = sum16(sq);
            sk = sum16(sk);
            if (lane16 == 0) {
                psq[hf * kChunk + r] = sq;
                pt[(8 + hf) * kChunk + r] = sk;
            }
        }
    }
    lds_barrier();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = lrow(16 * rb, e);
        const float sq = p.use_l2norm ? fq[r] * (psq[r] + psq[kChunk + r]) : 0.f;
        const float sk = p.use_l2norm ? fk[r] * (pt[8 * kChunk + r] + pt[9 * kChunk + r]) : 0.f;
        if (r < L) {
            float *dq = p.dqp + ((int64_t)(t0 + r) * HV + j) * K;
            float *dk = p.dkp + ((int64_t)(t0 + r) * HV + j) * K;
#pragma unroll
            for (int t = 0; t < NTK; ++t) {
                const int col = lcol(cbK(t));
                dq[col] = fq[r] * (dQ[t][e] - fq[r] * to_f(qr[r * KS + col]) * sq);
                dk[col] = fk[r] * (dK[t][e] - fk[r] * to_f(kr[r * KS + col]) * sk);
            }
        }
    }
}

// dq, dk [T_tot, H, K] = sum over the G value heads of each key head; four
// consecutive elements per thread (K is a multiple of 4)
template <typename E>
__global__ __launch_bounds__(kThreads) void bwd_reduce_kernel(const float *dqp, const float *dkp, E *dq, E *dk,
                                                             int64_t total4, int H, int G, int K) {
    const int64_t e4 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e4 >= total4) return;
    const int64_t e = 4 * e4;
    const int64_t row = e / K;   // t * H + jk
    const int c = (int)(e - row * K);
    const int64_t t = row / H;
    const int jk = (int)(row - t * H);
    f32x4 sq = {0.f, 0.f, 0.f, 0.f}, sk = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < G; ++g) {
        const int64_t at = (t * (int64_t)H * G + (int64_t)jk * G + g) * K + c;
        sq += *(const f32x4 *)(dqp + at);
        sk += *(const f32x4 *)(dkp + at);
    }
    typename VT<E>::v4 oq, ok;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        oq[u] = to_e<E>(sq[u]);
        ok[u] = to_e<E>(sk[u]);
    }
    *(typename VT<E>::v4 *)(dq + e) = oq;
    *(typename VT<E>::v4 *)(dk + e) = ok;
}

template <typename E, int K, int V>
hipError_t launch_kv(const BwdParams &p, int nc_max, hipStream_t st, Profiler *prof) {
    const dim3 blk(kThreads);
    if (p.cu_seqlens && p.N > 0) {
        if (prof) prof->begin(kBwdSetupKernel, st);
        hipLaunchKernelGGL(bwd_setup_kernel, dim3(1), blk, 0, st, p.cu_seqlens, p.N, p.chunk_offsets, p.seq_order);
        if (prof) prof->end(kBwdSetupKernel, st);
    }
    if (nc_max > 0) {
        if (prof) prof->begin(kBwdPrepKernel, st);
        hipLaunchKernelGGL((bwd_prep_kernel<E, K>), dim3(nc_max, p.HV), blk, 0, st, p);
        if (prof) prof->end(kBwdPrepKernel, st);
    }
    if (p.N > 0) {
        // Scan tiles (bf16 rows): 64 value columns and 8 waves when the
        // (sequence, value head, 64-column) workgroups fill the GPU; with fewer,
        // narrower tiles give each wave half the products of a chunk step, so
        // the serial chain runs faster while the workgroups still fit in one
        // round: 32 columns x 8 waves (at most 128 wide workgroups), 16 x 4
        // (at most 64).  fp32 rows need twice the LDS: 32 columns, 4 waves.
        const int64_t wide = (int64_t)p.N * p.HV * (V / 64);
        const int narrow = wide <= 64 ? 2 : wide <= 128 ? 1 : 0;
        if (nc_max > 0) {
            if (prof) prof->begin(kBwdFwdScanKernel, st);
            if constexpr (sizeof(E) == 2) {
                if (narrow == 2 && K == 128)
                    hipLaunchKernelGGL(bwd_fwd_scan_sk_kernel, dim3(p.N * p.HV, V / 16), dim3(512), 0, st, p);
                else if (narrow == 2)
                    hipLaunchKernelGGL((bwd_fwd_scan_kernel<E, K, 16, 256>), dim3(p.N * p.HV, V / 16), dim3(256), 0,
                                       st, p);
                else if (narrow == 1)
                    hipLaunchKernelGGL((bwd_fwd_scan_kernel<E, K, 32, 512>), dim3(p.N * p.HV, V / 32), dim3(512), 0,
                                       st, p);
                else
                    hipLaunchKernelGGL((bwd_fwd_scan_b16_kernel<K>), dim3(p.N * p.HV, V / 64), dim3(512), 0, st, p);
            } else {
                hipLaunchKernelGGL((bwd_fwd_scan_kernel<E, K, 32, 256>), dim3(p.N * p.HV, V / 32), dim3(256), 0, st,
                                   p);
            }
            if (prof) prof->end(kBwdFwdScanKernel, st);
        }
        if (prof) prof->begin(kBwdDhScanKernel, st);
        if constexpr (sizeof(E) == 2) {
            if (narrow == 2 && K == 128)
                hipLaunchKernelGGL(bwd_dh_scan_sk_kernel, dim3(p.N * p.HV, V / 16), dim3(512), 0, st, p);
            else if (narrow == 2)
                hipLaunchKernelGGL((bwd_dh_scan_kernel<E, K, 16, 256>), dim3(p.N * p.HV, V / 16), dim3(256), 0, st, p);
            else if (narrow == 1)
                hipLaunchKernelGGL((bwd_dh_scan_kernel<E, K, 32, 512>), dim3(p.N * p.HV, V / 32), dim3(512), 0, st, p);
            else
                hipLaunchKernelGGL((bwd_dh_scan_kernel<E, K, 64, 512>), dim3(p.N * p.HV, V / 64), dim3(512), 0, st, p);
        } else {
            hipLaunchKernelGGL((bwd_dh_scan_kernel<E, K, 32, 256>), dim3(p.N * p.HV, V / 32), dim3(256), 0, st, p);
        }
        if (prof) prof->end(kBwdDhScanKernel, st);
    }
    if (nc_max > 0) {
        if (prof) prof->begin(kBwdGradsKernel, st);
        hipLaunchKernelGGL((bwd_grads_kernel<E, K, V>), dim3(nc_max, p.HV), dim3(kGThreads), 0, st, p);
        if (prof) prof->end(kBwdGradsKernel, st);
        const int64_t total4 = (int64_t)p.T_tot * p.H * K / 4;
        if (total4 > 0) {
            if (prof) prof->begin(kBwdReduceKernel, st);
            hipLaunchKernelGGL(bwd_reduce_kernel<E>, dim3((unsigned)((total4 + kThreads - 1) / kThreads)), blk, 0, st,
                               p.dqp, p.dkp, (E *)p.dq, (E *)p.dk, total4, p.H, p.HV / p.H, K);
            if (prof) prof->end(kBwdReduceKernel, st);
        }
    }
    return hipGetLastError();
}

template <typename E>
hipError_t launch_dtype(const BwdParams &p, int nc_max, hipStream_t st, Profiler *prof) {
    if (p.K == 64) return p.V == 64 ? launch_kv<E, 64, 64>(p, nc_max, st, prof) : launch_kv<E, 64, 128>(p, nc_max, st, prof);
    return p.V == 64 ? launch_kv<E, 128, 64>(p, nc_max, st, prof) : launch_kv<E, 128, 128>(p, nc_max, st, prof);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

static int bwd_max_chunks(int B, int T, int N, bool varlen) {
    const int64_t t_tot = (int64_t)B * T;
    const int64_t nc = varlen ? (t_tot + kChunk - 1) / kChunk + N : (int64_t)B * ((T + kChunk - 1) / kChunk);
    return nc > INT32_MAX ? -1 : (int)nc;
}

BwdPlan plan_backward(int B, int T, int H, int HV, int K, int V, int N, bool varlen) {
    BwdPlan pl;
    const int64_t t_tot = (int64_t)B * T;
    pl.nc_max = bwd_max_chunks(B, T, N, varlen);
    if (pl.nc_max < 0) return pl;
    const size_t nc = (size_t)pl.nc_max;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    pl.off_co = take(sizeof(int32_t) * (size_t)(N + 1));
    pl.off_gam = take(sizeof(float) * (size_t)t_tot * HV);
    pl.off_tm = take(sizeof(float) * nc * HV * kTriFloats);
    pl.off_ag = take(sizeof(float) * nc * HV * kTriFloats);
    pl.off_pm = take(sizeof(float) * nc * HV * kTriFloats);
    pl.off_hs = take(sizeof(float) * nc * HV * K * V);
    pl.off_dhs = take(sizeof(float) * nc * HV * K * V);
    pl.off_vn = take(sizeof(float) * (size_t)t_tot * HV * V);
    pl.off_db = take(sizeof(float) * (size_t)t_tot * HV * V);
    pl.off_dqp = take(sizeof(float) * (size_t)t_tot * HV * K);
    pl.off_dkp = take(sizeof(float) * (size_t)t_tot * HV * K);
    if (varlen && N >= 2 && N <= kSeqOrderMax) {
        pl.ordered = true;
        pl.off_ord = take(sizeof(int32_t) * (size_t)N);
    }
    pl.bytes = off;
    return pl;
}

hipError_t launch_backward(BwdParams p, int dtype, const BwdPlan &plan, void *ws, hipStream_t stream,
                           Profiler *prof) {
    char *w = (char *)ws;
    p.chunk_offsets = (int32_t *)(w + plan.off_co);
    p.gam = (float *)(w + plan.off_gam);
    p.tm = (float *)(w + plan.off_tm);
    p.ag = (float *)(w + plan.off_ag);
    p.pm = (float *)(w + plan.off_pm);
    p.hs = (float *)(w + plan.off_hs);
    p.dhs = (float *)(w + plan.off_dhs);
    p.vn = (float *)(w + plan.off_vn);
    p.db = (float *)(w + plan.off_db);
    p.dqp = (float *)(w + plan.off_dqp);
    p.dkp = (float *)(w + plan.off_dkp);
    p.seq_order = plan.ordered && p.cu_seqlens ? (int32_t *)(w + plan.off_ord) : nullptr;
    p.T_tot = p.B * p.T;
    const int nc = p.T_tot > 0 ? plan.nc_max : 0;
    return dtype == 0 ? launch_dtype<bf16>(p, nc, stream, prof) : launch_dtype<float>(p, nc, stream, prof);
}

}  // namespace gdn
