// HIP kernels of the chunked gated delta rule forward pass for gfx950 (MI355X).
//
// The chunked algorithm follows the step list of the page "NPU Training
// Operators - GDN" (operator-semantics section): chunk-local gate cumsum, the
// gated beta*K*K^T product inside a chunk, the unit-lower-triangular solve,
// the W/U recompute, the inter-chunk state recurrence and the output readout;
// chunk length 64 as in that page's tiling section.  The per-chunk equations,
// derived from the recurrence in include/gdn.h, are (one sequence, one value
// head; gamma = inclusive gate cumsum inside the chunk; r, rho = L2-norm
// factors of k, q or 1; h = state at the chunk start, K x V):
//
//   A      = strict_lower( beta_i r_i r_j exp(gamma_i - gamma_j) k_i.k_j )
//   T      = (I + A)^-1
//   W      = T diag(beta e^gamma r) K          U = T diag(beta) V
//   V_new  = U - W h
//   O      = diag(scale rho e^gamma) Q h + P V_new,
//            P = causal( scale rho_i r_j exp(gamma_i - gamma_j) q_i.k_j )
//   h_next = e^{gamma_L} h + (diag(r e^{gamma_L - gamma}) K)^T V_new
//
// The L2 norm is folded in as the row scalings r and rho (exactly equal to
// normalising first), and every exponential takes a masked non-positive
// argument (i >= j) or gamma itself.
//
// Kernels (one stream, no host synchronisation):
//   chunk_index_kernel  packed batches only: chunk record -> sequence map
//   prep_kernel         per (chunk, value head): norms, cumsum, Gram products,
//                       solve_tril, W/U, P and the scaled Q, K^T records
//   scan_kernel         per (sequence, value head, 16-column value tile): the
//                       sequential state scan with the output readout fused in
//
// Matrix products use the gfx950 MFMA v_mfma_f32_16x16x32_bf16 (bf16 mode) or
// eight v_mfma_f32_16x16x4_f32 with the same register layout (fp32 check mode).
// Register layout of one 16x16x32 product, lane l = 16*grp + l16:
//   A (16 x 32): lane holds row l16, eight reduction slots of group grp
//   B (32 x 16): lane holds column l16, the same eight reduction slots
//   C (16 x 16): lane holds column l16, rows 4*grp .. 4*grp+3
// Which reduction index a slot stands for is free as long as A and B agree.
// The scan uses that freedom: slots 0-3 of group grp carry reduction rows
// 4*grp..4*grp+3 and slots 4-7 carry rows 16+4*grp..16+4*grp+3 of a 32-row
// step, which is exactly what two stacked C tiles hold.  So the fp32 state
// (a C tile stack) and V_new (another one) feed the next product as B
// operands without any data exchange between lanes.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

template <typename E> struct VT;
template <> struct VT<bf16> {
    typedef bf16x8 v8;    // one MFMA operand fragment
    typedef bf16x4 v4;    // half a fragment
    typedef bf16x8 v16b;  // 16 bytes
    static constexpr int kVec = 8;
};
template <> struct VT<float> {
    typedef f32x8 v8;
    typedef f32x4 v4;
    typedef f32x4 v16b;
    static constexpr int kVec = 4;
};

template <typename E> __device__ __forceinline__ E to_e(float x);
template <> __device__ __forceinline__ bf16 to_e<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float to_e<float>(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

// Eight consecutive elements (16-byte aligned) as one fragment.
template <typename E> __device__ __forceinline__ typename VT<E>::v8 ld8(const E *p);
template <> __device__ __forceinline__ bf16x8 ld8<bf16>(const bf16 *p) { return *(const bf16x8 *)p; }
template <> __device__ __forceinline__ f32x8 ld8<float>(const float *p) {
    f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Two runs of four elements, at p and p + 16, as one fragment (the scan's
// reduction-slot order).
template <typename E> __device__ __forceinline__ typename VT<E>::v8 ld4x2(const E *p) {
    typedef typename VT<E>::v4 v4;
    v4 a = *(const v4 *)p, b = *(const v4 *)(p + 16);
    typename VT<E>::v8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = a[e];
        r[4 + e] = b[e];
    }
    return r;
}

// Sequence offsets are read clamped to [0, T]: a malformed cu_seqlens then
// yields wrong rows, never an access outside the token range.
__device__ __forceinline__ int cu_at(const int32_t *cu, int n, int T) { return min(max(cu[n], 0), T); }

struct ChunkGeom {
    int n;        // sequence
    int64_t t0;   // first token (row of the flattened [B*T] token axis)
    int L;        // valid rows, 1..64
};

// Maps chunk record gc to its sequence and token range; false if the record is
// unused (packed batches allot an upper bound of records).
__device__ __forceinline__ bool resolve_chunk(int gc, const Params &p, ChunkGeom &cg) {
    if (p.cu_seqlens) {
        if (gc >= p.seq_chunk_off[p.N]) return false;
        const int n = p.chunk_seq[gc];
        const int c = gc - p.seq_chunk_off[n];
        const int s0 = cu_at(p.cu_seqlens, n, p.T), s1 = cu_at(p.cu_seqlens, n + 1, p.T);
        cg.n = n;
        cg.t0 = s0 + (int64_t)kChunk * c;
        cg.L = (int)min((int64_t)kChunk, s1 - cg.t0);
    } else {
        const int ncs = (p.T + kChunk - 1) / kChunk;
        if (gc >= p.N * ncs) return false;
        cg.n = gc / ncs;
        const int c = gc % ncs;
        cg.t0 = (int64_t)cg.n * p.T + (int64_t)kChunk * c;
        cg.L = min(kChunk, p.T - kChunk * c);
    }
    return cg.L > 0;
}

// ---------------------------------------------------------------------------
// Packed batches: chunk offsets of the sequences and the record -> sequence
// map, computed on the device (cu_seqlens never travels to the host).
// One workgroup of 1024 threads walks the sequences 1024 at a time.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024)
chunk_index_kernel(const int32_t *__restrict__ cu, int N, int T, int nc_max, int32_t *__restrict__ seq_chunk_off,
                   int32_t *__restrict__ chunk_seq) {
    __shared__ int s_off[1025];
    __shared__ int s_wave[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int carry = 0;
    for (int base = 0; base < N; base += 1024) {
        const int cnt_blk = min(1024, N - base);
        const int n = base + tid;
        int cnt = 0;
        if (tid < cnt_blk) cnt = (max(cu_at(cu, n + 1, T) - cu_at(cu, n, T), 0) + kChunk - 1) / kChunk;
        int x = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == 63) s_wave[wave] = x;
        __syncthreads();
        if (tid == 0) {
            int acc = 0;
            for (int w = 0; w < 16; ++w) {
                int t = s_wave[w];
                s_wave[w] = acc;
                acc += t;
            }
        }
        __syncthreads();
        // offsets are capped at nc_max so that inconsistent offsets can never
        // index past the records the workspace holds
        const int incl = min(carry + s_wave[wave] + x, nc_max);
        const int excl = min(carry + s_wave[wave] + x - cnt, nc_max);
        if (tid < cnt_blk) {
            s_off[tid] = excl;
            seq_chunk_off[n] = excl;
            if (tid == cnt_blk - 1) s_off[cnt_blk] = incl;
        }
        __syncthreads();
        const int first = s_off[0], last = s_off[cnt_blk];
        for (int gc = first + tid; gc < last; gc += 1024) {
            int lo = 0, hi = cnt_blk - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_off[mid] <= gc) lo = mid; else hi = mid - 1;
            }
            chunk_seq[gc] = base + lo;
        }
        carry = last;
        __syncthreads();
    }
    if (tid == 0) seq_chunk_off[N] = carry;
}

// ---------------------------------------------------------------------------
// Intra-chunk preparation, one workgroup (4 waves) per (chunk, value head).
// ---------------------------------------------------------------------------
__constant__ int kLowerTiles[10][2] = {{0, 0}, {1, 0}, {1, 1}, {2, 0}, {2, 1},
                                       {2, 2}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};
__constant__ int kUpperTiles[6][2] = {{0, 1}, {0, 2}, {0, 3}, {1, 2}, {1, 3}, {2, 3}};

template <typename E, int K, int V> struct PrepLds {
    static constexpr int kPad = 16 / sizeof(E);   // 16-byte row pad against bank conflicts
    static constexpr int KP = K + kPad, VP = V + kPad;
    E k[64][KP];
    union {
        E q[64][KP];       // raw q rows (until the Gram products and Qs are done)
        float T[64][65];   // (I + A)^-1
    } u;
    E v[64][VP];
    float A[64][65];
    float Y[3][16][17];
    float gam[64], beta[64], r[64], rho[64], wsc[64];
};

template <typename E, int K, int V>
__global__ void __launch_bounds__(256) prep_kernel(Params p) {
    typedef typename VT<E>::v8 v8;
    typedef typename VT<E>::v4 v4;
    typedef typename VT<E>::v16b v16b;
    constexpr int VEC = VT<E>::kVec;
    __shared__ PrepLds<E, K, V> s;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, grp = lane >> 4;
    const int gc = blockIdx.x / p.HV, j = blockIdx.x % p.HV;
    ChunkGeom cg;
    if (!resolve_chunk(gc, p, cg)) return;
    const int jk = j / (p.HV / p.H);
    const size_t rec = (size_t)gc * p.HV + j;
    const E *qg = (const E *)p.q, *kg = (const E *)p.k, *vg = (const E *)p.v;

    // 1. Stage the chunk's k, q (key head jk) and v (value head j) rows in
    //    LDS, zero rows past the end; gate cumsum and beta in wave 0.
    for (int idx = tid; idx < 64 * K / VEC; idx += 256) {
        const int i = idx / (K / VEC), c = (idx % (K / VEC)) * VEC;
        v16b kv = {}, qv = {};
        if (i < cg.L) {
            const size_t off = ((size_t)(cg.t0 + i) * p.H + jk) * K + c;
            kv = *(const v16b *)(kg + off);
            qv = *(const v16b *)(qg + off);
        }
        *(v16b *)&s.k[i][c] = kv;
        *(v16b *)&s.u.q[i][c] = qv;
    }
    for (int idx = tid; idx < 64 * V / VEC; idx += 256) {
        const int i = idx / (V / VEC), c = (idx % (V / VEC)) * VEC;
        v16b vv = {};
        if (i < cg.L) vv = *(const v16b *)(vg + ((size_t)(cg.t0 + i) * p.HV + j) * V + c);
        *(v16b *)&s.v[i][c] = vv;
    }
    if (wave == 0) {
        float gv = 0.f, bv = 0.f;
        if (lane < cg.L) {
            const size_t o = (size_t)(cg.t0 + lane) * p.HV + j;
            gv = p.g[o];
            bv = p.beta[o];
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(gv, o);
            if (lane >= o) gv += y;
        }
        s.gam[lane] = gv;
        s.beta[lane] = bv;
    }
    __syncthreads();

    // 2. Inverse L2 norms of the k and q rows (4 threads per row).
    {
        const int row = tid >> 2, part = tid & 3;
        float sk = 0.f, sq = 0.f;
#pragma unroll 8
        for (int c = part * (K / 4); c < (part + 1) * (K / 4); ++c) {
            const float a = to_f(s.k[row][c]), b = to_f(s.u.q[row][c]);
            sk += a * a;
            sq += b * b;
        }
        sk += __shfl_xor(sk, 1);
        sk += __shfl_xor(sk, 2);
        sq += __shfl_xor(sq, 1);
        sq += __shfl_xor(sq, 2);
        if (part == 0) {
            const float rk = p.use_l2norm ? 1.f / sqrtf(sk + 1e-6f) : 1.f;
            const float rq = p.use_l2norm ? 1.f / sqrtf(sq + 1e-6f) : 1.f;
            s.r[row] = rk;
            s.rho[row] = rq;
            s.wsc[row] = s.beta[row] * __expf(s.gam[row]) * rk;
        }
    }
    __syncthreads();

    // 3. Gram products on the lower 16x16 tiles: K K^T -> A (LDS, fp32) and
    //    Q K^T -> P (record, gated, causal, scaled).
    const float gl = s.gam[63];   // gamma at the last valid row (padding adds 0)
    E *pm = (E *)p.pm + rec * 64 * 64;
    for (int job = wave; job < 20; job += 4) {
        const bool isq = job >= 10;
        const int it = kLowerTiles[job % 10][0], jt = kLowerTiles[job % 10][1];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < K / 32; ++st) {
            const v8 a = isq ? ld8<E>(&s.u.q[16 * it + l16][32 * st + 8 * grp])
                             : ld8<E>(&s.k[16 * it + l16][32 * st + 8 * grp]);
            const v8 b = ld8<E>(&s.k[16 * jt + l16][32 * st + 8 * grp]);
            acc = mma(a, b, acc);
        }
        const int jj = 16 * jt + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * it + 4 * grp + e;
            if (!isq) {
                s.A[i][jj] = (i > jj) ? s.beta[i] * s.r[i] * s.r[jj] * __expf(s.gam[i] - s.gam[jj]) * acc[e]
                                      : 0.f;
            } else {
                const float val = (i >= jj) ? p.scale * s.rho[i] * s.r[jj] * __expf(s.gam[i] - s.gam[jj]) * acc[e]
                                            : 0.f;
                pm[i * 64 + jj] = to_e<E>(val);
            }
        }
    }
    for (int idx = tid; idx < 6 * 256; idx += 256) {
        const int t = idx >> 8, e = idx & 255;
        pm[(16 * kUpperTiles[t][0] + (e >> 4)) * 64 + 16 * kUpperTiles[t][1] + (e & 15)] = to_e<E>(0.f);
    }

    // 4. Scaled copies for the scan: Qs = diag(scale rho e^gamma) Q (rows) and
    //    Kt = (diag(r e^{gamma_L - gamma}) K)^T, plus the chunk decay.
    {
        E *qs = (E *)p.qs + rec * 64 * K;
        for (int idx = tid; idx < 64 * K / VEC; idx += 256) {
            const int i = idx / (K / VEC), c = (idx % (K / VEC)) * VEC;
            const float f = p.scale * s.rho[i] * __expf(s.gam[i]);
            v16b x = *(const v16b *)&s.u.q[i][c];
#pragma unroll
            for (int e = 0; e < VEC; ++e) x[e] = to_e<E>(f * to_f(x[e]));
            *(v16b *)(qs + i * K + c) = x;
        }
        E *kt = (E *)p.kt + rec * K * 64;
        for (int idx = tid; idx < K * 64 / VEC; idx += 256) {
            const int m = idx / (64 / VEC), i0 = (idx % (64 / VEC)) * VEC;
            v16b x;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int i = i0 + e;
                x[e] = to_e<E>(s.r[i] * __expf(gl - s.gam[i]) * to_f(s.k[i][m]));
            }
            *(v16b *)(kt + m * 64 + i0) = x;
        }
        if (tid == 0) p.decay[rec] = __expf(gl);
    }
    __syncthreads();   // raw q is dead from here on; its LDS becomes T

    // 5. solve_tril: T = (I + A)^-1 by 16x16 blocks.  Diagonal blocks by
    //    forward substitution, one block per 16-lane group of wave 0 (lane =
    //    column); then the off-diagonal blocks level by level:
    //    T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj.
    if (wave == 0) {
        const int b = grp, c = l16;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) acc -= s.A[16 * b + r][16 * b + m] * x[m];
            x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) s.u.T[16 * b + r][16 * b + c] = x[r];
    }
    __syncthreads();
    for (int d = 1; d <= 3; ++d) {
        const bool active = wave < 4 - d;
        const int bi = wave + d, bj = wave;
        if (active) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 4 * grp + e;
                float acc = 0.f;
                for (int kk = 16 * bj; kk < 16 * bi; ++kk) acc += s.A[16 * bi + rr][kk] * s.u.T[kk][16 * bj + l16];
                s.Y[wave][rr][l16] = acc;
            }
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 4 * grp + e;
                float acc = 0.f;
                for (int t = 0; t <= rr; ++t) acc += s.u.T[16 * bi + rr][16 * bi + t] * s.Y[wave][t][l16];
                s.u.T[16 * bi + rr][16 * bj + l16] = -acc;
            }
        }
        __syncthreads();
    }

    // 6. -W = -T diag(beta e^gamma r) K  and  U = T diag(beta) V  on MFMA.
    //    T is lower triangular, so output rows 0-31 only need tokens 0-31.
    E *wn = (E *)p.wneg + rec * 64 * K;
    E *ut = (E *)p.ut + rec * V * 64;
    constexpr int NWT = 4 * (K / 16), NUT = 4 * (V / 16);
    for (int job = wave; job < NWT + NUT; job += 4) {
        const bool isw = job < NWT;
        const int jb = isw ? job : job - NWT;
        const int it = jb & 3, ct = jb >> 2;
        const int i = 16 * it + l16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int nst = (it >= 2) ? 2 : 1;
        for (int st = 0; st < nst; ++st) {
            v8 a, b;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int jj = 32 * st + 8 * grp + e;
                const float tv = (jj <= i) ? s.u.T[i][jj] : 0.f;
                a[e] = to_e<E>(isw ? -tv * s.wsc[jj] : tv * s.beta[jj]);
                b[e] = isw ? s.k[jj][16 * ct + l16] : s.v[jj][16 * ct + l16];
            }
            acc = mma(a, b, acc);
        }
        if (isw) {
#pragma unroll
            for (int e = 0; e < 4; ++e) wn[(16 * it + 4 * grp + e) * K + 16 * ct + l16] = to_e<E>(acc[e]);
        } else {
            v4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = to_e<E>(acc[e]);
            *(v4 *)(ut + (16 * ct + l16) * 64 + 16 * it + 4 * grp) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// Sequential state scan with the output readout, one wave per
// (sequence, value head, 16-column value tile).  The K x 16 fp32 state tile
// lives in registers for the whole sequence.
// ---------------------------------------------------------------------------
template <typename E, int K, int V>
__global__ void __launch_bounds__(64) scan_kernel(Params p) {
    typedef typename VT<E>::v8 v8;
    typedef typename VT<E>::v4 v4;
    constexpr int NVT = V / 16, KT = K / 16, KS = K / 32;
    const int lane = threadIdx.x, l16 = lane & 15, grp = lane >> 4;
    // Workgroup ids go round-robin over the 8 XCDs; keep all value tiles of
    // one (sequence, head) pair on one XCD so that the chunk records they all
    // read come from HBM once and then from that XCD's L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int vt = slot % NVT;
    const int pair = (slot / NVT) * 8 + xcd;
    if (pair >= p.N * p.HV) return;
    const int n = pair / p.HV, j = pair % p.HV;
    const int col = 16 * vt + l16;

    int c0, c1;
    int64_t tok0, seq_end;
    if (p.cu_seqlens) {
        c0 = p.seq_chunk_off[n];
        c1 = p.seq_chunk_off[n + 1];
        tok0 = cu_at(p.cu_seqlens, n, p.T);
        seq_end = cu_at(p.cu_seqlens, n + 1, p.T);
    } else {
        const int ncs = (p.T + kChunk - 1) / kChunk;
        c0 = n * ncs;
        c1 = c0 + ncs;
        tok0 = (int64_t)n * p.T;
        seq_end = tok0 + p.T;
    }

    f32x4 h[KT];
    const size_t sbase = ((size_t)n * p.HV + j) * K * V;
    if (p.initial_state) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) h[t][e] = p.initial_state[sbase + (size_t)(16 * t + 4 * grp + e) * V + col];
    } else {
#pragma unroll
        for (int t = 0; t < KT; ++t) h[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    E *out = (E *)p.out;
    for (int c = c0; c < c1; ++c) {
        const size_t rec = (size_t)c * p.HV + j;
        const int64_t t0 = tok0 + (int64_t)(c - c0) * kChunk;
        const int L = (int)min((int64_t)kChunk, seq_end - t0);
        const E *W = (const E *)p.wneg + rec * 64 * K;
        const E *Q = (const E *)p.qs + rec * 64 * K;
        const E *KTm = (const E *)p.kt + rec * K * 64;
        const E *UT = (const E *)p.ut + rec * V * 64;
        const E *PM = (const E *)p.pm + rec * 64 * 64;
        const float dec = p.decay[rec];

        // state as B operand fragments
        v8 hb[KS];
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hb[s2][e] = to_e<E>(h[2 * s2][e]);
                hb[s2][4 + e] = to_e<E>(h[2 * s2 + 1][e]);
            }
        // V_new = U + (-W) h ;  O = Qs h
        f32x4 accv[4], acco[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const v4 u = *(const v4 *)(UT + col * 64 + 16 * ti + 4 * grp);
#pragma unroll
            for (int e = 0; e < 4; ++e) accv[ti][e] = to_f(u[e]);
            acco[ti] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) {
                const v8 aw = ld4x2<E>(W + (16 * ti + l16) * K + 32 * s2 + 4 * grp);
                accv[ti] = mma(aw, hb[s2], accv[ti]);
                const v8 aq = ld4x2<E>(Q + (16 * ti + l16) * K + 32 * s2 + 4 * grp);
                acco[ti] = mma(aq, hb[s2], acco[ti]);
            }
        // V_new as B operand fragments (reduction over the chunk's tokens)
        v8 vb[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vb[s2][e] = to_e<E>(accv[2 * s2][e]);
                vb[s2][4 + e] = to_e<E>(accv[2 * s2 + 1][e]);
            }
        // O += P V_new, then store the valid rows
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const v8 ap = ld4x2<E>(PM + (16 * ti + l16) * 64 + 32 * s2 + 4 * grp);
                acco[ti] = mma(ap, vb[s2], acco[ti]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * ti + 4 * grp + e;
                if (i < L) out[((size_t)(t0 + i) * p.HV + j) * V + col] = to_e<E>(acco[ti][e]);
            }
        }
        // h = e^{gamma_L} h + Kt V_new
#pragma unroll
        for (int mt = 0; mt < KT; ++mt) {
            h[mt] *= dec;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const v8 ak = ld4x2<E>(KTm + (16 * mt + l16) * 64 + 32 * s2 + 4 * grp);
                h[mt] = mma(ak, vb[s2], h[mt]);
            }
        }
    }
    if (p.final_state) {
#pragma unroll
        for (int t = 0; t < KT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) p.final_state[sbase + (size_t)(16 * t + 4 * grp + e) * V + col] = h[t][e];
    }
}

template <typename E, int K, int V> hipError_t launch_typed(const Params &p, hipStream_t st, Profiler *prof) {
    if (p.cu_seqlens) {
        if (prof) prof->begin(kIndexKernel, st);
        chunk_index_kernel<<<1, 1024, 0, st>>>(p.cu_seqlens, p.N, p.T, p.nc_max, p.seq_chunk_off, p.chunk_seq);
        if (prof) prof->end(kIndexKernel, st);
    }
    // equal-length batches use exactly N * ceil(T/64) records
    const int nrec = p.cu_seqlens ? p.nc_max : p.N * ((p.T + kChunk - 1) / kChunk);
    if (nrec > 0) {
        if (prof) prof->begin(kPrepKernel, st);
        prep_kernel<E, K, V><<<(unsigned)nrec * p.HV, 256, 0, st>>>(p);
        if (prof) prof->end(kPrepKernel, st);
    }
    const int pairs = p.N * p.HV;
    if (pairs > 0) {
        const unsigned grid = (unsigned)((pairs + 7) / 8) * 8 * (V / 16);
        if (prof) prof->begin(kScanKernel, st);
        scan_kernel<E, K, V><<<grid, 64, 0, st>>>(p);
        if (prof) prof->end(kScanKernel, st);
    }
    return hipGetLastError();
}

template <typename E> hipError_t launch_dim(const Params &p, hipStream_t st, Profiler *prof) {
    if (p.K == 64 && p.V == 64) return launch_typed<E, 64, 64>(p, st, prof);
    if (p.K == 64 && p.V == 128) return launch_typed<E, 64, 128>(p, st, prof);
    if (p.K == 128 && p.V == 64) return launch_typed<E, 128, 64>(p, st, prof);
    return launch_typed<E, 128, 128>(p, st, prof);
}

}  // namespace

const char *kernel_name(int kind) {
    switch (kind) {
        case kIndexKernel: return "chunk_index_kernel";
        case kPrepKernel: return "prep_kernel";
        case kScanKernel: return "scan_kernel";
        default: return "?";
    }
}

hipError_t launch_forward(const Params &p, int dtype, hipStream_t stream, Profiler *prof) {
    return dtype == 0 ? launch_dim<bf16>(p, stream, prof) : launch_dim<float>(p, stream, prof);
}

}  // namespace gdn
