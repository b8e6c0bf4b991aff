// Warp-specialized fused forward pass (bf16) for gfx950.
//
// Same mathematics as the single-role kernel in gdn_fused.hip (the step list
// of the page "NPU Training Operators - GDN", operator-semantics section, in
// the chunk form written out at the top of that file), scheduled differently:
// a workgroup has 12 waves, three per SIMD, in three roles.
//   waves 0-3   chain waves: each owns 16 state columns and runs everything
//               that depends on the state h: X, the block forward substitution
//               for V_new, the output, the state update, and Z = K h and
//               (Q h)^T of the next chunk.
//   waves 4-7   K-prep waves, one chunk ahead: gate cumsum, K K^T Gram tiles of
//               row tile w and the norms of the k rows of tiles 0..w, the
//               gated -A tiles, the diagonal-block inverse D_w; wave 7, which
//               has every norm, also the per-token state factors.
//   waves 8-11  Q-prep waves, one chunk ahead: the asynchronous copies of the
//               raw rows (two chunks ahead), gate cumsum, Q K^T Gram tiles of
//               row tile w, the norms of its q rows and of the k rows of tiles
//               0..w, the gated P tiles.
// The SIMDs interleave the serial state chain of chunk c with the
// preparation of chunk c+1.  Each step ends with the only workgroup barrier
// of the step; every prep wave computes the cumsum and norm values it needs
// itself, so the prep waves never wait for each other inside a step.
//
// Buffers: raw k and v rows in rings of three chunks (the chain reads chunk
// c's while c+1's is resident and c+2's streams in), raw q/g/beta and the prep
// outputs double-buffered by chunk parity.  Rows past the end of a sequence
// are copies of its last row; the cumsum reads their g and beta as 0, which
// makes their rows of A, X and V_new zero and leaves gamma_L at the last real
// token, so they contribute nothing.
//
// In-kernel gating: the copying wave fetches the raw gate words of chunk c+3
// (their own ring) and, at the start of the next step, turns those of chunk
// c+2 into g and beta in the g/beta ring, so every gate is computed once and
// off the step's barrier-to-barrier path.
#include <stddef.h>

#include <type_traits>

#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous global -> LDS copies: lane l's bytes land at lds + l * size.
// They are issued from inline assembly on purpose: the compiler does not track
// them, so it neither waits for them before unrelated LDS reads nor at the
// LDS fences of the barriers.  The code that consumes a copy waits for it
// explicitly (wait_vmem, then a barrier).  Vector memory counters retire in
// order, so the compiler's own counter waits stay correct (at worst they wait
// longer).
__device__ __forceinline__ void lds_copy16(const void *g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const void *g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(g), "s"(lds) : "memory", "m0");
}
// Wait until this wave's vector memory operations (its copies) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts by
// 1, 2, 4, 8 inside each row of 16 lanes (zero fill), then the running totals
// of rows 0 and 0..1 broadcast into the later rows.
template <int CTRL, int ROW_MASK> __device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    x += dpp_mov<0x111, 0xf>(x);   // row_shr:1
    x += dpp_mov<0x112, 0xf>(x);   // row_shr:2
    x += dpp_mov<0x114, 0xf>(x);   // row_shr:4
    x += dpp_mov<0x118, 0xf>(x);   // row_shr:8
    x += dpp_mov<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_mov<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

template <int N> struct IC { static constexpr int value = N; };

// Orders LDS writes of some lanes of a wave before LDS reads of other lanes of
// the same wave.  The hardware keeps a wave's LDS accesses in order; this only
// stops the compiler from moving the reads above the writes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// XOR swizzle of the 16-byte segments of a row of NSEG segments.
template <int NSEG> __device__ __forceinline__ int swz(int row) {
    static_assert(NSEG == 8 || NSEG % 16 == 0, "row length");
    return NSEG >= 16 ? (row & 15) : ((row >> 1) & 7);
}
template <int W> __device__ __forceinline__ int sw_off(int row, int col) {
    constexpr int NSEG = W / 8;
    return row * W + (((col >> 3) ^ swz<NSEG>(row)) << 3) + (col & 7);
}

// Per-chunk results of the prep waves that the chain waves read.
struct alignas(16) PrepOut {
    bf16 alo[64][68];         // -A in the off-diagonal 16x16 blocks below the diagonal
    bf16 p[64][72];           // P, columns in the key-slot order (see pcol); blocks (0,1), (2,3) zero
    bf16 dt[4][16][16];       // D_b transposed: dt[b][j][i] = D_b[i][j]
    float gam[64];            // gate cumsum, log2 units
    float beta[64];
    float bgr[64];            // beta e^gamma r
    float rq[64];             // L2-norm factor rho of q (1 without the norm)
    float kf[64];             // r e^{gamma_L - gamma}
    float decay;              // e^{gamma_L}
};

// Column of token j in PrepOut::p.  The output product reads P as the B
// operand of a 16x16x32 product whose lane-group g holds tokens
// 32 s + 4 g + e and 32 s + 16 + 4 g + e (e = 0..3); storing those eight
// columns next to each other makes each operand one 16-byte read.
__device__ __forceinline__ constexpr int pcol(int jt, int g) {   // first column of tile jt, group g
    return 32 * (jt >> 1) + 8 * g + 4 * (jt & 1);
}

template <int K, int VW> struct WsLds {
    bf16 kb[3][64 * K];       // raw k rows (swizzled), ring of three chunks
    bf16 qb[2][64 * K];       // raw q rows (swizzled)
    bf16 vb[3][64 * VW];      // raw v rows of this slice (swizzled), ring of three chunks
    float gb[2][64], bb[2][64];
    PrepOut po[2];
    float adiag[4][16 * 20];  // per K-prep wave: its diagonal block of A, fp32, transposed (A_ij at 20 j + i)
    float stk[4][3][64];      // per K-prep wave: gamma, beta, r of the chunk being prepared
    float stq[4][2][64];      // per Q-prep wave: gamma, r of the chunk being prepared
};
// With in-kernel gating: the raw gate words, by chunk parity, after the rest.
template <int K, int VW> struct WsLdsGated : WsLds<K, VW> {
    float ra[2][64], rb[2][64];
};

// The state h (K x V per value head) is held by the chain waves as K/16 tiles
// of 16 key rows x 16 value columns in the accumulator layout (lane: value
// column l16, tile rows 4 grp + e).  Tile mt row r stands for key dimension
//   kappa(mt, r) = 32 (mt / 2) + 8 (r / 4) + 4 (mt % 2) + r % 4,
// so that the eight key dimensions a lane group contributes to one 32-wide
// reduction step (rows 4 grp + e of tiles 2s and 2s+1) are consecutive:
// 32 s + 8 grp + 0..7.  Raw k/q fragments are then single 16-byte LDS reads.
// Every product that involves h (Z = K h, (Q h)^T, K^T V_new) uses the same
// assignment, and the state is read and written through it.
__device__ __forceinline__ constexpr int kappa(int mt, int r) {
    return 32 * (mt >> 1) + 8 * (r >> 2) + 4 * (mt & 1) + (r & 3);
}

// GATED: the gates come from the raw inputs (p.gates) instead of p.g / p.beta.
// POOL: the states live in a slot-indexed pool and/or are stored as bf16
// (p.state_indices, p.state_bf16).  Template parameters, so that the plain
// kernel carries none of their code.
template <int K, int V, bool GATED, bool POOL>
__global__ void __launch_bounds__(768) fused_ws_kernel(Params p) {
    typedef bf16 E;
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    typedef __attribute__((address_space(3))) bf16x4 lds_v4;
    typedef typename std::conditional<GATED, WsLdsGated<K, 64>, WsLds<K, 64>>::type Lds;
    constexpr int VW = 64, VEC = 8;
    constexpr int NSK = K / VEC, NSV = VW / VEC;
    constexpr int KT = K / 16, KS = K / 32;
    constexpr int KROW = 2 * K, VROW = 2 * VW;   // bytes per raw row in LDS
    static_assert(sizeof(Lds) <= 160 * 1024, "LDS budget");
    __shared__ Lds s;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int role = wave >> 2;   // 0 chain, 1 K-prep, 2 Q-prep
    const int w4 = wave & 3;      // chain: column tile; prep: row tile
    const int l16 = lane & 15, grp = lane >> 4;

    // Workgroup -> (sequence n, key head jk, value head j, value slice).  The
    // workgroups of one (n, jk) share q/k through L2 and sit on one XCD.
    const int G = p.HV / p.H;
    constexpr int VS = V / VW;
    const int per_group = G * VS;
    const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
    const int member = slot % per_group;
    const int group = (slot / per_group) * 8 + xcd;
    if (group >= p.N * p.H) return;
    const int n = group / p.H, jk = group % p.H;
    const int j = jk * G + member / VS;
    const int vcol0 = (member % VS) * VW;

    int64_t tok0;
    int len;
    if (p.cu_seqlens) {
        tok0 = cu_at(p.cu_seqlens, n, p.T);
        len = max(cu_at(p.cu_seqlens, n + 1, p.T) - (int)tok0, 0);
    } else {
        tok0 = (int64_t)n * p.T;
        len = p.T;
    }
    const int nchunks = (len + 63) / 64;

    // Raw gate inputs, when given: the head's constants, and which half of its
    // aligned 4-byte word a bf16 input occupies (HV is even, so the half is
    // the parity of j for every token).
    constexpr bool gated = GATED;
    const float negA = gated ? -expf(p.gates.A_log[j]) : 0.f;
    const float dtb = gated ? p.gates.dt_bias[j] : 0.f;
    const bool ghi = sizeof(E) == 2 && (j & 1);

    const E *__restrict__ qg = (const E *)p.q;
    const E *__restrict__ kg = (const E *)p.k;
    const E *__restrict__ vg = (const E *)p.v;
    E *__restrict__ og = (E *)p.out;
    const size_t kq_row = (size_t)p.H * K, v_row = (size_t)p.HV * V;

    // raw k/q fragment of row tile t, step s2: row 16 t + l16, key slots
    // 32 s2 + 8 grp .. +7 (one swizzled 16-byte segment)
    int fo[KS];
    {
        const int sw = swz<NSK>(l16);   // the swizzle of row 16 t + l16 does not depend on t
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) fo[s2] = l16 * KROW + (((4 * s2 + grp) ^ sw) << 4);
    }
    auto frag = [&](const E *buf, int t, int s2) {
        return *(const v8 *)((const char *)buf + fo[s2] + t * 16 * KROW);
    };
    auto tr = [&](const void *pt) { return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4 *)pt); };

    // gate cumsum of chunk c in log2 units (lane = token), and beta; rows past
    // the end of the sequence read 0
    auto cumsum = [&](int c, float &gam, float &b) {
        const int L = min(64, len - 64 * c);
        b = lane < L ? s.bb[c & 1][lane] : 0.f;
        gam = wave_inclusive_scan(lane < L ? s.gb[c & 1][lane] : 0.f) * 1.4426950408889634f;
    };
    // With raw gate inputs, the copying wave turns the landed raw words of
    // chunk c into g and beta (one wave computes each gate once).
    auto gate_chunk = [&](int c) {
        if constexpr (GATED) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");   // after the copies' wait
            s.gb[c & 1][lane] = gate_g(gate_raw<E>(s.ra[c & 1][lane], ghi), negA, dtb);
            s.bb[c & 1][lane] = gate_beta(gate_raw<E>(s.rb[c & 1][lane], ghi));
        }
    };

    // ---- asynchronous copies (Q-prep waves) --------------------------------
    // LDS destinations are byte addresses (wave-uniform); the per-lane source
    // offsets inside a full chunk are fixed, only the last chunk of a sequence
    // clamps its rows.
    const unsigned lds0 = (unsigned)(size_t)(lds_void *)&s;
    unsigned kqo[NSK / 4], vvo[NSV / 4];
#pragma unroll
    for (int i = 0; i < NSK / 4; ++i) {
        const int P = 64 * (w4 + 4 * i) + lane, row = P / NSK;
        kqo[i] = (unsigned)row * (unsigned)kq_row + (((P % NSK) ^ swz<NSK>(row)) * VEC);
    }
#pragma unroll
    for (int i = 0; i < NSV / 4; ++i) {
        const int P = 64 * (w4 + 4 * i) + lane, row = P / NSV;
        vvo[i] = (unsigned)row * (unsigned)v_row + (((P % NSV) ^ swz<NSV>(row)) * VEC);
    }
    auto issue = [&](int c) {
        const int64_t t0 = tok0 + 64LL * c;
        const int last = min(64, len - 64 * c) - 1;
        const unsigned kl = lds0 + offsetof(Lds, kb) + (c % 3) * (64 * K * 2);
        const unsigned ql = lds0 + offsetof(Lds, qb) + (c & 1) * (64 * K * 2);
        const unsigned vl = lds0 + offsetof(Lds, vb) + (c % 3) * (64 * VW * 2);
        const E *kc = kg + (size_t)t0 * kq_row + (size_t)jk * K;
        const E *qc = qg + (size_t)t0 * kq_row + (size_t)jk * K;
        const E *vc = vg + (size_t)t0 * v_row + (size_t)j * V + vcol0;
        if (last == 63) {
#pragma unroll
            for (int i = 0; i < NSK / 4; ++i) {
                const unsigned d = 1024u * (w4 + 4 * i);
                lds_copy16(kc + kqo[i], kl + d);
                lds_copy16(qc + kqo[i], ql + d);
            }
#pragma unroll
            for (int i = 0; i < NSV / 4; ++i) lds_copy16(vc + vvo[i], vl + 1024u * (w4 + 4 * i));
        } else {
#pragma unroll
            for (int i = 0; i < NSK / 4; ++i) {
                const int t = w4 + 4 * i;
                const int P = 64 * t + lane, row = P / NSK, seg = (P % NSK) ^ swz<NSK>(row);
                const unsigned off = (unsigned)min(row, last) * (unsigned)kq_row + seg * VEC;
                lds_copy16(kc + off, kl + 1024u * t);
                lds_copy16(qc + off, ql + 1024u * t);
            }
#pragma unroll
            for (int i = 0; i < NSV / 4; ++i) {
                const int t = w4 + 4 * i;
                const int P = 64 * t + lane, row = P / NSV, seg = (P % NSV) ^ swz<NSV>(row);
                lds_copy16(vc + (unsigned)min(row, last) * (unsigned)v_row + seg * VEC, vl + 1024u * t);
            }
        }
        if (w4 == 3 && !gated) {
            const size_t o = (size_t)(t0 + min(lane, last)) * p.HV + j;
            lds_copy4(p.g + o, lds0 + offsetof(Lds, gb) + (c & 1) * 256);
            lds_copy4(p.beta + o, lds0 + offsetof(Lds, bb) + (c & 1) * 256);
        }
    };
    // raw gate words of chunk c (in-kernel gating; the copying wave only):
    // the aligned 4-byte word that holds each token's input
    auto issue_gates = [&](int c) {
        if constexpr (GATED) {
            const int64_t t0 = tok0 + 64LL * c;
            const int last = min(64, len - 64 * c) - 1;
            const size_t wo = (((size_t)(t0 + min(lane, last)) * p.HV + j) * sizeof(E)) & ~(size_t)3;
            lds_copy4((const char *)p.gates.a + wo, (unsigned)(size_t)(lds_void *)&s.ra[c & 1][0]);
            lds_copy4((const char *)p.gates.b + wo, (unsigned)(size_t)(lds_void *)&s.rb[c & 1][0]);
        }
    };

    if (role == 2 && nchunks > 0) {
        issue(0);
        if (gated && w4 == 3) {
            issue_gates(0);
            if (nchunks > 1) issue_gates(1);
        }
        wait_vmem();
        if (gated && w4 == 3) gate_chunk(0);
    }
    // P blocks (0,1) and (2,3) are read by the output product but never
    // written by the epilogue: zero them once in both buffers.
    if (role == 0) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int idx = 256 * q4 + tid, b2 = idx >> 9, blk = (idx >> 8) & 1, r = (idx >> 4) & 15, jj = idx & 15;
            s.po[b2].p[32 * blk + r][pcol(2 * blk + 1, jj >> 2) + (jj & 3)] = (E)0.f;
        }
    }
    lds_barrier();

    // The three roles run separate loops with the same number of barriers, so
    // that none carries another's registers.
    if (role == 2) {
        // ============================ Q-prep ==================================
        for (int c = -1; c < nchunks; ++c) {
            const int cn = c + 1;
            if (c + 2 < nchunks) issue(c + 2);
            if (gated && w4 == 3) {
                if (c + 2 < nchunks) gate_chunk(c + 2);   // its raw words landed before the last barrier
                if (c + 3 < nchunks) issue_gates(c + 3);
            }
            if (cn < nchunks) {
                PrepOut &po = s.po[cn & 1];
                float *sg = s.stq[w4][0], *sr = s.stq[w4][1];
                {
                    float gam, b;
                    cumsum(cn, gam, b);
                    sg[lane] = gam;
                }
                const E *kb = s.kb[cn % 3], *qb = s.qb[cn & 1];
                // Transposed Gram tiles C[j][i] = k_j . q_i of row tile itq = w4
                // against column tiles jt <= itq, Q Q^T's diagonal tile, and the
                // diagonal tiles of K K^T for the norms of every k row
                auto qprep = [&](auto itq_c) {
                    constexpr int itq = decltype(itq_c)::value;
                    f32x4 gq[itq + 1], gd[itq + 1], gqq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int jt = 0; jt <= itq; ++jt) {
                        gq[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                        gd[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) {
                        v8 fk[itq + 1];
#pragma unroll
                        for (int t = 0; t <= itq; ++t) fk[t] = frag(kb, t, s2);
                        const v8 bq = frag(qb, itq, s2);
#pragma unroll
                        for (int jt = 0; jt <= itq; ++jt) {
                            gq[jt] = mma(fk[jt], bq, gq[jt]);
                            gd[jt] = mma(fk[jt], fk[jt], gd[jt]);
                        }
                        gqq = mma(bq, bq, gqq);
                    }
                    // norms of the k rows of tiles 0..itq from the diagonals: lane
                    // (l16, l16 / 4) holds row l16 at e = l16 % 4
                    {
                        const int e = l16 - 4 * grp;
                        if (e >= 0 && e < 4) {
#pragma unroll
                            for (int t = 0; t <= itq; ++t) sr[16 * t + l16] = p.use_l2norm ? rsqrtf(gd[t][e] + 1e-6f) : 1.f;
                        }
                    }
                    const float qq = __shfl(gqq[l16 & 3], (l16 >> 2) * 16 + l16);
                    const float rho = p.use_l2norm ? rsqrtf(qq + 1e-6f) : 1.f;
                    if (grp == 0) po.rq[16 * itq + l16] = rho;
                    wave_lds_sync();   // the staged gamma and r come from other lanes
                    const int iq = 16 * itq + l16;
                    const float giq = sg[iq], srq = p.scale * rho;
                    f32x4 gj[itq + 1], rj[itq + 1];
#pragma unroll
                    for (int jt = 0; jt <= itq; ++jt) {
                        gj[jt] = *(const f32x4 *)&sg[16 * jt + 4 * grp];
                        rj[jt] = *(const f32x4 *)&sr[16 * jt + 4 * grp];
                    }
#pragma unroll
                    for (int jt = 0; jt <= itq; ++jt) {
                        v4 o;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float v = srq * rj[jt][e] * fast_exp2(giq - gj[jt][e]) * gq[jt][e];
                            o[e] = (E)((jt < itq || iq >= 16 * jt + 4 * grp + e) ? v : 0.f);
                        }
                        *(v4 *)&po.p[iq][pcol(jt, grp)] = o;
                    }
                };
                switch (w4) {
                    case 0: qprep(IC<0>()); break;
                    case 1: qprep(IC<1>()); break;
                    case 2: qprep(IC<2>()); break;
                    default: qprep(IC<3>()); break;
                }
            }
            wait_vmem();   // this wave's copies of chunk c+2
            lds_barrier();
        }
        return;
    }

    if (role == 1) {
        // ============================ K-prep ==================================
        for (int c = -1; c < nchunks; ++c) {
            const int cn = c + 1;
            if (cn < nchunks) {
                PrepOut &po = s.po[cn & 1];
                float *sg = s.stk[w4][0], *sb = s.stk[w4][1], *sr = s.stk[w4][2];
                {
                    float gam, b;
                    cumsum(cn, gam, b);
                    sg[lane] = gam;
                    sb[lane] = b;
                    if (w4 == 0) {
                        po.gam[lane] = gam;
                        po.beta[lane] = b;
                    }
                }
                const E *kb = s.kb[cn % 3];
                // Transposed Gram tiles C[j][i] = k_j . k_i of row tile itk = w4
                // against column tiles jt <= itk, and the other diagonal tiles
                // for the norms of every k row
                auto kprep = [&](auto itk_c) {
                    constexpr int itk = decltype(itk_c)::value;
                    f32x4 gk[itk + 1], gd[itk + 1];
#pragma unroll
                    for (int jt = 0; jt <= itk; ++jt) {
                        gk[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                        gd[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) {
                        v8 fk[itk + 1];
#pragma unroll
                        for (int t = 0; t <= itk; ++t) fk[t] = frag(kb, t, s2);
#pragma unroll
                        for (int jt = 0; jt <= itk; ++jt) {
                            gk[jt] = mma(fk[jt], fk[itk], gk[jt]);
                            if (jt < itk) gd[jt] = mma(fk[jt], fk[jt], gd[jt]);
                        }
                    }
                    gd[itk] = gk[itk];
                    // norms of the rows of tiles 0..itk from the diagonals: lane
                    // (l16, l16 / 4) holds row l16 at e = l16 % 4
                    {
                        const int e = l16 - 4 * grp;
                        if (e >= 0 && e < 4) {
#pragma unroll
                            for (int t = 0; t <= itk; ++t) sr[16 * t + l16] = p.use_l2norm ? rsqrtf(gd[t][e] + 1e-6f) : 1.f;
                        }
                    }
                    wave_lds_sync();   // the staged gamma / beta / r come from other lanes
                    f32x4 gj[itk + 1], rj[itk + 1];
#pragma unroll
                    for (int jt = 0; jt <= itk; ++jt) {
                        gj[jt] = *(const f32x4 *)&sg[16 * jt + 4 * grp];
                        rj[jt] = *(const f32x4 *)&sr[16 * jt + 4 * grp];
                    }
                    const f32x4 bd = *(const f32x4 *)&sb[16 * itk + 4 * grp];
                    const int ik = 16 * itk + l16;
                    const float gik = sg[ik], rik = sr[ik], bik = sb[ik];
                    {   // diagonal tile -> A_itk,itk (fp32, transposed).  The raw Gram
                        // tile is symmetric, so the lane's values serve as rows
                        // i = 16 itk + 4 grp + e of column j = 16 itk + l16, which
                        // makes the transposed store one vector per lane.
                        f32x4 a;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float v = bd[e] * rj[itk][e] * rik * fast_exp2(gj[itk][e] - gik) * gk[itk][e];
                            a[e] = (4 * grp + e > l16) ? v : 0.f;
                        }
                        *(f32x4 *)&s.adiag[w4][20 * l16 + 4 * grp] = a;
                    }
                    {   // off-diagonal tiles of row tile itk -> -A (bf16)
                        const float bri = bik * rik;
#pragma unroll
                        for (int jt = 0; jt < itk; ++jt) {
                            v4 o;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                o[e] = (E)(-(bri * rj[jt][e] * fast_exp2(gik - gj[jt][e]) * gk[jt][e]));
                            *(v4 *)&po.alo[ik][16 * jt + 4 * grp] = o;
                        }
                    }
                    wave_lds_sync();   // A_itk,itk is read back across lanes by the solve
                };
                switch (w4) {
                    case 0: kprep(IC<0>()); break;
                    case 1: kprep(IC<1>()); break;
                    case 2: kprep(IC<2>()); break;
                    default: kprep(IC<3>()); break;
                }
                if (w4 == 3) {   // beta e^gamma r, r e^{gamma_L - gamma}, e^{gamma_L} for the chain
                    const float gi = sg[lane], gl = sg[63], ri = sr[lane];
                    po.bgr[lane] = sb[lane] * fast_exp2(gi) * ri;
                    po.kf[lane] = ri * fast_exp2(gl - gi);
                    if (lane == 0) po.decay = fast_exp2(gl);
                }
                // D_w = (I + A_w,w)^-1 by column-oriented forward substitution,
                // lane = column of D: once x_m is final it updates every later
                // row, so each step has up to 15 independent updates.  Columns
                // of A stream in a few steps ahead of their use.
                if (grp == 0) {
                    const float *AT = s.adiag[w4];
                    const int cc = l16;
                    constexpr int PF = 3;
                    float x[16];
                    f32x4 col[15][4];
                    auto load_col = [&](int m) {
#pragma unroll
                        for (int c4 = (m + 1) / 4; c4 < 4; ++c4) col[m][c4] = *(const f32x4 *)&AT[20 * m + 4 * c4];
                    };
#pragma unroll
                    for (int m = 0; m < PF; ++m) load_col(m);
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[r] = (r == cc) ? 1.f : 0.f;
#pragma unroll
                    for (int m = 0; m < 15; ++m) {
                        if (m + PF < 15) load_col(m + PF);
#pragma unroll
                        for (int r = m + 1; r < 16; ++r) x[r] -= col[m][r >> 2][r & 3] * x[m];
                        asm volatile("" ::: "memory");
                    }
                    // column cc of D is row cc of D^T: two 16-byte stores
                    v8 d0, d1;
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        d0[r] = (E)x[r];
                        d1[r] = (E)x[8 + r];
                    }
                    *(v8 *)&po.dt[w4][cc][0] = d0;
                    *(v8 *)&po.dt[w4][cc][8] = d1;
                }
            }
            lds_barrier();
        }
        return;
    }

    // ============================== chain ====================================
    // The chain is the serial part: it takes the SIMD's issue slots first, the
    // prep waves fill the gaps.
    __builtin_amdgcn_s_setprio(3);
    // transpose reads of K^T for state tile mt: lane (l16, grp) addresses token
    // row r0 + 4 grp + l16/4, key dims kappa(mt, 4 (l16 % 4)) .. +3
    int to[KT / 2];
    {
        const int rr = 4 * grp + (l16 >> 2), sw = swz<NSK>(rr);
#pragma unroll
        for (int m2 = 0; m2 < KT / 2; ++m2) to[m2] = rr * KROW + (((4 * m2 + (l16 & 3)) ^ sw) << 4);
    }
    // transpose read of the v tile: token row 16 ti + 4 grp + l16/4, value
    // columns c0 + 4 (l16 % 4) .. +3 of this wave's 16 columns
    const int c0 = 16 * w4;
    const int vo = (4 * grp + (l16 >> 2)) * VROW +
                   (((2 * w4 + ((l16 & 3) >> 1)) ^ swz<NSV>(4 * grp + (l16 >> 2))) << 4) + 8 * (l16 & 1);

    f32x4 h[KT];
    size_t sbase = ((size_t)n * p.HV + j) * K * V + vcol0;
    bool s_in = p.initial_state != nullptr, s_out = p.final_state != nullptr;
    if (POOL && p.state_indices) {   // state pool: the slot of sequence n (outside the pool: none)
        const int slot = p.state_indices[n];
        const bool ok = slot >= 0 && slot < p.pool_size;
        s_in = s_in && ok;
        s_out = s_out && ok;
        sbase = ((size_t)(ok ? slot : 0) * p.HV + j) * K * V + vcol0;
    }
    if (POOL && s_in && p.state_bf16) {
        const bf16 *__restrict__ s0 = (const bf16 *)p.initial_state + sbase;
#pragma unroll
        for (int mt = 0; mt < KT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) h[mt][e] = to_f(s0[(size_t)kappa(mt, 4 * grp + e) * V + c0 + l16]);
    } else if (s_in) {
        const float *__restrict__ s0 = p.initial_state + sbase;
#pragma unroll
        for (int mt = 0; mt < KT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) h[mt][e] = s0[(size_t)kappa(mt, 4 * grp + e) * V + c0 + l16];
    } else {
#pragma unroll
        for (int mt = 0; mt < KT; ++mt) h[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Z = K h and (Q h)^T of the next chunk, carried across the barrier.
    f32x4 zk[4], zq[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        zk[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        zq[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int c = -1; c < nchunks; ++c) {
        const int cn = c + 1;
        if (c >= 0) {
            const PrepOut &po = s.po[c & 1];
            const char *kb = (const char *)s.kb[c % 3];
            const char *vb = (const char *)s.vb[c % 3];
            const int64_t t0 = tok0 + 64LL * c;
            const int L = min(64, len - 64 * c);
            // X = diag(beta) V - diag(beta e^gamma r) Z
            f32x4 xz[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const v4 vv = tr(vb + vo + 16 * ti * VROW);
                const int r0 = 16 * ti + 4 * grp;
                const f32x4 be = *(const f32x4 *)&po.beta[r0];
                const f32x4 bgr = *(const f32x4 *)&po.bgr[r0];
#pragma unroll
                for (int e = 0; e < 4; ++e) xz[ti][e] = be[e] * (float)vv[e] - bgr[e] * zk[ti][e];
            }
            // V_new by block forward substitution, right-looking: as soon as
            // block m is final it is applied to every later block, so the
            // updates of different blocks overlap and only one product per block
            // sits on the dependency chain.
            v4 vb16[4];
            f32x4 vnf[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                v4 rbv;
#pragma unroll
                for (int e = 0; e < 4; ++e) rbv[e] = (E)xz[m][e];
                // D_m (row l16, columns 4 grp..+3) by a transpose read of D_m^T
                const v4 dfr = tr(&po.dt[m][4 * grp + (l16 >> 2)][4 * (l16 & 3)]);
                vnf[m] = mma_k16(dfr, rbv, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int e = 0; e < 4; ++e) vb16[m][e] = (E)vnf[m][e];
#pragma unroll
                for (int bi = m + 1; bi < 4; ++bi)
                    xz[bi] = mma_k16(*(const v4 *)&po.alo[16 * bi + l16][16 * m + 4 * grp], vb16[m], xz[bi]);
            }
            // V_new for the output product, diag(kf) V_new for the state
            v8 vnb[2], vkb[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const f32x4 k0 = *(const f32x4 *)&po.kf[32 * s2 + 4 * grp];
                const f32x4 k1 = *(const f32x4 *)&po.kf[32 * s2 + 16 + 4 * grp];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vnb[s2][e] = vb16[2 * s2][e];
                    vnb[s2][4 + e] = vb16[2 * s2 + 1][e];
                    vkb[s2][e] = (E)(k0[e] * vnf[2 * s2][e]);
                    vkb[s2][4 + e] = (E)(k1[e] * vnf[2 * s2 + 1][e]);
                }
            }
            // O^T tiles [value][token]: (Q h)^T scaled by scale rho e^gamma per
            // token, plus (P V_new)^T; and h <- e^{gamma_L} h + K^T diag(kf) V_new
            // (K^T by transpose loads).  The two are independent, so they sit in
            // one branch-free block and the scheduler interleaves them.
            f32x4 o[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const int i = 16 * ti + l16;
                o[ti] = zq[ti] * (p.scale * po.rq[i] * fast_exp2(po.gam[i]));
#pragma unroll
                for (int s2 = 0; s2 <= ti / 2; ++s2) o[ti] = mma(vnb[s2], *(const v8 *)&po.p[i][pcol(2 * s2, grp)], o[ti]);
            }
            const float dec = po.decay;
#pragma unroll
            for (int mt = 0; mt < KT; ++mt) {
                f32x4 acc = h[mt] * dec;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const char *pa = kb + to[mt >> 1] + 8 * (mt & 1) + 32 * s2 * KROW;
                    const v4 a0 = tr(pa), a1 = tr(pa + 16 * KROW);
                    v8 a;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a[e] = a0[e];
                        a[4 + e] = a1[e];
                    }
                    acc = mma(a, vkb[s2], acc);
                }
                h[mt] = acc;
            }
            E *dst = og + ((size_t)t0 * p.HV + j) * V + vcol0 + c0 + 4 * grp;
            const size_t orow = (size_t)p.HV * V;
            if (L == 64) {
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    v4 ov;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = (E)o[ti][e];
                    *(v4 *)__builtin_assume_aligned(dst + (16 * ti + l16) * orow, 8) = ov;
                }
            } else {
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    if (16 * ti + l16 < L) {
                        v4 ov;
#pragma unroll
                        for (int e = 0; e < 4; ++e) ov[e] = (E)o[ti][e];
                        *(v4 *)__builtin_assume_aligned(dst + (16 * ti + l16) * orow, 8) = ov;
                    }
                }
            }
        }
        if (cn < nchunks) {
            // Z = K h and (Q h)^T of chunk cn with the updated state
            const E *kb = s.kb[cn % 3], *qb = s.qb[cn & 1];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                zk[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                zq[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) {
                v8 hb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hb[e] = (E)h[2 * s2][e];
                    hb[4 + e] = (E)h[2 * s2 + 1][e];
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    zk[t] = mma(frag(kb, t, s2), hb, zk[t]);
                    zq[t] = mma(hb, frag(qb, t, s2), zq[t]);
                }
            }
        }
        lds_barrier();
    }

    if (POOL && s_out && p.state_bf16) {
        bf16 *__restrict__ sf = (bf16 *)p.final_state + sbase;
#pragma unroll
        for (int mt = 0; mt < KT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) sf[(size_t)kappa(mt, 4 * grp + e) * V + c0 + l16] = (bf16)h[mt][e];
    } else if (s_out) {
#pragma unroll
        for (int mt = 0; mt < KT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.final_state[sbase + (size_t)kappa(mt, 4 * grp + e) * V + c0 + l16] = h[mt][e];
    }
}

template <bool GATED, bool POOL>
hipError_t launch_ws_kv(const Params &p, unsigned grid, hipStream_t st) {
    if (p.K == 64 && p.V == 64) fused_ws_kernel<64, 64, GATED, POOL><<<grid, 768, 0, st>>>(p);
    else if (p.K == 64 && p.V == 128) fused_ws_kernel<64, 128, GATED, POOL><<<grid, 768, 0, st>>>(p);
    else if (p.K == 128 && p.V == 64) fused_ws_kernel<128, 64, GATED, POOL><<<grid, 768, 0, st>>>(p);
    else fused_ws_kernel<128, 128, GATED, POOL><<<grid, 768, 0, st>>>(p);
    return hipGetLastError();
}

}  // namespace

// One workgroup of 768 threads per (sequence, value head, 64 value columns).
hipError_t launch_fused_ws(const Params &p, hipStream_t st) {
    constexpr int VW = 64;
    const int groups = p.N * p.H;
    if (groups == 0) return hipSuccess;
    const int per_group = (p.HV / p.H) * (p.V / VW);
    const unsigned grid = (unsigned)((groups + 7) / 8) * 8 * per_group;
    const bool gated = p.gates.A_log != nullptr, pool = p.state_indices != nullptr || p.state_bf16;
    if (gated && pool) return launch_ws_kv<true, true>(p, grid, st);
    if (gated) return launch_ws_kv<true, false>(p, grid, st);
    if (pool) return launch_ws_kv<false, true>(p, grid, st);
    return launch_ws_kv<false, false>(p, grid, st);
}

}  // namespace gdn
