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
//   waves 4-7   K-prep waves, one chunk ahead: gate cumsum; wave w computes
//               its diagonal K K^T tile (A_ww and the diagonal-block inverse
//               D_w), two off-diagonal tiles (the gated -A tiles) and the
//               diagonal tiles whose norms those need, spread so that the four
//               waves carry 5, 5, 5 and 1 tiles; each publishes the per-token
//               state factors of its own 16 rows.
//   waves 8-11  Q-prep waves, one chunk ahead: the asynchronous copies of the
//               raw rows (two chunks ahead), gate cumsum, the ten causal Q K^T
//               tiles spread 7, 7, 7 and 3 tiles per wave (with the Q Q^T and
//               K K^T diagonals for the norms they need), the gated P tiles.
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
    float beta[64];
    float bgr[64];            // beta e^gamma r
    float osc[64];            // output scale of (Q h)^T: scale rho e^gamma
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
    float adiag[4][16 * 20];  // per K-prep wave: its diagonal block of A, fp32, by column: A_ij at 20 j + 4 (i % 4) + i / 4
    float stk[4][3][64];      // per K-prep wave: gamma, beta, r of the chunk being prepared
    float stq[4][2][64];      // per Q-prep wave: gamma, r of the chunk being prepared
    float ra[2][64], rb[2][64];  // in-kernel gating: raw gate words by chunk parity (unused otherwise)
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
    typedef WsLds<K, 64> Lds;
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
    const size_t kq_row = (size_t)p.H * K, v_row = (POOL && p.v_zero) ? 0 : (size_t)p.HV * V;

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
                // The ten causal tiles of Q K^T, spread so that no wave waits for
                // another inside the step; each wave also computes the diagonal
                // tiles of Q Q^T and K K^T for the norms its tiles need:
                //   wave 0: rows 0, 1 (tiles (0,0) (1,0) (1,1));  wave 1: row 2;
                //   wave 2: (3,0) (3,1) (3,2);  wave 3: (3,3)
                // (7, 7, 7 and 3 tiles, against 3, 5, 7 and 9 for whole row tiles).
                // Tiles are transposed: C[j][i] = k_j . q_i.
                auto qprep = [&](auto w_c) {
                    constexpr int W = decltype(w_c)::value;
                    constexpr int R0 = W == 0 ? 0 : W == 1 ? 2 : 3, R1 = W == 0 ? 1 : W == 1 ? 2 : 3;
                    constexpr int J0 = W == 3 ? 3 : 0, J1 = W == 0 ? 1 : W == 3 ? 3 : 2;
                    constexpr int NR = R1 - R0 + 1, NJ = J1 - J0 + 1;
                    f32x4 gq[NR][NJ], gd[NJ], gqq[NR];
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        gqq[r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int jj = 0; jj < NJ; ++jj) gq[r][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
                    }
#pragma unroll
                    for (int jj = 0; jj < NJ; ++jj) gd[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) {
                        v8 fk[NJ], bq[NR];
#pragma unroll
                        for (int jj = 0; jj < NJ; ++jj) fk[jj] = frag(kb, J0 + jj, s2);
#pragma unroll
                        for (int r = 0; r < NR; ++r) bq[r] = frag(qb, R0 + r, s2);
#pragma unroll
                        for (int jj = 0; jj < NJ; ++jj) {
                            gd[jj] = mma(fk[jj], fk[jj], gd[jj]);
#pragma unroll
                            for (int r = 0; r < NR; ++r)
                                if (J0 + jj <= R0 + r) gq[r][jj] = mma(fk[jj], bq[r], gq[r][jj]);
                        }
#pragma unroll
                        for (int r = 0; r < NR; ++r) gqq[r] = mma(bq[r], bq[r], gqq[r]);
                    }
                    // norms of the k rows of tiles J0..J1 from the diagonals: lane
                    // (l16, l16 / 4) holds row l16 at e = l16 % 4
                    {
                        const int e = l16 - 4 * grp;
                        if (e >= 0 && e < 4) {
#pragma unroll
                            for (int jj = 0; jj < NJ; ++jj)
                                sr[16 * (J0 + jj) + l16] = p.use_l2norm ? rsqrtf(gd[jj][e] + 1e-6f) : 1.f;
                        }
                    }
                    float rho[NR];
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        const float qq = __shfl(gqq[r][l16 & 3], (l16 >> 2) * 16 + l16);
                        rho[r] = p.use_l2norm ? rsqrtf(qq + 1e-6f) : 1.f;
                    }
                    wave_lds_sync();   // the staged gamma and r come from other lanes
                    f32x4 gj[NJ], rj[NJ];
#pragma unroll
                    for (int jj = 0; jj < NJ; ++jj) {
                        gj[jj] = *(const f32x4 *)&sg[16 * (J0 + jj) + 4 * grp];
                        rj[jj] = *(const f32x4 *)&sr[16 * (J0 + jj) + 4 * grp];
                    }
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        const int itq = R0 + r, iq = 16 * itq + l16;
                        const float giq = sg[iq], srq = p.scale * rho[r];
                        if (W != 2 && grp == 0) po.osc[iq] = srq * fast_exp2(giq);   // row 3: wave 3 publishes
#pragma unroll
                        for (int jj = 0; jj < NJ; ++jj) {
                            const int jt = J0 + jj;
                            if (jt > itq) continue;
                            v4 o;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float v = srq * rj[jj][e] * fast_exp2(giq - gj[jj][e]) * gq[r][jj][e];
                                o[e] = (E)((jt < itq || iq >= 16 * jt + 4 * grp + e) ? v : 0.f);
                            }
                            *(v4 *)&po.p[iq][pcol(jt, grp)] = o;
                        }
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
                    if (w4 == 0) po.beta[lane] = b;
                }
                const E *kb = s.kb[cn % 3];
                // The ten lower Gram tiles of K K^T are spread so that no wave
                // waits for another inside the step: wave W computes its own
                // diagonal tile (for A_WW and D_W), two off-diagonal tiles (i, j)
                // and the further diagonal tiles whose norms those need:
                //   W = 0: (1,0) (2,0), diagonals 0 1 2;  W = 1: (2,1) (3,1), 1 2 3;
                //   W = 2: (3,0) (3,2), diagonals 0 2 3;  W = 3: diagonal 3 only
                // (5, 5, 5 and 1 tiles, against 1, 3, 5 and 7 for whole row tiles).
                // Tiles are transposed: C[j][i] = k_j . k_i.
                auto kprep = [&](auto w_c) {
                    constexpr int W = decltype(w_c)::value;
                    constexpr int NOFF = W == 3 ? 0 : 2;
                    constexpr int OI0 = W == 0 ? 1 : W == 1 ? 2 : 3, OJ0 = W == 0 ? 0 : W == 1 ? 1 : 0;
                    constexpr int OI1 = W == 0 ? 2 : 3, OJ1 = W == 0 ? 0 : W == 1 ? 1 : 2;
                    constexpr int DM = W == 0 ? 0x7 : W == 1 ? 0xE : W == 2 ? 0xD : 0x8;
                    f32x4 gd[4], go[2];
#pragma unroll
                    for (int t = 0; t < 4; ++t) gd[t] = f32x4{0.f, 0.f, 0.f, 0.f};
                    go[0] = go[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) {
                        v8 fk[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            if (DM >> t & 1) fk[t] = frag(kb, t, s2);
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            if (DM >> t & 1) gd[t] = mma(fk[t], fk[t], gd[t]);
                        if (NOFF > 0) {
                            go[0] = mma(fk[OJ0], fk[OI0], go[0]);
                            go[1] = mma(fk[OJ1], fk[OI1], go[1]);
                        }
                    }
                    // norms of the rows of the computed diagonal tiles: lane
                    // (l16, l16 / 4) holds row l16 at e = l16 % 4
                    {
                        const int e = l16 - 4 * grp;
                        if (e >= 0 && e < 4) {
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                if (DM >> t & 1) sr[16 * t + l16] = p.use_l2norm ? rsqrtf(gd[t][e] + 1e-6f) : 1.f;
                        }
                    }
                    wave_lds_sync();   // the staged gamma / beta / r come from other lanes
                    {   // diagonal tile -> A_WW (fp32, by column).  The raw Gram tile
                        // is symmetric, so the lane's values serve as rows i = 4 grp + e
                        // (of the tile) of column j = l16.  Rows are stored in the
                        // order the solve's lanes take them (i % 4 major), so that
                        // each solve step reads one vector.
                        const f32x4 gw = *(const f32x4 *)&sg[16 * W + 4 * grp];
                        const f32x4 rw = *(const f32x4 *)&sr[16 * W + 4 * grp];
                        const f32x4 bw = *(const f32x4 *)&sb[16 * W + 4 * grp];
                        const int ik = 16 * W + l16;
                        const float gik = sg[ik], rik = sr[ik];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float v = bw[e] * rw[e] * rik * fast_exp2(gw[e] - gik) * gd[W][e];
                            s.adiag[W][20 * l16 + 4 * e + grp] = (4 * grp + e > l16) ? v : 0.f;
                        }
                    }
                    // off-diagonal tiles (i, j) -> -A (bf16): row 16 i + l16,
                    // columns 16 j + 4 grp + e
                    auto off = [&](auto oi_c, auto oj_c, const f32x4 &g) {
                        constexpr int OI = decltype(oi_c)::value, OJ = decltype(oj_c)::value;
                        const int ik = 16 * OI + l16;
                        const float gik = sg[ik], bri = sb[ik] * sr[ik];
                        const f32x4 gj = *(const f32x4 *)&sg[16 * OJ + 4 * grp];
                        const f32x4 rj = *(const f32x4 *)&sr[16 * OJ + 4 * grp];
                        v4 o;
#pragma unroll
                        for (int e = 0; e < 4; ++e) o[e] = (E)(-(bri * rj[e] * fast_exp2(gik - gj[e]) * g[e]));
                        *(v4 *)&po.alo[ik][16 * OJ + 4 * grp] = o;
                    };
                    if constexpr (NOFF > 0) {
                        off(IC<OI0>(), IC<OJ0>(), go[0]);
                        off(IC<OI1>(), IC<OJ1>(), go[1]);
                    }
                    // beta e^gamma r, r e^{gamma_L - gamma} for the rows of tile W,
                    // e^{gamma_L} (wave 0), for the chain
                    if (grp == 0) {
                        const int i = 16 * W + l16;
                        const float gi = sg[i], gl = sg[63], ri = sr[i];
                        po.bgr[i] = sb[i] * fast_exp2(gi) * ri;
                        po.kf[i] = ri * fast_exp2(gl - gi);
                        if (W == 0 && l16 == 0) po.decay = fast_exp2(gl);
                    }
                    wave_lds_sync();   // A_WW is read back across lanes by the solve
                };
                switch (w4) {
                    case 0: kprep(IC<0>()); break;
                    case 1: kprep(IC<1>()); break;
                    case 2: kprep(IC<2>()); break;
                    default: kprep(IC<3>()); break;
                }
                // D_w = (I + A_w,w)^-1 by column-oriented forward substitution
                // with every lane busy: the four lanes of quad c hold column c
                // of D, lane g of the quad rows g, g+4, g+8, g+12.  Once x_m is
                // final it is broadcast inside each quad (one DPP move) and
                // updates every row; A being strictly lower, the rows at or
                // above m take zeros, so each step is four branch-free FMAs.
                {
                    const float *AT = s.adiag[w4];
                    const int cc = lane >> 2, gg = lane & 3;
                    float x[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) x[q] = (4 * q + gg == cc) ? 1.f : 0.f;
                    f32x4 col[16];
#pragma unroll
                    for (int m = 0; m < 15; ++m) col[m] = *(const f32x4 *)&AT[20 * m + 4 * gg];
                    auto bcast = [&](auto m_c) {   // x_m from lane m % 4 of the quad
                        constexpr int m = decltype(m_c)::value, sl = m % 4;
                        return dpp_mov<sl | (sl << 2) | (sl << 4) | (sl << 6), 0xf>(x[m / 4]);
                    };
                    auto step = [&](auto m_c) {
                        constexpr int m = decltype(m_c)::value;
                        const float xm = bcast(m_c);
#pragma unroll
                        for (int q = 0; q < 4; ++q) x[q] -= col[m][q] * xm;
                    };
                    step(IC<0>()); step(IC<1>()); step(IC<2>()); step(IC<3>()); step(IC<4>());
                    step(IC<5>()); step(IC<6>()); step(IC<7>()); step(IC<8>()); step(IC<9>());
                    step(IC<10>()); step(IC<11>()); step(IC<12>()); step(IC<13>()); step(IC<14>());
                    // column cc of D is row cc of D^T
#pragma unroll
                    for (int q = 0; q < 4; ++q) po.dt[w4][cc][4 * q + gg] = (E)x[q];
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
    size_t sbase = ((size_t)n * p.HV + j) * K * V + vcol0, sbase_in = sbase;
    bool s_in = p.initial_state != nullptr, s_out = p.final_state != nullptr;
    if (POOL && p.state_indices) {   // state pool: the slot of sequence n (outside the pool: none)
        const int slot = p.state_indices[n];
        const bool ok = slot >= 0 && slot < p.pool_size;
        s_in = s_in && ok;
        s_out = s_out && ok;
        sbase = sbase_in = ((size_t)(ok ? slot : 0) * p.HV + j) * K * V + vcol0;
    }
    if (POOL && p.init_shared) sbase_in = (size_t)j * K * V + vcol0;   // one initial state for all
    if (POOL && s_in && p.state_bf16) {
        const bf16 *__restrict__ s0 = (const bf16 *)p.initial_state + sbase_in;
#pragma unroll
        for (int mt = 0; mt < KT; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) h[mt][e] = to_f(s0[(size_t)kappa(mt, 4 * grp + e) * V + c0 + l16]);
    } else if (s_in) {
        const float *__restrict__ s0 = p.initial_state + sbase_in;
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
                o[ti] = zq[ti] * po.osc[i];
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
    const bool gated = p.gates.A_log != nullptr,
               pool = p.state_indices != nullptr || p.state_bf16 || p.v_zero || p.init_shared;
    if (gated && pool) return launch_ws_kv<true, true>(p, grid, st);
    if (gated) return launch_ws_kv<true, false>(p, grid, st);
    if (pool) return launch_ws_kv<false, true>(p, grid, st);
    return launch_ws_kv<false, false>(p, grid, st);
}

}  // namespace gdn
