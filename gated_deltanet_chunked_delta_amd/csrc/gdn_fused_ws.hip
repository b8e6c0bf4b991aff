// Warp-specialized fused forward pass (bf16) for gfx950.
//
// Same mathematics as the single-role kernel in gdn_fused.hip (the step list
// of the page "NPU Training Operators - GDN", operator-semantics section, in
// the chunk form written out at the top of that file), scheduled differently:
// a workgroup has 12 waves, three per SIMD, in two or three roles.
//   chain waves: each owns 16 state columns and runs everything that depends
//               on the state h: the block forward substitution for V_new, the
//               output, the state update, and Z = K h and (Q h)^T of the next
//               chunk.
//   K-prep work, one chunk ahead, four row tiles w: gate cumsum; tile w's
//               diagonal K K^T tile (A_ww and the diagonal-block inverse D_w),
//               two off-diagonal tiles (the gated -A tiles) and the diagonal
//               tiles whose norms those need, spread so that the four carry 5,
//               5, 5 and 1 tiles; the per-token state factors of its 16 rows.
//   Q-prep work, one chunk ahead, four row tiles w: gate cumsum, the ten
//               causal Q K^T tiles spread 7, 7, 7 and 3 tiles per tile w (with
//               the Q Q^T and K K^T diagonals for the norms they need), the
//               gated P tiles.
// Two layouts (NCW chain waves):
//   NCW = 4: a workgroup per (sequence, value head, 64 value columns); waves
//            0-3 chain, 4-7 K-prep, 8-11 Q-prep.  Used when there are few
//            (sequence, value head) pairs, so that the grid fills the GPU.
//   NCW = 8: a workgroup per (sequence, value head) of 128 columns; waves 0-7
//            chain (two per SIMD, so that each hides the other's latencies),
//            8-11 prep waves doing both the K- and the Q-prep of their row
//            tile, once for all 128 columns.
// The prep waves also issue the asynchronous copies of the raw k and q rows
// and of the gates two chunks ahead; each chain wave copies its own v columns
// one chunk ahead.  The SIMDs interleave the
// serial state chain of chunk c with the preparation of chunk c+1.  Each step
// ends with the only workgroup barrier of the step; every prep wave computes
// the cumsum and norm values it needs itself, so the prep waves never wait for
// each other inside a step.
//
// Gate and norm factors travel as base-2 logarithms: with gamma the gate
// cumsum in log2 units and l_i = log2 r_i (the L2-norm factor of k_i, 0 when
// the norm is off),
//   A_ij = 2^(a_i - c_j) k_i.k_j,       a_i = gamma_i + log2 beta_i + l_i,
//   P_ij = 2^(a'_i - c_j) q_i.k_j,      a'_i = gamma_i + log2(scale rho_i),
//                                       c_j = gamma_j - l_j,
// so each gated element costs one subtraction and one exp2; beta = 0 gives
// a_i = -inf and a zero row.  The same factors give the per-token scalars:
// beta e^gamma r = 2^a_i, r e^{gamma_L - gamma} = 2^(gamma_L - c_i) and
// scale rho e^gamma = 2^a'_i.
//
// The diagonal-block inverses are published in three forms, D_b,
// D_b diag(beta) and -D_b diag(beta e^gamma r), so that the chain forms
//   V_b = D_b diag(beta) V_b - D_b diag(beta e^gamma r) Z_b
//         + D_b (-sum_{m<b} A_bm V_m)      (= D_b (X_b - sum A_bm V_m))
// entirely on the matrix cores, from the raw v rows and Z = K h.
//
// Buffers: raw k rows in a ring of three chunks (the chain reads chunk c's
// while c+1's is resident and c+2's streams in), raw q/g/beta, v and the prep
// outputs double-buffered by chunk parity.  Rows past the end of a sequence
// are copies of its last row; the cumsum reads their g and beta as 0, which
// makes their rows of A and V_new zero and leaves gamma_L at the last real
// token, so they contribute nothing.
//
// In-kernel gating: the gate-copying wave fetches the raw gate words of chunk
// c+3 (their own ring) and, at the start of the next step, turns those of
// chunk c+2 into g and beta in the g/beta ring, so every gate is computed once
// and off the step's barrier-to-barrier path.
#include <stddef.h>

#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Asynchronous global -> LDS copies: lane l's bytes land at lds + l * size.
// They are issued from inline assembly on purpose: the compiler does not track
// them, so it neither waits for them before unrelated LDS reads nor at the
// LDS fences of the barriers.  The code that consumes a copy waits for it
// explicitly (wait_vmem, then a barrier).  Vector memory counters retire in
// order, so the compiler's own counter waits stay correct (at worst they wait
// longer).
// lds_copy16s: 16 bytes per lane from a wave-uniform 64-bit base address plus
// a 32-bit per-lane byte offset (no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void lds_copy16s(const void *base, unsigned off, unsigned lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds) : "memory", "m0");
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

// XOR swizzle of the 16-byte segments of a row of NSEG segments.  Rows of 16
// segments (256 bytes) are swizzled in row pairs: rows 2x and 2x+1 take
// segments 2 h(x) and 2 h(x) + 1 (XOR the segment index), so the two lanes of
// each pair of a 16-byte fragment read (rows 16 t + l16) read the two halves
// of one 32-byte block, the form of a 16-byte-per-lane read that runs without
// bank conflicts on gfx950 (measured: the previous bit-pair exchange took
// twice the LDS cycles); and h(x) = 2 ((x & 3) ^ (x >> 2)) + (x >> 2) keeps
// the transposing reads of K^T (lane quads reading segments 4 m + 0..3 of
// eight rows per half wave) spread over all sixteen segments.
template <int NSEG> __device__ __forceinline__ int swz(int row) {
    static_assert(NSEG == 8 || NSEG == 16, "row length");
    if constexpr (NSEG == 16) {
        const int x = (row >> 1) & 7, h = 2 * ((x & 3) ^ (x >> 2)) + (x >> 2);
        return 2 * h + (row & 1);
    } else {
        return (row >> 1) & 7;
    }
}

// fp32 -> bf16, round to nearest even, two values per conversion instruction
// (the pairs are joined as 32-bit words, which keeps the compiler from
// merging them into one four-wide conversion that it would split per value).
__device__ __forceinline__ bf16x4 cvt4(f32x4 x) {
    const f32x2 a = {x[0], x[1]}, b = {x[2], x[3]};
    const bf16x2 ra = __builtin_convertvector(a, bf16x2), rb = __builtin_convertvector(b, bf16x2);
    const u32x2 u = {__builtin_bit_cast(unsigned, ra), __builtin_bit_cast(unsigned, rb)};
    return __builtin_bit_cast(bf16x4, u);
}
// Byte offset of a ring slot, kept wave-uniform (a scalar register).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// 2^x by the hardware exponential; log2 by the hardware logarithm.
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Per-chunk results of the prep waves that the chain waves read.
struct alignas(16) PrepOut {
    // -A in the six 16x16 blocks below the diagonal, block (i, m) at
    // i (i - 1) / 2 + m; element (r, 4 g + e) of a block at [g][r][e], so that
    // the 8-byte operand reads (lane: row l16, columns 4 grp ..) are linear
    bf16 alo[6][4][16][4];
    bf16 pp[3072];            // P by row pairs (see pel), columns in the key-slot order (see pcol)
    bf16 dt[3][4][16][16];    // transposed D_b, D_b diag(beta), -D_b diag(beta e^gamma r)
    float osc[64];            // output scale of (Q h)^T: scale rho e^gamma
    float kf[64];             // r e^{gamma_L - gamma}
    float decay;              // e^{gamma_L}
};
__device__ __forceinline__ constexpr int alo_blk(int i, int m) { return i * (i - 1) / 2 + m; }
// Element (i, col) of P.  Rows go in pairs: the 16-byte column units j of
// rows 2p and 2p+1 sit side by side, so that the two lanes of a pair read one
// 32-byte block; rows 0-31 keep the first four units (32 columns), rows 32-63
// all eight (blocks (0,1) and (2,3) are zero); the unit index is XOR-swizzled
// by the pair index so that the eight pairs of a 16-lane read hit different
// banks.
template <typename PO> __device__ __forceinline__ auto pel(PO &po, int i, int col) {
    const int p = i >> 1, j = col >> 3;
    const int e = i < 32 ? p * 64 + 16 * (j ^ ((p >> 1) & 3)) : 1024 + (p - 16) * 128 + 16 * (j ^ (p & 7));
    return &po.pp[e + 8 * (i & 1) + (col & 7)];
}

// Column of token j in P (PrepOut::pp).  The output product reads P as the B
// operand of a 16x16x32 product whose lane-group g holds tokens
// 32 s + 4 g + e and 32 s + 16 + 4 g + e (e = 0..3); storing those eight
// columns next to each other makes each operand one 16-byte read.
__device__ __forceinline__ constexpr int pcol(int jt, int g) {   // first column of tile jt, group g
    return 32 * (jt >> 1) + 8 * g + 4 * (jt & 1);
}

template <int K, int VW> struct WsLds {
    bf16 kb[3][64 * K];       // raw k rows (swizzled), ring of three chunks
    bf16 qb[2][64 * K];       // raw q rows (swizzled)
    bf16 vb[2][64 * VW];      // raw v rows by chunk parity: per chain wave its 64 x 16 columns, row-major
    float gb[2][64], bb[2][64];
    PrepOut po[2];
    float adiag[4][16 * 16];  // per K-prep wave: its diagonal block of A, fp32, by column: A_ij at 16 j + i
    float stk[4][4][64];      // per K-prep wave: gamma + log2 beta, gamma, log2 r, beta of the chunk being prepared
    float stq[4][4][64];      // per Q-prep wave: the same (the first and last unused)
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
template <int K, int V, int NCW, bool GATED, bool POOL, bool OUT>
__global__ void __launch_bounds__(768) fused_ws_kernel(Params p) {
    typedef bf16 E;
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    typedef __attribute__((address_space(3))) bf16x4 lds_v4;
    constexpr int VW = 16 * NCW, VEC = 8;   // value columns per workgroup
    constexpr bool MERGED = NCW == 8;       // four prep waves do both K- and Q-prep
    static_assert((NCW == 4 || NCW == 8) && V % VW == 0, "layout");
    typedef WsLds<K, VW> Lds;
    constexpr int NSK = K / VEC;
    constexpr int KT = K / 16, KS = K / 32;
    constexpr int KROW = 2 * K, VROW = 2 * VW;   // bytes per raw row in LDS
    static_assert(sizeof(Lds) <= 160 * 1024, "LDS budget");
    __shared__ Lds s;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // 0 chain, 1 K-prep, 2 Q-prep, 3 both preps
    const int role = wave < NCW ? 0 : MERGED ? 3 : (wave >> 2);
    const int w4 = wave & 3;      // prep: row tile, and index among the four copying waves
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
    // sequence n (longest first when the batch is packed and ordered), key head jk
    const int n = p.seq_order ? p.seq_order[group / p.H] : group / p.H, jk = group % p.H;
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
    // OUT = false (with POOL only): no output.  The sequence split's state and
    // transfer-map passes need only the final states, so the q rows, the P
    // tiles, (Q h)^T and the output product are skipped.
    static_assert(OUT || POOL, "the no-output variant is a pool variant");
    constexpr bool want_o = OUT;

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
    const float l2_scale = fast_log2(p.scale);

    const unsigned lds0 = (unsigned)(size_t)(lds_void *)&s;
    // raw k/q fragment of row tile t, step s2: row 16 t + l16, key slots
    // 32 s2 + 8 grp .. +7 (one swizzled 16-byte segment); byte offsets from the
    // start of a chunk's rows
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

    // ---- asynchronous copies ------------------------------------------------
    // Raw k and q rows are copied by the four K-prep and the four Q-prep waves
    // (NCW = 4), or by the prep wave with w4 = 3 alone (NCW = 8: its row tile
    // carries the least preparation work, and copies issued by the chain waves
    // stall them while the memory pipeline accepts a burst of eight waves'
    // copies); the gates by the prep wave with w4 = 3; each chain wave copies
    // its own v columns.  LDS
    // destinations are byte addresses (wave-uniform); the per-lane source
    // offsets inside a full chunk are fixed, only the last chunk of a
    // sequence clamps its rows.  Copy t of a chunk's rows moves 1 KB.
    constexpr int NCP = MERGED ? 1 : 4;          // waves sharing the copies of k (and of q)
    const int cpw = MERGED ? 0 : w4;             // this wave's index among them
    constexpr int NKQO = MERGED ? 1 : NSK / NCP;
    unsigned kqo[NKQO];   // byte offsets from the chunk's first row (NCP = 4)
#pragma unroll
    for (int i = 0; i < NKQO; ++i) {
        const int P = 64 * (cpw + NCP * i) + lane, row = P / NSK;
        kqo[i] = ((unsigned)row * (unsigned)kq_row + (((P % NSK) ^ swz<NSK>(row)) * VEC)) * sizeof(E);
    }
    // rows of k (or q) of chunk c into the LDS chunk slot at byte address dst
    auto issue_rows = [&](const E *src, int c, unsigned dst) {
        const int64_t t0 = tok0 + 64LL * c;
        const int last = min(64, len - 64 * c) - 1;
        const E *rc = src + (size_t)t0 * kq_row + (size_t)jk * K;
        if constexpr (NCP == 1) {
            // one wave copies all rows; its offsets are formed per copy instead
            // of being held in registers across the loop
#pragma unroll
            for (int t = 0; t < NSK; ++t) {
                const int P = 64 * t + lane, row = P / NSK, seg = (P % NSK) ^ swz<NSK>(row);
                lds_copy16s(rc, ((unsigned)min(row, last) * (unsigned)kq_row + seg * VEC) * sizeof(E), dst + 1024u * t);
            }
        } else if (last == 63) {
#pragma unroll
            for (int i = 0; i < NSK / NCP; ++i) lds_copy16s(rc, kqo[i], dst + 1024u * (cpw + NCP * i));
        } else {
#pragma unroll
            for (int i = 0; i < NSK / NCP; ++i) {
                const int t = cpw + NCP * i;
                const int P = 64 * t + lane, row = P / NSK, seg = (P % NSK) ^ swz<NSK>(row);
                lds_copy16s(rc, ((unsigned)min(row, last) * (unsigned)kq_row + seg * VEC) * sizeof(E), dst + 1024u * t);
            }
        }
    };
    auto issue_k = [&](int c) { issue_rows(kg, c, lds0 + offsetof(Lds, kb) + (c % 3) * (64 * K * 2)); };
    auto issue_q = [&](int c) { issue_rows(qg, c, lds0 + offsetof(Lds, qb) + (c & 1) * (64 * K * 2)); };
    // g and beta of chunk c (gates given as tensors; the gate-copying wave only)
    auto issue_gb = [&](int c) {
        if (!gated) {
            const int64_t t0 = tok0 + 64LL * c;
            const int last = min(64, len - 64 * c) - 1;
            const size_t o = (size_t)(t0 + min(lane, last)) * p.HV + j;
            lds_copy4(p.g + o, lds0 + offsetof(Lds, gb) + (c & 1) * 256);
            lds_copy4(p.beta + o, lds0 + offsetof(Lds, bb) + (c & 1) * 256);
        }
    };
    // raw gate words of chunk c (in-kernel gating; the gate-copying wave only):
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

    // the prep wave that copies (and, with raw inputs, computes) the gates
    const bool gate_wave = role == (MERGED ? 3 : 2) && w4 == 3;
    if (nchunks > 0) {
        if (MERGED ? gate_wave : role == 1) issue_k(0);
        if ((MERGED ? gate_wave : role == 2) && want_o) issue_q(0);
        if (gate_wave) {
            issue_gb(0);
            issue_gates(0);
            if (nchunks > 1) issue_gates(1);
        }
    }
    wait_vmem();
    if (gated && gate_wave) gate_chunk(0);
    // P blocks (0,1) and (2,3) are read by the output product but never
    // written by the epilogue: zero them once in both buffers.
    if (role == 0) {
#pragma unroll
        for (int q4 = 0; q4 < 16 / NCW; ++q4) {
            const int idx = 64 * NCW * q4 + tid, b2 = idx >> 9, blk = (idx >> 8) & 1, r = (idx >> 4) & 15, jj = idx & 15;
            *pel(s.po[b2], 32 * blk + r, pcol(2 * blk + 1, jj >> 2) + (jj & 3)) = (E)0.f;
        }
    }
    lds_barrier();

    // The three roles run separate loops with the same number of barriers, so
    // that none carries another's registers.
    // ============================ preparation ===============================
    // The work of row tile W for chunk cn: with DO_K the -A tiles, D_W (three
    // forms) and the state factors; with DO_Q the P tiles and the output
    // scale.  Tile assignment (tiles are transposed: C[j][i] = k_j . k_i or
    // k_j . q_i), spread so that no wave waits for another inside the step:
    //   K K^T: the diagonal tile W (for A_WW and D_W) and W = 0: (1,0) (2,0);
    //          W = 1: (2,1) (3,1);  W = 2: (3,0) (3,2);  W = 3: none
    //          (5, 5, 5 and 1 tiles, against 1, 3, 5 and 7 for whole rows);
    //   Q K^T: W = 0: rows 0, 1 ((0,0) (1,0) (1,1));  W = 1: row 2;
    //          W = 2: (3,0) (3,1) (3,2);  W = 3: (3,3);
    // and, with the L2 norm (NORM), the diagonal K K^T and Q Q^T tiles whose
    // norms those need.  With DO_K the diagonal tile W comes first, so that
    // the forward substitution for D_W (a chain of dependent steps) overlaps
    // the other products.
    auto prep_chunk = [&](auto w_c, auto k_c, auto q_c, auto n_c, int cn) {
        constexpr int W = decltype(w_c)::value;
        constexpr bool DO_K = decltype(k_c)::value != 0, DO_Q = decltype(q_c)::value != 0;
        constexpr bool NORM = decltype(n_c)::value != 0;
        constexpr int NOFF = (DO_K && W != 3) ? 2 : 0;
        constexpr int OI0 = W == 0 ? 1 : W == 1 ? 2 : 3, OJ0 = W == 0 ? 0 : W == 1 ? 1 : 0;
        constexpr int OI1 = W == 0 ? 2 : 3, OJ1 = W == 0 ? 0 : W == 1 ? 1 : 2;
        constexpr int R0 = W == 0 ? 0 : W == 1 ? 2 : 3, R1 = W == 0 ? 1 : W == 1 ? 2 : 3;
        constexpr int J0 = W == 3 ? 3 : 0, J1 = W == 0 ? 1 : W == 3 ? 3 : 2;
        constexpr int NR = DO_Q ? R1 - R0 + 1 : 0;
        constexpr int KDK = W == 0 ? 0x7 : W == 1 ? 0xE : W == 2 ? 0xD : 0x8;   // k tiles of the K work
        constexpr int KDQ = ((2 << J1) - 1) & ~((1 << J0) - 1);                // k tiles of the Q work
        constexpr int KD = (DO_K ? KDK : 0) | (DO_Q ? KDQ : 0);
        // k tiles whose fragments phase 2 loads (tile W's stay in registers from phase 1)
        constexpr int KL = DO_K ? (KD & ~(1 << W)) : KD;
        PrepOut &po = s.po[cn & 1];
        // staging of this wave: gamma + log2 beta, gamma, log2 r, beta by token
        float(*st)[64] = DO_K ? s.stk[w4] : s.stq[w4];
        float *sgb = st[0], *sg = st[1], *sl = st[2], *sb = st[3];
        // log2 r of token i, and of tokens i..i+3 (0 without the norm)
        auto lr = [&](int i) { return NORM ? sl[i] : 0.f; };
        auto lr4 = [&](int i) { return NORM ? *(const f32x4 *)&sl[i] : f32x4{0.f, 0.f, 0.f, 0.f}; };
        float gam, bt;   // this lane's token: gate cumsum (log2 units) and beta
        cumsum(cn, gam, bt);
        if constexpr (DO_K) {
            sgb[lane] = gam + fast_log2(bt);
            sb[lane] = bt;
        }
        sg[lane] = gam;
        const float gl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gam), 63));   // gamma_L
        const E *kb = (const E *)((const char *)s.kb[0] + uni((cn % 3) * 64 * KROW));
        const E *qb = (const E *)((const char *)s.qb[0] + uni((cn & 1) * 64 * KROW));
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        // lane (l16, l16 / 4) holds the diagonal entry of row l16 at e = l16 % 4
        const int ed = l16 - 4 * grp;
        const bool on_diag = ed >= 0 && ed < 4;

        // ---- phase 1 (DO_K): the diagonal tile W, A_WW, and the solve's operands
        v8 fkW[KS];
        f32x4 col[15];
        if constexpr (DO_K) {
            f32x4 gW = z4;
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) {
                fkW[s2] = frag(kb, W, s2);
                gW = mma(fkW[s2], fkW[s2], gW);
            }
            if (NORM && on_diag) sl[16 * W + l16] = -0.5f * fast_log2(gW[ed] + 1e-6f);
            wave_lds_sync();   // the staged factors come from other lanes
            {   // diagonal tile -> A_WW (fp32, by column).  The raw Gram tile is
                // symmetric, so the lane's values serve as rows i = 4 grp + e (of
                // the tile) of column j = l16: four consecutive entries.
                const f32x4 ai = *(const f32x4 *)&sgb[16 * W + 4 * grp] + lr4(16 * W + 4 * grp);
                const int jc = 16 * W + l16;
                const float cj = sg[jc] - lr(jc);
                f32x4 a;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = (4 * grp + e > l16) ? fast_exp2(ai[e] - cj) * gW[e] : 0.f;
                *(f32x4 *)&s.adiag[W][16 * l16 + 4 * grp] = a;
            }
            wave_lds_sync();   // A_WW is read back across lanes by the solve
        }

        // ---- phase 2: the other products, with the solve in between.  The
        // solve's 15 dependent steps are the prep's critical path; the chain
        // waves (priority 3) take the SIMD's issue slots first, so the K-side
        // prep raises its priority to 2 for this phase (wide and long 1-2 %
        // faster than at 0)
        if constexpr (DO_K) __builtin_amdgcn_s_setprio(2);
        f32x4 gd[4], go[2], gq[2][4], gqq[2];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            gd[t] = z4;
            gq[0][t] = gq[1][t] = z4;
        }
        go[0] = go[1] = gqq[0] = gqq[1] = z4;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            v8 fk[4], fq[2];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (KL >> t & 1) fk[t] = frag(kb, t, s2);
                else if (DO_K && t == W) fk[t] = fkW[s2];
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) fq[r] = frag(qb, R0 + r, s2);
            if constexpr (NORM) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (KL >> t & 1) gd[t] = mma(fk[t], fk[t], gd[t]);
            }
            if constexpr (NOFF > 0) {
                go[0] = mma(fk[OJ0], fk[OI0], go[0]);
                go[1] = mma(fk[OJ1], fk[OI1], go[1]);
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) {
#pragma unroll
                for (int jt = J0; jt <= J1; ++jt)
                    if (jt <= R0 + r) gq[r][jt] = mma(fk[jt], fq[r], gq[r][jt]);
                if constexpr (NORM) gqq[r] = mma(fq[r], fq[r], gqq[r]);
            }
        }
        // D_W = (I + A_WW)^-1 by column-oriented forward substitution with
        // every lane busy: the four lanes of quad cc hold column cc of D, lane
        // gg of the quad rows 4 gg .. 4 gg + 3.  Once x_m is final it is
        // broadcast inside each quad (one DPP move) and updates every row; A
        // being strictly lower, the rows at or above m take zeros, so each
        // step is four branch-free FMAs.
        float x[4];
        if constexpr (DO_K) {
            const int cc = lane >> 2, gg = lane & 3;
#pragma unroll
            for (int m = 0; m < 15; ++m) col[m] = *(const f32x4 *)&s.adiag[W][16 * m + 4 * gg];
#pragma unroll
            for (int q = 0; q < 4; ++q) x[q] = (4 * gg + q == cc) ? 1.f : 0.f;
            auto step = [&](auto m_c) {
                constexpr int m = decltype(m_c)::value, sl4 = m / 4;   // x_m from lane m / 4 of the quad
                const float xm = dpp_mov<sl4 | (sl4 << 2) | (sl4 << 4) | (sl4 << 6), 0xf>(x[m % 4]);
#pragma unroll
                for (int q = 0; q < 4; ++q) x[q] -= col[m][q] * xm;
            };
            step(IC<0>()); step(IC<1>()); step(IC<2>()); step(IC<3>()); step(IC<4>());
            step(IC<5>()); step(IC<6>()); step(IC<7>()); step(IC<8>()); step(IC<9>());
            step(IC<10>()); step(IC<11>()); step(IC<12>()); step(IC<13>()); step(IC<14>());
            // interleave the substitution's dependent steps with the products
            // above: one product, then four VALU instructions, in turn
            constexpr int NQ = DO_Q ? (W == 3 ? 1 : 3) : 0;
            constexpr int NM = KS * ((NORM ? __builtin_popcount(KL) + NR : 0) + NOFF + NQ);
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
        }
        if constexpr (DO_K) __builtin_amdgcn_s_setprio(0);
        // log2 of the norm factors of the other k rows this wave needs
        if constexpr (NORM) {
            if (on_diag) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (KL >> t & 1) sl[16 * t + l16] = -0.5f * fast_log2(gd[t][ed] + 1e-6f);
            }
        }
        float la[2];   // a'_i = gamma_i + log2(scale rho_i) of the lane's row in tile R0 + r
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            la[r] = l2_scale;
            if constexpr (NORM) {
                const float qq = __shfl(gqq[r][l16 & 3], (l16 >> 2) * 16 + l16);
                la[r] += -0.5f * fast_log2(qq + 1e-6f);
            }
        }
        if constexpr (NORM || !DO_K) wave_lds_sync();   // the staged factors come from other lanes
        if constexpr (DO_K) {
            // off-diagonal tiles (i, j) -> -A (bf16): row 16 i + l16, columns
            // 16 j + 4 grp + e
            auto off = [&](auto oi_c, auto oj_c, const f32x4 &g) {
                constexpr int OI = decltype(oi_c)::value, OJ = decltype(oj_c)::value;
                const int ik = 16 * OI + l16;
                const float ai = sgb[ik] + lr(ik);
                const f32x4 cj = *(const f32x4 *)&sg[16 * OJ + 4 * grp] - lr4(16 * OJ + 4 * grp);
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = -(fast_exp2(ai - cj[e]) * g[e]);
                *(v4 *)&po.alo[alo_blk(OI, OJ)][grp][l16][0] = cvt4(v);
            };
            if constexpr (NOFF > 0) {
                off(IC<OI0>(), IC<OJ0>(), go[0]);
                off(IC<OI1>(), IC<OJ1>(), go[1]);
            }
            // r e^{gamma_L - gamma} for the rows of tile W, e^{gamma_L} (W = 0)
            if (grp == 0) {
                const int i = 16 * W + l16;
                po.kf[i] = fast_exp2(gl - (sg[i] - lr(i)));
                if (W == 0 && l16 == 0) po.decay = fast_exp2(gl);
            }
        }
        if constexpr (DO_Q) {
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int itq = R0 + r, iq = 16 * itq + l16;
                const float ai = sg[iq] + la[r];
                if (W != 2 && grp == 0) po.osc[iq] = fast_exp2(ai);   // row 3: W = 3 publishes
#pragma unroll
                for (int jt = J0; jt <= J1; ++jt) {
                    if (jt > itq) continue;
                    const f32x4 cj = *(const f32x4 *)&sg[16 * jt + 4 * grp] - lr4(16 * jt + 4 * grp);
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[e] = fast_exp2(ai - cj[e]) * gq[r][jt][e];
                        if (jt == itq) v[e] = iq >= 16 * jt + 4 * grp + e ? v[e] : 0.f;
                    }
                    *(v4 *)pel(po, iq, pcol(jt, grp)) = cvt4(v);
                }
            }
        }
        if constexpr (DO_K) {
            // column cc of D is row cc of D^T; the column scalings of the two
            // scaled forms are the factors of token 16 W + cc
            const int cc = lane >> 2, gg = lane & 3;
            const int tc = 16 * W + cc;
            const float bc = sb[tc], bgr = fast_exp2(sgb[tc] + lr(tc));
            const f32x4 xv = {x[0], x[1], x[2], x[3]};
            *(v4 *)&po.dt[0][W][cc][4 * gg] = cvt4(xv);
            *(v4 *)&po.dt[1][W][cc][4 * gg] = cvt4(xv * bc);
            *(v4 *)&po.dt[2][W][cc][4 * gg] = cvt4(xv * -bgr);
        }
    };
    auto prep_tile = [&](auto k_c, auto q_c, auto n_c, int cn) {
        switch (w4) {
            case 0: prep_chunk(IC<0>(), k_c, q_c, n_c, cn); break;
            case 1: prep_chunk(IC<1>(), k_c, q_c, n_c, cn); break;
            case 2: prep_chunk(IC<2>(), k_c, q_c, n_c, cn); break;
            default: prep_chunk(IC<3>(), k_c, q_c, n_c, cn); break;
        }
    };

    // The prep waves: at step c, the copies of chunk c+2 (k, q, gates) and the
    // preparation of chunk c+1.  The chain and the prep waves run
    // separate loops with the same number of barriers, so that neither
    // carries the other's registers.
    auto prep_loop = [&](auto do_k_c, auto do_q_c, auto n_c) {
        constexpr bool DO_K = decltype(do_k_c)::value != 0, DO_Q = decltype(do_q_c)::value != 0;
        for (int c = -1; c < nchunks; ++c) {
            const int cn = c + 1;
            if constexpr (!MERGED) {
                if (DO_K && c + 2 < nchunks) issue_k(c + 2);
                if (DO_Q && want_o && c + 2 < nchunks) issue_q(c + 2);
            }
            if (gate_wave) {
                if (c + 2 < nchunks) issue_gb(c + 2);
                if (gated && c + 2 < nchunks) gate_chunk(c + 2);   // its raw words landed before the last barrier
                if (c + 3 < nchunks) issue_gates(c + 3);
                if constexpr (MERGED) {
                    if (c + 2 < nchunks) {
                        issue_k(c + 2);
                        if (want_o) issue_q(c + 2);
                    }
                }
            }
            if (cn < nchunks && (DO_K || want_o)) prep_tile(do_k_c, do_q_c, n_c, cn);
            wait_vmem();   // this wave's copies
            lds_barrier();
        }
    };
    if (role != 0) {
        // the prep code is compiled with and without the L2 norm
        auto roles = [&](auto n_c) {
            if constexpr (MERGED) {
                if constexpr (!want_o) prep_loop(IC<1>(), IC<0>(), n_c);   // no P tiles
                else prep_loop(IC<1>(), IC<1>(), n_c);
            } else if (role == 1) {
                prep_loop(IC<1>(), IC<0>(), n_c);
            } else {
                prep_loop(IC<0>(), IC<1>(), n_c);
            }
        };
        if (p.use_l2norm) roles(IC<1>());
        else roles(IC<0>());
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
    // This wave's v columns c0 .. c0 + 15 sit in their own 64 x 16 block of the
    // chunk's v buffer (32-byte rows), copied by this wave one chunk ahead:
    // copy i moves rows 32 i .. 32 i + 31, lane l one 16-byte half row.
    const int c0 = 16 * wave;
    const unsigned vslot0 = lds0 + offsetof(Lds, vb) + 2048u * wave;
    const unsigned vlo = (unsigned)(lane >> 1) * (unsigned)v_row * sizeof(E) + 16 * (lane & 1);
    auto issue_vw = [&](int c) {
        const int64_t t0 = tok0 + 64LL * c;
        const int last = min(64, len - 64 * c) - 1;
        const E *vc = vg + (size_t)t0 * v_row + (size_t)j * V + vcol0 + c0;
        const unsigned dst = vslot0 + (c & 1) * (64 * VROW);
        if (last == 63) {
            lds_copy16s(vc, vlo, dst);
            lds_copy16s(vc, vlo + 32u * (unsigned)v_row * sizeof(E), dst + 1024u);
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                lds_copy16s(vc, (unsigned)min(32 * i + (lane >> 1), last) * (unsigned)v_row * sizeof(E) + 16 * (lane & 1),
                            dst + 1024u * i);
        }
    };
    // transpose read of the v tile: token row 16 ti + 4 grp + l16/4, value
    // columns c0 + 4 (l16 % 4) .. +3
    const int vo = (4 * grp + (l16 >> 2)) * 32 + 8 * (l16 & 3);
    // transpose read of a 16x16 D block: row 4 grp + l16/4, columns 4 (l16 % 4) .. +3
    const int dto = (4 * grp + (l16 >> 2)) * 32 + 8 * (l16 & 3);

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
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    constexpr bool WO = want_o;
    for (int c = -1; c < nchunks; ++c) {
        const int cn = c + 1;
        // copy of v of chunk c+1 (this wave's columns) into the slot nothing
        // reads in this step; landed before the step's barrier.  Issued after
        // the block substitution: issued at the start of the step, the copies
        // of all chain waves queue up at once and hold back the first products.
        auto issue_copies = [&]() {
            if (cn < nchunks) issue_vw(cn);
        };
        if (c < 0) issue_copies();
        if (c >= 0) {
            const PrepOut &po = *(const PrepOut *)((const char *)s.po + uni((c & 1) * (int)sizeof(PrepOut)));
            const char *kb = (const char *)s.kb[0] + uni((c % 3) * 64 * KROW);
            const char *vbp = (const char *)s.vb[0] + 2048 * wave + uni((c & 1) * 64 * VROW) + vo;
            const char *dtp = (const char *)&po.dt[0][0][0][0] + dto;
            const int64_t t0 = tok0 + 64LL * c;
            const int L = min(64, len - 64 * c);
            // Start of each block of V_new: D_b diag(beta) V_b - D_b diag(beta e^gamma r) Z_b
            f32x4 acc[4], y[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const v4 vv = tr(vbp + 512 * b);
                const v4 fb = tr(dtp + (4 + b) * 512), fg = tr(dtp + (8 + b) * 512);
                acc[b] = mma_k16(fb, vv, zero4);
                acc[b] = mma_k16(fg, cvt4(zk[b]), acc[b]);
                y[b] = zero4;
            }
            // V_new by block forward substitution, right-looking: as soon as
            // block m is final it is applied to every later block, so the
            // updates of different blocks overlap and only two products per
            // block sit on the dependency chain.
            v4 vb16[4];
            f32x4 vnf[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (m > 0) acc[m] = mma_k16(tr(dtp + m * 512), cvt4(y[m]), acc[m]);
                vnf[m] = acc[m];
                vb16[m] = cvt4(acc[m]);
#pragma unroll
                for (int bi = m + 1; bi < 4; ++bi)
                    y[bi] = mma_k16(*(const v4 *)&po.alo[alo_blk(bi, m)][grp][l16][0], vb16[m], y[bi]);
            }
            issue_copies();
            // V_new for the output product, diag(kf) V_new for the state
            v8 vnb[2], vkb[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const f32x4 k0 = *(const f32x4 *)&po.kf[32 * s2 + 4 * grp];
                const f32x4 k1 = *(const f32x4 *)&po.kf[32 * s2 + 16 + 4 * grp];
                vnb[s2] = cat8(vb16[2 * s2], vb16[2 * s2 + 1]);
                vkb[s2] = cat8(cvt4(k0 * vnf[2 * s2]), cvt4(k1 * vnf[2 * s2 + 1]));
            }
            // O^T tiles [value][token]: (Q h)^T scaled by scale rho e^gamma per
            // token, plus (P V_new)^T; and h <- e^{gamma_L} h + K^T diag(kf) V_new
            // (K^T by transpose loads).  The two are independent, so they sit in
            // one branch-free block and the scheduler interleaves them.
            f32x4 o[4];
            if constexpr (WO) {
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    const int i = 16 * ti + l16;
                    o[ti] = zq[ti] * po.osc[i];
#pragma unroll
                    for (int s2 = 0; s2 <= ti / 2; ++s2) o[ti] = mma(vnb[s2], *(const v8 *)pel(po, i, pcol(2 * s2, grp)), o[ti]);
                }
            }
            const float dec = po.decay;
#pragma unroll
            for (int m2 = 0; m2 < KT / 2; ++m2) {
                const char *pm = kb + to[m2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int mt = 2 * m2 + hf;
                    f32x4 acc2 = h[mt] * dec;
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const char *pa = pm + 8 * hf + 32 * s2 * KROW;
                        acc2 = mma(cat8(tr(pa), tr(pa + 16 * KROW)), vkb[s2], acc2);
                    }
                    h[mt] = acc2;
                }
            }
            if constexpr (WO) {
                E *dst = og + ((size_t)t0 * p.HV + j) * V + vcol0 + c0 + 4 * grp;
                const size_t orow = (size_t)p.HV * V;
                if (L == 64) {
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti)
                        *(v4 *)__builtin_assume_aligned(dst + (16 * ti + l16) * orow, 8) = cvt4(o[ti]);
                } else {
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti)
                        if (16 * ti + l16 < L) *(v4 *)__builtin_assume_aligned(dst + (16 * ti + l16) * orow, 8) = cvt4(o[ti]);
                }
            }
        }
        if (cn < nchunks) {
            // Z = K h and (Q h)^T of chunk cn with the updated state
            const E *kb = (const E *)((const char *)s.kb[0] + uni((cn % 3) * 64 * KROW));
            const E *qb = (const E *)((const char *)s.qb[0] + uni((cn & 1) * 64 * KROW));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                zk[t] = zero4;
                zq[t] = zero4;
            }
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) {
                const v8 hb = cat8(cvt4(h[2 * s2]), cvt4(h[2 * s2 + 1]));
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    zk[t] = mma(frag(kb, t, s2), hb, zk[t]);
                    if constexpr (WO) zq[t] = mma(hb, frag(qb, t, s2), zq[t]);
                }
            }
        }
        wait_vmem();   // this wave's copies
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

template <int NCW, bool GATED, bool POOL, bool OUT>
hipError_t launch_ws_kv(const Params &p, hipStream_t st) {
    const int per_group = (p.HV / p.H) * (p.V / (16 * NCW));
    const unsigned grid = (unsigned)((p.N * p.H + 7) / 8) * 8 * per_group;
    if constexpr (NCW == 8) {
        if (p.K == 64) fused_ws_kernel<64, 128, 8, GATED, POOL, OUT><<<grid, 768, 0, st>>>(p);
        else fused_ws_kernel<128, 128, 8, GATED, POOL, OUT><<<grid, 768, 0, st>>>(p);
    } else {
        if (p.K == 64 && p.V == 64) fused_ws_kernel<64, 64, 4, GATED, POOL, OUT><<<grid, 768, 0, st>>>(p);
        else if (p.K == 64 && p.V == 128) fused_ws_kernel<64, 128, 4, GATED, POOL, OUT><<<grid, 768, 0, st>>>(p);
        else if (p.K == 128 && p.V == 64) fused_ws_kernel<128, 64, 4, GATED, POOL, OUT><<<grid, 768, 0, st>>>(p);
        else fused_ws_kernel<128, 128, 4, GATED, POOL, OUT><<<grid, 768, 0, st>>>(p);
    }
    return hipGetLastError();
}

template <bool GATED, bool POOL, bool OUT = true>
hipError_t launch_ws_layout(const Params &p, hipStream_t st) {
    // whole 128-column value heads once there are enough (sequence, value
    // head) pairs to give every CU a workgroup; 64-column slices otherwise
    if (p.V == 128 && (int64_t)p.N * p.HV >= 256) return launch_ws_kv<8, GATED, POOL, OUT>(p, st);
    return launch_ws_kv<4, GATED, POOL, OUT>(p, st);
}

}  // namespace

// One workgroup of 768 threads per (sequence, value head) or per (sequence,
// value head, 64 value columns).
hipError_t launch_fused_ws(const Params &p, hipStream_t st) {
    if (p.N * p.H == 0) return hipSuccess;
    const bool gated = p.gates.A_log != nullptr,
               pool = p.state_indices != nullptr || p.state_bf16 || p.v_zero || p.init_shared;
    if (pool && !p.out) {   // the sequence split's state and transfer-map passes
        if (gated) return launch_ws_layout<true, true, false>(p, st);
        return launch_ws_layout<false, true, false>(p, st);
    }
    if (gated && pool) return launch_ws_layout<true, true>(p, st);
    if (gated) return launch_ws_layout<true, false>(p, st);
    if (pool) return launch_ws_layout<false, true>(p, st);
    return launch_ws_layout<false, false>(p, st);
}

}  // namespace gdn
