// Fused chunked gated delta rule forward pass for gfx950: one kernel does
// every step of the chunked algorithm for one (sequence, value head, slice of
// VW value columns), walking the sequence's 64-token chunks in order with the
// K x VW fp32 state held in registers the whole time.  HBM traffic is the
// method's own: q, k, v, g, beta are read once per workgroup (the workgroups
// of one key head share their q/k reads through L2), o is written once, the
// states once each.
//
// Steps per chunk (the step list of the page "NPU Training Operators - GDN",
// operator-semantics section; chunk length 64 from its tiling section), with
// gamma the inclusive gate cumsum inside the chunk, r / rho the L2-norm
// factors of k / q (1 when the norm is off), h the state at the chunk start:
//
//   prologue  gamma, r, rho                       (fp32)
//   kkt       A = strict_lower(beta_i r_i r_j e^{gamma_i-gamma_j} k_i.k_j)
//             P = causal(scale rho_i r_j e^{gamma_i-gamma_j} q_i.k_j)
//   solve     D_b = (I + A_bb)^-1 for the four diagonal 16x16 blocks, by
//             forward substitution in fp32 (lane = column)
//   w/u       folded into the state step: with Z = K h,
//             X = diag(beta) V - diag(beta e^gamma r) Z  (= U - W h)
//             V_new = (I + A)^-1 X by block forward substitution
//             V_b = D_b (X_b - sum_{m<b} A_bm V_m)
//   fwd_h     h <- e^{gamma_L} h + (diag(r e^{gamma_L - gamma}) K)^T V_new
//   fwd_o     O = diag(scale rho e^gamma) Q h + P V_new
//
// (I + A)^-1 X equals U - W h of the WY form with W = T diag(beta e^gamma r) K
// and U = T diag(beta) V, T = (I + A)^-1; solving for the right-hand side
// directly needs no off-diagonal blocks of T.
//
// Work split inside a workgroup of NW waves: each wave owns CPW 16-column
// tiles of the state and runs the h-dependent chain (Z, X, V_new, O, h) for
// them alone, so the chain needs no data exchange between waves.  The
// h-independent work (cumsum, Gram tiles, diagonal inverses) is shared
// through LDS; the Gram tiles (and from their diagonals the squared row norms
// of k and q) are computed in the same pass over the K/Q fragments as Z, so
// every fragment is read from LDS once per wave.  Gram tiles and the output
// are produced transposed (B x A instead of A x B) so that each lane holds
// four consecutive columns and stores them with one vector write.  K^T and the
// v tile are read straight from the row-major raw rows with gfx950 transpose
// loads.  The next chunk's raw q/k/v/g/beta stream from HBM into the other
// half of a double-buffered LDS area (global_load_lds, no staging registers)
// while the current chunk computes.
#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous global -> LDS copies: lane l's bytes land at lds + l * size.
__device__ __forceinline__ void lds_copy16(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_copy4(const void *g, void *lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 4, 0, 0);
}
// Wait until this wave's asynchronous copies (and all its other vector memory
// operations) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// XOR swizzle of the 16-byte segments of an unpadded row of NSEG segments, so
// that the same segment of 16 consecutive rows falls in 16 different groups
// of 4 LDS banks.
template <int NSEG> __device__ __forceinline__ int swz(int row) {
    static_assert(NSEG == 8 || NSEG % 16 == 0, "row length");
    return NSEG >= 16 ? (row & 15) : ((row >> 1) & 7);
}
// Element offset of (row, col) in a swizzled buffer with rows of W elements.
template <typename E, int W> __device__ __forceinline__ int sw_off(int row, int col) {
    constexpr int VEC = 16 / sizeof(E), NSEG = W / VEC;
    return row * W + (((col / VEC) ^ swz<NSEG>(row)) * VEC) + (col % VEC);
}

template <typename E, int K, int VW, int NB> struct FusedLds {
    static constexpr int PE = 16 / sizeof(E);   // 16-byte row pad
    E kb[NB][64 * K];         // raw k rows (swizzled), double-buffered in bf16
    E qb[NB][64 * K];         // raw q rows (swizzled)
    E vb[NB][64 * VW];        // raw v rows of this slice (swizzled)
    float gb[NB][64], bb[NB][64];   // raw g, beta
    E alo[64][64 + PE];       // -A, off-diagonal 16x16 blocks below the diagonal
    E p[64][64 + PE];         // P; blocks (0,1) and (2,3) zeroed, others above unused
    E d[64][16 + PE];         // D_b row r at 16*b + r
    float adiag[4][272];      // diagonal 16x16 blocks of A, row r at 16*r (fp32)
    float gam[64], beta[64], rk[64], rq[64];   // gamma, beta, L2-norm factors of k and q
    float bz[64], oq[64], kf[64];   // beta e^gamma r,  scale rho e^gamma,  r e^{gamma_L - gamma}
    float decay;                    // e^{gamma_L}
};

template <typename E, int K, int V, int NW, int CPW>
__global__ void __launch_bounds__(64 * NW) fused_kernel(Params p) {
    typedef typename VT<E>::v8 v8;
    typedef typename VT<E>::v4 v4;
    typedef typename VT<E>::v16b v16b;
    constexpr int NT = 64 * NW;
    constexpr int VW = 16 * NW * CPW;
    constexpr int VEC = VT<E>::kVec;
    constexpr int NB = sizeof(E) == 2 ? 2 : 1;   // fp32 check mode: no room for a second buffer
    constexpr int NSK = K / VEC, NSV = VW / VEC; // 16-byte segments per k/q row and per v row
    constexpr int KT = K / 16, KS = K / 32;
    constexpr int RT = 4 / NW;                   // Gram row tiles per wave
    static_assert(NSK % NW == 0 && NSV % NW == 0, "copy instructions must split evenly over waves");
    static_assert(V % VW == 0 && (NW == 2 || NW == 4), "workgroup shape");
    __shared__ FusedLds<E, K, VW, NB> s;

    const int tid = threadIdx.x, lane = tid & 63;
    // the wave index is uniform inside a wave; say so, so that per-wave choices
    // compile to scalar branches instead of exec-mask juggling
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, grp = lane >> 4;

    // Workgroup -> (sequence n, key head jk, value head j, column slice).  Ids
    // go round-robin over the 8 XCDs; all workgroups of one (n, jk) group sit
    // on one XCD so that the q/k rows they all read come from HBM once.
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

    // Raw gate inputs, when given: the head's constants, and which half of its
    // aligned 4-byte word a bf16 input occupies (HV is even, so the half is
    // the parity of j for every token).
    const bool gated = p.gates.A_log != nullptr;
    const float negA = gated ? -expf(p.gates.A_log[j]) : 0.f;
    const float dtb = gated ? p.gates.dt_bias[j] : 0.f;
    const bool ghi = sizeof(E) == 2 && (j & 1);

    const E *__restrict__ qg = (const E *)p.q;
    const E *__restrict__ kg = (const E *)p.k;
    const E *__restrict__ vg = (const E *)p.v;
    E *__restrict__ og = (E *)p.out;

    // state: CPW column tiles x KT row tiles, C layout
    f32x4 h[CPW][KT];
    size_t sbase = ((size_t)n * p.HV + j) * K * V + vcol0;
    bool s_in = p.initial_state != nullptr, s_out = p.final_state != nullptr;
    if (p.state_indices) {   // state pool: the slot of sequence n (outside the pool: none)
        const int slot = p.state_indices[n];
        const bool ok = slot >= 0 && slot < p.pool_size;
        s_in = s_in && ok;
        s_out = s_out && ok;
        sbase = ((size_t)(ok ? slot : 0) * p.HV + j) * K * V + vcol0;
    }
    // init_shared: one initial state for every sequence
    const size_t sbase_in = p.init_shared ? (size_t)j * K * V + vcol0 : sbase;
    if (s_in) {
        const float *__restrict__ s0 = p.initial_state + sbase_in;
        const bf16 *__restrict__ s0h = (const bf16 *)p.initial_state + sbase_in;
#pragma unroll
        for (int ct = 0; ct < CPW; ++ct) {
            const int col = 16 * (wave * CPW + ct) + l16;
#pragma unroll
            for (int mt = 0; mt < KT; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const size_t o = (size_t)(16 * mt + 4 * grp + e) * V + col;
                    h[ct][mt][e] = p.state_bf16 ? to_f(s0h[o]) : s0[o];
                }
        }
    } else {
#pragma unroll
        for (int ct = 0; ct < CPW; ++ct)
#pragma unroll
            for (int mt = 0; mt < KT; ++mt) h[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Asynchronous copy of chunk c's raw rows into LDS buffer `buf`.  Rows past
    // the sequence end read the last valid row (so every address stays inside
    // the sequence) and are zeroed after arrival.
    // elements between token rows (v_zero: every token reads the one zero row)
    const size_t kq_row = (size_t)p.H * K, v_row = p.v_zero ? 0 : (size_t)p.HV * V;
    auto issue = [&](int c, int buf) {
        const int64_t t0 = tok0 + 64LL * c;
        const int last = min(64, len - 64 * c) - 1;
        const E *kc = kg + (size_t)t0 * kq_row + (size_t)jk * K;
        const E *qc = qg + (size_t)t0 * kq_row + (size_t)jk * K;
        const E *vc = vg + (size_t)t0 * v_row + (size_t)j * V + vcol0;
#pragma unroll
        for (int i = 0; i < NSK / NW; ++i) {
            const int t = wave + NW * i;
            const int P = 64 * t + lane, row = P / NSK, seg = (P % NSK) ^ swz<NSK>(row);
            const unsigned off = (unsigned)min(row, last) * (unsigned)kq_row + seg * VEC;
            lds_copy16(kc + off, &s.kb[buf][64 * t * VEC]);
            lds_copy16(qc + off, &s.qb[buf][64 * t * VEC]);
        }
#pragma unroll
        for (int i = 0; i < NSV / NW; ++i) {
            const int t = wave + NW * i;
            const int P = 64 * t + lane, row = P / NSV, seg = (P % NSV) ^ swz<NSV>(row);
            lds_copy16(vc + (unsigned)min(row, last) * (unsigned)v_row + seg * VEC, &s.vb[buf][64 * t * VEC]);
        }
        if (wave == NW - 1) {
            const size_t o = (size_t)(t0 + min(lane, last)) * p.HV + j;
            if (gated) {   // the aligned word that holds the raw input
                const size_t wo = (o * sizeof(E)) & ~(size_t)3;
                lds_copy4((const char *)p.gates.a + wo, &s.gb[buf][0]);
                lds_copy4((const char *)p.gates.b + wo, &s.bb[buf][0]);
            } else {
                lds_copy4(p.g + o, &s.gb[buf][0]);
                lds_copy4(p.beta + o, &s.bb[buf][0]);
            }
        }
    };

    if (nchunks > 0) issue(0, 0);
    for (int c = 0; c < nchunks; ++c) {
        const int buf = (NB == 2) ? (c & 1) : 0;
        const int64_t t0 = tok0 + 64LL * c;
        const int L = min(64, len - 64 * c);
        const E *kb = s.kb[buf];
        const E *qb = s.qb[buf];
        const E *vb = s.vb[buf];

        // ---- chunk c has arrived; start the next copy ----------------------
        wait_vmem();
        lds_barrier();
        if (L < 64) {   // zero the rows past the sequence end (uniform branch)
            for (int idx = tid; idx < (64 - L) * NSK; idx += NT) {
                const int o = L * K + idx * VEC;
                *(v16b *)&s.kb[buf][o] = v16b{};
                *(v16b *)&s.qb[buf][o] = v16b{};
            }
            for (int idx = tid; idx < (64 - L) * NSV; idx += NT) *(v16b *)&s.vb[buf][L * VW + idx * VEC] = v16b{};
            if (tid >= L && tid < 64) {
                s.gb[buf][tid] = 0.f;
                s.bb[buf][tid] = 0.f;
            }
            lds_barrier();
        }
        if (NB == 2 && c + 1 < nchunks) issue(c + 1, buf ^ 1);

        // ---- gate cumsum; Z = [K; Q] h, Gram tiles, squared row norms ------
        if (wave == 0) {
            float x = s.gb[buf][lane], bt = s.bb[buf][lane];
            if (gated) {   // gates from the raw inputs; rows past the end read 0
                x = lane < L ? gate_g(gate_raw<E>(x, ghi), negA, dtb) : 0.f;
                bt = lane < L ? gate_beta(gate_raw<E>(bt, ghi)) : 0.f;
            }
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(x, o);
                if (lane >= o) x += y;
            }
            s.gam[lane] = x * 1.4426950408889634f;   // gamma in log2 units: e^{a-b} = 2^{a2-b2}
            s.beta[lane] = bt;
        }
        // This wave's Gram tiles, all transposed (C[j][i]): K K^T row tiles
        // itk = wave + NW*i (columns jt <= itk), Q K^T row tiles itq = 3 - itk
        // (jt <= itq), and the diagonal tiles of Q Q^T at itq (for |q|^2).
        // Every wave gets 5 tiles (NW = 4) or 10 (NW = 2).
        auto itk_of = [&](int i) { return wave + NW * i; };
        auto itq_of = [&](int i) { return 3 - wave - NW * i; };
        auto kaddr = [&](int row, int col) { return &kb[sw_off<E, K>(row, col)]; };
        auto qaddr = [&](int row, int col) { return &qb[sw_off<E, K>(row, col)]; };
        auto frag = [&](auto addr, int t, int s2) {   // row tile t, reduction step s2, scan slot order
            const v4 a0 = *(const v4 *)addr(16 * t + l16, 32 * s2 + 4 * grp);
            const v4 a1 = *(const v4 *)addr(16 * t + l16, 32 * s2 + 16 + 4 * grp);
            v8 f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[e] = a0[e];
                f[4 + e] = a1[e];
            }
            return f;
        };
        f32x4 zk[CPW][4];   // Z_k = K h (token rows)
        f32x4 gk[RT][4], gq[RT][4], gqq[RT];
        {
#pragma unroll
            for (int ct = 0; ct < CPW; ++ct)
#pragma unroll
                for (int t = 0; t < 4; ++t) zk[ct][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < RT; ++i) {
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
                    gk[i][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    gq[i][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                gqq[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) {
                // state rows 32*s2 .. 32*s2+31: B operand of K h
                v8 hb[CPW];
#pragma unroll
                for (int ct = 0; ct < CPW; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hb[ct][e] = to_e<E>(h[ct][2 * s2][e]);
                        hb[ct][4 + e] = to_e<E>(h[ct][2 * s2 + 1][e]);
                    }
                v8 fk[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) fk[t] = frag(kaddr, t, s2);
#pragma unroll
                for (int ct = 0; ct < CPW; ++ct)
#pragma unroll
                    for (int t = 0; t < 4; ++t) zk[ct][t] = mma(fk[t], hb[ct], zk[ct][t]);
#pragma unroll
                for (int i = 0; i < RT; ++i) {
                    const int itk = itk_of(i), itq = itq_of(i);
                    // this wave's B operands, selected by address (no register indexing)
                    const v8 bk = frag(kaddr, itk, s2), bq = frag(qaddr, itq, s2);
                    // all four column tiles, also those above the diagonal: a few
                    // wasted products cost less than predicated accumulators
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt) {
                        gk[i][jt] = mma(fk[jt], bk, gk[i][jt]);
                        gq[i][jt] = mma(fk[jt], bq, gq[i][jt]);
                    }
                    gqq[i] = mma(bq, bq, gqq[i]);
                }
            }
        }
        // L2-norm factors from the diagonal tiles' squared norms: lane
        // (i = l16, j = 4*grp + e) holds entry (j, i); the diagonal is e = l16 - 4*grp
        {
            const int e = l16 - 4 * grp;
            if (e >= 0 && e < 4) {
#pragma unroll
                for (int i = 0; i < RT; ++i) {
                    f32x4 dk = gk[i][0];
#pragma unroll
                    for (int jt = 1; jt < 4; ++jt)
                        if (jt == itk_of(i)) dk = gk[i][jt];
                    s.rk[16 * itk_of(i) + l16] = p.use_l2norm ? rsqrtf(dk[e] + 1e-6f) : 1.f;
                    s.rq[16 * itq_of(i) + l16] = p.use_l2norm ? rsqrtf(gqq[i][e] + 1e-6f) : 1.f;
                }
            }
        }
        lds_barrier();

        // ---- per-token factors; Gram epilogue; diagonal inverses ----------
        if (wave == 0) {
            const float gi = s.gam[lane], gl = s.gam[63], ri = s.rk[lane];
            const float egi = fast_exp2(gi);
            s.bz[lane] = s.beta[lane] * egi * ri;
            s.oq[lane] = p.scale * s.rq[lane] * egi;
            s.kf[lane] = ri * fast_exp2(gl - gi);
            if (lane == 0) s.decay = fast_exp2(gl);
        }
#pragma unroll
        for (int ii = 0; ii < RT; ++ii) {
            // K K^T tiles: lane holds column i = 16*itk + l16, rows j = 16*jt + 4*grp + e
            const int itk = itk_of(ii), i = 16 * itk + l16;
            const float gi = s.gam[i], bri = s.beta[i] * s.rk[i];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                if (jt > itk) continue;
                const int j0 = 16 * jt + 4 * grp;
                const f32x4 gj = *(const f32x4 *)&s.gam[j0], rj = *(const f32x4 *)&s.rk[j0];
                f32x4 a;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = bri * rj[e] * fast_exp2(gi - gj[e]) * gk[ii][jt][e];
                    a[e] = (jt < itk || i > j0 + e) ? v : 0.f;
                }
                if (jt == itk) {
                    *(f32x4 *)&s.adiag[itk][16 * l16 + 4 * grp] = a;
                } else {
                    v4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = to_e<E>(-a[e]);
                    *(v4 *)&s.alo[i][j0] = o;
                }
            }
        }
#pragma unroll
        for (int ii = 0; ii < RT; ++ii) {
            // Q K^T tiles: lane holds column i = 16*itq + l16, rows j
            const int itq = itq_of(ii), i = 16 * itq + l16;
            const float gi = s.gam[i], sri = p.scale * s.rq[i];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                if (jt > itq) continue;
                const int j0 = 16 * jt + 4 * grp;
                const f32x4 gj = *(const f32x4 *)&s.gam[j0], rj = *(const f32x4 *)&s.rk[j0];
                v4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = sri * rj[e] * fast_exp2(gi - gj[e]) * gq[ii][jt][e];
                    o[e] = to_e<E>((jt < itq || i >= j0 + e) ? v : 0.f);
                }
                *(v4 *)&s.p[i][j0] = o;
            }
        }
        for (int idx = tid; idx < 512; idx += NT) {
            const int t = idx >> 8, e = idx & 255;
            s.p[32 * t + (e >> 4)][32 * t + 16 + (e & 15)] = to_e<E>(0.f);
        }
        // Each wave inverts the diagonal blocks it just wrote (no barrier: a
        // wave's own LDS writes are visible to its later reads).  Lane
        // (group b, column cc); the 16 lanes of group b solve block itk for
        // b < RT (RT = 1 or 2); rows are prefetched one step ahead.
        {
            const int b = grp, cc = l16;
            if (b < RT) {
                const float *A = s.adiag[itk_of(b)];
                float x[16];
                f32x4 cur[4] = {}, nxt[4] = {};
                x[0] = (cc == 0) ? 1.f : 0.f;
                cur[0] = *(const f32x4 *)&A[16 * 1];
#pragma unroll
                for (int r = 1; r < 16; ++r) {
                    if (r + 1 < 16) {
#pragma unroll
                        for (int m4 = 0; m4 < (r + 4) / 4; ++m4) nxt[m4] = *(const f32x4 *)&A[16 * (r + 1) + 4 * m4];
                    }
                    float acc0 = (r == cc) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
                    for (int m = 0; m < r; ++m) {
                        if (m & 1) acc1 -= cur[m >> 2][m & 3] * x[m];
                        else acc0 -= cur[m >> 2][m & 3] * x[m];
                    }
                    x[r] = acc0 + acc1;
#pragma unroll
                    for (int m4 = 0; m4 < 4; ++m4) cur[m4] = nxt[m4];
                    asm volatile("" ::: "memory");   // keep later rows' loads out of this step
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) s.d[16 * itk_of(b) + r][cc] = to_e<E>(x[r]);
            }
        }
        lds_barrier();

        // ---- the h-dependent chain: X, V_new, O, next h --------------------
        auto vaddr = [&](int row, int col) { return &vb[sw_off<E, VW>(row, col)]; };
#pragma unroll
        for (int ct = 0; ct < CPW; ++ct) {
            const int c0 = 16 * (wave * CPW + ct);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const v4 vv = ld_tr<E>(16 * ti, c0, vaddr);   // C layout of the v tile
                const f32x4 be = *(const f32x4 *)&s.beta[16 * ti + 4 * grp];
                const f32x4 bz = *(const f32x4 *)&s.bz[16 * ti + 4 * grp];
#pragma unroll
                for (int e = 0; e < 4; ++e) zk[ct][ti][e] = be[e] * to_f(vv[e]) - bz[e] * zk[ct][ti][e];
            }
        }
        const float dec = s.decay;
#pragma unroll
        for (int ct = 0; ct < CPW; ++ct) {
            const int c0 = 16 * (wave * CPW + ct);
            // V_new by block forward substitution (zk now holds X)
            v4 vb16[4];
            f32x4 vnf[4];
#pragma unroll
            for (int bi = 0; bi < 4; ++bi) {
                f32x4 rr = zk[ct][bi];
#pragma unroll
                for (int m = 0; m < bi; ++m) rr = mma_k16(*(const v4 *)&s.alo[16 * bi + l16][16 * m + 4 * grp], vb16[m], rr);
                v4 rbv;
#pragma unroll
                for (int e = 0; e < 4; ++e) rbv[e] = to_e<E>(rr[e]);
                vnf[bi] = mma_k16(*(const v4 *)&s.d[16 * bi + l16][4 * grp], rbv, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int e = 0; e < 4; ++e) vb16[bi][e] = to_e<E>(vnf[bi][e]);
            }
            // V_new fragments over 32-token steps; vkb scales the token rows by kf
            v8 vnb[2], vkb[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const f32x4 k0 = *(const f32x4 *)&s.kf[32 * s2 + 4 * grp];
                const f32x4 k1 = *(const f32x4 *)&s.kf[32 * s2 + 16 + 4 * grp];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vnb[s2][e] = vb16[2 * s2][e];
                    vnb[s2][4 + e] = vb16[2 * s2 + 1][e];
                    vkb[s2][e] = to_e<E>(k0[e] * vnf[2 * s2][e]);
                    vkb[s2][4 + e] = to_e<E>(k1[e] * vnf[2 * s2 + 1][e]);
                }
            }
            // O^T = (Q h)^T diag(oq) + V_new^T P^T: lane holds token i = 16*ti + l16
            // and value columns c0 + 4*grp .. +3.  (Q h)^T = h^T Q^T uses the
            // state fragments as the A operand and Q's as the B operand.
            f32x4 zq[4] = {};
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) {
                v8 hb;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    hb[e] = to_e<E>(h[ct][2 * s2][e]);
                    hb[4 + e] = to_e<E>(h[ct][2 * s2 + 1][e]);
                }
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) zq[ti] = mma(hb, frag(qaddr, ti, s2), zq[ti]);
            }
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const int i = 16 * ti + l16;
                f32x4 o = zq[ti] * s.oq[i];
#pragma unroll
                for (int s2 = 0; s2 <= ti / 2; ++s2) o = mma(vnb[s2], ld4x2<E>(&s.p[i][32 * s2 + 4 * grp]), o);
                if (i < L && og) {   // no output: the sequence split's state passes
                    v4 ov;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ov[e] = to_e<E>(o[e]);
                    // 4 consecutive columns: 8 (bf16) or 16 (fp32) bytes, aligned
                    v4 *dst = (v4 *)__builtin_assume_aligned(&og[((size_t)(t0 + i) * p.HV + j) * V + vcol0 + c0 + 4 * grp],
                                                            sizeof(v4));
                    *dst = ov;
                }
            }
            // h <- e^{gamma_L} h + K^T (kf V_new); K^T fragments by transpose loads
#pragma unroll
            for (int mt = 0; mt < KT; ++mt) {
                f32x4 acc = h[ct][mt] * dec;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const v4 a0 = ld_tr<E>(32 * s2, 16 * mt, kaddr);
                    const v4 a1 = ld_tr<E>(32 * s2 + 16, 16 * mt, kaddr);
                    v8 a;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a[e] = a0[e];
                        a[4 + e] = a1[e];
                    }
                    acc = mma(a, vkb[s2], acc);
                }
                h[ct][mt] = acc;
            }
        }
        if (NB == 1 && c + 1 < nchunks) {
            lds_barrier();   // single buffer: every wave is done with it
            issue(c + 1, 0);
        }
    }

    if (s_out) {
#pragma unroll
        for (int ct = 0; ct < CPW; ++ct) {
            const int col = 16 * (wave * CPW + ct) + l16;
#pragma unroll
            for (int mt = 0; mt < KT; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const size_t o = sbase + (size_t)(16 * mt + 4 * grp + e) * V + col;
                    if (p.state_bf16)
                        ((bf16 *)p.final_state)[o] = (bf16)h[ct][mt][e];
                    else
                        p.final_state[o] = h[ct][mt][e];
                }
        }
    }
}

template <typename E, int K, int V, int NW, int CPW>
hipError_t launch_fused_cfg(const Params &p, hipStream_t st) {
    constexpr int VW = 16 * NW * CPW;
    const int groups = p.N * p.H;
    if (groups == 0) return hipSuccess;
    const int per_group = (p.HV / p.H) * (V / VW);
    const unsigned grid = (unsigned)((groups + 7) / 8) * 8 * per_group;
    fused_kernel<E, K, V, NW, CPW><<<grid, 64 * NW, 0, st>>>(p);
    return hipGetLastError();
}

}  // namespace

// The fp32 check mode: 32 columns per workgroup on 2 waves, so that its LDS
// fits one CU.  (bf16 runs the warp-specialized kernel of gdn_fused_ws.hip.)
hipError_t launch_fused(const Params &p, int dtype, hipStream_t st) {
    (void)dtype;
    if (p.K == 64 && p.V == 64) return launch_fused_cfg<float, 64, 64, 2, 1>(p, st);
    if (p.K == 64 && p.V == 128) return launch_fused_cfg<float, 64, 128, 2, 1>(p, st);
    if (p.K == 128 && p.V == 64) return launch_fused_cfg<float, 128, 64, 2, 1>(p, st);
    return launch_fused_cfg<float, 128, 128, 2, 1>(p, st);
}

namespace {

// The sequences of a packed batch longest first: order[r] is the sequence of
// rank r by chunk count, descending, ties in index order (a strict total
// order, so the ranks are a permutation).  The prefill kernels take their
// sequences in this order, so that the workgroups of the longest sequences
// start first and the short ones fill in behind them (greedy longest-first
// list scheduling over the CUs) instead of a long sequence starting last.
// One workgroup: the chunk counts in LDS (padded with -1, which ranks below
// every count), each thread ranks one sequence against all of them, four
// counts per read.
__global__ void __launch_bounds__(1024) seq_order_kernel(const int32_t *__restrict__ cu, int N, int T,
                                                         int32_t *__restrict__ order) {
    __shared__ __attribute__((aligned(16))) int nc[kSeqOrderMax];
    const int t = threadIdx.x, N4 = (N + 3) & ~3;
    for (int n = t; n < N4; n += blockDim.x)
        nc[n] = n < N ? (max(dev::cu_at(cu, n + 1, T) - dev::cu_at(cu, n, T), 0) + 63) / 64 : -1;
    __syncthreads();
    for (int n = t; n < N; n += blockDim.x) {
        const int c = nc[n];
        int r = 0;
        for (int m = 0; m < N4; m += 4) {
            const int4 d = *(const int4 *)&nc[m];
            r += (d.x > c || (d.x == c && m < n)) + (d.y > c || (d.y == c && m + 1 < n)) +
                 (d.z > c || (d.z == c && m + 2 < n)) + (d.w > c || (d.w == c && m + 3 < n));
        }
        order[r] = n;
    }
}

}  // namespace

const char *kernel_name(int kind) {
    switch (kind) {
        case kFusedKernel: return "fused_kernel";
        case kFusedWsKernel: return "fused_ws_kernel";
        case kRecurrentKernel: return "recurrent_update_kernel";
        case kGatingKernel: return "gating_kernel";
        case kSplitSetupKernel: return "split_setup_kernel";
        case kSplitCombineKernel: return "split_combine_kernel";
        case kSplitFinalKernel: return "split_final_kernel";
        case kBwdSetupKernel: return "bwd_setup_kernel";
        case kBwdPrepKernel: return "bwd_prep_kernel";
        case kBwdFwdScanKernel: return "bwd_fwd_scan_kernel";
        case kBwdDhScanKernel: return "bwd_dh_scan_kernel";
        case kBwdGradsKernel: return "bwd_grads_kernel";
        case kBwdReduceKernel: return "bwd_reduce_kernel";
        case kSeqOrderKernel: return "seq_order_kernel";
        default: return "?";
    }
}

hipError_t launch_forward(const Params &p, int dtype, hipStream_t stream, Profiler *prof) {
    if (p.seq_order) {
        if (p.N < 2 || p.N > kSeqOrderMax || !p.cu_seqlens) return hipErrorInvalidValue;
        if (prof) prof->begin(kSeqOrderKernel, stream);
        seq_order_kernel<<<1, 1024, 0, stream>>>(p.cu_seqlens, p.N, p.T, (int32_t *)p.seq_order);
        const hipError_t e = hipGetLastError();
        if (prof) prof->end(kSeqOrderKernel, stream);
        if (e != hipSuccess) return e;
    }
    const int kind = dtype == 0 ? kFusedWsKernel : kFusedKernel;
    if (prof) prof->begin(kind, stream);
    const hipError_t err = dtype == 0 ? launch_fused_ws(p, stream) : launch_fused(p, dtype, stream);
    if (prof) prof->end(kind, stream);
    return err;
}

}  // namespace gdn
