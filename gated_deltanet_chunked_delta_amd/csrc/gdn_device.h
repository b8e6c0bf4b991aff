// Device-side helpers shared by the HIP kernels (types, MFMA wrappers,
// fragment loads).  Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace dev {

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

// Gates from the raw projections (the fused gating operator of the FastDeploy
// PR #7024 page, "Usage or Command" item 5): g = -exp(A_log) softplus(a +
// dt_bias) with negA = -exp(A_log), beta = sigmoid(b).  Every kernel uses
// these two functions, so in-kernel gates equal the stand-alone kernel's bit
// for bit.  They run on the hardware exp2 / log2 / reciprocal (about one ulp
// each):
//   softplus(x) = max(x, 0) + log1p(e),  e = e^-|x| in (0, 1],
//   log1p(e)    = ln(u) e / (u - 1),  u = 1 + e  (exact when u = 1: e),
// the rewrite that cancels the rounding of u (Goldberg, "What every computer
// scientist should know about floating-point arithmetic", on log1p), and
//   sigmoid(b)  = 1 / (1 + e^-b),
// which goes to 0 or 1 in the tails (the reciprocal of inf is 0).
__device__ __forceinline__ float gate_g(float a, float negA, float dt_bias) {
    const float x = a + dt_bias;
    const float e = __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f);
    const float u = 1.f + e;
    const float l1p = u == 1.f ? e : __builtin_amdgcn_logf(u) * 0.6931471805599453f * e * __builtin_amdgcn_rcpf(u - 1.f);
    return negA * (fmaxf(x, 0.f) + l1p);
}
__device__ __forceinline__ float gate_beta(float b) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-b * 1.4426950408889634f));
}

// One raw gate input of element type E from the 4-byte word that holds it: a
// bf16 sits in the low or high half (hi) of its aligned word.
template <typename E> __device__ __forceinline__ float gate_raw(float word, bool hi);
template <> __device__ __forceinline__ float gate_raw<float>(float word, bool) { return word; }
template <> __device__ __forceinline__ float gate_raw<bf16>(float word, bool hi) {
    const unsigned w = __float_as_uint(word);
    return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
}

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x8 a, f32x8 b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

// 16x16x16 product: A lane holds row l16 at reduction slots 4*grp..4*grp+3,
// B lane holds column l16 at the same slots, i.e. exactly the rows a C tile
// gives that lane.
__device__ __forceinline__ f32x4 mma_k16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k16(f32x4 a, f32x4 b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
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

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transposing LDS read of a 16x16 block of a row-major matrix M in LDS:
// lane (li = lane & 15, g = lane >> 4) gets r[e] = M[row0 + 4g + e][col0 + li],
// i.e. the block's transpose in the A/B-operand layout of a 16x16x16 product
// (lane = row of the transposed block, slots = 4 consecutive rows of M).
// `addr(row, col)` returns the element pointer of M(row, col).  bf16 uses the
// gfx950 transpose load (within each 16-lane group, lane li receives element e
// of the 8-byte row that lane 4e + li/4 addressed, at position li % 4); fp32
// gathers four scalars.
template <typename E, typename F>
__device__ __forceinline__ typename VT<E>::v4 ld_tr(int row0, int col0, F addr) {
    const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
    if constexpr (sizeof(E) == 2) {
        const E *pt = addr(row0 + 4 * g + (li >> 2), col0 + 4 * (li & 3));
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)pt);
    } else {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = *addr(row0 + 4 * g + e, col0 + li);
        return r;
    }
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// fences global memory, which makes the compiler wait for every outstanding
// vector memory operation (including asynchronous global->LDS copies that are
// meant to overlap the barrier); code that needs a copy waits for it itself.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 2^x by the hardware exponential (v_exp_f32).  Tiny results may flush to
// zero, which is the right limit for the decay factors it is used for.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sequence offsets are read clamped to [0, T]: a malformed cu_seqlens then
// yields wrong rows, never an access outside the token range.
__device__ __forceinline__ int cu_at(const int32_t *cu, int n, int T) { return min(max(cu[n], 0), T); }

}  // namespace dev
}  // namespace gdn
