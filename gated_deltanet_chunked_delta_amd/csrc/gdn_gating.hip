// Stand-alone gate computation for gfx950: for rows x HV (token, value head)
// pairs, g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b) in fp32,
// the fused gating operator of the FastDeploy PR #7024 page ("Usage or
// Command", item 5).  The prefill and decode kernels compute the same gates
// themselves when they are given the raw inputs; this kernel serves callers
// that keep g and beta as tensors.
//
// Elementwise and bound by HBM (a, b in; g, beta out).  Each thread handles
// eight consecutive elements per pass: with aligned buffers one 16-byte (bf16)
// or two 16-byte (fp32) loads per input and two 16-byte stores per output;
// otherwise element by element.
#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

template <typename E, bool VEC>
__global__ void __launch_bounds__(256) gating_kernel(Gates gt, int64_t n, int HV, float *__restrict__ g,
                                                    float *__restrict__ beta) {
    const E *__restrict__ a = (const E *)gt.a;
    const E *__restrict__ b = (const E *)gt.b;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
    for (int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; i0 < n; i0 += stride) {
        float av[8], bv[8];
        const bool full = VEC && i0 + 8 <= n;
        if (full) {
            if constexpr (sizeof(E) == 2) {
                const bf16x8 x = *(const bf16x8 *)(a + i0), y = *(const bf16x8 *)(b + i0);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    av[e] = (float)x[e];
                    bv[e] = (float)y[e];
                }
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f32x4 x = *(const f32x4 *)(a + i0 + 4 * h), y = *(const f32x4 *)(b + i0 + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        av[4 * h + e] = x[e];
                        bv[4 * h + e] = y[e];
                    }
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                av[e] = i0 + e < n ? to_f(a[i0 + e]) : 0.f;
                bv[e] = i0 + e < n ? to_f(b[i0 + e]) : 0.f;
            }
        }
        int j = (int)(i0 % HV);
        float gv[8], bt[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            gv[e] = gate_g(av[e], -expf(gt.A_log[j]), gt.dt_bias[j]);
            bt[e] = gate_beta(bv[e]);
            j = j + 1 == HV ? 0 : j + 1;
        }
        if (full) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                *(f32x4 *)(g + i0 + 4 * h) = f32x4{gv[4 * h], gv[4 * h + 1], gv[4 * h + 2], gv[4 * h + 3]};
                *(f32x4 *)(beta + i0 + 4 * h) = f32x4{bt[4 * h], bt[4 * h + 1], bt[4 * h + 2], bt[4 * h + 3]};
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (i0 + e < n) {
                    g[i0 + e] = gv[e];
                    beta[i0 + e] = bt[e];
                }
        }
    }
}

}  // namespace

hipError_t launch_gating(const Gates &gt, int64_t rows, int HV, int dtype, float *g, float *beta,
                         hipStream_t stream, Profiler *prof) {
    const int64_t n = rows * HV;
    if (n == 0) return hipSuccess;
    // one pass of 8 elements per thread where that takes fewer than 8192
    // workgroups; the loop covers the rest
    const int64_t want = (n + 2047) / 2048;
    const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
    // 16-byte vector accesses when every buffer allows them
    const bool vec = (((uintptr_t)gt.a | (uintptr_t)gt.b | (uintptr_t)g | (uintptr_t)beta) & 15u) == 0;
    if (prof) prof->begin(kGatingKernel, stream);
    if (dtype == 0) {
        if (vec) gating_kernel<bf16, true><<<grid, 256, 0, stream>>>(gt, n, HV, g, beta);
        else gating_kernel<bf16, false><<<grid, 256, 0, stream>>>(gt, n, HV, g, beta);
    } else {
        if (vec) gating_kernel<float, true><<<grid, 256, 0, stream>>>(gt, n, HV, g, beta);
        else gating_kernel<float, false><<<grid, 256, 0, stream>>>(gt, n, HV, g, beta);
    }
    const hipError_t err = hipGetLastError();
    if (prof) prof->end(kGatingKernel, stream);
    return err;
}

}  // namespace gdn
