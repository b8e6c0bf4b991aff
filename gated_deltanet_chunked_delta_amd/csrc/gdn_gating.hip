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

// ---------------------------------------------------------------------------
// Backward of the gate computation.  With x = a + dt_bias, s = sigmoid(x) and
// beta = sigmoid(b) (softplus' = sigmoid, sigmoid' = sigmoid (1 - sigmoid)):
//   da = dg * (-exp(A_log) s),  db = dbeta * beta (1 - beta),
//   dA_log[j] = sum_r dg g,  ddt_bias[j] = sum_r da  (over the rows r).
// gating_bwd_kernel: 64 rows per workgroup; lanes (row lane rl, column lane
// cl) walk the tile, write da, db and leave the workgroup's per-head sums in
// the workspace, reduced over the row lanes in a fixed order.
// gating_bwd_sum_kernel: one workgroup per head adds the workgroups' sums in a
// fixed order, so the result does not depend on scheduling.
// ---------------------------------------------------------------------------
constexpr int kGateTile = 64, kGateThreads = 256;

template <typename E>
__global__ void __launch_bounds__(kGateThreads) gating_bwd_kernel(Gates gt, int64_t rows, int HV,
                                                                 const float *__restrict__ dg,
                                                                 const float *__restrict__ dbeta, E *__restrict__ da,
                                                                 E *__restrict__ db, float *__restrict__ part) {
    __shared__ float red[2][kGateThreads];
    const E *__restrict__ a = (const E *)gt.a;
    const E *__restrict__ b = (const E *)gt.b;
    const int CL = HV < kGateThreads ? HV : kGateThreads;   // column lanes
    const int P = kGateThreads / CL;                          // row lanes
    const int cl = threadIdx.x % CL, rl = threadIdx.x / CL;
    const int64_t r0 = (int64_t)blockIdx.x * kGateTile;
    const int64_t r1 = r0 + kGateTile < rows ? r0 + kGateTile : rows;
    const int64_t nblk = gridDim.x;
    for (int j0 = 0; j0 < HV; j0 += CL) {   // the same trip count in every thread
        const int j = j0 + cl;
        float sA = 0.f, sD = 0.f;
        if (rl < P && j < HV) {
            const float negA = -expf(gt.A_log[j]), dtb = gt.dt_bias[j];
            for (int64_t r = r0 + rl; r < r1; r += P) {
                const int64_t e = r * HV + j;
                const float x = to_f(a[e]) + dtb;
                const float dgv = dg[e];
                const float dav = dgv * negA * gate_beta(x);
                const float bv = gate_beta(to_f(b[e]));
                da[e] = to_e<E>(dav);
                db[e] = to_e<E>(dbeta[e] * bv * (1.f - bv));
                sA = fmaf(dgv, gate_g(to_f(a[e]), negA, dtb), sA);
                sD += dav;
            }
        }
        red[0][threadIdx.x] = sA;
        red[1][threadIdx.x] = sD;
        __syncthreads();
        if (rl == 0 && j < HV) {
            float tA = 0.f, tD = 0.f;
            for (int u = 0; u < P; ++u) {
                tA += red[0][u * CL + cl];
                tD += red[1][u * CL + cl];
            }
            part[(int64_t)j * nblk + blockIdx.x] = tA;
            part[((int64_t)HV + j) * nblk + blockIdx.x] = tD;
        }
        __syncthreads();
    }
}

__global__ void __launch_bounds__(kGateThreads) gating_bwd_sum_kernel(const float *__restrict__ part, int64_t nblk,
                                                                     int HV, float *__restrict__ dA_log,
                                                                     float *__restrict__ ddt_bias) {
    __shared__ float red[2][kGateThreads];
    const int j = blockIdx.x;
    float tA = 0.f, tD = 0.f;
    for (int64_t u = threadIdx.x; u < nblk; u += kGateThreads) {
        tA += part[(int64_t)j * nblk + u];
        tD += part[((int64_t)HV + j) * nblk + u];
    }
    red[0][threadIdx.x] = tA;
    red[1][threadIdx.x] = tD;
    __syncthreads();
    for (int w = kGateThreads / 2; w > 0; w >>= 1) {   // fixed-order tree
        if ((int)threadIdx.x < w) {
            red[0][threadIdx.x] += red[0][threadIdx.x + w];
            red[1][threadIdx.x] += red[1][threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        dA_log[j] = red[0][0];
        ddt_bias[j] = red[1][0];
    }
}

}  // namespace

size_t gating_bwd_workspace_bytes(int64_t rows, int HV) {
    const int64_t nblk = (rows + kGateTile - 1) / kGateTile;
    return (size_t)(2 * nblk * (int64_t)HV) * sizeof(float);
}

hipError_t launch_gating_bwd(const Gates &gt, int64_t rows, int HV, int dtype, const float *dg, const float *dbeta,
                             void *da, void *db, float *dA_log, float *ddt_bias, float *ws, hipStream_t stream) {
    const int64_t nblk = (rows + kGateTile - 1) / kGateTile;
    if (nblk > 0) {
        if (dtype == 0)
            gating_bwd_kernel<bf16><<<(unsigned)nblk, kGateThreads, 0, stream>>>(gt, rows, HV, dg, dbeta, (bf16 *)da,
                                                                                 (bf16 *)db, ws);
        else
            gating_bwd_kernel<float><<<(unsigned)nblk, kGateThreads, 0, stream>>>(gt, rows, HV, dg, dbeta,
                                                                                  (float *)da, (float *)db, ws);
    }
    gating_bwd_sum_kernel<<<(unsigned)HV, kGateThreads, 0, stream>>>(ws, nblk, HV, dA_log, ddt_bias);
    return hipGetLastError();
}

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
