// Stand-alone gate computation for gfx950: for rows x HV (token, value head)
// pairs, g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b) in fp32,
// the fused gating operator of the FastDeploy PR #7024 page ("Usage or
// Command", item 5).  The prefill and decode kernels compute the same gates
// themselves when they are given the raw inputs; this kernel serves callers
// that keep g and beta as tensors.
//
// Elementwise and bound by HBM (a, b in; g, beta out).  Each thread handles
// four consecutive elements with one pass over the whole range per launch.
#include "gdn_device.h"

namespace gdn {
namespace {

using namespace dev;

template <typename E>
__global__ void __launch_bounds__(256) gating_kernel(Gates gt, int64_t n, int HV, float *__restrict__ g,
                                                    float *__restrict__ beta) {
    const E *__restrict__ a = (const E *)gt.a;
    const E *__restrict__ b = (const E *)gt.b;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
    for (int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i0 < n; i0 += stride) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t i = i0 + e;
            if (i < n) {
                const int j = (int)(i % HV);
                g[i] = gate_g(to_f(a[i]), -expf(gt.A_log[j]), gt.dt_bias[j]);
                beta[i] = gate_beta(to_f(b[i]));
            }
        }
    }
}

}  // namespace

hipError_t launch_gating(const Gates &gt, int64_t rows, int HV, int dtype, float *g, float *beta,
                         hipStream_t stream, Profiler *prof) {
    const int64_t n = rows * HV;
    if (n == 0) return hipSuccess;
    // enough workgroups to fill the chip several times over; the loop covers the rest
    const int64_t want = (n + 1023) / 1024;
    const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
    if (prof) prof->begin(kGatingKernel, stream);
    if (dtype == 0)
        gating_kernel<bf16><<<grid, 256, 0, stream>>>(gt, n, HV, g, beta);
    else
        gating_kernel<float><<<grid, 256, 0, stream>>>(gt, n, HV, g, beta);
    const hipError_t err = hipGetLastError();
    if (prof) prof->end(kGatingKernel, stream);
    return err;
}

}  // namespace gdn
