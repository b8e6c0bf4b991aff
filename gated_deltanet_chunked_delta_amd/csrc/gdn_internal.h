// Internal interface between the C-ABI host code (gdn_api.cpp) and the HIP
// kernels (gdn_fused.hip, gdn_fused_ws.hip, gdn_recurrent.hip, gdn_gating.hip).  Not part of
// the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace gdn {

constexpr int kChunk = 64;   // chunk length in tokens (the NPU page's tiling section: 64)

// Raw gate inputs: when A_log is non-null the kernels compute
// g = -exp(A_log) softplus(a + dt_bias) and beta = sigmoid(b) per (token,
// value head) themselves, and the g / beta pointers are not read.
struct Gates {
    const float *A_log, *dt_bias;    // [HV]
    const void *a, *b;               // [rows, HV], the element type of q/k/v
};

// Everything a launch needs.  Pointers are device pointers.
struct Params {
    // inputs
    const void *q, *k, *v;           // [T_tot, H, K], [T_tot, H, K], [T_tot, HV, V]
    const float *g, *beta;           // [T_tot, HV]
    const float *initial_state;      // [N, HV, K, V] or null
    const int32_t *cu_seqlens;       // [N+1] or null (equal-length mode)
    // outputs
    void *out;                       // [T_tot, HV, V]
    float *final_state;              // [N, HV, K, V] or null
    // sizes
    int B, T, H, HV, K, V, N;
    float scale;
    int use_l2norm;
    Gates gates;                     // used instead of g, beta when gates.A_log != null
    // State pool: when state_indices is non-null, initial_state and
    // final_state point at one pool [pool_size, HV, K, V] and sequence n uses
    // slot state_indices[n] (a slot outside the pool: zero start, no store).
    // state_bf16: the states (pool or not) are stored as bf16.
    const int32_t *state_indices;
    int pool_size;
    int state_bf16;
};

// The kernels of one forward pass, for the timing hook.
// fused_kernel: single-role prefill kernel (the fp32 check mode);
// fused_ws_kernel: warp-specialized prefill kernel (bf16);
// recurrent_update_kernel: the decode step;
// gating_kernel: the stand-alone gate computation.
enum KernelKind { kFusedKernel = 0, kFusedWsKernel = 1, kRecurrentKernel = 2, kGatingKernel = 3,
                  kNumKernelKinds = 4 };
const char *kernel_name(int kind);

// Timing hook: when given, the launch sequence calls begin/end around each
// kernel it enqueues (on the same stream).
struct Profiler {
    virtual void begin(int kind, hipStream_t stream) = 0;
    virtual void end(int kind, hipStream_t stream) = 0;
    virtual ~Profiler() {}
};

// Enqueues the whole forward pass.  Returns the HIP error of the launches.
hipError_t launch_forward(const Params &p, int dtype, hipStream_t stream, Profiler *prof);

// Everything a decode-step launch needs.  Pointers are device pointers.
struct DecodeParams {
    const void *q, *k, *v;           // [N, H, K], [N, H, K], [N, HV, V]
    const float *g, *beta;           // [N, HV]
    Gates gates;                     // used instead of g, beta when gates.A_log != null
    float *state_pool;               // [pool_size, HV, K, V], updated in place (bf16 when state_bf16)
    const int32_t *state_indices;    // [N]
    void *out;                       // [N, HV, V]
    int N, H, HV, K, V, pool_size;
    float scale;
    int use_l2norm;
    int state_bf16;
};

// Enqueues the decode step (gdn_recurrent.hip).
hipError_t launch_recurrent(const DecodeParams &p, int dtype, hipStream_t stream, Profiler *prof);

// Enqueues the stand-alone gate computation (gdn_gating.hip) for rows x HV
// gates into g and beta.
hipError_t launch_gating(const Gates &gt, int64_t rows, int HV, int dtype, float *g, float *beta,
                         hipStream_t stream, Profiler *prof);

// The single-role fused kernel's launch (gdn_fused.hip).
hipError_t launch_fused(const Params &p, int dtype, hipStream_t stream);
// The warp-specialized bf16 kernel's launch (gdn_fused_ws.hip).
hipError_t launch_fused_ws(const Params &p, hipStream_t stream);

}  // namespace gdn
