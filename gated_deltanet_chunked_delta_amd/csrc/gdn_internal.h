// Internal interface between the C-ABI host code (gdn_api.cpp) and the HIP
// kernels (gdn_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace gdn {

constexpr int kChunk = 64;   // chunk length in tokens (the NPU page's tiling section: 64)

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
    int nc_max;                      // chunk records allotted in the workspace
    float scale;
    int use_l2norm;
    // workspace regions
    int32_t *seq_chunk_off;          // [N+1]  (varlen) first chunk record of each sequence
    int32_t *chunk_seq;              // [nc_max] (varlen) sequence of each chunk record
    float *decay;                    // [nc_max, HV]     exp(gamma_last)
    void *wneg;                      // [nc_max, HV, 64, K]  -W
    void *qs;                        // [nc_max, HV, 64, K]  scale rho e^gamma Q
    void *kt;                        // [nc_max, HV, K, 64]  (diag(r e^{gamma_L - gamma}) K)^T
    void *ut;                        // [nc_max, HV, V, 64]  U^T
    void *pm;                        // [nc_max, HV, 64, 64] gated causal scale rho r Q K^T
};

// Chunk records allotted for a problem (an upper bound of the real count).
int64_t chunk_records(int B, int T, int N, bool varlen);

// Bytes per element for a dtype code (2 = bf16, 4 = fp32), 0 if unknown.
int elem_bytes(int dtype);

// The kernels of one forward pass, for the timing hook.
enum KernelKind { kIndexKernel = 0, kPrepKernel = 1, kScanKernel = 2, kNumKernelKinds = 3 };
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

}  // namespace gdn
