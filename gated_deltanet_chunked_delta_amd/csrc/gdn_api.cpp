// C-ABI entry points (include/gdn.h): host-side argument checks, workspace
// carving and the launch sequence.  Nothing here touches the device before
// every check has passed.
#include <limits.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "gdn.h"
#include "gdn_internal.h"

namespace gdn {
// Gate-input gradients (gdn_gating.hip).
size_t gating_bwd_workspace_bytes(int64_t rows, int HV);
hipError_t launch_gating_bwd(const Gates &gt, int64_t rows, int HV, int dtype, const float *dg, const float *dbeta,
                             void *da, void *db, float *dA_log, float *ddt_bias, float *ws, hipStream_t stream);
}  // namespace gdn

namespace gdn {

int elem_bytes(int dtype) { return dtype == GDN_BF16 ? 2 : dtype == GDN_F32 ? 4 : 0; }

}  // namespace gdn

namespace {

int check_shape(const gdn_shape *s) {
    if (!s) return GDN_ERR_NULL;
    if (s->B < 0 || s->T < 0 || s->N < 0 || s->H <= 0 || s->HV <= 0) return GDN_ERR_SHAPE;
    if (gdn::elem_bytes(s->dtype) == 0) return GDN_ERR_DTYPE;
    if ((s->K != 64 && s->K != 128) || (s->V != 64 && s->V != 128)) return GDN_ERR_UNSUPPORTED;
    if (s->HV % s->H != 0) return GDN_ERR_UNSUPPORTED;
    // every index the kernels form from these stays in range
    if ((int64_t)s->B * s->T > INT_MAX) return GDN_ERR_SHAPE;
    if ((int64_t)s->N * s->HV * (s->V / 16) > INT_MAX / 2) return GDN_ERR_SHAPE;
    return GDN_OK;
}

// Workspace for the sequence split of few, long, equal-length sequences
// (gdn_split.hip); 0 when these sizes are not split.
gdn::SplitPlan split_of(const gdn_shape &s) {
    if (s.N != s.B) return gdn::SplitPlan{};
    return gdn::plan_split(s.B, s.T, s.H, s.HV, s.K, s.V, gdn::elem_bytes(s.dtype));
}
// Workspace for the longest-first order of a packed batch of 2..kSeqOrderMax
// sequences (one int32 per sequence, 256-byte granules); 0 otherwise.
size_t order_bytes(const gdn_shape &s) {
    if (s.B != 1 || s.N < 2 || s.N > gdn::kSeqOrderMax) return 0;
    return ((size_t)s.N * 4 + 255) & ~(size_t)255;
}
size_t workspace_of(const gdn_shape &s) { return s.N != s.B ? order_bytes(s) : split_of(s).bytes; }

// Kernel timing hook (gdn_profile_enable / gdn_profile_read): HIP events
// recorded on the caller's stream around each kernel of every forward pass.
struct EventProfiler : gdn::Profiler {
    struct Rec {
        int kind;
        hipEvent_t a, b;
    };
    std::mutex mu;
    std::atomic<bool> on{false};
    std::vector<hipEvent_t> pool;
    std::vector<Rec> pending;
    hipEvent_t open[gdn::kNumKernelKinds] = {};
    double total_ms[gdn::kNumKernelKinds] = {};
    int64_t launches[gdn::kNumKernelKinds] = {};

    hipEvent_t take() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        // No system-scope fence: the timing events must not flush caches
        // between the launches they bracket.
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
        return e;
    }
    void begin(int kind, hipStream_t st) override {
        hipEvent_t e = take();
        if (e) (void)hipEventRecord(e, st);
        open[kind] = e;
    }
    void end(int kind, hipStream_t st) override {
        hipEvent_t e = take();
        if (e) (void)hipEventRecord(e, st);
        if (open[kind] && e) pending.push_back(Rec{kind, open[kind], e});
        open[kind] = nullptr;
    }
    void drain() {
        for (const Rec &r : pending) {
            float ms = 0.f;
            if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
                total_ms[r.kind] += ms;
                launches[r.kind] += 1;
            }
            pool.push_back(r.a);
            pool.push_back(r.b);
        }
        pending.clear();
    }
    void reset() {
        drain();
        for (int i = 0; i < gdn::kNumKernelKinds; ++i) {
            total_ms[i] = 0.0;
            launches[i] = 0;
        }
    }
};

EventProfiler g_prof;

// Runs launch(prof) with the timing hook while it is enabled, else with none;
// the hook's lock is taken only while timing is on.
template <class F>
hipError_t with_profiler(F &&launch) {
    if (!g_prof.on.load(std::memory_order_acquire)) return launch(nullptr);
    std::lock_guard<std::mutex> lock(g_prof.mu);
    return launch(g_prof.on.load(std::memory_order_relaxed) ? static_cast<gdn::Profiler *>(&g_prof) : nullptr);
}

const gdn_gates kNoGates = {nullptr, nullptr, nullptr, nullptr};

// Raw gate inputs: all four pointers given, a and b 4-byte aligned.
int check_gates(const gdn_gates &gt) {
    if (!gt.A_log || !gt.dt_bias || !gt.a || !gt.b) return GDN_ERR_NULL;
    if ((((uintptr_t)gt.a | (uintptr_t)gt.b) & 3u) != 0) return GDN_ERR_ALIGN;
    return GDN_OK;
}

// A state pool: data, indices given, a known dtype, at least one slot, data
// aligned for the decode kernel's vector accesses (16 bytes in fp32, 8 in bf16).
int check_pool(const gdn_state_pool &pl) {
    if (!pl.data || !pl.indices) return GDN_ERR_NULL;
    if (pl.dtype != GDN_BF16 && pl.dtype != GDN_F32) return GDN_ERR_DTYPE;
    if (pl.pool_size < 1) return GDN_ERR_SHAPE;
    if (((uintptr_t)pl.data & (pl.dtype == GDN_BF16 ? 7u : 15u)) != 0) return GDN_ERR_ALIGN;
    return GDN_OK;
}

// The prefill entry points: g / beta given (gates == null) or gates computed
// in the kernel from the raw inputs (gates != null).
int chunk_fwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
              const gdn_gates *gates, float scale, int use_l2norm, const float *initial_state,
              const int32_t *cu_seqlens, void *out, float *final_state, const gdn_shape *shape, void *workspace,
              size_t workspace_bytes, void *stream, const gdn_state_pool *pool = nullptr,
              bool check_only = false) {
    const int st = check_shape(shape);
    if (st != GDN_OK) return st;
    const gdn_shape &s = *shape;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen ? s.B != 1 : s.N != s.B) return GDN_ERR_SHAPE;
    const bool any_tokens = (int64_t)s.B * s.T > 0;
    if (any_tokens && (!q || !k || !v || !out)) return GDN_ERR_NULL;
    if (any_tokens && !gates && (!g || !beta)) return GDN_ERR_NULL;
    // the kernels move q, k, v, out and the states in 16-byte pieces and read
    // g, beta and cu_seqlens in 4-byte words
    const uintptr_t a16 = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out |
                          (uintptr_t)initial_state | (uintptr_t)final_state;
    const uintptr_t a4 = (uintptr_t)g | (uintptr_t)beta | (uintptr_t)cu_seqlens;
    if ((a16 & 15u) != 0 || (a4 & 3u) != 0) return GDN_ERR_ALIGN;
    if (any_tokens && gates) {
        const int gs = check_gates(*gates);
        if (gs != GDN_OK) return gs;
        // bf16 gate inputs are read through their aligned 4-byte word, whose
        // half is the same for every token only when HV is even
        if (s.dtype == GDN_BF16 && s.HV % 2 != 0) return GDN_ERR_UNSUPPORTED;
    }
    if (pool && s.N > 0) {
        const int ps = check_pool(*pool);
        if (ps != GDN_OK) return ps;
    }
    if (check_only) return GDN_OK;
    // The split runs only where it applies and the caller gave the workspace
    // for it (256-byte aligned); otherwise the sequences run unsplit.
    gdn::SplitPlan split;
    if (!pool && !varlen) {
        split = split_of(s);
        if (split.active && (!workspace || workspace_bytes < split.bytes || ((uintptr_t)workspace & 255u) != 0))
            split.active = false;
    }
    // A packed batch takes its sequences longest first where the caller gave
    // the workspace for the order (4-byte aligned); otherwise in index order.
    // Either way every sequence is computed the same, so the results are equal.
    const size_t ob = varlen ? order_bytes(s) : 0;
    const bool ordered = ob > 0 && workspace && workspace_bytes >= (size_t)s.N * 4 && ((uintptr_t)workspace & 3u) == 0;

    gdn::Params p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    if (any_tokens && gates) p.gates = gdn::Gates{gates->A_log, gates->dt_bias, gates->a, gates->b};
    p.initial_state = initial_state;
    p.cu_seqlens = cu_seqlens;
    p.out = out;
    p.final_state = final_state;
    p.B = s.B;
    p.T = s.T;
    p.H = s.H;
    p.HV = s.HV;
    p.K = s.K;
    p.V = s.V;
    p.N = s.N;
    p.scale = scale;
    p.use_l2norm = use_l2norm ? 1 : 0;
    if (ordered) p.seq_order = (const int32_t *)workspace;
    if (pool && s.N > 0) {
        p.initial_state = pool->read_initial ? (const float *)pool->data : nullptr;
        p.final_state = (float *)pool->data;
        p.state_indices = pool->indices;
        p.pool_size = pool->pool_size;
        p.state_bf16 = pool->dtype == GDN_BF16;
    }
    const hipError_t err = with_profiler([&](gdn::Profiler *prof) {
        return split.active ? gdn::launch_split(p, s.dtype, split, workspace, (hipStream_t)stream, prof)
                            : gdn::launch_forward(p, s.dtype, (hipStream_t)stream, prof);
    });
    return err == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

// The decode entry points, as chunk_fwd.
int recurrent_update(const void *q, const void *k, const void *v, const float *g, const float *beta,
                     const gdn_gates *gates, float scale, int use_l2norm, float *state_pool,
                     const int32_t *state_indices, void *out, const gdn_decode_shape *shape, void *stream,
                     bool state_bf16 = false) {
    if (!shape) return GDN_ERR_NULL;
    const gdn_decode_shape &s = *shape;
    if (s.N < 0 || s.H <= 0 || s.HV <= 0 || s.pool_size < 0) return GDN_ERR_SHAPE;
    if (gdn::elem_bytes(s.dtype) == 0) return GDN_ERR_DTYPE;
    if ((s.K != 64 && s.K != 128) || (s.V != 64 && s.V != 128) || s.HV % s.H != 0) return GDN_ERR_UNSUPPORTED;
    if (s.N > 0 && s.pool_size < 1) return GDN_ERR_SHAPE;
    // grid size and every index the kernel forms stay in range
    if ((int64_t)s.N * s.HV > INT_MAX) return GDN_ERR_SHAPE;
    if (s.N > 0 && (!q || !k || !v || !state_pool || !state_indices || !out)) return GDN_ERR_NULL;
    if (s.N > 0 && !gates && (!g || !beta)) return GDN_ERR_NULL;
    if (s.N > 0 && gates) {
        const int gs = check_gates(*gates);
        if (gs != GDN_OK) return gs;
    }
    if (s.N > 0 && ((uintptr_t)state_pool & (state_bf16 ? 7u : 15u)) != 0) return GDN_ERR_ALIGN;

    gdn::DecodeParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    if (s.N > 0 && gates) p.gates = gdn::Gates{gates->A_log, gates->dt_bias, gates->a, gates->b};
    p.state_pool = state_pool;
    p.state_indices = state_indices;
    p.out = out;
    p.N = s.N;
    p.H = s.H;
    p.HV = s.HV;
    p.K = s.K;
    p.V = s.V;
    p.pool_size = s.pool_size;
    p.scale = scale;
    p.use_l2norm = use_l2norm ? 1 : 0;
    p.state_bf16 = state_bf16 ? 1 : 0;
    const hipError_t err =
        with_profiler([&](gdn::Profiler *prof) { return gdn::launch_recurrent(p, s.dtype, (hipStream_t)stream, prof); });
    return err == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

// The backward pass.  The workspace slots are sized for packed sequences when
// B == 1 (ceil(T/64) + N chunks bound the chunks of any N sequences of T tokens
// in all) and for B equal-length sequences otherwise.
gdn::BwdPlan bwd_plan_of(const gdn_shape &s) {
    return gdn::plan_backward(s.B, s.T, s.H, s.HV, s.K, s.V, s.N, s.B == 1);
}

int chunk_bwd(const void *q, const void *k, const void *v, const float *g, const float *beta, const void *dout,
              const float *dht, float scale, int use_l2norm, const float *initial_state, const int32_t *cu_seqlens,
              void *dq, void *dk, void *dv, float *dg, float *dbeta, float *dh0, const gdn_shape *shape,
              void *workspace, size_t workspace_bytes, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN_OK) return st;
    const gdn_shape &s = *shape;
    const bool varlen = cu_seqlens != nullptr;
    if (varlen ? s.B != 1 : s.N != s.B) return GDN_ERR_SHAPE;
    const bool any_tokens = (int64_t)s.B * s.T > 0;
    if (any_tokens && (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta))
        return GDN_ERR_NULL;
    // the kernels read and write every tensor in 16-byte vectors
    const uintptr_t any = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)dout | (uintptr_t)dq |
                          (uintptr_t)dk | (uintptr_t)dv | (uintptr_t)dht | (uintptr_t)initial_state | (uintptr_t)dh0;
    if ((any & 15u) != 0) return GDN_ERR_ALIGN;
    const gdn::BwdPlan plan = bwd_plan_of(s);
    if (plan.nc_max < 0 || plan.bytes == 0) return GDN_ERR_SHAPE;
    if (!workspace || workspace_bytes < plan.bytes || ((uintptr_t)workspace & 255u) != 0) return GDN_ERR_WORKSPACE;
    if (s.N == 0 || (!any_tokens && !dh0)) return GDN_OK;

    gdn::BwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.dout = dout;
    p.dht = dht;
    p.initial_state = initial_state;
    p.cu_seqlens = cu_seqlens;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dg = dg;
    p.dbeta = dbeta;
    p.dh0 = dh0;
    p.B = s.B;
    p.T = s.T;
    p.H = s.H;
    p.HV = s.HV;
    p.K = s.K;
    p.V = s.V;
    p.N = s.N;
    p.scale = scale;
    p.use_l2norm = use_l2norm ? 1 : 0;
    const hipError_t err = with_profiler(
        [&](gdn::Profiler *prof) { return gdn::launch_backward(p, s.dtype, plan, workspace, (hipStream_t)stream, prof); });
    return err == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

size_t gdn_chunk_bwd_workspace_bytes(const gdn_shape *shape) {
    if (check_shape(shape) != GDN_OK) return 0;
    const gdn::BwdPlan plan = bwd_plan_of(*shape);
    return plan.nc_max < 0 ? 0 : plan.bytes;
}

int gdn_chunk_bwd(const void *q, const void *k, const void *v, const float *g, const float *beta, const void *dout,
                  const float *dht, float scale, int use_l2norm, const float *initial_state,
                  const int32_t *cu_seqlens, void *dq, void *dk, void *dv, float *dg, float *dbeta, float *dh0,
                  const gdn_shape *shape, void *workspace, size_t workspace_bytes, void *stream) {
    return chunk_bwd(q, k, v, g, beta, dout, dht, scale, use_l2norm, initial_state, cu_seqlens, dq, dk, dv, dg,
                     dbeta, dh0, shape, workspace, workspace_bytes, stream);
}

int gdn_profile_enable(int enable) {
    std::lock_guard<std::mutex> lock(g_prof.mu);
    g_prof.reset();
    g_prof.on.store(enable != 0, std::memory_order_release);
    return GDN_OK;
}

int gdn_profile_read(int max_kinds, const char **names, double *total_ms, int64_t *launches) {
    std::lock_guard<std::mutex> lock(g_prof.mu);
    g_prof.drain();
    const int n = max_kinds < gdn::kNumKernelKinds ? max_kinds : gdn::kNumKernelKinds;
    for (int i = 0; i < n; ++i) {
        if (names) names[i] = gdn::kernel_name(i);
        if (total_ms) total_ms[i] = g_prof.total_ms[i];
        if (launches) launches[i] = g_prof.launches[i];
    }
    return gdn::kNumKernelKinds;
}

size_t gdn_chunk_fwd_workspace_bytes(const gdn_shape *shape) {
    if (check_shape(shape) != GDN_OK) return 0;
    return workspace_of(*shape);
}

int gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
                  float scale, int use_l2norm, const float *initial_state, const int32_t *cu_seqlens,
                  void *out, float *final_state, const gdn_shape *shape, void *workspace,
                  size_t workspace_bytes, void *stream) {
    return chunk_fwd(q, k, v, g, beta, nullptr, scale, use_l2norm, initial_state, cu_seqlens, out, final_state,
                     shape, workspace, workspace_bytes, stream);
}

int gdn_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *g, const float *beta,
                          float scale, int use_l2norm, const float *initial_state, const int32_t *cu_seqlens,
                          void *out, float *final_state, const gdn_shape *shape, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN_OK) return st;
    // the split of equal-length sequences and the order of a packed batch
    // use scratch
    const size_t need = cu_seqlens ? order_bytes(*shape) : split_of(*shape).bytes;
    if (need > GDN_STATIC_SCRATCH_BYTES) return GDN_ERR_SCRATCH;
    void *scratch = nullptr;
    if (need > 0) {
        // chunk_fwd's checks come first, so that a call it refuses never
        // reaches the device; this second pass then runs it
        const int pre = chunk_fwd(q, k, v, g, beta, nullptr, scale, use_l2norm, initial_state, cu_seqlens, out,
                                  final_state, shape, nullptr, 0, stream, nullptr, /*check_only=*/true);
        if (pre != GDN_OK) return pre;
        if (gdn::static_scratch((hipStream_t)stream, &scratch) != hipSuccess) return GDN_ERR_LAUNCH;
    }
    return chunk_fwd(q, k, v, g, beta, nullptr, scale, use_l2norm, initial_state, cu_seqlens, out, final_state,
                     shape, scratch, need > 0 ? GDN_STATIC_SCRATCH_BYTES : 0, stream);
}

int gdn_chunk_fwd_gated(const void *q, const void *k, const void *v, const gdn_gates *gates, float scale,
                        int use_l2norm, const float *initial_state, const int32_t *cu_seqlens, void *out,
                        float *final_state, const gdn_shape *shape, void *workspace, size_t workspace_bytes,
                        void *stream) {
    return chunk_fwd(q, k, v, nullptr, nullptr, gates ? gates : &kNoGates, scale, use_l2norm, initial_state,
                     cu_seqlens, out, final_state, shape, workspace, workspace_bytes, stream);
}

int gdn_recurrent_update(const void *q, const void *k, const void *v, const float *g, const float *beta,
                         float scale, int use_l2norm, float *state_pool, const int32_t *state_indices,
                         void *out, const gdn_decode_shape *shape, void *stream) {
    return recurrent_update(q, k, v, g, beta, nullptr, scale, use_l2norm, state_pool, state_indices, out, shape,
                            stream);
}

int gdn_recurrent_update_gated(const void *q, const void *k, const void *v, const gdn_gates *gates, float scale,
                               int use_l2norm, float *state_pool, const int32_t *state_indices, void *out,
                               const gdn_decode_shape *shape, void *stream) {
    return recurrent_update(q, k, v, nullptr, nullptr, gates ? gates : &kNoGates, scale, use_l2norm, state_pool,
                            state_indices, out, shape, stream);
}

int gdn_chunk_fwd_pool(const void *q, const void *k, const void *v, const float *g, const float *beta,
                       const gdn_gates *gates, float scale, int use_l2norm, const gdn_state_pool *pool,
                       const int32_t *cu_seqlens, void *out, const gdn_shape *shape, void *workspace,
                       size_t workspace_bytes, void *stream) {
    if (!pool) return GDN_ERR_NULL;
    return chunk_fwd(q, k, v, g, beta, gates, scale, use_l2norm, nullptr, cu_seqlens, out, nullptr, shape,
                     workspace, workspace_bytes, stream, pool);
}

int gdn_recurrent_update_pool(const void *q, const void *k, const void *v, const float *g, const float *beta,
                              const gdn_gates *gates, float scale, int use_l2norm, const gdn_state_pool *pool,
                              void *out, const gdn_decode_shape *shape, void *stream) {
    if (!pool || !shape) return GDN_ERR_NULL;
    if (shape->N > 0) {
        const int ps = check_pool(*pool);
        if (ps != GDN_OK) return ps;
        if (shape->pool_size != pool->pool_size) return GDN_ERR_SHAPE;
    }
    return recurrent_update(q, k, v, g, beta, gates, scale, use_l2norm, (float *)pool->data, pool->indices, out,
                            shape, stream, pool->dtype == GDN_BF16);
}

int gdn_gating(const gdn_gates *gates, int64_t rows, int32_t HV, int32_t dtype, float *g, float *beta,
               void *stream) {
    if (rows < 0 || HV <= 0 || rows > ((int64_t)1 << 62) / HV) return GDN_ERR_SHAPE;
    if (gdn::elem_bytes(dtype) == 0) return GDN_ERR_DTYPE;
    if (rows == 0) return GDN_OK;
    if (!gates || !g || !beta) return GDN_ERR_NULL;
    const int st = check_gates(*gates);
    if (st != GDN_OK) return st;
    const gdn::Gates gt{gates->A_log, gates->dt_bias, gates->a, gates->b};
    const hipError_t err = with_profiler(
        [&](gdn::Profiler *prof) { return gdn::launch_gating(gt, rows, HV, dtype, g, beta, (hipStream_t)stream, prof); });
    return err == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

size_t gdn_gating_bwd_workspace_bytes(int64_t rows, int32_t HV) {
    if (rows < 0 || HV <= 0 || rows > ((int64_t)1 << 62) / HV) return 0;
    return gdn::gating_bwd_workspace_bytes(rows, HV);
}

int gdn_gating_bwd(const gdn_gates *gates, int64_t rows, int32_t HV, int32_t dtype, const float *dg,
                   const float *dbeta, void *da, void *db, float *dA_log, float *ddt_bias, void *workspace,
                   size_t workspace_bytes, void *stream) {
    if (rows < 0 || HV <= 0 || rows > ((int64_t)1 << 62) / HV) return GDN_ERR_SHAPE;
    if (gdn::elem_bytes(dtype) == 0) return GDN_ERR_DTYPE;
    if (!gates || !gates->A_log || !gates->dt_bias || !dA_log || !ddt_bias) return GDN_ERR_NULL;
    if (rows > 0) {
        if (!dg || !dbeta || !da || !db) return GDN_ERR_NULL;
        const int st = check_gates(*gates);
        if (st != GDN_OK) return st;
    }
    const size_t need = gdn::gating_bwd_workspace_bytes(rows, HV);
    if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15u) != 0))
        return GDN_ERR_WORKSPACE;
    const gdn::Gates gt{gates->A_log, gates->dt_bias, gates->a, gates->b};
    const hipError_t err = gdn::launch_gating_bwd(gt, rows, HV, dtype, dg, dbeta, da, db, dA_log, ddt_bias,
                                                  (float *)workspace, (hipStream_t)stream);
    return err == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

const char *gdn_status_str(int status) {
    switch (status) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
        case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: sizes negative or inconsistent";
        case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unknown dtype code";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: K/V not in {64,128} or HV % H != 0";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH: a kernel launch failed";
        case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: a pointer is not aligned as its argument requires";
        case GDN_ERR_SCRATCH:
            return "GDN_ERR_SCRATCH: the sizes need more than the static scratch (GDN_STATIC_SCRATCH_BYTES)";
        default: return "unknown gdn_status";
    }
}

}  // extern "C"
