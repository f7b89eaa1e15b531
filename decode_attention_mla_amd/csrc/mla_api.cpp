// Host side of the C ABI (include/mla_decode.h): argument checks, the
// context and its options, the split workspace (the context's own or a
// caller's), the host mirror of the split plan, and per-launch timing.  The
// kernels and their launch configuration are in mla_kernels.hip.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "context.h"
#include "launch.h"
#include "mla_decode.h"
#include "plan.h"

namespace {

using mla_host::fail;
using mla_host::hip_fail;

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15) == 0; }

int check(mla_ctx *ctx, const void *q, const void *kv, const int32_t *block_table,
          const int32_t *seqlens, float scale, const float *out, const float *lse,
          const mla_problem *p) {
    if (!p) return fail(ctx, MLA_ERR_INVALID_ARG, "problem description is NULL");
    if (!q || !kv || !seqlens || !out || !lse)
        return fail(ctx, MLA_ERR_INVALID_ARG, "q, kv_cache, seqlens, out and lse must be non-NULL");
    if (p->batch < 1) return fail(ctx, MLA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", p->batch);
    if (p->s_q < 1) return fail(ctx, MLA_ERR_INVALID_ARG, "s_q must be >= 1 (got %d)", p->s_q);
    if (p->num_heads < 1 || p->num_heads % 16)
        return fail(ctx, MLA_ERR_UNSUPPORTED, "num_heads must be a positive multiple of 16 (got %d)",
                    p->num_heads);
    if (p->head_dim_qk != MLA_HEAD_DIM_QK || p->head_dim_v != MLA_HEAD_DIM_V)
        return fail(ctx, MLA_ERR_UNSUPPORTED, "head dims must be %d/%d (got %d/%d)", MLA_HEAD_DIM_QK,
                    MLA_HEAD_DIM_V, p->head_dim_qk, p->head_dim_v);
    if ((int64_t)p->s_q * p->num_heads > (1 << 20))
        return fail(ctx, MLA_ERR_UNSUPPORTED, "s_q * num_heads too large");
    if (!isfinite(scale)) return fail(ctx, MLA_ERR_INVALID_ARG, "scale must be finite");
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out) || ((uintptr_t)lse & 3))
        return fail(ctx, MLA_ERR_INVALID_ARG,
                    "q, kv_cache and out must be 16-byte aligned, lse 4-byte aligned");
    int64_t capacity;
    if (p->page_size == 0) {
        if (block_table)
            return fail(ctx, MLA_ERR_INVALID_ARG, "block_table given but page_size is 0 (contiguous)");
        if (p->kv_capacity < 1 || p->kv_capacity > (int64_t)INT32_MAX)
            return fail(ctx, MLA_ERR_INVALID_ARG, "kv_capacity must be in [1, 2^31) (got %lld)",
                        (long long)p->kv_capacity);
        capacity = p->kv_capacity;
    } else {
        if (p->page_size < 0 || p->page_size % MLA_KEY_BLOCK)
            return fail(ctx, MLA_ERR_UNSUPPORTED, "page_size must be a positive multiple of %d (got %d)",
                        MLA_KEY_BLOCK, p->page_size);
        if (!block_table) return fail(ctx, MLA_ERR_INVALID_ARG, "paged layout needs a block_table");
        if (p->num_pages < 1 || p->max_pages < 1)
            return fail(ctx, MLA_ERR_INVALID_ARG, "num_pages and max_pages must be >= 1");
        capacity = (int64_t)p->max_pages * p->page_size;
        if (capacity > (int64_t)INT32_MAX)
            return fail(ctx, MLA_ERR_INVALID_ARG, "max_pages * page_size must be < 2^31");
    }
    if (p->seqlens_host) {
        for (int b = 0; b < p->batch; ++b) {
            const int32_t L = p->seqlens_host[b];
            if (L < p->s_q || (int64_t)L > capacity)
                return fail(ctx, MLA_ERR_INVALID_ARG,
                            "seqlens[%d] = %d outside [s_q = %d, capacity = %lld]", b, L, p->s_q,
                            (long long)capacity);
        }
    }
    return MLA_OK;
}

int64_t min_chunk_of(const mla_ctx *ctx) { return ctx->opt_min_chunk > 0 ? ctx->opt_min_chunk : mla::kDefaultMinChunk; }

}  // namespace

extern "C" {

const char *mla_version(void) { return "mla_decode 0.1 gfx950"; }

const char *mla_last_error(const mla_ctx *ctx) { return ctx ? ctx->err.c_str() : mla_host::thread_error().c_str(); }

int mla_validate(const void *q, const void *kv_cache, const int32_t *block_table,
                 const int32_t *seqlens, float scale, const float *out, const float *lse,
                 const mla_problem *p) {
    mla_host::thread_error().clear();
    return check(nullptr, q, kv_cache, block_table, seqlens, scale, out, lse, p);
}

int mla_plan(const int32_t *seqlens_host, int32_t batch, int32_t num_splits, int64_t min_chunk,
             mla_plan_segment *segs, int32_t max_segs, int32_t *n_segs, mla_plan_info *info) {
    using namespace mla;
    mla_host::thread_error().clear();
    if (!seqlens_host || batch < 1 || num_splits < 1 || !n_segs)
        return fail(nullptr, MLA_ERR_INVALID_ARG, "mla_plan: bad arguments");
    const HostLine ln = host_plan_line(seqlens_host, batch, num_splits, min_chunk);
    const int64_t total = ln.total, chunk = ln.chunk;
    int32_t count = 0, split_seqs = 0;
    int64_t st = 0;
    for (int b = 0; b < batch; ++b) {
        const int32_t L = seqlens_host[b] < 0 ? 0 : seqlens_host[b];
        const int64_t lp = padded_len(L);
        if (lp == 0) continue;
        const int g_first = (int)(st / chunk), g_last = (int)((st + lp - 1) / chunk);
        if (g_first != g_last) ++split_seqs;
        for (int g = g_first; g <= g_last; ++g) {
            const int64_t gs = (int64_t)g * chunk, ge = std::min(gs + chunk, total);
            if (segs && count < max_segs) {
                mla_plan_segment &s = segs[count];
                s.group = g;
                s.seq = b;
                s.key_begin = (int32_t)(std::max(gs, st) - st);
                s.key_end = (int32_t)std::min<int64_t>(std::min(ge, st + lp) - st, L);
                s.slot = g_first == g_last ? -1 : segment_slot(g, st, chunk);
            }
            ++count;
        }
        st += lp + ln.gap;
    }
    *n_segs = count;
    if (info) {
        info->chunk = chunk;
        info->total_keys = total;
        info->active_groups = (int32_t)((total + chunk - 1) / chunk);
        info->split_sequences = split_seqs;
        info->seq_gap = ln.gap;
    }
    if (segs && count > max_segs)
        return fail(nullptr, MLA_ERR_INVALID_ARG, "mla_plan: %d segments, room for %d", count, max_segs);
    return MLA_OK;
}

int mla_ctx_create(mla_ctx **out_ctx, void *stream) {
    mla_host::thread_error().clear();
    if (!out_ctx) return fail(nullptr, MLA_ERR_INVALID_ARG, "ctx out-pointer is NULL");
    *out_ctx = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(nullptr, e, "hipGetDevice");
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(nullptr, e, "hipDeviceGetAttribute");
    mla_ctx *ctx = new (std::nothrow) mla_ctx;
    if (!ctx) return fail(nullptr, MLA_ERR_WORKSPACE, "out of host memory");
    ctx->stream = (hipStream_t)stream;
    ctx->device = dev;
    ctx->cu_count = cus > 0 ? cus : 256;
    *out_ctx = ctx;
    return MLA_OK;
}

int mla_ctx_destroy(mla_ctx *ctx) {
    if (!ctx) return MLA_OK;
    int rc = MLA_OK;
    if ((ctx->ws && !ctx->ws_caller) || !ctx->ws_retired.empty()) {
        hipError_t e = hipStreamSynchronize(ctx->stream);
        if (e == hipSuccess && ctx->ws && !ctx->ws_caller) e = hipFree(ctx->ws);
        for (void *old : ctx->ws_retired)
            if (e == hipSuccess) e = hipFree(old);
        if (e != hipSuccess) rc = hip_fail(nullptr, e, "mla_ctx_destroy");
    }
    for (auto &t : ctx->timed) {
        (void)hipEventDestroy(t.start);
        (void)hipEventDestroy(t.stop);
    }
    for (auto e : ctx->spare) (void)hipEventDestroy(e);
    delete ctx;
    return rc;
}

int mla_ctx_set_option(mla_ctx *ctx, int option, int64_t value) {
    if (!ctx) return fail(nullptr, MLA_ERR_INVALID_ARG, "ctx is NULL");
    switch (option) {
    case MLA_OPT_NUM_SPLITS:
        if (value < 0 || value > (1 << 20)) return fail(ctx, MLA_ERR_INVALID_ARG, "bad split count");
        ctx->opt_splits = value;
        return MLA_OK;
    case MLA_OPT_MIN_CHUNK:
        if (value < 0 || value > ((int64_t)1 << 31)) return fail(ctx, MLA_ERR_INVALID_ARG, "bad min chunk");
        ctx->opt_min_chunk = value ? value : mla::kDefaultMinChunk;
        return MLA_OK;
    case MLA_OPT_KERNEL_TIMING:
        ctx->timing = value != 0;
        return MLA_OK;
    case MLA_OPT_P_BF16:
        if (value != 0 && value != 1) return fail(ctx, MLA_ERR_INVALID_ARG, "MLA_OPT_P_BF16 takes 0 or 1");
        ctx->p_bf16 = value != 0;
        return MLA_OK;
    default:
        return fail(ctx, MLA_ERR_INVALID_ARG, "unknown option %d", option);
    }
}

}  // extern "C"

namespace {

hipError_t take_event(mla_ctx *ctx, hipEvent_t *e) {
    if (!ctx->spare.empty()) {
        *e = ctx->spare.back();
        ctx->spare.pop_back();
        return hipSuccess;
    }
    return hipEventCreate(e);
}

// Event pairs around the split and combine launches of one call when timing
// is on (NULL when it is off or events are short).
mla::LaunchEvents *take_events(mla_ctx *ctx, mla::LaunchEvents *ev) {
    if (!ctx->timing) return nullptr;
    hipEvent_t *slots[4] = {&ev->split_start, &ev->split_stop, &ev->comb_start, &ev->comb_stop};
    for (int i = 0; i < 4; ++i) {
        if (take_event(ctx, slots[i]) != hipSuccess) {
            for (int j = 0; j < i; ++j) ctx->spare.push_back(*slots[j]);
            ctx->timing = false;
            return nullptr;
        }
    }
    ev->combine_ran = false;
    return ev;
}

// File the events of a call that was enqueued (or hand them back).
void keep_events(mla_ctx *ctx, mla::LaunchEvents *ev, bool launched) {
    if (!ev) return;
    if (launched) ctx->timed.push_back({ev->split_start, ev->split_stop, 0});
    else {
        ctx->spare.push_back(ev->split_start);
        ctx->spare.push_back(ev->split_stop);
    }
    if (launched && ev->combine_ran) ctx->timed.push_back({ev->comb_start, ev->comb_stop, 1});
    else {
        ctx->spare.push_back(ev->comb_start);
        ctx->spare.push_back(ev->comb_stop);
    }
}

int splits_for(const mla_ctx *ctx, int n_rb) {
    if (ctx->opt_splits > 0) return (int)ctx->opt_splits;
    return mla::default_splits(ctx->cu_count, n_rb);
}

// Make the context's workspace hold `need` bytes.  A caller's buffer is
// never replaced: a problem that needs more is refused.  The library's own
// buffer grows by allocating a larger one; the old one is retired (freed
// when the context is destroyed), so nothing enqueued or captured earlier
// ever finds it freed, and growing needs no synchronization.  Growing while
// the stream is being captured into a graph is refused: the allocation
// would not be part of the graph.
int ensure_workspace(mla_ctx *ctx, size_t need) {
    if (ctx->ws_bytes >= need) return MLA_OK;
    if (ctx->ws_caller)
        return fail(ctx, MLA_ERR_WORKSPACE,
                    "the caller's workspace holds %zu bytes, this problem needs %zu (mla_workspace_size)",
                    ctx->ws_bytes, need);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(ctx->stream, &cap);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamIsCapturing");
    if (cap != hipStreamCaptureStatusNone)
        return fail(ctx, MLA_ERR_WORKSPACE,
                    "workspace of %zu bytes needed while the stream is being captured: reserve it before the "
                    "capture (mla_ctx_reserve) or give the context a workspace (mla_ctx_set_workspace)",
                    need);
    void *fresh = nullptr;
    e = hipMalloc(&fresh, need);
    if (e != hipSuccess) return fail(ctx, MLA_ERR_WORKSPACE, "hipMalloc(%zu): %s", need, hipGetErrorString(e));
    if (ctx->ws) ctx->ws_retired.push_back(ctx->ws);
    ctx->ws = fresh;
    ctx->ws_bytes = need;
    return MLA_OK;
}

}  // namespace

extern "C" {

int mla_workspace_size(const mla_ctx *ctx, int32_t s_q, int32_t num_heads, size_t *bytes) {
    if (!ctx || !bytes) return fail(nullptr, MLA_ERR_INVALID_ARG, "ctx and bytes must be non-NULL");
    if (s_q < 1 || num_heads < 16 || num_heads % 16 || (int64_t)s_q * num_heads > (1 << 20))
        return fail(nullptr, MLA_ERR_INVALID_ARG, "bad s_q / num_heads (%d / %d)", s_q, num_heads);
    const int n_rb = s_q * num_heads / 16;
    *bytes = mla::workspace_bytes(splits_for(ctx, n_rb), n_rb);
    return MLA_OK;
}

int mla_ctx_set_workspace(mla_ctx *ctx, void *dev_ptr, size_t bytes) {
    if (!ctx) return fail(nullptr, MLA_ERR_INVALID_ARG, "ctx is NULL");
    ctx->err.clear();
    if (dev_ptr && ((uintptr_t)dev_ptr & 255))
        return fail(ctx, MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (dev_ptr && bytes == 0) return fail(ctx, MLA_ERR_INVALID_ARG, "workspace of 0 bytes");
    // The library's own buffer may still be in use by enqueued or captured
    // work: it is retired, freed when the context is destroyed.
    if (ctx->ws && !ctx->ws_caller) ctx->ws_retired.push_back(ctx->ws);
    ctx->ws = dev_ptr;
    ctx->ws_bytes = dev_ptr ? bytes : 0;
    ctx->ws_caller = dev_ptr != nullptr;
    return MLA_OK;
}

int mla_ctx_reserve(mla_ctx *ctx, int32_t s_q, int32_t num_heads) {
    if (!ctx) return fail(nullptr, MLA_ERR_INVALID_ARG, "ctx is NULL");
    ctx->err.clear();
    if (s_q < 1 || num_heads < 16 || num_heads % 16)
        return fail(ctx, MLA_ERR_INVALID_ARG, "bad s_q / num_heads");
    const int n_rb = s_q * num_heads / 16;
    return ensure_workspace(ctx, mla::workspace_bytes(splits_for(ctx, n_rb), n_rb));
}

}  // extern "C"

namespace {

// Enqueue the split kernel(s) and, when some sequence is split, the combine
// kernel on `stream`, with the partials in `ws` (mla::workspace_bytes(splits,
// n_rb) bytes).  Arguments are already checked.  `ectx` (may be NULL) takes
// the error message and, when timing is on, the launch events.
}  // namespace

extern "C" {

int mla_decode(mla_ctx *ctx, const void *q, const void *kv_cache, const int32_t *block_table,
               const int32_t *seqlens, float scale, float *out, float *lse, const mla_problem *p) {
    if (!ctx) return fail(nullptr, MLA_ERR_INVALID_ARG, "ctx is NULL");
    ctx->err.clear();
    int rc = check(ctx, q, kv_cache, block_table, seqlens, scale, out, lse, p);
    if (rc != MLA_OK) return rc;
    const int n_rb = p->s_q * p->num_heads / 16;
    const int splits = splits_for(ctx, n_rb);
    rc = ensure_workspace(ctx, mla::workspace_bytes(splits, n_rb));
    if (rc != MLA_OK) return rc;
    mla::LaunchEvents evs;
    mla::LaunchEvents *ev = take_events(ctx, &evs);
    const char *what = "launch";
    const hipError_t e = mla::launch_decode(ctx->stream, splits, min_chunk_of(ctx), ctx->p_bf16, ctx->ws, q,
                                            kv_cache, block_table, seqlens, scale, out, lse, p, ev, &what);
    keep_events(ctx, ev, e == hipSuccess);
    return e == hipSuccess ? MLA_OK : hip_fail(ctx, e, what);
}

int mla_ctx_kernel_times(mla_ctx *ctx, double *split_ms, int64_t *split_launches,
                         double *combine_ms, int64_t *combine_launches) {
    if (!ctx) return fail(nullptr, MLA_ERR_INVALID_ARG, "ctx is NULL");
    hipError_t e = hipStreamSynchronize(ctx->stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "hipStreamSynchronize");
    double ms[2] = {0.0, 0.0};
    int64_t n[2] = {0, 0};
    for (auto &t : ctx->timed) {
        float v = 0.f;
        e = hipEventElapsedTime(&v, t.start, t.stop);
        if (e != hipSuccess) return hip_fail(ctx, e, "hipEventElapsedTime");
        ms[t.kind] += v;
        n[t.kind] += 1;
        ctx->spare.push_back(t.start);
        ctx->spare.push_back(t.stop);
    }
    ctx->timed.clear();
    if (split_ms) *split_ms = ms[0];
    if (split_launches) *split_launches = n[0];
    if (combine_ms) *combine_ms = ms[1];
    if (combine_launches) *combine_launches = n[1];
    return MLA_OK;
}

}  // extern "C"
