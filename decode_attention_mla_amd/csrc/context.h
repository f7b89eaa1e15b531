// Internal to the library: the context object and the error helpers that
// the library's translation units share.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>
#include <vector>

#include "mla_decode.h"
#include "plan.h"

struct mla_ctx {
    hipStream_t stream = nullptr;
    int device = 0;
    int cu_count = 256;
    int64_t opt_splits = 0;
    int64_t opt_min_chunk = mla::kDefaultMinChunk;
    bool timing = false;
    bool p_bf16 = false;  // MLA_OPT_P_BF16
    // Split workspace: either the library's own (allocated on first use or
    // by mla_ctx_reserve, grown by allocating a larger one) or a caller's
    // buffer (mla_ctx_set_workspace).  A replaced buffer of the library's
    // own is kept until the context is destroyed, so that work already
    // enqueued or captured into a graph never sees it freed.
    void *ws = nullptr;
    size_t ws_bytes = 0;
    bool ws_caller = false;
    std::vector<void *> ws_retired;
    std::string err;
    // Event pairs around recorded launches: kind 0 = split, 1 = combine.
    struct Timed {
        hipEvent_t start, stop;
        int kind;
    };
    std::vector<Timed> timed;
    std::vector<hipEvent_t> spare;
};

namespace mla_host {

// The calling thread's last error of a context-free call.
inline std::string &thread_error() {
    static thread_local std::string e;
    return e;
}

// Record the message on ctx (or the calling thread when ctx is NULL) and
// return code.
inline int fail(mla_ctx *ctx, int code, const char *fmt, ...) __attribute__((format(printf, 3, 4)));
inline int fail(mla_ctx *ctx, int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (ctx) ctx->err = buf;
    else thread_error() = buf;
    return code;
}

inline int hip_fail(mla_ctx *ctx, hipError_t e, const char *what) {
    return fail(ctx, MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace mla_host
