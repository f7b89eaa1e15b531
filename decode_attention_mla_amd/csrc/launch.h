// Internal to the library: the launch interface between the host side of
// the C ABI (mla_api.cpp) and the kernels (mla_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mla_decode.h"

namespace mla {

// Events recorded around the split and combine launches of one call.
struct LaunchEvents {
    hipEvent_t split_start, split_stop, comb_start, comb_stop;
    bool combine_ran;  // set by launch_decode
};

// Row-block groups (of up to four 16-row blocks) that one split launch runs
// side by side for n_rb row blocks.
int groups_per_launch(int n_rb);

// Default number of key ranges per launch: the CU count over the row-block
// groups of one launch, so that the larger launch fills the GPU once.
int default_splits(int cu_count, int n_rb);

// Bytes of split workspace for `splits` key ranges and n_rb row blocks: two
// partial slots per range, each n_rb x 16 rows of 512 floats of O and one of
// LSE.
size_t workspace_bytes(int splits, int n_rb);

// Enqueue the split kernel(s) and, when some sequence is split across key
// ranges, the combine kernel on `stream`, with the partials in `ws`
// (workspace_bytes(splits, n_rb) bytes).  The arguments must already have
// passed the host checks of mla_decode.  `p_bf16`: P enters the PV product
// as one bf16 value in the kernels whose row blocks share key steps (see
// MLA_OPT_P_BF16).  `ev` (may be NULL) gets its events recorded.  On failure
// returns the HIP error and names the launch in *what.
hipError_t launch_decode(hipStream_t stream, int splits, int64_t min_chunk, bool p_bf16, void *ws, const void *q,
                         const void *kv_cache, const int32_t *block_table, const int32_t *seqlens, float scale,
                         float *out, float *lse, const mla_problem *p, LaunchEvents *ev, const char **what);

}  // namespace mla
