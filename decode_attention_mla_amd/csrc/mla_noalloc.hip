// mla_decode_noalloc: the attention of mla_decode for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid it).
//
// The split partials go to `scratch`, a file-scope device array of a fixed
// size that every GPU the library runs on holds from module load until the
// process ends.  Its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// ever handed to the kernels: in host code the array's name is a host-side
// stand-in, not a device address.  The call allocates and frees nothing,
// synchronizes nothing and needs no context; it launches the same kernels
// as mla_decode.
//
// Every call on one GPU shares that GPU's array, which keeps the last call's
// partials; nothing in it needs to start at zero (each partial the combine
// reads is written by the same call).  Calls that can overlap on one GPU
// (other streams, other host threads) race on it.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "context.h"
#include "launch.h"
#include "mla_decode.h"
#include "plan.h"

namespace {

using mla_host::fail;
using mla_host::hip_fail;

// Room for 2048 partial row blocks of 16 rows x (512 + 1) floats: two slots
// for each of 256 key ranges at four row blocks (s_q * heads = 64, e.g.
// 4 tokens x 16 heads), the default split plan of a 256-CU device up to that
// size.  64.1 MiB.
constexpr size_t kScratchRowBlocks = 2048;
constexpr size_t kScratchBytes = kScratchRowBlocks * 16 * (MLA_HEAD_DIM_V + 1) * sizeof(float) + 256;

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
    void *ptr = nullptr;  // device address of `scratch` on this device
    int cu_count = 0;
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

// The scratch address and CU count of the current device `dev`, looked up on
// the first call on that device.
int device_scratch(int dev, DeviceScratch *out) {
    if (dev < 0 || dev >= kMaxDevices) return fail(nullptr, MLA_ERR_UNSUPPORTED, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceScratch &d = g_dev[dev];
    if (!d.ptr) {
        void *ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(nullptr, e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(nullptr, MLA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return hip_fail(nullptr, e, "hipDeviceGetAttribute");
        d.cu_count = cus > 0 ? cus : 256;
        d.ptr = ptr;
    }
    *out = d;
    return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_noalloc_scratch_bytes(void) { return kScratchBytes; }

int mla_decode_noalloc(void *stream, const void *q, const void *kv_cache, const int32_t *block_table,
                       const int32_t *seqlens, float scale, float *out, float *lse, const mla_problem *p) {
    int rc = mla_validate(q, kv_cache, block_table, seqlens, scale, out, lse, p);
    if (rc != MLA_OK) return rc;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(nullptr, e, "hipGetDevice");
    DeviceScratch ds;
    rc = device_scratch(dev, &ds);
    if (rc != MLA_OK) return rc;

    // The default split plan when its partials fit the array, else the
    // largest split count that does (same result up to rounding).
    const int n_rb = p->s_q * p->num_heads / 16;
    const size_t max_splits = kScratchRowBlocks / (2 * (size_t)n_rb);
    if (max_splits < 1)
        return fail(nullptr, MLA_ERR_WORKSPACE,
                    "s_q * num_heads = %d needs %zu bytes of scratch for one key range; the static "
                    "scratch holds %zu (at most %zu query rows)",
                    p->s_q * p->num_heads, mla::workspace_bytes(1, n_rb), kScratchBytes,
                    kScratchRowBlocks / 2 * 16);
    int splits = mla::default_splits(ds.cu_count, n_rb);
    if ((size_t)splits > max_splits) splits = (int)max_splits;
    const size_t need = mla::workspace_bytes(splits, n_rb);
    if (need > kScratchBytes)
        return fail(nullptr, MLA_ERR_WORKSPACE, "needs %zu bytes of scratch, the static scratch holds %zu", need,
                    kScratchBytes);

    const char *what = "launch";
    e = mla::launch_decode((hipStream_t)stream, splits, mla::kDefaultMinChunk, false, ds.ptr, q, kv_cache,
                           block_table, seqlens, scale, out, lse, p, nullptr, &what);
    return e == hipSuccess ? MLA_OK : hip_fail(nullptr, e, what);
}

}  // extern "C"
