// Split-KV plan arithmetic shared by the host mirror (mla_plan) and the
// kernels, which evaluate it per workgroup from the device seqlens.
//
// The keys of all sequences are laid end to end, each sequence padded to a
// multiple of kKeyBlock, and the line is cut into `splits` equal ranges of
// `chunk` keys.  When that line would start some sequence inside a range,
// each sequence with keys is followed by kSeqGap line keys that hold no key,
// and the ranges are cut from that line instead.  Workgroup g owns range
// [g*chunk, (g+1)*chunk).  A range meets a sequence in a segment.  A
// sequence inside one range is finished by that workgroup; otherwise every
// segment writes a partial (normalized O and log2-domain LSE) into slot
// 2*g + (segment does not start the range) and the combine kernel merges the
// parts.  Each range holds at most one segment that starts it and one that
// does not and is partial, so two slots per range suffice.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_decode.h"

namespace mla {

constexpr int kKeyBlock = 16;   // keys per wave block
constexpr int kChunkAlign = kKeyBlock;  // range sizes are multiples of this
// Default smallest range: one 16-key block for each of a workgroup's four
// waves.  Small problems then spread over more workgroups (their time is
// round trips, not bytes); large ones never reach it.
constexpr int64_t kDefaultMinChunk = 64;

__host__ __device__ inline int64_t padded_len(int64_t len) {
    return (len + kKeyBlock - 1) / kKeyBlock * kKeyBlock;
}

__host__ __device__ inline int64_t plan_chunk(int64_t total, int32_t splits, int64_t min_chunk) {
    int64_t per = (total + splits - 1) / splits;
    int64_t c = per > min_chunk ? per : min_chunk;
    c = (c + kChunkAlign - 1) / kChunkAlign * kChunkAlign;
    return c > 0 ? c : kChunkAlign;
}

// Line keys after every sequence with keys when the plain line would start
// some sequence inside a range.  A range that holds several segments pays a
// fixed cost for each one after the first (the merge of the one before, the
// query load, the refill of the pipeline), about what its workgroup streams
// of this many keys in the meantime, so such a range takes fewer real keys.
constexpr int64_t kSeqGap = MLA_PLAN_SEQ_GAP;
static_assert(kSeqGap % kKeyBlock == 0, "sequences keep starting on a block boundary");

// The line as the host evaluates it from host lengths (negative lengths count
// as empty); every workgroup evaluates the same from the device lengths.
struct HostLine {
    int64_t total;  // keys on the line, gaps included
    int64_t chunk;  // keys per range
    int64_t gap;    // line keys after each sequence with keys: 0 or kSeqGap
};

inline HostLine host_plan_line(const int32_t *lens, int32_t batch, int32_t splits, int64_t min_chunk) {
    int64_t total = 0, with_keys = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t lp = padded_len(lens[b] < 0 ? 0 : lens[b]);
        total += lp;
        with_keys += lp > 0 ? 1 : 0;
    }
    const int64_t chunk0 = plan_chunk(total, splits, min_chunk);
    bool inside = false;
    int64_t st = 0;
    for (int b = 0; b < batch; ++b) {
        const int64_t lp = padded_len(lens[b] < 0 ? 0 : lens[b]);
        inside = inside || (lp > 0 && st % chunk0 != 0);
        st += lp;
    }
    HostLine ln;
    ln.gap = inside ? kSeqGap : 0;
    ln.total = total + ln.gap * with_keys;
    ln.chunk = inside ? plan_chunk(ln.total, splits, min_chunk) : chunk0;
    return ln;
}

// Partial slot of the segment that sequence starting at `seq_start` has in
// range g (only meaningful when the sequence is split).
__host__ __device__ inline int32_t segment_slot(int32_t g, int64_t seq_start, int64_t chunk) {
    return 2 * g + (seq_start > (int64_t)g * chunk ? 1 : 0);
}

// Length clamped into what the cache can hold.
__host__ __device__ inline int32_t clamp_len(int32_t len, int64_t capacity) {
    if (len < 0) return 0;
    return (int64_t)len > capacity ? (int32_t)capacity : len;
}

}  // namespace mla
