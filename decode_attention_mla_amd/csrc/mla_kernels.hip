// MLA decode attention for MI355X (gfx950): split kernel + combine kernel.
//
// What is computed ("FlashMLA-ETAP", gist.science technical summary,
// Methodology): S = Q K^T, P = softmax(S), O = P V over the shared latent
// KV rows (576 bf16 channels; V = the first 512).  The pages' design is for
// Hopper WGMMA, whose M >= 64 forces 16 heads to be padded (Problem
// Statement); their fix puts the KV length in the M slot (the transposed
// order S^T = K Q^T).  On CDNA4 the 16x16xK MFMA shapes take 16 heads with
// no padding, so the slot choice is free; this kernel still puts keys in M
// for QK^T, because then the score accumulator of a lane (one head, four
// keys) is exactly the B operand layout that the PV MFMA wants for P^T:
// P never leaves registers.
//
// Work decomposition (one workgroup = 4 waves of 64 lanes):
//   * A "row block" is 16 query rows: the 16 heads h0..h0+15 of one token.
//   * A workgroup owns key range g of the split plan (plan.h) and row
//     blocks 4y .. 4y+3 (nrb of them); range_and_group maps its id to (g, y)
//     so that the groups of one range share an XCD.  How they share the
//     keys is the kernel's mode (SplitMode): with one row block the four
//     waves split the keys, each an independent flash-decoding worker over
//     every 4th 16-key block with a private LDS ring and no barrier; with
//     two to four the waves of a key group compute the same 32- or 64-key
//     steps for different row blocks, fed through a shared two-slot LDS
//     ring, one barrier per step.
//   * At the end of a segment (the range's part of one sequence) the waves'
//     results are merged (through LDS where several waves share a row
//     block) into the final rows or into a partial for the combine kernel.
//
// Per 16 keys, per wave:
//   1. The 16 latent rows (1152 B each) arrive by direct-to-LDS 16-byte
//      loads, whole 128-byte lines, XOR-swizzled so that both operand reads
//      below are bank-conflict free; the next block or step is in flight
//      while the current one is computed.
//   2. S^T (16 keys x 16 heads) = 18 MFMA 16x16x32 bf16, fp32 accumulate;
//      the K operand is read from LDS, Q^T stays in registers.
//   3. Online softmax in fp32 (log2 domain); the accumulators are rescaled
//      only when a block's max passes the reference max by kMaxLag.
//   4. O^T (512 ch x 16 heads) += V^T P^T: 32 MFMA 16x16x32 bf16 per 16
//      keys, P split into bf16 hi + lo halves (so that rounding P costs no
//      accuracy) that the MFMA's k index carries; V^T comes from
//      transposing LDS reads.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <type_traits>
#include <utility>
#include <vector>

#include "launch.h"
#include "mla_decode.h"
#include "plan.h"

namespace mla {

constexpr int kDqk = MLA_HEAD_DIM_QK;          // 576
constexpr int kDv = MLA_HEAD_DIM_V;            // 512
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQkSteps = kDqk / 32;            // 18 MFMA k-steps of 32 channels
constexpr int kVSteps = kDv / 32;              // the first 16 of them are values
constexpr int kOutTiles = kDv / 16;            // 32 output tiles of 16 channels
constexpr int kBlockBytes = kKeyBlock * kDqk * 2;         // 18 KB: one 16-key block
constexpr int kStages = 2;                                 // LDS ring depth per wave
constexpr int kStageBytes = kWaves * kBlockBytes;          // one stage of all waves: 72 KB
// Shared rings (several row blocks per workgroup): per key group two 32-key
// steps of two blocks each, one computed while the next is in flight; the
// slot of parity s of key group kg is blocks 2kg, 2kg + 1 of stage array s.
constexpr int kPairBytes = 2 * kBlockBytes;
static_assert(2 * kPairBytes <= kStageBytes, "two key groups' slots fit in a stage array");
constexpr int kMergePitch = kDv + 4;           // floats per merge row (bank spread)
constexpr int kMergeWaveFloats = 16 * kMergePitch;          // one wave's O: 33 KB
static_assert(2 * kMergeWaveFloats * 4 + kWaves * 16 * 2 * 4 <= kStageBytes,
              "two waves' merge rows and the stats fit in one stage array");
constexpr int kCombineChannels = 32;           // channels per combine workgroup (64 and 128: slower)
constexpr int kCombineQuads = kCombineChannels / 4;       // threads per head, one float4 each
constexpr int kCombineThreads = 16 * kCombineQuads;      // 16 heads
constexpr int kCombineBatch = 16;              // partials merged per round trip
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNonTemporal = 2;                // cache-policy bits of a streaming load

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

struct Params {
    const uint16_t *q;
    const uint16_t *kv;
    const int32_t *block_table;
    const int32_t *seqlens;
    float *out;
    float *lse;
    float *part_o;     // [2*splits][n_rb][16][512]
    float *part_lse;   // [2*splits][n_rb][16], log2 domain
    int64_t kv_capacity;
    int64_t num_pages;
    int64_t capacity;  // keys one sequence can hold
    int64_t min_chunk;
    int32_t batch;
    int32_t s_q;
    int32_t heads;
    int32_t page_size;
    int32_t max_pages;
    int32_t n_rb;      // row blocks: s_q * heads / 16
    int32_t splits;    // key ranges (the split grid holds splits x n_groups workgroups when sized blind)
    int32_t y0;        // first row-block group of the launch
    int32_t n_groups;  // row-block groups in the launch (workgroups: key ranges x n_groups)
    int32_t line_gap;  // the plan's line keys after each sequence, from the host lengths;
                       // -1 without them (every workgroup then works it out)
    float scale_log2;  // scale * log2(e)
};

// ---------------------------------------------------------------- wave helpers

// Lane moves within the wave (DPP): row_shr:n takes lane i - n of the same
// 16-lane row, row_bcast:15 lane 15 of the row before, row_bcast:31 lane 31.
// Lanes whose row (row_mask) or 4-lane bank (bank_mask) is off, or whose
// source lies outside the row, read 0.  No LDS round trip is involved.
template <int kCtrl, int kRowMask, int kBankMask>
__device__ inline uint32_t dpp_move(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, kBankMask, true);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr3 = 0x113, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes: sums of up to four lanes back
// within a row, then of 4 and 8 back (the lanes that have them), then the
// row totals carried into the rows after them.
__device__ inline uint32_t wave_incl_scan_u32(uint32_t x) {
    uint32_t s = x + dpp_move<kRowShr1, 0xf, 0xf>(x);
    s += dpp_move<kRowShr2, 0xf, 0xf>(x);
    s += dpp_move<kRowShr3, 0xf, 0xf>(x);
    s += dpp_move<kRowShr4, 0xf, 0xe>(s);
    s += dpp_move<kRowShr8, 0xf, 0xc>(s);
    s += dpp_move<kRowBcast15, 0xa, 0xf>(s);
    s += dpp_move<kRowBcast31, 0xc, 0xf>(s);
    return s;
}

// Inclusive prefix sum of padded lengths (each below 2^32) over the lanes,
// as two 16-bit halves whose 64-lane sums fit in 32 bits.
__device__ inline int64_t wave_incl_scan_len(int64_t v) {
    const uint32_t hi = wave_incl_scan_u32((uint32_t)((uint64_t)v >> 16));
    const uint32_t lo = wave_incl_scan_u32((uint32_t)v & 0xffffu);
    return ((int64_t)hi << 16) + lo;
}

// Values that are the same in every lane, moved to scalar registers so that
// the compiler treats what depends on them as uniform.
__device__ inline int32_t uniform(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline int64_t uniform(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ inline int32_t lane_value(int32_t v, int j) { return __builtin_amdgcn_readlane(v, j); }
__device__ inline int64_t lane_value(int64_t v, int j) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, j);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), j);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Workgroup id -> key range g and row-block group grp.  The n_groups
// workgroups of one key range read the same keys.  Ids go round-robin over
// the 8 XCDs, so ids 8 apart share an XCD (and its L2) and are dispatched
// close together: each block of 8 x n_groups ids holds 8 ranges x n_groups
// groups, range-minor, so that the groups of a range read its keys in step
// and all but the first read them from that L2.  Ranges past the last
// multiple of 8 follow in plain order.  One group: g = id.
__device__ inline void range_and_group(int id, int n_groups, int ranges, int &g, int &grp) {
    const int full8 = ranges / 8 * 8;
    if (id < full8 * n_groups) {
        const int w = id % (8 * n_groups);
        g = id / (8 * n_groups) * 8 + w % 8;
        grp = w / 8;
    } else {
        const int t = id - full8 * n_groups, rem = ranges - full8;
        g = full8 + t % rem;
        grp = t / rem;
    }
}

__device__ inline int32_t seq_len(const Params &p, int b) {
    return clamp_len(p.seqlens[b], p.capacity);
}

// Length of sequence b0 + lane (0 past the batch); len0 holds it for the
// first 64 sequences, loaded once.
__device__ inline int32_t lane_len(const Params &p, int b0, int lane, int32_t len0) {
    const int bl = b0 + lane;
    return b0 == 0 ? len0 : (bl < p.batch ? seq_len(p, bl) : 0);
}

// The plan's line, the same arithmetic as host_plan_line: the padded lengths
// laid end to end, cut into p.splits ranges of `chunk` keys; when that line
// starts some sequence with keys inside a range, every sequence with keys is
// followed by kSeqGap line keys that hold no key, and the ranges are cut
// from that line.  len0: the lane's length among the first 64 sequences (0
// past the batch).
struct Line {
    int64_t total;  // keys on the line, gaps included
    int64_t chunk;  // keys per range
    int64_t gap;    // line keys after each sequence with keys: 0 or kSeqGap
};

// The gap of the line.  A launch with host lengths passes the host's choice
// (p.line_gap); without them every workgroup makes it from two passes over
// the lengths: the plain line's range size, then whether a sequence with keys
// starts inside one of its ranges.
__device__ inline int64_t plan_gap(const Params &p, int lane, int32_t len0) {
    if (p.line_gap >= 0) return p.line_gap;
    int64_t total = 0;
    for (int b0 = 0; b0 < p.batch; b0 += 64)
        total += lane_value(wave_incl_scan_len(padded_len(lane_len(p, b0, lane, len0))), 63);
    const int64_t chunk0 = plan_chunk(uniform(total), p.splits, p.min_chunk);
    bool inside = false;
    int64_t base = 0;
    for (int b0 = 0; b0 < p.batch && !inside; b0 += 64) {
        const int64_t lp = padded_len(lane_len(p, b0, lane, len0));
        const int64_t incl = wave_incl_scan_len(lp) + base;
        inside = __ballot(lp > 0 && (incl - lp) % chunk0 != 0) != 0;
        base = lane_value(incl, 63);
    }
    return inside ? kSeqGap : 0;
}

// Line keys of a sequence of padded length lp.
__device__ inline int64_t line_keys(int64_t lp, int64_t gap) { return lp > 0 ? lp + gap : 0; }

// The line, and where sequence b lies on it: its start and its padded length
// (every lane gets all of them; b < 0: none).  One pass over the lengths once
// the gap is known.
__device__ inline Line line_position(const Params &p, int b, int lane, int32_t len0, int64_t &start,
                                     int64_t &len) {
    Line ln;
    ln.gap = plan_gap(p, lane, len0);
    int64_t t = 0, s = 0, l = 0;
    for (int b0 = 0; b0 < p.batch; b0 += 64) {
        const int64_t lp = padded_len(lane_len(p, b0, lane, len0));
        const int64_t lnl = line_keys(lp, ln.gap);
        const int64_t incl = wave_incl_scan_len(lnl);
        if (b >= b0 && b < b0 + 64) {
            l = lane_value(lp, b - b0);
            s = t + lane_value(incl, b - b0) - lane_value(lnl, b - b0);
        }
        t += lane_value(incl, 63);
    }
    ln.total = uniform(t);
    ln.chunk = plan_chunk(ln.total, p.splits, p.min_chunk);
    start = uniform(s);
    len = uniform(l);
    return ln;
}

__device__ inline uint16_t bf16_bits(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ inline float bf16_value(uint16_t bits) {
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
}

// Wave-local ordering of LDS accesses: the same wave writes a tile and reads
// it back in another lane order; LDS executes one wave's accesses in order,
// this keeps the compiler from moving them across each other.
__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The 18 query chunks of a lane (Q^T operand: channels 32t + 8(l/16) ..+7
// of row l%16), loaded straight into accumulation registers, from which the
// MFMA reads its B operand, so the vector registers stay free for the hot
// loop.  All loads issue back to back and one wait at the end covers them
// (and any older load of the wave).
__device__ inline void load_q(bf16x8 (&qf)[kQkSteps], const uint16_t *qrow) {
    static_assert(kQkSteps == 18, "one load per 32-channel step");
    asm volatile(
        "global_load_dwordx4 %0, %18, off\n\t"
        "global_load_dwordx4 %1, %18, off offset:64\n\t"
        "global_load_dwordx4 %2, %18, off offset:128\n\t"
        "global_load_dwordx4 %3, %18, off offset:192\n\t"
        "global_load_dwordx4 %4, %18, off offset:256\n\t"
        "global_load_dwordx4 %5, %18, off offset:320\n\t"
        "global_load_dwordx4 %6, %18, off offset:384\n\t"
        "global_load_dwordx4 %7, %18, off offset:448\n\t"
        "global_load_dwordx4 %8, %18, off offset:512\n\t"
        "global_load_dwordx4 %9, %18, off offset:576\n\t"
        "global_load_dwordx4 %10, %18, off offset:640\n\t"
        "global_load_dwordx4 %11, %18, off offset:704\n\t"
        "global_load_dwordx4 %12, %18, off offset:768\n\t"
        "global_load_dwordx4 %13, %18, off offset:832\n\t"
        "global_load_dwordx4 %14, %18, off offset:896\n\t"
        "global_load_dwordx4 %15, %18, off offset:960\n\t"
        "global_load_dwordx4 %16, %18, off offset:1024\n\t"
        "global_load_dwordx4 %17, %18, off offset:1088\n\t"
        "s_waitcnt vmcnt(0)"
        : "=a"(qf[0]), "=a"(qf[1]), "=a"(qf[2]), "=a"(qf[3]), "=a"(qf[4]), "=a"(qf[5]),
          "=a"(qf[6]), "=a"(qf[7]), "=a"(qf[8]), "=a"(qf[9]), "=a"(qf[10]), "=a"(qf[11]),
          "=a"(qf[12]), "=a"(qf[13]), "=a"(qf[14]), "=a"(qf[15]), "=a"(qf[16]), "=a"(qf[17])
        : "v"(qrow)
        : "memory");
}

// ------------------------------------------------------------- per-wave state

struct WaveState {
    f32x4 acc[kOutTiles];  // O^T tiles: lane l -> head l%16, channels 16ct + 4(l/16) + i
    float m;               // running max of the scaled scores (log2 domain)
    float l;               // this lane's share of the running sum
};

struct BlockCtx {
    const uint16_t *kv;
    const int32_t *table_row;  // block table row of the sequence (paged)
    int64_t seq_base;          // contiguous: first row of the sequence
    int32_t page_size;         // 0 = contiguous
    int64_t num_pages;
    int32_t last_key;          // L - 1: loads of keys past it are clamped to it
};

__device__ inline BlockCtx block_ctx(const Params &p, int b, int32_t L) {
    BlockCtx bc;
    bc.kv = p.kv;
    bc.page_size = p.page_size;
    bc.num_pages = p.num_pages;
    bc.table_row = p.page_size ? p.block_table + (int64_t)b * p.max_pages : nullptr;
    bc.seq_base = (int64_t)b * p.kv_capacity;
    bc.last_key = L - 1;
    return bc;
}

// LDS image of one 16-key block (16 latent rows of 72 16-byte chunks):
// 18 slices of 1 KB.  Slice t = 9h + u holds rows 8h .. 8h+7, chunks
// 8u .. 8u+7 (channels 64u .. 64u+63): row 8h + r at slots 8r .. 8r+7,
// chunk 8u + w at slot 8r + (w ^ swz(r)), swz(r) = 4 bit1(r) + 2 bit2(r).
// Each direct load then fetches eight whole 128-byte lines, and both operand
// reads below spread over all LDS banks (the K read of a step hits every
// 16-byte bank group four times, a V^T read every 8-byte group twice).
__device__ inline int row_swz(int r) { return 4 * ((r >> 1) & 1) + 2 * ((r >> 2) & 1); }

// Block-table entry of the page that holds key `key` (clamped to the last
// key, which keeps the index inside the sequence's row), clamped into the
// pool.  The table is only read by this kernel, so it is read as constant
// memory through the scalar cache: the load then completes on the
// LDS/scalar counter and never makes the wave wait for the KV blocks still
// in flight on the vector-memory counter.  Contiguous caches need no entry.
__device__ inline int64_t page_of(const BlockCtx &c, int key) {
    if (!c.page_size) return 0;
    const int idx = uniform(min(key, c.last_key) / c.page_size);
    const auto *row = (const __attribute__((address_space(4))) int32_t *)(uintptr_t)uniform(
        (int64_t)(uintptr_t)c.table_row);
    const int64_t page = row[idx];
    return page < 0 ? 0 : (page >= c.num_pages ? c.num_pages - 1 : page);
}

// Issue the 18 direct-to-LDS 16-byte loads of the block starting at key kb,
// non-temporal (the cache is streamed once).  Lane l of load t = 9h + u
// fetches row 8h + l/8, chunk 8u + ((l % 8) ^ swz(l/8)); the hardware stores
// it at slice t, slot l.  A paged block lies in one page (`page`, from
// page_of): pages hold a multiple of 16 keys and blocks start at multiples
// of 16, and a key clamped to the last one stays in the block.
__device__ inline void issue_block(char *stage, const BlockCtx &c, int kb, int64_t page, int lane) {
    const int r = lane >> 3;
    const int w = (lane & 7) ^ row_swz(r);
    const uint16_t *rows[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int key = min(kb + 8 * h + r, c.last_key);
        if (c.page_size)
            rows[h] = c.kv + (page * c.page_size + key % c.page_size) * (int64_t)kDqk + 8 * w;
        else
            rows[h] = c.kv + (c.seq_base + key) * (int64_t)kDqk + 8 * w;
    }
#pragma unroll
    for (int t = 0; t < kQkSteps; ++t)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(rows[t / 9] + 64 * (t % 9)),
            (__attribute__((address_space(3))) void *)(stage + t * 1024), 16, 0, kNonTemporal);
}

// The same 18 loads in buffer form, for the shared kernel: a buffer
// resource spans the block's real rows, so rows past the last key read as
// zeros (they are masked out, and zero rows keep P V finite).  The compiler
// counts buffer-form direct loads on the vector-memory counter only, so the
// LDS reads issued while they fly keep exact waits; in the FLAT form it
// makes every such wait a full one.  vrow[h] is the lane's byte offset of
// its 16 bytes in rows 8h .. 8h+7 (row 8h + l/8, chunk (l%8) ^ swz(l/8)).
constexpr int kBufferWord3 = 0x00020000;  // gfx9 buffer descriptor: 32-bit data format
static_assert(kQkSteps * 1024 == kBlockBytes, "block B's slices follow block A's");
template <int T>
__device__ inline void buffer_load_slice(__amdgpu_buffer_rsrc_t rs, char *stage, const int (&vrow)[2]) {
    // The column-group offset goes in the scalar offset: an instruction
    // offset would move the LDS destination as well.
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(stage + T * 1024), 16,
                                             vrow[T / 9], 128 * (T % 9), 0, kNonTemporal);
}
template <int... T>
__device__ inline void buffer_load_slices(__amdgpu_buffer_rsrc_t rs, char *stage, const int (&vrow)[2],
                                          std::integer_sequence<int, T...>) {
    (buffer_load_slice<T>(rs, stage, vrow), ...);
}
__device__ inline __amdgpu_buffer_rsrc_t block_rsrc(const BlockCtx &c, int kb, int64_t page, bool live = true);
__device__ inline void issue_block_buffer(char *stage, const BlockCtx &c, int kb, int64_t page,
                                          const int (&vrow)[2]) {
    buffer_load_slices(block_rsrc(c, kb, page), stage, vrow, std::make_integer_sequence<int, kQkSteps>{});
}

// One wave's share of the 36 loads of a 32-key step (blocks A at kb and B
// at kb + 16, in buffer form): slices share, share + nshare, ... of the
// step's 36 (block A's 18, then block B's), so that the waves that compute
// a step also split its loads.  block_rsrc: the descriptor of the block at
// kb.  A block wholly past the last key (or any block when !live) gets an
// empty range: nothing is read and the stage fills with zeros.  The descriptor must be wave-uniform (scalar registers);
// readfirstlane states it, else the compiler wraps every load in a
// per-lane loop.
__device__ inline __amdgpu_buffer_rsrc_t block_rsrc(const BlockCtx &c, int kb, int64_t page, bool live) {
    const uint16_t *row0 = c.page_size ? c.kv + (page * c.page_size + kb % c.page_size) * (int64_t)kDqk
                                       : c.kv + (c.seq_base + kb) * (int64_t)kDqk;
    const int rows = live ? max(0, min(kKeyBlock, c.last_key + 1 - kb)) : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)uniform((int64_t)(uintptr_t)row0), 0,
                                             uniform(rows * kDqk * 2), kBufferWord3);
}
__device__ inline void issue_step_share(char *dst, const BlockCtx &c, int kb, int64_t page_a, int64_t page_b,
                                        const int (&vrow)[2], int share, int nshare) {
    const __amdgpu_buffer_rsrc_t ra = block_rsrc(c, kb, page_a);
    const __amdgpu_buffer_rsrc_t rb = block_rsrc(c, kb + kKeyBlock, page_b);
    for (int idx = share; idx < 2 * kQkSteps; idx += nshare) {
        const bool hb = idx >= kQkSteps;
        const int t = hb ? idx - kQkSteps : idx;
        // Slice t of block A or B sits at 1024 idx in the step's image.
        __builtin_amdgcn_raw_ptr_buffer_load_lds(hb ? rb : ra,
                                                 (__attribute__((address_space(3))) void *)(dst + 1024 * idx), 16,
                                                 t < 9 ? vrow[0] : vrow[1], 128 * (t < 9 ? t : t - 9), 0,
                                                 kNonTemporal);
    }
}

// One key group (kOneGroup) streams 64-key steps: four 16-key blocks, one
// per wave to load (wave w: block w, its 18 slices).  The loads of step
// i + 1 go out with the MFMAs of the first half of step i, one every
// kQuadEvery: issued in a burst they would hold every wave until the memory
// pipeline took them.
constexpr int kQuadBlocks = kWaves;
constexpr int kQuadBytes = kQuadBlocks * kBlockBytes;  // 72 KB
constexpr int kQuadEvery = 5;
static_assert(kQuadEvery * (kQkSteps - 1) < 2 * kQkSteps + 2 * kOutTiles, "within one pair's MFMAs");

struct QuadLoads {
    char *dst;                 // this wave's block in the step's slot
    __amdgpu_buffer_rsrc_t r;  // that block's rows
    int vrow[2];

    template <int T>
    __device__ void slice() {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)(dst + T * 1024), 16,
                                                 vrow[T / 9], 128 * (T % 9), 0, kNonTemporal);
    }
    template <int... T>
    __device__ void all(std::integer_sequence<int, T...>) {
        (slice<T>(), ...);
    }
    // The load that goes with MFMA g of the pair, if any.
    __device__ void operator()(int g) {
        if (g % kQuadEvery != 0 || g / kQuadEvery >= kQkSteps) return;
        switch (g / kQuadEvery) {  // compile-time after unrolling
        case 0: slice<0>(); break;
        case 1: slice<1>(); break;
        case 2: slice<2>(); break;
        case 3: slice<3>(); break;
        case 4: slice<4>(); break;
        case 5: slice<5>(); break;
        case 6: slice<6>(); break;
        case 7: slice<7>(); break;
        case 8: slice<8>(); break;
        case 9: slice<9>(); break;
        case 10: slice<10>(); break;
        case 11: slice<11>(); break;
        case 12: slice<12>(); break;
        case 13: slice<13>(); break;
        case 14: slice<14>(); break;
        case 15: slice<15>(); break;
        case 16: slice<16>(); break;
        default: slice<17>(); break;
        }
    }
};
static_assert(kQkSteps == 18, "QuadLoads lists the 18 slices of a block");

// Per-lane byte offsets of the operand reads within a block image.
//  K operand of QK^T step t (lane l -> key k = l%16, chunk 4t + l/16):
//    slice 9(k/8) + t/2, slot 8(k%8) + ((4(t%2) + l/16) ^ swz(k%8)),
//    i.e. k_off[t % 2] + 1024 * (t / 2).
//  V^T operand of output tile ct (transposing read; in-group lane m of
//  group g points at key 4g + m/4, channels 16ct + 4(m%4) .. +3: chunk
//  2ct + (m%4)/2, half m%2):  v_off[ct % 4] + 1024 * (ct / 4).
struct OperandOffsets {
    int k_off[2];
    uint32_t v_off[4];
};

__device__ inline OperandOffsets operand_offsets(int lane) {
    OperandOffsets o;
    {
        const int k = lane & 15, q = lane >> 4;
        const int h = k >> 3, r = k & 7;
        const int r1 = (r >> 1) & 1, r2 = (r >> 2) & 1;
        const int base = 9 * h * 1024 + 16 * (8 * r + (q ^ (2 * r2)));
        o.k_off[0] = base + 64 * r1;
        o.k_off[1] = base + 64 * (1 - r1);
    }
    {
        const int g = lane >> 4, m = lane & 15;
        const int key = 4 * g + (m >> 2);
        const int h = key >> 3, r = key & 7;
        const int r1 = (r >> 1) & 1, r2 = (r >> 2) & 1;
        const int b = (m & 3) >> 1;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            o.v_off[c4] = 9 * h * 1024 +
                          16 * (8 * r + b + 2 * ((c4 & 1) ^ r2) + 4 * (((c4 >> 1) & 1) ^ r1)) +
                          8 * (m & 1);
    }
    return o;
}

// The compiler does not track completion of direct-to-LDS loads, so the
// waits are explicit: at most N vector-memory operations may stay in flight.
// (s_waitcnt through the builtin, so the compiler's own wait insertion sees
// it; the empty asm statements keep memory accesses from moving across.)
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    asm volatile("" ::: "memory");
}

// Workgroup barrier without the memory fence of __syncthreads: that fence
// would wait for every outstanding load, including the direct loads of the
// next step.  Used only where each wave has already waited explicitly for
// what the others need (its share of direct loads, its own LDS reads).
__device__ inline void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ inline void wait_lgkm0() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (0x7 << 4));
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Eight transposing V^T reads (tiles 8G .. 8G+7; tile ct at
// v[ct % 4] + 1024 (ct / 4)), waited for inside the same statement so that
// the outputs are complete when it ends.  (The compiler would otherwise
// treat such a read as possibly aliasing the in-flight direct-to-LDS loads
// and wait for those.)
template <int G>
__device__ inline void read_vt8(s16x4 (&va)[kOutTiles], const uint32_t (&v)[4]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%12\n"
        "ds_read_b64_tr_b16 %1, %9 offset:%12\n"
        "ds_read_b64_tr_b16 %2, %10 offset:%12\n"
        "ds_read_b64_tr_b16 %3, %11 offset:%12\n"
        "ds_read_b64_tr_b16 %4, %8 offset:%13\n"
        "ds_read_b64_tr_b16 %5, %9 offset:%13\n"
        "ds_read_b64_tr_b16 %6, %10 offset:%13\n"
        "ds_read_b64_tr_b16 %7, %11 offset:%13\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(va[8 * G + 0]), "=&v"(va[8 * G + 1]), "=&v"(va[8 * G + 2]), "=&v"(va[8 * G + 3]),
          "=&v"(va[8 * G + 4]), "=&v"(va[8 * G + 5]), "=&v"(va[8 * G + 6]), "=&v"(va[8 * G + 7])
        : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "n"(2048 * G), "n"(2048 * G + 1024)
        : "memory");
}

// Scores of one block: S^T[key][head] for 16 keys x 16 heads, scaled into
// the log2 domain and masked; lane l holds head l%16, keys kb + 4(l/16) + i
// and mx is the block max of its head.  The A operand K comes from the
// block's LDS image (lane l -> key l%16, channels 32t + 8(l/16) .. +7, one
// contiguous 1 KB read per wave), the B operand Q^T from registers; two
// accumulators halve the dependent MFMA chain.  The first eight V^T
// operands are read here as well.
__device__ inline void block_scores(float (&sv)[4], float &mx, s16x4 (&va)[kOutTiles],
                                    const char *stage, const int (&k_off)[2],
                                    const uint32_t (&v_addr)[4], const bf16x8 (&qf)[kQkSteps],
                                    int kb, int key_end, float scale_log2, int lane) {
    bf16x8 ka[kQkSteps];
#pragma unroll
    for (int t = 0; t < kQkSteps; ++t)
        ka[t] = *reinterpret_cast<const bf16x8 *>(stage + k_off[t & 1] + 1024 * (t >> 1));
    // All K reads are issued before the first MFMA waits on one of them.
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < kQkSteps; t += 2) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t], qf[t], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[t + 1], qf[t + 1], s1, 0, 0, 0);
    }
    read_vt8<0>(va, v_addr);
    const f32x4 s = s0 + s1;
    const int k0 = kb + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (k0 + i < key_end) ? s[i] * scale_log2 : -INFINITY;
    mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
}

// P = exp2(s - m) and O^T += V^T P^T, P split into bf16 hi + lo, one
// 16x16x32 MFMA per output tile for both halves.  Its k index runs over
// (key, half): lane group g = l/16 holds k = 8g + j, which stands for key
// 4g + j%4, hi half for j < 4 and lo half for j >= 4.  The B operand is then
// the lane's own P^T values (head l%16, keys 4g + i: the score accumulator
// layout) as {hi[0..3], lo[0..3]}, and the A operand the lane's transposed
// V^T read (channel l%16, keys 4g + i) twice: sum_k A B = V^T (P_hi + P_lo).
// Tiles 0..7 were read with the scores; the others are read eight at a time.
__device__ inline void block_pv(WaveState &st, const float (&sv)[4], s16x4 (&va)[kOutTiles],
                                const uint32_t (&v_addr)[4]) {
    s16x8 pb;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float pr = __builtin_amdgcn_exp2f(sv[i] - st.m);
        psum += pr;
        const uint16_t h = bf16_bits(pr);
        pb[i] = (short)h;
        pb[4 + i] = (short)bf16_bits(pr - bf16_value(h));
    }
    const bf16x8 p8 = __builtin_bit_cast(bf16x8, pb);
    st.l += psum;
    // Tiles 8G .. 8G+7: group 0 was read with the scores; group G+1 is read
    // once the MFMAs of group G are issued, so its reads overlap them.
#pragma unroll
    for (int g = 0; g < kOutTiles / 8; ++g) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int ct = 8 * g + j;
            const bf16x8 a8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va[ct], va[ct], 0, 1, 2, 3, 0, 1, 2, 3));
            st.acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, p8, st.acc[ct], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        switch (g + 1) {  // compile-time after unrolling
        case 1: read_vt8<1>(va, v_addr); break;
        case 2: read_vt8<2>(va, v_addr); break;
        case 3: read_vt8<3>(va, v_addr); break;
        default: break;
        }
    }
}

// Move the reference max up to the block max and rescale (rare path).
__device__ inline void rescale(WaveState &ws, float mx) {
    const float m_new = fmaxf(ws.m, mx);
    const float alpha = __builtin_amdgcn_exp2f(ws.m - m_new);
#pragma unroll
    for (int ct = 0; ct < kOutTiles; ++ct) ws.acc[ct] *= alpha;
    ws.l *= alpha;
    ws.m = m_new;
}

// The running max m is only a reference point: P = exp2(s - m) may exceed 1
// as long as s - m <= kMaxLag, so the accumulators are rescaled only when a
// block's max passes m + kMaxLag (and for the first block).  The result is
// the same softmax; the rescale sits outside the hot loop.
constexpr float kMaxLag = 8.0f;

// ---- 32-key steps (shared rings): two 16-key blocks A and B per step ----

// One transposing V^T read, issued through the compiler's builtin so that it
// tracks the result and waits for it only where it is used.  Within 16
// lanes, lane i receives element i % 4 of the rows addressed by lanes
// i / 4 + 4r.
__device__ inline s16x4 read_vt(const char *addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(addr));
}

// Max of x over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups that
// hold one head's keys), with row-swapping permutes instead of LDS
// permutes: those would join the LDS counter, and waiting for their result
// would wait for every operand read issued before them.  Each swap of x
// with itself returns, per lane, x of the lane and of its partner.
__device__ inline float max_over_lane_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Compile-time slot parity of a shared-ring step.
template <int V>
struct Parity {
    static constexpr int value = V;
};

// The operand reads of one 32-key step of a row block form one stream: the
// 36 K reads (block A's 18 k-steps, then block B's) and then the 64 V^T
// reads (tile ct of block A is read 2ct, of block B 2ct + 1).  Each MFMA of
// the step is issued together with the read kAhead places further down the
// stream, so LDS latency overlaps the MFMAs instead of adding to them; the
// order is pinned with scheduling barriers and the compiler places the
// waits.
constexpr int kPairK = 2 * kQkSteps;
constexpr int kPairV = 2 * kOutTiles;
constexpr int kAhead = 12;
static_assert(kAhead <= kPairK, "the stream starts with K reads");


// Work issued with the MFMAs of a 32-key pair: side(g) runs after MFMA g
// (g = 0 .. 99: the 36 QK^T MFMAs, then the 64 PV ones).
struct NoSide {
    __device__ void operator()(int) const {}
};

struct PairReads {
    const char *stA, *stB;  // the step's blocks A and B
    int k_off[2];
    uint32_t v_off[4];
    bf16x8 ka[kPairK];
    s16x4 vr[kPairV];

    __device__ void read(int r) {
        if (r < kPairK) {
            const int t = r % kQkSteps;
            ka[r] = *reinterpret_cast<const bf16x8 *>((r < kQkSteps ? stA : stB) + k_off[t & 1] +
                                                      1024 * (t >> 1));
        } else if (r < kPairK + kPairV) {
            const int v = r - kPairK, ct = v >> 1;
            vr[v] = read_vt(((v & 1) ? stB : stA) + v_off[ct & 3] + 1024 * (ct >> 2));
        }
    }
};

// Scores of a step: lane l holds head l%16, keys 4(l/16) + i of block A
// (sv[i]) and of block B (sv[4 + i]), scaled into the log2 domain and
// masked; mx is their max over the head.  Leaves the first kAhead V^T reads
// of the stream in flight.
template <typename Side = NoSide>
__device__ inline void pair_scores(PairReads &rd, float (&sv)[8], float &mx, const bf16x8 (&qf)[kQkSteps],
                                   int kbA, int key_end, float scale_log2, int lane, Side side = Side{}) {
#pragma unroll
    for (int r = 0; r < kAhead; ++r) rd.read(r);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
    for (int n = 0; n < kPairK; ++n) {
        const int h = n / kQkSteps, t = n % kQkSteps;
        s[h][t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rd.ka[n], qf[t], s[h][t & 1], 0, 0, 0);
        rd.read(n + kAhead);
        side(n);
        __builtin_amdgcn_sched_barrier(0);
    }
    const int kA = kbA + 4 * (lane >> 4), kB = kA + kKeyBlock;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sv[i] = (kA + i < key_end) ? (s[0][0][i] + s[0][1][i]) * scale_log2 : -INFINITY;
        sv[4 + i] = (kB + i < key_end) ? (s[1][0][i] + s[1][1][i]) * scale_log2 : -INFINITY;
    }
    mx = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
    mx = max_over_lane_groups(mx);
}

// P = exp2(s - m) and O^T += V^T P^T over the step's 32 keys, continuing
// the stream at V^T read kAhead.  k slot 8(l/16) + i of a 16x16x32 MFMA is
// key 4(l/16) + i of block A for i < 4 and of block B for i >= 4, in both
// operands: P^T (B operand) is the joined score registers, split into bf16
// hi and lo halves (two MFMAs per tile), and V^T (A operand) joins one
// transposing read of each block.  Within a group of four tiles the hi
// MFMAs come before the lo ones, so no MFMA waits on the one before it.
// kHiOnly (the caller's MLA_OPT_P_BF16): P enters as its bf16 hi half alone,
// half the MFMAs, each P term rounded by at most 2^-8 of itself (bf16 keeps 8
// significant bits).
template <bool kHiOnly = false, typename Side = NoSide>
__device__ inline void pair_pv(PairReads &rd, WaveState &ws, const float (&sv)[8], Side side = Side{}) {
    bf16x8 phi, plo;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float pr = __builtin_amdgcn_exp2f(sv[i] - ws.m);
        psum += pr;
        const __bf16 hb = static_cast<__bf16>(pr);
        phi[i] = hb;
        if constexpr (!kHiOnly) plo[i] = static_cast<__bf16>(pr - static_cast<float>(hb));
    }
    ws.l += psum;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < 2 * kOutTiles; ++m) {
        const int ct = 4 * (m >> 3) + (m & 3);
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(rd.vr[2 * ct], rd.vr[2 * ct + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        // With kHiOnly the lo MFMAs drop out; the operand reads and the
        // loads that go with them keep their places in the stream.
        if (!(kHiOnly && (m & 4)))
            ws.acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, (!kHiOnly && (m & 4)) ? plo : phi, ws.acc[ct],
                                                                 0, 0, 0);
        rd.read(kPairK + kAhead + m);
        side(kPairK + m);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ------------------------------------------------- merging a segment's waves

// Where the waves' O rows and softmax stats go for the merge at the end of
// a segment (the two stage arrays, reused): waves 0 and 1 in the first,
// waves 2 and 3 and the stats (m, l: kWaves x 16 each) in the second.  (The
// address is computed, not looked up: an array of pointers indexed by the
// wave would be placed in memory.)
struct MergeArea {
    char *stage0, *stage1;
    float *m, *l;
    __device__ float *row(int w, int head) const {
        return reinterpret_cast<float *>(w < 2 ? stage0 : stage1) + ((w & 1) * 16 + head) * kMergePitch;
    }
    __device__ float *m_at(int w, int head) const { return m + w * 16 + head; }
    __device__ float *l_at(int w, int head) const { return l + w * 16 + head; }
};

// One row block per workgroup: each wave's O rows and stats go into its own
// two ring blocks, rows 0-7 into its stage-0 block with the stats after
// them and rows 8-15 into its stage-1 block, shifted by 32 floats so that
// the rows of heads h and h + 8 start on different banks.  No other wave
// touches those blocks, so a wave writes its rows as soon as its own last
// block is done.
constexpr int kMergeHiShift = 32;
static_assert(8 * kMergePitch * 4 + 32 * 4 <= kBlockBytes, "rows 0-7 and the stats fit in a block");
static_assert((kMergeHiShift + 8 * kMergePitch) * 4 <= kBlockBytes, "rows 8-15 fit in a block");
struct WaveMergeArea {
    char *stage0, *stage1;
    __device__ float *row(int w, int head) const {
        return head < 8 ? reinterpret_cast<float *>(stage0 + w * kBlockBytes) + head * kMergePitch
                        : reinterpret_cast<float *>(stage1 + w * kBlockBytes) + kMergeHiShift +
                              (head - 8) * kMergePitch;
    }
    __device__ float *m_at(int w, int head) const {
        return reinterpret_cast<float *>(stage0 + w * kBlockBytes) + 8 * kMergePitch + head;
    }
    __device__ float *l_at(int w, int head) const { return m_at(w, head) + 16; }
};

// One row block, while the next segment's first blocks land in the stage-0
// blocks: each wave's rows go through its stage-1 block half a row at a
// time (256 channels, pitch 260 floats), with the stats after them.
constexpr int kHalfCols = kDv / 2;
constexpr int kHalfPitch = kHalfCols + 4;
static_assert((16 * kHalfPitch + 32) * 4 <= kBlockBytes, "half rows and the stats fit in a block");
struct HalfMergeArea {
    char *stage1;
    __device__ float *row(int w, int head) const {
        return reinterpret_cast<float *>(stage1 + w * kBlockBytes) + head * kHalfPitch;
    }
    __device__ float *m_at(int w, int head) const {
        return reinterpret_cast<float *>(stage1 + w * kBlockBytes) + 16 * kHalfPitch + head;
    }
    __device__ float *l_at(int w, int head) const { return m_at(w, head) + 16; }
};

// Rows of row block rb0 + rbl from the NKG waves that computed them (waves
// rbl + nrb kg): the LSE-weighted sum of their O rows, normalized, written
// as the final rows (whole) or as the segment's part.  The area holds
// channels col0 .. col0 + kCols - 1 of each row (the LSE goes out with
// col0 = 0).  Every LDS read is issued before the first is used.  256
// threads: 16 heads x 16 quads.
template <int NKG, int kCols, typename Area>
__device__ inline void merge_waves(const Params &p, const Area &ma, int b, int rb0, int rbl, int nrb,
                                   bool whole, int slot, int col0) {
    const int head = threadIdx.x >> 4;
    const int cq = threadIdx.x & 15;
    float mw[NKG], lw[NKG];
    f32x4 ov[kCols / 64][NKG];
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg) {
        const int w = rbl + nrb * kg;
        mw[kg] = *ma.m_at(w, head);
        lw[kg] = *ma.l_at(w, head);
#pragma unroll
        for (int jc = 0; jc < kCols / 64; ++jc)
            ov[jc][kg] = *reinterpret_cast<const f32x4 *>(ma.row(w, head) + 4 * cq + 64 * jc);
    }
    __builtin_amdgcn_sched_barrier(0);
    float M = mw[0];
#pragma unroll
    for (int kg = 1; kg < NKG; ++kg) M = fmaxf(M, mw[kg]);
    float wgt[NKG];
    float lsum = 0.f;
#pragma unroll
    for (int kg = 0; kg < NKG; ++kg) {
        wgt[kg] = mw[kg] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[kg] - M);
        lsum += wgt[kg] * lw[kg];
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float lse2 = lsum > 0.f ? M + log2f(lsum) : -INFINITY;
    const int rbg = rb0 + rbl;
    const int hpt = p.heads >> 4;
    const int64_t row = ((int64_t)b * p.s_q + rbg / hpt) * p.heads + (rbg % hpt) * 16 + head;
    float *orow;
    if (whole) {
        orow = p.out + row * kDv + col0;
        if (cq == 0 && col0 == 0) p.lse[row] = lse2 * kLn2;
    } else {
        const int64_t r = ((int64_t)slot * p.n_rb + rbg) * 16 + head;
        orow = p.part_o + r * kDv + col0;
        if (cq == 0 && col0 == 0) p.part_lse[r] = lse2;
    }
#pragma unroll
    for (int jc = 0; jc < kCols / 64; ++jc) {
        f32x4 o = wgt[0] * ov[jc][0];
#pragma unroll
        for (int kg = 1; kg < NKG; ++kg) o += wgt[kg] * ov[jc][kg];
        *reinterpret_cast<f32x4 *>(orow + 4 * cq + 64 * jc) = o * inv;
    }
}

// A wave that alone computed its row block (one key group) writes the rows
// straight from its accumulators: normalized O (lane l: head l%16, channels
// 16ct + 4(l/16) .. +3 of tile ct) and the LSE, as the final rows (whole)
// or as the segment's part (log2-domain LSE).  Same values as merge_waves<1>.
__device__ inline void write_rows(const Params &p, const WaveState &ws, int b, int rb, bool whole, int slot,
                                  int lane) {
    const int head = lane & 15, grp = lane >> 4;
    float lt = ws.l;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse2 = lt > 0.f ? ws.m + log2f(lt) : -INFINITY;
    const int hpt = p.heads >> 4;
    const int64_t row = ((int64_t)b * p.s_q + rb / hpt) * p.heads + (rb % hpt) * 16 + head;
    float *orow;
    if (whole) {
        orow = p.out + row * kDv;
        if (grp == 0) p.lse[row] = lse2 * kLn2;
    } else {
        const int64_t r = ((int64_t)slot * p.n_rb + rb) * 16 + head;
        orow = p.part_o + r * kDv;
        if (grp == 0) p.part_lse[r] = lse2;
    }
#pragma unroll
    for (int ct = 0; ct < kOutTiles; ++ct)
        *reinterpret_cast<f32x4 *>(orow + 16 * ct + 4 * grp) = ws.acc[ct] * inv;
}

// --------------------------------------------------------------- split kernel

// How a workgroup's row blocks (nrb of them, of 16 query rows each) share
// the keys:
//  kOneBlock   nrb = 1: each wave streams its own 16-key blocks through a
//              private two-stage ring, no barrier.
//  kTwoGroups  nrb = 2: two key groups of two waves; the waves of a group
//              share each 32-key step through a two-slot ring.
//  kOneGroup   nrb = 3, 4: one key group of four waves sharing each 64-key
//              step through a two-slot ring; all four waves issue a quarter
//              of each step's loads, and each wave writes its rows itself.
//  kOneBlockNext  as kOneBlock, for launches where a workgroup may hold
//              several segments: each wave sends the first block of the
//              workgroup's next segment before the merge of the current one
//              (a separate instance: the extra path costs the single-segment
//              case a little in registers and time).
enum SplitMode { kOneBlock = 0, kTwoGroups = 1, kOneGroup = 2, kOneBlockNext = 3 };

template <int kMode, bool kHiOnly>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_split_kernel(Params p) {
    constexpr bool kOne = kMode == kOneBlock || kMode == kOneBlockNext;
    constexpr bool kShared = !kOne;
    char *stage0_base, *stage1_base;  // kOneBlock, kTwoGroups
    MergeArea ma{};
    if constexpr (kMode == kOneGroup) {
        // Two step-sized arrays, the ring's slots.  The compiler tells LDS
        // accesses of distinct arrays apart, so its own reads of one slot
        // never wait for direct loads still landing in the other.  (Each
        // wave writes its rows itself: no merge area.)
        __shared__ __attribute__((aligned(16))) char slot_a[kQuadBytes];
        __shared__ __attribute__((aligned(16))) char slot_b[kQuadBytes];
        stage0_base = slot_a;
        stage1_base = slot_b;
    } else {
        if constexpr (kMode == kTwoGroups) {
            // Two stage arrays, for the same reason.
            __shared__ __attribute__((aligned(16))) char stage_a[kStageBytes];
            __shared__ __attribute__((aligned(16))) char stage_b[kStageBytes];
            stage0_base = stage_a;
            stage1_base = stage_b;
        } else {
            __shared__ __attribute__((aligned(16))) char ring[kStages * kStageBytes];
            stage0_base = ring;
            stage1_base = ring + kStageBytes;
        }
        ma.stage0 = stage0_base;
        ma.stage1 = stage1_base;
        ma.m = reinterpret_cast<float *>(stage1_base) + 2 * kMergeWaveFloats;
        ma.l = ma.m + kWaves * 16;
    }
    const int lane = threadIdx.x & 63;
    // Wave-uniform (scalar) so that stage addresses stay in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int g, grp;
    range_and_group(blockIdx.x, p.n_groups, gridDim.x / p.n_groups, g, grp);
    const int rb0 = (p.y0 + grp) * kWaves;
    const int nrb = kOne ? 1 : kMode == kTwoGroups ? 2 : min(kWaves, p.n_rb - rb0);
    const int nkg = kWaves / nrb;
    const int my_rbl = wave % nrb;
    const int my_kg = wave / nrb;
    const bool active = my_kg < nkg;
    const int hpt = p.heads >> 4;
    const int rb = rb0 + my_rbl;
    const int tok = rb / hpt;
    const int h0 = (rb % hpt) * 16;

    // Plan (same arithmetic as mla_plan on the host).  The lengths of the
    // first 64 sequences are loaded once, for the line and for the walk
    // over the sequences below.
    const int32_t len0 = lane < p.batch ? seq_len(p, lane) : 0;
    const int64_t gap = plan_gap(p, lane, len0);
    const int64_t incl0 = wave_incl_scan_len(line_keys(padded_len(len0), gap));
    int64_t total_l = lane_value(incl0, 63);
    for (int b0 = 64; b0 < p.batch; b0 += 64) {
        const int bl = b0 + lane;
        total_l += lane_value(wave_incl_scan_len(line_keys(bl < p.batch ? padded_len(seq_len(p, bl)) : 0, gap)), 63);
    }
    const int64_t total = uniform(total_l);
    const int64_t chunk = plan_chunk(total, p.splits, p.min_chunk);
    const int64_t gs = (int64_t)g * chunk;
    if (gs >= total) return;  // uniform over the workgroup
    const int64_t ge = min(gs + chunk, total);

    const OperandOffsets offs = operand_offsets(lane);

    // One row block: this wave's blocks of a segment that starts at st on
    // the line and holds Ln keys.  The workgroup's blocks, over all its
    // segments, go to the waves in turn (turn_now: the wave that takes the
    // segment's first block), every nkg-th block from kf.
    auto one_block_share = [&](int64_t st, int32_t Ln, int turn_now, int &kf, int &nm, int &nblk) {
        const int lo = (int)(max(gs, st) - st);
        const int hi = (int)(min(ge, st + padded_len(Ln)) - st);
        const int lim = min(hi, Ln - p.s_q + tok + 1);
        nblk = lim > lo ? (lim - lo + kKeyBlock - 1) / kKeyBlock : 0;
        const int off = (my_kg - turn_now) & (kWaves - 1);
        nm = nblk > off ? (nblk - off + nkg - 1) / nkg : 0;
        kf = lo + kKeyBlock * off;
    };

    int64_t base = 0;
    int turn = 0;             // one row block: the wave that takes the next block
    bool prefetched = false;  // one row block: the segment's first blocks are already in flight
    for (int b0 = 0; b0 < p.batch && base < ge; b0 += 64) {
        const int32_t Ll = lane_len(p, b0, lane, len0);
        const int64_t lpl = padded_len(Ll);
        const int64_t lnl = line_keys(lpl, gap);
        const int64_t incl = (b0 == 0 ? incl0 : wave_incl_scan_len(lnl)) + base;
        const int64_t stl = incl - lnl;
        // Sequences with keys in this range (a gap holds none).
        uint64_t mask = __ballot(lpl > 0 && stl < ge && stl + lpl > gs);
        const int64_t next_base = lane_value(incl, 63);

        while (mask) {
            const int j = __builtin_ctzll(mask);
            mask &= mask - 1;
            const int b = b0 + j;
            const int64_t st_b = lane_value(stl, j);
            const int32_t L = lane_value(Ll, j);
            const int64_t lp = padded_len(L);
            const int seg_lo = (int)(max(gs, st_b) - st_b);
            const int seg_hi = (int)(min(ge, st_b + lp) - st_b);
            const bool whole = st_b >= gs && st_b + lp <= ge;
            const int slot = whole ? -1 : segment_slot(g, st_b, chunk);

            WaveState ws;
#pragma unroll
            for (int ct = 0; ct < kOutTiles; ++ct) ws.acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            ws.m = -INFINITY;
            ws.l = 0.f;

            const BlockCtx bc = block_ctx(p, b, L);
            const int vis_end = L - p.s_q + tok + 1;  // keys [0, vis_end) visible to this wave
            // This wave's keys.  One row block: every nkg-th 16-key block
            // from kfirst.  Several: the waves of a key group (same keys,
            // different row blocks) share each 32-key step, two 16-key
            // blocks, and the group takes every nkg-th step from kfirst.
            const int kgq = active ? my_kg : 0;
            const bool producer = active && my_rbl == 0;  // loads the keys of its group
            int kfirst, kstep, n_mine, n_iter = 0;
            if constexpr (!kShared) {
                int nblk;
                one_block_share(st_b, L, turn, kfirst, n_mine, nblk);
                kstep = kKeyBlock * nkg;
                turn = (turn + nblk) & (kWaves - 1);
            } else if constexpr (kMode == kOneGroup) {
                const int tok_last = (rb0 + nrb - 1) / hpt;  // sees the most keys
                const int lim = min(seg_hi, L - p.s_q + tok_last + 1);
                const int nblk = lim > seg_lo ? (lim - seg_lo + kKeyBlock - 1) / kKeyBlock : 0;
                n_iter = n_mine = (nblk + kQuadBlocks - 1) / kQuadBlocks;
                kstep = kQuadBlocks * kKeyBlock;
                kfirst = seg_lo;
            } else {
                const int tok_last = (rb0 + nrb - 1) / hpt;  // sees the most keys
                const int lim = min(seg_hi, L - p.s_q + tok_last + 1);
                const int nblk = lim > seg_lo ? (lim - seg_lo + kKeyBlock - 1) / kKeyBlock : 0;
                const int npair = (nblk + 1) / 2;
                n_iter = (npair + nkg - 1) / nkg;  // same in every wave
                n_mine = npair > kgq ? (npair - kgq + nkg - 1) / nkg : 0;
                kstep = 2 * kKeyBlock * nkg;
                kfirst = seg_lo + 2 * kKeyBlock * kgq;
            }
            // The first loads of the segment go out before the query is
            // fetched, so that the two round trips overlap.
            char *const first = stage0_base + (kShared ? kgq * kPairBytes : wave * kBlockBytes);  // not kOneGroup
            // Lane byte offsets of the buffer-form loads (shared kernel).
            int vrow[2];
            {
                const int r = lane >> 3;
                const int w = (lane & 7) ^ row_swz(r);
                vrow[0] = (r * kDqk + 8 * w) * 2;
                vrow[1] = vrow[0] + 8 * kDqk * 2;
            }
            // Pages of the next step to issue (shared kernels; kOneGroup: this
            // wave's block in pgA).
            int64_t pgA = 0, pgB = 0;
            if constexpr (kOne) {
                if (n_mine > 0 && !prefetched) issue_block(first, bc, kfirst, page_of(bc, kfirst), lane);
            } else if constexpr (kMode == kTwoGroups) {
                if (producer && n_mine > 0) {
                    issue_block_buffer(first, bc, kfirst, page_of(bc, kfirst), vrow);
                    issue_block_buffer(first + kBlockBytes, bc, kfirst + kKeyBlock, page_of(bc, kfirst + kKeyBlock),
                                       vrow);
                }
                pgA = page_of(bc, kfirst + kstep);
                pgB = page_of(bc, kfirst + kstep + kKeyBlock);
            } else {
                // Step 0, a quarter per wave.
                if (n_mine > 0) {
                    const int kbw = kfirst + wave * kKeyBlock;  // this wave's block
                    QuadLoads q0;
                    q0.dst = first + wave * kBlockBytes;
                    q0.r = block_rsrc(bc, kbw, page_of(bc, kbw));
                    q0.vrow[0] = vrow[0];
                    q0.vrow[1] = vrow[1];
                    q0.all(std::make_integer_sequence<int, kQkSteps>{});
                }
                pgA = page_of(bc, kfirst + kstep + wave * kKeyBlock);
            }
            bf16x8 qf[kQkSteps];  // B operand Q^T: lane l -> head l%16, channels 32t + 8(l/16)
            if (active)
                load_q(qf, p.q + (((int64_t)b * p.s_q + tok) * p.heads + h0 + (lane & 15)) * kDqk +
                                8 * (lane >> 4));

            if constexpr (!kShared) {
                // One row block: each wave streams its own blocks through a
                // private two-stage ring, no barrier.
                const int n_my = n_mine, step = kstep;
                char *stage0 = first;
                char *stage1 = stage1_base + wave * kBlockBytes;
                int64_t pg = page_of(bc, kfirst + step);  // pages are looked up a block ahead
                int i = 0;
                for (;;) {
                    float sv[4], mx = -INFINITY;
                    s16x4 va[kOutTiles];
                    uint32_t v_addr[4] = {0, 0, 0, 0};
                    bool lagged = false;
                    for (; i < n_my; ++i) {
                        char *cur = (i & 1) ? stage1 : stage0;
                        if (i + 1 < n_my) {
                            issue_block((i & 1) ? stage0 : stage1, bc, kfirst + (i + 1) * step, pg, lane);
                            pg = page_of(bc, kfirst + (i + 2) * step);
                            wait_vm<kQkSteps>();  // block i landed, block i+1 may fly
                        } else {
                            wait_vm<0>();
                        }
#pragma unroll
                        for (int c4 = 0; c4 < 4; ++c4)
                            v_addr[c4] = (uint32_t)(uintptr_t)cur + offs.v_off[c4];
                        block_scores(sv, mx, va, cur, offs.k_off, v_addr, qf, kfirst + i * step,
                                     vis_end, p.scale_log2, lane);
                        if (__any(mx > ws.m + kMaxLag)) {
                            lagged = true;
                            break;
                        }
                        block_pv(ws, sv, va, v_addr);
                        wait_lgkm0();  // this stage is refilled by the next block but one
                    }
                    if (!lagged) break;
                    rescale(ws, mx);
                    block_pv(ws, sv, va, v_addr);
                    wait_lgkm0();
                    ++i;
                }
            } else {
                // Several row blocks share each step of keys, which passes
                // through a two-slot ring (step i in slot i % 2, each slot an
                // LDS array of its own); a barrier per step publishes it and
                // frees the slot read one step ago, which then takes step
                // i + 1.  kTwoGroups: each key group's two waves share 32-key
                // steps and split their loads at the barrier.  kOneGroup: the
                // four waves share 64-key steps (two 32-key pairs), and every
                // wave, inactive ones too, issues a quarter of the next
                // step's loads with the MFMAs of the first pair.
                const int n_kg = n_mine, pstep = kstep;
                const int key_end = min(vis_end, seg_hi);
                char *slots[2];
                slots[0] = first;
                slots[1] = stage1_base + kgq * kPairBytes;
                // Step i with its slot fixed at compile time, so that every
                // LDS access and direct load names its array.
                PairReads rd;
                rd.k_off[0] = offs.k_off[0];
                rd.k_off[1] = offs.k_off[1];
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) rd.v_off[c4] = offs.v_off[c4];
                // One 32-key pair: blocks at `blocks` and blocks + 18 KB, keys kbp .. kbp + 31.
                auto pair = [&](const char *blocks, int kbp, auto side) __attribute__((always_inline)) {
                    rd.stA = blocks;
                    rd.stB = blocks + kBlockBytes;
                    float sv[8], mx;
                    pair_scores(rd, sv, mx, qf, kbp, key_end, p.scale_log2, lane, side);
                    if (__any(mx > ws.m + kMaxLag)) rescale(ws, mx);  // rare
                    pair_pv<kHiOnly>(rd, ws, sv, side);
                };
                auto step = [&](auto slot_idx, int i) __attribute__((always_inline)) {
                    constexpr int P = decltype(slot_idx)::value;
                    wait_vm<0>();    // this wave's share of step i landed
                    bare_barrier();  // step i is in; every wave is done with step i-1
                    // Only now is step i-1's slot free for step i + 1.
                    const int kb = kfirst + i * pstep;
                    if constexpr (kMode == kOneGroup) {
                        // Step i + 1's loads (empty ranges past the last
                        // step: the count stays fixed inside the MFMA stream).
                        const int kbw = kb + pstep + wave * kKeyBlock;  // this wave's block of step i + 1
                        QuadLoads ql;
                        ql.dst = slots[1 - P] + wave * kBlockBytes;
                        ql.r = block_rsrc(bc, kbw, pgA, i + 1 < n_kg);
                        ql.vrow[0] = vrow[0];
                        ql.vrow[1] = vrow[1];
                        pgA = page_of(bc, kbw + pstep);
                        if (active && kb < vis_end)
                            pair(slots[P], kb, ql);
                        else
                            ql.all(std::make_integer_sequence<int, kQkSteps>{});
                        if (active && kb + 2 * kKeyBlock < vis_end)
                            pair(slots[P] + 2 * kBlockBytes, kb + 2 * kKeyBlock, NoSide{});
                    } else {
                        if (active && i + 1 < n_kg) {
                            issue_step_share(slots[1 - P], bc, kb + pstep, pgA, pgB, vrow, my_rbl, nrb);
                            pgA = page_of(bc, kb + 2 * pstep);
                            pgB = page_of(bc, kb + 2 * pstep + kKeyBlock);
                        }
                        if (active && i < n_kg && kb < vis_end) pair(slots[P], kb, NoSide{});
                    }
                    wait_lgkm0();
                };
                for (int i = 0; i < n_iter; i += 2) {
                    step(Parity<0>{}, i);
                    if (i + 1 < n_iter) step(Parity<1>{}, i + 1);
                }
            }

            if constexpr (kMode == kOneGroup) {
                if (active) write_rows(p, ws, b, rb, whole, slot, lane);
                // Every wave is done with the ring, and every load into it
                // (the empty ones past the last step included) has landed,
                // before the next segment refills it.
                wait_vm<0>();
                bare_barrier();
            } else {
                // Merge the waves of this segment through LDS: each wave
                // puts its O rows and stats into the merge area, then all
                // threads merge them.
                // put_rows(area, ct0, stats): output tiles ct0 .. ct0 + n - 1
                // (n = the area's channels / 16) and, with stats, m and l.
                auto put_rows = [&](const auto &area, int ct0, bool stats) {
                    constexpr int n = std::is_same_v<std::decay_t<decltype(area)>, HalfMergeArea> ? kOutTiles / 2
                                                                                                 : kOutTiles;
                    const int head = lane & 15;
                    const int grp = lane >> 4;
                    float *dst = area.row(wave, head) + 4 * grp;
#pragma unroll
                    for (int ct = 0; ct < n; ++ct)
                        *reinterpret_cast<f32x4 *>(dst + 16 * ct) = ws.acc[ct0 + ct];
                    if (stats) {
                        float lt = ws.l;
                        lt += __shfl_xor(lt, 16);
                        lt += __shfl_xor(lt, 32);
                        if (grp == 0) {
                            *area.m_at(wave, head) = ws.m;
                            *area.l_at(wave, head) = lt;
                        }
                    }
                };
                if constexpr (kOne) {
                    // The workgroup's next segment, when it lies in the same
                    // 64 sequences: this wave sends its first block to its
                    // stage-0 block now, to land during the merge, and the
                    // rows go through the stage-1 blocks half a row at a
                    // time.  The barriers are bare: a full fence would wait
                    // for those loads.
                    prefetched = kMode == kOneBlockNext && mask != 0;
                    if (prefetched) {
                        const int jn = __builtin_ctzll(mask);
                        const int32_t Ln = lane_value(Ll, jn);
                        int kf, nm, nblk;
                        one_block_share(lane_value(stl, jn), Ln, turn, kf, nm, nblk);
                        if (nm > 0) {
                            const BlockCtx bn = block_ctx(p, b0 + jn, Ln);
                            issue_block(stage0_base + wave * kBlockBytes, bn, kf, page_of(bn, kf), lane);
                        }
                        const HalfMergeArea hma{stage1_base};
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            put_rows(hma, half * (kOutTiles / 2), half == 0);
                            wait_lgkm0();
                            bare_barrier();
                            merge_waves<4, kHalfCols>(p, hma, b, rb0, 0, 1, whole, slot, half * kHalfCols);
                            wait_lgkm0();
                            bare_barrier();
                        }
                    } else {
                        // Into this wave's own ring blocks, which it has
                        // finished reading: no wait for the other waves first.
                        const WaveMergeArea wma{stage0_base, stage1_base};
                        put_rows(wma, 0, true);
                        __syncthreads();
                        merge_waves<4, kDv>(p, wma, b, rb0, 0, 1, whole, slot, 0);
                        __syncthreads();
                    }
                } else {
                    // Into the ring, once every wave is done with it.
                    __syncthreads();
                    if (active) put_rows(ma, 0, true);
                    __syncthreads();
                    for (int rbl = 0; rbl < nrb; ++rbl)
                        merge_waves<2, kDv>(p, ma, b, rb0, rbl, nrb, whole, slot, 0);
                    __syncthreads();
                }
            }
        }
        base = next_base;
    }
}

// ------------------------------------------------------------- combine kernel

// Online merge of a sequence's parts g_first .. g_first + n_parts - 1 for
// one head and four channels, NB parts at a time: all loads of a batch are
// issued before any is used, so a batch costs one round trip.  Returns the
// log2-domain max M, the weight sum lsum and the weighted O sum o.
template <int NB>
__device__ inline void merge_parts(const Params &p, int rb, int head, int c, int g_first, int n_parts,
                                   int64_t st_b, int64_t chunk, float &M, float &lsum, f32x4 &o) {
    M = -INFINITY;
    lsum = 0.f;
    o = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < n_parts; k0 += NB) {
        float lv[NB];
        f32x4 ov[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int g = g_first + min(k0 + k, n_parts - 1);
            const int64_t r = ((int64_t)segment_slot(g, st_b, chunk) * p.n_rb + rb) * 16 + head;
            lv[k] = p.part_lse[r];
            ov[k] = *reinterpret_cast<const f32x4 *>(p.part_o + r * kDv + c);
        }
        __builtin_amdgcn_sched_barrier(0);  // all loads of the batch are in flight before any use
        float mb = -INFINITY;
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (k0 + k >= n_parts) lv[k] = -INFINITY;
            mb = fmaxf(mb, lv[k]);
        }
        const float m_new = fmaxf(M, mb);
        // Until some part holds a key every weight is 0; a finite reference
        // then keeps exp2 away from -inf - -inf.  (No branch here: a branch
        // on the LSEs would let the compiler sink the O loads below it.)
        const float m_ref = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(M - m_ref);
        lsum *= alpha;
        o *= alpha;
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const float w = __builtin_amdgcn_exp2f(lv[k] - m_ref);  // 0 for -inf parts
            lsum += w;
            o += w * ov[k];
        }
        M = m_new;
    }
}

// grid (batch, n_rb, 512 / kCombineChannels); 16 heads x kCombineQuads threads.
__global__ __launch_bounds__(kCombineThreads) void mla_combine_kernel(Params p) {
    const int b = blockIdx.x;
    const int rb = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int head = threadIdx.x / kCombineQuads;
    const int c = blockIdx.z * kCombineChannels + 4 * (threadIdx.x % kCombineQuads);

    int64_t st_b, lp;
    const int32_t len0 = lane < p.batch ? seq_len(p, lane) : 0;
    const int64_t chunk = line_position(p, b, lane, len0, st_b, lp).chunk;
    const int hpt = p.heads >> 4;
    const int t = rb / hpt;
    const int hh = (rb % hpt) * 16 + head;
    float *orow = p.out + (((int64_t)b * p.s_q + t) * p.heads + hh) * kDv + c;
    float *lrow = p.lse + ((int64_t)b * p.s_q + t) * p.heads + hh;
    if (lp == 0) {  // no key at all: defined empty result
        *reinterpret_cast<f32x4 *>(orow) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (threadIdx.x % kCombineQuads == 0 && blockIdx.z == 0) *lrow = -INFINITY;
        return;
    }
    // (There are p.splits ranges: the bound keeps every part read inside the
    // workspace.)
    const int g_first = (int)min(st_b / chunk, (int64_t)p.splits - 1);
    const int g_last = (int)min((st_b + lp - 1) / chunk, (int64_t)p.splits - 1);
    if (g_first == g_last) return;  // finished inside one range by the split kernel

    // Batches no wider than the parts of the sequence: a wider one would
    // repeat the last part's loads.
    const int n_parts = g_last - g_first + 1;
    float M, lsum;
    f32x4 o;
    if (n_parts <= 4)
        merge_parts<4>(p, rb, head, c, g_first, n_parts, st_b, chunk, M, lsum, o);
    else if (n_parts <= 8)
        merge_parts<8>(p, rb, head, c, g_first, n_parts, st_b, chunk, M, lsum, o);
    else
        merge_parts<kCombineBatch>(p, rb, head, c, g_first, n_parts, st_b, chunk, M, lsum, o);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    *reinterpret_cast<f32x4 *>(orow) = o * inv;
    if (threadIdx.x % kCombineQuads == 0 && blockIdx.z == 0)
        *lrow = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
}

}  // namespace mla

// ======================================================= launch configuration

namespace mla {

int groups_per_launch(int n_rb) {
    const int rem = n_rb % kWaves;
    const int full = n_rb / kWaves + (rem == 3 ? 1 : 0);
    return std::max(full, (rem == 1 || rem == 2) ? 1 : 0);
}

int default_splits(int cu_count, int n_rb) { return std::max(1, cu_count / groups_per_launch(n_rb)); }

size_t workspace_bytes(int splits, int n_rb) {
    const size_t rows = (size_t)2 * splits * n_rb * 16;
    return rows * (kDv + 1) * sizeof(float) + 256;
}

hipError_t launch_decode(hipStream_t stream, int splits, int64_t min_chunk, bool p_bf16, void *ws, const void *q,
                         const void *kv_cache, const int32_t *block_table, const int32_t *seqlens, float scale,
                         float *out, float *lse, const mla_problem *p, LaunchEvents *ev, const char **what) {
    const int n_rb = p->s_q * p->num_heads / 16;
    Params prm;
    prm.q = static_cast<const uint16_t *>(q);
    prm.kv = static_cast<const uint16_t *>(kv_cache);
    prm.block_table = p->page_size ? block_table : nullptr;
    prm.seqlens = seqlens;
    prm.out = out;
    prm.lse = lse;
    prm.part_o = static_cast<float *>(ws);
    prm.part_lse = prm.part_o + (size_t)2 * splits * n_rb * 16 * kDv;
    prm.kv_capacity = p->page_size ? 0 : p->kv_capacity;
    prm.num_pages = p->page_size ? p->num_pages : 0;
    prm.capacity = p->page_size ? (int64_t)p->max_pages * p->page_size : p->kv_capacity;
    prm.min_chunk = min_chunk;
    prm.batch = p->batch;
    prm.s_q = p->s_q;
    prm.heads = p->num_heads;
    prm.page_size = p->page_size;
    prm.max_pages = p->page_size ? p->max_pages : 0;
    prm.n_rb = n_rb;
    prm.splits = splits;
    prm.scale_log2 = scale * kLog2e;
    prm.line_gap = -1;

    // Launch sizes: with host lengths, only the ranges that hold keys, and
    // the combine only when some sequence is split.
    int grid_x = splits;
    bool need_combine = true;
    bool several_segments = p->batch > 1;  // some workgroup may take more than one sequence
    if (p->seqlens_host) {
        const HostLine ln = host_plan_line(p->seqlens_host, p->batch, splits, prm.min_chunk);
        const int64_t total = ln.total, chunk = ln.chunk;
        prm.line_gap = (int32_t)ln.gap;
        grid_x = (int)std::max<int64_t>(1, (total + chunk - 1) / chunk);
        // A workgroup can hold several segments only where a sequence with
        // keys starts inside a range (without gaps, exactly there).
        need_combine = false;
        several_segments = false;
        int64_t st = 0;
        for (int b = 0; b < p->batch; ++b) {
            const int64_t lp = padded_len(p->seqlens_host[b]);
            if (lp > 0) {
                need_combine = need_combine || st / chunk != (st + lp - 1) / chunk;
                several_segments = several_segments || st % chunk != 0;
                st += lp + ln.gap;
            }
        }
    }

    // Row-block groups of four (and a last group of three) run the one-group
    // kernel, a last group of two the two-group one and a group of one
    // (s_q * heads = 16, or the last group when n_rb % 4 == 1) the per-wave
    // one.  Each launch covers groups y0 .. y0 + n_groups - 1, with
    // grid_x x n_groups workgroups in one dimension (range_and_group).
    const int rem = n_rb % kWaves;
    const int full = n_rb / kWaves + (rem == 3 ? 1 : 0);
    if (ev) (void)hipEventRecord(ev->split_start, stream);
    hipError_t e = hipSuccess;
    if (full > 0) {
        prm.y0 = 0;
        prm.n_groups = full;
        if (p_bf16)
            hipLaunchKernelGGL((mla_split_kernel<kOneGroup, true>), dim3(grid_x * full), dim3(kThreads), 0, stream,
                               prm);
        else
            hipLaunchKernelGGL((mla_split_kernel<kOneGroup, false>), dim3(grid_x * full), dim3(kThreads), 0, stream,
                               prm);
        e = hipGetLastError();
        if (e != hipSuccess) {
            *what = "mla_split_kernel launch";
            return e;
        }
    }
    if (rem == 1 || rem == 2) {
        prm.y0 = n_rb / kWaves;
        prm.n_groups = 1;
        if (rem == 1 && several_segments)
            hipLaunchKernelGGL((mla_split_kernel<kOneBlockNext, false>), dim3(grid_x), dim3(kThreads), 0, stream,
                               prm);
        else if (rem == 1)
            hipLaunchKernelGGL((mla_split_kernel<kOneBlock, false>), dim3(grid_x), dim3(kThreads), 0, stream, prm);
        else if (p_bf16)
            hipLaunchKernelGGL((mla_split_kernel<kTwoGroups, true>), dim3(grid_x), dim3(kThreads), 0, stream, prm);
        else
            hipLaunchKernelGGL((mla_split_kernel<kTwoGroups, false>), dim3(grid_x), dim3(kThreads), 0, stream,
                               prm);
        e = hipGetLastError();
        if (e != hipSuccess) {
            *what = "mla_split_kernel launch";
            return e;
        }
    }
    if (ev) (void)hipEventRecord(ev->split_stop, stream);
    if (ev) ev->combine_ran = need_combine;
    if (need_combine) {
        if (ev) (void)hipEventRecord(ev->comb_start, stream);
        hipLaunchKernelGGL(mla_combine_kernel, dim3(p->batch, n_rb, kDv / kCombineChannels),
                           dim3(kCombineThreads), 0, stream, prm);
        e = hipGetLastError();
        if (e != hipSuccess) {
            *what = "mla_combine_kernel launch";
            return e;
        }
        if (ev) (void)hipEventRecord(ev->comb_stop, stream);
    }
        return hipSuccess;
}

}  // namespace mla
