// The MLA steps on either side of the attention kernel, for MI355X (gfx950).
//
// MLA keeps one latent row per token: the low-rank joint compression of the
// keys and values ("FlashMLA-ETAP", gist.science technical summary,
// Integration and Implementation).  Read as 512 compressed-KV channels and
// a 64-channel rotary key, the row lets each head's key up-projection be
// folded into its query (the absorbed query), and the value up-projection
// be applied once to the attention output:
//   * append:  the new tokens' latent rows go into the cache;
//   * absorb:  q[h] = [ W_UK[h]^T q_nope[h] , q_rope[h] ]  (576 wide, bf16);
//   * project: out[h] = W_UV[h] o[h]  (o: the 512-wide latent output).
//
// At decode sizes (a few to a few hundred query rows) the projections read
// each weight once and do 2 x rows flops per weight: below ~150 rows the
// weights' HBM bytes bound them, and at a few rows the latency of one
// memory round trip does.  So the kernels below issue every load of a wave
// at once and let MFMA do the arithmetic; they do not aim at data reuse.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "context.h"
#include "mla_decode.h"

namespace mla_steps {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

constexpr int kLatent = MLA_HEAD_DIM_V;                // 512 compressed channels
constexpr int kRope = MLA_HEAD_DIM_QK - MLA_HEAD_DIM_V;  // 64 rotary channels
constexpr int kRowBytes = MLA_HEAD_DIM_QK * 2;          // 1152

struct AppendParams {
    const uint16_t *rows;  // [B][s_q][576]
    uint16_t *kv;
    const int32_t *block_table;
    const int32_t *seqlens;
    int64_t kv_capacity;   // contiguous
    int64_t num_pages;     // paged
    int64_t capacity;      // keys one sequence can hold
    int32_t s_q;
    int32_t page_size;
    int32_t max_pages;
};

// One wave per new row: 72 chunks of 16 bytes.  The row is loaded before the
// length (and page id) that places it, so the two memory round trips overlap.
__global__ __launch_bounds__(64) void append_kernel(AppendParams p) {
    const int row = blockIdx.x;  // b * s_q + t
    const int lane = threadIdx.x;
    const int b = row / p.s_q, t = row % p.s_q;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(p.rows + (int64_t)row * MLA_HEAD_DIM_QK);
    constexpr int kChunks = kRowBytes / 16;  // 72
    const u32x4 v0 = src[lane];
    const u32x4 v1 = src[64 + (lane < kChunks - 64 ? lane : kChunks - 65)];  // no branch around loads
    int64_t L = p.seqlens[b];
    L = L < p.s_q ? p.s_q : (L > p.capacity ? p.capacity : L);
    const int64_t key = L - p.s_q + t;
    int64_t dst_row;
    if (p.page_size) {
        int64_t page = p.block_table[(int64_t)b * p.max_pages + key / p.page_size];
        page = page < 0 ? 0 : (page >= p.num_pages ? p.num_pages - 1 : page);
        dst_row = page * p.page_size + key % p.page_size;
    } else {
        dst_row = (int64_t)b * p.kv_capacity + key;
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(p.kv + dst_row * MLA_HEAD_DIM_QK);
    dst[lane] = v0;
    if (lane < kChunks - 64) dst[64 + lane] = v1;
}

// One MFMA operand (16x16x32, A or B: same layout) from 16 rows of `base`
// starting at row r0: lane l gets 8 consecutive bf16 of row r0 + l%16 at
// column k0 + 8(l/16).  Rows at or past `rows` read row rows-1 instead (no
// branch around the load); `zero_past` then clears them, after the wave has
// issued all its loads.
__device__ inline bf16x8 load_rows8(const uint16_t *base, int64_t row_stride, int r0, int rows, int k0,
                                    int lane) {
    const int r = r0 + (lane & 15);
    return *reinterpret_cast<const bf16x8 *>(base + (int64_t)(r < rows ? r : rows - 1) * row_stride + k0 +
                                             8 * (lane >> 4));
}

__device__ inline bf16x8 zero_past(bf16x8 v, int r0, int rows, int lane) {
    return r0 + (lane & 15) < rows ? v : bf16x8{};
}

// The projections take the 16-row tiles of up to kMaxTiles x 16 rows in one
// wave, with one load of its weights; the launch picks the fewest tiles that
// cover the rows (1, 2 or 4).
constexpr int kMaxTiles = 4;

struct AbsorbParams {
    const uint16_t *q_nope;  // [rows][H][d_nope]
    const uint16_t *q_rope;  // [rows][H][64]
    const uint16_t *w_uk;    // [H][512][d_nope]
    uint16_t *q_out;         // [rows][H][576]
    int32_t rows, heads, d_nope;
};

// One wave per (cg, h, rg): latent channels 16 kCh cg .. (kCh tiles of 16)
// of head h for the up to 16 kTiles rows from 16 kTiles rg.
// q_lat^T (channels x rows) = W_UK[h] (channels x d_nope) . q_nope^T
// (d_nope x rows): A from the weight rows, B from the query rows, 16
// contiguous bytes per lane each.  The reduction dimension goes in chunks of
// 128 whose loads (weights once, queries per tile) are all issued before
// the first MFMA, so the wave waits for memory once per chunk (once, for
// d_nope <= 128).  More channel tiles per wave read the query rows fewer
// times over.  D lane l: row l%16 of the tile, channels 4(l/16) .. +3 of
// the channel tile, stored as 4 bf16.  The waves of channel group 0 also
// copy the rotary part of their rows.
constexpr int kAbsorbChunk = 128;

template <int kTiles, int kCh>
__global__ __launch_bounds__(64) void absorb_kernel(AbsorbParams p) {
    const int lane = threadIdx.x;
    const int h = blockIdx.x, cg = blockIdx.y, r0 = blockIdx.z * 16 * kTiles;
    const int ch0 = cg * 16 * kCh;
    const int64_t q_stride = (int64_t)p.heads * p.d_nope;  // between rows
    const uint16_t *qn = p.q_nope + (int64_t)h * p.d_nope;
    const uint16_t *w = p.w_uk + ((int64_t)h * kLatent + ch0) * p.d_nope;
    constexpr int kK = kAbsorbChunk / 32;
    f32x4 acc[kCh][kTiles] = {};
    for (int c0 = 0; c0 < p.d_nope; c0 += kAbsorbChunk) {
        bf16x8 aw[kCh][kK], bq[kTiles][kK];
        // Reduction steps past d_nope load the last step again (no branch
        // around the loads) and are zeroed; so are rows past the last.
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
#pragma unroll
            for (int s = 0; s < kK; ++s) {
                const int k0 = c0 + 32 * s;
                aw[c][s] = load_rows8(w + 16 * c * p.d_nope, p.d_nope, 0, 16, k0 < p.d_nope ? k0 : p.d_nope - 32, lane);
            }
        }
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
#pragma unroll
            for (int s = 0; s < kK; ++s) {
                const int k0 = c0 + 32 * s;
                bq[t][s] = load_rows8(qn, q_stride, r0 + 16 * t, p.rows, k0 < p.d_nope ? k0 : p.d_nope - 32, lane);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the chunk in flight before any is used
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
#pragma unroll
            for (int s = 0; s < kK; ++s) aw[c][s] = c0 + 32 * s < p.d_nope ? aw[c][s] : bf16x8{};
        }
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
#pragma unroll
            for (int s = 0; s < kK; ++s) bq[t][s] = zero_past(bq[t][s], r0 + 16 * t, p.rows, lane);
        }
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
#pragma unroll
            for (int t = 0; t < kTiles; ++t) {
#pragma unroll
                for (int s = 0; s < kK; ++s)
                    acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[c][s], bq[t][s], acc[c][t], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const int r = r0 + 16 * t + (lane & 15);
        if (r < p.rows) {
            uint16_t *dst = p.q_out + ((int64_t)r * p.heads + h) * MLA_HEAD_DIM_QK + ch0 + 4 * (lane >> 4);
#pragma unroll
            for (int c = 0; c < kCh; ++c) {
                bf16x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = static_cast<__bf16>(acc[c][t][i]);  // to nearest even
                *reinterpret_cast<bf16x4 *>(dst + 16 * c) = v;
            }
        }
    }
    if (cg == 0) {
        // Rotary part: 128 B per row, lane l -> row l/4 of each 16, 32 bytes.
        u32x4 v[kTiles][2];
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
            const int rr = r0 + 16 * t + (lane >> 2);
            const u32x4 *src = reinterpret_cast<const u32x4 *>(
                                   p.q_rope + ((int64_t)(rr < p.rows ? rr : p.rows - 1) * p.heads + h) * kRope) +
                               2 * (lane & 3);
            v[t][0] = src[0];
            v[t][1] = src[1];
        }
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
            const int rr = r0 + 16 * t + (lane >> 2);
            if (rr < p.rows) {
                u32x4 *dst = reinterpret_cast<u32x4 *>(p.q_out + ((int64_t)rr * p.heads + h) * MLA_HEAD_DIM_QK + kLatent) +
                             2 * (lane & 3);
                dst[0] = v[t][0];
                dst[1] = v[t][1];
            }
        }
    }
}

struct ProjectParams {
    const float *o;         // [rows][H][512]
    const uint16_t *w_uv;   // [H][d_v][512]
    float *out;             // [rows][H][d_v]
    int32_t rows, heads, d_v;
};

// Workgroup (eg, h, rg) of four waves: value channels 16eg .. 16eg+15 of
// head h for the up to 16 kTiles rows from 16 kTiles rg; wave w takes
// latent channels 128w .. 128w+127 of the reduction.  out^T (d_v x rows) =
// W_UV[h] (d_v x 512) . o^T (512 x rows): A from the weight rows (loaded once
// for all tiles), B from the output rows split into bf16 hi + lo (two MFMAs
// per 32 channels).  All of a wave's loads are issued before its first
// MFMA.  The four partial tiles are summed through LDS in wave order (the
// same order on every run); D lane l: row l%16 of the tile, channels
// 4(l/16) .. +3, stored as 16 bytes.  (Eight or sixteen waves per workgroup
// measured 8% and 6% slower at 128 rows, and no faster at 16.)
constexpr int kProjectWaves = 4;
constexpr int kProjectSlice = kLatent / kProjectWaves;  // 128

template <int kTiles>
__global__ __launch_bounds__(64 * kProjectWaves) void project_kernel(ProjectParams p) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int h = blockIdx.x, eg = blockIdx.y, r0 = blockIdx.z * 16 * kTiles;
    const int k = wv * kProjectSlice + 8 * (lane >> 4);
    const uint16_t *w = p.w_uv + ((int64_t)h * p.d_v + eg * 16 + (lane & 15)) * kLatent + k;
    constexpr int kSteps = kProjectSlice / 32;
    bf16x8 aw[kSteps];
    f32x4 x[kTiles][2 * kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) aw[s] = *reinterpret_cast<const bf16x8 *>(w + 32 * s);
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        // Lanes past the last row read the last row (no branch around the
        // loads) and zero it.
        const int r = r0 + 16 * t + (lane & 15);
        const float *orow = p.o + ((int64_t)(r < p.rows ? r : p.rows - 1) * p.heads + h) * kLatent + k;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            x[t][2 * s] = *reinterpret_cast<const f32x4 *>(orow + 32 * s);
            x[t][2 * s + 1] = *reinterpret_cast<const f32x4 *>(orow + 32 * s + 4);
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load in flight before any is used
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        const bool live = r0 + 16 * t + (lane & 15) < p.rows;
#pragma unroll
        for (int i = 0; i < 2 * kSteps; ++i) x[t][i] = live ? x[t][i] : f32x4{};
    }
    __shared__ f32x4 part[kProjectWaves][kTiles][64];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
        f32x4 acc = {};
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            bf16x8 hi, lo;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xv = x[t][2 * s + j / 4][j % 4];
                const __bf16 hb = static_cast<__bf16>(xv);
                hi[j] = hb;
                lo[j] = static_cast<__bf16>(xv - static_cast<float>(hb));
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[s], hi, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[s], lo, acc, 0, 0, 0);
        }
        part[wv][t][lane] = acc;
    }
    __syncthreads();
    // Thread i sums tile i/64, lane i%64 over the waves.
    if (threadIdx.x < 64 * kTiles) {
        const int t = threadIdx.x >> 6;
        const int r = r0 + 16 * t + (lane & 15);
        if (r < p.rows) {
            f32x4 sum = part[0][t][lane];
#pragma unroll
            for (int i = 1; i < kProjectWaves; ++i) sum += part[i][t][lane];
            *reinterpret_cast<f32x4 *>(p.out + ((int64_t)r * p.heads + h) * p.d_v + eg * 16 + 4 * (lane >> 4)) = sum;
        }
    }
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15) == 0; }

int tiles_for(int rows) { return rows <= 16 ? 1 : rows <= 32 ? 2 : kMaxTiles; }

// Both projections launch with the head in blockIdx.x.  Workgroups go to
// the eight XCDs (each with its own L2) in turn by linear id, so with a head
// count that is a multiple of 8 every workgroup of head h runs on XCD h % 8,
// and the head's query or latent-output rows are fetched into one L2 only.
// Measured HBM fetches are then 1.01-1.03x the algorithmic bytes; with the
// channel group first every XCD fetched every head's rows (projection: 2.4x
// at 16 rows, 5.7x at 128).

}  // namespace mla_steps

using mla_host::fail;
using mla_host::hip_fail;

extern "C" {

int mla_append_kv(mla_ctx *ctx, const void *new_rows, void *kv_cache, const int32_t *block_table,
                  const int32_t *seqlens, const mla_problem *p) {
    using namespace mla_steps;
    if (!ctx) return fail(nullptr, MLA_ERR_INVALID_ARG, "ctx is NULL");
    ctx->err.clear();
    if (!p) return fail(ctx, MLA_ERR_INVALID_ARG, "problem description is NULL");
    if (!new_rows || !kv_cache || !seqlens)
        return fail(ctx, MLA_ERR_INVALID_ARG, "new_rows, kv_cache and seqlens must be non-NULL");
    if (p->batch < 1 || p->s_q < 1) return fail(ctx, MLA_ERR_INVALID_ARG, "batch and s_q must be >= 1");
    if ((int64_t)p->batch * p->s_q > INT32_MAX) return fail(ctx, MLA_ERR_UNSUPPORTED, "batch * s_q too large");
    if (p->head_dim_qk != MLA_HEAD_DIM_QK)
        return fail(ctx, MLA_ERR_UNSUPPORTED, "head_dim_qk must be %d (got %d)", MLA_HEAD_DIM_QK, p->head_dim_qk);
    if (!aligned16(new_rows) || !aligned16(kv_cache))
        return fail(ctx, MLA_ERR_INVALID_ARG, "new_rows and kv_cache must be 16-byte aligned");
    AppendParams ap{};
    ap.rows = static_cast<const uint16_t *>(new_rows);
    ap.kv = static_cast<uint16_t *>(kv_cache);
    ap.seqlens = seqlens;
    ap.s_q = p->s_q;
    if (p->page_size == 0) {
        if (block_table)
            return fail(ctx, MLA_ERR_INVALID_ARG, "block_table given but page_size is 0 (contiguous)");
        if (p->kv_capacity < p->s_q || p->kv_capacity > (int64_t)INT32_MAX)
            return fail(ctx, MLA_ERR_INVALID_ARG, "kv_capacity must be in [s_q, 2^31) (got %lld)",
                        (long long)p->kv_capacity);
        ap.kv_capacity = p->kv_capacity;
        ap.capacity = p->kv_capacity;
    } else {
        if (p->page_size < 0 || p->page_size % MLA_KEY_BLOCK)
            return fail(ctx, MLA_ERR_UNSUPPORTED, "page_size must be a positive multiple of %d (got %d)",
                        MLA_KEY_BLOCK, p->page_size);
        if (!block_table) return fail(ctx, MLA_ERR_INVALID_ARG, "paged layout needs a block_table");
        if (p->num_pages < 1 || p->max_pages < 1)
            return fail(ctx, MLA_ERR_INVALID_ARG, "num_pages and max_pages must be >= 1");
        ap.capacity = (int64_t)p->max_pages * p->page_size;
        if (ap.capacity < p->s_q || ap.capacity > (int64_t)INT32_MAX)
            return fail(ctx, MLA_ERR_INVALID_ARG, "max_pages * page_size must be in [s_q, 2^31)");
        ap.block_table = block_table;
        ap.page_size = p->page_size;
        ap.num_pages = p->num_pages;
        ap.max_pages = p->max_pages;
    }
    if (p->seqlens_host) {
        for (int b = 0; b < p->batch; ++b) {
            const int32_t L = p->seqlens_host[b];
            if (L < p->s_q || (int64_t)L > ap.capacity)
                return fail(ctx, MLA_ERR_INVALID_ARG, "seqlens[%d] = %d outside [s_q = %d, capacity = %lld]", b, L,
                            p->s_q, (long long)ap.capacity);
        }
    }
    hipLaunchKernelGGL(append_kernel, dim3(p->batch * p->s_q), dim3(64), 0, ctx->stream, ap);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MLA_OK : hip_fail(ctx, e, "append_kernel launch");
}

int mla_absorb_q(mla_ctx *ctx, const void *q_nope, const void *q_rope, const void *w_uk, void *q_out,
                 int32_t rows, int32_t heads, int32_t d_nope) {
    using namespace mla_steps;
    if (!ctx) return fail(nullptr, MLA_ERR_INVALID_ARG, "ctx is NULL");
    ctx->err.clear();
    if (!q_nope || !q_rope || !w_uk || !q_out)
        return fail(ctx, MLA_ERR_INVALID_ARG, "q_nope, q_rope, w_uk and q_out must be non-NULL");
    if (rows < 1 || heads < 1) return fail(ctx, MLA_ERR_INVALID_ARG, "rows and heads must be >= 1");
    if (d_nope < 32 || d_nope % 32)
        return fail(ctx, MLA_ERR_UNSUPPORTED, "d_nope must be a positive multiple of 32 (got %d)", d_nope);
    if (heads > 65535 || (rows + 15) / 16 > 65535 || (int64_t)heads * d_nope > (1 << 20))
        return fail(ctx, MLA_ERR_UNSUPPORTED, "rows or heads too large");
    if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(w_uk) || !aligned16(q_out))
        return fail(ctx, MLA_ERR_INVALID_ARG, "q_nope, q_rope, w_uk and q_out must be 16-byte aligned");
    AbsorbParams ap{static_cast<const uint16_t *>(q_nope), static_cast<const uint16_t *>(q_rope),
                    static_cast<const uint16_t *>(w_uk), static_cast<uint16_t *>(q_out), rows, heads, d_nope};
    // Few rows: one channel tile per wave, many waves.  More rows: four
    // channel tiles and four row tiles per wave, so the query rows are read
    // by 8 waves per head instead of 32.
    const int tiles = tiles_for(rows);
    if (tiles == 1)
        hipLaunchKernelGGL((absorb_kernel<1, 1>), dim3(heads, kLatent / 16, (rows + 15) / 16), dim3(64), 0,
                           ctx->stream, ap);
    else if (tiles == 2)
        hipLaunchKernelGGL((absorb_kernel<2, 1>), dim3(heads, kLatent / 16, (rows + 31) / 32), dim3(64), 0,
                           ctx->stream, ap);
    else
        hipLaunchKernelGGL((absorb_kernel<kMaxTiles, 4>), dim3(heads, kLatent / 64, (rows + 63) / 64), dim3(64), 0,
                           ctx->stream, ap);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MLA_OK : hip_fail(ctx, e, "absorb_kernel launch");
}

int mla_project_out(mla_ctx *ctx, const float *o, const void *w_uv, float *out, int32_t rows, int32_t heads,
                    int32_t d_v) {
    using namespace mla_steps;
    if (!ctx) return fail(nullptr, MLA_ERR_INVALID_ARG, "ctx is NULL");
    ctx->err.clear();
    if (!o || !w_uv || !out) return fail(ctx, MLA_ERR_INVALID_ARG, "o, w_uv and out must be non-NULL");
    if (rows < 1 || heads < 1) return fail(ctx, MLA_ERR_INVALID_ARG, "rows and heads must be >= 1");
    if (d_v < 16 || d_v % 16)
        return fail(ctx, MLA_ERR_UNSUPPORTED, "d_v must be a positive multiple of 16 (got %d)", d_v);
    if (heads > 65535 || (rows + 15) / 16 > 65535 || d_v / 16 > 65535)
        return fail(ctx, MLA_ERR_UNSUPPORTED, "rows, heads or d_v too large");
    if (!aligned16(o) || !aligned16(w_uv) || !aligned16(out))
        return fail(ctx, MLA_ERR_INVALID_ARG, "o, w_uv and out must be 16-byte aligned");
    ProjectParams pp{o, static_cast<const uint16_t *>(w_uv), out, rows, heads, d_v};
    const int tiles = tiles_for(rows);
    const dim3 grid(heads, d_v / 16, (rows + 16 * tiles - 1) / (16 * tiles));
    if (tiles == 1)
        hipLaunchKernelGGL(project_kernel<1>, grid, dim3(64 * kProjectWaves), 0, ctx->stream, pp);
    else if (tiles == 2)
        hipLaunchKernelGGL(project_kernel<2>, grid, dim3(64 * kProjectWaves), 0, ctx->stream, pp);
    else
        hipLaunchKernelGGL(project_kernel<kMaxTiles>, grid, dim3(64 * kProjectWaves), 0, ctx->stream, pp);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MLA_OK : hip_fail(ctx, e, "project_kernel launch");
}

}  // extern "C"
