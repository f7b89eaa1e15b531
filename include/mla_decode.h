/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) MLA decode-attention library.
 *
 * The operation is the attention step of Multi-head Latent Attention decode
 * as "FlashMLA-ETAP" states it (gist.science technical summary, Methodology,
 * the ETAP bullet): S = Q K^T, P = softmax(S), O = P V, over the latent KV
 * cache that MLA's low-rank joint compression leaves (same summary,
 * Integration and Implementation): one 576-wide bf16 row per token, shared
 * by all heads, with K = all 576 channels and V = the first 512 channels of
 * the same row (head dimension 576: arxivlens page, Limitations).  The
 * per-GPU shape is 16 heads (technical summary, Problem Statement: 128 heads
 * over 8 GPUs), a short query and a long context.
 *
 * Conventions for every entry point:
 *  - Tensors are plain pointers to DEVICE memory owned by the caller; the
 *    library never frees or retains them beyond the call.  Host pointers are
 *    marked "host".
 *  - All tensors are dense, row-major, in the element types stated.  bf16 is
 *    passed as its 16-bit pattern.
 *  - Return values are mla_status codes; nothing throws across the ABI.  On
 *    failure mla_last_error() describes the first problem found.
 *  - Argument checks are host code and run before any HIP call.
 *  - mla_decode only enqueues work on the context's stream: it never blocks
 *    the host.  With a caller's workspace (mla_ctx_set_workspace), or once
 *    the context's own workspace is large enough (mla_ctx_reserve), it never
 *    allocates either.
 *  - A context is used by one host thread at a time.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, bad length */
    MLA_ERR_UNSUPPORTED = -2, /* well-formed but outside what the kernels implement */
    MLA_ERR_WORKSPACE = -3,   /* workspace too small, or its allocation failed */
    MLA_ERR_HIP = -4          /* a HIP runtime call failed */
} mla_status;

/* Dimensions fixed by the latent layout. */
#define MLA_HEAD_DIM_QK 576
#define MLA_HEAD_DIM_V 512
/* Keys per kernel block: page sizes must be multiples of it. */
#define MLA_KEY_BLOCK 16
/* Line keys the split plan charges to the end of every sequence with keys
 * when, without them, some sequence would start inside a key range (see
 * mla_plan): a range that holds several segments pays a fixed cost for each
 * (merge, query load, pipeline refill), so it takes fewer real keys. */
#define MLA_PLAN_SEQ_GAP 128

/*
 * Sizes of one decode call (all counts in elements).
 *
 *  batch        B >= 1 sequences.
 *  s_q          query tokens per sequence, >= 1.  The new tokens are the last
 *               s_q positions of each sequence, so with s_q > 1 the mask is
 *               causal: token t (0-based) sees keys 0 .. L_b - s_q + t.
 *  num_heads    H, a multiple of 16.
 *  head_dim_qk  must be 576;  head_dim_v must be 512.
 *  page_size    0 for the contiguous layout; otherwise keys per page, a
 *               multiple of MLA_KEY_BLOCK.
 *  kv_capacity  contiguous layout: rows reserved per sequence (the stride
 *               between sequences is kv_capacity * 576 elements).  Ignored
 *               when paged.
 *  num_pages    paged layout: pages in the pool.  Ignored when contiguous.
 *  max_pages    paged layout: length of a block-table row.
 *  seqlens_host optional host copy of the device seqlens.  When given, the
 *               lengths are checked (s_q <= L_b <= capacity) and launches are
 *               sized to the work; when NULL nothing on the host reads the
 *               lengths and the kernels clamp them to [0, capacity].
 */
typedef struct {
    int32_t batch;
    int32_t s_q;
    int32_t num_heads;
    int32_t head_dim_qk;
    int32_t head_dim_v;
    int32_t page_size;
    int64_t kv_capacity;
    int64_t num_pages;
    int32_t max_pages;
    const int32_t *seqlens_host;
} mla_problem;

typedef struct mla_ctx mla_ctx;

/*
 * Create a context bound to the current HIP device and to `stream` (a
 * hipStream_t; NULL means the default stream).  Until it is given a
 * caller's workspace the context allocates its own on first use.  Returns
 * MLA_OK and sets *ctx, or an error code.
 */
int mla_ctx_create(mla_ctx **ctx, void *stream);

/* Release the context and the workspace it allocated itself (synchronizes
 * its stream first).  A caller's workspace is not touched.  NULL is
 * accepted. */
int mla_ctx_destroy(mla_ctx *ctx);

/*
 * Device workspace mla_decode needs on `ctx` for problems of up to `s_q`
 * query tokens and `num_heads` heads: the split partials (normalized O and
 * LSE of every key range that ends inside a sequence), 2 * splits *
 * (s_q * num_heads / 16) * 16 * 513 floats plus 256 bytes, where splits is
 * the key-range count of one launch (the device's CU count over the
 * row-block groups that share a launch, or MLA_OPT_NUM_SPLITS).  It does not
 * depend on the batch or the lengths.  Changing MLA_OPT_NUM_SPLITS changes
 * it.  Writes the byte count to *bytes.
 */
int mla_workspace_size(const mla_ctx *ctx, int32_t s_q, int32_t num_heads, size_t *bytes);

/*
 * Give the context a workspace owned by the caller: `bytes` bytes of device
 * memory at `dev_ptr`, 256-byte aligned, on the context's device.  From then
 * on mla_decode uses it for the split partials and never allocates, frees
 * or synchronizes; a problem that needs more than `bytes` (see
 * mla_workspace_size) is refused with MLA_ERR_WORKSPACE before anything is
 * enqueued.  The buffer holds no state between calls; it must stay valid
 * until the work enqueued with it (and any graph captured with it) has run,
 * and two contexts must not share it while their work can overlap.  The
 * context's own workspace, if any, is kept until mla_ctx_destroy (work
 * already enqueued may use it).  dev_ptr = NULL returns to a workspace the
 * context allocates itself.  No HIP call is made.
 */
int mla_ctx_set_workspace(mla_ctx *ctx, void *dev_ptr, size_t bytes);

/*
 * Make sure the context's own workspace holds the split partials for
 * problems with up to `s_q` tokens and `num_heads` heads, so that later
 * mla_decode calls of that size do not allocate (needed before capturing
 * mla_decode into a graph).  Allocates with hipMalloc when it must grow; the
 * smaller buffer it replaces is freed only by mla_ctx_destroy, so work
 * already enqueued or captured keeps a valid buffer and no synchronization
 * is needed.  With a caller's workspace set it only checks that it is large
 * enough (MLA_ERR_WORKSPACE if not).  Growing while the context's stream is
 * being captured is refused (MLA_ERR_WORKSPACE).
 */
int mla_ctx_reserve(mla_ctx *ctx, int32_t s_q, int32_t num_heads);

/*
 * Tuning knobs (they change speed, never results beyond rounding):
 *  MLA_OPT_NUM_SPLITS  number of key-range workgroups per row-block group
 *                      (default: the device's CU count divided by the
 *                      row-block groups that one launch runs side by side;
 *                      groups of four row blocks share a launch, a last
 *                      group of one or two runs in its own); 0 restores it.
 *  MLA_OPT_MIN_CHUNK   smallest key range given to one workgroup (default
 *                      64, rounded up to MLA_KEY_BLOCK); 0 restores it.
 *  MLA_OPT_KERNEL_TIMING  1: bracket every kernel launch with HIP events on
 *                      the context's stream (see mla_ctx_kernel_times); 0: off.
 *
 * A precision knob (default off; the only option that changes results):
 *  MLA_OPT_P_BF16      1: where several 16-row blocks of a sequence share
 *                      each key step (s_q * num_heads >= 32; a last lone
 *                      block of 16 rows is not affected), the softmax
 *                      weights P enter P V as one bf16 value each instead of
 *                      a bf16 high part plus a bf16 remainder, which halves
 *                      that product's MFMA work.  Each weight is then off by
 *                      at most 2^-8 of itself (bf16 keeps 8 significant
 *                      bits), so every O element moves by at most
 *                      2^-8 * max_j |V[j][c]| (plus fp32 rounding)
 *                      from the default result (the sum and the LSE keep
 *                      fp32 weights).  On N(0,1) inputs that
 *                      is an O RMSE of about 1e-5 at 64K keys and 1e-4 at 512.
 *                      With 16 rows (one block) it changes nothing: there
 *                      both parts cost one MFMA.  0: the default.
 */
typedef enum {
    MLA_OPT_NUM_SPLITS = 1,
    MLA_OPT_MIN_CHUNK = 2,
    MLA_OPT_KERNEL_TIMING = 3,
    MLA_OPT_P_BF16 = 4
} mla_option;
int mla_ctx_set_option(mla_ctx *ctx, int option, int64_t value);

/*
 * Per-kernel device time of the launches made since the last query while
 * MLA_OPT_KERNEL_TIMING was on: total milliseconds of the split kernel and
 * of the combine kernel, and how many of each ran.  Synchronizes the
 * context's stream, then forgets the recorded launches.
 */
int mla_ctx_kernel_times(mla_ctx *ctx, double *split_ms, int64_t *split_launches,
                         double *combine_ms, int64_t *combine_launches);

/* Text of the last error on `ctx` (or of the calling thread's last
 * context-free call when ctx is NULL).  Never NULL. */
const char *mla_last_error(const mla_ctx *ctx);

/*
 * MLA decode attention ("FlashMLA-ETAP", gist.science technical summary,
 * Methodology: S = Q K^T, P = softmax(S), O = P V), for every sequence b,
 * query token t and head h:
 *   s_j      = scale * sum_{c<576} q[b,t,h,c] * kv(b,j)[c]   for visible j
 *   out[b,t,h,c] = sum_j softmax(s)_j * kv(b,j)[c]           for c < 512
 *   lse[b,t,h]   = ln sum_j exp(s_j)
 *
 *  q            bf16 [B][s_q][H][576], 16-byte aligned.
 *  kv_cache     bf16, 16-byte aligned; contiguous: [B][kv_capacity][576];
 *               paged: pool [num_pages][page_size][576].
 *  block_table  NULL for the contiguous layout; paged: int32
 *               [B][max_pages], entry j of row b is the pool page holding
 *               keys j*page_size .. (j+1)*page_size-1 of sequence b.  Entries
 *               past ceil(L_b / page_size) and cache slots past L_b are
 *               never read (they may hold anything, NaN included).
 *  seqlens      int32 [B]: L_b, the number of cached keys including the s_q
 *               new ones.
 *  scale        multiplies q.k before the softmax (1/sqrt(576) for MLA).
 *  out          fp32 [B][s_q][H][512], 16-byte aligned.
 *  lse          fp32 [B][s_q][H], natural log.
 *  p            sizes, see mla_problem.
 *
 * A row that sees no key (only possible with unchecked lengths L_b < s_q)
 * gets out = 0 and lse = -inf.  Page ids are clamped into the pool.
 * Asynchronous on the context's stream.
 */
int mla_decode(mla_ctx *ctx, const void *q, const void *kv_cache,
               const int32_t *block_table, const int32_t *seqlens, float scale,
               float *out, float *lse, const mla_problem *p);

/*
 * mla_decode for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid device allocation.
 * Same arguments, checks and result as mla_decode (on the stream `stream`, a
 * hipStream_t, NULL for the default stream), but with no context: nothing
 * is allocated, freed or synchronized.  The split partials go to a static
 * scratch array of mla_noalloc_scratch_bytes() bytes (64.1 MiB) that every
 * GPU the library runs on holds until the process ends; its address is
 * looked up on the first call on each device.  The default split plan is
 * used when its partials fit the array, else the largest key-range count
 * that fits (the same result up to rounding); a problem of more than 16,384
 * query rows (s_q * num_heads) does not fit at all and is refused with
 * MLA_ERR_WORKSPACE before anything is enqueued.  All calls on one GPU share
 * its array: calls that may overlap on one GPU (several streams or threads)
 * race.  Errors go to mla_last_error(NULL).
 */
int mla_decode_noalloc(void *stream, const void *q, const void *kv_cache, const int32_t *block_table,
                       const int32_t *seqlens, float scale, float *out, float *lse, const mla_problem *p);

/* Size of the static scratch array of mla_decode_noalloc, in bytes. */
size_t mla_noalloc_scratch_bytes(void);

/*
 * Host-only argument check of mla_decode (the same checks, in the same
 * order, without a context or any HIP call).  Pointers are only tested for
 * NULL and alignment.  The message goes to mla_last_error(NULL).
 */
int mla_validate(const void *q, const void *kv_cache, const int32_t *block_table,
                 const int32_t *seqlens, float scale, const float *out,
                 const float *lse, const mla_problem *p);

/*
 * The split-KV plan, evaluated on the host exactly as every workgroup
 * evaluates it on the device.  The keys of all sequences are laid end to end
 * on a line, each sequence padded to a multiple of MLA_KEY_BLOCK; the line is
 * cut into `num_splits` equal ranges of `chunk` keys (a multiple of
 * MLA_KEY_BLOCK, at least `min_chunk`), and workgroup g takes range g.  When
 * that line would start some sequence with keys inside a range, every
 * sequence with keys is followed instead by MLA_PLAN_SEQ_GAP line keys that
 * hold no key, and the ranges are cut from that longer line.  A workgroup
 * range meets a sequence in a segment; a sequence that lies inside one range
 * is finished there, otherwise each segment writes a partial result into
 * slot 2*g + (segment does not start the range) and a merge combines them.
 *
 *  seqlens_host  host int32 [batch].
 *  segs          host output, room for max_segs segments (may be NULL to
 *                count only); *n_segs receives the total count.
 *  info          host output: chunk, keys on the line, active workgroups,
 *                number of sequences that need the merge, and the line keys
 *                after each sequence (0 or MLA_PLAN_SEQ_GAP).
 */
typedef struct {
    int32_t group;     /* workgroup (key range) index */
    int32_t seq;       /* sequence b */
    int32_t key_begin; /* first key of the segment, in sequence b */
    int32_t key_end;   /* one past the last real key (<= L_b) */
    int32_t slot;      /* partial slot, or -1 when the segment is the whole sequence */
} mla_plan_segment;

typedef struct {
    int64_t chunk;
    int64_t total_keys;      /* keys on the line, gaps included */
    int32_t active_groups;
    int32_t split_sequences;
    int64_t seq_gap;         /* line keys after each sequence with keys */
} mla_plan_info;

int mla_plan(const int32_t *seqlens_host, int32_t batch, int32_t num_splits,
             int64_t min_chunk, mla_plan_segment *segs, int32_t max_segs,
             int32_t *n_segs, mla_plan_info *info);

/* ------------------------------------------------------------------------
 * The MLA steps on either side of the attention.  MLA's low-rank joint
 * compression keeps one latent row per token (gist.science technical
 * summary, Integration and Implementation); the 576-wide row is read as the
 * 512-channel compressed KV followed by the 64-channel rotary key, and the
 * per-head up-projections are absorbed into the query and applied to the
 * attention output.  The per-head dimensions d_nope (query part without
 * rotary embedding) and d_v (value head) are arguments: the pages do not fix
 * them (DeepSeek-V3's are 128 and 128).  All three run on the context's
 * stream and never allocate.
 */

/*
 * Latent-cache append: the s_q new latent rows of each sequence become keys
 * L_b - s_q .. L_b - 1 of that sequence (token t at key L_b - s_q + t), in
 * the contiguous or the paged layout of mla_decode.  A byte copy.
 *
 *  new_rows     bf16 [B][s_q][576], 16-byte aligned.
 *  kv_cache     the cache of mla_decode (written), 16-byte aligned.
 *  block_table, seqlens, p   as for mla_decode; p->num_heads is not used.
 *               L_b are the lengths including the new tokens.
 *
 * Lengths outside [s_q, capacity] (device lengths are not checked on the
 * host when p->seqlens_host is NULL) are clamped to it; page ids are
 * clamped into the pool.
 */
int mla_append_kv(mla_ctx *ctx, const void *new_rows, void *kv_cache, const int32_t *block_table,
                  const int32_t *seqlens, const mla_problem *p);

/*
 * Absorbed query: for every row r (a query token of a sequence) and head h,
 *   q_out[r][h][c]       = bf16( sum_{d<d_nope} q_nope[r][h][d] * w_uk[h][c][d] ),  c < 512
 *   q_out[r][h][512 + j] = q_rope[r][h][j],                                            j < 64
 * i.e. the key up-projection of head h applied to its query, so that q.k
 * over the latent row equals the score against the up-projected key.
 * Accumulation in fp32, one rounding to bf16 (to nearest even).
 *
 *  q_nope  bf16 [rows][H][d_nope];  q_rope bf16 [rows][H][64]  (rotary
 *          embedding already applied);  w_uk bf16 [H][512][d_nope]: row c
 *          of head h holds the weights of latent channel c;  q_out bf16
 *          [rows][H][576], the query of mla_decode.  All 16-byte aligned.
 *  rows >= 1; heads >= 1; d_nope a positive multiple of 32.
 */
int mla_absorb_q(mla_ctx *ctx, const void *q_nope, const void *q_rope, const void *w_uk, void *q_out,
                 int32_t rows, int32_t heads, int32_t d_nope);

/*
 * Output up-projection: for every row r and head h,
 *   out[r][h][e] = sum_{c<512} o[r][h][c] * w_uv[h][e][c],   e < d_v
 * applied to the latent attention output o of mla_decode.  fp32 in, fp32
 * out; o enters the products split into a bf16 high and low part, so it
 * keeps about 16 significant bits.
 *
 *  o      fp32 [rows][H][512];  w_uv bf16 [H][d_v][512] (row e of head h
 *         holds the weights of value channel e);  out fp32 [rows][H][d_v].
 *         All 16-byte aligned.
 *  rows >= 1; heads >= 1; d_v a positive multiple of 16.
 */
int mla_project_out(mla_ctx *ctx, const float *o, const void *w_uv, float *out, int32_t rows, int32_t heads,
                    int32_t d_v);

/* Library version string, e.g. "mla_decode 0.1 gfx950". */
const char *mla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_DECODE_H */
