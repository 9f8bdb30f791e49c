/*
 * pa.h -- paged KV-cache attention on AMD MI355X (gfx950), C ABI.
 *
 * The operation
 * -------------
 * New query tokens attend to their own request's keys and values, which live
 * in a block-paged cache.  The inference-optimisation chapter ("Chapter 8:
 * Inference optimisation", section 8.3.1, Fig. 8-10) describes the layout
 * this follows: a sequence is cut into fixed-size logical blocks, each request
 * keeps a block table mapping logical block i to a physical block anywhere in
 * a shared pool, and attention recovers logical order through that table.
 * Several tables may reference the same physical block (shared prefixes,
 * section 8.3.2, Fig. 8-13).  Two workloads use it:
 *   - decode: one new token per request (same chapter, sections 8.1.1 and
 *     8.2.1), grouped-query heads, bound by HBM bandwidth;
 *   - chunked denoising: a chunk of latent tokens attends to the KV that
 *     earlier chunks left at the same noise level (PhysisServe teardown page,
 *     section "why autoregressive denoising can be pipelined", the update
 *     z_c^(d-1) = Phi_d(z_c^(d), K_<c^(d), cond_c)).
 *
 * For every slot r with n = ctx_lens[r] > 0 and m = q_lens[r] > 0, every new
 * row i < m (global row q_off[r] + i, q_off = exclusive running sum of q_lens)
 * and every query head h (KV head g = h / (num_q_heads / num_kv_heads)):
 *     K_r[j] = k_cache[block_table[r][j / 16]][g][j % 16][:]   (j < n)
 *     s_j    = scale * <q[row][h], K_r[j]>        over visible keys j
 *     out[row][h] = sum_j softmax(s)_j V_r[j]      (bf16, round to nearest even)
 *     lse[row][h] = ln sum_j exp(s_j)               (fp32, natural log)
 * Visible keys are all j < n (full mask), or j <= n - m + i with
 * PA_FLAG_CAUSAL.  n counts every key, including the new tokens' own K/V,
 * which the caller has already written into their pages.
 *
 * Finished ("zombie") slots ride along in an in-flight batch without a result
 * anyone reads (Photon pipelined-decoding page, section 5): a slot with
 * ctx_lens[r] == 0 or q_lens[r] == 0 writes nothing -- its out/lse bytes are
 * left exactly as they were.
 *
 * Data layout (all device memory, owned by the caller)
 *   q, out       bf16  [total_q][num_q_heads][head_dim], rows packed by slot
 *   k_cache,
 *   v_cache      bf16  [num_blocks][num_kv_heads][block_size][head_dim]
 *                      (one (block, KV head) tile = 16 x 128 x 2 B = 4 KiB)
 *   block_table  int32 [num_seqs][max_blocks_per_seq]
 *   ctx_lens,
 *   q_lens       int32 [num_seqs]
 *   lse          fp32  [total_q][num_q_heads]  (may be NULL)
 *
 * Conventions
 *   - Every device call only enqueues work on `stream` (a hipStream_t; NULL
 *     is the null stream) and returns; results are ordered on that stream.
 *     No device call allocates memory, synchronises, or reads device memory
 *     on the host, so calls may be captured in a HIP graph (cf. the Photon
 *     page, section 3: fixed buffers, no runtime allocation).
 *   - Apart from block pools (host objects the caller creates, owns and
 *     destroys; see pa_pool_create), the library keeps no state, and every
 *     device call is re-entrant.  The caller keeps every
 *     buffer alive and unmodified (and does not reuse `workspace`) until the
 *     stream has passed the call -- the "free only after the accelerator has
 *     stopped reading" rule of section 8.3.2.
 *   - Host-detectable errors return a status before anything is launched.
 *     Device-side contents (table entries < num_blocks, n <= 16 *
 *     max_blocks_per_seq, m <= n, n <= max_ctx_len, m <= max_q_len, the sum
 *     of q_lens <= total_q) are preconditions; pa_validate checks them on the
 *     device.  There is no retry and no fallback path.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL_ARG = 1,            /* a required pointer is NULL */
  PA_ERR_BAD_SHAPE = 2,           /* inconsistent or out-of-range sizes */
  PA_ERR_UNSUPPORTED = 3,         /* valid but not implemented (e.g. head_dim != 128) */
  PA_ERR_WORKSPACE_TOO_SMALL = 4, /* workspace_bytes < pa_workspace_size() */
  PA_ERR_LAUNCH = 5,              /* the HIP runtime rejected a kernel launch */
  PA_ERR_OUT_OF_BLOCKS = 6,       /* the block pool has too few free blocks; nothing changed */
  PA_ERR_SCRATCH_LIMIT = 7        /* pa_attend_noalloc: the call needs more scratch than
                                     PA_NOALLOC_SCRATCH_BYTES; nothing launched */
} pa_status;

/* Request rows may only see keys up to their own position (chunked prefill,
 * speculative verification).  Without it every row sees all n keys. */
#define PA_FLAG_CAUSAL 0x1u

/* Host-known sizes of one call.  The maxima are upper bounds the caller's
 * scheduler already knows; they size the launch grid without a device read. */
typedef struct pa_shape {
  int32_t num_seqs;           /* slots (rows of block_table, ctx_lens, q_lens) */
  int32_t total_q;            /* rows of q / out / lse */
  int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* Hkv */
  int32_t head_dim;           /* must be 128 */
  int32_t block_size;         /* tokens per block; must be 16 */
  int32_t max_blocks_per_seq; /* columns of block_table */
  int32_t max_q_len;          /* >= every q_lens[r]; 1 selects the decode path */
  int32_t max_ctx_len;        /* >= every ctx_lens[r] */
  int32_t partition_size;     /* split-KV partition in tokens: 0 = automatic,
                                 otherwise a positive multiple of block_size */
  int64_t num_blocks;         /* physical blocks in each of k_cache / v_cache */
  uint32_t flags;             /* PA_FLAG_* */
  uint32_t reserved;          /* must be 0 */
} pa_shape;

/* Bytes of scratch pa_attend (and pa_attend_kv, whatever the page format)
 * needs for this shape: one int32 counter per
 * (slot, KV head), then the split-KV partials (fp32 LSE and normalised fp32
 * output per partition and row).  0 when the call needs none.  Returns 0 for
 * a shape pa_attend would reject.
 * Why partials exist: a one-token decode step is too small to occupy the
 * whole GPU (OpScale page, section 2.1, Figure 7: one-token decode kernels
 * leave much of the SM allocation unused), so long contexts are cut into
 * partitions that run side by side and are merged by log-sum-exp.  The
 * caller allocates this buffer once and reuses it every step (Photon page,
 * section 3: working buffers are allocated once, at fixed addresses, so that
 * a step can be captured as a graph and replayed). */
size_t pa_workspace_size(const pa_shape* shape);

/* Prepare a workspace for this shape: zero its counter region (enqueued on
 * `stream` as a kernel, so it may be captured in a graph).  Required once
 * before a workspace is first used with a shape, and again before it is
 * reused with a different shape.  Every pa_attend call that completes leaves
 * the counters at zero again, so repeated calls (and graph replays) with the
 * same shape need no further initialisation.  Errors as for pa_attend. */
pa_status pa_workspace_init(const pa_shape* shape, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Number of split-KV partitions pa_attend will use for this shape (1 = no
 * split, or the path that does not split); 0 for an invalid shape. */
int32_t pa_num_partitions(const pa_shape* shape);

/* The same for pa_attend_kv with pages in `format` (a pa_kv_format): with
 * an automatic partition size, q8_0 / q4_0 pages are split into more
 * partitions than bf16 and FP8 ones; 0 for an invalid shape or format. */
int32_t pa_num_partitions_kv(const pa_shape* shape, int32_t format);

/* Attention of the new rows against the paged cache, as defined above.
 * `workspace` (initialised with pa_workspace_init for this shape) may be
 * NULL when pa_workspace_size() is 0.  One workspace must not be used by two
 * calls that can run at the same time.  `lse` may be NULL.
 * q and out must not overlap.  Errors: PA_ERR_NULL_ARG, PA_ERR_BAD_SHAPE,
 * PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE_TOO_SMALL (nothing launched), or
 * PA_ERR_LAUNCH. */
pa_status pa_attend(const pa_shape* shape, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_table,
                    const int32_t* ctx_lens, const int32_t* q_lens, float scale,
                    void* out, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Merge split-KV partials by their log-sum-exp weights.  No page states
 * this formula: it is the softmax of the definition above regrouped over
 * disjoint key sets (each partial o_p is the softmax-weighted mean over its
 * keys, lse_p the log of its sum of exponentials), so merging is exact up to
 * rounding.  Used for partitions of one request's keys and for a shared
 * prefix read once for several requests (chapter section 8.3.2).  For each
 * row:
 *   M = max_p lse_p,  w_p = exp(lse_p - M),
 *   lse = M + ln sum_p w_p,  out = sum_p w_p o_p / sum_p w_p  (bf16, RNE).
 * Partials with lse_p = -inf weigh zero and their outputs are never read; a
 * row whose partials are all -inf is left untouched (out and lse unchanged).
 *   partial_out  fp32 [num_partials][rows][head_dim] (each o_p normalised)
 *   partial_lse  fp32 [num_partials][rows]
 *   out          bf16 [rows][head_dim]
 *   lse          fp32 [rows] (may be NULL)
 * head_dim must be a positive multiple of 4, at most 1024.  Exported for
 * callers that produce partials themselves (context-parallel shards, or a
 * shared-prefix pass merged with per-request suffixes). */
pa_status pa_combine(int32_t num_partials, int32_t rows, int32_t head_dim,
                     const float* partial_out, const float* partial_lse,
                     void* out, float* lse, void* stream);

/* Copy every active slot's cached K (or V) rows into a dense buffer through
 * the same page addressing the attention kernels use -- the block-table
 * lookup of section 8.3.1, Fig. 8-10 (logical block j / 16 of a request maps
 * to whichever physical block its table names):
 *   dst[r][j][g][:] = cache[block_table[r][j / 16]][g][j % 16][:]  for j < n
 * dst is bf16 [num_seqs][max_ctx_len][num_kv_heads][head_dim]; rows j >= n
 * (and all rows of slots with n == 0) are left untouched.  For checking the
 * gather bit for bit. */
pa_status pa_gather_kv(const pa_shape* shape, const void* cache,
                       const int32_t* block_table, const int32_t* ctx_lens,
                       void* dst, void* stream);

/* Check the device-side preconditions of pa_attend for this shape and data,
 * so that a caller can reject a bad batch before submitting it (the PhyAI
 * parallel-serving page, failure handling: requests are checked before
 * submission, and failures are fail-fast with no retry).  Writes a bit mask
 * to *error_word (device int32, caller-owned): 0 if all hold, else PA_BAD_*
 * bits below.  `workspace` may be NULL; if given (with its size), the
 * split-KV counters pa_attend would use for this shape are also checked to
 * be zero -- a workspace that was not initialised for this shape, or whose
 * last call did not run to completion, would corrupt the merge silently.
 * Enqueued on `stream`; read the word after the stream passes.  Errors:
 * PA_ERR_NULL_ARG, PA_ERR_BAD_SHAPE / PA_ERR_UNSUPPORTED (as pa_attend),
 * PA_ERR_WORKSPACE_TOO_SMALL (a workspace smaller than its counter region),
 * PA_ERR_LAUNCH. */
#define PA_BAD_BLOCK_ID 0x1   /* a table entry in [0, ceil(n/16)) outside [0, num_blocks) */
#define PA_BAD_CTX_LEN 0x2    /* n < 0, n > max_ctx_len or n > 16 * max_blocks_per_seq */
#define PA_BAD_Q_LEN 0x4      /* m < 0, m > max_q_len, or m > n while n > 0 */
#define PA_BAD_TOTAL_Q 0x8    /* sum of q_lens exceeds total_q */
#define PA_BAD_WORKSPACE 0x10 /* a split-KV counter of this shape is not zero */
pa_status pa_validate(const pa_shape* shape, const int32_t* block_table,
                      const int32_t* ctx_lens, const int32_t* q_lens,
                      const void* workspace, size_t workspace_bytes,
                      int32_t* error_word, void* stream);

/* ------------------------------------------------------------------------
 * Prefix-grouped (cascade) decode
 * ------------------------------------------------------------------------
 * Requests that share a prefix reference the same physical blocks
 * (section 8.3.2, Figs. 8-13 / 8-14: one copy of the common context serves
 * several requests).  pa_attend_prefix computes exactly what pa_attend
 * computes, but reads each group's shared pages once per KV head for all of
 * the group's query rows -- (member, query head) pairs -- on the matrix
 * cores, attends each member to its own remaining keys, and merges both by
 * log-sum-exp.  Where the members' own keys are split (and 1, 2 or 4 query
 * heads share a KV head) both parts run in one launch; otherwise a prefix
 * pass runs first.
 *
 * Groups are runs of consecutive slots [group_start[k], group_start[k+1]).
 * Group k's prefix is its first L = prefix_len[k] keys, read as the
 * floor(L/16) whole pages they cover (the rest are ordinary keys).
 * Preconditions: for every member r, block_table[r][0 .. L/16) equals row
 * group_start[k]'s first L/16 entries, and ctx_lens[r] >= L for members with
 * new tokens.  Slots outside every group, and slots past a group's first
 * max_members, have no prefix (their keys are all read by the decode pass;
 * the result is the same).  Decode only (max_q_len == 1, 1, 2, 4 or 8
 * query heads per KV head): other shapes return PA_ERR_UNSUPPORTED. */
typedef struct pa_prefix_groups {
  int32_t num_groups;
  int32_t max_members;         /* prefix rows per group: a group's first max_members slots */
  int32_t max_prefix_len;      /* >= every prefix_len; a multiple of 16, <= max_ctx_len */
  int32_t min_prefix_len;      /* <= the prefix of every slot with new tokens (0 if some have
                                  none); a multiple of 16.  Sizes the suffix split only. */
  int32_t reserved;            /* must be 0 */
  int32_t reserved2;
  const int32_t* group_start;  /* device int32 [num_groups + 1], ascending */
  const int32_t* prefix_len;   /* device int32 [num_groups] */
} pa_prefix_groups;

/* Workspace bytes for pa_attend_prefix (never 0 for a valid shape); 0 for an
 * invalid shape or group description. */
size_t pa_prefix_workspace_size(const pa_shape* shape, const pa_prefix_groups* groups);

/* Prepare a workspace for pa_attend_prefix with this shape and group sizes
 * (zeroes its counters); as pa_workspace_init. */
pa_status pa_prefix_workspace_init(const pa_shape* shape, const pa_prefix_groups* groups,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Attention as pa_attend (same arguments and results), reading shared
 * prefixes once per group.  Errors as for pa_attend, plus PA_ERR_BAD_SHAPE
 * for an inconsistent group description. */
pa_status pa_attend_prefix(const pa_shape* shape, const pa_prefix_groups* groups, const void* q,
                           const void* k_cache, const void* v_cache, const int32_t* block_table,
                           const int32_t* ctx_lens, const int32_t* q_lens, float scale, void* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Quantised KV pages
 * ------------------------------------------------------------------------
 * The chapter's section 8.4.2 ("KV compression and read cost", Fig. 8-23)
 * stores KV in groups of 32 values with one 2-byte scale each: q8_0 keeps
 * one-byte codes (34 bytes per group where bf16 needs 64), q4_0 4-bit codes
 * (18 bytes).  Section 8.4.4 studies an FP8 cache and keeps the query in
 * bf16, as everything here does.  Reading fewer bytes pays when the
 * conversion costs less than the bytes saved: Delta T = Delta D / beta - T_c.
 *
 * Layouts (per layer, K and V alike; a group is 32 consecutive dims of one
 * token row of one KV head):
 *   PA_KV_BF16      codes = the bf16 cache of pa_attend
 *   PA_KV_FP8_E4M3  codes uint8 [num_blocks][Hkv][16][128], OCP E4M3 (bias 7,
 *                   no infinities, max 448); value = decode(code) * scale,
 *                   one fp32 scale per cache
 *   PA_KV_Q8_0      codes int8  [num_blocks][Hkv][16][128]; scales fp16
 *                   [num_blocks][Hkv][16][4]; value = code * scale
 *   PA_KV_Q4_0      codes uint8 [num_blocks][Hkv][16][64], byte b holding dim
 *                   2b in its low and 2b+1 in its high nibble; scales fp16
 *                   [num_blocks][Hkv][16][4]; value = (nibble - 8) * scale
 * Encoding (pa_write_kv_cache): q8_0 scale = max|x| / 127 and q4_0 scale =
 * (the group's value of largest magnitude) / -8, both rounded to fp16 (a
 * zero scale stored as +0); code
 * = x / stored scale in fp32, rounded half away from zero, clamped to the
 * code range; FP8 code = nearest E4M3 of x / scale (ties to even, saturating
 * at +-448). */
typedef enum pa_kv_format {
  PA_KV_BF16 = 0,
  PA_KV_FP8_E4M3 = 1,
  PA_KV_Q8_0 = 2,
  PA_KV_Q4_0 = 3
} pa_kv_format;

typedef struct pa_kv_cache {
  int32_t format;   /* pa_kv_format */
  int32_t reserved; /* must be 0 */
  void* k_codes;    /* layouts above (device memory) */
  void* v_codes;
  void* k_scales;   /* q8_0, q4_0: fp16 group scales; otherwise unused */
  void* v_scales;
  float k_scale;    /* FP8: per-cache scales; otherwise unused */
  float v_scale;
} pa_kv_cache;

/* pa_attend over a cache in any of the formats: the same definition, with
 * K and V the decoded values above.  PA_KV_BF16 is pa_attend itself.  The
 * quantised formats take the decode path only (max_q_len == 1 and a query
 * group of 1, 2 or 4 heads); other shapes return PA_ERR_UNSUPPORTED.  The
 * workspace is pa_workspace_size(shape), initialised with pa_workspace_init,
 * as for pa_attend (pa_num_partitions_kv gives the partition count).  Errors as for
 * pa_attend, plus PA_ERR_BAD_SHAPE for an unknown format, a non-finite or
 * non-positive FP8 scale, or reserved != 0. */
pa_status pa_attend_kv(const pa_shape* shape, const pa_kv_cache* cache, const void* q,
                       const int32_t* block_table, const int32_t* ctx_lens,
                       const int32_t* q_lens, float scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/* pa_write_kv into a cache in any of the formats: each new bf16 row is
 * encoded (per the rules above) into the codes and scales at its position.
 * PA_KV_BF16 is pa_write_kv itself.  Skips as pa_write_kv does. */
pa_status pa_write_kv_cache(const pa_shape* shape, const pa_kv_cache* cache, const void* k_new,
                            const void* v_new, const int32_t* block_table,
                            const int32_t* ctx_lens, const int32_t* q_lens, void* stream);

/* ------------------------------------------------------------------------
 * Appending new K/V, and the block pool that hands out pages
 * ------------------------------------------------------------------------
 * The chapter's sections 8.3.1 (Fig. 8-10) and 8.3.2 (Figs. 8-13 to 8-15)
 * describe the life of a page: a growing sequence takes a block from the
 * free pool when it needs a new one and records it in its block table;
 * tables may share blocks (a common prefix), each table entry being one
 * reference; a branch that writes into a shared block that is only partly
 * filled first takes a private copy of it; and a block goes back to the free
 * pool only when its last reference is dropped and the accelerator no longer
 * reads it (Fig. 8-14, and Fig. 8-16 for cancellation).
 */

/* Write the new tokens' K and V rows into their pages, the step that must
 * precede pa_attend with the same arguments.  For every slot r with
 * n = ctx_lens[r] > 0 and m = q_lens[r] > 0, new row i < m (global row
 * q_off[r] + i, as for pa_attend) is position j = n - m + i:
 *     k_cache[block_table[r][j / 16]][g][j % 16][:] = k_new[row][g][:]
 * and likewise V, for every KV head g.
 *   k_new, v_new  bf16 [total_q][num_kv_heads][head_dim]
 *   k_cache, v_cache as for pa_attend (written in place)
 * Uses num_seqs, total_q, num_kv_heads, head_dim, block_size,
 * max_blocks_per_seq, max_q_len and num_blocks of `shape` (num_q_heads only
 * has to be a valid multiple).  A position outside the block table or a
 * table entry outside [0, num_blocks) is skipped rather than written.  Only
 * enqueues work on `stream`.  Errors: PA_ERR_NULL_ARG, PA_ERR_BAD_SHAPE,
 * PA_ERR_UNSUPPORTED, PA_ERR_LAUNCH. */
pa_status pa_write_kv(const pa_shape* shape, const void* k_new, const void* v_new,
                      const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens,
                      void* k_cache, void* v_cache, void* stream);

/* Copy whole blocks (every KV head, K and V) src[i] -> dst[i] for
 * i < num_copies: the copy half of copy-on-write (section 8.3.2, Fig. 8-15).
 * src, dst: device int32 [num_copies]; no dst may equal any src or another
 * dst.  Entries outside [0, num_blocks) are skipped.  Caches as for
 * pa_attend, head_dim 128 and block_size 16. */
pa_status pa_copy_blocks(int32_t num_copies, const int32_t* src, const int32_t* dst,
                         int32_t num_kv_heads, int64_t num_blocks, void* k_cache, void* v_cache,
                         void* stream);

/* Host-side block pool: free pool, per-slot block tables, reference counts,
 * copy-on-write and fenced release.  Plain host memory, no device calls; not
 * thread-safe (the caller's scheduler owns it).  Blocks are handed out from
 * a free stack; which id a request gets is unspecified. */
typedef struct pa_pool pa_pool;

typedef struct pa_pool_stats {
  int32_t free_blocks;    /* ready to hand out */
  int32_t pending_blocks; /* released, waiting for their fence to retire */
  int32_t used_blocks;    /* referenced by at least one slot */
  int32_t reserved;
  int64_t references;     /* block-table entries over all slots */
} pa_pool_stats;

/* A pool of num_blocks blocks of block_size tokens (any positive size; the
 * attention kernels use 16) serving num_slots slots of at most
 * max_blocks_per_seq blocks each.  Errors: PA_ERR_NULL_ARG, PA_ERR_BAD_SHAPE. */
pa_status pa_pool_create(int32_t num_blocks, int32_t block_size, int32_t num_slots,
                         int32_t max_blocks_per_seq, pa_pool** pool);
void pa_pool_destroy(pa_pool* pool);

/* Make room for num_tokens more tokens in `slot` (section 8.3.1): new blocks
 * come from the free pool.  If the slot's last block is partly filled and
 * shared with another slot, the slot first gets a private copy of it
 * (section 8.3.2): *num_copies is then 1 and (copy_src[0], copy_dst[0])
 * names the copy the caller must make with pa_copy_blocks, on every layer's
 * caches, before writing into it; otherwise *num_copies is 0.  Returns
 * PA_ERR_OUT_OF_BLOCKS, changing nothing, when the free pool is too small,
 * and PA_ERR_BAD_SHAPE for a bad slot, a negative count or a sequence longer
 * than max_blocks_per_seq blocks. */
pa_status pa_pool_append(pa_pool* pool, int32_t slot, int32_t num_tokens, int32_t* copy_src,
                         int32_t* copy_dst, int32_t* num_copies);

/* Let the empty slot dst share the first num_tokens tokens of src (all of
 * them if num_tokens < 0): dst's table references src's first
 * ceil(num_tokens / block_size) blocks (section 8.3.2, Fig. 8-13).
 * PA_ERR_BAD_SHAPE if dst holds tokens, a slot is out of range or
 * num_tokens exceeds src's length. */
pa_status pa_pool_fork(pa_pool* pool, int32_t src, int32_t dst, int32_t num_tokens);

/* Drop every reference `slot` holds and empty it.  A block whose count
 * reaches zero becomes free once a fence >= `fence` is retired: the caller
 * names the work that may still read it (e.g. the number of the step whose
 * launches used it) and retires it when that work has finished (Fig. 8-14). */
pa_status pa_pool_release(pa_pool* pool, int32_t slot, uint64_t fence);

/* All work up to and including `fence` has finished: blocks released under
 * such fences return to the free pool. */
pa_status pa_pool_retire(pa_pool* pool, uint64_t fence);

/* Tokens held by `slot` (-1 for a bad slot or pool). */
int32_t pa_pool_length(const pa_pool* pool, int32_t slot);

/* The pool's block tables, host int32 [num_slots][max_blocks_per_seq], valid
 * until the pool is destroyed; entries past a slot's last block are 0.
 * Upload them (or the rows in use) for pa_write_kv / pa_attend. */
const int32_t* pa_pool_block_table(const pa_pool* pool);

/* References to `block` (-1 for a bad block or pool). */
int32_t pa_pool_refcount(const pa_pool* pool, int32_t block);

pa_status pa_pool_get_stats(const pa_pool* pool, pa_pool_stats* stats);

/* Static, NUL-terminated description of a status code. */
const char* pa_status_string(pa_status status);

/* ------------------------------------------------------------------------
 * pa_attend without a caller workspace
 * ------------------------------------------------------------------------
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, result, errors and kernels as pa_attend, minus
 * the workspace: the split-KV counters and partials live in a buffer built
 * into the library, PA_NOALLOC_SCRATCH_BYTES of device memory on every GPU
 * the library runs on, held until the process ends.  A call whose shape
 * needs more (pa_workspace_size(shape) > PA_NOALLOC_SCRATCH_BYTES) returns
 * PA_ERR_SCRATCH_LIMIT and launches nothing.  Nothing here allocates: the
 * first call on a device looks up that device's copy of the buffer and
 * enqueues a kernel that zeroes its counters; every later call finds them
 * zero again, since each completed call leaves them so.
 * The device is the current one (hipGetDevice), and `stream` must belong to
 * it.  All calls on one GPU share the buffer: two calls that can run at the
 * same time on one GPU (different streams, overlapping graph launches) race
 * on it and give wrong results; order them on one stream.  Errors as for
 * pa_attend, plus PA_ERR_SCRATCH_LIMIT, and PA_ERR_LAUNCH when the buffer's
 * address cannot be obtained. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pa_status pa_attend_noalloc(const pa_shape* shape, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_table,
                            const int32_t* ctx_lens, const int32_t* q_lens, float scale,
                            void* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
