// api.cpp -- the C ABI of libpa.so: argument checks, launch planning, launches.
//
// Host-side only.  Nothing here reads device memory, allocates, or waits on
// the stream, so every entry point can be captured in a HIP graph (fixed
// buffers and no runtime allocation, as the Photon pipelined-decoding page
// requires of its decode slots, section 3).  Errors that the host can detect
// are returned before anything is launched; there is no fallback path.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <climits>
#include <cmath>

#include "launch.h"
#include "pa.h"

namespace {

using namespace pa;

constexpr float kLog2e = 1.4426950408889634f;

struct Plan {
  bool empty = true;      // nothing to launch
  bool decode = false;    // split-KV decode path, else chunk path
  int group = 1;          // query heads per KV head
  int tokens = 1;         // decode: new tokens per slot the kernel is built for
  int part_pages = 0;     // pages per partition (decode)
  int num_parts = 1;      // partitions (decode)
  size_t rows = 0;        // total_q * num_q_heads
  size_t ws_bytes = 0;    // workspace bytes
  // Workspace layout (split decode): counters | partial LSE | partial out.
  size_t counters_bytes = 0;
  size_t lse_offset = 0;
  size_t out_offset = 0;
  unsigned grid = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

pa_status check_shape(const pa_shape* s) {
  if (!s) return PA_ERR_NULL_ARG;
  if (s->reserved != 0) return PA_ERR_BAD_SHAPE;
  if (s->num_seqs < 0 || s->total_q < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 ||
      s->head_dim <= 0 || s->block_size <= 0 || s->max_blocks_per_seq <= 0 ||
      s->max_q_len < 0 || s->max_ctx_len < 0 || s->partition_size < 0 || s->num_blocks < 0)
    return PA_ERR_BAD_SHAPE;
  if (s->num_q_heads % s->num_kv_heads != 0) return PA_ERR_BAD_SHAPE;
  if (s->head_dim != kHeadDim || s->block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
  if (s->partition_size % kBlockSize != 0) return PA_ERR_BAD_SHAPE;
  if ((long long)s->max_ctx_len > (long long)kBlockSize * s->max_blocks_per_seq) return PA_ERR_BAD_SHAPE;
  if (s->max_q_len > s->total_q && s->num_seqs > 0) return PA_ERR_BAD_SHAPE;
  if (s->num_blocks == 0 && s->max_ctx_len > 0) return PA_ERR_BAD_SHAPE;
  if (s->flags & ~PA_FLAG_CAUSAL) return PA_ERR_UNSUPPORTED;
  // Index arithmetic limits: rows and grid sizes must fit 32-bit counters.
  const long long rows = (long long)s->total_q * s->num_q_heads;
  if (rows > INT_MAX / 2) return PA_ERR_UNSUPPORTED;
  if ((long long)s->num_seqs * s->max_blocks_per_seq > (long long)INT_MAX) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

pa_status check_kv_cache(const pa_kv_cache& c) {
  if (c.reserved != 0) return PA_ERR_BAD_SHAPE;
  if (c.format < kFmtBF16 || c.format > kFmtQ4) return PA_ERR_BAD_SHAPE;
  if (c.format == kFmtFP8 && !(std::isfinite(c.k_scale) && std::isfinite(c.v_scale) &&
                               c.k_scale > 0.f && c.v_scale > 0.f))
    return PA_ERR_BAD_SHAPE;
  return PA_OK;
}

// Partition size when the caller leaves it to the library.  A decode
// workgroup (four waves, three pages in flight each) streams at close to its
// CU's share of HBM bandwidth, so what matters is how evenly the grid fills
// the CUs and how much fixed cost (start, merge) each partition carries:
//  - with at most two resident workgroups per CU for the whole grid, pick
//    the partition count whose grid fills its last round of CUs best, then
//    (bf16 and FP8 pages) the fewest partitions -- the least start and merge
//    per page -- or (q8_0 / q4_0 pages) the most;
//  - with more (slot, KV head) pairs than that, the grid is several rounds
//    anyway; long contexts are cut into partitions of at most 128 pages so
//    that a batch's longest requests do not finish last on their own.
// No partition is smaller than 8 pages (two per wave).
int auto_part_pages(const pa_shape* s, int max_pages, bool grouped) {
  constexpr int kMinPages = 8, kLongPages = 128;
  const long long pairs = (long long)s->num_seqs * s->num_kv_heads;
  const long long resident = (long long)kDecodeWGsPerCU * kNumCUs;
  if (pairs <= 0 || max_pages <= kMinPages) return kMinPages;
  if (pairs > resident) return std::max(kMinPages, ceil_div(max_pages, ceil_div(max_pages, kLongPages)));
  int best_pp = max_pages;
  double best_fill = -1.0;
  for (long long parts = 1; parts * pairs <= resident && parts <= max_pages; ++parts) {
    const int pp = ceil_div(max_pages, (int)parts);
    if (pp < kMinPages) break;
    if (ceil_div(max_pages, pp) != parts) continue;  // same grid as a smaller count
    const double rounds = (double)(pairs * parts) / kNumCUs;
    const double fill = rounds / std::ceil(rounds);
    // Ties in fill (within 1 %): bf16 and FP8 pages keep the fewer, longer
    // partitions (measured on the shared-prefix batch, 10 x 8447 keys: 3
    // partitions 34.7 us, 6 37.0 us per layer; FP8 on the Qwen3-8B-shaped
    // batch: 2 partitions 7 % faster than 4); q8_0 / q4_0 pages carry fewer
    // bytes for more per-page work (codes and group scales converted in
    // registers), so there more, smaller partitions -- more resident waves
    // per CU -- win (2 -> 4 partitions, 10-15 % faster).
    const bool better = fill > best_fill + 0.01 || (grouped && fill > best_fill - 0.01);
    if (better) {
      best_fill = std::max(best_fill, fill);  // (std::: HIP's unqualified max is the int one)
      best_pp = pp;
    }
  }
  return best_pp;
}

pa_status make_plan(const pa_shape* s, Plan* plan, bool grouped = false) {
  const pa_status st = check_shape(s);
  if (st != PA_OK) return st;
  Plan p;
  p.group = s->num_q_heads / s->num_kv_heads;
  p.rows = (size_t)s->total_q * (size_t)s->num_q_heads;
  if (s->num_seqs == 0 || s->total_q == 0 || s->max_q_len == 0 || s->max_ctx_len == 0) {
    *plan = p;  // nothing can be written
    return PA_OK;
  }
  p.empty = false;
  // Up to 8 new tokens per slot (tokens x group <= 32) stream the pages like
  // a one-token decode, the (token, query head) pairs as matrix columns;
  // longer chunks take the chunk path.
  p.tokens = decode_tokens_per_slot(p.group, s->max_q_len);
  p.decode = p.tokens > 0 && (p.tokens == 1 || !grouped);
  if (p.decode) {
    const int max_pages = ceil_div(s->max_ctx_len, kBlockSize);
    p.part_pages = s->partition_size > 0 ? s->partition_size / kBlockSize : auto_part_pages(s, max_pages, grouped);
    p.num_parts = ceil_div(max_pages, p.part_pages);
    const long long grid = (long long)s->num_kv_heads * s->num_seqs * p.num_parts;
    if (grid > INT_MAX) return PA_ERR_UNSUPPORTED;
    p.grid = (unsigned)grid;
    if (p.num_parts > 1) {
      p.counters_bytes = align256((size_t)s->num_seqs * s->num_kv_heads * sizeof(int32_t));
      p.lse_offset = p.counters_bytes;
      p.out_offset = p.lse_offset + align256((size_t)p.num_parts * p.rows * sizeof(float));
      p.ws_bytes = p.out_offset + (size_t)p.num_parts * p.rows * kHeadDim * sizeof(float);
    }
  } else {
    // One workgroup per 128 packed (token, query head of the group) rows of
    // a (slot, KV head).
    const int q_tiles = ceil_div(s->max_q_len * p.group, kChunkRows);
    const long long grid = (long long)s->num_seqs * s->num_kv_heads * q_tiles;
    if (grid > INT_MAX) return PA_ERR_UNSUPPORTED;
    p.grid = (unsigned)grid;
  }
  *plan = p;
  return PA_OK;
}

}  // namespace

#ifndef PA_PREFIX_ONE_LAUNCH
#define PA_PREFIX_ONE_LAUNCH 1
#endif
#ifndef PA_PREFIX_ITEM_PAGES
#define PA_PREFIX_ITEM_PAGES 0  // pages per prefix item (0: the prefix pass's partitions)
#endif

namespace {

// Kernel arguments of the decode path for a plan; `ws` holds the split-KV
// region at offset 0.
DecodeParams decode_params(const pa_shape* shape, const Plan& plan, const pa_kv_cache& kv,
                           const void* q, const int32_t* block_table, const int32_t* ctx_lens,
                           const int32_t* q_lens, float scale_log2, void* out, float* lse, char* ws) {
  DecodeParams d = {};
  d.q = static_cast<const uint16_t*>(q);
  d.k = static_cast<const uint16_t*>(kv.k_codes);
  d.v = static_cast<const uint16_t*>(kv.v_codes);
  d.block_table = block_table;
  d.ctx_lens = ctx_lens;
  d.q_lens = q_lens;
  d.out = static_cast<uint16_t*>(out);
  d.lse = lse;
  const bool split = plan.num_parts > 1;
  d.counters = split ? reinterpret_cast<int32_t*>(ws) : nullptr;
  d.part_lse = split ? reinterpret_cast<float*>(ws + plan.lse_offset) : nullptr;
  d.part_out = split ? reinterpret_cast<float*>(ws + plan.out_offset) : nullptr;
  d.scale_log2 = scale_log2;
  d.num_seqs = shape->num_seqs;
  d.num_q_heads = shape->num_q_heads;
  d.num_kv_heads = shape->num_kv_heads;
  d.max_blocks = shape->max_blocks_per_seq;
  d.total_q = shape->total_q;
  d.part_pages = plan.part_pages;
  d.num_parts = plan.num_parts;
  d.k_scales = static_cast<const uint16_t*>(kv.k_scales);
  d.v_scales = static_cast<const uint16_t*>(kv.v_scales);
  d.v_scale = kv.format == kFmtFP8 ? kv.v_scale : 1.f;
  d.causal = (shape->flags & PA_FLAG_CAUSAL) ? 1 : 0;
  return d;
}

// The attention call for any page format.  `kv` carries the codes (and
// scales); bf16 caches take either path, quantised ones the decode path.
pa_status attend_impl(const pa_shape* shape, const pa_kv_cache& kv, const void* q,
                      const int32_t* block_table, const int32_t* ctx_lens,
                      const int32_t* q_lens, float scale, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  const void* k_cache = kv.k_codes;
  const void* v_cache = kv.v_codes;
  const bool grouped = kv.format == kFmtQ8 || kv.format == kFmtQ4;
  Plan plan;
  const pa_status st = make_plan(shape, &plan, grouped);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale)) return PA_ERR_BAD_SHAPE;
  if (plan.empty) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !q_lens || !out)
    return PA_ERR_NULL_ARG;
  if (grouped && (!kv.k_scales || !kv.v_scales)) return PA_ERR_NULL_ARG;
  if (kv.format != kFmtBF16 && (!plan.decode || plan.tokens > 1)) return PA_ERR_UNSUPPORTED;
  if (plan.ws_bytes > 0) {
    if (!workspace) return PA_ERR_NULL_ARG;
    if (workspace_bytes < plan.ws_bytes) return PA_ERR_WORKSPACE_TOO_SMALL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // FP8: the K scale multiplies every score, so it joins the softmax scale.
  const float scale_log2 = scale * (kv.format == kFmtFP8 ? kv.k_scale : 1.f) * kLog2e;

  if (plan.decode) {
    const DecodeParams d = decode_params(shape, plan, kv, q, block_table, ctx_lens, q_lens, scale_log2,
                                         out, lse, static_cast<char*>(workspace));
    if (launch_decode(d, plan.group, kv.format, plan.tokens, plan.grid, s) != hipSuccess) return PA_ERR_LAUNCH;
    return PA_OK;
  }

  ChunkParams c = {};
  c.q = static_cast<const uint16_t*>(q);
  c.k = static_cast<const uint16_t*>(k_cache);
  c.v = static_cast<const uint16_t*>(v_cache);
  c.block_table = block_table;
  c.ctx_lens = ctx_lens;
  c.q_lens = q_lens;
  c.out = static_cast<uint16_t*>(out);
  c.lse = lse;
  c.scale_log2 = scale_log2;
  c.num_seqs = shape->num_seqs;
  c.num_q_heads = shape->num_q_heads;
  c.num_kv_heads = shape->num_kv_heads;
  c.max_blocks = shape->max_blocks_per_seq;
  c.q_tiles = ceil_div(shape->max_q_len * plan.group, kChunkRows);
  c.causal = (shape->flags & PA_FLAG_CAUSAL) ? 1 : 0;
  c.max_ctx = shape->max_ctx_len;
  c.max_q = shape->max_q_len;
  if (launch_chunk(c, plan.grid, s) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}


// Prefix-grouped decode: the suffix pass is the decode path with keys
// starting after each slot's prefix (sized for the longest possible suffix,
// max_ctx_len - min_prefix_len).  The prefix pass splits the longest prefix
// into partitions of at most kPrefixMaxTiles 32-key tiles (a workgroup holds
// its whole partition in LDS); when that leaves fewer workgroups than CUs it
// takes more partitions per (group, KV head, row tile), up to
// kPrefixFillParts (few enough that the suffix pass merges a row's partials
// in one batch), never less than one 32-key tile each.
// Workspace: [suffix split-KV region][slot prefix lengths]
// [prefix partial LSE][prefix partial out].
#ifndef PA_PREFIX_FILL_PARTS
#define PA_PREFIX_FILL_PARTS 24
#endif
constexpr int kPrefixFillParts = PA_PREFIX_FILL_PARTS;

struct PrefixPlan {
  Plan suffix;
  int row_tiles = 0;
  int pre_parts = 1;
  int pre_pages = 1;
  int suffix_pages = 0;  // pages of the longest suffix (the slots' own keys)
  unsigned pre_grid = 0;
  size_t plen_offset = 0, pre_lse_offset = 0, pre_out_offset = 0, ws_bytes = 0;
};

pa_status make_prefix_plan(const pa_shape* s, const pa_prefix_groups* gr, PrefixPlan* out) {
  pa_status st = check_shape(s);
  if (st != PA_OK) return st;
  if (!gr) return PA_ERR_NULL_ARG;
  if (gr->num_groups < 0 || gr->max_members < 0 || gr->max_prefix_len < 0 || gr->min_prefix_len < 0 ||
      gr->reserved != 0)
    return PA_ERR_BAD_SHAPE;
  if (gr->max_prefix_len % kBlockSize || gr->min_prefix_len % kBlockSize) return PA_ERR_BAD_SHAPE;
  if (gr->min_prefix_len > gr->max_prefix_len || gr->max_prefix_len > s->max_ctx_len) return PA_ERR_BAD_SHAPE;
  if (gr->max_members > s->num_seqs || gr->num_groups > s->num_seqs) return PA_ERR_BAD_SHAPE;
  const int G = s->num_q_heads / s->num_kv_heads;
  if (s->max_q_len > 1 || !decode_supports_group(G)) return PA_ERR_UNSUPPORTED;
  PrefixPlan pp;
  pa_shape suf = *s;
  suf.max_ctx_len = s->max_ctx_len - gr->min_prefix_len;
  if (suf.max_ctx_len < kBlockSize) suf.max_ctx_len = kBlockSize;
  st = make_plan(&suf, &pp.suffix);
  if (st != PA_OK) return st;
  pp.suffix_pages = ceil_div(suf.max_ctx_len, kBlockSize);
  const size_t rows = (size_t)s->total_q * s->num_q_heads;
  pp.row_tiles = ceil_div(gr->max_members * G, 64);
  const int max_pages = gr->max_prefix_len / kBlockSize;
  const long long base = (long long)gr->num_groups * s->num_kv_heads * pp.row_tiles;
  if (base > 0 && max_pages > 0) {
    long long parts = (long long)kNumCUs / base;
    parts = parts < 1 ? 1 : (parts > kPrefixFillParts ? kPrefixFillParts : parts);
    const long long need = ceil_div(max_pages, 2 * kPrefixMaxTiles);
    if (parts < need) parts = need;
    if (parts > ceil_div(max_pages, 2)) parts = ceil_div(max_pages, 2);
    pp.pre_pages = ceil_div(max_pages, (int)parts);
    pp.pre_parts = ceil_div(max_pages, pp.pre_pages);
    const long long grid = base * pp.pre_parts;
    if (grid + 1 > INT_MAX) return PA_ERR_UNSUPPORTED;
    pp.pre_grid = (unsigned)grid;
  }
  pp.plen_offset = align256(pp.suffix.ws_bytes);
  pp.pre_lse_offset = pp.plen_offset + align256((size_t)s->num_seqs * sizeof(int32_t));
  pp.pre_out_offset = pp.pre_lse_offset + align256((size_t)pp.pre_parts * rows * sizeof(float));
  pp.ws_bytes = pp.pre_out_offset + (size_t)pp.pre_parts * rows * kHeadDim * sizeof(float);
  *out = pp;
  return PA_OK;
}

}  // namespace

namespace pa {

// pa_attend with the workspace given by the caller of this function (the
// library's own scratch buffer, for pa_attend_noalloc).
pa_status attend_bf16(const pa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens,
                      float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream) {
  pa_kv_cache kv = {};
  kv.format = kFmtBF16;
  kv.k_codes = const_cast<void*>(k_cache);
  kv.v_codes = const_cast<void*>(v_cache);
  return attend_impl(shape, kv, q, block_table, ctx_lens, q_lens, scale, out, lse, workspace,
                     workspace_bytes, stream);
}

}  // namespace pa

extern "C" {

size_t pa_workspace_size(const pa_shape* shape) {
  Plan p, c;
  if (make_plan(shape, &p) != PA_OK || make_plan(shape, &c, true) != PA_OK) return 0;
  return p.ws_bytes > c.ws_bytes ? p.ws_bytes : c.ws_bytes;  // enough for every page format
}

int32_t pa_num_partitions(const pa_shape* shape) {
  Plan p;
  if (make_plan(shape, &p) != PA_OK) return 0;
  return p.decode ? p.num_parts : 1;
}

int32_t pa_num_partitions_kv(const pa_shape* shape, int32_t format) {
  if (format < kFmtBF16 || format > kFmtQ4) return 0;
  Plan p;
  if (make_plan(shape, &p, format == kFmtQ8 || format == kFmtQ4) != PA_OK) return 0;
  return p.decode ? p.num_parts : 1;
}

pa_status pa_attend(const pa_shape* shape, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_table,
                    const int32_t* ctx_lens, const int32_t* q_lens, float scale,
                    void* out, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream) {
  pa_kv_cache kv = {};
  kv.format = kFmtBF16;
  kv.k_codes = const_cast<void*>(k_cache);
  kv.v_codes = const_cast<void*>(v_cache);
  return attend_impl(shape, kv, q, block_table, ctx_lens, q_lens, scale, out, lse, workspace,
                     workspace_bytes, stream);
}

pa_status pa_workspace_init(const pa_shape* shape, void* workspace, size_t workspace_bytes,
                            void* stream) {
  // The counters sit at the start of the workspace whatever the page format
  // (only the partition count, and so the partials' extent, differs).
  Plan plan, comp;
  pa_status st = make_plan(shape, &plan);
  if (st != PA_OK) return st;
  st = make_plan(shape, &comp, true);
  if (st != PA_OK) return st;
  const size_t need = plan.ws_bytes > comp.ws_bytes ? plan.ws_bytes : comp.ws_bytes;
  const size_t counters = plan.counters_bytes > comp.counters_bytes ? plan.counters_bytes : comp.counters_bytes;
  if (need == 0) return PA_OK;
  if (!workspace) return PA_ERR_NULL_ARG;
  if (workspace_bytes < need) return PA_ERR_WORKSPACE_TOO_SMALL;
  if (launch_zero_i32(static_cast<int32_t*>(workspace), counters / sizeof(int32_t),
                      static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_combine(int32_t num_partials, int32_t rows, int32_t head_dim,
                     const float* partial_out, const float* partial_lse, void* out,
                     float* lse, void* stream) {
  if (num_partials <= 0 || rows < 0 || head_dim <= 0 || head_dim % 4 != 0 || head_dim > 1024)
    return PA_ERR_BAD_SHAPE;
  if ((long long)rows * head_dim * num_partials > (long long)1 << 40) return PA_ERR_UNSUPPORTED;
  if (rows == 0) return PA_OK;
  if (!partial_out || !partial_lse || !out) return PA_ERR_NULL_ARG;
  CombineParams c = {};
  c.part_out = partial_out;
  c.part_lse = partial_lse;
  c.out = static_cast<uint16_t*>(out);
  c.lse = lse;
  c.num_parts = num_partials;
  c.rows = rows;
  c.head_dim = head_dim;
  if (launch_combine(c, static_cast<hipStream_t>(stream)) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_gather_kv(const pa_shape* shape, const void* cache, const int32_t* block_table,
                       const int32_t* ctx_lens, void* dst, void* stream) {
  const pa_status st = check_shape(shape);
  if (st != PA_OK) return st;
  if (shape->num_seqs == 0 || shape->max_ctx_len == 0) return PA_OK;
  if (!cache || !block_table || !ctx_lens || !dst) return PA_ERR_NULL_ARG;
  GatherParams g = {};
  g.cache = static_cast<const uint16_t*>(cache);
  g.block_table = block_table;
  g.ctx_lens = ctx_lens;
  g.dst = static_cast<uint16_t*>(dst);
  g.num_seqs = shape->num_seqs;
  g.num_kv_heads = shape->num_kv_heads;
  g.max_blocks = shape->max_blocks_per_seq;
  g.max_ctx = shape->max_ctx_len;
  g.max_pages = ceil_div(shape->max_ctx_len, kBlockSize);
  if (launch_gather(g, static_cast<hipStream_t>(stream)) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_validate(const pa_shape* shape, const int32_t* block_table, const int32_t* ctx_lens,
                      const int32_t* q_lens, const void* workspace, size_t workspace_bytes,
                      int32_t* error_word, void* stream) {
  const pa_status st = check_shape(shape);
  if (st != PA_OK) return st;
  if (!error_word) return PA_ERR_NULL_ARG;
  if (shape->num_seqs > 0 && (!block_table || !ctx_lens || !q_lens)) return PA_ERR_NULL_ARG;
  ValidateParams v = {};
  // The counters sit at the start of the workspace for every page format
  // and for the suffix pass of pa_attend_prefix: one per (slot, KV head),
  // present whenever the shape needs a workspace.
  Plan plan, comp;
  if (workspace && make_plan(shape, &plan) == PA_OK && make_plan(shape, &comp, true) == PA_OK &&
      std::max(plan.ws_bytes, comp.ws_bytes) > 0) {
    const size_t bytes = std::max(plan.counters_bytes, comp.counters_bytes);
    if (workspace_bytes < bytes) return PA_ERR_WORKSPACE_TOO_SMALL;
    v.counters = static_cast<const int32_t*>(workspace);
    v.num_counters = (int32_t)(bytes / sizeof(int32_t));
  }
  v.block_table = block_table;
  v.ctx_lens = ctx_lens;
  v.q_lens = q_lens;
  v.error_word = error_word;
  v.num_blocks = shape->num_blocks;
  v.num_seqs = shape->num_seqs;
  v.max_blocks = shape->max_blocks_per_seq;
  v.max_ctx = shape->max_ctx_len;
  v.max_q = shape->max_q_len;
  v.total_q = shape->total_q;
  if (launch_validate(v, static_cast<hipStream_t>(stream)) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_write_kv(const pa_shape* shape, const void* k_new, const void* v_new,
                      const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens,
                      void* k_cache, void* v_cache, void* stream) {
  const pa_status st = check_shape(shape);
  if (st != PA_OK) return st;
  if (shape->num_seqs == 0 || shape->total_q == 0 || shape->max_q_len == 0) return PA_OK;
  if (!k_new || !v_new || !block_table || !ctx_lens || !q_lens || !k_cache || !v_cache)
    return PA_ERR_NULL_ARG;
  WriteParams w = {};
  w.k_new = static_cast<const uint16_t*>(k_new);
  w.v_new = static_cast<const uint16_t*>(v_new);
  w.block_table = block_table;
  w.ctx_lens = ctx_lens;
  w.q_lens = q_lens;
  w.k_cache = static_cast<uint16_t*>(k_cache);
  w.v_cache = static_cast<uint16_t*>(v_cache);
  w.num_blocks = shape->num_blocks;
  w.num_seqs = shape->num_seqs;
  w.num_kv_heads = shape->num_kv_heads;
  w.max_blocks = shape->max_blocks_per_seq;
  w.max_q_len = shape->max_q_len;
  w.total_q = shape->total_q;
  if ((long long)ceil_div(shape->max_q_len, 16) * shape->num_seqs > INT_MAX) return PA_ERR_UNSUPPORTED;
  if (launch_write_kv(w, static_cast<hipStream_t>(stream)) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_copy_blocks(int32_t num_copies, const int32_t* src, const int32_t* dst,
                         int32_t num_kv_heads, int64_t num_blocks, void* k_cache, void* v_cache,
                         void* stream) {
  if (num_copies < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_BAD_SHAPE;
  if ((long long)num_copies * num_kv_heads * 2 > INT_MAX) return PA_ERR_UNSUPPORTED;
  if (num_copies == 0) return PA_OK;
  if (!src || !dst || !k_cache || !v_cache) return PA_ERR_NULL_ARG;
  CopyParams c = {};
  c.src = src;
  c.dst = dst;
  c.k_cache = static_cast<uint16_t*>(k_cache);
  c.v_cache = static_cast<uint16_t*>(v_cache);
  c.num_blocks = num_blocks;
  c.num_copies = num_copies;
  c.num_kv_heads = num_kv_heads;
  if (launch_copy_blocks(c, static_cast<hipStream_t>(stream)) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_attend_kv(const pa_shape* shape, const pa_kv_cache* cache, const void* q,
                       const int32_t* block_table, const int32_t* ctx_lens,
                       const int32_t* q_lens, float scale, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!cache) return PA_ERR_NULL_ARG;
  const pa_status st = check_kv_cache(*cache);
  if (st != PA_OK) return st;
  return attend_impl(shape, *cache, q, block_table, ctx_lens, q_lens, scale, out, lse, workspace,
                     workspace_bytes, stream);
}

pa_status pa_write_kv_cache(const pa_shape* shape, const pa_kv_cache* cache, const void* k_new,
                            const void* v_new, const int32_t* block_table,
                            const int32_t* ctx_lens, const int32_t* q_lens, void* stream) {
  if (!cache) return PA_ERR_NULL_ARG;
  pa_status st = check_kv_cache(*cache);
  if (st != PA_OK) return st;
  if (cache->format == kFmtBF16)
    return pa_write_kv(shape, k_new, v_new, block_table, ctx_lens, q_lens, cache->k_codes,
                       cache->v_codes, stream);
  st = check_shape(shape);
  if (st != PA_OK) return st;
  if (shape->num_seqs == 0 || shape->total_q == 0 || shape->max_q_len == 0) return PA_OK;
  if (!k_new || !v_new || !block_table || !ctx_lens || !q_lens || !cache->k_codes || !cache->v_codes)
    return PA_ERR_NULL_ARG;
  const bool grouped = cache->format == kFmtQ8 || cache->format == kFmtQ4;
  if (grouped && (!cache->k_scales || !cache->v_scales)) return PA_ERR_NULL_ARG;
  if ((long long)ceil_div(shape->max_q_len, 16) * shape->num_seqs > INT_MAX) return PA_ERR_UNSUPPORTED;
  WriteQuantParams w = {};
  w.w.k_new = static_cast<const uint16_t*>(k_new);
  w.w.v_new = static_cast<const uint16_t*>(v_new);
  w.w.block_table = block_table;
  w.w.ctx_lens = ctx_lens;
  w.w.q_lens = q_lens;
  w.w.k_cache = static_cast<uint16_t*>(cache->k_codes);
  w.w.v_cache = static_cast<uint16_t*>(cache->v_codes);
  w.w.num_blocks = shape->num_blocks;
  w.w.num_seqs = shape->num_seqs;
  w.w.num_kv_heads = shape->num_kv_heads;
  w.w.max_blocks = shape->max_blocks_per_seq;
  w.w.max_q_len = shape->max_q_len;
  w.w.total_q = shape->total_q;
  w.k_scales = static_cast<uint16_t*>(cache->k_scales);
  w.v_scales = static_cast<uint16_t*>(cache->v_scales);
  w.k_scale = cache->k_scale;
  w.v_scale = cache->v_scale;
  if (launch_write_kv_quant(w, cache->format, static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

size_t pa_prefix_workspace_size(const pa_shape* shape, const pa_prefix_groups* groups) {
  PrefixPlan pp;
  if (make_prefix_plan(shape, groups, &pp) != PA_OK) return 0;
  return pp.ws_bytes;
}

pa_status pa_prefix_workspace_init(const pa_shape* shape, const pa_prefix_groups* groups,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  PrefixPlan pp;
  const pa_status st = make_prefix_plan(shape, groups, &pp);
  if (st != PA_OK) return st;
  if (!workspace) return PA_ERR_NULL_ARG;
  if (workspace_bytes < pp.ws_bytes) return PA_ERR_WORKSPACE_TOO_SMALL;
  if (pp.suffix.counters_bytes == 0) return PA_OK;
  if (launch_zero_i32(static_cast<int32_t*>(workspace), pp.suffix.counters_bytes / sizeof(int32_t),
                      static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_attend_prefix(const pa_shape* shape, const pa_prefix_groups* groups, const void* q,
                           const void* k_cache, const void* v_cache, const int32_t* block_table,
                           const int32_t* ctx_lens, const int32_t* q_lens, float scale, void* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  PrefixPlan pp;
  const pa_status st = make_prefix_plan(shape, groups, &pp);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale)) return PA_ERR_BAD_SHAPE;
  if (pp.suffix.empty) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_table || !ctx_lens || !q_lens || !out) return PA_ERR_NULL_ARG;
  if (groups->num_groups > 0 && (!groups->group_start || !groups->prefix_len)) return PA_ERR_NULL_ARG;
  if (!workspace) return PA_ERR_NULL_ARG;
  if (workspace_bytes < pp.ws_bytes) return PA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const float scale_log2 = scale * kLog2e;

  PrefixParams pr = {};
  pr.q = static_cast<const uint16_t*>(q);
  pr.k = static_cast<const uint16_t*>(k_cache);
  pr.v = static_cast<const uint16_t*>(v_cache);
  pr.block_table = block_table;
  pr.ctx_lens = ctx_lens;
  pr.q_lens = q_lens;
  pr.group_start = groups->group_start;
  pr.prefix_len = groups->prefix_len;
  pr.pre_out = reinterpret_cast<float*>(ws + pp.pre_out_offset);
  pr.pre_lse = reinterpret_cast<float*>(ws + pp.pre_lse_offset);
  pr.slot_plen = reinterpret_cast<int32_t*>(ws + pp.plen_offset);
  pr.scale_log2 = scale_log2;
  pr.num_seqs = shape->num_seqs;
  pr.num_q_heads = shape->num_q_heads;
  pr.num_kv_heads = shape->num_kv_heads;
  pr.max_blocks = shape->max_blocks_per_seq;
  pr.total_q = shape->total_q;
  pr.num_groups = groups->num_groups;
  pr.row_tiles = pp.row_tiles > 0 ? pp.row_tiles : 1;
  pr.pre_parts = pp.pre_parts;
  pr.part_pages = pp.pre_pages;
  pr.max_members = groups->max_members;

  pa_kv_cache kv = {};
  kv.format = kFmtBF16;
  kv.k_codes = const_cast<void*>(k_cache);
  kv.v_codes = const_cast<void*>(v_cache);
  DecodeParams d = decode_params(shape, pp.suffix, kv, q, block_table, ctx_lens, q_lens, scale_log2, out, lse, ws);
  d.slot_plen = pr.slot_plen;
  d.pre_out = pr.pre_out;
  d.pre_lse = pr.pre_lse;
  // Where every grouped slot has the same prefix, the partitions request
  // their first page ids for it before knowing their own.
  d.guess_plen = groups->min_prefix_len == groups->max_prefix_len ? groups->max_prefix_len : 0;

  // One launch for the shared and the own keys where the slots' own keys are
  // split (the workspace then has the counters, and the slots' merge counts
  // the prefix partials too): prefix items of kDecodeWaves x
  // prefix_chunk_members members each, placed first in the grid.  A prefix
  // item that arrives last for its members has to merge all of their rows
  // (up to 64) alone, so the plan keeps the prefix items ahead of the slots'
  // partitions: where the whole grid fits one workgroup per CU, it takes the
  // most slot partitions (up to the workspace's) for which prefix items of at
  // most half as many pages still fit beside them (a prefix page costs an
  // item about twice what a page costs a slot's partition: every wave scores
  // it), and as many prefix partitions as the remaining CUs hold (up to the
  // workspace's).  Otherwise the prefix pass's partitions and the slots' own
  // plan.  With fewer than 64 groups the partitions find their slot's group
  // themselves; otherwise the set-up workgroup (the slots' prefix lengths)
  // runs alone before.
  const int G = pp.suffix.group;
  const int mc = prefix_chunk_members(G);
  if (PA_PREFIX_ONE_LAUNCH && pp.pre_grid > 0 && pp.suffix.decode && pp.suffix.num_parts > 1 &&
      decode_prefix_supports_group(G)) {
    const int max_pages = groups->max_prefix_len / kBlockSize;
    const int chunks = ceil_div(groups->max_members, kDecodeWaves * mc);
    const long long units = (long long)groups->num_groups * shape->num_kv_heads * chunks;
    const long long pairs = (long long)shape->num_seqs * shape->num_kv_heads;
    const int suffix_pages = pp.suffix_pages;
    int pre_pages = PA_PREFIX_ITEM_PAGES > 0 ? PA_PREFIX_ITEM_PAGES : pp.pre_pages;
    int sparts = pp.suffix.num_parts;
    if (PA_PREFIX_ITEM_PAGES == 0 && units > 0) {
      const int s_lo = shape->partition_size > 0 ? sparts : 1;
      for (int ps = sparts; ps >= s_lo; --ps) {
        const long long left = (long long)kNumCUs - pairs * ps;
        if (left < units) continue;
        const long long fit = left / units;
        const int parts = (int)(fit < pp.pre_parts ? fit : pp.pre_parts);
        const int pages = ceil_div(max_pages, parts);
        if (2 * pages <= ceil_div(suffix_pages, ps)) {
          sparts = ps;
          pre_pages = pages;
          break;
        }
      }
    }
    const int pre_parts = ceil_div(max_pages, pre_pages);
    const long long items = units * pre_parts;
    const long long sgrid = pairs * sparts;
    if (pre_parts <= pp.pre_parts && items > 0 && items + sgrid <= INT_MAX) {
      d.num_parts = sparts;
      d.part_pages = sparts == pp.suffix.num_parts ? pp.suffix.part_pages : ceil_div(suffix_pages, sparts);
      if (groups->num_groups < 64) {
        d.slot_plen = nullptr;
        d.num_groups = groups->num_groups;
      } else if (launch_prefix(pr, 0, s) != hipSuccess) {
        return PA_ERR_LAUNCH;
      }
      d.pre_parts = pre_parts;
      d.pre_items = (int)items;
      d.pre_pages = pre_pages;
      d.pre_chunks = chunks;
      d.max_members = groups->max_members;
      d.group_start = groups->group_start;
      d.prefix_len = groups->prefix_len;
      if (launch_decode_prefix(d, G, (unsigned)(items + sgrid), s) != hipSuccess)
        return PA_ERR_LAUNCH;
      return PA_OK;
    }
  }
  if (launch_prefix(pr, pp.pre_grid, s) != hipSuccess) return PA_ERR_LAUNCH;
  d.pre_parts = pp.pre_grid > 0 ? pp.pre_parts : 0;
  if (launch_decode(d, G, kFmtBF16, 1, pp.suffix.grid, s) != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL_ARG: return "a required pointer is NULL";
    case PA_ERR_BAD_SHAPE: return "inconsistent or out-of-range sizes";
    case PA_ERR_UNSUPPORTED: return "valid but unsupported configuration";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than pa_workspace_size()";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_OUT_OF_BLOCKS: return "the block pool has too few free blocks";
    case PA_ERR_SCRATCH_LIMIT: return "the call needs more scratch than pa_attend_noalloc's built-in buffer";
  }
  return "unknown status";
}

}  // extern "C"
