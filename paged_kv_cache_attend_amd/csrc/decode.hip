// decode.hip -- paged decode attention, one new token per slot, split-KV with
// the log-sum-exp merge fused into the same launch.
//
// What it computes: for each active slot and query head, softmax attention of
// the one new query row over the slot's n cached keys, gathered through the
// block table (inference-optimisation chapter, section 8.3.1, Fig. 8-10).
// Decode reads every key and value of every request once per step, so the
// kernel is bound by HBM bandwidth (same chapter, section 8.2.1): per key and
// KV head it moves 512 bytes (K and V, 128 bf16 each) and does 4 FLOP per
// byte for a group of four query heads.  Everything is arranged around
// keeping enough of those bytes in flight:
//
// * Grid: one 256-thread workgroup per (KV head, slot, partition), where a
//   partition is a run of `part_pages` 16-token pages (split-KV, "flash
//   decoding"): short batches still put enough workgroups on 256 CUs.  The
//   hardware id is remapped so each XCD owns a contiguous range of
//   (KV head, slot, partition) work -- the partitions of one slot, and slots
//   that share prefix pages, read under one L2.
// * Each of the 4 waves takes every 4th page of the partition.  A page of one
//   KV head is a contiguous 4 KiB K tile and a 4 KiB V tile; a wave loads
//   each with four 128-bit loads per lane (fully coalesced, 1 KiB per
//   instruction) into a three-page register ring: two pages are in flight
//   while one is consumed, and a page's loads are issued as soon as its
//   buffer is free.  Page ids come from scalar loads one issue ahead.
// * Quantised pages (the chapter's section 8.4.2; FP8 E4M3, q8_0, q4_0) use
//   the same schedule: a lane loads the codes of the same (token, 8 dims)
//   chunks -- 8, 8 or 4 bytes instead of 16 -- plus, for q8_0 / q4_0, the
//   fp16 scale of each chunk's 32-value group, and turns the codes into bf16
//   in registers (exact: E4M3 values and small integers are bf16 values).
//   FP8's per-cache K scale is folded into the softmax scale and its V scale
//   into the result; group scales are applied as described below.
// * Each page runs on the matrix cores.  The K and V tiles go to LDS as bf16
//   (XOR-swizzled 16-byte chunks).  Scores S^T = K Q^T come from four
//   v_mfma_f32_16x16x32_bf16 (16 tokens x 32 dims each), with the group's
//   query heads as the first G of 16 columns (the rest a zero query); a
//   32-dim step is exactly one q8_0 / q4_0 group, so each step's product is
//   weighted by its tokens' K scales before the sum.  In that output layout
//   a lane holds 4 tokens of one head, so the online softmax (log2 domain,
//   scale * log2 e folded in) takes an in-lane max and two lane exchanges
//   (v_permlane16_swap, v_permlane32_swap); the reference max is only
//   raised (and the accumulators rescaled) when a score exceeds it by more
//   than 2^8, which keeps every weight <= 256.
// * PV: the same lanes hold P^T in exactly the B-operand layout of
//   v_mfma_f32_16x16x16_bf16, so the weights (times each token's V group
//   scale, one operand per 32-dim group) are used from registers; the V^T A
//   operand is read from the V tile with transposing LDS reads
//   (ds_read_b64_tr_b16), eight 16-dim blocks per page.  The weights reach
//   PV at close to fp32 accuracy although the operand is bf16: the query
//   heads also fill columns G .. 2G - 1 of the score tile (columns that would
//   otherwise hold a zero query), so those lanes compute the same weights w,
//   and they feed PV the remainder lo = w - hi(w) while lanes of columns < G
//   feed hi(w), w cut to bf16.  hi + lo is w to 2^-15 of w, and the two
//   output columns of a head are added once at the end: no extra matrix
//   product.  Rows past a slot's end are zeroed in the V tile
//   and get weight 0 by select, since their stored codes and scales may be
//   anything.
// * Epilogue: the four waves' (max, sum, acc) merge through LDS.  With one
//   partition the workgroup writes bf16 out and the LSE.  Otherwise it writes
//   its normalised fp32 partial and LSE to the workspace, and the last of the
//   slot's partitions to finish (an atomic counter per (slot, KV head),
//   reset to zero by that same workgroup) merges all partials by their LSE
//   and writes the result, all in the same launch.  Empty partitions and
//   slots with no keys take part with LSE = -inf; a slot whose partials are
//   all -inf writes nothing.
// * Prefix-grouped decode (pa_attend_prefix): a grouped slot's partitions
//   start after its group's shared prefix, and the merge also folds the
//   prefix pass's partials of the slot's rows (written by the launch before).

#include "device.h"

namespace pa {

namespace {

constexpr int kWaves = kDecodeWaves;
#ifndef PA_DECODE_RING
#define PA_DECODE_RING 3
#endif
constexpr int kRing = PA_DECODE_RING;                  // pages per wave in the register ring
constexpr int kTileBytes = kBlockSize * kHeadDim * 2;  // 4 KiB
constexpr float kRescaleSlack = 8.0f;                  // log2 units

// One page of one KV head as loaded: per lane, the codes of chunks
// c = lane + 64 k (k < 4) -- token c / 16, dims 8 (c % 16) .. +8 -- of the K
// and the V tile, and for the grouped formats the scale of each chunk.
template <int F>
struct Page;
template <>
struct Page<kFmtBF16> {
  u32x4_t k[4], v[4];
};
template <>
struct Page<kFmtFP8> {
  u32x2_t k[4], v[4];
};
// Grouped formats: lane L also holds the fp16 scale of (token L / 4, group
// L % 4) of the K and of the V tile -- the tile's 64 scales, one per lane.
template <>
struct Page<kFmtQ8> {
  u32x2_t k[4], v[4];
  uint32_t ks, vs;
};
template <>
struct Page<kFmtQ4> {
  uint32_t k[4], v[4];
  uint32_t ks, vs;
};

// Bytes of codes per (block, KV head) tile.
template <int F>
constexpr int tile_code_bytes() {
  return F == kFmtBF16 ? 4096 : (F == kFmtQ4 ? 1024 : 2048);
}

// Issue the loads of one page (K and V tiles of KV head g) into `b`.
template <int F>
__device__ __forceinline__ void issue_page(Page<F>& b, const DecodeParams& p, int32_t phys, int g,
                                           int lane) {
  const size_t ti = tile_index(phys, g, p.num_kv_heads);
  constexpr int kChunks = kBlockSize * kHeadDim / 8;  // 256 chunks of 8 values per tile
  if constexpr (F == kFmtBF16) {
    const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(p.k) + ti * kChunks + lane;
    const u32x4_t* vp = reinterpret_cast<const u32x4_t*>(p.v) + ti * kChunks + lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) b.k[k] = stream_load(kp + k * 64);
#pragma unroll
    for (int k = 0; k < 4; ++k) b.v[k] = stream_load(vp + k * 64);
  } else if constexpr (F == kFmtFP8 || F == kFmtQ8) {
    const u32x2_t* kp = reinterpret_cast<const u32x2_t*>(p.k) + ti * kChunks + lane;
    const u32x2_t* vp = reinterpret_cast<const u32x2_t*>(p.v) + ti * kChunks + lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) b.k[k] = stream_load(kp + k * 64);
#pragma unroll
    for (int k = 0; k < 4; ++k) b.v[k] = stream_load(vp + k * 64);
  } else {
    const uint32_t* kp = reinterpret_cast<const uint32_t*>(p.k) + ti * kChunks + lane;
    const uint32_t* vp = reinterpret_cast<const uint32_t*>(p.v) + ti * kChunks + lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) b.k[k] = stream_load(kp + k * 64);
#pragma unroll
    for (int k = 0; k < 4; ++k) b.v[k] = stream_load(vp + k * 64);
  }
  if constexpr (F == kFmtQ8 || F == kFmtQ4) {
    b.ks = stream_load(p.k_scales + ti * (kBlockSize * 4) + lane);
    b.vs = stream_load(p.v_scales + ti * (kBlockSize * 4) + lane);
  }
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Eight codes of one chunk -> eight bf16 values (exact for every format).
template <int F, typename T>
__device__ __forceinline__ u32x4_t chunk_to_bf16(const T& c) {
  if constexpr (F == kFmtBF16) {
    return c;
  } else if constexpr (F == kFmtFP8) {
    // Two E4M3 codes straight to two bf16 per instruction (scale 1: exact,
    // every E4M3 value is a bf16 value).
    u32x4_t r;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      r[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w], 1.0f, false));
      r[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[w], 1.0f, true));
    }
    return r;
  } else if constexpr (F == kFmtQ8) {
    u32x4_t r;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int32_t x = (int32_t)c[w];
      r[2 * w] = pack_bf16x2((float)((x << 24) >> 24), (float)((x << 16) >> 24));
      r[2 * w + 1] = pack_bf16x2((float)((x << 8) >> 24), (float)(x >> 24));
    }
    return r;
  } else {
    // Code n stands for n - 8.  With the top bit of every nibble flipped,
    // a nibble read as a signed 4-bit field is exactly n - 8, so a signed
    // bit-field extract (the shift pair) and one conversion give each value.
    const uint32_t x = c ^ 0x88888888u;
    u32x4_t r;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      r[w] = pack_bf16x2((float)((int)(x << (28 - 8 * w)) >> 28), (float)((int)(x << (24 - 8 * w)) >> 28));
    return r;
  }
}

// ---------------------------------------------------------------------------
// One page on the matrix cores (v_mfma_f32_16x16x32_bf16 for the scores,
// v_mfma_f32_16x16x16_bf16 for PV): S^T = K Q^T is 16 tokens x 16 columns
// (column n = query head n of the group, columns past G padded with a zero
// query), and O^T += V^T P^T with P^T taken straight from the score layout.
// ---------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ s16x4_t as_s16x4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(s16x4_t, u32x2_t{lo, hi});
}

// Two fp32 weights as a bf16 pair.  In the lanes of columns < G: hi(w), w
// truncated to bf16 (its top 16 bits); in the lanes of the duplicate columns:
// w - hi(w) (exact in fp32), truncated likewise.  hi + lo is w to within 2^-15
// of w, and both halves come from one byte permute per pair.
__device__ __forceinline__ uint32_t hi_or_lo(float w0, float w1, uint32_t lo_mask) {
  const float x0 = w0 - __uint_as_float(__float_as_uint(w0) & lo_mask);
  const float x1 = w1 - __uint_as_float(__float_as_uint(w1) & lo_mask);
  // bytes 2, 3 of x0 and 2, 3 of x1 -> (lo half, hi half) of the result
  return __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
}

template <int G>
struct WaveState {
  float m_ref;    // reference max (log2 domain) of head lane % 16
  float l_lane;   // this lane's share (tokens 4 (lane / 16) .. + 4 of each page) of that head's sum
  f32x4_t o[8];   // O^T block b: dims 16 b + 4 (lane / 16) + i of head lane % 16
  u32x4_t qb[4];  // Q^T operand of step s: dims 32 s + 8 (lane / 16) .. + 8 of head lane % 16
};

// `sk` / `sv` are this wave's 4 KiB LDS tiles, `sks` / `svs` its 16 x 4
// group scales (q8_0, q4_0).
template <int G, int F>
__device__ __forceinline__ void consume_page(WaveState<G>& st, Page<F>& b, uint8_t* sk, uint8_t* sv,
                                               float* sks, float* svs, int valid, float scale_log2, int lane) {
  const int pr = lane >> 4;
  const int pc = lane & 15;
  constexpr bool kGrouped = F == kFmtQ8 || F == kFmtQ4;

  // K and V tiles -> LDS as bf16, row t keeping its 16-byte chunk c at slot
  // c ^ t.  V rows past the end are zeroed: their codes may decode to
  // anything, NaN included, and a zero weight would not cancel that.
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = 4 * k + pr;
    *reinterpret_cast<u32x4_t*>(sk + t * 256 + ((pc ^ t) << 4)) = chunk_to_bf16<F>(b.k[k]);
    const u32x4_t vv = chunk_to_bf16<F>(b.v[k]);
    *reinterpret_cast<u32x4_t*>(sv + t * 256 + ((pc ^ t) << 4)) = t < valid ? vv : u32x4_t{0u, 0u, 0u, 0u};
  }
  if constexpr (kGrouped) {
    sks[lane] = half_bits_to_float(b.ks);  // [token][group]
    svs[lane] = half_bits_to_float(b.vs);
  }
  wave_lds_sync();

  // Scores: A = K (row = token pc, dims 32 s + 8 pr .. + 8 of step s), B = Q^T.
  // A group of 32 dims is one step, so grouped scales weight each step's
  // product (its own accumulator) before the sum.
  f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kGrouped) {
    f32x4_t ksc[4];  // K scales of this lane's tokens 4 pr + i, groups 0..3
#pragma unroll
    for (int i = 0; i < 4; ++i) ksc[i] = *reinterpret_cast<const f32x4_t*>(sks + (4 * pr + i) * 4);
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
      const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(sk + pc * 256 + (((4 * sg + pr) ^ pc) << 4));
      const f32x4_t part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(st.qb[sg]),
                                                                   f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) s4[i] = fmaf(ksc[i][sg], part[i], s4[i]);
    }
  } else {
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
      const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(sk + pc * 256 + (((4 * sg + pr) ^ pc) << 4));
      s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(st.qb[sg]), s4, 0, 0, 0);
    }
  }

  // Online softmax of column pc over the page's 16 tokens (this lane holds
  // tokens 4 pr .. + 4; the others sit in lanes ^ 16 and ^ 32).
  float sl[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sl[i] = 4 * pr + i < valid ? s4[i] * scale_log2 : -INFINITY;
    mloc = fmaxf(mloc, sl[i]);
  }
  mloc = fmaxf(mloc, other16(mloc));
  mloc = fmaxf(mloc, other_half(mloc));
  const bool raise = mloc > st.m_ref + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(raise) != 0) {
    const float m_new = fmaxf(st.m_ref, mloc);
    const float alpha = fast_exp2(st.m_ref - m_new);  // 0 on the first page (m_ref = -inf)
    st.m_ref = m_new;
    st.l_lane *= alpha;
#pragma unroll
    for (int bb = 0; bb < 8; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.o[bb][i] *= alpha;
  }
  float pw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pw[i] = fast_exp2(sl[i] - st.m_ref);  // 0 past the end
    st.l_lane += pw[i];
  }

  // V^T operand of block bb (dims 16 bb .. + 16, tokens 4 pr .. + 4): lane a
  // = pc points at token 4 pr + a / 4, dims 16 bb + 4 (a % 4) .. + 4, and
  // receives dim 16 bb + a of the four tokens (ds_read_b64_tr_b16).
  const int tv = 4 * pr + (pc >> 2);
  const uint8_t* vrow = sv + tv * 256 + (pc & 1) * 8;
  s16x4_t vt[8];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb)
    vt[bb] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4_t*)(vrow + (((2 * bb + ((pc & 3) >> 1)) ^ tv) << 4)));

  // P^T operand: this lane's tokens 4 pr .. + 4 of column pc, as bf16 (hi
  // in columns < G, lo in columns G .. 2G - 1); with grouped V scales one
  // operand per 32-dim group (tokens past the end get weight 0 by select:
  // their stored scales may be anything).
  const uint32_t lo_mask = pc >= G ? 0xffff0000u : 0u;  // lanes that feed lo subtract hi
  if constexpr (kGrouped) {
    f32x4_t vsc[4];  // V scales of tokens 4 pr + i, groups 0..3
#pragma unroll
    for (int i = 0; i < 4; ++i) vsc[i] = *reinterpret_cast<const f32x4_t*>(svs + (4 * pr + i) * 4);
#pragma unroll
    for (int gr = 0; gr < 4; ++gr) {
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = 4 * pr + i < valid ? pw[i] * vsc[i][gr] : 0.f;
      const s16x4_t pg = as_s16x4(hi_or_lo(w[0], w[1], lo_mask), hi_or_lo(w[2], w[3], lo_mask));
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        st.o[2 * gr + h2] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[2 * gr + h2], pg, st.o[2 * gr + h2], 0, 0, 0);
    }
  } else {
    const s16x4_t pg = as_s16x4(hi_or_lo(pw[0], pw[1], lo_mask), hi_or_lo(pw[2], pw[3], lo_mask));
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) st.o[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[bb], pg, st.o[bb], 0, 0, 0);
  }
}

template <int G, int F>
#ifndef PA_DECODE_MIN_WGS
#define PA_DECODE_MIN_WGS kDecodeWGsPerCU
#endif
__global__ __launch_bounds__(kDecodeThreads, PA_DECODE_MIN_WGS) void decode_kernel(DecodeParams p) {
  static_assert(G == 1 || G == 2 || G == 4, "group size");
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kWaves][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[G][kHeadDim * 2];
  __shared__ __attribute__((aligned(16))) float s_ks[kWaves][kBlockSize * 4];  // q8_0 / q4_0 K scales
  __shared__ __attribute__((aligned(16))) uint8_t s_v[kWaves][kTileBytes];
  __shared__ __attribute__((aligned(16))) float s_vs[kWaves][kBlockSize * 4];    // q8_0 / q4_0 V scales
  __shared__ __attribute__((aligned(16))) float s_acc[kWaves][G][kHeadDim];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The kernel arguments the start needs, fetched together (the compiler
  // would otherwise fetch some of them one round trip later).
  asm volatile("" ::"s"(p.q_lens), "s"(p.ctx_lens), "s"(p.block_table), "s"(p.slot_plen), "s"(p.pre_parts), "s"(p.num_parts),
               "s"(p.num_seqs), "s"(p.part_pages), "s"(p.max_blocks), "s"(gridDim.x));

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int P = p.num_parts;
  const int part = wg % P;
  const int rest = wg / P;
  const int seq = rest % p.num_seqs;
  const int g = rest / p.num_seqs;

  // Everything the start needs comes in one round trip, issued before the
  // first branch: the lengths, the prefix length, the slot's row offset (a
  // vector load and a wave sum) and the page ids of this wave's first four
  // pages as they are when the slot has no prefix (checked below, reloaded
  // otherwise).  Lengths and page ids are wave-uniform scalar loads, which do
  // not share the (in-order) vector load counter with the page stream.
  const int32_t* bt = p.block_table + (size_t)seq * p.max_blocks;
  const int spage0 = part * p.part_pages + wave;  // first page without a prefix
  const int m = scalar_load_i32(p.q_lens, seq);
  const int n = scalar_load_i32(p.ctx_lens, seq);
  // Prefix-grouped decode: this slot's keys start after its shared prefix,
  // whose partials the prefix pass has written; the last partition runs to
  // the slot's end whatever the prefix length.
  const int plen = p.slot_plen ? scalar_load_i32(p.slot_plen, seq) : 0;
  int32_t sid[kRing + 1];
#pragma unroll
  for (int k = 0; k <= kRing; ++k) sid[k] = scalar_load_i32(bt, min(spage0 + k * kWaves, p.max_blocks - 1));
  int qsum = 0;  // this lane's share of the row offset
  for (int i = lane; i < seq; i += 64) qsum += p.q_lens[i];
  // (Keeps the loads above the branch: the compiler would otherwise sink the
  // ones only the working path uses below it, one round trip later.  The
  // wave sum of the row offset waits until the first page is requested.)
#pragma unroll
  for (int k = 0; k <= kRing; ++k) asm volatile("" : "+s"(sid[k]));
  asm volatile("" : "+v"(qsum));
  if (m <= 0) return;  // no row: nothing to write, no partial to count
  const int npages = (n + kBlockSize - 1) / kBlockSize;
  const int npre = (plen > 0 && n > 0) ? p.pre_parts : 0;
  const int pstart = plen / kBlockSize + part * p.part_pages;
  const int pend = part == P - 1 ? npages : min(npages, pstart + p.part_pages);
  const bool has_work = n > 0 && pstart < pend;

  const int last_page = pend - 1;
  auto page_id = [&](int page) -> int32_t { return scalar_load_i32(bt, min(page, last_page)); };
  // Page id of this wave's k-th page (clamped to the partition's last page):
  // the early load when it is that page.
  auto first_id = [&](int k) -> int32_t {
    const int page = pstart + wave + k * kWaves;
    return (plen == 0 && page <= last_page) ? sid[k] : page_id(page);
  };

  const int h0 = g * G;
  const size_t rows = (size_t)p.total_q * p.num_q_heads;
  const int my_h = (threadIdx.x * 2) / kHeadDim;  // epilogue role: 2 dims of one head
  const int my_d = (threadIdx.x * 2) % kHeadDim;
  const bool my_out = threadIdx.x * 2 < G * kHeadDim;
  float my_o0 = 0.f, my_o1 = 0.f, my_lse = -INFINITY;  // this workgroup's partial

  // Prologue, in issue order: the wave's first page, the query (so that its
  // wait only covers that first page, needed next anyway), then pages 1 ..
  // kRing - 1.  Every load here is unconditional within the workgroup-
  // uniform has_work branch -- a wave with fewer pages than the ring re-reads
  // a valid page -- so the load counter's waits stay exact.
  Page<F> ring[kRing];
  const int page0 = pstart + wave;
  const int cnt = (has_work && page0 < pend) ? (pend - page0 + kWaves - 1) / kWaves : 0;
  int32_t next_id = 0;
  int q_row;
  if (has_work) {
    issue_page<F>(ring[0], p, first_id(0), g, lane);
    __builtin_amdgcn_sched_barrier(0);  // the first page goes out before the row-offset sum
    q_row = __builtin_amdgcn_readfirstlane(wave_sum_i32(qsum));
    const int qh = (threadIdx.x >> 4) % G, qc = threadIdx.x & 15;
    const u32x4_t qchunk =
        reinterpret_cast<const u32x4_t*>(p.q)[((size_t)q_row * p.num_q_heads + h0 + qh) * 16 + qc];
    issue_order_barrier();
#pragma unroll
    for (int r = 1; r < kRing; ++r) issue_page<F>(ring[r], p, first_id(r), g, lane);
    next_id = first_id(kRing);
    // Query of heads h0 .. h0+G-1 -> LDS, 16-byte chunk c of head h at slot c ^ h.
    if (threadIdx.x < G * 16) *reinterpret_cast<u32x4_t*>(&s_q[qh][(qc ^ qh) << 4]) = qchunk;
    __syncthreads();
  } else {
    q_row = __builtin_amdgcn_readfirstlane(wave_sum_i32(qsum));
  }

  if (has_work) {
    WaveState<G> st;
    st.m_ref = -INFINITY;
    st.l_lane = 0.f;
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) st.o[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Q^T operand from the staged query (head h keeps chunk c at slot c ^ h):
    // column n < 2G holds query head n % G (the second copy carries the lo
    // weights of PV); columns from 2G on get a zero query.
    {
      const int qn = lane & 15, qr = lane >> 4;
      const int qh = qn & (G - 1);
#pragma unroll
      for (int sg = 0; sg < 4; ++sg) {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(&s_q[qh][((4 * sg + qr) ^ qh) << 4]);
        st.qb[sg] = qn < 2 * G ? x : u32x4_t{0u, 0u, 0u, 0u};
      }
    }

    uint8_t* sk = s_k[wave];
    uint8_t* sv = s_v[wave];
    float* sks = s_ks[wave];
    float* svs = s_vs[wave];
    // This wave's pages are page0 + 4k for k < cnt; page k lives in ring
    // slot k % kRing.  The main loop reissues unconditionally, so the
    // (in-order) load counter sees the same pattern on every trip and each
    // wait leaves the other kRing - 1 pages in flight; the last pages are
    // peeled off.
    auto valid_of = [&](int k) { return min(kBlockSize, n - (page0 + kWaves * k) * kBlockSize); };
#define PA_CONSUME(RING, K) consume_page<G, F>(st, RING, sk, sv, sks, svs, valid_of(K), p.scale_log2, lane)
#define PA_REISSUE(RING, K)                                          \
  {                                                                  \
    issue_page<F>(RING, p, next_id, g, lane);                        \
    next_id = page_id(page0 + kWaves * ((K) + 1));                   \
  }
    int k = 0;
    for (; k + 2 * kRing - 1 < cnt; k += kRing) {
#pragma unroll
      for (int r = 0; r < kRing; ++r) {
        PA_CONSUME(ring[r], k + r);
        PA_REISSUE(ring[r], k + r + kRing);
      }
    }
    // At most 2 kRing - 1 pages left: k .. k + kRing - 1 in the ring (those
    // that exist), the rest still to be issued.
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      if (k + r < cnt) {
        PA_CONSUME(ring[r], k + r);
        if (k + r + kRing < cnt) PA_REISSUE(ring[r], k + r + kRing);
      }
    }
#pragma unroll
    for (int r = 0; r < kRing - 1; ++r)
      if (k + kRing + r < cnt) PA_CONSUME(ring[r], k + kRing + r);
#undef PA_CONSUME
#undef PA_REISSUE

    // Per-wave state -> LDS.  Column pc's sum is spread over lanes pc + 16 j;
    // its O^T block values are dims 16 b + 4 pr + i, to which the lo column
    // pc + G (lane ^ G, since pc < G and G is a power of two) is added.
    // FP8's V scale applies here, once.
    const int pr = lane >> 4;
    const int pc = lane & 15;
    float l_sum = st.l_lane + other16(st.l_lane);
    l_sum += other_half(l_sum);
    const float vs = F == kFmtFP8 ? p.v_scale : 1.f;
    f32x4_t o_tot[8];
#pragma unroll
    for (int bb = 0; bb < 8; ++bb)
#pragma unroll
      for (int i = 0; i < 4; ++i) o_tot[bb][i] = st.o[bb][i] + __shfl_xor(st.o[bb][i], G, 64);
    if (pc < G) {
      if (pr == 0) {
        s_m[wave][pc] = st.m_ref;
        s_l[wave][pc] = l_sum;
      }
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
        *reinterpret_cast<f32x4_t*>(&s_acc[wave][pc][16 * bb + 4 * pr]) = o_tot[bb] * vs;
    }
    __syncthreads();

    // Merge the waves: two adjacent dims of one head per thread.
    if (my_out) {
      const int h = my_h, d = my_d;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
      float L = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float sc = fast_exp2(s_m[w][h] - M);  // 0 for a wave with no page
        L = fmaf(sc, s_l[w][h], L);
        const float2 v = *reinterpret_cast<const float2*>(&s_acc[w][h][d]);
        a0 = fmaf(sc, v.x, a0);
        a1 = fmaf(sc, v.y, a1);
      }
      const float inv = 1.f / L;
      my_o0 = a0 * inv;
      my_o1 = a1 * inv;
      my_lse = (M + fast_log2(L)) * kLn2;  // natural log
    }
  }

  if (P == 1) {
    if (!my_out) return;
    const size_t row = (size_t)q_row * p.num_q_heads + h0 + my_h;
    if (npre == 0) {
      if (has_work) {
        reinterpret_cast<uint32_t*>(p.out)[(row * kHeadDim + my_d) / 2] = pack_bf16x2(my_o0, my_o1);
        if (my_d == 0 && p.lse) p.lse[row] = my_lse;
      }
      return;
    }
    // Own result and the prefix pass's partials of this row (written by the
    // previous launch).
    MergeState ms;
    if (has_work) merge_fold(ms, my_lse, my_o0, my_o1);
    merge_partials(ms, nullptr, nullptr, 0, p.pre_lse + row, p.pre_out + row * kHeadDim + my_d, npre, rows);
    if (ms.M != -INFINITY) {
      const float inv = 1.f / ms.W;
      reinterpret_cast<uint32_t*>(p.out)[(row * kHeadDim + my_d) / 2] = pack_bf16x2(ms.a0 * inv, ms.a1 * inv);
      if (my_d == 0 && p.lse) p.lse[row] = ms.M + fast_log2(ms.W) * kLn2;
    }
    return;
  }

  // Split: publish this partition's partial, count it, and let the last
  // partition of the (slot, KV head) to finish merge them all.  The partials
  // and the counter are exchanged with relaxed device-scope atomics; the
  // ordering that makes the merger see every partial is the hardware's, in
  // this order (a CPU test checks it on the gfx950 assembly):
  //   1. each thread's partial stores are device-scope (sc1): written through
  //      to the point of coherence that every XCD reads;
  //   2. s_waitcnt vmcnt(0): the stores are acknowledged there (on gfx9 the
  //      vector-memory counter also counts stores);
  //   3. s_barrier: every thread of the workgroup has passed step 2;
  //   4. one thread's counter atomic, whose returned value decides, through
  //      LDS and a second barrier, whether this workgroup merges;
  //   5. the merger's loads are device-scope (sc1) and issued after that
  //      decision, so each reads the point of coherence after every other
  //      partition's step 2.
  // This avoids device-scope release/acquire fences, which on this chip
  // write back and invalidate the whole L2 of the XCD.
  uint64_t* part_out64 = reinterpret_cast<uint64_t*>(p.part_out);
  if (my_out) {
    const size_t prow = (size_t)part * rows + (size_t)q_row * p.num_q_heads + h0 + my_h;
    if (has_work) {
      const uint64_t bits = (uint64_t)__float_as_uint(my_o0) | ((uint64_t)__float_as_uint(my_o1) << 32);
      __hip_atomic_store(part_out64 + (prow * kHeadDim + my_d) / 2, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (my_d == 0) __hip_atomic_store(p.part_lse + prow, my_lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_vm_stores();
  __syncthreads();
  int32_t* counter = p.counters + (size_t)seq * p.num_kv_heads + g;
  if (threadIdx.x == 0)
    s_last = (__hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == P - 1);
  __syncthreads();
  if (!s_last) return;

  // Merge by log-sum-exp weights: this slot's P partials and, with a shared
  // prefix, the prefix pass's npre, their loads issued in batches before any
  // is used; a partial with LSE = -inf (empty) gets weight 0 without its
  // output being read.
  if (my_out) {
    const size_t row = (size_t)q_row * p.num_q_heads + h0 + my_h;
    MergeState ms;
    merge_partials(ms, p.part_lse + row, p.part_out + row * kHeadDim + my_d, P,
                   p.pre_lse + row, p.pre_out + row * kHeadDim + my_d, npre, rows);
    if (ms.M != -INFINITY) {
      const float inv = 1.f / ms.W;
      reinterpret_cast<uint32_t*>(p.out)[(row * kHeadDim + my_d) / 2] = pack_bf16x2(ms.a0 * inv, ms.a1 * inv);
      if (my_d == 0 && p.lse) p.lse[row] = ms.M + fast_log2(ms.W) * kLn2;
    }
  }
  // Leave the counter at zero for the next call (the next launch sees it).
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void zero_kernel(int32_t* __restrict__ x, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    x[i] = 0;
}

}  // namespace

bool decode_supports_group(int group) { return group == 1 || group == 2 || group == 4; }

template <int F>
const void* decode_entry(int group) {
  switch (group) {
    case 1: return reinterpret_cast<const void*>(&decode_kernel<1, F>);
    case 2: return reinterpret_cast<const void*>(&decode_kernel<2, F>);
    case 4: return reinterpret_cast<const void*>(&decode_kernel<4, F>);
  }
  return nullptr;
}

hipError_t launch_decode(const DecodeParams& p, int group, int format, unsigned grid, hipStream_t s) {
  const void* fn = nullptr;
  switch (format) {
    case kFmtBF16: fn = decode_entry<kFmtBF16>(group); break;
    case kFmtFP8: fn = decode_entry<kFmtFP8>(group); break;
    case kFmtQ8: fn = decode_entry<kFmtQ8>(group); break;
    case kFmtQ4: fn = decode_entry<kFmtQ4>(group); break;
  }
  if (!fn) return hipErrorInvalidValue;
  DecodeParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, dim3(grid), dim3(kDecodeThreads), args, 0, s);
}

hipError_t launch_zero_i32(int32_t* x, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  int32_t* xa = x;
  size_t na = n;
  void* args[] = {&xa, &na};
  return hipLaunchKernel(reinterpret_cast<const void*>(&zero_kernel), dim3((unsigned)blocks), dim3(256), args, 0, s);
}

}  // namespace pa
