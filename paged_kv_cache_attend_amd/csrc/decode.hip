// decode.hip -- paged decode attention, one to eight new tokens per slot,
// split-KV with the log-sum-exp merge fused into the same launch.
//
// What it computes: for each active slot and query head, softmax attention of
// each new query row over the slot's n cached keys, gathered through the
// block table (inference-optimisation chapter, section 8.3.1, Fig. 8-10).
// A slot usually brings one new token; verifying several proposed tokens at
// once (section 8.5 of the same chapter) brings up to eight, and with
// PA_FLAG_CAUSAL new token t sees keys [0, n - m + t] (section 8.2.3).
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
//   product.  Where the columns leave no room for the lo copies (several
//   tokens per slot), the weights go in rounded to bf16 and the output is
//   divided by the sum of the rounded weights; a partition in which some
//   row sees fewer than kFewKeys keys also feeds the rounding's remainders
//   through a product of their own.  Rows past a slot's end are zeroed in the V tile
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
// * Several new tokens: the (token, query head) pairs of a KV head are the
//   columns of the score tile (see Cols below), so the pages are streamed
//   once for all of them; each column has its own causal limit.
// * Prefix-grouped decode (pa_attend_prefix): a grouped slot's partitions
//   start after its group's shared prefix, and the merge also folds the
//   prefix partials of the slot's rows: written by the launch before, or,
//   in the instance with prefix items, by the same launch's first
//   workgroups, which read each shared page once for up to 4 x 16/G members
//   (see prefix_item).

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
// Where a weight enters PV as one bf16 number (no room for the lo copies),
// a partial whose rows see few keys cannot average the rounding of its
// weights down: with fewer than this many keys for some row, the wave also
// feeds the rounding's remainders through a second product (the cost is
// twice the PV products on the few pages such a partial has).
constexpr int kFewKeys = 64;

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

// Columns of the score tile.  A slot's (token, query head) pairs of one KV
// head, token major -- column c is token c / G of query head g G + c % G --
// for up to M tokens per slot: C = G M real columns.  When two copies fit in
// a 16-column tile (2C <= 16, always so for one token with up to 8 heads per
// KV head), columns C .. 2C - 1 repeat the queries and carry the lo halves of
// the weights (see hi_or_lo); otherwise NT = ceil(C / 16) tiles of 16
// columns take the bf16-rounded weights, and a column's output is divided by
// the sum of those same rounded weights.
template <int G, int M>
struct Cols {
  static constexpr int C = G * M;
  static constexpr bool HL = 2 * C <= 16;
  static constexpr int NT = HL ? 1 : (C + 15) / 16;
  static constexpr int J = (C * kHeadDim / 2 + kDecodeThreads - 1) / kDecodeThreads;  // epilogue pairs per thread
};

template <int NT>
struct WaveState {
  float m_ref[NT];    // reference max (log2 domain) of column 16 ct + lane % 16
  float l_lane[NT];   // this lane's share (tokens 4 (lane / 16) .. + 4 of each page) of that column's sum
  float r_lane[NT];   // the same over the bf16-rounded weights (tiles without lo columns)
  f32x4_t o[NT][8];   // O^T block b: dims 16 b + 4 (lane / 16) + i of that column
  u32x4_t qb[NT][4];  // Q^T operand of step s: dims 32 s + 8 (lane / 16) .. + 8 of that column
};

// A page's K and V tiles -> the 4 KiB LDS tiles `sk` / `sv` as bf16, row t
// keeping its 16-byte chunk c at slot c ^ t; `sks` / `svs` take its 16 x 4
// group scales (q8_0, q4_0).  V rows past the end are zeroed: their codes
// may decode to anything, NaN included, and a zero weight would not cancel
// that.
template <int F>
__device__ __forceinline__ void stage_page(const Page<F>& b, uint8_t* sk, uint8_t* sv, float* sks, float* svs,
                                           int valid, int lane) {
  const int pr = lane >> 4;
  const int pc = lane & 15;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = 4 * k + pr;
    *reinterpret_cast<u32x4_t*>(sk + t * 256 + ((pc ^ t) << 4)) = chunk_to_bf16<F>(b.k[k]);
    const u32x4_t vv = chunk_to_bf16<F>(b.v[k]);
    *reinterpret_cast<u32x4_t*>(sv + t * 256 + ((pc ^ t) << 4)) = t < valid ? vv : u32x4_t{0u, 0u, 0u, 0u};
  }
  if constexpr (F == kFmtQ8 || F == kFmtQ4) {
    sks[lane] = half_bits_to_float(b.ks);  // [token][group]
    svs[lane] = half_bits_to_float(b.vs);
  }
}

// Scores and weighted values of one staged page for this wave's columns.
// `kbase` is the page's first key index and lim[ct] the last key this lane's
// column of tile ct may see (several tokens per slot only).
template <int G, int F, int M>
__device__ __forceinline__ void score_page(WaveState<Cols<G, M>::NT>& st, const uint8_t* sk, const uint8_t* sv,
                                           const float* sks, const float* svs, int valid, float scale_log2, int lane,
                                           int kbase, const int* lim, bool fine = false) {
  using CS = Cols<G, M>;
  constexpr int NT = CS::NT;
  const int pr = lane >> 4;
  const int pc = lane & 15;
  constexpr bool kGrouped = F == kFmtQ8 || F == kFmtQ4;
  static_assert(!kGrouped || M == 1, "grouped page formats decode one token per slot");

  // Scores: A = K (row = token pc, dims 32 s + 8 pr .. + 8 of step s), B = Q^T.
  // A group of 32 dims is one step, so grouped scales weight each step's
  // product (its own accumulator) before the sum.
  f32x4_t s4[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) s4[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (kGrouped) {
    f32x4_t ksc[4];  // K scales of this lane's tokens 4 pr + i, groups 0..3
#pragma unroll
    for (int i = 0; i < 4; ++i) ksc[i] = *reinterpret_cast<const f32x4_t*>(sks + (4 * pr + i) * 4);
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
      const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(sk + pc * 256 + (((4 * sg + pr) ^ pc) << 4));
      const f32x4_t part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(st.qb[0][sg]),
                                                                   f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) s4[0][i] = fmaf(ksc[i][sg], part[i], s4[0][i]);
    }
  } else {
#pragma unroll
    for (int sg = 0; sg < 4; ++sg) {
      const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(sk + pc * 256 + (((4 * sg + pr) ^ pc) << 4));
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
        s4[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(st.qb[ct][sg]), s4[ct], 0, 0, 0);
    }
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

#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    // Online softmax of column 16 ct + pc over the page's 16 tokens (this
    // lane holds tokens 4 pr .. + 4; the others sit in lanes ^ 16 and ^ 32).
    float sl[4];
    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool vis = 4 * pr + i < valid && (M == 1 || kbase + 4 * pr + i <= lim[ct]);
      sl[i] = vis ? s4[ct][i] * scale_log2 : -INFINITY;
      mloc = fmaxf(mloc, sl[i]);
    }
    mloc = fmaxf(mloc, other16(mloc));
    mloc = fmaxf(mloc, other_half(mloc));
    const bool raise = mloc > st.m_ref[ct] + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float m_new = fmaxf(st.m_ref[ct], mloc);
      // 0 on the first page (m_ref = -inf).  With several tokens, a column
      // that has seen no visible key yet keeps m = -inf (its sums are 0)
      // while another column raises: guard -inf - -inf.
      const float alpha = fast_exp2(st.m_ref[ct] - ((M > 1 && m_new == -INFINITY) ? 0.f : m_new));
      st.m_ref[ct] = m_new;
      st.l_lane[ct] *= alpha;
      st.r_lane[ct] *= alpha;
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.o[ct][bb][i] *= alpha;
    }
    // With several tokens a column can meet a page with no visible key
    // before any visible one (its reference max still -inf): weight 0.
    const float m_use = (M > 1 && st.m_ref[ct] == -INFINITY) ? 0.f : st.m_ref[ct];
    float pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = fast_exp2(sl[i] - m_use);  // 0 past the end
      st.l_lane[ct] += pw[i];
    }

    // P^T operand: this lane's tokens 4 pr .. + 4 of its column, as bf16 (hi
    // in columns < C and lo in columns C .. 2C - 1 when the tile holds both
    // copies, else rounded to nearest); with grouped V scales one operand per
    // 32-dim group (tokens past the end get weight 0 by select: their stored
    // scales may be anything).
    if constexpr (kGrouped) {
      const uint32_t lo_mask = pc >= CS::C ? 0xffff0000u : 0u;  // lanes that feed lo subtract hi
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
          st.o[0][2 * gr + h2] =
              __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[2 * gr + h2], pg, st.o[0][2 * gr + h2], 0, 0, 0);
      }
    } else {
      s16x4_t pg;
      if constexpr (CS::HL) {
        const uint32_t lo_mask = pc >= CS::C ? 0xffff0000u : 0u;  // lanes that feed lo subtract hi
        pg = as_s16x4(hi_or_lo(pw[0], pw[1], lo_mask), hi_or_lo(pw[2], pw[3], lo_mask));
      } else {
        const uint32_t w01 = pack_bf16x2(pw[0], pw[1]);
        const uint32_t w23 = pack_bf16x2(pw[2], pw[3]);
        st.r_lane[ct] += (bf16_lo(w01) + bf16_hi(w01)) + (bf16_lo(w23) + bf16_hi(w23));
        pg = as_s16x4(w01, w23);
      }
      if (!CS::HL && __builtin_expect(fine, 0)) {
        // Few keys (see kFewKeys): the rounding's remainders go through a
        // product of their own, so PV sums the fp32 weights, and their sum
        // is the divisor.
        const uint32_t hi01 = __builtin_bit_cast(u32x2_t, pg)[0], hi23 = __builtin_bit_cast(u32x2_t, pg)[1];
        st.r_lane[ct] += ((pw[0] + pw[1]) + (pw[2] + pw[3])) -
                         ((bf16_lo(hi01) + bf16_hi(hi01)) + (bf16_lo(hi23) + bf16_hi(hi23)));
        const s16x4_t pl = as_s16x4(lo_after(pw[0], pw[1], hi01), lo_after(pw[2], pw[3], hi23));
#pragma unroll
        for (int bb = 0; bb < 8; ++bb)
          st.o[ct][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[bb], pl, st.o[ct][bb], 0, 0, 0);
      }
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
        st.o[ct][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt[bb], pg, st.o[ct][bb], 0, 0, 0);
    }
  }
}

// One page of this wave's own: staged in its LDS tiles, then scored.
template <int G, int F, int M>
__device__ __forceinline__ void consume_page(WaveState<Cols<G, M>::NT>& st, Page<F>& b, uint8_t* sk, uint8_t* sv,
                                             float* sks, float* svs, int valid, float scale_log2, int lane,
                                             int kbase, const int* lim, bool fine) {
  stage_page<F>(b, sk, sv, sks, svs, valid, lane);
  wave_lds_sync();
  score_page<G, F, M>(st, sk, sv, sks, svs, valid, scale_log2, lane, kbase, lim, fine);
}

// Partitions of `parts` (of part_pages pages, the last running to the end)
// that hold any of a slot's `pages` own pages.
__device__ __forceinline__ int partitions_with_keys(int pages, int parts, int part_pages) {
  return min(parts, (max(pages, 0) + part_pages - 1) / part_pages);
}

// One prefix item of a prefix-grouped decode done in one launch (pre_items
// > 0): pages [pp pre_pages, ...) of one group's shared prefix for one KV
// head, read once for up to kWaves M of the group's members.  The waves take
// turns loading the pages (wave w the w-th of every kWaves) and stage them in
// LDS; after a barrier every wave scores all kWaves staged pages for its own
// M members: column c of wave w is member w M + c / G, query head h0 + c % G
// (each member brings at most one row on this path).  Each wave so ends with
// the whole range for its members, and the waves need no merge.  Two stages
// alternate (the second in the epilogue area, when that is large enough), so
// one barrier per step orders both the writes and the reuse.  A member sees
// the prefix up to its own length.  The item writes its members' partials to
// pre_out / pre_lse (normalised, with their LSE; -inf where no key is
// visible), counts them on each member's counter like a partition of that
// slot, and merges the slots it arrives last for, with the ordering of the
// partition path.
template <int G, int F, int M>
__device__ __forceinline__ void prefix_item(const DecodeParams& p, int pi, int lane, int wave,
                                            uint8_t (*s_k)[kTileBytes], uint8_t (*s_v)[kTileBytes],
                                            float (*s_acc)[Cols<G, M>::C][kHeadDim],
                                            float (*s_m)[Cols<G, M>::C], float (*s_l)[Cols<G, M>::C],
                                            float (*s_r)[Cols<G, M>::C], int* s_lastm) {
  using CS = Cols<G, M>;
  constexpr int C = CS::C;
  static_assert(CS::NT == 1 && F == kFmtBF16, "one bf16 column tile per wave");
  constexpr int kMembers = kWaves * M;
  static_assert(kMembers <= 64, "one lane per member");
  constexpr bool kTwoStages = sizeof(float) * kWaves * C * kHeadDim >= 2 * kWaves * kTileBytes;
  constexpr int kPRing = 2;  // pages per wave in flight; ring slot r uses stage r
  uint8_t (*s_k2)[kTileBytes] = reinterpret_cast<uint8_t (*)[kTileBytes]>(&s_acc[0][0][0]);
  uint8_t (*s_v2)[kTileBytes] = s_k2 + kWaves;

  const int ci = pi % p.pre_chunks;
  int rest = pi / p.pre_chunks;
  const int pp = rest % p.pre_parts;
  rest /= p.pre_parts;
  const int g = rest % p.num_kv_heads;
  const int gi = rest / p.num_kv_heads;

  // One round trip before the first page request when the group's first
  // slot is gi * max_members (full, consecutive groups): with the group's
  // bounds and prefix length come, for that guess, the ids of the item's
  // first 64 pages (one per lane, read with v_readlane: no memory wait, which
  // the step barriers would otherwise take for every prefetched id; further
  // pages, only where a prefix outruns the partitions, by scalar loads), the
  // members' lengths (lane j: member j of the item) and the row offset of
  // the slots before them.  A wrong guess costs one more round trip.
  const int pstart = pp * p.pre_pages;
  const int j0 = ci * kMembers;
  auto load_lanes = [&](int s0_, int& pid_, int& mq_, int& mn_, int& qs_) {
    const int32_t* bt_ = p.block_table + (size_t)s0_ * p.max_blocks;
    pid_ = bt_[min(pstart + lane, p.max_blocks - 1)];
    const int sl = min(s0_ + j0 + lane, p.num_seqs - 1);
    mq_ = p.q_lens[sl];
    mn_ = p.ctx_lens[sl];
    qs_ = 0;
    for (int i = lane; i < s0_ + j0; i += 64) qs_ += p.q_lens[i];
  };
  const int s0g = min(gi * p.max_members, max(p.num_seqs - 1, 0));
  int s0 = scalar_load_i32(p.group_start, gi);
  int s1 = scalar_load_i32(p.group_start, gi + 1);
  int plen = scalar_load_i32(p.prefix_len, gi);
  int pid, mq, mn, qsum;
  load_lanes(s0g, pid, mq, mn, qsum);
  asm volatile("" : "+s"(s0), "+s"(s1), "+s"(plen), "+v"(pid), "+v"(mq), "+v"(mn), "+v"(qsum));
  plen = max(plen, 0) & ~(kBlockSize - 1);  // whole pages, as the partitions read it
  const int members = min(s1 - s0, p.max_members);
  if (plen <= 0 || j0 >= members) return;
  if (s0 != s0g) load_lanes(s0, pid, mq, mn, qsum);
  const int jn = min(kMembers, members - j0);
  const int sf = s0 + j0;
  const int32_t* bt = p.block_table + (size_t)s0 * p.max_blocks;  // the group's shared pages
  // (the last partition runs to the group's prefix end, as in the prefix pass)
  const int pend = min(pp == p.pre_parts - 1 ? plen / kBlockSize : min(pstart + p.pre_pages, plen / kBlockSize),
                       p.max_blocks);
  const bool has_work = pstart < pend;
  const bool fine = !CS::HL && (pend - pstart) * kBlockSize < kFewKeys;
  const int last_page = pend - 1;
  auto page_id = [&](int page) -> int32_t {
    page = min(page, last_page) - pstart;
    return page < 64 ? __builtin_amdgcn_readlane(pid, page) : scalar_load_i32(bt, page + pstart);
  };
  const uint64_t rowmask = __builtin_amdgcn_ballot_w64(lane < jn && mq > 0);
  if (rowmask == 0) return;  // no rows: nothing to write, nothing to count

  Page<F> ring[kPRing];
  if (has_work) issue_page<F>(ring[0], p, page_id(pstart + wave), g, lane);
  __builtin_amdgcn_sched_barrier(0);  // the first page goes out before the row-offset sum
  const int q_row = __builtin_amdgcn_readfirstlane(wave_sum_i32(qsum));
  // This lane's column (the lo copy maps back to the hi one), its member,
  // whether that is live, the last key it may see and the member's row.
  const int pr = lane >> 4;
  const int pc = lane & 15;
  const int col = CS::HL ? (pc & (C - 1)) : pc;
  const int jm = wave * M + col / G;
  const int nm = __shfl(mn, jm, 64);
  const bool has_row = jm < jn && ((rowmask >> jm) & 1);
  const bool live = has_row && nm > 0;
  const int lim[1] = {min(plen, nm) - 1};
  const int qr = has_row ? q_row + __popcll(rowmask & ((1ull << jm) - 1)) : q_row;
  const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(p.q) + ((size_t)qr * p.num_q_heads + g * G + col % G) * 16;
  u32x4_t qv[4];
#pragma unroll
  for (int sg = 0; sg < 4; ++sg) qv[sg] = qp[4 * sg + pr];
  issue_order_barrier();
  if (has_work) {
#pragma unroll
    for (int r = 1; r < kPRing; ++r) issue_page<F>(ring[r], p, page_id(pstart + wave + r * kWaves), g, lane);
  }
  const bool wave_live = __builtin_amdgcn_ballot_w64(live) != 0;

  WaveState<1> st;
  st.m_ref[0] = -INFINITY;
  st.l_lane[0] = 0.f;
  st.r_lane[0] = 0.f;
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) st.o[0][bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sg = 0; sg < 4; ++sg) st.qb[0][sg] = live ? qv[sg] : u32x4_t{0u, 0u, 0u, 0u};

  // Step k: this wave's page pstart + wave + k kWaves (ring slot r = k %
  // kPRing) -> stage r, the slot reloaded for step k + kPRing; barrier; the
  // step's kWaves pages scored (only the last step can be short).  The main
  // loop reissues unconditionally, as the partition path does.
  auto step = [&](Page<F>& b, auto r_c, int k, bool reissue, bool full) {
    constexpr bool second = kTwoStages && decltype(r_c)::value == 1;
    uint8_t (*tk)[kTileBytes] = second ? s_k2 : s_k;
    uint8_t (*tv)[kTileBytes] = second ? s_v2 : s_v;
    stage_page<F>(b, tk[wave], tv[wave], nullptr, nullptr, kBlockSize, lane);
    if (reissue) issue_page<F>(b, p, page_id(pstart + wave + (k + kPRing) * kWaves), g, lane);
    __syncthreads();
    if (wave_live) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int page = pstart + k * kWaves + w;
        if (full || page < pend)
          score_page<G, F, M>(st, tk[w], tv[w], nullptr, nullptr, kBlockSize, p.scale_log2, lane, page * kBlockSize,
                              lim, fine);
      }
    }
    if (!kTwoStages) __syncthreads();
  };
  if (has_work) {
    const int nsteps = (pend - pstart + kWaves - 1) / kWaves;
    static_assert(kPRing == 2, "the steps below are unrolled by the ring depth");
    using R0 = std::integral_constant<int, 0>;
    using R1 = std::integral_constant<int, 1>;
    int k = 0;
    for (; k + 3 < nsteps; k += 2) {
      step(ring[0], R0{}, k, true, true);
      step(ring[1], R1{}, k + 1, true, true);
    }
    // At most 3 steps left: k, k + 1 in the ring (those that exist), k + 2
    // to be issued.
    if (k < nsteps) step(ring[0], R0{}, k, k + 2 < nsteps, false);
    if (k + 1 < nsteps) step(ring[1], R1{}, k + 1, false, false);
    if (k + 2 < nsteps) step(ring[0], R0{}, k + 2, false, false);
    if (kTwoStages) __syncthreads();  // the second stage is the area written next

    // This wave's columns -> LDS (a column's sum is spread over lanes pc +
    // 16 j; the lo copy, lane ^ C, is added when the tile holds one).
    if (wave_live) {
      float l_sum = st.l_lane[0] + other16(st.l_lane[0]);
      l_sum += other_half(l_sum);
      float r_sum = st.r_lane[0] + other16(st.r_lane[0]);
      r_sum += other_half(r_sum);
      f32x4_t o_tot[8];
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o_tot[bb][i] = CS::HL ? st.o[0][bb][i] + __shfl_xor(st.o[0][bb][i], C, 64) : st.o[0][bb][i];
      if (pc < C) {
        if (pr == 0) {
          s_m[wave][pc] = st.m_ref[0];
          s_l[wave][pc] = l_sum;
          s_r[wave][pc] = CS::HL ? l_sum : r_sum;
        }
#pragma unroll
        for (int bb = 0; bb < 8; ++bb) *reinterpret_cast<f32x4_t*>(&s_acc[wave][pc][16 * bb + 4 * pr]) = o_tot[bb];
      }
    }
    __syncthreads();
  }

  // Publish, count and merge with the ordering of the partition path (see
  // there): device-scope stores, their acknowledgement, a barrier, then each
  // member's counter; the merger's loads are device-scope.  Both the
  // publication and the merges take 16 lanes per column of the item, 8 dims
  // each (column wc = wave wc / C's column wc % C), so that a wave covers 4
  // columns at once.
  const size_t rows = (size_t)p.total_q * p.num_q_heads;
  constexpr int kTasks = kWaves * C * 16;
  static_assert(kTasks % kDecodeThreads == 0, "whole rounds of (column, 8 dims) tasks");
  auto row_of = [&](int c, int jc) -> size_t {
    return (size_t)(q_row + __popcll(rowmask & ((1ull << jc) - 1))) * p.num_q_heads + g * G + c % G;
  };
  float* pre_lse = const_cast<float*>(p.pre_lse);
  // (All LDS reads first, then the stores under their conditions: the
  // rounds' reads overlap instead of waiting behind each branch.)
  constexpr int kRounds = kTasks / kDecodeThreads;
  float pm[kRounds], pl[kRounds], prr[kRounds];
  f32x4_t pv0[kRounds], pv1[kRounds];
  bool pub[kRounds];
#pragma unroll
  for (int k = 0; k < kRounds; ++k) {
    const int t = k * kDecodeThreads + (int)threadIdx.x;
    const int wc = t >> 4, d8 = (t & 15) * 8;
    const int w = wc / C, c = wc % C, jc = w * M + c / G;
    const int njc = __shfl(mn, jc & 63, 64);
    pub[k] = jc < jn && ((rowmask >> jc) & 1) && njc > 0;
    pm[k] = has_work ? s_m[w][c] : -INFINITY;
    pl[k] = s_l[w][c];
    prr[k] = s_r[w][c];
    pv0[k] = *reinterpret_cast<const f32x4_t*>(&s_acc[w][c][d8]);
    pv1[k] = *reinterpret_cast<const f32x4_t*>(&s_acc[w][c][d8 + 4]);
  }
#pragma unroll
  for (int k = 0; k < kRounds; ++k) {
    if (!pub[k]) continue;
    const int t = k * kDecodeThreads + (int)threadIdx.x;
    const int wc = t >> 4, d8 = (t & 15) * 8;
    const int c = wc % C, jc = (wc / C) * M + c / G;
    const size_t prow = (size_t)pp * rows + row_of(c, jc);
    float lse = -INFINITY;
    if (pm[k] != -INFINITY) {
      const float inv = 1.f / prr[k];
      float* dst = const_cast<float*>(p.pre_out) + prow * kHeadDim + d8;
      store_coherent_x4(dst, pv0[k] * inv);
      store_coherent_x4(dst + 4, pv1[k] * inv);
      lse = (pm[k] + fast_log2(pl[k])) * kLn2;
    }
    if (d8 == 0) __hip_atomic_store(pre_lse + prow, lse, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // Lane j: member j's own partitions that hold keys, counted and merged
  // besides the prefix partitions (as the member's partitions count them).
  const int mps = partitions_with_keys((mn + kBlockSize - 1) / kBlockSize - plen / kBlockSize, p.num_parts,
                                       p.part_pages);
  wait_vm_stores();
  __syncthreads();
  if ((int)threadIdx.x < jn) {  // wave 0, lane = member
    int last = 0;
    if (((rowmask >> lane) & 1) && mn > 0) {
      int32_t* counter = p.counters + (size_t)(sf + lane) * p.num_kv_heads + g;
      last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             mps + p.pre_parts - 1;
    }
    s_lastm[lane] = last;
  }
  __syncthreads();
#pragma unroll 1
  for (int t = threadIdx.x; t < kTasks; t += kDecodeThreads) {
    const int wc = t >> 4, d8 = (t & 15) * 8;
    const int c = wc % C, jc = (wc / C) * M + c / G;
    const int njc = __shfl(mn, jc & 63, 64);
    const int pjc = __shfl(mps, jc & 63, 64);
    if (!(jc < jn && ((rowmask >> jc) & 1) && njc > 0 && s_lastm[jc])) continue;
    const size_t row = row_of(c, jc);
    MergeState8 ms;
    merge_partials8(ms, p.part_lse + row, p.part_out + row * kHeadDim + d8, pjc, p.pre_lse + row,
                    p.pre_out + row * kHeadDim + d8, p.pre_parts, rows);
    if (ms.M != -INFINITY) {
      const float inv = 1.f / ms.W;
      u32x4_t o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(ms.a[2 * j] * inv, ms.a[2 * j + 1] * inv);
      *reinterpret_cast<u32x4_t*>(p.out + row * kHeadDim + d8) = o;
      if (d8 == 0 && p.lse) p.lse[row] = ms.M + fast_log2(ms.W) * kLn2;
    }
  }
  if ((int)threadIdx.x < jn && s_lastm[lane])
    __hip_atomic_store(p.counters + (size_t)(sf + lane) * p.num_kv_heads + g, 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

#ifndef PA_DECODE_MIN_WGS
#define PA_DECODE_MIN_WGS kDecodeWGsPerCU
#endif
// kPre: the instance of a one-launch prefix-grouped decode, whose first
// pre_items workgroups are prefix items (one token per slot).
template <int G, int F, int M, bool kPre = false>
__global__ __launch_bounds__(kDecodeThreads, (Cols<G, M>::NT > 1 ? 1 : PA_DECODE_MIN_WGS)) void decode_kernel(
    const int32_t* block_table, const int32_t* q_lens, const int32_t* ctx_lens, const int32_t* slot_plen,
    int num_seqs, int num_parts, int part_pages, int max_blocks, int pre_items, int grid, DecodeParams p) {
  // The leading arguments repeat the fields of p that the start needs before
  // its first memory request; they arrive preloaded in scalar registers
  // (kernel-argument preloading), so the page-id requests need not wait for
  // a load of the argument block.
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  using CS = Cols<G, M>;
  constexpr int C = CS::C;
  constexpr int NT = CS::NT;
  static_assert(C <= 32, "at most two 16-column tiles");
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kWaves][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[C][kHeadDim * 2];
  __shared__ __attribute__((aligned(16))) float s_ks[kWaves][kBlockSize * 4];  // q8_0 / q4_0 K scales
  __shared__ __attribute__((aligned(16))) uint8_t s_v[kWaves][kTileBytes];
  __shared__ __attribute__((aligned(16))) float s_vs[kWaves][kBlockSize * 4];    // q8_0 / q4_0 V scales
  __shared__ __attribute__((aligned(16))) float s_acc[kWaves][C][kHeadDim];
  __shared__ float s_m[kWaves][C];
  __shared__ float s_l[kWaves][C];
  __shared__ float s_r[kWaves][C];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The kernel arguments the start needs, fetched together (the compiler
  // would otherwise fetch some of them one round trip later).
  asm volatile("" ::"s"(q_lens), "s"(ctx_lens), "s"(block_table), "s"(slot_plen), "s"(num_parts),
               "s"(pre_items), "s"(num_seqs), "s"(part_pages), "s"(max_blocks), "s"(grid));
  if constexpr (kPre)
    asm volatile("" ::"s"(p.num_groups), "s"(p.group_start), "s"(p.max_members), "s"(p.guess_plen), "s"(p.prefix_len));

  // One launch of prefix-grouped decode: the first pre_items workgroups are
  // prefix items (dispatched first); the rest are the slots' partitions.
  if constexpr (kPre) {
    static_assert(F == kFmtBF16 && M == 1, "prefix items: bf16 pages, one token per slot");
    if ((int)blockIdx.x < pre_items) {
      constexpr int PM = prefix_chunk_members(G);
      constexpr int PC = Cols<G, PM>::C;
      __shared__ __attribute__((aligned(16))) float s_pacc[kWaves][PC][kHeadDim];
      __shared__ float s_pm[kWaves][PC];
      __shared__ float s_pl[kWaves][PC];
      __shared__ float s_pr[kWaves][PC];
      __shared__ int s_lastm[kWaves * PM];
      prefix_item<G, F, PM>(p, xcd_remap(blockIdx.x, pre_items), lane, wave, s_k, s_v, s_pacc, s_pm, s_pl, s_pr,
                            s_lastm);
      return;
    }
  }
  const int wg = xcd_remap(blockIdx.x - pre_items, grid - pre_items);
  const int P = num_parts;
  const int part = wg % P;
  const int rest = wg / P;
  const int seq = rest % num_seqs;
  const int g = rest / num_seqs;

  // Everything the start needs comes in one round trip, issued before the
  // first branch: the lengths, the prefix length, the slot's row offset (a
  // vector load and a wave sum) and the page ids of this wave's first pages
  // as they are when the slot has no prefix (with prefix items: when its
  // prefix is guess_plen keys; checked below, reloaded otherwise).  Lengths
  // and page ids are wave-uniform scalar loads, which do not share the
  // (in-order) vector load counter with the page stream.
  const int32_t* bt = block_table + (size_t)seq * max_blocks;
  const int guess = kPre ? p.guess_plen : 0;
  const int spage0 = guess / kBlockSize + part * part_pages + wave;  // first page for that guess
  const int m = scalar_load_i32(q_lens, seq);
  const int n = scalar_load_i32(ctx_lens, seq);
  // Prefix-grouped decode: this slot's keys start after its shared prefix,
  // whose partials the prefix pass has written; the last partition runs to
  // the slot's end whatever the prefix length.
  int plen = slot_plen ? scalar_load_i32(slot_plen, seq) : 0;
  // (One launch with fewer than 64 groups: the slot's group is the last one
  // starting at or before it, found by the lanes among group_start, and its
  // prefix length is that group's lane of prefix_len.)
  int gsv = 0x7fffffff, plv = 0;
  if constexpr (kPre) {
    if (p.num_groups > 0 && lane <= p.num_groups) gsv = p.group_start[lane];
    if (p.num_groups > 0 && lane < p.num_groups) plv = p.prefix_len[lane];
  }
  int32_t sid[kRing + 1];
#pragma unroll
  for (int k = 0; k <= kRing; ++k) sid[k] = scalar_load_i32(bt, min(spage0 + k * kWaves, max_blocks - 1));
  int qsum = 0;  // this lane's share of the row offset
  for (int i = lane; i < seq; i += 64) qsum += q_lens[i];
  // (Keeps the loads above the branch: the compiler would otherwise sink the
  // ones only the working path uses below it, one round trip later.  The
  // wave sum of the row offset waits until the first page is requested.)
#pragma unroll
  for (int k = 0; k <= kRing; ++k) asm volatile("" : "+s"(sid[k]));
  asm volatile("" : "+v"(qsum));
  if constexpr (kPre) asm volatile("" : "+v"(gsv), "+v"(plv));
  if (m <= 0) return;  // no row: nothing to write, no partial to count
  if (kPre && p.num_groups > 0) {
    const int gsi = __popcll(__builtin_amdgcn_ballot_w64(gsv <= seq)) - 1;
    if (gsi >= 0 && gsi < p.num_groups && seq - __builtin_amdgcn_readlane(gsv, gsi) < p.max_members)
      plen = max(__builtin_amdgcn_readlane(plv, gsi), 0) & ~(kBlockSize - 1);
  }
  const int npages = (n + kBlockSize - 1) / kBlockSize;
  const int npre = (plen > 0 && n > 0) ? p.pre_parts : 0;
  // The slot's partitions that hold keys (the last runs to the slot's end):
  // the others have nothing to add and neither publish nor count, so a short
  // slot of a batch split for its longest costs one round trip per empty
  // partition, and a slot with one such partition writes its result itself.
  // (A prefix pass's partials from the launch before still need a merger:
  // partition 0, even without keys of its own.)
  const int ps = partitions_with_keys(npages - plen / kBlockSize, P, part_pages);
  const int Ps = (npre > 0 && pre_items == 0) ? max(ps, 1) : ps;
  if (part >= Ps) return;
  const int pstart = plen / kBlockSize + part * part_pages;
  const int pend = part == P - 1 ? npages : min(npages, pstart + part_pages);
  const bool has_work = n > 0 && pstart < pend;
  // Few keys: some live row sees between 1 and kFewKeys - 1 of this
  // partition's keys (token t of m sees keys up to n - m + t when causal; a
  // row that sees v keys has min(max(v - start, 0), the partition's keys) of
  // them here).
  bool fine = false;
  if constexpr (!CS::HL) {
    const int base = pstart * kBlockSize;
    fine = n > base && min(max((p.causal ? n - m + 1 : n) - base, 1), min(n, pend * kBlockSize) - base) < kFewKeys;
  }

  const int last_page = pend - 1;
  auto page_id = [&](int page) -> int32_t { return scalar_load_i32(bt, min(page, last_page)); };
  // Page id of this wave's k-th page (clamped to the partition's last page):
  // the early load when it is that page.
  auto first_id = [&](int k) -> int32_t {
    const int page = pstart + wave + k * kWaves;
    return (plen == guess && page <= last_page) ? sid[k] : page_id(page);
  };

  const int h0 = g * G;
  const size_t rows = (size_t)p.total_q * p.num_q_heads;

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
    // The queries of the C columns: 16-byte chunk qc of column c; tokens
    // past the slot's m read its last token (their columns are zeroed below).
    constexpr int kQChunks = (C * 16 + kDecodeThreads - 1) / kDecodeThreads;
    u32x4_t qchunk[kQChunks];
#pragma unroll
    for (int j = 0; j < kQChunks; ++j) {
      const int idx = threadIdx.x + j * kDecodeThreads;
      const int c = min(idx >> 4, C - 1), qc = idx & 15;
      const int tok = min(c / G, m - 1);
      qchunk[j] = reinterpret_cast<const u32x4_t*>(p.q)[((size_t)(q_row + tok) * p.num_q_heads + h0 + c % G) * 16 + qc];
    }
    issue_order_barrier();
#pragma unroll
    for (int r = 1; r < kRing; ++r) issue_page<F>(ring[r], p, first_id(r), g, lane);
    next_id = first_id(kRing);
    // Queries -> LDS, 16-byte chunk qc of column c at slot qc ^ (c % 16).
#pragma unroll
    for (int j = 0; j < kQChunks; ++j) {
      const int idx = threadIdx.x + j * kDecodeThreads;
      const int c = idx >> 4, qc = idx & 15;
      if (c < C) *reinterpret_cast<u32x4_t*>(&s_q[c][(qc ^ (c & 15)) << 4]) = qchunk[j];
    }
    __syncthreads();
  } else {
    q_row = __builtin_amdgcn_readfirstlane(wave_sum_i32(qsum));
  }

  // This lane's column per tile: its real column (the lo copy maps back to
  // the hi one), whether that column is a live token, and the last key it
  // may see (causal: token t of m sees keys up to n - m + t).
  const int pr = lane >> 4;
  const int pc = lane & 15;
  int col[NT];
  bool col_live[NT];
  int lim[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    const int n16 = ct * 16 + pc;
    col[ct] = CS::HL ? (n16 & (C - 1)) : n16;
    const bool in_tile = CS::HL ? n16 < 2 * C : n16 < C;
    col_live[ct] = in_tile && col[ct] / G < m;
    lim[ct] = p.causal ? n - m + col[ct] / G : n - 1;
  }

  if (has_work) {
    WaveState<NT> st;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      st.m_ref[ct] = -INFINITY;
      st.l_lane[ct] = 0.f;
      st.r_lane[ct] = 0.f;
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) st.o[ct][bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // Q^T operand from the staged queries; dead columns get a zero query.
      const int c = min(col[ct], C - 1);
#pragma unroll
      for (int sg = 0; sg < 4; ++sg) {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(&s_q[c][((4 * sg + pr) ^ (c & 15)) << 4]);
        st.qb[ct][sg] = col_live[ct] ? x : u32x4_t{0u, 0u, 0u, 0u};
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
#define PA_CONSUME(RING, K)                                                                            \
  consume_page<G, F, M>(st, RING, sk, sv, sks, svs, valid_of(K), p.scale_log2, lane,                   \
                        (page0 + kWaves * (K)) * kBlockSize, lim, fine)
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

    // Per-wave state -> LDS.  A column's sum is spread over lanes pc + 16 j;
    // its O^T block values are dims 16 b + 4 pr + i, to which the lo column
    // (lane ^ C, since pc < C and C is a power of two) is added when the tile
    // holds one.  FP8's V scale applies here, once.
    const float vs = F == kFmtFP8 ? p.v_scale : 1.f;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      float l_sum = st.l_lane[ct] + other16(st.l_lane[ct]);
      l_sum += other_half(l_sum);
      float r_sum = st.r_lane[ct] + other16(st.r_lane[ct]);
      r_sum += other_half(r_sum);
      f32x4_t o_tot[8];
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o_tot[bb][i] = CS::HL ? st.o[ct][bb][i] + __shfl_xor(st.o[ct][bb][i], C, 64) : st.o[ct][bb][i];
      const int c = ct * 16 + pc;
      if (c < C) {
        if (pr == 0) {
          s_m[wave][c] = st.m_ref[ct];
          s_l[wave][c] = l_sum;
          s_r[wave][c] = CS::HL ? l_sum : r_sum;
        }
#pragma unroll
        for (int bb = 0; bb < 8; ++bb)
          *reinterpret_cast<f32x4_t*>(&s_acc[wave][c][16 * bb + 4 * pr]) = o_tot[bb] * vs;
      }
    }
    __syncthreads();
  }

  // Epilogue: each thread takes J (column, dim pair) outputs: pair i covers
  // dims 2 (i % 64) .. + 2 of column i / 64, token c / G, head h0 + c % G.
  constexpr int J = CS::J;
  float my_o0[J], my_o1[J], my_lse[J];
  int my_c[J], my_d[J];
  bool my_out[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = threadIdx.x + j * kDecodeThreads;
    my_c[j] = min(i >> 6, C - 1);
    my_d[j] = (i & 63) * 2;
    my_out[j] = i < C * 64 && my_c[j] / G < m;
    my_o0[j] = 0.f;
    my_o1[j] = 0.f;
    my_lse[j] = -INFINITY;
    if (has_work && my_out[j]) {
      // Merge the waves (a wave with no page, or whose keys this column
      // cannot see, has max -inf and weight 0).
      const int c = my_c[j], d = my_d[j];
      float Mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) Mx = fmaxf(Mx, s_m[w][c]);
      if (Mx != -INFINITY) {
        float L = 0.f, R = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float sc = fast_exp2(s_m[w][c] - Mx);
          L = fmaf(sc, s_l[w][c], L);
          R = fmaf(sc, s_r[w][c], R);
          const float2 v = *reinterpret_cast<const float2*>(&s_acc[w][c][d]);
          a0 = fmaf(sc, v.x, a0);
          a1 = fmaf(sc, v.y, a1);
        }
        const float inv = 1.f / R;
        my_o0[j] = a0 * inv;
        my_o1[j] = a1 * inv;
        my_lse[j] = (Mx + fast_log2(L)) * kLn2;  // natural log
      }
    }
  }
  auto row_of = [&](int j) -> size_t {
    return (size_t)(q_row + my_c[j] / G) * p.num_q_heads + h0 + my_c[j] % G;
  };

  if (Ps == 1 && (pre_items == 0 || npre == 0)) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (!my_out[j]) continue;
      const size_t row = row_of(j);
      const int d = my_d[j];
      if (npre == 0) {
        if (my_lse[j] != -INFINITY) {
          reinterpret_cast<uint32_t*>(p.out)[(row * kHeadDim + d) / 2] = pack_bf16x2(my_o0[j], my_o1[j]);
          if (d == 0 && p.lse) p.lse[row] = my_lse[j];
        }
        continue;
      }
      // Own result and the prefix pass's partials of this row (written by the
      // previous launch).
      MergeState ms;
      if (has_work) merge_fold(ms, my_lse[j], my_o0[j], my_o1[j]);
      merge_partials(ms, nullptr, nullptr, 0, p.pre_lse + row, p.pre_out + row * kHeadDim + d, npre, rows);
      if (ms.M != -INFINITY) {
        const float inv = 1.f / ms.W;
        reinterpret_cast<uint32_t*>(p.out)[(row * kHeadDim + d) / 2] = pack_bf16x2(ms.a0 * inv, ms.a1 * inv);
        if (d == 0 && p.lse) p.lse[row] = ms.M + fast_log2(ms.W) * kLn2;
      }
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
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (!my_out[j]) continue;
    const size_t prow = (size_t)part * rows + row_of(j);
    if (my_lse[j] != -INFINITY) {
      const uint64_t bits = (uint64_t)__float_as_uint(my_o0[j]) | ((uint64_t)__float_as_uint(my_o1[j]) << 32);
      __hip_atomic_store(part_out64 + (prow * kHeadDim + my_d[j]) / 2, bits, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    if (my_d[j] == 0) __hip_atomic_store(p.part_lse + prow, my_lse[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  wait_vm_stores();
  __syncthreads();
  int32_t* counter = p.counters + (size_t)seq * p.num_kv_heads + g;
  if (threadIdx.x == 0)
    s_last = (__hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              Ps - 1 + (pre_items > 0 ? npre : 0));
  __syncthreads();
  if (!s_last) return;

  // Merge by log-sum-exp weights: this slot's Ps partials and, with a shared
  // prefix, the prefix pass's npre, their loads issued in batches before any
  // is used; a partial with LSE = -inf (empty) gets weight 0 without its
  // output being read.
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (!my_out[j]) continue;
    const size_t row = row_of(j);
    const int d = my_d[j];
    MergeState ms;
    merge_partials<J == 1>(ms, p.part_lse + row, p.part_out + row * kHeadDim + d, Ps, p.pre_lse + row,
                   p.pre_out + row * kHeadDim + d, npre, rows);
    if (ms.M != -INFINITY) {
      const float inv = 1.f / ms.W;
      reinterpret_cast<uint32_t*>(p.out)[(row * kHeadDim + d) / 2] = pack_bf16x2(ms.a0 * inv, ms.a1 * inv);
      if (d == 0 && p.lse) p.lse[row] = ms.M + fast_log2(ms.W) * kLn2;
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

bool decode_supports_group(int group) { return group == 1 || group == 2 || group == 4 || group == 8; }

int decode_tokens_per_slot(int group, int max_q_len) {
  if (!decode_supports_group(group) || max_q_len < 1) return 0;
  for (int mt = 1; mt <= 8; mt *= 2)
    if (max_q_len <= mt) return group * mt <= 32 ? mt : 0;
  return 0;
}

template <int F, int M>
const void* decode_entry(int group) {
  switch (group) {
    case 1: return reinterpret_cast<const void*>(&decode_kernel<1, F, M>);
    case 2: return reinterpret_cast<const void*>(&decode_kernel<2, F, M>);
    case 4: return reinterpret_cast<const void*>(&decode_kernel<4, F, M>);
    case 8:
      if constexpr (M <= 4) return reinterpret_cast<const void*>(&decode_kernel<8, F, M>);
      return nullptr;
  }
  return nullptr;
}

// The kernel's leading scalar arguments, then the whole parameter block.
static hipError_t launch_decode_fn(const void* fn, const DecodeParams& p, unsigned grid, hipStream_t s) {
  DecodeParams arg = p;
  const int32_t *bt = p.block_table, *ql = p.q_lens, *cl = p.ctx_lens, *sp = p.slot_plen;
  int ns = p.num_seqs, np = p.num_parts, pp = p.part_pages, mb = p.max_blocks, pi = p.pre_items;
  int gr = (int)grid;
  void* args[] = {&bt, &ql, &cl, &sp, &ns, &np, &pp, &mb, &pi, &gr, &arg};
  return hipLaunchKernel(fn, dim3(grid), dim3(kDecodeThreads), args, 0, s);
}

hipError_t launch_decode(const DecodeParams& p, int group, int format, int tokens, unsigned grid, hipStream_t s) {
  const void* fn = nullptr;
  if (tokens == 1) {
    switch (format) {
      case kFmtBF16: fn = decode_entry<kFmtBF16, 1>(group); break;
      case kFmtFP8: fn = decode_entry<kFmtFP8, 1>(group); break;
      case kFmtQ8: fn = decode_entry<kFmtQ8, 1>(group); break;
      case kFmtQ4: fn = decode_entry<kFmtQ4, 1>(group); break;
    }
  } else if (format == kFmtBF16) {
    switch (tokens) {
      case 2: fn = decode_entry<kFmtBF16, 2>(group); break;
      case 4: fn = decode_entry<kFmtBF16, 4>(group); break;
      case 8: fn = decode_entry<kFmtBF16, 8>(group); break;
    }
  }
  if (!fn) return hipErrorInvalidValue;
  return launch_decode_fn(fn, p, grid, s);
}

hipError_t launch_decode_prefix(const DecodeParams& p, int group, unsigned grid, hipStream_t s) {
  const void* fn = nullptr;
  switch (group) {
    case 1: fn = reinterpret_cast<const void*>(&decode_kernel<1, kFmtBF16, 1, true>); break;
    case 2: fn = reinterpret_cast<const void*>(&decode_kernel<2, kFmtBF16, 1, true>); break;
    case 4: fn = reinterpret_cast<const void*>(&decode_kernel<4, kFmtBF16, 1, true>); break;
  }
  if (!fn) return hipErrorInvalidValue;
  return launch_decode_fn(fn, p, grid, s);
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
