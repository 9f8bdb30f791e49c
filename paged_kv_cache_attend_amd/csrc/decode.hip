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
//   Group scales multiply the per-group partial scores of K and the PV
//   weights of V; FP8's per-cache K scale is folded into the softmax scale
//   and its V scale into the weights.
// * Scores: the K tile goes to LDS (XOR-swizzled 16-byte chunks, conflict
//   free); lane (token t = lane % 16, head h = lane / 16) forms the 128-long
//   dot product of its query head with key t using v_dot2c_f32_bf16 against
//   the query staged in LDS, so the group of query heads shares one read of
//   each key.
// * Online softmax in the log2 domain (scale * log2 e folded in): per-head
//   row max over the 16 tokens with DPP row rotations; the reference max is
//   only raised (and the accumulators rescaled) when a score exceeds it by
//   more than 2^8, which keeps every weight <= 256 and skips the rescale on
//   almost every page.
// * PV: the V tile stays in registers in its load layout (lane holds 8 dims
//   of tokens 4k + lane/16).  Weights reach that layout through a small LDS
//   buffer, are rounded to bf16 and paired by token; v_perm pairs the V
//   values the same way, and v_dot2c_f32_bf16 accumulates two tokens per
//   instruction in fp32.
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
    u32x4_t r;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      r[w] = pack_bf16x2((float)(int)((c >> (8 * w)) & 15u) - 8.f, (float)(int)((c >> (8 * w + 4)) & 15u) - 8.f);
    return r;
  }
}

template <int G>
struct WaveState {
  float m_ref;      // reference max (log2 domain) of head hq, uniform over its row
  float l_lane;     // this lane's running sum of weights
  float acc[G][8];  // PV layout accumulators
};

// One page: scores, online softmax, PV.  `sk` is this wave's 4 KiB LDS tile
// (bf16), `sks` its 16 x 4 K group scales, `sp` its 16 x 4 weight buffer,
// `salpha` its 4 rescale factors.
template <int G, int F>
__device__ __forceinline__ void consume_page(WaveState<G>& st, Page<F>& b, const uint8_t* sq,
                                             uint8_t* sk, float* sks, float* sp, float* salpha,
                                             int valid, float scale_log2, float v_scale, int lane) {
  const int tq = lane & 15;
  const int hq = (lane >> 4) % G;
  const int pr = lane >> 4;
  const int pc = lane & 15;
  constexpr bool kGrouped = F == kFmtQ8 || F == kFmtQ4;

  // K tile -> LDS as bf16.  Row t (256 B) keeps its 16-byte chunk c at slot c ^ t.
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = 4 * k + pr;
    *reinterpret_cast<u32x4_t*>(sk + t * 256 + ((pc ^ t) << 4)) = chunk_to_bf16<F>(b.k[k]);
  }
  if constexpr (kGrouped) sks[lane] = half_bits_to_float(b.ks);  // [token][group]
  wave_lds_sync();

  // Score of (token tq, head hq).  The query of head h keeps its 16-byte chunk
  // c at slot c ^ h, so the four heads' broadcast reads use different banks.
  float s = 0.f;
  if constexpr (kGrouped) {
#pragma unroll
    for (int gr = 0; gr < 4; ++gr) {
      float sg = 0.f;
#pragma unroll
      for (int i = 4 * gr; i < 4 * gr + 4; ++i) {
        const u32x4_t kk = *reinterpret_cast<const u32x4_t*>(sk + tq * 256 + ((i ^ tq) << 4));
        const u32x4_t qq = *reinterpret_cast<const u32x4_t*>(sq + hq * 256 + ((i ^ hq) << 4));
        sg = dot8_bf16(qq, kk, sg);
      }
      s = fmaf(sks[tq * 4 + gr], sg, s);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const u32x4_t kk = *reinterpret_cast<const u32x4_t*>(sk + tq * 256 + ((i ^ tq) << 4));
      const u32x4_t qq = *reinterpret_cast<const u32x4_t*>(sq + hq * 256 + ((i ^ hq) << 4));
      s = dot8_bf16(qq, kk, s);
    }
  }
  const float sl = (tq < valid) ? s * scale_log2 : -INFINITY;
  const float tmax = row16_max(sl);
  const bool raise = tmax > st.m_ref + kRescaleSlack;
  const bool any_raise = __builtin_amdgcn_ballot_w64(raise) != 0;
  float alpha = 1.f;
  if (any_raise) {
    const float m_new = fmaxf(st.m_ref, tmax);
    alpha = fast_exp2(st.m_ref - m_new);  // 0 on the first page (m_ref = -inf)
    st.m_ref = m_new;
    st.l_lane *= alpha;
  }
  const float w = fast_exp2(sl - st.m_ref);
  st.l_lane += w;
  if ((lane >> 4) < G) {
    sp[tq * 4 + hq] = w;
    if (tq == 0) salpha[hq] = alpha;
  }
  wave_lds_sync();

  if (any_raise) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a = salpha[h];
#pragma unroll
      for (int j = 0; j < 8; ++j) st.acc[h][j] *= a;
    }
  }

  // V scale of this lane's tokens t_k = 4k + pr (its group pc / 4); zero
  // past the end, where the stored scale may be anything.
  float vsc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float x = 1.f;
    // chunk 4 k + pr's group scale sits in lane 4 (4 k + pr) + pc / 4
    if constexpr (kGrouped) x = half_bits_to_float((uint32_t)__shfl((int)b.vs, 16 * k + 4 * pr + (pc >> 2), 64));
    if constexpr (F == kFmtFP8) x = v_scale;
    vsc[k] = (4 * k + pr < valid) ? x : 0.f;
  }

  // Weights of this lane's tokens, all heads, as bf16 pairs (t0, t1) and
  // (t2, t3), each times its V scale.
  uint32_t w01[G], w23[G];
  {
    const float4 p0 = *reinterpret_cast<const float4*>(sp + (0 + pr) * 4);
    const float4 p1 = *reinterpret_cast<const float4*>(sp + (4 + pr) * 4);
    const float4 p2 = *reinterpret_cast<const float4*>(sp + (8 + pr) * 4);
    const float4 p3 = *reinterpret_cast<const float4*>(sp + (12 + pr) * 4);
    const float a0[4] = {p0.x, p0.y, p0.z, p0.w};
    const float a1[4] = {p1.x, p1.y, p1.z, p1.w};
    const float a2[4] = {p2.x, p2.y, p2.z, p2.w};
    const float a3[4] = {p3.x, p3.y, p3.z, p3.w};
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if constexpr (F == kFmtBF16) {
        w01[h] = pack_bf16x2(a0[h], a1[h]);
        w23[h] = pack_bf16x2(a2[h], a3[h]);
      } else {
        w01[h] = pack_bf16x2(a0[h] * vsc[0], a1[h] * vsc[1]);
        w23[h] = pack_bf16x2(a2[h] * vsc[2], a3[h] * vsc[3]);
      }
    }
  }

  // V as bf16; tokens past the end hold anything (NaN included): zero them.
  u32x4_t vb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) vb[k] = chunk_to_bf16<F>(b.v[k]);
  if (valid < kBlockSize) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (4 * k + pr >= valid) vb[k] = u32x4_t{0u, 0u, 0u, 0u};
  }
  // V pairs: dims (2w, 2w+1) of tokens (t0, t1) and (t2, t3).
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    const uint32_t lo01 = __builtin_amdgcn_perm(vb[1][wd], vb[0][wd], 0x05040100u);
    const uint32_t hi01 = __builtin_amdgcn_perm(vb[1][wd], vb[0][wd], 0x07060302u);
    const uint32_t lo23 = __builtin_amdgcn_perm(vb[3][wd], vb[2][wd], 0x05040100u);
    const uint32_t hi23 = __builtin_amdgcn_perm(vb[3][wd], vb[2][wd], 0x07060302u);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      st.acc[h][2 * wd] = dot2_bf16(w01[h], lo01, st.acc[h][2 * wd]);
      st.acc[h][2 * wd] = dot2_bf16(w23[h], lo23, st.acc[h][2 * wd]);
      st.acc[h][2 * wd + 1] = dot2_bf16(w01[h], hi01, st.acc[h][2 * wd + 1]);
      st.acc[h][2 * wd + 1] = dot2_bf16(w23[h], hi23, st.acc[h][2 * wd + 1]);
    }
  }
}

template <int G, int F>
__global__ __launch_bounds__(kDecodeThreads, kDecodeWGsPerCU) void decode_kernel(DecodeParams p) {
  static_assert(G == 1 || G == 2 || G == 4, "group size");
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kWaves][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[G][kHeadDim * 2];
  __shared__ __attribute__((aligned(16))) float s_p[kWaves][kBlockSize * 4];
  __shared__ __attribute__((aligned(16))) float s_alpha[kWaves][4];
  __shared__ __attribute__((aligned(16))) float s_ks[kWaves][kBlockSize * 4];  // q8_0 / q4_0 K scales
  __shared__ __attribute__((aligned(16))) float s_acc[kWaves][4][G][kHeadDim];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ int s_last;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The kernel arguments the start needs, fetched together (the compiler
  // would otherwise fetch some of them one round trip later).
  asm volatile("" ::"s"(p.q_lens), "s"(p.ctx_lens), "s"(p.block_table), "s"(p.slot_plen), "s"(p.num_parts),
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
  int32_t sid[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) sid[k] = scalar_load_i32(bt, min(spage0 + k * kWaves, p.max_blocks - 1));
  int qsum = 0;  // this lane's share of the row offset
  for (int i = lane; i < seq; i += 64) qsum += p.q_lens[i];
  // (Keeps the loads above the branch: the compiler would otherwise sink the
  // ones only the working path uses below it, one round trip later.  The
  // wave sum of the row offset waits until the first page is requested.)
  asm volatile("" : "+s"(sid[0]), "+s"(sid[1]), "+s"(sid[2]), "+s"(sid[3]), "+v"(qsum));
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
  // wait only covers that first page, needed next anyway), the second and
  // third pages.  Every load here is unconditional within the workgroup-
  // uniform has_work branch -- a wave with fewer than three pages re-reads a
  // valid page -- so the load counter's waits stay exact.
  Page<F> ring0, ring1, ring2;
  const int page0 = pstart + wave;
  const int cnt = (has_work && page0 < pend) ? (pend - page0 + kWaves - 1) / kWaves : 0;
  int32_t next_id = 0;
  int q_row;
  if (has_work) {
    issue_page<F>(ring0, p, first_id(0), g, lane);
    __builtin_amdgcn_sched_barrier(0);  // the first page goes out before the row-offset sum
    q_row = __builtin_amdgcn_readfirstlane(wave_sum_i32(qsum));
    const int qh = (threadIdx.x >> 4) % G, qc = threadIdx.x & 15;
    const u32x4_t qchunk =
        reinterpret_cast<const u32x4_t*>(p.q)[((size_t)q_row * p.num_q_heads + h0 + qh) * 16 + qc];
    issue_order_barrier();
    issue_page<F>(ring1, p, first_id(1), g, lane);
    issue_page<F>(ring2, p, first_id(2), g, lane);
    next_id = first_id(3);
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
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) st.acc[h][j] = 0.f;

    uint8_t* sk = s_k[wave];
    float* sp = s_p[wave];
    float* sa = s_alpha[wave];
    float* sks = s_ks[wave];
    const uint8_t* sq = &s_q[0][0];
    // This wave's pages are page0 + 4k for k < cnt; page k lives in ring k % 3.
    // The main loop reissues unconditionally, so the (in-order) load counter
    // sees the same pattern on every trip and each wait leaves the other two
    // pages in flight; the last pages are peeled off.
    auto valid_of = [&](int k) { return min(kBlockSize, n - (page0 + kWaves * k) * kBlockSize); };
#define PA_CONSUME(RING, K) \
  consume_page<G, F>(st, RING, sq, sk, sks, sp, sa, valid_of(K), p.scale_log2, p.v_scale, lane)
#define PA_REISSUE(RING, K)                                          \
  {                                                                  \
    issue_page<F>(RING, p, next_id, g, lane);                        \
    next_id = page_id(page0 + kWaves * ((K) + 1));                   \
  }
    int k = 0;
    for (; k + 5 < cnt; k += 3) {
      PA_CONSUME(ring0, k);
      PA_REISSUE(ring0, k + 3);
      PA_CONSUME(ring1, k + 1);
      PA_REISSUE(ring1, k + 4);
      PA_CONSUME(ring2, k + 2);
      PA_REISSUE(ring2, k + 5);
    }
    // At most five pages left: k, k+1, k+2 in rings 0, 1, 2 (if they exist);
    // k+3 and k+4 still to be issued into rings 0 and 1.
    if (k < cnt) {
      PA_CONSUME(ring0, k);
      if (k + 3 < cnt) PA_REISSUE(ring0, k + 3);
      if (k + 1 < cnt) {
        PA_CONSUME(ring1, k + 1);
        if (k + 4 < cnt) PA_REISSUE(ring1, k + 4);
      }
      if (k + 2 < cnt) PA_CONSUME(ring2, k + 2);
      if (k + 3 < cnt) PA_CONSUME(ring0, k + 3);
      if (k + 4 < cnt) PA_CONSUME(ring1, k + 4);
    }
#undef PA_CONSUME
#undef PA_REISSUE

    // Per-wave state -> LDS.
    const int tq = lane & 15;
    const int hq = (lane >> 4) % G;
    const int pr = lane >> 4;
    const int pc = lane & 15;
    const float l_sum = row16_sum(st.l_lane);
    if ((lane >> 4) < G && tq == 0) {
      s_m[wave][hq] = st.m_ref;
      s_l[wave][hq] = l_sum;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(&s_acc[wave][pr][h][pc * 8]);
      dst[0] = make_float4(st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]);
      dst[1] = make_float4(st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]);
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
        float x0 = 0.f, x1 = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float2 v = *reinterpret_cast<const float2*>(&s_acc[w][r][h][d]);
          x0 += v.x;
          x1 += v.y;
        }
        a0 = fmaf(sc, x0, a0);
        a1 = fmaf(sc, x1, a1);
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
  // and the counter are exchanged with relaxed device-scope atomics, which
  // the compiler emits as cache-coherent (sc1) loads and stores; each thread
  // waits for its partial stores to complete before the workgroup bumps the
  // counter.  This avoids device-scope fences, which on this chip write back
  // and invalidate the whole L2 of the XCD.
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
