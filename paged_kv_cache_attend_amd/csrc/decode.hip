// decode.hip -- paged decode attention, one new token per slot, split-KV.
//
// What it computes: for each active slot and query head, softmax attention of
// the one new query row over the slot's n cached keys, gathered through the
// block table (inference-optimisation chapter, section 8.3.1, Fig. 8-10).
// Decode reads every key and value of every request once per step, so the
// kernel is bound by HBM bandwidth (same chapter, section 8.2.1): per key and
// KV head it moves 512 bytes (K and V, 128 bf16 each) and does 4 FLOP per
// byte for a group of four query heads.  Everything is arranged around
// streaming those bytes:
//
// * Grid: one 256-thread workgroup per (KV head, slot, partition), where a
//   partition is a run of `part_pages` 16-token pages (split-KV, "flash
//   decoding"): short batches still put enough workgroups on 256 CUs.  The
//   hardware id is remapped so each XCD owns a contiguous range of
//   (KV head, slot) pairs -- slots that share prefix pages read them under
//   one L2.
// * Each of the 4 waves takes every 4th page of the partition.  A page of one
//   KV head is a contiguous 4 KiB K tile and a 4 KiB V tile; a wave loads
//   each with four 128-bit loads per lane (fully coalesced 1 KiB per
//   instruction) and issues the next page's loads before working on the
//   current one.  The block table entries of the partition are read once into
//   lanes and broadcast with readlane.
// * Scores: the K tile goes to LDS (XOR-swizzled 16-byte chunks, conflict
//   free); lane (token t = lane % 16, head h = lane / 16) forms the full
//   128-long dot product of its query head with key t using bf16 dot2
//   instructions against the query held in registers.  The whole group of
//   query heads thus shares one read of each key.
// * Online softmax in the log2 domain (scale * log2 e folded in): running max
//   per head, row max over the 16 tokens with DPP row rotations, per-lane
//   running sums reduced once at the end.
// * PV: the V tile stays in registers in its load layout (lane holds 8 dims of
//   tokens 4k + lane/16); the probabilities reach that layout through a tiny
//   LDS buffer; fp32 FMA accumulation.
// * Epilogue: the four waves' (max, sum, acc) merge through LDS.  With one
//   partition the workgroup writes bf16 out and the LSE; otherwise it writes
//   the normalised fp32 partial and its LSE for the combine kernel.  Empty
//   partitions (and slots with no keys) write LSE = -inf partials so the merge
//   gives them zero weight; with one partition they write nothing at all.

#include "device.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kTileBytes = kBlockSize * kHeadDim * 2;  // 4 KiB

template <int G>
__global__ __launch_bounds__(kDecodeThreads, 2) void decode_kernel(DecodeParams p) {
  static_assert(G == 1 || G == 2 || G == 4, "group size");
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kWaves][kTileBytes];
  __shared__ __attribute__((aligned(16))) float s_p[kWaves][kBlockSize][4];
  __shared__ __attribute__((aligned(16))) float s_alpha[kWaves][4];
  __shared__ __attribute__((aligned(16))) float s_acc[kWaves][4][G][kHeadDim];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int P = p.num_parts;
  const int part = wg % P;
  const int rest = wg / P;
  const int seq = rest % p.num_seqs;
  const int g = rest / p.num_seqs;

  const int m = p.q_lens[seq];
  if (m <= 0) return;  // no row: nothing to write
  const int n = p.ctx_lens[seq];
  const int q_row = q_row_offset(p.q_lens, seq, lane);
  const int h0 = g * G;
  const int npages = (n + kBlockSize - 1) / kBlockSize;
  const int pstart = part * p.part_pages;
  const int pend = min(npages, pstart + p.part_pages);
  const size_t rows = (size_t)p.total_q * p.num_q_heads;

  if (n <= 0 || pstart >= pend) {
    // zombie slot or empty partition
    if (P > 1 && threadIdx.x < G) {
      p.part_lse[(size_t)part * rows + (size_t)q_row * p.num_q_heads + h0 + threadIdx.x] = -INFINITY;
    }
    return;
  }

  // Lane roles.  Score layout: token tq, head hq.  Load / PV layout: tokens
  // 4k + pr (k = 0..3), dims 8*pc .. 8*pc + 7.
  const int tq = lane & 15;
  const int hq = (lane >> 4) % G;
  const int pr = lane >> 4;
  const int pc = lane & 15;

  // Query of head h0 + hq, 128 bf16 = 16 x 16 bytes, held in registers.
  uint4 qv[16];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(p.q) +
                      ((size_t)q_row * p.num_q_heads + h0 + hq) * (kHeadDim / 8);
#pragma unroll
    for (int i = 0; i < 16; ++i) qv[i] = qp[i];
  }

  // Block table entries of this partition, one per lane, 64 at a time.
  const int32_t* bt = p.block_table + (size_t)seq * p.max_blocks;
  int bt_base = pstart;
  int bt_lane = (pstart + lane < pend) ? bt[pstart + lane] : 0;

  const uint4* kpool = reinterpret_cast<const uint4*>(p.k);
  const uint4* vpool = reinterpret_cast<const uint4*>(p.v);

  uint4 kn[4], vn[4];
  auto load_page = [&](int page) {
    if (page - bt_base >= 64) {
      bt_base += 64;
      bt_lane = (bt_base + lane < pend) ? bt[bt_base + lane] : 0;
    }
    const int phys = __builtin_amdgcn_readlane(bt_lane, page - bt_base);
    const size_t base = tile_index(phys, g, p.num_kv_heads) * (kTileBytes / 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) kn[k] = kpool[base + k * 64 + lane];
#pragma unroll
    for (int k = 0; k < 4; ++k) vn[k] = vpool[base + k * 64 + lane];
  };

  float m_run = -INFINITY;  // running max (log2 domain) of head hq
  float l_lane = 0.f;       // running sum of this lane's probabilities
  float acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;

  uint8_t* sk = s_k[wave];
  int page = pstart + wave;
  if (page < pend) load_page(page);

  for (; page < pend; page += kWaves) {
    // K tile -> LDS.  Row t (256 B) keeps its 16-byte chunk c at slot c ^ t.
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = 4 * k + pr;
      *reinterpret_cast<uint4*>(sk + t * 256 + ((pc ^ t) << 4)) = kn[k];
    }
    uint4 vc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) vc[k] = vn[k];
    const int valid = min(kBlockSize, n - page * kBlockSize);
    if (page + kWaves < pend) load_page(page + kWaves);
    wave_lds_sync();

    // Score of (token tq, head hq).
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 kk = *reinterpret_cast<const uint4*>(sk + tq * 256 + ((i ^ tq) << 4));
      s = dot8_bf16(qv[i], kk, s);
    }
    const float sl = (tq < valid) ? s * p.scale_log2 : -INFINITY;
    const float tmax = row16_max(sl);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    const float pw = fast_exp2(sl - m_new);
    l_lane = l_lane * alpha + pw;
    m_run = m_new;
    if ((lane >> 4) < G) {
      s_p[wave][tq][hq] = pw;
      if (tq == 0) s_alpha[wave][hq] = alpha;
    }
    wave_lds_sync();

    // PV in the load layout.
    float al[G];
#pragma unroll
    for (int h = 0; h < G; ++h) al[h] = s_alpha[wave][h];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[h][j] *= al[h];
    if (valid < kBlockSize) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (4 * k + pr >= valid) vc[k] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = 4 * k + pr;
      const float4 pt = *reinterpret_cast<const float4*>(&s_p[wave][t][0]);
      const float pk[4] = {pt.x, pt.y, pt.z, pt.w};
      float vf[8];
      vf[0] = bf16_lo(vc[k].x); vf[1] = bf16_hi(vc[k].x);
      vf[2] = bf16_lo(vc[k].y); vf[3] = bf16_hi(vc[k].y);
      vf[4] = bf16_lo(vc[k].z); vf[5] = bf16_hi(vc[k].z);
      vf[6] = bf16_lo(vc[k].w); vf[7] = bf16_hi(vc[k].w);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(pk[h], vf[j], acc[h][j]);
    }
  }

  // Per-wave state -> LDS.
  const float l_sum = row16_sum(l_lane);
  if ((lane >> 4) < G && tq == 0) {
    s_m[wave][hq] = m_run;
    s_l[wave][hq] = l_sum;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float4* dst = reinterpret_cast<float4*>(&s_acc[wave][pr][h][pc * 8]);
    dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
    dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
  }
  __syncthreads();

  // Merge the waves: two adjacent dims of one head per thread.
  for (int o = threadIdx.x * 2; o < G * kHeadDim; o += kDecodeThreads * 2) {
    const int h = o / kHeadDim;
    const int d = o % kHeadDim;
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
        x0 += s_acc[w][r][h][d];
        x1 += s_acc[w][r][h][d + 1];
      }
      a0 = fmaf(sc, x0, a0);
      a1 = fmaf(sc, x1, a1);
    }
    const float inv = 1.f / L;
    const float o0 = a0 * inv, o1 = a1 * inv;
    const float lse = (M + fast_log2(L)) * kLn2;
    const size_t row = (size_t)q_row * p.num_q_heads + h0 + h;
    if (P == 1) {
      reinterpret_cast<uint32_t*>(p.out)[(row * kHeadDim + d) / 2] = pack_bf16x2(o0, o1);
      if (d == 0 && p.lse) p.lse[row] = lse;
    } else {
      const size_t prow = (size_t)part * rows + row;
      reinterpret_cast<float2*>(p.part_out)[(prow * kHeadDim + d) / 2] = make_float2(o0, o1);
      if (d == 0) p.part_lse[prow] = lse;
    }
  }
}

}  // namespace

bool decode_supports_group(int group) { return group == 1 || group == 2 || group == 4; }

hipError_t launch_decode(const DecodeParams& p, int group, unsigned grid, hipStream_t s) {
  switch (group) {
    case 1: hipLaunchKernelGGL(decode_kernel<1>, dim3(grid), dim3(kDecodeThreads), 0, s, p); break;
    case 2: hipLaunchKernelGGL(decode_kernel<2>, dim3(grid), dim3(kDecodeThreads), 0, s, p); break;
    case 4: hipLaunchKernelGGL(decode_kernel<4>, dim3(grid), dim3(kDecodeThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
