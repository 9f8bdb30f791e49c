// prefix.hip -- the shared-prefix half of prefix-grouped (cascade) decode.
//
// Requests that share a prefix reference the same physical blocks through
// their block tables (inference-optimisation chapter, section 8.3.2,
// Figs. 8-13 / 8-14).  Decoding them one by one streams those blocks once per
// request.  Here a group's shared pages are read once per KV head for all of
// the group's query rows -- (member, query head) pairs, 40 for ten requests
// with four heads per KV head -- which turns the prefix part into a small
// dense contraction for the matrix cores; each member's private suffix is then
// decoded by the decode kernel, which merges this kernel's partials into its
// own by log-sum-exp (split-KV combine).
//
// Grid: one workgroup per (group, KV head, 64-row tile, prefix partition),
// plus one set-up workgroup that writes every slot's prefix length for the
// suffix pass.  A partition is at most eight 32-key tiles, and a workgroup
// requests all of its tiles at once, straight from memory into LDS
// (global_load_lds_dwordx4: K and V row-major with each row's 16-byte
// chunks permuted by key_swz, 128 KiB), so the pass costs one memory round
// trip rather than one per tile.  Eight waves: wave w takes rows
// 32 (w % 2) .. +32 of the tile and the tiles w / 2, w / 2 + 4 of the
// partition; at the end the quarters merge through LDS, each wave folding
// and storing one 32-dim block.
// S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_bf16 with the
// softmax mostly in-lane; the V^T operand
// comes from the row-major V tile through transposing LDS reads
// (ds_read_b64_tr_b16).  Keys past the partition, the prefix or a member's
// own length get -inf scores.  Output: the normalised fp32 partial and
// natural-log LSE of every live row, or LSE = -inf when the partition has no
// visible key.

#include "device.h"

namespace pa {

namespace {

constexpr int kThreads = 512;
constexpr int kTileKeys = 32;
constexpr int kRowBytes = kHeadDim * 2;           // 256: one key row of K or V
constexpr int kTileBytes = kTileKeys * kRowBytes; // 8 KiB (K or V)
constexpr float kRescaleSlack = 8.0f;             // log2 units
static_assert(kPrefixMaxTiles == 8, "two tiles per key quarter");

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& u) { return __builtin_bit_cast(bf16x8_t, u); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Byte offset of dims d .. of key row `key` in a swizzled K or V tile.
__device__ __forceinline__ int swz(int key, int d) {
  return key * kRowBytes + (((d >> 3) ^ key_swz(key)) << 4) + (d & 7) * 2;
}

// Set-up workgroup: slot_plen[r] = the prefix length of r's group in whole
// pages, for a group's first max_members slots (the rows this kernel
// computes); 0 elsewhere, where the decode pass reads all keys.
__device__ void write_slot_prefix(const PrefixParams& p) {
  for (int r = threadIdx.x; r < p.num_seqs; r += blockDim.x) p.slot_plen[r] = 0;
  __syncthreads();
  for (int k = 0; k < p.num_groups; ++k) {
    const int s0 = p.group_start[k], s1 = min(p.group_start[k + 1], s0 + p.max_members);
    const int plen = max(p.prefix_len[k], 0) & ~15;
    for (int r = s0 + (int)threadIdx.x; r < s1; r += blockDim.x)
      if (r >= 0 && r < p.num_seqs) p.slot_plen[r] = plen;
  }
}

__global__ __launch_bounds__(kThreads, 1) void prefix_kernel(PrefixParams p) {
  // The kernel arguments the start needs, fetched together: the index
  // arithmetic below uses the pinned copies, so the compiler cannot start it
  // on a first batch of arguments and fetch the rest round trips later.
  int grid = gridDim.x, parts = p.pre_parts, row_tiles = p.row_tiles, hkv = p.num_kv_heads, nhq = p.num_q_heads;
  int part_pages = p.part_pages, max_members = p.max_members, num_seqs = p.num_seqs, max_blocks = p.max_blocks;
  asm volatile("" : "+s"(grid), "+s"(parts), "+s"(row_tiles), "+s"(hkv), "+s"(nhq), "+s"(part_pages), "+s"(max_members),
                    "+s"(num_seqs), "+s"(max_blocks)
               : "s"(p.block_table), "s"(p.group_start), "s"(p.prefix_len));
  if (blockIdx.x == grid - 1) {
    write_slot_prefix(p);
    return;
  }
  // [tile][K | V], filled straight from memory; reused for the final merge.
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kPrefixMaxTiles][2][kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & 1;    // row group
  const int kq = wave >> 1;   // key quarter
  const int col = lane & 31;
  const int hh = lane >> 5;

  const int wg = xcd_remap(blockIdx.x, grid - 1);
  const int part = wg % parts;
  int rest = wg / parts;
  const int rt = rest % row_tiles;
  rest /= row_tiles;
  const int g = rest % hkv;
  const int grp = rest / hkv;
  const int G = nhq / hkv;

  // The group's table row is needed before any key can be requested.  The
  // row is guessed (groups of max_members consecutive slots) and its two
  // page ids for this wave's tile are requested together with the group's
  // bounds, saving a memory round trip when the guess holds.
  const int key0 = part * part_pages * kBlockSize;
  const int page0 = (key0 >> 4) + 2 * wave;  // first page of tile `wave`
  const int s_guess = (int)min((long long)grp * max_members, (long long)num_seqs - 1);
  const int32_t* bt_guess = uniform_ptr(p.block_table + (size_t)s_guess * max_blocks);
  int32_t id0 = scalar_load_i32(bt_guess, min(page0, max_blocks - 1));
  int32_t id1 = scalar_load_i32(bt_guess, min(page0 + 1, max_blocks - 1));
  int s0 = scalar_load_i32(p.group_start, grp);
  int s1 = scalar_load_i32(p.group_start, grp + 1);
  int plen = scalar_load_i32(p.prefix_len, grp);
  // (all five in flight before the first is used)
  asm volatile("" : "+s"(id0), "+s"(id1), "+s"(s0), "+s"(s1), "+s"(plen));
  plen &= ~15;  // whole pages, as the decode pass reads it
  const int members = s1 - s0;
  const int rows_here = members * G - rt * 64;  // rows of this tile that exist
  if (rows_here <= 0 || plen <= 0) return;

  // Keys of this partition: pages [part * part_pages, ...) of the prefix.
  const int kv_end = part == p.pre_parts - 1 ? plen : min(plen, (part + 1) * p.part_pages * kBlockSize);
  const int ntiles = kv_end > key0 ? (kv_end - key0 + kTileKeys - 1) / kTileKeys : 0;  // <= 8
  const int32_t* bt = uniform_ptr(p.block_table + (size_t)s0 * p.max_blocks);
  const int last_page = max(0, (kv_end - 1) >> 4);

  // Every tile of the partition goes out at once, before anything that
  // depends on the rows: wave w loads tile w (when it exists), its K and V
  // rows in eight instructions each (lane l fills LDS chunk slot l % 16 of
  // row l / 16 of the instruction's four rows, with the global chunk that
  // the swizzle puts there).  Keys past the partition re-read its last key
  // (finite), whose scores are masked and whose weights are 0.
  if (wave < ntiles) {
    const int t = wave;
    if (s0 != s_guess) {
      id0 = scalar_load_i32(bt, page0);
      id1 = scalar_load_i32(bt, min(page0 + 1, last_page));
    }
    // A tile exists only while its first page is in the partition; past the
    // prefix the second page is the first again.
    if (page0 + 1 > last_page) id1 = id0;
    uint8_t* sk = s_buf[t][0];
    uint8_t* sv = s_buf[t][1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = 4 * j + (lane >> 4);           // LDS row of this lane
      const int key = min(key0 + t * kTileKeys + row, kv_end - 1);
      const int32_t id = (key >> 4) == (key0 >> 4) + 2 * t ? id0 : id1;
      const int c = (lane & 15) ^ key_swz(row);      // global chunk for this slot
      const size_t off = cache_offset(id, g, key & 15, c * 8, p.num_kv_heads);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(p.k + off),
                                       (void __attribute__((address_space(3)))*)(sk + 4 * j * kRowBytes), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(p.v + off),
                                       (void __attribute__((address_space(3)))*)(sv + 4 * j * kRowBytes), 16, 0, 0);
    }
  }

  // This lane's row: member j, query head hq (of KV head g).  The tile's
  // members start at jf; one load per lane gives their query lengths, a
  // wave scan their row offsets.
  const int r_tile = rg * 32 + col;
  const int r = rt * 64 + r_tile;
  const int jf = (rt * 64) / G;
  const int jm = r_tile < rows_here ? r / G - jf : 0;  // 0 .. 63
  const int slot = s0 + jf + jm;
  const int ql = jf + lane < members ? p.q_lens[s0 + jf + lane] : 0;
  const int n_r = p.ctx_lens[slot];
  const int before = q_row_offset(p.q_lens, s0 + jf, lane);
  int incl = ql;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    incl += lane >= d ? y : 0;
  }
  const int m_r = __shfl(ql, jm, 64);
  const int q_off = before + __shfl(incl - ql, jm, 64);
  const int hq = r % G;
  // Rows of slots past the group's first max_members get no prefix (the
  // decode pass attends them to all their keys).
  const bool row_live = r_tile < rows_here && r / G < p.max_members && m_r > 0 && n_r > 0;
  const size_t grow = (size_t)q_off * p.num_q_heads + g * G + hq;  // global (row, head) index
  const int my_limit = min(plen, n_r) - 1;  // last visible key of this row

  // Q^T operand: lane (row, half) holds dims (hh*8 + s)*8 .. +8 for step s.
  u32x4_t qf[8];
  {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(p.q) + (row_live ? grow : 0) * (kHeadDim / 8);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = qp[hh * 8 + s];
  }

  f32x16_t o[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mb][i] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's share of the row sum (fp32 weights)
  float r_run = 0.f;  // the same over the bf16-rounded weights PV uses

  // Tile t of the partition (keys key0 + 32 t ..): S^T = K Q^T, online
  // softmax, O^T += V^T P^T.
  auto compute_tile = [&](int t) {
    const uint8_t* sk = s_buf[t][0];
    const uint8_t* svv = s_buf[t][1];
    u32x4_t kf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = hh * 8 + s;
      kf[s] = *reinterpret_cast<const u32x4_t*>(sk + col * kRowBytes + ((c ^ key_swz(col)) << 4));
    }
    f32x16_t st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[s]), as_bf16x8(qf[s]), st, 0, 0, 0);
    const int kbase = key0 + t * kTileKeys + 4 * hh;
    float sv[16];
    float mloc = -INFINITY;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int key = kbase + 8 * a + b;
        const float x = (key < kv_end && key <= my_limit) ? st[4 * a + b] * p.scale_log2 : -INFINITY;
        sv[4 * a + b] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, other_half(mloc));
    const bool raise = mloc > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = fast_exp2(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
      l_run *= alpha;
      r_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[mb][i] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = fast_exp2(sv[i] - m_use);
      lsum += sv[i];
    }
    l_run += lsum;
    // P^T operand for key steps 0 and 1: keys 16 ks + 4 hh + 0..3 and
    // 16 ks + 8 + 4 hh + 0..3.  The output is normalised by the sum of these
    // rounded weights, the LSE by the sum of the fp32 ones.
    u32x4_t pf[2];
    float rsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      pf[ks][0] = pack_bf16x2(sv[8 * ks + 0], sv[8 * ks + 1]);
      pf[ks][1] = pack_bf16x2(sv[8 * ks + 2], sv[8 * ks + 3]);
      pf[ks][2] = pack_bf16x2(sv[8 * ks + 4], sv[8 * ks + 5]);
      pf[ks][3] = pack_bf16x2(sv[8 * ks + 6], sv[8 * ks + 7]);
#pragma unroll
      for (int w = 0; w < 4; ++w) rsum += bf16_lo(pf[ks][w]) + bf16_hi(pf[ks][w]);
    }
    r_run += rsum;
    // V^T operand (lane: dim 32 mb + l % 32, the same keys) from the
    // row-major V tile through transposing reads: in each 16-lane group, lane
    // a points at 4 dims of key a / 4 and lane i receives dim i of the four
    // keys.  Key + 16 is 4096 bytes further with the same swizzle.
    const int grp16 = lane >> 4;
    const int a16 = lane & 15;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        s16x4_t v2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
          v2[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(
              svv + ks * 4096 + swz(8 * e + 4 * hh + (a16 >> 2), mb * 32 + (grp16 & 1) * 16 + 4 * (a16 & 3))));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, v2[0]);
        const u32x2_t h2 = __builtin_bit_cast(u32x2_t, v2[1]);
        const u32x4_t vf = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[ks]), o[mb], 0, 0, 0);
      }
  };

  // Every wave's tile loads (and the query) land, then one barrier puts the
  // whole partition in LDS for every wave.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), other counters unconstrained
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPrefixMaxTiles / 4; ++i)
    if (kq + 4 * i < ntiles) compute_tile(kq + 4 * i);
  __syncthreads();  // all tiles read before the area is reused

  // Merge the four key quarters of each row group through LDS (the tile
  // area, free now) behind one barrier: wave (rg, kq) folds output block
  // kq (dims 32 kq .. +32) of its rows from the other three quarters and
  // stores it, so the folding and the stores are spread over all eight
  // waves.  Region layout [block][row group][other quarter][chunk of 4
  // floats][lane]: 16-byte accesses by consecutive lanes.
  constexpr int kSlot = 4 * 64;  // float4s per (block, row group, quarter)
  float4* xacc = reinterpret_cast<float4*>(&s_buf[0][0][0]);
  float4* xml = xacc + 4 * 2 * 3 * kSlot;  // [row group][quarter][lane]: (m, l, rounded l)
  static_assert(4 * 2 * 3 * kSlot * sizeof(float4) + 2 * 4 * 64 * sizeof(float4) <= sizeof(s_buf),
                "merge buffer exceeds the tile area");
  xml[(rg * 4 + kq) * 64 + lane] = make_float4(m_run, l_run, r_run, 0.f);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (mb == kq) continue;
    float4* dst = xacc + ((mb * 2 + rg) * 3 + (kq < mb ? kq : kq - 1)) * kSlot;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      dst[c * 64 + lane] = make_float4(o[mb][4 * c], o[mb][4 * c + 1], o[mb][4 * c + 2], o[mb][4 * c + 3]);
  }
  __syncthreads();
  if (!row_live) return;  // both lanes of a row leave together

  float M = -INFINITY;
  float4 ml[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ml[q] = xml[(rg * 4 + q) * 64 + lane];
    M = fmaxf(M, ml[q].x);
  }
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float aw[4];
  float l = 0.f, lr = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    aw[q] = fast_exp2(ml[q].x - Mu);
    l = fmaf(ml[q].y, aw[q], l);
    lr = fmaf(ml[q].z, aw[q], lr);
  }
  const float l_tot = l + __shfl_xor(l, 32, 64);
  const float r_tot = lr + __shfl_xor(lr, 32, 64);
  const size_t rows = (size_t)p.total_q * p.num_q_heads;
  if (kq == 0 && hh == 0) p.pre_lse[(size_t)part * rows + grow] = l_tot > 0.f ? (M + fast_log2(l_tot)) * kLn2 : -INFINITY;
  if (l_tot == 0.f) return;  // no visible key in this partition: the output is never read
  const float inv = 1.f / r_tot;
  float* orow = p.pre_out + ((size_t)part * rows + grow) * kHeadDim;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (mb != kq) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float x0 = o[mb][4 * c] * aw[mb], x1 = o[mb][4 * c + 1] * aw[mb];
      float x2 = o[mb][4 * c + 2] * aw[mb], x3 = o[mb][4 * c + 3] * aw[mb];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q == mb) continue;
        const float4 y = xacc[((mb * 2 + rg) * 3 + (q < mb ? q : q - 1)) * kSlot + c * 64 + lane];
        x0 = fmaf(y.x, aw[q], x0);
        x1 = fmaf(y.y, aw[q], x1);
        x2 = fmaf(y.z, aw[q], x2);
        x3 = fmaf(y.w, aw[q], x3);
      }
      *reinterpret_cast<float4*>(orow + mb * 32 + 8 * c + 4 * hh) = make_float4(x0 * inv, x1 * inv, x2 * inv, x3 * inv);
    }
  }
}

}  // namespace

hipError_t launch_prefix(const PrefixParams& p, unsigned grid, hipStream_t s) {
  PrefixParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&prefix_kernel), dim3(grid + 1), dim3(kThreads), args, 0, s);
}

}  // namespace pa
