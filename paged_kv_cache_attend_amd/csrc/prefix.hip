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
// suffix pass.  Eight waves: wave w takes rows 32 (w % 2) .. +32 of the tile
// and a quarter (w / 2) of the partition's 32-key tiles; the quarters merge
// through LDS at the end.  Per tile: the quarter's 128 threads load K and V
// through the group leader's block-table row two tiles ahead into registers,
// store K row-major (swizzled) and V transposed (68-byte rows) to a
// double-buffered LDS area; S^T = K Q^T and O^T += V^T P^T run on
// v_mfma_f32_32x32x16_bf16 with the softmax mostly in-lane.  Keys past the
// partition, the prefix or a member's own length get -inf scores.  Output:
// the normalised fp32 partial and natural-log LSE of every live row, or
// LSE = -inf when the partition has no visible key.

#include "device.h"

namespace pa {

namespace {

constexpr int kThreads = 512;
constexpr int kQuarterThreads = 128;
constexpr int kTileKeys = 32;
constexpr int kKRowBytes = kHeadDim * 2;          // 256
constexpr int kVtRowBytes = kTileKeys * 2 + 4;    // 68: padded dim-major row (17 words)
constexpr int kKBytes = kTileKeys * kKRowBytes;   // 8 KiB
constexpr int kVtBytes = kHeadDim * kVtRowBytes;  // 8.5 KiB
constexpr int kStageBytes = kKBytes + kVtBytes;
constexpr float kRescaleSlack = 8.0f;             // log2 units

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& u) { return __builtin_bit_cast(bf16x8_t, u); }

// A loader thread holds chunk `lc` (dims 8 lc .. +8) of keys 4 lq .. 4 lq + 3
// of the tile, for K and for V: each load instruction of a wave reads whole
// 256-byte key rows.
struct TileRegs {
  u32x4_t k[4];
  u32x4_t v[4];
};

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
  if (blockIdx.x == gridDim.x - 1) {
    write_slot_prefix(p);
    return;
  }
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[4][2][kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & 1;    // row group
  const int kq = wave >> 1;   // key quarter
  const int lt = tid & (kQuarterThreads - 1);
  const int col = lane & 31;
  const int hh = lane >> 5;

  const int wg = xcd_remap(blockIdx.x, gridDim.x - 1);
  const int part = wg % p.pre_parts;
  int rest = wg / p.pre_parts;
  const int rt = rest % p.row_tiles;
  rest /= p.row_tiles;
  const int g = rest % p.num_kv_heads;
  const int grp = rest / p.num_kv_heads;
  const int G = p.num_q_heads / p.num_kv_heads;

  const int s0 = scalar_load_i32(p.group_start, grp);
  const int s1 = scalar_load_i32(p.group_start, grp + 1);
  const int plen = scalar_load_i32(p.prefix_len, grp) & ~15;  // whole pages, as the decode pass reads it
  const int members = s1 - s0;
  const int rows_here = members * G - rt * 64;  // rows of this tile that exist
  if (rows_here <= 0 || plen <= 0) return;

  // Keys of this partition: pages [part * part_pages, ...) of the prefix.
  const int key0 = part * p.part_pages * kBlockSize;
  const int kv_end = part == p.pre_parts - 1 ? plen : min(plen, (part + 1) * p.part_pages * kBlockSize);
  const int ntiles = kv_end > key0 ? (kv_end - key0 + kTileKeys - 1) / kTileKeys : 0;
  const int T = (ntiles + 3) / 4;          // tiles per quarter (all loop T times)
  const int tile0 = kq * T;
  const int32_t* bt = uniform_ptr(p.block_table + (size_t)s0 * p.max_blocks);
  const int last_page = max(0, (kv_end - 1) >> 4);

  const int lq = lt >> 4;   // keys 4 lq .. 4 lq + 3 of the tile (all in one page)
  const int lc = lt & 15;   // 16-byte chunk

  auto tile_key = [&](int it) { return key0 + (tile0 + it) * kTileKeys; };
  // Tiles past the quarter's share or the partition are not loaded; their
  // registers are never stored (store_tile zeroes keys past kv_end).
  auto load_tile = [&](TileRegs& t, int it) {
    if (it >= T || tile0 + it >= ntiles) return;
    const int page = tile_key(it) >> 4;
    const int32_t id0 = scalar_load_i32(bt, min(page, last_page));
    const int32_t id1 = scalar_load_i32(bt, min(page + 1, last_page));
    const int32_t idp = (lq >> 2) ? id1 : id0;
    const int slot0 = (4 * lq) & 15;
    const u32x4_t* ks = reinterpret_cast<const u32x4_t*>(p.k + cache_offset(idp, g, slot0, lc * 8, p.num_kv_heads));
    const u32x4_t* vs = reinterpret_cast<const u32x4_t*>(p.v + cache_offset(idp, g, slot0, lc * 8, p.num_kv_heads));
#pragma unroll
    for (int e = 0; e < 4; ++e) t.k[e] = stream_load(ks + e * (kHeadDim / 8));
#pragma unroll
    for (int e = 0; e < 4; ++e) t.v[e] = stream_load(vs + e * (kHeadDim / 8));
  };
  auto store_tile = [&](const TileRegs& t, int stage, int it) {
    uint8_t* sk = s_buf[kq][stage];
    uint8_t* svt = sk + kKBytes;
    const int base = tile_key(it) + 4 * lq;
    const bool tile_ok = it < T;
    const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
    u32x4_t kz[4], vz[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = tile_ok && base + e < kv_end;
      kz[e] = ok ? t.k[e] : zero;
      vz[e] = ok ? t.v[e] : zero;
      const int key = 4 * lq + e;
      *reinterpret_cast<u32x4_t*>(sk + key * kKRowBytes + ((lc ^ (key & 15)) << 4)) = kz[e];
    }
    // V^T: dim d's row holds the tile's keys in order; this thread writes the
    // two words of keys 4 lq .. 4 lq + 3 for each of its 8 dims.
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo01 = __builtin_amdgcn_perm(vz[1][w], vz[0][w], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(vz[1][w], vz[0][w], 0x07060302u);
      const uint32_t lo23 = __builtin_amdgcn_perm(vz[3][w], vz[2][w], 0x05040100u);
      const uint32_t hi23 = __builtin_amdgcn_perm(vz[3][w], vz[2][w], 0x07060302u);
      const int d = lc * 8 + 2 * w;
      uint32_t* r0 = reinterpret_cast<uint32_t*>(svt + d * kVtRowBytes + lq * 8);
      uint32_t* r1 = reinterpret_cast<uint32_t*>(svt + (d + 1) * kVtRowBytes + lq * 8);
      r0[0] = lo01;
      r0[1] = lo23;
      r1[0] = hi01;
      r1[1] = hi23;
    }
  };

  // The first two tiles go out before anything that depends on the rows.
  TileRegs ra, rb;
  load_tile(ra, 0);
  issue_order_barrier();
  load_tile(rb, 1);
  issue_order_barrier();

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
  float l_run = 0.f;

  auto compute_tile = [&](int it, int stage) {
    const uint8_t* sk = s_buf[kq][stage];
    const uint8_t* svt = sk + kKBytes;
    f32x16_t st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = hh * 8 + s;
      const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(sk + col * kKRowBytes + ((c ^ (col & 15)) << 4));
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[s]), st, 0, 0, 0);
    }
    const int kbase = tile_key(it) + 4 * hh;
    float sv[16];
    float mloc = -INFINITY;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int key = kbase + 8 * a + b;
        const float x = (it < T && key < kv_end && key <= my_limit) ? st[4 * a + b] * p.scale_log2 : -INFINITY;
        sv[4 * a + b] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const bool raise = mloc > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = fast_exp2(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
      l_run *= alpha;
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
    u32x4_t pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      pf[ks][0] = pack_bf16x2(sv[8 * ks + 0], sv[8 * ks + 1]);
      pf[ks][1] = pack_bf16x2(sv[8 * ks + 2], sv[8 * ks + 3]);
      pf[ks][2] = pack_bf16x2(sv[8 * ks + 4], sv[8 * ks + 5]);
      pf[ks][3] = pack_bf16x2(sv[8 * ks + 6], sv[8 * ks + 7]);
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int d = mb * 32 + col;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // keys 16 ks + 4 hh + 0..3 and 16 ks + 8 + 4 hh + 0..3 (4-byte reads:
        // the 68-byte rows keep only 4-byte alignment)
        const uint32_t* vrow = reinterpret_cast<const uint32_t*>(svt + d * kVtRowBytes + (16 * ks + 4 * hh) * 2);
        const u32x4_t vf = u32x4_t{vrow[0], vrow[1], vrow[4], vrow[5]};
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[ks]), o[mb], 0, 0, 0);
      }
    }
  };

  // Pipeline: tiles it+1, it+2 in registers while
  // tile it is computed from LDS; double-buffered LDS, one barrier per tile.
  if (T > 0) {
    store_tile(ra, 0, 0);
    issue_order_barrier();
    load_tile(ra, 2);
    issue_order_barrier();
    __syncthreads();
  }
  int it = 0;
  for (; it + 1 < T; it += 2) {
    store_tile(rb, 1, it + 1);
    issue_order_barrier();
    load_tile(rb, it + 3);
    issue_order_barrier();
    compute_tile(it, 0);
    __syncthreads();
    store_tile(ra, 0, it + 2);
    issue_order_barrier();
    load_tile(ra, it + 4);
    issue_order_barrier();
    compute_tile(it + 1, 1);
    __syncthreads();
  }
  if (it < T) {
    compute_tile(it, 0);
    __syncthreads();
  }

  // Merge the quarters into quarter 0 through LDS (the tile area, free
  // now), one accumulator block per round, each round in its own region so
  // one barrier per round suffices: quarters 1-3 write, quarter 0 folds.
  // Region layout [sender][chunk of 4 floats][lane]: 16-byte accesses by
  // consecutive lanes.
  constexpr int kRound = 6 * 4 * 64;  // float4s per round
  float4* xacc = reinterpret_cast<float4*>(&s_buf[0][0][0]);
  float2* xml = reinterpret_cast<float2*>(xacc + 4 * kRound);  // [sender][lane]: (m, l)
  static_assert((4 * kRound * sizeof(float4) + 6 * 64 * sizeof(float2)) <= sizeof(s_buf),
                "merge buffer exceeds the tile area");
  const int sender = (kq - 1) * 2 + rg;
  float a0 = 0.f, aq[3] = {0.f, 0.f, 0.f};
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    float4* rbuf = xacc + mb * kRound;
    if (kq != 0) {
      if (mb == 0) xml[sender * 64 + lane] = make_float2(m_run, l_run);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        rbuf[(sender * 4 + c) * 64 + lane] =
            make_float4(o[mb][4 * c], o[mb][4 * c + 1], o[mb][4 * c + 2], o[mb][4 * c + 3]);
    }
    __syncthreads();
    if (kq == 0) {
      if (mb == 0) {
        float2 ml[3];
        float M = m_run;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          ml[q] = xml[(q * 2 + rg) * 64 + lane];
          M = fmaxf(M, ml[q].x);
        }
        const float Mu = (M == -INFINITY) ? 0.f : M;
        a0 = fast_exp2(m_run - Mu);
        float l = l_run * a0;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          aq[q] = fast_exp2(ml[q].x - Mu);
          l = fmaf(ml[q].y, aq[q], l);
        }
        l_run = l;
        m_run = M;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float x0 = o[mb][4 * c] * a0, x1 = o[mb][4 * c + 1] * a0;
        float x2 = o[mb][4 * c + 2] * a0, x3 = o[mb][4 * c + 3] * a0;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const float4 y = rbuf[((q * 2 + rg) * 4 + c) * 64 + lane];
          x0 = fmaf(y.x, aq[q], x0);
          x1 = fmaf(y.y, aq[q], x1);
          x2 = fmaf(y.z, aq[q], x2);
          x3 = fmaf(y.w, aq[q], x3);
        }
        o[mb][4 * c] = x0;
        o[mb][4 * c + 1] = x1;
        o[mb][4 * c + 2] = x2;
        o[mb][4 * c + 3] = x3;
      }
    }
  }
  if (kq != 0 || !row_live) return;

  const size_t rows = (size_t)p.total_q * p.num_q_heads;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (hh == 0) p.pre_lse[(size_t)part * rows + grow] = l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  if (l_tot == 0.f) return;  // no visible key in this partition: the output is never read
  const float inv = 1.f / l_tot;
  float* orow = p.pre_out + ((size_t)part * rows + grow) * kHeadDim;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d = mb * 32 + 8 * a + 4 * hh;
      *reinterpret_cast<float4*>(orow + d) =
          make_float4(o[mb][4 * a] * inv, o[mb][4 * a + 1] * inv, o[mb][4 * a + 2] * inv, o[mb][4 * a + 3] * inv);
    }
}

}  // namespace

hipError_t launch_prefix(const PrefixParams& p, unsigned grid, hipStream_t s) {
  PrefixParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&prefix_kernel), dim3(grid + 1), dim3(kThreads), args, 0, s);
}

}  // namespace pa
