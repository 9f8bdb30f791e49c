// chunk.hip -- several new rows per slot against paged KV, on bf16 MFMA.
//
// Used for chunked autoregressive denoising: a chunk of latent tokens attends
// to the KV of earlier chunks at the same noise level plus its own (PhysisServe
// teardown page, section "why autoregressive denoising can be pipelined"),
// with a full mask over the slot's n keys; with PA_FLAG_CAUSAL row i sees keys
// [0, n - m + i] instead (chunked prefill, inference-optimisation chapter,
// section 8.2.3).  Both products are dense contractions, so they run on the
// matrix cores: v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// Rows: the (new token, query head) pairs of one KV head of a slot, token
// major -- packed row j is token j / G of query head g G + j % G, G being the
// query heads per KV head -- so the G heads that share a KV head read its
// pages once, and a few tokens with grouped heads (speculative verification:
// 5 to 8 tokens times 4 heads) fill a tile instead of leaving most of it
// idle.  With one query head per KV head (the denoising workload) a row is a
// token.
//
// Workgroup: 8 waves over 128 packed rows of one (slot, KV head).  Wave w
// takes the rows r with r % 4 == w % 4 (32 of them) and one half of the
// keys (w / 4); the two halves merge through LDS at the end.  Each half
// walks its keys in 32-key tiles (two 16-token pages):
//   1. the tile's K and V rows go straight from memory into LDS
//      (global_load_lds_dwordx4), row-major with each row's 16-byte chunks
//      permuted (key_swz in device.h: no LDS bank conflicts for the reads
//      below), into a four-stage ring: three tiles are in flight while one
//      is computed, no registers hold them and no store instructions move
//      them.  Each lane's source chunk is the one the permutation puts at its
//      LDS slot; page ids come from scalar loads one tile ahead.  One barrier
//      per tile;
//   2. each wave computes S^T = K Q^T (32 keys x 32 rows, 8 MFMAs over the 128
//      dims, all eight K fragments read before the first product).  In the
//      MFMA output layout a lane holds 16 keys of ONE query row, so the row
//      max and sum of the online softmax are mostly in-lane; the other 16
//      keys of the row sit in lane ^ 32 (v_permlane32_swap).  The
//      accumulators are only rescaled when the row max grows by more than
//      2^8; masked keys become -inf in place, tiles that every row sees whole
//      skip the masking, and the scale folds into the exponent's FMA;
//   3. probabilities are rounded to bf16 and used directly, from registers, as
//      the B operand of O^T += V^T P^T (4 x 32 dims, 2 key steps, 8 MFMAs);
//      the V^T A operand is read from the row-major V tile with transposing
//      LDS reads (ds_read_b64_tr_b16), issued before the softmax so that they
//      complete under it.  The output is divided by the sum of those rounded
//      weights, so it is an exact weighted mean of the V rows under the
//      weights PV used (a single dominant key comes back exactly); the LSE
//      takes the sum of the fp32 weights.  A key half in which some row
//      sees fewer than kFewKeys of the half's keys -- too few to average the
//      rounding down -- makes a second pass over its tiles after the loop,
//      adding the rounding's remainders (each scaled to the row's final
//      reference max) through a product of their own; its divisor is then
//      the fp32 sum.
// Keys past the end load the last key (finite) and get -inf scores.  The
// 128 x 128 bf16 output tile is staged in LDS and stored as whole rows.

#include <type_traits>

#include "device.h"

namespace pa {

namespace {

constexpr int kThreads = 512;
constexpr int kTileKeys = 32;
constexpr int kRowBytes = kHeadDim * 2;           // 256: one key row of K or V
constexpr int kTileBytes = kTileKeys * kRowBytes; // 8 KiB (K or V)
constexpr int kStages = 4;                        // LDS stages per key half
constexpr float kRescaleSlack = 8.0f;             // log2 units
constexpr int kMergeBytes = 72 * 1024;            // merge buffer at the start of the tile area
// Rows that see fewer than this many of a key half's keys get the second,
// remainder pass (see above).
constexpr int kFewKeys = 64;

static_assert(kChunkRows == 4 * 32, "four row groups of 32 rows");

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& u) { return __builtin_bit_cast(bf16x8_t, u); }

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Byte offset of dims d .. of key row `key` in a swizzled K or V tile.
__device__ __forceinline__ int swz(int key, int d) {
  return key * kRowBytes + (((d >> 3) ^ key_swz(key)) << 4) + (d & 7) * 2;
}

__global__ __launch_bounds__(kThreads, 1) void chunk_kernel(ChunkParams p) {
  // [key half][stage][K tile | V tile], both row-major with swizzled 16-byte
  // chunks, filled straight from memory; reused for the final merge.
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[2][kStages][2][kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & 3;    // row group
  const int kh = wave >> 2;   // key half
  const int wh = wave & 3;    // wave within the half (loader role)
  const int col = lane & 31;  // query row within the wave / MFMA column
  const int hh = lane >> 5;   // lane half
  // The kernel arguments the start needs, fetched together: the index
  // arithmetic below uses the pinned copies, so the compiler cannot start it
  // on a first batch of arguments and fetch the rest one round trip later.
  int grid = gridDim.x, q_tiles = p.q_tiles, hq = p.num_q_heads, hkv = p.num_kv_heads;
  asm volatile("" : "+s"(grid), "+s"(q_tiles), "+s"(hq), "+s"(hkv)
               : "s"(p.q_lens), "s"(p.ctx_lens), "s"(p.block_table), "s"(p.max_blocks), "s"(p.max_ctx),
                 "s"(p.max_q), "s"(p.causal));

  const int wg = xcd_remap(blockIdx.x, grid);
  const int qt = wg % q_tiles;
  const int sg = wg / q_tiles;
  const int g = sg % hkv;
  const int seq = sg / hkv;
  const int G = hq / hkv;

  // The keys this half needs depend on the slot's lengths.  The page ids of
  // its first four tiles are requested together with the lengths, for the
  // tiles the declared maxima (max_ctx_len, max_q_len) give, and requested
  // again only when the lengths differ: a memory round trip saved before the
  // first tile request when the slot is full length.
  const int32_t* bt = p.block_table + (size_t)seq * p.max_blocks;
  auto half_tiles = [&](int m_, int n_, int& tile0_, int& last_page_, int& kv_end_) {
    int kv = n_;
    if (p.causal) {
      const int last_token = (min(m_ * G, (qt + 1) * kChunkRows) - 1) / G;  // of the tile's last live row
      kv = min(n_, n_ - m_ + last_token + 1);
    }
    kv_end_ = kv;
    const int nt = (max(kv, 1) + kTileKeys - 1) / kTileKeys;
    tile0_ = kh * ((nt + 1) / 2);
    last_page_ = max(0, (kv - 1) >> 4);
  };
  int32_t ids[8];  // pages 2 tile0 .. + 7: tiles 0 .. 3 of this half
  auto request_ids = [&](int tile0_, int last_page_) {
#pragma unroll
    for (int j = 0; j < 8; ++j) ids[j] = scalar_load_i32(bt, min(2 * tile0_ + j, last_page_));
  };
  int tile0_g, last_page_g, kv_end_g;
  half_tiles(p.max_q, p.max_ctx, tile0_g, last_page_g, kv_end_g);
  request_ids(tile0_g, last_page_g);
  int m = scalar_load_i32(p.q_lens, seq);
  int n = scalar_load_i32(p.ctx_lens, seq);
  // The row offset of the slot (the sum of q_lens over the slots before it)
  // in the same round trip: the first sixteen terms (indices clamped into
  // the array, the extra ones masked below).
  int x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) x[j] = scalar_load_i32(p.q_lens, max(0, min(j, seq - 1)));
  // (all in flight before the first is used)
  asm volatile("" : "+s"(ids[0]), "+s"(ids[1]), "+s"(ids[2]), "+s"(ids[3]), "+s"(ids[4]), "+s"(ids[5]),
               "+s"(ids[6]), "+s"(ids[7]), "+s"(m), "+s"(n));
  asm volatile("" : "+s"(x[0]), "+s"(x[1]), "+s"(x[2]), "+s"(x[3]), "+s"(x[4]), "+s"(x[5]), "+s"(x[6]),
               "+s"(x[7]), "+s"(x[8]), "+s"(x[9]), "+s"(x[10]), "+s"(x[11]), "+s"(x[12]), "+s"(x[13]),
               "+s"(x[14]), "+s"(x[15]));
  if (m <= 0 || n <= 0 || qt * kChunkRows >= m * G) return;
  int q_row0 = 0;  // row offset of the slot
#pragma unroll
  for (int j = 0; j < 16; ++j) q_row0 += j < seq ? x[j] : 0;
  // Slots past the sixteenth: further batches of sixteen independent scalar
  // loads, one wait each.
  for (int i = 16; i < seq; i += 16) {
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = scalar_load_i32(p.q_lens, min(i + j, seq - 1));
    asm volatile("" : "+s"(x[0]), "+s"(x[1]), "+s"(x[2]), "+s"(x[3]), "+s"(x[4]), "+s"(x[5]), "+s"(x[6]),
                 "+s"(x[7]), "+s"(x[8]), "+s"(x[9]), "+s"(x[10]), "+s"(x[11]), "+s"(x[12]), "+s"(x[13]),
                 "+s"(x[14]), "+s"(x[15]));
#pragma unroll
    for (int j = 0; j < 16; ++j) q_row0 += i + j < seq ? x[j] : 0;
  }
  // Packed row within the slot: the tile's rows are dealt to the four row
  // groups in turn (row 4 c + rg is column c of row group rg), so a tile
  // with few live rows (a few tokens' grouped heads) still keeps every SIMD
  // busy instead of leaving three row groups idle.
  const int prow = qt * kChunkRows + 4 * col + rg;
  const bool row_live = prow < m * G;
  const int tok = row_live ? prow / G : 0;           // its token; rows past the end use token 0 of
  const int h = g * G + (row_live ? prow % G : 0);   // head g G (their results are never written)

  // Q^T operand: lane (row, half) holds dims (hh*8 + s)*8 .. +8 for step s
  // (requested just before the first tiles, below).
  u32x4_t qf[8];
  auto load_q = [&]() {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(p.q) +
                        ((size_t)(q_row0 + tok) * p.num_q_heads + h) * (kHeadDim / 8);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = qp[hh * 8 + s];
  };

  // Keys this workgroup needs, split in two halves of whole tiles.
  int tile0, last_page, kv_end;
  half_tiles(m, n, tile0, last_page, kv_end);
  const int ntiles = (kv_end + kTileKeys - 1) / kTileKeys;
  const int T = (ntiles + 1) / 2;       // tiles per half (both halves loop T times)
  const int my_limit = p.causal ? (n - m + tok) : (n - 1);  // last visible key of this row
  // Few keys in a half: some live row sees between 1 and kFewKeys - 1 of
  // the half's keys (a row that sees v keys has min(max(v - base, 0), T * 32)
  // of those of the half starting at key base).  Both halves' flags, since
  // the remainder pass's barriers are the workgroup's.
  bool fine, fine_any;
  {
    const int t_first = (qt * kChunkRows) / G;
    const int t_last = (min(m * G, (qt + 1) * kChunkRows) - 1) / G;
    const int v_lo = p.causal ? n - m + t_first + 1 : n;
    const int v_hi = p.causal ? n - m + t_last + 1 : n;
    auto few = [&](int base) { return v_hi > base && min(max(v_lo - base, 1), T * kTileKeys) < kFewKeys; };
    const bool f0 = few(0), f1 = few(T * kTileKeys);
    fine = kh == 0 ? f0 : f1;
    fine_any = f0 || f1;
  }
  // Tiles ending at or before this key count are visible to every row of the
  // workgroup (under the causal mask: to the tile's first token).
  const int open_end = p.causal ? min(kv_end, n - m + (qt * kChunkRows) / G + 1) : kv_end;
  if (m != p.max_q || n != p.max_ctx) request_ids(tile0, last_page);

  // Loads straight into LDS (global_load_lds_dwordx4: lane l of a wave
  // writes bytes 16 l .. of the instruction's LDS base).  Each of a half's
  // four waves fills key rows 8 wh .. 8 wh + 7 of a tile's K and V with four
  // instructions of four rows each; lane l takes LDS chunk slot l % 16 of
  // row l / 16 and so loads the global chunk that the swizzle puts there.
  // Keys past the end re-read the last key (finite: tail slots are never
  // read), whose scores are masked and whose probabilities are 0.
  // In the loop, the page ids of the next tile to load are read one load
  // ahead.
  int32_t nid0 = 0, nid1 = 0;
  auto fetch_ids = [&](int it) {
    const int t = tile0 + it;
    nid0 = scalar_load_i32(bt, min(2 * t, last_page));
    nid1 = scalar_load_i32(bt, min(2 * t + 1, last_page));
  };
  auto issue_tile = [&](int it, int stage, int32_t id0, int32_t id1) {
    const int t = tile0 + it;
    uint8_t* sk = s_buf[kh][stage][0];
    uint8_t* sv = s_buf[kh][stage][1];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 8 * wh + 4 * j + (lane >> 4);  // LDS row of this lane
      const int key = min(t * kTileKeys + r, kv_end - 1);
      const int32_t id = (key >> 4) & 1 ? id1 : id0;
      const int c = (lane & 15) ^ key_swz(r);      // global chunk for this slot
      const size_t off = cache_offset(id, g, key & 15, c * 8, p.num_kv_heads);
      const int lds_off = (8 * wh + 4 * j) * kRowBytes;  // wave-uniform
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(p.k + off),
                                       (void __attribute__((address_space(3)))*)(sk + lds_off), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(p.v + off),
                                       (void __attribute__((address_space(3)))*)(sv + lds_off), 16, 0, 0);
    }
  };
  auto load_tile = [&](int it, int stage) {
    const int32_t id0 = nid0, id1 = nid1;
    fetch_ids(it + 1);
    issue_tile(it, stage, id0, id1);
  };

  f32x16_t o[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mb][i] = 0.f;
  float m_run = -INFINITY;  // reference max of this row (log2 domain)
  float l_run = 0.f;        // this lane's share of the row sum (fp32 weights)
  float r_run = 0.f;        // the same over the bf16-rounded weights PV uses

  // The stage is a compile-time constant (the loop below is unrolled by the
  // ring depth), so every LDS address is a per-lane register plus an
  // immediate offset.
  auto compute_tile = [&](int it, auto stage_c) {
    constexpr int stage = decltype(stage_c)::value;
    const uint8_t* sk = s_buf[kh][stage][0];
    // S^T = K Q^T: A = K rows (key = col), B = Q^T (row = col).
    f32x16_t st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
    // All eight K fragments are read before the first product, so the LDS
    // latency is paid once rather than before every MFMA.
    u32x4_t kf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = hh * 8 + s;
      kf[s] = *reinterpret_cast<const u32x4_t*>(sk + col * kRowBytes + ((c ^ key_swz(col)) << 4));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int s = 0; s < 8; ++s)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[s]), as_bf16x8(qf[s]), st, 0, 0, 0);
    // The V^T operand of O^T += V^T P^T (lane: dim mb*32 + l % 32, keys
    // 16 ks + 4 hh + {0..3, 8..11}) comes from the row-major V tile through
    // transposing reads (ds_read_b64_tr_b16): in each 16-lane group, lane a
    // points at 4 dims of key a / 4, and lane i receives dim i of the four
    // keys.  The sixteen reads are issued here, in an asm block, so that they
    // complete under the softmax; a second block waits for them.  (Through
    // the builtin, the compiler would also wait for the loads into LDS still
    // in flight, which it cannot tell apart from this stage, already
    // complete: its loads were waited for before the barrier.)  Key + 16 is
    // 4096 bytes further with the same swizzle; key + 8 has its own address.
    const int grp16 = lane >> 4;
    const int a16 = lane & 15;
    // (stage 0's V tile; the stage is the reads' immediate offset)
    const uint32_t vbase = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)s_buf[kh][0][1];
    constexpr int voff = stage * 2 * kTileBytes;
    u32x2_t vr[16];  // vr[4 mb + 2 ks + e]: keys 16 ks + 8 e + 4 hh + 0..3
    {
      uint32_t va[8];  // va[2 mb + e]: key 8 e + 4 hh + a / 4, 4 dims of block mb
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          va[2 * mb + e] = vbase + swz(8 * e + 4 * hh + (a16 >> 2), mb * 32 + (grp16 & 1) * 16 + 4 * (a16 & 3));
      asm volatile(
          "ds_read_b64_tr_b16 %0, %16 offset:%24\n\t"
          "ds_read_b64_tr_b16 %1, %17 offset:%24\n\t"
          "ds_read_b64_tr_b16 %2, %16 offset:%25\n\t"
          "ds_read_b64_tr_b16 %3, %17 offset:%25\n\t"
          "ds_read_b64_tr_b16 %4, %18 offset:%24\n\t"
          "ds_read_b64_tr_b16 %5, %19 offset:%24\n\t"
          "ds_read_b64_tr_b16 %6, %18 offset:%25\n\t"
          "ds_read_b64_tr_b16 %7, %19 offset:%25\n\t"
          "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
          "ds_read_b64_tr_b16 %9, %21 offset:%24\n\t"
          "ds_read_b64_tr_b16 %10, %20 offset:%25\n\t"
          "ds_read_b64_tr_b16 %11, %21 offset:%25\n\t"
          "ds_read_b64_tr_b16 %12, %22 offset:%24\n\t"
          "ds_read_b64_tr_b16 %13, %23 offset:%24\n\t"
          "ds_read_b64_tr_b16 %14, %22 offset:%25\n\t"
          "ds_read_b64_tr_b16 %15, %23 offset:%25"
          : "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]), "=&v"(vr[6]),
            "=&v"(vr[7]), "=&v"(vr[8]), "=&v"(vr[9]), "=&v"(vr[10]), "=&v"(vr[11]), "=&v"(vr[12]),
            "=&v"(vr[13]), "=&v"(vr[14]), "=&v"(vr[15])
          : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7]),
            "i"(voff), "i"(voff + 4096));
    }

    // Online softmax over this lane's 16 keys of its row (log2 domain).
    // The scale folds into the exponent's FMA (and into the max, taken over
    // the raw scores); masked keys become -inf in place.  Tiles that every
    // row of the workgroup sees whole skip the masking.  A scale that is not positive would turn the max of the raw
    // scores into the min of the scaled ones, so then the masking pass
    // applies the scale itself and the FMA multiplies by 1.
    const int kbase = (tile0 + it) * kTileKeys + 4 * hh;
    const bool pos = p.scale_log2 > 0.f;
    const float sc = pos ? p.scale_log2 : 1.f;
    if ((tile0 + it + 1) * kTileKeys > open_end || !pos) {
      if (!pos) {
#pragma unroll
        for (int i = 0; i < 16; ++i) st[i] *= p.scale_log2;
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int key = kbase + 8 * a + b;
          if (key > my_limit) st[4 * a + b] = -INFINITY;
        }
    }
    float mloc = st[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, st[i]);
    mloc *= sc;
    mloc = fmaxf(mloc, other_half(mloc));
    const bool raise = mloc > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      // A row with no visible key so far keeps m = -inf (its sums are 0);
      // guard the difference so -inf - -inf never makes a NaN.
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
      st[i] = fast_exp2(fmaf(st[i], sc, -m_use));
      lsum += st[i];
    }
    l_run += lsum;
    // P^T operand for key steps 0 and 1: keys 16ks + 4hh + 0..3, 16ks + 8 + 4hh + 0..3.
    // The sum of the rounded weights is a dot product of each packed pair
    // with (1, 1): exact products, fp32 sums.
    u32x4_t pf[2];
    float rsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pf[ks][w] = pack_bf16x2(st[8 * ks + 2 * w], st[8 * ks + 2 * w + 1]);
        rsum = bf16x2_sum_into(pf[ks][w], rsum);
      }
    }
    r_run += rsum;
    // The transposed reads must have landed (the operands pass through this
    // block, so nothing reads them before it).
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(vr[0]), "+v"(vr[1]), "+v"(vr[2]), "+v"(vr[3]), "+v"(vr[4]), "+v"(vr[5]), "+v"(vr[6]),
                   "+v"(vr[7]), "+v"(vr[8]), "+v"(vr[9]), "+v"(vr[10]), "+v"(vr[11]), "+v"(vr[12]),
                   "+v"(vr[13]), "+v"(vr[14]), "+v"(vr[15]));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x2_t l2 = vr[4 * mb + 2 * ks];
        const u32x2_t h2 = vr[4 * mb + 2 * ks + 1];
        const u32x4_t vf = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[ks]), o[mb], 0, 0, 0);
      }
  };

  // Pipeline: tile it sits in stage it % 4; the loads of tiles it + 1 ..
  // it + 3 are in flight while it is computed.  Iteration it waits for its
  // own loads, crosses one barrier (every wave's loads of tile it are then
  // in LDS, and every wave has finished computing tile it - 1), refills the
  // stage of tile it - 1 with tile it + 3, and computes.  Loads are
  // unconditional (a tile index past the half clamps to the last key), so
  // the load counter sees the same pattern on every trip.
  // The query first, then three tiles: the first wait of the loop (all but
  // the last two tiles' eight loads) covers exactly the query and tile 0.
  load_q();
  if (T > 0) {
    issue_tile(0, 0, ids[0], ids[1]);
    issue_tile(1, 1, ids[2], ids[3]);
    issue_tile(2, 2, ids[4], ids[5]);
    nid0 = ids[6];
    nid1 = ids[7];
  }
  auto step = [&](int it, auto stage_c) {
    constexpr int stage = decltype(stage_c)::value;
    // this wave's loads of tile it (and before the first tile, the query's)
    // are older than those of it + 1, it + 2 (4 instructions each).
    __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8), other counters unconstrained
    __syncthreads();
    load_tile(it + 3, (stage + 3) & (kStages - 1));
    compute_tile(it, stage_c);
  };
  static_assert(kStages == 4, "the loop below is unrolled by the ring depth");
  for (int it = 0; it < T; it += 4) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 >= T) break;
    step(it + 1, std::integral_constant<int, 1>{});
    if (it + 2 >= T) break;
    step(it + 2, std::integral_constant<int, 2>{});
    if (it + 3 >= T) break;
    step(it + 3, std::integral_constant<int, 3>{});
  }
  // The loads past the last tile must land before the tile area is reused,
  // and every wave must be done computing.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  // Remainder pass (few keys in a half): the half's tiles again, one at a
  // time through stage 0.  The scores, the masking and the lazy reference
  // max are recomputed exactly as above, so each tile's weights w and their
  // bf16 roundings hi are the ones PV used; the remainders w - hi, scaled by
  // 2^(reference at the tile - final reference) as the rescales scaled that
  // tile's share of o, go through PV as bf16.  o then sums the fp32 weights,
  // so the divisor becomes their fp32 sum.
  if (fine_any) {
    const float m_fin = m_run;
    float m2 = -INFINITY;
    const bool pos = p.scale_log2 > 0.f;
    const float sc = pos ? p.scale_log2 : 1.f;
    const int grp16 = lane >> 4;
    const int a16 = lane & 15;
#pragma unroll 1
    for (int it = 0; it < T; ++it) {
      const int t = tile0 + it;
      issue_tile(it, 0, scalar_load_i32(bt, min(2 * t, last_page)), scalar_load_i32(bt, min(2 * t + 1, last_page)));
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
      if (fine) {
        const uint8_t* sk = s_buf[kh][0][0];
        const uint8_t* svv = s_buf[kh][0][1];
        f32x16_t st;
#pragma unroll
        for (int i = 0; i < 16; ++i) st[i] = 0.f;
        u32x4_t kf[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int c = hh * 8 + s;
          kf[s] = *reinterpret_cast<const u32x4_t*>(sk + col * kRowBytes + ((c ^ key_swz(col)) << 4));
        }
#pragma unroll
        for (int s = 0; s < 8; ++s)
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[s]), as_bf16x8(qf[s]), st, 0, 0, 0);
        const int kbase = t * kTileKeys + 4 * hh;
        if ((t + 1) * kTileKeys > open_end || !pos) {
          if (!pos) {
#pragma unroll
            for (int i = 0; i < 16; ++i) st[i] *= p.scale_log2;
          }
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
              if (kbase + 8 * a + b > my_limit) st[4 * a + b] = -INFINITY;
        }
        float mloc = st[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, st[i]);
        mloc *= sc;
        mloc = fmaxf(mloc, other_half(mloc));
        if (__builtin_amdgcn_ballot_w64(mloc > m2 + kRescaleSlack) != 0) m2 = fmaxf(m2, mloc);
        const float m_use = (m2 == -INFINITY) ? 0.f : m2;
        const float to_fin = m_fin == -INFINITY ? 0.f : fast_exp2(m_use - m_fin);
        u32x4_t pl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float w0 = fast_exp2(fmaf(st[8 * ks + 2 * w], sc, -m_use));
            const float w1 = fast_exp2(fmaf(st[8 * ks + 2 * w + 1], sc, -m_use));
            const uint32_t hi = pack_bf16x2(w0, w1);
            pl[ks][w] = pack_bf16x2((w0 - bf16_lo(hi)) * to_fin, (w1 - bf16_hi(hi)) * to_fin);
          }
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
            o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pl[ks]), o[mb], 0, 0, 0);
          }
      }
      __syncthreads();  // stage 0 is loaded again next
    }
    if (fine) r_run = l_run;
  }

  // Merge the key halves through LDS (the tile area) behind one barrier:
  // wave (rg, kh) keeps output blocks 2 kh, 2 kh + 1 (dims 64 kh .. +64) of
  // its rows, hands the other two to its partner (rg, 1 - kh), folds the two
  // it receives and stores its 64 dims, so both halves share the folding
  // and the stores.  Layout [row group][sender half][block][chunk of 4
  // floats][lane]: 16-byte accesses by consecutive lanes.
  float4* xacc = reinterpret_cast<float4*>(&s_buf[0][0][0][0]);
  float4* xml = xacc + 4 * 2 * 2 * 4 * 64;  // [row group][half][lane]: (m, l, rounded l)
  static_assert(4 * 2 * 2 * 4 * 64 * sizeof(float4) + 4 * 2 * 64 * sizeof(float4) <= kMergeBytes &&
                    kMergeBytes + kChunkRows * kRowBytes <= sizeof(s_buf),
                "merge buffer and output tile exceed the tile area");
  xml[(rg * 2 + kh) * 64 + lane] = make_float4(m_run, l_run, r_run, 0.f);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if ((mb >> 1) == kh) continue;
    float4* dst = xacc + ((rg * 2 + kh) * 2 + (mb & 1)) * 4 * 64;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      dst[c * 64 + lane] = make_float4(o[mb][4 * c], o[mb][4 * c + 1], o[mb][4 * c + 2], o[mb][4 * c + 3]);
  }
  __syncthreads();

  const float4 ml = xml[(rg * 2 + (1 - kh)) * 64 + lane];
  const float M = fmaxf(m_run, ml.x);
  const float Mu = (M == -INFINITY) ? 0.f : M;
  const float s0 = fast_exp2(m_run - Mu);
  const float s1 = fast_exp2(ml.x - Mu);
  const float l = l_run * s0 + ml.y * s1;
  const float l_tot = l + __shfl_xor(l, 32, 64);
  const float r = r_run * s0 + ml.z * s1;
  const float inv = 1.f / (r + __shfl_xor(r, 32, 64));
  // The bf16 output of the tile goes through LDS (past the merge buffer), so
  // that every output row leaves as 16 lanes storing its 256 contiguous
  // bytes: the wave's own lanes hold 8 bytes of 32 different rows per
  // value, and stored from there the rows reach memory in 16-byte pieces
  // (measured: 0.4 - 0.9 us per launch more).  Tile row j = packed row qt 128 + j,
  // the 16-byte chunk c at position c ^ ((j / 4) % 16), so the wave's 32
  // rows (j = 4 col + rg) write distinct positions.
  uint8_t* otile = &s_buf[0][0][0][0] + kMergeBytes;
  {
    const int j = 4 * col + rg;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if ((mb >> 1) != kh) continue;
      const float4* src = xacc + ((rg * 2 + (1 - kh)) * 2 + (mb & 1)) * 4 * 64;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4 y = src[a * 64 + lane];
        const int d = mb * 32 + 8 * a + 4 * hh;
        uint2 w;
        w.x = pack_bf16x2((o[mb][4 * a + 0] * s0 + y.x * s1) * inv, (o[mb][4 * a + 1] * s0 + y.y * s1) * inv);
        w.y = pack_bf16x2((o[mb][4 * a + 2] * s0 + y.z * s1) * inv, (o[mb][4 * a + 3] * s0 + y.w * s1) * inv);
        *reinterpret_cast<uint2*>(otile + j * kRowBytes + (((d >> 3) ^ (col & 15)) << 4) + (d & 7) * 2) = w;
      }
    }
  }
  if (row_live && kh == 0 && hh == 0 && p.lse)
    p.lse[(size_t)(q_row0 + tok) * p.num_q_heads + h] = (M + fast_log2(l_tot)) * kLn2;
  __syncthreads();
  // 128 rows x 16 chunks, four per thread: 16 consecutive threads per row.
  const int rows_live = min(kChunkRows, m * G - qt * kChunkRows);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int idx = k * kThreads + tid;
    const int j = idx >> 4;
    const int c = idx & 15;
    if (j < rows_live) {
      const int pj = qt * kChunkRows + j;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(otile + j * kRowBytes + ((c ^ ((j >> 2) & 15)) << 4));
      // (non-temporal: written once, not read again by this kernel; measured
      // 0.2 - 0.7 us per launch faster than an ordinary store)
      const size_t orow = (size_t)(q_row0 + pj / G) * p.num_q_heads + g * G + pj % G;
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p.out + orow * kHeadDim + c * 8));
    }
  }
}

}  // namespace

hipError_t launch_chunk(const ChunkParams& p, unsigned grid, hipStream_t s) {
  ChunkParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&chunk_kernel), dim3(grid), dim3(kThreads), args, 0, s);
}

}  // namespace pa
