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
// Workgroup: 8 waves over 128 query rows of one (slot, query head).  Wave w
// takes rows 32 (w % 4) .. +32 and one half of the keys (w / 4); the two
// halves merge through LDS at the end.  Each half walks its keys in 32-key
// tiles (two 16-token pages):
//   1. its 256 threads load a tile's K and V rows through the block table
//      (page ids by scalar loads; a thread holds one 16-byte chunk of two
//      adjacent keys, so each wave instruction reads four whole 256-byte key
//      rows) two tiles ahead into a two-deep register ring, and store each
//      tile to a double-buffered LDS area: K row-major with XOR-swizzled
//      16-byte chunks, V transposed (dim-major, rows padded to 68 bytes, 17
//      words, which keeps the transposed stores and 4-byte reads spread over
//      the banks).  One barrier per tile;
//   2. each wave computes S^T = K Q^T (32 keys x 32 rows, 8 MFMAs over the 128
//      dims, all eight K fragments read before the first product).  In the
//      MFMA output layout a lane holds 16 keys of ONE query row, so the row
//      max and sum of the online softmax are mostly in-lane; the other 16
//      keys of the row sit in lane ^ 32 (v_permlane32_swap).  The
//      accumulators are only rescaled when the row max grows by more than 2^8;
//   3. probabilities are rounded to bf16 and used directly, from registers, as
//      the B operand of O^T += V^T P^T (4 x 32 dims, 2 key steps, 8 MFMAs); the
//      V^T A operand is read from the transposed LDS tile with the same key
//      order the probabilities already have.
// Keys >= n are never loaded (zeros) and get -inf scores.

#include "device.h"

namespace pa {

namespace {

constexpr int kThreads = 512;
constexpr int kHalfThreads = 256;
constexpr int kTileKeys = 32;
constexpr int kKRowBytes = kHeadDim * 2;          // 256
constexpr int kVtRowBytes = kTileKeys * 2 + 4;    // 68: padded dim-major row (17 words)
constexpr int kKBytes = kTileKeys * kKRowBytes;   // 8 KiB
constexpr int kVtBytes = kHeadDim * kVtRowBytes;  // 9 KiB
constexpr int kStageBytes = kKBytes + kVtBytes;   // one tile
constexpr float kRescaleSlack = 8.0f;             // log2 units

static_assert(kChunkRows == 4 * 32, "four row groups of 32 rows");

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& u) { return __builtin_bit_cast(bf16x8_t, u); }

struct TileRegs {
  u32x4_t k[2];  // keys 2 lv_kp, 2 lv_kp + 1, chunk lv_c
  u32x4_t v[2];
};

__global__ __launch_bounds__(kThreads, 1) void chunk_kernel(ChunkParams p) {
  // [key half][stage][K tile | V^T tile]; reused for the final merge.
  __shared__ __attribute__((aligned(16))) uint8_t s_buf[2][2][kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & 3;    // row group
  const int kh = wave >> 2;   // key half
  const int lt = tid & (kHalfThreads - 1);  // loader id within the half
  const int col = lane & 31;  // query row within the wave / MFMA column
  const int hh = lane >> 5;   // lane half

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = wg % p.q_tiles;
  const int sh = wg / p.q_tiles;
  const int h = sh % p.num_q_heads;
  const int seq = sh / p.num_q_heads;
  const int g = h / (p.num_q_heads / p.num_kv_heads);

  const int m = scalar_load_i32(p.q_lens, seq);
  const int n = scalar_load_i32(p.ctx_lens, seq);
  if (m <= 0 || n <= 0 || qt * kChunkRows >= m) return;
  int q_row0 = 0;
  for (int i = 0; i < seq; ++i) q_row0 += scalar_load_i32(p.q_lens, i);
  const int row = qt * kChunkRows + rg * 32 + col;  // row within the slot
  const bool row_live = row < m;

  // Q^T operand: lane (row, half) holds dims (hh*8 + s)*8 .. +8 for step s
  // (loaded after the first tiles are requested, below).  Rows past m read
  // row 0's query (their results are never written).
  u32x4_t qf[8];
  auto load_q = [&]() {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(p.q) +
                        ((size_t)(q_row0 + (row_live ? row : 0)) * p.num_q_heads + h) * (kHeadDim / 8);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = qp[hh * 8 + s];
  };

  // Keys this workgroup needs, split in two halves of whole tiles.
  int kv_end = n;
  if (p.causal) {
    const int last_row = min(m, (qt + 1) * kChunkRows) - 1;
    kv_end = min(n, n - m + last_row + 1);
  }
  const int ntiles = (kv_end + kTileKeys - 1) / kTileKeys;
  const int T = (ntiles + 1) / 2;       // tiles per half (both halves loop T times)
  const int tile0 = kh * T;             // this half's first tile
  const int my_limit = p.causal ? (n - m + row) : (n - 1);  // last visible key of this row

  const int32_t* bt = p.block_table + (size_t)seq * p.max_blocks;
  const int last_page = (kv_end - 1) >> 4;

  // Loader roles (within the half): keys 2 lv_kp and 2 lv_kp + 1 (same
  // page), 16-byte chunk lv_c, for K and for V -- each wave instruction reads
  // four whole 256-byte key rows.
  const int lv_kp = lt >> 4;
  const int lv_c = lt & 15;

  // Loads are unconditional (page ids clamped to the last live page, so every
  // address is inside the pool) and keys past the end are zeroed when the
  // tile is stored: the load counter then sees a fixed pattern and its waits
  // leave the next tile in flight.
  auto load_tile = [&](TileRegs& r, int it) {
    const int t = tile0 + it;
    const int32_t id0 = scalar_load_i32(bt, min(2 * t, last_page));
    const int32_t id1 = scalar_load_i32(bt, min(2 * t + 1, last_page));
    const int32_t idv = ((2 * lv_kp) >> 4) ? id1 : id0;
    const size_t off = cache_offset(idv, g, (2 * lv_kp) & 15, lv_c * 8, p.num_kv_heads);
    r.k[0] = *reinterpret_cast<const u32x4_t*>(p.k + off);
    r.k[1] = *reinterpret_cast<const u32x4_t*>(p.k + off + kHeadDim);
    r.v[0] = *reinterpret_cast<const u32x4_t*>(p.v + off);
    r.v[1] = *reinterpret_cast<const u32x4_t*>(p.v + off + kHeadDim);
  };
  auto store_tile = [&](const TileRegs& r, int stage, int it) {
    uint8_t* sk = s_buf[kh][stage];
    uint8_t* svt = sk + kKBytes;
    const int base = (tile0 + it) * kTileKeys;
    const bool tile_ok = it < T;
    const bool v0_ok = tile_ok && base + 2 * lv_kp < kv_end;
    const bool v1_ok = tile_ok && base + 2 * lv_kp + 1 < kv_end;
    const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = 2 * lv_kp + e;
      *reinterpret_cast<u32x4_t*>(sk + key * kKRowBytes + ((lv_c ^ (key & 15)) << 4)) =
          (e ? v1_ok : v0_ok) ? r.k[e] : zero;
    }
    const u32x4_t va = v0_ok ? r.v[0] : zero;
    const u32x4_t vb = v1_ok ? r.v[1] : zero;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // dims 8*lv_c + 2w (low halves) and + 2w + 1 (high halves)
      const uint32_t lo = __builtin_amdgcn_perm(vb[w], va[w], 0x05040100u);
      const uint32_t hi = __builtin_amdgcn_perm(vb[w], va[w], 0x07060302u);
      const int d = lv_c * 8 + 2 * w;
      *reinterpret_cast<uint32_t*>(svt + d * kVtRowBytes + lv_kp * 4) = lo;
      *reinterpret_cast<uint32_t*>(svt + (d + 1) * kVtRowBytes + lv_kp * 4) = hi;
    }
  };

  f32x16_t o[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mb][i] = 0.f;
  float m_run = -INFINITY;  // reference max of this row (log2 domain)
  float l_run = 0.f;        // this lane's share of the row sum

  auto compute_tile = [&](int it, int stage) {
    const uint8_t* sk = s_buf[kh][stage];
    const uint8_t* svt = sk + kKBytes;
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
      kf[s] = *reinterpret_cast<const u32x4_t*>(sk + col * kKRowBytes + ((c ^ (col & 15)) << 4));
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int s = 0; s < 8; ++s)
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[s]), as_bf16x8(qf[s]), st, 0, 0, 0);
    // Online softmax over this lane's 16 keys of its row (log2 domain).
    const int kbase = (tile0 + it) * kTileKeys + 4 * hh;
    float sv[16];
    float mloc = -INFINITY;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int key = kbase + 8 * a + b;
        const float x = (it < T && key <= my_limit) ? st[4 * a + b] * p.scale_log2 : -INFINITY;
        sv[4 * a + b] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, other_half(mloc));
    const bool raise = mloc > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      // A row with no visible key so far keeps m = -inf (its sums are 0);
      // guard the difference so -inf - -inf never makes a NaN.
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
    // P^T operand for key steps 0 and 1: keys 16ks + 4hh + 0..3, 16ks + 8 + 4hh + 0..3.
    u32x4_t pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      pf[ks][0] = pack_bf16x2(sv[8 * ks + 0], sv[8 * ks + 1]);
      pf[ks][1] = pack_bf16x2(sv[8 * ks + 2], sv[8 * ks + 3]);
      pf[ks][2] = pack_bf16x2(sv[8 * ks + 4], sv[8 * ks + 5]);
      pf[ks][3] = pack_bf16x2(sv[8 * ks + 6], sv[8 * ks + 7]);
    }
    // O^T += V^T P^T.
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int d = mb * 32 + col;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // (4-byte reads: the 68-byte rows keep only 4-byte alignment)
        const uint32_t* vrow = reinterpret_cast<const uint32_t*>(svt + d * kVtRowBytes + (16 * ks + 4 * hh) * 2);
        const u32x4_t vf = u32x4_t{vrow[0], vrow[1], vrow[4], vrow[5]};
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[ks]), o[mb], 0, 0, 0);
      }
    }
  };

  // Pipeline: a ring of two tiles in registers per half; tile it goes to
  // LDS stage it % 2, its ring slot is refilled with tile it + 2, one
  // barrier, then it is computed.  Two stages suffice: a wave reaches tile
  // it + 2's store only after the barrier of tile it + 1, which every wave
  // passes after computing tile it.  Ring loads past the half's last tile
  // re-read a valid page and are never stored.
  TileRegs rr[2];
  if (T > 0) {
    load_tile(rr[0], 0);
    issue_order_barrier();
    load_tile(rr[1], 1);
    issue_order_barrier();
  }
  load_q();
  issue_order_barrier();
#define PA_CHUNK_STEP(K, IT, RELOAD)           \
  do {                                         \
    store_tile(rr[K], (IT) & 1, IT);           \
    issue_order_barrier();                     \
    if (RELOAD) load_tile(rr[K], (IT) + 2);    \
    issue_order_barrier();                     \
    __syncthreads();                           \
    compute_tile(IT, (IT) & 1);                \
  } while (0)
  int it = 0;
  for (; it + 4 <= T; it += 2) {  // every reload is a real tile
    PA_CHUNK_STEP(0, it, true);
    PA_CHUNK_STEP(1, it + 1, true);
  }
  // The last 0 .. 3 tiles.
  if (it < T) PA_CHUNK_STEP(0, it, it + 2 < T);
  if (it + 1 < T) PA_CHUNK_STEP(1, it + 1, false);
  if (it + 2 < T) PA_CHUNK_STEP(0, it + 2, false);
#undef PA_CHUNK_STEP
  __syncthreads();  // all computes done before the tile area is reused

  // Merge the key halves: half 1 hands (m, l, o) to half 0 through LDS, in
  // four rounds of 16 accumulators (16 KiB per round, inside the tile area).
  float* xbuf = reinterpret_cast<float*>(&s_buf[0][0][0]);  // [rg][18][64] floats
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if (kh == 1) {
      float* dst = xbuf + (size_t)rg * 18 * 64;
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[i * 64 + lane] = o[mb][i];
      if (mb == 0) {
        dst[16 * 64 + lane] = m_run;
        dst[17 * 64 + lane] = l_run;
      }
    }
    __syncthreads();
    if (kh == 0) {
      const float* src = xbuf + (size_t)rg * 18 * 64;
      const float m1 = src[16 * 64 + lane];
      const float l1 = src[17 * 64 + lane];
      const float M = fmaxf(m_run, m1);
      const float Mu = (M == -INFINITY) ? 0.f : M;
      const float s0 = fast_exp2(m_run - Mu);
      const float s1 = fast_exp2(m1 - Mu);
#pragma unroll
      for (int i = 0; i < 16; ++i) o[mb][i] = o[mb][i] * s0 + src[i * 64 + lane] * s1;
      if (mb == 3) {
        l_run = l_run * s0 + l1 * s1;
        m_run = M;
      }
    }
    __syncthreads();
  }
  if (kh == 1 || !row_live) return;

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  uint16_t* orow = p.out + ((size_t)(q_row0 + row) * p.num_q_heads + h) * kHeadDim;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d = mb * 32 + 8 * a + 4 * hh;
      uint2 w;
      w.x = pack_bf16x2(o[mb][4 * a + 0] * inv, o[mb][4 * a + 1] * inv);
      w.y = pack_bf16x2(o[mb][4 * a + 2] * inv, o[mb][4 * a + 3] * inv);
      *reinterpret_cast<uint2*>(orow + d) = w;
    }
  if (hh == 0 && p.lse) p.lse[(size_t)(q_row0 + row) * p.num_q_heads + h] = (m_run + fast_log2(l_tot)) * kLn2;
}

}  // namespace

hipError_t launch_chunk(const ChunkParams& p, unsigned grid, hipStream_t s) {
  ChunkParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&chunk_kernel), dim3(grid), dim3(kThreads), args, 0, s);
}

}  // namespace pa
