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
// Workgroup: 4 waves, 128 query rows (32 per wave) of one (slot, query head).
// Loop over 32-key tiles (two 16-token pages):
//   1. all 256 threads load the tile's K and V rows through the block table
//      (16-byte loads, one key row per 8 / 16 threads) into registers one tile
//      ahead, then store them to LDS: K row-major with XOR-swizzled 16-byte
//      chunks, V transposed (dim-major, rows padded to 72 bytes so the
//      transposed reads are conflict free);
//   2. each wave computes S^T = K Q^T (32 keys x 32 rows, 8 MFMAs over the 128
//      dims).  In the MFMA output layout a lane holds 16 keys of ONE query row,
//      so the row max and row sum of the online softmax are mostly in-lane;
//      the other 16 keys of the row sit in lane + 32;
//   3. probabilities are rounded to bf16 and used directly, from registers, as
//      the B operand of O^T += V^T P^T (4 x 32 dims, 2 key steps, 8 MFMAs); the
//      V^T A operand is read from the transposed LDS tile with the same key
//      order the probabilities already have.
// Keys >= n are never loaded (zeros) and get -inf scores.

#include "device.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kTileKeys = 32;
constexpr int kKRowBytes = kHeadDim * 2;         // 256
constexpr int kVtRowBytes = kTileKeys * 2 + 8;   // 72: padded dim-major row
constexpr int kKBytes = kTileKeys * kKRowBytes;  // 8 KiB
constexpr int kVtBytes = kHeadDim * kVtRowBytes; // 9 KiB

static_assert(kChunkRows == 4 * 32, "four waves of 32 rows");

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

__global__ __launch_bounds__(kThreads, 2) void chunk_kernel(ChunkParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kKBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_vt[kVtBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;  // query row within the wave / MFMA column
  const int hh = lane >> 5;   // lane half

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = wg % p.q_tiles;
  const int sh = wg / p.q_tiles;
  const int h = sh % p.num_q_heads;
  const int seq = sh / p.num_q_heads;
  const int g = h / (p.num_q_heads / p.num_kv_heads);

  const int m = p.q_lens[seq];
  const int n = p.ctx_lens[seq];
  if (m <= 0 || n <= 0 || qt * kChunkRows >= m) return;
  const int q_row0 = q_row_offset(p.q_lens, seq, lane);
  const int row = qt * kChunkRows + wave * 32 + col;  // row within the slot
  const bool row_live = row < m;

  // Q^T operand: lane (row, half) holds dims (hh*8 + s)*8 .. +8 for step s.
  uint4 qf[8];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(p.q) +
                      ((size_t)(q_row0 + row) * p.num_q_heads + h) * (kHeadDim / 8);
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = row_live ? qp[hh * 8 + s] : make_uint4(0u, 0u, 0u, 0u);
  }

  // Keys this workgroup needs.
  int kv_end = n;
  if (p.causal) {
    const int last_row = min(m, (qt + 1) * kChunkRows) - 1;
    kv_end = min(n, n - m + last_row + 1);
  }
  const int ntiles = (kv_end + kTileKeys - 1) / kTileKeys;
  const int my_limit = p.causal ? (n - m + row) : (n - 1);  // last visible key of this row

  const int32_t* bt = p.block_table + (size_t)seq * p.max_blocks;
  const uint16_t* kpool = p.k;
  const uint16_t* vpool = p.v;

  // Loader roles.  K: key kk = tid / 8, chunks 2*(tid%8), +1.  V: keys
  // 2*(tid/16), +1, chunk tid % 16.
  const int lk_key = tid >> 3;
  const int lk_c = (tid & 7) * 2;
  const int lv_kp = tid >> 4;
  const int lv_c = tid & 15;
  uint4 rk[2], rv[2];
  auto load_tile = [&](int kt) {
    const int base = kt * kTileKeys;
    {
      const int j = base + lk_key;
      if (j < kv_end) {
        const uint4* src = reinterpret_cast<const uint4*>(
            kpool + cache_offset(bt[j >> 4], g, j & 15, lk_c * 8, p.num_kv_heads));
        rk[0] = src[0];
        rk[1] = src[1];
      } else {
        rk[0] = rk[1] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = base + 2 * lv_kp + e;
      if (j < kv_end) {
        rv[e] = *reinterpret_cast<const uint4*>(
            vpool + cache_offset(bt[j >> 4], g, j & 15, lv_c * 8, p.num_kv_heads));
      } else {
        rv[e] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = lk_c + e;
      *reinterpret_cast<uint4*>(s_k + lk_key * kKRowBytes + ((c ^ (lk_key & 15)) << 4)) = rk[e];
    }
    const uint32_t a[4] = {rv[0].x, rv[0].y, rv[0].z, rv[0].w};
    const uint32_t b[4] = {rv[1].x, rv[1].y, rv[1].z, rv[1].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // dims 8*lv_c + 2w (low halves) and + 2w + 1 (high halves)
      const uint32_t lo = (a[w] & 0xffffu) | (b[w] << 16);
      const uint32_t hi = (a[w] >> 16) | (b[w] & 0xffff0000u);
      const int d = lv_c * 8 + 2 * w;
      *reinterpret_cast<uint32_t*>(s_vt + d * kVtRowBytes + lv_kp * 4) = lo;
      *reinterpret_cast<uint32_t*>(s_vt + (d + 1) * kVtRowBytes + lv_kp * 4) = hi;
    }
  };

  f32x16_t o[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[mb][i] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  if (ntiles > 0) load_tile(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (kt + 1 < ntiles) load_tile(kt + 1);

    // S^T = K Q^T: A = K rows (key = col), B = Q^T (row = col).
    f32x16_t st;
#pragma unroll
    for (int i = 0; i < 16; ++i) st[i] = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = hh * 8 + s;
      const uint4 kf = *reinterpret_cast<const uint4*>(s_k + col * kKRowBytes + ((c ^ (col & 15)) << 4));
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[s]), st, 0, 0, 0);
    }

    // Online softmax over this lane's 16 keys of its row (log2 domain).
    const int kbase = kt * kTileKeys + 4 * hh;
    float sv[16];
    float mloc = -INFINITY;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int key = kbase + 8 * a + b;
        const float x = (key <= my_limit) ? st[4 * a + b] * p.scale_log2 : -INFINITY;
        sv[4 * a + b] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = fast_exp2(sv[i] - m_use);
      lsum += sv[i];
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[mb][i] *= alpha;

    // P^T operand for key steps 0 and 1: keys 16ks + 4hh + 0..3, 16ks + 8 + 4hh + 0..3.
    uint4 pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      pf[ks].x = pack_bf16x2(sv[8 * ks + 0], sv[8 * ks + 1]);
      pf[ks].y = pack_bf16x2(sv[8 * ks + 2], sv[8 * ks + 3]);
      pf[ks].z = pack_bf16x2(sv[8 * ks + 4], sv[8 * ks + 5]);
      pf[ks].w = pack_bf16x2(sv[8 * ks + 6], sv[8 * ks + 7]);
    }

    // O^T += V^T P^T.
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int d = mb * 32 + col;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const uint8_t* vrow = s_vt + d * kVtRowBytes + (16 * ks + 4 * hh) * 2;
        const uint2 v0 = *reinterpret_cast<const uint2*>(vrow);
        const uint2 v1 = *reinterpret_cast<const uint2*>(vrow + 16);
        const uint4 vf = make_uint4(v0.x, v0.y, v1.x, v1.y);
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[ks]), o[mb], 0, 0, 0);
      }
    }
  }

  if (!row_live) return;
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
