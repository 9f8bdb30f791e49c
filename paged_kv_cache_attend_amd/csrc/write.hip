// write.hip -- appending new K/V rows to their pages, and whole-block copies.
//
// write_kv_kernel is the write half of paged allocation (inference-
// optimisation chapter, section 8.3.1, Fig. 8-10): new token i of a slot with
// n visible tokens and m new ones sits at position n - m + i, i.e. in block
// table[(n - m + i) / 16] at slot (n - m + i) % 16.  One workgroup per
// (slot, 16 new rows); each thread moves 16-byte chunks, so a row of
// Hkv x 128 bf16 is written with coalesced 16-byte stores per (KV head,
// 256-byte row).  Positions are resolved through cache_offset, the same
// routine the attention kernels read with.
//
// copy_blocks_kernel makes the copies of copy-on-write (section 8.3.2,
// Fig. 8-15): one workgroup per (copy, KV head, K or V) moves one 4 KiB tile.
//
// Both kernels are bandwidth-trivial next to attention; they skip (rather
// than write through) a position beyond the block table, a block id outside
// the pool, or a source row beyond total_q.

#include "device.h"

namespace pa {

namespace {

constexpr int kRowsPerGroup = 16;
constexpr int kChunksPerRow = kHeadDim / 8;  // 16-byte chunks per (row, head)

__global__ __launch_bounds__(256) void write_kv_kernel(WriteParams p) {
  const int groups = (p.max_q_len + kRowsPerGroup - 1) / kRowsPerGroup;
  const int seq = blockIdx.x / groups;
  const int i0 = (blockIdx.x % groups) * kRowsPerGroup;
  const int lane = threadIdx.x & 63;
  const int m = scalar_load_i32(p.q_lens, seq);
  const int n = scalar_load_i32(p.ctx_lens, seq);
  if (m <= 0 || n <= 0 || i0 >= m) return;
  const int rows = min(kRowsPerGroup, m - i0);
  const int row0 = q_row_offset(p.q_lens, seq, lane) + i0;
  const int per_row = p.num_kv_heads * kChunksPerRow;
  const int32_t* bt = p.block_table + (size_t)seq * p.max_blocks;
  for (int e = threadIdx.x; e < rows * per_row * 2; e += blockDim.x) {
    const int which = e / (rows * per_row);  // 0: K, 1: V
    const int f = e % (rows * per_row);
    const int r = f / per_row;
    const int g = (f % per_row) / kChunksPerRow;
    const int c = f % kChunksPerRow;
    const int j = n - m + i0 + r;
    if (j < 0 || j >= kBlockSize * p.max_blocks || row0 + r >= p.total_q) continue;
    const int32_t phys = bt[j / kBlockSize];
    if (phys < 0 || (int64_t)phys >= p.num_blocks) continue;
    const size_t src = (((size_t)(row0 + r)) * p.num_kv_heads + g) * kHeadDim + c * 8;
    const size_t dst = cache_offset(phys, g, j % kBlockSize, c * 8, p.num_kv_heads);
    const u32x4_t* from = reinterpret_cast<const u32x4_t*>((which ? p.v_new : p.k_new) + src);
    *reinterpret_cast<u32x4_t*>((which ? p.v_cache : p.k_cache) + dst) = *from;
  }
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyParams p) {
  const int copy = blockIdx.x / (p.num_kv_heads * 2);
  const int g = (blockIdx.x / 2) % p.num_kv_heads;
  const int which = blockIdx.x % 2;
  const int32_t src = p.src[copy];
  const int32_t dst = p.dst[copy];
  if (src < 0 || dst < 0 || (int64_t)src >= p.num_blocks || (int64_t)dst >= p.num_blocks) return;
  uint16_t* cache = which ? p.v_cache : p.k_cache;
  const u32x4_t* from = reinterpret_cast<const u32x4_t*>(cache + cache_offset(src, g, 0, 0, p.num_kv_heads));
  u32x4_t* to = reinterpret_cast<u32x4_t*>(cache + cache_offset(dst, g, 0, 0, p.num_kv_heads));
  constexpr int kVecs = kBlockSize * kHeadDim * 2 / 16;  // 256 per 4 KiB tile
  for (int e = threadIdx.x; e < kVecs; e += blockDim.x) to[e] = from[e];
}

// Quantising append (the chapter's section 8.4.2, Fig. 8-23): one thread per
// (K or V, new row, KV head, group of 32 dims).  The thread reads the group's
// 64 bytes of bf16, and writes its codes (32, 32 or 16 bytes) and, for the
// grouped formats, its fp16 scale.  Encoding rules as declared in pa.h: fp32
// arithmetic, correctly rounded division by the stored (fp16) scale, codes
// rounded half away from zero, a zero scale stored as +0; FP8 through the
// hardware E4M3 conversion
// (round to nearest even) after clamping to +-448.
template <int F>
__global__ __launch_bounds__(256) void write_kv_quant_kernel(WriteQuantParams q) {
  const WriteParams& p = q.w;
  const int groups = (p.max_q_len + kRowsPerGroup - 1) / kRowsPerGroup;
  const int seq = blockIdx.x / groups;
  const int i0 = (blockIdx.x % groups) * kRowsPerGroup;
  const int lane = threadIdx.x & 63;
  const int m = scalar_load_i32(p.q_lens, seq);
  const int n = scalar_load_i32(p.ctx_lens, seq);
  if (m <= 0 || n <= 0 || i0 >= m) return;
  const int rows = min(kRowsPerGroup, m - i0);
  const int row0 = q_row_offset(p.q_lens, seq, lane) + i0;
  const int per_row = p.num_kv_heads * 4;  // (head, group) pairs per row
  const int32_t* bt = p.block_table + (size_t)seq * p.max_blocks;
  for (int e = threadIdx.x; e < 2 * rows * per_row; e += blockDim.x) {
    const int which = e / (rows * per_row);  // 0: K, 1: V
    const int f = e % (rows * per_row);
    const int r = f / per_row;
    const int g = (f % per_row) / 4;
    const int grp = f % 4;
    const int j = n - m + i0 + r;
    if (j < 0 || j >= kBlockSize * p.max_blocks || row0 + r >= p.total_q) continue;
    const int32_t phys = bt[j / kBlockSize];
    if (phys < 0 || (int64_t)phys >= p.num_blocks) continue;
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(
        (which ? p.v_new : p.k_new) + (((size_t)(row0 + r)) * p.num_kv_heads + g) * kHeadDim + grp * 32);
    float x[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4_t w = src[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * c + 2 * i] = bf16_lo(w[i]);
        x[8 * c + 2 * i + 1] = bf16_hi(w[i]);
      }
    }
    const size_t rowi = tile_index(phys, g, p.num_kv_heads) * kBlockSize + (size_t)(j % kBlockSize);
    uint8_t* codes = reinterpret_cast<uint8_t*>(which ? p.v_cache : p.k_cache);
    if constexpr (F == kFmtFP8) {
      const float sc = which ? q.v_scale : q.k_scale;
      u32x4_t out[2];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = fminf(fmaxf(x[4 * c + i] / sc, -448.f), 448.f);
        int word = 0;
        word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], word, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
        out[c / 4][c % 4] = (uint32_t)word;
      }
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + rowi * kHeadDim + grp * 32);
      dst[0] = out[0];
      dst[1] = out[1];
    } else {
      float d;
      if constexpr (F == kFmtQ8) {
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
        d = amax / 127.f;
      } else {
        float best = x[0];
#pragma unroll
        for (int i = 1; i < 32; ++i) best = fabsf(x[i]) > fabsf(best) ? x[i] : best;
        d = best / -8.f;
      }
      const _Float16 h = (_Float16)d;
      const float ds = (float)h;
      const uint16_t h_bits = ds == 0.f ? (uint16_t)0 : __builtin_bit_cast(uint16_t, h);  // zero as +0
      constexpr float kLo = F == kFmtQ8 ? -127.f : -8.f;
      constexpr float kHi = F == kFmtQ8 ? 127.f : 7.f;
      int code[32];
#pragma unroll
      for (int i = 0; i < 32; ++i)
        code[i] = ds == 0.f ? 0 : (int)fminf(fmaxf(roundf(x[i] / ds), kLo), kHi);
      uint16_t* scales = which ? q.v_scales : q.k_scales;
      scales[rowi * 4 + grp] = h_bits;
      if constexpr (F == kFmtQ8) {
        u32x4_t out[2];
#pragma unroll
        for (int w = 0; w < 8; ++w)
          out[w / 4][w % 4] = (uint32_t)(code[4 * w] & 255) | ((uint32_t)(code[4 * w + 1] & 255) << 8) |
                              ((uint32_t)(code[4 * w + 2] & 255) << 16) | ((uint32_t)(code[4 * w + 3] & 255) << 24);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + rowi * kHeadDim + grp * 32);
        dst[0] = out[0];
        dst[1] = out[1];
      } else {
        u32x4_t out;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t word = 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) word |= (uint32_t)(code[8 * w + i] + 8) << (4 * i);
          out[w] = word;
        }
        *reinterpret_cast<u32x4_t*>(codes + rowi * (kHeadDim / 2) + grp * 16) = out;
      }
    }
  }
}

}  // namespace

hipError_t launch_write_kv_quant(const WriteQuantParams& p, int format, hipStream_t s) {
  const long long groups = (p.w.max_q_len + kRowsPerGroup - 1) / kRowsPerGroup;
  const long long grid = groups * p.w.num_seqs;
  if (grid <= 0) return hipSuccess;
  const void* fn = nullptr;
  switch (format) {
    case kFmtFP8: fn = reinterpret_cast<const void*>(&write_kv_quant_kernel<kFmtFP8>); break;
    case kFmtQ8: fn = reinterpret_cast<const void*>(&write_kv_quant_kernel<kFmtQ8>); break;
    case kFmtQ4: fn = reinterpret_cast<const void*>(&write_kv_quant_kernel<kFmtQ4>); break;
    default: return hipErrorInvalidValue;
  }
  WriteQuantParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, s);
}

hipError_t launch_write_kv(const WriteParams& p, hipStream_t s) {
  const long long groups = (p.max_q_len + kRowsPerGroup - 1) / kRowsPerGroup;
  const long long grid = groups * p.num_seqs;
  if (grid <= 0) return hipSuccess;
  WriteParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&write_kv_kernel), dim3((unsigned)grid), dim3(256),
                         args, 0, s);
}

hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t s) {
  const long long grid = (long long)p.num_copies * p.num_kv_heads * 2;
  if (grid <= 0) return hipSuccess;
  CopyParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&copy_blocks_kernel), dim3((unsigned)grid),
                         dim3(256), args, 0, s);
}

}  // namespace pa
