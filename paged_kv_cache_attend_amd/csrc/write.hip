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

}  // namespace

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
