// combine.hip -- log-sum-exp merge of split-KV partials.
//
// Softmax over a union of disjoint key ranges weighs range p by exp(lse_p)
// relative to the others, so for one output row
//     M = max_p lse_p,  w_p = exp(lse_p - M),
//     lse = M + ln sum_p w_p,  out = sum_p w_p o_p / sum_p w_p.
// Partials with lse_p = -inf (empty ranges) weigh zero and their outputs are
// never read (they may hold anything, NaN included).  A row whose partials are
// all -inf -- a slot with no keys -- is left untouched.
//
// Layout: half a wave (32 lanes) per row, four fp32 dims per lane per step,
// so one row of 128 dims is a single coalesced 512-byte read per partial.
// The work is a few percent of the decode kernel's bytes; it is bound by the
// partial reads.

#include "device.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 32;
constexpr int kRowsPerBlock = kThreads / kLanesPerRow;

__device__ __forceinline__ float half_wave_max(float x) {
  for (int off = 16; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 32));
  return x;
}
__device__ __forceinline__ float half_wave_sum(float x) {
  for (int off = 16; off > 0; off >>= 1) x += __shfl_xor(x, off, 32);
  return x;
}

__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams c) {
  const int sub = threadIdx.x & (kLanesPerRow - 1);
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x / kLanesPerRow);
  if (row >= c.rows) return;  // whole half-wave leaves together
  const size_t rows = (size_t)c.rows;
  const float* pl = c.part_lse + row;

  float M = -INFINITY;
  for (int p = sub; p < c.num_parts; p += kLanesPerRow) M = fmaxf(M, pl[(size_t)p * rows]);
  M = half_wave_max(M);
  if (M == -INFINITY) return;  // no live partial: leave the row untouched

  float W = 0.f;
  for (int p = sub; p < c.num_parts; p += kLanesPerRow) {
    const float l = pl[(size_t)p * rows];
    W += (l == -INFINITY) ? 0.f : __expf(l - M);
  }
  W = half_wave_sum(W);
  const float inv = 1.f / W;

  const int nvec = c.head_dim / 4;
  for (int v = sub; v < nvec; v += kLanesPerRow) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = 0; p < c.num_parts; ++p) {
      const float l = pl[(size_t)p * rows];
      if (l == -INFINITY) continue;
      const float w = __expf(l - M);
      const float4 o = reinterpret_cast<const float4*>(c.part_out + ((size_t)p * rows + row) * c.head_dim)[v];
      a.x = fmaf(w, o.x, a.x);
      a.y = fmaf(w, o.y, a.y);
      a.z = fmaf(w, o.z, a.z);
      a.w = fmaf(w, o.w, a.w);
    }
    uint2 packed;
    packed.x = pack_bf16x2(a.x * inv, a.y * inv);
    packed.y = pack_bf16x2(a.z * inv, a.w * inv);
    reinterpret_cast<uint2*>(c.out + (size_t)row * c.head_dim)[v] = packed;
  }
  if (sub == 0 && c.lse) c.lse[row] = M + __logf(W);
}

}  // namespace

hipError_t launch_combine(const CombineParams& c, hipStream_t s) {
  const unsigned grid = (unsigned)((c.rows + kRowsPerBlock - 1) / kRowsPerBlock);
  CombineParams arg = c;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel), dim3(grid), dim3(kThreads), args, 0, s);
}

}  // namespace pa
