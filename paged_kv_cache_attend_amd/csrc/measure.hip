// measure.hip -- the measured ceilings of pa_measure.h: a read-only stream of
// scattered 4 KiB K/V tiles with the decode kernel's loads, and a bf16
// matrix-core throughput loop.  Neither computes attention.

#include <hip/hip_runtime.h>

#include "device.h"
#include "pa_measure.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

// Wave w of a workgroup takes tiles w, w + 4, ... of the workgroup's range;
// per tile a lane loads the same four 16-byte chunks of K and of V as the
// decode kernel (chunk lane + 64 k), two tiles ahead of their use.
__global__ __launch_bounds__(kThreads, 2) void read_tiles_kernel(const u32x4_t* __restrict__ k,
                                                                 const u32x4_t* __restrict__ v,
                                                                 const int32_t* __restrict__ tiles,
                                                                 int64_t num_tiles, int tiles_per_wg,
                                                                 uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t first = (int64_t)blockIdx.x * tiles_per_wg;
  const int64_t last = first + tiles_per_wg < num_tiles ? first + tiles_per_wg : num_tiles;
  uint32_t acc = 0;
  for (int64_t t = first + wave; t < last; t += 4 * 3) {
    u32x4_t kk[3][4], vv[3][4];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int64_t ti = t + 4 * r < last ? t + 4 * r : t;  // repeat a valid tile past the end
      const size_t base = (size_t)tiles[ti] * 256 + lane;
#pragma unroll
      for (int c = 0; c < 4; ++c) kk[r][c] = stream_load(k + base + 64 * c);
#pragma unroll
      for (int c = 0; c < 4; ++c) vv[r][c] = stream_load(v + base + 64 * c);
    }
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc ^= kk[r][c][0] ^ kk[r][c][3] ^ vv[r][c][1] ^ vv[r][c][2];
  }
  __shared__ uint32_t s_acc[4];
  acc = (uint32_t)wave_sum_i32((int)acc);
  if (lane == 0) s_acc[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3];
}

__global__ __launch_bounds__(kThreads, 2) void mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((lane + e) & 7);
    b[e] = (__bf16)(float)((lane * 3 + e) & 7);
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_measure_read_tiles(const void* k_cache, const void* v_cache, const int32_t* tiles,
                                           int64_t num_tiles, int32_t tiles_per_wg, uint32_t* sink,
                                           void* stream) {
  if (num_tiles < 0 || tiles_per_wg < 1) return PA_ERR_BAD_SHAPE;
  if (num_tiles == 0) return PA_OK;
  if (!k_cache || !v_cache || !tiles || !sink) return PA_ERR_NULL_ARG;
  const int64_t grid = (num_tiles + tiles_per_wg - 1) / tiles_per_wg;
  if (grid > 0x7fffffff) return PA_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(pa::read_tiles_kernel, dim3((unsigned)grid), dim3(pa::kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const pa::u32x4_t*>(k_cache),
                     static_cast<const pa::u32x4_t*>(v_cache), tiles, num_tiles, (int)tiles_per_wg, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

extern "C" pa_status pa_measure_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (workgroups < 1 || iters < 1) return PA_ERR_BAD_SHAPE;
  if (!sink) return PA_ERR_NULL_ARG;
  hipLaunchKernelGGL(pa::mfma_kernel, dim3((unsigned)workgroups), dim3(pa::kThreads), 0,
                     static_cast<hipStream_t>(stream), (int)iters, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
