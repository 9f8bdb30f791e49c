// gather.hip -- page-table gather to a dense buffer, and precondition checks.
//
// gather_kernel copies each active slot's keys (or values) through the same
// page addressing the attention kernels use (cache_offset in device.h), so a
// byte-for-byte comparison with an independent host gather checks the
// addressing itself.  One workgroup per (slot, logical page); each thread
// moves 16-byte chunks.
//
// validate_kernel checks the device-side preconditions of pa_attend (table
// entries inside the pool, lengths inside their declared maxima) with one
// workgroup, accumulating a bit mask in LDS and storing it once.

#include "device.h"
#include "pa.h"

namespace pa {

namespace {

__global__ __launch_bounds__(256) void gather_kernel(GatherParams p) {
  const int seq = blockIdx.x / p.max_pages;
  const int page = blockIdx.x % p.max_pages;
  const int n = p.ctx_lens[seq];
  if (page * kBlockSize >= n) return;
  const int32_t phys = p.block_table[(size_t)seq * p.max_blocks + page];
  const int chunks = p.num_kv_heads * kBlockSize * (kHeadDim / 8);
  for (int e = threadIdx.x; e < chunks; e += blockDim.x) {
    const int c = e % (kHeadDim / 8);
    const int slot = (e / (kHeadDim / 8)) % kBlockSize;
    const int g = e / (kBlockSize * (kHeadDim / 8));
    const int j = page * kBlockSize + slot;
    if (j >= n || j >= p.max_ctx) continue;
    const uint4 val = *reinterpret_cast<const uint4*>(p.cache + cache_offset(phys, g, slot, c * 8, p.num_kv_heads));
    const size_t dst = (((size_t)seq * p.max_ctx + j) * p.num_kv_heads + g) * kHeadDim + c * 8;
    *reinterpret_cast<uint4*>(p.dst + dst) = val;
  }
}

__global__ __launch_bounds__(256) void validate_kernel(ValidateParams p) {
  __shared__ int s_bits;
  __shared__ long long s_total;
  if (threadIdx.x == 0) {
    s_bits = 0;
    s_total = 0;
  }
  __syncthreads();
  int bits = 0;
  long long total = 0;
  for (int r = threadIdx.x; r < p.num_seqs; r += blockDim.x) {
    const int n = p.ctx_lens[r];
    const int m = p.q_lens[r];
    if (n < 0 || n > p.max_ctx || (long long)n > (long long)kBlockSize * p.max_blocks) bits |= PA_BAD_CTX_LEN;
    if (m < 0 || m > p.max_q || (n > 0 && m > n)) bits |= PA_BAD_Q_LEN;
    if (m > 0) total += m;
  }
  // Table entries of every slot's live pages.
  for (int r = 0; r < p.num_seqs; ++r) {
    const int n = p.ctx_lens[r];
    if (n <= 0 || (long long)n > (long long)kBlockSize * p.max_blocks) continue;
    const int pages = (n + kBlockSize - 1) / kBlockSize;
    for (int j = threadIdx.x; j < pages; j += blockDim.x) {
      const int32_t b = p.block_table[(size_t)r * p.max_blocks + j];
      if (b < 0 || (int64_t)b >= p.num_blocks) bits |= PA_BAD_BLOCK_ID;
    }
  }
  // Split-KV counters: every call that completes leaves them at zero.
  for (int i = threadIdx.x; i < p.num_counters; i += blockDim.x)
    if (p.counters[i] != 0) bits |= PA_BAD_WORKSPACE;
  if (bits) atomicOr(&s_bits, bits);
  if (total) atomicAdd(reinterpret_cast<unsigned long long*>(&s_total), (unsigned long long)total);
  __syncthreads();
  if (threadIdx.x == 0) {
    int out = s_bits;
    if (s_total > (long long)p.total_q) out |= PA_BAD_TOTAL_Q;
    *p.error_word = out;
  }
}

}  // namespace

hipError_t launch_gather(const GatherParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)p.num_seqs * (unsigned)p.max_pages;
  GatherParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gather_kernel), dim3(grid), dim3(256), args, 0, s);
}

hipError_t launch_validate(const ValidateParams& p, hipStream_t s) {
  ValidateParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&validate_kernel), dim3(1), dim3(256), args, 0, s);
}

}  // namespace pa
