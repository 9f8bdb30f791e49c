// noalloc.hip -- pa_attend without a caller workspace (pa_attend_noalloc).
//
// The split-KV counters and partials live in `scratch`, a file-scope device
// array: every GPU the library runs on holds its own copy from module load
// until the process ends, so a call needs no hipMalloc, hipFree or workspace
// argument (callers under graph capture, or that may not allocate).
//
// In host code the array's name only stands for the symbol; its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and that address is what the kernels receive.  The lookup also
// enqueues a kernel that zeroes the counter region on the caller's stream; a
// call that completes leaves its counters at zero, so later calls need no
// clearing.  Calls that overlap on one GPU share the array and race.

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "pa.h"

namespace pa {
namespace {

static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mutex;

// This device's address of `scratch`, fetched (and its counter region zeroed
// on `stream`) on first use.  Null if the lookup fails.
void* device_scratch(int dev, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  // The counters sit at the start of the workspace, one int32 per (slot, KV
  // head) of the call; zero enough for any shape the buffer can serve (the
  // partials need no initial value).
  constexpr size_t kZeroInts = (size_t)1 << 20;  // 4 MiB: 1 Mi (slot, KV head) pairs
  static_assert(kZeroInts * sizeof(int32_t) <= PA_NOALLOC_SCRATCH_BYTES, "zeroed region exceeds the buffer");
  if (launch_zero_i32(static_cast<int32_t*>(ptr), kZeroInts, stream) != hipSuccess) return nullptr;
  g_scratch_ptr[dev] = ptr;
  return ptr;
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_attend_noalloc(const pa_shape* shape, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_table,
                                       const int32_t* ctx_lens, const int32_t* q_lens, float scale,
                                       void* out, float* lse, void* stream) {
  if (!shape) return PA_ERR_NULL_ARG;
  // Shape errors first (pa_workspace_size is 0 for a shape pa_attend rejects;
  // attend_bf16 then returns the precise status).
  const size_t need = pa_workspace_size(shape);
  if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH_LIMIT;
  // Counters: one per (slot, KV head) on the decode path, one per 128-row
  // tile of a (slot, query head) on the chunk path; bounded by slots x query
  // heads x row tiles either way.
  const size_t counters = (size_t)(shape->num_seqs > 0 ? shape->num_seqs : 0) *
                          (size_t)(shape->num_q_heads > 0 ? shape->num_q_heads : 0) *
                          (size_t)((shape->max_q_len + 127) / 128 > 1 ? (shape->max_q_len + 127) / 128 : 1);
  if (need > 0 && counters > ((size_t)1 << 20)) return PA_ERR_SCRATCH_LIMIT;  // beyond the zeroed region
  void* ws = nullptr;
  if (need > 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= pa::kMaxDevices) return PA_ERR_LAUNCH;
    ws = pa::device_scratch(dev, static_cast<hipStream_t>(stream));
    if (!ws) return PA_ERR_LAUNCH;
  }
  return pa::attend_bf16(shape, q, k_cache, v_cache, block_table, ctx_lens, q_lens, scale, out, lse, ws,
                         need > 0 ? PA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
