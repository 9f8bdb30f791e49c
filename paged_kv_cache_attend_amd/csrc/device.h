// device.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// Native vectors for 16-byte data in registers (HIP's uint4 is a struct whose
// copies can end up in scratch memory).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Page addressing.  Logical key j of a slot lives in logical block j / 16 at
// slot j % 16; the block table names the physical block.  One (physical
// block, KV head) tile is 16 x 128 bf16 = 4 KiB, contiguous.  Every kernel
// that touches the cache goes through these two functions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ size_t tile_index(int32_t phys, int g, int num_kv_heads) {
  return (size_t)phys * (size_t)num_kv_heads + (size_t)g;
}
// Element offset of (phys, g, slot, dim) in a cache pool.
__device__ __forceinline__ size_t cache_offset(int32_t phys, int g, int slot, int dim,
                                               int num_kv_heads) {
  return (tile_index(phys, g, num_kv_heads) * kBlockSize + (size_t)slot) * kHeadDim + (size_t)dim;
}

// ---------------------------------------------------------------------------
// Work distribution over the 8 XCDs.  Workgroups are handed to XCDs round
// robin (id % 8); this maps hardware id -> logical id so that each XCD gets a
// contiguous range of logical ids, i.e. neighbouring work (same KV head,
// same shared pages) runs under one L2.  A bijection for any grid size.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int q = nblocks / kNumXCDs;
  const int r = nblocks % kNumXCDs;
  const int x = bid % kNumXCDs;
  const int k = bid / kNumXCDs;
  return x * q + (x < r ? x : r) + k;
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  Widening is exact (bf16 is the top half of binary32);
// narrowing uses the hardware convert, round to nearest even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// The remainders w - hi of two fp32 weights after their bf16 pair hi (as
// pack_bf16x2 rounds them), truncated to bf16: exact in fp32 before the
// truncation, so hi + lo is w to within 2^-16 of w.
__device__ __forceinline__ uint32_t lo_after(float w0, float w1, uint32_t hi) {
  const float x0 = w0 - bf16_lo(hi);
  const float x1 = w1 - bf16_hi(hi);
  return __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
}

// Two fp32 weights as a bf16 pair, split for a weight fed to a matrix
// product as hi + lo: with lo_mask 0, hi(w), w truncated to bf16 (its top 16
// bits); with lo_mask 0xffff0000, w - hi(w) (exact in fp32), truncated
// likewise.  hi + lo is w to within 2^-15 of w, and either half comes from
// one byte permute per pair.
__device__ __forceinline__ uint32_t hi_or_lo(float w0, float w1, uint32_t lo_mask) {
  const float x0 = w0 - __uint_as_float(__float_as_uint(w0) & lo_mask);
  const float x1 = w1 - __uint_as_float(__float_as_uint(w1) & lo_mask);
  // bytes 2, 3 of x0 and 2, 3 of x1 -> (lo half, hi half) of the result
  return __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
}

// The swizzle of the 32-key K and V tiles that the chunk and prefix kernels
// stage in LDS (256-byte rows of 16 chunks): the 16-byte chunk c of key row
// `key` sits at chunk position c ^ key_swz(key), where key_swz permutes the
// key's low four bits k3 k2 k1 k0 into (k1 ^ k3) k0 k1 k2.  Two read patterns must be free of
// LDS bank conflicts, whether the LDS serves 128 or 256 bytes per cycle:
//  * the K fragment reads: 8 or 16 lanes read one chunk of as many
//    consecutive keys: key_swz is a permutation of 16 keys that is also one
//    of any 8 aligned keys in its low three bits;
//  * the transposing V reads: 16 lanes read chunks 2j, 2j + 1 of four
//    consecutive keys 4i .. 4i + 3 (32 lanes: chunks 4j .. 4j + 3): bits 2-1
//    and bits 3-2 of key_swz each take all four values over those keys, so
//    the positions cover 8 (16) distinct chunks mod 8 (16).
// (XORing with the key itself put keys 4i and 4i + 1 of the V reads on the
// same banks.)
__device__ __forceinline__ int key_swz(int key) {
  const int k0 = key & 1, k1 = (key >> 1) & 1, k2 = (key >> 2) & 1, k3 = (key >> 3) & 1;
  return ((k1 ^ k3) << 3) | (k0 << 2) | (k1 << 1) | k2;
}

// acc + lo + hi of a packed bf16 pair, in one VALU operation (a dot product
// with (1, 1): the products are exact, the sum is fp32).
__device__ __forceinline__ float bf16x2_sum_into(uint32_t u, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u), __builtin_bit_cast(bf16x2_t, 0x3f803f80u),
                                         acc, false);
}

// Sum over the whole 64-lane wave (result in every lane).
__device__ __forceinline__ int wave_sum_i32(int x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Row of slot `seq`'s first new token: sum of q_lens[0 .. seq).
__device__ __forceinline__ int q_row_offset(const int32_t* q_lens, int seq, int lane) {
  int s = 0;
  for (int i = lane; i < seq; i += 64) s += q_lens[i];
  return wave_sum_i32(s);
}

// Orders LDS traffic between the lanes of one wave: LDS operations of a wave
// execute in program order, this keeps the compiler from moving them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wave-uniform read of read-only data through the scalar cache (s_load).
// The pointer is viewed in the constant address space, which is only valid
// for memory no kernel writes while this one runs (e.g. the block table).
// Scalar loads are counted apart from vector loads, so waiting for one does
// not drain the vector loads in flight.
__device__ __forceinline__ int32_t scalar_load_i32(const int32_t* p, int idx) {
  const __attribute__((address_space(4))) int32_t* cp =
      (const __attribute__((address_space(4))) int32_t*)(p);
  return cp[__builtin_amdgcn_readfirstlane(idx)];
}

// A pointer the compiler may hold in vector registers, made wave-uniform (in
// scalar registers), so that loads through it can be scalar loads.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Compiler-only barrier for memory operations: keeps the issue order of the
// loads on either side (emits no instruction).
__device__ __forceinline__ void issue_order_barrier() { asm volatile("" ::: "memory"); }

// Wait until this thread's outstanding vector-memory operations (loads and
// stores) have completed: s_waitcnt vmcnt(0), the other counters left
// unconstrained (expcnt 7, lgkmcnt 15 in the gfx9 encoding).
__device__ __forceinline__ void wait_vm_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Device-coherent store of 16 bytes: written through to the point of
// coherence that every XCD reads (the sc1 bit), as the relaxed agent-scope
// atomic stores of up to 8 bytes are, in one instruction instead of two
// (HIP has no 16-byte atomic store).  The compiler does not count this store
// in its waits, so the caller waits for it with wait_vm_stores() before
// announcing the data; the s_nop keeps the data registers from being
// overwritten in the cycle after the store reads them.
__device__ __forceinline__ void store_coherent_x4(float* dst, const f32x4_t& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(dst), "v"(v) : "memory");
}

// Load of data read once per pass (cached K/V pages): a non-temporal load,
// which does not keep the lines in the caches and streams measurably faster
// from HBM than an ordinary load for scattered 4 KiB tiles.
__device__ __forceinline__ u32x4_t stream_load(const u32x4_t* p) {
#if PA_STREAM_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

#if PA_STREAM_NT
__device__ __forceinline__ u32x2_t stream_load(const u32x2_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint32_t stream_load(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint32_t stream_load(const uint16_t* p) {
  return (uint32_t)__builtin_nontemporal_load(p);
}
#else
__device__ __forceinline__ u32x2_t stream_load(const u32x2_t* p) { return *p; }
__device__ __forceinline__ uint32_t stream_load(const uint32_t* p) { return *p; }
__device__ __forceinline__ uint32_t stream_load(const uint16_t* p) { return (uint32_t)*p; }
#endif

// The value of the same register in lane l ^ 32 (the other half of the
// wave), through v_permlane32_swap: the swap leaves lanes 0-31 of the first
// result and lanes 32-63 of the second holding this lane's own value, the
// other two holding the partner's.
__device__ __forceinline__ float other_half(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// The value of lane ^ 16 (v_permlane16_swap; its lane layout was checked on
// the device: rows 0 and 2 find the partner in the second result, rows 1
// and 3 in the first).
__device__ __forceinline__ float other16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  return __uint_as_float((lane >> 4) & 1 ? r[0] : r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLn2 = 0.69314718055994530942f;

// Online log-sum-exp merge of split-KV partials (each a normalised output
// and its natural-log LSE) for one thread's two adjacent dims of one row:
// the result is (a0, a1) / W with LSE M + ln W.  A partial with LSE = -inf
// weighs 0 and its output is never read.
struct MergeState {
  float M = -INFINITY;
  float W = 0.f;
  float a0 = 0.f;
  float a1 = 0.f;
};

__device__ __forceinline__ void merge_fold(MergeState& s, float l, float o0, float o1) {
  if (l == -INFINITY) return;
  const float M2 = fmaxf(s.M, l);
  const float sc = fast_exp2((s.M - M2) * 1.4426950408889634f);  // 0 when M = -inf
  const float w = fast_exp2((l - M2) * 1.4426950408889634f);
  s.W = fmaf(s.W, sc, w);
  s.a0 = fmaf(s.a0, sc, w * o0);
  s.a1 = fmaf(s.a1, sc, w * o1);
  s.M = M2;
}

// Fold the partials of one row from two sets: set A's partial i has its LSE
// at lse_a[i * rows] and its two dims at out_a[i * rows * 128 + 0, 1]
// (likewise B).  Device-coherent relaxed loads (partials of this launch may
// come from workgroups on any XCD), in batches whose loads are all issued
// before any is used: 2, 4, 8 (or 16) partials for short merges, else 28 (56 loads
// in flight, within the 6-bit load counter).
template <int kBatch>
__device__ __forceinline__ void merge_batches(MergeState& s, const float* lse_a, const float* out_a, int na,
                                              const float* lse_b, const float* out_b, int n, size_t rows) {
  const size_t ostride = rows * 128 / 2;
  for (int q0 = 0; q0 < n; q0 += kBatch) {
    float lv[kBatch];
    uint64_t ov[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int q = min(q0 + i, n - 1);
      const bool a = q < na;
      const int k = a ? q : q - na;
      const float* lp = (a ? lse_a : lse_b) + (size_t)k * rows;
      const uint64_t* op = reinterpret_cast<const uint64_t*>(a ? out_a : out_b) + (size_t)k * ostride;
      lv[i] = __hip_atomic_load(lp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ov[i] = __hip_atomic_load(op, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (q0 + i < n)
        merge_fold(s, lv[i], __uint_as_float((uint32_t)ov[i]), __uint_as_float((uint32_t)(ov[i] >> 32)));
  }
}

// The same for eight adjacent dims of a row (four 8-byte device-coherent
// loads per partial), in batches of 8 partials (40 loads in flight).
struct MergeState8 {
  float M = -INFINITY;
  float W = 0.f;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
};

__device__ __forceinline__ void merge_partials8(MergeState8& s, const float* lse_a, const float* out_a, int na,
                                                const float* lse_b, const float* out_b, int nb, size_t rows) {
  constexpr int kBatch = 8;
  const int n = na + nb;
  const size_t ostride = rows * 128 / 2;
  for (int q0 = 0; q0 < n; q0 += kBatch) {
    float lv[kBatch];
    uint64_t ov[kBatch][4];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int q = min(q0 + i, n - 1);
      const bool a = q < na;
      const int k = a ? q : q - na;
      const float* lp = (a ? lse_a : lse_b) + (size_t)k * rows;
      const uint64_t* op = reinterpret_cast<const uint64_t*>(a ? out_a : out_b) + (size_t)k * ostride;
      lv[i] = __hip_atomic_load(lp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int j = 0; j < 4; ++j) ov[i][j] = __hip_atomic_load(op + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float l = lv[i];
      if (q0 + i >= n || l == -INFINITY) continue;
      const float M2 = fmaxf(s.M, l);
      const float sc = fast_exp2((s.M - M2) * 1.4426950408889634f);  // 0 when M = -inf
      const float w = fast_exp2((l - M2) * 1.4426950408889634f);
      s.W = fmaf(s.W, sc, w);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s.a[2 * j] = fmaf(s.a[2 * j], sc, w * __uint_as_float((uint32_t)ov[i][j]));
        s.a[2 * j + 1] = fmaf(s.a[2 * j + 1], sc, w * __uint_as_float((uint32_t)(ov[i][j] >> 32)));
      }
      s.M = M2;
    }
  }
}

// kBatch16: also a batch of 16 for 9 - 16 partials (callers that merge one
// (row, dim pair) per thread; with several unrolled per thread the extra
// variant costs more scalar registers than it saves).
template <bool kBatch16 = false>
__device__ __forceinline__ void merge_partials(MergeState& s, const float* lse_a, const float* out_a, int na,
                                               const float* lse_b, const float* out_b, int nb, size_t rows) {
  const int n = na + nb;
  if (n <= 0) return;
  if (n <= 2)
    merge_batches<2>(s, lse_a, out_a, na, lse_b, out_b, n, rows);
  else if (n <= 4)
    merge_batches<4>(s, lse_a, out_a, na, lse_b, out_b, n, rows);
  else if (n <= 8)
    merge_batches<8>(s, lse_a, out_a, na, lse_b, out_b, n, rows);
  else if (kBatch16 && n <= 16)
    merge_batches<16>(s, lse_a, out_a, na, lse_b, out_b, n, rows);
  else
    merge_batches<28>(s, lse_a, out_a, na, lse_b, out_b, n, rows);
}

}  // namespace pa
