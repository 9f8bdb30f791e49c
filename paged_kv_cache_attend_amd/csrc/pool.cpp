// pool.cpp -- host-side block pool: paged allocation, sharing, copy-on-write
// and fenced release.
//
// Follows the inference-optimisation chapter ("Chapter 8: Inference
// optimisation"): section 8.3.1 (Fig. 8-10) for growing a sequence block by
// block through its table, section 8.3.2 for shared blocks with reference
// counts (Figs. 8-13, 8-14), copy-on-write of a shared, partly filled tail
// block (Fig. 8-15), and release only after the accelerator has finished the
// work that reads a block (Figs. 8-14, 8-16).
//
// Data structures: a stack of free block ids (O(1) take and return), one
// reference count per block, one fixed-size table row per slot (the layout
// the kernels read, so a row can be uploaded as is), and a list of released
// blocks waiting for their fence.  All host memory, no device calls.

#include <stdint.h>

#include <utility>
#include <vector>

#include "pa.h"

struct pa_pool {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  int32_t num_slots = 0;
  int32_t max_blocks = 0;
  std::vector<int32_t> free_stack;  // next block to hand out at the back
  std::vector<int32_t> refs;        // references per block
  std::vector<int32_t> table;       // [num_slots][max_blocks]
  std::vector<int32_t> length;      // tokens per slot
  std::vector<int32_t> held;        // blocks per slot
  std::vector<std::pair<uint64_t, int32_t>> pending;  // (fence, block)
  int32_t used = 0;
  int64_t references = 0;

  int32_t take() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    refs[b] = 1;
    ++used;
    return b;
  }
  void drop(int32_t b, uint64_t fence) {
    if (--refs[b] == 0) {
      --used;
      pending.emplace_back(fence, b);
    }
  }
  int32_t* row(int32_t slot) { return table.data() + (size_t)slot * max_blocks; }
  bool slot_ok(int32_t slot) const { return slot >= 0 && slot < num_slots; }
};

namespace {

int64_t blocks_for(int64_t tokens, int32_t block_size) {
  return (tokens + block_size - 1) / block_size;
}

}  // namespace

extern "C" {

pa_status pa_pool_create(int32_t num_blocks, int32_t block_size, int32_t num_slots,
                         int32_t max_blocks_per_seq, pa_pool** pool) {
  if (!pool) return PA_ERR_NULL_ARG;
  *pool = nullptr;
  if (num_blocks <= 0 || block_size <= 0 || num_slots < 0 || max_blocks_per_seq <= 0)
    return PA_ERR_BAD_SHAPE;
  if ((int64_t)num_slots * max_blocks_per_seq > ((int64_t)1 << 31) - 1) return PA_ERR_BAD_SHAPE;
  pa_pool* p = new pa_pool;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->num_slots = num_slots;
  p->max_blocks = max_blocks_per_seq;
  p->free_stack.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) p->free_stack[i] = num_blocks - 1 - i;  // 0 first
  p->refs.assign(num_blocks, 0);
  p->table.assign((size_t)num_slots * max_blocks_per_seq, 0);
  p->length.assign(num_slots, 0);
  p->held.assign(num_slots, 0);
  *pool = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

pa_status pa_pool_append(pa_pool* pool, int32_t slot, int32_t num_tokens, int32_t* copy_src,
                         int32_t* copy_dst, int32_t* num_copies) {
  if (!pool || !copy_src || !copy_dst || !num_copies) return PA_ERR_NULL_ARG;
  *num_copies = 0;
  if (!pool->slot_ok(slot) || num_tokens < 0) return PA_ERR_BAD_SHAPE;
  const int32_t len = pool->length[slot];
  const int32_t have = pool->held[slot];
  const int64_t new_len = (int64_t)len + num_tokens;
  const int64_t need = blocks_for(new_len, pool->block_size);
  if (need > pool->max_blocks) return PA_ERR_BAD_SHAPE;
  int32_t* row = pool->row(slot);
  // Writing into a shared block that is only partly filled needs a private
  // copy first; full shared blocks are never written again.
  const bool cow = num_tokens > 0 && len % pool->block_size != 0 && pool->refs[row[have - 1]] > 1;
  const int64_t grow = need - have;
  if (grow + (cow ? 1 : 0) > (int64_t)pool->free_stack.size()) return PA_ERR_OUT_OF_BLOCKS;
  if (cow) {
    const int32_t old = row[have - 1];
    const int32_t fresh = pool->take();
    --pool->refs[old];  // still referenced by another slot
    row[have - 1] = fresh;
    copy_src[0] = old;
    copy_dst[0] = fresh;
    *num_copies = 1;
  }
  for (int64_t i = 0; i < grow; ++i) row[have + i] = pool->take();
  pool->references += grow;
  pool->held[slot] = (int32_t)need;
  pool->length[slot] = (int32_t)new_len;
  return PA_OK;
}

pa_status pa_pool_fork(pa_pool* pool, int32_t src, int32_t dst, int32_t num_tokens) {
  if (!pool) return PA_ERR_NULL_ARG;
  if (!pool->slot_ok(src) || !pool->slot_ok(dst) || src == dst) return PA_ERR_BAD_SHAPE;
  if (pool->length[dst] != 0 || pool->held[dst] != 0) return PA_ERR_BAD_SHAPE;
  const int32_t n = num_tokens < 0 ? pool->length[src] : num_tokens;
  if (n > pool->length[src]) return PA_ERR_BAD_SHAPE;
  const int32_t k = (int32_t)blocks_for(n, pool->block_size);
  const int32_t* from = pool->row(src);
  int32_t* to = pool->row(dst);
  for (int32_t i = 0; i < k; ++i) {
    to[i] = from[i];
    ++pool->refs[from[i]];
  }
  pool->references += k;
  pool->held[dst] = k;
  pool->length[dst] = n;
  return PA_OK;
}

pa_status pa_pool_release(pa_pool* pool, int32_t slot, uint64_t fence) {
  if (!pool) return PA_ERR_NULL_ARG;
  if (!pool->slot_ok(slot)) return PA_ERR_BAD_SHAPE;
  int32_t* row = pool->row(slot);
  for (int32_t i = 0; i < pool->held[slot]; ++i) {
    pool->drop(row[i], fence);
    row[i] = 0;
  }
  pool->references -= pool->held[slot];
  pool->held[slot] = 0;
  pool->length[slot] = 0;
  return PA_OK;
}

pa_status pa_pool_retire(pa_pool* pool, uint64_t fence) {
  if (!pool) return PA_ERR_NULL_ARG;
  size_t keep = 0;
  for (size_t i = 0; i < pool->pending.size(); ++i) {
    if (pool->pending[i].first <= fence)
      pool->free_stack.push_back(pool->pending[i].second);
    else
      pool->pending[keep++] = pool->pending[i];
  }
  pool->pending.resize(keep);
  return PA_OK;
}

int32_t pa_pool_length(const pa_pool* pool, int32_t slot) {
  if (!pool || !pool->slot_ok(slot)) return -1;
  return pool->length[slot];
}

const int32_t* pa_pool_block_table(const pa_pool* pool) {
  return pool ? pool->table.data() : nullptr;
}

int32_t pa_pool_refcount(const pa_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= pool->num_blocks) return -1;
  return pool->refs[block];
}

pa_status pa_pool_get_stats(const pa_pool* pool, pa_pool_stats* stats) {
  if (!pool || !stats) return PA_ERR_NULL_ARG;
  stats->free_blocks = (int32_t)pool->free_stack.size();
  stats->pending_blocks = (int32_t)pool->pending.size();
  stats->used_blocks = pool->used;
  stats->reserved = 0;
  stats->references = pool->references;
  return PA_OK;
}

}  // extern "C"
