// launch.h -- internal interface between the C-ABI front end (api.cpp) and the
// HIP kernels.  Host-only types: nothing here is visible outside libpa.so.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kHeadDim = 128;    // only head size built
constexpr int kBlockSize = 16;   // tokens per KV block
constexpr int kNumCUs = 256;     // MI355X compute units (8 XCDs x 32)
constexpr int kNumXCDs = 8;
#ifndef PA_STREAM_NT
#define PA_STREAM_NT 1
#endif
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 4
#endif
constexpr int kDecodeWaves = PA_DECODE_WAVES;          // waves per decode workgroup
constexpr int kDecodeWGsPerCU = 8 / kDecodeWaves;      // resident per CU (2 waves per SIMD)

// Page formats of the K/V caches (values of pa_kv_format in pa.h).
constexpr int kFmtBF16 = 0;
constexpr int kFmtFP8 = 1;   // OCP E4M3 codes, one fp32 scale per cache
constexpr int kFmtQ8 = 2;    // q8_0: int8 codes, fp16 scale per 32 values
constexpr int kFmtQ4 = 3;    // q4_0: 4-bit codes, fp16 scale per 32 values

// Split-KV decode: one workgroup per (KV head, slot, partition).
struct DecodeParams {
  const uint16_t* q;          // bf16 [total_q][Hq][128]
  const uint16_t* k;          // page codes: bf16 [num_blocks][Hkv][16][128], or the
  const uint16_t* v;          // byte layouts of the quantised formats
  const uint16_t* k_scales;   // fp16 [num_blocks][Hkv][16][4] (q8_0, q4_0)
  const uint16_t* v_scales;
  float v_scale;              // FP8: per-cache V scale (K's is folded into scale_log2)
  // Prefix-grouped decode: a slot's keys start at slot_plen[slot] (null: 0),
  // and slots with a prefix also merge pre_parts partials of the prefix pass.
  const int32_t* slot_plen;
  const float* pre_out;       // fp32 [pre_parts][total_q*Hq][128]
  const float* pre_lse;       // fp32 [pre_parts][total_q*Hq]
  int32_t pre_parts;
  const int32_t* block_table; // [num_seqs][max_blocks]
  const int32_t* ctx_lens;
  const int32_t* q_lens;
  uint16_t* out;              // bf16 [total_q][Hq][128]: the result
  float* lse;                 // fp32 [total_q][Hq] or null
  float* part_out;            // fp32 [num_parts][total_q*Hq][128] (split: num_parts > 1)
  float* part_lse;            // fp32 [num_parts][total_q*Hq]
  int32_t* counters;          // [num_seqs][Hkv] finished partitions; zero between calls
  float scale_log2;           // softmax scale * log2(e)
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t total_q;
  int32_t part_pages;         // 16-token pages per partition
  int32_t num_parts;
  int32_t causal;             // several tokens per slot: token t of m sees keys [0, n - m + t]
  // Prefix-grouped decode in one launch: the first pre_items workgroups each
  // stream a run of pre_pages shared pages of one group and KV head once for
  // up to M of its members (the members' rows as the token columns) and
  // write pre_out / pre_lse; the rest are the members' own-key partitions.
  // A slot with a prefix then merges once all num_parts + pre_parts
  // partials of it have arrived.  0 pre_items: the prefix pass ran before.
  int32_t pre_items;
  int32_t pre_pages;          // pages per prefix partition
  int32_t pre_chunks;         // member chunks (of kDecodeWaves M members) per group
  int32_t max_members;        // members of a group that share its prefix
  const int32_t* group_start; // [num_groups + 1]: a group's slots are [group_start[i], group_start[i + 1])
  const int32_t* prefix_len;  // [num_groups]: shared tokens (read as whole pages)
  // With slot_plen null, the slots' partitions look their group up among
  // the num_groups (< 64) groups themselves; 0: no lookup.
  int32_t num_groups;
  int32_t guess_plen;         // prefix length (whole pages) the first page-id requests assume
};

// Chunk path (several new rows per slot): bf16 MFMA for S = QK^T and O = PV.
struct ChunkParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* q_lens;
  uint16_t* out;
  float* lse;
  float scale_log2;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t q_tiles;            // ceil(max_q_len / rows per workgroup)
  int32_t causal;
  int32_t max_ctx;            // max_ctx_len and max_q_len: the lengths the
  int32_t max_q;              // first page ids are requested for, unverified
};

struct CombineParams {
  const float* part_out;      // [P][rows][D]
  const float* part_lse;      // [P][rows]
  uint16_t* out;              // bf16 [rows][D]
  float* lse;                 // [rows] or null
  int32_t num_parts;
  int32_t rows;
  int32_t head_dim;
};

struct GatherParams {
  const uint16_t* cache;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  uint16_t* dst;              // [num_seqs][max_ctx][Hkv][128]
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t max_pages;
};

struct ValidateParams {
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* q_lens;
  const int32_t* counters;    // split-KV counters to check for zero, or null
  int32_t num_counters;
  int32_t* error_word;
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t max_q;
  int32_t total_q;
};

// Decode kernels exist for these query-per-KV head group sizes, and for up
// to 8 new tokens per slot (bf16 pages) while tokens x group <= 32.
bool decode_supports_group(int group);
// Tokens per slot the decode kernel is built for that cover max_q_len
// (1, 2, 4 or 8), or 0 when the decode path does not apply.
int decode_tokens_per_slot(int group, int max_q_len);
constexpr int kDecodeThreads = 64 * kDecodeWaves;
// Members per wave of a prefix item in a one-launch prefix-grouped decode:
// as many as fill the 16 columns of one score tile with their query heads (8
// with one head per KV head, where the tile takes each column twice, hi and
// lo).  An item covers kDecodeWaves times as many.
constexpr int prefix_chunk_members(int group) { return group == 1 ? 8 : 16 / group; }
hipError_t launch_decode(const DecodeParams& p, int group, int format, int tokens, unsigned grid, hipStream_t s);
// The one-launch prefix-grouped decode (bf16 pages, one token per slot):
// pre_items prefix items, then the slots' partitions.  Built for 1, 2 and 4
// query heads per KV head (with 8, the prefix items' LDS would leave one
// workgroup per CU).
constexpr bool decode_prefix_supports_group(int group) { return group == 1 || group == 2 || group == 4; }
hipError_t launch_decode_prefix(const DecodeParams& p, int group, unsigned grid, hipStream_t s);
hipError_t launch_zero_i32(int32_t* x, size_t n, hipStream_t s);

constexpr int kChunkRows = 128;  // query rows per chunk workgroup
hipError_t launch_chunk(const ChunkParams& p, unsigned grid, hipStream_t s);

hipError_t launch_combine(const CombineParams& p, hipStream_t s);
struct WriteParams {
  const uint16_t* k_new;      // bf16 [total_q][Hkv][128]
  const uint16_t* v_new;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* q_lens;
  uint16_t* k_cache;          // bf16 [num_blocks][Hkv][16][128]
  uint16_t* v_cache;
  int64_t num_blocks;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t max_q_len;
  int32_t total_q;            // rows of k_new / v_new
};

// Shared-prefix pass of prefix-grouped decode.  A partition is at most
// kPrefixMaxTiles 32-key tiles (all held in LDS at once).
constexpr int kPrefixMaxTiles = 8;
struct PrefixParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_table;
  const int32_t* ctx_lens;
  const int32_t* q_lens;
  const int32_t* group_start;  // [num_groups + 1]
  const int32_t* prefix_len;   // [num_groups]
  float* pre_out;              // fp32 [pre_parts][total_q*Hq][128]
  float* pre_lse;              // fp32 [pre_parts][total_q*Hq]
  int32_t* slot_plen;          // [num_seqs], written by the set-up workgroup
  float scale_log2;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t total_q;
  int32_t num_groups;
  int32_t row_tiles;           // 64-row tiles of (member, query head) rows per group
  int32_t pre_parts;           // partitions of the prefix
  int32_t part_pages;          // pages per prefix partition (<= 2 kPrefixMaxTiles)
  int32_t max_members;         // rows of a group's first max_members slots only
};

// Quantising append: new bf16 rows -> codes (+ scales) at their positions.
struct WriteQuantParams {
  WriteParams w;              // rows, table, lengths; k_cache / v_cache hold the codes
  uint16_t* k_scales;         // fp16 [num_blocks][Hkv][16][4] (q8_0, q4_0)
  uint16_t* v_scales;
  float k_scale;              // FP8: per-cache scales (codes of x / scale)
  float v_scale;
};

struct CopyParams {
  const int32_t* src;         // [num_copies] block ids
  const int32_t* dst;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int64_t num_blocks;
  int32_t num_copies;
  int32_t num_kv_heads;
};

hipError_t launch_gather(const GatherParams& p, hipStream_t s);
hipError_t launch_write_kv(const WriteParams& p, hipStream_t s);
hipError_t launch_copy_blocks(const CopyParams& p, hipStream_t s);
hipError_t launch_write_kv_quant(const WriteQuantParams& p, int format, hipStream_t s);
hipError_t launch_prefix(const PrefixParams& p, unsigned grid, hipStream_t s);
hipError_t launch_validate(const ValidateParams& p, hipStream_t s);

// pa_attend on bf16 pages with an explicit workspace (api.cpp).
pa_status attend_bf16(const pa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens,
                      float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream);

}  // namespace pa
