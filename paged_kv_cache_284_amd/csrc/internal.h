// Internal declarations shared by the device translation units of libpagedkv.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace pa {

constexpr int kBlockSize = 16;  // tokens per KV block (the only size the kernels take)

// Everything one decode launch needs.  Pointers are device pointers.
struct DecodeArgs {
  float* out;                 // [B][Hq][D]
  const void* q;              // [B][Hq][D]
  const void* k;              // [NB][Hkv][bs][D]
  const void* v;              // [NB][Hkv][D][bs]
  const float* k_scale;       // [NB][Hkv] (int8)
  const float* v_scale;       // [NB][Hkv] (int8)
  const int32_t* tables;      // [B][max_blocks]
  const int32_t* seq_lens;    // [B]
  float* ws_m;                // [B][Hq][np_max]  running max (log2 domain)
  float* ws_l;                // [B][Hq][np_max]  running sum
  float* ws_o;                // [B][Hq][np_max][D] normalised partial outputs
  int32_t max_blocks, max_seq_len;
  int32_t B, Hq, Hkv, D, NB;
  int32_t partition;          // tokens per partition (multiple of 64)
  int32_t np_max;             // ceil(max_seq_len / partition), >= 1
  int32_t nw;                 // balanced schedule: workgroups (0 = fixed partitions)
  int32_t* ws_merge;          // balanced schedule: per-workgroup merge records [nw][4]
  float scale_log2;           // softmax scale * log2(e)
  // Shared-prefix decode (all null / 0 otherwise).  A group is a run of consecutive sequences
  // whose tables start with the same physical block; its reference is its longest member.
  int32_t* pstart;            // [B] leading tokens of a non-reference member read by the
                              //     prefix pass (multiple of 32; 0 for references / no group)
  int32_t* ref_p;             // [B] at a reference: tokens its group's prefix pass covers
  int32_t* grp_ref;           // [B] reference sequence of each sequence's group, -1 when none
  float* pf_m;                // [B][Hq][pf_parts] prefix-pass states: max (log2 domain)
  float* pf_l;                //                   sum of weights
  float* pf_o;                // [B][Hq][pf_parts][D] normalised output
  int32_t pf_parts;           // prefix-pass parts per output row (ceil(max_seq_len / pf_tokens))
  int32_t pf_tokens;          // tokens per prefix-pass part (multiple of 32)
  int32_t pf_gmax;            // bound on the number of groups (B / 2)
  float* sf_m;                // [B][Hq] state of a whole segment past a shared prefix: max,
  float* sf_l;                //         sum of weights,
  float* sf_o;                // [B][Hq][D] normalised output (folded with the prefix states and
  int32_t* sf_mark;           // [B][Hkv] written out by the merge launch); 1 where it was written
};

// Everything one chunked-prefill launch needs.  Pointers are device pointers.
// Cache element kinds the matrix-core kernels are templated on.
constexpr int kKvBf16 = 0, kKvI8 = 1, kKvI4 = 2;

struct PrefillArgs {
  float* out;                 // [T][Hq][D]
  const void* q;              // [T][Hq][D] bf16
  const void* k;              // [NB][Hkv][bs][D] bf16 / int8, [NB][Hkv][bs][D/2] packed int4
  const void* v;              // [NB][Hkv][D][bs] bf16 / int8, [NB][Hkv][D][bs/2] packed int4
  const int32_t* tables;      // [B][max_blocks]
  const int32_t* seq_lens;    // [B] context length, the chunk included
  const int32_t* cu_q;        // [B + 1] first query row of each sequence's chunk
  int32_t max_blocks, max_seq_len;
  int32_t B, T, Hq, Hkv, D, NB;
  int32_t max_tiles;          // grid bound on the number of 64-query workgroups
  float scale_log2;
  int32_t kv_kind;            // 0 bf16, 1 int8, 2 packed int4 cache
  const float* k_scale;       // [NB][Hkv], quantised caches
  const float* v_scale;
};

// Upper bound on balanced-schedule workgroups; sizes the workspace.
constexpr int kMaxBalancedWorkgroups = 1024;
// Largest batch / group size the balanced schedule takes (its prefix sums and per-wave states
// live in LDS).
constexpr int kMaxBalancedBatch = 8192;
constexpr int kMaxBalancedGroup = 8;
// Most prefix-pass parts one output row folds in (parts are at least 1024 tokens).
constexpr int kMaxPrefixParts = 8;
// Resident workgroups of the balanced MFMA kernel per compute unit.
int mfma_workgroups_per_cu();

// pa_decode in two steps.  decode_check: the host-side argument checks (no HIP call); *nothing
// is set when the call has no work (B == 0).  decode_run: schedule, workspace layout and
// launches; exact_size: the workspace is a fixed buffer that must hold what this call's schedule
// uses (PA_ERR_TOO_LARGE otherwise), else it must hold pa_decode_workspace_size().
int decode_check(const float* out, const void* q, int32_t q_dtype, const void* k_cache,
                 const void* v_cache, int32_t kv_dtype, const float* k_scale,
                 const float* v_scale, const int32_t* block_tables, int32_t max_blocks,
                 const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t Hq,
                 int32_t Hkv, int32_t D, int32_t bs, int32_t NB, float scale,
                 int32_t partition_tokens, bool* nothing);
int decode_run(float* out, const void* q, int32_t q_dtype, const void* k_cache,
               const void* v_cache, int32_t kv_dtype, const float* k_scale, const float* v_scale,
               const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
               int32_t max_seq_len, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t NB,
               float scale, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
               bool exact_size, void* stream);

// Partition length the fixed-partition schedule uses when the caller passes 0.
int32_t auto_partition(int32_t B, int32_t Hkv);

// table_index / tables may be NULL; otherwise the launch also patches the block tables.
// lens_in / lens_out may be NULL; otherwise the launch also copies the sequence lengths.
hipError_t launch_kv_append(const void* k_new, const void* v_new, const int64_t* slots,
                            void* k_cache, void* v_cache, int32_t B, int32_t Hkv, int32_t D,
                            int32_t NB, int32_t elem_bytes, const int32_t* table_index,
                            int32_t* tables, int32_t max_blocks, const int32_t* lens_in,
                            int32_t* lens_out, hipStream_t stream);
// Quantising append into an int8 cache; new tokens in bf16 (bf16_new) or fp32.
hipError_t launch_kv_append_i8(const void* k_new, const void* v_new, bool bf16_new,
                               const int64_t* slots, int8_t* k_cache, int8_t* v_cache,
                               float* k_scale, float* v_scale, int32_t B, int32_t Hkv, int32_t D,
                               int32_t NB, hipStream_t stream);
// Quantising append into a packed int4 cache; new tokens in bf16 (bf16_new) or fp32.
hipError_t launch_kv_append_i4(const void* k_new, const void* v_new, bool bf16_new,
                               const int64_t* slots, uint8_t* k_cache, uint8_t* v_cache,
                               float* k_scale, float* v_scale, int32_t B, int32_t Hkv, int32_t D,
                               int32_t NB, hipStream_t stream);
// Whole-block copies from one pool to another of the same layout (scales optional);
// block_bytes = bytes of one block of K (= of V), a multiple of 16.
hipError_t launch_copy_tiles(const void* src_k, const void* src_v, const float* src_ks,
                             const float* src_vs, int32_t src_blocks, void* dst_k, void* dst_v,
                             float* dst_ks, float* dst_vs, int32_t dst_blocks,
                             const int32_t* pairs, int32_t n, int32_t Hkv, int64_t block_bytes,
                             hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* pairs, int32_t n, int32_t Hkv, int32_t NB,
                              int64_t block_bytes, hipStream_t stream);
hipError_t launch_update_tables(int32_t* tables, int32_t max_blocks, const int64_t* slots,
                                const int32_t* table_index, int32_t B, hipStream_t stream);

// Returns hipErrorNotSupported when no kernel of this family takes the combination.
hipError_t launch_decode_generic(const DecodeArgs& a, int q_dtype, int kv_dtype,
                                 hipStream_t stream);
// bf16 query; bf16, int8 or int4 cache (PA_BF16 / PA_I8 / PA_I4; the quantised ones with
// k_scale / v_scale set); D 64/128; group size 1, 2, 4, 8 or 16.
hipError_t launch_decode_mfma(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
// Shared-prefix decode on the matrix cores: the group plan, the prefix pass, then the balanced
// decode of every sequence past its prefix (a.nw workgroups) folding in the prefix states.
// bf16 query; bf16, int8 or int4 cache; D 64/128; group size 1, 2, 4 or 8.
hipError_t launch_decode_shared_prefix(const DecodeArgs& a, int kv_dtype, hipStream_t stream);
hipError_t launch_splitk_reduce(const DecodeArgs& a, hipStream_t stream);
// bf16 query and cache; D 64/128; group size 1, 2, 4, 8 or 16.
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream);

}  // namespace pa
