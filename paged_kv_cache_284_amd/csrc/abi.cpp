// C-ABI device entry points: host-side argument checks, then dispatch to the kernels.
// Nothing here touches the device before every argument has been checked.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"
#include "pagedkv.h"

namespace {

int elem_bytes(int32_t dtype) {  // whole bytes per element (0: none, or not a byte type)
  switch (dtype) {
    case PA_F32: return 4;
    case PA_BF16: return 2;
    case PA_I8: return 1;
    default: return 0;
  }
}

bool known_kv(int32_t dtype) { return elem_bytes(dtype) != 0 || dtype == PA_I4; }
bool quantised(int32_t dtype) { return dtype == PA_I8 || dtype == PA_I4; }

// Bytes of one block of K (or of V): Hkv tiles of bs x D elements.
int64_t block_bytes(int32_t dtype, int32_t Hkv, int32_t D) {
  const int64_t elems = static_cast<int64_t>(Hkv) * pa::kBlockSize * D;
  return dtype == PA_I4 ? elems / 2 : elems * elem_bytes(dtype);
}

int status_of(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
  return PA_ERR_DEVICE;
}

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace

namespace pa {

// Partition length of the fixed-partition schedule when the caller passes 0.  A batch whose
// (sequence, KV head) pairs alone give every compute unit four workgroups is not split below the
// largest partition (no merge pass for sequences up to 8192 tokens); a smaller batch is split
// into 512-token partitions, so long sequences spread over the device.  Depends only on sizes the
// workspace query also sees.
int32_t auto_partition(int32_t B, int32_t Hkv) {
  constexpr int64_t kFillWorkgroups = 4 * 256;
  return static_cast<int64_t>(B) * Hkv >= kFillWorkgroups ? 8192 : 512;
}

}  // namespace pa

extern "C" {

int pa_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                 void* k_cache, void* v_cache, int32_t B, int32_t Hkv, int32_t D, int32_t bs,
                 int32_t NB, int32_t kv_dtype, void* stream) {
  if (B < 0 || Hkv < 1 || NB < 1 || (D != 64 && D != 128)) return PA_ERR_INVALID;
  if (bs != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (kv_dtype != PA_F32 && kv_dtype != PA_BF16) {
    return quantised(kv_dtype) ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID;
  }
  if (B == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID;
  return status_of(pa::launch_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, B, Hkv, D,
                                        NB, elem_bytes(kv_dtype), nullptr, nullptr, 0, nullptr,
                                        nullptr, static_cast<hipStream_t>(stream)));
}

int pa_kv_append_int8(const void* k_new, const void* v_new, int32_t new_dtype,
                      const int64_t* slot_mapping, int8_t* k_cache, int8_t* v_cache,
                      float* k_scale, float* v_scale, int32_t B, int32_t Hkv, int32_t D,
                      int32_t bs, int32_t NB, void* stream) {
  if (B < 0 || Hkv < 1 || NB < 1 || (D != 64 && D != 128)) return PA_ERR_INVALID;
  if (bs != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (new_dtype != PA_F32 && new_dtype != PA_BF16) return PA_ERR_INVALID;
  if (B == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale)
    return PA_ERR_INVALID;
  return status_of(pa::launch_kv_append_i8(k_new, v_new, new_dtype == PA_BF16, slot_mapping,
                                           k_cache, v_cache, k_scale, v_scale, B, Hkv, D, NB,
                                           static_cast<hipStream_t>(stream)));
}

int pa_kv_append_int4(const void* k_new, const void* v_new, int32_t new_dtype,
                      const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                      float* k_scale, float* v_scale, int32_t B, int32_t Hkv, int32_t D,
                      int32_t bs, int32_t NB, void* stream) {
  if (B < 0 || Hkv < 1 || NB < 1 || (D != 64 && D != 128)) return PA_ERR_INVALID;
  if (bs != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (new_dtype != PA_F32 && new_dtype != PA_BF16) return PA_ERR_INVALID;
  if (B == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale)
    return PA_ERR_INVALID;
  return status_of(pa::launch_kv_append_i4(k_new, v_new, new_dtype == PA_BF16, slot_mapping,
                                           k_cache, v_cache, k_scale, v_scale, B, Hkv, D, NB,
                                           static_cast<hipStream_t>(stream)));
}

int pa_append_step(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                   const int32_t* table_index, const int32_t* seq_lens_in, int32_t* seq_lens_out,
                   void* k_cache, void* v_cache, int32_t* block_tables, int32_t max_blocks,
                   int32_t B, int32_t Hkv, int32_t D, int32_t bs, int32_t NB, int32_t kv_dtype,
                   void* stream) {
  if (B < 0 || Hkv < 1 || NB < 1 || max_blocks < 0 || (D != 64 && D != 128))
    return PA_ERR_INVALID;
  if (bs != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (kv_dtype != PA_F32 && kv_dtype != PA_BF16) {
    return quantised(kv_dtype) ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID;
  }
  if (B == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID;
  if (table_index && !block_tables) return PA_ERR_INVALID;
  if ((seq_lens_in == nullptr) != (seq_lens_out == nullptr)) return PA_ERR_INVALID;
  return status_of(pa::launch_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, B, Hkv, D,
                                        NB, elem_bytes(kv_dtype), table_index, block_tables,
                                        max_blocks, seq_lens_in, seq_lens_out,
                                        static_cast<hipStream_t>(stream)));
}

int pa_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                   const int32_t* pairs, int32_t n, int32_t Hkv, int32_t D, int32_t bs,
                   int32_t NB, int32_t kv_dtype, void* stream) {
  if (n < 0 || Hkv < 1 || NB < 1 || (D != 64 && D != 128)) return PA_ERR_INVALID;
  if (bs != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (!known_kv(kv_dtype)) return PA_ERR_INVALID;
  if (n == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_ERR_INVALID;
  if (quantised(kv_dtype) && (!k_scale || !v_scale)) return PA_ERR_INVALID;
  if (!quantised(kv_dtype)) k_scale = v_scale = nullptr;
  return status_of(pa::launch_copy_blocks(k_cache, v_cache, k_scale, v_scale, pairs, n, Hkv,
                                          NB, block_bytes(kv_dtype, Hkv, D),
                                          static_cast<hipStream_t>(stream)));
}

int pa_swap_blocks(const void* src_k, const void* src_v, const float* src_k_scale,
                   const float* src_v_scale, int32_t src_blocks, void* dst_k, void* dst_v,
                   float* dst_k_scale, float* dst_v_scale, int32_t dst_blocks,
                   const int32_t* pairs, int32_t n, int32_t Hkv, int32_t D, int32_t bs,
                   int32_t kv_dtype, void* stream) {
  if (n < 0 || Hkv < 1 || src_blocks < 1 || dst_blocks < 1 || (D != 64 && D != 128))
    return PA_ERR_INVALID;
  if (bs != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (!known_kv(kv_dtype)) return PA_ERR_INVALID;
  if (n == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return PA_ERR_INVALID;
  if (quantised(kv_dtype)) {
    if (!src_k_scale || !src_v_scale || !dst_k_scale || !dst_v_scale) return PA_ERR_INVALID;
  } else {
    src_k_scale = src_v_scale = nullptr;
    dst_k_scale = dst_v_scale = nullptr;
  }
  return status_of(pa::launch_copy_tiles(src_k, src_v, src_k_scale, src_v_scale, src_blocks,
                                         dst_k, dst_v, dst_k_scale, dst_v_scale, dst_blocks,
                                         pairs, n, Hkv, block_bytes(kv_dtype, Hkv, D),
                                         static_cast<hipStream_t>(stream)));
}

int pa_update_block_tables(int32_t* block_tables, int32_t max_blocks, const int64_t* slots,
                           const int32_t* table_index, int32_t B, int32_t bs, void* stream) {
  if (B < 0 || max_blocks < 0) return PA_ERR_INVALID;
  if (bs != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (B == 0) return PA_OK;
  if (!block_tables || !slots || !table_index) return PA_ERR_INVALID;
  return status_of(pa::launch_update_tables(block_tables, max_blocks, slots, table_index, B,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Fixed partitions: m, l [B][Hq][np] and o [B][Hq][np][D].
int64_t fixed_bytes(int32_t B, int32_t Hq, int32_t D, int64_t np) {
  if (np <= 1) return 0;
  const int64_t rows = static_cast<int64_t>(B) * Hq * np;
  return 2 * align256(rows * 4) + align256(rows * D * 4);
}

// Balanced schedule: m, l [nw][2][G], o [nw][2][G][D], merge records [nw][4].
int64_t balanced_bytes(int32_t G, int32_t D, int64_t nw) {
  const int64_t rows = nw * 2 * G;
  return 2 * align256(rows * 4) + align256(rows * D * 4) + align256(nw * 16);
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cached[dev] = n;
  return n;
}

// Workgroups of the balanced schedule: the resident ones, no more than there are units, a
// multiple of 8 (one per XCD) when there are 8 or more; 0 when the device cannot be queried.
int64_t balanced_workgroups(int32_t B, int32_t Hkv, int32_t max_seq_len) {
  const int cus = cu_count();
  if (cus <= 0) return 0;
  int64_t nw = static_cast<int64_t>(cus) * pa::mfma_workgroups_per_cu();
  if (nw > pa::kMaxBalancedWorkgroups) nw = pa::kMaxBalancedWorkgroups;
  const int64_t units = static_cast<int64_t>(Hkv) * B * ((max_seq_len + 31) / 32);
  if (nw > units) nw = units;
  if (nw >= 8) nw -= nw % 8;
  if (nw < 1) nw = 1;
  return nw;
}

// Shared-prefix decode: tokens per prefix-pass part and parts per output row.  A part is one
// workgroup item; at most 8 parts per row keep the states' memory below 8 (D + 2) floats per
// row.
void prefix_parts(int32_t max_seq_len, int32_t* tokens, int32_t* parts) {
  constexpr int64_t kMinPart = 1024, kMaxParts = pa::kMaxPrefixParts;
  int64_t np = (static_cast<int64_t>(max_seq_len) + kMinPart - 1) / kMinPart;
  if (np > kMaxParts) np = kMaxParts;
  if (np < 1) np = 1;
  int64_t pt = (static_cast<int64_t>(max_seq_len) + np - 1) / np;
  pt = (pt + 31) / 32 * 32;
  if (pt < 32) pt = 32;
  *tokens = static_cast<int32_t>(pt);
  *parts = static_cast<int32_t>((max_seq_len + pt - 1) / pt < 1 ? 1 : (max_seq_len + pt - 1) / pt);
}

// Shared-prefix decode workspace past the balanced schedule's: pstart, ref_p, grp_ref [B]; the
// prefix states m, l [B][Hq][parts] and o [B][Hq][parts][D]; the whole-segment states m, l
// [B][Hq], o [B][Hq][D] and their marks [B][Hkv].
int64_t shared_extra_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t max_seq_len) {
  int32_t pt = 0, np = 0;
  prefix_parts(max_seq_len, &pt, &np);
  const int64_t rows = static_cast<int64_t>(B) * Hq * np;
  const int64_t srows = static_cast<int64_t>(B) * Hq;
  return 3 * align256(static_cast<int64_t>(B) * 4) + 2 * align256(rows * 4) +
         align256(rows * D * 4) + 2 * align256(srows * 4) + align256(srows * D * 4) +
         align256(static_cast<int64_t>(B) * Hkv * 4);
}

// Whether pa_decode_shared_prefix runs its own schedule (else it is pa_decode).
bool shared_schedule(int32_t q_dtype, int32_t kv_dtype, int32_t B, int32_t Hq, int32_t Hkv) {
  const int G = Hq / Hkv;
  return q_dtype == PA_BF16 &&
         (kv_dtype == PA_BF16 || kv_dtype == PA_I8 || kv_dtype == PA_I4) &&
         (G == 1 || G == 2 || G == 4 || G == 8) && B <= pa::kMaxBalancedBatch;
}

}  // namespace

extern "C" {

size_t pa_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t max_seq_len, int32_t partition_tokens) {
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D < 1 || max_seq_len < 0 ||
      partition_tokens < 0)
    return 0;
  const int32_t P =
      partition_tokens ? partition_tokens : pa::auto_partition(B, Hkv);
  const int64_t np = (static_cast<int64_t>(max_seq_len) + P - 1) / P;
  int64_t bytes = fixed_bytes(B, Hq, D, np);
  if (partition_tokens == 0 && B <= pa::kMaxBalancedBatch && Hq / Hkv <= pa::kMaxBalancedGroup) {
    const int64_t bal = balanced_bytes(Hq / Hkv, D, pa::kMaxBalancedWorkgroups);
    bytes = bytes > bal ? bytes : bal;
  }
  return static_cast<size_t>(bytes < 256 ? 256 : bytes);
}

}  // extern "C"

namespace pa {

int decode_check(const float* out, const void* q, int32_t q_dtype, const void* k_cache,
                 const void* v_cache, int32_t kv_dtype, const float* k_scale,
                 const float* v_scale, const int32_t* block_tables, int32_t max_blocks,
                 const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t Hq,
                 int32_t Hkv, int32_t D, int32_t bs, int32_t NB, float scale,
                 int32_t partition_tokens, bool* nothing) {
  *nothing = false;
  if (B < 0 || Hq < 1 || Hkv < 1 || NB < 1 || max_blocks < 0 || max_seq_len < 0)
    return PA_ERR_INVALID;
  if (Hq % Hkv != 0 || (D != 64 && D != 128)) return PA_ERR_INVALID;
  if (Hq / Hkv > 16) return PA_ERR_UNSUPPORTED;
  if (bs != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (q_dtype != PA_F32 && q_dtype != PA_BF16) return PA_ERR_INVALID;
  if (!known_kv(kv_dtype)) return PA_ERR_INVALID;
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks) * bs)
    return PA_ERR_INVALID;
  if (partition_tokens != 0 &&
      (partition_tokens < 64 || partition_tokens > 8192 || partition_tokens % 64 != 0))
    return PA_ERR_INVALID;
  if (!(scale == scale)) return PA_ERR_INVALID;
  if (B == 0) {
    *nothing = true;
    return PA_OK;
  }
  if (!out || !q || !k_cache || !v_cache || !seq_lens || (max_blocks > 0 && !block_tables))
    return PA_ERR_INVALID;
  if (quantised(kv_dtype) && (!k_scale || !v_scale)) return PA_ERR_INVALID;
  const int32_t G = Hq / Hkv;  // int4 runs on the matrix-core kernel only
  const bool mfma_group = G == 1 || G == 2 || G == 4 || G == 8 || G == 16;
  if (kv_dtype == PA_I4 && (q_dtype != PA_BF16 || !mfma_group)) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int decode_run(float* out, const void* q, int32_t q_dtype, const void* k_cache,
               const void* v_cache, int32_t kv_dtype, const float* k_scale, const float* v_scale,
               const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
               int32_t max_seq_len, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t NB,
               float scale, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
               bool exact_size, void* stream) {
  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.tables = block_tables;
  a.seq_lens = seq_lens;
  a.max_blocks = max_blocks;
  a.max_seq_len = max_seq_len;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.NB = NB;
  a.partition = partition_tokens ? partition_tokens : pa::auto_partition(B, Hkv);
  const int64_t np = (static_cast<int64_t>(max_seq_len) + a.partition - 1) / a.partition;
  a.np_max = static_cast<int32_t>(np < 1 ? 1 : np);
  a.scale_log2 = scale * kLog2e;

  const int G = Hq / Hkv;
  const bool mfma = q_dtype == PA_BF16 &&
                    (kv_dtype == PA_BF16 || kv_dtype == PA_I8 || kv_dtype == PA_I4) &&
                    (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
  const bool balanced = mfma && partition_tokens == 0 && B <= pa::kMaxBalancedBatch &&
                        G <= pa::kMaxBalancedGroup;
  int64_t nw = 0;
  if (balanced) {
    nw = balanced_workgroups(B, Hkv, max_seq_len);
    if (nw <= 0) return PA_ERR_DEVICE;
  }
  if (exact_size) {
    // a fixed buffer: exactly what this call's schedule uses must fit
    const int64_t need = balanced ? balanced_bytes(G, D, nw) : fixed_bytes(B, Hq, D, a.np_max);
    if (static_cast<uint64_t>(need) > workspace_bytes) return PA_ERR_TOO_LARGE;
  } else if (!workspace ||
             workspace_bytes < pa_decode_workspace_size(B, Hq, Hkv, D, max_seq_len,
                                                        partition_tokens)) {
    return PA_ERR_INVALID;
  }
  char* base = static_cast<char*>(workspace);
  if (balanced) {
    a.nw = static_cast<int32_t>(nw);
    const int64_t rows = nw * 2 * G;
    a.ws_m = reinterpret_cast<float*>(base);
    a.ws_l = reinterpret_cast<float*>(base + align256(rows * 4));
    a.ws_o = reinterpret_cast<float*>(base + 2 * align256(rows * 4));
    a.ws_merge = reinterpret_cast<int32_t*>(base + 2 * align256(rows * 4) +
                                            align256(rows * D * 4));
  } else if (a.np_max > 1) {
    const int64_t rows = static_cast<int64_t>(B) * Hq * a.np_max;
    a.ws_m = reinterpret_cast<float*>(base);
    a.ws_l = reinterpret_cast<float*>(base + align256(rows * 4));
    a.ws_o = reinterpret_cast<float*>(base + 2 * align256(rows * 4));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = mfma ? pa::launch_decode_mfma(a, kv_dtype, s)
                      : pa::launch_decode_generic(a, q_dtype, kv_dtype, s);
  if (e != hipSuccess) return status_of(e);
  if (balanced) return PA_OK;
  return status_of(pa::launch_splitk_reduce(a, s));
}

}  // namespace pa

extern "C" {

int pa_decode(float* out, const void* q, int32_t q_dtype, const void* k_cache,
              const void* v_cache, int32_t kv_dtype, const float* k_scale, const float* v_scale,
              const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
              int32_t max_seq_len, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs,
              int32_t NB, float scale, int32_t partition_tokens, void* workspace,
              size_t workspace_bytes, void* stream) {
  bool nothing = false;
  const int st = pa::decode_check(out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                                  block_tables, max_blocks, seq_lens, max_seq_len, B, Hq, Hkv,
                                  D, bs, NB, scale, partition_tokens, &nothing);
  if (st != PA_OK || nothing) return st;
  return pa::decode_run(out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                        block_tables, max_blocks, seq_lens, max_seq_len, B, Hq, Hkv, D, NB,
                        scale, partition_tokens, workspace, workspace_bytes, false, stream);
}

size_t pa_decode_shared_prefix_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                              int32_t max_seq_len) {
  const size_t plain = pa_decode_workspace_size(B, Hq, Hkv, D, max_seq_len, 0);
  if (plain == 0 || B > pa::kMaxBalancedBatch || Hq / Hkv > pa::kMaxBalancedGroup) return plain;
  const int64_t bytes = balanced_bytes(Hq / Hkv, D, pa::kMaxBalancedWorkgroups) +
                        shared_extra_bytes(B, Hq, Hkv, D, max_seq_len);
  return static_cast<size_t>(bytes) > plain ? static_cast<size_t>(bytes) : plain;
}

int pa_decode_shared_prefix(float* out, const void* q, int32_t q_dtype, const void* k_cache,
                            const void* v_cache, int32_t kv_dtype, const float* k_scale,
                            const float* v_scale, const int32_t* block_tables, int32_t max_blocks,
                            const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t Hq,
                            int32_t Hkv, int32_t D, int32_t bs, int32_t NB, float scale,
                            void* workspace, size_t workspace_bytes, void* stream) {
  bool nothing = false;
  const int st = pa::decode_check(out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                                  block_tables, max_blocks, seq_lens, max_seq_len, B, Hq, Hkv,
                                  D, bs, NB, scale, 0, &nothing);
  if (st != PA_OK || nothing) return st;
  if (!workspace ||
      workspace_bytes < pa_decode_shared_prefix_workspace_size(B, Hq, Hkv, D, max_seq_len))
    return PA_ERR_INVALID;
  if (!shared_schedule(q_dtype, kv_dtype, B, Hq, Hkv))
    return pa::decode_run(out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                          block_tables, max_blocks, seq_lens, max_seq_len, B, Hq, Hkv, D, NB,
                          scale, 0, workspace, workspace_bytes, false, stream);
  const int64_t nw = balanced_workgroups(B, Hkv, max_seq_len);
  if (nw <= 0) return PA_ERR_DEVICE;
  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.tables = block_tables;
  a.seq_lens = seq_lens;
  a.max_blocks = max_blocks;
  a.max_seq_len = max_seq_len;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.NB = NB;
  a.partition = 512;  // unused by the balanced schedule
  a.np_max = 1;
  a.scale_log2 = scale * kLog2e;
  a.nw = static_cast<int32_t>(nw);
  const int G = Hq / Hkv;
  char* base = static_cast<char*>(workspace);
  const int64_t rows = nw * 2 * G;
  a.ws_m = reinterpret_cast<float*>(base);
  a.ws_l = reinterpret_cast<float*>(base + align256(rows * 4));
  a.ws_o = reinterpret_cast<float*>(base + 2 * align256(rows * 4));
  a.ws_merge =
      reinterpret_cast<int32_t*>(base + 2 * align256(rows * 4) + align256(rows * D * 4));
  char* p = base + balanced_bytes(G, D, nw);
  const int64_t bb = align256(static_cast<int64_t>(B) * 4);
  a.pstart = reinterpret_cast<int32_t*>(p);
  a.ref_p = reinterpret_cast<int32_t*>(p + bb);
  a.grp_ref = reinterpret_cast<int32_t*>(p + 2 * bb);
  prefix_parts(max_seq_len, &a.pf_tokens, &a.pf_parts);
  const int64_t prow = static_cast<int64_t>(B) * Hq * a.pf_parts;
  a.pf_m = reinterpret_cast<float*>(p + 3 * bb);
  a.pf_l = reinterpret_cast<float*>(p + 3 * bb + align256(prow * 4));
  a.pf_o = reinterpret_cast<float*>(p + 3 * bb + 2 * align256(prow * 4));
  char* q2 = p + 3 * bb + 2 * align256(prow * 4) + align256(prow * D * 4);
  const int64_t srow = static_cast<int64_t>(B) * Hq;
  a.sf_m = reinterpret_cast<float*>(q2);
  a.sf_l = reinterpret_cast<float*>(q2 + align256(srow * 4));
  a.sf_o = reinterpret_cast<float*>(q2 + 2 * align256(srow * 4));
  a.sf_mark = reinterpret_cast<int32_t*>(q2 + 2 * align256(srow * 4) + align256(srow * D * 4));
  a.pf_gmax = B / 2 + 1;
  return status_of(pa::launch_decode_shared_prefix(a, kv_dtype, static_cast<hipStream_t>(stream)));
}

int pa_prefill(float* out, const void* q, int32_t q_dtype, const void* k_cache,
               const void* v_cache, int32_t kv_dtype, const float* k_scale, const float* v_scale,
               const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
               const int32_t* cu_q, int32_t max_seq_len, int32_t B, int32_t T, int32_t Hq,
               int32_t Hkv, int32_t D, int32_t bs, int32_t NB, float scale, void* stream) {
  if (B < 0 || T < 0 || Hq < 1 || Hkv < 1 || NB < 1 || max_blocks < 0 || max_seq_len < 0)
    return PA_ERR_INVALID;
  if (Hq % Hkv != 0 || (D != 64 && D != 128)) return PA_ERR_INVALID;
  const int32_t G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return PA_ERR_UNSUPPORTED;
  if (bs != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (q_dtype != PA_BF16 || kv_dtype == PA_F32) {
    const bool known = (q_dtype == PA_F32 || q_dtype == PA_BF16) && known_kv(kv_dtype);
    return known ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID;
  }
  if (!known_kv(kv_dtype)) return PA_ERR_INVALID;
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks) * bs)
    return PA_ERR_INVALID;
  if (!(scale == scale)) return PA_ERR_INVALID;
  if (B == 0 || T == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !seq_lens || !cu_q || (max_blocks > 0 && !block_tables))
    return PA_ERR_INVALID;
  if (quantised(kv_dtype) && (!k_scale || !v_scale)) return PA_ERR_INVALID;
  pa::PrefillArgs a{};
  a.kv_kind = kv_dtype == PA_I8 ? pa::kKvI8 : (kv_dtype == PA_I4 ? pa::kKvI4 : pa::kKvBf16);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = block_tables;
  a.seq_lens = seq_lens;
  a.cu_q = cu_q;
  a.max_blocks = max_blocks;
  a.max_seq_len = max_seq_len;
  a.B = B;
  a.T = T;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.NB = NB;
  const int64_t tiles = (static_cast<int64_t>(T) + 63) / 64 + B;  // sum of ceil(n_b / 64)
  // one workgroup per (query group, KV head, block of up to 4 heads) in a 1-D grid; query
  // positions and key reaches stay within +-(T + max_seq_len)
  if (tiles * Hq > INT32_MAX || static_cast<int64_t>(T) + max_seq_len > INT32_MAX / 2)
    return PA_ERR_INVALID;
  a.max_tiles = static_cast<int32_t>(tiles);
  a.scale_log2 = scale * kLog2e;
  return status_of(pa::launch_prefill_mfma(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
