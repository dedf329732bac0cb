// pa_decode_no_alloc: pa_decode with its workspace in a fixed device array of the library, for
// callers that cannot allocate device memory (graph capture, tight serving loops).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "internal.h"
#include "pagedkv.h"

// The scratch of every pa_decode_no_alloc call on a GPU: each GPU the library runs on holds its
// own copy, at its own address, until the process ends.
static __device__ __align__(256) unsigned char scratch[PA_DECODE_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on each GPU, looked up once per device with that device current.
// (In host code the array's name is only a stand-in for the symbol, never an address.)
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_no_alloc(float* out, const void* q, int32_t q_dtype,
                                  const void* k_cache, const void* v_cache, int32_t kv_dtype,
                                  const float* k_scale, const float* v_scale,
                                  const int32_t* block_tables, int32_t max_blocks,
                                  const int32_t* seq_lens, int32_t max_seq_len, int32_t B,
                                  int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t NB,
                                  float scale, int32_t partition_tokens, void* stream) {
  bool nothing = false;
  int st = pa::decode_check(out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                            block_tables, max_blocks, seq_lens, max_seq_len, B, Hq, Hkv, D, bs,
                            NB, scale, partition_tokens, &nothing);
  if (st != PA_OK || nothing) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != PA_OK) return st;
  return pa::decode_run(out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                        block_tables, max_blocks, seq_lens, max_seq_len, B, Hq, Hkv, D, NB,
                        scale, partition_tokens, ws, PA_DECODE_SCRATCH_BYTES, true, stream);
}
