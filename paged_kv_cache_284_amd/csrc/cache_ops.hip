// Writes into the paged cache: token append, copy-on-write block copies, block-table patches.
//
// Append ("How LLM Inference Serving Works", "What the KV Cache Is, and How Big It Gets": every
// decode step appends one token's K and V; "The Life of a Request": into the request's current
// block).  Copy-on-write ("Sharing comes for free": a shared block is copied only when a branch
// writes to it).  All three are bit copies; they move a few KiB to a few MiB per step and are
// bound by launch latency, so they favour simple, fully coalesced addressing over occupancy
// tuning.
#include "internal.h"

namespace pa {
namespace {

// One workgroup per sequence.  Its first thread reads the sequence's slot (and table index and
// length) once -- those arrays may live in pinned host memory, where every read crosses the bus
// -- and the workgroup's threads then copy the Hkv x D elements.  K rows are contiguous in the
// tile; V is dim-major, so consecutive d land 32 B (bf16) apart -- the write is small enough for
// that not to matter.  With a table (the fused step) the first thread also patches the
// sequence's block-table entry when the step gave it a new or copied block, and with lens_out it
// copies the sequence's new length.
template <typename T>
__global__ void __launch_bounds__(256) kv_append_kernel(const T* __restrict__ k_new,
                                                        const T* __restrict__ v_new,
                                                        const int64_t* __restrict__ slots,
                                                        T* __restrict__ k_cache,
                                                        T* __restrict__ v_cache, int32_t Hkv,
                                                        int32_t D, int32_t NB,
                                                        const int32_t* __restrict__ table_index,
                                                        int32_t* __restrict__ tables,
                                                        int32_t max_blocks,
                                                        const int32_t* __restrict__ lens_in,
                                                        int32_t* __restrict__ lens_out) {
  const int32_t b = blockIdx.x;
  __shared__ int64_t slot_s;
  __shared__ int32_t index_s;
  // three threads issue the three reads at once: one bus round trip
  if (threadIdx.x == 0) {
    const int64_t slot = slots[b];
    slot_s = (slot >= 0 && slot < static_cast<int64_t>(NB) * kBlockSize) ? slot : -1;
  } else if (threadIdx.x == 1) {
    index_s = tables ? table_index[b] : -1;
  } else if (threadIdx.x == 2 && lens_out) {
    lens_out[b] = lens_in[b];
  }
  __syncthreads();
  const int64_t slot = slot_s;
  if (slot < 0) return;
  if (threadIdx.x == 0 && index_s >= 0 && index_s < max_blocks)
    tables[static_cast<int64_t>(b) * max_blocks + index_s] = static_cast<int32_t>(slot / kBlockSize);
  const int64_t blk = slot / kBlockSize;
  const int32_t off = static_cast<int32_t>(slot % kBlockSize);
  const int32_t n = Hkv * D;
  const T* kn = k_new + static_cast<int64_t>(b) * n;
  const T* vn = v_new + static_cast<int64_t>(b) * n;
  for (int32_t e = threadIdx.x; e < n; e += blockDim.x) {
    const int32_t g = e / D, d = e % D;
    const int64_t tile = blk * Hkv + g;
    k_cache[(tile * kBlockSize + off) * D + d] = kn[e];
    v_cache[(tile * D + d) * kBlockSize + off] = vn[e];
  }
}

// One workgroup per pair; its threads stride over the 16-byte chunks of the K and V tiles.
__global__ void __launch_bounds__(256) copy_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          float* __restrict__ k_scale,
                                                          float* __restrict__ v_scale,
                                                          const int32_t* __restrict__ pairs,
                                                          int32_t chunks, int32_t Hkv,
                                                          int32_t NB) {
  __shared__ int32_t pair_s[2];  // read once: the pairs may live in pinned host memory
  if (threadIdx.x < 2) pair_s[threadIdx.x] = pairs[2 * blockIdx.x + threadIdx.x];
  __syncthreads();
  const int32_t src = pair_s[0], dst = pair_s[1];
  if (src < 0 || src >= NB || dst < 0 || dst >= NB) return;
  const int64_t s0 = static_cast<int64_t>(src) * chunks;
  const int64_t d0 = static_cast<int64_t>(dst) * chunks;
  for (int32_t c = threadIdx.x; c < chunks; c += blockDim.x) {
    k_cache[d0 + c] = k_cache[s0 + c];
    v_cache[d0 + c] = v_cache[s0 + c];
  }
  if (k_scale) {
    for (int32_t g = threadIdx.x; g < Hkv; g += blockDim.x) {
      k_scale[static_cast<int64_t>(dst) * Hkv + g] = k_scale[static_cast<int64_t>(src) * Hkv + g];
      v_scale[static_cast<int64_t>(dst) * Hkv + g] = v_scale[static_cast<int64_t>(src) * Hkv + g];
    }
  }
}

__global__ void __launch_bounds__(256) update_tables_kernel(int32_t* __restrict__ tables,
                                                            int32_t max_blocks,
                                                            const int64_t* __restrict__ slots,
                                                            const int32_t* __restrict__ table_index,
                                                            int32_t B) {
  const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B) return;
  const int32_t j = table_index[i];
  const int64_t slot = slots[i];
  if (j < 0 || j >= max_blocks || slot < 0) return;
  tables[static_cast<int64_t>(i) * max_blocks + j] = static_cast<int32_t>(slot / kBlockSize);
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int64_t* slots,
                            void* k_cache, void* v_cache, int32_t B, int32_t Hkv, int32_t D,
                            int32_t NB, int32_t elem_bytes, const int32_t* table_index,
                            int32_t* tables, int32_t max_blocks, const int32_t* lens_in,
                            int32_t* lens_out, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (!table_index) tables = nullptr;
  if (!lens_in) lens_out = nullptr;
  const dim3 grid(static_cast<unsigned>(B));
  if (elem_bytes == 4) {
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint32_t*>(k_new), static_cast<const uint32_t*>(v_new),
                       slots, static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache),
                       Hkv, D, NB, table_index, tables, max_blocks, lens_in, lens_out);
  } else if (elem_bytes == 2) {
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       slots, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                       Hkv, D, NB, table_index, tables, max_blocks, lens_in, lens_out);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* pairs, int32_t n, int32_t Hkv, int32_t D,
                              int32_t NB, int32_t elem_bytes, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t tile_bytes = static_cast<int64_t>(Hkv) * kBlockSize * D * elem_bytes;
  const int32_t chunks = static_cast<int32_t>(tile_bytes / 16);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n), dim3(256), 0, stream,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), k_scale, v_scale,
                     pairs, chunks, Hkv, NB);
  return hipGetLastError();
}

hipError_t launch_update_tables(int32_t* tables, int32_t max_blocks, const int64_t* slots,
                                const int32_t* table_index, int32_t B, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(update_tables_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, tables,
                     max_blocks, slots, table_index, B);
  return hipGetLastError();
}

}  // namespace pa
