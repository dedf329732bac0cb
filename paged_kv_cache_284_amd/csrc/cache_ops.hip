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

// Quantising append into an int8 cache.  One wave per (batch entry, KV head); the wave of the
// first entry of a run of consecutive entries that write into the same block takes the whole
// run in order (a block's scale and codes evolve token by token), the others exit.  Per token
// and for K and V alike (all fp32, IEEE division, round-half-to-even): c = max|x| / 127; a fresh
// block (offset 0) takes scale c; otherwise a larger c grows the scale to c and re-rounds the
// block's earlier codes by old/c; the new slot gets clamp(rint(x / scale), -127, 127) (0 for a
// zero scale).  Lane l only ever touches dims d = l (mod 64) of the tile, so the re-rounding
// reads back only what the same lane wrote.
template <typename TIn>
__device__ __forceinline__ float widen(TIn x);
template <>
__device__ __forceinline__ float widen<float>(float x) { return x; }
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

template <typename TIn>
__device__ void quantise_token(const TIn* __restrict__ x, int8_t* tile, float* scale_slot,
                               float* scale_reg, bool fresh, int off, int D, bool token_major) {
  const int lane = threadIdx.x;
  float amax = 0.f;
  for (int d = lane; d < D; d += 64) amax = fmaxf(amax, fabsf(widen<TIn>(x[d])));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float cand = amax / 127.f;
  float scale;
  if (fresh) {
    scale = cand;
  } else {
    const float old = *scale_reg;
    scale = old;
    if (cand > old) {
      const float r = old / cand;
      for (int d = lane; d < D; d += 64) {
        for (int row = 0; row < off; ++row) {
          int8_t* c = token_major ? tile + row * D + d : tile + d * kBlockSize + row;
          const float q = __builtin_rintf(static_cast<float>(*c) * r);
          *c = static_cast<int8_t>(fminf(fmaxf(q, -127.f), 127.f));
        }
      }
      scale = cand;
    }
  }
  for (int d = lane; d < D; d += 64) {
    float q = 0.f;
    if (scale > 0.f) q = fminf(fmaxf(__builtin_rintf(widen<TIn>(x[d]) / scale), -127.f), 127.f);
    int8_t* c = token_major ? tile + off * D + d : tile + d * kBlockSize + off;
    *c = static_cast<int8_t>(q);
  }
  *scale_reg = scale;
  if (lane == 0) *scale_slot = scale;
}

template <typename TIn>
__global__ void __launch_bounds__(64) kv_append_i8_kernel(const TIn* __restrict__ k_new,
                                                           const TIn* __restrict__ v_new,
                                                           const int64_t* __restrict__ slots,
                                                           int8_t* k_cache, int8_t* v_cache,
                                                           float* k_scale, float* v_scale,
                                                           int32_t B, int32_t Hkv, int32_t D,
                                                           int32_t NB) {
  const int i = blockIdx.x, g = blockIdx.y;
  const int64_t cap = static_cast<int64_t>(NB) * kBlockSize;
  auto block_of = [&](int64_t s) -> int64_t { return (s >= 0 && s < cap) ? s / kBlockSize : -1; };
  const int64_t blk = block_of(slots[i]);
  if (blk < 0) return;
  if (i > 0 && block_of(slots[i - 1]) == blk) return;  // not the first entry of its run
  const int64_t tile = blk * Hkv + g;
  int8_t* kt = k_cache + tile * kBlockSize * D;
  int8_t* vt = v_cache + tile * kBlockSize * D;
  float ks_reg = k_scale[tile], vs_reg = v_scale[tile];  // the block's scales so far
  for (int j = i; j < B; ++j) {
    const int64_t sj = slots[j];
    if (block_of(sj) != blk) break;
    const int off = static_cast<int>(sj % kBlockSize);
    const int64_t src = (static_cast<int64_t>(j) * Hkv + g) * D;
    quantise_token<TIn>(k_new + src, kt, k_scale + tile, &ks_reg, off == 0, off, D, true);
    quantise_token<TIn>(v_new + src, vt, v_scale + tile, &vs_reg, off == 0, off, D, false);
  }
}

// Quantising append into a packed int4 cache: the int8 rule with 7 in place of 127, codes
// stored as nibbles c + 8 (a 4-byte group holds 8 consecutive elements of a row: 0..3 in the
// low nibbles, 4..7 in the high ones).  K rows are dims of one token: lane l owns byte l of the
// row (two dims), so a token's row is written whole.  V rows are tokens of one dim: lane l owns
// dims l, l + 64, and a token is one nibble, read-modified-written by its dim's lane.
__device__ __forceinline__ int nibble_code(uint8_t byte, int hi) {
  return static_cast<int>((byte >> (4 * hi)) & 0xf) - 8;
}
__device__ __forceinline__ uint8_t with_nibble(uint8_t byte, int hi, int code) {
  const uint8_t u = static_cast<uint8_t>(code + 8) & 0xf;
  return hi ? static_cast<uint8_t>((byte & 0x0f) | (u << 4)) : static_cast<uint8_t>((byte & 0xf0) | u);
}
__device__ __forceinline__ int quant7(float x, float scale) {
  if (!(scale > 0.f)) return 0;
  return static_cast<int>(fminf(fmaxf(__builtin_rintf(x / scale), -7.f), 7.f));
}
__device__ __forceinline__ int requant7(int code, float r) {
  return static_cast<int>(fminf(fmaxf(__builtin_rintf(static_cast<float>(code) * r), -7.f), 7.f));
}
__device__ __forceinline__ float wave_absmax(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// New scale of a block for a token whose own scale would be `cand` (see the int8 kernel).
__device__ __forceinline__ float next_scale(bool fresh, float old, float cand, bool* grew) {
  *grew = !fresh && cand > old;
  return (fresh || cand > old) ? cand : old;
}

template <typename TIn>
__device__ void append_i4_k(const TIn* __restrict__ x, uint8_t* tile, float* scale_slot,
                            float* scale_reg, bool fresh, int off, int D) {
  const int lane = threadIdx.x;
  const int row_bytes = D / 2;
  const bool mine = lane < row_bytes;
  const int e_lo = 8 * (lane / 4) + lane % 4, e_hi = e_lo + 4;  // the dims of byte `lane`
  const float x_lo = mine ? widen<TIn>(x[e_lo]) : 0.f;
  const float x_hi = mine ? widen<TIn>(x[e_hi]) : 0.f;
  const float cand = wave_absmax(fmaxf(fabsf(x_lo), fabsf(x_hi))) / 7.f;
  bool grew;
  const float scale = next_scale(fresh, *scale_reg, cand, &grew);
  if (grew && mine) {
    const float r = *scale_reg / cand;
    for (int row = 0; row < off; ++row) {
      uint8_t* p = tile + row * row_bytes + lane;
      const uint8_t b = *p;
      *p = with_nibble(with_nibble(b, 0, requant7(nibble_code(b, 0), r)), 1,
                       requant7(nibble_code(b, 1), r));
    }
  }
  if (mine) {
    tile[off * row_bytes + lane] =
        with_nibble(with_nibble(0, 0, quant7(x_lo, scale)), 1, quant7(x_hi, scale));
  }
  *scale_reg = scale;
  if (lane == 0) *scale_slot = scale;
}

template <typename TIn>
__device__ void append_i4_v(const TIn* __restrict__ x, uint8_t* tile, float* scale_slot,
                            float* scale_reg, bool fresh, int off, int D) {
  const int lane = threadIdx.x;
  constexpr int kRowBytes = kBlockSize / 2;
  float amax = 0.f;
  for (int d = lane; d < D; d += 64) amax = fmaxf(amax, fabsf(widen<TIn>(x[d])));
  const float cand = wave_absmax(amax) / 7.f;
  bool grew;
  const float scale = next_scale(fresh, *scale_reg, cand, &grew);
  auto at = [](int t) { return 4 * (t / 8) + t % 4; };  // byte of token t in a dim row
  for (int d = lane; d < D; d += 64) {
    uint8_t* row = tile + d * kRowBytes;
    if (grew) {
      const float r = *scale_reg / cand;
      for (int t = 0; t < off; ++t) {
        const int hi = (t % 8) / 4;
        row[at(t)] = with_nibble(row[at(t)], hi, requant7(nibble_code(row[at(t)], hi), r));
      }
    }
    const int hi = (off % 8) / 4;
    row[at(off)] = with_nibble(row[at(off)], hi, quant7(widen<TIn>(x[d]), scale));
  }
  *scale_reg = scale;
  if (lane == 0) *scale_slot = scale;
}

template <typename TIn>
__global__ void __launch_bounds__(64) kv_append_i4_kernel(const TIn* __restrict__ k_new,
                                                           const TIn* __restrict__ v_new,
                                                           const int64_t* __restrict__ slots,
                                                           uint8_t* k_cache, uint8_t* v_cache,
                                                           float* k_scale, float* v_scale,
                                                           int32_t B, int32_t Hkv, int32_t D,
                                                           int32_t NB) {
  const int i = blockIdx.x, g = blockIdx.y;
  const int64_t cap = static_cast<int64_t>(NB) * kBlockSize;
  auto block_of = [&](int64_t s) -> int64_t { return (s >= 0 && s < cap) ? s / kBlockSize : -1; };
  const int64_t blk = block_of(slots[i]);
  if (blk < 0) return;
  if (i > 0 && block_of(slots[i - 1]) == blk) return;  // not the first entry of its run
  const int64_t tile = blk * Hkv + g;
  uint8_t* kt = k_cache + tile * kBlockSize * (D / 2);
  uint8_t* vt = v_cache + tile * kBlockSize * (D / 2);
  float ks_reg = k_scale[tile], vs_reg = v_scale[tile];
  for (int j = i; j < B; ++j) {
    const int64_t sj = slots[j];
    if (block_of(sj) != blk) break;
    const int off = static_cast<int>(sj % kBlockSize);
    const int64_t src = (static_cast<int64_t>(j) * Hkv + g) * D;
    append_i4_k<TIn>(k_new + src, kt, k_scale + tile, &ks_reg, off == 0, off, D);
    append_i4_v<TIn>(v_new + src, vt, v_scale + tile, &vs_reg, off == 0, off, D);
  }
}

// One workgroup per pair; its threads stride over the 16-byte chunks of the K and V tiles.
// Source and destination pools may be the same (copy-on-write) or different (swapping to and
// from a host pool in pinned memory, which the kernel reads or writes over the bus).
__global__ void __launch_bounds__(256) copy_tiles_kernel(const uint4* src_k, const uint4* src_v,
                                                         const float* src_ks, const float* src_vs,
                                                         int32_t src_blocks, uint4* dst_k,
                                                         uint4* dst_v, float* dst_ks,
                                                         float* dst_vs, int32_t dst_blocks,
                                                         const int32_t* __restrict__ pairs,
                                                         int32_t chunks, int32_t Hkv) {
  __shared__ int32_t pair_s[2];  // read once: the pairs may live in pinned host memory
  if (threadIdx.x < 2) pair_s[threadIdx.x] = pairs[2 * blockIdx.x + threadIdx.x];
  __syncthreads();
  const int32_t src = pair_s[0], dst = pair_s[1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const int64_t s0 = static_cast<int64_t>(src) * chunks;
  const int64_t d0 = static_cast<int64_t>(dst) * chunks;
  for (int32_t c = threadIdx.x; c < chunks; c += blockDim.x) {
    dst_k[d0 + c] = src_k[s0 + c];
    dst_v[d0 + c] = src_v[s0 + c];
  }
  if (src_ks) {
    for (int32_t g = threadIdx.x; g < Hkv; g += blockDim.x) {
      dst_ks[static_cast<int64_t>(dst) * Hkv + g] = src_ks[static_cast<int64_t>(src) * Hkv + g];
      dst_vs[static_cast<int64_t>(dst) * Hkv + g] = src_vs[static_cast<int64_t>(src) * Hkv + g];
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

hipError_t launch_kv_append_i8(const void* k_new, const void* v_new, bool bf16_new,
                               const int64_t* slots, int8_t* k_cache, int8_t* v_cache,
                               float* k_scale, float* v_scale, int32_t B, int32_t Hkv, int32_t D,
                               int32_t NB, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(B), static_cast<unsigned>(Hkv));
  if (bf16_new) {
    hipLaunchKernelGGL(kv_append_i8_kernel<uint16_t>, grid, dim3(64), 0, stream,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       slots, k_cache, v_cache, k_scale, v_scale, B, Hkv, D, NB);
  } else {
    hipLaunchKernelGGL(kv_append_i8_kernel<float>, grid, dim3(64), 0, stream,
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new), slots,
                       k_cache, v_cache, k_scale, v_scale, B, Hkv, D, NB);
  }
  return hipGetLastError();
}

hipError_t launch_kv_append_i4(const void* k_new, const void* v_new, bool bf16_new,
                               const int64_t* slots, uint8_t* k_cache, uint8_t* v_cache,
                               float* k_scale, float* v_scale, int32_t B, int32_t Hkv, int32_t D,
                               int32_t NB, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(B), static_cast<unsigned>(Hkv));
  if (bf16_new) {
    hipLaunchKernelGGL(kv_append_i4_kernel<uint16_t>, grid, dim3(64), 0, stream,
                       static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       slots, k_cache, v_cache, k_scale, v_scale, B, Hkv, D, NB);
  } else {
    hipLaunchKernelGGL(kv_append_i4_kernel<float>, grid, dim3(64), 0, stream,
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new), slots,
                       k_cache, v_cache, k_scale, v_scale, B, Hkv, D, NB);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                              const int32_t* pairs, int32_t n, int32_t Hkv, int32_t NB,
                              int64_t block_bytes, hipStream_t stream) {
  return launch_copy_tiles(k_cache, v_cache, k_scale, v_scale, NB, k_cache, v_cache, k_scale,
                           v_scale, NB, pairs, n, Hkv, block_bytes, stream);
}

hipError_t launch_copy_tiles(const void* src_k, const void* src_v, const float* src_ks,
                             const float* src_vs, int32_t src_blocks, void* dst_k, void* dst_v,
                             float* dst_ks, float* dst_vs, int32_t dst_blocks,
                             const int32_t* pairs, int32_t n, int32_t Hkv, int64_t block_bytes,
                             hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int32_t chunks = static_cast<int32_t>(block_bytes / 16);
  hipLaunchKernelGGL(copy_tiles_kernel, dim3(n), dim3(256), 0, stream,
                     static_cast<const uint4*>(src_k), static_cast<const uint4*>(src_v), src_ks,
                     src_vs, src_blocks, static_cast<uint4*>(dst_k), static_cast<uint4*>(dst_v),
                     dst_ks, dst_vs, dst_blocks, pairs, chunks, Hkv);
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
