// Writes into the paged cache: token append, copy-on-write block copies, block-table patches.
//
// Append ("How LLM Inference Serving Works", "What the KV Cache Is, and How Big It Gets": the
// cache grows by one token's K and V per decode step; "The Life of a Request": that token lands
// in the request's last block).  Copy-on-write ("Sharing comes for free": a block held by
// several sequences is duplicated when one of them writes into it).  All three are bit copies; they move a few KiB to a few MiB per step and are
// bound by launch latency, so they favour simple, fully coalesced addressing over occupancy
// tuning.
#include <type_traits>

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
  // the new token's values do not depend on the slot: request them before the slot, so the
  // HBM read overlaps the bus round trip to the step's arrays (at most 4 elements per thread
  // for Hkv * D <= 1024; larger rows take the loop below)
  constexpr int kPre = 4;
  const int32_t n = Hkv * D;
  const T* kn = k_new + static_cast<int64_t>(b) * n;
  const T* vn = v_new + static_cast<int64_t>(b) * n;
  T kv[kPre], vv[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int32_t e = threadIdx.x + i * static_cast<int32_t>(blockDim.x);
    if (e < n) {
      kv[i] = kn[e];
      vv[i] = vn[e];
    }
  }
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
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int32_t e = threadIdx.x + i * static_cast<int32_t>(blockDim.x);
    if (e < n) {
      const int32_t g = e / D, d = e % D;
      const int64_t tile = blk * Hkv + g;
      k_cache[(tile * kBlockSize + off) * D + d] = kv[i];
      v_cache[(tile * D + d) * kBlockSize + off] = vv[i];
    }
  }
  for (int32_t e = threadIdx.x + kPre * static_cast<int32_t>(blockDim.x); e < n;
       e += blockDim.x) {
    const int32_t g = e / D, d = e % D;
    const int64_t tile = blk * Hkv + g;
    k_cache[(tile * kBlockSize + off) * D + d] = kn[e];
    v_cache[(tile * D + d) * kBlockSize + off] = vn[e];
  }
}

// Quantising appends into int8 and packed int4 caches.  One wave per (batch entry, KV head), four
// entries to a workgroup; the wave of the first entry of a run of consecutive entries that write
// into the same block takes the whole run in order (a block's scale and codes evolve token by
// token), the others exit.
// Per token and for K and V alike (all fp32, IEEE division, round-half-to-even): c = max|x| /
// qmax (qmax 127 for int8, 7 for int4); a fresh block (offset 0) takes scale c; otherwise a
// larger c grows the scale to c and re-rounds the block's earlier rows by old/c; the new row gets
// clamp(rint(x / scale), -qmax, qmax) (0 for a zero scale).  The wave holds the whole (block,
// head) tile's codes in registers for the run -- each lane a fixed share of the elements of
// every row -- and writes the tile and its scales back once at the end.
//
// Element ownership.  K rows are the dims of one token: int8 lane l owns dims l + 64 j; int4 lane
// l owns byte l of a row (dims 8 (l / 4) + l % 4 and that + 4: a 4-byte group holds 8
// consecutive elements, 0..3 in the low nibbles, 4..7 in the high ones).  V rows are the 16
// tokens of one dim: lane l owns dims l + 64 j for both widths.
template <typename TIn>
__device__ __forceinline__ float widen(TIn x);
template <>
__device__ __forceinline__ float widen<float>(float x) { return x; }
template <>
__device__ __forceinline__ float widen<uint16_t>(uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

template <int kQMax>
__device__ __forceinline__ int quant_code(float x, float scale) {
  if (!(scale > 0.f)) return 0;
  return static_cast<int>(fminf(fmaxf(__builtin_rintf(x / scale), -float(kQMax)), float(kQMax)));
}
template <int kQMax>
__device__ __forceinline__ int requant_code(int code, float r) {
  return static_cast<int>(
      fminf(fmaxf(__builtin_rintf(static_cast<float>(code) * r), -float(kQMax)), float(kQMax)));
}
// Maximum over the wave of non-negative values, by register moves only: DPP rotations and quad
// permutes inside each 16-lane row, then the gfx950 row and half swaps.  (Exact: max does not
// depend on the order.)
template <int kCtrl>
__device__ __forceinline__ float max_dpp(float v) {
  const int o = __builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xf, 0xf, false);
  return fmaxf(v, __int_as_float(o));
}
__device__ __forceinline__ float wave_absmax(float v) {
  v = max_dpp<0x128>(v);  // row_ror:8
  v = max_dpp<0x124>(v);  // row_ror:4
  v = max_dpp<0x4e>(v);   // quad_perm [2, 3, 0, 1]
  v = max_dpp<0xb1>(v);   // quad_perm [1, 0, 3, 2]
  auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
}
// byte and nibble of element t (0..15) in a packed 8-byte row
__device__ __forceinline__ int nib_byte(int t) { return 4 * (t / 8) + t % 4; }
__device__ __forceinline__ int nib_shift(int t) { return 4 * ((t % 8) / 4); }

// One token's rule on the codes of one tile held as code[row][k] (k < kK: the elements this
// lane owns in each row), with the token's values x[k] and the tile's scale so far.
template <int kQMax, int kK>
__device__ __forceinline__ void quantise_row(int (&code)[kBlockSize][kK], const float (&x)[kK],
                                             float* scale, int off) {
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < kK; ++k) amax = fmaxf(amax, fabsf(x[k]));
  const float cand = wave_absmax(amax) / static_cast<float>(kQMax);
  const float old = *scale;
  // every row is visited with a select, so that each code stays in its own register
  if (off != 0 && cand > old) {
    const float r = old / cand;
#pragma unroll
    for (int row = 0; row < kBlockSize; ++row)
#pragma unroll
      for (int k = 0; k < kK; ++k)
        code[row][k] = row < off ? requant_code<kQMax>(code[row][k], r) : code[row][k];
  }
  const float sc = (off == 0 || cand > old) ? cand : old;
#pragma unroll
  for (int k = 0; k < kK; ++k) {
    const int q = quant_code<kQMax>(x[k], sc);
#pragma unroll
    for (int row = 0; row < kBlockSize; ++row) code[row][k] = row == off ? q : code[row][k];
  }
  *scale = sc;
}

constexpr int kAppendWaves = 4;  // entries (one wave each) per workgroup of the quantising append

// blockIdx.z = 0 quantises K, 1 quantises V: the two evolve independently, so each wave carries
// only one token-by-token chain.
template <typename TIn, int D, int kQMax>
__global__ void __launch_bounds__(64 * kAppendWaves) kv_append_quant_kernel(
    const TIn* __restrict__ k_new, const TIn* __restrict__ v_new,
    const int64_t* __restrict__ slots, uint8_t* k_cache, uint8_t* v_cache, float* k_scale,
    float* v_scale, int32_t B, int32_t Hkv, int32_t NB) {
  constexpr bool kI4 = kQMax == 7;
  constexpr int kJ = D / 64;                       // dims per lane (int8 K, and V)
  constexpr int kKE = kI4 ? 2 : kJ;                // K elements per lane and row
  constexpr int kRowK = kI4 ? D / 2 : D;           // bytes per K row
  constexpr int kRowV = kI4 ? kBlockSize / 2 : kBlockSize;  // bytes per V row
  const int lane = threadIdx.x % 64;
  const int i = blockIdx.x * kAppendWaves + static_cast<int>(threadIdx.x) / 64;  // wave's entry
  const int g = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  if (i >= B) return;  // the waves of a workgroup are independent: no barrier follows
  const int64_t cap = static_cast<int64_t>(NB) * kBlockSize;
  auto block_of = [&](int64_t s) -> int64_t { return (s >= 0 && s < cap) ? s / kBlockSize : -1; };
  const int64_t blk = block_of(slots[i]);
  if (blk < 0) return;
  if (i > 0 && block_of(slots[i - 1]) == blk) return;  // not the first entry of its run
  const int64_t tile = blk * Hkv + g;
  const bool kmine = !kI4 || lane < D / 2;        // int4 K: lanes past the row's bytes own none
  const int e_lo = 8 * (lane / 4) + lane % 4;      // int4 K: the dims of byte `lane`
  const TIn* x_new = is_v ? v_new : k_new;
  float* scale_slot = (is_v ? v_scale : k_scale) + tile;

  // the run's entries, 16 at a time: lane t reads entry j0 + t's slot, a ballot gives the run's
  // length; each entry's values are requested while the previous entry is quantised
  auto run = [&](auto& code, auto kk_tag, auto fetch) {
    constexpr int kK = decltype(kk_tag)::value;
    float sc = *scale_slot;  // the block's scale so far
    for (int j0 = i;;) {
      const bool in_batch = lane < kBlockSize && j0 + lane < B;
      const int64_t my_slot = in_batch ? slots[j0 + lane] : -1;
      const uint64_t same = __ballot(in_batch && block_of(my_slot) == blk);
      const int n = __builtin_ctzll(~same);  // leading entries in the block (at most 16)
      const int my_off = static_cast<int>(my_slot % kBlockSize);
      float x[kK];
      fetch(j0, x);  // n >= 1: entry j0 is in the block
      for (int t = 0; t < n; ++t) {
        float nx[kK];
        if (t + 1 < n) fetch(j0 + t + 1, nx);
        quantise_row<kQMax, kK>(code, x, &sc, __builtin_amdgcn_readlane(my_off, t));
        if (t + 1 < n) {
#pragma unroll
          for (int k = 0; k < kK; ++k) x[k] = nx[k];
        }
      }
      if (n < kBlockSize) break;  // the run ended inside this group of 16
      j0 += kBlockSize;           // 16 entries all in the block (repeated slots): go on
    }
    if (lane == 0) *scale_slot = sc;
  };

  if (!is_v) {
    uint8_t* kt = k_cache + tile * kBlockSize * kRowK;
    int kc[kBlockSize][kKE] = {};
#pragma unroll
    for (int row = 0; row < kBlockSize; ++row) {
      if constexpr (kI4) {
        if (kmine) {
          const uint8_t byte = kt[row * kRowK + lane];
          kc[row][0] = static_cast<int>(byte & 0xf) - 8;
          kc[row][1] = static_cast<int>(byte >> 4) - 8;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kJ; ++j)
          kc[row][j] =
              static_cast<int>(reinterpret_cast<const int8_t*>(kt)[row * kRowK + lane + 64 * j]);
      }
    }
    run(kc, std::integral_constant<int, kKE>{}, [&](int j, float (&x)[kKE]) {
      const TIn* src = x_new + (static_cast<int64_t>(j) * Hkv + g) * D;
      if constexpr (kI4) {
        x[0] = kmine ? widen<TIn>(src[e_lo]) : 0.f;
        x[1] = kmine ? widen<TIn>(src[e_lo + 4]) : 0.f;
      } else {
#pragma unroll
        for (int k = 0; k < kJ; ++k) x[k] = widen<TIn>(src[lane + 64 * k]);
      }
    });
#pragma unroll
    for (int row = 0; row < kBlockSize; ++row) {
      if constexpr (kI4) {
        if (kmine)
          kt[row * kRowK + lane] = static_cast<uint8_t>(((kc[row][0] + 8) & 0xf) |
                                                        (((kc[row][1] + 8) & 0xf) << 4));
      } else {
#pragma unroll
        for (int j = 0; j < kJ; ++j)
          reinterpret_cast<int8_t*>(kt)[row * kRowK + lane + 64 * j] =
              static_cast<int8_t>(kc[row][j]);
      }
    }
  } else {
    uint8_t* vt = v_cache + tile * D * kRowV;
    int vc[kBlockSize][kJ] = {};
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const uint8_t* vrow = vt + (lane + 64 * j) * kRowV;
#pragma unroll
      for (int t = 0; t < kBlockSize; ++t) {
        if constexpr (kI4) {
          vc[t][j] = static_cast<int>((vrow[nib_byte(t)] >> nib_shift(t)) & 0xf) - 8;
        } else {
          vc[t][j] = static_cast<int>(reinterpret_cast<const int8_t*>(vrow)[t]);
        }
      }
    }
    run(vc, std::integral_constant<int, kJ>{}, [&](int j, float (&x)[kJ]) {
      const TIn* src = x_new + (static_cast<int64_t>(j) * Hkv + g) * D;
#pragma unroll
      for (int k = 0; k < kJ; ++k) x[k] = widen<TIn>(src[lane + 64 * k]);
    });
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      uint8_t* vrow = vt + (lane + 64 * j) * kRowV;
      if constexpr (kI4) {
        uint8_t bytes[kRowV] = {};
#pragma unroll
        for (int t = 0; t < kBlockSize; ++t)
          bytes[nib_byte(t)] |= static_cast<uint8_t>(((vc[t][j] + 8) & 0xf) << nib_shift(t));
#pragma unroll
        for (int e = 0; e < kRowV; ++e) vrow[e] = bytes[e];
      } else {
#pragma unroll
        for (int t = 0; t < kBlockSize; ++t)
          reinterpret_cast<int8_t*>(vrow)[t] = static_cast<int8_t>(vc[t][j]);
      }
    }
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

template <int kQMax>
hipError_t launch_kv_append_quant(const void* k_new, const void* v_new, bool bf16_new,
                                  const int64_t* slots, uint8_t* k_cache, uint8_t* v_cache,
                                  float* k_scale, float* v_scale, int32_t B, int32_t Hkv,
                                  int32_t D, int32_t NB, hipStream_t stream) {
  if (B == 0) return hipSuccess;
  if (D != 64 && D != 128) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((B + kAppendWaves - 1) / kAppendWaves),
                  static_cast<unsigned>(Hkv), 2);
  auto go = [&](auto kernel, auto tin) {
    using T = decltype(tin);
    hipLaunchKernelGGL(kernel, grid, dim3(64 * kAppendWaves), 0, stream,
                       static_cast<const T*>(k_new), static_cast<const T*>(v_new), slots, k_cache,
                       v_cache, k_scale, v_scale, B, Hkv, NB);
  };
  if (bf16_new) {
    if (D == 128) go(kv_append_quant_kernel<uint16_t, 128, kQMax>, uint16_t{});
    else go(kv_append_quant_kernel<uint16_t, 64, kQMax>, uint16_t{});
  } else {
    if (D == 128) go(kv_append_quant_kernel<float, 128, kQMax>, float{});
    else go(kv_append_quant_kernel<float, 64, kQMax>, float{});
  }
  return hipGetLastError();
}

hipError_t launch_kv_append_i8(const void* k_new, const void* v_new, bool bf16_new,
                               const int64_t* slots, int8_t* k_cache, int8_t* v_cache,
                               float* k_scale, float* v_scale, int32_t B, int32_t Hkv, int32_t D,
                               int32_t NB, hipStream_t stream) {
  return launch_kv_append_quant<127>(k_new, v_new, bf16_new, slots,
                                     reinterpret_cast<uint8_t*>(k_cache),
                                     reinterpret_cast<uint8_t*>(v_cache), k_scale, v_scale, B,
                                     Hkv, D, NB, stream);
}

hipError_t launch_kv_append_i4(const void* k_new, const void* v_new, bool bf16_new,
                               const int64_t* slots, uint8_t* k_cache, uint8_t* v_cache,
                               float* k_scale, float* v_scale, int32_t B, int32_t Hkv, int32_t D,
                               int32_t NB, hipStream_t stream) {
  return launch_kv_append_quant<7>(k_new, v_new, bf16_new, slots, k_cache, v_cache, k_scale,
                                   v_scale, B, Hkv, D, NB, stream);
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
