// Portable decode-attention kernel: any query/KV dtype pair, any group size up to 16, D 64/128.
//
// What it computes ("How LLM Inference Serving Works", "What the KV Cache Is, and How Big It
// Gets": the new token's query is scored against every cached key and the values are mixed by
// those weights; "PagedAttention: Virtual Memory for the KV Cache": K and V are gathered through
// the block table; grouped-query attention: query head h reads KV head h / G).
//
// Layout of the work: one workgroup per (partition, KV head, sequence).  It walks its
// partition in chunks of 256 tokens: one thread scores one token for all G heads of the group,
// a wave per head folds the chunk into the running max / sum (online softmax, exp2 domain), and
// one thread per (head, dim) accumulates the P.V column.  It is the path for the fp32 cache and
// fp32 queries, where the matrix-core kernels do not apply; it is built for short latency
// chains rather than bandwidth: a thread requests its whole K row, and its V column a block of
// 16 tokens at a time, as 16-byte pieces before it uses the first of them.
#include <cfloat>

#include "internal.h"
#include "pagedkv.h"

namespace pa {
namespace {

constexpr int kChunk = 256;
constexpr int kGMax = 16;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element loaders: get reads element i; unpack takes element e of a 16-byte piece (kE elements)
struct F32 {
  using T = float;
  static constexpr int kE = 4;
  static __device__ __forceinline__ float get(const T* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ float unpack(u32x4 x, int e) { return __uint_as_float(x[e]); }
};
struct BF16 {
  using T = uint16_t;
  static constexpr int kE = 8;
  static __device__ __forceinline__ float get(const T* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
  }
  static __device__ __forceinline__ float unpack(u32x4 x, int e) {
    return __uint_as_float(e % 2 ? x[e / 2] & 0xffff0000u : x[e / 2] << 16);
  }
};
struct I8 {
  using T = int8_t;
  static constexpr int kE = 16;
  static __device__ __forceinline__ float get(const T* p, int64_t i) {
    return static_cast<float>(p[i]);
  }
  static __device__ __forceinline__ float unpack(u32x4 x, int e) {
    return static_cast<float>(static_cast<int8_t>((x[e / 4] >> (8 * (e % 4))) & 0xffu));
  }
};

template <typename T>
__device__ __forceinline__ u32x4 piece(const T* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename QL, typename KL, int D>
__global__ void __launch_bounds__(256) decode_generic_kernel(DecodeArgs a, int G) {
  using QT = typename QL::T;
  using KT = typename KL::T;
  constexpr bool kQuant = sizeof(KT) == 1;
  constexpr int kPairs = (kGMax * D + 255) / 256;

  __shared__ float q_s[kGMax][D];
  __shared__ float s_s[kGMax][kChunk];
  __shared__ int32_t blk_s[kChunk / kBlockSize];
  __shared__ float ks_s[kChunk / kBlockSize];
  __shared__ float vs_s[kChunk / kBlockSize];
  __shared__ float m_s[kGMax], l_s[kGMax], alpha_s[kGMax];

  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int nparts = max(1, (L + a.partition - 1) / a.partition);
  if (p >= nparts) return;
  const int start = p * a.partition;
  const int end = min(start + a.partition, L);

  const QT* q = static_cast<const QT*>(a.q);
  const KT* kc = static_cast<const KT*>(a.k);
  const KT* vc = static_cast<const KT*>(a.v);
  const int64_t qbase = (static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G) * D;
  for (int i = tid; i < G * D; i += 256) q_s[i / D][i % D] = QL::get(q, qbase + i);
  if (tid < G) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  float acc[kPairs];
#pragma unroll
  for (int k = 0; k < kPairs; ++k) acc[k] = 0.f;
  __syncthreads();

  const int32_t* table = a.tables + static_cast<int64_t>(b) * a.max_blocks;
  for (int c0 = start; c0 < end; c0 += kChunk) {
    const int n = min(kChunk, end - c0);
    if (tid < kChunk / kBlockSize) {
      int32_t blk = -1;
      if (c0 + tid * kBlockSize < end) {
        blk = table[c0 / kBlockSize + tid];
        if (blk < 0 || blk >= a.NB) blk = -1;
      }
      blk_s[tid] = blk;
      if (kQuant) {
        const int64_t si = static_cast<int64_t>(max(blk, 0)) * a.Hkv + g;
        ks_s[tid] = blk >= 0 ? a.k_scale[si] : 0.f;
        vs_s[tid] = blk >= 0 ? a.v_scale[si] : 0.f;
      }
    }
    __syncthreads();

    // scores: thread t <-> token c0 + t, its K row requested whole
    {
      constexpr int kE = KL::kE;
      const int t = tid;
      const int32_t blk = t < n ? blk_s[t / kBlockSize] : -1;
      if (blk >= 0) {
        const KT* krow = kc + ((static_cast<int64_t>(blk) * a.Hkv + g) * kBlockSize +
                               t % kBlockSize) * D;
        u32x4 kp[D / kE];
#pragma unroll
        for (int c = 0; c < D / kE; ++c) kp[c] = piece(krow + c * kE);
        const float f = a.scale_log2 * (kQuant ? ks_s[t / kBlockSize] : 1.f);
        for (int h = 0; h < G; ++h) {
          float dot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int d = 0; d < D; ++d)
            dot[d % 4] = fmaf(q_s[h][d], KL::unpack(kp[d / kE], d % kE), dot[d % 4]);
          s_s[h][t] = ((dot[0] + dot[1]) + (dot[2] + dot[3])) * f;
        }
      } else {
        for (int h = 0; h < G; ++h) s_s[h][t] = -INFINITY;
      }
    }
    __syncthreads();

    // online softmax over the chunk, one wave per head
    {
      const int wave = tid / 64, lane = tid % 64;
      for (int h = wave; h < G; h += 4) {
        float mx = -INFINITY;
        for (int k = 0; k < kChunk / 64; ++k) mx = fmaxf(mx, s_s[h][lane + 64 * k]);
        mx = wave_max(mx);
        const float m_old = m_s[h];
        const float m_new = fmaxf(m_old, mx);
        float sum = 0.f;
        for (int k = 0; k < kChunk / 64; ++k) {
          const float s = s_s[h][lane + 64 * k];
          const float pv = (s == -INFINITY) ? 0.f : exp2f(s - m_new);
          s_s[h][lane + 64 * k] = pv;
          sum += pv;
        }
        sum = wave_sum(sum);
        if (lane == 0) {
          const float alpha = (m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new);
          alpha_s[h] = alpha;
          l_s[h] = l_s[h] * alpha + sum;
          m_s[h] = m_new;
        }
      }
    }
    __syncthreads();

    // P.V: thread <-> (head, dim) pairs; the 16 tokens of dim d in a block are contiguous in
    // the dim-major V tile, one to four 16-byte pieces
#pragma unroll
    for (int k = 0; k < kPairs; ++k) {
      const int idx = tid + 256 * k;
      if (idx < G * D) {
        constexpr int kE = KL::kE;
        const int h = idx / D, d = idx % D;
        float sum[2] = {0.f, 0.f};
        const int nb = (n + kBlockSize - 1) / kBlockSize;
#pragma unroll 2
        for (int j = 0; j < nb; ++j) {
          const int32_t blk = blk_s[j];
          if (blk < 0) continue;  // its P are 0 and its V is not read
          const KT* vcol = vc + ((static_cast<int64_t>(blk) * a.Hkv + g) * D + d) * kBlockSize;
          u32x4 vp[kBlockSize / kE];
#pragma unroll
          for (int c = 0; c < kBlockSize / kE; ++c) vp[c] = piece(vcol + c * kE);
          const float vsc = kQuant ? vs_s[j] : 1.f;
          const int lim = n - j * kBlockSize;  // tokens of the block inside the chunk
#pragma unroll
          for (int e = 0; e < kBlockSize; ++e) {
            // tokens past the chunk's end may hold anything, also NaN: skipped, not weighted
            if (e < lim)
              sum[e % 2] = fmaf(s_s[h][j * kBlockSize + e], KL::unpack(vp[e / kE], e % kE) * vsc,
                                sum[e % 2]);
          }
        }
        acc[k] = acc[k] * alpha_s[h] + (sum[0] + sum[1]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int k = 0; k < kPairs; ++k) {
    const int idx = tid + 256 * k;
    if (idx < G * D) {
      const int h = idx / D, d = idx % D;
      const float l = l_s[h];
      const float o = l > 0.f ? acc[k] / l : 0.f;
      const int64_t row = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + h;
      if (nparts == 1) {
        a.out[row * D + d] = o;
      } else {
        const int64_t slot = row * a.np_max + p;
        a.ws_o[slot * D + d] = o;
        if (d == 0) {
          a.ws_m[slot] = m_s[h];
          a.ws_l[slot] = l;
        }
      }
    }
  }
}

// Merge the partitions of each (sequence, query head): M = max m_p, w_p = l_p 2^(m_p - M),
// out = sum w_p o_p / sum w_p.  Sequences with one partition were written directly.
__global__ void __launch_bounds__(128) splitk_reduce_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int nparts = max(1, (L + a.partition - 1) / a.partition);
  if (nparts == 1 || d >= a.D) return;
  const int64_t row = static_cast<int64_t>(b) * a.Hq + h;
  const int64_t base = row * a.np_max;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.ws_m[base + p]);
  float num = 0.f, den = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float w = a.ws_l[base + p] * exp2f(a.ws_m[base + p] - M);
    den += w;
    num = fmaf(w, a.ws_o[(base + p) * a.D + d], num);
  }
  a.out[row * a.D + d] = den > 0.f ? num / den : 0.f;
}

template <typename QL, typename KL>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.np_max, a.Hkv, a.B);
  const int G = a.Hq / a.Hkv;
  if (a.D == 64)
    hipLaunchKernelGGL((decode_generic_kernel<QL, KL, 64>), grid, dim3(256), 0, stream, a, G);
  else if (a.D == 128)
    hipLaunchKernelGGL((decode_generic_kernel<QL, KL, 128>), grid, dim3(256), 0, stream, a, G);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_generic(const DecodeArgs& a, int q_dtype, int kv_dtype,
                                 hipStream_t stream) {
  if (a.Hq / a.Hkv > kGMax) return hipErrorNotSupported;
  if (q_dtype == PA_F32) {
    if (kv_dtype == PA_F32) return launch_typed<F32, F32>(a, stream);
    if (kv_dtype == PA_BF16) return launch_typed<F32, BF16>(a, stream);
    if (kv_dtype == PA_I8) return launch_typed<F32, I8>(a, stream);
  } else if (q_dtype == PA_BF16) {
    if (kv_dtype == PA_F32) return launch_typed<BF16, F32>(a, stream);
    if (kv_dtype == PA_BF16) return launch_typed<BF16, BF16>(a, stream);
    if (kv_dtype == PA_I8) return launch_typed<BF16, I8>(a, stream);
  }
  return hipErrorNotSupported;
}

hipError_t launch_splitk_reduce(const DecodeArgs& a, hipStream_t stream) {
  if (a.np_max <= 1) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(a.Hq, a.B), dim3(128), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
