// bf16 paged decode attention on the gfx950 matrix cores.
//
// What it computes ("How LLM Inference Serving Works", "What the KV Cache Is, and How Big It
// Gets": the new token's query is scored against every cached key and the values are mixed by
// the softmax weights; "PagedAttention: Virtual Memory for the KV Cache": the kernel follows the
// block table to gather K and V; grouped-query attention: query heads h of one group share KV
// head h / G).
//
// Decode reads every cached byte once and does 4 flops per byte, so it is bound by HBM.  The
// design goal is to keep enough 16-byte loads in flight and to spend as few issue slots as
// possible on everything else; the two small contractions run on MFMA so the vector ALUs only do
// the softmax.
//
// Work split.  One workgroup = 4 waves = one (partition, KV head, sequence).  A partition is a
// run of whole blocks; the waves take its block *pairs* (32 tokens) in turn and keep private
// softmax state; the workgroup merges the 4 states in LDS at the end.  Long sequences span
// several partitions whose normalised outputs are merged by splitk_reduce_kernel.
//
// One pair (blocks A, B of one KV head) per wave iteration, v_mfma_f32_16x16x32_bf16 throughout:
//   scores  S = K . q^T as two 16(token) x 16(head) tiles, K tiles token-major in HBM (each lane
//           loads 16 contiguous bytes of one token row), q^T columns replicated 16/G times;
//   P.V     O += P . V as 16(head) x 16(dim) tiles over the pair's 32 tokens, V tiles dim-major in
//           HBM (each lane loads 8 consecutive tokens of one dim: 16 contiguous bytes).
// The token order of the two score tiles is chosen so that lane l ends up holding the scores of
// exactly the 8 tokens it must supply as its P operand (tokens 8*(l/16)..+7 of the pair for head
// (l%16)%G): softmax and P.V need no cross-lane transposition.  P is fed as a bf16 hi/lo pair
// (p = hi + lo to ~16 bits) so the rounding of P stays far below the bf16 tolerance.
#include <cmath>

#include "internal.h"
#include "pagedkv.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kPair = 2 * kBlockSize;  // tokens per wave iteration

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <int D>
struct PairRegs {
  static constexpr int kSteps = D / 32;  // k-steps of the score MFMAs
  static constexpr int kTiles = D / 16;  // output dim tiles of P.V
  u32x4 k1[kSteps];   // score tile 1 rows (tokens A0-3, A8-11, B0-3, B8-11)
  u32x4 k2[kSteps];   // score tile 2 rows (tokens A4-7, A12-15, B4-7, B12-15)
  u32x4 v[kTiles];    // 8 tokens x 1 dim per tile
  int32_t blk_a, blk_b;  // physical blocks, -1 when masked
};

template <int G, int D>
__global__ void __launch_bounds__(64 * kWaves) decode_mfma_kernel(DecodeArgs a) {
  using Regs = PairRegs<D>;
  constexpr int kSteps = Regs::kSteps;
  constexpr int kTiles = Regs::kTiles;

  __shared__ float m_s[kWaves][G];
  __shared__ float l_s[kWaves][G];
  __shared__ float o_s[kWaves][G][D];

  const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int nparts = max(1, (L + a.partition - 1) / a.partition);
  if (p >= nparts) return;
  const int start = p * a.partition;
  const int end = min(start + a.partition, L);
  const int n_pairs = (end - start + kPair - 1) / kPair;

  const int lane = threadIdx.x % 64;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int r = lane % 16;   // row / column index inside an MFMA tile
  const int qg = lane / 16;  // k-group of the lane

  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(a.v);
  const int32_t* __restrict__ table = a.tables + static_cast<int64_t>(b) * a.max_blocks;
  const int NB = a.NB, Hkv = a.Hkv;

  // q^T operand: lane holds q[head (r % G)][dims 32 s + 8 qg .. +8] for each k-step s
  u32x4 qv[kSteps];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) +
                        (static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + r % G) * D;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qv[s] = load16(q + 32 * s + 8 * qg);
  }

  // token rows of the two score tiles, relative to the pair start
  const int tok1 = (r / 8) * 16 + ((r / 4) % 2) * 8 + (r % 4);
  const int tok2 = tok1 + 4;
  const int vblk_sel = qg / 2;         // which block of the pair this lane's P.V tokens are in
  const int vtok = 8 * (qg % 2);       // first of its 8 tokens inside that block

  auto load_pair = [&](int i, Regs& R) {
    const int tok0 = start + i * kPair;
    const int j = tok0 / kBlockSize;
    int32_t ba = table[j];
    int32_t bb = (tok0 + kBlockSize < end) ? table[j + 1] : -1;
    ba = (ba >= 0 && ba < NB) ? ba : -1;
    bb = (bb >= 0 && bb < NB) ? bb : -1;
    R.blk_a = ba;
    R.blk_b = bb;
    const int64_t tile_a = (static_cast<int64_t>(ba < 0 ? 0 : ba) * Hkv + g) * (kBlockSize * D);
    const int64_t tile_b = (static_cast<int64_t>(bb < 0 ? 0 : bb) * Hkv + g) * (kBlockSize * D);
    const uint16_t* k1 = kc + (tok1 < 16 ? tile_a : tile_b) + (tok1 % 16) * D + 8 * qg;
    const uint16_t* k2 = kc + (tok2 < 16 ? tile_a : tile_b) + (tok2 % 16) * D + 8 * qg;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      R.k1[s] = load16(k1 + 32 * s);
      R.k2[s] = load16(k2 + 32 * s);
    }
    const uint16_t* v = vc + (vblk_sel ? tile_b : tile_a) + r * kBlockSize + vtok;
#pragma unroll
    for (int n = 0; n < kTiles; ++n) R.v[n] = load16(v + 16 * n * kBlockSize);
  };

  float m_run = -INFINITY;  // running max (log2 domain) of head r % G
  float l_run = 0.f;        // lane-partial running sum over this lane's tokens
  f32x4 acc[kTiles];
#pragma unroll
  for (int n = 0; n < kTiles; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute_pair = [&](int i, Regs& R) {
    const int tok0 = start + i * kPair;
    // scores
    f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k1[s]), as_bf16x8(qv[s]), s1, 0, 0, 0);
      s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k2[s]), as_bf16x8(qv[s]), s2, 0, 0, 0);
    }
    // this lane's 8 tokens: pair tokens 8 qg + e, e = 0..7
    const int t_first = tok0 + 8 * qg;
    const int32_t my_blk = vblk_sel ? R.blk_b : R.blk_a;
    const bool tail = (tok0 + kPair > end) || R.blk_b < 0 || R.blk_a < 0;
    float sc[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc[e] = s1[e] * a.scale_log2;
      sc[4 + e] = s2[e] * a.scale_log2;
    }
    if (tail) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (t_first + e >= end || my_blk < 0) sc[e] = -INFINITY;
      // masked tokens must not reach P.V even with p = 0 (their V may be anything)
      uint32_t keep[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool k0 = my_blk >= 0 && t_first + 2 * c < end;
        const bool k1 = my_blk >= 0 && t_first + 2 * c + 1 < end;
        keep[c] = (k0 ? 0x0000ffffu : 0u) | (k1 ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int n = 0; n < kTiles; ++n)
#pragma unroll
        for (int c = 0; c < 4; ++c) R.v[n][c] &= keep[c];
    }
    float bmax = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) bmax = fmaxf(bmax, sc[e]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float m_new = fmaxf(m_run, bmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    f32x8 pv;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
      psum += pv[e];
    }
    l_run = l_run * alpha + psum;
    // rescale the accumulators: rows 4 qg + j hold head (4 qg + j) % G
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float aj;
      if constexpr (G <= 4) {
        aj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), j % G));
      } else {
        aj = __shfl(alpha, (4 * qg + j) % G, 64);
      }
#pragma unroll
      for (int n = 0; n < kTiles; ++n) acc[n][j] *= aj;
    }
    // P as bf16 hi + lo
    const bf16x8 p_hi = __builtin_convertvector(pv, bf16x8);
    const u32x4 hi_bits = __builtin_bit_cast(u32x4, p_hi);
    f32x8 rest;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      rest[2 * c] = pv[2 * c] - __uint_as_float(hi_bits[c] << 16);
      rest[2 * c + 1] = pv[2 * c + 1] - __uint_as_float(hi_bits[c] & 0xffff0000u);
    }
    const bf16x8 p_lo = __builtin_convertvector(rest, bf16x8);
#pragma unroll
    for (int n = 0; n < kTiles; ++n) {
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_hi, as_bf16x8(R.v[n]), acc[n], 0, 0, 0);
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_lo, as_bf16x8(R.v[n]), acc[n], 0, 0, 0);
    }
  };

  // software pipeline: the next pair's loads are in flight while the current one is computed
  {
    Regs ra, rb;
    int i = w;
    if (i < n_pairs) load_pair(i, ra);
    while (i < n_pairs) {
      if (i + kWaves < n_pairs) load_pair(i + kWaves, rb);
      compute_pair(i, ra);
      i += kWaves;
      if (i >= n_pairs) break;
      if (i + kWaves < n_pairs) load_pair(i + kWaves, ra);
      compute_pair(i, rb);
      i += kWaves;
    }
  }

  // per-wave state -> LDS
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (qg == 0 && r < G) {
    m_s[w][r] = m_run;
    l_s[w][r] = l_tot;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = 4 * qg + j;
    if (h < G) {
#pragma unroll
      for (int n = 0; n < kTiles; ++n) o_s[w][h][16 * n + r] = acc[n][j];
    }
  }
  __syncthreads();

  // merge the waves and write
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * kWaves) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, m_s[v][h]);
    float num = 0.f, den = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float f = __builtin_amdgcn_exp2f(m_s[v][h] - M);
        num += f * o_s[v][h][d];
        den += f * l_s[v][h];
      }
    }
    const float o = den > 0.f ? num / den : 0.f;
    const int64_t row = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + h;
    if (nparts == 1) {
      a.out[row * D + d] = o;
    } else {
      const int64_t slot = row * a.np_max + p;
      a.ws_o[slot * D + d] = o;
      if (d == 0) {
        a.ws_m[slot] = M;
        a.ws_l[slot] = den;
      }
    }
  }
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.np_max, a.Hkv, a.B);
  if (a.D == 128)
    hipLaunchKernelGGL((decode_mfma_kernel<G, 128>), grid, dim3(64 * kWaves), 0, stream, a);
  else if (a.D == 64)
    hipLaunchKernelGGL((decode_mfma_kernel<G, 64>), grid, dim3(64 * kWaves), 0, stream, a);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 4: return launch_g<4>(a, stream);
    case 8: return launch_g<8>(a, stream);
    case 16: return launch_g<16>(a, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pa
