// Chunked-prefill attention over the paged cache on the gfx950 matrix cores.
//
// What it computes ("How LLM Inference Serving Works", "Two Phases: Prefill and Decode": prefill
// runs the prompt's tokens in parallel, each depending on all earlier ones; "Prefix Caching and
// Chunked Prefill" / "Chunked prefill": a long prefill runs as a series of chunks).  Sequence b
// brings a chunk of n_b query tokens, the last n_b of its L_b cached tokens; query i sits at
// position p = L_b - n_b + i and attends to tokens 0..p of the sequence through its block table.
//
// Unlike decode this is a dense contraction with reuse: 16 queries share every K and V tile, so
// the path is bound by the matrix cores, not by HBM.  The layout mirrors the decode kernel with
// the 16 columns of each MFMA tile holding 16 *queries* of one head instead of the replicated
// heads of a group:
//   scores  S^T = K . Q^T: two 16(token) x 16(query) tiles per block pair (32 tokens); with the
//           decode kernel's token order, lane l ends up with the 8 scores of tokens
//           8*(l/16)..+7 for query l%16 -- exactly its P operand for P . V;
//   P . V   O^T += V^T . P^T as 16(dim) x 16(query) tiles, V tiles dim-major in HBM, so a
//           lane's accumulator column is its own query;
// online softmax per query (exp2 domain) with a lazily moved maximum, the causal limit p applied
// per lane on the pairs that reach it.
// A wave takes 16 queries of up to four query heads of one KV head: each K/V operand it loads
// feeds the MFMAs of all its heads.  A workgroup holds four such waves on consecutive 16-query
// tiles of one sequence, which read the same K/V tiles back to back and share them in cache.
#include <cmath>

#include "internal.h"
#include "pagedkv.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;              // queries per wave
constexpr int kPairTok = 2 * kBlockSize;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Reductions over the four 16-lane groups (lanes r, r + 16, r + 32, r + 48) with the gfx950
// row and half swaps.
__device__ __forceinline__ float max_across_groups(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_groups(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr float kLazyLog2 = 8.f;  // slack of the running maximum, in log2 units

template <int D>
struct KVRegs {
  u32x4 k1[D / 32];
  u32x4 k2[D / 32];
  u32x4 v[D / 16];
  int32_t blk_a, blk_b;
};

// Sequence and group of global group index `group`: groups of kGroup queries are numbered
// sequence by sequence, ceil(n_b / kGroup) per sequence.  Every lane of the wave returns the
// same answer; b = -1 when the index is past the last group.
template <int kGroup>
__device__ void locate_group(const int32_t* __restrict__ cu_q, int B, int group, int* b_out,
                             int* j_out) {
  const int lane = threadIdx.x % 64;
  int base = 0;  // groups before the current chunk of 64 sequences
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int n = b < B ? max(cu_q[b + 1] - cu_q[b], 0) : 0;
    const int t = (n + kGroup - 1) / kGroup;
    int incl = t;  // inclusive prefix over the chunk
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    const int excl = incl - t;
    const bool mine = b < B && group >= base + excl && group < base + incl;
    const unsigned long long hit = __ballot(mine);
    if (hit) {
      const int src = __ffsll(static_cast<long long>(hit)) - 1;
      *b_out = b0 + src;
      *j_out = group - base - __shfl(excl, src, 64);
      return;
    }
    base += __shfl(incl, 63, 64);
  }
  *b_out = -1;
  *j_out = 0;
}

// Query heads per wave: the group's heads, at most 4 (larger groups span blockIdx.z).  Every
// K/V operand a wave loads feeds the MFMAs of all its heads.
template <int G>
constexpr int kHeadsPerWave = G < 4 ? G : 4;
constexpr int kWavesPerWG = 4;                       // consecutive 16-query tiles
constexpr int kGroupQueries = kTile * kWavesPerWG;   // queries per workgroup

template <int G, int D>
__global__ void __launch_bounds__(64 * kWavesPerWG) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_mfma_kernel(PrefillArgs a) {
  constexpr int kSteps = D / 32;
  constexpr int kTiles = D / 16;
  constexpr int kH = kHeadsPerWave<G>;
  const int lane = threadIdx.x % 64;
  const int w = threadIdx.x / 64;
  const int r = lane % 16, qg = lane / 16;
  const int g = blockIdx.y;
  const int h0 = g * G + blockIdx.z * kH;  // this wave's first query head

  int b, jg;
  locate_group<kGroupQueries>(a.cu_q, a.B, blockIdx.x, &b, &jg);
  if (b < 0) return;
  const int row0 = a.cu_q[b];
  const int n = a.cu_q[b + 1] - row0;
  const int qi0 = jg * kGroupQueries + w * kTile;
  if (qi0 >= n) return;                           // no barrier follows: idle waves just leave
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int q_last = min(qi0 + kTile, n) - 1;    // last query of the tile
  const int p_max = L - n + q_last;               // its position: the tile's causal reach
  const int kv_end = min(L, p_max + 1);
  // this lane's query (column r) and its causal limit
  const int my_q = qi0 + r;
  const int my_p = L - n + my_q;
  const int32_t* __restrict__ table = a.tables + static_cast<int64_t>(b) * a.max_blocks;
  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(a.v);
  const int NB = a.NB, Hkv = a.Hkv;

  // Scores enter the exponent as fma(s, c, -m) with c = |scale log2 e| > 0; a negative scale
  // flips the sign of q instead (exact in bf16), and c = 0 is raised to the least normal float,
  // which leaves every score's product with it a zero of the exponent's rounding.
  const float c = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
  const uint32_t q_sign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  // Q^T operands: query column r of head h0 + hh, dims 32 s + 8 qg .. +8 (row clamped)
  u32x4 qv[kH][kSteps];
  {
    const int qrow = min(max(row0 + min(my_q, n - 1), 0), a.T - 1);
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) {
      const uint16_t* q = static_cast<const uint16_t*>(a.q) +
                          (static_cast<int64_t>(qrow) * a.Hq + h0 + hh) * D;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) qv[hh][s] = ld16(q + 32 * s + 8 * qg) ^ q_sign;
    }
  }

  const int tok1 = (r / 8) * 16 + ((r / 4) % 2) * 8 + (r % 4);
  const int tok2 = tok1 + 4;
  const int vsel = qg / 2, vtok = 8 * (qg % 2);

  auto load_pair = [&](int i, KVRegs<D>& R) {
    const int tok0 = i * kPairTok;
    const int jb = tok0 / kBlockSize;
    int32_t ba = table[jb];
    int32_t bb = (tok0 + kBlockSize < kv_end) ? table[jb + 1] : -1;
    ba = (ba >= 0 && ba < NB) ? ba : -1;
    bb = (bb >= 0 && bb < NB) ? bb : -1;
    R.blk_a = ba;
    R.blk_b = bb;
    const int64_t ta = (static_cast<int64_t>(ba < 0 ? 0 : ba) * Hkv + g) * (kBlockSize * D);
    const int64_t tb = (static_cast<int64_t>(bb < 0 ? 0 : bb) * Hkv + g) * (kBlockSize * D);
    const uint16_t* k1 = kc + (tok1 < 16 ? ta : tb) + (tok1 % 16) * D + 8 * qg;
    const uint16_t* k2 = kc + (tok2 < 16 ? ta : tb) + (tok2 % 16) * D + 8 * qg;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      R.k1[s] = ld16(k1 + 32 * s);
      R.k2[s] = ld16(k2 + 32 * s);
    }
    const uint16_t* v = vc + (vsel ? tb : ta) + r * kBlockSize + vtok;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) R.v[t] = ld16(v + 16 * t * kBlockSize);
  };

  float m_run[kH], l_run[kH];
  f32x4 acc[kH][kTiles];
#pragma unroll
  for (int hh = 0; hh < kH; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.f;
#pragma unroll
    for (int t = 0; t < kTiles; ++t) acc[hh][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int p_first = L - n + qi0;  // position of the tile's first query
  auto compute_pair = [&](int i, KVRegs<D>& R) {
    const int tok0 = i * kPairTok;
    const int t_first = tok0 + 8 * qg;
    const int32_t my_blk = vsel ? R.blk_b : R.blk_a;
    // Only pairs that reach past the tile's first query, past the context or into a missing
    // block need masks (wave-uniform test).
    const bool edge =
        tok0 + kPairTok - 1 > p_first || tok0 + kPairTok > L || R.blk_a < 0 || R.blk_b < 0;
    // causal and context limits: token t is kept for this lane's query when t <= my_p, t < L
    const int limit = min(my_p, L - 1);
    if (tok0 + kPairTok > L || R.blk_a < 0 || R.blk_b < 0) {
      // tokens past the context (or of a missing block) must not reach P.V even with p = 0
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const bool k0 = my_blk >= 0 && t_first + 2 * cc < L;
        const bool k1 = my_blk >= 0 && t_first + 2 * cc + 1 < L;
        const uint32_t keep = (k0 ? 0x0000ffffu : 0u) | (k1 ? 0xffff0000u : 0u);
#pragma unroll
        for (int t = 0; t < kTiles; ++t) R.v[t][cc] &= keep;
      }
    }
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) {
      f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k1[s]), as_bf16x8(qv[hh][s]), s1,
                                                      0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k2[s]), as_bf16x8(qv[hh][s]), s2,
                                                      0, 0, 0);
      }
      float sr[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sr[e] = s1[e];
        sr[4 + e] = s2[e];
      }
      if (edge) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (t_first + e > limit || my_blk < 0) sr[e] = -INFINITY;
      }
      float bmax = sr[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) bmax = fmaxf(bmax, sr[e]);
      bmax = max_across_groups(bmax);
      const float bm = bmax * c;  // the pair's largest scaled score of this lane's query
      // Lazy rescaling: the running maximum moves only when a score exceeds it by more than
      // kLazyLog2, so P stays below 2^kLazyLog2 and most pairs skip the accumulator rescale.
      const bool grow = bm > m_run[hh] + kLazyLog2;
      if (__ballot(grow)) {
        const float m_new = grow ? bm : m_run[hh];
        const float alpha = __builtin_amdgcn_exp2f(m_run[hh] - m_new);
        m_run[hh] = m_new;
        l_run[hh] *= alpha;
#pragma unroll
        for (int t = 0; t < kTiles; ++t) acc[hh][t] *= alpha;
      }
      const float m_use = m_run[hh] == -INFINITY ? 0.f : m_run[hh];
      f32x8 pv;
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = __builtin_amdgcn_exp2f(fmaf(sr[e], c, -m_use));
        psum += pv[e];
      }
      l_run[hh] += psum;
      // O^T += V^T . P^T: V rows are dims, P^T columns are this lane's query, so the
      // accumulator column of a lane is its own query and the rescale above needs no shuffle.
      // P enters as a bf16 pair hi + lo, which carries it to about 16 bits.
      const bf16x8 p_hi = __builtin_convertvector(pv, bf16x8);
      const u32x4 hb = __builtin_bit_cast(u32x4, p_hi);
      f32x8 rest;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        rest[2 * cc] = pv[2 * cc] - __uint_as_float(hb[cc] << 16);
        rest[2 * cc + 1] = pv[2 * cc + 1] - __uint_as_float(hb[cc] & 0xffff0000u);
      }
      const bf16x8 p_lo = __builtin_convertvector(rest, bf16x8);
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        acc[hh][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.v[t]), p_hi, acc[hh][t],
                                                              0, 0, 0);
        acc[hh][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.v[t]), p_lo, acc[hh][t],
                                                              0, 0, 0);
      }
    }
  };

  const int n_pairs = kv_end > 0 ? (kv_end + kPairTok - 1) / kPairTok : 0;
  {
    KVRegs<D> ra, rb;
    int i = 0;
    if (i < n_pairs) load_pair(i, ra);
    while (i < n_pairs) {
      if (i + 1 < n_pairs) load_pair(i + 1, rb);
      compute_pair(i, ra);
      if (++i >= n_pairs) break;
      if (i + 1 < n_pairs) load_pair(i + 1, ra);
      compute_pair(i, rb);
      ++i;
    }
  }

  // l summed over the four lane groups is query r's; a lane holds dims 16 t + 4 qg .. +3 of it
  const int out_row = row0 + my_q;
  const bool store = my_q < n && out_row < a.T && out_row >= 0;
#pragma unroll
  for (int hh = 0; hh < kH; ++hh) {
    const float lq = sum_across_groups(l_run[hh]);
    if (store) {
      float* o = a.out + (static_cast<int64_t>(out_row) * a.Hq + h0 + hh) * D + 4 * qg;
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const f32x4 y = lq > 0.f ? acc[hh][t] / lq : f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(o + 16 * t) = y;
      }
    }
  }
}

template <int G, int D>
hipError_t launch_gd(const PrefillArgs& a, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.max_tiles), static_cast<unsigned>(a.Hkv),
                  static_cast<unsigned>(G / kHeadsPerWave<G>));
  hipLaunchKernelGGL((prefill_mfma_kernel<G, D>), grid, dim3(64 * kWavesPerWG), 0, stream, a);
  return hipGetLastError();
}

template <int G>
hipError_t launch_g(const PrefillArgs& a, hipStream_t stream) {
  if (a.D == 128) return launch_gd<G, 128>(a, stream);
  if (a.D == 64) return launch_gd<G, 64>(a, stream);
  return hipErrorNotSupported;
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t stream) {
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
