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
// softmax per query (exp2 domain) against a fixed reference, the causal limit p applied per lane
// on the pairs that reach it.
// A wave takes 16 queries of up to four query heads of one KV head: each K/V operand it loads
// feeds the MFMAs of all its heads.  A workgroup holds four such waves on consecutive 16-query
// tiles of one sequence, which read the same K/V tiles back to back and share them in cache.
#include <climits>
#include <cmath>

#include "device_load.h"
#include "internal.h"
#include "pagedkv.h"
#include "quant_f16.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

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

constexpr float kOverPQ = 16384.f;         // 2^14: a pair's fp16 P sum (times the V scale) above
                                           // this asks for a rerun against the exact maximum
constexpr float kUnderL = 8.6736174e-19f;  // 2^-60: a final l below this asks for a rerun

struct Pair {
  int32_t a, b;  // the blocks of tokens 0..15 and 16..31 of a 32-token pair
};

// Integer reduction over the wave (rows of 16 with DPP rotations and quad permutations, then
// the row swaps), returned as a wave-uniform value.
template <class Op>
__device__ __forceinline__ int wave_reduce(int v, Op op) {
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x128, 0xf, 0xf, false));  // row_ror:8
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x124, 0xf, 0xf, false));  // row_ror:4
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0x4e, 0xf, 0xf, false));   // quad_perm [2, 3, 0, 1]
  v = op(v, __builtin_amdgcn_mov_dpp(v, 0xb1, 0xf, 0xf, false));   // quad_perm [1, 0, 3, 2]
  auto h = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v),
                                            false, false);
  v = op(static_cast<int>(h[0]), static_cast<int>(h[1]));
  h = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false,
                                       false);
  v = op(static_cast<int>(h[0]), static_cast<int>(h[1]));
  return __builtin_amdgcn_readfirstlane(v);
}

// Work order.  A sequence with L cached tokens and an n-query chunk splits into ceil(n / kGroup)
// groups of kGroup queries; group j's last query reaches key L - n + min(kGroup (j + 1), n),
// and a workgroup's time grows with that reach.  Groups are handed out longest reach first
// (ties in sequence order), so the long workgroups start first and the short ones fill the
// compute units behind them instead of leaving a tail.  The reach grows strictly with j, so a
// sequence holds at most one group of any given reach.
struct SeqGroups {
  int n, J, base;  // chunk size, number of groups, L - n
};
template <int kGroup>
__device__ __forceinline__ SeqGroups seq_groups(const PrefillArgs& a, int b) {
  if (b >= a.B) return SeqGroups{0, 0, 0};
  const int n = min(max(a.cu_q[b + 1] - a.cu_q[b], 0), a.T);
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  return SeqGroups{n, (n + kGroup - 1) / kGroup, L - n};
}
// groups of the sequence whose reach is at least v
template <int kGroup>
__device__ __forceinline__ int groups_reaching(SeqGroups s, int v) {
  const int d = v - s.base;  // reach >= v  <=>  min(kGroup (j + 1), n) >= d
  if (s.J == 0 || d > s.n) return 0;
  return s.J - (d <= kGroup ? 0 : (d + kGroup - 1) / kGroup - 1);
}
// Sequence b and group j of the group ranked `rank` in that order, by bisection on the reach:
// the largest reach v with more than `rank` groups reaching v is the group's own; the groups
// reaching further come first, then those of reach v in sequence order.  Every lane returns
// the same answer; b = -1 past the last group.
template <int kGroup>
__device__ void group_of_rank(const PrefillArgs& a, int rank, int* b_out, int* j_out) {
  const int lane = threadIdx.x % 64;
  const SeqGroups s0 = seq_groups<kGroup>(a, lane);  // the first 64 sequences stay in registers
  auto chunk = [&](int b0) { return b0 == 0 ? s0 : seq_groups<kGroup>(a, b0 + lane); };
  auto add = [](int x, int y) { return x + y; };
  int n_groups = 0, lo = INT_MAX, hi = INT_MIN;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const SeqGroups s = chunk(b0);
    n_groups += s.J;
    if (s.J > 0) {
      lo = min(lo, s.base + min(kGroup, s.n));
      hi = max(hi, s.base + s.n);
    }
  }
  n_groups = wave_reduce(n_groups, add);
  *b_out = -1;
  *j_out = 0;
  if (rank >= n_groups) return;
  lo = wave_reduce(lo, [](int x, int y) { return min(x, y); });      // every group reaches lo
  hi = wave_reduce(hi, [](int x, int y) { return max(x, y); }) + 1;  // none reaches hi
  auto reaching = [&](int v) {
    int c = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) c += groups_reaching<kGroup>(chunk(b0), v);
    return wave_reduce(c, add);
  };
  int above = 0;  // groups reaching hi
  while (hi - lo > 1) {
    const int mid = lo + (hi - lo) / 2;
    const int c = reaching(mid);
    if (c > rank) {
      lo = mid;
    } else {
      hi = mid;
      above = c;
    }
  }
  int want = rank - above;  // among the groups of reach exactly lo, in sequence order
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const SeqGroups s = chunk(b0);
    const int ge = groups_reaching<kGroup>(s, lo);
    const bool has = ge > groups_reaching<kGroup>(s, lo + 1);
    const uint64_t m = __ballot(has);
    const int cnt = __popcll(m);
    if (want < cnt) {
      const int before = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(
                                                       static_cast<uint32_t>(m), 0u));
      const uint64_t pick = __ballot(has && before == want);
      const int src = __ffsll(static_cast<long long>(pick)) - 1;
      *b_out = b0 + src;
      *j_out = __shfl(s.J - ge, src, 64);
      return;
    }
    want -= cnt;
  }
}

// Query heads per wave: the group's heads, at most 4 (larger groups take several blocks of heads).  Every
// K/V operand a wave loads feeds the MFMAs of all its heads.
template <int G>
constexpr int kHeadsPerWave = G < 4 ? G : 4;
constexpr int kWavesPerWG = 4;                       // consecutive 16-query tiles
constexpr int kGroupQueries = kTile * kWavesPerWG;   // queries per workgroup

// Operand registers of one block pair for each cache kind.  bf16: K rows (two 16-token halves
// of the score tile) and V rows as 16-byte loads.  int8: 16 dims of a K row per load (two
// k-steps), 8 tokens of a V row per 8-byte load.  int4: the 4-byte groups of packed nibbles a
// lane feeds one k-step (K) or its 8 tokens of one dim (V).
template <int kKV, int D>
struct KOps;
template <int D>
struct KOps<kKvBf16, D> {
  u32x4 k1[D / 32], k2[D / 32];
  float ks_a, ks_b;
};
template <int D>
struct KOps<kKvI8, D> {
  u32x4 k1[D / 64], k2[D / 64];
  float ks_a, ks_b;
};
template <int D>
struct KOps<kKvI4, D> {
  uint32_t k1[D / 32], k2[D / 32];
  float ks_a, ks_b;
};
template <int kKV, int D>
struct VOps;
template <int D>
struct VOps<kKvBf16, D> {
  u32x4 v[D / 16];
  float vs_a, vs_b;
};
template <int D>
struct VOps<kKvI8, D> {
  u32x2 v[D / 16];
  float vs_a, vs_b;
};
template <int D>
struct VOps<kKvI4, D> {
  uint32_t v[D / 16];
  float vs_a, vs_b;
};

template <int G, int D, int kKV>
__global__ void __launch_bounds__(64 * kWavesPerWG) __attribute__((amdgpu_waves_per_eu(1, 1)))
prefill_mfma_kernel(PrefillArgs a) {
  constexpr int kSteps = D / 32;
  constexpr int kTiles = D / 16;
  constexpr int kH = kHeadsPerWave<G>;
  constexpr bool kQ = kKV != kKvBf16;  // quantised cache: fp16 matrix-core operands
  // code offset removed from the sums; int4 carries it inside its weighted sums (two offsets,
  // one per half of each 8-element operand group)
  constexpr float kOffset = kKV == kKvI4 ? 1.f : kCodeOffset;
  const int lane = threadIdx.x % 64;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int r = lane % 16, qg = lane / 16;
  // blockIdx.x = (rank of the query group) x (KV head, block of kH heads) with the KV heads
  // innermost: with 8 | Hkv, the workgroups of one KV head share an XCD and its L2
  const int per_group = a.Hkv * (G / kH);
  const int hz = blockIdx.x % per_group;
  const int g = hz % a.Hkv;
  const int h0 = g * G + (hz / a.Hkv) * kH;  // this wave's first query head

  int b, jg;
  group_of_rank<kGroupQueries>(a, blockIdx.x / per_group, &b, &jg);
  // wave-uniform from here on (the compiler cannot see it through the search): the block
  // table then is read through the scalar cache and the loop bounds stay scalar
  b = __builtin_amdgcn_readfirstlane(b);
  jg = __builtin_amdgcn_readfirstlane(jg);
  if (b < 0) return;
  const int row0 = __builtin_amdgcn_readfirstlane(a.cu_q[b]);
  const int n = __builtin_amdgcn_readfirstlane(a.cu_q[b + 1]) - row0;
  const int qi0 = jg * kGroupQueries + w * kTile;
  if (qi0 >= n) return;                           // no barrier follows: idle waves just leave
  const int L = __builtin_amdgcn_readfirstlane(min(max(a.seq_lens[b], 0), a.max_seq_len));
  const int q_last = min(qi0 + kTile, n) - 1;    // last query of the tile
  const int p_max = L - n + q_last;               // its position: the tile's causal reach
  const int kv_end = min(L, p_max + 1);
  // this lane's query (column r) and its causal limit
  const int my_q = qi0 + r;
  const int my_p = L - n + my_q;
  const int32_t* __restrict__ table = a.tables + static_cast<int64_t>(b) * a.max_blocks;
  const int NB = a.NB, Hkv = a.Hkv;

  // bf16: scores enter the exponent as fma(s, c, -m) with c = |scale log2 e| > 0; a negative
  // scale flips the sign of q instead (exact), and c = 0 is raised to the least normal float,
  // which leaves every score's product with it a zero of the exponent's rounding.  Quantised
  // caches fold c with the block's K scale into the score itself (cx = 1 below).
  const float c = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
  const float cx = kQ ? 1.f : c;
  const bool q_neg = a.scale_log2 < 0.f;
  // Q^T operands: query column r of head h0 + hh (row clamped).  bf16: step s covers dims
  // 32 s + 8 qg .. +8.  Quantised: fp16 (bf16 -> fp16 is exact in fp16's normal range); int8
  // step s covers dims 16 (qg + 4 (s / 2)) + 8 (s % 2) .. +8 (the 16-dim K loads), int4 step s
  // dims 8 kSteps qg + 8 s .. +8 (the packed 4-byte groups).  qsum: the sum of the rounded fp16
  // q over the head's dims, which takes the code offset out of the scores.
  u32x4 qv[kH][kSteps];
  float qsum[kH];
  {
    const int qrow = min(max(row0 + min(my_q, n - 1), 0), a.T - 1);
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) {
      const uint16_t* q = static_cast<const uint16_t*>(a.q) +
                          (static_cast<int64_t>(qrow) * a.Hq + h0 + hh) * D;
      float part = 0.f;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        if constexpr (kQ) {
          const u32x4 raw = kKV == kKvI4 ? ld16(q + 8 * kSteps * qg + 8 * s)
                                         : ld16(q + 16 * (qg + 4 * (s / 2)) + 8 * (s % 2));
          f32x8 f;
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            f[2 * cc] = __uint_as_float((raw[cc] << 16) ^ (q_neg ? 0x80000000u : 0u));
            f[2 * cc + 1] = __uint_as_float((raw[cc] & 0xffff0000u) ^ (q_neg ? 0x80000000u : 0u));
          }
          f16x8 h = __builtin_convertvector(f, f16x8);
          if constexpr (kKV == kKvI4) {
            // elements 4..7 meet codes expanded at 16 times their value
#pragma unroll
            for (int e = 4; e < 8; ++e) h[e] *= static_cast<_Float16>(0.0625f);
          }
          qv[hh][s] = __builtin_bit_cast(u32x4, h);
          const f32x8 back = __builtin_convertvector(h, f32x8);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            part += kKV == kKvI4 ? back[e] * (e < 4 ? kNibbleOffset : kNibbleOffsetHi16) : back[e];
        } else {
          qv[hh][s] = ld16(q + 32 * s + 8 * qg) ^ (q_neg ? 0x80008000u : 0u);
        }
      }
      qsum[hh] = kQ ? sum_across_groups(part) : 0.f;
    }
  }

  const int tok1 = (r / 8) * 16 + ((r / 4) % 2) * 8 + (r % 4);
  const int tok2 = tok1 + 4;
  const int vsel = qg / 2, vtok = 8 * (qg % 2);

  // Blocks of pair i (two consecutive table entries; -1 marks a missing or unused block).
  auto blocks_of = [&](int i) -> Pair {
    const int tok0 = __builtin_amdgcn_readfirstlane(i * kPairTok);
    const int jb = tok0 / kBlockSize;
    // entries past the row are never read (a table with no columns may be NULL)
    int32_t ba = jb < a.max_blocks ? uniform_load(table, jb) : -1;
    int32_t bb = (tok0 + kBlockSize < kv_end && jb + 1 < a.max_blocks) ? uniform_load(table, jb + 1) : -1;
    return Pair{(ba >= 0 && ba < NB) ? ba : -1, (bb >= 0 && bb < NB) ? bb : -1};
  };
  auto tile_idx = [&](int32_t blk) {  // (block, KV head) tile number
    return static_cast<int64_t>(blk < 0 ? 0 : blk) * Hkv + g;
  };
  KOps<kKV, D> ko;
  VOps<kKV, D> vo;
  auto load_k = [&](Pair bl) {
    const int64_t ia = tile_idx(bl.a), ib = tile_idx(bl.b);
    if constexpr (kKV == kKvBf16) {
      const uint16_t* kc = static_cast<const uint16_t*>(a.k);
      const uint16_t* p1 = kc + (tok1 < 16 ? ia : ib) * (kBlockSize * D) + (tok1 % 16) * D + 8 * qg;
      const uint16_t* p2 = kc + (tok2 < 16 ? ia : ib) * (kBlockSize * D) + (tok2 % 16) * D + 8 * qg;
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        ko.k1[s] = ld16(p1 + 32 * s);
        ko.k2[s] = ld16(p2 + 32 * s);
      }
    } else {
      // a missing block reads block 0's scale entry in its place; its scores are replaced by
      // -inf whatever that scale gives (mask_scores)
      ko.ks_a = uniform_load(a.k_scale, ia);
      ko.ks_b = uniform_load(a.k_scale, ib);
      const uint8_t* kc = static_cast<const uint8_t*>(a.k);
      if constexpr (kKV == kKvI8) {
        const uint8_t* p1 = kc + (tok1 < 16 ? ia : ib) * (kBlockSize * D) + (tok1 % 16) * D + 16 * qg;
        const uint8_t* p2 = kc + (tok2 < 16 ? ia : ib) * (kBlockSize * D) + (tok2 % 16) * D + 16 * qg;
#pragma unroll
        for (int cc = 0; cc < kSteps / 2; ++cc) {
          ko.k1[cc] = *reinterpret_cast<const u32x4*>(p1 + 64 * cc);
          ko.k2[cc] = *reinterpret_cast<const u32x4*>(p2 + 64 * cc);
        }
      } else {  // int4: tiles of bs * D / 2 bytes
        const uint8_t* p1 = kc + (tok1 < 16 ? ia : ib) * (kBlockSize * D / 2) +
                            (tok1 % 16) * (D / 2) + 4 * kSteps * qg;
        const uint8_t* p2 = kc + (tok2 < 16 ? ia : ib) * (kBlockSize * D / 2) +
                            (tok2 % 16) * (D / 2) + 4 * kSteps * qg;
#pragma unroll
        for (int cc = 0; cc < kSteps; ++cc) {
          ko.k1[cc] = *reinterpret_cast<const uint32_t*>(p1 + 4 * cc);
          ko.k2[cc] = *reinterpret_cast<const uint32_t*>(p2 + 4 * cc);
        }
      }
    }
  };
  auto load_v = [&](Pair bl) {
    const int64_t it = tile_idx(vsel ? bl.b : bl.a);
    if constexpr (kKV == kKvBf16) {
      const uint16_t* pv = static_cast<const uint16_t*>(a.v) + it * (kBlockSize * D) +
                           r * kBlockSize + vtok;
#pragma unroll
      for (int t = 0; t < kTiles; ++t) vo.v[t] = ld16(pv + 16 * t * kBlockSize);
    } else {
      // block 0's entry for a missing block; zeroed where it is used
      vo.vs_a = uniform_load(a.v_scale, tile_idx(bl.a));
      vo.vs_b = uniform_load(a.v_scale, tile_idx(bl.b));
      const uint8_t* vc = static_cast<const uint8_t*>(a.v);
      if constexpr (kKV == kKvI8) {
        const uint8_t* pv = vc + it * (kBlockSize * D) + r * kBlockSize + vtok;
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
          vo.v[t] = *reinterpret_cast<const u32x2*>(pv + 16 * t * kBlockSize);
      } else {
        const uint8_t* pv = vc + it * (kBlockSize * D / 2) + r * (kBlockSize / 2) + 4 * (qg % 2);
#pragma unroll
        for (int t = 0; t < kTiles; ++t)
          vo.v[t] = *reinterpret_cast<const uint32_t*>(pv + 16 * t * (kBlockSize / 2));
      }
    }
  };

  // Softmax against a fixed reference per query instead of a running maximum: P = 2^(s c - ref)
  // and the accumulators are never rescaled; the quotient acc / l is the same for any ref.  The
  // reference is the scaled maximum of the first pair (tokens 0..31), a score the sum contains,
  // so the largest P is at least 1 and nothing that matters underflows.  Should a later pair's
  // P sum leave range (past 2^61 for bf16; for quantised caches, P times the V scale past 2^14,
  // so that the fp16 P operand stays finite), or the final l stay below 2^-60 (the first pair
  // had no key for this query), the wave sweeps its keys once for the exact maximum and runs the
  // tile again with that as the reference, which no score can exceed.
  float ref[kH], l_run[kH], c_run[kH];
  f32x4 acc[kH][kTiles];
  const int p_first = L - n + qi0;     // position of the tile's first query
  const int limit = min(my_p, L - 1);  // keys t <= limit count for this lane's query
  const int n_pairs = kv_end > 0 ? (kv_end + kPairTok - 1) / kPairTok : 0;

  f32x4 s1[kH], s2[kH];
  // Scores of the pair in ko: bf16 leaves the raw products (scaled in the exponent); quantised
  // caches turn them into log2-domain scores, ks (sum q (offset + c) - offset qsum) |scale log2 e|,
  // with the K scale of the block this lane's tokens come from.
  auto scores = [&]() {
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) {
      s1[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
      s2[hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        if constexpr (kKV == kKvBf16) {
          s1[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ko.k1[s]),
                                                            as_bf16x8(qv[hh][s]), s1[hh], 0, 0, 0);
          s2[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ko.k2[s]),
                                                            as_bf16x8(qv[hh][s]), s2[hh], 0, 0, 0);
        } else {
          f16x8 a1, a2;
          if constexpr (kKV == kKvI8) {
            a1 = codes_to_f16(ko.k1[s / 2][2 * (s % 2)], ko.k1[s / 2][2 * (s % 2) + 1]);
            a2 = codes_to_f16(ko.k2[s / 2][2 * (s % 2)], ko.k2[s / 2][2 * (s % 2) + 1]);
          } else {
            a1 = nibbles_to_f16_hi16(ko.k1[s]);
            a2 = nibbles_to_f16_hi16(ko.k2[s]);
          }
          const f16x8 qh = __builtin_bit_cast(f16x8, qv[hh][s]);
          s1[hh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qh, s1[hh], 0, 0, 0);
          s2[hh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, qh, s2[hh], 0, 0, 0);
        }
      }
      if constexpr (kQ) {
        const float f = (vsel ? ko.ks_b : ko.ks_a) * c;
        const float c0 = -kOffset * qsum[hh] * f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s1[hh][e] = fmaf(s1[hh][e], f, c0);
          s2[hh][e] = fmaf(s2[hh][e], f, c0);
        }
      }
    }
  };
  // -inf for keys past this lane's query, past the context or in a missing block
  auto mask_scores = [&](int tok0, int32_t my_blk) {
    const int t_first = tok0 + 8 * qg;
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (t_first + e > limit || my_blk < 0) s1[hh][e] = -INFINITY;
        if (t_first + 4 + e > limit || my_blk < 0) s2[hh][e] = -INFINITY;
      }
    }
  };
  auto is_edge = [&](int tok0, Pair bl) {  // pairs that need masks (wave-uniform)
    return tok0 + kPairTok > L || bl.a < 0 || bl.b < 0 || tok0 + kPairTok - 1 > p_first;
  };
  // scaled maximum over the scores in s1, s2 of this lane's query (all four lane groups)
  auto pair_max = [&](int hh) {
    float m = fmaxf(fmaxf(fmaxf(s1[hh][0], s1[hh][1]), fmaxf(s1[hh][2], s1[hh][3])),
                    fmaxf(fmaxf(s2[hh][0], s2[hh][1]), fmaxf(s2[hh][2], s2[hh][3])));
    return max_across_groups(m) * cx;
  };
  // exact maximum over all keys of the tile (the rare second pass)
  auto sweep_max = [&]() {
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) ref[hh] = -INFINITY;
    Pair cur = blocks_of(0);
    load_k(cur);
    for (int i = 0; i < n_pairs; ++i) {
      const Pair nxt = blocks_of(min(i + 1, n_pairs - 1));
      scores();
      load_k(nxt);
      if (is_edge(i * kPairTok, cur)) mask_scores(i * kPairTok, vsel ? cur.b : cur.a);
#pragma unroll
      for (int hh = 0; hh < kH; ++hh) ref[hh] = fmaxf(ref[hh], pair_max(hh));
      cur = nxt;
    }
  };

  if (n_pairs > 0) {
    const Pair b0 = blocks_of(0);
    load_k(b0);
    scores();
    if (is_edge(0, b0)) mask_scores(0, vsel ? b0.b : b0.a);
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) ref[hh] = pair_max(hh);
  }
  for (int pass = 0; pass < 2; ++pass) {
    float r0[kH];
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) {
      r0[hh] = ref[hh] == -INFINITY ? 0.f : ref[hh];
      l_run[hh] = 0.f;
      c_run[hh] = 0.f;
#pragma unroll
      for (int t = 0; t < kTiles; ++t) acc[hh][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bool over = false;
    // requested even when the tile has no pairs (block ids are clamped, so the loads stay in
    // bounds): the loop below is then entered only with these loads outstanding, which keeps
    // its first wait to this pair's K
    Pair cur = blocks_of(0);
    load_k(cur);
    load_v(cur);
    // One pair of blocks per step, single-buffered: the next pair's K is requested once every
    // head's scores have consumed this pair's K, and its V once P . V has consumed this V.
    // Every step requests the same loads (the last pair requests itself again, a cache hit):
    // vector loads complete in order, and a step without them would make the waits after the
    // join cover the next pair's loads too.
    for (int i = 0; i < n_pairs; ++i) {
      const int tok0 = i * kPairTok;
      const int t_first = tok0 + 8 * qg;
      const Pair nxt = blocks_of(min(i + 1, n_pairs - 1));
      const int32_t my_blk = vsel ? cur.b : cur.a;
      scores();
      load_k(nxt);
      if constexpr (kKV == kKvBf16) {
        if (tok0 + kPairTok > L || cur.a < 0 || cur.b < 0) {
          // tokens past the context (or of a missing block) must not reach P.V even with
          // p = 0 (their V may be anything); quantised codes are always finite, so there
          // p = 0 is enough
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            const bool k0 = my_blk >= 0 && t_first + 2 * cc < L;
            const bool k1b = my_blk >= 0 && t_first + 2 * cc + 1 < L;
            const uint32_t keep = (k0 ? 0x0000ffffu : 0u) | (k1b ? 0xffff0000u : 0u);
#pragma unroll
            for (int t = 0; t < kTiles; ++t) vo.v[t][cc] &= keep;
          }
        }
      }
      if (is_edge(tok0, cur)) mask_scores(tok0, my_blk);
      // a missing block's V scale is never read as a number (its P are 0, and 0 * scale must
      // stay 0 whatever the unused entry holds).  The choice is made here, at the use, where
      // the value is waited for anyway: made where the scales are loaded, it would wait for
      // those loads (and every scalar load in flight) one pair early.
      const float vsc = kQ ? (my_blk >= 0 ? (vsel ? vo.vs_b : vo.vs_a) : 0.f) : 1.f;
      // bf16 cache: V tiles as fp16 operands, converted once for all heads of the wave (exact
      // for |V| in fp16's normal range), so P . V takes one fp16 MFMA per tile
      f16x8 vh[kKV == kKvBf16 ? kTiles : 1];
      if constexpr (kKV == kKvBf16) {
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          f32x8 vf;
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            vf[2 * cc] = __uint_as_float(vo.v[t][cc] << 16);
            vf[2 * cc + 1] = __uint_as_float(vo.v[t][cc] & 0xffff0000u);
          }
          vh[t] = __builtin_convertvector(vf, f16x8);
        }
      }
#pragma unroll
      for (int hh = 0; hh < kH; ++hh) {
        f32x8 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(fmaf(s1[hh][e], cx, -r0[hh]));
          pv[4 + e] = __builtin_amdgcn_exp2f(fmaf(s2[hh][e], cx, -r0[hh]));
        }
        const float psum = ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
        l_run[hh] += psum;
        // O^T += V^T . P^T: V rows are dims, P^T columns are this lane's query, so the
        // accumulator column of a lane is its own query
        if constexpr (kKV == kKvBf16) {
          // P as one fp16 operand (11-bit significand); its range bound asks for the exact-
          // maximum pass like the quantised path's
          over = over || !(psum <= kOverPQ);
          const f16x8 p16 = __builtin_convertvector(pv, f16x8);
#pragma unroll
          for (int t = 0; t < kTiles; ++t)
            acc[hh][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh[t], p16, acc[hh][t], 0, 0, 0);
        } else {
          over = over || !(psum * vsc <= kOverPQ);
          // P times the block's V scale as one fp16 operand next to the fp16 codes; the code
          // offset comes out with the sum of exactly these rounded operands, so it cancels
          // int4: elements 4..7 meet codes expanded at 16 times their value
          const float vsc_hi = kKV == kKvI4 ? vsc * 0.0625f : vsc;
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] *= e < 4 ? vsc : vsc_hi;
          const f16x8 p16 = __builtin_convertvector(pv, f16x8);
          const f32x8 pr = __builtin_convertvector(p16, f32x8);
          if constexpr (kKV == kKvI4) {
            c_run[hh] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) * kNibbleOffset +
                         ((pr[4] + pr[5]) + (pr[6] + pr[7])) * kNibbleOffsetHi16;
          } else {
            c_run[hh] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
          }
#pragma unroll
          for (int t = 0; t < kTiles; ++t) {
            f16x8 vop;
            if constexpr (kKV == kKvI8) {
              vop = codes_to_f16(vo.v[t][0], vo.v[t][1]);
            } else {
              vop = nibbles_to_f16_hi16(vo.v[t]);
            }
            acc[hh][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, p16, acc[hh][t], 0, 0, 0);
          }
        }
      }
      load_v(nxt);
      cur = nxt;
    }
    if (pass == 1) break;
    // queries of this lane's column whose keys were all masked keep l = 0 in both passes
#pragma unroll
    for (int hh = 0; hh < kH; ++hh) over = over || l_run[hh] < kUnderL;
    if (!__ballot(over)) break;
    sweep_max();
  }

  // l summed over the four lane groups is query r's; a lane holds dims 16 t + 4 qg .. +3 of it
  const int out_row = row0 + my_q;
  const bool store = my_q < n && out_row < a.T && out_row >= 0;
#pragma unroll
  for (int hh = 0; hh < kH; ++hh) {
    const float lq = sum_across_groups(l_run[hh]);
    const float off = kQ ? kOffset * sum_across_groups(c_run[hh]) : 0.f;
    if (store) {
      float* o = a.out + (static_cast<int64_t>(out_row) * a.Hq + h0 + hh) * D + 4 * qg;
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const f32x4 y = lq > 0.f ? (acc[hh][t] - off) / lq : f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(o + 16 * t) = y;
      }
    }
  }
}

template <int G, int D, int kKV>
hipError_t launch_gdk(const PrefillArgs& a, hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(a.max_tiles) * a.Hkv * (G / kHeadsPerWave<G>);
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_mfma_kernel<G, D, kKV>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * kWavesPerWG), 0, stream, a);
  return hipGetLastError();
}

template <int G, int D>
hipError_t launch_gd(const PrefillArgs& a, hipStream_t stream) {
  switch (a.kv_kind) {
    case kKvBf16: return launch_gdk<G, D, kKvBf16>(a, stream);
    case kKvI8: return launch_gdk<G, D, kKvI8>(a, stream);
    case kKvI4: return launch_gdk<G, D, kKvI4>(a, stream);
    default: return hipErrorNotSupported;
  }
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
