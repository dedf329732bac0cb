// Paged decode attention on the gfx950 matrix cores: bf16 q over a bf16, int8 or packed int4
// cache.
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
// Work split.  The unit of work is a block *pair* (32 tokens) of one (KV head, sequence) segment.
// A workgroup has 8 waves, two per SIMD.  Two schedules decide who takes which pairs:
//   balanced (default): all segments are laid end to end (KV-head-major, then sequence) and the
//     unit range is cut into equal contiguous spans, one per resident workgroup, so every
//     workgroup moves the same number of bytes whatever the length mix.  Each wave streams its
//     own contiguous eighth of the span with no barriers, keeping one softmax state per segment
//     it walks through and writing it out directly when it holds the whole segment; states of
//     segments it shares with other waves are merged in LDS at the end.  A segment cut by a
//     span boundary leaves a partial state per workgroup, merged by streamk_reduce_kernel.
//   fixed partitions (caller-given length): one workgroup per (partition, KV head, sequence),
//     its waves taking the pairs in turn, merged by splitk_reduce_kernel.
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
// Quantised caches score with exact integer products on v_mfma_i32_16x16x64_i8 (the codes as
// they are, q as two int8 parts on its absmax scale) and run P.V on v_mfma_f32_16x16x32_f16:
// codes expand to fp16 values offset + c (a byte permute for int8, a nibble mask and permute for
// int4), P is one fp16 operand, and the offset part of P.V comes out through one more MFMA of
// the same rounded P against a tile of the offsets, so it cancels exactly.  Loads of up to
// kDepth pairs are in flight per wave.
//
// Shared prefixes (pa_decode_shared_prefix) run the same pair loop in two more modes: a prefix
// pass whose 16 MFMA columns hold the query heads of up to 16/G members of a group, reading the
// blocks they share once, and a suffix pass, the balanced schedule over each sequence's tokens
// past its prefix; the merge launch folds the prefix states into the rows.
#include <cmath>
#include <type_traits>

#include "device_load.h"
#include "internal.h"
#include "pagedkv.h"
#include "quant_f16.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
// Waves per workgroup of the decode kernel.  bf16 caches with up to 4 query heads per KV head
// keep one pair in flight per wave instead of two, which leaves them at ~160 VGPRs, so three
// waves share each SIMD (12 per workgroup); the others run two per SIMD.
template <int G, int kKV>
constexpr int kWavesOf = (G <= 4 && kKV == kKvBf16) ? 12 : kWaves;
constexpr int kPrefixWaves = 8;  // the shared-prefix pass's workgroup
constexpr int kPair = 2 * kBlockSize;  // tokens per wave iteration

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Maximum and integer sum over the four 16-lane groups (lanes r, r + 16, r + 32, r + 48), every
// lane receiving the result, with the gfx950 half and row swaps: plain VALU work, where a lane
// shuffle goes through the LDS crossbar and its wait would also cover the scalar loads of the
// block table and scales that are in flight (used by the quantised kinds)
__device__ __forceinline__ float group_max(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int group_sum(int x) {
  const auto h = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(x),
                                                  static_cast<uint32_t>(x), false, false);
  x = static_cast<int>(h[0]) + static_cast<int>(h[1]);
  const auto r = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(x),
                                                  static_cast<uint32_t>(x), false, false);
  return static_cast<int>(r[0]) + static_cast<int>(r[1]);
}

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// K/V tiles are read exactly once per launch: non-temporal loads keep them from displacing
// lines that are reused (tables, q, the last-level cache's other contents).  Measured on the
// Llama-3.1-8B-shaped batch: 121.5 -> 112.5 us for the same bytes.
struct StreamLoad {
  template <typename T>
  __device__ __forceinline__ T get(const void* p) const {
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  }
};

template <int D>
struct PairRegs {
  static constexpr int kSteps = D / 32;  // k-steps of the score MFMAs
  static constexpr int kTiles = D / 16;  // output dim tiles of P.V
  u32x4 k1[kSteps];   // score tile 1 rows (tokens A0-3, A8-11, B0-3, B8-11)
  u32x4 k2[kSteps];   // score tile 2 rows (tokens A4-7, A12-15, B4-7, B12-15)
  u32x4 v[kTiles];    // 8 tokens x 1 dim per tile
  int32_t blk_a, blk_b;  // physical blocks, -1 when masked
};

// int8 cache: the same tiles at one byte per element, plus the (block, head) scales.
template <int D>
struct PairRegsI8 {
  static constexpr int kSteps = D / 32;
  static constexpr int kTiles = D / 16;
  u32x4 k1[kSteps / 2];  // 16 dims per load = two k-steps
  u32x4 k2[kSteps / 2];
  u32x2 v[kTiles];       // 8 tokens x 1 dim per tile
  int32_t blk_a, blk_b;
  float ks_a, ks_b, vs_a, vs_b;
};

// int4 cache tiles: K [bs][D/2] bytes, V [D][bs/2] bytes; one 4-byte group holds the 8 dims a
// lane feeds one k-step (K) or its 8 tokens of one dim (V).
template <int D>
struct PairRegsI4 {
  static constexpr int kSteps = D / 32;
  static constexpr int kTiles = D / 16;
  uint32_t k1[kSteps];
  uint32_t k2[kSteps];
  uint32_t v[kTiles];
  int32_t blk_a, blk_b;
  float ks_a, ks_b, vs_a, vs_b;
};

// Pairs each cache kind keeps in flight per wave.  Eight waves per CU already keep enough bytes
// in flight; the quantised kinds are bound by issue slots, and deeper look-ahead only adds
// register pressure (measured: bf16 1 and 2 equal, int8 best at 1, int4 best at 2).
constexpr int kDepthBf16 = 2, kDepthI8 = 1, kDepthI4 = 2;

// Cost of a segment start in the balanced schedule, in pairs of the cache's kind (see the span
// computation).  A start costs about the same time whatever the kind, so it is worth more of
// the cheaper int4 pairs (4 KB against 8 KB int8 and 16 KB bf16).
template <int kKV>
constexpr int kSegCostOf = kKV == kKvI4 ? 3 : 2;

// Schedules of decode_mfma_kernel.
constexpr int kFixed = 0;     // one workgroup per (partition, KV head, sequence)
constexpr int kBalanced = 1;  // equal spans of block pairs per workgroup
constexpr int kSuffix = 2;    // kBalanced over the pairs past each sequence's shared prefix, with
                              // the prefix pass's states folded into every final output
constexpr int kPrefix = 3;    // the shared-prefix pass (16 query columns of a group's members)

// Tokens of sequence b that the prefix pass covered (0 when it has no shared prefix).
__device__ __forceinline__ int prefix_tokens(const DecodeArgs& a, int b, int L) {
  const int ps = a.pstart[b] + a.ref_p[b];
  return min(max(ps, 0), L) & ~(2 * kBlockSize - 1);
}

// Prefix-pass parts that output rows of a sequence with ps prefix tokens fold in.
__device__ __forceinline__ int prefix_parts_of(const DecodeArgs& a, int ps) {
  return ps > 0 ? min((ps + a.pf_tokens - 1) / a.pf_tokens, a.pf_parts) : 0;
}

// One prefix-pass state of element d of output row `row`, part k: (m, l, o).
struct PrefixState {
  float m, l, o;
};
__device__ __forceinline__ PrefixState load_prefix(const DecodeArgs& a, int64_t row, int k,
                                                   int d) {
  const int64_t slot = row * a.pf_parts + k;
  return {a.pf_m[slot], a.pf_l[slot], a.pf_o[slot * a.D + d]};
}

// Folds a prefix state into the running state (M, num, den) of one element: M the max (log2
// domain), num the weighted sum of values and den the sum of weights, both relative to M.
// Callers load the states of all their elements first and fold them after, so one round trip
// to memory serves them all.
__device__ __forceinline__ void fold_state(float& M, float& num, float& den, PrefixState p) {
  if (!(p.l > 0.f)) return;
  const float mn = fmaxf(M, p.m);
  const float c = __builtin_amdgcn_exp2f(M - mn);  // 0 while the running state is empty
  const float f = p.l * __builtin_amdgcn_exp2f(p.m - mn);
  num = num * c + f * p.o;
  den = den * c + f;
  M = mn;
}

// Plain (cached) loads: the prefix pass reads each shared tile once per column block, and the
// column blocks of one tile run side by side on one XCD, so the second read comes from its L2.
struct CachedLoad {
  template <typename T>
  __device__ __forceinline__ T get(const void* p) const {
    return *reinterpret_cast<const T*>(p);
  }
};

// The decode of one workgroup: workgroup wg of the nwg that share the balanced schedule or
// the prefix pass (the fixed schedule takes its partition, head and sequence from the grid).
template <int G, int D, int kMode, int kKV>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, const int wg, const int nwg) {
  constexpr bool kStream = kMode == kBalanced || kMode == kSuffix;  // balanced schedule
  constexpr bool kFold = kMode == kSuffix;
  constexpr bool kPre = kMode == kPrefix;
  constexpr int kW = kPre ? kPrefixWaves : kWavesOf<G, kKV>;  // waves per workgroup
  // column tiles per wave: the prefix pass takes two column blocks (32 query columns) on every
  // pair it loads, so each load serves twice the columns
  constexpr int CT = kPre ? 2 : 1;
  static_assert(!kPre || G == 16, "the prefix pass fills all 16 columns of its tiles");
  constexpr bool kI4 = kKV == kKvI4;
  constexpr bool kI8 = kKV == kKvI8 || kI4;  // a quantised cache (scales, offset codes)
  // quantised caches: int8 score tiles of 64 dims per v_mfma_i32_16x16x64_i8
  constexpr int kK8 = D / 64;
  using Regs = std::conditional_t<kI4, PairRegsI4<D>,
                                  std::conditional_t<kI8, PairRegsI8<D>, PairRegs<D>>>;
  // pairs in flight per wave (the prefix pass keeps one: two waves per SIMD cover each other's
  // waits better than one wave with four pairs in flight)
  constexpr int kDepth =
      kPre ? 1 : (kI4 ? kDepthI4 : (kI8 ? kDepthI8 : (kW == 12 ? 1 : kDepthBf16)));
  constexpr int kSteps = D / 32;
  constexpr int kTiles = D / 16;

  // Per-wave softmax states waiting to be merged: one slot per wave for the fixed schedule (the
  // piece the whole workgroup shares), two for the balanced one (the first and the last piece of
  // the wave's span, when a neighbouring wave holds the rest of it).  o holds acc - 128 c (the
  // int8 offset already taken out).
  constexpr int kSlots = kStream ? 2 : 1;
  // balanced schedule: pair-count prefix sums cum_s[0..B], then cost prefix sums cc_s[0..B]
  extern __shared__ int32_t cum_s[];
  __shared__ float m_s[kW][kSlots][G];
  __shared__ float l_s[kW][kSlots][G];
  __shared__ float o_s[kW][kSlots][G][D];
  __shared__ int32_t wave_tot[kW];
  // prefix pass: output row (-1: unused) and token limit of each query column of the item
  __shared__ int32_t colrow_s[kPre ? 16 * CT : 1], collim_s[kPre ? 16 * CT : 1];

  const int lane = threadIdx.x % 64;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int r = lane % 16;   // row / column index inside an MFMA tile
  const int qg = lane / 16;  // k-group of the lane

  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(a.v);
  const uint8_t* __restrict__ kc8 = static_cast<const uint8_t*>(a.k);
  const uint8_t* __restrict__ vc8 = static_cast<const uint8_t*>(a.v);
  const int NB = a.NB, Hkv = a.Hkv;

  // token rows of the two score tiles, relative to the pair start
  const int tok1 = (r / 8) * 16 + ((r / 4) % 2) * 8 + (r % 4);
  const int tok2 = tok1 + 4;
  const int vblk_sel = qg / 2;         // which block of the pair this lane's P.V tokens are in
  const int vtok = 8 * (qg % 2);       // first of its 8 tokens inside that block

  // One piece: pairs [i0, i1) of KV head g of sequence b (L tokens).
  //   solo = false: every wave of the workgroup calls it with the same arguments, the waves take
  //     the pairs in turn and merge in LDS; dest 0 = final output, 1 = fixed-partition slot
  //     `part`.
  //   solo = true: the calling wave takes every pair itself; with lds_slot >= 0 it leaves its
  //     state in LDS slot (w, lds_slot), otherwise it writes the result: dest 0 = final output,
  //     2 = balanced-schedule slot `part`.
  //   ps (kSuffix): tokens of b the prefix pass covered; a final output folds in its states.
  //   kPrefix: b is the group's reference sequence (its table is read), the query columns and
  //     their token limits come from colrow_s / collim_s, and the merged states go to prefix
  //     part `part` of each column's row.
  auto run_piece = [&](int b, int g, int L, int i0, int i1, bool solo, int dest, int64_t part,
                       int lds_slot, int ps) {
    const int32_t* __restrict__ table = a.tables + static_cast<int64_t>(b) * a.max_blocks;
    const int end = L;

    // q^T operand, head (r % G).  bf16 cache: step s covers dims 32 s + 8 qg .. +8.
    // Quantised caches score with exact integer products (v_mfma_i32_16x16x64_i8): q enters as
    // two int8 parts on the head's absmax scale sq = max|q| / 127, q ~ sq (hi + lo / 128)
    // (within sq / 256, about 15 bits of the largest element), the codes as they are (int4:
    // nibbles unpacked to bytes c + 8).  Lane group qg holds dims of tile t in the order the K
    // operand has them: int8 16 qg + 64 t + m, int4 (D / 4) qg + 16 t + m, m < 16; both read
    // as the 8-dim groups s = 2 t, 2 t + 1 of the loads below.
    // (one set per column tile ct: the prefix pass's lane holds columns r and 16 + r)
    u32x4 qv[CT][kI8 ? 1 : kSteps];
    i32x4 qh[CT][kI8 ? kK8 : 1], ql[CT][kI8 ? kK8 : 1];
    float qscale[CT];  // quantised: sq / 128, the weight of one unit of hi * 128 + lo
    int q8[CT];        // int4: 8 * sum_d (128 hi + lo), the nibbles' +8 times q
    int lim_tok[CT];   // kPrefix: tokens of the lane's column (its pairs from lim_tok on are masked)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      qscale[ct] = 0.f;
      q8[ct] = 0;
      lim_tok[ct] = 0;
      int64_t qrow = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + r % G;
      if constexpr (kPre) {
        const int cr = colrow_s[16 * ct + r];
        qrow = cr >= 0 ? cr : colrow_s[0];  // an unused column computes on a valid row
        lim_tok[ct] = collim_s[16 * ct + r];
      }
      const uint16_t* q = static_cast<const uint16_t*>(a.q) + qrow * D;
      if constexpr (kI8) {
        f32x8 f[kSteps];
        float amax = 0.f;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          const u32x4 raw = kI4 ? load16(q + (D / 4) * qg + 8 * s)
                                : load16(q + 16 * (qg + 4 * (s / 2)) + 8 * (s % 2));
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            f[s][2 * c] = __uint_as_float(raw[c] << 16);
            f[s][2 * c + 1] = __uint_as_float(raw[c] & 0xffff0000u);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[s][e]));
        }
        amax = group_max(amax);
        const float sq = amax > 0.f ? amax / 127.f : 1.f;
        const float inv = amax > 0.f ? 127.f / amax : 1.f;
        qscale[ct] = sq * (1.f / 128.f);
        int qtot = 0;
#pragma unroll
        for (int t = 0; t < kK8; ++t) {
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {  // 4 dims per word: group s = 2 t + c / 2
            uint32_t hb = 0, lb = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = f[2 * t + c / 2][4 * (c % 2) + e] * inv;
              const float hi = __builtin_rintf(x);
              const float lo = __builtin_rintf((x - hi) * 128.f);
              const int hv = static_cast<int>(hi), lv = static_cast<int>(lo);
              qtot += 128 * hv + lv;
              hb |= (static_cast<uint32_t>(hv) & 0xffu) << (8 * e);
              lb |= (static_cast<uint32_t>(lv) & 0xffu) << (8 * e);
            }
            hw[c] = hb;
            lw[c] = lb;
          }
          qh[ct][t] = i32x4{static_cast<int32_t>(hw[0]), static_cast<int32_t>(hw[1]),
                        static_cast<int32_t>(hw[2]), static_cast<int32_t>(hw[3])};
          ql[ct][t] = i32x4{static_cast<int32_t>(lw[0]), static_cast<int32_t>(lw[1]),
                        static_cast<int32_t>(lw[2]), static_cast<int32_t>(lw[3])};
        }
        if constexpr (kI4) {
          qtot = group_sum(qtot);
          q8[ct] = 8 * qtot;
        }
      } else {
#pragma unroll
        for (int s = 0; s < kSteps; ++s) qv[ct][s] = load16(q + 32 * s + 8 * qg);
      }
    }

    auto load_pair = [&](int i, Regs& R) {
      const int tok0 = __builtin_amdgcn_readfirstlane(i * kPair);
      const int j = tok0 / kBlockSize;
      int32_t ba = uniform_load(table, j);
      int32_t bb = (tok0 + kBlockSize < end) ? uniform_load(table, j + 1) : -1;
      ba = (ba >= 0 && ba < NB) ? ba : -1;
      bb = (bb >= 0 && bb < NB) ? bb : -1;
      R.blk_a = ba;
      R.blk_b = bb;
      const int64_t ta = static_cast<int64_t>(ba < 0 ? 0 : ba) * Hkv + g;  // (block, head) tiles
      const int64_t tb = static_cast<int64_t>(bb < 0 ? 0 : bb) * Hkv + g;
      const int64_t tile_a = ta * (kBlockSize * D);
      const int64_t tile_b = tb * (kBlockSize * D);
      if constexpr (kI8) {
        // a masked block reads block 0's entries in its place: its scores become -inf whatever
        // the K scale gives, and its V scale is zeroed where it is used
        R.ks_a = uniform_load(a.k_scale, ta);
        R.ks_b = uniform_load(a.k_scale, tb);
        R.vs_a = uniform_load(a.v_scale, ta);
        R.vs_b = uniform_load(a.v_scale, tb);
      }
      const std::conditional_t<kPre, CachedLoad, StreamLoad> ld;
      if constexpr (kI4) {
        const int64_t h_a = tile_a / 2, h_b = tile_b / 2;  // tiles of bs * D / 2 bytes
        const uint8_t* k1 = kc8 + (tok1 < 16 ? h_a : h_b) + (tok1 % 16) * (D / 2) + 4 * kSteps * qg;
        const uint8_t* k2 = kc8 + (tok2 < 16 ? h_a : h_b) + (tok2 % 16) * (D / 2) + 4 * kSteps * qg;
        if constexpr (kSteps == 4) {
          const u32x4 x1 = ld.template get<u32x4>(k1);
          const u32x4 x2 = ld.template get<u32x4>(k2);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            R.k1[c] = x1[c];
            R.k2[c] = x2[c];
          }
        } else {
          const u32x2 x1 = ld.template get<u32x2>(k1);
          const u32x2 x2 = ld.template get<u32x2>(k2);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            R.k1[c] = x1[c];
            R.k2[c] = x2[c];
          }
        }
        // V: two dim rows (16 tokens of 4 bits each) per 16-byte load, 64 dims per load over the
        // wave: lane group qg reads block qg / 2, dims 64 t + 32 (qg % 2) + 2 r and + 1 (rows of
        // 8 bytes); compute_pair pairs up the half rows with the neighbouring lane group
        const uint8_t* v = vc8 + (vblk_sel ? h_b : h_a) + 256 * (qg % 2) + 16 * r;
#pragma unroll
        for (int t = 0; t < kTiles / 4; ++t) {
          const u32x4 x = ld.template get<u32x4>(v + 512 * t);
#pragma unroll
          for (int c = 0; c < 4; ++c) R.v[4 * t + c] = x[c];
        }
      } else if constexpr (kI8) {
        const uint8_t* k1 = kc8 + (tok1 < 16 ? tile_a : tile_b) + (tok1 % 16) * D + 16 * qg;
        const uint8_t* k2 = kc8 + (tok2 < 16 ? tile_a : tile_b) + (tok2 % 16) * D + 16 * qg;
#pragma unroll
        for (int c = 0; c < kSteps / 2; ++c) {
          R.k1[c] = ld.template get<u32x4>(k1 + 64 * c);
          R.k2[c] = ld.template get<u32x4>(k2 + 64 * c);
        }
        // V: one whole dim row (16 tokens) per 16-byte load, dims 32 t + 16 (qg % 2) + r of
        // block qg / 2; words 0, 1 are token half 0, words 2, 3 half 1 (compute_pair pairs the
        // halves up with the neighbouring lane group)
        const uint8_t* v = vc8 + (vblk_sel ? tile_b : tile_a) + (16 * (qg % 2) + r) * kBlockSize;
#pragma unroll
        for (int t = 0; t < kTiles / 2; ++t) {
          const u32x4 x = ld.template get<u32x4>(v + 32 * t * kBlockSize);
          R.v[2 * t] = u32x2{x[0], x[1]};
          R.v[2 * t + 1] = u32x2{x[2], x[3]};
        }
      } else {
        const uint16_t* k1 = kc + (tok1 < 16 ? tile_a : tile_b) + (tok1 % 16) * D + 8 * qg;
        const uint16_t* k2 = kc + (tok2 < 16 ? tile_a : tile_b) + (tok2 % 16) * D + 8 * qg;
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          R.k1[s] = ld.template get<u32x4>(k1 + 32 * s);
          R.k2[s] = ld.template get<u32x4>(k2 + 32 * s);
        }
        const uint16_t* v = vc + (vblk_sel ? tile_b : tile_a) + r * kBlockSize + vtok;
#pragma unroll
        for (int n = 0; n < kTiles; ++n) R.v[n] = ld.template get<u32x4>(v + 16 * n * kBlockSize);
      }
    };

    float m_run[CT], l_run[CT];  // running max (log2 domain) of the lane's column (head r % G)
                                 // and the lane-partial running sum over this lane's tokens
    f32x4 acc[CT][kTiles];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      m_run[ct] = -INFINITY;
      l_run[ct] = 0.f;
#pragma unroll
      for (int n = 0; n < kTiles; ++n) acc[ct][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // quantised caches: the codes enter P.V as offset + code (offset 1152 for int8; 1032 for
    // int4 elements 0..3 and 1152 for 4..7, whose codes come at 16 times their value); accc
    // collects sum_t P_t offset_t with one more MFMA against a tile of the offsets, rounded and
    // summed exactly as the value tiles' offset parts, and is taken out at the end
    f32x4 accc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) accc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    f16x8 offs;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      offs[e] = static_cast<_Float16>(kI4 && e < 4 ? kNibbleOffset : kCodeOffset);

    auto compute_pair = [&](int i, Regs& R) {
      const int tok0 = i * kPair;
      // this lane's 8 tokens: pair tokens 8 qg + e, e = 0..7
      const int t_first = tok0 + 8 * qg;
      const int32_t my_blk = vblk_sel ? R.blk_b : R.blk_a;
      const bool tail = (tok0 + kPair > end) || R.blk_b < 0 || R.blk_a < 0;
      if (tail && !kI8) {
        // masked tokens must not reach P.V even with p = 0 (their V may be anything); int8
        // codes always convert to finite values, so there p = 0 is enough
        uint32_t keep[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bool k0 = my_blk >= 0 && t_first + 2 * c < end;
          const bool k1 = my_blk >= 0 && t_first + 2 * c + 1 < end;
          keep[c] = (k0 ? 0x0000ffffu : 0u) | (k1 ? 0xffff0000u : 0u);
        }
        if constexpr (!kI8) {
#pragma unroll
          for (int n = 0; n < kTiles; ++n)
#pragma unroll
            for (int c = 0; c < 4; ++c) R.v[n][c] &= keep[c];
        }
      }
      // quantised caches: the K operands of the integer score MFMAs, shared by the column tiles
      i32x4 ka1[kI8 ? kK8 : 1], ka2[kI8 ? kK8 : 1];
      if constexpr (kI8) {
#pragma unroll
        for (int t = 0; t < kK8; ++t) {
          if constexpr (kI4) {
            // nibble bytes c + 8 of dims (D / 4) qg + 16 t + m: words 2 t, 2 t + 1, each split
            // into its low nibbles (dims +0..3) and high nibbles (+4..7)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const uint32_t x1 = R.k1[2 * t + c], x2 = R.k2[2 * t + c];
              ka1[t][2 * c] = static_cast<int32_t>(x1 & 0x0f0f0f0fu);
              ka1[t][2 * c + 1] = static_cast<int32_t>((x1 >> 4) & 0x0f0f0f0fu);
              ka2[t][2 * c] = static_cast<int32_t>(x2 & 0x0f0f0f0fu);
              ka2[t][2 * c + 1] = static_cast<int32_t>((x2 >> 4) & 0x0f0f0f0fu);
            }
          } else {
            ka1[t] = __builtin_bit_cast(i32x4, R.k1[t]);
            ka2[t] = __builtin_bit_cast(i32x4, R.k2[t]);
          }
        }
      }
      f16x8 p16[CT];
      bf16x8 p_hi[CT], p_lo[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
        i32x4 h1 = {0, 0, 0, 0}, l1 = {0, 0, 0, 0}, h2 = {0, 0, 0, 0}, l2 = {0, 0, 0, 0};
        if constexpr (kI8) {
#pragma unroll
          for (int t = 0; t < kK8; ++t) {
            h1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka1[t], qh[ct][t], h1, 0, 0, 0);
            l1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka1[t], ql[ct][t], l1, 0, 0, 0);
            h2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka2[t], qh[ct][t], h2, 0, 0, 0);
            l2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ka2[t], ql[ct][t], l2, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int s = 0; s < kSteps; ++s) {
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k1[s]), as_bf16x8(qv[ct][s]),
                                                         s1, 0, 0, 0);
            s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(R.k2[s]), as_bf16x8(qv[ct][s]),
                                                         s2, 0, 0, 0);
          }
        }
        float sc[8];
        if constexpr (kI8) {
          // score = k_scale * sq / 128 * sum_d c_d (128 hi_d + lo_d), the sum exact in int32
          // (int4: the bytes hold c + 8, whose 8 (128 hi + lo) summed over d is q8)
          const float f = (vblk_sel ? R.ks_b : R.ks_a) * a.scale_log2 * qscale[ct];
          const float c0 = kI4 ? -static_cast<float>(q8[ct]) * f : 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sc[e] = fmaf(static_cast<float>((h1[e] << 7) + l1[e]), f, c0);
            sc[4 + e] = fmaf(static_cast<float>((h2[e] << 7) + l2[e]), f, c0);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sc[e] = s1[e] * a.scale_log2;
            sc[4 + e] = s2[e] * a.scale_log2;
          }
        }
        if (tail) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (t_first + e >= end || my_blk < 0) sc[e] = -INFINITY;
        }
        if constexpr (kPre) {
          // column limits are multiples of a pair; the reference's tokens below the group's
          // prefix length are all live, so p = 0 keeps a masked column's values out
          if (tok0 >= lim_tok[ct]) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[e] = -INFINITY;
          }
        }
        float bmax = sc[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) bmax = fmaxf(bmax, sc[e]);
        if constexpr (kI8) {
          bmax = group_max(bmax);
        } else {
          // bf16 keeps the lane shuffles: with the swaps it measured 0.6% slower
          bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
          bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
        }
        const float m_new = fmaxf(m_run[ct], bmax);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[ct] - m_use);
        // quantised caches spend their issue slots on ALU work, so they skip the accumulator
        // rescale (alpha is exactly 1) on pairs where no column's maximum grew, most pairs once
        // a few hundred tokens are in; bf16 waits on memory and rescales unconditionally
        const bool rescale = !kI8 || __ballot(m_new != m_run[ct]) != 0;
        m_run[ct] = m_new;
        f32x8 pv;
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
          psum += pv[e];
        }
        l_run[ct] = l_run[ct] * alpha + psum;
        if constexpr (kI8) {
          // fold this block's V scale into P and round it to the fp16 operand once; the offset
          // tile meets exactly those operands, so the offsets cancel
          // (a masked block's scale is never read as a number: its P are 0, and 0 * scale must
          // stay 0 whatever the unused entry holds; chosen here, at the use, so that the wave
          // does not wait for the look-ahead's scalar loads a pair early)
          const float vs = my_blk >= 0 ? (vblk_sel ? R.vs_b : R.vs_a) : 0.f;
          // int4: elements 4..7 meet codes expanded at 16 times their value
          const float vs_hi = kI4 ? vs * 0.0625f : vs;
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] *= e < 4 ? vs : vs_hi;
          p16[ct] = __builtin_convertvector(pv, f16x8);
        } else {
          // P as bf16 hi + lo
          p_hi[ct] = __builtin_convertvector(pv, bf16x8);
          const u32x4 hi_bits = __builtin_bit_cast(u32x4, p_hi[ct]);
          f32x8 rest;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            rest[2 * c] = pv[2 * c] - __uint_as_float(hi_bits[c] << 16);
            rest[2 * c + 1] = pv[2 * c + 1] - __uint_as_float(hi_bits[c] & 0xffff0000u);
          }
          p_lo[ct] = __builtin_convertvector(rest, bf16x8);
        }
        // rescale the accumulators: rows 4 qg + j hold head (4 qg + j) % G
        if (rescale) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float aj;
            if constexpr (G <= 4) {
              aj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), j % G));
            } else {
              aj = __shfl(alpha, (4 * qg + j) % G, 64);
            }
#pragma unroll
            for (int n = 0; n < kTiles; ++n) acc[ct][n][j] *= aj;
            if constexpr (kI8) accc[ct][j] *= aj;
          }
        }
        if constexpr (kI8) accc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(p16[ct], offs, accc[ct], 0, 0, 0);
      }
      if constexpr (kI8) {
        // P as one fp16 operand (11-bit significand: its rounding stays far inside the int8 /
        // int4 tolerance) next to fp16 codes
        // int4: words 4 t + 2 e and 4 t + 2 e + 1 of a lane hold the token halves 0 and 1 of its
        // dim row 64 t + 32 (qg % 2) + 2 r + e.  One row swap between the lane groups of a block
        // (qg = 2 i and 2 i + 1) leaves every lane the half its own group contracts over, of the
        // even group's row (word 4 t + 2 e) and of the odd group's (word 4 t + 2 e + 1); tile
        // n = 4 t + 2 s + e takes the even (s = 0) or odd (s = 1) rows, so its column r is dim
        // 64 t + 32 s + 2 r + e (dim_of).
        // int8: R.v[2 t] / R.v[2 t + 1] hold the token halves 0 / 1 of the lane's dim row
        // 32 t + 16 (qg % 2) + r; the same swap leaves each lane its group's half of the even
        // group's row (tile 2 t, dims 32 t + r) and of the odd group's (tile 2 t + 1), so the
        // tiles keep the plain column map 16 n + r
        u32x2 v8[kI4 || !kI8 ? 1 : kTiles];
        if constexpr (kI8 && !kI4) {
#pragma unroll
          for (int t = 0; t < kTiles / 2; ++t) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const auto sw = __builtin_amdgcn_permlane16_swap(R.v[2 * t][c], R.v[2 * t + 1][c],
                                                               false, false);
              v8[2 * t][c] = sw[0];
              v8[2 * t + 1][c] = sw[1];
            }
          }
        }
        uint32_t vw[kI4 ? kTiles : 1];
        if constexpr (kI4) {
#pragma unroll
          for (int q2 = 0; q2 < kTiles / 2; ++q2) {
            const auto sw = __builtin_amdgcn_permlane16_swap(R.v[2 * q2], R.v[2 * q2 + 1], false,
                                                             false);
            vw[2 * q2] = sw[0];
            vw[2 * q2 + 1] = sw[1];
          }
        }
#pragma unroll
        for (int n = 0; n < kTiles; ++n) {
          f16x8 vop;
          if constexpr (kI4) {
            // tile n = 4 t + 2 s + e: word 4 t + 2 e + s after the swap
            vop = nibbles_to_f16_hi16(vw[4 * (n / 4) + 2 * (n % 2) + (n / 2) % 2]);
          } else {
            vop = codes_to_f16(v8[n][0], v8[n][1]);
          }
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            acc[ct][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(p16[ct], vop, acc[ct][n], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int n = 0; n < kTiles; ++n) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            acc[ct][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_hi[ct], as_bf16x8(R.v[n]),
                                                                 acc[ct][n], 0, 0, 0);
            acc[ct][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(p_lo[ct], as_bf16x8(R.v[n]),
                                                                 acc[ct][n], 0, 0, 0);
          }
        }
      }
    };

    // software pipeline: the loads of the next kDepth - 1 pairs are in flight while the
    // current pair is computed (kDepth 1: the wave waits for each pair; the other waves of the
    // CU keep the memory busy).  The loop is unrolled kDepth times so every buffer index is
    // static.
    // Every iteration issues the same loads: near the end of the piece the look-ahead reloads
    // the wave's last pair (a cache hit) instead of skipping, because a path without loads
    // would make the wait before each compute cover the look-ahead loads as well (vector
    // loads complete in order, and the wait at the join must hold on both paths).
    {
      const int step = solo ? 1 : kW;
      int i = solo ? i0 : i0 + w;
      if (i < i1) {
        const int last = i + (i1 - 1 - i) / step * step;  // the wave's last pair of the piece
        Regs R[kDepth];
#pragma unroll
        for (int j = 0; j + 1 < kDepth; ++j) load_pair(min(i + j * step, last), R[j]);
        while (i < i1) {
#pragma unroll
          for (int j = 0; j < kDepth; ++j) {
            load_pair(min(i + (kDepth - 1) * step, last), R[(j + kDepth - 1) % kDepth]);
            // keep the look-ahead loads ahead of this pair's first use of its data: hoisting
            // an MFMA above them would wait for the look-ahead's predecessors before issuing it
            __builtin_amdgcn_sched_barrier(0);
            compute_pair(i, R[j]);
            i += step;
            if (i >= i1) break;
          }
        }
      }
    }

    // the dim of column r of accumulator tile n (int4: see compute_pair)
    auto dim_of = [&](int n) {
      return kI4 ? 64 * (n / 4) + 32 * ((n / 2) % 2) + 2 * r + n % 2 : 16 * n + r;
    };
    // reduce the lane partials over the four lane groups: l_tot belongs to head r % G
    float l_tot[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      l_tot[ct] = l_run[ct] + __shfl_xor(l_run[ct], 16, 64);
      l_tot[ct] += __shfl_xor(l_tot[ct], 32, 64);
    }
    // accumulator rows 4 qg + j hold head (4 qg + j) % G; the copy with 4 qg + j < G is written
    auto to_lds = [&](int slot, int ct) {
      if (qg == 0 && r < G) {
        m_s[w][slot][r] = m_run[ct];
        l_s[w][slot][r] = l_tot[ct];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int h = 4 * qg + j;
        const float cj = kI8 ? accc[ct][j] : 0.f;  // row 4 qg + j's offset sum
        if (h < G) {
#pragma unroll
          for (int n = 0; n < kTiles; ++n) o_s[w][slot][h][dim_of(n)] = acc[ct][n][j] - cj;
        }
      }
    };
    if (solo) {  // (one column tile: CT is 2 only for the prefix pass, which never runs solo)
      if (lds_slot >= 0) {
        to_lds(lds_slot, 0);
        return;
      }
      // kSuffix: a whole segment of a sequence with a shared prefix leaves its state for the
      // merge launch, which folds the prefix states in
      const bool to_sf = kFold && dest == 0 && ps > 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int h = 4 * qg + j;
        const float lj = __shfl(l_tot[0], h % G, 64);
        const float mj = __shfl(m_run[0], h % G, 64);
        const float cj = kI8 ? accc[0][j] : 0.f;
        if (h < G) {
          const int64_t row = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + h;
          const int64_t slot = part * G + h;
#pragma unroll
          for (int n = 0; n < kTiles; ++n) {
            const float o = lj > 0.f ? (acc[0][n][j] - cj) / lj : 0.f;
            if (to_sf) {
              a.sf_o[row * D + dim_of(n)] = o;
            } else if (dest == 0) {
              a.out[row * D + dim_of(n)] = o;
            } else {
              a.ws_o[slot * D + dim_of(n)] = o;
            }
          }
          if (r == 0) {
            if (to_sf) {
              a.sf_m[row] = mj;
              a.sf_l[row] = lj;
            } else if (dest != 0) {
              a.ws_m[slot] = mj;
              a.ws_l[slot] = lj;
            }
          }
        }
      }
      if (to_sf && lane == 0) a.sf_mark[static_cast<int64_t>(b) * Hkv + g] = 1;
      return;
    }

    // merge the waves and write, one column tile at a time (the LDS states hold one)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
    if (ct > 0) __syncthreads();  // the previous tile's merge has read LDS
    to_lds(0, ct);
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * kW) {
      const int h = idx / D, d = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < kW; ++v) M = fmaxf(M, m_s[v][0][h]);
      float num = 0.f, den = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int v = 0; v < kW; ++v) {
          const float f = __builtin_amdgcn_exp2f(m_s[v][0][h] - M);
          num += f * o_s[v][0][h][d];
          den += f * l_s[v][0][h];
        }
      }
      const float o = den > 0.f ? num / den : 0.f;
      if constexpr (kPre) {
        // a column with no tokens in this part writes nothing: its row folds in only the
        // parts below its limit
        const int64_t row = colrow_s[16 * ct + h];
        if (row < 0 || collim_s[16 * ct + h] <= i0 * kPair) continue;
        const int64_t slot = row * a.pf_parts + part;
        a.pf_o[slot * D + d] = o;
        if (d == 0) {
          a.pf_m[slot] = M;
          a.pf_l[slot] = den;
        }
        continue;
      }
      const int64_t row = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + h;
      if (dest == 0) {
        a.out[row * D + d] = o;
        continue;
      }
      const int64_t slot = row * a.np_max + part;
      a.ws_o[slot * D + d] = o;
      if (d == 0) {
        a.ws_m[slot] = M;
        a.ws_l[slot] = den;
      }
    }
    }
    __syncthreads();  // LDS is reused by the next piece
  };

  if constexpr (kMode == kFixed) {
    const int p = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
    const int nparts = max(1, (L + a.partition - 1) / a.partition);
    if (p >= nparts) return;
    const int ppp = a.partition / kPair;  // pairs per partition
    const int n_b = (L + kPair - 1) / kPair;
    run_piece(b, g, L, p * ppp, min(n_b, (p + 1) * ppp), false, nparts == 1 ? 0 : 1, p, -1, 0);
  } else if constexpr (kPre) {
    // The shared-prefix pass.  Every workgroup first lists the groups with a prefix from the
    // plan (groups are runs of equal grp_ref inside aligned windows of 64 sequences), in batch
    // order.  A group of M members with a prefix of P tokens splits into items (KV head g,
    // part of pf_tokens tokens, column block cb of 16 CT = 32 query columns = member-major
    // (member, head) pairs, two MFMA column tiles that every loaded pair serves); its items are
    // numbered in runs of 8 (g, part) items per column block, so the column blocks of one
    // (g, part) sit 8 item numbers apart and, with a grid that is a multiple of 8, run at the
    // same time on the same XCD: a further read of the shared blocks is served by that XCD's
    // L2.  Items go to workgroups round-robin; the waves of a workgroup take an item's pairs in
    // turn and merge in LDS.
    const int B = a.B;
    const int Gs = a.Hq / Hkv;  // query heads per KV head of the sequences
    const int PT = a.pf_tokens;
    const int nwin = (B + 63) / 64;
    int32_t* grp_off = cum_s;                     // [gmax + 1] first item of each group
    int32_t* grp_s = cum_s + a.pf_gmax + 1;       // [gmax] first member | members << 16
    int32_t* grp_p = grp_s + a.pf_gmax;           // [gmax] prefix tokens
    constexpr int kMaxWindows = kMaxBalancedBatch / 64;
    __shared__ int32_t win_g[kMaxWindows + 1], win_i[kMaxWindows + 1];
    // Lane values of window win: is the lane the first member of a group with a prefix; if so
    // its members, prefix tokens (the longest member prefix: the reference's entry is 0) and
    // items.
    auto scan_window = [&](int win, int& members, int& ptok, int& items) -> bool {
      const int i = win * 64 + lane;
      const int gr = i < B ? a.grp_ref[i] : -1;
      const int ps = i < B ? a.pstart[i] : 0;
      const int gr_up = __shfl_up(gr, 1, 64);
      const int gr_dn = __shfl_down(gr, 1, 64);
      const bool start = gr >= 0 && (lane == 0 || gr_up != gr);
      const bool end = gr >= 0 && (lane == 63 || gr_dn != gr);
      int P = ps;  // max over this lane and the later lanes of its group (members are contiguous)
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_down(P, o, 64);
        const int g2 = __shfl_down(gr, o, 64);
        if (lane + o < 64 && g2 == gr) P = max(P, v);
      }
      const uint64_t em = __ballot(end);
      const int M = start ? __builtin_ctzll(em >> lane) + 1 : 0;
      const bool act = start && P > 0;
      const int np = (P + PT - 1) / PT, ncb = (M * Gs + 16 * CT - 1) / (16 * CT);
      members = M;
      ptok = P;
      items = act ? (Hkv * np + 7) / 8 * 8 * ncb : 0;
      return act;
    };
    for (int win = w; win < nwin; win += kW) {
      int m, pt, it;
      const bool act = scan_window(win, m, pt, it);
      int isum = it;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) isum += __shfl_xor(isum, o, 64);
      const uint64_t am = __ballot(act);
      if (lane == 0) {
        win_g[win] = __popcll(am);
        win_i[win] = isum;
      }
    }
    __syncthreads();
    if (w == 0) {
      // exclusive prefix sums over the windows (at most 128: two per lane)
      int g0 = lane < nwin ? win_g[lane] : 0, i0 = lane < nwin ? win_i[lane] : 0;
      int g1 = lane + 64 < nwin ? win_g[lane + 64] : 0, i1 = lane + 64 < nwin ? win_i[lane + 64] : 0;
      int sg0 = g0, si0 = i0, sg1 = g1, si1 = i1;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int a0 = __shfl_up(sg0, o, 64), b0 = __shfl_up(si0, o, 64);
        const int a1 = __shfl_up(sg1, o, 64), b1 = __shfl_up(si1, o, 64);
        if (lane >= o) {
          sg0 += a0;
          si0 += b0;
          sg1 += a1;
          si1 += b1;
        }
      }
      const int tg0 = __shfl(sg0, 63, 64), ti0 = __shfl(si0, 63, 64);
      if (lane < nwin) {
        win_g[lane] = sg0 - g0;
        win_i[lane] = si0 - i0;
      }
      if (lane + 64 < nwin) {
        win_g[lane + 64] = tg0 + sg1 - g1;
        win_i[lane + 64] = ti0 + si1 - i1;
      }
      if (lane == 63) {
        win_g[nwin] = tg0 + sg1;
        win_i[nwin] = ti0 + si1;
      }
    }
    __syncthreads();
    for (int win = w; win < nwin; win += kW) {
      int m, pt, it;
      const bool act = scan_window(win, m, pt, it);
      const uint64_t am = __ballot(act);
      const int rank = __popcll(am & ((1ull << lane) - 1));
      int x = it;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (act) {
        const int k = win_g[win] + rank;
        grp_off[k] = win_i[win] + x - it;
        grp_s[k] = (win * 64 + lane) | (m << 16);
        grp_p[k] = pt;
      }
    }
    const int ngroups = win_g[nwin], nitems = win_i[nwin];
    if (threadIdx.x == 0) grp_off[ngroups] = nitems;
    __syncthreads();
    for (int it = wg; it < nitems; it += nwg) {
      int lo = 0, hi = ngroups - 1;  // the group holding item it: last k with grp_off[k] <= it
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (grp_off[mid] <= it) lo = mid; else hi = mid - 1;
      }
      const int first = grp_s[lo] & 0xffff, M = grp_s[lo] >> 16, P = grp_p[lo];
      const int np = (P + PT - 1) / PT, ncb = (M * Gs + 16 * CT - 1) / (16 * CT);
      const int local = it - grp_off[lo];
      const int cb = local % (8 * ncb) / 8;
      const int qi = local / (8 * ncb) * 8 + local % 8;
      if (qi >= Hkv * np) continue;  // padding of the last run of 8
      const int g = qi / np, part = qi % np;
      const int ref = a.grp_ref[first];
      if (threadIdx.x < 16 * CT) {
        const int c = cb * 16 * CT + threadIdx.x;
        const int mi = c / Gs;
        int row = -1, lim = 0;
        if (mi < M) {
          const int mb = first + mi;
          row = mb * a.Hq + g * Gs + c % Gs;
          lim = mb == ref ? P : a.pstart[mb];
        }
        colrow_s[threadIdx.x] = row;
        collim_s[threadIdx.x] = lim;
      }
      if (threadIdx.x == 0 && qi == 0 && cb == 0) a.ref_p[ref] = P;
      __syncthreads();
      const int ptp = PT / kPair;
      run_piece(ref, g, P, part * ptp, min(P / kPair, (part + 1) * ptp), false, 3, part, -1, 0);
    }
  } else {
    // pair counts -> prefix sums cum_s[0..B], and costs -> cc_s[0..B]: the spans are cut so that
    // every workgroup and wave gets the same cost, a nonempty segment costing kSegCostOf pairs
    // more than its pairs (the latency of a segment start: its table entries, q and first tiles
    // come from memory with nothing in flight behind them).  Pieces and merges work on units.
    const int B = a.B;
    int32_t* cc_s = cum_s + B + 1;
    __shared__ int32_t wave_cost[kW];
    // kSuffix: tokens of b the prefix pass covered
    auto ps_of = [&](int b) {
      return prefix_tokens(a, b, min(max(a.seq_lens[b], 0), a.max_seq_len));
    };
    int carry = 0, carry_c = 0;
    if (threadIdx.x == 0) {
      cum_s[0] = 0;
      cc_s[0] = 0;
    }
    for (int base = 0; base < B; base += 64 * kW) {
      const int i = base + threadIdx.x;
      const int L = i < B ? min(max(a.seq_lens[i], 0), a.max_seq_len) : 0;
      int x = (L + kPair - 1) / kPair;
      if constexpr (kFold) {
        if (i < B) x -= prefix_tokens(a, i, L) / kPair;  // the pairs past the shared prefix
      }
      int c = x > 0 ? x + kSegCostOf<kKV> : 0;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        const int yc = __shfl_up(c, o, 64);
        if (lane >= o) {
          x += y;
          c += yc;
        }
      }
      if (lane == 63) {
        wave_tot[w] = x;
        wave_cost[w] = c;
      }
      __syncthreads();
      int add = carry, add_c = carry_c;
      for (int v = 0; v < w; ++v) {
        add += wave_tot[v];
        add_c += wave_cost[v];
      }
      if (i < B) {
        cum_s[i + 1] = add + x;
        cc_s[i + 1] = add_c + c;
      }
      int tot = 0, tot_c = 0;
      for (int v = 0; v < kW; ++v) {
        tot += wave_tot[v];
        tot_c += wave_cost[v];
      }
      if (base + 64 * kW < B) __syncthreads();  // wave_tot is rewritten next round
      carry += tot;
      carry_c += tot_c;
    }
    __syncthreads();
    const int64_t T = carry;              // pairs per KV head
    const int64_t U = T * Hkv;            // all units
    const int64_t CT = carry_c;           // cost per KV head
    const int64_t CU = CT * Hkv;          // all costs
    // the first unit at or after cost position x (a segment's start costs come before its first
    // pair)
    auto unit_at = [&](int64_t x) -> int64_t {
      if (x >= CU) return U;
      const int g = static_cast<int>(x / CT);
      const int r = static_cast<int>(x - static_cast<int64_t>(g) * CT);
      int b = B - 1;
      for (int base = 0; base < B; base += 64) {
        const int i = base + lane;
        const uint64_t hit = __ballot(i < B && cc_s[i + 1] > r);
        if (hit != 0) {
          b = base + __builtin_ctzll(hit);
          break;
        }
      }
      b = __builtin_amdgcn_readfirstlane(b);
      return static_cast<int64_t>(g) * T + cum_s[b] + max(r - cc_s[b] - kSegCostOf<kKV>, 0);
    };
    const int NW = nwg;
    const int wl = wg;
    // empty sequences produce zeros (kSuffix: a sequence whose prefix covers every token is
    // written by the merge launch, from the prefix pass's states alone)
    for (int b = wl; b < B; b += NW) {
      if (cum_s[b + 1] != cum_s[b]) continue;
      if (kFold && ps_of(b) > 0) continue;  // only the prefix: the merge launch writes it
      for (int i = threadIdx.x; i < a.Hq * D; i += 64 * kW)
        a.out[static_cast<int64_t>(b) * a.Hq * D + i] = 0.f;
    }
    // workgroup span [u0, u1); wave w streams its own eighth [v0, v1) of it with no barriers
    const int64_t X0 = CU * wl / NW, X1 = CU * (wl + 1) / NW;
    const int64_t u0 = unit_at(X0), u1 = unit_at(X1);
    // Merge record for the reduce kernel: the segment that starts in this span and runs past
    // its end (at most one), as {b, g, last workgroup holding a piece, slot of the piece here}.
    // An empty span marks its slot 0 as holding nothing.
    if (threadIdx.x == 0) {
      int4 rec = {-1, 0, 0, 0};
      if (u0 < u1) {
        const int g = static_cast<int>((u1 - 1) / T);
        const int rem = static_cast<int>(u1 - 1 - static_cast<int64_t>(g) * T);
        int lo = 0, hi = B - 1;
        while (lo < hi) {
          const int mid = (lo + hi) / 2;
          if (cum_s[mid + 1] > rem) hi = mid; else lo = mid + 1;
        }
        const int64_t s0 = static_cast<int64_t>(g) * T + cum_s[lo];
        const int64_t s1 = s0 + (cum_s[lo + 1] - cum_s[lo]);
        if (s0 >= u0 && s1 > u1) {
          // the workgroup holding unit s1 - 1: the one whose cost span holds its cost
          const int64_t xl = static_cast<int64_t>(g) * CT + cc_s[lo + 1] - 1;
          const int64_t wb = ((xl + 1) * NW + CU - 1) / CU - 1;
          rec = int4{lo, g, static_cast<int>(wb), s0 == u0 ? 0 : 1};
        }
      }
      reinterpret_cast<int4*>(a.ws_merge)[wl] = rec;
    }
    if (u0 == u1 && threadIdx.x < G) {
      a.ws_m[static_cast<int64_t>(wl) * 2 * G + threadIdx.x] = -INFINITY;
      a.ws_l[static_cast<int64_t>(wl) * 2 * G + threadIdx.x] = 0.f;
    }
    const int64_t v0 = unit_at(X0 + (X1 - X0) * w / kW);
    const int64_t v1 = unit_at(X0 + (X1 - X0) * (w + 1) / kW);
    __shared__ int64_t tag_s[kW][2];   // workgroup piece (first unit) held in each LDS slot
    __shared__ int32_t info_s[kW][2][4];  // its b, g, destination, partial slot
    if (lane < 2) tag_s[w][lane] = -1;
    int64_t u = v0;
    // first sequence b with cum_s[b + 1] > rem: 64 candidates per LDS read and ballot (rem is
    // below cum_s[B], so a window below B holds it)
    auto seq_at = [&](int rem) {
      int b = B - 1;
      for (int base = 0; base < B; base += 64) {
        const int i = base + lane;
        const uint64_t hit = __ballot(i < B && cum_s[i + 1] > rem);
        if (hit != 0) {
          b = base + __builtin_ctzll(hit);
          break;
        }
      }
      return __builtin_amdgcn_readfirstlane(b);
    };
    while (u < v1) {
      const int g = static_cast<int>(u / T);
      const int rem = static_cast<int>(u - static_cast<int64_t>(g) * T);
      const int b = seq_at(rem);
      const int n_b = cum_s[b + 1] - cum_s[b];
      const int i0 = rem - cum_s[b];
      const int take = static_cast<int>(min(static_cast<int64_t>(n_b - i0), v1 - u));
      const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
      const int64_t s0 = static_cast<int64_t>(g) * T + cum_s[b], s1 = s0 + n_b;
      const int64_t p0 = max(s0, u0), p1 = min(s1, u1);  // this workgroup's piece of the segment
      const bool whole = (p0 == s0 && p1 == s1);
      const int dest = whole ? 0 : 2;
      const int64_t part = static_cast<int64_t>(wl) * 2 + (p0 == u0 ? 0 : 1);
      int slot = -1;
      if (p0 != u || p1 != u + take) {
        // shared with a neighbouring wave: the wave's first or last piece
        slot = (u == v0) ? 0 : 1;
        if (lane == 0) {
          tag_s[w][slot] = p0;
          info_s[w][slot][0] = b;
          info_s[w][slot][1] = g;
          info_s[w][slot][2] = dest;
          info_s[w][slot][3] = static_cast<int32_t>(part);
        }
      }
      const int ps = kFold ? ps_of(b) : 0;
      const int off = ps / kPair;  // kSuffix: units count the pairs past the prefix
      run_piece(b, g, L, i0 + off, i0 + off + take, true, dest, part, slot, ps);
      u += take;
    }
    __syncthreads();
    // Merge the pieces that waves share.  The 2 kW LDS entries e = 2 w + slot are in unit
    // order, and the entries of one segment (equal tags) are consecutive among the used ones.
    // First the entries' (m, l) become per-entry weights 2^(m - M) and per-group sums (one
    // thread per entry and head); then every thread reads its element of all entries at once
    // and sums each group in entry order, so the result does not depend on timing.
    constexpr int kE = 2 * kW;
    __shared__ float wt_s[kE][G];   // entry weight 2^(m - M_group) (0 for unused entries)
    __shared__ float gm_s[kE][G];   // at a group's last entry: the group's M and l
    __shared__ float gl_s[kE][G];
    __shared__ uint32_t mask_s[2];  // used entries, last entries of groups
    // kSuffix: prefix tokens of each entry's sequence when the entry's segment is written out
    // (dest 0)
    __shared__ int32_t eps_s[kFold ? kE : 1];
    const float* mf = &m_s[0][0][0];
    const float* lf = &l_s[0][0][0];
    const float* of = &o_s[0][0][0][0];
    // one thread per (entry, head): the group of an entry is every used entry with its tag
    for (int t = threadIdx.x; t < kE * G; t += 64 * kW) {
      const int e = t / G, h = t % G;
      int64_t tg[kE];
      float mm[kE], ll[kE];
#pragma unroll
      for (int o = 0; o < kE; ++o) {
        tg[o] = tag_s[o / 2][o % 2];
        mm[o] = mf[o * G + h];
        ll[o] = lf[o * G + h];
      }
      const int64_t mine = tag_s[e / 2][e % 2];
      const float me = mf[e * G + h];
      const bool used = mine >= 0;
      float M = -INFINITY;
#pragma unroll
      for (int o = 0; o < kE; ++o)
        if (used && tg[o] == mine) M = fmaxf(M, mm[o]);
      const bool live = used && M != -INFINITY;
      float den = 0.f;
#pragma unroll
      for (int o = 0; o < kE; ++o)
        if (live && tg[o] == mine) den += __builtin_amdgcn_exp2f(mm[o] - M) * ll[o];
      wt_s[e][h] = live ? __builtin_amdgcn_exp2f(me - M) : 0.f;
      gm_s[e][h] = M;
      gl_s[e][h] = den;
      if constexpr (kFold) {
        if (h == 0)
          eps_s[e] = (used && info_s[e / 2][e % 2][2] == 0) ? ps_of(info_s[e / 2][e % 2][0]) : 0;
      }
    }
    if (w == kW - 1) {
      // used entries, and the last entry of each group (on the last wave, which the weights
      // above leave idle for G <= 8, so the two run side by side)
      const int64_t mine = lane < kE ? tag_s[lane / 2][lane % 2] : -1;
      bool last = mine >= 0;
#pragma unroll
      for (int o = 0; o < kE; ++o)
        if (o > lane && tag_s[o / 2][o % 2] == mine) last = false;
      const uint64_t um = __ballot(mine >= 0), em = __ballot(last);
      if (lane == 0) {
        mask_s[0] = static_cast<uint32_t>(um);
        mask_s[1] = static_cast<uint32_t>(em);
      }
    }
    __syncthreads();
    const uint32_t um = mask_s[0], em = mask_s[1];
    if (um != 0) {
      for (int idx = threadIdx.x; idx < G * D; idx += 64 * kW) {
        const int h = idx / D, d = idx % D;
        float ov[kE];
#pragma unroll
        for (int e = 0; e < kE; ++e) ov[e] = of[e * G * D + idx];  // all reads in flight at once
        float num = 0.f;
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          if ((um >> e) & 1u) num += wt_s[e][h] * ov[e];
          if ((em >> e) & 1u) {
            const int* inf = info_s[e / 2][e % 2];
            const int b = inf[0], g = inf[1], dest = inf[2], part = inf[3];
            const float den = gl_s[e][h];
            const float o = den > 0.f ? num / den : 0.f;
            const int64_t row = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + h;
            if (kFold && dest == 0 && eps_s[e] > 0) {
              // a whole segment past a shared prefix: its state, for the merge launch
              a.sf_o[row * D + d] = o;
              if (d == 0) {
                a.sf_m[row] = gm_s[e][h];
                a.sf_l[row] = den;
                if (h == 0) a.sf_mark[static_cast<int64_t>(b) * Hkv + g] = 1;
              }
            } else if (dest == 0) {
              a.out[row * D + d] = o;
            } else {
              const int64_t slot = static_cast<int64_t>(part) * G + h;
              a.ws_o[slot * D + d] = o;
              if (d == 0) {
                a.ws_m[slot] = gm_s[e][h];
                a.ws_l[slot] = den;
              }
            }
            num = 0.f;
          }
        }
      }
    }
  }
}

template <int G, int D, int kMode, int kKV>
__global__ void __launch_bounds__((64 * kWavesOf<G, kKV>))
    __attribute__((amdgpu_waves_per_eu((kWavesOf<G, kKV> / 4), (kWavesOf<G, kKV> / 4))))
decode_mfma_kernel(DecodeArgs a) {
  decode_body<G, D, kMode, kKV>(a, blockIdx.x, gridDim.x);
}

// The shared-prefix pass: eight waves per workgroup, two per SIMD, each with 32 query columns
// (two column blocks) and one pair of loads in flight, which fits two waves' registers.
template <int D, int kKV>
__global__ void __launch_bounds__(64 * kPrefixWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_prefix_kernel(DecodeArgs a) {
  decode_body<16, D, kPrefix, kKV>(a, blockIdx.x, gridDim.x);
}

// Merge the partial pieces of the segments the balanced schedule cut: one workgroup per decode
// workgroup wa, reading the record wa left.  The pieces sit in slot `first` of wa and in slot 0
// of wa + 1 .. wb (an empty span's slot 0 holds l = 0 and is skipped).  Pieces are combined in
// workgroup order, so the result does not depend on timing.  The states of both slots of wa and
// slot 0 of wa + 1 (every cut segment has those) are requested together with the record, so
// the common two-piece merge costs one round trip to memory instead of two.
// kFold (shared-prefix decode): the segment's sequence may have a shared prefix whose states are
// folded in; workgroups nw .. nw + B Hkv - 1 then write the segments past a prefix that no cut
// left to a record (fold_segment).
template <int G, int D>
__device__ void fold_segment(const DecodeArgs& a, int seg);

template <int G, int D, bool kFold>
__global__ void __launch_bounds__(256) streamk_reduce_kernel(DecodeArgs a) {
  if constexpr (kFold) {
    if (static_cast<int>(blockIdx.x) >= a.nw) {
      fold_segment<G, D>(a, blockIdx.x - a.nw);
      return;
    }
  }
  const int wa = blockIdx.x;
  const bool has_next = wa + 1 < a.nw;
  const int4 rec = reinterpret_cast<const int4*>(a.ws_merge)[wa];
  constexpr int kPer = (G * D + 255) / 256;
  float pm[3][kPer], pl[3][kPer], po[3][kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int idx = threadIdx.x + 256 * k;
    if (idx >= G * D) break;
    const int h = idx / D, d = idx % D;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      if (c == 2 && !has_next) break;
      const int64_t slot = static_cast<int64_t>(2 * wa + c) * G + h;  // c = 2: slot 0 of wa + 1
      pm[c][k] = a.ws_m[slot];
      pl[c][k] = a.ws_l[slot];
      po[c][k] = a.ws_o[slot * D + d];
    }
  }
  if (rec.x < 0) return;
  const int b = rec.x, g = rec.y, wb = rec.z, first = rec.w;
  float M[kPer], num[kPer], den[kPer];
  auto add = [&](int k, float m, float l, float o) {
    if (!(l > 0.f)) return;
    const float m_new = fmaxf(M[k], m);
    const float c = __builtin_amdgcn_exp2f(M[k] - m_new);  // 0 for the first piece
    const float f = l * __builtin_amdgcn_exp2f(m - m_new);
    den[k] = den[k] * c + f;
    num[k] = num[k] * c + f * o;
    M[k] = m_new;
  };
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    M[k] = -INFINITY;
    num[k] = 0.f;
    den[k] = 0.f;
    if (threadIdx.x + 256 * k >= G * D) continue;
    // a record always has wb > wa, so wa + 1 exists
    if (first == 0) {
      add(k, pm[0][k], pl[0][k], po[0][k]);
    } else {
      add(k, pm[1][k], pl[1][k], po[1][k]);
    }
    add(k, pm[2][k], pl[2][k], po[2][k]);
  }
  // segments longer than a span have pieces in more workgroups: request them 16 at a time
  constexpr int kBatch = 16;
  for (int v0 = wa + 2; v0 <= wb; v0 += kBatch) {
    float mm[kBatch][kPer], ll[kBatch][kPer], oo[kBatch][kPer];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int idx = threadIdx.x + 256 * k;
        ll[u][k] = 0.f;
        if (v0 + u <= wb && idx < G * D) {
          const int h = idx / D, d = idx % D;
          const int64_t slot = static_cast<int64_t>(2 * (v0 + u)) * G + h;
          mm[u][k] = a.ws_m[slot];
          ll[u][k] = a.ws_l[slot];
          oo[u][k] = a.ws_o[slot * D + d];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int k = 0; k < kPer; ++k) add(k, mm[u][k], ll[u][k], oo[u][k]);
  }
  if constexpr (kFold) {
    const int ps = prefix_tokens(a, b, min(max(a.seq_lens[b], 0), a.max_seq_len));
    const int np = prefix_parts_of(a, ps);
    for (int part = 0; part < np; ++part) {
      PrefixState st[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int idx = threadIdx.x + 256 * k;
        if (idx < G * D) {
          const int64_t row = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + idx / D;
          st[k] = load_prefix(a, row, part, idx % D);
        }
      }
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        if (threadIdx.x + 256 * k < G * D) fold_state(M[k], num[k], den[k], st[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int idx = threadIdx.x + 256 * k;
    if (idx >= G * D) break;
    const int h = idx / D, d = idx % D;
    const int64_t row = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + h;
    a.out[row * D + d] = den[k] > 0.f ? num[k] / den[k] : 0.f;
  }
}

// Output of segment (b, g) = seg / Hkv, seg % Hkv of a sequence with a shared prefix that the
// suffix decode did not cut across workgroups: its whole-segment state (sf_*, when it had pairs
// past the prefix) folded with the prefix parts in order.  Cut segments are written by their
// merge record; sequences without a prefix by the decode itself.
template <int G, int D>
__device__ void fold_segment(const DecodeArgs& a, int seg) {
  const int b = seg / a.Hkv, g = seg % a.Hkv;
  // what decides the work is requested in one round trip: length, prefix and the mark
  const int L = min(max(a.seq_lens[b], 0), a.max_seq_len);
  const int ps = prefix_tokens(a, b, L);
  const bool whole = a.sf_mark[seg] != 0;
  if (ps == 0) return;
  const int nb = (L + 2 * kBlockSize - 1) / (2 * kBlockSize) - ps / (2 * kBlockSize);
  if (nb > 0 && !whole) return;  // cut: its merge record writes it
  constexpr int kPer = (G * D + 255) / 256;
  const int np = prefix_parts_of(a, ps);
  // then every state this thread folds (the suffix's, each prefix part's), all requested
  // before the first is folded
  PrefixState sf[kPer], pf[kMaxPrefixParts][kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int idx = threadIdx.x + 256 * k;
    if (idx >= G * D) continue;
    const int64_t row = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + idx / D;
    if (whole) sf[k] = PrefixState{a.sf_m[row], a.sf_l[row], a.sf_o[row * D + idx % D]};
#pragma unroll
    for (int part = 0; part < kMaxPrefixParts; ++part)
      if (part < np) pf[part][k] = load_prefix(a, row, part, idx % D);
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int idx = threadIdx.x + 256 * k;
    if (idx >= G * D) break;
    float M = -INFINITY, num = 0.f, den = 0.f;
    if (whole) fold_state(M, num, den, sf[k]);
#pragma unroll
    for (int part = 0; part < kMaxPrefixParts; ++part)
      if (part < np) fold_state(M, num, den, pf[part][k]);
    const int64_t row = static_cast<int64_t>(b) * a.Hq + static_cast<int64_t>(g) * G + idx / D;
    a.out[row * D + idx % D] = den > 0.f ? num / den : 0.f;
  }
}

// Shared-prefix plan, one wave per sequence b.  b's group is the run of consecutive sequences
// around it, inside b's aligned window of 64, whose tables start with the same valid block (a
// sequence with no tokens has no group).  The reference is the group's longest member (the
// first on ties).  Every other member b shares with it the tokens below min(L_b, 16 k) where k
// counts the leading table entries that are equal and valid in both: those tokens sit in the
// same physical slots, so their keys and values are the same bytes.  The prefix pass takes b's
// shared tokens rounded down to a pair (pstart[b]); the reference's own prefix length, the
// largest of its members', is set by the prefix pass (ref_p).  The plan trusts nothing but the
// tables: any run of sequences gives the same attention as without it.
__global__ void __launch_bounds__(256) prefix_plan_kernel(DecodeArgs a) {
  const int lane = threadIdx.x % 64;
  const int b = blockIdx.x * 4 + static_cast<int>(threadIdx.x / 64);
  const int B = a.B, NB = a.NB;
  if (b >= B) return;
  const int w0 = b & ~63, pos = b - w0;
  const int i = w0 + lane;
  int key = -1, Li = 0;
  if (i < B) {
    Li = min(max(a.seq_lens[i], 0), a.max_seq_len);
    if (Li > 0 && a.max_blocks > 0) {
      const int t = a.tables[static_cast<int64_t>(i) * a.max_blocks];
      key = (t >= 0 && t < NB) ? t : -1;
    }
  }
  const int kb = __shfl(key, pos, 64);
  const uint64_t same = __ballot(i < B && key >= 0 && key == kb);
  for (int g = lane; g < a.Hkv; g += 64) a.sf_mark[static_cast<int64_t>(b) * a.Hkv + g] = 0;
  auto put = [&](int ps, int gr) {
    if (lane == 0) {
      a.pstart[b] = ps;
      a.grp_ref[b] = gr;
      a.ref_p[b] = 0;
    }
  };
  if (kb < 0) {
    put(0, -1);
    return;
  }
  // the maximal run of set bits of `same` through bit pos
  const uint64_t below = ~same & ((1ull << pos) - 1);
  const uint64_t above = ~same & ~((2ull << pos) - 1);  // bits above pos (none for pos 63)
  const int s = below ? 64 - __builtin_clzll(below) : 0;
  const int e = above ? __builtin_ctzll(above) : 64;
  if (e - s < 2) {
    put(0, -1);
    return;
  }
  const bool in = lane >= s && lane < e;
  int best = in ? Li : -1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) best = max(best, __shfl_xor(best, o, 64));
  const int ref = w0 + __builtin_ctzll(__ballot(in && Li == best));
  if (ref == b) {
    put(0, ref);
    return;
  }
  const int Lb = __shfl(Li, pos, 64);
  const int n = min((Lb + kBlockSize - 1) / kBlockSize, (best + kBlockSize - 1) / kBlockSize);
  const int32_t* tb = a.tables + static_cast<int64_t>(b) * a.max_blocks;
  const int32_t* tr = a.tables + static_cast<int64_t>(ref) * a.max_blocks;
  int k = n;  // leading entries equal and valid in both tables
  for (int c = 0; c < n; c += 64) {
    const int j = c + lane;
    bool diff = false;
    if (j < n) {
      const int x = tb[j], y = tr[j];
      diff = x != y || x < 0 || x >= NB;
    }
    const uint64_t dm = __ballot(diff);
    if (dm != 0) {
      k = c + __builtin_ctzll(dm);
      break;
    }
  }
  put(min(Lb, kBlockSize * k) & ~(2 * kBlockSize - 1), ref);
}

// Dynamic LDS of a balanced-schedule launch: the prefix sums cum_s[0..B] and cc_s[0..B], every
// entry the kernel touches (sizing it one short left cc_s[B] to the rounding of the allocation).
size_t balanced_lds(int32_t B) {
  return static_cast<size_t>(2 * static_cast<int64_t>(B) + 2) * sizeof(int32_t);
}

template <int G, int D, int kKV>
hipError_t launch_gd(const DecodeArgs& a, hipStream_t stream) {
  if (a.nw == 0 || G > kMaxBalancedGroup) {
    const dim3 grid(a.np_max, a.Hkv, a.B);
    hipLaunchKernelGGL((decode_mfma_kernel<G, D, kFixed, kKV>), grid, dim3(64 * kWavesOf<G, kKV>), 0, stream,
                       a);
    return hipGetLastError();
  }
  constexpr int Gb = G <= kMaxBalancedGroup ? G : kMaxBalancedGroup;  // never launched for G > 8
  const size_t lds = balanced_lds(a.B);
  hipLaunchKernelGGL((decode_mfma_kernel<Gb, D, kBalanced, kKV>), dim3(a.nw), dim3(64 * kWavesOf<Gb, kKV>),
                     lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((streamk_reduce_kernel<Gb, D, false>), dim3(a.nw), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Shared-prefix decode: plan, prefix pass (a.nw workgroups), suffix decode, merge.
template <int G, int D, int kKV>
hipError_t launch_gd_shared(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (G > kMaxBalancedGroup) {
    return hipErrorNotSupported;
  } else {
    hipLaunchKernelGGL(prefix_plan_kernel, dim3((a.B + 3) / 4), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds_pre = static_cast<size_t>(3 * a.pf_gmax + 1) * sizeof(int32_t);
    hipLaunchKernelGGL((decode_prefix_kernel<D, kKV>), dim3(a.nw), dim3(64 * kPrefixWaves),
                       lds_pre, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = balanced_lds(a.B);
    hipLaunchKernelGGL((decode_mfma_kernel<G, D, kSuffix, kKV>), dim3(a.nw), dim3(64 * kWavesOf<G, kKV>),
                       lds, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t grid = static_cast<int64_t>(a.nw) + static_cast<int64_t>(a.B) * a.Hkv;
    hipLaunchKernelGGL((streamk_reduce_kernel<G, D, true>), dim3(static_cast<uint32_t>(grid)),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
  }
}

template <int G, int kKV, bool kShared>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (kShared) {
    if (a.D == 128) return launch_gd_shared<G, 128, kKV>(a, stream);
    if (a.D == 64) return launch_gd_shared<G, 64, kKV>(a, stream);
  } else {
    if (a.D == 128) return launch_gd<G, 128, kKV>(a, stream);
    if (a.D == 64) return launch_gd<G, 64, kKV>(a, stream);
  }
  return hipErrorNotSupported;
}

template <int kKV, bool kShared = false>
hipError_t launch_kv(const DecodeArgs& a, hipStream_t stream) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_g<1, kKV, kShared>(a, stream);
    case 2: return launch_g<2, kKV, kShared>(a, stream);
    case 4: return launch_g<4, kKV, kShared>(a, stream);
    case 8: return launch_g<8, kKV, kShared>(a, stream);
    case 16: return launch_g<16, kKV, kShared>(a, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

int mfma_workgroups_per_cu() {
  static int cached = 0;
  if (cached == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<4, 128, kBalanced, kKvBf16>,
                                                     64 * kWavesOf<4, kKvBf16>, 1024) != hipSuccess ||
        n < 1)
      n = 1;
    cached = n;
  }
  return cached;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  if (kv_dtype == PA_I8) return launch_kv<kKvI8>(a, stream);
  if (kv_dtype == PA_I4) return launch_kv<kKvI4>(a, stream);
  return launch_kv<kKvBf16>(a, stream);
}

hipError_t launch_decode_shared_prefix(const DecodeArgs& a, int kv_dtype, hipStream_t stream) {
  if (kv_dtype == PA_I8) return launch_kv<kKvI8, true>(a, stream);
  if (kv_dtype == PA_I4) return launch_kv<kKvI4, true>(a, stream);
  return launch_kv<kKvBf16, true>(a, stream);
}

}  // namespace pa
