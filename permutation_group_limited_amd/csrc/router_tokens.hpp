// Group-limited top-k router: the per-token routing routine shared by the
// router kernel and the fused router + index kernel. The method and its
// mapping onto CDNA lanes are described in router.hip.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace moe {
namespace {

// Load EPL consecutive elements of dtype D (one vector load of EPL * size
// bytes when that is 4, 8 or a multiple of 16) and widen them to fp32.
template <typename D, int EPL>
__device__ __forceinline__ void load_row(float (&dst)[EPL],
                                         const typename D::storage* __restrict__ p) {
  constexpr int kBytes = EPL * D::kBytes;
  if constexpr (kBytes == 2) {
    dst[0] = D::widen_bits(static_cast<uint32_t>(p[0]));
  } else {
    constexpr int kWords = kBytes / 4;
    uint32_t w[kWords];
    if constexpr (kBytes % 16 == 0) {
#pragma unroll
      for (int q = 0; q < kWords; q += 4) {
        const u32x4 v = reinterpret_cast<const u32x4*>(p)[q / 4];
        w[q] = v.x;
        w[q + 1] = v.y;
        w[q + 2] = v.z;
        w[q + 3] = v.w;
      }
    } else if constexpr (kBytes == 8) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(p);
      w[0] = v.x;
      w[1] = v.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
    if constexpr (D::kBytes == 4) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) dst[i] = D::widen_bits(w[i]);
    } else {
#pragma unroll
      for (int q = 0; q < kWords; ++q) {
        dst[2 * q] = D::widen_bits(w[q] & 0xFFFFu);
        dst[2 * q + 1] = D::widen_hi(w[q]);
      }
    }
  }
}

// Cross-lane moves inside rows of 16 lanes. Every control used here reads a
// lane of the same row, so no lane is left without a source; the moves are
// written so that the compiler can fold them into the consuming VALU op.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, true));
}
// v_writelane_b32: `value` (wave-uniform) into lane `lane` of `v`, other
// lanes unchanged.
extern "C" __device__ int moe_amdgcn_writelane(int value, int lane, int v) __asm(
    "llvm.amdgcn.writelane.i32");
__device__ __forceinline__ uint32_t write_lane(uint32_t value, int lane, uint32_t v) {
  return static_cast<uint32_t>(
      moe_amdgcn_writelane(static_cast<int>(value), lane, static_cast<int>(v)));
}

constexpr int kXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kMirror = 0x140;      // lane i <-> 15-i within each row

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// Merge the (largest, second largest) pair of order-preserving keys of this
// lane with the pair of the lane that holds a disjoint set of experts.
__device__ __forceinline__ void merge_top2_keys(uint32_t& m1, uint32_t& m2, uint32_t o1,
                                                uint32_t o2) {
  m2 = umax(umin(m1, o1), umax(m2, o2));
  m1 = umax(m1, o1);
}

// Top-2 keys over groups of `lpg` adjacent lanes (lpg a power of two,
// groups aligned). Each step pairs lanes whose partial results cover
// disjoint experts: xor 1 and xor 2 (quad_perm), then the mirrored half-row
// and row (every lane of a quad, resp. half-row, already holds the same
// pair), then xor 16 (ds_swizzle) and xor 32 (ds_bpermute).
__device__ __forceinline__ void group_top2_keys(uint32_t& m1, uint32_t& m2, int lpg) {
  if (lpg >= 2) merge_top2_keys(m1, m2, dpp_u<kXor1>(m1), dpp_u<kXor1>(m2));
  if (lpg >= 4) merge_top2_keys(m1, m2, dpp_u<kXor2>(m1), dpp_u<kXor2>(m2));
  if (lpg >= 8) merge_top2_keys(m1, m2, dpp_u<kHalfMirror>(m1), dpp_u<kHalfMirror>(m2));
  if (lpg >= 16) merge_top2_keys(m1, m2, dpp_u<kMirror>(m1), dpp_u<kMirror>(m2));
  if (lpg >= 32) {
    const uint32_t o1 =
        static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(m1), 0x401F));
    const uint32_t o2 =
        static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(m2), 0x401F));
    merge_top2_keys(m1, m2, o1, o2);
  }
  if (lpg >= 64)
    merge_top2_keys(m1, m2, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m1), 32, kWave)),
                    static_cast<uint32_t>(__shfl_xor(static_cast<int>(m2), 32, kWave)));
}

// Sum over groups of `lpg` adjacent lanes, same lane pairing as group_top2_keys.
__device__ __forceinline__ int group_sum(int x, int lpg) {
  if (lpg >= 2) x += __builtin_amdgcn_mov_dpp(x, kXor1, 0xF, 0xF, true);
  if (lpg >= 4) x += __builtin_amdgcn_mov_dpp(x, kXor2, 0xF, 0xF, true);
  if (lpg >= 8) x += __builtin_amdgcn_mov_dpp(x, kHalfMirror, 0xF, 0xF, true);
  if (lpg >= 16) x += __builtin_amdgcn_mov_dpp(x, kMirror, 0xF, 0xF, true);
  if (lpg >= 32) x += __builtin_amdgcn_ds_swizzle(x, 0x401F);
  if (lpg >= 64) x += __shfl_xor(x, 32, kWave);
  return x;
}

// Maximum of v over the token's LPT lanes, returned to every lane of the
// segment: xor 1 and xor 2 inside quads, mirrored half-rows and rows (by
// then each quad, resp. half-row, is uniform), xor 16 by ds_swizzle; for a
// full wave, the row maxima are carried across rows by the row_bcast:15 and
// row_bcast:31 moves (lane 63 ends with the wave maximum) and read back
// with one v_readlane.
template <int LPT>
__device__ __forceinline__ uint32_t segment_max(uint32_t v) {
  if (LPT >= 2) v = umax(v, dpp_u<kXor1>(v));
  if (LPT >= 4) v = umax(v, dpp_u<kXor2>(v));
  if (LPT >= 8) v = umax(v, dpp_u<kHalfMirror>(v));
  if (LPT >= 16) v = umax(v, dpp_u<kMirror>(v));
  if constexpr (LPT == 32) {
    v = umax(v, static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x401F)));
  } else if constexpr (LPT == kWave) {
    // rows outside the row mask take 0, the identity of the maximum
    v = umax(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v),
                                                                  kRowBcast15, 0xA, 0xF, false)));
    v = umax(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v),
                                                                  kRowBcast31, 0xC, 0xF, false)));
    v = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), kWave - 1));
  }
  return v;
}

// One compare-exchange of the descending sort below: position a (< b)
// keeps the larger of the two (key, rel) pairs, ordered as the 64-bit
// values key << 32 | rel. One 64-bit compare and four 32-bit selects (on
// the packed values the compiler would form a maximum and a minimum, with a
// compare each).
template <int EPL>
__device__ __forceinline__ void compare_exchange(uint32_t (&key)[EPL], uint32_t (&rel)[EPL], int a,
                                                 int b) {
  const uint64_t va = (static_cast<uint64_t>(key[a]) << 32) | rel[a];
  const uint64_t vb = (static_cast<uint64_t>(key[b]) << 32) | rel[b];
  const bool sw = va < vb;
  const uint32_t ka = key[a], kb = key[b], ra = rel[a], rb = rel[b];
  key[a] = sw ? kb : ka;
  key[b] = sw ? ka : kb;
  rel[a] = sw ? rb : ra;
  rel[b] = sw ? ra : rb;
}

// Descending sort of EPL (a power of two) pairs with distinct packed values
// by Batcher's odd-even merge sort (5, 19 and 63 compare-exchanges for 4, 8
// and 16 elements, against 6, 24 and 80 for a bitonic network), unrolled at
// compile time.
template <int EPL>
__device__ __forceinline__ void sort_desc_pairs(uint32_t (&key)[EPL], uint32_t (&rel)[EPL]) {
#pragma unroll
  for (int p = 1; p < EPL; p <<= 1) {
#pragma unroll
    for (int k = p; k >= 1; k >>= 1) {
#pragma unroll
      for (int j = k % p; j + k < EPL; j += 2 * k) {
#pragma unroll
        for (int i = 0; i < k; ++i) {
          if (i < EPL - j - k && (i + j) / (2 * p) == (i + j + k) / (2 * p))
            compare_exchange<EPL>(key, rel, i + j, i + j + k);
        }
      }
    }
  }
}

// Score functions applied to logits before routing (the page's optional
// scores_input_fn): evaluated in binary64, rounded once to binary32.
constexpr int kScoreLoad = 0;
constexpr int kScoreSigmoid = 1;
constexpr int kScoreSoftmax = 2;

// 1 / n! rounded once (n! is exact in binary64 for n <= 18); folded by the
// compiler, whose constant arithmetic rounds to nearest even.
constexpr double inv_factorial(int n) {
  double f = 1.0;
  for (int i = 2; i <= n; ++i) f *= static_cast<double>(i);
  return 1.0 / f;
}

// 2^n for -1022 <= n <= 1023, built from its exponent field.
__device__ __forceinline__ double pow2_normal(int n) {
  return __longlong_as_double(static_cast<long long>(n + 1023) << 52);
}

// Binary64 exponential by a fixed published method, so that its bits do
// not depend on a math library: Cody and Waite's reduction (Software Manual
// for the Elementary Functions, 1980) x = k ln2 + r, k = round-to-even of
// x / ln2, r = (x - k LN2_HI) - k LN2_LO with ln2 split into its nearest
// binary64 value and the nearest binary64 value of the remainder, each
// step one fused multiply-add; exp(r) as its Taylor polynomial up to
// r^13 / 13! by Horner's rule with fused multiply-adds; then 2^k applied as
// two exact powers of two, 2^(k/2) and 2^(k - k/2), so that only the last
// product rounds. 0 below -745.2, +inf above 709.78, NaN kept.
__device__ __forceinline__ double exp_f64(double x) {
  constexpr double kLn2Hi = 0x1.62e42fefa39efp-1;
  constexpr double kLn2Lo = 0x1.abc9e3b39803fp-56;
  constexpr double kInvLn2 = 0x1.71547652b82fep+0;
  const double xc = __builtin_fmin(__builtin_fmax(x, -745.2), 709.78);
  const double kd = __builtin_rint(xc * kInvLn2);
  double r = __builtin_fma(-kd, kLn2Hi, xc);
  r = __builtin_fma(-kd, kLn2Lo, r);
  double p = inv_factorial(13);
#pragma unroll
  for (int n = 12; n >= 0; --n) p = __builtin_fma(p, r, inv_factorial(n));
  const int k = static_cast<int>(kd);
  const int k1 = k / 2;
  double y = (p * pow2_normal(k1)) * pow2_normal(k - k1);
  y = x > 709.78 ? __builtin_inf() : y;
  y = x < -745.2 ? 0.0 : y;
  return x != x ? x : y;
}

__device__ __forceinline__ float sigmoid_f64(float x) {
  return static_cast<float>(1.0 / (1.0 + exp_f64(-static_cast<double>(x))));
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// Pairwise sum of the token's E' = EPL * LPT values in expert order: a
// balanced tree inside the lane's EPL consecutive experts, then the xor
// butterfly over the token's LPT lanes, which continues the same tree (step
// `off` adds the partial sums of the neighbouring blocks of off lanes; each
// add is commutative, so every lane of the segment ends with the root).
template <int EPL, int LPT>
__device__ __forceinline__ double pairwise_sum_f64(const double (&v)[EPL]) {
  double t[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) t[i] = v[i];
#pragma unroll
  for (int w = 1; w < EPL; w *= 2) {
#pragma unroll
    for (int i = 0; i + w < EPL; i += 2 * w) t[i] = t[i] + t[i + w];
  }
  double s = t[0];
#pragma unroll
  for (int off = 1; off < LPT; off <<= 1) s += __shfl_xor(s, off, kWave);
  return s;
}

// Routes the tokens of workgroup `block` (WPB waves of kWave / LPT tokens
// each) and writes their expert_indices and expert_weights rows. A
// workgroup past the last token (grid padding) returns at once.
//
// GEN = false: E = EPL * LPT, a power of two, and groups of S = E / n_groups
// experts cover whole lanes (S >= EPL), so the group stage is a lane
// butterfly. GEN = true: any E_rt <= EPL * 64 (one wave per token, LPT =
// 64); lane l holds experts [l * EPL, l * EPL + EPL) of which those >= E_rt
// are absent, and the group stage goes through LDS: the biased scores are
// staged per wave, lane g scans group g, and the kept groups form a mask.
template <typename DS, typename DB, int EPL, int LPT, int FN, int WPB, bool GEN = false>
__device__ __forceinline__ void route_tokens(
    int32_t* __restrict__ out_idx, typename DS::storage* __restrict__ out_w,
    const typename DS::storage* __restrict__ scores, const typename DB::storage* __restrict__ bias,
    int64_t T, int32_t K, int32_t n_groups, int32_t topk_group, int32_t norm_weights,
    float scale, int32_t mode, uint32_t block, int32_t E_rt = 0,
    RouterHist hist = RouterHist{nullptr, 0u}) {
  static_assert(!GEN || LPT == kWave, "the general-E form routes one token per wave");
  const int32_t E = GEN ? E_rt : EPL * LPT;
  constexpr int TPW = kWave / LPT;  // tokens per wave
  const int64_t t0 = static_cast<int64_t>(block) * WPB * TPW;  // first token
  if (t0 >= T) return;  // uniform over the workgroup, before any barrier
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int sub = lane & (LPT - 1);
  const int tok_lane0 = lane & ~(LPT - 1);
  const int64_t t = t0 + static_cast<int64_t>(wave) * TPW + lane / LPT;
  const bool tok_ok = t < T;
  const int e0 = sub * EPL;
  const uint64_t segmask =
      (LPT == kWave) ? ~0ull : (((1ull << (LPT & 63)) - 1ull) << tok_lane0);

  float s[EPL], bi[EPL], b[EPL];
  bool present[EPL];  // expert e0 + i exists (always, unless GEN)
#pragma unroll
  for (int i = 0; i < EPL; ++i) present[i] = !GEN || e0 + i < E;
  if constexpr (GEN) {
    // rows of E elements need not be 16-byte multiples: element loads
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      s[i] = (tok_ok && present[i]) ? load_f32<DS>(scores, t * E + e0 + i) : 0.0f;
      bi[i] = present[i] ? load_f32<DB>(bias, e0 + i) : 0.0f;
    }
  } else {
    if (tok_ok) {
      load_row<DS, EPL>(s, scores + t * E + e0);
    } else {
#pragma unroll
      for (int i = 0; i < EPL; ++i) s[i] = 0.0f;
    }
    load_row<DB, EPL>(bi, bias + e0);
  }
  // scores from logits (FN != kScoreLoad)
  double sm_max = 0.0, sm_sum = 1.0;
  if constexpr (FN == kScoreSigmoid) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) s[i] = sigmoid_f64(s[i]);
  } else if constexpr (FN == kScoreSoftmax) {
    uint32_t km = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) km = present[i] ? umax(km, ordered_key(s[i])) : km;
    sm_max = static_cast<double>(key_to_float(segment_max<LPT>(km)));
    double ex[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      ex[i] = present[i] ? exp_f64(static_cast<double>(s[i]) - sm_max) : 0.0;
    sm_sum = pairwise_sum_f64<EPL, LPT>(ex);
#pragma unroll
    for (int i = 0; i < EPL; ++i) s[i] = static_cast<float>(ex[i] / sm_sum);
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) b[i] = s[i] + bi[i];
  // order-preserving keys of the biased scores (group stage and top-K)
  uint32_t bk[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) bk[i] = ordered_key(b[i]);

  // ---- group stage: keep the best topk_group groups ------------------------
  bool kept[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) kept[i] = true;
  if constexpr (GEN) {
    if (topk_group < n_groups) {
      // Stage the token's biased scores in this wave's LDS row; LDS
      // operations of one wave take effect in order, so its lanes may read
      // each other's stores after a wave-level scheduling barrier.
      __shared__ float staged[WPB][EPL * kWave];
      float* row = staged[wave];
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (present[i]) row[e0 + i] = b[i];
      __builtin_amdgcn_wave_barrier();
      const int S = E / n_groups;
      float gs = -__builtin_inff();
      if (lane < n_groups) {
        float m1 = -__builtin_inff(), m2 = -__builtin_inff();
        for (int j = lane * S; j < lane * S + S; ++j) {
          const float v = row[j];
          m2 = fmaxf(m2, fminf(m1, v));
          m1 = fmaxf(m1, v);
        }
        gs = (mode == MOE_GROUP_MAX || S == 1) ? m1 : m1 + m2;
      }
      // rank of group `lane` = groups that beat it (ties: lower index)
      int beats = 0;
      for (int j = 0; j < n_groups; ++j) {
        const float o = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gs), j));
        beats += (o > gs) || (o == gs && j < lane);
      }
      const uint64_t keep = __ballot(lane < n_groups && beats < topk_group);
      // group of expert e = floor((e + 1/2) / S), exact in binary32 for
      // e, S < 2^10: the quotient stays at least 1/(2S) from an integer
      const float inv_s = 1.0f / static_cast<float>(S);
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int g = static_cast<int>((static_cast<float>(e0 + i) + 0.5f) * inv_s);
        kept[i] = present[i] && ((keep >> (g & 63)) & 1ull) != 0;
      }
    }
  } else if (topk_group < n_groups) {
    // E, n_groups and EPL are powers of two: shifts, not divisions
    const int lg_groups = __builtin_ctz(static_cast<uint32_t>(n_groups));
    const int S = E >> lg_groups;
    const int LPG = S / EPL;  // lanes per group, a power of two
    const int lg_lpg = __builtin_ctz(static_cast<uint32_t>(LPG));
    // top-2 of the group on the order-preserving keys (exact integer max /
    // min; key 0 lies below every finite score), then back to binary32 for
    // the group score: the same values as the scores themselves (-0 reads
    // back as +0, which compares equal)
    uint32_t k1 = 0u, k2 = 0u;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      k2 = umax(umin(k1, k2), umin(umax(k1, k2), bk[i]));  // median of three: k1 >= k2
      k1 = umax(k1, bk[i]);
    }
    group_top2_keys(k1, k2, LPG);
    const float g1 = key_to_float(k1);
    const float gs = (mode == MOE_GROUP_MAX || S == 1) ? g1 : g1 + key_to_float(k2);
    // rank of my group = groups that beat it; the LPG lanes of a group split
    // the comparisons (lane q of the group tests groups q, q + LPG, ...) and
    // add their counts
    const int my_g = sub >> lg_lpg;
    int beats = 0;
    for (int j = sub & (LPG - 1); j < n_groups; j += LPG) {
      const float o = __shfl(gs, tok_lane0 + j * LPG, kWave);
      beats += (o > gs) || (o == gs && j < my_g);
    }
    const bool k_lane = group_sum(beats, LPG) < topk_group;
#pragma unroll
    for (int i = 0; i < EPL; ++i) kept[i] = k_lane;
  }

  // ---- top-K: K rounds of segment max over the lanes' sorted heads ---------
  // Keys preserve the order of the biased scores (0 = not a candidate). Each
  // lane sorts its EPL elements by (key desc, element asc), packed as
  // key << 32 | (EPL - 1 - element) so that all packed values of a lane are
  // distinct. A round takes the segment maximum of the lane heads' keys;
  // among lanes whose head key equals it the lowest lane wins, which is the
  // lowest expert id because lanes hold ascending, disjoint id ranges. The
  // winner pops its head. Round k yields slot k.
  uint32_t kv[EPL], rel[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    kv[i] = (tok_ok && kept[i] && present[i]) ? bk[i] : 0u;
    rel[i] = static_cast<uint32_t>(EPL - 1 - i);
  }
  sort_desc_pairs<EPL>(kv, rel);
  // The sorted list as keys plus one word of 4-bit element indices (element
  // of position i in bits 4i..4i+3): a pop shifts the keys by one register
  // and the index word by 4 bits (two tokens per wave: see below).
  using IdxWord = typename std::conditional<(EPL > 8), uint64_t, uint32_t>::type;
  IdxWord iw = 0;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    iw |= static_cast<IdxWord>((EPL - 1) - rel[i]) << (4 * i);

  // LDS scratch of each wave (power-of-two layouts with several experts per
  // lane): its sorted lists during the top-K of two tokens per wave, then
  // its scores for the weights. One word where unused.
  // Scores are stored with a lane stride of EPL + 4 words from 8 experts a
  // lane up: the 16-byte stores of 8 consecutive lanes then cover all 32
  // banks once (a stride of EPL words would put two lanes on each bank).
  constexpr int kScoreStride = EPL >= 8 ? EPL + 4 : EPL;
  constexpr int kScratchWords =
      (!GEN && EPL > 1) ? ((EPL + 1) > kScoreStride ? EPL + 1 : kScoreStride) * kWave : 1;
  __shared__ __align__(16) uint32_t wave_lds[WPB][kScratchWords];
  uint32_t my_id = 0;
  if constexpr (LPT == kWave / 2 && EPL > 1) {
    // Two tokens per wave (K <= 32, checked by the host): each half's
    // winner is the lowest set bit of its half of the ballot (every half
    // has one: its maximum is one of its heads), so both winners, their
    // elements and the two slot ids are wave-uniform; slot k of the tokens
    // goes to lanes k and 32 + k. The sorted lists sit in this wave's LDS
    // scratch, position p of lane l at word p * 64 + l (position EPL holds
    // the empty key): a pop advances the lane's position and reads its next
    // head, instead of shifting EPL registers.
#pragma unroll
    for (int p = 0; p < EPL; ++p) wave_lds[wave][p * kWave + lane] = kv[p];
    wave_lds[wave][EPL * kWave + lane] = 0u;
    __builtin_amdgcn_wave_barrier();
    static_assert(EPL <= 8, "two tokens per wave take E <= 256: 4-bit indices in one word");
    uint32_t pos = 0u;
    for (int k = 0; k < K; ++k) {
      // A lane is popped at most EPL times while its token has candidates
      // left; a half without a valid token (the ragged end of the batch)
      // keeps popping its lowest lane, which stays on the empty row.
      const uint32_t at = pos < static_cast<uint32_t>(EPL) ? pos : static_cast<uint32_t>(EPL);
      const uint32_t head = wave_lds[wave][at * kWave + lane];
      const uint64_t top = __ballot(head == segment_max<LPT>(head));
      const int w_lo = __builtin_ctz(static_cast<uint32_t>(top));
      const int w_hi = 32 + __builtin_ctz(static_cast<uint32_t>(top >> 32));
      const int e4 = static_cast<int>(__builtin_amdgcn_ubfe(iw, 4u * at, 4u));  // past EPL: unused
      const uint32_t el_lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(e4, w_lo));
      const uint32_t el_hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(e4, w_hi));
      my_id = write_lane(static_cast<uint32_t>(w_lo * EPL) + el_lo, k, my_id);
      my_id = write_lane(static_cast<uint32_t>((w_hi - 32) * EPL) + el_hi, 32 + k, my_id);
      // the two winners advance (a uniform lane mask, no per-lane compares)
      pos += __builtin_amdgcn_inverse_ballot_w64((1ull << w_lo) | (1ull << w_hi)) ? 1u : 0u;
    }
    __builtin_amdgcn_wave_barrier();  // the scratch is rewritten with the scores below
  } else {
    for (int k = 0; k < K; ++k) {
      const uint32_t head = kv[0];
      const uint64_t top = __ballot(head == segment_max<LPT>(head));
      bool pop;
      if constexpr (LPT == kWave) {
        // the winner and its element are wave-uniform; slot k goes to lane k
        const int win = __builtin_ctzll(static_cast<unsigned long long>(top));
        const uint32_t elem =
            static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(iw & 0xFu), win));
        my_id = write_lane(static_cast<uint32_t>(win * EPL) + elem, k, my_id);
        pop = lane == win;
      } else {
        // one expert per lane, several tokens per wave
        static_assert(EPL == 1, "several tokens per wave need one expert per lane or two tokens");
        const int win = __builtin_ctzll(static_cast<unsigned long long>(top & segmask));
        if (sub == k) my_id = static_cast<uint32_t>(win - tok_lane0);
        pop = lane == win;
      }
      if (pop) {
#pragma unroll
        for (int i = 0; i + 1 < EPL; ++i) kv[i] = kv[i + 1];
        kv[EPL - 1] = 0u;
        iw >>= 4;
      }
    }
  }

  // ---- weights from the unbiased scores -----------------------------------
  // Slot `sub`'s score is still in the registers of the lane that holds
  // its expert. Powers of two with several experts per lane: every lane
  // stores its scores in this wave's LDS scratch and each slot reads its
  // own, without reading the input again
  // (LDS operations of one wave take effect in order). Otherwise one
  // ds_bpermute per element register.
  const bool slot = tok_ok && sub < K;
  if (my_id >= static_cast<uint32_t>(E)) my_id = 0;  // unreachable with finite scores
  float u = 0.0f;
  if constexpr (!GEN && EPL > 1) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) wave_lds[wave][lane * kScoreStride + i] = __float_as_uint(s[i]);
    __builtin_amdgcn_wave_barrier();
    u = __uint_as_float(
        wave_lds[wave][(tok_lane0 + static_cast<int>(my_id) / EPL) * kScoreStride + my_id % EPL]);
  } else {
    const int owner = tok_lane0 + static_cast<int>(my_id / EPL);
    const int elem = static_cast<int>(my_id % EPL);
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float v = __shfl(s[i], owner, kWave);
      u = (i == elem) ? v : u;
    }
  }
  // Normalise and scale in binary64, rounded once to binary32: the sum of
  // the K selected scores in slot order (each widened exactly), a correctly
  // rounded divide, then the product with the scaling factor.
  double wd = static_cast<double>(u);
  if (norm_weights) {
    double d = 0.0;
    if constexpr (LPT == kWave) {
      for (int q = 0; q < K; ++q)
        d += static_cast<double>(
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, u), q)));
    } else {
      for (int q = 0; q < K; ++q) d += static_cast<double>(__shfl(u, tok_lane0 + q, kWave));
    }
    wd = wd / d;
  }
  const float w = static_cast<float>(wd * static_cast<double>(scale));
  if (slot) {
    out_idx[t * K + sub] = static_cast<int32_t>(my_id);
    out_w[t * K + sub] = to_storage<DS>(w);
  }
  // Histogram of the index step: one counter per (chunk, expert), summed
  // with relaxed atomics (integer sums do not depend on their order). Same-
  // address device-scope atomics serialise, and a popular expert appears in
  // most tokens, so the workgroup first merges its slots: each slot's key
  // (chunk offset from the workgroup's first chunk, expert) goes to LDS in
  // slot order, then wave 0 groups equal keys (peer masks from ballots) and
  // one lane per distinct key issues the global add. A workgroup holds at
  // most 256 slots and a chunk at least 256, so the offset is 0 or 1.
  if (hist.fine != nullptr) {  // uniform: ranked form of the index step
    // Each slot's expert goes to LDS in slot order; wave 0 then walks the
    // workgroup's slots 64 at a time in that order, with a running count
    // per expert in LDS: a slot's rank is the count before its round plus
    // its peers in lower lanes (ballot peer masks), the lowest peer adds the
    // round's count, to the running count and (several chunks) to its
    // chunk's row of the counts (relaxed atomics: integer sums do not depend
    // on their order). Stores (rank << 10) | expert for the slot, then the
    // workgroup's row of counts.
    constexpr int kThreads = WPB * kWave;
    __shared__ uint32_t slot_expert[kThreads];
    __shared__ uint32_t running[kRankedMaxExperts];
    const int64_t t1 = (t0 + WPB * TPW < T) ? t0 + WPB * TPW : T;
    const int nslots = static_cast<int>((t1 - t0) * K);
    if (slot) slot_expert[(t - t0) * K + sub] = my_id;
    __syncthreads();
    if (wave == 0) {
      for (int x = lane; x < E; x += kWave) running[x] = 0u;
      __builtin_amdgcn_wave_barrier();
      int nb = 0;
      while ((1 << nb) < E) ++nb;
      uint32_t* packed = hist.packed + static_cast<uint64_t>(t0) * K;
      const int32_t stride = ranked_stride(E);
      uint32_t* crow = hist.counts == nullptr
                           ? nullptr
                           : hist.counts + static_cast<uint64_t>(block / hist.rows_per_chunk) *
                                               stride;
      for (int r = 0; r < nslots; r += kWave) {
        const bool ok = r + lane < nslots;
        const uint32_t e = ok ? slot_expert[r + lane] : 0u;
        const uint64_t peers = match_any(e, nb, __ballot(ok));
        const uint32_t before = ok ? running[e] : 0u;
        __builtin_amdgcn_wave_barrier();  // every lane reads before the update
        if (ok && (__ffsll(static_cast<unsigned long long>(peers)) - 1) == lane) {
          const uint32_t n = static_cast<uint32_t>(__popcll(peers));
          running[e] = before + n;
          if (crow != nullptr)  // one lane per distinct expert of the round
            __hip_atomic_fetch_add(crow + e, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (ok) packed[r + lane] = ((before + popc_below(peers)) << kPackedExpertBits) | e;
        __builtin_amdgcn_wave_barrier();
      }
      uint32_t* row = hist.fine + static_cast<uint64_t>(block) * stride;
      for (int x = lane; x < stride; x += kWave) row[x] = x < E ? running[x] : 0u;
    }
  } else if (hist.counts != nullptr) {  // uniform: chunked form
    constexpr int kThreads = WPB * kWave;
    __shared__ uint32_t keys[kThreads];
    const int64_t t1 = (t0 + WPB * TPW < T) ? t0 + WPB * TPW : T;
    const int nslots = static_cast<int>((t1 - t0) * K);
    const uint32_t c0 = static_cast<uint32_t>((t0 * K) / hist.chunk);
    if (slot) {
      const uint32_t dc = static_cast<uint32_t>(t * K + sub) / hist.chunk - c0;
      if (dc < 2u) {
        keys[(t - t0) * K + sub] = (dc << 10) | my_id;
      } else {  // not reached with the launch shapes used; kept correct anyway
        keys[(t - t0) * K + sub] = 0xFFFFFFFFu;
        __hip_atomic_fetch_add(hist.counts + static_cast<size_t>(c0 + dc) * E + my_id, 1u,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (wave == 0) {
      for (int r = 0; r < nslots; r += kWave) {
        const uint32_t key =
            r + lane < nslots ? keys[r + lane] : 0xFFFFFFFFu;
        const bool ok = key != 0xFFFFFFFFu;
        const uint64_t peers = match_any(key, 11, __ballot(ok));
        if (ok && (__ffsll(static_cast<unsigned long long>(peers)) - 1) == lane)
          __hip_atomic_fetch_add(
              hist.counts + static_cast<size_t>(c0 + (key >> 10)) * E + (key & 1023u),
              static_cast<uint32_t>(__popcll(peers)), __ATOMIC_RELAXED,
              __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}


// Picks the instance for (score dtype, bias dtype, score function, E) and
// calls L<DS, DB, EPL, LPT, FN>::run(args...). E = LPT * EPL: for E >= 64 a
// token fills a wave (LPT = 64), below that it takes E lanes.
template <template <typename, typename, int, int, int> class L, typename DS, typename DB, int FN,
          typename... A>
moe_status_t dispatch_router_e(int32_t E, A... args) {
  switch (E) {
    case 1: return L<DS, DB, 1, 1, FN>::run(args...);
    case 2: return L<DS, DB, 1, 2, FN>::run(args...);
    case 4: return L<DS, DB, 1, 4, FN>::run(args...);
    case 8: return L<DS, DB, 1, 8, FN>::run(args...);
    case 16: return L<DS, DB, 1, 16, FN>::run(args...);
    case 32: return L<DS, DB, 1, 32, FN>::run(args...);
    case 64: return L<DS, DB, 1, 64, FN>::run(args...);
    case 128: return L<DS, DB, 2, 64, FN>::run(args...);
    case 256: return L<DS, DB, 4, 64, FN>::run(args...);
    case 512: return L<DS, DB, 8, 64, FN>::run(args...);
    case 1024: return L<DS, DB, 16, 64, FN>::run(args...);
    default: return MOE_ERR_UNSUPPORTED;
  }
}

template <template <typename, typename, int, int, int> class L, typename DS, typename DB,
          typename... A>
moe_status_t dispatch_router_fn(int32_t fn, int32_t E, A... args) {
  switch (fn) {
    case kScoreLoad: return dispatch_router_e<L, DS, DB, kScoreLoad>(E, args...);
    case kScoreSigmoid: return dispatch_router_e<L, DS, DB, kScoreSigmoid>(E, args...);
    case kScoreSoftmax: return dispatch_router_e<L, DS, DB, kScoreSoftmax>(E, args...);
    default: return MOE_ERR_INVALID_ARG;
  }
}

// Score / bias dtype pairs with an instance: equal, or an fp32 bias.
template <template <typename, typename, int, int, int> class L, typename... A>
moe_status_t dispatch_router(moe_dtype_t sd, moe_dtype_t bd, int32_t fn, int32_t E, A... args) {
  if (sd == MOE_DTYPE_F32 && bd == MOE_DTYPE_F32)
    return dispatch_router_fn<L, DF32, DF32>(fn, E, args...);
  if (sd == MOE_DTYPE_BF16 && bd == MOE_DTYPE_BF16)
    return dispatch_router_fn<L, DBF16, DBF16>(fn, E, args...);
  if (sd == MOE_DTYPE_BF16 && bd == MOE_DTYPE_F32)
    return dispatch_router_fn<L, DBF16, DF32>(fn, E, args...);
  if (sd == MOE_DTYPE_F16 && bd == MOE_DTYPE_F16)
    return dispatch_router_fn<L, DF16, DF16>(fn, E, args...);
  if (sd == MOE_DTYPE_F16 && bd == MOE_DTYPE_F32)
    return dispatch_router_fn<L, DF16, DF32>(fn, E, args...);
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace moe
