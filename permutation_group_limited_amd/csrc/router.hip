// Group-limited top-k router for gfx950.
//
// Computes what the group_limited_router_kernel page (Modular MAX Mojo API,
// nn/moe) describes: biased scores for selection, the best topk_group of
// n_groups expert groups, the top-K experts inside them, and weights from
// the unbiased scores, optionally normalised, times routed_scaling_factor.
//
// Mapping (CDNA-specific; the page's one-thread-per-expert block is not
// used): a token is owned by LPT consecutive lanes of a wave64, each lane
// holding EPL consecutive experts (E = LPT * EPL). For E >= 64 a token fills
// a whole wave (E = 256: 4 experts = one 16-byte load per lane); for E < 64
// several tokens share a wave. A group of S = E / n_groups experts is then
// LPG = S / EPL adjacent lanes, so group top-2 is a log2(LPG)-step xor
// butterfly; the top-K is K rounds of a lexicographic argmax over the token's
// lanes on 64-bit keys (ordered score, inverted expert id), which breaks
// ties towards the lower expert id by construction.
#include "common.hpp"

namespace moe {
namespace {

template <int EPL>
__device__ __forceinline__ void load_row(float (&dst)[EPL], const float* __restrict__ p) {
  if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int i = 0; i < EPL; i += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p + i);
      dst[i] = v.x;
      dst[i + 1] = v.y;
      dst[i + 2] = v.z;
      dst[i + 3] = v.w;
    }
  } else if constexpr (EPL == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    dst[0] = v.x;
    dst[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) dst[i] = p[i];
  }
}

template <int EPL, int LPT>
__global__ __launch_bounds__(kBlock) void router_kernel(
    int32_t* __restrict__ out_idx, float* __restrict__ out_w, const float* __restrict__ scores,
    const float* __restrict__ bias, int64_t T, int32_t K, int32_t n_groups, int32_t topk_group,
    int32_t norm_weights, float scale, int32_t mode) {
  constexpr int E = EPL * LPT;
  constexpr int TPW = kWave / LPT;  // tokens per wave
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int sub = lane & (LPT - 1);
  const int tok_lane0 = lane & ~(LPT - 1);
  const int64_t t =
      (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave) * TPW + lane / LPT;
  const bool tok_ok = t < T;
  const int e0 = sub * EPL;

  float s[EPL], bi[EPL], b[EPL];
  if (tok_ok) {
    load_row<EPL>(s, scores + t * E + e0);
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) s[i] = 0.0f;
  }
  load_row<EPL>(bi, bias + e0);
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    b[i] = s[i] + bi[i];
    if (b[i] == 0.0f) b[i] = 0.0f;  // one zero: -0 and +0 tie anyway
  }

  // ---- group stage: keep the best topk_group groups ------------------------
  bool kept = true;
  if (topk_group < n_groups) {
    const int S = E / n_groups;
    const int LPG = S / EPL;  // lanes per group, a power of two
    float m1 = -__builtin_inff(), m2 = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (b[i] > m1) {
        m2 = m1;
        m1 = b[i];
      } else if (b[i] > m2) {
        m2 = b[i];
      }
    }
    for (int off = 1; off < LPG; off <<= 1) {
      const float o1 = __shfl_xor(m1, off, kWave);
      const float o2 = __shfl_xor(m2, off, kWave);
      const float n2 = fmaxf(fminf(m1, o1), fmaxf(m2, o2));
      m1 = fmaxf(m1, o1);
      m2 = n2;
    }
    const float gs = (mode == MOE_GROUP_MAX || S == 1) ? m1 : m1 + m2;
    const int my_g = sub / LPG;
    int rank = 0;
    for (int g = 0; g < n_groups; ++g) {
      const float o = __shfl(gs, tok_lane0 + g * LPG, kWave);
      rank += (o > gs) || (o == gs && g < my_g);
    }
    kept = rank < topk_group;
  }

  // ---- top-K over the surviving experts -----------------------------------
  // key = ordered(b) << 32 | ~e; 0 marks "not a candidate" (every finite
  // score has ordered key >= 0x00800000).
  uint64_t keys[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    keys[i] = (tok_ok && kept)
                  ? (static_cast<uint64_t>(ordered_key(b[i])) << 32) |
                        static_cast<uint32_t>(~static_cast<uint32_t>(e0 + i))
                  : 0ull;
  }
  // lane-local descending sort (EPL <= 16, insertion network, unrolled)
#pragma unroll
  for (int i = 1; i < EPL; ++i) {
#pragma unroll
    for (int j = i; j > 0; --j) {
      const uint64_t hi = keys[j - 1] > keys[j] ? keys[j - 1] : keys[j];
      const uint64_t lo = keys[j - 1] > keys[j] ? keys[j] : keys[j - 1];
      keys[j - 1] = hi;
      keys[j] = lo;
    }
  }

  uint64_t mine = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = keys[0];
#pragma unroll
    for (int off = 1; off < LPT; off <<= 1) {
      const uint64_t o = shfl_xor_u64(best, off);
      best = o > best ? o : best;
    }
    if (sub == k) mine = best;
    if (keys[0] == best) {  // the owner pops its head
#pragma unroll
      for (int i = 0; i + 1 < EPL; ++i) keys[i] = keys[i + 1];
      keys[EPL - 1] = 0ull;
    }
  }

  // ---- weights from the unbiased scores -----------------------------------
  const bool slot = tok_ok && sub < K;
  uint32_t e_sel = ~static_cast<uint32_t>(mine);
  if (e_sel >= static_cast<uint32_t>(E)) e_sel = 0;  // only reachable with NaN scores
  const float u = slot ? scores[t * E + e_sel] : 0.0f;
  float w;
  if (norm_weights) {
    float d = 0.0f;
    for (int k = 0; k < K; ++k) d += __shfl(u, tok_lane0 + k, kWave);
    w = (u / d) * scale;
  } else {
    w = u * scale;
  }
  if (slot) {
    out_idx[t * K + sub] = static_cast<int32_t>(e_sel);
    out_w[t * K + sub] = w;
  }
}

template <int EPL, int LPT>
moe_status_t launch_router_t(int32_t* idx, float* w, const float* s, const float* b, int64_t T,
                             int32_t K, int32_t G, int32_t TG, int32_t norm, float scale,
                             int32_t mode, hipStream_t stream) {
  constexpr int TPB = kWavesPerBlock * (kWave / LPT);  // tokens per block
  const int64_t blocks = (T + TPB - 1) / TPB;
  hipLaunchKernelGGL((router_kernel<EPL, LPT>), dim3(static_cast<uint32_t>(blocks)), dim3(kBlock),
                     0, stream, idx, w, s, b, T, K, G, TG, norm, scale, mode);
  return check_launch();
}

}  // namespace

moe_status_t launch_router(int32_t* idx, float* w, const float* s, const float* b, int64_t T,
                           int32_t E, int32_t K, int32_t G, int32_t TG, int32_t norm, float scale,
                           int32_t mode, hipStream_t stream) {
  switch (E) {
    case 1: return launch_router_t<1, 1>(idx, w, s, b, T, K, G, TG, norm, scale, mode, stream);
    case 2: return launch_router_t<1, 2>(idx, w, s, b, T, K, G, TG, norm, scale, mode, stream);
    case 4: return launch_router_t<1, 4>(idx, w, s, b, T, K, G, TG, norm, scale, mode, stream);
    case 8: return launch_router_t<1, 8>(idx, w, s, b, T, K, G, TG, norm, scale, mode, stream);
    case 16: return launch_router_t<1, 16>(idx, w, s, b, T, K, G, TG, norm, scale, mode, stream);
    case 32: return launch_router_t<1, 32>(idx, w, s, b, T, K, G, TG, norm, scale, mode, stream);
    case 64: return launch_router_t<1, 64>(idx, w, s, b, T, K, G, TG, norm, scale, mode, stream);
    case 128: return launch_router_t<2, 64>(idx, w, s, b, T, K, G, TG, norm, scale, mode, stream);
    case 256: return launch_router_t<4, 64>(idx, w, s, b, T, K, G, TG, norm, scale, mode, stream);
    case 512: return launch_router_t<8, 64>(idx, w, s, b, T, K, G, TG, norm, scale, mode, stream);
    case 1024: return launch_router_t<16, 64>(idx, w, s, b, T, K, G, TG, norm, scale, mode, stream);
    default: return MOE_ERR_UNSUPPORTED;
  }
}

}  // namespace moe
