// Per-lane helpers of the encode path, shared by the encode kernels and the
// streaming attention kernel's append phase (which must produce the same
// codes): fp16 row loads and stores, and the normalized Walsh-Hadamard
// rotation of a head vector held as one sub-vector per lane (in-lane
// butterflies over the low index bits, cross-lane ones over the lane bits),
// the same butterflies in the same order wherever it is used.
#pragma once
#include "vq_internal.h"

#include <type_traits>

namespace vq {
namespace {

template <int DS>
__device__ __forceinline__ void load_f16(const __half* __restrict__ p, float (&x)[DS]) {
  if constexpr (DS == 1) {
    x[0] = __half2float(p[0]);
  } else if constexpr (DS == 2) {
    float2 f = __half22float2(*reinterpret_cast<const __half2*>(p));
    x[0] = f.x; x[1] = f.y;
  } else if constexpr (DS == 4) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    float2 f0 = __half22float2(*reinterpret_cast<const __half2*>(&u.x));
    float2 f1 = __half22float2(*reinterpret_cast<const __half2*>(&u.y));
    x[0] = f0.x; x[1] = f0.y; x[2] = f1.x; x[3] = f1.y;
  } else {
#pragma unroll
    for (int i = 0; i < DS; i += 8) {
      uint4 u = *reinterpret_cast<const uint4*>(p + i);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float2 f = __half22float2(*reinterpret_cast<const __half2*>(&w[k]));
        x[i + 2 * k] = f.x; x[i + 2 * k + 1] = f.y;
      }
    }
  }
}

// The DS fp16 values at p as raw bits (halves packed two per word), to be
// converted once they are needed.
template <int DS>
struct RawHalves {
  uint32_t w[(DS + 1) / 2];
};
template <int DS>
__device__ __forceinline__ RawHalves<DS> load_raw_f16(const __half* __restrict__ p) {
  RawHalves<DS> r;
  if constexpr (DS == 1) {
    r.w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else if constexpr (DS == 2) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (DS == 4) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    r.w[0] = u.x; r.w[1] = u.y;
  } else {
#pragma unroll
    for (int i = 0; i < DS / 8; ++i) {
      const uint4 u = reinterpret_cast<const uint4*>(p)[i];
      r.w[4 * i] = u.x; r.w[4 * i + 1] = u.y; r.w[4 * i + 2] = u.z; r.w[4 * i + 3] = u.w;
    }
  }
  return r;
}
template <int DS>
__device__ __forceinline__ void cvt_raw_f16(const RawHalves<DS>& r, float (&x)[DS]) {
#pragma unroll
  for (int e = 0; e < DS; ++e) {
    const uint16_t b = (uint16_t)(r.w[e / 2] >> (16 * (e & 1)));
    x[e] = __half2float(*reinterpret_cast<const __half*>(&b));
  }
}

template <int DS>
__device__ __forceinline__ void store_f16(__half* __restrict__ p, const float (&x)[DS]) {
  if constexpr (DS == 1) {
    p[0] = __float2half_rn(x[0]);
  } else if constexpr (DS == 2) {
    *reinterpret_cast<__half2*>(p) = __floats2half2_rn(x[0], x[1]);
  } else if constexpr (DS == 4) {
    __half2 a = __floats2half2_rn(x[0], x[1]), b = __floats2half2_rn(x[2], x[3]);
    uint2 u;
    u.x = *reinterpret_cast<uint32_t*>(&a);
    u.y = *reinterpret_cast<uint32_t*>(&b);
    *reinterpret_cast<uint2*>(p) = u;
  } else {
#pragma unroll
    for (int i = 0; i < DS; i += 8) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        __half2 h = __floats2half2_rn(x[i + 2 * k], x[i + 2 * k + 1]);
        w[k] = *reinterpret_cast<uint32_t*>(&h);
      }
      *reinterpret_cast<uint4*>(p + i) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

template <int DS>
__device__ __forceinline__ void store_f32(float* __restrict__ p, const float (&x)[DS]) {
  if constexpr (DS == 1) {
    p[0] = x[0];
  } else if constexpr (DS == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
  } else {
#pragma unroll
    for (int i = 0; i < DS; i += 4)
      *reinterpret_cast<float4*>(p + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
  }
}

// Unnormalized Walsh-Hadamard butterflies over the index bits held inside the
// lane (element e of sub-vector j is index j * DS + e).
template <int DS>
__device__ __forceinline__ void wht_in_lane(float (&x)[DS]) {
#pragma unroll
  for (int h = 1; h < DS; h <<= 1) {
#pragma unroll
    for (int i = 0; i < DS; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
}

// Butterflies over the index bits that select the lane (sub-vector j): the
// partner of lane j for bit m is lane j ^ m in the same token-head group.
template <int NSUB, int DS>
__device__ __forceinline__ void wht_cross_lane(float (&x)[DS], int j) {
  // Lane j gets x + x(j ^ M) where bit M of j is clear and x(j ^ M) - x
  // where it is set: fma(sg, a, b) with sg = -1 / +1, which rounds as that
  // sum or difference.  The partner's value comes without a trip through
  // LDS: DPP quad permutes (M = 1, 2), row shifts into alternate 4-lane
  // banks (M = 4), a row rotation (M = 8); v_permlane16/32_swap of x with
  // itself (M = 16, 32) returns (own, partner) where bit M is clear and
  // (partner, own) where it is set, so fma(sg, second, first) needs no select.
  auto butterfly = [](float v, float sg, auto mc) {
    constexpr int M = decltype(mc)::value;
    const int vi = __float_as_int(v);
    if constexpr (M == 1) {
      return fmaf(sg, v, __int_as_float(__builtin_amdgcn_mov_dpp(vi, 0xb1, 0xf, 0xf, false)));
    } else if constexpr (M == 2) {
      return fmaf(sg, v, __int_as_float(__builtin_amdgcn_mov_dpp(vi, 0x4e, 0xf, 0xf, false)));
    } else if constexpr (M == 4) {
      const int t = __builtin_amdgcn_update_dpp(0, vi, 0x104, 0xf, 0x5, false);
      return fmaf(sg, v, __int_as_float(__builtin_amdgcn_update_dpp(t, vi, 0x114, 0xf, 0xa, false)));
    } else if constexpr (M == 8) {
      return fmaf(sg, v, __int_as_float(__builtin_amdgcn_update_dpp(0, vi, 0x128, 0xf, 0xf, false)));
    } else if constexpr (M == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap((unsigned)vi, (unsigned)vi, false, false);
      return fmaf(sg, __uint_as_float(r[1]), __uint_as_float(r[0]));
    } else {
      static_assert(M == 32, "lane bit");
      const auto r = __builtin_amdgcn_permlane32_swap((unsigned)vi, (unsigned)vi, false, false);
      return fmaf(sg, __uint_as_float(r[1]), __uint_as_float(r[0]));
    }
  };
  auto stage = [&](auto mc) {
    constexpr int M = decltype(mc)::value;
    if constexpr (M < NSUB) {
      const float sg = (j & M) ? -1.f : 1.f;
#pragma unroll
      for (int e = 0; e < DS; ++e) x[e] = butterfly(x[e], sg, mc);
    }
  };
  stage(std::integral_constant<int, 1>{});
  stage(std::integral_constant<int, 2>{});
  stage(std::integral_constant<int, 4>{});
  stage(std::integral_constant<int, 8>{});
  stage(std::integral_constant<int, 16>{});
  stage(std::integral_constant<int, 32>{});
}

template <int D, int DS>
__device__ __forceinline__ void wht(float (&x)[DS], int j) {
  wht_in_lane<DS>(x);
  wht_cross_lane<D / DS, DS>(x, j);
  const float nrm = WhtNorm<D>::value;
#pragma unroll
  for (int e = 0; e < DS; ++e) x[e] *= nrm;
}

}  // namespace
}  // namespace vq
