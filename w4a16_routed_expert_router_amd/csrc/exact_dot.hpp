// Exact FP16 dot products: the FP32 value nearest (ties to even) to the exact
// real sum of FP16 products, computed as a 128-bit fixed-point integer.
#pragma once

#include "common.hpp"

namespace moe {

__device__ __forceinline__ void f16_fixed(uint16_t b, int32_t& m, int32_t& sh) {
  // FP16 value = m * 2^sh * 2^-24 with |m| < 2^11, 0 <= sh <= 29.
  const int32_t e = (b >> 10) & 0x1F;
  const int32_t f = b & 0x3FF;
  if (e == 0) {
    m = f;
    sh = 0;
  } else {
    m = 1024 + f;
    sh = e - 1;
  }
  if (b & 0x8000) m = -m;
}

__device__ __forceinline__ int clz128(unsigned __int128 v) {
  const uint64_t hi = (uint64_t)(v >> 64);
  const uint64_t lo = (uint64_t)v;
  return hi ? __clzll(hi) : 64 + (lo ? __clzll(lo) : 64);
}

// Nearest FP32 (ties to even) to S * 2^exp2; S*2^exp2 is always in FP32's
// normal range here (|S| < 2^92, exp2 = -48).
__device__ inline float round_i128_to_f32(__int128 S, int exp2) {
  if (S == 0) return 0.0f;
  const bool neg = S < 0;
  const unsigned __int128 m = neg ? (unsigned __int128)(-S) : (unsigned __int128)S;
  const int nb = 128 - clz128(m);
  float f;
  if (nb <= 24) {
    f = ldexpf((float)(uint32_t)m, exp2);
  } else {
    const int sh = nb - 24;
    unsigned __int128 q = m >> sh;
    const unsigned __int128 r = m & ((((unsigned __int128)1) << sh) - 1);
    const unsigned __int128 half = ((unsigned __int128)1) << (sh - 1);
    if (r > half || (r == half && (q & 1))) q += 1;
    f = ldexpf((float)(uint32_t)q, sh + exp2);  // q <= 2^24: exact
  }
  return neg ? -f : f;
}

// Exact dot product of FP16 rows a, b of length H, over the whole wave.
// Every lane returns the correctly rounded FP32 result.  b is in global memory.
__device__ inline float exact_dot_wave(const uint16_t* a, const uint16_t* b, int H, int lane) {
  __int128 acc = 0;
  for (int k = lane * 8; k < H; k += kWave * 8) {
    const uint4 av = *reinterpret_cast<const uint4*>(a + k);
    const uint4 bv = ldg_u4(b + k);
    const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
    const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t ah = (uint16_t)(aw[i >> 1] >> (16 * (i & 1)));
      const uint16_t bh = (uint16_t)(bw[i >> 1] >> (16 * (i & 1)));
      int32_t ma, sa, mb, sb;
      f16_fixed(ah, ma, sa);
      f16_fixed(bh, mb, sb);
      acc += ((__int128)(ma * mb)) << (sa + sb);
    }
  }
  uint64_t lo = (uint64_t)acc;
  int64_t hi = (int64_t)(acc >> 64);
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const uint64_t lo2 = __shfl_xor(lo, o, kWave);
    const int64_t hi2 = __shfl_xor(hi, o, kWave);
    const uint64_t nlo = lo + lo2;
    hi = hi + hi2 + (nlo < lo ? 1 : 0);
    lo = nlo;
  }
  const __int128 S = (((__int128)hi) << 64) | (__int128)lo;
  return round_i128_to_f32(S, -48);
}


// Certified tier: products of FP16 values are exact in FP32; they are summed in
// FP64 with sum |p|, which bounds the FP64 error (each product passes through at
// most `depth` additions).  Returns the FP32 rounding when the whole error
// interval lies strictly between the two rounding midpoints of that value, so
// it equals the rounding of the exact sum; otherwise falls back to the exact
// tier.  All lanes of the wave must call it and get the same result.
__device__ inline float certified_dot_wave(const uint16_t* a, const uint16_t* b, int H, int lane,
                                           int exact_always) {
  if (!exact_always) {
    double acc = 0.0, asum = 0.0;
    for (int k = lane * 8; k < H; k += kWave * 8) {
      const uint4 av = *reinterpret_cast<const uint4*>(a + k);
      const uint4 bv = *reinterpret_cast<const uint4*>(b + k);
      const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
      const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = half_bits_to_float((uint16_t)(aw[i >> 1] >> (16 * (i & 1))));
        const float y = half_bits_to_float((uint16_t)(bw[i >> 1] >> (16 * (i & 1))));
        const double p = (double)(x * y);
        acc += p;
        asum += fabs(p);
      }
    }
    // xor butterfly: every lane ends with bit-identical sums
    for (int o = kWave / 2; o > 0; o >>= 1) {
      acc += __shfl_xor(acc, o, kWave);
      asum += __shfl_xor(asum, o, kWave);
    }
    const int depth = 8 * ((H + 511) / 512) + 6;
    const double eps = (double)(depth + 2) * 0x1p-52 * asum;
    const float r = (float)acc;
    if (r != 0.0f && isfinite(r) && isfinite(acc)) {
      const double rd = (double)r;
      const double m_lo = 0.5 * (rd + (double)nextafterf(r, -INFINITY));
      const double m_hi = 0.5 * (rd + (double)nextafterf(r, INFINITY));
      if (acc - eps > m_lo && acc + eps < m_hi) return r;
    }
  }
  return exact_dot_wave(a, b, H, lane);
}

}  // namespace moe
