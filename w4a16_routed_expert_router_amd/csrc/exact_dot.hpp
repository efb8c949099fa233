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

// Exact dot product of FP16 rows a, b of length H (a multiple of 8), over the
// whole wave.  Every lane returns the correctly rounded FP32 result.  b is in
// global memory.  Each lane loads up to four 8-element chunks before it uses
// any, so the row costs one or two memory round trips.
__device__ inline float exact_dot_wave(const uint16_t* a, const uint16_t* b, int H, int lane) {
  constexpr int kAhead = 4;
  __int128 acc = 0;
  for (int k0 = lane * 8; k0 < H; k0 += kAhead * kWave * 8) {
    uint4 av[kAhead], bv[kAhead];
#pragma unroll
    for (int c = 0; c < kAhead; ++c) {
      const int k = k0 + c * kWave * 8;
      av[c] = k < H ? *reinterpret_cast<const uint4*>(a + k) : make_uint4(0u, 0u, 0u, 0u);
      bv[c] = k < H ? ldg_u4(b + k) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int c = 0; c < kAhead; ++c) {
      const uint32_t aw[4] = {av[c].x, av[c].y, av[c].z, av[c].w};
      const uint32_t bw[4] = {bv[c].x, bv[c].y, bv[c].z, bv[c].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t ah = (uint16_t)(aw[i >> 1] >> (16 * (i & 1)));
        const uint16_t bh = (uint16_t)(bw[i >> 1] >> (16 * (i & 1)));
        int32_t ma, sa, mb, sb;
        f16_fixed(ah, ma, sa);
        f16_fixed(bh, mb, sb);
        acc += ((__int128)(ma * mb)) << (sa + sb);  // a zero chunk adds zero
      }
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



// Exact partial dot product of FP16 rows a, b over [k0, k1) (k0, k1 multiples
// of 8, 8-element chunks dealt over the lanes), as a 128-bit fixed-point
// integer in units of 2^-48 summed over the wave: every lane returns it.  Exact
// partial sums add exactly, so any split of a row over waves gives the same
// total as exact_dot_wave.
__device__ inline __int128 exact_partial_wave(const uint16_t* a, const uint16_t* b, int k0, int k1, int lane) {
  constexpr int kAhead = 4;
  __int128 acc = 0;
  for (int kb = k0 + lane * 8; kb < k1; kb += kAhead * kWave * 8) {
    uint4 av[kAhead], bv[kAhead];
#pragma unroll
    for (int c = 0; c < kAhead; ++c) {
      const int k = kb + c * kWave * 8;
      av[c] = k < k1 ? *reinterpret_cast<const uint4*>(a + k) : make_uint4(0u, 0u, 0u, 0u);
      bv[c] = k < k1 ? ldg_u4(b + k) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int c = 0; c < kAhead; ++c) {
      const uint32_t aw[4] = {av[c].x, av[c].y, av[c].z, av[c].w};
      const uint32_t bw[4] = {bv[c].x, bv[c].y, bv[c].z, bv[c].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int32_t ma, sa, mb, sb;
        f16_fixed((uint16_t)(aw[i >> 1] >> (16 * (i & 1))), ma, sa);
        f16_fixed((uint16_t)(bw[i >> 1] >> (16 * (i & 1))), mb, sb);
        acc += ((__int128)(ma * mb)) << (sa + sb);  // a zero chunk adds zero
      }
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
  return (((__int128)hi) << 64) | (__int128)lo;
}

// exact_dot_wave with one chunk of each row in flight and no unrolling: the
// same exact sum (so the same result) for a caller with little register room,
// where the exact tier is a rare fallback.
__device__ inline float exact_dot_wave_lean(const uint16_t* a, const uint16_t* b, int H, int lane) {
  __int128 acc = 0;
#pragma unroll 1
  for (int k0 = lane * 8; k0 < H; k0 += kWave * 8) {
    const uint4 av = *reinterpret_cast<const uint4*>(a + k0);
    const uint4 bv = ldg_u4(b + k0);
    const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
    const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll 1
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

}  // namespace moe
