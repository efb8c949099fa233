// Top-k selection by one wavefront, for the router of the fused decode path.
//
// The order is (logit descending, expert id ascending).  Each candidate is a
// 64-bit key: the order-preserving image of its FP32 logit above the
// complemented expert id, so one unsigned comparison orders two candidates
// and distinct experts never tie.  A key's rank is the number of keys greater
// than it, counted by every lane against all keys read from LDS (broadcast
// reads, independent comparisons: no chain of lane-to-lane steps).  Every
// result is a function of the keys alone, so every wave that runs it on the
// same keys derives the same bits.
#pragma once

#include "common.hpp"

namespace moe {

// Order-preserving image of an FP32 value (never 0 for a finite value or an
// infinity; 0 marks an empty slot).
__device__ __forceinline__ uint32_t order_bits(float v) {
  const uint32_t vb = __builtin_bit_cast(uint32_t, v);
  return (vb & 0x80000000u) ? ~vb : (vb | 0x80000000u);
}
__device__ __forceinline__ float unorder_bits(uint32_t ob) {
  return __builtin_bit_cast(float, (ob & 0x80000000u) ? (ob & 0x7fffffffu) : ~ob);
}

__device__ __forceinline__ uint32_t rdlane(uint32_t v, int j) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, j);
}

// 64-bit selection key of expert `id` with logit v: ordered like (logit desc,
// id asc) by one unsigned comparison (larger key = earlier rank); distinct
// for distinct ids and never 0.  -0 is taken as +0, so that the two zeros
// tie like equal values and the id decides.
__device__ __forceinline__ uint64_t sel_key(float v, int id) {
  return ((uint64_t)order_bits(v + 0.0f) << 32) | (uint32_t)(0xffffffffu - (uint32_t)id);
}
__device__ __forceinline__ int key_id(uint64_t key) { return (int)(0xffffffffu - (uint32_t)key); }
__device__ __forceinline__ float key_value(uint64_t key) { return unorder_bits((uint32_t)(key >> 32)); }

// Rank of the keys k0 (slot lane) and k1 (slot lane + 64) among the n keys of
// slots 0 .. n-1 (n <= 128, keys distinct, an empty slot holds 0): the number
// of keys greater than each.  scr: 128 LDS words of this wave.  Every lane
// reads every key (broadcast reads), so no lane waits for another.
__device__ __forceinline__ void wave_rank(uint64_t k0, uint64_t k1, int n, uint64_t* scr, int lane, int& r0,
                                          int& r1) {
  scr[lane] = k0;
  scr[lane + kWave] = k1;
  int a = 0, b = 0;
#pragma unroll 4
  for (int j = 0; j < n; j += 2) {
    const uint4 two = *reinterpret_cast<const uint4*>(scr + j);
    const uint64_t x0 = ((uint64_t)two.y << 32) | two.x, x1 = ((uint64_t)two.w << 32) | two.z;
    a += (int)(x0 > k0) + (int)(x1 > k0);
    b += (int)(x0 > k1) + (int)(x1 > k1);
  }
  r0 = a;
  r1 = b;
}

// Rank of this lane's key among the 64 keys of the wave (one per lane, keys
// distinct): the number of keys greater than it.  Reads 16 keys per batch so
// that the LDS latency is paid a few times, not once per key.
__device__ __forceinline__ int wave_rank64(uint64_t key, uint64_t* scr, int lane) {
  scr[lane] = key;
  int r = 0;
#pragma unroll 1
  for (int j0 = 0; j0 < kWave; j0 += 16) {
    uint4 t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = *reinterpret_cast<const uint4*>(scr + j0 + 2 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint64_t x0 = ((uint64_t)t[i].y << 32) | t[i].x, x1 = ((uint64_t)t[i].w << 32) | t[i].z;
      r += (int)(x0 > key) + (int)(x1 > key);
    }
  }
  return r;
}

// Ranks skip .. skip+k-1 of 64 keys (one per lane): out[r - skip] = the key of
// rank r.  Returns this lane's rank.
__device__ __forceinline__ int wave_top64(uint64_t key, int k, int skip, uint64_t* scr, uint64_t* out, int lane) {
  const int r = wave_rank64(key, scr, lane);
  if (r >= skip && r < skip + k) out[r - skip] = key;
  return r;
}

// Ranks skip .. skip+k-1 of the n candidate keys cand[0 .. n) (n <= 128).
__device__ __forceinline__ void wave_top_cands(const uint64_t* cand, int n, int k, int skip, uint64_t* scr,
                                               uint64_t* out, int lane) {
  const uint64_t k0 = lane < n ? cand[lane] : 0ull;
  const uint64_t k1 = lane + kWave < n ? cand[lane + kWave] : 0ull;
  int r0, r1;
  wave_rank(k0, k1, (n + 1) & ~1, scr, lane, r0, r1);
  if (lane < n && r0 >= skip && r0 < skip + k) out[r0 - skip] = k0;
  if (lane + kWave < n && r1 >= skip && r1 < skip + k) out[r1 - skip] = k1;
}

// Ranks 0 .. k-1 of the n distinct keys list[0 .. n) (any n): out[r] = the
// key of rank r.  Each lane ranks the keys of its slots lane + 64 c against
// the whole list, read from LDS two keys at a time (list 16-byte aligned;
// list[n] is read when n is odd and must exist: it is never counted).
__device__ __forceinline__ void wave_top_list(const uint64_t* list, int n, int k, uint64_t* out, int lane) {
#pragma unroll 1
  for (int c0 = 0; c0 < n; c0 += kWave) {
    const bool own = c0 + lane < n;
    const uint64_t key = own ? list[c0 + lane] : 0ull;
    int r = 0;
#pragma unroll 4
    for (int j = 0; j < n; j += 2) {
      const uint4 two = *reinterpret_cast<const uint4*>(list + j);
      const uint64_t x0 = ((uint64_t)two.y << 32) | two.x, x1 = ((uint64_t)two.w << 32) | two.z;
      r += (int)(x0 > key) + (int)(j + 1 < n && x1 > key);
    }
    if (own && r < k) out[r] = key;
  }
}

}  // namespace moe
