// Device helpers shared by the fused decode kernels (decode_fused.hip and
// decode_spec.hip): epoch-tagged exchange words, INT4 -> FP16 MFMA operands,
// router dot products with certified FP32 rounding.
#pragma once

#include "common.hpp"
#include "exact_dot.hpp"
#include "launch.hpp"

namespace moe {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kFT = 512;
constexpr int kFW = kFT / kWave;  // 8 waves
constexpr uint32_t kSpinLimit = 1u << 18;  // polls of one word before giving up

// ---- epoch-tagged words ----------------------------------------------------------
__device__ __forceinline__ void st_tag(uint64_t* p, uint32_t tag, uint32_t v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tag_is(uint64_t w, uint32_t tag) { return (uint32_t)(w >> 32) == tag; }

// Polls one word until it carries `tag` (or the wait is abandoned).
__device__ __forceinline__ uint32_t wait_word(const uint64_t* p, uint64_t w, uint32_t tag, bool& bail) {
  uint32_t spins = 0;
  while (!tag_is(w, tag) && !bail) {
    if (++spins > kSpinLimit) {
      bail = true;
      break;
    }
    w = ld_tag(p);
  }
  return (uint32_t)w;
}

// Cooperative read of n tagged words by NT threads (thread index `tid` among
// them): sink(i, payload) for each.  A thread holds up to NF words in flight;
// every poll round re-issues all of its words that are not current yet, so one
// round trip refreshes them all.
template <int NT, int NF = 8, class F>
__device__ __forceinline__ void read_tagged_n(const uint64_t* src, int n, uint32_t tag, bool& bail, int tid,
                                              F&& sink) {
  for (int i0 = tid; i0 < n; i0 += NF * NT) {
    uint64_t w[NF];
#pragma unroll
    for (int u = 0; u < NF; ++u) {
      const int i = i0 + u * NT;
      w[u] = i < n ? ld_tag(src + i) : ((uint64_t)tag << 32);
    }
    uint32_t spins = 0;
    while (!bail) {
      bool all = true;
#pragma unroll
      for (int u = 0; u < NF; ++u) all &= tag_is(w[u], tag);
      if (all) break;
      if (++spins > kSpinLimit) {
        bail = true;
        break;
      }
#pragma unroll
      for (int u = 0; u < NF; ++u)
        if (!tag_is(w[u], tag)) w[u] = ld_tag(src + i0 + u * NT);
    }
#pragma unroll
    for (int u = 0; u < NF; ++u) {
      const int i = i0 + u * NT;
      if (i < n) sink(i, (uint32_t)w[u]);
    }
  }
}

// Block-cooperative read of n tagged words (every thread of the block).
template <class F>
__device__ __forceinline__ void read_tagged(const uint64_t* src, int n, uint32_t tag, bool& bail, F&& sink) {
  read_tagged_n<kFT>(src, n, tag, bail, (int)threadIdx.x, sink);
}

// INT4 dword of 8 K values -> the 8 FP16 operands of one MFMA step.
__device__ __forceinline__ h8 decode_h8(uint32_t d) {
  h2 p[4];
  dequant8(d, p);
  h8 r;
  r[0] = p[0][0]; r[1] = p[0][1]; r[2] = p[1][0]; r[3] = p[1][1];
  r[4] = p[2][0]; r[5] = p[2][1]; r[6] = p[3][0]; r[7] = p[3][1];
  return r;
}

__device__ __forceinline__ uint32_t dword_of(const uint4& q, int i) {
  return i == 0 ? q.x : (i == 1 ? q.y : (i == 2 ? q.z : q.w));
}

// One wave's part of a router row: chunks c < nc of 512 FP16, 8 per lane.
template <int H>
__device__ __forceinline__ void load_router_part(const uint16_t* part_row, int nc, int lane,
                                                 uint4 (&q)[H / 512]) {
#pragma unroll
  for (int c = 0; c < H / 512; ++c)
    if (c < nc) q[c] = ldg_u4(part_row + c * 512 + lane * 8);
}

// FP64 partial dot of LDS x with a router part already in registers; every
// lane ends with the wave's sums (bit-identical in all lanes).
// Products of FP16 values are exact in FP32; |p| is summed alongside.
template <int H>
__device__ __forceinline__ void partial_dot(const _Float16* x, const uint4 (&q)[H / 512], int nc, int lane,
                                            double& acc, double& asum) {
  acc = 0.0;
  asum = 0.0;
#pragma unroll
  for (int c = 0; c < H / 512; ++c) {
    if (c < nc) {
      const uint4 av = *reinterpret_cast<const uint4*>(x + c * 512 + lane * 8);
      const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
      const uint32_t bw[4] = {q[c].x, q[c].y, q[c].z, q[c].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xv = half_bits_to_float((uint16_t)(aw[i >> 1] >> (16 * (i & 1))));
        const float yv = half_bits_to_float((uint16_t)(bw[i >> 1] >> (16 * (i & 1))));
        const double p = (double)(xv * yv);
        acc += p;
        asum += fabs(p);
      }
    }
  }
  acc = wave_sum(acc);
  asum = wave_sum(asum);
}

// Certified rounding: an FP64 sum of FP16 products whose sum of magnitudes
// asum is below kExactSumBound is exact, so its FP32 rounding is the logit;
// otherwise the FP32 rounding of an FP64 sum whose error is at most
// (depth + 2) * 2^-52 * asum equals the rounding of the exact sum when the
// whole error interval lies strictly between the two rounding midpoints of
// that value.  Returns false when neither is proven.
__device__ __forceinline__ bool certify(double acc, double asum, int depth, float& out) {
  const double eps = (double)(depth + 2) * 0x1p-52 * asum;
  const float r = (float)acc;
  if (r != 0.0f && isfinite(r) && isfinite(acc) && isfinite(asum)) {
    const double rd = (double)r;
    const double m_lo = 0.5 * (rd + (double)nextafterf(r, -INFINITY));
    const double m_hi = 0.5 * (rd + (double)nextafterf(r, INFINITY));
    if (asum < kExactSumBound || (acc - eps > m_lo && acc + eps < m_hi)) {
      out = r;
      return true;
    }
  }
  return false;
}

// Phase timestamp (instrumentation) of thread `who`, kept in the kernel's LDS
// stamp buffer until the launch ends.
template <class S>
__device__ __forceinline__ void stamp(S& s, const FusedArgs& a, int l, int ev, int who = 0) {
  if (a.stamps && (int)threadIdx.x == who && l - a.l0 < kStampLayers) {
    const int i = (l - a.l0) * kStampsPerLayer + ev;
    s.stampbuf[0][i] = __builtin_amdgcn_s_memrealtime();
    s.stampbuf[1][i] = __builtin_amdgcn_s_memtime();
  }
}

// OR of a per-thread flag over the block (all threads call it).
__device__ __forceinline__ bool block_any(bool v) { return __syncthreads_or(v ? 1 : 0) != 0; }

}  // namespace moe
