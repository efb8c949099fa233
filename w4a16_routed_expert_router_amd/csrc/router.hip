// Router: logits, softmax and top-k of one MoE layer.
//
// Routing (each token picks its top-k experts, "Horizon RunMap", "The complete
// execution path"; 8 of 64 per layer in "An expert-offloading engine, from
// scratch", "Terms used here"; 10 of 512 in "F51 Nitro / Nitro-MoE",
// "The thesis").  The router matrix is an FP16 non-routed weight
// ("Horizon RunMap", "Architecture invariants").
//
// logit[t,e] is defined as the FP32 value nearest (ties to even) to the exact
// real dot product of the FP16 inputs, so the selected experts do not depend on
// summation order.  It is reached in two tiers:
//   1. every FP16 x FP16 product is exact in FP32; products are summed in FP64
//      together with sum |p|, which bounds the FP64 error; the FP64 sum is
//      rounded to FP32 and accepted when the whole error interval rounds to the
//      same FP32 value (it lies strictly between that value's two rounding
//      midpoints);
//   2. otherwise (about one logit in 10^6) the wave recomputes the sum exactly
//      as a 128-bit fixed-point integer (unit 2^-48) and rounds it once.
#include "common.hpp"
#include "launch.hpp"
#include "exact_dot.hpp"

namespace moe {

constexpr int kRtTok = 4;  // tokens per logits work item
constexpr int kRtExp = 4;  // experts per logits work item
constexpr int kCombos = kRtTok * kRtExp;

// Sum 2*kCombos doubles across the wave, each lane keeping one index:
// afterwards lane l holds the full sum of value index (l >> 1) in v[0].
__device__ __forceinline__ void transpose_reduce32(double (&v)[2 * kCombos], int lane) {
  int n = 2 * kCombos;
  int o = kWave / 2;
  for (; n > 1; o >>= 1) {
    const int half = n >> 1;
    const bool up = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const double send = up ? v[i] : v[i + half];
      const double keep = up ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, o, kWave);
    }
    n = half;
  }
  for (; o > 0; o >>= 1) v[0] += __shfl_xor(v[0], o, kWave);
}

// grid (ceil(E/4), ceil(T/4)), block 64: one wave per 4 tokens x 4 experts.
__global__ __launch_bounds__(64) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           int T, int E, int H,
                                                           float* __restrict__ logits,
                                                           int exact_always) {
  const int lane = threadIdx.x;
  const int e0 = blockIdx.x * kRtExp;
  const int t0 = blockIdx.y * kRtTok;

  double v[2 * kCombos];
#pragma unroll
  for (int i = 0; i < 2 * kCombos; ++i) v[i] = 0.0;

  if (!exact_always) {
    for (int k = lane * 8; k < H; k += kWave * 8) {
      float xf[kRtTok][8], wf[kRtExp][8];
#pragma unroll
      for (int ti = 0; ti < kRtTok; ++ti) {
        const int t = min(t0 + ti, T - 1);
        const uint4 q = *reinterpret_cast<const uint4*>(x + (int64_t)t * H + k);
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) xf[ti][i] = half_bits_to_float((uint16_t)(u[i >> 1] >> (16 * (i & 1))));
      }
#pragma unroll
      for (int ei = 0; ei < kRtExp; ++ei) {
        const int e = min(e0 + ei, E - 1);
        const uint4 q = *reinterpret_cast<const uint4*>(wr + (int64_t)e * H + k);
        const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) wf[ei][i] = half_bits_to_float((uint16_t)(u[i >> 1] >> (16 * (i & 1))));
      }
#pragma unroll
      for (int ti = 0; ti < kRtTok; ++ti)
#pragma unroll
        for (int ei = 0; ei < kRtExp; ++ei)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const double p = (double)(xf[ti][i] * wf[ei][i]);  // exact in FP32
            v[ti * kRtExp + ei] += p;
            v[kCombos + ti * kRtExp + ei] += fabs(p);
          }
    }
    transpose_reduce32(v, lane);
  }
  // lanes 2c hold the sum of combo c, lanes 32+2c the sum of its |p|
  const double asum = __shfl(v[0], (lane + 32) & 63, kWave);
  const int c = lane >> 1;
  const int t = t0 + c / kRtExp;
  const int e = e0 + c % kRtExp;
  const bool mine = (lane < 32) && ((lane & 1) == 0) && t < T && e < E;
  bool certified = false;
  if (mine && !exact_always) {
    const double s = v[0];
    // additions any product went through: 8 per 512-wide chunk, then 6 levels
    const int depth = 8 * ((H + 511) / 512) + 6;
    const double eps = (double)(depth + 2) * 0x1p-52 * asum;
    const float r = (float)s;  // round to nearest even
    if (r != 0.0f && isfinite(r) && isfinite(s)) {
      const double rd = (double)r;
      const double m_lo = 0.5 * (rd + (double)nextafterf(r, -INFINITY));
      const double m_hi = 0.5 * (rd + (double)nextafterf(r, INFINITY));
      if (s - eps > m_lo && s + eps < m_hi) {
        certified = true;
        logits[(int64_t)t * E + e] = r;
      }
    }
  }
  uint64_t todo = __ballot(mine && !certified);
  while (todo) {
    const int l = __builtin_ctzll(todo);
    todo &= todo - 1;
    const int cc = l >> 1;
    const int tt = t0 + cc / kRtExp;
    const int ee = e0 + cc % kRtExp;
    const float r = exact_dot_wave(x + (int64_t)tt * H, wr + (int64_t)ee * H, H, lane);
    if (lane == 0) logits[(int64_t)tt * E + ee] = r;
  }
}

__device__ __forceinline__ uint64_t rank_key(float v, int id) {
  uint32_t u = __float_as_uint(v + 0.0f);  // -0 -> +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)id);
}

// grid T, block 64: softmax + top-k (or forced ids) for one token per wave.
__global__ __launch_bounds__(64) void router_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int renorm,
                                                         const int32_t* __restrict__ forced,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w,
                                                         uint32_t* __restrict__ err) {
  constexpr int kMaxV = 16;  // E <= 1024
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* lg = logits + (int64_t)t * E;
  float v[kMaxV];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kMaxV; ++i) {
    const int e = i * kWave + lane;
    v[i] = (e < E) ? lg[e] : -INFINITY;
    mx = fmaxf(mx, v[i]);
  }
  mx = wave_max(mx);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxV; ++i)
    if (i * kWave + lane < E) s += expf(v[i] - mx);
  s = wave_sum(s);

  int my_id = 0;
  if (forced) {
    int e = (lane < k) ? forced[(int64_t)t * k + lane] : 0;
    bool bad = lane < k && (e < 0 || e >= E);
    bool dup = false;
    for (int j = 0; j < k; ++j) {
      const int other = __shfl(e, j, kWave);
      if (lane < k && j != lane && other == e) dup = true;
    }
    const bool any_bad = __any(bad);
    const bool any_dup = __any(dup);
    if (any_bad || any_dup) {
      if (lane == 0) atomic_or_err(err, (any_bad ? kErrBadId : 0u) | (any_dup ? kErrDupId : 0u));
      e = lane;
    }
    my_id = e;
  } else {
    uint32_t removed = 0;
    for (int r = 0; r < k; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < kMaxV; ++i) {
        const int e = i * kWave + lane;
        if (e < E && !((removed >> i) & 1u)) {
          const uint64_t key = rank_key(v[i], e);
          best = key > best ? key : best;
        }
      }
      best = wave_max_u64(best);  // DPP network: no LDS round trips
      const int id = (int)(~(uint32_t)best);
      if (lane == (id & (kWave - 1))) removed |= 1u << (id / kWave);
      if (lane == r) my_id = id;
    }
  }
  float my_w = 0.0f;
  if (lane < k) my_w = expf(lg[my_id] - mx) / s;
  if (renorm) {
    const float tot = wave_sum(lane < k ? my_w : 0.0f);
    my_w = my_w / tot;
  }
  if (lane < k) {
    ids[(int64_t)t * k + lane] = my_id;
    w[(int64_t)t * k + lane] = my_w;
  }
}

void launch_router_logits(const RouterArgs& a, hipStream_t stream) {
  dim3 g1((a.E + kRtExp - 1) / kRtExp, (a.T + kRtTok - 1) / kRtTok);
  hipLaunchKernelGGL(router_logits_kernel, g1, dim3(64), 0, stream, a.x, a.wr, a.T, a.E, a.H,
                     a.logits, a.exact_always);
}

void launch_router_topk(const RouterArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(router_topk_kernel, dim3(a.T), dim3(64), 0, stream, a.logits, a.T, a.E,
                     a.k, a.renorm, a.forced, a.ids, a.w, a.err);
}

}  // namespace moe
