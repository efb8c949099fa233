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
//   1. every FP16 x FP16 product is exact in FP32 (and FP64); products are
//      summed in FP64 together with S = sum |p|.  Every product, and so every
//      partial sum, is an integer multiple of 2^-48, and every partial sum is
//      at most S in magnitude: with S below 2^5 = 2^53 * 2^-48 no FP64
//      addition rounds, the FP64 sum is the exact sum and its FP32 rounding is
//      the logit (kExactSumBound).  Otherwise S bounds the FP64 error, and the
//      FP32 rounding of the FP64 sum is accepted when the whole error interval
//      rounds to the same FP32 value (it lies strictly between that value's
//      two rounding midpoints).  Shapes with a multiple of 16 experts run this
//      tier on the FP64 matrix cores;
//   2. otherwise the sum is recomputed exactly as a 128-bit fixed-point
//      integer (unit 2^-48) and rounded once.
#include "common.hpp"
#include "launch.hpp"
#include "exact_dot.hpp"
#include "topk_wave.hpp"

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
    if (r != 0.0f && isfinite(r) && isfinite(s) && isfinite(asum)) {
      const double rd = (double)r;
      const double m_lo = 0.5 * (rd + (double)nextafterf(r, -INFINITY));
      const double m_hi = 0.5 * (rd + (double)nextafterf(r, INFINITY));
      if (asum < kExactSumBound || (s - eps > m_lo && s + eps < m_hi)) {
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

constexpr int kTopkMaxK = 16;  // largest top-k a context accepts

// LDS scratch of one wave's top-k (KV = ceil(E / 64) keys per lane).
template <int KV>
struct TopkScratch {
  alignas(16) uint64_t scr[kWave];                  // lane maxima (rank scratch)
  alignas(16) uint64_t cand[kTopkMaxK * KV + 2];    // keys at or above the bound
  uint64_t top[kTopkMaxK];                          // keys of ranks 0 .. k-1
};

// Softmax + top-k (or the forced ids) of one token, by one wave.  lg holds the
// token's E logits (global memory or LDS); KV = ceil(E / 64) logits per lane.
// Selection: lane l holds the keys of experts l + 64 i (one 64-bit key per
// expert, ordered like (logit desc, id asc) by one unsigned compare).  The
// rank of each lane's largest key among the 64 lane maxima takes one pass of
// comparisons; the lane maximum of rank k-1 bounds the k-th largest key from
// below (the k lanes above it hold k keys at least as large), so the keys at
// or above it -- at most k lanes x KV keys -- contain the top k, which are
// ranked exactly.  With KV = 1 the lane maxima are the keys themselves.
template <int KV>
__device__ __forceinline__ void topk_token(const float* lg, int t, int E, int k, int renorm,
                                           const int32_t* __restrict__ forced,
                                           int32_t* __restrict__ ids, float* __restrict__ w,
                                           uint32_t* __restrict__ err, TopkScratch<KV>& ts, int lane) {
  float v[KV];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < KV; ++i) {
    const int e = i * kWave + lane;
    v[i] = (e < E) ? lg[e] : -INFINITY;
    mx = fmaxf(mx, v[i]);
  }
  mx = wave_max(mx);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < KV; ++i)
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
    uint64_t kv[KV];
    uint64_t mk = 0;  // 0: a lane without experts (never selected, k <= E)
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int e = i * kWave + lane;
      kv[i] = e < E ? sel_key(v[i], e) : 0ull;
      mk = kv[i] > mk ? kv[i] : mk;
    }
    const int r = wave_rank64(mk, ts.scr, lane);
    if (KV == 1) {
      if (r < k) ts.top[r] = mk;
    } else {
      const int tl = __builtin_ctzll(__ballot(r == k - 1));  // exactly one lane
      const uint64_t th = ((uint64_t)rdlane((uint32_t)(mk >> 32), tl) << 32) | rdlane((uint32_t)mk, tl);
      const uint64_t below = (1ull << lane) - 1ull;
      int n = 0;
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const bool c = kv[i] >= th;  // empty keys (0) never qualify
        const uint64_t bal = __ballot(c);
        if (c) ts.cand[n + __popcll(bal & below)] = kv[i];
        n += __popcll(bal);
      }
      if (lane == 0) ts.cand[n] = 0ull;  // read (never counted) when n is odd
      wave_top_list(ts.cand, n, k, ts.top, lane);
    }
    if (lane < k) my_id = key_id(ts.top[lane]);
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

// grid T, block 64: softmax + top-k (or forced ids) for one token per wave.
__global__ __launch_bounds__(64) void router_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int renorm,
                                                         const int32_t* __restrict__ forced,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w,
                                                         uint32_t* __restrict__ err) {
  (void)T;
  const int t = blockIdx.x;
  __shared__ TopkScratch<16> ts;
  topk_token<16>(logits + (int64_t)t * E, t, E, k, renorm, forced, ids, w, err, ts, threadIdx.x);  // E <= 1024
}

// ---- FP64 matrix-core logits -----------------------------------------------------
// The certified tier on v_mfma_f64_16x16x4_f64, in two launches.
//
// router_partial_kernel: every FP16 value is exact in FP64 and so is every
// product (22 significant bits), so the only rounding is in the accumulation.
// Block (x, y, z) covers the 16x16 tile of tokens 16y.., experts 16x.. over
// the K range [z*4*KR, (z+1)*4*KR); its wave w takes the KR-wide part w of
// that range.  Lane (r, q) = (lane % 16, lane / 16) loads 8 consecutive K of
// token row r and of expert row r; MFMA (c, e) takes K index 32c + 8q + e from
// lane group q for both operands, so A and B see the same permutation of K
// and the tile is the plain dot product.  The four wave tiles are added in
// LDS in wave order and written as the block's FP64 partial, together with
// the partial of |x_i| |w_i| (FP16 matrix cores, FP32 accumulation: every
// product is exact and every rounding of these positive sums is below 2^-24
// of the sum, so the partial is within a relative 2^-16 of the exact one).
//
// router_select_kernel (one block per token, one wave per 64 experts, at
// least 4 waves): adds the partials of the K blocks in order and certifies
// each logit with S = sum |x_i w_i| (the added |x| |w| partials):
//   * every FP16 value is an integer multiple of 2^-24, so every product is
//     one of 2^-48, and so is every partial sum.  While a partial sum stays
//     below 2^53 * 2^-48 = 2^5 in magnitude it is representable in FP64, so
//     no addition rounds; every partial sum of either chain is bounded by the
//     sum of |x_i w_i| over its terms.  So when S < 2^5 both FP64 sums are
//     exact, and the FP32 rounding of the logit's sum is the logit
//     (kExactSumBound).
//   * otherwise every rounding has an error of at most 2^-53 of the sum it
//     produces, which is at most the sum of |x_i w_i| over that sum's terms.
//     A wave's two chains (one per product parity) take at most KR / 2
//     roundings each over disjoint terms, so together at most
//     KR / 2 * 2^-53 * S_wave (S_wave: the sum of |x_i w_i| over the wave's K
//     range); the addition of the two chains, 3 additions in the block and
//     KB - 1 over the K blocks add at most (1 + 3 + KB - 1) * 2^-53 * S, so
//     the error is below (KR / 2 + KB + 3) * 2^-53 * S (one more unit covers
//     the second-order growth of the partial sums; the factor 1 + 2^-12 covers
//     the error of the computed S).  The logit is certified when the interval of
//     half-width (KR / 2 + KB + 4) * 2^-53 * S around the FP64 sum lies
//     strictly between the rounding midpoints of its FP32 rounding.
// The block's waves then compute each logit that neither test certifies
// exactly, every wave the 128-bit fixed-point sum of one K slice, added
// exactly and rounded once.  Softmax and top-k follow.
typedef double d4 __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
constexpr int kRmTile = 16;  // tokens and experts per MFMA tile
constexpr int kRmWaves = 4;  // K parts per block
constexpr int kRmMaxKB = 8;  // K blocks

template <int KR>
__global__ __launch_bounds__(kRmWaves * kWave) void router_partial_kernel(RouterArgs a, double* __restrict__ part,
                                                                          double* __restrict__ pabs) {
  __shared__ double sp[kRmWaves][kRmTile * kRmTile];
  __shared__ double sa[kRmWaves][kRmTile * kRmTile];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int T = a.T, E = a.E, H = a.H;
  const int e0 = blockIdx.x * kRmTile, t0 = blockIdx.y * kRmTile, kb = blockIdx.z;
  const int k0 = (kb * kRmWaves + wv) * KR;
  const int tr = min(t0 + r, T - 1);
  const uint16_t* xa = a.x + (int64_t)tr * H + k0 + 8 * q;
  const uint16_t* wb = a.wr + (int64_t)(e0 + r) * H + k0 + 8 * q;
  constexpr int NC = KR / 32;  // 32-wide K chunks, all loaded up front
  uint4 av[NC], bv[NC];
  if (a.hres) {
    // x = fp16(RMSNorm(h)) of the lane's chunks, from the residual and its
    // sums of squares; the blocks of expert tile 0 write x for the later
    // kernels (every (token, K chunk) once)
    const float* hr = a.hres + (int64_t)tr * H + k0 + 8 * q;
    float4 hv[NC][2];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      hv[c][0] = *reinterpret_cast<const float4*>(hr + 32 * c);
      hv[c][1] = *reinterpret_cast<const float4*>(hr + 32 * c + 4);
      bv[c] = ldg_u4(wb + 32 * c);
    }
    float tot = 0.0f;
    for (int i = 0; i < a.nssq; ++i) tot += a.ssq[(int64_t)tr * a.nssq + i];
    const float rr = 1.0f / sqrtf(tot / (float)H + 1e-5f);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float f[8] = {hv[c][0].x, hv[c][0].y, hv[c][0].z, hv[c][0].w,
                          hv[c][1].x, hv[c][1].y, hv[c][1].z, hv[c][1].w};
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const _Float16 lo = (_Float16)(f[2 * e] * rr), hi = (_Float16)(f[2 * e + 1] * rr);
        w4[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      av[c] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      if (blockIdx.x == 0 && t0 + r < T)
        *reinterpret_cast<uint4*>(a.xw + (int64_t)tr * H + k0 + 8 * q + 32 * c) = av[c];
    }
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      av[c] = *reinterpret_cast<const uint4*>(xa + 32 * c);
      bv[c] = ldg_u4(wb + 32 * c);
    }
  }
  // two independent accumulation chains (even and odd e), added at the end
  d4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
  // sum of |x| |w| on the FP16 matrix cores (lane (r, q) holds K 32c + 8q + e
  // of token row r and expert row r, which is the A and B fragment layout of
  // v_mfma_f32_16x16x32_f16; subnormal inputs are kept)
  f4v sab = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint32_t au[4] = {av[c].x, av[c].y, av[c].z, av[c].w};
    const uint32_t bu[4] = {bv[c].x, bv[c].y, bv[c].z, bv[c].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double xv = (double)half_bits_to_float((uint16_t)(au[e >> 1] >> (16 * (e & 1))));
      const double wvv = (double)half_bits_to_float((uint16_t)(bu[e >> 1] >> (16 * (e & 1))));
      if (e & 1)
        acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(xv, wvv, acc1, 0, 0, 0);
      else
        acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(xv, wvv, acc0, 0, 0, 0);
    }
    const uint4 xa_abs = make_uint4(av[c].x & 0x7fff7fffu, av[c].y & 0x7fff7fffu, av[c].z & 0x7fff7fffu,
                                    av[c].w & 0x7fff7fffu);
    const uint4 wb_abs = make_uint4(bv[c].x & 0x7fff7fffu, bv[c].y & 0x7fff7fffu, bv[c].z & 0x7fff7fffu,
                                    bv[c].w & 0x7fff7fffu);
    sab = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8v, xa_abs), __builtin_bit_cast(h8v, wb_abs),
                                                  sab, 0, 0, 0);
  }
  const d4 acc = acc0 + acc1;
  // lane holds D[token q + 4i][expert r] of the FP64 MFMA and D[token 4q + i]
  // [expert r] of the FP16 one
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sp[wv][(q + 4 * i) * kRmTile + r] = acc[i];
    sa[wv][(4 * q + i) * kRmTile + r] = (double)sab[i];
  }
  __syncthreads();
  // one output per thread: tid = 16 * token + expert
  const int ti = tid >> 4, ei = tid & 15;
  if (t0 + ti < T) {
    const int64_t o = ((int64_t)kb * T + t0 + ti) * E + e0 + ei;
    part[o] = ((sp[0][tid] + sp[1][tid]) + sp[2][tid]) + sp[3][tid];
    pabs[o] = ((sa[0][tid] + sa[1][tid]) + sa[2][tid]) + sa[3][tid];
  }
}

// grid T, block 64 * max(ceil(E / 64), 4): wave w < KV = ceil(E / 64)
// certifies experts 64w .. 64w + 63 of the token; the logits it cannot
// certify are then computed exactly by all waves of the block together (each
// one K slice, exact integer partial sums added in LDS); then wave 0 does
// softmax and top-k over all of them (KV logits per lane there).
template <int KV>
constexpr int select_waves() { return KV < 4 ? 4 : KV; }
template <int KV>
__global__ __launch_bounds__(select_waves<KV>() * 64) void router_select_kernel(RouterArgs a,
                                                                              const double* __restrict__ part,
                                                                              const double* __restrict__ pabs,
                                                                              int KB, int KR) {
  constexpr int NW = select_waves<KV>();
  __shared__ float slg[KV * kWave];
  __shared__ TopkScratch<KV> ts;
  __shared__ uint64_t unc[KV];     // per certifying wave: lanes whose logit was not certified
  __shared__ uint64_t xlo[NW], xhi[NW];  // exact partial sums of one logit, per wave
  const int t = blockIdx.x, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int T = a.T, E = a.E;
  if (wv < KV) {
    const int e = wv * kWave + lane;
    const int ec = min(e, E - 1);
    // every partial is loaded before any is added (at most kRmMaxKB of each)
    double sv[kRmMaxKB], av[kRmMaxKB];
#pragma unroll
    for (int kb = 0; kb < kRmMaxKB; ++kb) {
      sv[kb] = kb < KB ? part[((int64_t)kb * T + t) * E + ec] : 0.0;
      av[kb] = kb < KB ? pabs[((int64_t)kb * T + t) * E + ec] : 0.0;
    }
    double s = 0.0, sab = 0.0;
#pragma unroll
    for (int kb = 0; kb < kRmMaxKB; ++kb)
      if (kb < KB) {  // fixed order
        s += sv[kb];
        sab += av[kb];
      }
    bool certified = false;
    if (e < E) {
      const float rr = (float)s;  // round to nearest even
      if (rr != 0.0f && isfinite(rr) && isfinite(s) && isfinite(sab)) {
        if (sab < kExactSumBound) {
          certified = true;  // the FP64 sum is the exact sum: rr is its FP32 rounding
        } else {
          const double eps = (double)(KR / 2 + KB + 4) * 0x1p-53 * (sab * (1.0 + 0x1p-12));
          const double rd = (double)rr;
          const double m_lo = 0.5 * (rd + (double)nextafterf(rr, -INFINITY));
          const double m_hi = 0.5 * (rd + (double)nextafterf(rr, INFINITY));
          certified = s - eps > m_lo && s + eps < m_hi;
        }
      }
      if (certified) slg[e] = rr;
    }
    const uint64_t m = __ballot(e < E && !certified);
    if (lane == 0) unc[wv] = m;
  }
  __syncthreads();
  // the uncertified logits, one at a time (block-uniform loop): wave w adds
  // the exact products of its K slice, and thread 0 adds the waves' sums
  {
    const int H = a.H;
    const int ks = ((H / 8 + NW - 1) / NW) * 8;  // K slice per wave (multiple of 8)
    const int k0 = min(H, wv * ks), k1 = min(H, k0 + ks);
    const uint16_t* xr = a.x + (int64_t)t * H;
    for (int w = 0; w < KV; ++w) {
      uint64_t m = unc[w];
      while (m) {
        const int ee = w * kWave + __builtin_ctzll(m);
        m &= m - 1;
        const __int128 ps = exact_partial_wave(xr, a.wr + (int64_t)ee * H, k0, k1, lane);
        if (lane == 0) {
          xlo[wv] = (uint64_t)ps;
          xhi[wv] = (uint64_t)(ps >> 64);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
          __int128 S = 0;
          for (int i = 0; i < NW; ++i) S += (__int128)(((unsigned __int128)xhi[i] << 64) | (unsigned __int128)xlo[i]);
          slg[ee] = round_i128_to_f32(S, -48);
        }
        __syncthreads();
      }
    }
  }
  if (wv < KV) {
    const int e = wv * kWave + lane;
    if (e < E) a.logits[(int64_t)t * E + e] = slg[e];
  }
  if (wv == 0) topk_token<KV>(slg, t, E, a.k, a.renorm, a.forced, a.ids, a.w, a.err, ts, lane);
}

// K per wave of the matrix-core router (0: the shape does not take it).
static int mfma_router_kr(int H, int E) {
  if (E % kRmTile != 0 || E > 1024) return 0;
  for (int kr = 128; kr >= 64; kr /= 2)
    if (H % (kRmWaves * kr) == 0 && H / (kRmWaves * kr) <= kRmMaxKB) return kr;
  return 0;
}

size_t router_scratch_bytes(int max_tokens, int E, int H) {
  const int kr = mfma_router_kr(H, E);
  if (!kr) return 0;
  const int64_t KB = H / (kRmWaves * kr);
  return (size_t)(2 * KB * (int64_t)max_tokens * E * 8);
}

bool router_takes_mfma(int H, int E, int exact_always) { return !exact_always && mfma_router_kr(H, E) != 0; }

// Logits + softmax/top-k.  Returns false (nothing launched) when the shape
// does not take the matrix-core router.
bool launch_router(const RouterArgs& a, double* scratch, hipStream_t stream) {
  const int kr = mfma_router_kr(a.H, a.E);
  if (a.exact_always || !kr || !scratch) return false;
  const int KB = a.H / (kRmWaves * kr);
  double* part = scratch;
  double* pabs = part + (int64_t)KB * a.T * a.E;
  dim3 g(a.E / kRmTile, (a.T + kRmTile - 1) / kRmTile, KB);
  if (kr == 128)
    hipLaunchKernelGGL((router_partial_kernel<128>), g, dim3(kRmWaves * kWave), 0, stream, a, part, pabs);
  else
    hipLaunchKernelGGL((router_partial_kernel<64>), g, dim3(kRmWaves * kWave), 0, stream, a, part, pabs);
  const int kv = (a.E + kWave - 1) / kWave;
  const dim3 gs(a.T);
  if (kv == 1)
    hipLaunchKernelGGL((router_select_kernel<1>), gs, dim3(kWave * select_waves<1>()), 0, stream, a, part, pabs, KB,
                       kr);
  else if (kv == 2)
    hipLaunchKernelGGL((router_select_kernel<2>), gs, dim3(kWave * select_waves<2>()), 0, stream, a, part, pabs, KB,
                       kr);
  else if (kv <= 4)
    hipLaunchKernelGGL((router_select_kernel<4>), gs, dim3(kWave * select_waves<4>()), 0, stream, a, part, pabs, KB,
                       kr);
  else if (kv <= 8)
    hipLaunchKernelGGL((router_select_kernel<8>), gs, dim3(kWave * select_waves<8>()), 0, stream, a, part, pabs, KB,
                       kr);
  else
    hipLaunchKernelGGL((router_select_kernel<16>), gs, dim3(kWave * select_waves<16>()), 0, stream, a, part,
                       pabs, KB, kr);
  return true;
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
