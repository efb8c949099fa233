// Fused decode path: one persistent kernel runs every layer of a stack step
// for a small batch (a few tokens).
//
// Per layer it does what the separate kernels do -- RMSNorm, router logits,
// softmax + top-k, grouping, gate/up + SwiGLU, down, rank-ordered combine into
// the FP32 residual -- in three phases separated by grid-wide barriers:
//   A  every block normalises the residual into LDS; router logits
//      (exact-rounded, see exact_dot.hpp) are spread over all waves;
//   B  every block redundantly selects the experts from the logits, groups the
//      (token, rank) pairs by expert, then runs gate/up tiles of 16 rows: the
//      8 waves of a block split {gate, up} x 4 K-quarters, each wave streams
//      16-byte INT4 chunks of 16 rows, decodes them in registers and feeds
//      v_mfma_f32_16x16x32_f16 with the tokens as the A operand (rows = tokens,
//      zero-padded to 16); K-quarter partials are summed in LDS, SwiGLU applied;
//   C  every working block stages the FP16 intermediates of all pairs in LDS,
//      then takes a tile of 16 output rows: each wave runs the down projection
//      of active experts on MFMA, and the block sums the per-(token, rank) rows
//      in rank order and adds them to the residual.
// INT4 weights are read once per step, straight from their packed form (the
// experts are executed from compact INT4 with FP16 group scales, "Horizon
// RunMap", "Architecture invariants").  Loads that do not depend on the data
// of the phase being waited for are issued before the barrier wait: the next
// layer's router rows before barrier A, the first down tile's weights before
// barrier C.
//
// MFMA 16x16x32 operand layout on gfx950 (checked on the device): lane l holds
// A[l%16][8*(l/16)+e], B[8*(l/16)+e][l%16] (e = 0..7) and D[4*(l/16)+r][l%16].
// Each lane loads 16 contiguous bytes of one weight row = 32 consecutive K,
// i.e. one dword per MFMA step; the K index of MFMA step st, lane group q,
// element e is kb + 32q + 8st + e, and the activations are read with the same
// mapping, so the contraction covers [kb, kb+128) = one scale group.
//
// Cross-block data (router logits, FP16 intermediates, the residual) is only
// ever accessed with device-coherent loads and stores (agent-scope atomic
// accesses: write-through, never served from a stale L2 line of another XCD);
// weights and router rows are read-only during the kernel and stay cacheable.
// The grid barrier is a flag per block: every wave waits for its stores to
// complete, then one thread stores the block's barrier count to its flag; a
// waiting block polls all flags with coherent loads.  No L2 writeback or
// invalidation is needed, so the weights and code stay in L2 across barriers.
// Spinning is bounded; on timeout the block sets an error bit and continues,
// so the kernel always terminates.  The grid never exceeds the number of
// compute units, so all blocks are resident together.
#include "common.hpp"
#include "exact_dot.hpp"
#include "launch.hpp"

namespace moe {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kFT = 512;
constexpr int kFW = kFT / kWave;  // 8 waves
constexpr uint32_t kSpinLimit = 1u << 18;  // ~0.3 s of polling, then give up

struct FusedSmem {
  _Float16 x[kFMaxT * 2048];                 // normalised tokens
  _Float16 hst[kFStageHalves];               // phase C: FP16 intermediates of all pairs
  union {
    float logit[kFMaxTE];                    // phase B: logits of the step
    float red[2][kFW][256];                  // phase B: K-quarter partial tiles (2 tasks)
    float y[kFMaxP + kFMaxT][16];            // phase C: per-(token, rank) output rows
  } u;
  float cval[kFMaxT][kFMaxCand];
  int cid[kFMaxT][kFMaxCand];
  int prank[kFW][kWave], prank2[kFW][kWave];  // partial ranks per wave
  float psum[kFMaxT][kFW], pmax[kFMaxT][kFW];
  float rmax[kFMaxT], rsum[kFMaxT];
  int ids[kFMaxP];
  float w[kFMaxP];
  int act_slot[kFMaxP + 1];
  int pair_of[(kFMaxP + 1) * kFMaxT];        // [active][token] -> pair, -1
  int nact;
  float part[kFW];
};

__device__ __forceinline__ void stamp(const FusedArgs& a, int l, int ev) {
  if (a.stamps && threadIdx.x == 0) {
    const int64_t i = (int64_t)blockIdx.x * kStampStride + (l - a.l0) * kStampsPerLayer + ev;
    a.stamps[i] = __builtin_amdgcn_s_memrealtime();
    a.stamps[(int64_t)gridDim.x * kStampStride + i] = __builtin_amdgcn_s_memtime();
  }
}

// Device-coherent accesses to data exchanged between blocks.
__device__ __forceinline__ float ld_coh(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_coh(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coh(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival half of the grid barrier (all threads call it): every wave waits
// until its coherent stores have completed before the flag is raised.
__device__ __forceinline__ void barrier_arrive(uint32_t* flags, uint32_t target) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(&flags[blockIdx.x], target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waiting half (all threads call it).
__device__ __forceinline__ void barrier_wait(uint32_t* flags, uint32_t target, uint32_t* err) {
  if (threadIdx.x < kWave) {
    const int nb = gridDim.x;
    uint32_t spins = 0;
    while (true) {
      bool mine = true;
      for (int i = threadIdx.x; i < nb; i += kWave) {
        const uint32_t f = __hip_atomic_load(&flags[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((int32_t)(f - target) < 0) mine = false;
      }
      if (__all(mine)) break;
      if (++spins > kSpinLimit) {
        if (threadIdx.x == 0) atomic_or_err(err, kErrBarrier);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
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

__device__ __forceinline__ float beats(float v, int e, float w, int f) {
  // 1 when (w, f) ranks before (v, e): larger logit, then smaller id
  return (w > v || (w == v && f < e)) ? 1.0f : 0.0f;
}

__device__ __forceinline__ float bcast(float v, int j) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
}

// How many of the 64 (value, id) pairs held one per lane in (wreg, freg)
// rank before (v, e); lanes with id < 0 hold no pair.  Each lane's pair is
// broadcast in turn with v_readlane (no LDS round trips).
__device__ __forceinline__ int wave_beating(float v, int e, float wreg, int freg) {
  int rank = 0;
#pragma unroll 8
  for (int j = 0; j < kWave; ++j) {
    const float w = bcast(wreg, j);
    const int f = __builtin_amdgcn_readlane(freg, j);
    rank += (f >= 0 && (w > v || (w == v && f < e))) ? 1 : 0;
  }
  return rank;
}

__device__ __forceinline__ int wave_rank(float v, int e) { return wave_beating(v, e, v, e); }

// Router row of one logit item, 8 FP16 per lane per 512-wide chunk (H <= 2048).
template <int H>
__device__ __forceinline__ void load_router_row(const uint16_t* row, int lane, uint4 (&q)[H / 512]) {
#pragma unroll
  for (int c = 0; c < H / 512; ++c) q[c] = *reinterpret_cast<const uint4*>(row + c * 512 + lane * 8);
}

// Certified FP64 dot of LDS x with a router row already in registers; same
// contract as certified_dot_wave (exact fallback reads the row again).
template <int H>
__device__ float certified_dot_regs(const _Float16* x, const uint4 (&q)[H / 512], const uint16_t* row,
                                    int lane, int exact_always) {
  if (!exact_always) {
    double acc = 0.0, asum = 0.0;
#pragma unroll
    for (int c = 0; c < H / 512; ++c) {
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
    for (int o = kWave / 2; o > 0; o >>= 1) {
      acc += __shfl_xor(acc, o, kWave);
      asum += __shfl_xor(asum, o, kWave);
    }
    const int depth = 8 * (H / 512) + 6;
    const double eps = (double)(depth + 2) * 0x1p-52 * asum;
    const float r = (float)acc;
    if (r != 0.0f && isfinite(r) && isfinite(acc)) {
      const double rd = (double)r;
      const double m_lo = 0.5 * (rd + (double)nextafterf(r, -INFINITY));
      const double m_hi = 0.5 * (rd + (double)nextafterf(r, INFINITY));
      if (acc - eps > m_lo && acc + eps < m_hi) return r;
    }
  }
  return exact_dot_wave(reinterpret_cast<const uint16_t*>(x), row, H, lane);
}

template <int H, int I>
__global__ __launch_bounds__(kFT) void fused_decode_kernel(FusedArgs a) {
  __shared__ FusedSmem s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nb = gridDim.x, b = blockIdx.x;
  const int T = a.T, E = a.E, k = a.k;
  const int P = T * k;
  const int gw = b * kFW + wv, nw = nb * kFW;
  const int m = lane & 15, lg = lane >> 4;
  constexpr int KQ = H / 4;      // K per quarter in gate/up
  constexpr int GQ = KQ / 128;   // scale groups per quarter
  constexpr int GD = I / 128;    // scale groups of the down projection
  constexpr int NR = H / 512;    // router chunks per lane
  uint32_t target = __hip_atomic_load(&a.flags[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  uint4 rq[NR];                  // router row of this wave's first logit item
  if (gw < T * E) load_router_row<H>(a.layers[a.l0].router + (int64_t)(gw % E) * H, lane, rq);

  for (int l = a.l0; l < a.l1; ++l) {
    const FusedLayer L = a.layers[l];
    stamp(a, l, 0);

    // ---------------- phase A: RMSNorm (every block), router logits ----------------
    for (int t = 0; t < T; ++t) {
      const float* hr = a.h + (int64_t)t * H;
      float hv[H / kFT];
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < H / kFT; ++i) {
        hv[i] = ld_coh(hr + tid + i * kFT);
        ss += hv[i] * hv[i];
      }
      ss = wave_sum_xor(ss, kWave);
      if (lane == 0) s.part[wv] = ss;
      __syncthreads();
      float tot = 0.0f;
#pragma unroll
      for (int w = 0; w < kFW; ++w) tot += s.part[w];
      const float r = 1.0f / sqrtf(tot / (float)H + 1e-5f);
#pragma unroll
      for (int i = 0; i < H / kFT; ++i) {
        const _Float16 xv = (_Float16)(hv[i] * r);
        s.x[t * H + tid + i * kFT] = xv;
        if (b == 0 && a.x_trace)
          reinterpret_cast<_Float16*>(a.x_trace)[((int64_t)l * T + t) * H + tid + i * kFT] = xv;
      }
      __syncthreads();
    }
    stamp(a, l, 1);
    for (int item = gw; item < T * E; item += nw) {
      const int t = item / E, e = item - t * E;
      const uint16_t* row = L.router + (int64_t)e * H;
      if (item != gw) load_router_row<H>(row, lane, rq);
      const float r = certified_dot_regs<H>(s.x + t * H, rq, row, lane, a.exact_always);
      if (lane == 0) st_coh(a.logits + item, r);
    }
    stamp(a, l, 2);
    barrier_arrive(a.flags, ++target);
    barrier_wait(a.flags, target, a.err);
    stamp(a, l, 3);

    // ---------------- phase B: selection, grouping, gate/up + SwiGLU ----------------
    for (int i = tid; i < T * E; i += kFT) s.u.logit[i] = ld_coh(a.logits + i);
    for (int i = tid; i < (kFMaxP + 1) * kFMaxT; i += kFT) s.pair_of[i] = -1;
    __syncthreads();
    stamp(a, l, 4);
    // selection: rank of every expert among its chunk of 64 (all waves share
    // the comparisons), then among the chunks' candidates; branch-free compares
    // of LDS-broadcast values, partial ranks summed in LDS in a fixed order
    if (a.forced) {
      if (wv == 0) {
        const int p = lane;
        const bool valid = p < P;
        const int t = valid ? p / k : 0;
        int e = valid ? a.forced[((int64_t)l * T) * k + p] : 0;
        const bool bad = valid && (e < 0 || e >= E);
        bool dup = false;
        for (int q = 0; q < P; ++q) {
          const int other = __shfl(e, q, kWave);
          dup |= valid && q != p && q / k == t && other == e;
        }
        // a token with any bad or repeated id gets ids 0..k-1
        const uint64_t badm = __ballot(bad || dup);
        const uint64_t bm = __ballot(bad), dm = __ballot(dup);
        bool tok_bad = false;
        for (int j = 0; j < k; ++j) tok_bad |= valid && ((badm >> (t * k + j)) & 1ull);
        if (lane == 0 && badm) atomic_or_err(a.err, (bm ? kErrBadId : 0u) | (dm ? kErrDupId : 0u));
        if (valid) s.ids[p] = tok_bad ? (p - t * k) : e;
      }
    } else {
      const int nch = E / kWave;
      const int nrank = T * nch;
      int wpu = 1;                        // waves sharing one (token, chunk) unit
      while (wpu * 2 * nrank <= kFW) wpu *= 2;
      const int span = kWave / wpu;
      for (int r0 = 0; r0 < nrank; r0 += kFW / wpu) {
        const int u = r0 + wv / wpu, sl = wv % wpu;
        const int t = u / nch, c = u - (u / nch) * nch;
        const bool on = u < nrank;
        const float vi = on ? s.u.logit[t * E + c * kWave + lane] : 0.0f;
        int pr = 0;
        if (on) {
          const float* row = s.u.logit + t * E + c * kWave + sl * span;
#pragma unroll 8
          for (int jj = 0; jj < span; ++jj) {
            const float vj = row[jj];
            const int j = sl * span + jj;
            pr += (int)(vj > vi) | ((int)(vj == vi) & (int)(j < lane));
          }
        }
        s.prank[wv][lane] = pr;
        __syncthreads();
        if (on && sl == 0) {
          int rank = 0;
          for (int q = 0; q < wpu; ++q) rank += s.prank[wv + q][lane];
          const int e = c * kWave + lane;
          if (rank < k) {
            if (nch == 1) {
              s.ids[t * k + rank] = e;
            } else {
              s.cval[t][c * k + rank] = vi;   // chunk c's candidates in rank order
              s.cid[t][c * k + rank] = e;
            }
          }
        }
        __syncthreads();
      }
      if (nch > 1) {
        // nch*k <= 128 candidates per token: lanes hold candidates lane, lane+64
        const int n = nch * k;
        int wpu2 = 1;
        while (wpu2 * 2 * T <= kFW) wpu2 *= 2;
        const int span2 = (n + wpu2 - 1) / wpu2;
        for (int t0 = 0; t0 < T; t0 += kFW / wpu2) {
          const int t = t0 + wv / wpu2, sl = wv % wpu2;
          const bool on = t < T;
          const int ca = lane, cb = lane + kWave;
          const float va = on && ca < n ? s.cval[t][ca] : 0.0f;
          const float vb = on && cb < n ? s.cval[t][cb] : 0.0f;
          const int ea = on && ca < n ? s.cid[t][ca] : 0x7fffffff;
          const int eb = on && cb < n ? s.cid[t][cb] : 0x7fffffff;
          int pa = 0, pb = 0;
          if (on) {
            const int j0 = sl * span2, j1 = min(n, j0 + span2);
            for (int j = j0; j < j1; ++j) {
              const float vj = s.cval[t][j];
              const int ej = s.cid[t][j];
              pa += (int)(vj > va) | ((int)(vj == va) & (int)(ej < ea));
              pb += (int)(vj > vb) | ((int)(vj == vb) & (int)(ej < eb));
            }
          }
          s.prank[wv][lane] = pa;
          s.prank2[wv][lane] = pb;
          __syncthreads();
          if (on && sl == 0) {
            int ra = 0, rb = 0;
            for (int q = 0; q < wpu2; ++q) {
              ra += s.prank[wv + q][lane];
              rb += s.prank2[wv + q][lane];
            }
            if (ca < n && ra < k) s.ids[t * k + ra] = ea;
            if (cb < n && rb < k) s.ids[t * k + rb] = eb;
          }
          __syncthreads();
        }
      }
    }
    __syncthreads();
    stamp(a, l, 5);
    // softmax denominators: the maximum is the first-ranked logit (reduced over
    // the block when the ids are forced); the sum of exp(l - max) is reduced
    // over the whole block in a fixed order
    if (a.forced) {
      for (int t = 0; t < T; ++t) {
        float mx = -INFINITY;
        for (int e = tid; e < E; e += kFT) mx = fmaxf(mx, s.u.logit[t * E + e]);
        for (int o = kWave / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
        if (lane == 0) s.pmax[t][wv] = mx;
      }
      __syncthreads();
    }
    for (int t = 0; t < T; ++t) {
      float mx = s.u.logit[t * E + s.ids[t * k]];
      if (a.forced) {
        mx = s.pmax[t][0];
#pragma unroll
        for (int w = 1; w < kFW; ++w) mx = fmaxf(mx, s.pmax[t][w]);
      }
      float sm = 0.0f;
      for (int e = tid; e < E; e += kFT) sm += expf(s.u.logit[t * E + e] - mx);
      sm = wave_sum_xor(sm, kWave);
      if (lane == 0) s.psum[t][wv] = sm;
      if (tid == 0) s.rmax[t] = mx;
    }
    __syncthreads();
    if (tid < T) {
      float tot = 0.0f;
#pragma unroll
      for (int w = 0; w < kFW; ++w) tot += s.psum[tid][w];
      s.rsum[tid] = tot;
    }
    __syncthreads();
    float wtmp = 0.0f;
    if (tid < P) {
      const int t = tid / k;
      wtmp = expf(s.u.logit[t * E + s.ids[tid]] - s.rmax[t]) / s.rsum[t];
      s.w[tid] = wtmp;
    }
    __syncthreads();
    if (tid < P) {
      if (a.renorm) {
        const int t = tid / k;
        float tot = 0.0f;
        for (int j = 0; j < k; ++j) tot += s.w[t * k + j];
        wtmp = wtmp / tot;
      }
      if (b == 0 && a.ids_trace) a.ids_trace[(int64_t)l * P + tid] = s.ids[tid];
      if (b == 0 && a.w_trace) a.w_trace[(int64_t)l * P + tid] = wtmp;
    }
    __syncthreads();
    if (tid < P) s.w[tid] = wtmp;
    // grouping: distinct experts in order of first appearance
    if (wv == 0) {
      const int p = lane;
      const bool valid = p < P;
      const int e = valid ? s.ids[p] : -1;
      int q0 = p;   // first pair naming the same expert (ids of one token are distinct)
      if (T > 1) {
#pragma unroll 8
        for (int q = kWave - 1; q >= 0; --q) {
          const int eq = s.ids[q];
          q0 = ((q < p) & (eq == e)) ? q : q0;
        }
      }
      const bool first = valid && q0 == p;
      const uint64_t fm = __ballot(first);
      const int ap = __popcll(fm & ((1ull << q0) - 1ull));
      if (first) {
        int slot = L.map ? L.map[e] : e;
        if (slot < 0) {
          atomic_or_err(a.err, kErrNotResident);
          slot = 0;
        }
        s.act_slot[ap] = slot;
      }
      if (valid) s.pair_of[ap * T + p / k] = p;
      const int U = __popcll(fm);
      if (a.has_shared && p < T) s.pair_of[U * T + p] = P + p;
      if (lane == 0) s.nact = U;
    }
    __syncthreads();
    stamp(a, l, 6);
    const int U = s.nact;
    const int nunits = U + (a.has_shared ? 1 : 0);
    {
      constexpr int RB = I / 16;
      const int ntask = nunits * RB;
      const int q4 = wv & 3, mat = wv >> 2;
      // two tasks per round so that both tiles' loads are in flight together
      for (int base = b; base < ntask; base += 2 * nb) {
        uint4 qv[2][GQ];
        float scl[2][GQ];
        int tau[2], trb[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int task = base + h * nb;
          tau[h] = -1;
          trb[h] = 0;
          if (task < ntask) {
            const int au = task / RB, rb = task - au * RB;
            tau[h] = au;
            trb[h] = rb;
            const uint8_t* blob = au < U ? L.store + (int64_t)s.act_slot[au] * a.blob_stride : L.shared;
            const int n = rb * 16 + m;
            const uint8_t* rowp = blob + a.lay.codes(mat) + (int64_t)n * (H / 2) + q4 * (KQ / 2) + lg * 16;
            const uint16_t* sc = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(mat)) +
                                 (int64_t)n * (H / 128) + q4 * GQ;
#pragma unroll
            for (int g = 0; g < GQ; ++g) {
              qv[h][g] = *reinterpret_cast<const uint4*>(rowp + g * 64);
              scl[h][g] = half_bits_to_float(sc[g]);
            }
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (tau[h] < 0) continue;
          f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int g = 0; g < GQ; ++g) {
            f4 ag = {0.f, 0.f, 0.f, 0.f};
            const int kb = q4 * KQ + g * 128 + 32 * lg;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              h8 av = {};
              if (m < T) av = *reinterpret_cast<const h8*>(s.x + m * H + kb + 8 * st);
              ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, decode_h8(dword_of(qv[h][g], st)), ag, 0, 0, 0);
            }
            acc += ag * scl[h][g];
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) s.u.red[h][wv][(4 * lg + r) * 16 + m] = acc[r];
        }
        __syncthreads();
        {
          const int h = tid >> 8;              // 2 x 256 threads: one task each
          const int e = tid & 255;
          const int i = e >> 4, j = e & 15;
          float hv = 0.0f;
          if (tau[h] >= 0 && i < T) {
            const float g = (s.u.red[h][0][e] + s.u.red[h][1][e]) + (s.u.red[h][2][e] + s.u.red[h][3][e]);
            const float u = (s.u.red[h][4][e] + s.u.red[h][5][e]) + (s.u.red[h][6][e] + s.u.red[h][7][e]);
            hv = g / (1.0f + expf(-g)) * u;
          }
          // rows j and j+1 (adjacent lanes) go out as one coherent 32-bit store
          const float hn = __shfl_down(hv, 1, kWave);
          if (tau[h] >= 0 && i < T && (j & 1) == 0) {
            const int p = s.pair_of[tau[h] * T + i];
            if (p >= 0) {
              const h2 pr = {(_Float16)hv, (_Float16)hn};
              st_coh(reinterpret_cast<uint32_t*>(a.hbuf + (int64_t)p * I + trb[h] * 16 + j),
                     __builtin_bit_cast(uint32_t, pr));
            }
          }
        }
        __syncthreads();
      }
    }
    stamp(a, l, 7);
    barrier_arrive(a.flags, ++target);
    // prefetch the first down tile's weights of this wave while waiting
    uint4 dq[GD];
    float dscl[GD];
    const int c_task0 = b;
    if (c_task0 < H / 16 && wv < nunits) {
      const int au = wv;
      const uint8_t* blob = au < U ? L.store + (int64_t)s.act_slot[au] * a.blob_stride : L.shared;
      const int n = c_task0 * 16 + m;
      const uint8_t* rowp = blob + a.lay.codes(2) + (int64_t)n * (I / 2) + lg * 16;
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(2)) + (int64_t)n * (I / 128);
#pragma unroll
      for (int g = 0; g < GD; ++g) {
        dq[g] = *reinterpret_cast<const uint4*>(rowp + g * 64);
        dscl[g] = half_bits_to_float(sc[g]);
      }
    }
    barrier_wait(a.flags, target, a.err);
    stamp(a, l, 8);

    // ---------------- phase C: down projection, rank-ordered combine ----------------
    if (b < H / 16) {
      // stage the FP16 intermediates of every (token, rank) pair and shared token
      const int rows = P + (a.has_shared ? T : 0);
      const int words = rows * I / 2;
      for (int c = tid; c < words; c += kFT)
        reinterpret_cast<uint32_t*>(s.hst)[c] = ld_coh(reinterpret_cast<const uint32_t*>(a.hbuf) + c);
      __syncthreads();
      for (int task = b; task < H / 16; task += nb) {
        const int n = task * 16 + m;
        for (int au = wv; au < nunits; au += kFW) {
          if (!(task == c_task0 && au == wv)) {
            const uint8_t* blob = au < U ? L.store + (int64_t)s.act_slot[au] * a.blob_stride : L.shared;
            const uint8_t* rowp = blob + a.lay.codes(2) + (int64_t)n * (I / 2) + lg * 16;
            const uint16_t* sc = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(2)) + (int64_t)n * (I / 128);
#pragma unroll
            for (int g = 0; g < GD; ++g) {
              dq[g] = *reinterpret_cast<const uint4*>(rowp + g * 64);
              dscl[g] = half_bits_to_float(sc[g]);
            }
          }
          const int pm = m < T ? s.pair_of[au * T + m] : -1;
          const _Float16* hrow = s.hst + (pm < 0 ? 0 : pm) * I;
          f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int g = 0; g < GD; ++g) {
            f4 ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              h8 av = {};
              if (pm >= 0) av = *reinterpret_cast<const h8*>(hrow + g * 128 + 32 * lg + 8 * st);
              ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, decode_h8(dword_of(dq[g], st)), ag, 0, 0, 0);
            }
            acc += ag * dscl[g];
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * lg + r;
            if (i < T) {
              const int p = s.pair_of[au * T + i];
              if (p >= 0) s.u.y[p][m] = acc[r];
            }
          }
        }
        __syncthreads();
        if (tid < T * 16) {
          const int t = tid >> 4, j = tid & 15;
          float o = 0.0f;
          for (int jj = 0; jj < k; ++jj) o += s.w[t * k + jj] * s.u.y[t * k + jj][j];
          if (a.has_shared) o += s.u.y[P + t][j];
          float* hp = a.h + (int64_t)t * H + task * 16 + j;
          st_coh(hp, ld_coh(hp) + o);
        }
        __syncthreads();
      }
    }
    stamp(a, l, 9);
    if (l + 1 < a.l1) {
      barrier_arrive(a.flags, ++target);
      // prefetch the next layer's router row of this wave's first logit item
      if (gw < T * E) load_router_row<H>(a.layers[l + 1].router + (int64_t)(gw % E) * H, lane, rq);
      barrier_wait(a.flags, target, a.err);
    }
    stamp(a, l, 10);
  }
}

bool fused_supported(int H, int I) { return H == 2048 && (I == 1024 || I == 512); }

void launch_fused_decode(const FusedArgs& a, int grid, hipStream_t stream) {
  if (a.I == 1024)
    hipLaunchKernelGGL((fused_decode_kernel<2048, 1024>), dim3(grid), dim3(kFT), 0, stream, a);
  else
    hipLaunchKernelGGL((fused_decode_kernel<2048, 512>), dim3(grid), dim3(kFT), 0, stream, a);
}

}  // namespace moe
