// Fused decode path: one persistent kernel runs every layer of a stack step
// for a small batch (T <= 8 tokens).
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
//   C  tiles of 16 output rows: each wave takes active experts, runs the down
//      projection on MFMA from the FP16 intermediate, the block sums the
//      per-(token, rank) rows in rank order and adds them to the residual.
// INT4 weights are read once per step, straight from their packed form (the
// experts are executed from compact INT4 with FP16 group scales, "Horizon
// RunMap", "Architecture invariants").
//
// MFMA 16x16x32 operand layout on gfx950 (checked on the device): lane l holds
// A[l%16][8*(l/16)+e], B[8*(l/16)+e][l%16] (e = 0..7) and D[4*(l/16)+r][l%16].
// Each lane loads 16 contiguous bytes of one weight row = 32 consecutive K,
// i.e. one dword per MFMA step; the K index of MFMA step st, lane group q,
// element e is kb + 32q + 8st + e, and the activations are read with the same
// mapping, so the contraction covers [kb, kb+128) = one scale group.
//
// The grid barrier is a flag per block: a block publishes its arrival by
// storing its barrier count (after a device-scope release fence) and waits
// until every flag has reached the count (then an acquire fence).  Spinning is
// bounded; on timeout the block sets an error bit and continues, so the kernel
// always terminates.  The grid never exceeds the number of compute units, so
// all blocks are resident together.
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
  _Float16 x[kFMaxT * 2048];  // normalised tokens
  union {
    float logit[kFMaxTE];           // phase B: logits of the step
    float red[kFW][256];            // phase B: K-quarter partial tiles
    float y[kFMaxP + kFMaxT][16];   // phase C: per-(token, rank) output rows
  } u;
  float cval[kFMaxT][kFMaxCand];
  int cid[kFMaxT][kFMaxCand];
  int ncand[kFMaxT];
  float rmax[kFMaxT], rsum[kFMaxT];
  int ids[kFMaxP];
  float w[kFMaxP];
  int act_slot[kFMaxP + 1];
  int pair_of[(kFMaxP + 1) * kFMaxT];  // [active][token] -> pair, -1
  int nact;
  float part[kFW];
};

__device__ __forceinline__ void grid_barrier(uint32_t* flags, uint32_t target, uint32_t* err) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    __hip_atomic_store(&flags[blockIdx.x], target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
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
      __builtin_amdgcn_s_sleep(2);
    }
    __threadfence();
  }
  __syncthreads();
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

template <int H, int I>
__global__ __launch_bounds__(kFT) void fused_decode_kernel(FusedArgs a) {
  __shared__ FusedSmem s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nb = gridDim.x, b = blockIdx.x;
  const int T = a.T, E = a.E, k = a.k;
  const int P = T * k;
  constexpr int KQ = H / 4;      // K per quarter in gate/up
  constexpr int GQ = KQ / 128;   // scale groups per quarter
  constexpr int GD = I / 128;    // scale groups of the down projection
  uint32_t target = __hip_atomic_load(&a.flags[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  for (int l = a.l0; l < a.l1; ++l) {
    const FusedLayer L = a.layers[l];

    // ---------------- phase A: RMSNorm (every block), router logits ----------------
    for (int t = 0; t < T; ++t) {
      const float* hr = a.h + (int64_t)t * H;
      float ss = 0.0f;
      for (int i = tid; i < H; i += kFT) ss += hr[i] * hr[i];
      ss = wave_sum_xor(ss, kWave);
      if (lane == 0) s.part[wv] = ss;
      __syncthreads();
      float tot = 0.0f;
#pragma unroll
      for (int w = 0; w < kFW; ++w) tot += s.part[w];
      const float r = 1.0f / sqrtf(tot / (float)H + 1e-5f);
      for (int i = tid; i < H; i += kFT) {
        const _Float16 xv = (_Float16)(hr[i] * r);
        s.x[t * H + i] = xv;
        if (b == 0 && a.x_trace)
          reinterpret_cast<_Float16*>(a.x_trace)[((int64_t)l * T + t) * H + i] = xv;
      }
      __syncthreads();
    }
    {
      const int gw = b * kFW + wv, nw = nb * kFW;
      for (int item = gw; item < T * E; item += nw) {
        const int t = item / E, e = item - t * E;
        const float r = certified_dot_wave(reinterpret_cast<const uint16_t*>(s.x + t * H),
                                           L.router + (int64_t)e * H, H, lane, a.exact_always);
        if (lane == 0) a.logits[item] = r;
      }
    }
    grid_barrier(a.flags, ++target, a.err);

    // ---------------- phase B: selection, grouping, gate/up + SwiGLU ----------------
    for (int i = tid; i < T * E; i += kFT) s.u.logit[i] = a.logits[i];
    if (tid < kFMaxT) s.ncand[tid] = 0;
    for (int i = tid; i < (kFMaxP + 1) * kFMaxT; i += kFT) s.pair_of[i] = -1;
    __syncthreads();
    for (int t = wv; t < T; t += kFW) {
      float mx = -INFINITY;
      for (int e = lane; e < E; e += kWave) mx = fmaxf(mx, s.u.logit[t * E + e]);
      for (int o = kWave / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
      float sm = 0.0f;
      for (int e = lane; e < E; e += kWave) sm += expf(s.u.logit[t * E + e] - mx);
      sm = wave_sum_xor(sm, kWave);
      if (lane == 0) {
        s.rmax[t] = mx;
        s.rsum[t] = sm;
      }
    }
    if (a.forced) {
      if (wv == 0) {
        const int p = lane;
        const bool valid = p < P;
        const int t = valid ? p / k : 0;
        int e = valid ? a.forced[((int64_t)l * T) * k + p] : 0;
        bool bad = valid && (e < 0 || e >= E);
        bool dup = false;
        for (int q = 0; q < P; ++q) {
          const int other = __shfl(e, q, kWave);
          if (valid && q != p && q / k == t && other == e) dup = true;
        }
        // a token with any bad or repeated id gets ids 0..k-1
        const uint64_t badm = __ballot(bad || dup);
        bool tok_bad = false;
        for (int j = 0; j < k; ++j) tok_bad |= valid && ((badm >> (t * k + j)) & 1ull);
        const uint64_t bm = __ballot(bad), dm = __ballot(dup);
        if (lane == 0 && badm) atomic_or_err(a.err, (bm ? kErrBadId : 0u) | (dm ? kErrDupId : 0u));
        if (valid) s.ids[p] = tok_bad ? (p - t * k) : e;
      }
    } else {
      const int nch = (E + kWave - 1) / kWave;
      for (int u = wv; u < T * nch; u += kFW) {
        const int t = u / nch, c = u - t * nch;
        const int e = c * kWave + lane;
        const bool valid = e < E;
        const float v = valid ? s.u.logit[t * E + e] : 0.0f;
        const int cend = min(kWave, E - c * kWave);
        float rank = 0.0f;
        for (int j = 0; j < cend; ++j) {
          const int f = c * kWave + j;
          rank += beats(v, e, s.u.logit[t * E + f], f);
        }
        if (valid && rank < (float)k) {
          if (nch == 1) {
            s.ids[t * k + (int)rank] = e;
          } else {
            const int slot = atomicAdd(&s.ncand[t], 1);
            s.cval[t][slot] = v;
            s.cid[t][slot] = e;
          }
        }
      }
      __syncthreads();
      if (nch > 1) {
        for (int t = wv; t < T; t += kFW) {
          const int n = s.ncand[t];
          for (int ci = lane; ci < n; ci += kWave) {
            const float v = s.cval[t][ci];
            const int e = s.cid[t][ci];
            float rank = 0.0f;
            for (int cj = 0; cj < n; ++cj) rank += beats(v, e, s.cval[t][cj], s.cid[t][cj]);
            if (rank < (float)k) s.ids[t * k + (int)rank] = e;
          }
        }
      }
    }
    __syncthreads();
    float wtmp = 0.0f;
    if (tid < P) {
      const int t = tid / k;
      wtmp = expf(s.u.logit[t * E + s.ids[tid]] - s.rmax[t]) / s.rsum[t];
      s.w[tid] = wtmp;
    }
    __syncthreads();
    if (a.renorm && tid < P) {
      const int t = tid / k;
      float tot = 0.0f;
      for (int j = 0; j < k; ++j) tot += s.w[t * k + j];
      wtmp = wtmp / tot;
    }
    __syncthreads();
    if (tid < P) {
      s.w[tid] = wtmp;
      if (b == 0 && a.ids_trace) a.ids_trace[(int64_t)l * P + tid] = s.ids[tid];
      if (b == 0 && a.w_trace) a.w_trace[(int64_t)l * P + tid] = wtmp;
    }
    // grouping: distinct experts in order of first appearance
    if (wv == 0) {
      const int p = lane;
      const bool valid = p < P;
      const int e = valid ? s.ids[p] : -1;
      int q0 = p;
      for (int q = 0; q < p; ++q)
        if (s.ids[q] == e) {
          q0 = q;
          break;
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
    const int U = s.nact;
    const int nunits = U + (a.has_shared ? 1 : 0);
    {
      constexpr int RB = I / 16;
      const int ntask = nunits * RB;
      const int q4 = wv & 3, mat = wv >> 2;
      const int m = lane & 15, lg = lane >> 4;
      for (int task = b; task < ntask; task += nb) {
        const int au = task / RB, rb = task - au * RB;
        const uint8_t* blob = au < U ? L.store + (int64_t)s.act_slot[au] * a.blob_stride : L.shared;
        const int n = rb * 16 + m;
        const uint8_t* rowp = blob + a.lay.codes(mat) + (int64_t)n * (H / 2) + q4 * (KQ / 2) + lg * 16;
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(mat)) +
                             (int64_t)n * (H / 128) + q4 * GQ;
        uint4 qv[GQ];
        float scl[GQ];
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
          qv[g] = *reinterpret_cast<const uint4*>(rowp + g * 64);
          scl[g] = half_bits_to_float(sc[g]);
        }
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
          f4 ag = {0.f, 0.f, 0.f, 0.f};
          const int kb = q4 * KQ + g * 128 + 32 * lg;
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            h8 av = {};
            if (m < T) av = *reinterpret_cast<const h8*>(s.x + m * H + kb + 8 * st);
            ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, decode_h8(dword_of(qv[g], st)), ag, 0, 0, 0);
          }
          acc += ag * scl[g];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) s.u.red[wv][(4 * lg + r) * 16 + m] = acc[r];
        __syncthreads();
        if (tid < 256) {
          const int i = tid >> 4, j = tid & 15;
          const float g = (s.u.red[0][tid] + s.u.red[1][tid]) + (s.u.red[2][tid] + s.u.red[3][tid]);
          const float u = (s.u.red[4][tid] + s.u.red[5][tid]) + (s.u.red[6][tid] + s.u.red[7][tid]);
          if (i < T) {
            const int p = s.pair_of[au * T + i];
            if (p >= 0)
              reinterpret_cast<_Float16*>(a.hbuf)[(int64_t)p * I + rb * 16 + j] =
                  (_Float16)(g / (1.0f + expf(-g)) * u);
          }
        }
        __syncthreads();
      }
    }
    grid_barrier(a.flags, ++target, a.err);

    // ---------------- phase C: down projection, rank-ordered combine ----------------
    {
      const int m = lane & 15, lg = lane >> 4;
      for (int task = b; task < H / 16; task += nb) {
        const int n = task * 16 + m;
        for (int au = wv; au < nunits; au += kFW) {
          const uint8_t* blob = au < U ? L.store + (int64_t)s.act_slot[au] * a.blob_stride : L.shared;
          const uint8_t* rowp = blob + a.lay.codes(2) + (int64_t)n * (I / 2) + lg * 16;
          const uint16_t* sc = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(2)) + (int64_t)n * (I / 128);
          uint4 qv[GD];
          float scl[GD];
#pragma unroll
          for (int g = 0; g < GD; ++g) {
            qv[g] = *reinterpret_cast<const uint4*>(rowp + g * 64);
            scl[g] = half_bits_to_float(sc[g]);
          }
          const int pm = m < T ? s.pair_of[au * T + m] : -1;
          const _Float16* hrow = reinterpret_cast<const _Float16*>(a.hbuf) + (int64_t)(pm < 0 ? 0 : pm) * I;
          f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int g = 0; g < GD; ++g) {
            f4 ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              h8 av = {};
              if (pm >= 0) av = *reinterpret_cast<const h8*>(hrow + g * 128 + 32 * lg + 8 * st);
              ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, decode_h8(dword_of(qv[g], st)), ag, 0, 0, 0);
            }
            acc += ag * scl[g];
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
          a.h[(int64_t)t * H + task * 16 + j] += o;
        }
        __syncthreads();
      }
    }
    if (l + 1 < a.l1) grid_barrier(a.flags, ++target, a.err);
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
