// Fused decode path: one persistent kernel runs every layer of a stack step
// for a small batch (a few tokens).
//
// Per layer it does what the separate kernels do -- RMSNorm, router logits,
// softmax + top-k, grouping, gate/up + SwiGLU, down, rank-ordered combine into
// the FP32 residual.  Blocks hand data to each other only through three
// epoch-tagged exchanges per layer; there is no grid barrier:
//   E1  residual: every block owns 8 rows of the residual and publishes them;
//       every block reads the whole residual, normalises it into LDS;
//   E2  router logits: each XCD computes all logits of the step itself (the
//       32 blocks of XCD c = blockIdx % 8 share them through a replica of
//       their own), so the exchange stays within one XCD when the step has
//       few logits; with many logits one chip-wide copy is shared instead;
//   E3  FP16 intermediates: the gate/up tasks publish SwiGLU outputs of the
//       routed (token, expert) pairs; every block reads all of them into LDS.
// Each exchanged 64-bit word carries the epoch of the layer that wrote it in
// its high half and one FP32 value (or two FP16) in its low half; a reader
// polls a word until its epoch is the expected one.  Words are written and
// read with single-copy-atomic device-coherent 64-bit accesses, so no flag,
// fence or cache maintenance is needed and a value is consumed as soon as
// it lands.  Every wait is bounded: on time-out the block sets an error bit
// and stops waiting, so the kernel always ends.
//
// Work split (OLMoE-shaped step, T = 1, 8 routed experts, 256 blocks):
//   gate/up  one wave = 8 intermediate rows of one expert, gate and up (16
//            MFMA columns), one K half; the two halves of a row group run in
//            sibling waves and are summed in LDS, then SwiGLU;
//   down     one block = 8 output rows of the residual for every routed
//            expert; one wave = 2 experts x 8 rows (16 MFMA columns) over
//            half of K; the A operand holds the intermediates of the
//            (expert, token) pairs of those two experts.
// Right after the experts are known, every wave issues the loads of its first
// gate/up task and of its first down task, so the whole layer's INT4 weights
// stream from HBM while gate/up computes and while E3 completes.  INT4 codes
// are decoded in registers and fed to v_mfma_f32_16x16x32_f16 with the tokens
// as the zero-padded A operand; weights are never expanded in memory ("Horizon
// RunMap", "Architecture invariants": routed experts run from compact INT4
// data with FP16 scales).
//
// MFMA 16x16x32 operand layout on gfx950: lane l holds A[l%16][8*(l/16)+e],
// B[8*(l/16)+e][l%16] (e = 0..7) and D[4*(l/16)+r][l%16].  Each lane loads 16
// contiguous bytes of one weight row = 32 consecutive K; the K index of MFMA
// step st, lane group q, element e is kb + 32q + 8st + e for both operands,
// so one 4-step chain covers one 128-wide scale group.
//
// Every reduction runs in a fixed order, so every block derives bit-identical
// normalised inputs, expert choices and weights, and repeated runs give
// bit-identical results.  The grid is exactly 256 blocks (one per compute
// unit, all resident together), each owning H / 256 = 8 residual rows.
#include "fused_common.hpp"
#include "topk_wave.hpp"

namespace moe {

template <int I>
struct FusedSmem {
  alignas(16) _Float16 x[kFMaxT * 2048];     // normalised tokens (gate/up A operand)
  alignas(16) _Float16 xz[32];               // zeros: the A operand of padding rows
  union alignas(16) {
    struct {
      float logit[kFMaxTE];                  // logits of the step
      float cval[kFMaxT][kFMaxCand];         // per-chunk candidates (E > 64)
      int cid[kFMaxT][kFMaxCand];
      int prank[kFW][kWave];                 // partial ranks of the waves
      alignas(16) int prankT[kWave][kFW];    // the same by lane (one token)
      int prank2[kFW][kWave];
      uint64_t key[kFW][kWave];              // per-wave (logit, id) sort keys
      uint64_t cand[kFMaxCand];              // one-token candidates (keys)
      uint64_t scr[2 * kWave];               // rank scratch of wave 0
      uint64_t top[kFMaxP];                  // keys of ranks 0 .. k-1
      uint64_t candT[kFMaxT][kFMaxCand];     // the same per token (a few tokens)
      uint64_t scrT[kFMaxT][2 * kWave];
      uint64_t topT[kFMaxT][kFMaxP];
    } sel;
    _Float16 hst[kFStageHalves];             // intermediates of every pair (down A operand)
    float hfull[kFStageHalves / 2];          // residual of every token (E1 staging)
  } u;
  float red[kFW][kFMaxT][16];                // gate/up K-half partials
  float ypart[2][kFMaxP + kFMaxT][kFRows];   // down K-part outputs per pair
  float hown[kFMaxT][kFRows];                // residual rows owned by the block
  float part[kFMaxT][kFW];
  double lgacc[kFW], lgsum[kFW];             // logit partial sums of the waves
  int ids[kFMaxP];
  float w[kFMaxP];
  int unit_slot[kFMaxP + 1];                 // blob slot of each routed expert
  int pair_of[(kFMaxP + 1) * kFMaxT];        // [unit][token] -> pair, -1
  int nunits;
  // down-projection weights of each wave's current task, written by direct
  // global->LDS loads: codes [group][lane] 16 B, scales [lane] 2 groups
  uint4 dpre[kFW][I / 128][kWave];
  uint32_t dsc[kFW][kWave];
  // phase timestamps (instrumentation): kept in LDS during the call and
  // written out at its end, so that no timestamp store is in flight while a
  // phase waits for its own memory operations
  uint64_t stampbuf[2][kStampStride];
};

template <int H, int I>
__global__ __launch_bounds__(kFT) void fused_decode_kernel(FusedArgs a) {
  __shared__ FusedSmem<I> s;
  static_assert(H / kFRows == kFGrid, "one block per 8 residual rows");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int b = blockIdx.x;
  const int T = a.T, E = a.E, k = a.k;
  const int P = T * k;
  const int TE = T * E;
  const int n16 = lane & 15, q = lane >> 4;
  const int R = a.lg_reps;                 // logit replicas: 8 (one per XCD) or 1
  const int rep = b % R, rb = b / R, nrb = kFGrid / R;
  const int r0 = b * kFRows;               // residual rows owned by this block
  // logit items: `sub` waves of one block share an item, each over H / sub of
  // it; item of round r for this wave = (r * nrb + rb) * ipb + islot
  const int sub = a.lg_sub;
  const int ipb = kFW / sub, islot = wv / sub, lpart = wv - islot * sub;
  const int nchunk = (H / 512) / sub;
  const int item0 = rb * ipb + islot;
  const int lpoff = lpart * (H / sub);     // first K of the wave's part
  constexpr int GPU = I / 8;               // gate/up row groups per expert
  constexpr int GH = H / 256;              // scale groups per K half of gate/up
  constexpr int GDM = I / 128;             // scale groups of a whole down row
  const uint32_t ep = __hip_atomic_load(&a.epoch[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool bail = false;
  uint32_t errs = 0;

  if (tid < 32) s.xz[tid] = (_Float16)0.0f;
  uint4 rq[H / 512];  // router part of the wave's first logit item
  if (item0 < TE) load_router_part<H>(a.layers[a.l0].router + (int64_t)(item0 % E) * H + lpoff, nchunk, lane, rq);

  for (int l = a.l0; l < a.l1; ++l) {
    // Lane-derived indices are formed anew in every layer (from an opaque
    // copy of the thread index): hoisted out of the loop, they and the
    // addresses built from them would hold registers for the whole kernel.
    int tid_l = tid;
    asm volatile("" : "+v"(tid_l));
    const int tid = tid_l, lane = tid_l & 63, n16 = lane & 15, q = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid_l >> 6);
    const FusedLayer L = a.layers[l];
    // the next layer's router, read early so that its prefetch at the end of
    // this layer does not wait for the descriptor
    const uint16_t* next_router = l + 1 < a.l1 ? a.layers[l + 1].router : nullptr;
    const int li = l - a.l0;
    const uint32_t tag = ep + (uint32_t)li + 1u;  // epoch of the data this layer writes
    stamp(s, a, l, 0);

    // ---------------- E1: residual -> RMSNorm -> x in LDS ----------------
    if (li == 0) {
      const float* hin = a.h_in ? a.h_in : a.h;
      for (int i = tid; i < T * H; i += kFT) s.u.hfull[i] = hin[i];
    } else {
      read_tagged(a.xh + (int64_t)(li & 1) * kFMaxT * H, T * H, tag - 1u, bail,
                  [&](int i, uint32_t v) { s.u.hfull[i] = __builtin_bit_cast(float, v); });
    }
    bail = block_any(bail);
    // single-layer call in place: announce that this block has read the
    // caller's residual (its loads have returned: their values are in LDS)
    if (li == 0 && a.l1 - a.l0 == 1 && !a.h_in && tid == 0) st_tag(a.xgate + b, tag, 0u);
    if (tid < T * kFRows) s.hown[tid / kFRows][tid % kFRows] = s.u.hfull[(tid / kFRows) * H + r0 + tid % kFRows];
    for (int t = 0; t < T; ++t) {
      float ss = 0.0f;
#pragma unroll
      for (int j = 0; j < H / kFT; ++j) {
        const float v = s.u.hfull[t * H + tid + j * kFT];
        ss += v * v;
      }
      ss = wave_sum(ss);
      if (lane == 0) s.part[t][wv] = ss;
    }
    __syncthreads();
    for (int t = 0; t < T; ++t) {
      float tot = 0.0f;
#pragma unroll
      for (int w = 0; w < kFW; ++w) tot += s.part[t][w];
      const float r = 1.0f / sqrtf(tot / (float)H + 1e-5f);
#pragma unroll
      for (int j = 0; j < H / kFT; ++j) {
        const int i = tid + j * kFT;
        const _Float16 xv = (_Float16)(s.u.hfull[t * H + i] * r);
        s.x[t * H + i] = xv;
        if (b == 0 && a.x_trace) reinterpret_cast<_Float16*>(a.x_trace)[((int64_t)l * T + t) * H + i] = xv;
      }
    }
    __syncthreads();
    stamp(s, a, l, 1);

    // ---------------- router logits of this replica ----------------
    {
      const int nlr = (TE + nrb * ipb - 1) / (nrb * ipb);
      for (int r = 0; r < nlr; ++r) {
        const int item = (r * nrb + rb) * ipb + islot;
        const bool on = item < TE;
        const int t = on ? item / E : 0, e = on ? item - t * E : 0;
        const uint16_t* row = L.router + (int64_t)e * H;
        double acc = 0.0, asum = 0.0;
        if (on) {
          if (r > 0) load_router_part<H>(row + lpoff, nchunk, lane, rq);
          partial_dot<H>(s.x + t * H + lpoff, rq, nchunk, lane, acc, asum);
        }
        if (sub > 1) {
          if (lane == 0) {
            s.lgacc[wv] = acc;
            s.lgsum[wv] = asum;
          }
          __syncthreads();
          if (lpart == 0) {
            acc = s.lgacc[wv];
            asum = s.lgsum[wv];
            for (int j = 1; j < sub; ++j) {
              acc += s.lgacc[wv + j];
              asum += s.lgsum[wv + j];
            }
          }
          __syncthreads();
        }
        if (on && lpart == 0) {
          float v;
          if (a.exact_always || !certify(acc, asum, 8 * (H / 512) + 9, v))
            v = exact_dot_wave(reinterpret_cast<const uint16_t*>(s.x + t * H), row, H, lane);
          if (lane == 0) st_tag(a.xlg + (int64_t)rep * kFMaxTE + item, tag, __builtin_bit_cast(uint32_t, v));
        }
      }
    }
    stamp(s, a, l, 2);

    // ---------------- E2: logits -> LDS ----------------
    read_tagged(a.xlg + (int64_t)rep * kFMaxTE, TE, tag, bail,
                [&](int i, uint32_t v) { s.u.sel.logit[i] = __builtin_bit_cast(float, v); });
    for (int i = tid; i < (kFMaxP + 1) * kFMaxT; i += kFT) s.pair_of[i] = -1;
    bail = block_any(bail);
    stamp(s, a, l, 3);

    // ---------------- selection: top-k by (logit desc, id asc) ----------------
    const int nch = E >> 6;
    if (T == 1 && nch <= kFW && !a.forced) {
      // One token, at most 512 experts.  Lane l holds the keys of experts
      // l + 64 j, ordered like (logit desc, id asc) by one unsigned compare.
      // (1) The largest key of each lane; (2) the rank of each lane maximum
      // among the 64, its 64 x 64 comparisons split over the waves (wave w
      // takes lanes 8w .. 8w+7) and summed through LDS; (3) the lane maximum
      // of rank k-1 bounds the k-th largest key from below (the k lanes above
      // it hold k keys at least as large), so the keys at or above it -- at
      // most k lanes x nch keys -- contain the top k, which wave 0 ranks
      // exactly.  With 64 experts the lane maxima are the keys themselves and
      // step (2) is the whole ranking.
      const float* lg = s.u.sel.logit;
      uint64_t kj[kFW];
      uint64_t m = 0;
#pragma unroll
      for (int j = 0; j < kFW; ++j) {
        kj[j] = j < nch ? sel_key(lg[j * kWave + lane], j * kWave + lane) : 0ull;
        m = kj[j] > m ? kj[j] : m;
      }
      constexpr int kLanesPerWave = kWave / kFW;
      int pr = 0;
#pragma unroll
      for (int i = 0; i < kLanesPerWave; ++i) {
        const int src = wv * kLanesPerWave + i;
        const uint64_t mo = ((uint64_t)rdlane((uint32_t)(m >> 32), src) << 32) | rdlane((uint32_t)m, src);
        pr += (int)(mo > m);
      }
      s.u.sel.prankT[lane][wv] = pr;  // a lane's partial ranks side by side: two reads
      __syncthreads();
      stamp(s, a, l, 10);
      if (wv == 0) {
        const uint4 p0 = *reinterpret_cast<const uint4*>(&s.u.sel.prankT[lane][0]);
        const uint4 p1 = *reinterpret_cast<const uint4*>(&s.u.sel.prankT[lane][4]);
        const int r = (int)(((p0.x + p0.y) + (p0.z + p0.w)) + ((p1.x + p1.y) + (p1.z + p1.w)));
        uint64_t* top = s.u.sel.top;
        if (nch == 1) {
          // every lane holds its own expert: the weights are formed where the
          // logits are, in rank order only for the renormalisation's sum
          const int l0 = __builtin_ctzll(__ballot(r == 0));
          const float mx = key_value(((uint64_t)rdlane((uint32_t)(m >> 32), l0) << 32) | rdlane((uint32_t)m, l0));
          const float v = key_value(m);
          const float sm = wave_sum(expf(v - mx));
          float wj = r < k ? expf(v - mx) / sm : 0.0f;
          if (a.renorm) {
            if (r < k) s.w[r] = wj;
            const float wr = lane < k ? s.w[lane] : 0.0f;
            wj = wj / wave_sum(wr);
          }
          stamp(s, a, l, 11);
          if (r < k) {
            s.ids[r] = lane;
            s.w[r] = wj;
            if (b == 0 && a.ids_trace) a.ids_trace[(int64_t)l * P + r] = lane;
            if (b == 0 && a.w_trace) a.w_trace[(int64_t)l * P + r] = wj;
            int slot = L.map ? ldg<int32_t>(L.map + lane) : lane;
            if (slot < 0) {
              errs |= kErrNotResident;
              slot = 0;
            }
            s.unit_slot[r] = slot;
            s.pair_of[r] = r;
          }
          if (lane == 0) {
            if (a.has_shared) s.pair_of[k] = P;
            s.nunits = k;
          }
        } else {
          const int tl = __builtin_ctzll(__ballot(r == k - 1));  // exactly one lane
          const uint64_t th = ((uint64_t)rdlane((uint32_t)(m >> 32), tl) << 32) | rdlane((uint32_t)m, tl);
          const uint64_t below = (1ull << lane) - 1ull;
          int n = 0;
#pragma unroll
          for (int j = 0; j < kFW; ++j) {
            const bool c = kj[j] >= th;  // empty keys (0) never qualify
            const uint64_t bal = __ballot(c);
            if (c) s.u.sel.cand[n + __popcll(bal & below)] = kj[j];
            n += __popcll(bal);
          }
          wave_top_cands(s.u.sel.cand, n, k, 0, s.u.sel.scr, top, lane);
          // softmax over all E logits, in the same order as for several tokens
          // (the logits are the keys' values; -0 is +0 there, same exponential)
          const float mx = key_value(top[0]);
          float sm = 0.0f;
#pragma unroll
          for (int c = 0; c < kFW; ++c)
            if (c < nch) sm += expf(key_value(kj[c]) - mx);
          sm = wave_sum(sm);
          const uint64_t kt = lane < k ? top[lane] : 0ull;
          const int ej = lane < k ? key_id(kt) : 0;
          float wj = lane < k ? expf(key_value(kt) - mx) / sm : 0.0f;
          if (a.renorm) wj = wj / wave_sum(wj);
          stamp(s, a, l, 11);
          if (lane < k) {
            s.ids[lane] = ej;
            s.w[lane] = wj;
            if (b == 0 && a.ids_trace) a.ids_trace[(int64_t)l * P + lane] = ej;
            if (b == 0 && a.w_trace) a.w_trace[(int64_t)l * P + lane] = wj;
            // unit u = rank u; pair u
            int slot = L.map ? ldg<int32_t>(L.map + ej) : ej;
            if (slot < 0) {
              errs |= kErrNotResident;
              slot = 0;
            }
            s.unit_slot[lane] = slot;
            s.pair_of[lane] = lane;
          }
          if (lane == 0) {
            if (a.has_shared) s.pair_of[k] = P;
            s.nunits = k;
          }
        }
      }
      __syncthreads();
    } else {
      if (a.forced) {
        if (wv == 0) {
          const int p = lane;
          const bool valid = p < P;
          const int t = valid ? p / k : 0;
          const int e = valid ? a.forced[((int64_t)l * T) * k + p] : 0;
          const bool bad = valid && (e < 0 || e >= E);
          bool dup = false;
#pragma unroll 1
          for (int qq = 0; qq < P; ++qq) {
            const int other = __shfl(e, qq, kWave);
            dup |= valid && qq != p && qq / k == t && other == e;
          }
          // a token with any bad or repeated id gets ids 0..k-1
          const uint64_t badm = __ballot(bad || dup);
          const uint64_t bm = __ballot(bad), dm = __ballot(dup);
          bool tok_bad = false;
          for (int j = 0; j < k; ++j) tok_bad |= valid && ((badm >> (t * k + j)) & 1ull);
          if (lane == 0 && badm) errs |= (bm ? kErrBadId : 0u) | (dm ? kErrDupId : 0u);
          if (valid) s.ids[p] = tok_bad ? (p - t * k) : e;
        }
      } else if (nch <= kFW) {
        // a few tokens, at most 512 experts: wave t selects token t by itself,
        // as for one token but without the split over waves -- the rank of
        // each lane's largest key among the 64 lane maxima, then the exact
        // ranking of the keys at or above the k-th lane maximum
        if (wv < T) {
          const int t = wv;
          const float* lg = s.u.sel.logit + t * E;
          uint64_t kj[kFW];
          uint64_t m = 0;
#pragma unroll
          for (int j = 0; j < kFW; ++j) {
            kj[j] = j < nch ? sel_key(lg[j * kWave + lane], j * kWave + lane) : 0ull;
            m = kj[j] > m ? kj[j] : m;
          }
          const int r = wave_rank64(m, s.u.sel.key[wv], lane);
          if (nch == 1) {
            if (r < k) s.ids[t * k + r] = lane;
          } else {
            const int tl = __builtin_ctzll(__ballot(r == k - 1));  // exactly one lane
            const uint64_t th = ((uint64_t)rdlane((uint32_t)(m >> 32), tl) << 32) | rdlane((uint32_t)m, tl);
            const uint64_t below = (1ull << lane) - 1ull;
            uint64_t* cand = s.u.sel.candT[t];
            int n = 0;
#pragma unroll
            for (int j = 0; j < kFW; ++j) {
              const bool c = kj[j] >= th;  // empty keys (0) never qualify
              const uint64_t bal = __ballot(c);
              if (c) cand[n + __popcll(bal & below)] = kj[j];
              n += __popcll(bal);
            }
            uint64_t* top = s.u.sel.topT[t];
            wave_top_cands(cand, n, k, 0, s.u.sel.scrT[t], top, lane);
            if (lane < k) s.ids[t * k + lane] = key_id(top[lane]);
          }
        }
      } else {
        // rank of every expert within its chunk of 64: `wpt` waves share one
        // (token, chunk) task, each comparing all 64 lanes against a slice of
        // the chunk read with batched LDS broadcasts; partial ranks are summed
        const int ntask = T * nch;
        int wpt = 1;
        while (wpt * 2 * ntask <= kFW) wpt *= 2;
        const int span = kWave / wpt, sl = wv % wpt;
        for (int t0 = 0; t0 < ntask; t0 += kFW / wpt) {
          const int task = t0 + wv / wpt;
          const bool on = task < ntask;
          const int t = on ? task / nch : 0, c = on ? task - t * nch : 0;
          const float* row = s.u.sel.logit + t * E + c * kWave;
          const float v = row[lane];
          int pr = 0;
          if (on) {
            for (int j0 = sl * span; j0 < (sl + 1) * span; j0 += 8) {
              float vj[8];
  #pragma unroll
              for (int u = 0; u < 8; ++u) vj[u] = row[j0 + u];
  #pragma unroll
              for (int u = 0; u < 8; ++u) pr += (int)(vj[u] > v) | ((int)(vj[u] == v) & (int)(j0 + u < lane));
            }
          }
          s.u.sel.prank[wv][lane] = pr;
          __syncthreads();
          if (on && sl == 0) {
            int rank = 0;
            for (int qq = 0; qq < wpt; ++qq) rank += s.u.sel.prank[wv + qq][lane];
            if (rank < k) {
              if (nch == 1) {
                s.ids[t * k + rank] = lane;
              } else {
                s.u.sel.cval[t][c * k + rank] = v;
                s.u.sel.cid[t][c * k + rank] = c * kWave + lane;
              }
            }
          }
          __syncthreads();
        }
        if (nch > 1) {
          // rank among the chunks' candidates (<= 128 per token): lanes hold
          // candidates lane and lane + 64; `wpt2` waves share a token, each
          // comparing against a slice of the candidates
          const int n = nch * k;
          int wpt2 = 1;
          while (wpt2 * 2 * T <= kFW) wpt2 *= 2;
          const int span2 = (n + wpt2 - 1) / wpt2, sl2 = wv % wpt2;
          for (int t0 = 0; t0 < T; t0 += kFW / wpt2) {
            const int t = t0 + wv / wpt2;
            const bool on = t < T;
            const int tt = on ? t : 0;
            const bool ha = on && lane < n, hb = on && lane + kWave < n;
            const float va = ha ? s.u.sel.cval[tt][lane] : 0.0f;
            const float vb = hb ? s.u.sel.cval[tt][lane + kWave] : 0.0f;
            const int ea = ha ? s.u.sel.cid[tt][lane] : 0;
            const int eb = hb ? s.u.sel.cid[tt][lane + kWave] : 0;
            int ra = 0, rbk = 0;
            if (on) {
              const int j1 = min(n, (sl2 + 1) * span2);
              for (int j0 = sl2 * span2; j0 < j1; j0 += 8) {
                float vj[8];
                int ej[8];
  #pragma unroll
                for (int u = 0; u < 8; ++u) {
                  const bool in = j0 + u < j1;
                  vj[u] = in ? s.u.sel.cval[tt][j0 + u] : -INFINITY;
                  ej[u] = in ? s.u.sel.cid[tt][j0 + u] : 0x7fffffff;
                }
  #pragma unroll
                for (int u = 0; u < 8; ++u) {
                  ra += (int)(vj[u] > va) | ((int)(vj[u] == va) & (int)(ej[u] < ea));
                  rbk += (int)(vj[u] > vb) | ((int)(vj[u] == vb) & (int)(ej[u] < eb));
                }
              }
            }
            s.u.sel.prank[wv][lane] = ra;
            s.u.sel.prank2[wv][lane] = rbk;
            __syncthreads();
            if (on && sl2 == 0) {
              int rsa = 0, rsb = 0;
              for (int qq = 0; qq < wpt2; ++qq) {
                rsa += s.u.sel.prank[wv + qq][lane];
                rsb += s.u.sel.prank2[wv + qq][lane];
              }
              if (ha && rsa < k) s.ids[t * k + rsa] = ea;
              if (hb && rsb < k) s.ids[t * k + rsb] = eb;
            }
            __syncthreads();
          }
        }
      }
      __syncthreads();
      stamp(s, a, l, 10);
      // softmax weights of the chosen experts: one wave per token; sums over the
      // experts and the renormalisation run as fixed-order wave reductions
      if (wv < T) {
        const int t = wv;
        const float* lg = s.u.sel.logit + t * E;
        float mx;
        if (a.forced) {
          mx = -INFINITY;
          for (int c = 0; c < nch; ++c) mx = fmaxf(mx, lg[c * kWave + lane]);
          mx = wave_max(mx);
        } else {
          mx = lg[s.ids[t * k]];
        }
        float sm = 0.0f;
        for (int c = 0; c < nch; ++c) sm += expf(lg[c * kWave + lane] - mx);
        sm = wave_sum(sm);
        float wj = 0.0f;
        if (lane < k) wj = expf(lg[s.ids[t * k + lane]] - mx) / sm;
        if (a.renorm) {
          const float tot = wave_sum(lane < k ? wj : 0.0f);
          wj = wj / tot;
        }
        if (lane < k) {
          s.w[t * k + lane] = wj;
          if (b == 0 && a.ids_trace) a.ids_trace[(int64_t)l * P + t * k + lane] = s.ids[t * k + lane];
          if (b == 0 && a.w_trace) a.w_trace[(int64_t)l * P + t * k + lane] = wj;
        }
      }
      __syncthreads();
      stamp(s, a, l, 11);
      // grouping: distinct experts ("units") in order of first appearance
      if (wv == 0) {
        const int p = lane;
        const bool valid = p < P;
        const int e = valid ? s.ids[p] : -1;
        int q0 = p;  // first pair naming the same expert (ids of one token are distinct)
        if (T > 1) {
          // once per distinct expert: the lowest pair not yet grouped leads,
          // and every pair naming its expert takes it as its first
          uint64_t rem = __ballot(valid);
          while (rem) {
            const int ld = __builtin_ctzll(rem);
            const int ev = __builtin_amdgcn_readlane(e, ld);
            const bool same = valid && e == ev;
            if (same) q0 = ld;
            rem &= ~__ballot(same);
          }
        }
        const bool first = valid && q0 == p;
        const uint64_t fm = __ballot(first);
        const int ap = __popcll(fm & ((1ull << q0) - 1ull));
        if (first) {
          int slot = L.map ? ldg<int32_t>(L.map + e) : e;
          if (slot < 0) {
            errs |= kErrNotResident;
            slot = 0;
          }
          s.unit_slot[ap] = slot;
        }
        if (valid) s.pair_of[ap * T + p / k] = p;
        const int U = __popcll(fm);
        if (a.has_shared && p < T) s.pair_of[U * T + p] = P + p;
        if (lane == 0) s.nunits = U;
      }
      __syncthreads();
    }
    stamp(s, a, l, 4);

    // ---------------- weights: first gate/up task and first down task ----------------
    const int U = s.nunits;
    const int UU = U + a.has_shared;                  // units incl. the shared expert
    const int ntask_gu = UU * GPU * 2;
    const int nround_gu = (ntask_gu + kFGrid * kFW - 1) / (kFGrid * kFW);
    const int ncg = (UU + 1) >> 1;                    // down column groups (2 units each)
    const int ks = (ncg <= kFW / 2 && I >= 512) ? 2 : 1;
    const int ntask_d = ncg * ks;
    const int nround_d = (ntask_d + kFW - 1) / kFW;
    const int ngd = GDM / ks;                         // scale groups per down task

    auto unit_blob = [&](int u) -> const uint8_t* {
      return u < U ? L.store + (int64_t)s.unit_slot[u] * a.blob_stride : L.shared;
    };
    static_assert(GH == 8, "one 16-byte load carries the 8 group scales of a half row");
    uint4 gq[GH];
    uint4 gs;  // FP16 scales of the half row's GH groups
    auto load_gu = [&](int task) {
      const int g = task >> 1, half = task & 1;
      const int u = g / GPU, i0 = (g - u * GPU) * 8;
      const uint8_t* blob = unit_blob(u);
      const int mat = n16 >> 3;  // columns 0-7 gate rows, 8-15 up rows
      const int row = i0 + (n16 & 7);
      const uint8_t* cp = blob + a.lay.codes(mat) + code_offset(row, half * (H / 4) + q * 16, H / 2);
      const uint16_t* sp = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(mat)) + (int64_t)row * (H / 128) + half * GH;
#pragma unroll
      for (int g2 = 0; g2 < GH; ++g2) gq[g2] = ldg_u4(cp + g2 * kCodeGroupStride);
      // one 16-byte load for the scales: 2-byte loads cost the address unit
      // about as much per instruction as a whole 16-byte-per-lane load
      gs = ldg_u4(sp);
    };
    // down weights go straight to LDS: no registers are held for them while
    // gate/up runs and E3 completes.  Addresses are formed before any load of
    // the burst is issued, so forming them waits on nothing.
    struct DPtr {
      const uint8_t* cp;
      const uint16_t* sp;
    };
    auto d_ptrs = [&](int task) -> DPtr {
      const int cg = task / ks, kp = task - cg * ks;
      const int u = min(cg * 2 + (n16 >> 3), UU - 1);  // a dead column re-reads a live row
      const uint8_t* blob = unit_blob(u);
      const int row = r0 + (n16 & 7);
      return DPtr{blob + a.lay.codes(2) + code_offset(row, kp * (I / 2 / ks) + q * 16, I / 2),
                  reinterpret_cast<const uint16_t*>(blob + a.lay.scales(2)) + (int64_t)row * GDM + kp * ngd + 2 * q};
    };
    auto load_d = [&](const DPtr& d) {
#pragma unroll
      for (int g2 = 0; g2 < GDM; ++g2)
        if (g2 < ngd) dma_lds16(d.cp + g2 * kCodeGroupStride, lds_addr(&s.dpre[wv][g2][0]));
      // lane (n, q) fetches the scales of groups 2q, 2q+1 of column n
      if (2 * q < ngd) dma_lds4(d.sp, lds_addr(&s.dsc[wv][0]));
    };
    const int gu_task0 = b * kFW + wv;
    const DPtr d0 = d_ptrs(wv < ntask_d ? wv : 0);
    // the gate/up loads are issued now; the down weights' direct loads only
    // once the wave's gate/up weights have arrived, so that the whole chip's
    // gate/up weights lead the burst (the down weights are needed only after
    // the intermediates have been exchanged)
    if (gu_task0 < ntask_gu) load_gu(gu_task0);
    stamp(s, a, l, 5);

    // ---------------- gate/up + SwiGLU -> E3 publication ----------------
    // one round: MFMA over the wave's K half, LDS sum of the halves, SwiGLU,
    // publication.  Round 0 runs outside the loop so that its loads are
    // waited for one group at a time.
    // `next`: the wave's task of the following round, whose weights are
    // loaded as soon as this round's MFMAs have taken theirs (the registers
    // are free then), so that their latency runs under the round's exchange
    auto gu_round = [&](int task, bool first, int next) __attribute__((always_inline)) {
      const bool on = task < ntask_gu;
      if (on) {
        const int half = task & 1;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g2 = 0; g2 < GH; ++g2) {
          f4 ag = {0.f, 0.f, 0.f, 0.f};
          const int kb = half * (H / 2) + g2 * 128 + 32 * q;
          // padding rows (n16 >= T) read 32 zeros; all four reads issue together
          const _Float16* ap = n16 < T ? s.x + n16 * H + kb : s.xz;
          h8 av[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) av[st] = *reinterpret_cast<const h8*>(ap + 8 * st);
#pragma unroll
          for (int st = 0; st < 4; ++st)
            ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st], decode_h8(dword_of(gq[g2], st)), ag, 0, 0, 0);
          acc += ag * half_bits_to_float((uint16_t)(dword_of(gs, g2 >> 1) >> (16 * (g2 & 1))));
          // decode one group at a time: keeps the decoded operands of later
          // groups from being hoisted (and held in registers) early
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (4 * q + rr < T) s.red[wv][4 * q + rr][n16] = acc[rr];
      }
      if (next < ntask_gu) load_gu(next);
      if (first && wv < ntask_d) load_d(d0);
      stamp(s, a, l, 13);
      __syncthreads();
      stamp(s, a, l, 14);
      if (on && (wv & 1) == 0) {
        // sum the two K halves (sibling waves), SwiGLU, publish FP16 pairs
        const int m = lane >> 3, n = lane & 7;
        float hv = 0.0f;
        if (m < T) {
          const float gsum = s.red[wv][m][n] + s.red[wv + 1][m][n];
          const float usum = s.red[wv][m][n + 8] + s.red[wv + 1][m][n + 8];
          hv = swiglu(gsum, usum);
        }
        const float hn = __shfl_down(hv, 1, kWave);
        if (m < T && (n & 1) == 0) {
          const int g = task >> 1, u = g / GPU, i0 = (g - u * GPU) * 8;
          const int p = s.pair_of[u * T + m];
          if (p >= 0) {
            const h2 pr = {(_Float16)hv, (_Float16)hn};
            st_tag(a.xhb + (int64_t)p * (I / 2) + (i0 + n) / 2, tag, __builtin_bit_cast(uint32_t, pr));
          }
        }
      }
    };
    constexpr int kGuStride = kFGrid * kFW;  // tasks per round
    gu_round(gu_task0, true, nround_gu > 1 ? gu_task0 + kGuStride : ntask_gu);
    for (int r = 1; r < nround_gu; ++r) {
      const int task = gu_task0 + r * kGuStride;
      __syncthreads();  // red is reused
      gu_round(task, false, r + 1 < nround_gu ? task + kGuStride : ntask_gu);
    }
    stamp(s, a, l, 6);

    // ---------------- down weights of the first down task -> registers ----------------
    // When the wave has a single down task, its direct loads are waited for
    // and the INT4 codes of its first kPre scale groups decoded (with their
    // scales) before the intermediates are exchanged: the exchange is a wait,
    // and after it less work remains for the down projection.
    constexpr int kPre = 4;
    const bool pre = nround_d == 1 && wv < ntask_d;
    h8 bd[kPre][4];
    float bsc[kPre];
    if (pre) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int g2 = 0; g2 < kPre; ++g2) {
        if (g2 < ngd) {
          const uint4 dq = s.dpre[wv][g2][lane];
#pragma unroll
          for (int st = 0; st < 4; ++st) bd[g2][st] = decode_h8(dword_of(dq, st));
          const uint32_t sw = s.dsc[wv][n16 + 16 * (g2 >> 1)];
          bsc[g2] = half_bits_to_float((uint16_t)(sw >> (16 * (g2 & 1))));
        } else {
#pragma unroll
          for (int st = 0; st < 4; ++st) bd[g2][st] = h8{};
          bsc[g2] = 0.0f;
        }
        // keep the decoded operands here, ahead of the exchange
#pragma unroll
        for (int st = 0; st < 4; ++st) asm volatile("" : "+v"(bd[g2][st]));
      }
    }

    // ---------------- E3: intermediates of every pair -> LDS ----------------
    const int npairs = P + (a.has_shared ? T : 0);
    read_tagged(a.xhb, npairs * (I / 2), tag, bail,
                [&](int i, uint32_t v) { reinterpret_cast<uint32_t*>(s.u.hst)[i] = v; });
    bail = block_any(bail);
    stamp(s, a, l, 7);

    // ---------------- down projection of the block's 8 rows ----------------
    for (int r = 0; r < nround_d; ++r) {
      const int task = wv + r * kFW;
      const bool on = task < ntask_d;
      if (r > 0 && on) load_d(d_ptrs(task));
      // this wave's direct loads into its LDS region have landed
      if (!pre) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (r == 0) stamp(s, a, l, 12);
      if (on) {
        const int cg = task / ks, kp = task - cg * ks;
        // A row m: unit cg*2 + m/T, token m%T
        const int us = n16 / T, t = n16 - us * T;
        const int ua = cg * 2 + us;
        const int pa = (us < 2 && ua < UU) ? s.pair_of[ua * T + t] : -1;
        const _Float16* hrow = s.u.hst + (pa < 0 ? 0 : pa) * I;
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g2 = 0; g2 < GDM; ++g2) {
          if (g2 < ngd) {
            f4 ag = {0.f, 0.f, 0.f, 0.f};
            const int kb = kp * (I / ks) + g2 * 128 + 32 * q;
            const uint4 dq = s.dpre[wv][g2][lane];
            const _Float16* ap = pa >= 0 ? hrow + kb : s.xz;
            h8 av[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) av[st] = *reinterpret_cast<const h8*>(ap + 8 * st);
            if (g2 < kPre && pre) {
#pragma unroll
              for (int st = 0; st < 4; ++st)
                ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st], bd[g2 < kPre ? g2 : 0][st], ag, 0, 0, 0);
              acc += ag * bsc[g2 < kPre ? g2 : 0];
            } else {
#pragma unroll
              for (int st = 0; st < 4; ++st)
                ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st], decode_h8(dword_of(dq, st)), ag, 0, 0, 0);
              const uint32_t sw = s.dsc[wv][n16 + 16 * (g2 >> 1)];
              acc += ag * half_bits_to_float((uint16_t)(sw >> (16 * (g2 & 1))));
            }
          }
        }
        // D[m][n]: row m = (unit m/T, token m%T), column n = (unit n/8, row n%8)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int m = 4 * q + rr;
          const int um = m / T;
          if (m < 2 * T && um == (n16 >> 3)) {
            const int uu = cg * 2 + um;
            if (uu < UU) {
              const int p = s.pair_of[uu * T + (m - um * T)];
              if (p >= 0) s.ypart[kp][p][n16 & 7] = acc[rr];
            }
          }
        }
      }
    }
    // the next layer's router part of this wave's first item streams in
    // during the combine and the residual exchange
    if (next_router && item0 < TE)
      load_router_part<H>(next_router + (int64_t)(item0 % E) * H + lpoff, nchunk, lane, rq);
    __syncthreads();
    stamp(s, a, l, 8);

    // ---------------- rank-ordered combine, residual update, E1 publication ----------------
    const bool last = l + 1 == a.l1;
    if (last && li == 0 && !a.h_in) {
      // single-layer call in place: the caller's residual is overwritten only
      // after every block has read it
      read_tagged(a.xgate, kFGrid, tag, bail, [&](int, uint32_t) {});
      bail = block_any(bail);
    }
    if (tid < T * kFRows) {
      const int t = tid / kFRows, row = tid - t * kFRows;
      float o = 0.0f;
      // rank order; the LDS reads of four ranks are issued together
      for (int j0 = 0; j0 < k; j0 += 4) {
        float y[4], wq[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int p = t * k + min(j0 + u, k - 1);
          y[u] = ks == 2 ? s.ypart[0][p][row] + s.ypart[1][p][row] : s.ypart[0][p][row];
          wq[u] = s.w[p];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (j0 + u < k) o += wq[u] * y[u];
      }
      if (a.has_shared) {
        const int p = P + t;
        o += ks == 2 ? s.ypart[0][p][row] + s.ypart[1][p][row] : s.ypart[0][p][row];
      }
      const float hn = s.hown[t][row] + o;
      if (last)
        a.h[(int64_t)t * H + r0 + row] = hn;
      else
        st_tag(a.xh + (int64_t)((li + 1) & 1) * kFMaxT * H + t * H + r0 + row, tag, __builtin_bit_cast(uint32_t, hn));
    }
    stamp(s, a, l, 9);
  }
  if (a.stamps && tid == 0) {
    const int n = min(a.l1 - a.l0, kStampLayers) * kStampsPerLayer;
    for (int i = 0; i < n; ++i) {
      a.stamps[(int64_t)b * kStampStride + i] = s.stampbuf[0][i];
      a.stamps[(int64_t)(kFGrid + b) * kStampStride + i] = s.stampbuf[1][i];
    }
  }
  if (bail) errs |= kErrBarrier;
  if (tid == 0) __hip_atomic_store(&a.epoch[b], ep + (uint32_t)(a.l1 - a.l0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (errs) atomic_or_err(a.err, errs);
}

bool fused_supported(int H, int I) { return H == 2048 && (I == 1024 || I == 512); }

void launch_fused_decode(const FusedArgs& a, hipStream_t stream) {
  if (a.I == 1024)
    hipLaunchKernelGGL((fused_decode_kernel<2048, 1024>), dim3(kFGrid), dim3(kFT), 0, stream, a);
  else
    hipLaunchKernelGGL((fused_decode_kernel<2048, 512>), dim3(kFGrid), dim3(kFT), 0, stream, a);
}

}  // namespace moe
