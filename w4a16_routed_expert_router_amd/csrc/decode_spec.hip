// Batch-1 decode with the next layer's experts guessed ahead: one persistent
// kernel runs every layer of a stack step for a single token.
//
// What each layer computes is that of the general fused path (RMSNorm, exact
// router logits, softmax + top-k, gate/up + SwiGLU, down, rank-ordered
// combine into the FP32 residual).  At batch 1 a layer is a chain of short
// dependent phases, each bounded by memory latency: the residual exchange,
// the logits and their exchange, the selection, the exchange of the
// intermediates, the down projection and the combine.  The routed experts'
// weights (26 MB per OLMoE-shaped layer) would add a burst to that chain;
// here they are loaded ahead, on a guess of the layer's experts made during
// the previous layer: that layer's router applied to the previous layer's
// normalised input, the guess the expert-offloading page uses for its
// next-layer prefetch ("An expert-offloading engine, from scratch", "Terms
// used here", "What the numbers say").
//
// The waves of a block take two roles that never wait for each other at a
// block barrier, only on LDS flags for the data they hand over:
//   chain waves (0-3) run the latency chain: every exchange read, the
//     RMSNorm, one router logit each (an exact logit of this layer or a
//     guess logit of the next), the selection and the guess, the combine;
//   weight waves (4-7) own the weights: each loads its row group's gate/up
//     rows and its down rows of the guessed experts into LDS during the
//     previous layer (direct global->LDS loads, counted in its own vmcnt),
//     computes gate/up + SwiGLU for the guessed expert as soon as x is
//     known, publishes it once the selection confirms the guess (or loads
//     and computes the chosen expert's rows when it does not) and runs the
//     down projection once the intermediates are in LDS.
// Chain waves never have a weight load in flight, so their exchange reads
// never wait behind one in their own vmcnt.  The guess decides only what is
// loaded and computed early, never what is published.
//
// Hand-overs (LDS flags hold the layer index):
//   f_x     chain -> weight   x of layer l is in LDS
//   f_sel   chain -> weight   units of layer l (expert per unit) are chosen
//   f_e3    chain -> weight   the intermediates of layer l are in LDS
//   f_down  weight -> chain   a weight wave's down partials of layer l
//   guess_layer  chain -> weight   the guessed experts of layer l+1
#include "fused_common.hpp"
#include "topk_wave.hpp"

namespace moe {

constexpr int kPW = 4;                // chain waves
constexpr int kPT = kPW * kWave;      // chain threads
constexpr int kMW = kFW - kPW;        // weight waves
constexpr int kSMaxU = 12;            // units (routed experts + shared) per layer
constexpr int kSMaxE = 512;           // experts per layer
constexpr int kSMaxK = 16;            // routed experts per token
constexpr int kSMaxNgd = 4;           // scale groups per down task
constexpr int kCand = 2 * kWave;      // candidates of a two-stage selection
constexpr uint32_t kLdsSpinLimit = 1u << 26;  // LDS flag polls before giving up

template <int H, int I>
struct SpecSmem {
  alignas(16) _Float16 x[H];                // normalised token (gate/up A operand)
  alignas(16) _Float16 xz[32];              // zeros: the A operand of padding rows
  union alignas(16) {
    float hfull[H];                         // residual (E1 staging)
    _Float16 hst[kSMaxU * I];               // intermediates of every unit (down A operand)
  } u;
  float logit[2 * kSMaxE];                  // exact logits of the layer, then the next layer's guess
  // gate/up rows of each weight wave's row group (8 gate + 8 up rows, all of
  // K): codes [group][lane] 16 B, scales [K half][lane] 2 groups
  uint4 gw[kMW][H / 128][kWave];
  uint32_t gsc[kMW][2][kWave];
  // down rows of each down task slot: codes [group][lane], scales [lane]
  uint4 dw[2 * kMW][kSMaxNgd][kWave];
  uint32_t dsc[2 * kMW][kWave];
  float ypart[2][kSMaxU][kFRows];           // down K-part outputs per unit
  float hown[kFRows];                       // residual rows owned by the block
  float part[kPW];
  alignas(16) uint64_t cand[2][kCand];      // per-chunk top keys: exact selection, guess
  alignas(16) uint64_t scr[kPW][kCand];     // per-wave ranking scratch
  uint64_t top[kPW][kSMaxK];                // per-wave ranking result (keys in rank order)
  // unit matching: per expert the layer tag and the rank (chosen) or the
  // unit (guessed)
  uint64_t sflag[kSMaxE];
  uint64_t gflag[kSMaxE];
  int nr[kSMaxK];                           // ranks of the chosen experts nobody guessed
  int unit_e[kSMaxU];                       // expert of each unit (-1 the shared expert)
  int uor[kSMaxK];                          // unit of each rank
  float sw[kSMaxK];                         // combine weight of each rank
  // guessed experts of a layer (guess rank order), by layer parity: the
  // guess of layer l+1 is written while layer l's may still be read
  int guess[2][kSMaxK];
  int guess_layer[2];                       // layer each guess is for, -1 none
  int f_x, f_sel, f_e3;
  int f_down[kMW];
  int pcnt;                                 // chain-wave barrier arrivals
  int bailf;                                // a wait was abandoned: every wait ends
  uint64_t stampbuf[2][kStampStride];
};

// LDS hand-over flags.  A flag is written after the data it covers has left
// the writing wave (lgkmcnt(0)); a wave's LDS reads are performed in order,
// so reads issued after the flag was seen return that data.
__device__ __forceinline__ void lds_settle() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ int lds_ld(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void flag_set(int* f, int v, int lane) {
  lds_settle();
  if (lane == 0) __hip_atomic_store(f, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Waits until *f >= v (or == v when `exact`); false if the wait was
// abandoned (here or by another wave).
__device__ __forceinline__ bool flag_wait(const int* f, int v, int* bailf, bool sleepy, bool exact = false) {
  uint32_t spins = 0;
  for (;;) {
    const int cur = lds_ld(f);
    if (exact ? cur == v : cur >= v) break;
    if (lds_ld(bailf)) return false;
    if (++spins > kLdsSpinLimit) {
      __hip_atomic_store(bailf, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return false;
    }
    if (sleepy) __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
  return true;
}

// s_waitcnt vmcnt(n) for the counts the weight waves use (an immediate in
// the instruction); any other count waits for everything
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

template <int H, int I>
__global__ __launch_bounds__(kFT) void spec_decode_kernel(FusedArgs a) {
  __shared__ SpecSmem<H, I> s;
  static_assert(H / kFRows == kFGrid, "one block per 8 residual rows");
  constexpr int GPU = I / 8;               // gate/up row groups per expert
  constexpr int GK = H / 128;              // scale groups along K of a gate/up row
  constexpr int GDM = I / 128;             // scale groups of a whole down row
  const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform
  const bool pw = wv < kPW;
  const int b = blockIdx.x;
  const int E = a.E, k = a.k, nch = E >> 6;
  const int UU = k + a.has_shared;
  const int R = a.lg_reps, rep = b % R, rb = b / R;
  const int r0 = b * kFRows;
  const uint32_t ep = __hip_atomic_load(&a.epoch[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int64_t xlg_rep = (int64_t)rep * kFMaxTE;
  const bool guessing = a.guess_mode != 3;
  // test hooks of the guess: mode 1 ranks the negated guess logits (the k
  // lowest; nearly every row group is recomputed), mode 2 takes guess ranks
  // k/2 .. k/2 + k - 1 (about half are)
  const float gsign = a.guess_mode == 1 ? -1.0f : 1.0f;
  const int gskip = a.guess_mode == 2 ? k / 2 : 0;

  if (threadIdx.x < 32) s.xz[threadIdx.x] = (_Float16)0.0f;
  if (threadIdx.x < 2) s.guess_layer[threadIdx.x] = -1;
  if (threadIdx.x < kMW) s.f_down[threadIdx.x] = -1;
  if (threadIdx.x == 0) {
    s.f_x = s.f_sel = s.f_e3 = -1;
    s.pcnt = 0;
    s.bailf = 0;
  }
  for (int e = threadIdx.x; e < kSMaxE; e += kFT) s.sflag[e] = s.gflag[e] = 0ull;
  __syncthreads();  // the only block barrier before the end of the call

  auto blob_of = [&](const FusedLayer& L, int e) -> const uint8_t* {
    return e >= 0 ? L.store + (int64_t)e * a.blob_stride : L.shared;
  };

  if (pw) {
    // ============================ chain waves ============================
    const int item = rb * kPW + wv;  // logit item: < E exact, < 2E guess of the next layer
    int pgen = 0;
    bool bail = false;
    // barrier of the four chain waves
    auto pbar = [&](int lane) {
      lds_settle();
      pgen += kPW;
      if (lane == 0) __hip_atomic_fetch_add(&s.pcnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (!flag_wait(&s.pcnt, pgen, &s.bailf, false)) bail = true;
    };
    uint4 rq[H / 512];
    {
      const uint16_t* row = nullptr;
      if (item < E) row = a.layers[a.l0].router + (int64_t)item * H;
      else if (item < 2 * E && a.l0 + 1 < a.l1 && guessing) row = a.layers[a.l0 + 1].router + (int64_t)(item - E) * H;
      if (row) load_router_part<H>(row, H / 512, (int)threadIdx.x & 63, rq);
    }
    for (int l = a.l0; l < a.l1; ++l) {
      int tid_l = threadIdx.x;
      asm volatile("" : "+v"(tid_l));
      const int tid = tid_l, lane = tid_l & 63;
      const FusedLayer L = a.layers[l];
      const bool has_next = l + 1 < a.l1;
      const bool guess_next = has_next && guessing;
      const int li = l - a.l0;
      const uint32_t tag = ep + (uint32_t)li + 1u;  // epoch of the data this layer writes
      stamp(s, a, l, 0);

      // ---------------- E1: residual -> RMSNorm -> x ----------------
      if (li == 0) {
        for (int i = tid; i < H; i += kPT) s.u.hfull[i] = (a.h_in ? a.h_in : a.h)[i];
      } else {
        // the staging buffer also holds the previous layer's intermediates:
        // every weight wave has finished its down projection
        for (int w = 0; w < kMW; ++w)
          if (!flag_wait(&s.f_down[w], l - 1, &s.bailf, false)) bail = true;
        read_tagged_n<kPT, H / kPT>(a.xh + (int64_t)(li & 1) * kFMaxT * H, H, tag - 1u, bail, tid,
                                    [&](int i, uint32_t v) { s.u.hfull[i] = __builtin_bit_cast(float, v); });
      }
      if (bail) __hip_atomic_store(&s.bailf, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      {
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < H / kPT; ++j) {
          const float v = s.u.hfull[tid + j * kPT];
          ss += v * v;
        }
        ss = wave_sum(ss);
        if (lane == 0) s.part[wv] = ss;
      }
      pbar(lane);
      // single-layer call in place: announce that this block has read the caller's residual
      if (li == 0 && a.l1 - a.l0 == 1 && !a.h_in && tid == 0) st_tag(a.xgate + b, tag, 0u);
      if (tid < kFRows) s.hown[tid] = s.u.hfull[r0 + tid];
      {
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < kPW; ++w) tot += s.part[w];
        const float r = 1.0f / sqrtf(tot / (float)H + 1e-5f);
#pragma unroll
        for (int j = 0; j < H / kPT; ++j) {
          const int i = tid + j * kPT;
          const _Float16 xv = (_Float16)(s.u.hfull[i] * r);
          s.x[i] = xv;
          if (b == 0 && a.x_trace) reinterpret_cast<_Float16*>(a.x_trace)[(int64_t)l * H + i] = xv;
        }
      }
      pbar(lane);
      flag_set(&s.f_x, l, tid);
      stamp(s, a, l, 1);

      // ---------------- logits: one exact or one guess item per chain wave ----------------
      if (item < E) {
        double acc, asum;
        partial_dot<H>(s.x, rq, H / 512, lane, acc, asum);
        float v;
        if (a.exact_always || !certify(acc, asum, 8 * (H / 512) + 9, v))
          v = exact_dot_wave_lean(reinterpret_cast<const uint16_t*>(s.x), L.router + (int64_t)item * H, H, lane);
        if (lane == 0) st_tag(a.xlg + xlg_rep + item, tag, __builtin_bit_cast(uint32_t, v));
      } else if (item < 2 * E && guess_next) {
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < H / 512; ++c) {
          const uint4 av = *reinterpret_cast<const uint4*>(s.x + c * 512 + lane * 8);
          const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
          const uint32_t bw[4] = {rq[c].x, rq[c].y, rq[c].z, rq[c].w};
#pragma unroll
          for (int i = 0; i < 8; ++i)
            acc += half_bits_to_float((uint16_t)(aw[i >> 1] >> (16 * (i & 1)))) *
                   half_bits_to_float((uint16_t)(bw[i >> 1] >> (16 * (i & 1))));
        }
        acc = wave_sum(acc);
        if (lane == 0) st_tag(a.xlg + xlg_rep + item, tag, __builtin_bit_cast(uint32_t, acc));
      }
      stamp(s, a, l, 2);
      // ---------------- E2: the exact logits and the guess -> LDS ----------------
      read_tagged_n<kPT, 2 * kSMaxE / kPT>(a.xlg + xlg_rep, guess_next ? 2 * E : E, tag, bail, tid,
                                          [&](int i, uint32_t v) { s.logit[i] = __builtin_bit_cast(float, v); });
      if (bail) __hip_atomic_store(&s.bailf, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      pbar(lane);
      stamp(s, a, l, 3);

      // ---------------- selection (wave 0) and the next layer's guess (wave 1) ----------------
      if (nch > 1) {
        // each chain wave ranks 64-expert chunks; the chunks' top k hold the layer's top k
        for (int c = wv; c < nch; c += kPW)
          wave_top64(sel_key(s.logit[lane + kWave * c], lane + kWave * c), k, 0, s.scr[wv], s.cand[0] + c * k, lane);
        if (guess_next)
          for (int c = wv; c < nch; c += kPW)
            wave_top64(sel_key(gsign * s.logit[E + lane + kWave * c], lane + kWave * c), k + gskip, 0, s.scr[wv],
                       s.cand[1] + c * (k + gskip), lane);
        pbar(lane);
      }
      if (wv == 0) {
        uint64_t* top = s.top[0];
        if (nch == 1) wave_top64(sel_key(s.logit[lane], lane), k, 0, s.scr[0], top, lane);
        else wave_top_cands(s.cand[0], nch * k, k, 0, s.scr[0], top, lane);
        stamp(s, a, l, 5);
        // softmax weights; the sums in the order of the general path
        const bool valid = lane < k;
        const uint64_t mykey = valid ? top[lane] : 0ull;
        const int sid = valid ? key_id(mykey) : -1;
        const float mx = key_value(top[0]);
        float sm = 0.0f;
        for (int c = 0; c < nch; ++c) sm += expf(s.logit[lane + kWave * c] - mx);
        sm = wave_sum(sm);
        float wj = valid ? expf(key_value(mykey) - mx) / sm : 0.0f;
        if (a.renorm) {
          const float tot = wave_sum(valid ? wj : 0.0f);
          wj = wj / tot;
        }
        if (b == 0 && valid) {
          if (a.ids_trace) a.ids_trace[(int64_t)l * k + lane] = sid;
          if (a.w_trace) a.w_trace[(int64_t)l * k + lane] = wj;
        }
        // Units 0..k-1 carry the routed experts, unit k the shared one.  A
        // unit keeps the expert guessed for it when that expert was chosen;
        // the chosen experts nobody guessed take the remaining units in rank
        // order.  Per expert, tables tagged with this layer's epoch hold its
        // rank (chosen) and its unit (guessed).
        const bool gv = s.guess_layer[l & 1] == l;
        const int gid = (gv && valid) ? s.guess[l & 1][lane] : -1;
        const uint64_t mtag = (uint64_t)tag << 32;
        if (valid) s.sflag[sid] = mtag | (uint32_t)lane;
        if (gid >= 0) s.gflag[gid] = mtag | (uint32_t)lane;
        const uint64_t sg = gid >= 0 ? s.sflag[gid] : 0ull;
        const uint64_t gs = valid ? s.gflag[sid] : 0ull;
        const bool keep = gid >= 0 && (sg >> 32) == tag;  // unit lane: its guess was chosen
        const bool in_g = valid && (gs >> 32) == tag;    // rank lane: its expert was guessed
        const uint64_t miss_m = __ballot(valid && !keep);
        const uint64_t new_m = __ballot(valid && !in_g);
        if (valid && !in_g) s.nr[__popcll(new_m & ((1ull << lane) - 1ull))] = lane;
        const int m = __popcll(miss_m & ((1ull << lane) - 1ull));
        const int rank_g = min((int)(uint32_t)sg, k - 1);
        const int ur = keep ? rank_g : (valid ? s.nr[m] : 0);  // rank carried by unit lane
        if (valid) {
          s.unit_e[lane] = key_id(top[ur]);
          s.uor[ur] = lane;
          s.sw[lane] = wj;
        }
        if (lane == k && a.has_shared) s.unit_e[k] = -1;
        flag_set(&s.f_sel, l, lane);
        stamp(s, a, l, 4);
      } else if (wv == 1 && guess_next) {
        uint64_t* top = s.top[1];
        if (nch == 1) wave_top64(sel_key(gsign * s.logit[E + lane], lane), k, gskip, s.scr[1], top, lane);
        else wave_top_cands(s.cand[1], nch * (k + gskip), k, gskip, s.scr[1], top, lane);
        if (lane < k) s.guess[(l + 1) & 1][lane] = key_id(top[lane]);
        flag_set(&s.guess_layer[(l + 1) & 1], l + 1, lane);
      }
      // the router row of this chain wave's next item streams in while the
      // intermediates are exchanged
      if (has_next) {
        const FusedLayer& LN = a.layers[l + 1];
        const uint16_t* row = nullptr;
        if (item < E) row = LN.router + (int64_t)item * H;
        else if (item < 2 * E && l + 2 < a.l1 && guessing) row = a.layers[l + 2].router + (int64_t)(item - E) * H;
        if (row) load_router_part<H>(row, H / 512, lane, rq);
      }

      // ---------------- E3: intermediates of every unit -> LDS ----------------
      read_tagged_n<kPT, 16>(a.xhb, UU * (I / 2), tag, bail, tid,
                            [&](int i, uint32_t v) { reinterpret_cast<uint32_t*>(s.u.hst)[i] = v; });
      if (bail) __hip_atomic_store(&s.bailf, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      pbar(lane);
      flag_set(&s.f_e3, l, tid);
      stamp(s, a, l, 7);

      // ---------------- rank-ordered combine, residual update, E1 publication ----------------
      if (wv == 0) {
        for (int w = 0; w < kMW; ++w)
          if (!flag_wait(&s.f_down[w], l, &s.bailf, false)) bail = true;
        stamp(s, a, l, 8);
        const bool last = !has_next;
        if (last && li == 0 && !a.h_in) {
          // single-layer call in place: the caller's residual is overwritten
          // only after every block has read it
          read_tagged_n<kWave, kFGrid / kWave>(a.xgate, kFGrid, tag, bail, lane, [&](int, uint32_t) {});
        }
        const int ks = ((UU + 1) / 2 <= kFW / 2 && I >= 512) ? 2 : 1;
        const int row = lane & 7;
        float y[kSMaxK], wj[kSMaxK];
#pragma unroll
        for (int j = 0; j < kSMaxK; ++j) {
          if (j < k) {
            const int u = s.uor[j];
            y[j] = ks == 2 ? s.ypart[0][u][row] + s.ypart[1][u][row] : s.ypart[0][u][row];
            wj[j] = s.sw[j];
          }
        }
        float o = 0.0f;
#pragma unroll
        for (int j = 0; j < kSMaxK; ++j)
          if (j < k) o += wj[j] * y[j];
        if (a.has_shared) o += ks == 2 ? s.ypart[0][k][row] + s.ypart[1][k][row] : s.ypart[0][k][row];
        const float hnew = s.hown[row] + o;
        if (lane < kFRows) {
          if (last)
            a.h[r0 + row] = hnew;
          else
            st_tag(a.xh + (int64_t)((li + 1) & 1) * kFMaxT * H + r0 + row, tag, __builtin_bit_cast(uint32_t, hnew));
        }
        stamp(s, a, l, 9);
      }
    }
    if (bail) __hip_atomic_store(&s.bailf, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    // ============================ weight waves ============================
    const int mw = wv - kPW;
    const int rg = b * kMW + mw;          // this wave's gate/up row group
    const int nrg = UU * GPU;             // row groups of a layer
    const int ncg = (UU + 1) >> 1;
    const int ks = (ncg <= kFW / 2 && I >= 512) ? 2 : 1;
    const int ntask_d = ncg * ks;
    const int ngd = GDM / ks;
    // direct loads this wave issues for its down slots (mw, mw + kMW)
    const int ndl = ((mw < ntask_d) + (mw + kMW < ntask_d)) * (ngd + 1);
    // what this wave's LDS holds of the coming layer: the expert of the
    // gate/up rows (-3 none) and the expert pairs of the down slots
    int pre_gu = -3;
    int pre_d[2] = {-3, -3};
    bool bail = false;

    for (int l = a.l0; l < a.l1 && !bail; ++l) {
      int tid_l = threadIdx.x;
      asm volatile("" : "+v"(tid_l));
      const int lane = tid_l & 63, n16 = lane & 15, q = lane >> 4;
      const FusedLayer L = a.layers[l];
      const bool has_next = l + 1 < a.l1;
      const bool guess_next = has_next && guessing;
      const uint32_t tag = ep + (uint32_t)(l - a.l0) + 1u;

      // direct loads of this wave's gate/up row group of expert e
      auto dma_gu = [&](const FusedLayer& LL, int e) {
        const int i0 = (rg % GPU) * 8;
        const uint8_t* blob = blob_of(LL, e);
        const int mat = n16 >> 3;  // columns 0-7 gate rows, 8-15 up rows
        const int row = i0 + (n16 & 7);
        const uint8_t* cp = blob + a.lay.codes(mat) + code_offset(row, q * 16, H / 2);
        const uint16_t* sp = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(mat)) + (int64_t)row * (H / 128) + 2 * q;
#pragma unroll 1
        for (int g = 0; g < GK; ++g) dma_lds16(cp + g * kCodeGroupStride, lds_addr(&s.gw[mw][g][0]));
        dma_lds4(sp, lds_addr(&s.gsc[mw][0][0]));
        dma_lds4(sp + GK / 2, lds_addr(&s.gsc[mw][1][0]));
      };
      // direct loads of down slot `slot` (units 2cg, 2cg+1 with experts e0, e1)
      auto dma_d = [&](const FusedLayer& LL, int slot, int e0, int e1) {
        const int cg = slot / ks, kp = slot - cg * ks;
        const uint8_t* blob = blob_of(LL, (n16 >> 3) ? e1 : e0);
        const int row = r0 + (n16 & 7);
        const uint8_t* cp = blob + a.lay.codes(2) + code_offset(row, kp * (I / 2 / ks) + q * 16, I / 2);
        // lanes with 2q >= ngd have no scales of their own: they re-read lane
        // group 0's (never used), which keeps every read inside the row
        const int qs = 2 * q < ngd ? q : 0;
        const uint16_t* sp = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(2)) + (int64_t)row * GDM + kp * ngd + 2 * qs;
#pragma unroll 1
        for (int g2 = 0; g2 < ngd; ++g2) dma_lds16(cp + g2 * kCodeGroupStride, lds_addr(&s.dw[slot][g2][0]));
        dma_lds4(sp, lds_addr(&s.dsc[slot][0]));
      };
      // expert pair of down slot `slot` for unit experts ue(u), as one key
      auto down_key = [&](auto&& ue, int slot, int& e0, int& e1) -> int {
        const int cg = slot / ks;
        e0 = ue(cg * 2);
        e1 = ue(min(cg * 2 + 1, UU - 1));  // a dead column re-reads a live row
        return (e0 + 1) * 1024 + (e1 + 1);
      };
      // gate/up of this wave's row group over all of K: the MFMA sums of
      // column n16 (row 0) scaled per group and added in group order
      auto gateup = [&]() -> float {
        f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int g = 0; g < GK; ++g) {
          f4 ag = {0.f, 0.f, 0.f, 0.f};
          const int kb = g * 128 + 32 * q;
          const _Float16* ap = n16 == 0 ? s.x + kb : s.xz;
          h8 av[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) av[st] = *reinterpret_cast<const h8*>(ap + 8 * st);
          const uint4 gq = s.gw[mw][g][lane];
#pragma unroll
          for (int st = 0; st < 4; ++st)
            ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st], decode_h8(dword_of(gq, st)), ag, 0, 0, 0);
          const int g2 = g % (GK / 2);
          const uint32_t sw2 = s.gsc[mw][g / (GK / 2)][n16 + 16 * (g2 >> 1)];
          acc += ag * half_bits_to_float((uint16_t)(sw2 >> (16 * (g2 & 1))));
        }
        return acc[0];
      };

      // ---------------- gate/up of the guessed expert, once x is known ----------------
      if (!flag_wait(&s.f_x, l, &s.bailf, true)) { bail = true; break; }
      const bool have_rows = pre_gu != -3 && rg < nrg;
      float pg = 0.0f;
      if (have_rows) {
        wait_vmcnt(pre_d[0] != -3 || pre_d[1] != -3 ? ndl : 0);  // the gate/up rows (the down rows may still fly)
        pg = gateup();
      }
      stamp(s, a, l, 13, kPT);

      // ---------------- the selection: publish, or compute the chosen expert ----------------
      if (!flag_wait(&s.f_sel, l, &s.bailf, true)) { bail = true; break; }
      auto ue_lds = [&](int u) -> int { return s.unit_e[u]; };
      if (rg < nrg) {
        const int u = rg / GPU, i0 = (rg - u * GPU) * 8;
        const int e = s.unit_e[u];
        if (!(have_rows && e == pre_gu)) {
          dma_gu(L, e);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          pg = gateup();
        }
        // SwiGLU: lanes 0..7 end with the result of row i0 + lane (v) and of the next row (vn)
        const float up = __builtin_bit_cast(float, dpp32<0x108, 0xf>(__builtin_bit_cast(uint32_t, pg), 0u));  // row_shl:8
        const float v = swiglu(pg, up);
        const float vn = __builtin_bit_cast(float, dpp32<0x101, 0xf>(__builtin_bit_cast(uint32_t, v), 0u));  // row_shl:1
        if (lane < 8 && (lane & 1) == 0) {
          const h2 pr = {(_Float16)v, (_Float16)vn};
          st_tag(a.xhb + (int64_t)u * (I / 2) + (i0 + lane) / 2, tag, __builtin_bit_cast(uint32_t, pr));
        }
      }
      pre_gu = -3;
      // the down rows of the chosen experts
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int slot = mw + kMW * t;
        if (slot < ntask_d) {
          int e0, e1;
          const int key = down_key(ue_lds, slot, e0, e1);
          if (key != pre_d[t]) dma_d(L, slot, e0, e1);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      stamp(s, a, l, 12, kPT);
      // the first down slot's operands, decoded while the intermediates arrive
      h8 bd[kSMaxNgd][4];
      float bsc[kSMaxNgd];
#pragma unroll
      for (int g2 = 0; g2 < kSMaxNgd; ++g2) {
        if (mw < ntask_d && g2 < ngd) {
          const uint4 dq = s.dw[mw][g2][lane];
#pragma unroll
          for (int st = 0; st < 4; ++st) bd[g2][st] = decode_h8(dword_of(dq, st));
          const uint32_t sw2 = s.dsc[mw][n16 + 16 * (g2 >> 1)];
          bsc[g2] = half_bits_to_float((uint16_t)(sw2 >> (16 * (g2 & 1))));
        } else {
#pragma unroll
          for (int st = 0; st < 4; ++st) bd[g2][st] = h8{};
          bsc[g2] = 0.0f;
        }
      }
      stamp(s, a, l, 15, kPT);

      // ---------------- down projection of the block's 8 rows ----------------
      if (!flag_wait(&s.f_e3, l, &s.bailf, false)) { bail = true; break; }
      stamp(s, a, l, 10, kPT);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int slot = mw + kMW * t;
        if (slot < ntask_d) {
          const int cg = slot / ks, kp = slot - cg * ks;
          // A row m (= n16): unit cg*2 + m for m < 2, zero rows otherwise
          const int ua = cg * 2 + n16;
          const bool ra = n16 < 2 && ua < UU;
          const _Float16* hrow = s.u.hst + (ra ? ua : 0) * I;
          f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int g2 = 0; g2 < kSMaxNgd; ++g2) {
            if (g2 < ngd) {
              f4 ag = {0.f, 0.f, 0.f, 0.f};
              const int kb = kp * (I / ks) + g2 * 128 + 32 * q;
              const _Float16* ap = ra ? hrow + kb : s.xz;
              h8 av[4];
#pragma unroll
              for (int st = 0; st < 4; ++st) av[st] = *reinterpret_cast<const h8*>(ap + 8 * st);
              if (t == 0) {
#pragma unroll
                for (int st = 0; st < 4; ++st)
                  ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st], bd[g2][st], ag, 0, 0, 0);
                acc += ag * bsc[g2];
              } else {
                const uint4 dq = s.dw[slot][g2][lane];
#pragma unroll
                for (int st = 0; st < 4; ++st)
                  ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st], decode_h8(dword_of(dq, st)), ag, 0, 0, 0);
                const uint32_t sw2 = s.dsc[slot][n16 + 16 * (g2 >> 1)];
                acc += ag * half_bits_to_float((uint16_t)(sw2 >> (16 * (g2 & 1))));
              }
            }
          }
          // D[m][n]: row m = unit cg*2 + m, column n = (unit n/8, row n%8)
          if (q == 0) {
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
              const int uu = cg * 2 + rr;
              if (rr == (n16 >> 3) && uu < UU) s.ypart[kp][uu][n16 & 7] = acc[rr];
            }
          }
        }
      }
      flag_set(&s.f_down[mw], l, lane);
      stamp(s, a, l, 11, kPT);

      // ---------------- the next layer's guessed rows ----------------
      pre_d[0] = pre_d[1] = -3;
      if (guess_next) {
        if (!flag_wait(&s.guess_layer[(l + 1) & 1], l + 1, &s.bailf, true, true)) { bail = true; break; }
        const FusedLayer& LN = a.layers[l + 1];
        const int gl = (l + 1) & 1;
        auto ue_guess = [&](int u) -> int { return u < k ? s.guess[gl][u] : -1; };
        if (rg < nrg) {
          pre_gu = ue_guess(rg / GPU);
          dma_gu(LN, pre_gu);
        }
        // down rows last: the next layer's first wait leaves them in flight
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int slot = mw + kMW * t;
          if (slot < ntask_d) {
            int e0, e1;
            pre_d[t] = down_key(ue_guess, slot, e0, e1);
            dma_d(LN, slot, e0, e1);
          }
        }
        stamp(s, a, l, 14, kPT);
      }
    }
    // no direct load may still be in flight when the block's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (bail) __hip_atomic_store(&s.bailf, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }

  __syncthreads();
  if (a.stamps && threadIdx.x == 0) {
    const int n = min(a.l1 - a.l0, kStampLayers) * kStampsPerLayer;
    for (int i = 0; i < n; ++i) {
      a.stamps[(int64_t)b * kStampStride + i] = s.stampbuf[0][i];
      a.stamps[(int64_t)(kFGrid + b) * kStampStride + i] = s.stampbuf[1][i];
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.epoch[b], ep + (uint32_t)(a.l1 - a.l0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0 && s.bailf) atomic_or_err(a.err, kErrBarrier);
}

bool spec_supported(int H, int I, int E, int k, int shared_inter) {
  if (H != 2048 || (I != 1024 && I != 512)) return false;
  if (E % 64 != 0 || E > kSMaxE || k < 1 || k > kSMaxK || k > E) return false;
  if (shared_inter != 0 && shared_inter != I) return false;
  const int UU = k + (shared_inter ? 1 : 0);
  if (UU > kSMaxU) return false;
  if (UU * (I / 8) > kFGrid * kMW) return false;                    // one gate/up row group per weight wave
  const int ncg = (UU + 1) / 2, ks = (ncg <= kFW / 2 && I >= 512) ? 2 : 1;
  const int ngd = (I / 128) / ks;
  if (ncg * ks > 2 * kMW || ngd > kSMaxNgd) return false;           // two down slots per weight wave
  if (ngd != 2 && ngd != 4) return false;                           // the load counts wait_vmcnt knows
  // candidates of the two-stage selection (with the guess hook's extra ranks)
  if ((E / 64) * (k + k / 2) > kCand) return false;
  return 2 * E <= kFGrid * kPW;                                     // one logit item per chain wave
}

void launch_spec_decode(const FusedArgs& a, hipStream_t stream) {
  if (a.I == 1024)
    hipLaunchKernelGGL((spec_decode_kernel<2048, 1024>), dim3(kFGrid), dim3(kFT), 0, stream, a);
  else
    hipLaunchKernelGGL((spec_decode_kernel<2048, 512>), dim3(kFGrid), dim3(kFT), 0, stream, a);
}

}  // namespace moe
