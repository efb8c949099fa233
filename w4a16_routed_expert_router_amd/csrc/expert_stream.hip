// Expert FFN for experts that receive few tokens (batched decode, the small
// experts of a prefill, the shared expert of a small batch): a persistent
// weight-streaming kernel on FP16 MFMA.
//
// The experts run straight from packed INT4 codes with FP16 group scales and
// FP16 activations; weights are never expanded in memory ("Horizon RunMap",
// "Architecture invariants").  With at most 32 tokens per expert the work is
// bound by streaming the weights, so the kernel is shaped for that:
//   * one block per compute unit takes a contiguous run of work items
//     (expert, tile of output rows), so consecutive items are mostly row tiles
//     of the same expert and its activation tile stays in LDS;
//   * at K = 2048 and 512 an item's scale groups are split between two waves
//     on the same rows, which add their sums in LDS at the item's end (items
//     of half the rows divide more evenly over the blocks; k_halves);
//   * every wave streams "units" (one 128-wide scale group of its two 16-row
//     weight sub-tiles, 2 KiB) through a ring of kRing units in registers; the
//     ring runs across item boundaries, so the weight stream never drains
//     between items and no barrier stops it (a barrier is taken only when the
//     next item belongs to another expert and its activations are loaded);
//   * the FP16 scales of an item's rows come in one 16-byte load per lane and
//     unit (2-byte loads cost the address unit about as much per instruction
//     as 16-byte ones), and each step takes the scale of its group and row
//     from the lane that holds it (ds_bpermute);
//   * the tokens of the expert (<= 32, zero-padded to one or two 16-token
//     sub-tiles; the second only when the expert has more than 16) are the A
//     operand of v_mfma_f32_16x16x32_f16; INT4 codes are decoded in registers to the
//     exact FP16 values q - 8, and each 128-wide group's FP32 MFMA result is
//     multiplied by its FP16 scale before it is added to the accumulator.
// MFMA operand layout (gfx950): lane l holds A[l%16][8*(l/16)+e],
// B[8*(l/16)+e][l%16], D[4*(l/16)+r][l%16]; the K index of step st, lane group
// q, element e is 128g + 32q + 8st + e for both operands.
#include <algorithm>
#include <utility>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t word_of(const u4& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}

constexpr int kSW = 8;          // waves per block
// weight units per wave in the ring (one in use, the rest in flight): 4 for the
// 2048- and 1024-wide K (3 to 4 measured 3 % faster, deeper rings slower); 3 for
// K = 512, whose 4-slot ring the compiler built with a slot copied on the loop's
// back edge while its load was in flight (tests/test_ring_asm.py checks every
// instantiation)
template <int K>
constexpr int ring_units() { return K == 512 ? 3 : 4; }
constexpr int kTok = 32;        // tokens per expert handled here (two sub-tiles of 16)
constexpr int kPad = 8;         // LDS row padding (halves)
constexpr int kMaxList = 1024;  // experts per call
constexpr int kBlockEntries = 8;  // list entries a block keeps when it groups the call itself
constexpr int kGroupScans = 4;    // values scanned over the experts by that grouping
// K halves per item.  With 2, waves w and w + kSW / 2 take the same rows of
// an item, each one half of its scale groups, and add their sums in LDS at the
// item's end: an item is half as many rows, so that the items of a call
// divide more evenly over the blocks (the Qwen3-Next-like batch of 16 has 140
// experts x 4 items of 128 gate/up rows for 256 blocks: 3 items on the busiest
// block against 2.2 on average; with 64-row items 5 against 4.4; measured
// gate/up 45.6 -> 41.5 us, down at K = 512 25.8 -> 24.8 us).  The down
// projection at K = 1024 keeps whole rows per wave: the OLMoE-shaped batch of
// 64 already divides evenly, and there the split measured 21.4 -> 22.9 us.
template <int K>
constexpr int k_halves() { return K == 1024 ? 1 : 2; }

// 8 INT4 codes -> (q - 8) as FP16 (exact); the group scale is applied to the
// FP32 MFMA result of the group instead (one FMA per output, fewer VALU
// instructions per weight than scaling every weight when few tokens share it).
__device__ __forceinline__ h8 decode_unscaled(uint32_t d, uint32_t mlo, uint32_t mhi) {
  h2 p[4];
  dequant8_v(d, p, mlo, mhi);
  h8 r;
  r[0] = p[0][0]; r[1] = p[0][1]; r[2] = p[1][0]; r[3] = p[1][1];
  r[4] = p[2][0]; r[5] = p[2][1]; r[6] = p[3][0]; r[7] = p[3][1];
  return r;
}

template <int K>
struct StreamSmem {
  alignas(16) _Float16 a[kTok * (K + kPad)];  // activation tile of the current expert
  f4 red[k_halves<K>() == 2 ? kSW / 2 : 1][4][kWave];  // second K half's sums: [row wave][sub-tile pair][lane]
  int slot[kMaxList];             // small experts of the call: blob slot, count, offset
  int count[kMaxList];
  int offset[kMaxList];
  int tok[kTok];
  int ns;
  int scan[kSW];
  int ptok[kBlockEntries][kTok];  // grouping in the kernel: tokens of the block's list entries
};

}  // namespace

// Exclusive prefix sums of N values per thread over the block (thread order)
// and their totals.  scratch: N x kSW ints, used once (no barrier after the
// reads).
template <int N>
__device__ __forceinline__ void stream_block_scan(const int (&v)[N], int (&excl)[N], int (&tot)[N], int* scratch) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    incl[i] = wave_incl_scan(v[i]);
    if (lane == 63) scratch[i * kSW + wv] = incl[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    int pre = 0, t = 0;
#pragma unroll
    for (int w = 0; w < kSW; ++w) {
      const int x = scratch[i * kSW + w];
      pre += w < wv ? x : 0;
      t += x;
    }
    excl[i] = pre + incl[i] - v[i];
    tot[i] = t;
  }
}

// Bytes of the tile's LDS the in-kernel grouping takes: ids, (64-token chunk,
// expert) masks and their prefix counts, four per-expert arrays, the scans'
// scratch.
__host__ __device__ inline size_t group_in_kernel_bytes(int T, int k, int E) {
  const size_t P = (size_t)T * k, NC = ((size_t)T + 63) / 64;
  return ((P * 4 + 7) & ~(size_t)7) + NC * E * 8 + NC * E * 4 + (size_t)E * 4 * 4 + (size_t)kGroupScans * kSW * 4;
}

// MODE 0: gate/up + SwiGLU (K = H, rows = I, 128 rows per item);
// MODE 1: down (K = I, rows = H, 256 rows per item).
template <int MODE, int K>
__global__ __launch_bounds__(kSW * kWave) void stream_expert_kernel(ExpertArgs a) {
  __shared__ StreamSmem<K> s;
  constexpr int LD = K + kPad;
  constexpr int NG = K / kGroup;
  constexpr int KS = k_halves<K>();
  constexpr int RW = kSW / KS;  // waves per K half
  constexpr int ROWS = MODE == 0 ? RW * 16 : RW * 32;
  constexpr int NGW = NG / KS;  // scale groups of a wave per item
  static_assert(NG % KS == 0, "scale groups per K half");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wr = wv % RW, kh = wv / RW;  // row wave, K half
  const int n = lane & 15, q = lane >> 4;
  const int N = MODE == 0 ? a.I : a.H;
  const int ntn = N / ROWS;

  // ---- the call's experts with at most 32 tokens (and below the MFMA
  // threshold), listed by the grouping, then the shared expert if it rides
  // along; the block takes a contiguous run of items (expert, row tile) and
  // keeps the list entries of its experts in LDS (slot -1 marks the shared
  // expert)
  // With group_in_kernel (gate/up only) every block groups the call's pairs
  // itself, the same way as the one-pass grouping kernel: ids validated per
  // token, a bit per (64-token chunk, expert), per-expert counts, offsets and
  // list entries (chunks of at most kStreamTokens tokens) by block scans; the
  // arrays live in the activation tile's LDS until the first tile is loaded.
  // Block 0 writes the grouping's outputs (positions, the permutation, the
  // lists and their counts, errors) for the down kernel and the combine.
  const bool gik = MODE == 0 && a.group_in_kernel;
  const GroupArgs& g = a.grp;
  const int gE = g.E, gT = g.T, gk = g.k, gP = gT * gk, gNC = (gT + 63) / 64;
  uint8_t* gbase = reinterpret_cast<uint8_t*>(s.a);
  int* gid = reinterpret_cast<int*>(gbase);                                                   // [P]
  unsigned long long* gmask = reinterpret_cast<unsigned long long*>(gbase + ((gP * 4 + 7) & ~7));  // [NC][E]
  int* gcum = reinterpret_cast<int*>(gmask + gNC * gE);  // [NC][E]: the expert's pairs in earlier chunks
  int* ecnt = gcum + gNC * gE;
  int* eoff = ecnt + gE;
  int* esidx = eoff + gE;
  int* eslot = esidx + gE;
  int* escan = eslot + gE;  // [kGroupScans][kSW]
  const int ept = (gE + kSW * kWave - 1) / (kSW * kWave);  // experts per thread (contiguous)
  int nrouted;
  if (gik) {
    int slot_pre[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid * ept + i;
      slot_pre[i] = (i < ept && e < gE && g.slot_map) ? g.slot_map[e] : e;
    }
    for (int i = tid; i < gNC * gE; i += kSW * kWave) gmask[i] = 0ull;
    for (int p = tid; p < gP; p += kSW * kWave) gid[p] = g.ids_in[p];
    __syncthreads();
    uint32_t errbits = 0;
    for (int t = tid; t < gT; t += kSW * kWave) {
      int rv[kMaxTopK], v[kMaxTopK];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) rv[j] = j < gk ? gid[t * gk + j] : -1;
      validate_token(rv, gk, gE, v, errbits);
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j >= gk) break;
        gid[t * gk + j] = v[j];
        atomicOr(&gmask[(t >> 6) * gE + v[j]], 1ull << (t & 63));
      }
    }
    __syncthreads();
    int c[2] = {0, 0}, vs[kGroupScans] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid * ept + i;
      if (i < ept && e < gE) {
        int cc = 0;
        for (int ch = 0; ch < gNC; ++ch) {
          gcum[ch * gE + e] = cc;
          cc += __popcll(gmask[ch * gE + e]);
        }
        c[i] = cc;
        vs[0] += cc;                                                               // positions
        vs[1] += cc >= g.mfma_min ? (cc + kMfmaTileTokens - 1) / kMfmaTileTokens : 0;  // MFMA token tiles
        vs[2] += cc > 0 ? 1 : 0;                                                   // active experts
        vs[3] += (cc + kStreamTokens - 1) / kStreamTokens;                         // list entries
      }
    }
    int ex[kGroupScans], tt[kGroupScans];
    stream_block_scan<kGroupScans>(vs, ex, tt, escan);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid * ept + i;
      if (i < ept && e < gE) {
        const int cc = c[i];
        int slot = 0;
        if (cc > 0) {
          slot = slot_pre[i];
          if (slot < 0) {
            errbits |= kErrNotResident;
            slot = 0;
          }
        }
        ecnt[e] = cc;
        eoff[e] = ex[0];
        esidx[e] = ex[3];
        eslot[e] = slot;
        if (blockIdx.x == 0) {
          if (cc > 0) {
            g.mtile_off[ex[2]] = ex[1];
            g.active[ex[2]] = ActiveExpert{e, slot, cc, ex[0]};
          }
          for (int j = 0; j * kStreamTokens < cc; ++j)
            g.small[ex[3] + j] =
                ActiveExpert{e, slot, min(kStreamTokens, cc - j * kStreamTokens), ex[0] + j * kStreamTokens};
        }
        ex[0] += cc;
        ex[1] += cc >= g.mfma_min ? (cc + kMfmaTileTokens - 1) / kMfmaTileTokens : 0;
        ex[2] += cc > 0 ? 1 : 0;
        ex[3] += (cc + kStreamTokens - 1) / kStreamTokens;
      }
    }
    if (blockIdx.x == 0) {
      if (errbits) atomic_or_err(g.err, errbits);
      if (tid == 0) {
        g.mtile_off[tt[2]] = tt[1];
        *g.n_active = tt[2];
        *g.n_small = tt[3];
      }
    }
    __syncthreads();
    if (blockIdx.x == 0) {
      for (int p = tid; p < gP; p += kSW * kWave) {
        const int e = gid[p], t = p / gk, ch = t >> 6, tl = t & 63;
        const int pos = eoff[e] + gcum[ch * gE + e] + __popcll(gmask[ch * gE + e] & ((1ull << tl) - 1ull));
        g.perm_tok[pos] = t;
        g.pos_of[p] = pos;
      }
    }
    nrouted = tt[3];
  } else {
    nrouted = a.fixed_blob ? 1 : *a.n_small;
  }
  const int ns = nrouted + (a.shared_blob ? 1 : 0);
  const int items = ns * ntn;
  const int per = (items + gridDim.x - 1) / gridDim.x;
  const int lo = blockIdx.x * per;
  const int hi = min(items, lo + per);
  if (lo >= hi) return;  // uniform over the block
  const int nv = (hi - lo) * NGW;  // units of every wave
  const int se0 = lo / ntn;       // first expert of the block (list index)
  if (gik) {
    // the block's list entries (at most kBlockEntries) and their tokens
    const int ne = (hi - 1) / ntn - se0 + 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid * ept + i;
      if (i < ept && e < gE) {
        const int cc = ecnt[e];
        for (int j = 0; j * kStreamTokens < cc; ++j) {
          const int idx = esidx[e] + j - se0;
          if (idx >= 0 && idx < ne) {
            s.slot[idx] = eslot[e];
            s.count[idx] = min(kStreamTokens, cc - j * kStreamTokens);
            s.offset[idx] = eoff[e] + j * kStreamTokens;
          }
        }
      }
    }
    if (tid == 0 && a.shared_blob && nrouted - se0 >= 0 && nrouted - se0 < ne) {
      s.slot[nrouted - se0] = -1;
      s.count[nrouted - se0] = a.shared_count;
      s.offset[nrouted - se0] = 0;
    }
    for (int p = tid; p < gP; p += kSW * kWave) {
      const int e = gid[p], t = p / gk, ch = t >> 6, tl = t & 63;
      const int r = gcum[ch * gE + e] + __popcll(gmask[ch * gE + e] & ((1ull << tl) - 1ull));
      const int idx = esidx[e] + r / kStreamTokens - se0;
      if (idx >= 0 && idx < ne) s.ptok[idx][r % kStreamTokens] = t;
    }
  } else if (tid <= (hi - 1) / ntn - se0) {
    if (a.fixed_blob) {
      s.slot[0] = 0;
      s.count[0] = a.fixed_count;
      s.offset[0] = a.fixed_offset;
    } else if (se0 + tid == nrouted) {
      s.slot[tid] = -1;
      s.count[tid] = a.shared_count;
      s.offset[tid] = 0;
    } else {
      const ActiveExpert e = a.small[se0 + tid];
      s.slot[tid] = e.slot;
      s.count[tid] = e.count;
      s.offset[tid] = e.offset;
    }
  }

  // ---- weight stream: unit v = (item lo + v / NGW, scale group kh * NGW + v % NGW)
  // The unit loads are issued as inline assembly and waited for explicitly:
  // every unit issues exactly kUnitLoads loads (its two code loads and the
  // scale load of its item; the tail re-reads the last unit), so the loads
  // younger than unit v are always (kRing - 1) * kUnitLoads and "vmcnt <=
  // that" means unit v has landed (loads return in order; stores and the
  // activation-tile loads only make the wait longer).  The compiler tracks
  // none of these loads, so it never drains the ring.
  constexpr int kUnitLoads = 3;
  constexpr int SB = NG * 2;                   // scale bytes of one row
  static_assert(SB == 32 || SB == 16 || SB == 8, "rows of 8 to 32 bytes of scales");
  constexpr int kRing = ring_units<K>();
  u4 bq[kRing][2];
  u4 bsv[kRing];  // scales of the unit's item (used from its first unit)
  auto load_unit = [&](int v, int slot_) __attribute__((always_inline)) {
    const int it = lo + v / NGW, g = kh * NGW + (v - (v / NGW) * NGW);
    const int se = it / ntn, nt = it - se * ntn;
    const int sl = s.slot[se - se0];
    const uint8_t* blob = a.fixed_blob ? a.fixed_blob
                          : sl < 0    ? a.shared_blob
                                      : a.blobs + (int64_t)sl * a.blob_stride;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int mat = MODE == 0 ? j : 2;
      const int r = MODE == 0 ? nt * ROWS + wr * 16 + n : nt * ROWS + wr * 32 + j * 16 + n;
      const uint8_t* cp = blob + a.lay.codes(mat) + code_offset(r, g * kCodeGroupBytes + q * 16, K / 2);
      asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(bq[slot_][j]) : "v"(cp) : "memory");
    }
    // lane (n, q) holds the 16-byte aligned chunk of scales [8 (q & 1), +8)
    // of row n of sub-tile q >> 1 (rows of 16 bytes: the lanes q & 1 == 1
    // repeat the row's load; rows of 8 bytes: the chunk holds rows n & ~1 and
    // n | 1).  The item's later units repeat its first unit's load, which
    // keeps the count of loads per unit fixed and costs the address unit one
    // instruction.  (Every ring register is a 16-byte vector: a ring slot of
    // another width was seen copied at the loop's back edge while its load was
    // in flight.)
    const int j = q >> 1;
    const int mat = MODE == 0 ? j : 2;
    const int r = MODE == 0 ? nt * ROWS + wr * 16 + n : nt * ROWS + wr * 32 + j * 16 + n;
    const int h = SB == 32 ? (q & 1) : 0;
    const uint8_t* sp = blob + a.lay.scales(mat) + (((int64_t)r * SB) & ~(int64_t)15) + h * 16;
    asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(bsv[slot_]) : "v"(sp) : "memory");
  };
  auto wait_unit = [&](int slot_) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(%3)"
                 : "+v"(bq[slot_][0]), "+v"(bq[slot_][1]), "+v"(bsv[slot_])
                 : "n"((kRing - 1) * kUnitLoads)
                 : "memory");
  };
  // ---- activation tile of one expert: rows = its tokens, zero past the count
  int cur = -1;  // small-expert index whose tile is in LDS
  bool two = false;  // its tile has a second 16-token sub-tile (uniform)
  auto load_tile = [&](int se) __attribute__((always_inline)) {
    __syncthreads();  // every wave is done with the previous tile (and the list is in LDS)
    const int cnt = s.count[se - se0], off = s.offset[se - se0];
    const bool shared = s.slot[se - se0] < 0;  // uniform
    if (tid < kTok) {
      int v = -1;
      if (tid < cnt)
        v = (a.fixed_blob || shared) ? tid
            : MODE == 1              ? off + tid
            : gik                    ? s.ptok[se - se0][tid]
                                     : a.perm_tok[off + tid];
      s.tok[tid] = v;
    }
    __syncthreads();
    const uint16_t* src = MODE == 0 ? a.x : (shared ? a.shared_h : a.hbuf);
    // rows of the sub-tiles the MFMAs read; past the count they are zero.
    // Each thread loads a batch of four 16-byte chunks before it stores any,
    // so a tile costs at most four memory round trips.
    const int rows = cnt > 16 ? kTok : 16;
    constexpr int kB = 4;  // chunks per thread and batch
    for (int c0 = 0; c0 < rows * (K / 8); c0 += kB * kSW * kWave) {
      u4 v[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        const int c = c0 + i * kSW * kWave + tid;
        const int r = c / (K / 8), col = (c - r * (K / 8)) * 8;
        v[i] = u4{0u, 0u, 0u, 0u};
        if (r < cnt) {
          const int t = s.tok[r];
          // gate/up reads token rows of x; down reads the rows of hbuf at the
          // expert's positions (the shared expert: positions offset + t)
          const int64_t src_row = MODE == 0 ? (int64_t)t : (a.fixed_blob ? (int64_t)off + t : (int64_t)t);
          v[i] = *reinterpret_cast<const u4*>(src + src_row * K + col);
        }
      }
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        const int c = c0 + i * kSW * kWave + tid;
        const int r = c / (K / 8), col = (c - r * (K / 8)) * 8;
        if (r < rows) *reinterpret_cast<u4*>(&s.a[r * LD + col]) = v[i];
      }
    }
    __syncthreads();
    cur = se;
    two = cnt > 16;
  };
  // the weight stream starts as soon as the block's list is in LDS; the first
  // expert's tile is loaded while it is in flight (its data arrives with the
  // ring's first units, which the first step needs anyway)
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kRing - 1; ++u) load_unit(min(u, nv - 1), u);
  load_tile(se0);

  f4 acc[2][2];  // [sub-tile][weight sub-tile]
#pragma unroll
  for (int m = 0; m < 2; ++m) acc[m][0] = acc[m][1] = f4{0.f, 0.f, 0.f, 0.f};
  uint32_t mlo = 0x000F000Fu, mhi = 0x00F000F0u;
  asm("" : "+v"(mlo), "+v"(mhi));  // the decode masks live in VGPRs
  u4 cs = {0u, 0u, 0u, 0u};  // scales of the current item (see load_unit)
  // Every round runs all kRing steps, so that the count of loads between a
  // unit's issue and its wait is the same on every path; the last round's
  // steps past nv only keep that count (they load and wait, and compute and
  // store nothing).
  auto step = [&](int v, auto uc) __attribute__((always_inline)) {
    constexpr int U = decltype(uc)::value;
    const bool live = v < nv;  // uniform
    const int vl = live ? v : nv - 1;
    const int it = lo + vl / NGW, gi = vl - (vl / NGW) * NGW, g = kh * NGW + gi;
    const int se = it / ntn;
    if (live && gi == 0 && se != cur) load_tile(se);  // uniform: same v sequence in every wave
    load_unit(min(v + kRing - 1, nv - 1), (U + kRing - 1) % kRing);
    wait_unit(U);
    if (!live) return;
    if (gi == 0) cs = bsv[U];  // uniform
    f4 ag[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m) ag[m][0] = ag[m][1] = f4{0.f, 0.f, 0.f, 0.f};
    if (two) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const h8 b0 = decode_unscaled(bq[U][0][st], mlo, mhi), b1 = decode_unscaled(bq[U][1][st], mlo, mhi);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const h8 af = *reinterpret_cast<const h8*>(&s.a[(16 * m + n) * LD + g * kGroup + 32 * q + 8 * st]);
          ag[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b0, ag[m][0], 0, 0, 0);
          ag[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b1, ag[m][1], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const h8 af = *reinterpret_cast<const h8*>(&s.a[n * LD + g * kGroup + 32 * q + 8 * st]);
        ag[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, decode_unscaled(bq[U][0][st], mlo, mhi), ag[0][0], 0, 0, 0);
        ag[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, decode_unscaled(bq[U][1][st], mlo, mhi), ag[0][1], 0, 0, 0);
      }
    }
    // scale of group g, row n of sub-tile j: lane n + 16 (2 j + g / 8), 16-bit
    // word g % 8 of its load (rows of 8 bytes: word g + 4 (n & 1))
    const int w = (g & 7) >> 1;  // uniform
    const uint32_t sw = SB == 8 ? ((n & 1) ? word_of(cs, w + 2) : word_of(cs, w)) : word_of(cs, w);
    const int src = n + 16 * (g >> 3);
    const uint32_t sv0 = (uint32_t)__shfl((int)sw, src, kWave);
    const uint32_t sv1 = (uint32_t)__shfl((int)sw, src + 32, kWave);
    const int sh = 16 * (g & 1);
    const float s0 = half_bits_to_float((uint16_t)(sv0 >> sh)), s1 = half_bits_to_float((uint16_t)(sv1 >> sh));
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      acc[m][0] += ag[m][0] * s0;
      acc[m][1] += ag[m][1] * s1;
    }
    if (gi == NGW - 1) {
      // item done: the second K half hands its sums to the first (the first
      // barrier keeps the buffer until the last item's sums have been read)
      if constexpr (KS == 2) {
        __syncthreads();
        if (kh == 1) {
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int j = 0; j < 2; ++j) s.red[wr][2 * m + j][lane] = acc[m][j];
        }
        __syncthreads();
        if (kh == 0) {
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[m][j] += s.red[wr][2 * m + j][lane];
        }
      }
      if (kh == 0) {
        // lane holds D[token 16m + 4q + r][row n] of both weight sub-tiles
        const int nt = it - se * ntn;
        const int cnt = s.count[se - se0], off = s.offset[se - se0];
        const bool shared = s.slot[se - se0] < 0;  // uniform
        _Float16* hout = reinterpret_cast<_Float16*>(shared ? a.shared_h : a.hbuf);
        float* yout = shared ? a.shared_y : a.ybuf;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tr = 16 * m + 4 * q + r;
            if (tr < cnt) {
              const int64_t pos = off + tr;
              if (MODE == 0) {
                const int row = nt * ROWS + wr * 16 + n;
                const float gv = acc[m][0][r], uv = acc[m][1][r];
                hout[pos * a.I + row] = (_Float16)swiglu(gv, uv);
              } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) yout[pos * a.H + nt * ROWS + wr * 32 + j * 16 + n] = acc[m][j][r];
              }
            }
          }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) acc[m][0] = acc[m][1] = f4{0.f, 0.f, 0.f, 0.f};
    }
  };
  for (int v0 = 0; v0 < nv; v0 += kRing) {
    [&]<int... Us>(std::integer_sequence<int, Us...>) {
      (step(v0 + Us, std::integral_constant<int, Us>{}), ...);
    }(std::make_integer_sequence<int, kRing>{});
  }
}

bool stream_group_in_kernel_ok(int T, int k, int E, int I, int grid, bool shared_rides) {
  if (E > 2 * kSW * kWave || T <= 0) return false;
  if (group_in_kernel_bytes(T, k, E) > sizeof(StreamSmem<2048>::a)) return false;
  // list entries: every active expert in chunks of kStreamTokens tokens, at
  // most min(E, P) + P / kStreamTokens of them, plus the shared expert; a run
  // of `per` consecutive items spans at most ceil(per / ntn) + 1 entries
  const int64_t P = (int64_t)T * k;
  const int ntn = I / (kSW / k_halves<2048>() * 16);
  if (ntn <= 0) return false;
  const int64_t ns = std::min<int64_t>(E, P) + P / kStreamTokens + (shared_rides ? 1 : 0);
  const int64_t per = (ns * ntn + grid - 1) / grid;
  return (per + ntn - 1) / ntn + 1 <= kBlockEntries;
}

bool stream_supported(int mode, int K, int rows) {
  const int ks = K == 1024 ? k_halves<1024>() : K == 512 ? k_halves<512>() : k_halves<2048>();
  const int per_item = mode == 0 ? kSW / ks * 16 : kSW / ks * 32;
  if (rows % per_item) return false;
  return mode == 0 ? K == 2048 : (K == 1024 || K == 512);
}

void launch_stream_expert(const ExpertArgs& a, int mode, int grid, hipStream_t stream) {
  if (mode == 0) {
    hipLaunchKernelGGL((stream_expert_kernel<0, 2048>), dim3(grid), dim3(kSW * kWave), 0, stream, a);
  } else if (a.I == 1024) {
    hipLaunchKernelGGL((stream_expert_kernel<1, 1024>), dim3(grid), dim3(kSW * kWave), 0, stream, a);
  } else {
    hipLaunchKernelGGL((stream_expert_kernel<1, 512>), dim3(grid), dim3(kSW * kWave), 0, stream, a);
  }
}

}  // namespace moe
