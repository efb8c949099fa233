// Grouped GEMM on FP16 MFMA for experts that receive many tokens (batched
// decode, prefill).  The expert FFN runs straight from packed INT4 weights with
// FP16 group scales and FP16 activations ("Horizon RunMap", "Architecture
// invariants"); this is the dense-contraction form of the same arithmetic as
// the GEMV kernels.
//
// Work is a list of tiles (active expert, tile of up to 128 gathered tokens,
// tile of output rows) built from the grouping's per-expert token counts, so
// an expert with at most 128 tokens streams its weights exactly once.  A block
// of 8 waves (one block per compute unit):
//   * stages the tile's 128-wide K slice of activations (rows gathered by
//     token, zero past the expert's count) in LDS, double buffered: the next
//     group's rows are loaded into registers while the current one computes;
//   * each wave owns NB 16-row weight sub-tiles (gate/up: NB/2 blocks of 16
//     rows, each taken from both the gate and the up matrix, so SwiGLU is
//     applied in registers; down: 16*NB consecutive rows) and keeps a ring of
//     scale groups of INT4 codes in registers, loads running ahead of the
//     group being used.  Four sub-tiles per wave (the default) let every
//     activation fragment read from LDS feed four MFMAs, which halves the LDS
//     traffic of two and makes one block cover 256 intermediate (gate/up) or
//     512 hidden (down) rows, so a 512-token prefill of 64 experts is a single
//     round of 256 blocks;
//   * the codes of a group are decoded once, multiplied by their FP16 group
//     scale (rounding each weight to FP16, a relative error of at most 2^-11)
//     and fed to v_mfma_f32_16x16x32_f16 for every 16-token sub-tile.
// All global loads in the main loop are unconditional (indices are clamped),
// so the compiler's wait counters track each load exactly and the prefetch
// overlaps the MFMA work.
// Tiles are mapped to blocks so that the row tiles of one token tile land on
// the same XCD (blocks are dispatched round-robin over the 8 XCDs) and share
// its L2 for the activation rows.
// MFMA operand layout (gfx950): A[l%16][8*(l/16)+e], B[8*(l/16)+e][l%16],
// D[4*(l/16)+r][l%16]; the K index of step st, lane group q, element e is
// kb + 32q + 8st + e for both operands.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));  // native vector: stays in registers

constexpr int kMW = 8;                  // waves per block
constexpr int kMT = kMfmaTileTokens;    // tokens per tile (8 sub-tiles of 16)
constexpr int kKC = 128;                // K per main-loop step (= one scale group)
constexpr int kAPad = 8;                // LDS row padding (halves) against bank conflicts
// weight groups held per wave (current + kRing - 1 in flight); four sub-tiles
// per wave hold twice the registers per group
template <int NB, int MS>
constexpr int ring_depth() { return NB == 4 ? (MS <= 4 ? 4 : MS <= 6 ? 3 : 2) : 4; }
constexpr int kXcd = 8;                 // XCDs; blocks go round-robin over them

// 8 INT4 codes (one dword) -> 8 FP16 weights (q - 8) * scale.
__device__ __forceinline__ h8 decode_scaled(uint32_t d, h2 s2) {
  h2 p[4];
  dequant8_v(d, p, 0x000F000Fu, 0x00F000F0u);
  p[0] *= s2; p[1] *= s2; p[2] *= s2; p[3] *= s2;
  h8 r;
  r[0] = p[0][0]; r[1] = p[0][1]; r[2] = p[1][0]; r[3] = p[1][1];
  r[4] = p[2][0]; r[5] = p[2][1]; r[6] = p[3][0]; r[7] = p[3][1];
  return r;
}


// (16-byte alignment lets the 16-byte operand reads be single instructions)
struct MfmaSmem {
  alignas(16) _Float16 a[2][kMT + 1][kKC + kAPad];   // row kMT takes the stores of padding rows
  int tok[kMT];
};

// Tiles of few tokens keep their whole activation block (all K) in LDS, so the
// main loop has no barrier and no activation traffic and only streams weights,
// with a deeper ring of weight groups in flight.  Fits when MS * K <= 4096.
template <int NB>
constexpr int full_ring_depth() { return NB == 4 ? 4 : 8; }
constexpr int kAFullHalves = 64 * (1024 + kAPad);  // >= MS*16 x (K + pad) for MS*K <= 4096
struct MfmaSmemFull {
  alignas(16) _Float16 a[kAFullHalves];
  int tok[kMT];
};
union MfmaShared {
  MfmaSmem d;
  MfmaSmemFull f;
};
// Rows of the wave's weight sub-tiles: a block covers block_rows<MODE, NB>()
// consecutive output rows (gate/up: rows of I, each in both matrices).
template <int MODE, int NB>
constexpr int wave_rows() { return MODE == 0 ? 8 * NB : 16 * NB; }
template <int MODE, int NB>
constexpr int block_rows() { return kMW * wave_rows<MODE, NB>(); }

// A pointer that is the same in every lane, moved to scalar registers so that
// loads address it as scalar base + per-lane 32-bit offset.
template <class T>
__device__ __forceinline__ const T* wave_uniform(const T* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// Weight sub-tile bases of a wave (uniform) and the lane's offsets into them:
// lane (n, q) reads row n of a sub-tile, bytes [16q, 16q + 16) of each 64-byte
// group of codes, and the row's scale of each group.
template <int MODE, int NB>
struct WaveTiles {
  const uint8_t* code[NB];
  const uint8_t* scale[NB];
  uint32_t lane_code, lane_scale;  // byte offsets
  int row[NB];                     // output row of each sub-tile for this lane
  __device__ __forceinline__ WaveTiles(const MfmaArgs& a, const uint8_t* blob, int K, int nt, int wv, int n,
                                       int q) {
    const int ng = K / kKC;
    const int base = nt * block_rows<MODE, NB>() + wv * wave_rows<MODE, NB>();
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      // gate/up: sub-tiles 2p (gate) and 2p + 1 (up) share rows base + 16p + n
      const int mat = MODE == 0 ? (j & 1) : 2;
      const int r0 = base + 16 * (MODE == 0 ? (j >> 1) : j);
      row[j] = r0 + n;
      code[j] = wave_uniform(blob + a.lay.codes(mat) + code_offset(r0, 0, K / 2));  // r0 % 16 == 0
      scale[j] = wave_uniform(blob + a.lay.scales(mat) + (int64_t)r0 * ng * 2);
    }
    lane_code = (uint32_t)(n * kCodeGroupBytes + q * 16);
    lane_scale = (uint32_t)(n * ng * 2);
  }
  // global (not flat) loads: flat loads would also hold up every LDS wait
  __device__ __forceinline__ u4 codes(int j, int g) const {
    return ldg<u4>(code[j] + (lane_code + (uint32_t)(g * kCodeGroupStride)));
  }
  __device__ __forceinline__ uint32_t scale_of(int j, int g) const {
    return ldg<uint16_t>(scale[j] + (lane_scale + (uint32_t)g * 2u));
  }
};

// One tile with MS 16-token sub-tiles (MS*16 >= tokens in the tile).
// MODE 0: gate/up + SwiGLU -> hbuf FP16 [position, I]; MODE 1: down -> ybuf FP32 [position, H].
template <int MODE, int MS, int NB>
__device__ __forceinline__ void mfma_tile(const MfmaArgs& a, MfmaSmem& s, const ActiveExpert& ae, int m0,
                                          int mcount, int nt) {
  constexpr int NA = (MS + 1) / 2;  // activation chunks of 16 B per thread and group
  constexpr int R = ring_depth<NB, MS>();
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int K = MODE == 0 ? a.H : a.I;
  const int ng = K / kKC;
  const uint8_t* blob = a.blobs + (int64_t)ae.slot * a.blob_stride;

  // the wave's weight sub-tiles
  const WaveTiles<MODE, NB> wt(a, blob, K, nt, wv, n, q);
  const int(&row)[NB] = wt.row;

  u4 bq[R][NB];
  uint32_t bs[R][NB];
  auto load_b = [&](int g, u4 (&dq)[NB], uint32_t (&ds)[NB]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      dq[j] = wt.codes(j, g);
      ds[j] = wt.scale_of(j, g);
    }
  };
  // the first R - 1 weight groups go out before the token rows are known
#pragma unroll
  for (int u = 0; u < R - 1; ++u) load_b(min(u, ng - 1), bq[u], bs[u]);

  // activation rows: token ids (gate/up) or sorted positions (down)
  if (tid < kMT) {
    int v = -1;
    if (tid < mcount) v = MODE == 0 ? a.perm_tok[ae.offset + m0 + tid] : ae.offset + m0 + tid;
    s.tok[tid] = v;
  }
  __syncthreads();
  // rows past the tile's tokens stay zero in both buffers
  for (int c = tid; c < MS * 16 * (kKC / 8); c += kMW * kWave) {
    const int r = c >> 4, col = (c & 15) * 8;
    if (r >= mcount) {
      *reinterpret_cast<uint4*>(&s.a[0][r][col]) = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(&s.a[1][r][col]) = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // activation chunks of this thread: a padding row loads a valid row and
  // stores it into the spare LDS row, so loads and stores are unconditional
  const uint16_t* abase[NA];
  int arow[NA], acol[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int c = tid + i * kMW * kWave;
    const int r = c >> 4;
    const bool valid = r < mcount;
    arow[i] = valid ? r : kMT;
    acol[i] = (c & 15) * 8;
    abase[i] = (MODE == 0 ? a.x : a.hbuf) + (int64_t)s.tok[valid ? r : 0] * K + acol[i];
  }

  // activation chunks of the next group: loaded at the top of step g and
  // staged into LDS at its end (group g + 1)
  u4 av[NA];
  auto load_a = [&](int g, u4 (&dst)[NA]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; ++i) dst[i] = *reinterpret_cast<const u4*>(abase[i] + g * kKC);
  };
  auto store_a = [&](int buf, const u4 (&src)[NA]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; ++i) *reinterpret_cast<u4*>(&s.a[buf][arow[i]][acol[i]]) = src[i];
  };

  f4 acc[MS][NB];
#pragma unroll
  for (int mi = 0; mi < MS; ++mi)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mi][j] = f4{0.f, 0.f, 0.f, 0.f};

  // prologue: group 0 of activations in LDS
  load_a(0, av);
  store_a(0, av);
  __syncthreads();

  // one K group: prefetch, decode + MFMA, stage the next activations.  U is
  // the group's ring slot (g mod R), P its activation register set (g mod 2).
  auto step = [&](int g, auto uc, auto pc) __attribute__((always_inline)) {
    constexpr int U = decltype(uc)::value;
    constexpr int P = decltype(pc)::value;
    // activations first, then weights: the wait for the activations staged
    // at the end of the step (loaded one step earlier) then leaves this
    // step's loads in flight (loads complete in issue order).  The
    // scheduling barriers keep this order and keep the loads at the top
    // instead of next to their first use.
    load_a(min(g + 1, ng - 1), av);
    __builtin_amdgcn_sched_barrier(0);
    const int gl = min(g + R - 1, ng - 1);
    const _Float16(*sa)[kKC + kAPad] = s.a[P];
    h2 s2[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)bs[U][j]);
      s2[j] = h2{sv, sv};
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      h8 b[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) b[j] = decode_scaled(bq[U][j][st], s2[j]);
      // the weight loads of group g + R - 1 are spread over the K slices so
      // that the vector memory unit works while the slices compute
#pragma unroll
      for (int j = st * NB / 4; j < (st + 1) * NB / 4; ++j) {
        bq[(U + R - 1) % R][j] = wt.codes(j, gl);
        bs[(U + R - 1) % R][j] = wt.scale_of(j, gl);
      }
#pragma unroll
      for (int mi = 0; mi < MS; ++mi) {
        const h8 af = *reinterpret_cast<const h8*>(&sa[mi * 16 + n][32 * q + 8 * st]);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[mi][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b[j], acc[mi][j], 0, 0, 0);
      }
      // one K slice at a time: operands of later slices are not hoisted
      __builtin_amdgcn_sched_barrier(0);
    }
    store_a(P ^ 1, av);
    __syncthreads();
  };
  // groups in whole periods of lcm(R, 2) steps, so that both ring indices
  // are compile-time constants; the tail runs the first steps of a period
  constexpr int PER = R % 2 == 0 ? R : 2 * R;
  auto period = [&](int g0, int count) __attribute__((always_inline)) {
    [&]<int... Us>(std::integer_sequence<int, Us...>) {
      ((Us < count ? step(g0 + Us, std::integral_constant<int, Us % R>{},
                          std::integral_constant<int, Us % 2>{})
                   : void()),
       ...);
    }(std::make_integer_sequence<int, PER>{});
  };
  int g = 0;
  for (; g + PER <= ng; g += PER) period(g, PER);
  if (g < ng) period(g, ng - g);

  // epilogue: lane holds D[token 4q + r][row n] of each sub-tile
#pragma unroll
  for (int mi = 0; mi < MS; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = mi * 16 + 4 * q + r;
      if (tr >= mcount) continue;
      const int pos = ae.offset + m0 + tr;
      if (MODE == 0) {
#pragma unroll
        for (int p = 0; p < NB / 2; ++p) {
          const float gv = acc[mi][2 * p][r], uv = acc[mi][2 * p + 1][r];
          reinterpret_cast<_Float16*>(a.hbuf)[(int64_t)pos * a.I + row[2 * p]] =
              (_Float16)swiglu(gv, uv);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) a.ybuf[(int64_t)pos * a.H + row[j]] = acc[mi][j][r];
      }
    }
  }
}

// Same arithmetic and summation order as mfma_tile, activation block resident.
template <int MODE, int MS, int NB>
__device__ __forceinline__ void mfma_tile_full(const MfmaArgs& a, MfmaSmemFull& s, const ActiveExpert& ae,
                                               int m0, int mcount, int nt) {
  constexpr int K = MODE == 0 ? 2048 : 1024;  // H (gate/up) or I (down) of the shapes that take this path
  constexpr int LD = K + kAPad;               // LDS row stride (halves)
  constexpr int NG = K / kKC;
  constexpr int R = full_ring_depth<NB>();
  static_assert(MS * 16 * LD <= kAFullHalves, "activation block fits");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const uint8_t* blob = a.blobs + (int64_t)ae.slot * a.blob_stride;
  const WaveTiles<MODE, NB> wt(a, blob, K, nt, wv, n, q);
  const int(&row)[NB] = wt.row;
  // the activation block goes straight to LDS (direct loads: no registers),
  // 512 halves of one row per wave instruction; rows past the tile's tokens
  // are zero; then the first R - 1 weight groups go out
  if (tid < kMT) {
    int v = -1;
    if (tid < mcount) v = MODE == 0 ? a.perm_tok[ae.offset + m0 + tid] : ae.offset + m0 + tid;
    s.tok[tid] = v;
  }
  __syncthreads();
  {
    const uint16_t* src = MODE == 0 ? a.x : a.hbuf;
    constexpr int SEG = K / 512;                      // 1-KB segments per row
    for (int c = wv; c < MS * 16 * SEG; c += kMW) {   // wave-uniform
      const int r = c / SEG, b = c - r * SEG;
      _Float16* dst = &s.a[r * LD + b * 512];
      if (r < mcount)
        dma_lds16(src + (int64_t)s.tok[r] * K + b * 512 + lane * 8, lds_addr(dst));
      else
        *reinterpret_cast<u4*>(dst + lane * 8) = u4{0u, 0u, 0u, 0u};
    }
  }
  u4 bq[R][NB];
  uint32_t bs[R][NB];
  auto load_b = [&](int g, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      bq[slot][j] = wt.codes(j, g);
      bs[slot][j] = wt.scale_of(j, g);
    }
  };
#pragma unroll
  for (int u = 0; u < R - 1; ++u) load_b(min(u, NG - 1), u);
  // the direct loads were issued first, so they have landed once all but the
  // weight loads issued after them are done; the barrier publishes them
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f4 acc[MS][NB];
#pragma unroll
  for (int mi = 0; mi < MS; ++mi)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[mi][j] = f4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](int g, auto uc) __attribute__((always_inline)) {
    constexpr int U = decltype(uc)::value;
    load_b(min(g + R - 1, NG - 1), (U + R - 1) % R);
    __builtin_amdgcn_sched_barrier(0);
    h2 s2[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)bs[U][j]);
      s2[j] = h2{sv, sv};
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      h8 b[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) b[j] = decode_scaled(bq[U][j][st], s2[j]);
#pragma unroll
      for (int mi = 0; mi < MS; ++mi) {
        const h8 af = *reinterpret_cast<const h8*>(&s.a[(mi * 16 + n) * LD + g * kKC + 32 * q + 8 * st]);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[mi][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b[j], acc[mi][j], 0, 0, 0);
      }
    }
  };
  static_assert(NG % R == 0, "whole rings of groups");
  for (int g = 0; g < NG; g += R) {
    [&]<int... Us>(std::integer_sequence<int, Us...>) {
      (step(g + Us, std::integral_constant<int, Us>{}), ...);
    }(std::make_integer_sequence<int, R>{});
  }
#pragma unroll
  for (int mi = 0; mi < MS; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = mi * 16 + 4 * q + r;
      if (tr >= mcount) continue;
      const int pos = ae.offset + m0 + tr;
      if (MODE == 0) {
#pragma unroll
        for (int p = 0; p < NB / 2; ++p) {
          const float gv = acc[mi][2 * p][r], uv = acc[mi][2 * p + 1][r];
          reinterpret_cast<_Float16*>(a.hbuf)[(int64_t)pos * a.I + row[2 * p]] =
              (_Float16)swiglu(gv, uv);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j) a.ybuf[(int64_t)pos * a.H + row[j]] = acc[mi][j][r];
      }
    }
  }
}

template <int MODE, int NB>
__global__ __launch_bounds__(kMW * kWave) void mfma_expert_kernel(MfmaArgs a) {
  __shared__ MfmaShared sh;
  MfmaSmem& s = sh.d;
  const int ntn = (MODE == 0 ? a.I : a.H) / block_rows<MODE, NB>();
  // block -> (token tile mg, row tile nt): the ntn row tiles of a token tile
  // share an XCD; token tiles are dealt round-robin over the XCDs
  const int xcd = blockIdx.x % kXcd, j = blockIdx.x / kXcd;
  const int nt = j % ntn;
  const int mg = (j / ntn) * kXcd + xcd;
  // the active expert owning token tile mg: every thread tests one expert's
  // tile range (one round of loads instead of a dependent binary search)
  __shared__ int sh_ai, sh_m0;
  const int na = *a.n_active;
  if (threadIdx.x == 0) sh_ai = -1;
  __syncthreads();
  for (int t = threadIdx.x; t < na; t += kMW * kWave) {
    const int o0 = a.mtile_off[t], o1 = a.mtile_off[t + 1];
    if (o0 <= mg && mg < o1) {
      sh_ai = t;
      sh_m0 = (mg - o0) * kMT;
    }
  }
  __syncthreads();
  const int ai = sh_ai;
  if (ai < 0) return;  // past the last token tile (uniform over the block)
  const ActiveExpert ae = a.active[ai];
  const int m0 = sh_m0;
  const int mcount = min(kMT, ae.count - m0);
  // exactly as many 16-token sub-tiles as the tile needs: MFMA work is not
  // padded beyond the next multiple of 16 tokens
  // the resident-activation tiles serve the two shapes it is built for
  const bool full_ok = (MODE == 0 ? a.H : a.I) == (MODE == 0 ? 2048 : 1024);
  switch ((mcount + 15) >> 4) {
    case 1:
      if (full_ok) mfma_tile_full<MODE, 1, NB>(a, sh.f, ae, m0, mcount, nt);
      else mfma_tile<MODE, 1, NB>(a, s, ae, m0, mcount, nt);
      break;
    case 2:
      if (full_ok) mfma_tile_full<MODE, 2, NB>(a, sh.f, ae, m0, mcount, nt);
      else mfma_tile<MODE, 2, NB>(a, s, ae, m0, mcount, nt);
      break;
    case 3:
      if (MODE == 1 && full_ok) mfma_tile_full<1, 3, NB>(a, sh.f, ae, m0, mcount, nt);
      else mfma_tile<MODE, 3, NB>(a, s, ae, m0, mcount, nt);
      break;
    case 4:
      if (MODE == 1 && full_ok) mfma_tile_full<1, 4, NB>(a, sh.f, ae, m0, mcount, nt);
      else mfma_tile<MODE, 4, NB>(a, s, ae, m0, mcount, nt);
      break;
    case 5: mfma_tile<MODE, 5, NB>(a, s, ae, m0, mcount, nt); break;
    case 6: mfma_tile<MODE, 6, NB>(a, s, ae, m0, mcount, nt); break;
    case 7: mfma_tile<MODE, 7, NB>(a, s, ae, m0, mcount, nt); break;
    default: mfma_tile<MODE, 8, NB>(a, s, ae, m0, mcount, nt); break;
  }
}

// Four sub-tiles per wave where the rows divide into blocks of that size,
// else two.
static int mfma_nb(int mode, int rows) {
  return rows % (mode == 0 ? block_rows<0, 4>() : block_rows<1, 4>()) == 0 ? 4 : 2;
}

static int rows_per_block(int mode, int nb) {
  if (mode == 0) return nb == 4 ? block_rows<0, 4>() : block_rows<0, 2>();
  return nb == 4 ? block_rows<1, 4>() : block_rows<1, 2>();
}

int mfma_max_tiles(int T, int k, int E, int rows, int mode, int mfma_min) {
  const int pairs = T * k;
  // sum over those experts of ceil(n_e / kMT) <= ceil(pairs / kMT) + their
  // number, which is at most min(E, pairs / mfma_min)
  const int max_mtiles = (pairs + kMT - 1) / kMT + std::min(E, pairs / std::max(mfma_min, 1));
  const int ntn = rows / rows_per_block(mode, mfma_nb(mode, rows));
  // the block mapping covers token tiles in multiples of the XCD count
  return ((max_mtiles + kXcd - 1) / kXcd) * kXcd * ntn;
}

void launch_mfma_gateup(const MfmaArgs& a, int max_tiles, hipStream_t stream) {
  if (max_tiles <= 0) return;
  if (mfma_nb(0, a.I) == 4)
    hipLaunchKernelGGL((mfma_expert_kernel<0, 4>), dim3(max_tiles), dim3(kMW * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((mfma_expert_kernel<0, 2>), dim3(max_tiles), dim3(kMW * kWave), 0, stream, a);
}

void launch_mfma_down(const MfmaArgs& a, int max_tiles, hipStream_t stream) {
  if (max_tiles <= 0) return;
  if (mfma_nb(1, a.H) == 4)
    hipLaunchKernelGGL((mfma_expert_kernel<1, 4>), dim3(max_tiles), dim3(kMW * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((mfma_expert_kernel<1, 2>), dim3(max_tiles), dim3(kMW * kWave), 0, stream, a);
}

}  // namespace moe
