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
//   * each wave owns two 16-row weight sub-tiles (gate/up: the same 16 rows of
//     the gate and the up matrix, so SwiGLU is applied in registers; down: 32
//     consecutive rows) and keeps a ring of four scale groups of INT4 codes in
//     registers, loads running three groups ahead of the one being used;
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
constexpr int kRing = 4;                // weight groups held per wave: current + 3 in flight
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
constexpr int kFullRing = 8;
constexpr int kAFullHalves = 64 * (1024 + kAPad);  // >= MS*16 x (K + pad) for MS*K <= 4096
struct MfmaSmemFull {
  alignas(16) _Float16 a[kAFullHalves];
  int tok[kMT];
};
union MfmaShared {
  MfmaSmem d;
  MfmaSmemFull f;
};
template <int MODE, int MS>
constexpr bool afull_fits(int K) { return MS * K <= 4096; }

// One tile with MS 16-token sub-tiles (MS*16 >= tokens in the tile).
// MODE 0: gate/up + SwiGLU -> hbuf FP16 [position, I]; MODE 1: down -> ybuf FP32 [position, H].
template <int MODE, int MS>
__device__ __forceinline__ void mfma_tile(const MfmaArgs& a, MfmaSmem& s, const ActiveExpert& ae, int m0,
                                          int mcount, int nt) {
  constexpr int NA = (MS + 1) / 2;  // activation chunks of 16 B per thread and group
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int K = MODE == 0 ? a.H : a.I;
  const int ng = K / kKC;
  const uint8_t* blob = a.blobs + (int64_t)ae.slot * a.blob_stride;

  // the wave's two weight sub-tiles
  const uint8_t* codes[2];
  const uint16_t* scales[2];
  int row[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int mat, r;
    if (MODE == 0) {
      mat = j;                                   // 0 gate, 1 up: same rows
      r = nt * (kMW * 16) + wv * 16 + n;
    } else {
      mat = 2;
      r = nt * (kMW * 32) + wv * 32 + j * 16 + n;
    }
    row[j] = r;
    codes[j] = blob + a.lay.codes(mat) + (int64_t)r * (K / 2) + q * 16;
    scales[j] = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(mat)) + (int64_t)r * (K / kKC);
  }

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

  u4 bq[kRing][2];
  uint32_t bs[kRing][2];
  auto load_b = [&](int g, u4 (&dq)[2], uint32_t (&ds)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      dq[j] = *reinterpret_cast<const u4*>(codes[j] + g * 64);
      ds[j] = scales[j][g];
    }
  };
  // activation chunks of two groups in flight: group g + 1 is staged into
  // LDS during step g, group g + 2 is being loaded
  u4 av[2][NA];
  auto load_a = [&](int g, u4 (&dst)[NA]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; ++i) dst[i] = *reinterpret_cast<const u4*>(abase[i] + g * kKC);
  };
  auto store_a = [&](int buf, const u4 (&src)[NA]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; ++i) *reinterpret_cast<u4*>(&s.a[buf][arow[i]][acol[i]]) = src[i];
  };

  f4 acc[MS][2];
#pragma unroll
  for (int mi = 0; mi < MS; ++mi) acc[mi][0] = acc[mi][1] = f4{0.f, 0.f, 0.f, 0.f};

  // prologue: groups 0..kRing-2 of weights in flight, group 0 of activations
  // in LDS, group 1 in flight
  load_a(0, av[0]);
  load_a(min(1, ng - 1), av[1]);
#pragma unroll
  for (int u = 0; u < kRing - 1; ++u) load_b(min(u, ng - 1), bq[u], bs[u]);
  store_a(0, av[0]);
  __syncthreads();

  // one K group: prefetch, decode + MFMA, stage the next activations
  auto step = [&](int g, auto uc) __attribute__((always_inline)) {
    constexpr int U = decltype(uc)::value;
    // activations first, then weights: the wait for the activations staged
    // at the end of the step (loaded one step earlier) then leaves this
    // step's loads in flight (loads complete in issue order).  The
    // scheduling barriers keep this order and keep the loads at the top
    // instead of next to their first use.
    load_a(min(g + 2, ng - 1), av[U & 1]);
    __builtin_amdgcn_sched_barrier(0);
    load_b(min(g + kRing - 1, ng - 1), bq[(U + kRing - 1) % kRing], bs[(U + kRing - 1) % kRing]);
    __builtin_amdgcn_sched_barrier(0);
    const _Float16(*sa)[kKC + kAPad] = s.a[g & 1];
    h2 s2[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)bs[U][j]);
      s2[j] = h2{sv, sv};
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const h8 b0 = decode_scaled(bq[U][0][st], s2[0]);
      const h8 b1 = decode_scaled(bq[U][1][st], s2[1]);
#pragma unroll
      for (int mi = 0; mi < MS; ++mi) {
        const h8 af = *reinterpret_cast<const h8*>(&sa[mi * 16 + n][32 * q + 8 * st]);
        acc[mi][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b0, acc[mi][0], 0, 0, 0);
        acc[mi][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b1, acc[mi][1], 0, 0, 0);
      }
    }
    store_a((g + 1) & 1, av[(U + 1) & 1]);
    __syncthreads();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  int g = 0;
  for (; g + kRing <= ng; g += kRing) {
    step(g, C0{});
    step(g + 1, C1{});
    step(g + 2, C2{});
    step(g + 3, C3{});
  }
  if (g < ng) {  // ng is even: a tail of two groups
    step(g, C0{});
    step(g + 1, C1{});
  }

  // epilogue: lane holds D[token 4q + r][row n] of each sub-tile
#pragma unroll
  for (int mi = 0; mi < MS; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = mi * 16 + 4 * q + r;
      if (tr >= mcount) continue;
      const int pos = ae.offset + m0 + tr;
      if (MODE == 0) {
        const float gv = acc[mi][0][r], uv = acc[mi][1][r];
        reinterpret_cast<_Float16*>(a.hbuf)[(int64_t)pos * a.I + row[0]] =
            (_Float16)(gv / (1.0f + expf(-gv)) * uv);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) a.ybuf[(int64_t)pos * a.H + row[j]] = acc[mi][j][r];
      }
    }
  }
}

// Same arithmetic and summation order as mfma_tile, activation block resident.
template <int MODE, int MS>
__device__ __forceinline__ void mfma_tile_full(const MfmaArgs& a, MfmaSmemFull& s, const ActiveExpert& ae,
                                               int m0, int mcount, int nt) {
  constexpr int K = MODE == 0 ? 2048 : 1024;  // H (gate/up) or I (down) of the shapes that take this path
  constexpr int LD = K + kAPad;               // LDS row stride (halves)
  constexpr int NG = K / kKC;
  static_assert(MS * 16 * LD <= kAFullHalves, "activation block fits");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, q = lane >> 4;
  const uint8_t* blob = a.blobs + (int64_t)ae.slot * a.blob_stride;
  const uint8_t* codes[2];
  const uint16_t* scales[2];
  int row[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int mat, r;
    if (MODE == 0) {
      mat = j;
      r = nt * (kMW * 16) + wv * 16 + n;
    } else {
      mat = 2;
      r = nt * (kMW * 32) + wv * 32 + j * 16 + n;
    }
    row[j] = r;
    codes[j] = blob + a.lay.codes(mat) + (int64_t)r * (K / 2) + q * 16;
    scales[j] = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(mat)) + (int64_t)r * NG;
  }
  // the activation block goes straight to LDS (direct loads: no registers),
  // 512 halves of one row per wave instruction; rows past the tile's tokens
  // are zero; then the first kFullRing - 1 weight groups go out
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
  u4 bq[kFullRing][2];
  uint32_t bs[kFullRing][2];
  auto load_b = [&](int g, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bq[slot][j] = *reinterpret_cast<const u4*>(codes[j] + g * 64);
      bs[slot][j] = scales[j][g];
    }
  };
#pragma unroll
  for (int u = 0; u < kFullRing - 1; ++u) load_b(min(u, NG - 1), u);
  // the direct loads were issued first, so they have landed once all but the
  // weight loads issued after them are done; the barrier publishes them
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f4 acc[MS][2];
#pragma unroll
  for (int mi = 0; mi < MS; ++mi) acc[mi][0] = acc[mi][1] = f4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](int g, auto uc) __attribute__((always_inline)) {
    constexpr int U = decltype(uc)::value;
    load_b(min(g + kFullRing - 1, NG - 1), (U + kFullRing - 1) % kFullRing);
    __builtin_amdgcn_sched_barrier(0);
    h2 s2[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const _Float16 sv = __builtin_bit_cast(_Float16, (uint16_t)bs[U][j]);
      s2[j] = h2{sv, sv};
    }
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const h8 b0 = decode_scaled(bq[U][0][st], s2[0]);
      const h8 b1 = decode_scaled(bq[U][1][st], s2[1]);
#pragma unroll
      for (int mi = 0; mi < MS; ++mi) {
        const h8 af = *reinterpret_cast<const h8*>(&s.a[(mi * 16 + n) * LD + g * kKC + 32 * q + 8 * st]);
        acc[mi][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b0, acc[mi][0], 0, 0, 0);
        acc[mi][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, b1, acc[mi][1], 0, 0, 0);
      }
    }
  };
  static_assert(NG % kFullRing == 0, "whole rings of groups");
  for (int g = 0; g < NG; g += kFullRing) {
    [&]<int... Us>(std::integer_sequence<int, Us...>) {
      (step(g + Us, std::integral_constant<int, Us>{}), ...);
    }(std::make_integer_sequence<int, kFullRing>{});
  }
#pragma unroll
  for (int mi = 0; mi < MS; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = mi * 16 + 4 * q + r;
      if (tr >= mcount) continue;
      const int pos = ae.offset + m0 + tr;
      if (MODE == 0) {
        const float gv = acc[mi][0][r], uv = acc[mi][1][r];
        reinterpret_cast<_Float16*>(a.hbuf)[(int64_t)pos * a.I + row[0]] =
            (_Float16)(gv / (1.0f + expf(-gv)) * uv);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) a.ybuf[(int64_t)pos * a.H + row[j]] = acc[mi][j][r];
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(kMW * kWave) void mfma_expert_kernel(MfmaArgs a) {
  __shared__ MfmaShared sh;
  MfmaSmem& s = sh.d;
  const int rows_per_block = kMW * (MODE == 0 ? 16 : 32);
  const int ntn = (MODE == 0 ? a.I : a.H) / rows_per_block;
  // block -> (token tile mg, row tile nt): the ntn row tiles of a token tile
  // share an XCD; token tiles are dealt round-robin over the XCDs
  const int xcd = blockIdx.x % kXcd, j = blockIdx.x / kXcd;
  const int nt = j % ntn;
  const int mg = (j / ntn) * kXcd + xcd;
  const int na = *a.n_active;
  if (mg >= a.mtile_off[na]) return;
  int lo = 0, hi = na - 1;  // largest ai with mtile_off[ai] <= mg
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.mtile_off[mid] <= mg) lo = mid; else hi = mid - 1;
  }
  const ActiveExpert ae = a.active[lo];
  const int m0 = (mg - a.mtile_off[lo]) * kMT;
  const int mcount = min(kMT, ae.count - m0);
  // exactly as many 16-token sub-tiles as the tile needs: MFMA work is not
  // padded beyond the next multiple of 16 tokens
  // the resident-activation tiles serve the two shapes it is built for
  const bool full_ok = (MODE == 0 ? a.H : a.I) == (MODE == 0 ? 2048 : 1024);
  switch ((mcount + 15) >> 4) {
    case 1:
      if (full_ok) mfma_tile_full<MODE, 1>(a, sh.f, ae, m0, mcount, nt);
      else mfma_tile<MODE, 1>(a, s, ae, m0, mcount, nt);
      break;
    case 2:
      if (full_ok) mfma_tile_full<MODE, 2>(a, sh.f, ae, m0, mcount, nt);
      else mfma_tile<MODE, 2>(a, s, ae, m0, mcount, nt);
      break;
    case 3:
      if (MODE == 1 && full_ok) mfma_tile_full<1, 3>(a, sh.f, ae, m0, mcount, nt);
      else mfma_tile<MODE, 3>(a, s, ae, m0, mcount, nt);
      break;
    case 4:
      if (MODE == 1 && full_ok) mfma_tile_full<1, 4>(a, sh.f, ae, m0, mcount, nt);
      else mfma_tile<MODE, 4>(a, s, ae, m0, mcount, nt);
      break;
    case 5: mfma_tile<MODE, 5>(a, s, ae, m0, mcount, nt); break;
    case 6: mfma_tile<MODE, 6>(a, s, ae, m0, mcount, nt); break;
    case 7: mfma_tile<MODE, 7>(a, s, ae, m0, mcount, nt); break;
    default: mfma_tile<MODE, 8>(a, s, ae, m0, mcount, nt); break;
  }
}

static int rows_per_block(int mode) { return kMW * (mode == 0 ? 16 : 32); }

int mfma_max_tiles(int T, int k, int E, int rows, int mode) {
  const int pairs = T * k;
  const int max_mtiles = (pairs + kMT - 1) / kMT + std::min(E, pairs);
  const int ntn = rows / rows_per_block(mode);
  // the block mapping covers token tiles in multiples of the XCD count
  return ((max_mtiles + kXcd - 1) / kXcd) * kXcd * ntn;
}

void launch_mfma_gateup(const MfmaArgs& a, int max_tiles, hipStream_t stream) {
  if (max_tiles > 0)
    hipLaunchKernelGGL((mfma_expert_kernel<0>), dim3(max_tiles), dim3(kMW * kWave), 0, stream, a);
}

void launch_mfma_down(const MfmaArgs& a, int max_tiles, hipStream_t stream) {
  if (max_tiles > 0)
    hipLaunchKernelGGL((mfma_expert_kernel<1>), dim3(max_tiles), dim3(kMW * kWave), 0, stream, a);
}

}  // namespace moe
