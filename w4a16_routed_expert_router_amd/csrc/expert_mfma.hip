// Grouped GEMM on FP16 MFMA for experts that receive many tokens (batched
// decode, prefill).  The expert FFN runs straight from packed INT4 weights with
// FP16 group scales and FP16 activations ("Horizon RunMap", "Architecture
// invariants"); this is the dense-contraction form of the same arithmetic as
// the GEMV kernels.
//
// Work is a list of tiles (active expert, tile of 64 gathered tokens, tile of
// output rows) built from the grouping's per-expert token counts.  A block of
// 8 waves:
//   * stages the 64 x 128 FP16 activation slice of the current scale group in
//     LDS (rows gathered by token, zero past the expert's count), double
//     buffered, the next group's rows loaded while the current one computes;
//   * each wave owns 2 x 16 weight rows, loads 16 contiguous INT4 bytes per row
//     and lane per group (prefetched two groups ahead), decodes them once, and
//     runs (token sub-tiles holding tokens, up to 4) x 2 (row sub-tiles) x 4 K-steps of
//     v_mfma_f32_16x16x32_f16; each 128-wide group is accumulated separately
//     and added to the FP32 result times the row's FP16 scale.
// Gate/up tiles pair the same 16 gate and up rows in a wave, so SwiGLU is
// applied in registers; down tiles write FP32 rows per (token, rank) position.
// MFMA operand layout (gfx950): A[l%16][8*(l/16)+e], B[8*(l/16)+e][l%16],
// D[4*(l/16)+r][l%16]; the K index of step st, lane group q, element e is
// kb + 32q + 8st + e for both operands.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace moe {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kMT = 64;    // tokens per tile
constexpr int kMW = 8;     // waves per block
constexpr int kKC = 128;   // K per step of the main loop (= one scale group)
constexpr int kAPad = 8;   // LDS row padding (halves) against bank conflicts

__device__ __forceinline__ h8 decode_dword(uint32_t d) {
  h2 p[4];
  dequant8(d, p);
  h8 r;
  r[0] = p[0][0]; r[1] = p[0][1]; r[2] = p[1][0]; r[3] = p[1][1];
  r[4] = p[2][0]; r[5] = p[2][1]; r[6] = p[3][0]; r[7] = p[3][1];
  return r;
}

__device__ __forceinline__ uint32_t dw(const uint4& q, int i) {
  return i == 0 ? q.x : (i == 1 ? q.y : (i == 2 ? q.z : q.w));
}

// Tile -> (active expert, token tile, row tile); false if past the end.
__device__ __forceinline__ bool find_tile(const MfmaArgs& a, int tile, int ntn, int& ai, int& mt,
                                          int& nt) {
  nt = tile % ntn;
  const int mg = tile / ntn;
  const int na = *a.n_active;
  if (mg >= a.mtile_off[na]) return false;
  int lo = 0, hi = na - 1;  // largest ai with mtile_off[ai] <= mg
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.mtile_off[mid] <= mg) lo = mid; else hi = mid - 1;
  }
  ai = lo;
  mt = mg - a.mtile_off[lo];
  return true;
}

// MODE 0: gate/up + SwiGLU (K = H; a wave owns 32 gate rows and the same 32 up
//         rows: 4 sub-tiles; 256 + 256 rows per tile; output h FP16)
// MODE 1: down (K = I; a wave owns 16*NSUB output rows; output y FP32)
template <int MODE, int NSUB>
__global__ __launch_bounds__(kMW * kWave) void mfma_expert_kernel(MfmaArgs a) {
  static_assert(MODE == 1 || NSUB == 4, "gate/up tiles pair 2 gate + 2 up sub-tiles");
  __shared__ __align__(16) _Float16 sa[2][kMT][kKC + kAPad];
  __shared__ int stok[kMT];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int K = MODE == 0 ? a.H : a.I;
  const int rows_per_wave = 16 * (MODE == 0 ? NSUB / 2 : NSUB);
  const int rows_per_tile = kMW * rows_per_wave;
  const int nrows = MODE == 0 ? a.I : a.H;
  const int ntn = nrows / rows_per_tile;
  int ai, mt, nt;
  if (!find_tile(a, blockIdx.x, ntn, ai, mt, nt)) return;
  const ActiveExpert ae = a.active[ai];
  const uint8_t* blob = a.blobs + (int64_t)ae.slot * a.blob_stride;
  const int m0 = mt * kMT;
  const int mcount = min(kMT, ae.count - m0);
  // rows of A: token ids (gate/up) or sorted positions (down); -1 = padding
  if (tid < kMT) {
    int v = -1;
    if (tid < mcount) v = MODE == 0 ? a.perm_tok[ae.offset + m0 + tid] : ae.offset + m0 + tid;
    stok[tid] = v;
  }
  __syncthreads();

  const int n = lane & 15, q = lane >> 4;
  // weight sub-tile j: 16 rows of one matrix
  int row[NSUB];
  const uint8_t* codes[NSUB];
  const uint16_t* scales[NSUB];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    int r, mat;
    if (MODE == 0) {
      mat = j / 2;                                   // 0,1 gate; 2,3 up
      r = nt * rows_per_tile + wv * rows_per_wave + (j & 1) * 16 + n;
    } else {
      mat = 2;
      r = nt * rows_per_tile + wv * rows_per_wave + j * 16 + n;
    }
    row[j] = r;
    codes[j] = blob + a.lay.codes(mat) + (int64_t)r * (K / 2);
    scales[j] = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(mat)) + (int64_t)r * (K / 128);
  }

  // A staging: 64 rows x 128 halves = 1024 chunks of 16 B, 2 per thread
  auto load_a = [&](int g, uint4 (&buf)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * kMW * kWave;
      const int r = c >> 4, col = (c & 15) * 8;
      const int src = stok[r];
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (src >= 0) {
        const uint16_t* base = MODE == 0 ? a.x + (int64_t)src * K : a.hbuf + (int64_t)src * K;
        v = *reinterpret_cast<const uint4*>(base + g * kKC + col);
      }
      buf[i] = v;
    }
  };
  auto store_a = [&](int s, const uint4 (&buf)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * kMW * kWave;
      const int r = c >> 4, col = (c & 15) * 8;
      *reinterpret_cast<uint4*>(&sa[s][r][col]) = buf[i];
    }
  };
  // weights of group g for every sub-tile: 16 contiguous bytes per row and lane
  auto load_b = [&](int g, uint4 (&bq)[NSUB], float (&bs)[NSUB]) {
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      bq[j] = *reinterpret_cast<const uint4*>(codes[j] + g * 64 + q * 16);
      bs[j] = half_bits_to_float(scales[j][g]);
    }
  };

  const int ng = K / kKC;
  const int msub = (mcount + 15) >> 4;   // 16-token sub-tiles that hold tokens
  f4 acc[4][NSUB];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[mi][j] = f4{0.f, 0.f, 0.f, 0.f};

  uint4 bq[NSUB], nq[NSUB];
  float bs[NSUB], ns[NSUB];
  load_b(0, bq, bs);
  uint4 abuf[2];
  load_a(0, abuf);
  store_a(0, abuf);
  __syncthreads();

  for (int g = 0; g < ng; ++g) {
    const int s = g & 1;
    const bool more = g + 1 < ng;
    if (more) {
      load_b(g + 1, nq, ns);
      load_a(g + 1, abuf);
    }
    // decode this group's weights once; each A fragment then feeds NSUB MFMAs
    h8 bf[NSUB][4];
#pragma unroll
    for (int j = 0; j < NSUB; ++j)
#pragma unroll
      for (int st = 0; st < 4; ++st) bf[j][st] = decode_dword(dw(bq[j], st));
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (mi < msub) {
        h8 af[4];
#pragma unroll
        for (int st = 0; st < 4; ++st)
          af[st] = *reinterpret_cast<const h8*>(&sa[s][mi * 16 + n][32 * q + 8 * st]);
#pragma unroll
        for (int j = 0; j < NSUB; ++j) {
          f4 ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < 4; ++st) ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[st], bf[j][st], ag, 0, 0, 0);
          acc[mi][j] += ag * bs[j];
        }
      }
    }
    if (more) store_a(s ^ 1, abuf);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      bq[j] = nq[j];
      bs[j] = ns[j];
    }
  }

  // epilogue: lane holds D[token 4q + r][row n] of each sub-tile
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tr = mi * 16 + 4 * q + r;
      if (tr >= mcount) continue;
      const int pos = ae.offset + m0 + tr;
      if (MODE == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float gv = acc[mi][j][r], uv = acc[mi][j + 2][r];
          reinterpret_cast<_Float16*>(a.hbuf)[(int64_t)pos * a.I + row[j]] =
              (_Float16)(gv / (1.0f + expf(-gv)) * uv);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NSUB; ++j) a.ybuf[(int64_t)pos * a.H + row[j]] = acc[mi][j][r];
      }
    }
  }
}

static int down_nsub(int H) { return H % (kMW * 64) == 0 ? 4 : 2; }

int mfma_max_tiles(int T, int k, int E, int rows, int mode) {
  const int pairs = T * k;
  const int max_mtiles = (pairs + kMT - 1) / kMT + std::min(E, pairs);
  const int rows_per_tile = mode == 0 ? kMW * 32 : kMW * 16 * down_nsub(rows);
  return max_mtiles * (rows / rows_per_tile);
}

void launch_mfma_gateup(const MfmaArgs& a, int max_tiles, hipStream_t stream) {
  if (max_tiles > 0)
    hipLaunchKernelGGL((mfma_expert_kernel<0, 4>), dim3(max_tiles), dim3(kMW * kWave), 0, stream, a);
}

void launch_mfma_down(const MfmaArgs& a, int max_tiles, hipStream_t stream) {
  if (max_tiles <= 0) return;
  if (down_nsub(a.H) == 4)
    hipLaunchKernelGGL((mfma_expert_kernel<1, 4>), dim3(max_tiles), dim3(kMW * kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((mfma_expert_kernel<1, 2>), dim3(max_tiles), dim3(kMW * kWave), 0, stream, a);
}

}  // namespace moe
