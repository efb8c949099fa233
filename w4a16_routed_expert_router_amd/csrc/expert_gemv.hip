// Expert FFN of routed (and shared) experts from packed INT4 weights, GEMV form,
// plus the rank-ordered combine and the stack's RMSNorm.
//
// The experts run straight from compact INT4 codes with FP16 group scales and
// FP16 activations; weights are never expanded in HBM ("Horizon RunMap",
// "Architecture invariants" and "What is implemented").
//
// Work split: one wave per (active expert, tile of rows).  A tile is 4 x 1 KiB
// of codes per matrix: each lane issues 4 coalesced 16-byte loads per matrix
// (64 lanes x 16 B = 1 KiB contiguous per load instruction), keeps the decoded
// FP16 pairs in registers, and reuses them for every token routed to the
// expert.  Each 16-byte chunk is 32 consecutive K of one row, so it lies in one
// 128-wide scale group.  A row of K elements spans K/32 lanes (CPR); partial
// sums are scaled per lane and reduced across those lanes with shuffles.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kLoads = 4;          // 16-byte loads per lane per matrix
constexpr int kWavesPerBlock = 4;  // independent waves per 256-thread block

__device__ __forceinline__ void decode_chunk(const uint4 q, h2 out[16]) {
  dequant8(q.x, out + 0);
  dequant8(q.y, out + 4);
  dequant8(q.z, out + 8);
  dequant8(q.w, out + 12);
}

__device__ __forceinline__ void load_act_chunk(const uint16_t* p, h2 out[16]) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = q[i];
    out[4 * i + 0] = as_h2(v.x);
    out[4 * i + 1] = as_h2(v.y);
    out[4 * i + 2] = as_h2(v.z);
    out[4 * i + 3] = as_h2(v.w);
  }
}

__device__ __forceinline__ float dot32(const h2 w[16], const h2 x[16]) {
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc = dot2(w[j], x[j], acc);
  return acc;
}

__device__ __forceinline__ bool resolve(const ExpertArgs& a, int ai, const uint8_t*& blob,
                                        int& cnt, int& off) {
  if (a.fixed_blob) {
    if (ai > 0) return false;
    blob = a.fixed_blob;
    cnt = a.fixed_count;
    off = a.fixed_offset;
    return true;
  }
  if (ai >= *a.n_active) return false;
  const ActiveExpert ae = a.active[ai];
  if (ae.count >= a.mfma_min) return false;  // handled by the MFMA kernels
  blob = a.blobs + (int64_t)ae.slot * a.blob_stride;
  cnt = ae.count;
  off = ae.offset;
  return true;
}

// gate/up + SwiGLU: h[pos, n] = silu(x.Wg[n]) * (x.Wu[n]); K = H, CPR = H/32.
template <int CPR>
__global__ __launch_bounds__(256) void gateup_gemv_kernel(ExpertArgs a) {
  constexpr int RPL = kWave / CPR;  // rows per load
  constexpr int RT = kLoads * RPL;  // rows per wave tile
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int tiles = a.I / RT;
  const int ai = wave / tiles;
  const int tile = wave - ai * tiles;
  const uint8_t* blob;
  int cnt, off;
  if (!resolve(a, ai, blob, cnt, off)) return;
  const int H = a.H;
  const int kc = lane % CPR;
  const int rsub = lane / CPR;
  const int row0 = tile * RT;
  const int row_bytes = H / 2;
  const uint8_t* gc = blob + a.lay.codes(0);
  const uint8_t* uc = blob + a.lay.codes(1);
  const uint16_t* gs = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(0));
  const uint16_t* us = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(1));
  const int ngroups = H / kGroup;

  uint4 gq[kLoads], uq[kLoads];
  float gsc[kLoads], usc[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = row0 + i * RPL + rsub;
    gq[i] = *reinterpret_cast<const uint4*>(gc + code_offset(r, kc * 16, row_bytes));
    uq[i] = *reinterpret_cast<const uint4*>(uc + code_offset(r, kc * 16, row_bytes));
    gsc[i] = half_bits_to_float(gs[(int64_t)r * ngroups + (kc >> 2)]);
    usc[i] = half_bits_to_float(us[(int64_t)r * ngroups + (kc >> 2)]);
  }
  h2 gw[kLoads][16], uw[kLoads][16];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    decode_chunk(gq[i], gw[i]);
    decode_chunk(uq[i], uw[i]);
  }
  for (int it = 0; it < cnt; ++it) {
    const int pos = off + it;
    const int t = a.fixed_blob ? it : a.perm_tok[pos];
    h2 xv[16];
    load_act_chunk(a.x + (int64_t)t * H + kc * 32, xv);
    float g[kLoads], u[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      g[i] = dot32(gw[i], xv) * gsc[i];
      u[i] = dot32(uw[i], xv) * usc[i];
    }
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      g[i] = wave_sum_xor(g[i], CPR);
      u[i] = wave_sum_xor(u[i], CPR);
    }
    if (kc == 0) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int r = row0 + i * RPL + rsub;
        const float hv = swiglu(g[i], u[i]);
        reinterpret_cast<_Float16*>(a.hbuf)[(int64_t)pos * a.I + r] = (_Float16)hv;
      }
    }
  }
}

// down: y[pos, n] = h[pos] . Wd[n]; K = I, CPR = I/32.
template <int CPR>
__global__ __launch_bounds__(256) void down_gemv_kernel(ExpertArgs a) {
  constexpr int RPL = kWave / CPR;
  constexpr int RT = kLoads * RPL;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int tiles = a.H / RT;
  const int ai = wave / tiles;
  const int tile = wave - ai * tiles;
  const uint8_t* blob;
  int cnt, off;
  if (!resolve(a, ai, blob, cnt, off)) return;
  const int I = a.I;
  const int kc = lane % CPR;
  const int rsub = lane / CPR;
  const int row0 = tile * RT;
  const int row_bytes = I / 2;
  const uint8_t* dc = blob + a.lay.codes(2);
  const uint16_t* ds = reinterpret_cast<const uint16_t*>(blob + a.lay.scales(2));
  const int ngroups = I / kGroup;

  uint4 dq[kLoads];
  float dsc[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = row0 + i * RPL + rsub;
    dq[i] = *reinterpret_cast<const uint4*>(dc + code_offset(r, kc * 16, row_bytes));
    dsc[i] = half_bits_to_float(ds[(int64_t)r * ngroups + (kc >> 2)]);
  }
  h2 dw[kLoads][16];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) decode_chunk(dq[i], dw[i]);
  for (int it = 0; it < cnt; ++it) {
    const int pos = off + it;
    h2 hv[16];
    load_act_chunk(a.hbuf + (int64_t)pos * I + kc * 32, hv);
    float y[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) y[i] = wave_sum_xor(dot32(dw[i], hv) * dsc[i], CPR);
    if (kc == 0) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int r = row0 + i * RPL + rsub;
        a.ybuf[(int64_t)pos * a.H + r] = y[i];
      }
    }
  }
}

#define MOE_DISPATCH_CPR(cpr, KERNEL, grid, stream, args)                          \
  switch (cpr) {                                                                   \
    case 8: hipLaunchKernelGGL(KERNEL<8>, grid, dim3(256), 0, stream, args); break;   \
    case 16: hipLaunchKernelGGL(KERNEL<16>, grid, dim3(256), 0, stream, args); break; \
    case 32: hipLaunchKernelGGL(KERNEL<32>, grid, dim3(256), 0, stream, args); break; \
    case 64: hipLaunchKernelGGL(KERNEL<64>, grid, dim3(256), 0, stream, args); break; \
    default: break;                                                                \
  }

static int work_items(const ExpertArgs& a, int rows, int cpr) {
  const int rt = kLoads * (kWave / cpr);
  const int n_exp = a.fixed_blob ? 1 : a.max_active;
  return n_exp * (rows / rt);
}

void launch_gateup_gemv(const ExpertArgs& a, hipStream_t stream) {
  const int cpr = a.H / 32;
  const int waves = work_items(a, a.I, cpr);
  dim3 grid((waves + kWavesPerBlock - 1) / kWavesPerBlock);
  MOE_DISPATCH_CPR(cpr, gateup_gemv_kernel, grid, stream, a);
}

void launch_down_gemv(const ExpertArgs& a, hipStream_t stream) {
  const int cpr = a.I / 32;
  const int waves = work_items(a, a.H, cpr);
  dim3 grid((waves + kWavesPerBlock - 1) / kWavesPerBlock);
  MOE_DISPATCH_CPR(cpr, down_gemv_kernel, grid, stream, a);
}

// out[t] = sum_j w[t,j] * y[pos_of[t,j]] (+ yshared[t]), summed in rank order
// in FP32.  grid (ceil(H/1024), T), block 256, 4 columns per thread.  Stack
// mode (resid): resid[t] += that, and with ssq each block also writes the sum
// of squares of its 1024 updated columns (for the next layer's RMSNorm).
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * 4;
  float ss = 0.0f;  // this thread's part of the new residual's sum of squares
  if (n < a.H) {    // H is a multiple of 256: a wave is wholly in or out
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < a.k; ++j) {
      const int p = a.pos_of[(int64_t)t * a.k + j];
      const float wj = a.w[(int64_t)t * a.k + j];
      const float4 y = *reinterpret_cast<const float4*>(a.ybuf + (int64_t)p * a.H + n);
      acc.x += wj * y.x;
      acc.y += wj * y.y;
      acc.z += wj * y.z;
      acc.w += wj * y.w;
    }
    if (a.yshared) {
      const float4 y = *reinterpret_cast<const float4*>(a.yshared + (int64_t)t * a.H + n);
      acc.x += y.x;
      acc.y += y.y;
      acc.z += y.z;
      acc.w += y.w;
    }
    if (a.resid) {
      float4* r = reinterpret_cast<float4*>(a.resid + (int64_t)t * a.H + n);
      float4 v = *r;
      v.x += acc.x;
      v.y += acc.y;
      v.z += acc.z;
      v.w += acc.w;
      *r = v;
      ss = ((v.x * v.x + v.y * v.y) + v.z * v.z) + v.w * v.w;
    } else {
      _Float16* o = reinterpret_cast<_Float16*>(a.out) + (int64_t)t * a.H + n;
      o[0] = (_Float16)acc.x;
      o[1] = (_Float16)acc.y;
      o[2] = (_Float16)acc.z;
      o[3] = (_Float16)acc.w;
    }
  }
  if (a.ssq) {  // uniform
    __shared__ float part[4];
    ss = wave_sum_xor(ss, kWave);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) a.ssq[(int64_t)t * gridDim.x + blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
  }
}

void launch_combine(const CombineArgs& a, hipStream_t stream) {
  dim3 grid((a.H + 1023) / 1024, a.T);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, a);
}

// x[t] = fp16(h[t] / sqrt(mean(h[t]^2) + eps)); grid T, block 256, H <= 2048.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ h, int H, float eps,
                                                      uint16_t* __restrict__ x) {
  constexpr int kPer = 8;  // H <= 2048: at most 8 values per thread, held in registers
  __shared__ float part[4];
  const int t = blockIdx.x;
  const float* row = h + (int64_t)t * H;
  float v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) v[j] = threadIdx.x + 256 * j < H ? row[threadIdx.x + 256 * j] : 0.0f;
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (threadIdx.x + 256 * j < H) ss += v[j] * v[j];
  ss = wave_sum_xor(ss, kWave);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  _Float16* xo = reinterpret_cast<_Float16*>(x) + (int64_t)t * H;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (threadIdx.x + 256 * j < H) xo[threadIdx.x + 256 * j] = (_Float16)(v[j] * r);
}

void launch_rmsnorm(const float* h, int T, int H, float eps, uint16_t* x, hipStream_t stream) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(256), 0, stream, h, H, eps, x);
}

// Publication of slot-pool changes in stream order.
__global__ void publish_kernel(PublishArgs a) {
  const int i = threadIdx.x;
  if (i < a.n) a.map[a.u[i].expert] = a.u[i].slot;
}

void launch_publish(const PublishArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(publish_kernel, dim3(1), dim3(kMaxPublish), 0, stream, a);
}

}  // namespace moe
