// Device-side helpers shared by the HIP kernels of the W4A16 MoE library.
// gfx950 only: 64-lane wavefronts, v_dot2_f32_f16, packed FP16 arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kGroup = 128;  // INT4 quantisation group along K

// Below this S = sum |x_i w_i| an FP64 sum of FP16 products x_i w_i is exact:
// every FP16 value is an integer multiple of 2^-24, so every product and every
// partial sum is one of 2^-48, and a partial sum (at most S in magnitude)
// below 2^5 = 2^53 * 2^-48 is representable in FP64, so no addition rounds.
// Had the exact S reached 2^5, a computed S (relative error below 2^-16)
// would exceed 2^5 (1 - 2^-16), so the computed S is tested against 31.
constexpr double kExactSumBound = 31.0;

// Device error word bits (see moe_check_device_errors).
constexpr uint32_t kErrBadId = 1u;
constexpr uint32_t kErrDupId = 2u;
constexpr uint32_t kErrNotResident = 4u;
constexpr uint32_t kErrBarrier = 8u;

// One active expert of a call, produced by the grouping kernel.
struct ActiveExpert {
  int32_t expert;  // routed expert id
  int32_t slot;    // index of its blob in the layer's expert storage
  int32_t count;   // tokens routed to it
  int32_t offset;  // first position of its tokens in the sorted order
};

// Byte offsets of the parts of one expert blob in HBM (device layout):
//   [gate codes I*H/2][up codes I*H/2][down codes H*I/2]
//   [gate scales I*H/128 fp16][up scales][down scales]
// Scales are row-major.  Codes come in blocks of 16 rows; inside a block the
// 64 bytes of scale group g of row n sit at g * 1024 + n * 64, so the 16 rows'
// bytes of one group (what one MFMA B fragment load of a wave takes) are one
// contiguous 1 KiB run, and a row block's groups follow one another.
constexpr int kCodeRowBlock = 16;
constexpr int kCodeGroupBytes = kGroup / 2;                            // 64
constexpr int kCodeGroupStride = kCodeRowBlock * kCodeGroupBytes;      // 1024
// Offset of byte `b` of row `row`'s codes in a matrix with `row_bytes` (= K/2)
// code bytes per row.
__host__ __device__ __forceinline__ int64_t code_offset(int row, int b, int row_bytes) {
  return (int64_t)(row / kCodeRowBlock) * kCodeRowBlock * row_bytes + (b / kCodeGroupBytes) * kCodeGroupStride +
         (row % kCodeRowBlock) * kCodeGroupBytes + (b % kCodeGroupBytes);
}
struct BlobLayout {
  int64_t code_bytes;   // one matrix
  int64_t scale_bytes;  // one matrix
  __host__ __device__ int64_t codes(int m) const { return m * code_bytes; }
  __host__ __device__ int64_t scales(int m) const { return 3 * code_bytes + m * scale_bytes; }
  __host__ __device__ int64_t total() const { return 3 * (code_bytes + scale_bytes); }
};

// ---- INT4 -> FP16 --------------------------------------------------------------
// Device code layout: within each 32-bit word holding k0..k7 of a row, nibble
// position p holds k[perm(p)] with positions (0,4,1,5,2,6,3,7) <- (k0..k7), so
// that masking with 0x000F000F / 0x00F000F0 yields the pairs (k0,k1), (k2,k3)
// and after an 8-bit shift (k4,k5), (k6,k7).  OR-ing a nibble into the FP16
// pattern 0x6400 (= 1024, ulp 1) gives 1024 + q exactly; a nibble in bits 4..7
// gives 1024 + 16q.  Both are turned into q - 8 exactly.
__device__ __forceinline__ void dequant8(uint32_t d, h2 out[4]) {
  const uint32_t d8 = d >> 8;
  const h2 lo0 = __builtin_bit_cast(h2, (d & 0x000F000Fu) | 0x64006400u);
  const h2 hi0 = __builtin_bit_cast(h2, (d & 0x00F000F0u) | 0x64006400u);
  const h2 lo1 = __builtin_bit_cast(h2, (d8 & 0x000F000Fu) | 0x64006400u);
  const h2 hi1 = __builtin_bit_cast(h2, (d8 & 0x00F000F0u) | 0x64006400u);
  const h2 k1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const h2 k16th = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 km72 = {(_Float16)-72.0f, (_Float16)-72.0f};
  out[0] = lo0 - k1032;
  out[1] = hi0 * k16th + km72;
  out[2] = lo1 - k1032;
  out[3] = hi1 * k16th + km72;
}

// Load through a pointer that addresses global memory.  A pointer read from
// memory (rather than passed as a kernel argument) is generic to the compiler,
// which then emits flat loads; those also count against the LDS wait counter,
// so every later LDS access would wait for them.  This keeps them global loads.
template <class T>
__device__ __forceinline__ T ldg(const void* p) {
  return *(const __attribute__((address_space(1))) T*)(uintptr_t)p;
}
__device__ __forceinline__ uint4 ldg_u4(const void* p) {
  typedef uint32_t v4 __attribute__((ext_vector_type(4)));
  const v4 v = ldg<v4>(p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// (a & m) | o in one VALU instruction.  gfx9 VOP3 takes one scalar operand,
// so the mask comes in a VGPR (callers keep it in one across their loop).
__device__ __forceinline__ uint32_t and_or_b32(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "s"(o));
  return r;
}

// dequant8 with the masks held in VGPRs (mlo = 0x000F000F, mhi = 0x00F000F0):
// five instructions form the four FP16 pairs, four more turn them into q - 8.
__device__ __forceinline__ void dequant8_v(uint32_t d, h2 out[4], uint32_t mlo, uint32_t mhi) {
  const uint32_t d8 = d >> 8;
  const h2 lo0 = __builtin_bit_cast(h2, and_or_b32(d, mlo, 0x64006400u));
  const h2 hi0 = __builtin_bit_cast(h2, and_or_b32(d, mhi, 0x64006400u));
  const h2 lo1 = __builtin_bit_cast(h2, and_or_b32(d8, mlo, 0x64006400u));
  const h2 hi1 = __builtin_bit_cast(h2, and_or_b32(d8, mhi, 0x64006400u));
  const h2 k1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
  const h2 k16th = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 km72 = {(_Float16)-72.0f, (_Float16)-72.0f};
  out[0] = lo0 - k1032;
  out[1] = hi0 * k16th + km72;
  out[2] = lo1 - k1032;
  out[3] = hi1 * k16th + km72;
}

// SwiGLU of one gate/up pair: silu(g) * u = g * u / (1 + e^-g), with the
// hardware base-2 exponential and reciprocal (about one ulp each, far below
// the FP16 rounding of the result).  Large negative g gives e^-g = inf and a
// zero result, as the limit has it.
__device__ __forceinline__ float swiglu(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ float dot2(h2 a, h2 b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// ---- wave reductions -------------------------------------------------------------
__device__ __forceinline__ float wave_sum_xor(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Direct global -> LDS loads (gfx950 LDS DMA): lane l's `bytes` land at the
// wave-uniform LDS address `lds` + l * bytes.  Written as inline assembly so
// that the compiler neither stalls on them when it reuses their address
// registers nor waits for them before unrelated loads; they still count in
// vmcnt, and the LDS data is read only after an explicit vmcnt(0).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma_lds16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}
__device__ __forceinline__ void dma_lds4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}

// Wave reductions on the DPP network (no LDS round trips): inclusive sums
// within each row of 16 lanes, then row broadcasts, leave the total in lane 63,
// which is broadcast to every lane.  The order of the additions is fixed, so
// every lane -- and every wave given the same inputs -- gets the same bits.
template <int CTRL, int RM>
__device__ __forceinline__ uint32_t dpp32(uint32_t v, uint32_t ident) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)v, CTRL, RM, 0xf, false);
}
template <int CTRL, int RM>
__device__ __forceinline__ float dppf(float v, float ident) {
  return __builtin_bit_cast(float, dpp32<CTRL, RM>(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, ident)));
}
template <int CTRL, int RM>
__device__ __forceinline__ double dppd(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = dpp32<CTRL, RM>((uint32_t)u, 0u);
  const uint32_t hi = dpp32<CTRL, RM>((uint32_t)(u >> 32), 0u);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float bcast63(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dppf<0x111, 0xf>(x, 0.0f);  // row_shr:1
  x += dppf<0x112, 0xf>(x, 0.0f);  // row_shr:2
  x += dppf<0x114, 0xf>(x, 0.0f);  // row_shr:4
  x += dppf<0x118, 0xf>(x, 0.0f);  // row_shr:8
  x += dppf<0x142, 0xa>(x, 0.0f);  // row_bcast:15
  x += dppf<0x143, 0xc>(x, 0.0f);  // row_bcast:31
  return bcast63(x);
}
__device__ __forceinline__ double wave_sum(double x) {
  x += dppd<0x111, 0xf>(x);
  x += dppd<0x112, 0xf>(x);
  x += dppd<0x114, 0xf>(x);
  x += dppd<0x118, 0xf>(x);
  x += dppd<0x142, 0xa>(x);
  x += dppd<0x143, 0xc>(x);
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dppf<0x111, 0xf>(x, -INFINITY));
  x = fmaxf(x, dppf<0x112, 0xf>(x, -INFINITY));
  x = fmaxf(x, dppf<0x114, 0xf>(x, -INFINITY));
  x = fmaxf(x, dppf<0x118, 0xf>(x, -INFINITY));
  x = fmaxf(x, dppf<0x142, 0xa>(x, -INFINITY));
  x = fmaxf(x, dppf<0x143, 0xc>(x, -INFINITY));
  return bcast63(x);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp32<0x111, 0xf>(x, 0u));
  x = max(x, dpp32<0x112, 0xf>(x, 0u));
  x = max(x, dpp32<0x114, 0xf>(x, 0u));
  x = max(x, dpp32<0x118, 0xf>(x, 0u));
  x = max(x, dpp32<0x142, 0xa>(x, 0u));
  x = max(x, dpp32<0x143, 0xc>(x, 0u));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
// Largest 64-bit key of the wave: the largest high half, then the largest
// low half among the lanes holding that high half.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  const uint32_t hi = (uint32_t)(x >> 32);
  const uint32_t hm = wave_max_u32(hi);
  const uint32_t lm = wave_max_u32(hi == hm ? (uint32_t)x : 0u);
  return ((uint64_t)hm << 32) | lm;
}

// Inclusive prefix sum over the lanes of a wave, on the same DPP network.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += (int)dpp32<0x111, 0xf>((uint32_t)x, 0u);
  x += (int)dpp32<0x112, 0xf>((uint32_t)x, 0u);
  x += (int)dpp32<0x114, 0xf>((uint32_t)x, 0u);
  x += (int)dpp32<0x118, 0xf>((uint32_t)x, 0u);
  x += (int)dpp32<0x142, 0xa>((uint32_t)x, 0u);
  x += (int)dpp32<0x143, 0xc>((uint32_t)x, 0u);
  return x;
}

__device__ __forceinline__ void atomic_or_err(uint32_t* err, uint32_t bits) {
  if (err) atomicOr(err, bits);
}

constexpr int kMaxTopK = 16;  // largest top-k a context accepts

// Validates the k ids of token t: an id out of range or repeated within the
// token flags the call (errbits) and the token gets ids 0..k-1 (valid and
// distinct) instead.
__device__ __forceinline__ void validate_token(const int (&rv)[kMaxTopK], int k, int E, int (&out)[kMaxTopK],
                                               uint32_t& errbits) {
  bool bad = false, dup = false;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      bad |= rv[j] < 0 || rv[j] >= E;
#pragma unroll
      for (int jj = 0; jj < j; ++jj) dup |= rv[jj] == rv[j];
    }
  }
  if (bad) errbits |= kErrBadId;
  if (dup) errbits |= kErrDupId;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) out[j] = (bad || dup) ? j : rv[j];
}

}  // namespace moe
