// Grouping of a call's (token, rank) pairs by expert.
//
// The pages execute each token's routed expert group ("Horizon RunMap",
// "Partial-residency contract": a request acquires its routed expert group)
// and name a grouped executor ("Grouped T3").  Here the T*k pairs are sorted
// stably by (expert, token): expert e's tokens occupy positions
// [offset_e, offset_e + count_e) in ascending token order, so every expert's
// weights are streamed once per call and the work layout depends only on ids.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kGroupThreads = 1024;
constexpr int kMaxExperts = 1024;
constexpr int kChunk = 64;  // tokens per stable-placement round

__device__ int block_exclusive_scan(int v, int* sh_warp, int* total) {
  // 1024 threads = 16 waves
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) sh_warp[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    int s = (lane < kGroupThreads / 64) ? sh_warp[lane] : 0;
    int si = s;
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(si, o, 64);
      if (lane >= o) si += n;
    }
    if (lane < kGroupThreads / 64) sh_warp[lane] = si - s;
    if (lane == kGroupThreads / 64 - 1) *total = si;
  }
  __syncthreads();
  const int r = sh_warp[wid] + incl - v;
  __syncthreads();
  return r;
}

// One block of 1024 threads.
__global__ __launch_bounds__(kGroupThreads) void group_kernel(GroupArgs a) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ unsigned long long mask[kMaxExperts];
  __shared__ int sh_warp[16];
  __shared__ int sh_total;
  const int tid = threadIdx.x;
  const int T = a.T, k = a.k, E = a.E;
  const int P = T * k;

  for (int e = tid; e < E; e += kGroupThreads) cnt[e] = 0;
  // validate each token's ids; a bad token gets ids 0..k-1 (valid, distinct)
  uint32_t errbits = 0;
  for (int t = tid; t < T; t += kGroupThreads) {
    const int32_t* row = a.ids_in + (int64_t)t * k;
    bool bad = false, dup = false;
    for (int j = 0; j < k; ++j) {
      const int e = row[j];
      if (e < 0 || e >= E) bad = true;
      for (int jj = 0; jj < j; ++jj)
        if (row[jj] == e) dup = true;
    }
    if (bad) errbits |= kErrBadId;
    if (dup) errbits |= kErrDupId;
    for (int j = 0; j < k; ++j) a.ids_s[(int64_t)t * k + j] = (bad || dup) ? j : row[j];
  }
  if (errbits) atomic_or_err(a.err, errbits);
  __syncthreads();
  for (int p = tid; p < P; p += kGroupThreads) atomicAdd(&cnt[a.ids_s[p]], 1);
  __syncthreads();

  // offsets and the active list (ascending expert id); E <= 1024 = one per thread
  const int c = (tid < E) ? cnt[tid] : 0;
  const int off = block_exclusive_scan(c, sh_warp, &sh_total);
  const int mtiles = c >= a.mfma_min ? (c + kMfmaTileTokens - 1) / kMfmaTileTokens : 0;
  const int moff = block_exclusive_scan(mtiles, sh_warp, &sh_total);
  const int mtotal = sh_total;
  const int act = block_exclusive_scan(c > 0 ? 1 : 0, sh_warp, &sh_total);
  if (c > 0) a.mtile_off[act] = moff;
  if (tid == 0) a.mtile_off[sh_total] = mtotal;
  if (tid < E) {
    base[tid] = off;
    if (c > 0) {
      int slot = a.slot_map ? a.slot_map[tid] : tid;
      if (slot < 0) {
        atomic_or_err(a.err, kErrNotResident);
        slot = 0;
      }
      a.active[act] = ActiveExpert{tid, slot, c, off};
    }
  }
  if (tid == 0) *a.n_active = sh_total;
  __syncthreads();

  // stable placement: within an expert, positions follow token order
  for (int t0 = 0; t0 < T; t0 += kChunk) {
    for (int e = tid; e < E; e += kGroupThreads) mask[e] = 0ull;
    __syncthreads();
    const int nt = min(kChunk, T - t0);
    const int np = nt * k;
    int e = -1, tl = 0, p = 0;
    if (tid < np) {
      p = t0 * k + tid;
      tl = tid / k;
      e = a.ids_s[p];
      atomicOr(&mask[e], 1ull << tl);
    }
    __syncthreads();
    if (e >= 0) {
      const int pos = base[e] + __popcll(mask[e] & ((1ull << tl) - 1ull));
      a.perm_tok[pos] = t0 + tl;
      a.pos_of[p] = pos;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kGroupThreads) base[ee] += __popcll(mask[ee]);
    __syncthreads();
  }
}

void launch_group(const GroupArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(group_kernel, dim3(1), dim3(kGroupThreads), 0, stream, a);
}

}  // namespace moe
