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
constexpr int kLdsPairs = 16384;  // validated ids are kept in LDS up to this many pairs
constexpr int kRounds = 4;        // placement chunks per round at most

// Exclusive prefix sums of N values per thread over the block (1024 threads =
// 16 waves) and their block totals; three barriers for all N.
template <int N>
__device__ void block_exclusive_scan(const int (&v)[N], int (&excl)[N], int (&total)[N], int (*sh_warp)[16],
                                     int* sh_tot) {
  constexpr int NW = kGroupThreads / 64;
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int incl[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    incl[i] = wave_incl_scan(v[i]);
    if (lane == 63) sh_warp[i][wid] = incl[i];
  }
  __syncthreads();
  if (wid == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int s = lane < NW ? sh_warp[i][lane] : 0;
      const int si = wave_incl_scan(s);
      if (lane < NW) sh_warp[i][lane] = si - s;
      if (lane == NW - 1) sh_tot[i] = si;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    excl[i] = sh_warp[i][wid] + incl[i] - v[i];
    total[i] = sh_tot[i];
  }
  __syncthreads();
}

// The call's plan from the per-expert token counts (c of thread e < E):
// positions of each expert's first pair (ascending expert id), the active
// list, the MFMA token-tile offsets and the few-token kernel's list.  Every
// thread of the block calls it (barriers inside); base[e] is set on return.
struct ListPlan {
  int c, slot, off, moff, mtotal, act, nact, sidx, nsmall, nchunk;
};
__device__ ListPlan plan_lists(const GroupArgs& a, int c, int slot_pre, int* base, int (*sh_warp)[16], int* sh_tot) {
  const int tid = threadIdx.x, E = a.E;
  ListPlan L;
  L.c = c;
  const int mtiles = c >= a.mfma_min ? (c + kMfmaTileTokens - 1) / kMfmaTileTokens : 0;
  // entries of the few-token kernel's list: one for an expert with at most
  // kStreamTokens tokens below the MFMA threshold, or (chunk_all) one per
  // chunk of kStreamTokens tokens of every active expert
  L.nchunk = a.chunk_all ? (c + kStreamTokens - 1) / kStreamTokens
                         : (c > 0 && c <= kStreamTokens && c < a.mfma_min ? 1 : 0);
  const int sv[4] = {c, mtiles, c > 0 ? 1 : 0, L.nchunk};
  int sx[4], st[4];
  block_exclusive_scan<4>(sv, sx, st, sh_warp, sh_tot);
  L.off = sx[0];
  L.moff = sx[1];
  L.mtotal = st[1];
  L.act = sx[2];
  L.nact = st[2];
  L.sidx = sx[3];
  L.nsmall = st[3];
  L.slot = 0;
  if (tid < E) {
    base[tid] = L.off;
    if (c > 0) {
      L.slot = slot_pre;
      if (L.slot < 0) {
        atomic_or_err(a.err, kErrNotResident);
        L.slot = 0;
      }
    }
  }
  return L;
}

// The plan's global lists (thread e writes expert e's entries).
__device__ void store_lists(const GroupArgs& a, const ListPlan& L) {
  const int tid = threadIdx.x;
  if (L.c > 0) {
    a.mtile_off[L.act] = L.moff;
    a.active[L.act] = ActiveExpert{tid, L.slot, L.c, L.off};
  }
  for (int i = 0; i < L.nchunk; ++i)
    a.small[L.sidx + i] =
        ActiveExpert{tid, L.slot, min(kStreamTokens, L.c - i * kStreamTokens), L.off + i * kStreamTokens};
  if (tid == 0) {
    a.mtile_off[L.nact] = L.mtotal;
    *a.n_active = L.nact;
    *a.n_small = L.nsmall;
  }
}

// One pass over the pairs, for calls whose (64-token chunk, expert) bit masks
// and validated ids fit in LDS.  Each thread validates whole tokens as their
// ids arrive and sets the token's bit in the mask of each of its experts; an
// expert's count and its pairs in earlier chunks then come from one walk over
// its masks, and a pair's position is its expert's base + the expert's pairs
// in earlier chunks + the expert's earlier tokens in the pair's own chunk.
constexpr int kOnePassMaskWords = 4096;
__global__ __launch_bounds__(kGroupThreads) void group_onepass_kernel(GroupArgs a) {
  __shared__ unsigned long long mask[kOnePassMaskWords];  // [chunk][expert]
  __shared__ int cum[kOnePassMaskWords];                  // [chunk][expert]: pairs in earlier chunks
  __shared__ int base[kMaxExperts];
  __shared__ int sh_warp[4][16];
  __shared__ int sh_tot[4];
  __shared__ int16_t sid[kLdsPairs];  // validated ids by pair
  const int tid = threadIdx.x;
  const int T = a.T, k = a.k, E = a.E;
  const int P = T * k, NC = (T + kChunk - 1) / kChunk;
  // the slot map is loaded first: its latency overlaps everything up to the lists
  const int slot_pre = tid < E && a.slot_map ? a.slot_map[tid] : tid;
  for (int i = tid; i < NC * E; i += kGroupThreads) mask[i] = 0ull;
  __syncthreads();
  uint32_t errbits = 0;
  for (int t = tid; t < T; t += kGroupThreads) {
    int rv[kMaxTopK], v[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) rv[j] = j < k ? a.ids_in[(int64_t)t * k + j] : -1;
    validate_token(rv, k, E, v, errbits);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= k) break;
      sid[t * k + j] = (int16_t)v[j];
      atomicOr(&mask[(t / kChunk) * E + v[j]], 1ull << (t % kChunk));
    }
  }
  if (errbits) atomic_or_err(a.err, errbits);
  __syncthreads();
  int c = 0;
  if (tid < E)
    for (int ch = 0; ch < NC; ++ch) {
      cum[ch * E + tid] = c;
      c += __popcll(mask[ch * E + tid]);
    }
  const ListPlan L = plan_lists(a, c, slot_pre, base, sh_warp, sh_tot);
  __syncthreads();
  for (int p = tid; p < P; p += kGroupThreads) {
    const int t = p / k, e = sid[p];
    const int ch = t / kChunk, tl = t % kChunk;
    const int pos = base[e] + cum[ch * E + e] + __popcll(mask[ch * E + e] & ((1ull << tl) - 1ull));
    a.perm_tok[pos] = t;
    a.pos_of[p] = pos;
  }
  store_lists(a, L);
}

// General form (any T and E): ids stay in LDS up to kLdsPairs pairs, else in
// the global scratch, and the placement runs in rounds of chunks.
// One block of 1024 threads.
__global__ __launch_bounds__(kGroupThreads) void group_kernel(GroupArgs a) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ unsigned long long mask[kRounds][kMaxExperts];
  __shared__ int sh_warp[4][16];
  __shared__ int sh_tot[4];
  __shared__ int16_t sid[kLdsPairs];    // ids by pair (validated in place)
  __shared__ int16_t sperm[kLdsPairs];  // token at each sorted position
  __shared__ int16_t spos[kLdsPairs];   // sorted position of each pair
  const int tid = threadIdx.x;
  const int T = a.T, k = a.k, E = a.E;
  const int P = T * k;
  // Ids, positions and the permutation live in LDS when they fit (else in
  // their global buffers), and every global store is issued at the end: a
  // barrier waits for the block's outstanding stores, so stores issued
  // between the placement rounds would stall each round.
  const bool lds_ids = P <= kLdsPairs;
  auto get_id = [&](int p) -> int { return lds_ids ? (int)sid[p] : a.ids_s[p]; };

  for (int e = tid; e < E; e += kGroupThreads) cnt[e] = 0;
  // the caller's ids, read coalesced (out-of-range values are clamped into
  // int16 so that they stay out of range)
  if (lds_ids) {
    for (int p = tid; p < P; p += kGroupThreads) {
      const int v = a.ids_in[p];
      sid[p] = (int16_t)(v < 0 || v >= E ? -1 : v);
    }
    __syncthreads();
  }
  // validate each token's ids; a bad token gets ids 0..k-1 (valid, distinct)
  uint32_t errbits = 0;
  for (int t = tid; t < T; t += kGroupThreads) {
    int rv[kMaxTopK], v[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      rv[j] = j < k ? (lds_ids ? (int)sid[t * k + j] : a.ids_in[(int64_t)t * k + j]) : -1;
    validate_token(rv, k, E, v, errbits);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= k) break;
      if (lds_ids)
        sid[t * k + j] = (int16_t)v[j];
      else
        a.ids_s[(int64_t)t * k + j] = v[j];
    }
  }
  if (errbits) atomic_or_err(a.err, errbits);
  __syncthreads();
  for (int p = tid; p < P; p += kGroupThreads) atomicAdd(&cnt[get_id(p)], 1);
  __syncthreads();

  // offsets and the active list (ascending expert id); E <= 1024 = one per thread
  const int c = (tid < E) ? cnt[tid] : 0;
  const ListPlan L = plan_lists(a, c, tid < E && a.slot_map ? a.slot_map[tid] : tid, base, sh_warp, sh_tot);
  for (int i = tid; i < kRounds * kMaxExperts; i += kGroupThreads) (&mask[0][0])[i] = 0ull;
  __syncthreads();

  // stable placement: within an expert, positions follow token order.  One
  // round places R consecutive chunks of 64 tokens (R * 64 * k <= 1024 pairs):
  // a pair's position is its expert's base, plus the expert's pairs in the
  // round's earlier chunks, plus its earlier tokens within its own chunk.
  const int R = max(1, min(kRounds, kGroupThreads / (kChunk * k)));
  for (int t0 = 0; t0 < T; t0 += R * kChunk) {
    const int np = min(R * kChunk, T - t0) * k;
    int e = -1, tl = 0, ci = 0, p = 0;
    if (tid < np) {
      p = t0 * k + tid;
      const int tr = tid / k;  // token within the round
      ci = tr / kChunk;
      tl = tr - ci * kChunk;
      e = get_id(p);
      atomicOr(&mask[ci][e], 1ull << tl);
    }
    __syncthreads();
    if (e >= 0) {
      int pos = base[e] + __popcll(mask[ci][e] & ((1ull << tl) - 1ull));
      for (int cc = 0; cc < ci; ++cc) pos += __popcll(mask[cc][e]);
      const int t = t0 + ci * kChunk + tl;
      if (lds_ids) {
        sperm[pos] = (int16_t)t;
        spos[p] = (int16_t)pos;
      } else {
        a.perm_tok[pos] = t;
        a.pos_of[p] = pos;
      }
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kGroupThreads) {
      int add = 0;
      for (int cc = 0; cc < R; ++cc) {
        add += __popcll(mask[cc][ee]);
        mask[cc][ee] = 0ull;
      }
      base[ee] += add;
    }
    __syncthreads();
  }

  // global results
  if (lds_ids) {
    for (int p = tid; p < P; p += kGroupThreads) {
      a.perm_tok[p] = sperm[p];
      a.pos_of[p] = spos[p];
    }
  }
  store_lists(a, L);
}

void launch_group(const GroupArgs& a, hipStream_t stream) {
  const int64_t nc = (a.T + kChunk - 1) / kChunk;
  if ((int64_t)a.T * a.k <= kLdsPairs && nc * a.E <= kOnePassMaskWords)
    hipLaunchKernelGGL(group_onepass_kernel, dim3(1), dim3(kGroupThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(kGroupThreads), 0, stream, a);
}

}  // namespace moe
