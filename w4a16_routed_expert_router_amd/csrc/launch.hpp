// Internal launcher interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

struct RouterArgs {
  const uint16_t* x;      // [T,H] fp16
  const uint16_t* wr;     // [E,H] fp16
  int T, E, H, k, renorm;
  float* logits;          // [T,E] fp32 out
  const int32_t* forced;  // [T,k] or null
  int32_t* ids;           // [T,k] out
  float* w;               // [T,k] out
  uint32_t* err;
  int exact_always;
  // stack layers after the first, on the matrix-core router: x is formed in
  // the partial-logit kernel as fp16(RMSNorm(hres)) from the residual's sums
  // of squares ssq ([T][nssq] blocks of it, written by the previous layer's
  // combine) and written to xw (= x); hres null: x is given
  const float* hres;
  const float* ssq;
  int nssq;
  uint16_t* xw;
};
void launch_router_logits(const RouterArgs& a, hipStream_t stream);
// logits + softmax/top-k on the FP64 matrix cores, using `scratch` of
// router_scratch_bytes(); returns false, launching nothing, when the shape or
// the flags do not take that path (then launch_router_logits + _topk)
bool launch_router(const RouterArgs& a, double* scratch, hipStream_t stream);
// whether launch_router takes the matrix-core path for this shape and flag
bool router_takes_mfma(int H, int E, int exact_always);
size_t router_scratch_bytes(int max_tokens, int E, int H);
void launch_router_topk(const RouterArgs& a, hipStream_t stream);

struct GroupArgs {
  const int32_t* ids_in;    // [T,k] caller ids
  int T, k, E;
  const int32_t* slot_map;  // [E] expert -> slot, or null (identity)
  int32_t* ids_s;           // [T,k] validated ids
  ActiveExpert* active;     // [E]
  int32_t* n_active;        // [1]
  int32_t* perm_tok;        // [T*k] token at sorted position
  int32_t* pos_of;          // [T*k] sorted position of pair t*k+j
  uint32_t* err;
  int mfma_min;             // experts with at least this many tokens take the MFMA path
  int32_t* mtile_off;       // [E+1] MFMA token-tile offsets over the active list
  ActiveExpert* small;      // [E + ceil(T*k / kStreamTokens)] the few-token kernel's list: active
                            // experts with at most kStreamTokens tokens (below mfma_min), or with
                            // chunk_all every active expert as chunks of at most kStreamTokens
  int32_t* n_small;         // [1]
  int chunk_all;            // 1: every active expert goes to the few-token list, in chunks
};
void launch_group(const GroupArgs& a, hipStream_t stream);

// Grouped GEMM on MFMA (expert_mfma.hip)
constexpr int kMfmaTileTokens = 128;  // tokens of one expert per MFMA tile
struct MfmaArgs {
  const uint8_t* blobs;
  int64_t blob_stride;
  BlobLayout lay;
  const ActiveExpert* active;
  const int32_t* n_active;
  const int32_t* mtile_off;   // [n_active+1]
  int H, I;
  const uint16_t* x;          // [T,H] (gate/up input)
  const int32_t* perm_tok;    // token at each sorted position
  uint16_t* hbuf;             // [positions, I] fp16
  float* ybuf;                // [positions, H] fp32
};
// Blocks of a grouped-GEMM launch: enough token tiles for any routing of the
// call in which only experts with at least mfma_min tokens take the grouped GEMM.
int mfma_max_tiles(int T, int k, int E, int rows, int mode, int mfma_min);
void launch_mfma_gateup(const MfmaArgs& a, int max_tiles, hipStream_t stream);
void launch_mfma_down(const MfmaArgs& a, int max_tiles, hipStream_t stream);

// Test support (debug.hip): a bounded wait of `microseconds` on `stream`.
void launch_copy_delay(hipStream_t stream, int microseconds);

struct ExpertArgs {
  const uint8_t* blobs;       // expert storage of the layer (slot-indexed)
  int64_t blob_stride;        // bytes per slot
  BlobLayout lay;             // offsets inside one blob (for this expert kind)
  const ActiveExpert* active; // routed mode: active list from the grouping
  const int32_t* n_active;
  int max_active;             // upper bound of *n_active (sizes the grid)
  const uint8_t* fixed_blob;  // shared-expert mode: its blob (then active unused)
  int fixed_count;            // shared-expert mode: tokens (= T)
  int fixed_offset;           // shared-expert mode: first position
  int H, I;
  const uint16_t* x;          // [T,H] fp16 (gate/up input)
  const int32_t* perm_tok;    // token at each sorted position (routed mode)
  uint16_t* hbuf;             // [positions, I] fp16
  float* ybuf;                // [positions, H] fp32
  int mfma_min;               // routed experts with count >= this are skipped (MFMA path)
  const ActiveExpert* small;  // routed experts (or chunks of them) with at most kStreamTokens tokens
  const int32_t* n_small;
  // streaming kernel, routed mode: the shared expert taken as one more list
  // entry after the small experts (null: none); its tokens are 0..T-1 and its
  // rows live in shared_h / shared_y
  const uint8_t* shared_blob;
  int shared_count;
  uint16_t* shared_h;         // [T, I] fp16
  float* shared_y;            // [T, H] fp32
  // streaming gate/up kernel: 1 when every block groups the call's pairs
  // itself from grp (stream_group_in_kernel_ok), block 0 writing the
  // grouping's outputs for the later kernels; small / n_small then come from
  // grp, and no grouping kernel runs
  int group_in_kernel;
  GroupArgs grp;
};
void launch_gateup_gemv(const ExpertArgs& a, hipStream_t stream);
// Persistent weight-streaming expert kernel (expert_stream.hip) for experts with
// at most kStreamTokens tokens (and below mfma_min); mode 0 gate/up, 1 down.
constexpr int kStreamTokens = 32;
// Whether a T-token call whose experts all take the streaming kernels can have
// its pairs grouped inside the gate/up streaming kernel: the ids, bit masks
// and per-expert lists fit in the kernel's LDS and no block's run of items can
// span more list entries than it keeps.
bool stream_group_in_kernel_ok(int T, int k, int E, int I, int grid, bool shared_rides);
// with at least this many (token, expert) pairs per expert on average (a
// prefill) every expert takes the grouped GEMM
constexpr int kPrefillPairsPerExpert = 16;
bool stream_supported(int mode, int K, int rows);
void launch_stream_expert(const ExpertArgs& a, int mode, int grid, hipStream_t stream);
void launch_down_gemv(const ExpertArgs& a, hipStream_t stream);

struct CombineArgs {
  const float* ybuf;          // [P, H] routed outputs by sorted position
  const float* yshared;       // [T, H] shared-expert output or null
  const int32_t* pos_of;      // [T*k]
  const float* w;             // [T*k]
  int T, k, H;
  uint16_t* out;              // [T,H] fp16 (if resid == null)
  float* resid;               // [T,H] fp32: resid += combined (stack mode)
  // stack mode: [T][ceil(H/1024)] sums of squares of the updated residual,
  // one per block of 1024 columns (for the next layer's RMSNorm), or null
  float* ssq;
};
void launch_combine(const CombineArgs& a, hipStream_t stream);

void launch_rmsnorm(const float* h, int T, int H, float eps, uint16_t* x, hipStream_t stream);

// Fused persistent decode path (decode_fused.hip)
constexpr int kFMaxT = 4;      // tokens per call
constexpr int kFMaxP = 64;     // (token, rank) pairs per call
constexpr int kFMaxTE = 4096;  // T * E
constexpr int kFMaxCand = 128; // ceil(E/64) * k
constexpr int kFStageHalves = 32768;  // (T*k + shared T) * I FP16 staged in LDS
constexpr int kFGrid = 256;    // blocks: one per compute unit
constexpr int kFRows = 8;      // residual rows per block (H / kFGrid)
constexpr int kFLogitReps = 8; // logit replicas (one per XCD) for small steps
constexpr int kStampsPerLayer = 16;   // phase timestamps per layer (instrumentation)
constexpr int kStampLayers = 16;      // layers of a call that are stamped
constexpr int kStampStride = kStampLayers * kStampsPerLayer;  // per block
struct FusedLayer {
  const uint16_t* router;
  const uint8_t* store;
  const int32_t* map;
  const uint8_t* shared;
};
struct FusedArgs {
  const FusedLayer* layers;   // device array, indexed by absolute layer
  int l0, l1, T, E, I, k, renorm, has_shared, exact_always;
  int lg_reps;                // logit replicas: kFLogitReps or 1
  int lg_sub;                 // waves sharing one logit item: 1, 2 or 4
  BlobLayout lay;             // routed and shared blobs (shared inter == inter)
  int64_t blob_stride;
  float* h;                   // [T,H] residual, updated in place
  const float* h_in;          // [T,H] the first layer's input residual (null: h)
  uint64_t* xh;               // [2][kFMaxT][H] tagged residual exchange
  uint64_t* xlg;              // [kFLogitReps][kFMaxTE] tagged logits
  uint64_t* xhb;              // [kFStageHalves/2] tagged FP16 pairs of intermediates
  uint64_t* xgate;            // [kFGrid] tagged "residual read" marks
  uint32_t* epoch;            // [kFGrid] per-block epoch counters
  const int32_t* forced;      // [L,T,k] or null
  uint16_t* x_trace;
  int32_t* ids_trace;
  float* w_trace;
  uint32_t* err;
  uint64_t* stamps;           // [grid][kStampStride] phase timestamps or null
  int guess_mode;             // batch-1 path: 0 the router's guess; test hooks 1 the
                              // k lowest guess logits, 2 guess ranks k/2 .. k/2+k-1;
                              // 3 no guess (weights loaded after each selection)
};
bool fused_supported(int H, int I);
void launch_fused_decode(const FusedArgs& a, hipStream_t stream);
// Batch-1 fused decode with the next layer's weights loaded during the
// current layer (decode_spec.hip); resident layers, no forced ids.  Uses
// xlg[rep * kFMaxTE + E ..] for the guess logits.
bool spec_supported(int H, int I, int E, int k, int shared_inter);
void launch_spec_decode(const FusedArgs& a, hipStream_t stream);
// words of each exchange buffer
constexpr int64_t kFXhWords = 2ll * kFMaxT * 2048;
constexpr int64_t kFXlgWords = (int64_t)kFLogitReps * kFMaxTE;
constexpr int64_t kFXhbWords = kFStageHalves / 2;

struct PublishUpdate {
  int32_t expert;
  int32_t slot;  // -1 = evicted
};
constexpr int kMaxPublish = 64;
struct PublishArgs {
  int32_t* map;
  int n;
  PublishUpdate u[kMaxPublish];
};
void launch_publish(const PublishArgs& a, hipStream_t stream);

}  // namespace moe
