// C ABI of the W4A16 routed-expert MoE library: context, weight registration,
// dispatch of the hot path and the expert-slot pool transport.
//
// Expert-slot pool ("Horizon RunMap", "Partial-residency contract: immutable
// authority and miss lifecycle"; "F51 Nitro / Nitro-MoE", "Layer 1 - expert
// persistence cache"):
//   - every expert of a pooled layer lives in pinned host memory that is
//     written once at registration and never again (immutable authority);
//   - a miss copies one contiguous expert blob host -> device on a side stream
//     (H2D only; eviction discards the device copy, nothing is written back);
//   - the side stream first waits for the layer's "retired" event, recorded
//     after the last compute that read the layer's slots, so a victim slot is
//     not overwritten while an earlier kernel may still read it;
//   - the caller's stream waits for the "ready" event of the call's copies and
//     only then runs the small kernel that writes the expert -> slot map in HBM
//     (publication after complete transfer, in stream order);
//   - capacity is fixed at creation; a routed group larger than it fails.
#include <hip/hip_runtime.h>
#include <string.h>

#include <condition_variable>
#include <cstdlib>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/moe_w4a16.h"
#include "launch.hpp"
#include "policy.hpp"

using namespace moe;

// Scratch of moe_expert_forward_noalloc: a fixed array in every GPU's memory,
// held until the process ends and shared by every call on that GPU.  Host
// code never passes this name to a kernel (on the host it is only a stand-in
// for the symbol): it uses the device address that hipGetSymbolAddress
// returned for the current device, kept in g_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_create_error;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on `device`, which must be the current device;
// looked up once per device.  Returns null when the lookup fails.
void* scratch_on_device(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[device] = p;
  }
  return g_scratch_ptr[device];
}

// Host copy into pinned staging, split over a few persistent threads (the
// caller takes one part): one thread cannot fill a staging buffer as fast as
// the link drains it.
class CopyPool {
 public:
  explicit CopyPool(int workers) {
    for (int i = 0; i < workers; ++i) th_.emplace_back([this, i] { run(i); });
  }
  ~CopyPool() {
    {
      std::lock_guard<std::mutex> lk(m_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  void copy(uint8_t* dst, const uint8_t* src, size_t bytes) {
    const size_t parts = th_.size() + 1;
    const size_t part = ((bytes + parts - 1) / parts + 63) & ~(size_t)63;
    {
      std::lock_guard<std::mutex> lk(m_);
      dst_ = dst;
      src_ = src;
      bytes_ = bytes;
      part_ = part;
      pending_ = (int)th_.size();
      ++gen_;
    }
    cv_.notify_all();
    piece(th_.size(), dst, src, bytes, part);  // the caller's part
    std::unique_lock<std::mutex> lk(m_);
    done_.wait(lk, [this] { return pending_ == 0; });
  }

 private:
  static void piece(size_t i, uint8_t* dst, const uint8_t* src, size_t bytes, size_t part) {
    const size_t b = i * part;
    if (b < bytes) memcpy(dst + b, src + b, std::min(part, bytes - b));
  }
  void run(int i) {
    uint64_t seen = 0;
    for (;;) {
      uint8_t* dst;
      const uint8_t* src;
      size_t bytes, part;
      {
        std::unique_lock<std::mutex> lk(m_);
        cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
        if (stop_) return;
        seen = gen_;
        dst = dst_;
        src = src_;
        bytes = bytes_;
        part = part_;
      }
      piece((size_t)i, dst, src, bytes, part);
      {
        std::lock_guard<std::mutex> lk(m_);
        if (--pending_ == 0) done_.notify_one();
      }
    }
  }
  std::mutex m_;
  std::condition_variable cv_, done_;
  std::vector<std::thread> th_;
  uint8_t* dst_ = nullptr;
  const uint8_t* src_ = nullptr;
  size_t bytes_ = 0, part_ = 0;
  uint64_t gen_ = 0;
  int pending_ = 0;
  bool stop_ = false;
};

struct LayerState {
  bool registered = false;
  uint16_t* router = nullptr;  // dev [E,H] fp16
  uint8_t* store = nullptr;    // dev: E blobs (resident) or C slot blobs (pool)
  uint8_t* shared = nullptr;   // dev: shared-expert blob
  int32_t* map = nullptr;      // dev [E]: expert -> slot, -1 = not resident
  uint8_t* backing = nullptr;  // host [E blobs] (pool only): pinned, or pageable RAM (staged transport)
  bool pageable = false;
  bool spare = false;  // spare rows: misses land in rows no generation reads
  // with spare rows: logical slot -> GPU row (-1 empty), and the rows no
  // generation reads, each with the event after which its last reader of an
  // older generation has retired (null: never read)
  std::vector<int32_t> phys;
  struct FreeRow {
    int32_t row;
    std::shared_ptr<ihipEvent_t> lease;
  };
  std::vector<FreeRow> free_rows;
  std::unique_ptr<PolicyEngine> policy;
  hipEvent_t retired = nullptr;
  hipEvent_t ready = nullptr;
  hipEvent_t pf_ready = nullptr;  // after the latest prefetch copies of the layer
  bool pf_recorded = false;
  moe_cache_counters stats{};
  std::vector<std::pair<hipEvent_t, hipEvent_t>> timing;
  int inject = 0;  // test hook: 1 fail before publication, 2 fail after it
};

}  // namespace

struct moe_ctx {
  moe_config cfg{};
  BlobLayout lay{}, shared_lay{};
  std::vector<LayerState> layers;
  float* logits = nullptr;
  double* rscratch = nullptr;  // FP64 partial logits and sums of magnitudes of the matrix-core router
  int32_t* ids = nullptr;
  float* w = nullptr;
  int32_t* ids_s = nullptr;
  ActiveExpert* active = nullptr;
  int32_t* n_active = nullptr;
  int32_t* perm_tok = nullptr;
  int32_t* pos_of = nullptr;
  int32_t* mtile_off = nullptr;
  uint16_t* hbuf = nullptr;
  uint16_t* hshared = nullptr;
  float* ybuf = nullptr;
  float* yshared = nullptr;
  uint16_t* xbuf = nullptr;
  float* ssq = nullptr;        // [max_tokens][ceil(H/1024)] residual sums of squares (per-layer stack)
  uint32_t* err = nullptr;
  hipStream_t side = nullptr;
  int copy_delay_us = 0;       // test hook: wait before every host-to-device blob copy
  // slot pools: recorded after every call that publishes or reads the pool,
  // on that call's stream; the next such call waits for it first
  hipEvent_t pool_tail = nullptr;
  bool sync_each = false;      // MOE_SYNC_EACH_CALL=1 at creation
  std::string last_error;
  bool faulted = false;
  // fused decode path
  std::vector<FusedLayer> hlayers;
  FusedLayer* dlayers = nullptr;
  uint64_t* xh = nullptr;      // tagged exchange buffers of the fused path
  uint64_t* xlg = nullptr;
  uint64_t* xhb = nullptr;
  uint64_t* xgate = nullptr;
  uint32_t* epoch = nullptr;   // per-block epoch counters
  int grid = 0;
  int ncu = 1;                 // compute units (grid of the streaming kernel)
  uint64_t* stamps = nullptr;  // caller-owned phase-timestamp buffer or null
  // staged transport: pinned staging buffers (one blob each), reused after the
  // transfer out of each has completed
  std::vector<uint8_t*> stage;
  std::vector<hipEvent_t> stage_ev;
  std::vector<char> stage_used;
  int stage_next = 0;
  std::unique_ptr<CopyPool> copier;
  // natural routing over slot pools (moe_stack_forward_pooled)
  uint16_t* pool_x = nullptr;   // dev FP16 [max_tokens, H]: x of the current layer
  int32_t* pool_ids = nullptr;  // dev [n_layers, T, k] (room for max_tokens): routed ids, forced ids of the layer calls
  float* pool_w = nullptr;      // dev [max_tokens, k]
  int32_t* pool_gids = nullptr; // dev [max_tokens, k]: next layer's guessed ids
  int32_t* pool_cids = nullptr; // dev [n_layers, max_tokens, k]: forced ids of a token chunk
  int32_t* pool_ids_h = nullptr;   // pinned host [2, max_tokens, k]: routed + guessed ids
  // kernel timer
  int timer_kind = -1;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> timer_events;
  size_t timer_used = 0;
};

namespace {

moe_status fail(moe_ctx* c, moe_status st, const std::string& msg) {
  if (c)
    c->last_error = msg;
  else
    g_create_error = msg;
  return st;
}

#define HIPCHK(ctx, call)                                                           \
  do {                                                                              \
    hipError_t e_ = (call);                                                         \
    if (e_ != hipSuccess)                                                           \
      return fail(ctx, MOE_E_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

bool valid_dim(int v) { return v >= 256 && v <= 2048 && v % 256 == 0; }

// Canonical packing has k0..k7 of a row in nibbles 0..7 of a little-endian
// word; the device layout puts the even k in nibbles 0..3 and the odd k in
// nibbles 4..7 (see dequant8 in common.hpp).
inline uint32_t compress_low_nibbles(uint32_t v) {
  v &= 0x0F0F0F0Fu;
  v = (v | (v >> 4)) & 0x00FF00FFu;
  v = (v | (v >> 8)) & 0x0000FFFFu;
  return v;
}
inline uint32_t to_device_word(uint32_t c) {
  return compress_low_nibbles(c) | (compress_low_nibbles(c >> 4) << 16);
}

// One expert's canonical (codes [3][cb], scales [3][sc]) -> device blob bytes.
// Canonical codes are row-major: gate and up [I][H/2], down [H][I/2]
// (I = 2 * cb / H); on the device they go in blocks of 16 rows (code_offset).
void repack_expert(const uint8_t* q, const uint16_t* s, int64_t cb, int64_t sc, int H, uint8_t* dst) {
  const int I = (int)(2 * cb / H);
  for (int m = 0; m < 3; ++m) {
    const int rows = m < 2 ? I : H, rb = m < 2 ? H / 2 : I / 2;
    const uint8_t* src = q + m * cb;
    uint8_t* d = dst + m * cb;
    for (int r = 0; r < rows; ++r)
      for (int b = 0; b < rb; b += 4) {
        uint32_t w;
        memcpy(&w, src + (int64_t)r * rb + b, 4);
        w = to_device_word(w);
        memcpy(d + code_offset(r, b, rb), &w, 4);
      }
  }
  memcpy(dst + 3 * cb, s, 3 * sc * sizeof(uint16_t));
}

// Repack E experts with a few host threads.
void repack_many(const uint8_t* q, const uint16_t* s, int n, int64_t cb, int64_t sc, int H,
                 uint8_t* dst, int64_t blob) {
  unsigned nt = std::thread::hardware_concurrency();
  nt = nt == 0 ? 1 : (nt > 16 ? 16 : nt);
  if ((int64_t)n * blob < (64ll << 20)) nt = 1;
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back([=] {
      for (int e = (int)t; e < n; e += (int)nt)
        repack_expert(q + (int64_t)e * 3 * cb, s + (int64_t)e * 3 * sc, cb, sc, H, dst + e * blob);
    });
  for (auto& x : th) x.join();
}

moe_status check_ctx(moe_ctx* c) {
  if (!c) return MOE_E_ARG;
  if (c->faulted) return fail(c, MOE_E_FAULTED, "context is faulted");
  return MOE_OK;
}

moe_status check_layer(moe_ctx* c, int layer) {
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, MOE_E_ARG, "layer index out of range");
  if (!c->layers[layer].registered) return fail(c, MOE_E_NOT_REGISTERED, "layer not registered");
  return MOE_OK;
}

bool pooled(const moe_ctx* c) { return c->cfg.policy != MOE_RESIDENT_ALL; }

// Keeps the timing events of a layer's transfers bounded: once many are held,
// the pairs whose transfers have completed are folded into h2d_seconds (the
// rest are kept for moe_cache_stats, which waits for them).
void note_transfer(LayerState& L, hipEvent_t t0, hipEvent_t t1) {
  L.timing.emplace_back(t0, t1);
  if (L.timing.size() < 256) return;
  size_t keep = 0;
  for (auto& p : L.timing) {
    float ms = 0.0f;
    if (hipEventQuery(p.second) == hipSuccess && hipEventElapsedTime(&ms, p.first, p.second) == hipSuccess) {
      L.stats.h2d_seconds += ms * 1e-3;
      (void)hipEventDestroy(p.first);
      (void)hipEventDestroy(p.second);
    } else {
      (void)hipGetLastError();  // not complete yet (hipErrorNotReady)
      L.timing[keep++] = p;
    }
  }
  L.timing.resize(keep);
}

// GPU row that holds logical slot `slot` of a pooled layer.
int32_t row_of(const LayerState& L, int32_t slot) { return L.spare ? L.phys[slot] : slot; }

// Row state of a pool with spare rows, saved before a transaction so that a
// failure before publication leaves the old generation as it was.
struct RowState {
  std::vector<int32_t> phys;
  std::vector<LayerState::FreeRow> free_rows;
};
RowState save_rows(const LayerState& L) { return RowState{L.phys, L.free_rows}; }
void restore_rows(LayerState& L, RowState&& r) {
  L.phys = std::move(r.phys);
  L.free_rows = std::move(r.free_rows);
}

// Enqueues the transfers of `fills` (decisions that load an expert into a
// logical slot) on the side stream, between the timing events t0 and t1, and
// records `done` after them.  Returns false if one could not be enqueued; the
// caller then restores the policy and row state it saved.
//   in-place slots (no spare rows): the side stream first waits for the
//     layer's last reader (`retired`), then copies each blob into its slot;
//   spare rows: each fill takes the lowest free GPU row (after that row's
//     lease).  The rows the victims leave are freed after this call with a
//     lease recorded now on `s`: every reader of the old generation is
//     enqueued before it, so no transfer waits for the current readers and
//     none overwrites a row they still read.
// A blob comes straight from the pinned backing, or (staged transport) from
// the pageable source through the next pinned staging buffer, after a host
// wait until that buffer's previous transfer has completed.
// Calls from several streams on a pooled context.  The calls that publish or
// read the slot pool (and use the context's scratch) run on the GPU one after
// another in the order they were made, whatever their streams: each first
// makes its stream wait for the previous one's end (the wait takes that record
// as it stands when the wait is enqueued; the next record comes after it).
// Transfers still run on the side stream beside them.  A row's lease, recorded
// on the stream of the call that vacates it after that wait, and each layer's
// `retired` event, recorded by its latest reader, therefore cover every
// earlier reader on every stream.
moe_status pool_order_begin(moe_ctx* c, hipStream_t s) {
  if (!pooled(c) || !c->pool_tail) return MOE_OK;
  HIPCHK(c, hipStreamWaitEvent(s, c->pool_tail, 0));
  return MOE_OK;
}
moe_status pool_order_end(moe_ctx* c, hipStream_t s) {
  if (!pooled(c)) return MOE_OK;
  if (!c->pool_tail) HIPCHK(c, hipEventCreateWithFlags(&c->pool_tail, hipEventDisableTiming));
  HIPCHK(c, hipEventRecord(c->pool_tail, s));
  return MOE_OK;
}

// Test hook: occupies the side stream for the set time before a blob copy.
void delay_copy(moe_ctx* c) {
  if (c->copy_delay_us > 0) launch_copy_delay(c->side, c->copy_delay_us);
}

bool enqueue_fills(moe_ctx* c, LayerState& L, const std::vector<PolicyEngine::Decision>& fills, hipStream_t s,
                   hipEvent_t t0, hipEvent_t t1, hipEvent_t done) {
  const int64_t blob = c->lay.total();
  bool good = true;
  if (!L.spare) {
    good = hipStreamWaitEvent(c->side, L.retired, 0) == hipSuccess;
    good = good && hipEventRecord(t0, c->side) == hipSuccess;
    for (const auto& d : fills) {
      if (!good) break;
      delay_copy(c);
      good = hipMemcpyAsync(L.store + (int64_t)d.slot * blob, L.backing + (int64_t)d.expert * blob,
                            (size_t)blob, hipMemcpyHostToDevice, c->side) == hipSuccess;
    }
  } else {
    std::shared_ptr<ihipEvent_t> lease;
    bool vacates = false;
    for (const auto& d : fills) vacates = vacates || L.phys[d.slot] >= 0;
    if (vacates) {
      hipEvent_t ev = nullptr;
      if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) return false;
      lease.reset(ev, [](hipEvent_t e) { (void)hipEventDestroy(e); });
      good = hipEventRecord(ev, s) == hipSuccess;
    }
    good = good && hipEventRecord(t0, c->side) == hipSuccess;
    std::vector<LayerState::FreeRow> released;
    for (const auto& d : fills) {
      if (!good || L.free_rows.empty()) {
        good = false;  // (spare_rows >= the fills of one call: a free row exists)
        break;
      }
      size_t bi = 0;
      for (size_t i = 1; i < L.free_rows.size(); ++i)
        if (L.free_rows[i].row < L.free_rows[bi].row) bi = i;
      const LayerState::FreeRow fr = L.free_rows[bi];
      L.free_rows.erase(L.free_rows.begin() + bi);
      if (fr.lease) good = hipStreamWaitEvent(c->side, fr.lease.get(), 0) == hipSuccess;
      if (!good) break;
      if (L.pageable) {
        const int si = c->stage_next;
        c->stage_next = (c->stage_next + 1) % (int)c->stage.size();
        if (c->stage_used[si]) good = hipEventSynchronize(c->stage_ev[si]) == hipSuccess;
        if (!good) break;
        c->copier->copy(c->stage[si], L.backing + (int64_t)d.expert * blob, (size_t)blob);
        delay_copy(c);
        good = hipMemcpyAsync(L.store + (int64_t)fr.row * blob, c->stage[si], (size_t)blob,
                              hipMemcpyHostToDevice, c->side) == hipSuccess;
        good = good && hipEventRecord(c->stage_ev[si], c->side) == hipSuccess;
        c->stage_used[si] = 1;
      } else {
        delay_copy(c);
        good = hipMemcpyAsync(L.store + (int64_t)fr.row * blob, L.backing + (int64_t)d.expert * blob,
                              (size_t)blob, hipMemcpyHostToDevice, c->side) == hipSuccess;
      }
      if (L.phys[d.slot] >= 0) released.push_back({L.phys[d.slot], lease});
      L.phys[d.slot] = fr.row;
    }
    for (auto& r : released) L.free_rows.push_back(std::move(r));
  }
  good = good && hipEventRecord(t1, c->side) == hipSuccess;
  good = good && hipEventRecord(done, c->side) == hipSuccess;
  return good;
}

enum KernelKind {
  kKindLogits = 0, kKindTopk, kKindGroup, kKindGateUp, kKindDown, kKindCombine, kKindNorm, kKindFused,
  kKindMfmaGateUp, kKindMfmaDown
};

constexpr int kMfmaMinTokens = 8;  // per-expert token count from which MFMA is used

bool fused_eligible(const moe_ctx* c, int T) {
  const moe_config& g = c->cfg;
  if (g.flags & MOE_FLAG_NO_FUSED) return false;
  if (T > kFMaxT || T * g.top_k > kFMaxP || T * g.n_experts > kFMaxTE) return false;
  if (g.n_experts % 64 != 0 || (g.n_experts / 64) * g.top_k > kFMaxCand) return false;
  if (g.shared_inter != 0 && g.shared_inter != g.inter) return false;
  if ((int64_t)(T * g.top_k + (g.shared_inter ? T : 0)) * g.inter > kFStageHalves) return false;
  return c->grid == kFGrid && fused_supported(g.hidden, g.inter);
}

// Brackets one launch with a recorded event pair when the timer is on for `kind`.
struct ScopedTimer {
  moe_ctx* c;
  hipStream_t s;
  hipEvent_t stop = nullptr;
  ScopedTimer(moe_ctx* ctx, int kind, hipStream_t stream) : ScopedTimer(ctx, true, kind, stream) {}
  // enabled = false: never times (and never creates events)
  ScopedTimer(moe_ctx* ctx, bool enabled, int kind, hipStream_t stream) : c(ctx), s(stream) {
    if (!enabled || c->timer_kind != kind) return;
    if (c->timer_used == c->timer_events.size()) {
      hipEvent_t a = nullptr, b = nullptr;
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return;
      c->timer_events.emplace_back(a, b);
    }
    auto& p = c->timer_events[c->timer_used++];
    (void)hipEventRecord(p.first, s);
    stop = p.second;
  }
  ~ScopedTimer() {
    if (stop) (void)hipEventRecord(stop, s);
  }
};

int max_active(const moe_ctx* c, int T) {
  const int64_t p = (int64_t)T * c->cfg.top_k;
  return (int)(p < c->cfg.n_experts ? p : c->cfg.n_experts);
}

void run_router(moe_ctx* c, const RouterArgs& ra, hipStream_t s) {
  {
    ScopedTimer tm(c, kKindLogits, s);
    if (launch_router(ra, c->rscratch, s)) return;
    launch_router_logits(ra, s);
  }
  ScopedTimer tm(c, kKindTopk, s);
  launch_router_topk(ra, s);
}

// Device scratch of the expert path of one call: the grouping's outputs, the
// FP16 intermediates and the FP32 expert outputs.  Every word the kernels read
// is written earlier in the same call, so nothing has to start at zero.
// Entries of the active-expert lists of a T-token call: the active list (E),
// then the few-token kernel's list (E, or with chunks of kStreamTokens tokens
// E + ceil(T*k / kStreamTokens)).
size_t active_list_entries(const moe_config& g, int T) {
  return (size_t)2 * g.n_experts + ((size_t)T * g.top_k + kStreamTokens - 1) / kStreamTokens;
}

struct ExpertScratch {
  int32_t* ids_s;          // [P]
  ActiveExpert* active;    // [active_list_entries]: active list, then the few-token kernel's list
  int32_t* n_active;       // [2]
  int32_t* perm_tok;       // [P]
  int32_t* pos_of;         // [P]
  int32_t* mtile_off;      // [E+1]
  uint16_t* hbuf;          // [P + T, max(I, Is)] fp16
  float* ybuf;             // [P, H]
  uint16_t* hshared;       // [T, Is] fp16 (shared expert only)
  float* yshared;          // [T, H]   (shared expert only)
};

ExpertScratch ctx_scratch(moe_ctx* c) {
  return ExpertScratch{c->ids_s, c->active, c->n_active, c->perm_tok, c->pos_of,
                       c->mtile_off, c->hbuf, c->ybuf, c->hshared, c->yshared};
}

// Carves the scratch of a T-token call out of `base` (256-byte aligned parts);
// returns the bytes used, whether or not base is null.
size_t carve_scratch(const moe_config& g, int T, uint8_t* base, ExpertScratch* out) {
  const size_t P = (size_t)T * g.top_k;
  const size_t Imax = (size_t)std::max(g.inter, g.shared_inter);
  size_t off = 0;
  auto take = [&](size_t bytes) -> uint8_t* {
    uint8_t* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  ExpertScratch x{};
  x.ids_s = (int32_t*)take(P * 4);
  x.active = (ActiveExpert*)take(active_list_entries(g, T) * sizeof(ActiveExpert));
  x.n_active = (int32_t*)take(2 * 4);
  x.perm_tok = (int32_t*)take(P * 4);
  x.pos_of = (int32_t*)take(P * 4);
  x.mtile_off = (int32_t*)take((size_t)(g.n_experts + 1) * 4);
  x.hbuf = (uint16_t*)take((P + T) * Imax * 2);
  x.ybuf = (float*)take(P * g.hidden * 4);
  if (g.shared_inter) {
    x.hshared = (uint16_t*)take((size_t)T * g.shared_inter * 2);
    x.yshared = (float*)take((size_t)T * g.hidden * 4);
  }
  if (out) *out = x;
  return off;
}

// group -> gate/up -> down (routed and shared) -> combine into out or resid.
// `timed`: launches may be bracketed by the kernel timer's events (which it
// creates on first use); the allocation-free entry point passes false.
moe_status run_experts(moe_ctx* c, int layer, const uint16_t* x, int T, const int32_t* ids,
                       const float* w, uint16_t* out, float* resid, hipStream_t s,
                       const ExpertScratch& sc, bool timed = true, float* ssq = nullptr) {
  LayerState& L = c->layers[layer];
  const moe_config& g = c->cfg;

  // experts with at least mfma_min tokens run on the MFMA grouped GEMM; the
  // choice depends only on the token counts
  // experts with few tokens take the persistent streaming kernel where the
  // shapes allow it (then every expert with up to kStreamTokens tokens), else
  // the GEMV kernels
  const bool force_gemv = (g.flags & MOE_FLAG_FORCE_GEMV) != 0;
  // with at least kPrefillPairsPerExpert pairs per expert on average (prefill)
  // every expert runs on the grouped GEMM and the few-token kernels are not
  // launched
  const bool all_mfma = !force_gemv && ((g.flags & MOE_FLAG_FORCE_MFMA) ||
                                        (int64_t)T * g.top_k >= (int64_t)kPrefillPairsPerExpert * g.n_experts);
  const bool stream_gu = !force_gemv && stream_supported(0, g.hidden, g.inter);
  const bool stream_dn = !force_gemv && stream_supported(1, g.inter, g.hidden);
  // below the prefill threshold with both streaming kernels available, they
  // take every expert (one with more than kStreamTokens tokens as several
  // list entries, each streaming the weights again): no grouped-GEMM launch,
  // which costs several microseconds even when it finds no tile
  const bool chunk_all = !force_gemv && !all_mfma && stream_gu && stream_dn;
  const int mfma_min = force_gemv ? INT32_MAX
                       : all_mfma ? 1
                       : chunk_all ? INT32_MAX
                       : (stream_gu ? kStreamTokens + 1 : kMfmaMinTokens);
  GroupArgs ga{ids, T, g.top_k, g.n_experts, L.map, sc.ids_s, sc.active, sc.n_active,
               sc.perm_tok, sc.pos_of, c->err, mfma_min, sc.mtile_off,
               sc.active + g.n_experts, sc.n_active + 1, chunk_all ? 1 : 0};
  // a shared expert of the routed experts' shape rides along in the streaming
  // launches as one more list entry (one weight stream over the whole chip
  // instead of two launches of its own)
  const bool shared_in_stream = g.shared_inter == g.inter && !all_mfma && stream_gu && stream_dn &&
                                T <= kStreamTokens;
  // when every expert takes the streaming kernels, the gate/up kernel groups
  // the pairs itself where that fits (no grouping launch, and its blocks start
  // from LDS lists instead of reading them back)
  const bool group_in_kernel =
      chunk_all && stream_group_in_kernel_ok(T, g.top_k, g.n_experts, g.inter, c->ncu, shared_in_stream);
  if (!group_in_kernel) {
    ScopedTimer tm(c, timed, kKindGroup, s);
    launch_group(ga, s);
  }
  const bool any_mfma = T >= mfma_min;
  MfmaArgs ma{L.store, c->lay.total(), c->lay, sc.active, sc.n_active, sc.mtile_off,
              g.hidden, g.inter, x, sc.perm_tok, sc.hbuf, sc.ybuf};
  ExpertArgs ea{};
  ea.mfma_min = mfma_min;
  ea.blobs = L.store;
  ea.blob_stride = c->lay.total();
  ea.lay = c->lay;
  ea.active = sc.active;
  ea.n_active = sc.n_active;
  ea.small = sc.active + g.n_experts;
  ea.n_small = sc.n_active + 1;
  ea.max_active = max_active(c, T);
  ea.H = g.hidden;
  ea.I = g.inter;
  ea.x = x;
  ea.perm_tok = sc.perm_tok;
  ea.hbuf = sc.hbuf;
  ea.ybuf = sc.ybuf;
  if (shared_in_stream) {
    ea.shared_blob = L.shared;
    ea.shared_count = T;
    ea.shared_h = sc.hshared;
    ea.shared_y = sc.yshared;
  }
  if (group_in_kernel) {
    ea.group_in_kernel = 1;
    ea.grp = ga;
  }
  if (!all_mfma) {
    ScopedTimer tm(c, timed, kKindGateUp, s);
    if (stream_gu) launch_stream_expert(ea, 0, c->ncu, s);
    else launch_gateup_gemv(ea, s);
  }
  if (any_mfma) {
    ScopedTimer tm(c, timed, kKindMfmaGateUp, s);
    launch_mfma_gateup(ma, mfma_max_tiles(T, g.top_k, g.n_experts, g.inter, 0, mfma_min), s);
  }
  if (!all_mfma) {
    ScopedTimer tm(c, timed, kKindDown, s);
    if (stream_dn && stream_gu) launch_stream_expert(ea, 1, c->ncu, s);
    else launch_down_gemv(ea, s);
  }
  if (any_mfma) {
    ScopedTimer tm(c, timed, kKindMfmaDown, s);
    launch_mfma_down(ma, mfma_max_tiles(T, g.top_k, g.n_experts, g.hidden, 1, mfma_min), s);
  }
  if (g.shared_inter && !shared_in_stream) {
    ExpertArgs sa = ea;
    sa.group_in_kernel = 0;  // one fixed expert: no list
    sa.shared_blob = nullptr;
    sa.lay = c->shared_lay;
    sa.fixed_blob = L.shared;
    sa.fixed_count = T;
    sa.fixed_offset = 0;
    sa.I = g.shared_inter;
    sa.hbuf = sc.hshared;
    sa.ybuf = sc.yshared;
    const bool st_gu = !force_gemv && T <= kStreamTokens && stream_supported(0, g.hidden, g.shared_inter);
    const bool st_dn = st_gu && stream_supported(1, g.shared_inter, g.hidden);
    if (st_gu) launch_stream_expert(sa, 0, c->ncu, s);
    else launch_gateup_gemv(sa, s);
    if (st_dn) launch_stream_expert(sa, 1, c->ncu, s);
    else launch_down_gemv(sa, s);
  }
  CombineArgs ca{sc.ybuf, g.shared_inter ? sc.yshared : nullptr, sc.pos_of, w, T, g.top_k,
                 g.hidden, out, resid, ssq};
  {
    ScopedTimer tm(c, timed, kKindCombine, s);
    launch_combine(ca, s);
  }
  if (pooled(c)) HIPCHK(c, hipEventRecord(L.retired, s));
  HIPCHK(c, hipGetLastError());
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(const moe_ctx* ctx) {
  return ctx ? ctx->last_error.c_str() : g_create_error.c_str();
}

moe_status moe_create(const moe_config* cfg, moe_ctx** out) {
  if (!out) return fail(nullptr, MOE_E_ARG, "out is NULL");
  *out = nullptr;
  if (!cfg) return fail(nullptr, MOE_E_ARG, "cfg is NULL");
  const moe_config g = *cfg;
  if (!valid_dim(g.hidden) || !valid_dim(g.inter) || (g.shared_inter && !valid_dim(g.shared_inter)))
    return fail(nullptr, MOE_E_SHAPE, "hidden/inter/shared_inter must be multiples of 256 in [256, 2048]");
  if (g.n_experts < 1 || g.n_experts > 1024) return fail(nullptr, MOE_E_SHAPE, "n_experts must be in [1, 1024]");
  if (g.top_k < 1 || g.top_k > 16 || g.top_k > g.n_experts) return fail(nullptr, MOE_E_SHAPE, "top_k must be in [1, min(16, E)]");
  if (g.group != 128) return fail(nullptr, MOE_E_SHAPE, "group must be 128");
  if (g.n_layers < 1) return fail(nullptr, MOE_E_SHAPE, "n_layers must be >= 1");
  if (g.max_tokens < 1 || g.max_tokens > 8192) return fail(nullptr, MOE_E_SHAPE, "max_tokens must be in [1, 8192]");
  if (g.policy < 0 || g.policy > 3) return fail(nullptr, MOE_E_ARG, "unknown policy");
  if (g.policy != MOE_RESIDENT_ALL) {
    const int64_t need = std::min<int64_t>(g.n_experts, (int64_t)g.max_tokens * g.top_k);
    if (g.slots_per_layer < need || g.slots_per_layer > g.n_experts)
      return fail(nullptr, MOE_E_CAPACITY,
                  "slots_per_layer must be >= min(E, max_tokens*k) and <= E");
  }
  const bool staged = g.policy != MOE_RESIDENT_ALL && (g.flags & MOE_FLAG_STAGED_TRANSPORT);
  const bool spare = g.policy != MOE_RESIDENT_ALL && (staged || g.spare_rows > 0);
  if (g.spare_rows < 0) return fail(nullptr, MOE_E_ARG, "spare_rows must be >= 0");
  if (spare) {
    const int64_t need = std::min<int64_t>(g.slots_per_layer, (int64_t)g.max_tokens * g.top_k);
    if ((staged && g.staging_blobs < 1) || g.spare_rows < need)
      return fail(nullptr, MOE_E_CAPACITY,
                  "spare rows need spare_rows >= min(C, max_tokens*k), and the staged transport "
                  "staging_blobs >= 1");
  }
  std::unique_ptr<moe_ctx> c(new moe_ctx());
  c->cfg = g;
  if (const char* v = std::getenv("MOE_SYNC_EACH_CALL")) c->sync_each = std::string(v) == "1";
  const int64_t cb = (int64_t)g.inter * g.hidden / 2, sc = (int64_t)g.inter * g.hidden / 128;
  c->lay = BlobLayout{cb, sc * 2};
  const int64_t scb = (int64_t)g.shared_inter * g.hidden / 2, ssc = (int64_t)g.shared_inter * g.hidden / 128;
  c->shared_lay = BlobLayout{scb, ssc * 2};
  hipError_t e = hipSetDevice(g.device);
  if (e != hipSuccess) return fail(nullptr, MOE_E_HIP, std::string("hipSetDevice: ") + hipGetErrorString(e));
  // the allocation-free entry point's scratch on this device (its address is
  // looked up here, with the device current, once per device)
  if (!scratch_on_device(g.device))
    return fail(nullptr, MOE_E_HIP, "hipGetSymbolAddress of the static scratch failed");

  auto dalloc = [&](void** p, size_t bytes) -> bool {
    if (hipMalloc(p, bytes < 256 ? 256 : bytes) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    return true;
  };
  c->layers.resize(g.n_layers);
  const int64_t blob = c->lay.total();
  const int nslots = g.policy == MOE_RESIDENT_ALL ? g.n_experts
                                                  : g.slots_per_layer + (spare ? g.spare_rows : 0);
  bool ok = true;
  for (int l = 0; l < g.n_layers && ok; ++l) {
    LayerState& L = c->layers[l];
    L.spare = spare;
    ok = ok && dalloc((void**)&L.router, (size_t)g.n_experts * g.hidden * 2);
    ok = ok && dalloc((void**)&L.store, (size_t)nslots * blob);
    ok = ok && dalloc((void**)&L.map, (size_t)g.n_experts * 4);
    if (g.shared_inter) ok = ok && dalloc((void**)&L.shared, (size_t)c->shared_lay.total());
    if (ok && staged) {
      // the complete host source in pageable RAM, touched page by page when the
      // layer is registered, immutable afterwards
      L.backing = new (std::nothrow) uint8_t[(size_t)g.n_experts * blob];
      L.pageable = true;
      ok = L.backing != nullptr;
    } else if (ok && g.policy != MOE_RESIDENT_ALL) {
      if (hipHostMalloc((void**)&L.backing, (size_t)g.n_experts * blob, hipHostMallocDefault) != hipSuccess) {
        (void)hipGetLastError();
        L.backing = nullptr;
        ok = false;
      }
    }
    if (ok) {
      if (hipEventCreateWithFlags(&L.retired, hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&L.ready, hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&L.pf_ready, hipEventDisableTiming) != hipSuccess)
        ok = false;
    }
  }
  const int64_t P = (int64_t)g.max_tokens * g.top_k;
  const int Imax = g.inter;
  ok = ok && dalloc((void**)&c->logits, (size_t)g.max_tokens * g.n_experts * 4);
  if (const size_t rb = router_scratch_bytes(g.max_tokens, g.n_experts, g.hidden))
    ok = ok && dalloc((void**)&c->rscratch, rb);
  ok = ok && dalloc((void**)&c->ids, (size_t)P * 4);
  ok = ok && dalloc((void**)&c->w, (size_t)P * 4);
  ok = ok && dalloc((void**)&c->ids_s, (size_t)P * 4);
  // active list, then the list of the experts the few-token kernel takes
  ok = ok && dalloc((void**)&c->active, active_list_entries(g, g.max_tokens) * sizeof(ActiveExpert));
  ok = ok && dalloc((void**)&c->n_active, 2 * 4);
  ok = ok && dalloc((void**)&c->perm_tok, (size_t)P * 4);
  ok = ok && dalloc((void**)&c->pos_of, (size_t)P * 4);
  ok = ok && dalloc((void**)&c->mtile_off, (size_t)(g.n_experts + 1) * 4);
  // rows: routed (token, rank) pairs, then the shared expert's tokens
  ok = ok && dalloc((void**)&c->hbuf, (size_t)(P + g.max_tokens) * std::max(Imax, g.shared_inter) * 2);
  ok = ok && dalloc((void**)&c->dlayers, (size_t)g.n_layers * sizeof(FusedLayer));
  c->hlayers.assign(g.n_layers, FusedLayer{nullptr, nullptr, nullptr, nullptr});
  {
    // the fused path runs one block per compute unit on exactly kFGrid of them
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, g.device) != hipSuccess) ncu = 0;
    c->grid = ncu >= kFGrid ? kFGrid : 0;
    c->ncu = ncu > 0 ? ncu : 1;
    ok = ok && dalloc((void**)&c->xh, (size_t)kFXhWords * 8);
    ok = ok && dalloc((void**)&c->xlg, (size_t)kFXlgWords * 8);
    ok = ok && dalloc((void**)&c->xhb, (size_t)kFXhbWords * 8);
    ok = ok && dalloc((void**)&c->xgate, (size_t)kFGrid * 8);
    ok = ok && dalloc((void**)&c->epoch, (size_t)kFGrid * 4);
    // tag 0 never names a layer: every later launch starts at epoch 1
    if (ok) ok = hipMemset(c->xh, 0, (size_t)kFXhWords * 8) == hipSuccess;
    if (ok) ok = hipMemset(c->xlg, 0, (size_t)kFXlgWords * 8) == hipSuccess;
    if (ok) ok = hipMemset(c->xhb, 0, (size_t)kFXhbWords * 8) == hipSuccess;
    if (ok) ok = hipMemset(c->xgate, 0, (size_t)kFGrid * 8) == hipSuccess;
    if (ok) ok = hipMemset(c->epoch, 0, (size_t)kFGrid * 4) == hipSuccess;
  }
  ok = ok && dalloc((void**)&c->ybuf, (size_t)P * g.hidden * 4);
  ok = ok && dalloc((void**)&c->xbuf, (size_t)g.max_tokens * g.hidden * 2);
  ok = ok && dalloc((void**)&c->ssq, (size_t)g.max_tokens * ((g.hidden + 1023) / 1024) * sizeof(float));
  ok = ok && dalloc((void**)&c->err, 4);
  if (g.shared_inter) {
    ok = ok && dalloc((void**)&c->hshared, (size_t)g.max_tokens * g.shared_inter * 2);
    ok = ok && dalloc((void**)&c->yshared, (size_t)g.max_tokens * g.hidden * 4);
  }
  if (g.policy != MOE_RESIDENT_ALL) {
    ok = ok && dalloc((void**)&c->pool_x, (size_t)g.max_tokens * g.hidden * 2);
    ok = ok && dalloc((void**)&c->pool_ids, (size_t)g.n_layers * P * 4);
    ok = ok && dalloc((void**)&c->pool_w, (size_t)P * 4);
    ok = ok && dalloc((void**)&c->pool_gids, (size_t)P * 4);
    ok = ok && dalloc((void**)&c->pool_cids, (size_t)g.n_layers * P * 4);
    if (ok && hipHostMalloc((void**)&c->pool_ids_h, (size_t)2 * P * 4, hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      c->pool_ids_h = nullptr;
      ok = false;
    }
  }
  if (ok && staged) {
    for (int i = 0; i < g.staging_blobs && ok; ++i) {
      uint8_t* p = nullptr;
      hipEvent_t ev = nullptr;
      if (hipHostMalloc((void**)&p, (size_t)blob, hipHostMallocDefault) != hipSuccess) {
        (void)hipGetLastError();
        ok = false;
        break;
      }
      c->stage.push_back(p);
      if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
        (void)hipGetLastError();
        ok = false;
        break;
      }
      c->stage_ev.push_back(ev);
      c->stage_used.push_back(0);
    }
    if (ok) c->copier.reset(new CopyPool(3));
  }
  if (ok && hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess) ok = false;
  if (ok) {
    const uint32_t zero = 0;
    ok = hipMemcpy(c->err, &zero, 4, hipMemcpyHostToDevice) == hipSuccess;
  }
  if (!ok) {
    moe_destroy(c.release());
    return fail(nullptr, MOE_E_OOM, "device or pinned allocation failed");
  }
  *out = c.release();
  return MOE_OK;
}

void moe_destroy(moe_ctx* c) {
  if (!c) return;
  (void)hipSetDevice(c->cfg.device);
  (void)hipDeviceSynchronize();
  for (LayerState& L : c->layers) {
    (void)hipFree(L.router);
    (void)hipFree(L.store);
    (void)hipFree(L.map);
    (void)hipFree(L.shared);
    if (L.backing && L.pageable) delete[] L.backing;
    else if (L.backing) (void)hipHostFree(L.backing);
    L.free_rows.clear();  // releases the lease events
    if (L.retired) (void)hipEventDestroy(L.retired);
    if (L.ready) (void)hipEventDestroy(L.ready);
    if (L.pf_ready) (void)hipEventDestroy(L.pf_ready);
    for (auto& p : L.timing) {
      (void)hipEventDestroy(p.first);
      (void)hipEventDestroy(p.second);
    }
  }
  void* bufs[] = {c->logits, c->rscratch, c->ids,  c->w,    c->ids_s,   c->active,  c->n_active, c->perm_tok,
                  c->pos_of, c->hbuf, c->ybuf, c->xbuf,    c->ssq,     c->err,      c->hshared,  c->yshared,
                  c->dlayers, c->mtile_off, c->xh, c->xlg, c->xhb, c->xgate, c->epoch,
                  c->pool_x, c->pool_ids, c->pool_w, c->pool_gids, c->pool_cids};
  for (void* p : bufs) (void)hipFree(p);
  if (c->pool_ids_h) (void)hipHostFree(c->pool_ids_h);
  c->copier.reset();
  for (uint8_t* p : c->stage) (void)hipHostFree(p);
  for (hipEvent_t e : c->stage_ev) (void)hipEventDestroy(e);
  if (c->side) (void)hipStreamDestroy(c->side);
  if (c->pool_tail) (void)hipEventDestroy(c->pool_tail);
  for (auto& p : c->timer_events) {
    (void)hipEventDestroy(p.first);
    (void)hipEventDestroy(p.second);
  }
  delete c;
}

moe_status moe_register_layer(moe_ctx* c, int32_t layer, const uint16_t* router, const uint8_t* q,
                              const uint16_t* s, const uint8_t* shared_q, const uint16_t* shared_s) {
  if (moe_status st = check_ctx(c)) return st;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, MOE_E_ARG, "layer index out of range");
  if (!router || !q || !s) return fail(c, MOE_E_ARG, "router, q and s are required");
  const moe_config& g = c->cfg;
  if (g.shared_inter && (!shared_q || !shared_s)) return fail(c, MOE_E_ARG, "shared expert weights required");
  if (!g.shared_inter && (shared_q || shared_s)) return fail(c, MOE_E_ARG, "no shared expert configured");
  HIPCHK(c, hipSetDevice(g.device));
  HIPCHK(c, hipDeviceSynchronize());
  LayerState& L = c->layers[layer];
  const int64_t cb = c->lay.code_bytes, sc = c->lay.scale_bytes / 2, blob = c->lay.total();
  HIPCHK(c, hipMemcpy(L.router, router, (size_t)g.n_experts * g.hidden * 2, hipMemcpyHostToDevice));
  std::vector<int32_t> map(g.n_experts);
  if (pooled(c)) {
    repack_many(q, s, g.n_experts, cb, sc, g.hidden, L.backing, blob);
    for (int e = 0; e < g.n_experts; ++e) map[e] = -1;
    L.policy.reset(new PolicyEngine(g.policy, g.n_experts, g.slots_per_layer, layer));
    L.stats = moe_cache_counters{};
    if (L.spare) {
      L.phys.assign(g.slots_per_layer, -1);
      L.free_rows.clear();
      for (int r = 0; r < g.slots_per_layer + g.spare_rows; ++r) L.free_rows.push_back({r, nullptr});
    }
  } else {
    // stage in chunks of experts through pinned memory
    const int chunk = 16;
    uint8_t* stage = nullptr;
    HIPCHK(c, hipHostMalloc((void**)&stage, (size_t)chunk * blob, hipHostMallocDefault));
    hipError_t err = hipSuccess;
    for (int e0 = 0; e0 < g.n_experts && err == hipSuccess; e0 += chunk) {
      const int n = std::min(chunk, g.n_experts - e0);
      repack_many(q + (int64_t)e0 * 3 * cb, s + (int64_t)e0 * 3 * sc, n, cb, sc, g.hidden, stage, blob);
      err = hipMemcpy(L.store + (int64_t)e0 * blob, stage, (size_t)n * blob, hipMemcpyHostToDevice);
    }
    (void)hipHostFree(stage);
    if (err != hipSuccess) return fail(c, MOE_E_HIP, std::string("hipMemcpy: ") + hipGetErrorString(err));
    for (int e = 0; e < g.n_experts; ++e) map[e] = e;
  }
  HIPCHK(c, hipMemcpy(L.map, map.data(), map.size() * 4, hipMemcpyHostToDevice));
  if (g.shared_inter) {
    const int64_t scb = c->shared_lay.code_bytes, ssc = c->shared_lay.scale_bytes / 2;
    std::vector<uint8_t> tmp((size_t)c->shared_lay.total());
    repack_expert(shared_q, shared_s, scb, ssc, g.hidden, tmp.data());
    HIPCHK(c, hipMemcpy(L.shared, tmp.data(), tmp.size(), hipMemcpyHostToDevice));
  }
  // full residency: slot = expert, the fused path skips the map lookup
  c->hlayers[layer] = FusedLayer{L.router, L.store, pooled(c) ? L.map : nullptr, L.shared};
  HIPCHK(c, hipMemcpy(c->dlayers + layer, &c->hlayers[layer], sizeof(FusedLayer), hipMemcpyHostToDevice));
  L.registered = true;
  return MOE_OK;
}

static moe_status moe_route_call(moe_ctx* c, int32_t layer, const void* x, int32_t T, const int32_t* forced_ids,
                     int32_t* ids, float* w, float* logits, void* stream) {
  if (moe_status st = check_ctx(c)) return st;
  if (moe_status st = check_layer(c, layer)) return st;
  if (!x || !ids || !w) return fail(c, MOE_E_ARG, "x, ids and w are required");
  if (T < 1 || T > c->cfg.max_tokens) return fail(c, MOE_E_ARG, "T out of range [1, max_tokens]");
  const moe_config& g = c->cfg;
  RouterArgs ra{(const uint16_t*)x, c->layers[layer].router, T, g.n_experts, g.hidden, g.top_k,
                g.renorm, logits ? logits : c->logits, forced_ids, ids, w, c->err,
                (int)(g.flags & MOE_FLAG_ROUTER_EXACT_ALWAYS)};
  run_router(c, ra, (hipStream_t)stream);
  HIPCHK(c, hipGetLastError());
  return MOE_OK;
}

static moe_status moe_expert_forward_call(moe_ctx* c, int32_t layer, const void* x, int32_t T, const int32_t* ids,
                              const float* w, void* out, void* stream) {
  if (moe_status st = check_ctx(c)) return st;
  if (moe_status st = check_layer(c, layer)) return st;
  if (!x || !ids || !w || !out) return fail(c, MOE_E_ARG, "x, ids, w and out are required");
  if (x == out) return fail(c, MOE_E_ARG, "out must not alias x");
  if (T < 1 || T > c->cfg.max_tokens) return fail(c, MOE_E_ARG, "T out of range [1, max_tokens]");
  return run_experts(c, layer, (const uint16_t*)x, T, ids, w, (uint16_t*)out, nullptr,
                     (hipStream_t)stream, ctx_scratch(c));
}

static moe_status moe_expert_forward_noalloc_call(moe_ctx* c, int32_t layer, const void* x, int32_t T, const int32_t* ids,
                                      const float* w, void* out, void* stream) {
  if (moe_status st = check_ctx(c)) return st;
  if (moe_status st = check_layer(c, layer)) return st;
  if (!x || !ids || !w || !out) return fail(c, MOE_E_ARG, "x, ids, w and out are required");
  if (x == out) return fail(c, MOE_E_ARG, "out must not alias x");
  if (T < 1 || T > c->cfg.max_tokens) return fail(c, MOE_E_ARG, "T out of range [1, max_tokens]");
  const size_t need = carve_scratch(c->cfg, T, nullptr, nullptr);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(c, MOE_E_ARG, "T needs " + std::to_string(need) + " bytes of scratch, more than the " +
                                  std::to_string((size_t)MOE_NOALLOC_SCRATCH_BYTES) + " of the static scratch");
  uint8_t* base = (uint8_t*)g_scratch_ptr[c->cfg.device];  // looked up by moe_create on this device
  if (!base) return fail(c, MOE_E_HIP, "static scratch address unknown on this device");
  ExpertScratch sc{};
  carve_scratch(c->cfg, T, base, &sc);
  return run_experts(c, layer, (const uint16_t*)x, T, ids, w, (uint16_t*)out, nullptr, (hipStream_t)stream, sc,
                     false);
}

// h_in: the first layer's input residual when it is not h (else null).
static moe_status moe_stack_forward_call(moe_ctx* c, int32_t layer_begin, int32_t layer_end, float* h, int32_t T,
                             const int32_t* forced_ids, void* x_trace, int32_t* ids_trace,
                             float* w_trace, void* stream, const float* h_in = nullptr) {
  if (moe_status st = check_ctx(c)) return st;
  const moe_config& g = c->cfg;
  if (layer_begin < 0 || layer_end > g.n_layers || layer_begin >= layer_end)
    return fail(c, MOE_E_ARG, "bad layer range");
  for (int l = layer_begin; l < layer_end; ++l)
    if (moe_status st = check_layer(c, l)) return st;
  if (!h) return fail(c, MOE_E_ARG, "h is required");
  if (T < 1 || T > g.max_tokens) return fail(c, MOE_E_ARG, "T out of range [1, max_tokens]");
  if (pooled(c) && !forced_ids) return fail(c, MOE_E_ARG, "a slot pool needs forced_ids");
  hipStream_t s = (hipStream_t)stream;
  const int64_t tk = (int64_t)T * g.top_k, th = (int64_t)T * g.hidden;
  if (fused_eligible(c, T)) {
    FusedArgs fa{};
    fa.layers = c->dlayers;
    fa.l0 = layer_begin;
    fa.l1 = layer_end;
    fa.T = T;
    fa.E = g.n_experts;
    fa.I = g.inter;
    fa.k = g.top_k;
    fa.renorm = g.renorm;
    fa.has_shared = g.shared_inter ? 1 : 0;
    fa.exact_always = (int)(g.flags & MOE_FLAG_ROUTER_EXACT_ALWAYS);
    fa.lay = c->lay;
    fa.blob_stride = c->lay.total();
    fa.lg_reps = T * g.n_experts <= 256 ? kFLogitReps : 1;
    {
      // split each logit over up to 4 waves while every wave of a replica
      // still has at most one item
      const int waves = (kFGrid / fa.lg_reps) * 8;
      fa.lg_sub = 1;
      while (fa.lg_sub < 4 && T * g.n_experts * fa.lg_sub * 2 <= waves) fa.lg_sub *= 2;
    }
    fa.h = h;
    fa.h_in = h_in;
    fa.xh = c->xh;
    fa.xlg = c->xlg;
    fa.xhb = c->xhb;
    fa.xgate = c->xgate;
    fa.epoch = c->epoch;
    fa.forced = forced_ids;
    fa.x_trace = (uint16_t*)x_trace;
    fa.ids_trace = ids_trace;
    fa.w_trace = w_trace;
    fa.err = c->err;
    fa.stamps = c->stamps;
    // one token over resident layers, routed by the router: the next layer's
    // guessed experts are loaded during the current layer
    const bool spec = (g.flags & MOE_FLAG_GUESS_AHEAD) && T == 1 && !forced_ids && !pooled(c) &&
                      spec_supported(g.hidden, g.inter, g.n_experts, g.top_k, g.shared_inter);
    if (spec) {
      fa.guess_mode = (g.flags & MOE_FLAG_TEST_GUESS_NONE)      ? 3
                      : (g.flags & MOE_FLAG_TEST_GUESS_LOWEST)  ? 1
                      : (g.flags & MOE_FLAG_TEST_GUESS_SHIFTED) ? 2
                                                                : 0;
      // one logit item (an exact logit, or a guess logit of the next layer)
      // per polling wave, 4 per block: one replica per XCD while each XCD
      // has a wave per item
      constexpr int kPollWaves = 4;
      const int items = fa.guess_mode == 3 ? g.n_experts : 2 * g.n_experts;
      fa.lg_reps = items <= (kFGrid / kFLogitReps) * kPollWaves ? kFLogitReps : 1;
      fa.lg_sub = 1;
    }
    {
      ScopedTimer tm(c, kKindFused, s);
      if (spec)
        launch_spec_decode(fa, s);
      else
        launch_fused_decode(fa, s);
    }
    HIPCHK(c, hipGetLastError());
    if (pooled(c))
      for (int l = layer_begin; l < layer_end; ++l) HIPCHK(c, hipEventRecord(c->layers[l].retired, s));
    return MOE_OK;
  }
  if (h_in) HIPCHK(c, hipMemcpyAsync(h, h_in, (size_t)th * sizeof(float), hipMemcpyDeviceToDevice, s));
  // after the first layer, the combine leaves the residual's sums of squares
  // and the matrix-core router's partial-logit kernel forms x itself (no
  // RMSNorm launch)
  const int exact_always = (int)(g.flags & MOE_FLAG_ROUTER_EXACT_ALWAYS);
  const bool norm_in_router = router_takes_mfma(g.hidden, g.n_experts, exact_always);
  const int nssq = (g.hidden + 1023) / 1024;
  for (int l = layer_begin; l < layer_end; ++l) {
    uint16_t* x = x_trace ? (uint16_t*)x_trace + l * th : c->xbuf;
    int32_t* ids = ids_trace ? ids_trace + l * tk : c->ids;
    float* w = w_trace ? w_trace + l * tk : c->w;
    const bool fused_norm = norm_in_router && l > layer_begin;
    if (!fused_norm) {
      ScopedTimer tm(c, kKindNorm, s);
      launch_rmsnorm(h, T, g.hidden, 1e-5f, x, s);
    }
    RouterArgs ra{x, c->layers[l].router, T, g.n_experts, g.hidden, g.top_k, g.renorm, c->logits,
                  forced_ids ? forced_ids + l * tk : nullptr, ids, w, c->err, exact_always};
    if (fused_norm) {
      ra.hres = h;
      ra.ssq = c->ssq;
      ra.nssq = nssq;
      ra.xw = x;
    }
    run_router(c, ra, s);
    if (moe_status st = run_experts(c, l, x, T, ids, w, nullptr, h, s, ctx_scratch(c), true,
                                    norm_in_router && l + 1 < layer_end ? c->ssq : nullptr))
      return st;
  }
  return MOE_OK;
}

moe_status moe_check_device_errors(moe_ctx* c, void* stream, uint32_t* bits) {
  if (!c) return MOE_E_ARG;
  HIPCHK(c, hipStreamSynchronize((hipStream_t)stream));
  uint32_t v = 0;
  const uint32_t zero = 0;
  HIPCHK(c, hipMemcpy(&v, c->err, 4, hipMemcpyDeviceToHost));
  HIPCHK(c, hipMemcpy(c->err, &zero, 4, hipMemcpyHostToDevice));
  if (bits) *bits = v;
  if (v) return fail(c, MOE_E_DEVICE, "device error word " + std::to_string(v));
  return MOE_OK;
}

static moe_status moe_cache_ensure_call(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n,
                            int32_t* slots, int32_t step, void* stream) {
  if (moe_status st = check_ctx(c)) return st;
  if (moe_status st = check_layer(c, layer)) return st;
  if (n < 0 || (n > 0 && (!experts || !slots))) return fail(c, MOE_E_ARG, "bad experts/slots");
  const moe_config& g = c->cfg;
  for (int i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= g.n_experts) return fail(c, MOE_E_ARG, "expert id out of range");
  if (!pooled(c)) {
    for (int i = 0; i < n; ++i) slots[i] = experts[i];
    return MOE_OK;
  }
  LayerState& L = c->layers[layer];
  if (n > g.slots_per_layer) return fail(c, MOE_E_CAPACITY, "routed group larger than the slot pool");
  hipStream_t s = (hipStream_t)stream;
  const PolicyEngine saved = *L.policy;
  std::vector<PolicyEngine::Decision> dec;
  const int rc = L.policy->access(experts, n, step, dec);
  if (rc == 1) return fail(c, MOE_E_ARG, "repeated expert in group");
  if (rc == 2) return fail(c, MOE_E_CAPACITY, "routed group larger than the slot pool");
  const int64_t blob = c->lay.total();
  int nmiss = 0, nevict = 0, nfirst = 0;
  for (const auto& d : dec) {
    if (!d.hit) {
      ++nmiss;
      if (d.victim >= 0) ++nevict;
    }
    if (d.kind == PolicyEngine::kPrefetchHit) ++nfirst;
  }
  // a prefetched copy is published on its first use, after its transfer
  // (ordered before any copy of this call is enqueued)
  if (nfirst > 0 && L.pf_recorded && hipStreamWaitEvent(s, L.pf_ready, 0) != hipSuccess) {
    (void)hipGetLastError();
    *L.policy = saved;
    L.stats.failures += 1;
    return fail(c, MOE_E_TRANSFER, "could not order the first use of a prefetched copy");
  }
  if (nmiss > 0) {
    // transport of the misses, then `stream` waits for all of them
    bool good = L.inject != 1;
    hipEvent_t t0 = nullptr, t1 = nullptr;
    good = good && hipEventCreate(&t0) == hipSuccess && hipEventCreate(&t1) == hipSuccess;
    RowState rows = save_rows(L);
    std::vector<PolicyEngine::Decision> fills;
    for (const auto& d : dec)
      if (!d.hit) fills.push_back(d);
    good = good && enqueue_fills(c, L, fills, s, t0, t1, L.ready);
    good = good && hipStreamWaitEvent(s, L.ready, 0) == hipSuccess;
    if (!good) {
      (void)hipGetLastError();
      if (t0) (void)hipEventDestroy(t0);
      if (t1) (void)hipEventDestroy(t1);
      restore_rows(L, std::move(rows));
      *L.policy = saved;  // the old generation stays authoritative
      L.inject = 0;
      L.stats.failures += 1;
      return fail(c, MOE_E_TRANSFER, "miss transfer failed before publication");
    }
    note_transfer(L, t0, t1);
  }
  if (nmiss > 0 || nfirst > 0) {
    // publication in stream order, after the copies
    PublishArgs pa{};
    pa.map = L.map;
    auto push = [&](int32_t e, int32_t slot) {
      if (pa.n == kMaxPublish) {
        launch_publish(pa, s);
        pa.n = 0;
      }
      pa.u[pa.n++] = PublishUpdate{e, slot};
    };
    for (const auto& d : dec) {
      if (d.kind == PolicyEngine::kPrefetchHit) push(d.expert, row_of(L, d.slot));
      if (d.hit) continue;
      if (d.victim >= 0) push(d.victim, -1);
      push(d.expert, row_of(L, d.slot));
    }
    if (pa.n) launch_publish(pa, s);
    if (hipGetLastError() != hipSuccess || (nmiss > 0 && L.inject == 2)) {
      c->faulted = true;
      L.inject = 0;
      L.stats.failures += 1;
      return fail(c, MOE_E_FAULTED, "failure after publication: context faulted");
    }
  }
  L.stats.accesses += n;
  L.stats.hits += n - nmiss;
  L.stats.misses += nmiss;
  L.stats.evictions += nevict;
  L.stats.h2d_bytes += (uint64_t)nmiss * blob;
  L.stats.prefetch_used += nfirst;
  for (int i = 0; i < n; ++i) slots[i] = L.policy->slot_of(experts[i]);
  return MOE_OK;
}

static moe_status moe_cache_prefetch_call(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n, int32_t step,
                              void* stream) {
  if (moe_status st = check_ctx(c)) return st;
  if (moe_status st = check_layer(c, layer)) return st;
  if (n < 0 || (n > 0 && !experts)) return fail(c, MOE_E_ARG, "bad experts");
  const moe_config& g = c->cfg;
  for (int i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= g.n_experts) return fail(c, MOE_E_ARG, "expert id out of range");
  if (!pooled(c)) return MOE_OK;
  LayerState& L = c->layers[layer];
  if (n > g.slots_per_layer) return fail(c, MOE_E_CAPACITY, "guessed group larger than the slot pool");
  hipStream_t s = (hipStream_t)stream;
  const PolicyEngine saved = *L.policy;
  std::vector<PolicyEngine::Decision> dec;
  const int rc = L.policy->prefetch(experts, n, step, dec);
  if (rc == 1) return fail(c, MOE_E_ARG, "repeated expert in guessed group");
  if (rc == 2) return fail(c, MOE_E_CAPACITY, "guessed group larger than the slot pool");
  if (dec.empty()) return MOE_OK;
  const int64_t blob = c->lay.total();
  // transport only: nothing is published until an ensure() names the expert
  bool good = L.inject != 1;
  hipEvent_t t0 = nullptr, t1 = nullptr;
  good = good && hipEventCreate(&t0) == hipSuccess && hipEventCreate(&t1) == hipSuccess;
  RowState rows = save_rows(L);
  good = good && enqueue_fills(c, L, dec, s, t0, t1, L.pf_ready);
  if (!good) {
    (void)hipGetLastError();
    if (t0) (void)hipEventDestroy(t0);
    if (t1) (void)hipEventDestroy(t1);
    restore_rows(L, std::move(rows));
    *L.policy = saved;
    L.inject = 0;
    L.stats.failures += 1;
    return fail(c, MOE_E_TRANSFER, "prefetch transfer failed; nothing was published");
  }
  L.pf_recorded = true;
  note_transfer(L, t0, t1);
  // the victims' old copies are being overwritten: their map entries go to -1
  // in `stream` order, so no later kernel can read a victim through a stale map
  PublishArgs pa{};
  pa.map = L.map;
  int nevict = 0;
  for (const auto& d : dec) {
    if (d.victim < 0) continue;
    ++nevict;
    if (pa.n == kMaxPublish) {
      launch_publish(pa, s);
      pa.n = 0;
    }
    pa.u[pa.n++] = PublishUpdate{d.victim, -1};
  }
  if (pa.n) launch_publish(pa, s);
  if (hipGetLastError() != hipSuccess) {
    c->faulted = true;
    L.stats.failures += 1;
    return fail(c, MOE_E_FAULTED, "failure after a prefetch was enqueued: context faulted");
  }
  L.stats.prefetches += dec.size();
  L.stats.evictions += nevict;
  L.stats.h2d_bytes += (uint64_t)dec.size() * blob;
  return MOE_OK;
}

static moe_status moe_cache_pin_call(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n, int32_t step,
                         void* stream) {
  if (moe_status st = check_ctx(c)) return st;
  if (moe_status st = check_layer(c, layer)) return st;
  if (n < 0 || (n > 0 && !experts)) return fail(c, MOE_E_ARG, "bad experts");
  const moe_config& g = c->cfg;
  for (int i = 0; i < n; ++i)
    if (experts[i] < 0 || experts[i] >= g.n_experts) return fail(c, MOE_E_ARG, "expert id out of range");
  if (!pooled(c)) return MOE_OK;
  LayerState& L = c->layers[layer];
  hipStream_t s = (hipStream_t)stream;
  const PolicyEngine saved = *L.policy;
  std::vector<PolicyEngine::Decision> dec;
  const int rc = L.policy->pin(experts, n, step, dec);
  if (rc == 2) return fail(c, MOE_E_CAPACITY, "a hot set must leave at least one dynamic slot");
  if (rc == 3) return fail(c, MOE_E_ARG, "a hot set is pinned on a cold pool only");
  if (rc != 0) return fail(c, MOE_E_ARG, "repeated expert in hot set");
  if (dec.empty()) return MOE_OK;
  const int64_t blob = c->lay.total();
  bool good = true;
  hipEvent_t t0 = nullptr, t1 = nullptr;
  good = good && hipEventCreate(&t0) == hipSuccess && hipEventCreate(&t1) == hipSuccess;
  RowState rows = save_rows(L);
  good = good && enqueue_fills(c, L, dec, s, t0, t1, L.ready);
  good = good && hipStreamWaitEvent(s, L.ready, 0) == hipSuccess;
  if (!good) {
    (void)hipGetLastError();
    if (t0) (void)hipEventDestroy(t0);
    if (t1) (void)hipEventDestroy(t1);
    restore_rows(L, std::move(rows));
    *L.policy = saved;
    L.stats.failures += 1;
    return fail(c, MOE_E_TRANSFER, "hot-set transfer failed; nothing was published");
  }
  note_transfer(L, t0, t1);
  PublishArgs pa{};
  pa.map = L.map;
  for (const auto& d : dec) {
    if (pa.n == kMaxPublish) {
      launch_publish(pa, s);
      pa.n = 0;
    }
    pa.u[pa.n++] = PublishUpdate{d.expert, row_of(L, d.slot)};
  }
  if (pa.n) launch_publish(pa, s);
  if (hipGetLastError() != hipSuccess) {
    c->faulted = true;
    L.stats.failures += 1;
    return fail(c, MOE_E_FAULTED, "failure after a hot set was published: context faulted");
  }
  L.stats.pinned += dec.size();
  L.stats.h2d_bytes += (uint64_t)dec.size() * blob;
  return MOE_OK;
}

static moe_status moe_stack_forward_pooled_call(moe_ctx* c, int32_t layer_begin, int32_t layer_end, float* h, int32_t T,
                                    int32_t prefetch, int32_t step, int32_t* ids_trace, int32_t* guess_trace,
                                    void* stream) {
  if (moe_status st = check_ctx(c)) return st;
  const moe_config& g = c->cfg;
  if (!pooled(c)) return fail(c, MOE_E_ARG, "moe_stack_forward_pooled needs a slot pool");
  if (!h || T < 1 || T > g.max_tokens) return fail(c, MOE_E_ARG, "bad h/T");
  if (layer_begin < 0 || layer_end > g.n_layers || layer_begin >= layer_end)
    return fail(c, MOE_E_ARG, "bad layer range");
  for (int l = layer_begin; l < layer_end; ++l)
    if (moe_status st = check_layer(c, l)) return st;
  hipStream_t s = (hipStream_t)stream;
  const int k = g.top_k, P = T * k;
  int32_t* ids_h = c->pool_ids_h;
  int32_t* gids_h = c->pool_ids_h + (int64_t)g.max_tokens * k;
  // distinct ids of tokens [t0, t1), ascending
  auto group_of = [&](const int32_t* v, int t0, int t1, std::vector<int32_t>& grp) {
    grp.assign(v + (int64_t)t0 * k, v + (int64_t)t1 * k);
    std::sort(grp.begin(), grp.end());
    grp.erase(std::unique(grp.begin(), grp.end()), grp.end());
  };
  std::vector<int32_t> grp, next, guess, slots;
  for (int l = layer_begin; l < layer_end; ++l) {
    int32_t* ids_l = c->pool_ids + (int64_t)l * P;  // forced ids of the layer call: [L, T, k]
    const bool guess_next = prefetch && l + 1 < layer_end;
    if (moe_status st = moe_rmsnorm(c, h, T, c->pool_x, stream)) return st;
    if (moe_status st = moe_route(c, l, c->pool_x, T, nullptr, ids_l, c->pool_w, nullptr, stream)) return st;
    // the next layer's router on the current state guesses its experts
    if (guess_next)
      if (moe_status st = moe_route(c, l + 1, c->pool_x, T, nullptr, c->pool_gids, c->pool_w, nullptr, stream))
        return st;
    if (ids_trace) HIPCHK(c, hipMemcpyAsync(ids_trace + (int64_t)l * P, ids_l, (size_t)P * 4, hipMemcpyDeviceToDevice, s));
    if (guess_next && guess_trace)
      HIPCHK(c, hipMemcpyAsync(guess_trace + (int64_t)(l + 1) * P, c->pool_gids, (size_t)P * 4,
                               hipMemcpyDeviceToDevice, s));
    HIPCHK(c, hipMemcpyAsync(ids_h, ids_l, (size_t)P * 4, hipMemcpyDeviceToHost, s));
    if (guess_next) HIPCHK(c, hipMemcpyAsync(gids_h, c->pool_gids, (size_t)P * 4, hipMemcpyDeviceToHost, s));
    HIPCHK(c, hipStreamSynchronize(s));
    const PolicyEngine& eng = *c->layers[l].policy;
    const int dyn = g.slots_per_layer - eng.pinned_count();  // slots outside the hot set
    auto outside = [&](const std::vector<int32_t>& v) {
      int n = 0;
      for (int e : v) n += eng.is_pinned(e) ? 0 : 1;
      return n;
    };
    auto do_prefetch = [&]() -> moe_status {
      if (!guess_next) return MOE_OK;
      group_of(gids_h, 0, T, guess);
      // a guess that does not fit the pool's dynamic slots is not prefetched
      // (the engine is left unchanged by that refusal)
      if ((int32_t)guess.size() > g.slots_per_layer) return MOE_OK;
      const moe_status st = moe_cache_prefetch(c, l + 1, guess.data(), (int32_t)guess.size(), step, stream);
      return st == MOE_E_CAPACITY ? MOE_OK : st;
    };
    group_of(ids_h, 0, T, grp);
    if (outside(grp) <= dyn) {
      slots.resize(grp.size());
      if (moe_status st = moe_cache_ensure(c, l, grp.data(), (int32_t)grp.size(), slots.data(), step, stream))
        return st;
      if (moe_status st = do_prefetch()) return st;
      // the layer itself, routed by the ids just read (the same router, the same x)
      if (moe_status st = moe_stack_forward(c, l, l + 1, h, T, c->pool_ids, nullptr, nullptr, nullptr, stream))
        return st;
      continue;
    }
    // The batch's routed group does not fit the slots outside the hot set: the
    // layer runs over contiguous token chunks, each the longest run from its
    // first token whose group fits, one after another (each chunk's group is
    // ensured, then computed, so a later chunk may evict an expert only after
    // the earlier chunk that read it has retired).
    if (moe_status st = do_prefetch()) return st;
    for (int t0 = 0; t0 < T;) {
      int t1 = t0 + 1;
      group_of(ids_h, t0, t1, grp);
      if (outside(grp) > dyn)
        return fail(c, MOE_E_CAPACITY, "one token's experts exceed the pool's slots outside the hot set");
      while (t1 < T) {
        group_of(ids_h, t0, t1 + 1, next);
        if (outside(next) > dyn) break;
        grp.swap(next);
        ++t1;
      }
      slots.resize(grp.size());
      if (moe_status st = moe_cache_ensure(c, l, grp.data(), (int32_t)grp.size(), slots.data(), step, stream))
        return st;
      const int Tc = t1 - t0;
      int32_t* cids = c->pool_cids + (int64_t)l * Tc * k;  // forced ids of the chunk call: [L, Tc, k]
      HIPCHK(c, hipMemcpyAsync(cids, ids_l + (int64_t)t0 * k, (size_t)Tc * k * 4, hipMemcpyDeviceToDevice, s));
      if (moe_status st = moe_stack_forward(c, l, l + 1, h + (int64_t)t0 * g.hidden, Tc, c->pool_cids, nullptr,
                                            nullptr, nullptr, stream))
        return st;
      t0 = t1;
    }
  }
  return MOE_OK;
}

static moe_status moe_rmsnorm_call(moe_ctx* c, const float* h, int32_t T, void* x, void* stream) {
  if (moe_status st = check_ctx(c)) return st;
  if (!h || !x || T < 1 || T > c->cfg.max_tokens) return fail(c, MOE_E_ARG, "bad h/x/T");
  launch_rmsnorm(h, T, c->cfg.hidden, 1e-5f, reinterpret_cast<uint16_t*>(x), (hipStream_t)stream);
  HIPCHK(c, hipGetLastError());
  return MOE_OK;
}

moe_status moe_cache_stats(moe_ctx* c, int32_t layer, moe_cache_counters* out) {
  if (!c || !out) return MOE_E_ARG;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, MOE_E_ARG, "layer index out of range");
  LayerState& L = c->layers[layer];
  for (auto& p : L.timing) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.second) == hipSuccess && hipEventElapsedTime(&ms, p.first, p.second) == hipSuccess)
      L.stats.h2d_seconds += ms * 1e-3;
    (void)hipEventDestroy(p.first);
    (void)hipEventDestroy(p.second);
  }
  L.timing.clear();
  *out = L.stats;
  return MOE_OK;
}

moe_status moe_cache_event_log(const moe_ctx* c, int32_t layer, moe_cache_event* buf, int32_t cap,
                               int32_t* n) {
  if (!c || !n) return MOE_E_ARG;
  if (layer < 0 || layer >= c->cfg.n_layers) return MOE_E_ARG;
  const LayerState& L = c->layers[layer];
  *n = 0;
  if (!L.policy) return MOE_OK;
  const auto& lg = L.policy->log();
  const int32_t m = std::min<int32_t>(cap < 0 ? 0 : cap, (int32_t)lg.size());
  if (m > 0 && !buf) return MOE_E_ARG;
  for (int32_t i = 0; i < m; ++i) buf[i] = lg[i];
  *n = m;
  return MOE_OK;
}

moe_status moe_timer_enable(moe_ctx* c, int32_t kind) {
  if (!c) return MOE_E_ARG;
  if (kind < -1 || kind > kKindMfmaDown) return fail(c, MOE_E_ARG, "unknown kernel kind");
  c->timer_kind = kind;
  return MOE_OK;
}

moe_status moe_timer_read(moe_ctx* c, double* total_ms, int64_t* launches) {
  if (!c || !total_ms || !launches) return MOE_E_ARG;
  double tot = 0.0;
  for (size_t i = 0; i < c->timer_used; ++i) {
    auto& p = c->timer_events[i];
    HIPCHK(c, hipEventSynchronize(p.second));
    float ms = 0.0f;
    HIPCHK(c, hipEventElapsedTime(&ms, p.first, p.second));
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int64_t)c->timer_used;
  c->timer_used = 0;
  return MOE_OK;
}

moe_status moe_fused_phase_stamps(moe_ctx* c, uint64_t* dev_buf, int64_t count, int32_t* grid,
                                  int32_t* stride, int32_t* per_layer) {
  if (!c) return MOE_E_ARG;
  if (dev_buf && count < 2 * (int64_t)kFGrid * kStampStride)
    return fail(c, MOE_E_ARG, "stamp buffer smaller than 2 * grid * stride");
  c->stamps = dev_buf;
  if (grid) *grid = kFGrid;
  if (stride) *stride = kStampStride;
  if (per_layer) *per_layer = kStampsPerLayer;
  return MOE_OK;
}

moe_status moe_debug_inject_transfer_failure(moe_ctx* c, int32_t layer, int32_t mode) {
  if (!c) return MOE_E_ARG;
  if (layer < 0 || layer >= c->cfg.n_layers || mode < 0 || mode > 2)
    return fail(c, MOE_E_ARG, "bad layer or mode");
  c->layers[layer].inject = mode;
  return MOE_OK;
}

// Every call that enqueues GPU work: on a pooled context it first waits for
// the previous such call (pool_order_begin) and records its own end after its
// work (pool_order_end).
// MOE_SYNC_EACH_CALL=1: every call that enqueues GPU work waits for its
// stream and the side stream and reads the device error word, so that an
// asynchronous error is reported by the call that caused it.
moe_status sync_each_call(moe_ctx* c, void* stream, moe_status st, const char* what) {
  if (st != MOE_OK || !c || !c->sync_each) return st;
  HIPCHK(c, hipStreamSynchronize((hipStream_t)stream));
  if (c->side) HIPCHK(c, hipStreamSynchronize(c->side));
  uint32_t v = 0;
  HIPCHK(c, hipMemcpy(&v, c->err, 4, hipMemcpyDeviceToHost));
  if (v)
    return fail(c, MOE_E_DEVICE, std::string(what) + ": device error word " + std::to_string(v) +
                                     " (MOE_SYNC_EACH_CALL; moe_check_device_errors clears it)");
  return MOE_OK;
}

moe_status moe_route(moe_ctx* c, int32_t layer, const void* x, int32_t T, const int32_t* forced_ids,
                     int32_t* ids, float* w, float* logits, void* stream) {
  if (c && !c->faulted)
    if (moe_status st = pool_order_begin(c, (hipStream_t)stream)) return st;
  moe_status st = moe_route_call(c, layer, x, T, forced_ids, ids, w, logits, stream);
  if (st == MOE_OK && c) st = pool_order_end(c, (hipStream_t)stream);
  return sync_each_call(c, stream, st, "moe_route");
}

moe_status moe_expert_forward(moe_ctx* c, int32_t layer, const void* x, int32_t T, const int32_t* ids,
                              const float* w, void* out, void* stream) {
  if (c && !c->faulted)
    if (moe_status st = pool_order_begin(c, (hipStream_t)stream)) return st;
  moe_status st = moe_expert_forward_call(c, layer, x, T, ids, w, out, stream);
  if (st == MOE_OK && c) st = pool_order_end(c, (hipStream_t)stream);
  return sync_each_call(c, stream, st, "moe_expert_forward");
}

moe_status moe_expert_forward_noalloc(moe_ctx* c, int32_t layer, const void* x, int32_t T, const int32_t* ids,
                                      const float* w, void* out, void* stream) {
  if (c && !c->faulted)
    if (moe_status st = pool_order_begin(c, (hipStream_t)stream)) return st;
  moe_status st = moe_expert_forward_noalloc_call(c, layer, x, T, ids, w, out, stream);
  if (st == MOE_OK && c) st = pool_order_end(c, (hipStream_t)stream);
  return sync_each_call(c, stream, st, "moe_expert_forward_noalloc");
}

moe_status moe_stack_forward(moe_ctx* c, int32_t layer_begin, int32_t layer_end, float* h, int32_t T,
                             const int32_t* forced_ids, void* x_trace, int32_t* ids_trace,
                             float* w_trace, void* stream) {
  if (c && !c->faulted)
    if (moe_status st = pool_order_begin(c, (hipStream_t)stream)) return st;
  moe_status st = moe_stack_forward_call(c, layer_begin, layer_end, h, T, forced_ids, x_trace, ids_trace, w_trace, stream);
  if (st == MOE_OK && c) st = pool_order_end(c, (hipStream_t)stream);
  return sync_each_call(c, stream, st, "moe_stack_forward");
}

moe_status moe_stack_forward_into(moe_ctx* c, int32_t layer_begin, int32_t layer_end, const float* h_in,
                                  float* h, int32_t T, const int32_t* forced_ids, void* x_trace,
                                  int32_t* ids_trace, float* w_trace, void* stream) {
  if (!h_in) return c ? fail(c, MOE_E_ARG, "h_in is required") : MOE_E_ARG;
  if (c && !c->faulted) {
    if (h_in != h && c->cfg.hidden > 0 && T > 0) {
      const uintptr_t a0 = (uintptr_t)h_in, b0 = (uintptr_t)h;
      const uintptr_t n = (uintptr_t)T * (uintptr_t)c->cfg.hidden * sizeof(float);
      if (a0 < b0 + n && b0 < a0 + n) return fail(c, MOE_E_ARG, "h_in and h overlap without being equal");
    }
    if (moe_status st = pool_order_begin(c, (hipStream_t)stream)) return st;
  }
  moe_status st = moe_stack_forward_call(c, layer_begin, layer_end, h, T, forced_ids, x_trace, ids_trace, w_trace,
                                         stream, h_in == h ? nullptr : h_in);
  if (st == MOE_OK && c) st = pool_order_end(c, (hipStream_t)stream);
  return sync_each_call(c, stream, st, "moe_stack_forward_into");
}

moe_status moe_cache_ensure(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n,
                            int32_t* slots, int32_t step, void* stream) {
  if (c && !c->faulted)
    if (moe_status st = pool_order_begin(c, (hipStream_t)stream)) return st;
  moe_status st = moe_cache_ensure_call(c, layer, experts, n, slots, step, stream);
  if (st == MOE_OK && c) st = pool_order_end(c, (hipStream_t)stream);
  return sync_each_call(c, stream, st, "moe_cache_ensure");
}

moe_status moe_cache_prefetch(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n, int32_t step,
                              void* stream) {
  if (c && !c->faulted)
    if (moe_status st = pool_order_begin(c, (hipStream_t)stream)) return st;
  moe_status st = moe_cache_prefetch_call(c, layer, experts, n, step, stream);
  if (st == MOE_OK && c) st = pool_order_end(c, (hipStream_t)stream);
  return sync_each_call(c, stream, st, "moe_cache_prefetch");
}

moe_status moe_cache_pin(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n, int32_t step,
                         void* stream) {
  if (c && !c->faulted)
    if (moe_status st = pool_order_begin(c, (hipStream_t)stream)) return st;
  moe_status st = moe_cache_pin_call(c, layer, experts, n, step, stream);
  if (st == MOE_OK && c) st = pool_order_end(c, (hipStream_t)stream);
  return sync_each_call(c, stream, st, "moe_cache_pin");
}

moe_status moe_stack_forward_pooled(moe_ctx* c, int32_t layer_begin, int32_t layer_end, float* h, int32_t T,
                                    int32_t prefetch, int32_t step, int32_t* ids_trace, int32_t* guess_trace,
                                    void* stream) {
  if (c && !c->faulted)
    if (moe_status st = pool_order_begin(c, (hipStream_t)stream)) return st;
  moe_status st = moe_stack_forward_pooled_call(c, layer_begin, layer_end, h, T, prefetch, step, ids_trace, guess_trace, stream);
  if (st == MOE_OK && c) st = pool_order_end(c, (hipStream_t)stream);
  return sync_each_call(c, stream, st, "moe_stack_forward_pooled");
}

moe_status moe_rmsnorm(moe_ctx* c, const float* h, int32_t T, void* x, void* stream) {
  if (c && !c->faulted)
    if (moe_status st = pool_order_begin(c, (hipStream_t)stream)) return st;
  moe_status st = moe_rmsnorm_call(c, h, T, x, stream);
  if (st == MOE_OK && c) st = pool_order_end(c, (hipStream_t)stream);
  return sync_each_call(c, stream, st, "moe_rmsnorm");
}

moe_status moe_debug_delay_copies(moe_ctx* c, int32_t microseconds) {
  if (!c) return MOE_E_ARG;
  if (microseconds < 0 || microseconds > MOE_MAX_COPY_DELAY_US)
    return fail(c, MOE_E_ARG, "the copy delay must be in [0, " + std::to_string(MOE_MAX_COPY_DELAY_US) + "] microseconds");
  c->copy_delay_us = microseconds;
  return MOE_OK;
}

}  // extern "C"
