// C-ABI of libmoba: argument checks, workspace layout and the launch sequence
// (pool -> gate/top-k -> query lists -> block attention -> merge). Every entry
// point only enqueues on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/moba.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;
std::atomic<int> g_poison_workspace{0};   // moba_debug_poison_workspace

constexpr int kMaxDevices = 64;

struct DeviceState {
  std::once_flag once;
  hipError_t init_error = hipSuccess;
  bool gfx950 = false;
  int num_cus = 0;
  int device = 0;
  std::once_flag pool_once;   // the workspace pool is created on the first call that needs one
  hipError_t pool_error = hipSuccess;
  hipMemPool_t pool = nullptr;
};

DeviceState g_devices[kMaxDevices];

int hip_fail(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return MOBA_ERR_HIP;
}

void init_device(int dev, DeviceState* st) {
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    st->init_error = e;
    return;
  }
  st->gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  st->num_cus = prop.multiProcessorCount;
  st->device = dev;
}

void init_pool(DeviceState* st) {
  hipMemPoolProps props;
  std::memset(&props, 0, sizeof(props));
  props.allocType = hipMemAllocationTypePinned;
  props.handleTypes = hipMemHandleTypeNone;
  props.location.type = hipMemLocationTypeDevice;
  props.location.id = st->device;
  hipError_t e = hipMemPoolCreate(&st->pool, &props);
  if (e != hipSuccess) {
    st->pool_error = e;
    return;
  }
  uint64_t keep = ~0ull;  // keep freed workspace in the pool across calls
  e = hipMemPoolSetAttribute(st->pool, hipMemPoolAttrReleaseThreshold, &keep);
  if (e != hipSuccess) st->pool_error = e;
}

// Resolves the current device; returns a moba status.
int current_device(DeviceState** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return MOBA_ERR_UNSUPPORTED;
  DeviceState* st = &g_devices[dev];
  std::call_once(st->once, init_device, dev, st);
  if (st->init_error != hipSuccess) return hip_fail(st->init_error);
  if (!st->gfx950) return MOBA_ERR_UNSUPPORTED;
  *out = st;
  return MOBA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point (no HIP calls).
int check_shape(int64_t N, int32_t H, int32_t D, int32_t B) {
  if (N < 1 || H < 1 || B < 1) return MOBA_ERR_INVALID_ARG;
  if (N % B != 0) return MOBA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return MOBA_ERR_UNSUPPORTED;
  if (B % 64 != 0) return MOBA_ERR_UNSUPPORTED;
  if (N >= (int64_t{1} << 28)) return MOBA_ERR_UNSUPPORTED;
  if (N / B > MOBA_MAX_BLOCKS) return MOBA_ERR_UNSUPPORTED;
  if (H > 65535) return MOBA_ERR_UNSUPPORTED;
  return MOBA_OK;
}

// The dense causal path of the bf16 prefill and backward: every query keeps
// every block (top_k >= n, n > 1).
bool dense_path(int64_t N, int32_t B, int32_t topk, bool is_f32) {
  return !is_f32 && N / B > 1 && topk >= N / B;
}

int check_topk(int64_t N, int32_t B, int32_t topk) {
  if (topk < 1) return MOBA_ERR_INVALID_ARG;
  const int64_t n = N / B;
  if (topk > MOBA_MAX_TOPK && topk < n) return MOBA_ERR_UNSUPPORTED;
  return MOBA_OK;
}

moba::Problem make_problem(int64_t N, int32_t H, int32_t D, int32_t B, int32_t topk, bool is_f32) {
  moba::Problem p;
  p.N = N;
  p.H = H;
  p.D = D;
  p.B = B;
  p.n = static_cast<int>(N / B);
  // A query of block j keeps min(topk, j + 1) <= n blocks: a larger topk
  // selects the same blocks as topk = n, so the internal selection rows are n
  // wide at most (moba_gate_topk still fills the caller's topk-wide rows).
  p.topk = static_cast<int>(std::min<int64_t>(topk, p.n));
  p.lmax = static_cast<int>(std::min<int64_t>(topk - 1, p.n - 1));
  p.ntiles = static_cast<int>((N + moba::kQTile - 1) / moba::kQTile);
  int64_t pairs_per_head = 0;  // sum over blocks j of B * min(topk - 1, j)
  for (int j = 0; j < p.n; ++j) pairs_per_head += static_cast<int64_t>(B) * std::min(topk - 1, j);
  p.p_off = pairs_per_head * H;
  p.max_items = p.p_off / moba::kAttnTile + static_cast<int64_t>(H) * p.n;
  p.diag_items = static_cast<int64_t>(H) * p.n * ((B + moba::kAttnTile - 1) / moba::kAttnTile);
  p.is_f32 = is_f32;
  return p;
}

struct Layout {
  size_t total = 0;
  size_t add(size_t bytes) {
    const size_t o = total;
    total += (bytes + 255) & ~size_t{255};
    return o;
  }
};

// Workspace offsets for the requested stages.
struct WsPlan {
  size_t kbar, kpieces, cnt, totals, offs, istart, rk, qidx, inv, items, counters, part_diag, lse_diag, part_off,
      lse_off, sel, delta, part_dq, blo;
  size_t total;
};

// What a call runs after the gate: nothing (gate only), the query lists
// alone, the lists and the forward partials, or the lists and the backward's
// Delta and dQ partials.
enum class Stages { gate, lists, forward, backward };

// Workspace offsets for the requested stages. With Stages::lists the caller
// owns sel, offs and qidx, so the workspace holds none of them.
WsPlan plan(const moba::Problem& p, Stages stages, bool packed = false) {
  Layout L;
  WsPlan w;
  std::memset(&w, 0, sizeof(w));
  const int64_t hn = static_cast<int64_t>(p.H) * p.n;
  const int64_t hN = static_cast<int64_t>(p.H) * p.N;
  const size_t es = p.is_f32 ? 4 : 2;
  const bool own_lists = stages != Stages::lists;
  w.kbar = L.add(hn * p.D * 4);
  w.kpieces = L.add(p.is_f32 ? 0 : hn * 3 * p.D * 2);
  if (stages != Stages::gate) {
    w.cnt = L.add(hn * p.ntiles * 4);
    w.totals = L.add(hn * 4);
    w.offs = L.add(own_lists ? (hn + 1) * 4 : 0);   // list starts, then the total
    w.istart = L.add(hn * 4);
    w.rk = L.add(hN * p.lmax * 4);
    w.qidx = L.add(own_lists ? p.p_off * 4 : 0);
    w.inv = L.add(hN * p.lmax * 4);
    w.items = L.add(p.max_items * sizeof(moba::WorkItem));
    w.counters = L.add(moba::kCounterInts * 4);
    if (stages == Stages::forward) {
      // With the merge fused into the own-block pass there are no own-block partials.
      const bool fused = moba::merge_fused(p);
      w.part_diag = L.add(fused ? 0 : (hN + moba::kDumpRows) * p.D * es);
      w.lse_diag = L.add(fused ? 0 : (hN + moba::kDumpRows) * 4);
      w.part_off = L.add((p.p_off + moba::kDumpRows) * p.D * es);
      w.lse_off = L.add((p.p_off + moba::kDumpRows) * 4);
    } else if (stages == Stages::backward) {
      w.delta = L.add(hN * 4);
      w.part_dq = L.add(p.p_off * p.D * 4);
    }
    w.sel = L.add(own_lists ? hN * p.topk * 4 : 0);
  }
  if (packed) w.blo = L.add(static_cast<size_t>(p.n) * 4);
  w.total = L.total;
  return w;
}

moba::Workspace bind(const WsPlan& w, char* base, bool full) {
  moba::Workspace ws;
  std::memset(&ws, 0, sizeof(ws));
  ws.kbar = reinterpret_cast<float*>(base + w.kbar);
  ws.kpieces = reinterpret_cast<moba::bf16*>(base + w.kpieces);
  if (full) {
    ws.cnt = reinterpret_cast<int32_t*>(base + w.cnt);
    ws.totals = reinterpret_cast<int32_t*>(base + w.totals);
    ws.offs = reinterpret_cast<int32_t*>(base + w.offs);
    ws.istart = reinterpret_cast<int32_t*>(base + w.istart);
    ws.rk = reinterpret_cast<int32_t*>(base + w.rk);
    ws.qidx = reinterpret_cast<int32_t*>(base + w.qidx);
    ws.inv = reinterpret_cast<int32_t*>(base + w.inv);
    ws.items = reinterpret_cast<moba::WorkItem*>(base + w.items);
    ws.counters = reinterpret_cast<int32_t*>(base + w.counters);
    ws.part_diag = base + w.part_diag;
    ws.lse_diag = reinterpret_cast<float*>(base + w.lse_diag);
    ws.part_off = base + w.part_off;
    ws.lse_off = reinterpret_cast<float*>(base + w.lse_off);
    ws.sel = reinterpret_cast<int32_t*>(base + w.sel);
  }
  return ws;
}

int alloc_ws(DeviceState* st, size_t bytes, hipStream_t stream, char** out) {
  // A stream under capture would record the pool allocation and its free as
  // graph memory nodes, which the allocating calls do not support: they
  // refuse capture before anything is enqueued. (The allocation-free decode
  // step takes its workspace from a fixed device array instead.)
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  const hipError_t ce = hipStreamIsCapturing(stream, &capture);
  if (ce != hipSuccess) return hip_fail(ce);
  if (capture != hipStreamCaptureStatusNone) return MOBA_ERR_UNSUPPORTED;
  std::call_once(st->pool_once, init_pool, st);
  if (st->pool_error != hipSuccess) return hip_fail(st->pool_error);
  void* p = nullptr;
  hipError_t e = hipMallocFromPoolAsync(&p, bytes ? bytes : 256, st->pool, stream);
  if (e == hipErrorOutOfMemory) {
    (void)hipGetLastError();
    return MOBA_ERR_OUT_OF_MEMORY;
  }
  if (e != hipSuccess) return hip_fail(e);
  *out = static_cast<char*>(p);
  if (g_poison_workspace.load(std::memory_order_relaxed) != 0) {
    // Layout rounds every piece to 256 bytes, so the total is a multiple of 16.
    e = moba::launch_fill(p, bytes, 0xFFFFFFFFu, stream);
    if (e != hipSuccess) {
      (void)hipFreeAsync(p, stream);
      return hip_fail(e);
    }
  }
  return MOBA_OK;
}

int finish(hipError_t launch_error, char* ws, hipStream_t stream) {
  hipError_t fe = hipFreeAsync(ws, stream);
  if (launch_error != hipSuccess) return hip_fail(launch_error);
  if (fe != hipSuccess) return hip_fail(fe);
  return MOBA_OK;
}

// Block pooling of the gate's keys: a MOBA_POOL_* mode and, for the weighted
// mode, the caller's [H][N] fp32 weights.
struct Pooling {
  int mode = MOBA_POOL_MEAN;
  const float* weights = nullptr;
};

int check_pooling(const Pooling& pl) {
  if (pl.mode != MOBA_POOL_MEAN && pl.mode != MOBA_POOL_MAX && pl.mode != MOBA_POOL_WEIGHTED)
    return MOBA_ERR_INVALID_ARG;
  if (pl.mode == MOBA_POOL_WEIGHTED && pl.weights == nullptr) return MOBA_ERR_INVALID_ARG;
  if (pl.mode == MOBA_POOL_WEIGHTED && reinterpret_cast<uintptr_t>(pl.weights) % 4 != 0) return MOBA_ERR_UNSUPPORTED;
  return MOBA_OK;
}

// Several sequences packed along N, each a whole number of blocks.
struct Packed {
  moba::SeqStarts st;          // block-unit starts (passed by value to the table kernel)
  int max_blocks = 0;          // blocks of the longest sequence
  int64_t pairs_per_head = 0;  // sum over sequences and their blocks jj of B * min(topk - 1, jj)
};

// Validates the host array cu_seqlens[0..num_seqs] (token offsets: 0, then
// non-decreasing, every length a multiple of B) and fills `pk` and the total
// token count.
int parse_packed(const int64_t* cu, int32_t num_seqs, int32_t B, int32_t topk, Packed* pk, int64_t* total) {
  if (cu == nullptr || num_seqs < 1 || B < 1 || topk < 1) return MOBA_ERR_INVALID_ARG;
  if (num_seqs > moba::kMaxSeqs) return MOBA_ERR_UNSUPPORTED;
  if (cu[0] != 0) return MOBA_ERR_INVALID_ARG;
  pk->st.nseq = num_seqs;
  pk->max_blocks = 0;
  pk->pairs_per_head = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t len = cu[s + 1] - cu[s];
    if (len < 0 || len % B != 0) return MOBA_ERR_INVALID_ARG;
    if (cu[s + 1] >= (int64_t{1} << 28)) return MOBA_ERR_UNSUPPORTED;
    const int nb = static_cast<int>(len / B);
    pk->st.start[s] = static_cast<int32_t>(cu[s] / B);
    pk->max_blocks = std::max(pk->max_blocks, nb);
    for (int jj = 0; jj < nb; ++jj) pk->pairs_per_head += static_cast<int64_t>(B) * std::min(topk - 1, jj);
  }
  pk->st.start[num_seqs] = static_cast<int32_t>(cu[num_seqs] / B);
  *total = cu[num_seqs];
  if (*total < 1) return MOBA_ERR_INVALID_ARG;
  if (topk > MOBA_MAX_TOPK && topk < pk->max_blocks) return MOBA_ERR_UNSUPPORTED;
  return MOBA_OK;
}

// The problem of packed sequences: list sizes from the sequences' own blocks.
void apply_packed(const Packed& pk, moba::Problem* p) {
  p->p_off = pk.pairs_per_head * p->H;
  p->topk = std::max(1, std::min(p->topk, pk.max_blocks));   // the longest sequence bounds the kept blocks
  p->lmax = std::max(0, std::min(p->topk - 1, pk.max_blocks - 1));
  p->max_items = p->p_off / moba::kAttnTile + static_cast<int64_t>(p->H) * p->n;
}

int block_mean_keys_impl(const void* k, float* kbar, int64_t N, int32_t H, int32_t D, int32_t B, hipStream_t stream,
                         bool is_f32, const Pooling& pl = Pooling()) {
  if (k == nullptr || kbar == nullptr) return MOBA_ERR_INVALID_ARG;
  int s = check_shape(N, H, D, B);
  if (s != MOBA_OK) return s;
  if ((s = check_pooling(pl)) != MOBA_OK) return s;
  if (!aligned16(k) || !aligned16(kbar)) return MOBA_ERR_UNSUPPORTED;
  DeviceState* st = nullptr;
  if ((s = current_device(&st)) != MOBA_OK) return s;
  hipError_t e = moba::launch_pool(k, is_f32, kbar, nullptr, N, H, D, B, stream, pl.mode, pl.weights);
  return e == hipSuccess ? MOBA_OK : hip_fail(e);
}

int gate_impl(const void* q, const void* k, int32_t* sel, int64_t N, int32_t H, int32_t D, int32_t B, int32_t topk,
              hipStream_t stream, bool is_f32, const Pooling& pl = Pooling(), const Packed* pk = nullptr) {
  if (q == nullptr || k == nullptr || sel == nullptr) return MOBA_ERR_INVALID_ARG;
  int s = check_shape(N, H, D, B);
  if (s != MOBA_OK) return s;
  if (pk == nullptr && (s = check_topk(N, B, topk)) != MOBA_OK) return s;
  if ((s = check_pooling(pl)) != MOBA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(sel)) return MOBA_ERR_UNSUPPORTED;
  DeviceState* st = nullptr;
  if ((s = current_device(&st)) != MOBA_OK) return s;
  moba::Problem p = make_problem(N, H, D, B, topk, is_f32);
  if (pk != nullptr) apply_packed(*pk, &p);
  p.topk = topk;   // the caller's rows are topk wide (entries past j + 1 are -1)
  const WsPlan w = plan(p, Stages::gate, pk != nullptr);
  char* base = nullptr;
  if ((s = alloc_ws(st, w.total, stream, &base)) != MOBA_OK) return s;
  moba::Workspace ws = bind(w, base, false);
  hipError_t e = hipSuccess;
  if (pk != nullptr) {
    int32_t* blo = reinterpret_cast<int32_t*>(base + w.blo);
    p.blo = blo;
    e = moba::launch_seq_lo(pk->st, blo, p.n, stream);
  }
  if (e == hipSuccess)
    e = moba::launch_pool(k, is_f32, ws.kbar, is_f32 ? nullptr : ws.kpieces, N, H, D, B, stream, pl.mode, pl.weights);
  if (e == hipSuccess) e = moba::launch_gate(p, q, ws, sel, false, st->num_cus, stream);
  return finish(e, base, stream);
}

// Pooling, gate and the query lists of the prefill, with the lists written
// into the caller's offs / qidx and the selection into the caller's sel.
int query_lists_impl(const void* q, const void* k, int32_t* sel, int32_t* offs, int32_t* qidx, int64_t qidx_len,
                     int64_t N, int32_t H, int32_t D, int32_t B, int32_t topk, hipStream_t stream) {
  if (q == nullptr || k == nullptr || sel == nullptr || offs == nullptr || qidx == nullptr) return MOBA_ERR_INVALID_ARG;
  int s = check_shape(N, H, D, B);
  if (s != MOBA_OK) return s;
  if ((s = check_topk(N, B, topk)) != MOBA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(sel) || !aligned16(offs) || !aligned16(qidx))
    return MOBA_ERR_UNSUPPORTED;
  moba::Problem p = make_problem(N, H, D, B, topk, false);
  if (p.p_off >= (int64_t{1} << 31)) return MOBA_ERR_UNSUPPORTED;
  if (qidx_len < p.p_off) return MOBA_ERR_INVALID_ARG;
  p.topk = topk;   // the caller's rows are topk wide (entries past j + 1 are -1)
  DeviceState* st = nullptr;
  if ((s = current_device(&st)) != MOBA_OK) return s;
  const WsPlan w = plan(p, Stages::lists);
  char* base = nullptr;
  if ((s = alloc_ws(st, w.total, stream, &base)) != MOBA_OK) return s;
  moba::Workspace ws = bind(w, base, true);
  ws.offs = offs;
  ws.qidx = qidx;
  ws.sel = sel;
  hipError_t e = moba::launch_pool(k, false, ws.kbar, ws.kpieces, N, H, D, B, stream, MOBA_POOL_MEAN, nullptr);
  if (e == hipSuccess) e = moba::launch_gate(p, q, ws, sel, true, st->num_cus, stream);
  if (e == hipSuccess) e = moba::launch_csr(p, ws, sel, stream);
  return finish(e, base, stream);
}

int prefill_impl(const void* q, const void* k, const void* v, void* out, float* lse, int64_t N, int32_t H, int32_t D,
                 int32_t B, int32_t topk, hipStream_t stream, bool is_f32, hipEvent_t* events = nullptr,
                 const Pooling& pl = Pooling(), const Packed* pk = nullptr) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || lse == nullptr) return MOBA_ERR_INVALID_ARG;
  int s = check_shape(N, H, D, B);
  if (s != MOBA_OK) return s;
  if (pk == nullptr && (s = check_topk(N, B, topk)) != MOBA_OK) return s;
  if ((s = check_pooling(pl)) != MOBA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse))
    return MOBA_ERR_UNSUPPORTED;
  // Every block kept (top_k >= n): the attended set of a query is every key up
  // to itself, i.e. MoBA with one block of N tokens and top-1. That form needs
  // no pooling, gate, query lists or partials (dense causal path).
  const bool dense = pk == nullptr && dense_path(N, B, topk, is_f32);
  moba::Problem p = dense ? make_problem(N, H, D, static_cast<int32_t>(N), 1, is_f32)
                          : make_problem(N, H, D, B, topk, is_f32);
  if (pk != nullptr) apply_packed(*pk, &p);
  if (p.p_off >= (int64_t{1} << 31)) return MOBA_ERR_UNSUPPORTED;
  DeviceState* st = nullptr;
  if ((s = current_device(&st)) != MOBA_OK) return s;
  const WsPlan w = plan(p, Stages::forward, pk != nullptr);
  char* base = nullptr;
  if ((s = alloc_ws(st, w.total, stream, &base)) != MOBA_OK) return s;
  moba::Workspace ws = bind(w, base, true);
  auto mark = [&](int i) { return events && events[i] ? hipEventRecord(events[i], stream) : hipSuccess; };
  hipError_t e = mark(0);
  if (e == hipSuccess && pk != nullptr) {
    int32_t* blo = reinterpret_cast<int32_t*>(base + w.blo);
    p.blo = blo;
    e = moba::launch_seq_lo(pk->st, blo, p.n, stream);
  }
  if (e == hipSuccess && !dense)
    e = moba::launch_pool(k, is_f32, ws.kbar, is_f32 ? nullptr : ws.kpieces, N, H, D, B, stream, pl.mode, pl.weights);
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess && !dense) e = moba::launch_gate(p, q, ws, ws.sel, true, st->num_cus, stream);
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess && !dense) e = moba::launch_csr(p, ws, ws.sel, stream);
  if (e == hipSuccess) e = mark(3);
  if (e == hipSuccess) e = moba::launch_attention(p, q, k, v, ws, out, lse, st->num_cus, stream, mark);
  if (e == hipSuccess) e = mark(5);
  if (e == hipSuccess && !moba::merge_fused(p)) e = moba::launch_merge(p, ws, out, lse, stream);
  if (e == hipSuccess) e = mark(6);
  return finish(e, base, stream);
}

int backward_impl(const void* q, const void* k, const void* v, const void* out, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, int64_t N, int32_t H, int32_t D, int32_t B, int32_t topk,
                  hipStream_t stream, const Pooling& pl = Pooling(), const Packed* pk = nullptr) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || lse == nullptr || dout == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return MOBA_ERR_INVALID_ARG;
  int s = check_shape(N, H, D, B);
  if (s != MOBA_OK) return s;
  if (pk == nullptr && (s = check_topk(N, B, topk)) != MOBA_OK) return s;
  if ((s = check_pooling(pl)) != MOBA_OK) return s;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse) || !aligned16(dout) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return MOBA_ERR_UNSUPPORTED;
  const bool dense = pk == nullptr && dense_path(N, B, topk, false);   // see prefill_impl
  moba::Problem p = dense ? make_problem(N, H, D, static_cast<int32_t>(N), 1, false)
                          : make_problem(N, H, D, B, topk, false);
  if (pk != nullptr) apply_packed(*pk, &p);
  if (p.p_off >= (int64_t{1} << 31)) return MOBA_ERR_UNSUPPORTED;
  DeviceState* st = nullptr;
  if ((s = current_device(&st)) != MOBA_OK) return s;
  const WsPlan w = plan(p, Stages::backward, pk != nullptr);
  char* base = nullptr;
  if ((s = alloc_ws(st, w.total, stream, &base)) != MOBA_OK) return s;
  moba::Workspace ws = bind(w, base, true);
  moba::BwdArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const moba::bf16*>(q);
  a.k = static_cast<const moba::bf16*>(k);
  a.v = static_cast<const moba::bf16*>(v);
  a.out = static_cast<const moba::bf16*>(out);
  a.dout = static_cast<const moba::bf16*>(dout);
  a.lse = lse;
  a.dq = static_cast<moba::bf16*>(dq);
  a.dk = static_cast<moba::bf16*>(dk);
  a.dv = static_cast<moba::bf16*>(dv);
  a.delta = reinterpret_cast<float*>(base + w.delta);
  a.part_dq = reinterpret_cast<float*>(base + w.part_dq);
  a.qidx = ws.qidx;
  a.offs = ws.offs;
  a.totals = ws.totals;
  a.inv = ws.inv;
  a.items = ws.items;
  a.counters = ws.counters;
  a.N = N;
  a.H = H;
  a.D = D;
  a.B = p.B;
  a.n = p.n;
  a.topk = p.topk;
  a.lmax = p.lmax;
  a.max_items = p.lmax > 0 ? p.max_items : 0;
  a.has_lists = dense ? 0 : 1;
  a.num_cus = st->num_cus;
  a.scale = 1.0f / std::sqrt(static_cast<float>(D));
  a.scale_log2 = 1.4426950408889634f / std::sqrt(static_cast<float>(D));
  hipError_t e = hipSuccess;
  if (pk != nullptr) {
    int32_t* blo = reinterpret_cast<int32_t*>(base + w.blo);
    p.blo = blo;
    a.blo = blo;
    e = moba::launch_seq_lo(pk->st, blo, p.n, stream);
  }
  if (!dense && e == hipSuccess) {
    e = moba::launch_pool(k, false, ws.kbar, ws.kpieces, N, H, D, B, stream, pl.mode, pl.weights);
    if (e == hipSuccess) e = moba::launch_gate(p, q, ws, ws.sel, true, st->num_cus, stream);
    if (e == hipSuccess) e = moba::launch_csr(p, ws, ws.sel, stream);
  }
  if (e == hipSuccess) e = moba::launch_backward(a, stream);
  return finish(e, base, stream);
}

// ext_ws: caller-provided workspace of ext_cap bytes (the allocation-free
// entry point); nullptr takes it from the pool.
int decode_impl(const void* q, const void* k, const void* v, const float* kbar, int32_t kbar_blocks, void* out,
                float* lse, int32_t* sel, int64_t N, int32_t H, int32_t D, int32_t B, int32_t topk,
                hipStream_t stream, char* ext_ws = nullptr, size_t ext_cap = 0) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || lse == nullptr) return MOBA_ERR_INVALID_ARG;
  if (N < 1 || H < 1 || B < 1 || topk < 1) return MOBA_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return MOBA_ERR_UNSUPPORTED;
  if (N >= (int64_t{1} << 40) || H > 65535) return MOBA_ERR_UNSUPPORTED;
  const int64_t j = (N - 1) / B;   // the new token's block; blocks 0..j-1 are complete
  if (j >= (int64_t{1} << 24)) return MOBA_ERR_UNSUPPORTED;
  if (topk > MOBA_MAX_TOPK && topk <= j) return MOBA_ERR_UNSUPPORTED;
  if (sel != nullptr && topk > MOBA_MAX_BLOCKS) return MOBA_ERR_UNSUPPORTED;
  if (kbar != nullptr && kbar_blocks < j) return MOBA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(lse) ||
      (kbar != nullptr && !aligned16(kbar)) || (sel != nullptr && !aligned16(sel)))
    return MOBA_ERR_UNSUPPORTED;
  int s;
  DeviceState* st = nullptr;
  if ((s = current_device(&st)) != MOBA_OK) return s;
  moba::DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.N = N;
  a.H = H;
  a.D = D;
  a.B = B;
  a.j = static_cast<int>(j);
  a.topk = topk;
  a.S = static_cast<int>(std::min<int64_t>(topk, j + 1));
  // Keys per unit: the largest of 512, 256, 128, 64 that still gives two units per CU.
  a.chunk = moba::kDecMaxChunk;
  while (a.chunk > 64 && static_cast<int64_t>(H) * a.S * ((B + a.chunk - 1) / a.chunk) < 2 * st->num_cus)
    a.chunk /= 2;
  a.chunks = (B + a.chunk - 1) / a.chunk;
  if (static_cast<int64_t>(a.S) * a.chunks >= (int64_t{1} << 31)) return MOBA_ERR_UNSUPPORTED;
  a.units = a.S * a.chunks;
  a.scale_log2 = 1.4426950408889634f / std::sqrt(static_cast<float>(D));
  a.q = static_cast<const moba::bf16*>(q);
  a.k = static_cast<const moba::bf16*>(k);
  a.v = static_cast<const moba::bf16*>(v);
  a.kbar = kbar;
  a.kbar_blocks = kbar_blocks;
  a.sel_out = sel;
  a.out = static_cast<moba::bf16*>(out);
  a.lse = lse;
  if (moba::decode_fused(a)) {
    // Caller's block means and few kept keys: one launch, no workspace.
    const hipError_t e = moba::launch_decode_fused(a, stream);
    return e == hipSuccess ? MOBA_OK : hip_fail(e);
  }
  const bool own_kbar = kbar == nullptr && topk < j + 1;   // block means only matter when the gate chooses
  Layout L;
  const size_t o_sel = L.add(static_cast<size_t>(H) * a.S * 4);
  const size_t o_sc = L.add(static_cast<size_t>(H) * j * 4);
  const size_t o_po = L.add(static_cast<size_t>(H) * a.units * D * 4);
  const size_t o_ml = L.add(static_cast<size_t>(H) * a.units * 2 * 4);
  const size_t o_kb = L.add(own_kbar ? static_cast<size_t>(H) * j * D * 4 : 0);
  char* base = nullptr;
  if (ext_ws != nullptr) {
    if (L.total > ext_cap) return MOBA_ERR_UNSUPPORTED;
    base = ext_ws;
    if (g_poison_workspace.load(std::memory_order_relaxed) != 0) {
      const hipError_t pe = moba::launch_fill(base, L.total, 0xFFFFFFFFu, stream);
      if (pe != hipSuccess) return hip_fail(pe);
    }
  } else if ((s = alloc_ws(st, L.total, stream, &base)) != MOBA_OK) {
    return s;
  }
  a.q = static_cast<const moba::bf16*>(q);
  a.k = static_cast<const moba::bf16*>(k);
  a.v = static_cast<const moba::bf16*>(v);
  a.kbar = own_kbar ? reinterpret_cast<const float*>(base + o_kb) : kbar;
  a.kbar_blocks = own_kbar ? static_cast<int>(j) : kbar_blocks;
  a.sel = reinterpret_cast<int32_t*>(base + o_sel);
  a.sel_out = sel;
  a.scores = reinterpret_cast<float*>(base + o_sc);
  a.part_o = reinterpret_cast<float*>(base + o_po);
  a.part_ml = reinterpret_cast<float*>(base + o_ml);
  a.out = static_cast<moba::bf16*>(out);
  a.lse = lse;
  hipError_t e = hipSuccess;
  if (own_kbar)
    e = moba::launch_pool(k, false, reinterpret_cast<float*>(base + o_kb), nullptr, j * B, H, D, B, stream);
  if (e == hipSuccess) e = moba::launch_decode(a, stream);
  if (ext_ws != nullptr) return e == hipSuccess ? MOBA_OK : hip_fail(e);
  return finish(e, base, stream);
}

}  // namespace

namespace moba {

int fail_hip(hipError_t e) { return hip_fail(e); }

int decode_with_workspace(const void* q, const void* k, const void* v, const float* kbar, int32_t kbar_blocks,
                          void* out, float* lse, int32_t* sel, int64_t N, int32_t H, int32_t D, int32_t block_size,
                          int32_t topk, hipStream_t stream, char* ws, size_t ws_bytes) {
  return decode_impl(q, k, v, kbar, kbar_blocks, out, lse, sel, N, H, D, block_size, topk, stream, ws, ws_bytes);
}

}  // namespace moba

extern "C" {

int moba_block_mean_keys(const void* k, float* kbar, int64_t N, int32_t H, int32_t D, int32_t block_size,
                         hipStream_t stream) {
  return block_mean_keys_impl(k, kbar, N, H, D, block_size, stream, false);
}

int moba_block_mean_keys_f32(const float* k, float* kbar, int64_t N, int32_t H, int32_t D, int32_t block_size,
                             hipStream_t stream) {
  return block_mean_keys_impl(k, kbar, N, H, D, block_size, stream, true);
}

int moba_gate_topk(const void* q, const void* k, int32_t* sel, int64_t N, int32_t H, int32_t D, int32_t block_size,
                   int32_t topk, hipStream_t stream) {
  return gate_impl(q, k, sel, N, H, D, block_size, topk, stream, false);
}

int moba_gate_topk_f32(const float* q, const float* k, int32_t* sel, int64_t N, int32_t H, int32_t D,
                       int32_t block_size, int32_t topk, hipStream_t stream) {
  return gate_impl(q, k, sel, N, H, D, block_size, topk, stream, true);
}

int moba_block_query_lists(const void* q, const void* k, int32_t* sel, int32_t* offs, int32_t* qidx,
                           int64_t qidx_len, int64_t N, int32_t H, int32_t D, int32_t block_size, int32_t topk,
                           hipStream_t stream) {
  return query_lists_impl(q, k, sel, offs, qidx, qidx_len, N, H, D, block_size, topk, stream);
}

int moba_prefill_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int64_t N, int32_t H,
                     int32_t D, int32_t block_size, int32_t topk, hipStream_t stream) {
  return prefill_impl(q, k, v, out, lse, N, H, D, block_size, topk, stream, false);
}

int moba_prefill_fwd_timed(const void* q, const void* k, const void* v, void* out, float* lse, int64_t N, int32_t H,
                           int32_t D, int32_t block_size, int32_t topk, hipStream_t stream, hipEvent_t* events) {
  return prefill_impl(q, k, v, out, lse, N, H, D, block_size, topk, stream, false, events);
}

int moba_prefill_fwd_f32(const float* q, const float* k, const float* v, float* out, float* lse, int64_t N, int32_t H,
                         int32_t D, int32_t block_size, int32_t topk, hipStream_t stream) {
  return prefill_impl(q, k, v, out, lse, N, H, D, block_size, topk, stream, true);
}

int moba_decode_fwd(const void* q, const void* k, const void* v, const float* kbar, int32_t kbar_blocks, void* out,
                    float* lse, int32_t* sel, int64_t N, int32_t H, int32_t D, int32_t block_size, int32_t topk,
                    hipStream_t stream) {
  return decode_impl(q, k, v, kbar, kbar_blocks, out, lse, sel, N, H, D, block_size, topk, stream);
}

int moba_prefill_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int64_t N, int32_t H, int32_t D,
                     int32_t block_size, int32_t topk, hipStream_t stream) {
  return backward_impl(q, k, v, out, lse, dout, dq, dk, dv, N, H, D, block_size, topk, stream);
}

int moba_block_pool_keys(const void* k, const float* weights, float* kbar, int64_t N, int32_t H, int32_t D,
                         int32_t block_size, int32_t pooling, hipStream_t stream) {
  Pooling pl;
  pl.mode = pooling;
  pl.weights = weights;
  return block_mean_keys_impl(k, kbar, N, H, D, block_size, stream, false, pl);
}

int moba_gate_topk_pooled(const void* q, const void* k, const float* weights, int32_t* sel, int64_t N, int32_t H,
                          int32_t D, int32_t block_size, int32_t topk, int32_t pooling, hipStream_t stream) {
  Pooling pl;
  pl.mode = pooling;
  pl.weights = weights;
  return gate_impl(q, k, sel, N, H, D, block_size, topk, stream, false, pl);
}

int moba_prefill_fwd_pooled(const void* q, const void* k, const void* v, const float* weights, void* out, float* lse,
                            int64_t N, int32_t H, int32_t D, int32_t block_size, int32_t topk, int32_t pooling,
                            hipStream_t stream) {
  Pooling pl;
  pl.mode = pooling;
  pl.weights = weights;
  return prefill_impl(q, k, v, out, lse, N, H, D, block_size, topk, stream, false, nullptr, pl);
}

int moba_prefill_bwd_pooled(const void* q, const void* k, const void* v, const float* weights, const void* out,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv, int64_t N, int32_t H,
                            int32_t D, int32_t block_size, int32_t topk, int32_t pooling, hipStream_t stream) {
  Pooling pl;
  pl.mode = pooling;
  pl.weights = weights;
  return backward_impl(q, k, v, out, lse, dout, dq, dk, dv, N, H, D, block_size, topk, stream, pl);
}

int moba_gate_topk_varlen(const void* q, const void* k, int32_t* sel, const int64_t* cu_seqlens, int32_t num_seqs,
                          int32_t H, int32_t D, int32_t block_size, int32_t topk, hipStream_t stream) {
  Packed pk;
  int64_t T = 0;
  const int s = parse_packed(cu_seqlens, num_seqs, block_size, topk, &pk, &T);
  if (s != MOBA_OK) return s;
  return gate_impl(q, k, sel, T, H, D, block_size, topk, stream, false, Pooling(), &pk);
}

int moba_prefill_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                            const int64_t* cu_seqlens, int32_t num_seqs, int32_t H, int32_t D, int32_t block_size,
                            int32_t topk, hipStream_t stream) {
  Packed pk;
  int64_t T = 0;
  const int s = parse_packed(cu_seqlens, num_seqs, block_size, topk, &pk, &T);
  if (s != MOBA_OK) return s;
  return prefill_impl(q, k, v, out, lse, T, H, D, block_size, topk, stream, false, nullptr, Pooling(), &pk);
}

int moba_prefill_bwd_varlen(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, void* dq, void* dk, void* dv, const int64_t* cu_seqlens,
                            int32_t num_seqs, int32_t H, int32_t D, int32_t block_size, int32_t topk,
                            hipStream_t stream) {
  Packed pk;
  int64_t T = 0;
  const int s = parse_packed(cu_seqlens, num_seqs, block_size, topk, &pk, &T);
  if (s != MOBA_OK) return s;
  return backward_impl(q, k, v, out, lse, dout, dq, dk, dv, T, H, D, block_size, topk, stream, Pooling(), &pk);
}

int32_t moba_topk_for_sparsity(int64_t N, int32_t block_size, double sparsity) {
  if (N < 1 || block_size < 1 || N % block_size != 0 || !(sparsity >= 0.0 && sparsity < 1.0))
    return -MOBA_ERR_INVALID_ARG;
  const int64_t n = N / block_size;
  const double kk = std::nearbyint((1.0 - sparsity) * static_cast<double>(N) / static_cast<double>(block_size));
  return static_cast<int32_t>(std::min<double>(static_cast<double>(n), std::max(1.0, kk)));
}

const char* moba_status_string(int status) {
  switch (status) {
    case MOBA_OK: return "MOBA_OK";
    case MOBA_ERR_INVALID_ARG: return "MOBA_ERR_INVALID_ARG";
    case MOBA_ERR_UNSUPPORTED: return "MOBA_ERR_UNSUPPORTED";
    case MOBA_ERR_HIP: return "MOBA_ERR_HIP";
    case MOBA_ERR_OUT_OF_MEMORY: return "MOBA_ERR_OUT_OF_MEMORY";
    default: return "MOBA_ERR_UNKNOWN";
  }
}

int moba_last_hip_error(void) { return g_last_hip_error; }

int moba_debug_poison_workspace(int on) { return g_poison_workspace.exchange(on != 0 ? 1 : 0); }

}  // extern "C"
