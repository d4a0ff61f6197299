// Regrouping of the queries by key block (the second half of the query lists).
//
// The pages' implementation reorders the queries by their block assignment so
// that attention runs block by block (智东西 report, section 二, implementation
// steps 1-2). Here every (head, past block) pair gets a list of the queries
// that kept that block, ordered by query position:
//   1. scan_tiles: per (head, block), exclusive prefix of the per-tile counts
//      written by the gate, and the list length;
//   2. build_lists (one 1024-thread workgroup): global start of every list and
//      of its work items (at most kAttnTile list entries each);
//   3. scatter (one workgroup per query tile and head): every (query, kept
//      past block) pair lands at start(list) + prefix(tile) + rank-in-tile,
//      written as the tile's run of each list; the position is also kept per
//      query so the merge can find its partial outputs again; and the work
//      items.
// Only integer arithmetic in fixed orders: the lists are deterministic.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moba {

namespace {

// Workgroup-wide exclusive scan of one int64 value per thread (NT threads, a
// multiple of 64): shuffle scans inside each wave, then a scan of the wave totals.
template <int NT>
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t x, int64_t* sh, int64_t* total) {
  constexpr int kW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t v = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int64_t wv = lane < kW ? sh[lane] : 0;
#pragma unroll
    for (int off = 1; off < kW; off <<= 1) {
      const int64_t y = __shfl_up(wv, off);
      if (lane >= off) wv += y;
    }
    if (lane < kW) sh[lane] = wv;
  }
  __syncthreads();
  const int64_t base = wave > 0 ? sh[wave - 1] : 0;
  *total = sh[kW - 1];
  __syncthreads();
  return base + v - x;
}

__global__ __launch_bounds__(256) void scan_tiles_kernel(int32_t* __restrict__ cnt, int32_t* __restrict__ totals,
                                                         int ntiles) {
  __shared__ int64_t sh[4];
  const int64_t e = blockIdx.x;
  int32_t* row = cnt + e * ntiles;
  const int per = (ntiles + 255) / 256;
  const int lo = min(ntiles, static_cast<int>(threadIdx.x) * per);
  const int hi = min(ntiles, lo + per);
  int64_t s = 0;
  for (int i = lo; i < hi; ++i) s += row[i];
  int64_t total;
  int64_t run = block_exclusive_scan<256>(s, sh, &total);
  for (int i = lo; i < hi; ++i) {
    const int32_t c = row[i];
    row[i] = static_cast<int32_t>(run);
    run += c;
  }
  if (threadIdx.x == 0) totals[e] = static_cast<int32_t>(total);
}

constexpr int kListThreads = 1024;

// List starts and work-item starts of every (head, block): two exclusive
// scans over the E list lengths (one workgroup; E = H * n is small), the total
// list length (offs[E]) and the number of work items. The items themselves
// are written by the scatter.
__global__ __launch_bounds__(kListThreads) void build_lists_kernel(const int32_t* __restrict__ totals,
                                                                   int32_t* __restrict__ offs,
                                                                   int32_t* __restrict__ istart,
                                                                   int32_t* __restrict__ counters, int64_t E) {
  __shared__ int64_t sh[kListThreads / 64];
  const int64_t per = (E + kListThreads - 1) / kListThreads;
  const int64_t lo = min(E, static_cast<int64_t>(threadIdx.x) * per);
  const int64_t hi = min(E, lo + per);
  int64_t s_len = 0, s_items = 0;
  for (int64_t e = lo; e < hi; ++e) {
    const int64_t len = totals[e];
    s_len += len;
    s_items += (len + kAttnTile - 1) / kAttnTile;
  }
  int64_t tot_len, tot_items;
  int64_t pos = block_exclusive_scan<kListThreads>(s_len, sh, &tot_len);
  int64_t it = block_exclusive_scan<kListThreads>(s_items, sh, &tot_items);
  for (int64_t e = lo; e < hi; ++e) {
    const int64_t len = totals[e];
    offs[e] = static_cast<int32_t>(pos);
    istart[e] = static_cast<int32_t>(it);
    pos += len;
    it += (len + kAttnTile - 1) / kAttnTile;
  }
  if (threadIdx.x == 0) {
    counters[0] = static_cast<int32_t>(tot_items);
    offs[E] = static_cast<int32_t>(tot_len);
  }
  if (threadIdx.x < kXcds) counters[kCursorStride * (1 + threadIdx.x)] = 0;
}

// One workgroup per (query tile, head). Every (query, kept past block) pair
// of the tile lands at start(list) + prefix(tile) + rank-in-tile. The pairs
// are first sorted by block in LDS (the tile's share of each list is one
// contiguous run of the list), so the query indices leave in runs of
// consecutive addresses; the list positions are written per query
// (contiguous rows). The workgroup also writes the work items of the lists
// b = tile, tile + ntiles, ... of its head.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ sel, const int32_t* __restrict__ rk,
                                                      const int32_t* __restrict__ cnt,
                                                      const int32_t* __restrict__ totals,
                                                      const int32_t* __restrict__ offs,
                                                      const int32_t* __restrict__ istart, int32_t* __restrict__ qidx,
                                                      int32_t* __restrict__ inv, WorkItem* __restrict__ items,
                                                      int64_t N, int H, int B, int n, int topk, int lmax, int ntiles,
                                                      const int32_t* __restrict__ blo) {
  extern __shared__ int32_t csm[];
  __shared__ int64_t sh[4];
  __shared__ int32_t s_total;
  const int tile = static_cast<int>(blockIdx.x);
  const int h = static_cast<int>(blockIdx.y);
  const int tid = static_cast<int>(threadIdx.x);
  const int64_t hn = static_cast<int64_t>(h) * n;

  // Work items of this workgroup's lists (written last: nothing below waits on them).
  auto write_items = [&]() {
    for (int b = tile; b < n; b += ntiles) {
      const int64_t e = hn + b;
      const int len = totals[e];
      const int i0 = istart[e], p0 = offs[e];
      for (int c = tid; c * kAttnTile < len; c += 256) {
        WorkItem wi;
        wi.h = h;
        wi.b = b;
        wi.start = p0 + c * kAttnTile;
        wi.count = min(kAttnTile, len - c * kAttnTile);
        items[i0 + c] = wi;
      }
    }
  };
  const int64_t t0 = static_cast<int64_t>(tile) * kQTile;
  const int64_t t1 = min(N, t0 + kQTile);
  const int jmax = static_cast<int>((t1 - 1) / B);   // the tile's past blocks are all below its last block
  if (lmax == 0 || jmax == 0) {
    write_items();
    return;
  }
  // (query, kept past block) pair i of the tile: query t0 + i / lmax, slot i % lmax.
  const int nq = static_cast<int>(t1 - t0);
  auto load_pair = [&](int i, int& b, int& r, int64_t& t) -> bool {
    const int qi = i / lmax, s = i - qi * lmax;
    t = t0 + qi;
    const int j = static_cast<int>(t / B);
    if (s >= kept_past(j, blo != nullptr ? blo[j] : 0, topk)) return false;
    const int64_t g = static_cast<int64_t>(h) * N + t;
    b = sel[g * topk + s];
    r = rk[g * lmax + s];
    return true;
  };
  // The thread's first pair is read before the list positions (it does not
  // depend on them), so the two reads overlap.
  int b_first = 0, r_first = 0;
  int64_t t_first = 0;
  const bool has_first = tid < nq * lmax && load_pair(tid, b_first, r_first, t_first);
  // Per-block share of the tile (its count), then the exclusive prefix over
  // blocks; and the list position of the tile's first entry in each list.
  const int jpad = (jmax + 3) & ~3;
  int32_t* const pre = csm;                                              // [jmax]
  int32_t* const first = csm + jpad;                                     // [jmax]
  int2* const ent = reinterpret_cast<int2*>(csm + 2 * jpad);             // [kQTile * lmax]: (position, query)
  const int per = (jmax + 255) / 256;
  const int b0 = min(jmax, tid * per), b1 = min(jmax, b0 + per);
  int64_t sum = 0;
  for (int b = b0; b < b1; ++b) {
    const int64_t e = hn + b;
    const int before = cnt[e * ntiles + tile];
    const int c = (tile + 1 < ntiles ? cnt[e * ntiles + tile + 1] : totals[e]) - before;
    pre[b] = c;
    first[b] = offs[e] + before;
    sum += c;
  }
  int64_t total;
  int64_t run = block_exclusive_scan<256>(sum, sh, &total);
  for (int b = b0; b < b1; ++b) {
    const int c = pre[b];
    pre[b] = static_cast<int32_t>(run);
    run += c;
  }
  if (tid == 0) s_total = static_cast<int32_t>(total);
  __syncthreads();
  // Pairs in query order: coalesced reads of sel and rk and writes of inv.
  for (int i = tid; i < nq * lmax; i += 256) {
    int b, r;
    int64_t t;
    if (i == tid) {
      if (!has_first) continue;
      b = b_first;
      r = r_first;
      t = t_first;
    } else if (!load_pair(i, b, r, t)) {
      continue;
    }
    const int qi = i / lmax, s = i - qi * lmax;
    const int64_t g = static_cast<int64_t>(h) * N + t0 + qi;
    const int32_t pos = first[b] + r;
    inv[g * lmax + s] = pos;
    ent[pre[b] + r] = make_int2(pos, static_cast<int32_t>(t));
  }
  __syncthreads();
  const int tot = s_total;
  for (int k = tid; k < tot; k += 256) {
    const int2 x = ent[k];
    qidx[x.x] = x.y;
  }
  write_items();
}

}  // namespace

hipError_t launch_csr(const Problem& p, const Workspace& ws, const int32_t* sel, hipStream_t stream) {
  const int64_t E = static_cast<int64_t>(p.H) * p.n;
  scan_tiles_kernel<<<static_cast<unsigned>(E), 256, 0, stream>>>(ws.cnt, ws.totals, p.ntiles);
  build_lists_kernel<<<1, kListThreads, 0, stream>>>(ws.totals, ws.offs, ws.istart, ws.counters, E);
  // LDS: the per-block prefix and first list positions of a tile's past blocks
  // (at most n each) and its (position, query) pairs.
  const size_t smem = static_cast<size_t>((p.n + 3) & ~3) * 8 + static_cast<size_t>(kQTile) * p.lmax * 8;
  dim3 grid(static_cast<unsigned>(p.ntiles), static_cast<unsigned>(p.H));
  scatter_kernel<<<grid, 256, smem, stream>>>(sel, ws.rk, ws.cnt, ws.totals, ws.offs, ws.istart, ws.qidx, ws.inv,
                                              ws.items, p.N, p.H, p.B, p.n, p.topk, p.lmax, p.ntiles, p.blo);
  return hipGetLastError();
}

namespace {

__global__ __launch_bounds__(256) void fill_kernel(uint4* __restrict__ p, size_t n16, uint32_t value) {
  const uint4 x = make_uint4(value, value, value, value);
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += static_cast<size_t>(gridDim.x) * 256)
    p[i] = x;
}

}  // namespace

hipError_t launch_fill(void* p, size_t bytes, uint32_t value, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n16 + 255) / 256, 4096);
  fill_kernel<<<static_cast<unsigned>(blocks), 256, 0, stream>>>(static_cast<uint4*>(p), n16, value);
  return hipGetLastError();
}

namespace {

__global__ __launch_bounds__(256) void seq_lo_kernel(SeqStarts st, int32_t* __restrict__ blo, int n) {
  const int j = static_cast<int>(blockIdx.x) * 256 + threadIdx.x;
  if (j >= n) return;
  // The last sequence whose first block is <= j (empty sequences share their
  // start with the next one, so the last such sequence is the one holding j).
  int lo = 0, hi = st.nseq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (st.start[mid] <= j) lo = mid;
    else hi = mid - 1;
  }
  blo[j] = st.start[lo];
}

}  // namespace

hipError_t launch_seq_lo(const SeqStarts& st, int32_t* blo, int n, hipStream_t stream) {
  seq_lo_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(st, blo, n);
  return hipGetLastError();
}

}  // namespace moba
