// Regrouping of the queries by key block (the second half of the query lists).
//
// The pages' implementation reorders the queries by their block assignment so
// that attention runs block by block (智东西 report, section 二, implementation
// steps 1-2). Here every (head, past block) pair gets a list of the queries
// that kept that block, ordered by query position:
//   1. scan_tiles: per (head, block), exclusive prefix of the per-tile counts
//      written by the gate, and the list length;
//   2. build_lists (one 1024-thread workgroup): global start of every list and the work
//      items of at most kAttnTile list entries each;
//   3. scatter: every (query, kept past block) pair lands at
//      start(list) + prefix(tile) + rank-in-tile; the position is also kept per
//      query so the merge can find its partial outputs again.
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

__global__ __launch_bounds__(kListThreads) void build_lists_kernel(const int32_t* __restrict__ totals,
                                                                   int32_t* __restrict__ offs,
                                                                   WorkItem* __restrict__ items,
                                                                   int32_t* __restrict__ counters, int n, int64_t E) {
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
    for (int64_t c = 0; c < len; c += kAttnTile) {
      WorkItem w;
      w.h = static_cast<int32_t>(e / n);
      w.b = static_cast<int32_t>(e % n);
      w.start = static_cast<int32_t>(pos + c);
      w.count = static_cast<int32_t>(len - c < kAttnTile ? len - c : kAttnTile);
      items[it++] = w;
    }
    pos += len;
  }
  if (threadIdx.x == 0) counters[0] = static_cast<int32_t>(tot_items);
  if (threadIdx.x < kXcds) counters[kCursorStride * (1 + threadIdx.x)] = 0;
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ sel, const int32_t* __restrict__ rk,
                                                      const int32_t* __restrict__ cnt,
                                                      const int32_t* __restrict__ offs, int32_t* __restrict__ qidx,
                                                      int32_t* __restrict__ inv, int64_t N, int H, int B, int n,
                                                      int topk, int lmax, int ntiles, const int32_t* __restrict__ blo) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (g >= N * H) return;
  const int h = static_cast<int>(g / N);
  const int64_t t = g % N;
  const int j = static_cast<int>(t / B);
  const int L = kept_past(j, blo != nullptr ? blo[j] : 0, topk);   // kept past blocks, ascending in sel
  const int tile = static_cast<int>(t / kQTile);
  const int32_t* srow = sel + g * topk;
  const int32_t* rrow = rk + g * lmax;
  int32_t* irow = inv + g * lmax;
  for (int s = 0; s < L; ++s) {
    const int b = srow[s];
    const int64_t e = static_cast<int64_t>(h) * n + b;
    const int32_t pos = offs[e] + cnt[e * ntiles + tile] + rrow[s];
    qidx[pos] = static_cast<int32_t>(t);
    irow[s] = pos;
  }
}

}  // namespace

hipError_t launch_csr(const Problem& p, const Workspace& ws, const int32_t* sel, hipStream_t stream) {
  const int64_t E = static_cast<int64_t>(p.H) * p.n;
  scan_tiles_kernel<<<static_cast<unsigned>(E), 256, 0, stream>>>(ws.cnt, ws.totals, p.ntiles);
  build_lists_kernel<<<1, kListThreads, 0, stream>>>(ws.totals, ws.offs, ws.items, ws.counters, p.n, E);
  const int64_t threads = p.N * p.H;
  if (p.lmax > 0)
    scatter_kernel<<<static_cast<unsigned>((threads + 255) / 256), 256, 0, stream>>>(
        sel, ws.rk, ws.cnt, ws.offs, ws.qidx, ws.inv, p.N, p.H, p.B, p.n, p.topk, p.lmax, p.ntiles, p.blo);
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
