// Gate and causal top-k (with the first half of the per-block query lists).
//
// For query t in block j the gate score of past block i < j is <q_t, kbar_i>
// in fp32, with no scale (pomoai MoBA overview, "核心原理" step 2; 智东西 report,
// section 二, relevance score). The current block j is always kept and the
// topk - 1 best past blocks are added, ranked by score and then by lower block
// index; future blocks are never scored (wzjinhao.cn MoBA article, section 3,
// causal_mask and current_block_force). Rows with j < topk keep all of 0..j.
//
// bf16 path: persistent workgroups of 4 waves x 32 queries (one 128-query
// tile at a time), each owning one head and walking every grid.x-th tile of
// it. The scores of 32 blocks x 32
// queries come from bf16 MFMA (v_mfma_f32_32x32x16_bf16) with the block means
// as the A operand (rows = blocks) and the queries as the B operand (columns =
// queries), so each lane ends up holding 16 block scores of one query. The
// fp32 mean is fed as its exact 3-way bf16 split (hi + mid + lo), and since q
// is bf16 every product is exact and the score carries only fp32 accumulation
// error. The head's split means are staged once in LDS (padded rows, so the
// 16-byte operand reads of 16 rows hit distinct banks) when they fit, else
// read from L2; the next tile pair's queries are loaded while the current one
// is scored. Each lane keeps a sorted register list of the best keys and
// merges it with the lane 32 away, which holds the other 16 blocks.
//
// fp32 path: the same lane layout, but each lane forms full fp32 dot products
// for every other block with vector FMAs.
//
// When the query lists are wanted, the workgroup also records, per past block,
// which of its 128 queries kept it (an LDS bitmap built with integer ORs), and
// writes the per-tile count and each query's rank inside the tile. The lists
// come out ordered by query position, independent of scheduling.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moba {

namespace {

struct GateArgs {
  int32_t* sel;
  int32_t* cnt;   // null: no query-list bookkeeping
  int32_t* rk;
  int64_t N;
  int H, B, n, topk, lmax, ntiles;
  const int32_t* blo;   // first block of each block's sequence (packed sequences) or nullptr
};

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), m);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), m);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Per-lane running top-KCAP of (score, block), best first, for the bf16
// path: blocks arrive in increasing order within a lane, so a plain
// "strictly greater" test leaves equal scores in block order (lower block
// first), as the ranking requires. Empty slots hold -inf. -0 and +0 compare
// equal, as in the orderable key.
template <int KCAP>
struct ScoreList {
  float s[KCAP];
  int b[KCAP];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < KCAP; ++i) {
      s[i] = -INFINITY;
      b[i] = 0;
    }
  }
  // Insert a block later in order than every block already held.
  __device__ __forceinline__ void push(float x, int blk) {
    bool gt[KCAP];
#pragma unroll
    for (int i = 0; i < KCAP; ++i) gt[i] = x > s[i];
#pragma unroll
    for (int i = KCAP - 1; i > 0; --i) {
      s[i] = gt[i - 1] ? s[i - 1] : (gt[i] ? x : s[i]);
      b[i] = gt[i - 1] ? b[i - 1] : (gt[i] ? blk : b[i]);
    }
    s[0] = gt[0] ? x : s[0];
    b[0] = gt[0] ? blk : b[0];
  }
  // The 64-bit ranking keys (0 for empty slots), merged with the lane 32
  // away, which holds the other blocks of the same query.
  __device__ __forceinline__ void to_keys(uint64_t (&list)[KCAP]) const {
#pragma unroll
    for (int i = 0; i < KCAP; ++i) list[i] = s[i] > -INFINITY ? rank_key(s[i], b[i]) : 0ull;
  }
};

template <int KCAP>
__device__ __forceinline__ void merge_with_partner(uint64_t (&list)[KCAP]) {
  uint64_t other[KCAP];
#pragma unroll
  for (int s = 0; s < KCAP; ++s) other[s] = shfl_xor_u64(list[s], 32);
#pragma unroll
  for (int s = 0; s < KCAP; ++s) topk_insert<KCAP>(list, other[s]);
}

// Writes the selection row of this lane's query and, if requested, the query
// list bookkeeping. Called by all 256 threads of the workgroup (it has barriers).
template <int KCAP>
__device__ __forceinline__ void finalize(const GateArgs& a, const uint64_t (&list)[KCAP], int64_t t, bool valid,
                                         int j, int lo, uint32_t* bm, int tile) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int qn = lane & 31;
  const int half = lane >> 5;
  const int h = blockIdx.y;
  const int topk = a.topk;
  const bool ranked = j - lo >= topk;   // more eligible past blocks than slots: the gate decides
  const int nk = topk - 1;         // past blocks kept when ranked

  // Position of each kept past block in ascending block order.
  int pos[KCAP];
#pragma unroll
  for (int s = 0; s < KCAP; ++s) {
    int p = 0;
#pragma unroll
    for (int u = 0; u < KCAP; ++u)
      p += (u < nk && key_block(list[u]) < key_block(list[s])) ? 1 : 0;
    pos[s] = p;
  }

  if (valid && half == 0) {
    int32_t* srow = a.sel + (static_cast<int64_t>(h) * a.N + t) * topk;
    if (!ranked) {
      for (int s = 0; s < topk; ++s) srow[s] = lo + s <= j ? lo + s : -1;
    } else {
#pragma unroll
      for (int s = 0; s < KCAP; ++s)
        if (s < nk) srow[pos[s]] = key_block(list[s]);
      srow[nk] = j;
    }
  }

  if (a.cnt == nullptr) return;

  const int n = a.n;
  for (int i = threadIdx.x; i < 4 * n; i += 256) bm[i] = 0u;
  __syncthreads();
  if (valid && half == 0) {
    uint32_t* mine = bm + w * n;
    const uint32_t bit = 1u << qn;
    if (!ranked) {
      for (int b = lo; b < j; ++b) atomicOr(mine + b, bit);
    } else {
#pragma unroll
      for (int s = 0; s < KCAP; ++s)
        if (s < nk) atomicOr(mine + key_block(list[s]), bit);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < n; b += 256) {
    const int c = __popc(bm[b]) + __popc(bm[n + b]) + __popc(bm[2 * n + b]) + __popc(bm[3 * n + b]);
    a.cnt[(static_cast<int64_t>(h) * n + b) * a.ntiles + tile] = c;
  }
  if (valid && half == 0) {
    int32_t* rrow = a.rk + (static_cast<int64_t>(h) * a.N + t) * a.lmax;
    const uint32_t below = (1u << qn) - 1u;
    auto rank_of = [&](int b) {
      int r = __popc(bm[w * n + b] & below);
      for (int u = 0; u < w; ++u) r += __popc(bm[u * n + b]);
      return r;
    };
    if (!ranked) {
      for (int b = lo; b < j; ++b) rrow[b - lo] = rank_of(b);
    } else {
#pragma unroll
      for (int s = 0; s < KCAP; ++s)
        if (s < nk) rrow[pos[s]] = rank_of(key_block(list[s]));
    }
  }
}

// Bytes of one block's row of split means in LDS: 3 pieces of D bf16 plus 16
// bytes of padding (row stride = 4 banks mod 64).
template <int D>
constexpr int gate_lds_row() { return 3 * D * 2 + 16; }
constexpr int kGateLdsPieces = 64 * 1024;      // largest LDS image of the split means
constexpr int kGateBitmapDouble = 64 * 1024;   // largest double-buffered bitmap (2 x 4n words)

template <int D, int KCAP, bool kLds>
__global__ __launch_bounds__(256) void gate_mfma_kernel(const bf16* __restrict__ q, const bf16* __restrict__ pieces,
                                                        GateArgs a) {
  extern __shared__ __attribute__((aligned(16))) char gsm[];
  constexpr int kRow = gate_lds_row<D>();
  const int n = a.n;
  const int h = blockIdx.y;
  char* const plds = gsm;
  // Query-list bitmaps: two buffers of 4n words when they fit (a buffer is
  // then rewritten two iterations after it was read), else one buffer and an
  // extra barrier per iteration.
  uint32_t* const bmb = reinterpret_cast<uint32_t*>(gsm + (kLds ? n * kRow : 0));
  const bool two_bm = a.cnt != nullptr && 32 * n <= kGateBitmapDouble;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int qn = lane & 31;
  const int half = lane >> 5;
  const bf16* hp = pieces + static_cast<int64_t>(h) * n * 3 * D;
  if (kLds) {
    constexpr int kChunks = 3 * D / 8;   // 16-byte chunks per block row
    for (int i = threadIdx.x; i < n * kChunks; i += 256) {
      const int row = i / kChunks, c = i - row * kChunks;
      *reinterpret_cast<uint4*>(plds + row * kRow + 16 * c) = load_u4(hp + static_cast<int64_t>(row) * 3 * D + 8 * c);
    }
    __syncthreads();
  }
  auto load_q = [&](int tile, bf16x8 (&op)[D / 16]) {
    const int64_t t = static_cast<int64_t>(tile) * kQTile + w * 32 + qn;
    const int64_t tc = t < a.N ? t : a.N - 1;
    const bf16* qrow = q + (tc * a.H + h) * D + 8 * half;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) op[c] = load_bf16x8(qrow + 16 * c);
  };
  bf16x8 qop[D / 16];
  load_q(blockIdx.x, qop);
  int buf = 0;
  for (int tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int64_t t0w = static_cast<int64_t>(tile) * kQTile + w * 32;
    const int64_t t = t0w + qn;
    const bool valid = t < a.N;
    const int64_t tc = valid ? t : a.N - 1;
    const int j = static_cast<int>(tc / a.B);
    const int lo = a.blo != nullptr ? a.blo[j] : 0;   // first block of the query's sequence
    const int64_t tlast = (t0w + 31 < a.N) ? t0w + 31 : a.N - 1;
    const int jw = static_cast<int>(tlast / a.B);   // largest block of the wave
    // Next tile's queries, in flight while this tile is scored.
    bf16x8 qnext[D / 16];
    const int nxt = tile + static_cast<int>(gridDim.x);
    load_q(nxt < a.ntiles ? nxt : tile, qnext);

    uint64_t list[KCAP];
#pragma unroll
    for (int s = 0; s < KCAP; ++s) list[s] = 0;
    if (jw >= a.topk && a.topk > 1 && t0w < a.N) {
      ScoreList<KCAP> sl;
      sl.clear();
      for (int bc = 0; bc * 32 < jw; ++bc) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        const int brow = min(bc * 32 + qn, n - 1);
#pragma unroll
        for (int pc = 0; pc < 3; ++pc) {
          // All operands of one piece are read before its products, so the
          // reads overlap one another instead of each product waiting for its own.
          bf16x8 av[D / 16];
#pragma unroll
          for (int c = 0; c < D / 16; ++c)
            av[c] = kLds ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                               plds + brow * kRow + pc * D * 2 + 32 * c + 16 * half))
                         : load_bf16x8(hp + static_cast<int64_t>(brow) * 3 * D + pc * D + 16 * c + 8 * half);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int c = 0; c < D / 16; ++c) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[c], qop[c], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int b = bc * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          sl.push(b < j && b >= lo ? acc[r] : -INFINITY, b);
        }
      }
      sl.to_keys(list);
      merge_with_partner<KCAP>(list);
    }
    finalize<KCAP>(a, list, t, valid, j, lo, bmb + buf * 4 * n, tile);
    if (two_bm) buf ^= 1;
    else if (a.cnt != nullptr) __syncthreads();
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qop[c] = qnext[c];
  }
}

template <int D, int KCAP>
__global__ __launch_bounds__(256) void gate_f32_kernel(const float* __restrict__ q, const float* __restrict__ kbar,
                                                       GateArgs a) {
  extern __shared__ uint32_t bm[];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int qn = lane & 31;
  const int half = lane >> 5;
  const int h = blockIdx.y;
  const int64_t t0w = static_cast<int64_t>(blockIdx.x) * kQTile + w * 32;
  const int64_t t = t0w + qn;
  const bool valid = t < a.N;
  const int64_t tc = valid ? t : a.N - 1;
  const int j = static_cast<int>(tc / a.B);
  const int lo = a.blo != nullptr ? a.blo[j] : 0;
  const int64_t tlast = (t0w + 31 < a.N) ? t0w + 31 : a.N - 1;
  const int jw = static_cast<int>(tlast / a.B);

  uint64_t list[KCAP];
#pragma unroll
  for (int s = 0; s < KCAP; ++s) list[s] = 0;

  if (jw >= a.topk && a.topk > 1 && t0w < a.N) {
    float qr[D];
    const float* qrow = q + (tc * a.H + h) * D;
#pragma unroll
    for (int d = 0; d < D; d += 4) {
      const float4 x = *reinterpret_cast<const float4*>(qrow + d);
      qr[d] = x.x; qr[d + 1] = x.y; qr[d + 2] = x.z; qr[d + 3] = x.w;
    }
    for (int b = half; b < jw; b += 2) {
      const float* kb = kbar + (static_cast<int64_t>(h) * a.n + b) * D;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qr[d], kb[d], s);
      topk_insert<KCAP>(list, b < j && b >= lo ? rank_key(s, b) : 0ull);
    }
    merge_with_partner<KCAP>(list);
  }
  finalize<KCAP>(a, list, t, valid, j, lo, bm, blockIdx.x);
}

template <int D, int KCAP>
hipError_t launch_gate_t(const Problem& p, const void* q, const Workspace& ws, int32_t* sel, bool csr, int num_cus,
                         hipStream_t stream) {
  GateArgs a;
  a.sel = sel;
  a.cnt = csr ? ws.cnt : nullptr;
  a.rk = csr ? ws.rk : nullptr;
  a.N = p.N;
  a.H = p.H;
  a.B = p.B;
  a.n = p.n;
  a.topk = p.topk;
  a.lmax = p.lmax;
  a.ntiles = p.ntiles;
  a.blo = p.blo;
  if (p.is_f32) {
    dim3 grid(p.ntiles, p.H);
    const size_t smem = csr ? static_cast<size_t>(4) * p.n * sizeof(uint32_t) : 0;
    gate_f32_kernel<D, KCAP><<<grid, 256, smem, stream>>>(static_cast<const float*>(q), ws.kbar, a);
    return hipGetLastError();
  }
  // Persistent: three workgroups per CU (as many as the staged means of a
  // 64-block head leave room for in LDS) over all heads, each walking every
  // grid.x-th tile of its head.
  const int per_head = std::max(1, std::min(p.ntiles, (3 * num_cus + p.H - 1) / p.H));
  dim3 grid(per_head, p.H);
  const size_t lds_pieces = static_cast<size_t>(p.n) * gate_lds_row<D>();
  const size_t bm1 = static_cast<size_t>(4) * p.n * sizeof(uint32_t);
  const size_t bm = !csr ? 0 : (2 * bm1 <= static_cast<size_t>(kGateBitmapDouble) ? 2 * bm1 : bm1);
  if (lds_pieces <= kGateLdsPieces)
    gate_mfma_kernel<D, KCAP, true><<<grid, 256, lds_pieces + bm, stream>>>(static_cast<const bf16*>(q), ws.kpieces, a);
  else
    gate_mfma_kernel<D, KCAP, false><<<grid, 256, bm, stream>>>(static_cast<const bf16*>(q), ws.kpieces, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_gate_d(const Problem& p, const void* q, const Workspace& ws, int32_t* sel, bool csr, int num_cus,
                         hipStream_t stream) {
  const int need = p.topk - 1;  // ranked slots (only used when a row has more past blocks than that)
  if (need <= 2) return launch_gate_t<D, 2>(p, q, ws, sel, csr, num_cus, stream);
  if (need <= 4) return launch_gate_t<D, 4>(p, q, ws, sel, csr, num_cus, stream);
  if (need <= 8) return launch_gate_t<D, 8>(p, q, ws, sel, csr, num_cus, stream);
  if (need <= 12) return launch_gate_t<D, 12>(p, q, ws, sel, csr, num_cus, stream);
  if (need <= 16) return launch_gate_t<D, 16>(p, q, ws, sel, csr, num_cus, stream);
  return launch_gate_t<D, 32>(p, q, ws, sel, csr, num_cus, stream);
}

}  // namespace

hipError_t launch_gate(const Problem& p, const void* q, const Workspace& ws, int32_t* sel, bool csr, int num_cus,
                       hipStream_t stream) {
  return p.D == 128 ? launch_gate_d<128>(p, q, ws, sel, csr, num_cus, stream)
                    : launch_gate_d<64>(p, q, ws, sel, csr, num_cus, stream);
}

}  // namespace moba
