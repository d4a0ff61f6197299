// Block attention: every work item is one key block of one head and up to
// kAttnTile queries attending it (智东西 report, section 二, implementation step 3:
// attention per KV block over the queries routed to it). Two kinds of items:
//   * past-block items: queries gathered from the block's query list; no mask;
//   * own-block items: a run of consecutive queries of the block itself, with
//     the causal mask inside the block (keys up to the query's own position).
// Each item writes, per query, the softmax-normalised partial output over its
// keys and the partial log-sum-exp; the merge kernel combines them.
//
// bf16 kernel (gfx950): 8 waves per workgroup (two per SIMD), each wave owns
// one 32-query column block, 64-key tiles of K and V staged row-major in LDS
// (padded rows, double buffered through registers). Per wave and 32-key half
// tile:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, keys on the rows and queries on
//                 the columns; Q stays in registers as the B operand;
//   softmax       in registers per query column, exp2 with the 1/sqrt(D)
//                 scale folded into one FMA; the running maximum is only
//                 refreshed (and O rescaled) when it grows by more than 2^8,
//                 which keeps every exponent <= 8 and is exact after the final
//                 normalisation;
//   O^T += V^T P^T  P stays in registers as the B operand; the V^T operand is
//                 read with ds_read_b64_tr_b16 (LDS transpose read) in the key
//                 order the S accumulator layout hands to P.
// Workgroups are persistent; each XCD walks its own contiguous share of the
// item list through an atomic cursor, so the items of one key block run close
// together on one L2.
//
// fp32 kernel: one thread per query, K/V tiles in LDS, fp32 FMA throughout.
#include "common.h"
#include "kernels.h"

namespace moba {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The running maximum is refreshed only when it grows by more than this many
// powers of two.
constexpr float kRescaleThreshold = 8.0f;

template <typename T>
struct AttnArgs {
  const T* q;
  const T* k;
  const T* v;
  const int32_t* qidx;
  const WorkItem* items;
  int32_t* counters;
  T* part_diag;
  float* lse_diag;
  T* part_off;
  float* lse_off;
  int64_t N;
  int H, B, n;
  int qt_per_block;     // own-block items per block: ceil(B / kAttnTile)
  int64_t diag_items;   // H * n * qt_per_block
  float scale_log2;     // log2(e) / sqrt(D)
};

// Resolved work item.
struct Item {
  int h, b, count, q0;     // q0: first query position inside the block (own-block items)
  bool causal;
  int64_t list_start;      // past-block items: first list position
};

__device__ __forceinline__ bool next_item(const int32_t* counters, int32_t* cursor, int64_t diag_items,
                                          const WorkItem* items, int n, int qt_per_block, int B, int* s_it,
                                          Item* out) {
  const int xcd = blockIdx.x % kXcds;
  const int64_t n_off = counters[0];
  const int64_t oa = n_off * xcd / kXcds, ob = n_off * (xcd + 1) / kXcds;
  const int64_t da = diag_items * xcd / kXcds, db = diag_items * (xcd + 1) / kXcds;
  if (threadIdx.x == 0) *s_it = atomicAdd(cursor + kCursorStride * xcd, 1);
  __syncthreads();
  const int64_t it = *s_it;
  __syncthreads();
  if (it < ob - oa) {
    const WorkItem w = items[oa + it];
    out->h = w.h;
    out->b = w.b;
    out->count = w.count;
    out->q0 = 0;
    out->causal = false;
    out->list_start = w.start;
    return true;
  }
  const int64_t d = da + (it - (ob - oa));
  if (d >= db) return false;
  const int64_t e = d / qt_per_block;
  const int qt = static_cast<int>(d % qt_per_block);
  out->h = static_cast<int>(e / n);
  out->b = static_cast<int>(e % n);
  out->q0 = qt * kAttnTile;
  out->count = min(kAttnTile, B - out->q0);
  out->causal = true;
  out->list_start = 0;
  return true;
}

// ------------------------------------------------------------------------------------------
// bf16 MFMA kernel
// ------------------------------------------------------------------------------------------

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct Tile {
  static constexpr int kChunks = D / 8;                      // 16-byte chunks per key row
  static constexpr int kRowBytes = D * 2;
  // Padded LDS row strides. K rows get 16 extra bytes, so the 16 rows one
  // 16-byte-per-lane operand read touches per LDS cycle hit distinct banks;
  // V rows get 32, so the 4 rows x 32 bytes of one transpose read do. Plain
  // padding (not a swizzle) keeps every operand address an immediate offset
  // from one per-lane base.
  static constexpr int kKStride = kRowBytes + 16;
  static constexpr int kVStride = kRowBytes + 32;
  static constexpr int kKSlotsRow = kKStride / 16;
  static constexpr int kVSlotsRow = kVStride / 16;
  static constexpr int kKBytes = kKTile * kKStride;
  static constexpr int kVBytes = kKTile * kVStride;
  // Direct global->LDS loads (16 bytes per lane, 1 KB per wave instruction).
  // Every wave issues the same number per tile; instructions whose 1 KB
  // window lies past the end of a tile write into a 1 KB dump area that
  // follows the tile in the same LDS object.
  static constexpr int kDump = 1024;
  static constexpr int kKDma = (kKTile * kKSlotsRow + 511) / 512;
  static constexpr int kVDma = (kKTile * kVSlotsRow + 511) / 512;
  static constexpr int kDmaPerTile = kKDma + kVDma;
};

constexpr int kAttnThreads = 512;
constexpr int kStages = 4;          // LDS tile buffers; up to kStages - 1 tiles in flight

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate for "vmcnt(n)" with the other counters unconstrained (gfx9 encoding).
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Per-lane byte offsets (inside one tile of one tensor) of the direct
// global->LDS loads of this lane: load u fills slot (u * 8 + w) * 64 + lane of
// the tile's padded LDS image. Windows past the end of the tile re-load row 0
// and go to the dump area (see dma_tile). Padding slots re-load chunk 0.
template <int D, int kSlotsRow, int kDma>
__device__ __forceinline__ void dma_offsets(int64_t row_stride, uint32_t (&off)[kDma]) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  constexpr int kSlots = kKTile * kSlotsRow;
#pragma unroll
  for (int u = 0; u < kDma; ++u) {
    const int first = (u * 8 + w) * 64;
    const int slot = first < kSlots ? first + lane : lane;
    const int row = slot / kSlotsRow;
    int c = slot % kSlotsRow;
    c = c < Tile<D>::kChunks ? c : 0;
    off[u] = static_cast<uint32_t>((row * row_stride + 8 * c) * 2);
  }
}

// Issue the direct-to-LDS loads of one tensor tile whose first row is at the
// (wave-uniform) address `tile` into the LDS stage `lds` (tile image of
// kSlotsRow * 64 slots followed by the dump area).
//
// The loads are written as inline asm on purpose. With the compiler builtin,
// the compiler's wait-count pass cannot tell which ring stage a later LDS read
// touches and inserts "wait for every outstanding load" before reads, which
// drains the ring and exposes the full memory latency on most tiles. As asm
// the loads are invisible to that pass; every wait they need is explicit (see
// tile_step): each thread waits on the vector-memory counter for its own
// loads of a tile, then the workgroup barrier publishes the tile. The loads
// have no register results (they write LDS), so nothing the compiler
// allocates can be overwritten by a load in flight; M0 is written right before
// each load inside the same asm statement, with the one wait state a write of
// M0 needs before an LDS DMA.
template <int kSlotsRow, int kDma>
__device__ __forceinline__ void dma_tile(const bf16* tile, const uint32_t* off, char* lds) {
  const int w = threadIdx.x >> 6;
  constexpr int kSlots = kKTile * kSlotsRow;
  // The base is wave-uniform; move it to SGPRs. readfirstlane returns a signed
  // int: each half goes through uint32_t so that widening never sign-extends.
  const uint64_t base = reinterpret_cast<uint64_t>(tile);
  const uint32_t base_lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(base)));
  const uint32_t base_hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(base >> 32)));
  const uint64_t sbase = (static_cast<uint64_t>(base_hi) << 32) | static_cast<uint64_t>(base_lo);
#pragma unroll
  for (int u = 0; u < kDma; ++u) {
    const int first = (u * 8 + w) * 64;              // first slot of this wave's 1 KB window
    char* dst = lds + (first < kSlots ? first * 16 : kSlots * 16);
    // LDS byte offset of the window: the low half of the generic address of an
    // LDS object is its offset inside the workgroup's LDS allocation.
    const uint32_t m0 = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst)))));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(m0), "v"(off[u]), "s"(sbase)
                 : "memory");
  }
}

// One 64-key tile of work for one wave: S^T = K Q^T, online softmax and
// O^T += V^T P^T in two halves of 32 keys.
template <int D>
__device__ __forceinline__ void tile_compute(const char* ks, const char* vs, const bf16x8 (&qop)[D / 16],
                                             f32x16 (&o)[D / 32], float& m, float& l, int kt, bool causal,
                                             int first_pos, int qpos, int half, float c2, bool first_tile) {
  using T = Tile<D>;
  constexpr int kDC = D / 32;
  constexpr int kQC = D / 16;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const int kbase = kt * kKTile + 32 * kh;
    if (causal && kbase > first_pos + 31) break;   // the whole half is in the future
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int c = 0; c < kQC; ++c) {
      const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ks + 32 * kh * T::kKStride + 32 * c));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[c], s, 0, 0, 0);
    }
    if (causal && kbase + 31 > first_pos) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kbase + 8 * (r >> 2) + 4 * half + (r & 3) > qpos) s[r] = -INFINITY;
    }
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[r], s[r + 1]));
    mx = wave_max_pair(mx);
    const float m_new = fmaxf(m, mx);
    if (first_tile && kh == 0) {
      m = m_new;                         // O and l are still zero
    } else if (__builtin_amdgcn_ballot_w64((m_new - m) * c2 > kRescaleThreshold) != 0) {
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c2);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int c = 0; c < kDC; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
    }
    const float mc = m * c2;
    bf16x8 p[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -mc));
      l += e;
      p[r >> 3][r & 7] = static_cast<bf16>(e);
    }
#pragma unroll
    for (int dc = 0; dc < kDC; ++dc) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const char* vp = vs + (32 * kh + 16 * g) * T::kVStride + 64 * dc;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 8 * T::kVStride));
        const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo);
        const bf16x4 h4 = __builtin_bit_cast(bf16x4, hi);
        const bf16x8 va = {l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
        o[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[g], o[dc], 0, 0, 0);
      }
    }
  }
}

// The LDS tile ring. Each stage is a separate __shared__ object so that the
// compiler can tell a read of one stage from the direct-to-LDS writes still in
// flight into the others (it would otherwise wait for all of them).
template <int D> struct Ring {
  static constexpr int kK = Tile<D>::kKBytes + Tile<D>::kDump, kV = Tile<D>::kVBytes + Tile<D>::kDump;
};
#define MOBA_RING(D)                                                  \
  __shared__ __attribute__((aligned(16))) char k0[Ring<D>::kK];     \
  __shared__ __attribute__((aligned(16))) char k1[Ring<D>::kK];     \
  __shared__ __attribute__((aligned(16))) char k2[Ring<D>::kK];     \
  __shared__ __attribute__((aligned(16))) char k3[Ring<D>::kK];     \
  __shared__ __attribute__((aligned(16))) char v0[Ring<D>::kV];     \
  __shared__ __attribute__((aligned(16))) char v1[Ring<D>::kV];     \
  __shared__ __attribute__((aligned(16))) char v2[Ring<D>::kV];     \
  __shared__ __attribute__((aligned(16))) char v3[Ring<D>::kV];
static_assert(kStages == 4, "the ring below has four stages");

struct ItemCtx {
  const bf16* kblk;
  const bf16* vblk;
  int64_t tile_stride;
  int nkt, last_tile, first_pos, qpos;
  bool causal, has;
};

// One pipeline step: tile kt sits in stage (ks, vs); the loads of tile
// kt + kStages - 1 go to stage (kn, vn), which held tile kt - 1. Every step
// issues the same loads (a tile past the end re-loads the item's last tile
// into a stage nobody reads again), so exactly (kStages - 2) * kDmaPerTile
// loads are younger than tile kt's at the wait below.
template <int D>
__device__ __forceinline__ void tile_step(int kt, const ItemCtx& c, const char* ks, const char* vs, char* kn, char* vn,
                                          const uint32_t (&koff)[Tile<D>::kKDma],
                                          const uint32_t (&voff)[Tile<D>::kVDma], int k_lane, int v_lane,
                                          const bf16x8 (&qop)[D / 16], f32x16 (&o)[D / 32], float& m, float& l,
                                          int half, float c2) {
  using T = Tile<D>;
  __builtin_amdgcn_s_waitcnt(wait_vmcnt((kStages - 2) * T::kDmaPerTile));
  // Tile kt is in LDS for everyone and everyone is done reading tile kt - 1.
  // A bare barrier (no fence): the only LDS writes here are this thread's
  // direct loads, already waited for above, and a fence would also wait for
  // the later tiles still in flight. The memory clobber keeps the compiler
  // from moving LDS accesses across it.
  asm volatile("s_barrier" ::: "memory");
  const int nxt = min(kt + kStages - 1, c.last_tile);
  dma_tile<T::kKSlotsRow, T::kKDma>(c.kblk + nxt * c.tile_stride, koff, kn);
  dma_tile<T::kVSlotsRow, T::kVDma>(c.vblk + nxt * c.tile_stride, voff, vn);
  if (c.has && (!c.causal || kt * kKTile <= c.first_pos + 31))
    tile_compute<D>(ks + k_lane, vs + v_lane, qop, o, m, l, kt, c.causal, c.first_pos, c.qpos, half, c2, kt == 0);
}

template <int D>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_bf16_kernel(AttnArgs<bf16> a) {
  using T = Tile<D>;
  constexpr int kDC = D / 32;   // 32-row blocks of O^T
  constexpr int kQC = D / 16;   // 16-deep contraction steps of S
  MOBA_RING(D)
  __shared__ int s_it;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int qn = lane & 31;
  const int half = lane >> 5;
  const float c2 = a.scale_log2;
  // Per-lane LDS offsets of the operand reads. K operand (row qn, dims
  // 8*half..): one 16-byte read per 16 dims. V^T operand through the
  // transpose read: within each 16-lane group, lane (4*e + q) addresses key
  // row e of the group's 4 keys and dims 4*q..4*q+3 of the group's 16 dims.
  const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
  const int k_lane = qn * T::kKStride + 16 * half;
  const int v_lane = (4 * (tg >> 1) + te) * T::kVStride + 2 * (16 * (tg & 1) + 4 * tq);
  // Query block of this wave. Waves w and w + 4 share a SIMD; giving them
  // blocks w and 7 - w evens out the causal triangle of own-block items.
  const int qblk = w < 4 ? w : 11 - w;

  const int64_t row_stride = static_cast<int64_t>(a.H) * D;
  uint32_t koff[T::kKDma], voff[T::kVDma];
  dma_offsets<D, T::kKSlotsRow, T::kKDma>(row_stride, koff);
  dma_offsets<D, T::kVSlotsRow, T::kVDma>(row_stride, voff);

  Item item;
  while (next_item(a.counters, a.counters + kCursorStride, a.diag_items, a.items, a.n, a.qt_per_block, a.B, &s_it, &item)) {
    const int h = item.h;
    ItemCtx c;
    c.causal = item.causal;
    c.has = 32 * qblk < item.count;
    const int slot = 32 * qblk + qn;
    const int sc = slot < item.count ? slot : item.count - 1;
    const int64_t qrow = item.causal ? static_cast<int64_t>(item.b) * a.B + item.q0 + sc
                                     : static_cast<int64_t>(a.qidx[item.list_start + sc]);
    c.first_pos = item.q0 + 32 * qblk;   // own-block items: position of the block's first query
    c.qpos = item.q0 + slot;
    c.nkt = item.causal ? (item.q0 + item.count + kKTile - 1) / kKTile : a.B / kKTile;
    c.last_tile = c.nkt - 1;
    c.tile_stride = static_cast<int64_t>(kKTile) * row_stride;
    c.kblk = a.k + (static_cast<int64_t>(item.b) * a.B * a.H + h) * D;
    c.vblk = a.v + (static_cast<int64_t>(item.b) * a.B * a.H + h) * D;

    // The first kStages - 1 tiles, then the Q operands, then one full wait:
    // Q and the first tiles arrive together, and from here on the compiler
    // sees no load of its own in flight, so it adds no waits inside the tile
    // loop (the ring loads are managed by the explicit waits in tile_step).
    dma_tile<T::kKSlotsRow, T::kKDma>(c.kblk, koff, k0);
    dma_tile<T::kVSlotsRow, T::kVDma>(c.vblk, voff, v0);
    dma_tile<T::kKSlotsRow, T::kKDma>(c.kblk + min(1, c.last_tile) * c.tile_stride, koff, k1);
    dma_tile<T::kVSlotsRow, T::kVDma>(c.vblk + min(1, c.last_tile) * c.tile_stride, voff, v1);
    dma_tile<T::kKSlotsRow, T::kKDma>(c.kblk + min(2, c.last_tile) * c.tile_stride, koff, k2);
    dma_tile<T::kVSlotsRow, T::kVDma>(c.vblk + min(2, c.last_tile) * c.tile_stride, voff, v2);
    bf16x8 qop[kQC];
    {
      const bf16* qp = a.q + (qrow * a.H + h) * D + 8 * half;
#pragma unroll
      for (int cc = 0; cc < kQC; ++cc) qop[cc] = load_bf16x8(qp + 16 * cc);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));

    f32x16 o[kDC];
#pragma unroll
    for (int cc = 0; cc < kDC; ++cc)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[cc][r] = 0.f;
    float m = -INFINITY;   // running maximum of the raw scores (shared by the lane pair of a query)
    float l = 0.f;         // this lane's share of the softmax denominator

    for (int kt = 0; kt < c.nkt; kt += kStages) {
      tile_step<D>(kt, c, k0, v0, k3, v3, koff, voff, k_lane, v_lane, qop, o, m, l, half, c2);
      if (kt + 1 >= c.nkt) break;
      tile_step<D>(kt + 1, c, k1, v1, k0, v0, koff, voff, k_lane, v_lane, qop, o, m, l, half, c2);
      if (kt + 2 >= c.nkt) break;
      tile_step<D>(kt + 2, c, k2, v2, k1, v1, koff, voff, k_lane, v_lane, qop, o, m, l, half, c2);
      if (kt + 3 >= c.nkt) break;
      tile_step<D>(kt + 3, c, k3, v3, k2, v2, koff, voff, k_lane, v_lane, qop, o, m, l, half, c2);
    }

    // ---- epilogue: normalise, stage the wave's 32 x D output block in LDS
    // (the ring is free once everyone is past the last tile) and write whole
    // rows: an item's partial rows are consecutive in memory, so each wave
    // stores one contiguous run of 32 rows. ----
    const float l_tot = l + __shfl_xor(l, 32);
    const float inv_l = 1.f / l_tot;
    // Retire this thread's loads (the last steps re-load tiles into stages no
    // one reads; they must not land on the staged output), then wait for all
    // waves to be done with the ring.
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    asm volatile("s_barrier" ::: "memory");
    char* stage = (w < 2 ? k0 : w < 4 ? k1 : w < 6 ? k2 : k3) + (w & 1) * (32 * 2 * D);
#pragma unroll
    for (int cc = 0; cc < kDC; ++cc) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bf16x4 vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = static_cast<bf16>(o[cc][4 * i + e] * inv_l);
        *reinterpret_cast<uint2*>(stage + (qn * D + 32 * cc + 8 * i + 4 * half) * 2) = __builtin_bit_cast(uint2, vv);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
    if (c.has) {
      const int rows = min(32, item.count - 32 * qblk);          // valid rows of this wave's block
      const int64_t orow0 = item.causal ? static_cast<int64_t>(h) * a.N + static_cast<int64_t>(item.b) * a.B +
                                              item.q0 + 32 * qblk
                                        : item.list_start + 32 * qblk;
      bf16* po = (item.causal ? a.part_diag : a.part_off) + orow0 * D;
      constexpr int kRowChunks = D / 8;                            // 16-byte chunks per row
      constexpr int kRowsPerPass = 64 / kRowChunks;
#pragma unroll
      for (int r0 = 0; r0 < 32; r0 += kRowsPerPass) {
        const int r = r0 + lane / kRowChunks;
        const int ch = lane % kRowChunks;
        if (r < rows)
          *reinterpret_cast<uint4*>(po + r * D + 8 * ch) = *reinterpret_cast<const uint4*>(stage + (r * D + 8 * ch) * 2);
      }
      if (half == 0 && slot < item.count) {
        float* pl = (item.causal ? a.lse_diag : a.lse_off) + orow0;
        pl[qn] = (m * c2 + log2f(l_tot)) * kLn2;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// fp32 kernel
// ------------------------------------------------------------------------------------------

constexpr int kF32Keys = 32;

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs<float> a) {
  __shared__ float sk[kF32Keys][D];
  __shared__ float sv[kF32Keys][D];
  __shared__ int s_it;
  const int tid = threadIdx.x;
  const int64_t row_stride = static_cast<int64_t>(a.H) * D;

  Item item;
  while (next_item(a.counters, a.counters + kCursorStride, a.diag_items, a.items, a.n, a.qt_per_block, a.B, &s_it, &item)) {
    const int h = item.h;
    const bool valid = tid < item.count;
    const int qs = valid ? tid : item.count - 1;
    const int64_t qrow = item.causal ? static_cast<int64_t>(item.b) * a.B + item.q0 + qs
                                     : static_cast<int64_t>(a.qidx[item.list_start + qs]);
    const int qpos = item.q0 + tid;
    float qr[D], o[D];
    const float* qp = a.q + (qrow * a.H + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      qr[d] = qp[d];
      o[d] = 0.f;
    }
    float m_run = -INFINITY, l_run = 0.f;
    const int keys = item.causal ? item.q0 + item.count : a.B;
    const float* kblk = a.k + (static_cast<int64_t>(item.b) * a.B * a.H + h) * D;
    const float* vblk = a.v + (static_cast<int64_t>(item.b) * a.B * a.H + h) * D;
    for (int k0 = 0; k0 < keys; k0 += kF32Keys) {
      for (int i = tid; i < kF32Keys * D / 4; i += 256) {
        const int r = i / (D / 4), c4 = i % (D / 4);
        const int64_t off = static_cast<int64_t>(k0 + r) * row_stride + 4 * c4;
        const bool in = k0 + r < a.B;
        const float4 kv = in ? *reinterpret_cast<const float4*>(kblk + off) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 vv = in ? *reinterpret_cast<const float4*>(vblk + off) : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(&sk[r][4 * c4]) = kv;
        *reinterpret_cast<float4*>(&sv[r][4 * c4]) = vv;
      }
      __syncthreads();
      if (valid) {
        float x[kF32Keys];
        float mx = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < kF32Keys; ++kk) {
          float s = 0.f;
#pragma unroll
          for (int d = 0; d < D; ++d) s = fmaf(qr[d], sk[kk][d], s);
          s *= a.scale_log2;
          const int kpos = k0 + kk;
          if (kpos >= keys || (item.causal && kpos > qpos)) s = -INFINITY;
          x[kk] = s;
          mx = fmaxf(mx, s);
        }
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
        for (int kk = 0; kk < kF32Keys; ++kk) {
          const float p = exp2f(x[kk] - m_new);
          l_run += p;
#pragma unroll
          for (int d = 0; d < D; ++d) o[d] = fmaf(p, sv[kk][d], o[d]);
        }
      }
      __syncthreads();
    }
    if (valid) {
      const int64_t orow = item.causal ? static_cast<int64_t>(h) * a.N + qrow : item.list_start + tid;
      float* po = (item.causal ? a.part_diag : a.part_off) + orow * D;
      const float inv_l = 1.f / l_run;
#pragma unroll
      for (int d = 0; d < D; ++d) po[d] = o[d] * inv_l;
      (item.causal ? a.lse_diag : a.lse_off)[orow] = (m_run + log2f(l_run)) * kLn2;
    }
  }
}

template <typename T>
AttnArgs<T> make_args(const Problem& p, const void* q, const void* k, const void* v, const Workspace& ws) {
  AttnArgs<T> a;
  a.q = static_cast<const T*>(q);
  a.k = static_cast<const T*>(k);
  a.v = static_cast<const T*>(v);
  a.qidx = ws.qidx;
  a.items = ws.items;
  a.counters = ws.counters;
  a.part_diag = static_cast<T*>(ws.part_diag);
  a.lse_diag = ws.lse_diag;
  a.part_off = static_cast<T*>(ws.part_off);
  a.lse_off = ws.lse_off;
  a.N = p.N;
  a.H = p.H;
  a.B = p.B;
  a.n = p.n;
  a.qt_per_block = (p.B + kAttnTile - 1) / kAttnTile;
  a.diag_items = p.diag_items;
  a.scale_log2 = kLog2e / sqrtf(static_cast<float>(p.D));
  return a;
}

}  // namespace

hipError_t launch_attention(const Problem& p, const void* q, const void* k, const void* v, const Workspace& ws,
                            int num_cus, hipStream_t stream) {
  const int64_t total = p.max_items + p.diag_items;
  int64_t grid = static_cast<int64_t>(num_cus) * (p.is_f32 ? 2 : 1);
  grid = std::min<int64_t>(grid, ((total + kXcds - 1) / kXcds) * kXcds);
  if (p.is_f32) {
    auto a = make_args<float>(p, q, k, v, ws);
    if (p.D == 128)
      attn_f32_kernel<128><<<static_cast<unsigned>(grid), 256, 0, stream>>>(a);
    else
      attn_f32_kernel<64><<<static_cast<unsigned>(grid), 256, 0, stream>>>(a);
  } else {
    auto a = make_args<bf16>(p, q, k, v, ws);
    if (p.D == 128)
      attn_bf16_kernel<128><<<static_cast<unsigned>(grid), kAttnThreads, 0, stream>>>(a);
    else
      attn_bf16_kernel<64><<<static_cast<unsigned>(grid), kAttnThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moba
