// Block attention: every work item is one key block of one head and up to
// kAttnTile queries attending it (智东西 report, section 二, implementation step 3:
// attention per KV block over the queries routed to it). Two kinds of items:
//   * past-block items: queries gathered from the block's query list; no mask;
//   * own-block items: a run of consecutive queries of the block itself, with
//     the causal mask inside the block (keys up to the query's own position).
// Each past-block item writes, per query, the softmax-normalised partial
// output over its keys and the partial log-sum-exp. The LSE merge of those
// partials runs inside the own-block items when every query keeps at most
// kFusedMaxPast past blocks, else in the merge kernel after both passes.
//
// bf16 kernel (gfx950): 8 waves per workgroup (two per SIMD), each wave owns
// one 32-query column block of the item's 256 queries. Q tiles and the 64-key
// K and V tiles are brought straight from HBM into LDS by buffer-to-LDS loads
// (global_load_lds_dwordx4) through a 3-slot ring whose loads run two steps
// ahead, across item boundaries. Per wave and 32-key half tile:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, keys on the rows and queries on
//                 the columns; Q stays in registers as the B operand;
//   softmax       in registers per query column, exp2 with the 1/sqrt(D)
//                 scale folded into one FMA against a running reference; the
//                 reference is only raised (and O rescaled) when a half's
//                 probabilities sum past 2^64 or are not finite, which is
//                 rare and exact after the final normalisation;
//   O^T += V^T P^T  P stays in registers as the B operand; the V^T operand is
//                 read with ds_read_b64_tr_b16 (LDS transpose read) in the key
//                 order the S accumulator layout hands to P.
// The schedule is static and XCD-aware: each XCD takes a contiguous share of
// the past-block items, so the items of one key block run close together on
// one L2 (details above the kernel).
//
// fp32 kernel: one thread per query, K/V tiles in LDS, fp32 FMA throughout;
// its workgroups take items through a per-XCD atomic cursor.
#include "common.h"
#include "kernels.h"

namespace moba {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
struct AttnArgs {
  const T* q;
  const T* k;
  const T* v;
  const int32_t* qidx;
  const int32_t* inv;   // [H][N][lmax] list position of each past-block selection
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
  int64_t p_off;        // past-block list entries (rows of part_off before the dump rows)
  int64_t own_items;    // own-block items of the MFMA kernel: H * n * ceil(B / kAttnTile)
  int topk, lmax;
  const int32_t* blo;   // first block of each block's sequence (packed sequences) or nullptr
  T* out;               // final output [N][H][D] (own-block kernel with the merge fused in)
  float* lse_out;       // final lse [H][N]
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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;                  // two waves per SIMD, 32 queries each
constexpr int kThreads = kWaves * kWave;
constexpr int kSlots = 3;                  // LDS ring slots
constexpr int kAhead = kSlots - 1;         // loads run this many steps ahead, into the slot of
                                           // the previous step (all its reads are consumed
                                           // within that step)
static_assert(kAhead == 2, "the wait counts below track the two previous steps");
// Per-wave staging of the item's output rows: 32 rows of 64 dims (128 bytes,
// 16-byte chunks swizzled by row), so that the rows leave in full 128-byte lines.
constexpr int kStageBytes = 32 * 128;
constexpr int kQTileRows = kAttnTile / 2;  // queries per Q tile (the first or last four waves)
constexpr int kQBuf = 2 * kAttnTile;       // query-index entries per buffer (one 4-byte load per lane)
// Own-block items with the merge fused in: list positions of the item's past
// selections, [query][lmax], loaded into LDS in kInvRounds 4-byte loads per lane.
constexpr int kFusedMaxPast = 16;
constexpr int kInvInts = kAttnTile * kFusedMaxPast;
constexpr int kInvRounds = kInvInts / (kWaves * kWave);

// LDS image of one ring slot. A slot holds either one 64-key tile of K and V
// (row-major, keys on rows) or 128 query rows. Rows are padded (K and Q by
// 16 bytes, V by 32) so that the 16-byte operand reads of consecutive rows
// (K, Q) fall on distinct banks; of the paddings tried for V (16, 32, 48
// bytes) 32 gave the fastest past-block launch. The slot is filled in
// 1 KB windows (one 16-byte load per lane); wave w takes windows w, w + 8, ...
template <int D>
struct Lay {
  static constexpr int kKStride = 2 * D + 16;
  static constexpr int kVStride = 2 * D + 32;
  static constexpr int kKBytes = kKTile * kKStride;
  static constexpr int kVBytes = kKTile * kVStride;
  static constexpr int kKSlots16 = kKStride / 16;   // 16-byte units per padded row
  static constexpr int kVSlots16 = kVStride / 16;
  // Windows per slot: a multiple of 8 plus 4, so that exactly waves 0-3 take
  // one more round than waves 4-7 (the partial steps below rely on it).
  static constexpr int kWindows = ((kKBytes + kVBytes + 1023) / 1024 + 3) / 8 * 8 + 4;
  static constexpr int kSlot = kWindows * 1024;
  static constexpr int kRoundsHi = (kWindows + kWaves - 1) / kWaves;   // loads per step, waves < kWindows % 8
  static constexpr int kRoundsLo = kWindows / kWaves;                  // loads per step, the others
  static constexpr int kChunks = D / 8;             // 16-byte chunks of one row
  // Partial steps (own-block items with the merge fused in): per query of the
  // item, kPC 32-dim blocks of one past partial row (kSegChunks 16-byte
  // chunks, swizzled by query), then the partials' log-sum-exps (one float per
  // query) in the windows of round kRoundsLo, which only waves 0-3 take.
  static constexpr int kPC = D == 128 ? 2 : 1;
  static constexpr int kSegChunks = kPC * 4;
  static constexpr int kLseOff = kAttnTile * kSegChunks * 16;
  static_assert(kWindows % kWaves == 4, "waves 0-3 take one more round");
  static_assert(kLseOff == kRoundsLo * kWaves * 1024, "the log-sum-exps fill the last round");
  static_assert(kQTileRows * kKStride <= kSlot, "a Q tile must fit one slot");
  static_assert((kKBytes / 16) % 64 == 0, "K/V boundary must fall on a window");
};

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate for "vmcnt(n)" with the other counters unconstrained (gfx9 encoding).
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  // The low half of the generic address of an LDS object is its offset in the
  // workgroup's LDS allocation.
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(x)));
}

__device__ __forceinline__ uint64_t uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  // readfirstlane works on 32-bit ints; each half goes through uint32_t so
  // that widening never sign-extends.
  const uint32_t lo = uniform_u32(static_cast<uint32_t>(v));
  const uint32_t hi = uniform_u32(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// The direct global->LDS loads and the partial-output stores are inline asm on
// purpose: the kernel keeps its own exact count of vector-memory operations in
// flight (every wave issues the same sequence) and waits on that count, so no
// memory operation may be hidden from, added to or merged by the compiler's
// wait-count pass. None of them has a register result, so nothing the compiler
// allocates can be overwritten by an operation in flight. M0 is written in the
// same statement as the load that reads it, with the one wait state that an
// LDS DMA needs after an M0 write.
//
// They carry no "memory" clobber: the only compiler-visible memory they touch
// is LDS, and a load always targets a slot no wave reads in the current ring
// step; every ordering that matters (reads of a slot after the barrier that
// publishes it, and before the barrier after which it is reloaded) is fixed by
// the barrier statements, which do clobber memory. Without the clobber the
// compiler may read the (read-only) work list through scalar loads.
__device__ __forceinline__ void dma16(uint32_t m0, uint32_t voff, uint64_t sbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(uniform_u32(m0)), "v"(voff), "s"(sbase));
}

__device__ __forceinline__ void dma16_addr(uint32_t m0, const void* addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(uniform_u32(m0)), "v"(addr));
}

__device__ __forceinline__ void dma4(uint32_t m0, uint32_t voff, uint64_t sbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(uniform_u32(m0)), "v"(voff), "s"(sbase));
}

typedef int i32x4v __attribute__((ext_vector_type(4)));

// Stores read their data registers at issue; the trailing s_nop covers the
// wait state before those registers may be rewritten.
__device__ __forceinline__ void store16(void* addr, uint4 d) {
  const i32x4v data = {static_cast<int>(d.x), static_cast<int>(d.y), static_cast<int>(d.z), static_cast<int>(d.w)};
  asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" ::"v"(addr), "v"(data));
}

__device__ __forceinline__ void store4(void* addr, float data) {
  asm volatile("global_store_dword %0, %1, off\n\ts_nop 1" ::"v"(addr), "v"(data));
}

// One work item as the kernel sees it. Past-block items: head h, block b, list
// entries [start, start + count). Own-block items: queries [start, start +
// count) of block b. nkt: 64-key tiles to visit; np: partial steps (own-block
// items with the merge fused in: two per past selection of the block's queries).
struct Desc {
  int h, b, start, count, nkt, np;
  int64_t kv_row;   // the block's first key / value row of head h, in rows of D elements
};

template <bool kCausal, bool kFused>
__device__ __forceinline__ Desc item_desc(const AttnArgs<bf16>& a, int64_t idx) {
  Desc d;
  d.np = 0;
  if (!kCausal) {
    // Scalar load of the 16-byte descriptor, waited for in the same statement
    // (the list was written by an earlier kernel and is read-only here).
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    i32x4 v;
    const uint64_t addr = uniform_ptr(a.items + idx);
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(addr));
    d.h = v.x;
    d.b = v.y;
    d.start = v.z;
    d.count = v.w;
    d.nkt = a.B / kKTile;
  } else {
    // Query tiles of a block in zig-zag order (first, last, second, second
    // last, ...): the causal work of a tile grows with its position, so a
    // workgroup's contiguous range of items mixes light and heavy tiles.
    const int per_block = (a.B + kAttnTile - 1) / kAttnTile;
    const int64_t e = idx / per_block;
    const int zz = static_cast<int>(idx - e * per_block);
    const int qt = (zz & 1) ? per_block - 1 - (zz >> 1) : (zz >> 1);
    d.h = static_cast<int>(e / a.n);
    d.b = static_cast<int>(e - static_cast<int64_t>(d.h) * a.n);
    d.start = qt * kAttnTile;
    d.count = min(kAttnTile, a.B - d.start);
    d.nkt = (d.start + d.count) / kKTile;
    if (kFused) {
      int lo = 0;
      if (a.blo != nullptr) {
        // Scalar load, waited for in the same statement (written by an earlier kernel).
        const uint64_t addr = uniform_ptr(a.blo + uniform_u32(d.b));
        asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(lo) : "s"(addr));
      }
      d.np = 2 * kept_past(d.b, lo, a.topk);
    }
  }
  d.h = static_cast<int>(uniform_u32(d.h));
  d.b = static_cast<int>(uniform_u32(d.b));
  d.start = static_cast<int>(uniform_u32(d.start));
  d.count = static_cast<int>(uniform_u32(d.count));
  d.nkt = static_cast<int>(uniform_u32(d.nkt));
  d.np = static_cast<int>(uniform_u32(d.np));
  d.kv_row = static_cast<int64_t>(d.b) * a.B * a.H + d.h;
  return d;
}

// The 32-query block (item position 32 * blk) of wave i. Own-block items pair
// the blocks i and 7 - i on the two waves of a SIMD (waves i and i + 4), which
// evens out the causal triangle across the SIMDs.
template <bool kCausal>
__device__ __forceinline__ int wave_block(int i) {
  return kCausal ? (i < 4 ? i : 11 - i) : i;
}

// Attention over one 64-key K/V tile for the wave's 32 queries, in 32-key
// halves.
//   S^T = K Q^T      keys on rows, queries on columns; K from LDS, Q in registers;
//   causal mask      on the scores, when a half holds the diagonal;
//   softmax          p = exp2(s * c2 - m * c2) against the running reference m;
//                    m is only raised (and O, l rescaled) when a half's
//                    probabilities sum past 2^64 or are not finite, i.e. when
//                    a score exceeds m by a wide margin: rare, decided
//                    wave-wide, and exact after the final normalisation. l sums
//                    the bf16 probabilities that actually multiply V;
//   O^T += V^T P^T   V^T read with the LDS transpose read in the key order the
//                    S accumulator layout hands to P.
constexpr float kSumLimit = 0x1p64f;   // largest accepted sum of one half's probabilities

template <int D>
__device__ __forceinline__ f32x16 scores(const char* kp, const bf16x8 (&q)[D / 16]) {
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kp + 32 * c));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, q[c], s, 0, 0, 0);
  }
  return s;
}

__device__ __forceinline__ void mask_scores(f32x16& s, int kbase, int qpos, int half) {
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (kbase + 8 * (r >> 2) + 4 * half + (r & 3) > qpos) s[r] = -INFINITY;
}

// bf16 probabilities of one half against reference mc = m * c2; returns their sum.
__device__ __forceinline__ float probs(const f32x16& s, float c2, float mc, bf16x8 (&p)[2]) {
  const bf16x2 ones = {static_cast<bf16>(1.f), static_cast<bf16>(1.f)};
  float lh = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const bf16x2 pr = {static_cast<bf16>(__builtin_amdgcn_exp2f(fmaf(s[r], c2, -mc))),
                       static_cast<bf16>(__builtin_amdgcn_exp2f(fmaf(s[r + 1], c2, -mc)))};
    p[r >> 3][r & 7] = pr[0];
    p[r >> 3][(r & 7) + 1] = pr[1];
    lh = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lh, false);
  }
  return lh;
}

// The rare path: raise m to the half's maximum (both lanes of a query agree),
// rescale O and l, recompute the half's probabilities. Taken by the whole wave
// when any lane's sum is out of range (always on an item's first half, where
// m = -inf).
template <int D>
__device__ __forceinline__ void settle(const f32x16& s, float& m, float& l, f32x16 (&o)[D / 32], bf16x8 (&p)[2],
                                       float& lh, float c2) {
  if (__builtin_amdgcn_ballot_w64(!(lh <= kSumLimit)) == 0) return;
  float mx = fmaxf(s[0], s[1]);
#pragma unroll
  for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[r], s[r + 1]));
  const float m_new = fmaxf(m, fmaxf(mx, __shfl_xor(mx, 32)));
  const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c2);   // 0 when m was -inf
  m = m_new;
  l *= alpha;
#pragma unroll
  for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dc][r] *= alpha;
  lh = probs(s, c2, m * c2, p);
}

// V^T operands of one half (transpose reads, two per 16-key group and 32 dims).
template <int D>
__device__ __forceinline__ void v_operands(const char* vp, bf16x8 (&va)[D / 32][2]) {
  using L = Lay<D>;
#pragma unroll
  for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const char* vq = vp + 16 * g * L::kVStride + 64 * dc;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vq));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vq + 8 * L::kVStride));
      const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo);
      const bf16x4 h4 = __builtin_bit_cast(bf16x4, hi);
      va[dc][g] = bf16x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
    }
}

template <int D>
__device__ __forceinline__ void pv(const bf16x8 (&va)[D / 32][2], const bf16x8 (&p)[2], f32x16 (&o)[D / 32]) {
#pragma unroll
  for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
    for (int g = 0; g < 2; ++g) o[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dc][g], p[g], o[dc], 0, 0, 0);
}

// Scheduling hint for the current region: n groups of (d LDS reads, one
// MFMA, v VALU instructions), so that the MFMAs of one half are issued in
// between the VALU work of the other.
template <int N, int D, int V>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, D, 0);   // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, V, 0);   // VALU
  }
}

// Both halves of a tile, software-pipelined inside the wave so that the MFMAs
// of one half run while the VALU work of the other is issued:
//   S(h0) | S(h1) + softmax(h0) | PV(h0) + softmax(h1) | PV(h1).
// mask1: the second half holds the diagonal (own-block items).
// issue(0) and issue(1) put the tile loads of a later ring step in between the
// phases, so that the address unit works through them while the MFMAs run
// instead of in one burst at the start of the step.
template <int D, typename F>
__device__ __forceinline__ void tile_pair(const char* kp, const char* vp, const bf16x8 (&q)[D / 16],
                                          f32x16 (&o)[D / 32], float& m, float& l, bool mask1, int kbase1, int qpos,
                                          int half, float c2, F&& issue) {
  using L = Lay<D>;
  constexpr int kQC = D / 16;
  // The first half's K operands all requested before its products (the step
  // opens with them, right after the barrier).
  bf16x8 ka[kQC];
#pragma unroll
  for (int c = 0; c < kQC; ++c) ka[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kp + 32 * c));
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s0;
#pragma unroll
  for (int r = 0; r < 16; ++r) s0[r] = 0.f;
#pragma unroll
  for (int c = 0; c < kQC; ++c) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], q[c], s0, 0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue(0);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s1 = scores<D>(kp + 32 * L::kKStride, q);
  bf16x8 p0[2], va0[D / 32][2];
  float lh0 = probs(s0, c2, m * c2, p0);
  v_operands<D>(vp, va0);
  interleave<kQC, 3, 6>();
  settle<D>(s0, m, l, o, p0, lh0, c2);
  l += lh0;
  if (mask1) mask_scores(s1, kbase1, qpos, half);
  __builtin_amdgcn_sched_barrier(0);
  issue(1);
  __builtin_amdgcn_sched_barrier(0);
  pv<D>(va0, p0, o);
  bf16x8 p1[2], va1[D / 32][2];
  float lh1 = probs(s1, c2, m * c2, p1);
  v_operands<D>(vp + 32 * L::kVStride, va1);
  interleave<2 * (D / 32), 2, 6>();
  settle<D>(s1, m, l, o, p1, lh1, c2);
  l += lh1;
  pv<D>(va1, p1, o);
}

// Past-block tiles (no mask), pipelined across ring steps: the PV of a
// tile's second half runs at the start of the next step, from probabilities
// and V^T operands kept in registers, so that each step opens with MFMAs
// that need no LDS read while the K reads of the new tile are in flight:
//   PV(t-1, h1) + S(t, h0) | S(t, h1) + softmax(t, h0) | PV(t, h0) + softmax(t, h1).
// p1 is zero on an item's first tile (the PV then adds exactly zero).
template <int D, typename F>
__device__ __forceinline__ void tile_step(const char* kp, const char* vp, const bf16x8 (&q)[D / 16],
                                          f32x16 (&o)[D / 32], float& m, float& l, float c2, bf16x8 (&p1)[2],
                                          bf16x8 (&va1)[D / 32][2], F&& issue) {
  using L = Lay<D>;
  constexpr int kQC = D / 16;
  pv<D>(va1, p1, o);
  f32x16 s0 = scores<D>(kp, q);
  __builtin_amdgcn_sched_barrier(0);
  issue(0);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 s1 = scores<D>(kp + 32 * L::kKStride, q);
  bf16x8 p0[2], va0[D / 32][2];
  float lh0 = probs(s0, c2, m * c2, p0);
  v_operands<D>(vp, va0);
  interleave<kQC, 3, 6>();
  settle<D>(s0, m, l, o, p0, lh0, c2);
  l += lh0;
  __builtin_amdgcn_sched_barrier(0);
  issue(1);
  __builtin_amdgcn_sched_barrier(0);
  pv<D>(va0, p0, o);
  float lh1 = probs(s1, c2, m * c2, p1);
  v_operands<D>(vp + 32 * L::kVStride, va1);
  interleave<2 * (D / 32), 2, 6>();
  settle<D>(s1, m, l, o, p1, lh1, c2);
  l += lh1;
}

// One half only (own-block items: the tile whose first half holds the diagonal).
template <int D>
__device__ __forceinline__ void tile_first_half(const char* kp, const char* vp, const bf16x8 (&q)[D / 16],
                                                f32x16 (&o)[D / 32], float& m, float& l, int kbase, int qpos,
                                                int half, float c2) {
  f32x16 s0 = scores<D>(kp, q);
  mask_scores(s0, kbase, qpos, half);
  bf16x8 p0[2], va0[D / 32][2];
  float lh0 = probs(s0, c2, m * c2, p0);
  v_operands<D>(vp, va0);
  settle<D>(s0, m, l, o, p0, lh0, c2);
  l += lh0;
  pv<D>(va0, p0, o);
}

// Persistent block-attention kernel over one kind of work item (past-block
// items from the query lists, or own-block items with the causal mask).
//
// Schedule: static. Past-block items: XCD x (= blockIdx % 8) takes a
// contiguous 1/8 of the item list and its workgroups take every (G/8)-th item
// of it, so the workgroups of one XCD work on neighbouring items (the same key
// blocks) at the same time. Own-block items: every workgroup takes a
// contiguous range, so the query tiles of a block run back to back.
//
// Pipeline: each item is a sequence of ring steps: two Q tiles (the item's 256
// query rows, gathered through the query list into LDS; waves 0-3 take their
// rows from the first, waves 4-7 from the second), then its 64-key K/V tiles.
// The loads of step p + kAhead are issued at step p, across item boundaries,
// into the slot of step p - 1. Every wave issues a fixed number of loads per
// step (its share of the slot's windows), plus one query-index load at the
// first step of an item (for the item after it) and the item's stores after
// its last step, so the number of this wave's memory operations younger than
// step p's loads is known exactly; step p waits for that count, then a
// workgroup barrier publishes the slot.
//
// kFused (own-block items, at most kFusedMaxPast past selections per query):
// after its K/V tiles the item takes two more ring steps per past selection,
// which bring that selection's partial rows (gathered by list position) and
// their log-sum-exps into a slot; the waves fold them into their rows (LSE
// merge) and the item ends by writing the final out and lse rows.
template <int D, bool kCausal, bool kFused>
__global__ __launch_bounds__(kThreads, 1) void attn_mfma_kernel(AttnArgs<bf16> a) {
  using L = Lay<D>;
  constexpr int kQC = D / 16, kDC = D / 32;
  // Item stores: four 16-byte stores per 64-dim round, and the log-sum-exps.
  constexpr int kStoresPerItem = 4 * (kDC / 2) + 1;
  // Extra loads at an item's first step: the next item's query indices
  // (past-block items) or this item's list positions (fused own-block items).
  constexpr int kXq = kCausal ? (kFused ? kInvRounds : 0) : 1;
  static_assert(!kFused || kCausal, "the merge is fused into own-block items only");
  static_assert((kAhead - 1) * L::kRoundsHi + kStoresPerItem + kXq < 64, "vmcnt holds at most 63");
  // Tail buffer: the double-buffered query indices (past-block items) or the
  // list positions of the item's past selections (fused own-block items).
  constexpr int kTailBytes = kFused ? kInvInts * 4 : 2 * kQBuf * 4;
  __shared__ __attribute__((aligned(16))) char smem[kSlots * L::kSlot + kWaves * kStageBytes + kTailBytes];
  char* const ring = smem;
  char* const stage = smem + kSlots * L::kSlot;
  int32_t* const qbuf = reinterpret_cast<int32_t*>(smem + kSlots * L::kSlot + kWaves * kStageBytes);

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int qn = lane & 31;
  const int half = lane >> 5;
  const float c2 = a.scale_log2;
  const int64_t row_el = static_cast<int64_t>(a.H) * D;        // elements between consecutive tokens
  const int64_t tile_el = kKTile * row_el;                      // elements between consecutive K/V tiles
  const uint32_t row_bytes = static_cast<uint32_t>(row_el * 2);
  const bool hi_rounds = w < L::kWindows % kWaves || L::kWindows % kWaves == 0;

  // ---- static schedule of this workgroup ----
  int64_t first, stride;
  int cnt;
  int gper = 0, gside = 0;   // grouped own-block schedule: group size and this workgroup's place in it
  if (!kCausal) {
    const int64_t M = a.counters[0];
    const int xcd = blockIdx.x % kXcds, c = blockIdx.x / kXcds, nper = gridDim.x / kXcds;
    const int64_t xa = M * xcd / kXcds, xb = M * (xcd + 1) / kXcds;
    first = xa + c;
    stride = nper;
    cnt = first < xb ? static_cast<int>((xb - first + nper - 1) / nper) : 0;
  } else {
    const int per = a.qt_per_block;
    const int64_t nblk = a.own_items / per;
    const int G = static_cast<int>(gridDim.x);
    if (per > 1 && G % (kXcds * per) == 0) {
      // The per query tiles of a block run at the same time on `per`
      // workgroups of one XCD, which then read the block's K/V tiles once from
      // HBM and share them in L2; the tiles rotate over the group's workgroups
      // from one block to the next, which evens out the causal work.
      const int x = static_cast<int>(blockIdx.x) % kXcds, sx = static_cast<int>(blockIdx.x) / kXcds;
      const int64_t groups = G / per;
      first = static_cast<int64_t>(x) * (G / kXcds / per) + sx / per;   // this group's first block
      stride = groups;
      gper = per;
      gside = sx % per;
      cnt = first < nblk ? static_cast<int>((nblk - first + groups - 1) / groups) : 0;
    } else {
      const int64_t lo = a.own_items * blockIdx.x / gridDim.x, hi = a.own_items * (blockIdx.x + 1) / gridDim.x;
      first = lo;
      stride = 1;
      cnt = static_cast<int>(hi - lo);
    }
  }
  cnt = static_cast<int>(uniform_u32(cnt));
  if (cnt <= 0) return;
  // The m-th item of this workgroup.
  auto sched = [&](int m) -> int64_t {
    const int64_t base = first + static_cast<int64_t>(m) * stride;
    return (kCausal && gper > 0) ? base * gper + (gside + m) % gper : base;
  };

  // ---- per-lane offsets of the K/V tile loads (tile-relative) ----
  uint32_t kvoff[L::kRoundsHi];
  uint32_t vmask = 0;   // bit u: window of round u holds V rows (else K rows or padding)
#pragma unroll
  for (int u = 0; u < L::kRoundsHi; ++u) {
    const int win = u * kWaves + w;
    const int s16 = win * 64 + lane;             // 16-byte unit of the slot
    int row = 0, ch = 0;
    if (s16 < L::kKBytes / 16) {
      row = s16 / L::kKSlots16;
      ch = s16 % L::kKSlots16;
    } else if (s16 < (L::kKBytes + L::kVBytes) / 16) {
      const int t = s16 - L::kKBytes / 16;
      row = t / L::kVSlots16;
      ch = t % L::kVSlots16;
      vmask |= 1u << u;
    }
    ch = ch < L::kChunks ? ch : 0;               // padding units re-load chunk 0
    kvoff[u] = static_cast<uint32_t>(row) * row_bytes + 16u * ch;
  }
  vmask = uniform_u32(vmask);
  // Past-block items: row (within a 128-row Q tile) and byte offset in that
  // row of each of the lane's Q loads; units past the tile's rows or chunks
  // reload the tile's last row or a row's first chunk.
  int qrow[kCausal ? 1 : L::kRoundsHi], qch16[kCausal ? 1 : L::kRoundsHi];
  if (!kCausal) {
#pragma unroll
    for (int u = 0; u < L::kRoundsHi; ++u) {
      const int s16 = (u * kWaves + w) * 64 + lane;
      const int r = s16 / L::kKSlots16, ch = s16 % L::kKSlots16;
      qrow[u] = r < kQTileRows ? r : kQTileRows - 1;
      qch16[u] = 16 * (ch < L::kChunks ? ch : 0);
    }
  }
  const uint32_t ring_lds = lds_addr(ring);
  const uint32_t qbuf_lds = lds_addr(qbuf);

  // Loads of one ring step (Q tile, K/V tile or partial step) of item d into slot `sl`.
  auto issue_step = [&](const Desc& d, int j, int sl, int qb, int u0, int u1) {
    const uint32_t m0base = ring_lds + sl * L::kSlot + w * 1024;
    if (kFused && j >= 2 + d.nkt) {
      // Partial step jp: past selection jp / 2, 32-dim blocks kPC * (jp % 2)
      // onwards, gathered by list position (the item's inv rows in the tail
      // buffer). Unit (q, c') of the slot takes chunk c' ^ (q % kSegChunks) of
      // query q's segment; the hi round takes the partials' log-sum-exps.
      const int jp = j - 2 - d.nkt, sp = jp >> 1;
      const int dim0 = 32 * L::kPC * (jp & 1);
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int u = 0; u < L::kRoundsHi; ++u) {
        if (u >= u0 && u < u1 && u < L::kRoundsLo) {
          const int s16 = (u * kWaves + w) * 64 + ln;
          const int q = s16 / L::kSegChunks, cs = s16 % L::kSegChunks;
          const int ps = qbuf[min(q, d.count - 1) * a.lmax + sp];
          dma16_addr(m0base + u * kWaves * 1024,
                     a.part_off + static_cast<int64_t>(ps) * D + dim0 + 8 * (cs ^ (q % L::kSegChunks)));
        } else if (u >= u0 && u < u1 && u == L::kRoundsLo && hi_rounds) {
          const int ps = qbuf[min(w * 64 + ln, d.count - 1) * a.lmax + sp];
          dma4(ring_lds + sl * L::kSlot + L::kLseOff + w * 256, static_cast<uint32_t>(ps) * 4u, uniform_ptr(a.lse_off));
        }
      }
    } else if (j >= 2) {
      // Rows b * B + kKTile * (j - 2) onwards: the item's offset plus j - 2 tile strides.
      const int64_t off = d.kv_row * D + static_cast<int64_t>(j - 2) * tile_el;
      const uint64_t kb = uniform_ptr(a.k + off), vb = uniform_ptr(a.v + off);
#pragma unroll
      for (int u = 0; u < L::kRoundsHi; ++u)
        if (u >= u0 && u < u1 && (u < L::kRoundsLo || hi_rounds))
          dma16(m0base + u * kWaves * 1024, kvoff[u], ((vmask >> u) & 1) ? vb : kb);
    } else if (!kCausal) {
      // Past-block items: the lane's rows and chunk offsets of a Q tile come
      // from the per-kernel table (row qrow[u] of the tile, i.e. item position
      // 128 j + qrow[u]); the query index comes from the list entries in LDS.
      const int32_t* qi_lds = qbuf + qb * kQBuf;
      const uint64_t qh = uniform_ptr(a.q + static_cast<int64_t>(d.h) * D);
#pragma unroll
      for (int u = 0; u < L::kRoundsHi; ++u) {
        if (u >= u0 && u < u1 && (u < L::kRoundsLo || hi_rounds)) {
          const int pos = min(kQTileRows * j + qrow[u], d.count - 1);
          const uint64_t tok = static_cast<uint32_t>(qi_lds[pos]);
          dma16_addr(m0base + u * kWaves * 1024,
                     reinterpret_cast<const void*>(qh + tok * row_bytes + static_cast<uint32_t>(qch16[u])));
        }
      }
    } else {
      const int32_t* qi_lds = qbuf + qb * kQBuf;
      // Opaque copy of the lane index: keeps the per-lane address arithmetic
      // below from being hoisted out of the loops as long-lived registers.
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int u = 0; u < L::kRoundsHi; ++u) {
        if (u >= u0 && u < u1 && (u < L::kRoundsLo || hi_rounds)) {
          const int s16 = (u * kWaves + w) * 64 + ln;
          int r = s16 / L::kKSlots16, ch = s16 % L::kKSlots16;
          r = r < kQTileRows ? r : kQTileRows - 1;
          ch = ch < L::kChunks ? ch : 0;
          const int wi = 4 * j + (r >> 5);                      // wave that reads row r
          const int pos = min(32 * wave_block<kCausal>(wi) + (r & 31), d.count - 1);
          const int64_t tok = kCausal ? static_cast<int64_t>(d.b) * a.B + d.start + pos
                                      : static_cast<int64_t>(qi_lds[pos]);
          dma16_addr(m0base + u * kWaves * 1024, a.q + (tok * a.H + d.h) * D + 8 * ch);
        }
      }
    }
  };
  // Query-list entries of a past-block item into qbuf[qb] (one 4-byte load per
  // lane; entries past the item's count repeat its last one).
  auto issue_qidx = [&](const Desc& d, int qb) {
    const int i = min(w * 64 + lane, d.count - 1);
    dma4(qbuf_lds + qb * kQBuf * 4 + w * 256, static_cast<uint32_t>(i) * 4u, uniform_ptr(a.qidx + d.start));
  };

  // List positions of the past selections of an own-block item's queries,
  // [query][lmax] for its 256 query slots (slots past its count repeat the
  // last query), into the tail buffer; a fixed kInvRounds loads per lane.
  auto issue_inv = [&](const Desc& d) {
    const int64_t row0 = (static_cast<int64_t>(d.h) * a.N + static_cast<int64_t>(d.b) * a.B + d.start) * a.lmax;
    const int last = max(d.count * a.lmax - 1, 0);
    // No past selections at all: load (and ignore) the first ints of q instead.
    const uint64_t src = a.lmax > 0 ? uniform_ptr(a.inv + row0) : uniform_ptr(a.q);
    int ln = lane;   // opaque copy: the offsets below are not kept live across the item
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int u = 0; u < kInvRounds; ++u) {
      const int e = min((u * kWaves + w) * 64 + ln, last);
      dma4(qbuf_lds + (u * kWaves + w) * 256, static_cast<uint32_t>(e) * 4u, src);
    }
  };

  // ---- prologue ----
  Desc dd = item_desc<kCausal, kFused>(a, sched(0));   // item being loaded
  int md = 0, jd = 0;                         // load cursor: item ordinal, step within item
  bool ddone = false;
  int qstep0 = -1000, qstep1 = -1000;         // ring step at which each qbuf was requested
  if (!kCausal) {
    issue_qidx(dd, 0);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    asm volatile("s_barrier" ::: "memory");
  }
  auto advance_load = [&]() {
    if (ddone) return;
    if (++jd == 2 + dd.nkt + dd.np) {
      if (md + 1 < cnt) {
        ++md;
        jd = 0;
        dd = item_desc<kCausal, kFused>(a, sched(md));
      } else {
        ddone = true;   // keep re-loading the last K/V tile (into slots nobody reads again)
        jd = 2 + dd.nkt - 1;
      }
    }
  };
  // Issue the loads of the load cursor's step into slot sl during ring step
  // `now`: rounds [u0, u1) of it; the part that ends with the last round also
  // moves the cursor on.
  auto load_part = [&](int now, int sl, int u0, int u1) {
    if (u0 == 0 && !kCausal && jd < 2 && !ddone && now < ((md & 1) ? qstep1 : qstep0) + kAhead) {
      // The query indices of this item may still be in flight: drain and sync.
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
      asm volatile("s_barrier" ::: "memory");
    }
    if (u0 == 0 && kFused && jd >= 2 + dd.nkt && !ddone && now < qstep0 + kAhead) {
      // The list positions of this item may still be in flight: drain and sync.
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
      asm volatile("s_barrier" ::: "memory");
    }
    issue_step(dd, jd, sl, md & 1, u0, u1);
    if (u1 == L::kRoundsHi) advance_load();
  };
  auto load_next = [&](int now, int sl) { load_part(now, sl, 0, L::kRoundsHi); };
#pragma unroll
  for (int i = 0; i < kAhead; ++i) load_next(0, i);

  // ---- main loop: items, each two Q steps and nkt K/V steps ----
  const int k_lane = qn * L::kKStride + 16 * half;
  const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
  const int v_lane = L::kKBytes + (4 * (tg >> 1) + te) * L::kVStride + 2 * (16 * (tg & 1) + 4 * tq);
  const int q_lane = (32 * (w & 3) + qn) * L::kKStride + 16 * half;
  const int pos0 = 32 * wave_block<kCausal>(w);    // this wave's queries: item positions pos0 .. pos0 + 31

  int p = 0;   // ring step
  // Operations issued after the tile loads of step p - kAhead (= p - 2):
  // query-index or list-position loads at step p - 1 (they precede the step's
  // tile loads), item stores at steps p - 1 and p - 2 (they follow them; at
  // most one item's, items being at least three steps long).
  int qh1 = 0, sh1 = 0, sh2 = 0;
  // Start ring step p: wait for this wave's loads of the step, publish the slot
  // to the workgroup, issue the loads of step p + kAhead. Returns the slot of step p.
  // With `defer`, the loads of step p + kAhead are left to the caller (split
  // into two parts by the tile computation).
  auto ring_step = [&](int qidx_buf, const Desc& nd, bool defer) -> const char* {
    const bool xs = (sh1 | sh2) != 0;
    const bool xq = qh1 != 0;
    constexpr int kHi = (kAhead - 1) * L::kRoundsHi, kLo = (kAhead - 1) * L::kRoundsLo;
    if (hi_rounds) {
      if (xs) {
        if (xq) __builtin_amdgcn_s_waitcnt(wait_vmcnt(kHi + kStoresPerItem + kXq));
        else __builtin_amdgcn_s_waitcnt(wait_vmcnt(kHi + kStoresPerItem));
      } else {
        if (xq) __builtin_amdgcn_s_waitcnt(wait_vmcnt(kHi + kXq));
        else __builtin_amdgcn_s_waitcnt(wait_vmcnt(kHi));
      }
    } else {
      if (xs) {
        if (xq) __builtin_amdgcn_s_waitcnt(wait_vmcnt(kLo + kStoresPerItem + kXq));
        else __builtin_amdgcn_s_waitcnt(wait_vmcnt(kLo + kStoresPerItem));
      } else {
        if (xq) __builtin_amdgcn_s_waitcnt(wait_vmcnt(kLo + kXq));
        else __builtin_amdgcn_s_waitcnt(wait_vmcnt(kLo));
      }
    }
    // This wave's reads of earlier slots have returned before the barrier
    // after which other waves may reload them.
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    const bool qnow = kXq > 0 && qidx_buf >= 0;
    if (qnow) {
      if (kCausal) {
        issue_inv(nd);
        qstep0 = p;
      } else {
        issue_qidx(nd, qidx_buf);
        if (qidx_buf) qstep1 = p;
        else qstep0 = p;
      }
    }
    if (!defer) load_next(p, (p + kAhead) % kSlots);
    const char* slot = ring + (p % kSlots) * L::kSlot;
    sh2 = sh1;
    sh1 = 0;
    qh1 = qnow ? 1 : 0;
    ++p;
    return slot;
  };

  // Writes the wave's 32 output rows (item positions pos0 .. pos0 + 31, each
  // query's values times `scale`) through the wave's staging area, one 64-dim
  // round at a time: lane (qn, half) puts its values into 16-byte chunks
  // swizzled by row, then 8 lanes per row read them back and store 128-byte
  // lines. rowp(pos): first element of the output row of item position pos.
  // The wave's LDS operations run in order, so the staging area needs no barrier.
  auto store_tile = [&](const f32x16 (&ov)[kDC], float scale, auto&& rowp) {
    char* const st = stage + w * kStageBytes;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int wr = ln & 31, wh = ln >> 5;   // writer: row, half
    const int rr = ln >> 3, rc = ln & 7;    // reader: row within a group of 8, chunk
#pragma unroll
    for (int rd = 0; rd < kDC / 2; ++rd) {
#pragma unroll
      for (int dl = 0; dl < 2; ++dl)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x4 vv;
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[e] = static_cast<bf16>(ov[2 * rd + dl][4 * i + e] * scale);
          const int c = 4 * dl + i;
          *reinterpret_cast<uint2*>(st + wr * 128 + 16 * (c ^ (wr & 7)) + 8 * wh) = __builtin_bit_cast(uint2, vv);
        }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + rr;
        const uint4 x = *reinterpret_cast<const uint4*>(st + r * 128 + 16 * (rc ^ rr));
        store16(rowp(pos0 + r) + 64 * rd + 8 * rc, x);
      }
      asm volatile("" ::: "memory");
    }
  };

  bf16x8 p1[2], va1[kDC][2];
#pragma unroll
  for (int dc = 0; dc < kDC; ++dc)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) va1[dc][g][e] = static_cast<bf16>(0.f);

  for (int mc = 0; mc < cnt; ++mc) {
    const Desc cd = item_desc<kCausal, kFused>(a, sched(mc));
    bf16x8 q[kQC];
    {
      // The first Q step also requests the query indices of the next item
      // (past-block items) or this item's list positions (fused merge).
      const bool more = mc + 1 < cnt;
      Desc nd = cd;
      if (!kCausal && more) nd = item_desc<kCausal, kFused>(a, sched(mc + 1));
      const char* slot = ring_step(kFused ? 0 : (!kCausal && more ? (mc + 1) & 1 : -1), nd, false);
      if (w < 4) {
#pragma unroll
        for (int c = 0; c < kQC; ++c)
          q[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(slot + q_lane + 32 * c));
      }
      slot = ring_step(-1, nd, false);
      if (w >= 4) {
#pragma unroll
        for (int c = 0; c < kQC; ++c)
          q[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(slot + q_lane + 32 * c));
      }
    }
    f32x16 o[kDC];
#pragma unroll
    for (int dc = 0; dc < kDC; ++dc)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dc][r] = 0.f;
    float m = -INFINITY, l = 0.f;
    const bool wave_valid = pos0 < cd.count;
    const int f = cd.start + pos0;                 // own-block items: block position of the first query
    const int qpos = f + qn;
    // Past-block items: probabilities and V^T operands of the previous
    // tile's second half (its PV runs in the next step).
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) p1[g][e] = static_cast<bf16>(0.f);
    for (int t = 0; t < cd.nkt; ++t) {
      const int kbase = t * kKTile;
      const char* slot = ring_step(-1, cd, true);
      const int now = p - 1, sl = (now + kAhead) % kSlots;
      constexpr int kSplit = (L::kRoundsHi + 1) / 2;
      auto issue = [&](int part) {
        if (part == 0) load_part(now, sl, 0, kSplit);
        else load_part(now, sl, kSplit, L::kRoundsHi);
      };
      if (!kCausal && wave_valid) {
        tile_step<D>(slot + k_lane, slot + v_lane, q, o, m, l, c2, p1, va1, issue);
      } else if (wave_valid && (!kCausal || kbase < f)) {
        // Both halves visible (the second may hold the diagonal).
        tile_pair<D>(slot + k_lane, slot + v_lane, q, o, m, l, kCausal && kbase + 32 == f, kbase + 32, qpos, half,
                     c2, issue);
      } else {
        load_next(now, sl);
        if (kCausal && wave_valid && kbase == f)
          tile_first_half<D>(slot + k_lane, slot + v_lane, q, o, m, l, kbase, qpos, half, c2);
      }
    }
    if (!kCausal && wave_valid) pv<D>(va1, p1, o);   // the last tile's second half
    // ---- epilogue: normalise and store the item's partial rows ----
    if (kFused) {
      // LSE merge with the query's past-block partials (natural-log lse_s,
      // normalised rows O_s): lse = log(exp(lse_own) + sum_s exp(lse_s)),
      // out = sum over all partials of exp(lse_x - lse) O_x, accumulated in
      // log2 units with a running maximum. The partial rows come through the
      // ring in the item's partial steps, two per past selection (kPC 32-dim
      // blocks each); the first of the two also carries their log-sum-exps.
      const int pos = pos0 + qn;
      const bool valid = pos < cd.count;
      const float l_tot = l + __shfl_xor(l, 32);
      float mm = m * c2 + log2f(l_tot);
      float ww = 1.f;
      {
        const float inv_l = 1.f / l_tot;
#pragma unroll
        for (int dc = 0; dc < kDC; ++dc)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dc][r] *= inv_l;
      }
      for (int sp = 0; sp < cd.np / 2; ++sp) {
        // This lane's bytes of its query's segment and the query's swizzle,
        // from an opaque copy of the lane index (nothing of the merge is kept
        // live across the item's tiles).
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lpos = pos0 + (ln & 31);
        const int seg = lpos * L::kSegChunks * 16 + 8 * (ln >> 5);
        const int sw = lpos % L::kSegChunks;
        float ca = 1.f, cb = 0.f;
#pragma unroll
        for (int pc = 0; pc < 2; ++pc) {
          const char* slot = ring_step(-1, cd, false);
          if (pc == 0) {
            const float ls = *reinterpret_cast<const float*>(slot + L::kLseOff + 4 * lpos) * kLog2e;
            const float nm = fmaxf(mm, ls);
            ca = __builtin_amdgcn_exp2f(mm - nm);
            cb = __builtin_amdgcn_exp2f(ls - nm);
            ww = fmaf(ww, ca, cb);
            mm = nm;
          }
#pragma unroll
          for (int dl = 0; dl < L::kPC; ++dl)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const bf16x4 x = __builtin_bit_cast(
                  bf16x4, *reinterpret_cast<const uint2*>(slot + seg + 16 * ((4 * dl + i) ^ sw)));
#pragma unroll
              for (int e = 0; e < 4; ++e)
                o[L::kPC * pc + dl][4 * i + e] =
                    fmaf(o[L::kPC * pc + dl][4 * i + e], ca, static_cast<float>(x[e]) * cb);
            }
        }
      }
      const int64_t tok = static_cast<int64_t>(cd.b) * a.B + cd.start + pos;
      // Slots without a query write to the dump rows of the past-block partials.
      store_tile(o, 1.f / ww, [&](int ps) -> bf16* {
        return ps < cd.count ? a.out + ((static_cast<int64_t>(cd.b) * a.B + cd.start + ps) * a.H + cd.h) * D
                             : a.part_off + (a.p_off + ps) * D;
      });
      store4(valid ? a.lse_out + static_cast<int64_t>(cd.h) * a.N + tok : a.lse_off + a.p_off + pos,
             (mm + log2f(ww)) * kLn2);
    } else {
      const float l_tot = l + __shfl_xor(l, 32);
      const float inv_l = 1.f / l_tot;
      const int pos = pos0 + qn;
      // Output row of item position ps: the item's list entries (past
      // blocks) or queries (own block); slots without one write to dump rows.
      auto row_of = [&](int ps) -> int64_t {
        if (kCausal)
          return ps < cd.count ? static_cast<int64_t>(cd.h) * a.N + static_cast<int64_t>(cd.b) * a.B + cd.start + ps
                               : static_cast<int64_t>(a.H) * a.N + ps;
        return ps < cd.count ? static_cast<int64_t>(cd.start) + ps : a.p_off + ps;
      };
      store_tile(o, inv_l, [&](int ps) -> bf16* { return (kCausal ? a.part_diag : a.part_off) + row_of(ps) * D; });
      const int64_t row = row_of(pos);
      store4((kCausal ? a.lse_diag : a.lse_off) + row, (m * c2 + log2f(l_tot)) * kLn2);
    }
    sh1 = 1;
  }
  // Retire the trailing (unused) loads before the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
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
  a.inv = ws.inv;
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
  a.p_off = p.p_off;
  a.own_items = static_cast<int64_t>(p.H) * p.n * ((p.B + kAttnTile - 1) / kAttnTile);
  a.topk = p.topk;
  a.lmax = p.lmax;
  a.blo = p.blo;
  a.out = nullptr;
  a.lse_out = nullptr;
  a.scale_log2 = kLog2e / sqrtf(static_cast<float>(p.D));
  return a;
}

}  // namespace

bool merge_fused(const Problem& p) { return !p.is_f32 && p.lmax <= kFusedMaxPast; }

hipError_t launch_attention(const Problem& p, const void* q, const void* k, const void* v, const Workspace& ws,
                            void* out, float* lse, int num_cus, hipStream_t stream,
                            const std::function<hipError_t(int)>& mark) {
  if (p.is_f32) {
    const int64_t total = p.max_items + p.diag_items;
    int64_t grid = static_cast<int64_t>(num_cus) * 2;
    grid = std::min<int64_t>(grid, ((total + kXcds - 1) / kXcds) * kXcds);
    auto a = make_args<float>(p, q, k, v, ws);
    if (p.D == 128)
      attn_f32_kernel<128><<<static_cast<unsigned>(grid), 256, 0, stream>>>(a);
    else
      attn_f32_kernel<64><<<static_cast<unsigned>(grid), 256, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? mark(4) : e;
  }
  auto a = make_args<bf16>(p, q, k, v, ws);
  a.out = static_cast<bf16*>(out);
  a.lse_out = lse;
  // Past-block items (their number is only known on the device): one
  // workgroup per CU, a multiple of the XCD count.
  if (p.lmax > 0) {
    const int64_t grid = std::max<int64_t>(kXcds, (num_cus / kXcds) * kXcds);
    if (p.D == 128)
      attn_mfma_kernel<128, false, false><<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(a);
    else
      attn_mfma_kernel<64, false, false><<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = mark(4);
  if (e != hipSuccess) return e;
  // Own-block items after them (same stream), with the merge fused in when
  // every query keeps at most kFusedMaxPast past blocks.
  const int64_t grid = std::min<int64_t>(num_cus, a.own_items);
  const bool fused = merge_fused(p);
  if (p.D == 128) {
    if (fused)
      attn_mfma_kernel<128, true, true><<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(a);
    else
      attn_mfma_kernel<128, true, false><<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(a);
  } else {
    if (fused)
      attn_mfma_kernel<64, true, true><<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(a);
    else
      attn_mfma_kernel<64, true, false><<<static_cast<unsigned>(grid), kThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moba
