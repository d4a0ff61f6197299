// Shared device-side types and helpers of libmoba (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moba {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
// Queries per gate tile (4 waves x 32 queries).
constexpr int kQTile = 128;
// Queries per block-attention work item (8 waves x 32 queries).
constexpr int kAttnTile = 256;
// Extra partial-output rows past the end of each partial buffer: work-item
// slots without a query write there, so every lane of the attention kernel
// stores unconditionally.
constexpr int kDumpRows = kAttnTile;
// Keys per attention tile staged in LDS.
constexpr int kKTile = 64;
// Number of XCDs (L2 domains) of an MI355X; workgroups are dealt to them round-robin.
constexpr int kXcds = 8;
// Spacing (in int32) of the per-XCD work cursors: atomics from different XCDs
// on one cache line serialise.
constexpr int kCursorStride = 64;
constexpr int kCounterInts = kCursorStride * (1 + kXcds);

// One work item of the block-attention kernel over the off-diagonal (past block)
// query lists: head h, key block b, and `count` (<= kAttnTile) consecutive entries
// of the block's query list starting at global list position `start`.
struct WorkItem {
  int32_t h;
  int32_t b;
  int32_t start;
  int32_t count;
};

// Offsets (in bytes) and sizes of the per-call device workspace.
struct Workspace {
  float* kbar;          // [H][n][D] fp32 block mean keys
  bf16* kpieces;        // [H][n][3][D] bf16 exact 3-way split of kbar (bf16 path)
  int32_t* cnt;         // [H*n][ntiles] per-tile off-diagonal counts -> exclusive prefix
  int32_t* totals;      // [H*n] off-diagonal list length of every (head, block)
  int32_t* offs;        // [H*n + 1] global start of every (head, block) list, then the total
  int32_t* istart;      // [H*n] first work item of every (head, block) list
  int32_t* rk;          // [H][N][Lmax] rank of a query inside its tile's share of a list
  int32_t* qidx;        // [P_off] query of every list entry
  int32_t* inv;         // [H][N][Lmax] list position of each off-diagonal selection
  WorkItem* items;      // [max_items]
  int32_t* counters;    // [0]: number of off-diagonal items; per-XCD item cursors at
                        // [kCursorStride * (1 + x)], one cache line apart
  void* part_diag;      // [H][N][D] own-block partial outputs (bf16 or fp32)
  float* lse_diag;      // [H][N]
  void* part_off;       // [P_off][D] past-block partial outputs
  float* lse_off;       // [P_off]
  int32_t* sel;         // [H][N][topk] (prefill only; gate_topk writes the caller's)
};

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ uint4 load_u4(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Order-preserving map of an fp32 score onto uint32 (larger score -> larger
// key). -0 is folded onto +0 so that equal scores compare equal.
__device__ __forceinline__ uint32_t orderable(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Ranking key of (score, block): higher score first, then lower block index.
__device__ __forceinline__ uint64_t rank_key(float score, int block) {
  return (static_cast<uint64_t>(orderable(score)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(block));
}

__device__ __forceinline__ int key_block(uint64_t key) {
  return static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

// Insert `key` into the descending list `a` of KCAP distinct keys, dropping the
// smallest (0 marks an empty slot; every real key is > 0).
template <int KCAP>
__device__ __forceinline__ void topk_insert(uint64_t (&a)[KCAP], uint64_t key) {
#pragma unroll
  for (int i = KCAP - 1; i > 0; --i) {
    const uint64_t lo = a[i - 1] < key ? a[i - 1] : key;
    a[i] = a[i] > lo ? a[i] : lo;
  }
  a[0] = a[0] > key ? a[0] : key;
}

__device__ __forceinline__ float wave_max_pair(float x) {  // max with the lane 32 away
  return fmaxf(x, __shfl_xor(x, 32));
}

}  // namespace moba
