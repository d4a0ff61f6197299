// Launchers of the libmoba kernels (host side). Every launcher only enqueues on
// `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <functional>

#include "common.h"

namespace moba {

// Parameters of the gate / CSR / attention / merge stages of one call.
struct Problem {
  int64_t N;
  int H, D, B, n, topk;
  int lmax;        // largest number of past blocks a query keeps: min(topk - 1, n - 1)
  int ntiles;      // ceil(N / kQTile) gate tiles per head
  int64_t p_off;   // total number of (query, past block) pairs over all heads
  int64_t max_items;   // upper bound on off-diagonal work items
  int64_t diag_items;  // own-block work items: H * n * ceil(B / kAttnTile)
  bool is_f32;
  // Several sequences packed along N (each a whole number of blocks): blo[j]
  // is the first block of block j's sequence, the lowest block its queries may
  // select. nullptr: one sequence (blo[j] = 0).
  const int32_t* blo = nullptr;
};

// Past blocks a query of block j keeps: min(topk - 1, j - lo) with lo the first
// block of its sequence.
__host__ __device__ inline int kept_past(int j, int lo, int topk) { return j - lo < topk - 1 ? j - lo : topk - 1; }

// Sequence starts in block units for the blo table (at most kMaxSeqs sequences).
constexpr int kMaxSeqs = 512;
struct SeqStarts {
  int32_t nseq;
  int32_t start[kMaxSeqs + 1];   // start[s] = first block of sequence s; start[nseq] = n
};
hipError_t launch_seq_lo(const SeqStarts& st, int32_t* blo, int n, hipStream_t stream);

// Fills `bytes` (a multiple of 16) at the 16-byte aligned `p` with copies of `value`.
hipError_t launch_fill(void* p, size_t bytes, uint32_t value, hipStream_t stream);

// Block pooling modes (MOBA_POOL_* in moba.h).
constexpr int kPoolMean = 0, kPoolMax = 1, kPoolWeighted = 2;
// Block keys (and their 3-way bf16 split when `pieces` is not null). `weights`
// [H][N] is read in the weighted mode only.
hipError_t launch_pool(const void* k, bool is_f32, float* kbar, bf16* pieces, int64_t N, int H, int D, int B,
                       hipStream_t stream, int mode = kPoolMean, const float* weights = nullptr);

// Gate + causal top-k; writes sel and, when `ws_csr` is true, the per-tile
// counts and in-tile ranks of the off-diagonal selections.
hipError_t launch_gate(const Problem& p, const void* q, const Workspace& ws, int32_t* sel, bool ws_csr, int num_cus,
                       hipStream_t stream);

// Scans, list scatter and work-list construction.
hipError_t launch_csr(const Problem& p, const Workspace& ws, const int32_t* sel, hipStream_t stream);

// Block attention over the off-diagonal work items and the own-block items.
// When merge_fused(p), the own-block pass also performs the LSE merge and
// writes out and lse; launch_merge is then not needed.
// `mark(4)` is called between the past-block and the own-block launches (stage timing).
bool merge_fused(const Problem& p);
hipError_t launch_attention(const Problem& p, const void* q, const void* k, const void* v, const Workspace& ws,
                            void* out, float* lse, int num_cus, hipStream_t stream,
                            const std::function<hipError_t(int)>& mark);

// Log-sum-exp merge of the partial outputs into out and lse.
hipError_t launch_merge(const Problem& p, const Workspace& ws, void* out, float* lse, hipStream_t stream);

// Decode step (bf16): the token at position N - 1 of a K/V cache.
constexpr int kDecMaxChunk = 512;   // largest number of keys per attention unit
struct DecodeArgs {
  const bf16* q;        // [H][D] query of the new token
  const bf16* k;        // [N][H][D] cache (the new token's key and value are the last rows)
  const bf16* v;
  const float* kbar;    // [H][kbar_blocks][D] fp32 means of the complete blocks (at least j of them)
  int kbar_blocks;
  int32_t* sel;         // [H][S] kept blocks, ascending (own block last); unused when S == j + 1
  int32_t* sel_out;     // optional [H][topk] copy, -1 padded
  float* scores;        // [H][j] gate scores (used when j exceeds the LDS capacity)
  float* part_o;        // [H][units][D] unnormalised partial outputs
  float* part_ml;       // [H][units][2] partial (max, sum) in log2 units
  bf16* out;            // [H][D]
  float* lse;           // [H] natural log
  int64_t N;
  int H, D, B, j, topk, S;
  int chunk;            // keys per unit (64 .. 512)
  int chunks;           // units per kept block: ceil(B / chunk)
  int units;            // S * chunks
  float scale_log2;     // log2(e) / sqrt(D)
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Records `e` as the calling thread's last HIP error; returns MOBA_ERR_HIP.
int fail_hip(hipError_t e);
// moba_decode_fwd with its workspace in the caller's `ws` (ws_bytes long)
// instead of the library's pool: argument checks, then every launch on
// `stream`; MOBA_ERR_UNSUPPORTED when the call needs more than ws_bytes.
// Returns a moba status.
int decode_with_workspace(const void* q, const void* k, const void* v, const float* kbar, int32_t kbar_blocks,
                          void* out, float* lse, int32_t* sel, int64_t N, int32_t H, int32_t D, int32_t block_size,
                          int32_t topk, hipStream_t stream, char* ws, size_t ws_bytes);
// One-launch gated decode (no workspace): the caller's block means, a gate
// choice to make, at most 2048 past blocks and kDecFusedMaxKeys kept keys.
constexpr int kDecFusedMaxKeys = 8192;
bool decode_fused(const DecodeArgs& a);
hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t stream);

// Backward pass of the bf16 prefill: dQ, dK, dV of the output (the selection
// and the query lists come from the gate and list stages of the same call).
struct BwdArgs {
  const bf16* q;        // [N][H][D]
  const bf16* k;
  const bf16* v;
  const bf16* out;      // forward output [N][H][D]
  const bf16* dout;     // upstream gradient of out [N][H][D]
  const float* lse;     // forward log-sum-exp [H][N], natural log
  bf16* dq;             // [N][H][D]
  bf16* dk;
  bf16* dv;
  float* delta;         // [H][N] workspace: sum over d of dout * out
  float* part_dq;       // [P_off][D] workspace: past-block dQ partials in list order (unscaled)
  const int32_t* qidx;  // list entries (token of every (query, past block) pair)
  const int32_t* offs;  // [H*n] list starts
  const int32_t* totals;  // [H*n] list lengths
  const int32_t* inv;   // [H][N][lmax] list position of each past selection
  const WorkItem* items;  // past-block work items (count in counters[0])
  const int32_t* counters;
  int64_t N;
  int H, D, B, n, topk, lmax;
  int64_t max_items;
  int num_cus;            // compute units of the device (0: unknown)
  int has_lists;        // 0: no query lists (every block kept; one block of N tokens)
  const int32_t* blo;   // per-block first block of its sequence (packed sequences), or nullptr
  float scale;          // 1 / sqrt(D)
  float scale_log2;     // log2(e) / sqrt(D)
};
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);

}  // namespace moba
