// Gate and causal top-k (with the first half of the per-block query lists).
//
// For query t in block j the gate score of past block i < j is <q_t, kbar_i>
// in fp32, with no scale (pomoai MoBA overview, "核心原理" step 2; 智东西 report,
// section 二, relevance score). The current block j is always kept and the
// topk - 1 best past blocks are added, ranked by score and then by lower block
// index; future blocks are never scored (wzjinhao.cn MoBA article, section 3,
// causal_mask and current_block_force). Rows with j < topk keep all of 0..j.
//
// bf16 path: one workgroup = 4 waves x 32 queries. The scores of 32 blocks x
// 32 queries come from bf16 MFMA (v_mfma_f32_32x32x16_bf16) with the block
// means as the A operand (rows = blocks) and the queries as the B operand
// (columns = queries), so each lane ends up holding 16 block scores of one
// query. The fp32 mean is fed as its exact 3-way bf16 split (hi + mid + lo),
// and since q is bf16 every product is exact and the score carries only fp32
// accumulation error. Each lane keeps a sorted register list of the best keys
// and merges it with the lane 32 away, which holds the other 16 blocks.
//
// fp32 path: the same lane layout, but each lane forms full fp32 dot products
// for every other block with vector FMAs.
//
// When the query lists are wanted, the workgroup also records, per past block,
// which of its 128 queries kept it (an LDS bitmap built with integer ORs), and
// writes the per-tile count and each query's rank inside the tile. The lists
// come out ordered by query position, independent of scheduling.
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
};

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), m);
  const uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), m);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

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
                                         int j, uint32_t* bm) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int qn = lane & 31;
  const int half = lane >> 5;
  const int h = blockIdx.y;
  const int topk = a.topk;
  const bool ranked = j >= topk;   // more past blocks than slots: the gate decides
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
      for (int s = 0; s < topk; ++s) srow[s] = s <= j ? s : -1;
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
      for (int b = 0; b < j; ++b) atomicOr(mine + b, bit);
    } else {
#pragma unroll
      for (int s = 0; s < KCAP; ++s)
        if (s < nk) atomicOr(mine + key_block(list[s]), bit);
    }
  }
  __syncthreads();
  const int tile = blockIdx.x;
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
      for (int b = 0; b < j; ++b) rrow[b] = rank_of(b);
    } else {
#pragma unroll
      for (int s = 0; s < KCAP; ++s)
        if (s < nk) rrow[pos[s]] = rank_of(key_block(list[s]));
    }
  }
}

template <int D, int KCAP>
__global__ __launch_bounds__(256) void gate_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ pieces,
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
  const int64_t tlast = (t0w + 31 < a.N) ? t0w + 31 : a.N - 1;
  const int jw = static_cast<int>(tlast / a.B);   // largest block of the wave

  uint64_t list[KCAP];
#pragma unroll
  for (int s = 0; s < KCAP; ++s) list[s] = 0;

  if (jw >= a.topk && a.topk > 1 && t0w < a.N) {
    bf16x8 qop[D / 16];
    const bf16* qrow = q + (tc * a.H + h) * D + 8 * half;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qop[c] = load_bf16x8(qrow + 16 * c);

    for (int bc = 0; bc * 32 < jw; ++bc) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      const int brow = min(bc * 32 + qn, a.n - 1);
      const bf16* prow = pieces + (static_cast<int64_t>(h) * a.n + brow) * 3 * D + 8 * half;
#pragma unroll
      for (int p = 0; p < 3; ++p) {
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_bf16x8(prow + p * D + 16 * c), qop[c], acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int b = bc * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        topk_insert<KCAP>(list, b < j ? rank_key(acc[r], b) : 0ull);
      }
    }
    merge_with_partner<KCAP>(list);
  }
  finalize<KCAP>(a, list, t, valid, j, bm);
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
      topk_insert<KCAP>(list, b < j ? rank_key(s, b) : 0ull);
    }
    merge_with_partner<KCAP>(list);
  }
  finalize<KCAP>(a, list, t, valid, j, bm);
}

template <int D, int KCAP>
hipError_t launch_gate_t(const Problem& p, const void* q, const Workspace& ws, int32_t* sel, bool csr,
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
  dim3 grid(p.ntiles, p.H);
  const size_t smem = csr ? static_cast<size_t>(4) * p.n * sizeof(uint32_t) : 0;
  if (p.is_f32)
    gate_f32_kernel<D, KCAP><<<grid, 256, smem, stream>>>(static_cast<const float*>(q), ws.kbar, a);
  else
    gate_bf16_kernel<D, KCAP><<<grid, 256, smem, stream>>>(static_cast<const bf16*>(q), ws.kpieces, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_gate_d(const Problem& p, const void* q, const Workspace& ws, int32_t* sel, bool csr,
                         hipStream_t stream) {
  const int need = p.topk - 1;  // ranked slots (only used when a row has more past blocks than that)
  if (need <= 2) return launch_gate_t<D, 2>(p, q, ws, sel, csr, stream);
  if (need <= 4) return launch_gate_t<D, 4>(p, q, ws, sel, csr, stream);
  if (need <= 8) return launch_gate_t<D, 8>(p, q, ws, sel, csr, stream);
  if (need <= 12) return launch_gate_t<D, 12>(p, q, ws, sel, csr, stream);
  if (need <= 16) return launch_gate_t<D, 16>(p, q, ws, sel, csr, stream);
  return launch_gate_t<D, 32>(p, q, ws, sel, csr, stream);
}

}  // namespace

hipError_t launch_gate(const Problem& p, const void* q, const Workspace& ws, int32_t* sel, bool csr,
                       hipStream_t stream) {
  return p.D == 128 ? launch_gate_d<128>(p, q, ws, sel, csr, stream) : launch_gate_d<64>(p, q, ws, sel, csr, stream);
}

}  // namespace moba
