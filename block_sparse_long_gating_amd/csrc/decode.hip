// Decode step: the newest token of a K/V cache attends its gated blocks.
//
// After the prefill, generation adds one token at a time; the pages run that
// step as full attention or, gated like a prefill row, as MoBA (wzjinhao.cn
// MoBA article, section 3). The token at position t = N - 1 (its key and value
// are the last rows of the cache) sits in block j = floor(t / B), which may be
// partial. Its gate scores the fp32 means of the complete past blocks
// 0 .. j-1 (same rule as the prefill gate: no scale, fp32 scores, ranking by
// score and then lower block index), keeps the k-1 best and always its own
// block; with k > j every past block is kept (full attention).
//
// Three launches, all tiny except the attention:
//   decode_gate_kernel    one workgroup per head: fp32 scores, k-1 rounds of a
//                         workgroup arg-max over 64-bit ranking keys, sorted
//                         selection row (own block included);
//   decode_attn_kernel    split over (head, selected block, chunk of
//                         kDecChunk keys): flash-decoding partial (m, l, o)
//                         per unit, 16-byte coalesced key/value rows, 8 dims
//                         per lane and D/8 lanes per key;
//   decode_combine_kernel one workgroup per head: log-sum-exp combination of
//                         the units into out (bf16) and lse (natural log).
// Memory-bound: the attention reads 4D bytes per attended key.
#include "common.h"
#include "kernels.h"

namespace moba {

namespace {

constexpr float kDecLn2 = 0.6931471805599453f;
constexpr int kDecMaxPast = 31;   // ranked past blocks kept (the boundary rejects more)

__global__ __launch_bounds__(256) void decode_gate_kernel(DecodeArgs a) {
  __shared__ uint64_t red[256];
  __shared__ int chosen[kDecMaxPast];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int j = a.j;
  const int S = a.S;                 // min(topk, j + 1) kept blocks
  int32_t* row = a.sel + static_cast<int64_t>(h) * S;
  if (a.sel_out != nullptr) {
    int32_t* ro = a.sel_out + static_cast<int64_t>(h) * a.topk;
    for (int s = S + tid; s < a.topk; s += 256) ro[s] = -1;
  }
  if (j + 1 <= a.topk) {
    // Every block 0..j is kept.
    for (int s = tid; s < S; s += 256) {
      row[s] = s;
      if (a.sel_out != nullptr) a.sel_out[static_cast<int64_t>(h) * a.topk + s] = s;
    }
    return;
  }
  // Scores of the past blocks i < j, kept in the workspace.
  float* sc = a.scores + static_cast<int64_t>(h) * a.j;
  const bf16* qh = a.q + static_cast<int64_t>(h) * a.D;
  for (int i = tid; i < j; i += 256) {
    const float* kb = a.kbar + (static_cast<int64_t>(h) * a.kbar_blocks + i) * a.D;
    float s = 0.f;
    for (int d = 0; d < a.D; ++d) s = fmaf(static_cast<float>(qh[d]), kb[d], s);
    sc[i] = s;
  }
  __syncthreads();
  // k - 1 rounds of arg-max over (score desc, block asc), skipping chosen blocks.
  const int nk = a.topk - 1;
  for (int r = 0; r < nk; ++r) {
    uint64_t best = 0;
    for (int i = tid; i < j; i += 256) {
      bool taken = false;
      for (int c = 0; c < r; ++c) taken |= chosen[c] == i;
      if (!taken) {
        const uint64_t key = rank_key(sc[i], i);
        best = key > best ? key : best;
      }
    }
    red[tid] = best;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (tid < off) red[tid] = red[tid] > red[tid + off] ? red[tid] : red[tid + off];
      __syncthreads();
    }
    if (tid == 0) chosen[r] = key_block(red[0]);
    __syncthreads();
  }
  // Ascending row: the chosen past blocks and the own block j (largest).
  if (tid < nk) {
    const int b = chosen[tid];
    int pos = 0;
    for (int c = 0; c < nk; ++c) pos += chosen[c] < b ? 1 : 0;
    row[pos] = b;
    if (a.sel_out != nullptr) a.sel_out[static_cast<int64_t>(h) * a.topk + pos] = b;
  }
  if (tid == 0) {
    row[nk] = j;
    if (a.sel_out != nullptr) a.sel_out[static_cast<int64_t>(h) * a.topk + nk] = j;
  }
}

// Partial attention of one (head, kept block, chunk) unit.
template <int D>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeArgs a) {
  constexpr int kLanes = D / 8;              // lanes per key (8 dims each)
  constexpr int kGroups = 256 / kLanes;      // keys in flight per workgroup
  __shared__ float sm_m[kGroups], sm_l[kGroups];
  __shared__ float sm_o[kGroups][D];
  const int h = blockIdx.y;
  const int u = blockIdx.x;                  // unit = slot * chunks + chunk
  const int slot = u / a.chunks, chunk = u % a.chunks;
  const int tid = threadIdx.x;
  const int li = tid % kLanes, g = tid / kLanes;
  const int b = a.sel[static_cast<int64_t>(h) * a.S + slot];
  const int64_t t = a.N - 1;
  int64_t k0 = static_cast<int64_t>(b) * a.B + static_cast<int64_t>(chunk) * kDecChunk;
  int64_t k1 = min(k0 + kDecChunk, static_cast<int64_t>(b + 1) * a.B);
  k1 = min(k1, t + 1);                       // the own block stops at the token itself
  const int64_t row_el = static_cast<int64_t>(a.H) * D;
  float qf[8];
  {
    const bf16x8 q8 = load_bf16x8(a.q + static_cast<int64_t>(h) * D + 8 * li);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = static_cast<float>(q8[e]) * a.scale_log2;
  }
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int64_t kk = k0 + g; kk < k1; kk += kGroups) {
    const int64_t off = kk * row_el + static_cast<int64_t>(h) * D + 8 * li;
    const bf16x8 k8 = load_bf16x8(a.k + off);
    const bf16x8 v8 = load_bf16x8(a.v + off);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(qf[e], static_cast<float>(k8[e]), s);
#pragma unroll
    for (int w = 1; w < kLanes; w <<= 1) s += __shfl_xor(s, w);
    const float mn = fmaxf(m, s);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);   // 0 when m was -inf
    const float p = __builtin_amdgcn_exp2f(s - mn);
    l = fmaf(l, alpha, p);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = fmaf(o[e], alpha, p * static_cast<float>(v8[e]));
    m = mn;
  }
  if (li == 0) {
    sm_m[g] = m;
    sm_l[g] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm_o[g][8 * li + e] = o[e];
  __syncthreads();
  // Combine the groups (fixed order): one thread per dim.
  float mt = -INFINITY;
  for (int x = 0; x < kGroups; ++x) mt = fmaxf(mt, sm_m[x]);
  const int64_t pu = static_cast<int64_t>(h) * a.units + u;
  for (int d = tid; d < D; d += 256) {
    float od = 0.f, lt = 0.f;
    for (int x = 0; x < kGroups; ++x) {
      const float w = sm_m[x] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm_m[x] - mt);
      od = fmaf(sm_o[x][d], w, od);
      lt = fmaf(sm_l[x], w, lt);
    }
    a.part_o[pu * D + d] = od;
    if (d == 0) {
      a.part_ml[2 * pu] = mt;
      a.part_ml[2 * pu + 1] = lt;
    }
  }
}

// Log-sum-exp combination of a head's units into out and lse.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int d = threadIdx.x;
  const int64_t p0 = static_cast<int64_t>(h) * a.units;
  float mt = -INFINITY;
  for (int u = 0; u < a.units; ++u) mt = fmaxf(mt, a.part_ml[2 * (p0 + u)]);
  float od = 0.f, lt = 0.f;
  for (int u = 0; u < a.units; ++u) {
    const float mu = a.part_ml[2 * (p0 + u)];
    const float w = mu == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mu - mt);
    od = fmaf(a.part_o[(p0 + u) * D + d], w, od);
    lt = fmaf(a.part_ml[2 * (p0 + u) + 1], w, lt);
  }
  a.out[static_cast<int64_t>(h) * D + d] = static_cast<bf16>(od / lt);
  if (d == 0) a.lse[h] = (mt + log2f(lt)) * kDecLn2;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  decode_gate_kernel<<<a.H, 256, 0, stream>>>(a);
  dim3 grid(a.units, a.H);
  if (a.D == 128) {
    decode_attn_kernel<128><<<grid, 256, 0, stream>>>(a);
    decode_combine_kernel<128><<<a.H, 128, 0, stream>>>(a);
  } else {
    decode_attn_kernel<64><<<grid, 256, 0, stream>>>(a);
    decode_combine_kernel<64><<<a.H, 64, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moba
