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
// Launches, in stream order:
//   decode_gate_kernel    (gated only) one workgroup per head: fp32 scores
//                         (8 dims per lane, several block rows in flight),
//                         k-1 rounds of a workgroup arg-max over 64-bit
//                         ranking keys, sorted selection row (own block
//                         included); with every block kept the selection is
//                         the identity and this launch is skipped;
//   decode_attn_kernel    split over (head, kept block, chunk of keys):
//                         flash-decoding partial (m, l, o) per unit, 16-byte
//                         coalesced key/value rows, 8 dims per lane, D/8
//                         lanes per key and kDecKeys keys in flight per lane group;
//   decode_combine_kernel one workgroup per head: log-sum-exp combination of
//                         the head's units (float4 columns, units split over
//                         the workgroup) into out (bf16) and lse (natural log).
// Memory-bound: the attention reads 4D bytes per attended key.
#include "common.h"
#include "kernels.h"

namespace moba {

namespace {

constexpr float kDecLn2 = 0.6931471805599453f;
constexpr int kDecMaxPast = 31;   // ranked past blocks kept (the boundary rejects more)
constexpr int kDecLdsScores = 2048;   // gate scores held in LDS up to this many past blocks
constexpr int kDecKeys = 2;           // keys in flight per lane group in the attention

__device__ __forceinline__ float dot8(const float (&q)[8], const float4& x0, const float4& x1) {
  float s = q[0] * x0.x;
  s = fmaf(q[1], x0.y, s);
  s = fmaf(q[2], x0.z, s);
  s = fmaf(q[3], x0.w, s);
  s = fmaf(q[4], x1.x, s);
  s = fmaf(q[5], x1.y, s);
  s = fmaf(q[6], x1.z, s);
  s = fmaf(q[7], x1.w, s);
  return s;
}

template <int D>
__global__ __launch_bounds__(256) void decode_gate_kernel(DecodeArgs a) {
  constexpr int kL = D / 8;          // lanes per block-mean row, 8 dims each
  constexpr int kRows = 256 / kL;    // rows per pass of the workgroup
  constexpr int kU = 4;              // passes in flight
  __shared__ uint64_t red[4];
  __shared__ int chosen[kDecMaxPast];
  __shared__ float sc_lds[kDecLdsScores];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int j = a.j;                 // > topk - 1 here: the gate has a choice to make
  const int S = a.S;                 // topk kept blocks
  int32_t* row = a.sel + static_cast<int64_t>(h) * S;
  int32_t* ro = a.sel_out != nullptr ? a.sel_out + static_cast<int64_t>(h) * a.topk : nullptr;
  // Scores of the past blocks i < j: in LDS, or in the workspace when there are many.
  float* sc = j <= kDecLdsScores ? sc_lds : a.scores + static_cast<int64_t>(h) * j;
  const int li = tid % kL;
  float qf[8];
  {
    const bf16x8 q8 = load_bf16x8(a.q + static_cast<int64_t>(h) * D + 8 * li);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = static_cast<float>(q8[e]);
  }
  const float* kb = a.kbar + static_cast<int64_t>(h) * a.kbar_blocks * D + 8 * li;
  for (int i0 = tid / kL; i0 < j; i0 += kU * kRows) {
    float4 x[kU][2];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(i0 + u * kRows, j - 1);   // rows past j - 1 re-read the last one and are dropped
      const float4* p = reinterpret_cast<const float4*>(kb + static_cast<int64_t>(i) * D);
      x[u][0] = p[0];
      x[u][1] = p[1];
    }
    float s[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) s[u] = dot8(qf, x[u][0], x[u][1]);
#pragma unroll
    for (int w = 1; w < kL; w <<= 1) {
#pragma unroll
      for (int u = 0; u < kU; ++u) s[u] += __shfl_xor(s[u], w);
    }
    if (li == 0) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (i0 + u * kRows < j) sc[i0 + u * kRows] = s[u];
    }
  }
  __syncthreads();
  // k - 1 rounds of arg-max over (score desc, block asc), skipping chosen blocks.
  const int nk = a.topk - 1;
  const int lane = tid & 63, wave = tid >> 6;
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
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
      const uint64_t o = __shfl_xor(best, w);
      best = o > best ? o : best;
    }
    if (lane == 0) red[wave] = best;
    __syncthreads();
    if (tid == 0) {
      uint64_t m = red[0];
#pragma unroll
      for (int x = 1; x < 4; ++x) m = red[x] > m ? red[x] : m;
      chosen[r] = key_block(m);
    }
    __syncthreads();
  }
  // Ascending row: the chosen past blocks and the own block j (largest).
  if (tid < nk) {
    const int b = chosen[tid];
    int pos = 0;
    for (int c = 0; c < nk; ++c) pos += chosen[c] < b ? 1 : 0;
    row[pos] = b;
    if (ro != nullptr) ro[pos] = b;
  }
  if (tid == 0) {
    row[nk] = j;
    if (ro != nullptr) ro[nk] = j;
  }
}

typedef unsigned u32x4nt __attribute__((ext_vector_type(4)));

// 16-byte non-temporal load (data read once).
__device__ __forceinline__ bf16x8 load_stream(const bf16* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4nt*>(p)));
}

// Partial attention of one (head, kept block, chunk) unit; the last unit of a
// head to finish also combines the head.
template <int D>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeArgs a) {
  constexpr int kLanes = D / 8;              // lanes per key (8 dims each)
  constexpr int kGroups = 256 / kLanes;      // lane groups per workgroup
  __shared__ float sm_m[kGroups], sm_l[kGroups];
  __shared__ float sm_o[kGroups][D];
  const int h = blockIdx.y;
  const int u = blockIdx.x;                  // unit = slot * chunks + chunk
  const int slot = u / a.chunks, chunk = u % a.chunks;
  const int tid = threadIdx.x;
  const int li = tid % kLanes, g = tid / kLanes;
  const int b = a.S == a.j + 1 ? slot : a.sel[static_cast<int64_t>(h) * a.S + slot];   // all kept: identity
  const int64_t t = a.N - 1;
  const int64_t k0 = static_cast<int64_t>(b) * a.B + static_cast<int64_t>(chunk) * a.chunk;
  int64_t k1 = min(k0 + a.chunk, static_cast<int64_t>(b + 1) * a.B);
  k1 = min(k1, t + 1);                       // the own block stops at the token itself
  const int64_t row_el = static_cast<int64_t>(a.H) * D;
  const int64_t col = static_cast<int64_t>(h) * D + 8 * li;
  float qf[8];
  {
    const bf16x8 q8 = load_bf16x8(a.q + col);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = static_cast<float>(q8[e]) * a.scale_log2;
  }
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int64_t kk = k0 + g; kk < k1; kk += kDecKeys * kGroups) {
    // kDecKeys keys per lane group, kGroups apart (a key past the end re-reads
    // kk and is masked out).
    // This path serves the long attended sets (every block kept, or more keys
    // than the one-launch step takes), whose keys and values stream through
    // once: non-temporal loads (h32, every block kept: 113.6 -> 100.0 us).
    bf16x8 k8[kDecKeys], v8[kDecKeys];
#pragma unroll
    for (int x = 0; x < kDecKeys; ++x) {
      const int64_t kx = kk + x * kGroups < k1 ? kk + x * kGroups : kk;
      k8[x] = load_stream(a.k + kx * row_el + col);
      v8[x] = load_stream(a.v + kx * row_el + col);
    }
    float s[kDecKeys];
#pragma unroll
    for (int x = 0; x < kDecKeys; ++x) {
      s[x] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s[x] = fmaf(qf[e], static_cast<float>(k8[x][e]), s[x]);
    }
#pragma unroll
    for (int w = 1; w < kLanes; w <<= 1) {
#pragma unroll
      for (int x = 0; x < kDecKeys; ++x) s[x] += __shfl_xor(s[x], w);
    }
    float mn = m;
#pragma unroll
    for (int x = 0; x < kDecKeys; ++x) {
      if (kk + x * kGroups >= k1) s[x] = -INFINITY;
      mn = fmaxf(mn, s[x]);
    }
    const float alpha = __builtin_amdgcn_exp2f(m - mn);   // 0 when m was -inf
    float p[kDecKeys];
    float ps = 0.f;
#pragma unroll
    for (int x = 0; x < kDecKeys; ++x) {
      p[x] = __builtin_amdgcn_exp2f(s[x] - mn);            // 0 for a masked key
      ps += p[x];
    }
    l = fmaf(l, alpha, ps);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float pv = 0.f;
#pragma unroll
      for (int x = 0; x < kDecKeys; ++x) pv = fmaf(p[x], static_cast<float>(v8[x][e]), pv);
      o[e] = fmaf(o[e], alpha, pv);
    }
    m = mn;
  }
  if (li == 0) {
    sm_m[g] = m;
    sm_l[g] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm_o[g][8 * li + e] = o[e];
  __syncthreads();
  // Combine the lane groups (fixed order): one thread per dim.
  const int64_t p0 = static_cast<int64_t>(h) * a.units;
  const int64_t pu = p0 + u;
  if (tid < D) {
    float mt = -INFINITY;
    for (int x = 0; x < kGroups; ++x) mt = fmaxf(mt, sm_m[x]);
    float od = 0.f, lt = 0.f;
    for (int x = 0; x < kGroups; ++x) {
      const float w = sm_m[x] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm_m[x] - mt);
      od = fmaf(sm_o[x][tid], w, od);
      lt = fmaf(sm_l[x], w, lt);
    }
    a.part_o[pu * D + tid] = od;
    if (tid == 0) {
      a.part_ml[2 * pu] = mt;
      a.part_ml[2 * pu + 1] = lt;
    }
  }
}

// Log-sum-exp combination of a head's units into out and lse.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int kQ = D / 4;          // float4 columns of a partial output
  constexpr int kSp = 256 / kQ;      // unit splits over the workgroup
  __shared__ float4 s_o[kSp][kQ];
  __shared__ float s_m[kSp], s_l[kSp];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int c = tid % kQ, sp = tid / kQ;
  if (a.S == a.j + 1 && a.sel_out != nullptr) {
    // All blocks kept (no gate launch): the selection row is the identity.
    for (int s = tid; s < a.topk; s += 256) a.sel_out[static_cast<int64_t>(h) * a.topk + s] = s < a.S ? s : -1;
  }
  const int64_t p0 = static_cast<int64_t>(h) * a.units;
  const float4* po = reinterpret_cast<const float4*>(a.part_o);
  float m = -INFINITY;
  for (int x = sp; x < a.units; x += kSp) m = fmaxf(m, a.part_ml[2 * (p0 + x)]);
  float4 od = make_float4(0.f, 0.f, 0.f, 0.f);
  float lt = 0.f;
  for (int x = sp; x < a.units; x += kSp) {
    const float mu = a.part_ml[2 * (p0 + x)];
    const float w = mu == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mu - m);
    const float4 o4 = po[(p0 + x) * kQ + c];
    od.x = fmaf(o4.x, w, od.x);
    od.y = fmaf(o4.y, w, od.y);
    od.z = fmaf(o4.z, w, od.z);
    od.w = fmaf(o4.w, w, od.w);
    lt = fmaf(a.part_ml[2 * (p0 + x) + 1], w, lt);
  }
  s_o[sp][c] = od;
  if (c == 0) {
    s_m[sp] = m;
    s_l[sp] = lt;
  }
  __syncthreads();
  if (tid < kQ) {
    float mt = -INFINITY;
#pragma unroll
    for (int x = 0; x < kSp; ++x) mt = fmaxf(mt, s_m[x]);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
#pragma unroll
    for (int x = 0; x < kSp; ++x) {
      const float w = s_m[x] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[x] - mt);
      o.x = fmaf(s_o[x][tid].x, w, o.x);
      o.y = fmaf(s_o[x][tid].y, w, o.y);
      o.z = fmaf(s_o[x][tid].z, w, o.z);
      o.w = fmaf(s_o[x][tid].w, w, o.w);
      l = fmaf(s_l[x], w, l);
    }
    bf16* dst = a.out + static_cast<int64_t>(h) * D + 4 * tid;
    dst[0] = static_cast<bf16>(o.x / l);
    dst[1] = static_cast<bf16>(o.y / l);
    dst[2] = static_cast<bf16>(o.z / l);
    dst[3] = static_cast<bf16>(o.w / l);
    if (tid == 0) a.lse[h] = (mt + log2f(l)) * kDecLn2;
  }
}

// Gated decode in one launch: one 1024-thread workgroup per head gates, attends
// its kept keys and combines them in LDS (no workspace). For a few thousand
// kept keys, where three launches and a workspace cost more than the work.
constexpr int kFusedThreads = 1024;
constexpr int kFusedKeys = 8;          // keys in flight per lane group

template <int D>
__global__ __launch_bounds__(kFusedThreads) void decode_fused_kernel(DecodeArgs a) {
  constexpr int kL = D / 8;                          // lanes per row (8 dims each)
  constexpr int kGroups = kFusedThreads / kL;        // lane groups
  constexpr int kWavesF = kFusedThreads / 64;
  __shared__ float sc[kDecLdsScores];
  __shared__ uint64_t red[kWavesF];
  __shared__ int chosen[kDecMaxPast];
  __shared__ int srow[kDecMaxPast + 1];
  __shared__ float sm_m[kGroups], sm_l[kGroups];
  __shared__ float sm_o[kGroups][D];
  const int h = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = tid % kL, g = tid / kL;
  const int j = a.j, S = a.S;                        // j >= topk here: the gate chooses
  // ---- gate: fp32 scores of the complete past blocks, then k - 1 arg-max rounds ----
  float qf[8];
  {
    const bf16x8 q8 = load_bf16x8(a.q + static_cast<int64_t>(h) * D + 8 * li);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[e] = static_cast<float>(q8[e]);
  }
  const float* kb = a.kbar + static_cast<int64_t>(h) * a.kbar_blocks * D + 8 * li;
  for (int i0 = g; i0 < j; i0 += 4 * kGroups) {
    float4 x[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = min(i0 + u * kGroups, j - 1);
      const float4* p = reinterpret_cast<const float4*>(kb + static_cast<int64_t>(i) * D);
      x[u][0] = p[0];
      x[u][1] = p[1];
    }
    float sv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) sv[u] = dot8(qf, x[u][0], x[u][1]);
#pragma unroll
    for (int w = 1; w < kL; w <<= 1)
#pragma unroll
      for (int u = 0; u < 4; ++u) sv[u] += __shfl_xor(sv[u], w);
    if (li == 0)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u * kGroups < j) sc[i0 + u * kGroups] = sv[u];
  }
  __syncthreads();
  const int nk = a.topk - 1;
  for (int r = 0; r < nk; ++r) {
    uint64_t best = 0;
    for (int i = tid; i < j; i += kFusedThreads) {
      bool taken = false;
      for (int c = 0; c < r; ++c) taken |= chosen[c] == i;
      if (!taken) {
        const uint64_t key = rank_key(sc[i], i);
        best = key > best ? key : best;
      }
    }
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
      const uint64_t o = __shfl_xor(best, w);
      best = o > best ? o : best;
    }
    if (lane == 0) red[wave] = best;
    __syncthreads();
    if (tid == 0) {
      uint64_t m = red[0];
      for (int x = 1; x < kWavesF; ++x) m = red[x] > m ? red[x] : m;
      chosen[r] = key_block(m);
    }
    __syncthreads();
  }
  if (tid < nk) {
    const int b = chosen[tid];
    int pos = 0;
    for (int c = 0; c < nk; ++c) pos += chosen[c] < b ? 1 : 0;
    srow[pos] = b;
  }
  if (tid == 0) srow[nk] = j;
  __syncthreads();
  if (a.sel_out != nullptr && tid < a.topk)
    a.sel_out[static_cast<int64_t>(h) * a.topk + tid] = tid < S ? srow[tid] : -1;
  // ---- attention over the kept keys: (S - 1) full blocks, then the own block up to t ----
  const int64_t t = a.N - 1;
  const int nkeys = (S - 1) * a.B + static_cast<int>(t - static_cast<int64_t>(j) * a.B) + 1;
  const int64_t row_el = static_cast<int64_t>(a.H) * D;
  const int64_t col = static_cast<int64_t>(h) * D + 8 * li;
#pragma unroll
  for (int e = 0; e < 8; ++e) qf[e] *= a.scale_log2;
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  // This lane group's kept key f = g, g + kGroups, ... as (slot, offset in the
  // block), advanced incrementally (no division per key).
  int slot = g / a.B, off = g % a.B;
  int64_t last_key = t;                                 // the final kept key (the token itself)
  for (int f0 = g; f0 < nkeys; f0 += kFusedKeys * kGroups) {
    bf16x8 k8[kFusedKeys], v8[kFusedKeys];
#pragma unroll
    for (int x = 0; x < kFusedKeys; ++x) {
      // Past the end: re-read the last key (masked below).
      const int64_t key = f0 + x * kGroups < nkeys ? static_cast<int64_t>(srow[slot]) * a.B + off : last_key;
      k8[x] = load_bf16x8(a.k + key * row_el + col);
      v8[x] = load_bf16x8(a.v + key * row_el + col);
      off += kGroups;
      while (off >= a.B && slot < S - 1) {
        off -= a.B;
        ++slot;
      }
    }
    float sv[kFusedKeys];
#pragma unroll
    for (int x = 0; x < kFusedKeys; ++x) {
      sv[x] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[x] = fmaf(qf[e], static_cast<float>(k8[x][e]), sv[x]);
    }
#pragma unroll
    for (int w = 1; w < kL; w <<= 1)
#pragma unroll
      for (int x = 0; x < kFusedKeys; ++x) sv[x] += __shfl_xor(sv[x], w);
    float mn = m;
#pragma unroll
    for (int x = 0; x < kFusedKeys; ++x) {
      if (f0 + x * kGroups >= nkeys) sv[x] = -INFINITY;
      mn = fmaxf(mn, sv[x]);
    }
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    float ps = 0.f, pr[kFusedKeys];
#pragma unroll
    for (int x = 0; x < kFusedKeys; ++x) {
      pr[x] = __builtin_amdgcn_exp2f(sv[x] - mn);
      ps += pr[x];
    }
    l = fmaf(l, alpha, ps);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float pv = 0.f;
#pragma unroll
      for (int x = 0; x < kFusedKeys; ++x) pv = fmaf(pr[x], static_cast<float>(v8[x][e]), pv);
      o[e] = fmaf(o[e], alpha, pv);
    }
    m = mn;
  }
  if (li == 0) {
    sm_m[g] = m;
    sm_l[g] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm_o[g][8 * li + e] = o[e];
  __syncthreads();
  if (tid < D) {
    float mt = -INFINITY;
    for (int x = 0; x < kGroups; ++x) mt = fmaxf(mt, sm_m[x]);
    float od = 0.f, lt = 0.f;
    for (int x = 0; x < kGroups; ++x) {
      const float w = sm_m[x] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm_m[x] - mt);
      od = fmaf(sm_o[x][tid], w, od);
      lt = fmaf(sm_l[x], w, lt);
    }
    a.out[static_cast<int64_t>(h) * D + tid] = static_cast<bf16>(od / lt);
    if (tid == 0) a.lse[h] = (mt + log2f(lt)) * kDecLn2;
  }
}

}  // namespace

bool decode_fused(const DecodeArgs& a) {
  const int64_t keys = static_cast<int64_t>(a.S - 1) * a.B + (a.N - 1 - static_cast<int64_t>(a.j) * a.B) + 1;
  return a.kbar != nullptr && a.S < a.j + 1 && a.j <= kDecLdsScores && keys <= kDecFusedMaxKeys;
}

hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t stream) {
  if (a.D == 128) decode_fused_kernel<128><<<a.H, kFusedThreads, 0, stream>>>(a);
  else decode_fused_kernel<64><<<a.H, kFusedThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.units, a.H);
  const bool gated = a.S < a.j + 1;
  if (a.D == 128) {
    if (gated) decode_gate_kernel<128><<<a.H, 256, 0, stream>>>(a);
    decode_attn_kernel<128><<<grid, 256, 0, stream>>>(a);
    decode_combine_kernel<128><<<a.H, 256, 0, stream>>>(a);
  } else {
    if (gated) decode_gate_kernel<64><<<a.H, 256, 0, stream>>>(a);
    decode_attn_kernel<64><<<grid, 256, 0, stream>>>(a);
    decode_combine_kernel<64><<<a.H, 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moba
