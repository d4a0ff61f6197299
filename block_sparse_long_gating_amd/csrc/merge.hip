// Log-sum-exp merge of the per-block partial outputs (the "online softmax"
// combination and output reordering of the 智东西 report, section 二,
// implementation steps 4-5; the LSE-weighted fusion of the pomoai MoBA overview,
// "核心原理" step 3).
//
// For query t of head h the partials are its own-block partial and one partial
// per kept past block, each normalised over its own keys and carrying its own
// lse_s. Then lse = log sum_s exp(lse_s) and out = sum_s exp(lse_s - lse) * O_s,
// which equals one softmax over the union of the keys (the key sets are
// disjoint). HBM-bound: every partial is read once, out and lse written once.
//
// D/8 lanes per (token, head); consecutive lane groups take consecutive
// (token, head) pairs so the [N][H][D] output rows are written contiguously.
#include "common.h"
#include "kernels.h"

namespace moba {

namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]);

template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float (&x)[8]) {
  const bf16x8 v = load_bf16x8(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(v[e]);
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&x)[8]);

template <>
__device__ __forceinline__ void store8<bf16>(bf16* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = static_cast<bf16>(x[e]);
  *reinterpret_cast<uint4*>(p) = __builtin_bit_cast(uint4, v);
}

template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&x)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

template <typename T>
struct MergeArgs {
  const T* part_diag;
  const float* lse_diag;
  const T* part_off;
  const float* lse_off;
  const int32_t* inv;
  T* out;
  float* lse;
  int64_t N;
  int H, B, topk, lmax;
  const int32_t* blo;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs<T> a) {
  constexpr int kLanes = D / 8;
  const int64_t g = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / kLanes;
  const int sub = threadIdx.x % kLanes;
  if (g >= a.N * a.H) return;
  const int64_t t = g / a.H;
  const int h = static_cast<int>(g % a.H);
  const int j = static_cast<int>(t / a.B);
  const int L = kept_past(j, a.blo != nullptr ? a.blo[j] : 0, a.topk);
  const int64_t dr = static_cast<int64_t>(h) * a.N + t;
  const int32_t* irow = a.inv + dr * a.lmax;

  const float ld = a.lse_diag[dr];
  float m = ld;
  for (int s = 0; s < L; ++s) m = fmaxf(m, a.lse_off[irow[s]]);
  float z = expf(ld - m);
  for (int s = 0; s < L; ++s) z += expf(a.lse_off[irow[s]] - m);
  const float lse = m + logf(z);

  float acc[8], x[8];
  {
    const float wgt = expf(ld - lse);
    load8<T>(a.part_diag + dr * D + 8 * sub, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = wgt * x[e];
  }
  for (int s = 0; s < L; ++s) {
    const int32_t pos = irow[s];
    const float wgt = expf(a.lse_off[pos] - lse);
    load8<T>(a.part_off + static_cast<int64_t>(pos) * D + 8 * sub, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(wgt, x[e], acc[e]);
  }
  store8<T>(a.out + (t * a.H + h) * D + 8 * sub, acc);
  if (sub == 0) a.lse[dr] = lse;
}

template <typename T, int D>
hipError_t launch_merge_t(const Problem& p, const Workspace& ws, void* out, float* lse, hipStream_t stream) {
  MergeArgs<T> a;
  a.part_diag = static_cast<const T*>(ws.part_diag);
  a.lse_diag = ws.lse_diag;
  a.part_off = static_cast<const T*>(ws.part_off);
  a.lse_off = ws.lse_off;
  a.inv = ws.inv;
  a.out = static_cast<T*>(out);
  a.lse = lse;
  a.N = p.N;
  a.H = p.H;
  a.B = p.B;
  a.topk = p.topk;
  a.lmax = p.lmax;
  a.blo = p.blo;
  const int64_t threads = p.N * p.H * (D / 8);
  merge_kernel<T, D><<<static_cast<unsigned>((threads + 255) / 256), 256, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const Problem& p, const Workspace& ws, void* out, float* lse, hipStream_t stream) {
  if (p.is_f32)
    return p.D == 128 ? launch_merge_t<float, 128>(p, ws, out, lse, stream)
                      : launch_merge_t<float, 64>(p, ws, out, lse, stream);
  return p.D == 128 ? launch_merge_t<bf16, 128>(p, ws, out, lse, stream)
                    : launch_merge_t<bf16, 64>(p, ws, out, lse, stream);
}

}  // namespace moba
