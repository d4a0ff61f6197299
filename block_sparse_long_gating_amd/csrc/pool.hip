// Block mean-pool of the keys: kbar[h][i][:] = mean of the block_size keys of block i.
//
// Mean pooling gives each block the "representative" key the gate scores
// against (wzjinhao.cn MoBA article, section 3, score_pooling = mean; pomoai MoBA
// overview, "核心原理" step 2). HBM-bound: every key is read exactly once.
//
// One workgroup per (block, head). Each thread owns 8 consecutive head-dim
// lanes of a strided subset of the block's rows (16-byte loads, rows of one
// token are contiguous), sums them in fp64 in a fixed order, and the per-row
// group partial sums are combined in LDS in a fixed order, so the result is
// deterministic and, whenever the fp64 sum is exact, the correctly rounded mean.
// The bf16 path also writes the exact 3-way bf16 split (hi + mid + lo == fp32
// mean) that the MFMA gate consumes.
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

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_keys_kernel(const T* __restrict__ k, float* __restrict__ kbar,
                                                        bf16* __restrict__ pieces, int H, int B, int n) {
  constexpr int kChunks = D / 8;              // threads per token row
  constexpr int kRowsPerPass = 256 / kChunks; // token rows covered per pass
  __shared__ double red[256][8];

  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int c = threadIdx.x % kChunks;
  const int r0 = threadIdx.x / kChunks;
  const int64_t row_stride = static_cast<int64_t>(H) * D;
  const T* base = k + (static_cast<int64_t>(i) * B * H + h) * D + c * 8;

  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;

  int r = r0;
  for (; r + 3 * kRowsPerPass < B; r += 4 * kRowsPerPass) {
    float x0[8], x1[8], x2[8], x3[8];
    load8<T>(base + static_cast<int64_t>(r) * row_stride, x0);
    load8<T>(base + static_cast<int64_t>(r + kRowsPerPass) * row_stride, x1);
    load8<T>(base + static_cast<int64_t>(r + 2 * kRowsPerPass) * row_stride, x2);
    load8<T>(base + static_cast<int64_t>(r + 3 * kRowsPerPass) * row_stride, x3);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] += static_cast<double>(x0[e]);
      acc[e] += static_cast<double>(x1[e]);
      acc[e] += static_cast<double>(x2[e]);
      acc[e] += static_cast<double>(x3[e]);
    }
  }
  for (; r < B; r += kRowsPerPass) {
    float x0[8];
    load8<T>(base + static_cast<int64_t>(r) * row_stride, x0);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += static_cast<double>(x0[e]);
  }

#pragma unroll
  for (int e = 0; e < 8; ++e) red[threadIdx.x][e] = acc[e];
  __syncthreads();

  if (threadIdx.x < kChunks) {
    double s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.0;
    for (int g = 0; g < kRowsPerPass; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += red[g * kChunks + c][e];
    }
    const int64_t o = (static_cast<int64_t>(h) * n + i) * D + c * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float m = static_cast<float>(s[e] / static_cast<double>(B));
      kbar[o + e] = m;
      if (pieces != nullptr) {
        const bf16 hi = static_cast<bf16>(m);
        const float r1 = m - static_cast<float>(hi);
        const bf16 mid = static_cast<bf16>(r1);
        const float r2 = r1 - static_cast<float>(mid);
        const bf16 lo = static_cast<bf16>(r2);
        const int64_t po = ((static_cast<int64_t>(h) * n + i) * 3) * D + c * 8 + e;
        pieces[po] = hi;
        pieces[po + D] = mid;
        pieces[po + 2 * D] = lo;
      }
    }
  }
}

}  // namespace

hipError_t launch_pool(const void* k, bool is_f32, float* kbar, bf16* pieces, int64_t N, int H, int D, int B,
                       hipStream_t stream) {
  const int n = static_cast<int>(N / B);
  dim3 grid(n, H);
  if (is_f32) {
    if (D == 128)
      pool_keys_kernel<float, 128><<<grid, 256, 0, stream>>>(static_cast<const float*>(k), kbar, pieces, H, B, n);
    else
      pool_keys_kernel<float, 64><<<grid, 256, 0, stream>>>(static_cast<const float*>(k), kbar, pieces, H, B, n);
  } else {
    if (D == 128)
      pool_keys_kernel<bf16, 128><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(k), kbar, pieces, H, B, n);
    else
      pool_keys_kernel<bf16, 64><<<grid, 256, 0, stream>>>(static_cast<const bf16*>(k), kbar, pieces, H, B, n);
  }
  return hipGetLastError();
}

}  // namespace moba
