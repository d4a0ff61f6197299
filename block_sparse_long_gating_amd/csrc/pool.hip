// Block pooling of the keys: kbar[h][i][:] = the representative key of block i.
//
// Mean pooling gives each block the "representative" key the gate scores
// against (wzjinhao.cn MoBA article, section 3, score_pooling = mean; pomoai MoBA
// overview, "核心原理" step 2). The same article's closing section suggests
// max or weighted pooling instead: the per-dimension maximum over the block's
// keys, or the average of the block's keys under non-negative per-(head,
// token) weights (all-zero weights pool to zero). HBM-bound: every key is read
// exactly once.
//
// One workgroup per (block, group of up to 8 heads). Each thread owns 8
// consecutive dims of one head on a strided subset of the block's rows
// (16-byte loads, two batches of eight rows in flight; the group's heads of
// one token are one contiguous run), sums them in fp64 in a fixed order, and the per-row-group partial sums are
// combined in LDS in a fixed order, so the result is deterministic and,
// whenever the fp64 sum is exact, the correctly rounded mean.
// The bf16 path also writes the exact 3-way bf16 split (hi + mid + lo == fp32
// mean) that the MFMA gate consumes.
#include "common.h"
#include "kernels.h"

namespace moba {

namespace {

// Eight consecutive values of one row as loaded (one 16-byte load for bf16,
// two for fp32), widened to float on use. The keys are streamed: the loads
// are non-temporal, so they do not displace cache lines that later stages
// reuse (measured at h32: the pool 49.8 -> 43.9 us, the gate after it ~4 us
// faster).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Raw8;

template <>
struct Raw8<bf16> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16* p) {
    v = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
  }
  __device__ __forceinline__ void widen(float (&x)[8]) const {
    const bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(b[e]);
  }
};

template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)));
    b = __builtin_bit_cast(float4, __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4)));
  }
  __device__ __forceinline__ void widen(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

template <typename T, int D, int kMode>
__global__ __launch_bounds__(256) void pool_keys_kernel(const T* __restrict__ k, const float* __restrict__ weights,
                                                        float* __restrict__ kbar, bf16* __restrict__ pieces, int H,
                                                        int B, int n, int hg) {
  __shared__ double red[256][8];
  __shared__ double redw[kMode == kPoolWeighted ? 256 : 1];

  const int i = blockIdx.x;
  const int h0 = blockIdx.y * hg;             // this workgroup's heads h0 .. h0 + hg - 1
  const int chunks = hg * (D / 8);            // threads per token row (16-byte chunks of hg heads)
  const int rows_per_pass = 256 / chunks;
  const int c = threadIdx.x % chunks;
  const int r0 = threadIdx.x / chunks;
  const int64_t row_stride = static_cast<int64_t>(H) * D;
  // The hg heads of one token are contiguous: each row pass reads hg * 2D bytes in one run.
  const T* base = k + (static_cast<int64_t>(i) * B * H + h0) * D + c * 8;

  const int hc = h0 + c / (D / 8);            // this thread's head
  // Weights of this thread's head for the block's tokens (weighted mode).
  const float* wrow =
      kMode == kPoolWeighted ? weights + static_cast<int64_t>(hc) * n * B + static_cast<int64_t>(i) * B : nullptr;

  double acc[8];
  double wacc = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = kMode == kPoolMax ? -INFINITY : 0.0;
  auto add = [&](const float (&x)[8], int row) {
    if (kMode == kPoolMax) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmax(acc[e], static_cast<double>(x[e]));
    } else if (kMode == kPoolWeighted) {
      const double wt = static_cast<double>(wrow[row]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wt * static_cast<double>(x[e]);   // exact product
      wacc += wt;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += static_cast<double>(x[e]);
    }
  };

  // Rows in batches of eight, added in row order; the next batch's loads are
  // in flight while the current one is added (two batches of registers).
  const int rows = r0 < B ? (B - r0 + rows_per_pass - 1) / rows_per_pass : 0;   // this thread's rows
  const int batches = rows / 8;
  auto load_batch = [&](Raw8<T> (&buf)[8], int bt) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      buf[u].load(base + static_cast<int64_t>(r0 + (8 * bt + u) * rows_per_pass) * row_stride);
  };
  auto add_batch = [&](const Raw8<T> (&buf)[8], int bt) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float x[8];
      buf[u].widen(x);
      add(x, r0 + (8 * bt + u) * rows_per_pass);
    }
  };
  Raw8<T> b0[8], b1[8];
  if (batches > 0) load_batch(b0, 0);
  for (int bt = 0; bt < batches; bt += 2) {
    if (bt + 1 < batches) load_batch(b1, bt + 1);
    add_batch(b0, bt);
    if (bt + 1 < batches) {
      if (bt + 2 < batches) load_batch(b0, bt + 2);
      add_batch(b1, bt + 1);
    }
  }
  for (int rr = 8 * batches; rr < rows; ++rr) {
    Raw8<T> one;
    one.load(base + static_cast<int64_t>(r0 + rr * rows_per_pass) * row_stride);
    float x[8];
    one.widen(x);
    add(x, r0 + rr * rows_per_pass);
  }

#pragma unroll
  for (int e = 0; e < 8; ++e) red[threadIdx.x][e] = acc[e];
  if (kMode == kPoolWeighted) redw[threadIdx.x] = wacc;
  __syncthreads();

  if (threadIdx.x < chunks) {
    double s[8];
    double ws = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = kMode == kPoolMax ? -INFINITY : 0.0;
    for (int g = 0; g < rows_per_pass; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        s[e] = kMode == kPoolMax ? fmax(s[e], red[g * chunks + c][e]) : s[e] + red[g * chunks + c][e];
      if (kMode == kPoolWeighted) ws += redw[g * chunks + c];
    }
    const int h = hc;
    const int d0 = (c % (D / 8)) * 8;
    const int64_t o = (static_cast<int64_t>(h) * n + i) * D + d0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float m;
      if (kMode == kPoolMax) m = static_cast<float>(s[e]);
      else if (kMode == kPoolWeighted) m = ws > 0.0 ? static_cast<float>(s[e] / ws) : 0.f;
      else m = static_cast<float>(s[e] / static_cast<double>(B));
      kbar[o + e] = m;
      if (pieces != nullptr) {
        const bf16 hi = static_cast<bf16>(m);
        const float r1 = m - static_cast<float>(hi);
        const bf16 mid = static_cast<bf16>(r1);
        const float r2 = r1 - static_cast<float>(mid);
        const bf16 lo = static_cast<bf16>(r2);
        const int64_t po = ((static_cast<int64_t>(h) * n + i) * 3) * D + d0 + e;
        pieces[po] = hi;
        pieces[po + D] = mid;
        pieces[po + 2 * D] = lo;
      }
    }
  }
}

template <typename T, int D>
void launch_pool_mode(dim3 grid, const T* k, const float* weights, float* kbar, bf16* pieces, int H, int B, int n,
                      int hg, int mode, hipStream_t stream) {
  if (mode == kPoolMax)
    pool_keys_kernel<T, D, kPoolMax><<<grid, 256, 0, stream>>>(k, weights, kbar, pieces, H, B, n, hg);
  else if (mode == kPoolWeighted)
    pool_keys_kernel<T, D, kPoolWeighted><<<grid, 256, 0, stream>>>(k, weights, kbar, pieces, H, B, n, hg);
  else
    pool_keys_kernel<T, D, kPoolMean><<<grid, 256, 0, stream>>>(k, weights, kbar, pieces, H, B, n, hg);
}

}  // namespace

hipError_t launch_pool(const void* k, bool is_f32, float* kbar, bf16* pieces, int64_t N, int H, int D, int B,
                       hipStream_t stream, int mode, const float* weights) {
  const int n = static_cast<int>(N / B);
  // Heads per workgroup: the largest of 8, 4, 2, 1 that divides H (longer
  // contiguous runs per token row) while leaving at least 512 workgroups (two
  // per CU) to keep enough loads in flight, and with a row pass of at most 256
  // threads (measured at 32 heads: 512 workgroups of 4 heads beat 1024 of 2).
  int hg = 8;
  while (hg > 1 && (H % hg != 0 || hg * (D / 8) > 256 || static_cast<int64_t>(n) * (H / hg) < 512)) hg /= 2;
  dim3 grid(n, H / hg);
  if (is_f32) {
    const float* kf = static_cast<const float*>(k);
    if (D == 128) launch_pool_mode<float, 128>(grid, kf, weights, kbar, pieces, H, B, n, hg, mode, stream);
    else launch_pool_mode<float, 64>(grid, kf, weights, kbar, pieces, H, B, n, hg, mode, stream);
  } else {
    const bf16* kb = static_cast<const bf16*>(k);
    if (D == 128) launch_pool_mode<bf16, 128>(grid, kb, weights, kbar, pieces, H, B, n, hg, mode, stream);
    else launch_pool_mode<bf16, 64>(grid, kb, weights, kbar, pieces, H, B, n, hg, mode, stream);
  }
  return hipGetLastError();
}

}  // namespace moba
