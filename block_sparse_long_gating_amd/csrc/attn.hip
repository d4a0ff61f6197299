// Block attention: every work item is one key block of one head and up to
// kQTile queries attending it (智东西 report, section 二, implementation step 3:
// attention per KV block over the queries routed to it). Two kinds of items:
//   * past-block items: queries gathered from the block's query list; no mask;
//   * own-block items: a run of consecutive queries of the block itself, with
//     the causal mask inside the block (keys up to the query's own position).
// Each item writes, per query, the softmax-normalised partial output over its
// keys and the partial log-sum-exp; the merge kernel combines them.
//
// bf16 kernel (gfx950): 4 waves x 32 queries per workgroup, 64-key tiles of K
// and V staged in LDS with double buffering. Per wave and tile:
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16, keys on the rows, queries on the
//                  columns, Q held in registers as the B operand)
//   online softmax in the exp2 domain, per query column in registers
//   O^T += V^T P^T (P stays in registers as the B operand; V is staged
//                  transposed, in the key order the S accumulator layout gives)
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
  int qt_per_block;     // own-block items per block: ceil(B / kQTile)
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
  if (threadIdx.x == 0) *s_it = atomicAdd(cursor + xcd, 1);
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
  out->q0 = qt * kQTile;
  out->count = min(kQTile, B - out->q0);
  out->causal = true;
  out->list_start = 0;
  return true;
}

// ------------------------------------------------------------------------------------------
// bf16 MFMA kernel
// ------------------------------------------------------------------------------------------

template <int D>
struct Bf16Tile {
  static constexpr int kKStride = D + 8;        // K rows [key][d], padded
  static constexpr int kVStride = kKTile + 8;   // V^T rows [d][key position], padded
  static constexpr int kKElems = kKTile * kKStride;
  static constexpr int kVElems = D * kVStride;
  static constexpr int kKChunks = kKTile * D / 8 / 256;   // 16-byte K chunks per thread
  static constexpr int kVUnits = (kKTile / 4) * (D / 8);  // 4-key x 8-dim V units
};

// Position of key `kk` (0..63) of a tile inside a V^T row: within every group of
// 16 keys, bits 2 and 3 of the key index are swapped. That is the key order in
// which a lane's S accumulator registers reach the PV MFMA as its B operand.
__device__ __forceinline__ int vt_pos(int kk) {
  return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

template <int D>
__device__ __forceinline__ void load_tile_bf16(const bf16* __restrict__ kbase, const bf16* __restrict__ vbase,
                                               int64_t row_stride, uint4 (&kr)[Bf16Tile<D>::kKChunks],
                                               uint4 (&vr)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < Bf16Tile<D>::kKChunks; ++u) {
    const int ci = tid + 256 * u;
    const int row = ci / (D / 8);
    const int c8 = ci % (D / 8);
    kr[u] = load_u4(kbase + row * row_stride + 8 * c8);
  }
  if (tid < Bf16Tile<D>::kVUnits) {
    const int kg = tid % 16;
    const int dc = tid / 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = load_u4(vbase + (4 * kg + i) * row_stride + 8 * dc);
  }
}

template <int D>
__device__ __forceinline__ void store_tile_bf16(bf16* sk, bf16* svt, const uint4 (&kr)[Bf16Tile<D>::kKChunks],
                                                const uint4 (&vr)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < Bf16Tile<D>::kKChunks; ++u) {
    const int ci = tid + 256 * u;
    const int row = ci / (D / 8);
    const int c8 = ci % (D / 8);
    *reinterpret_cast<uint4*>(sk + row * Bf16Tile<D>::kKStride + 8 * c8) = kr[u];
  }
  if (tid < Bf16Tile<D>::kVUnits) {
    const int kg = tid % 16;
    const int dc = tid / 16;
    const int pos = vt_pos(4 * kg);
    const uint32_t w[4][4] = {{vr[0].x, vr[0].y, vr[0].z, vr[0].w},
                              {vr[1].x, vr[1].y, vr[1].z, vr[1].w},
                              {vr[2].x, vr[2].y, vr[2].z, vr[2].w},
                              {vr[3].x, vr[3].y, vr[3].z, vr[3].w}};
#pragma unroll
    for (int cp = 0; cp < 4; ++cp) {
      // dims 8*dc + 2*cp (low halves) and 8*dc + 2*cp + 1 (high halves) of the 4 keys
      uint2 even, odd;
      even.x = (w[0][cp] & 0xFFFFu) | (w[1][cp] << 16);
      even.y = (w[2][cp] & 0xFFFFu) | (w[3][cp] << 16);
      odd.x = (w[0][cp] >> 16) | (w[1][cp] & 0xFFFF0000u);
      odd.y = (w[2][cp] >> 16) | (w[3][cp] & 0xFFFF0000u);
      *reinterpret_cast<uint2*>(svt + (8 * dc + 2 * cp) * Bf16Tile<D>::kVStride + pos) = even;
      *reinterpret_cast<uint2*>(svt + (8 * dc + 2 * cp + 1) * Bf16Tile<D>::kVStride + pos) = odd;
    }
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs<bf16> a) {
  using Tl = Bf16Tile<D>;
  __shared__ bf16 sk[2][Tl::kKElems];
  __shared__ bf16 svt[2][Tl::kVElems];
  __shared__ int s_it;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int qn = lane & 31;
  const int half = lane >> 5;
  const int64_t row_stride = static_cast<int64_t>(a.H) * D;

  Item item;
  while (next_item(a.counters, a.counters + 8, a.diag_items, a.items, a.n, a.qt_per_block, a.B, &s_it, &item)) {
    const int h = item.h;
    const int qi = 32 * w + qn;                 // query slot inside the item
    const bool lvalid = qi < item.count;
    const int qs = lvalid ? qi : item.count - 1;
    int64_t qrow;                               // token index of this lane's query
    if (item.causal)
      qrow = static_cast<int64_t>(item.b) * a.B + item.q0 + qs;
    else
      qrow = a.qidx[item.list_start + qs];
    const int qpos = item.q0 + qi;              // position inside the block (own-block items)
    const int wave_last = item.q0 + 32 * w + 31;
    const bool wave_has = 32 * w < item.count;

    bf16x8 qop[D / 16];
    {
      const bf16* qp = a.q + (qrow * a.H + h) * D + 8 * half;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) qop[c] = load_bf16x8(qp + 16 * c);
    }

    f32x16 o[D / 32];
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[c][r] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;

    const int nkt = item.causal ? (item.q0 + item.count + kKTile - 1) / kKTile : a.B / kKTile;
    const bf16* kblk = a.k + (static_cast<int64_t>(item.b) * a.B * a.H + h) * D;
    const bf16* vblk = a.v + (static_cast<int64_t>(item.b) * a.B * a.H + h) * D;

    uint4 kr[Tl::kKChunks];
    uint4 vr[4];
    load_tile_bf16<D>(kblk, vblk, row_stride, kr, vr);
    store_tile_bf16<D>(sk[0], svt[0], kr, vr);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nkt) {
        const int64_t adv = static_cast<int64_t>(kt + 1) * kKTile * row_stride;
        load_tile_bf16<D>(kblk + adv, vblk + adv, row_stride, kr, vr);
      }
      const bool active = wave_has && (!item.causal || kt * kKTile <= wave_last);
      if (active) {
        const bf16* kl = sk[buf] + qn * Tl::kKStride + 8 * half;
        f32x16 s0, s1;
#pragma unroll
        for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_bf16x8(kl + 16 * c), qop[c], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_bf16x8(kl + 32 * Tl::kKStride + 16 * c), qop[c], s1,
                                                       0, 0, 0);
        }
        // scale into the exp2 domain, causal mask, tile maximum
        const bool need_mask = item.causal && (kt * kKTile + kKTile - 1 > item.q0 + 32 * w);
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x0 = s0[r] * a.scale_log2;
          float x1 = s1[r] * a.scale_log2;
          if (need_mask) {
            const int kk = kt * kKTile + 8 * (r >> 2) + 4 * half + (r & 3);
            if (kk > qpos) x0 = -INFINITY;
            if (kk + 32 > qpos) x1 = -INFINITY;
          }
          s0[r] = x0;
          s1[r] = x1;
          mx = fmaxf(mx, fmaxf(x0, x1));
        }
        mx = wave_max_pair(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        bf16x8 p[4];
        float lsum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e0 = __builtin_amdgcn_exp2f(s0[r] - m_new);
          const float e1 = __builtin_amdgcn_exp2f(s1[r] - m_new);
          lsum += e0 + e1;
          p[r >> 3][r & 7] = static_cast<bf16>(e0);
          p[2 + (r >> 3)][r & 7] = static_cast<bf16>(e1);
        }
        l_run = l_run * alpha + lsum;
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[c][r] *= alpha;
        // O^T += V^T P^T over the 4 groups of 16 keys
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
          const bf16* vl = svt[buf] + (32 * c + qn) * Tl::kVStride + 8 * half;
#pragma unroll
          for (int g = 0; g < 4; ++g)
            o[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(load_bf16x8(vl + 16 * g), p[g], o[c], 0, 0, 0);
        }
      }
      if (kt + 1 < nkt) store_tile_bf16<D>(sk[buf ^ 1], svt[buf ^ 1], kr, vr);
      __syncthreads();
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (lvalid) {
      const int64_t orow = item.causal ? static_cast<int64_t>(h) * a.N + qrow : item.list_start + qi;
      bf16* po = (item.causal ? a.part_diag : a.part_off) + orow * D;
      const float inv_l = 1.f / l_tot;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x4 vv;
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[e] = static_cast<bf16>(o[c][4 * i + e] * inv_l);
          *reinterpret_cast<uint2*>(po + 32 * c + 8 * i + 4 * half) = __builtin_bit_cast(uint2, vv);
        }
      }
      if (half == 0) {
        float* pl = item.causal ? a.lse_diag : a.lse_off;
        pl[orow] = (m_run + log2f(l_tot)) * kLn2;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// fp32 kernel
// ------------------------------------------------------------------------------------------

constexpr int kF32Keys = 32;

template <int D>
__global__ __launch_bounds__(128) void attn_f32_kernel(AttnArgs<float> a) {
  __shared__ float sk[kF32Keys][D];
  __shared__ float sv[kF32Keys][D];
  __shared__ int s_it;
  const int tid = threadIdx.x;
  const int64_t row_stride = static_cast<int64_t>(a.H) * D;

  Item item;
  while (next_item(a.counters, a.counters + 8, a.diag_items, a.items, a.n, a.qt_per_block, a.B, &s_it, &item)) {
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
      for (int i = tid; i < kF32Keys * D / 4; i += 128) {
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
  a.qt_per_block = (p.B + kQTile - 1) / kQTile;
  a.diag_items = p.diag_items;
  a.scale_log2 = kLog2e / sqrtf(static_cast<float>(p.D));
  return a;
}

}  // namespace

hipError_t launch_attention(const Problem& p, const void* q, const void* k, const void* v, const Workspace& ws,
                            int num_cus, hipStream_t stream) {
  const int64_t total = p.max_items + p.diag_items;
  if (p.is_f32) {
    auto a = make_args<float>(p, q, k, v, ws);
    int64_t grid = static_cast<int64_t>(num_cus) * 4;
    grid = std::min<int64_t>(grid, ((total + kXcds - 1) / kXcds) * kXcds);
    if (p.D == 128)
      attn_f32_kernel<128><<<static_cast<unsigned>(grid), 128, 0, stream>>>(a);
    else
      attn_f32_kernel<64><<<static_cast<unsigned>(grid), 128, 0, stream>>>(a);
  } else {
    auto a = make_args<bf16>(p, q, k, v, ws);
    int64_t grid = static_cast<int64_t>(num_cus) * 2;
    grid = std::min<int64_t>(grid, ((total + kXcds - 1) / kXcds) * kXcds);
    if (p.D == 128)
      attn_bf16_kernel<128><<<static_cast<unsigned>(grid), 256, 0, stream>>>(a);
    else
      attn_bf16_kernel<64><<<static_cast<unsigned>(grid), 256, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moba
