// Backward pass of the MoBA causal prefill (bf16): dQ, dK, dV of the output.
//
// The pages train and continually pretrain with MoBA (智东西 report, section
// 三); the gate is a top-k choice with no gradient, so the selection of the
// forward pass is recomputed and held fixed, and the gradients are those of
// the block-sparse softmax attention (P the probabilities over the attended
// keys, dO the upstream gradient):
//   dV = Pᵀ dO,  dP = dO Vᵀ,  dS = P ⊙ (dP − Δ) with Δ_t = Σ_d dO_t O_t,
//   dQ = dS K / √D,  dK = dSᵀ Q / √D.
// P is rebuilt from the scores and the forward's log-sum-exp.
//
// Kernels (v_mfma_f32_32x32x16_bf16 for every product; C layout: lane l holds
// column l % 32 and rows 8 (r / 4) + 4 (l / 32) + r % 4 of accumulator
// element r; the 16-row groups that feed a second product are taken in that
// same row order, through the LDS transpose read where the operand is
// row-major in LDS):
//   bwd_delta_kernel   Δ per (head, query): D/8 lanes per row.
//   bwd_dkdv_kernel    key-stationary: one workgroup per (head, key block,
//                      128-key chunk) walks every query that attends the
//                      chunk: the block's query list (past selections) and
//                      the block's own later queries (causal mask), in
//                      64-query tiles staged in LDS (double-buffered through
//                      registers, list entries looked up a tile ahead). Eight
//                      waves in two kinds, one of each per SIMD, working on
//                      consecutive tiles at the same time: waves 0-3 hold K
//                      and V of key group w (32 keys) in registers and turn
//                      tile i into
//                        S = Q Kᵀ, dP = dO Vᵀ (queries on the rows), P, dS,
//                      which go to a double-buffered LDS exchange as bf16;
//                      waves 4-7 add tile i - 1 into all D dims of key group
//                      w - 4:
//                        dVᵀ += dOᵀ P, dKᵀ += Qᵀ dS (dOᵀ, Qᵀ by transpose reads).
//                      Each key is owned by one workgroup: no atomics.
//   bwd_dq_kernel      query-stationary over the same work items as the
//                      forward pass (a block and up to 256 of its queries;
//                      eight waves of 32 queries with Q and dO in registers),
//                      walking the block's 64-key tiles in LDS:
//                        Sᵀ = K Qᵀ, dPᵀ = V dOᵀ (keys on the rows),
//                        dQᵀ += Kᵀ dSᵀ (Kᵀ by transpose reads).
//                      Past-block items write fp32 partial rows in list
//                      order; the own-block items run afterwards, add the
//                      query's past partials (list positions from the scatter)
//                      and write dQ.
#include "common.h"
#include "kernels.h"

namespace moba {

namespace {

typedef short s16x4b __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4b lds_s16x4b;

constexpr float kBwdLog2e = 1.4426950408889634f;
constexpr int kBwdQTile = 64;      // queries per LDS tile of the dK/dV kernel
constexpr int kBwdKeys = 128;      // keys per dK/dV workgroup (4 waves x 32)
constexpr int kBwdKTile = 64;      // keys per LDS tile of the dQ kernel

template <int D>
struct BwdLay {
  // Padded LDS row (bytes): rows are read both as 16-byte row pieces and by the
  // transpose read; this padding keeps both free of bank conflicts (measured:
  // 10% faster backward than 2D + 16).
  static constexpr int kRow = 2 * D + (D == 128 ? 48 : 32);
  static constexpr int kTile = 64 * kRow;          // one 64-row tile
  static constexpr int kChunks = D / 8;            // 16-byte chunks per row
};

// MFMA over D: rows from a row-major LDS tile (A operand, per-lane pointer to
// row l % 32 at byte 16 (l / 32)), columns from registers (B operand).
// All D / 16 row pieces are read before the products, so the reads overlap one
// another instead of each product waiting for its own.
template <int D>
__device__ __forceinline__ f32x16 rows_by_regs(const char* ap, const bf16x8 (&b)[D / 16]) {
  f32x16 s;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
  bf16x8 av[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) av[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ap + 32 * c));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < D / 16; ++c) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[c], b[c], s, 0, 0, 0);
  return s;
}

// A operand "columns of a row-major LDS tile as rows": for a 16-row group
// starting at `p` (already offset by the lane's transpose-read position) and
// 32 columns starting at column 32 dc, the 8 rows the C layout pairs with this
// lane (4 (l / 32) + 0..3, then 8 + 4 (l / 32) + 0..3).
template <int kRow>
__device__ __forceinline__ bf16x8 tr_operand(const char* p) {
  const s16x4b lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4b*)(p));
  const s16x4b hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4b*)(p + 8 * kRow));
  const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo);
  const bf16x4 h4 = __builtin_bit_cast(bf16x4, hi);
  return bf16x8{l4[0], l4[1], l4[2], l4[3], h4[0], h4[1], h4[2], h4[3]};
}

__device__ __forceinline__ void pack16(const f32x16& x, bf16x8 (&p)[2]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) p[r >> 3][r & 7] = static_cast<bf16>(x[r]);
}

__device__ __forceinline__ uint4 ld16(const bf16* p) { return *reinterpret_cast<const uint4*>(p); }

// Scalar load of work item idx (wave-uniform), waited for in the same
// statement. The list was written by an earlier kernel and is read-only here;
// inside a loop that also stores, the compiler would use a vector load, and
// waiting for that would wait for every vector load and store in flight.
__device__ __forceinline__ WorkItem load_item(const WorkItem* items, int idx) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const uint64_t p = reinterpret_cast<uint64_t>(items + __builtin_amdgcn_readfirstlane(idx));
  // readfirstlane works on 32-bit ints; each half goes through uint32_t so that
  // widening never sign-extends.
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p))));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(p >> 32))));
  const uint64_t addr = (static_cast<uint64_t>(hi) << 32) | lo;
  i32x4 v;
  asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(addr));
  WorkItem it;
  it.h = v.x;
  it.b = v.y;
  it.start = v.z;
  it.count = v.w;
  return it;
}

__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  const int kl = a.D / 8;                          // lanes per row
  const int rows = 256 / kl;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * rows + threadIdx.x / kl;   // g = t * H + h
  const int li = threadIdx.x % kl;
  float s = 0.f;
  if (g < a.N * a.H) {
    const bf16x8 o8 = __builtin_bit_cast(bf16x8, ld16(a.out + g * a.D + 8 * li));
    const bf16x8 d8 = __builtin_bit_cast(bf16x8, ld16(a.dout + g * a.D + 8 * li));
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(static_cast<float>(o8[e]), static_cast<float>(d8[e]), s);
  }
  for (int w = 1; w < kl; w <<= 1) s += __shfl_xor(s, w);
  if (g < a.N * a.H && li == 0) {
    const int64_t t = g / a.H;
    const int h = static_cast<int>(g % a.H);
    a.delta[static_cast<int64_t>(h) * a.N + t] = s;
  }
}

// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------

// Eight waves over 128 keys in a two-stage pipeline over the 64-query tiles:
// wave w < 4 computes S, dP, P and dS of tile i for key group w (32 keys, K
// and V in registers) and hands P and dS over through LDS; wave w + 4, on the
// same SIMD, meanwhile accumulates dKᵀ and dVᵀ of key group w over tile i - 1.
template <int D>
__global__ __launch_bounds__(512) void bwd_dkdv_kernel(BwdArgs a) {
  using L = BwdLay<D>;
  constexpr int kXRow = 2 * kBwdQTile + 8;         // P / dS exchange row (one key, 64 queries, bf16; 34 dwords: conflict-free)
  constexpr int kX = 32 * kXRow;                   // one key group
  __shared__ __align__(16) char tiles[2][2 * L::kTile];   // [buffer][Q tile, dO tile]
  __shared__ __align__(16) char xch[2][2][4 * kX];         // [buffer][P, dS][key group]
  __shared__ __align__(16) float s_lse[2][kBwdQTile];
  __shared__ __align__(16) float s_del[2][kBwdQTile];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int kg = w & 3;                            // key group
  const int chunks = (a.B + kBwdKeys - 1) / kBwdKeys;
  // XCD-aware order: the chunks of one (head, block) run on one XCD at the same
  // time (they read the same query rows), consecutive (head, block) pairs go
  // round-robin over the XCDs, and blocks are taken in ascending order (their
  // query lists get shorter).
  const int G = static_cast<int>(gridDim.x);
  int li = static_cast<int>(blockIdx.x);
  if (G % (kXcds * chunks) == 0) {
    const int xcd = li % kXcds, slot = li / kXcds;
    li = ((slot / chunks) * kXcds + xcd) * chunks + slot % chunks;
  }
  const int c = li % chunks;
  const int rest = li / chunks;
  const int h = rest % a.H, b = rest / a.H;
  const int kofs = kBwdKeys * c + 32 * kg;         // this wave's first key inside the block
  const bool active = kofs < a.B;
  const int64_t key0 = static_cast<int64_t>(b) * a.B + kofs;
  const int64_t hb = static_cast<int64_t>(h) * a.n + b;
  const int lstart = a.has_lists ? a.offs[hb] : 0, llen = a.has_lists ? a.totals[hb] : 0;
  const int own0 = kBwdKeys * c;                   // first own query (offset in the block) that sees the chunk
  const int t_past = (llen + kBwdQTile - 1) / kBwdQTile;
  const int t_all = t_past + (a.B - own0 + kBwdQTile - 1) / kBwdQTile;
  const int64_t hd = static_cast<int64_t>(h) * D;
  const int64_t row_el = static_cast<int64_t>(a.H) * D;


  // Tile rows: the token of row r of tile i (-1: no query). Tokens stay 32-bit
  // (N < 2^31): a widened list entry would make the compiler wait for the
  // entry, and with it for every older load of the tile, right after the lookup.
  auto token = [&](int i, int r) -> int {
    if (i >= t_all) return -1;
    if (i < t_past) {
      const int e = kBwdQTile * i + r;
      return e < llen ? a.qidx[lstart + e] : -1;
    }
    const int o = own0 + kBwdQTile * (i - t_past) + r;
    return o < a.B ? b * a.B + o : -1;
  };
  // Loader: 64 rows x kChunks 16-byte chunks of Q and dO; the rows' tokens are
  // looked up one tile ahead of the row loads.
  constexpr int kPer = kBwdQTile * L::kChunks / 512;
  uint4 pq[kPer], pd[kPer];
  int tok[kPer];
  int tok_l = -1;
  float plse = INFINITY, pdel = 0.f;
  auto lookup = [&](int i) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) tok[u] = token(i, (tid + 512 * u) / L::kChunks);
    if (tid < kBwdQTile) tok_l = token(i, tid);
  };
  auto fetch = [&]() {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int ch = (tid + 512 * u) % L::kChunks;
      const bool ok = tok[u] >= 0;
      const int64_t off = static_cast<int64_t>(ok ? tok[u] : 0) * row_el + hd + 8 * ch;
      pq[u] = ok ? ld16(a.q + off) : make_uint4(0, 0, 0, 0);
      pd[u] = ok ? ld16(a.dout + off) : make_uint4(0, 0, 0, 0);
    }
    if (tid < kBwdQTile) {
      const bool ok = tok_l >= 0;
      plse = ok ? a.lse[static_cast<int64_t>(h) * a.N + tok_l] : INFINITY;   // scaled at the commit
      pdel = ok ? a.delta[static_cast<int64_t>(h) * a.N + tok_l] : 0.f;
    }
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int idx = tid + 512 * u;
      const int r = idx / L::kChunks, ch = idx % L::kChunks;
      *reinterpret_cast<uint4*>(&tiles[buf][r * L::kRow + 16 * ch]) = pq[u];
      *reinterpret_cast<uint4*>(&tiles[buf][L::kTile + r * L::kRow + 16 * ch]) = pd[u];
    }
    if (tid < kBwdQTile) {
      s_lse[buf][tid] = plse * kBwdLog2e;
      s_del[buf][tid] = pdel;
    }
  };

  const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
  const int row_lane = col * L::kRow + 16 * half;
  const int tr_lane = (4 * (tg >> 1) + te) * L::kRow + 2 * (16 * (tg & 1) + 4 * tq);
  const int xrow = kg * kX + col * kXRow;          // this lane's key row in a P or dS exchange area
  // Own tiles: block offset of tile i's first query.
  auto tile_q0 = [&](int i) { return own0 + kBwdQTile * (i - t_past); };
  lookup(0);
  fetch();
  commit(0);
  lookup(1);
  __syncthreads();
  // Pipeline step st (0 .. t_all): the rows of tile st + 1 are loaded into
  // registers, waves 0-3 turn tile st into P and dS while waves 4-7 add tile
  // st - 1 into dV and dK (so every SIMD holds one wave of each kind), then,
  // after a barrier, tile st + 1 goes into the buffer that tile st - 1 held,
  // and a second barrier publishes it. Both kinds of wave pass the same
  // barriers: 2 (t_all + 1) each.
  auto step_begin = [&](int st) {
    if (st + 1 < t_all) {
      fetch();          // rows of tile st + 1 (tokens looked up one step earlier)
      lookup(st + 2);
    }
  };
  auto step_end = [&](int st) {
    __syncthreads();
    if (st + 1 < t_all) commit((st + 1) & 1);
    __syncthreads();
  };
  if (w < 4) {
    // K and V of the key group in registers; per tile, S = Q Kᵀ and dP = dO Vᵀ
    // (queries on the rows) for each 32-query half, then P and dS as bf16 into
    // the tile's exchange buffer.
    bf16x8 kr[D / 16], vr[D / 16];
    {
      const int64_t kk = active ? key0 + col : 0;
#pragma unroll
      for (int cc = 0; cc < D / 16; ++cc) {
        kr[cc] = __builtin_bit_cast(bf16x8, ld16(a.k + kk * row_el + hd + 16 * cc + 8 * half));
        vr[cc] = __builtin_bit_cast(bf16x8, ld16(a.v + kk * row_el + hd + 16 * cc + 8 * half));
      }
    }
    for (int st = 0; st <= t_all; ++st) {
      step_begin(st);
      const int buf = st & 1;
      const bool own = st >= t_past;
      const int q0 = tile_q0(st);
      // Nothing to do past the last tile, and nothing to write when every key
      // of the group comes after every query of the tile (the consumer skips it).
      if (active && st < t_all && !(own && kofs > q0 + kBwdQTile - 1)) {
        const char* qt = tiles[buf];
        const char* dt = tiles[buf] + L::kTile;
        char* xp = xch[buf][0] + xrow;
        char* xs = xch[buf][1] + xrow;
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          if (own && kofs > q0 + 32 * qh + 31) {
            // Every key of the group comes after every query of the half: P = dS = 0.
            const bf16x4 z4 = {static_cast<bf16>(0.f), static_cast<bf16>(0.f), static_cast<bf16>(0.f),
                               static_cast<bf16>(0.f)};
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int rq = qh * 32 + 8 * g4 + 4 * half;
              *reinterpret_cast<bf16x4*>(xp + 2 * rq) = z4;
              *reinterpret_cast<bf16x4*>(xs + 2 * rq) = z4;
            }
            continue;
          }
          const f32x16 sc = rows_by_regs<D>(qt + qh * 32 * L::kRow + row_lane, kr);
          const f32x16 dp = rows_by_regs<D>(dt + qh * 32 * L::kRow + row_lane, vr);
          auto softmax = [&](auto masked) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int rq = qh * 32 + 8 * g4 + 4 * half;
              const float4 l4 = *reinterpret_cast<const float4*>(&s_lse[buf][rq]);
              const float4 d4 = *reinterpret_cast<const float4*>(&s_del[buf][rq]);
              const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
              const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
              bf16x4 p4, ds4;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                float pr = __builtin_amdgcn_exp2f(fmaf(sc[r], a.scale_log2, -lv[e]));
                if constexpr (decltype(masked)::value)
                  if (kofs + col > q0 + rq + e) pr = 0.f;   // key after the query
                p4[e] = static_cast<bf16>(pr);
                ds4[e] = static_cast<bf16>(pr * (dp[r] - dv[e]));
              }
              *reinterpret_cast<bf16x4*>(xp + 2 * rq) = p4;
              *reinterpret_cast<bf16x4*>(xs + 2 * rq) = ds4;
            }
          };
          // Only own tiles whose (key group, query half) square crosses the
          // diagonal hold keys after a query; the rest skip the mask (uniform branch).
          if (own && kofs + 31 > q0 + 32 * qh) softmax(std::true_type{});
          else softmax(std::false_type{});
        }
      }
      step_end(st);
    }
    return;
  }
  // Waves 4-7: dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS over all D dims of the key group,
  // for tile st - 1 (dOᵀ, Qᵀ by transpose reads; P, dS from the exchange).
  f32x16 adv[D / 32], adk[D / 32];
#pragma unroll
  for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
    for (int r = 0; r < 16; ++r) adv[dc][r] = adk[dc][r] = 0.f;
  for (int st = 0; st <= t_all; ++st) {
    step_begin(st);
    const int i = st - 1;
    if (active && i >= 0 && !(i >= t_past && kofs > tile_q0(i) + kBwdQTile - 1)) {   // (all P = 0 otherwise)
      const int buf = i & 1;
      const char* qt = tiles[buf];
      const char* dt = tiles[buf] + L::kTile;
      const char* xp = xch[buf][0] + xrow;
      const char* xs = xch[buf][1] + xrow;
      // Operands of one 16-query group; the next group's are read before the
      // current group's products are issued.
      struct Ops {
        bf16x8 dot[D / 32], qtr[D / 32], pp, dsp;
      };
      auto read_ops = [&](int g, Ops& o) {
        const int q16 = 16 * g + 4 * half;
        const bf16x4 pa = *reinterpret_cast<const bf16x4*>(xp + 2 * q16);
        const bf16x4 pb = *reinterpret_cast<const bf16x4*>(xp + 2 * (q16 + 8));
        const bf16x4 sa = *reinterpret_cast<const bf16x4*>(xs + 2 * q16);
        const bf16x4 sb = *reinterpret_cast<const bf16x4*>(xs + 2 * (q16 + 8));
        o.pp = bf16x8{pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
        o.dsp = bf16x8{sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
        const int roff = 16 * g * L::kRow + tr_lane;
#pragma unroll
        for (int dc = 0; dc < D / 32; ++dc) {
          o.dot[dc] = tr_operand<L::kRow>(dt + roff + 64 * dc);
          o.qtr[dc] = tr_operand<L::kRow>(qt + roff + 64 * dc);
        }
      };
      auto products = [&](const Ops& o) {
#pragma unroll
        for (int dc = 0; dc < D / 32; ++dc) {
          adv[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.dot[dc], o.pp, adv[dc], 0, 0, 0);
          adk[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.qtr[dc], o.dsp, adk[dc], 0, 0, 0);
        }
      };
      Ops o0, o1;
      read_ops(0, o0);
      read_ops(1, o1);
      products(o0);
      read_ops(2, o0);
      products(o1);
      read_ops(3, o1);
      products(o0);
      products(o1);
    }
    step_end(st);
  }
  if (!active) return;
  // dKᵀ / dVᵀ rows are dims 32 dc + 8 g4 + 4 half + 0..3 of this lane's key.
  const int64_t base = (key0 + col) * row_el + hd;
#pragma unroll
  for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * dc + 8 * g4 + 4 * half;
      bf16x4 kv4, vv4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv4[e] = static_cast<bf16>(adk[dc][4 * g4 + e] * a.scale);
        vv4[e] = static_cast<bf16>(adv[dc][4 * g4 + e]);
      }
      *reinterpret_cast<bf16x4*>(a.dk + base + d0) = kv4;
      *reinterpret_cast<bf16x4*>(a.dv + base + d0) = vv4;
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------

template <int D, bool kOwn>
__global__ __launch_bounds__(512) void bwd_dq_kernel(BwdArgs a) {
  using L = BwdLay<D>;
  __shared__ __align__(16) char tiles[2][2 * L::kTile];   // [buffer][K tile, V tile]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int pos = 32 * w + col;                    // this lane's query inside an item
  // Past items: persistent workgroups on a static, XCD-aware schedule (XCD x =
  // blockIdx % 8 takes a contiguous eighth of the item list and its
  // workgroups every (G/8)-th item of it), so the items of one key block run
  // on one XCD at the same time and share its K/V rows in that XCD's L2. The
  // list entries of a workgroup's next item are requested at the start of the
  // current one. Own items: one item per workgroup.
  int ii = 0, iend = 1, istep = 1;
  int tok_next = 0;
  if (!kOwn) {
    const int nitems = a.counters[0];
    const int G = static_cast<int>(gridDim.x);
    if (G % kXcds == 0) {
      const int x = static_cast<int>(blockIdx.x) % kXcds;
      ii = static_cast<int>(static_cast<int64_t>(nitems) * x / kXcds) + static_cast<int>(blockIdx.x) / kXcds;
      iend = static_cast<int>(static_cast<int64_t>(nitems) * (x + 1) / kXcds);
      istep = G / kXcds;
    } else {
      ii = static_cast<int>(blockIdx.x);
      iend = nitems;
      istep = G;
    }
    if (ii >= iend) return;
    const WorkItem it = load_item(a.items, ii);
    if (pos < it.count) tok_next = a.qidx[it.start + pos];
  }
  for (;;) {
    int h, b, count;
    int64_t t0 = 0;         // own items: first query
    int lstart = 0;         // past items: first list position
    if (kOwn) {
      // Within a block, later query tiles (more keys) are dispatched first.
      const int per = (a.B + kAttnTile - 1) / kAttnTile;
      const int x = per - 1 - static_cast<int>(blockIdx.x % per);
      const int rest = blockIdx.x / per;
      h = rest % a.H;
      b = rest / a.H;
      t0 = static_cast<int64_t>(b) * a.B + static_cast<int64_t>(x) * kAttnTile;
      count = min(kAttnTile, a.B - x * kAttnTile);
    } else {
      const WorkItem it = load_item(a.items, ii);
      h = it.h;
      b = it.b;
      lstart = it.start;
      count = it.count;
    }
    const int64_t hd = static_cast<int64_t>(h) * D;
    const int64_t row_el = static_cast<int64_t>(a.H) * D;
    const bool valid = pos < count;
    int64_t t = 0;
    if (valid) t = kOwn ? t0 + pos : tok_next;
    bf16x8 qr[D / 16], dr[D / 16];
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) {
      const int64_t off = t * row_el + hd + 16 * cc + 8 * half;
      qr[cc] = valid ? __builtin_bit_cast(bf16x8, ld16(a.q + off)) : bf16x8{};
      dr[cc] = valid ? __builtin_bit_cast(bf16x8, ld16(a.dout + off)) : bf16x8{};
    }
    float lse_raw = valid ? a.lse[static_cast<int64_t>(h) * a.N + t] : INFINITY;   // scaled below
    const float del = valid ? a.delta[static_cast<int64_t>(h) * a.N + t] : 0.f;
    if (!kOwn) {
      // The next item's list entries, after this item's row loads.
      tok_next = 0;
      if (ii + istep < iend) {
        const WorkItem it = load_item(a.items, ii + istep);
        if (pos < it.count) tok_next = a.qidx[it.start + pos];
      }
    }
    f32x16 acc[D / 32];
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dc][r] = 0.f;

    int inv0 = 0, inv1 = 0;   // own items: list positions of the first two past partials

    // Key tiles of block b; the own block stops at the item's last query.
    const int64_t kb0 = static_cast<int64_t>(b) * a.B;
    const int nkeys = kOwn ? static_cast<int>(t0 - kb0) + count : a.B;
    const int ntiles = (nkeys + kBwdKTile - 1) / kBwdKTile;
    constexpr int kPer = kBwdKTile * L::kChunks / 512;
    uint4 pk[kPer], pv[kPer];
    auto fetch = [&](int i) {
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int idx = tid + 512 * u;
        const int r = idx / L::kChunks, ch = idx % L::kChunks;
        const int64_t off = (kb0 + kBwdKTile * i + r) * row_el + hd + 8 * ch;   // always inside block b
        pk[u] = ld16(a.k + off);
        pv[u] = ld16(a.v + off);
      }
    };
    auto commit = [&](int buf) {
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int idx = tid + 512 * u;
        const int r = idx / L::kChunks, ch = idx % L::kChunks;
        *reinterpret_cast<uint4*>(&tiles[buf][r * L::kRow + 16 * ch]) = pk[u];
        *reinterpret_cast<uint4*>(&tiles[buf][L::kTile + r * L::kRow + 16 * ch]) = pv[u];
      }
    };
    const int tg = lane >> 4, te = (lane >> 2) & 3, tq = lane & 3;
    const int row_lane = col * L::kRow + 16 * half;
    const int tr_lane = (4 * (tg >> 1) + te) * L::kRow + 2 * (16 * (tg & 1) + 4 * tq);
    // This wave's last query (wave-uniform): key halves after it are all masked
    // (own items), and a wave without queries has nothing to add.
    const int64_t wlast = 32 * w < count ? (kOwn ? t0 + min(32 * w + 31, count - 1) : INT64_MAX) : -1;
    fetch(0);
    if (kOwn && valid) {
      // Requested after the first tile's loads (the block's sequence start may
      // have to arrive first) and used after the key loop.
      const int np = kept_past(b, a.blo != nullptr ? a.blo[b] : 0, a.topk);
      const int64_t ibase = (static_cast<int64_t>(h) * a.N + t) * a.lmax;
      if (np > 0) inv0 = a.inv[ibase];
      if (np > 1) inv1 = a.inv[ibase + 1];
    }
    commit(0);
    __syncthreads();
    // Scaled only here, where every load above has been waited for: a multiply
    // right after the load would hold the first tile's loads back until then
    // (the empty asm keeps the compiler from moving it there).
    asm volatile("" : "+v"(lse_raw));
    const float lse2 = lse_raw * kBwdLog2e;
    for (int i = 0; i < ntiles; ++i) {
      const int buf = i & 1;
      if (i + 1 < ntiles) fetch(i + 1);
      const char* kt = tiles[buf];
      const char* vt = tiles[buf] + L::kTile;
      // Past items test only whether the wave holds queries (once per tile),
      // which leaves both halves in one block for the scheduler; own items
      // also skip the halves that lie wholly after the wave's queries.
      if (kOwn || wlast >= 0) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int64_t kbase = kb0 + kBwdKTile * i + 32 * kh;
          if (kOwn && kbase > wlast) continue;
          const f32x16 s = rows_by_regs<D>(kt + kh * 32 * L::kRow + row_lane, qr);
          const f32x16 dp = rows_by_regs<D>(vt + kh * 32 * L::kRow + row_lane, dr);
          f32x16 ds;
          auto softmax = [&](auto masked) {
            const int rel = masked ? static_cast<int>(t - kbase) - 4 * half : 0;   // |t - kbase| < B
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float pr = __builtin_amdgcn_exp2f(fmaf(s[r], a.scale_log2, -lse2));
              if constexpr (decltype(masked)::value)
                if (8 * (r >> 2) + (r & 3) > rel) pr = 0.f;   // key after the query
              ds[r] = pr * (dp[r] - del);
            }
          };
          // Own items: only a key half that crosses the diagonal of the wave's
          // queries holds keys after a query (uniform branch).
          if (kOwn && kbase + 31 > t0 + 32 * w) softmax(std::true_type{});
          else softmax(std::false_type{});
          bf16x8 dsp[2];
          pack16(ds, dsp);
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int roff = (kh * 32 + 16 * g) * L::kRow + tr_lane;
#pragma unroll
            for (int dc = 0; dc < D / 32; ++dc) {
              const bf16x8 ktr = tr_operand<L::kRow>(kt + roff + 64 * dc);
              acc[dc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktr, dsp[g], acc[dc], 0, 0, 0);
            }
          }
        }
      }
      // Buffer buf ^ 1 was last read by tile i - 1, which every wave finished
      // before the previous barrier: one barrier per tile suffices.
      if (i + 1 < ntiles) commit(buf ^ 1);
      __syncthreads();
    }
    // dQᵀ rows are dims 32 dc + 8 g4 + 4 half + 0..3 of this lane's query.
    if (!kOwn) {
      if (valid) {
        float* dst = a.part_dq + static_cast<int64_t>(lstart + pos) * D;
#pragma unroll
        for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<float4*>(dst + 32 * dc + 8 * g4 + 4 * half) =
                make_float4(acc[dc][4 * g4], acc[dc][4 * g4 + 1], acc[dc][4 * g4 + 2], acc[dc][4 * g4 + 3]);
      }
      ii += istep;
      if (ii >= iend) return;
      continue;   // the loop's last barrier ended every wave's reads of the tiles
    }
    if (!valid) return;
    // Own block: add the query's past partials (two rows in flight at a time, in
    // list order), scale, write dQ.
    const int np = kept_past(b, a.blo != nullptr ? a.blo[b] : 0, a.topk);
    const int64_t ibase = (static_cast<int64_t>(h) * a.N + t) * a.lmax;
    for (int s2 = 0; s2 < np; s2 += 2) {
      const bool two = s2 + 1 < np;
      const int r0 = s2 == 0 ? inv0 : a.inv[ibase + s2];
      const int r1 = !two ? r0 : s2 == 0 ? inv1 : a.inv[ibase + s2 + 1];
      const float* src0 = a.part_dq + static_cast<int64_t>(r0) * D;
      const float* src1 = a.part_dq + static_cast<int64_t>(r1) * D;
      float4 x0[D / 8], x1[D / 8];
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const int d0 = 32 * (c >> 2) + 8 * (c & 3) + 4 * half;
        x0[c] = *reinterpret_cast<const float4*>(src0 + d0);
        x1[c] = *reinterpret_cast<const float4*>(src1 + d0);
      }
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        acc[c >> 2][4 * (c & 3)] += x0[c].x;
        acc[c >> 2][4 * (c & 3) + 1] += x0[c].y;
        acc[c >> 2][4 * (c & 3) + 2] += x0[c].z;
        acc[c >> 2][4 * (c & 3) + 3] += x0[c].w;
      }
      if (two) {
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
          acc[c >> 2][4 * (c & 3)] += x1[c].x;
          acc[c >> 2][4 * (c & 3) + 1] += x1[c].y;
          acc[c >> 2][4 * (c & 3) + 2] += x1[c].z;
          acc[c >> 2][4 * (c & 3) + 3] += x1[c].w;
        }
      }
    }
    bf16* dq = a.dq + t * row_el + hd;
#pragma unroll
    for (int dc = 0; dc < D / 32; ++dc)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = static_cast<bf16>(acc[dc][4 * g4 + e] * a.scale);
        *reinterpret_cast<bf16x4*>(dq + 32 * dc + 8 * g4 + 4 * half) = v4;
      }
    return;
  }
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = a.N * a.H;
  const int per = 256 / (a.D / 8);
  bwd_delta_kernel<<<static_cast<unsigned>((rows + per - 1) / per), 256, 0, stream>>>(a);
  const unsigned kv_grid = static_cast<unsigned>(static_cast<int64_t>(a.n) * a.H * ((a.B + kBwdKeys - 1) / kBwdKeys));
  const unsigned own_grid = static_cast<unsigned>(static_cast<int64_t>(a.n) * a.H * ((a.B + kAttnTile - 1) / kAttnTile));
  // dQ past items: one persistent workgroup per CU (one fits at a time).
  const unsigned past_grid = static_cast<unsigned>(a.num_cus > 0 ? std::min<int64_t>(a.max_items, a.num_cus) : a.max_items);
  if (a.D == 128) {
    bwd_dkdv_kernel<128><<<kv_grid, 512, 0, stream>>>(a);
    if (a.max_items > 0) bwd_dq_kernel<128, false><<<past_grid, 512, 0, stream>>>(a);
    bwd_dq_kernel<128, true><<<own_grid, 512, 0, stream>>>(a);
  } else {
    bwd_dkdv_kernel<64><<<kv_grid, 512, 0, stream>>>(a);
    if (a.max_items > 0) bwd_dq_kernel<64, false><<<past_grid, 512, 0, stream>>>(a);
    bwd_dq_kernel<64, true><<<own_grid, 512, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moba
