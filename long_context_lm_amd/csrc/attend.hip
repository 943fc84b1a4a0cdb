// Grouped cross-attention over retrieved chunks: forward and backward.
//
// [Notes, Key designs: GCA]: every token of the current chunk attends to each retrieved chunk
// separately, with its own softmax; the per-chunk outputs are fused with weights given by a
// softmax of the retrieval scores, so the scores receive gradients of the language-model loss
// [Notes, Background: entry point].  K/V are shared by all retrieval groups [Notes, Key
// designs: GCA].
//
// Tiles.  A chunk is 64 tokens, the head dim is 64, so one retrieved chunk of one head is a
// 64x64 K tile and a 64x64 V tile, and one (query chunk, head) is a 64x64 Q tile.  A workgroup
// of two waves owns one 64-query tile (forward and query-major backward) or one 64-key tile
// (key-major backward); each wave owns 32 rows and all 64 columns.  Each per-chunk softmax
// covers exactly one 64-key tile, so it is computed whole, without an online rescaling.
//
// Layout trick (see gca_device.hpp): S^T = K Q^T is computed with the K rows loaded through
// the permutation pi, which leaves each lane holding 16 consecutive keys of one query per
// 32-key tile; that register block is directly the B operand (P^T) of O^T = V^T P^T, so the
// probabilities never leave registers.  Operands that must be read down a column of a row-major
// tile (V in the forward, K in dQ, Q and dO in dK/dV) are staged transposed in LDS.
//
// Backward without floating-point atomics.  dQ and the per-slot sums of e = <dO, O_k> are
// produced query-major (one workgroup per query tile).  dK and dV are produced key-major: an
// inverse index lists, per (batch row, key chunk), the (group, row, slot) retrievals that
// selected it, in a fixed order, and one workgroup per (batch row, head, key chunk) walks that
// list and accumulates in registers.  d(score) sums the per-head partials in head order.
#include "gca_device.hpp"
#include "gca_internal.hpp"

namespace gca {
namespace {

constexpr int kThreads = 128;  // two waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2f = 0.6931471805599453f;

template <typename T>
struct TileCfg {
  static constexpr int kVec = 16 / static_cast<int>(sizeof(T));      // elements per 16 bytes
  static constexpr int kLd = kDim + kVec;                             // LDS row stride
  static constexpr int kChunksPerRow = kDim / kVec;
  static constexpr int kChunks = kChunk * kChunksPerRow;              // 16-byte pieces per tile
  static constexpr int kPerThread = kChunks / kThreads;
};

__device__ __forceinline__ uint16_t elem16(const u32x4_t& x, int e) {
  return static_cast<uint16_t>(x[e >> 1] >> ((e & 1) * 16));
}

// Copy a 64x64 tile (row stride 64 in global memory) to LDS, row-major and/or transposed.
template <typename T, bool kRow, bool kTrans>
__device__ __forceinline__ void stage_tile(const T* __restrict__ src, T* rowm, T* trans) {
  using C = TileCfg<T>;
  const int tid = threadIdx.x;
  u32x4_t x[C::kPerThread];
#pragma unroll
  for (int n = 0; n < C::kPerThread; ++n) {
    const int c = tid + n * kThreads;
    const int u = c / C::kChunksPerRow, col = (c % C::kChunksPerRow) * C::kVec;
    x[n] = *reinterpret_cast<const u32x4_t*>(src + u * kDim + col);
  }
#pragma unroll
  for (int n = 0; n < C::kPerThread; ++n) {
    const int c = tid + n * kThreads;
    const int u = c / C::kChunksPerRow, col = (c % C::kChunksPerRow) * C::kVec;
    if (kRow) *reinterpret_cast<u32x4_t*>(rowm + u * C::kLd + col) = x[n];
    if (kTrans) {
      if constexpr (sizeof(T) == 2) {
        uint16_t* t16 = reinterpret_cast<uint16_t*>(trans);
#pragma unroll
        for (int e = 0; e < 8; ++e) t16[(col + e) * C::kLd + u] = elem16(x[n], e);
      } else {
        float* t32 = reinterpret_cast<float*>(trans);
#pragma unroll
        for (int e = 0; e < 4; ++e) t32[(col + e) * C::kLd + u] = __uint_as_float(x[n][e]);
      }
    }
  }
}

// Slot table of one retrieval row: valid slots (0 <= j < n_kv) in slot order, with the fusion
// weights w = softmax over the valid slots of the clean scores.
struct SlotTable {
  int32_t j[kMaxTopk];
  int32_t slot[kMaxTopk];
  float w[kMaxTopk];
  int n;
};

__device__ void fusion_weights(const int32_t* idx_row, const float* score_row, int K, int64_t n_kv,
                               float* w_out, bool* valid_out) {
  float mx = -__builtin_inff();
  for (int k = 0; k < K; ++k) {
    const int32_t j = idx_row[k];
    const bool ok = j >= 0 && j < n_kv;
    valid_out[k] = ok;
    if (ok) mx = fmaxf(mx, score_row[k]);
  }
  float sum = 0.f;
  for (int k = 0; k < K; ++k) {
    const float e = valid_out[k] ? expf(score_row[k] - mx) : 0.f;
    w_out[k] = e;
    sum += e;
  }
  for (int k = 0; k < K; ++k) w_out[k] = valid_out[k] ? w_out[k] / sum : 0.f;
}

__device__ void build_slot_table(SlotTable& st, const AttendParams& p, int g, int b, int64_t row) {
  st.n = 0;
  if (row < 0) return;
  const int64_t base = ((static_cast<int64_t>(g) * p.B + b) * p.n_q + row) * p.K;
  float w[kMaxTopk];
  bool valid[kMaxTopk];
  fusion_weights(p.idx + base, p.score + base, p.K, p.n_kv, w, valid);
  for (int k = 0; k < p.K; ++k) {
    if (!valid[k]) continue;
    st.j[st.n] = p.idx[base + k];
    st.slot[st.n] = k;
    st.w[st.n] = w[k];
    ++st.n;
  }
}

struct QTileCoord {
  int b, h, g;
  int64_t t;
};

__device__ __forceinline__ QTileCoord query_tile_coord(const AttendParams& p) {
  const int64_t lid = xcd_logical_block(blockIdx.x, gridDim.x);
  QTileCoord c;
  c.t = lid % p.n_q;
  int64_t rest = lid / p.n_q;
  c.g = static_cast<int>(rest % p.G);
  rest /= p.G;
  c.h = static_cast<int>(rest % p.H);
  c.b = static_cast<int>(rest / p.H);
  return c;
}

// ------------------------------------------------------------------------------ forward
template <typename T>
__global__ __launch_bounds__(kThreads) void attend_fwd_kernel(AttendParams p) {
  using C = TileCfg<T>;
  __shared__ __align__(16) T Ks[kChunk * C::kLd];
  __shared__ __align__(16) T Vt[kDim * C::kLd];
  __shared__ float lse_s[kChunk * kMaxTopk];
  __shared__ SlotTable st;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hl = lane >> 5;
  const QTileCoord c = query_tile_coord(p);
  const int64_t Lq = p.n_q * kChunk;
  const int64_t qrow0 = ((static_cast<int64_t>(c.g) * p.B + c.b) * p.H + c.h) * Lq + c.t * kChunk;
  const int my_q = 32 * wave + li;

  if (tid == 0) build_slot_table(st, p, c.g, c.b, c.t - p.shift);
  for (int e = tid; e < kChunk * kMaxTopk; e += kThreads) lse_s[e] = -__builtin_inff();

  Frag<T> qf[4];
  const T* q = static_cast<const T*>(p.q) + (qrow0 + my_q) * kDim;
#pragma unroll
  for (int s = 0; s < 4; ++s) qf[s].load(q + 16 * s + 8 * hl);

  f32x16_t oacc[2] = {zero16(), zero16()};
  const float c2 = p.attn_scale * kLog2e;
  const T* kbase = static_cast<const T*>(p.k) + (static_cast<int64_t>(c.b) * p.H + c.h) * p.n_kv * kChunk * kDim;
  const T* vbase = static_cast<const T*>(p.v) + (static_cast<int64_t>(c.b) * p.H + c.h) * p.n_kv * kChunk * kDim;
  __syncthreads();

  for (int n = 0; n < st.n; ++n) {
    const int64_t j = st.j[n];
    stage_tile<T, true, false>(kbase + j * kChunk * kDim, Ks, nullptr);
    stage_tile<T, false, true>(vbase + j * kChunk * kDim, nullptr, Vt);
    __syncthreads();

    f32x16_t sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = zero16();
      const T* arow = Ks + (32 * tt + pi_row(li)) * C::kLd + 8 * hl;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Frag<T> a;
        a.load(arow + 16 * s);
        sacc[tt] = mma(a, qf[s], sacc[tt]);
      }
    }
    // softmax over the 64 keys of this chunk (32 here, 32 in lane ^ 32)
    float mx = sacc[0][0];
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(sacc[0][r], sacc[1][r]));
    mx = xor32_max(mx);
    const float bias = -mx * c2;
    float l = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = fast_exp2(__builtin_fmaf(sacc[tt][r], c2, bias));
        sacc[tt][r] = e;
        l += e;
      }
    l = xor32_sum(l);
    if (hl == 0) lse_s[my_q * kMaxTopk + st.slot[n]] = mx * p.attn_scale + __builtin_amdgcn_logf(l) * kLn2f;
    const float f = st.w[n] / l;
    Frag<T> pf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = sacc[s >> 1][8 * (s & 1) + e] * f;
      pf[s].set(x);
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const T* arow = Vt + (32 * dt + li) * C::kLd + 16 * hl;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Frag<T> a;
        a.load(arow + 32 * (s >> 1) + 8 * (s & 1));
        oacc[dt] = mma(a, pf[s], oacc[dt]);
      }
    }
    __syncthreads();
  }

  T* o = static_cast<T*>(p.o) + (qrow0 + my_q) * kDim;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      store4(o + 32 * dt + 8 * a + 4 * hl, oacc[dt][4 * a], oacc[dt][4 * a + 1], oacc[dt][4 * a + 2],
             oacc[dt][4 * a + 3]);
  if (p.lse) {
    __syncthreads();
    float* lse = p.lse + qrow0 * p.K;
    for (int e = tid; e < kChunk * p.K; e += kThreads) lse[e] = lse_s[(e / p.K) * kMaxTopk + e % p.K];
  }
}

// ------------------------------------------------------------- backward, query-major (dQ)
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_query_kernel(AttendParams p) {
  using C = TileCfg<T>;
  __shared__ __align__(16) T Ks[kChunk * C::kLd];
  __shared__ __align__(16) T Kt[kDim * C::kLd];
  __shared__ __align__(16) T Vs[kChunk * C::kLd];
  __shared__ float dw_s[2][kMaxTopk];
  __shared__ SlotTable st;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hl = lane >> 5;
  const QTileCoord c = query_tile_coord(p);
  const int64_t Lq = p.n_q * kChunk;
  const int64_t qrow0 = ((static_cast<int64_t>(c.g) * p.B + c.b) * p.H + c.h) * Lq + c.t * kChunk;
  const int my_q = 32 * wave + li;
  const int64_t row = c.t - p.shift;

  if (tid == 0) build_slot_table(st, p, c.g, c.b, row);
  if (tid < 2 * kMaxTopk) dw_s[tid / kMaxTopk][tid % kMaxTopk] = 0.f;

  Frag<T> qf[4], df[4];
  const T* q = static_cast<const T*>(p.q) + (qrow0 + my_q) * kDim;
  const T* dout = static_cast<const T*>(p.dout) + (qrow0 + my_q) * kDim;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qf[s].load(q + 16 * s + 8 * hl);
    df[s].load(dout + 16 * s + 8 * hl);
  }
  f32x16_t dqacc[2] = {zero16(), zero16()};
  const float c2 = p.attn_scale * kLog2e;
  const T* kbase = static_cast<const T*>(p.k) + (static_cast<int64_t>(c.b) * p.H + c.h) * p.n_kv * kChunk * kDim;
  const T* vbase = static_cast<const T*>(p.v) + (static_cast<int64_t>(c.b) * p.H + c.h) * p.n_kv * kChunk * kDim;
  __syncthreads();

  for (int n = 0; n < st.n; ++n) {
    const int64_t j = st.j[n];
    const int slot = st.slot[n];
    stage_tile<T, true, true>(kbase + j * kChunk * kDim, Ks, Kt);
    stage_tile<T, true, false>(vbase + j * kChunk * kDim, Vs, nullptr);
    const float lse_b = p.lse_in[(qrow0 + my_q) * p.K + slot] * kLog2e;
    __syncthreads();

    f32x16_t sacc[2], pacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      sacc[tt] = zero16();
      pacc[tt] = zero16();
      const T* krow = Ks + (32 * tt + pi_row(li)) * C::kLd + 8 * hl;
      const T* vrow = Vs + (32 * tt + pi_row(li)) * C::kLd + 8 * hl;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Frag<T> a, bv;
        a.load(krow + 16 * s);
        bv.load(vrow + 16 * s);
        sacc[tt] = mma(a, qf[s], sacc[tt]);
        pacc[tt] = mma(bv, df[s], pacc[tt]);
      }
    }
    // P = exp(z - lse); e = sum_u P dP'
    float e = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(__builtin_fmaf(sacc[tt][r], c2, -lse_b));
        sacc[tt][r] = pr;
        e = __builtin_fmaf(pr, pacc[tt][r], e);
      }
    e = xor32_sum(e);
    if (hl == 0) p.delta[(qrow0 + my_q) * p.K + slot] = e;
    // per-wave sum of e over its 32 queries, fixed butterfly order
    float es = e;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) es += __shfl_xor(es, off, 64);
    if (lane == 0) dw_s[wave][slot] = es;
    const float w = st.w[n];
    Frag<T> zf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
#pragma unroll
      for (int ee = 0; ee < 8; ++ee) {
        const int tt = s >> 1, r = 8 * (s & 1) + ee;
        x[ee] = w * sacc[tt][r] * (pacc[tt][r] - e);
      }
      zf[s].set(x);
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const T* arow = Kt + (32 * dt + li) * C::kLd + 16 * hl;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Frag<T> a;
        a.load(arow + 32 * (s >> 1) + 8 * (s & 1));
        dqacc[dt] = mma(a, zf[s], dqacc[dt]);
      }
    }
    __syncthreads();
  }

  T* dq = static_cast<T*>(p.dq) + (qrow0 + my_q) * kDim;
  const float sc = p.attn_scale;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      store4(dq + 32 * dt + 8 * a + 4 * hl, sc * dqacc[dt][4 * a], sc * dqacc[dt][4 * a + 1],
             sc * dqacc[dt][4 * a + 2], sc * dqacc[dt][4 * a + 3]);
  if (row >= 0 && tid < p.K) {
    const int64_t o = (((static_cast<int64_t>(c.g) * p.B + c.b) * p.n_q + row) * p.H + c.h) * p.K + tid;
    p.dw_part[o] = dw_s[0][tid] + dw_s[1][tid];
  }
}

// ------------------------------------------------------------- backward, key-major (dK, dV)
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_key_kernel(AttendParams p) {
  using C = TileCfg<T>;
  __shared__ __align__(16) T Qs[kChunk * C::kLd];
  __shared__ __align__(16) T Qt[kDim * C::kLd];
  __shared__ __align__(16) T Ds[kChunk * C::kLd];
  __shared__ __align__(16) T Dt[kDim * C::kLd];
  __shared__ __align__(16) float lse_s[kChunk];
  __shared__ __align__(16) float del_s[kChunk];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hl = lane >> 5;
  const int64_t lid = xcd_logical_block(blockIdx.x, gridDim.x);
  const int64_t j = lid % p.n_kv;
  const int64_t bh = lid / p.n_kv;
  const int h = static_cast<int>(bh % p.H);
  const int b = static_cast<int>(bh / p.H);
  const int my_u = 32 * wave + li;

  const int64_t krow = (bh * p.n_kv + j) * kChunk + my_u;
  Frag<T> kf[4], vf[4];
  const T* kp = static_cast<const T*>(p.k) + krow * kDim;
  const T* vp = static_cast<const T*>(p.v) + krow * kDim;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    kf[s].load(kp + 16 * s + 8 * hl);
    vf[s].load(vp + 16 * s + 8 * hl);
  }
  f32x16_t dkacc[2] = {zero16(), zero16()};
  f32x16_t dvacc[2] = {zero16(), zero16()};
  const float c2 = p.attn_scale * kLog2e;
  const int64_t Lq = p.n_q * kChunk;
  const int32_t* seg = p.seg + static_cast<int64_t>(b) * (p.n_kv + 1);
  const int32_t beg = seg[j], end = seg[j + 1];
  const int32_t* pairs = p.pairs + static_cast<int64_t>(b) * p.pair_cap;

  for (int32_t pr = beg; pr < end; ++pr) {
    const int32_t code = pairs[pr];
    const int slot = code % p.K;
    const int64_t gr = code / p.K;  // g * n_q + row
    const int64_t row = gr % p.n_q;
    const int g = static_cast<int>(gr / p.n_q);
    const int64_t t = row + p.shift;
    const float w = p.wts[((static_cast<int64_t>(g) * p.B + b) * p.n_q + row) * p.K + slot];
    const int64_t qrow0 = ((static_cast<int64_t>(g) * p.B + b) * p.H + h) * Lq + t * kChunk;
    stage_tile<T, true, true>(static_cast<const T*>(p.q) + qrow0 * kDim, Qs, Qt);
    stage_tile<T, true, true>(static_cast<const T*>(p.dout) + qrow0 * kDim, Ds, Dt);
    if (tid < kChunk) lse_s[tid] = p.lse_in[(qrow0 + tid) * p.K + slot] * kLog2e;
    else del_s[tid - kChunk] = p.delta[(qrow0 + tid - kChunk) * p.K + slot];
    __syncthreads();

    // S[q][u] and dP'[q][u] for the 64 queries (two tiles) and this wave's 32 keys.
    f32x16_t sacc[2], pacc[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      sacc[qt] = zero16();
      pacc[qt] = zero16();
      const T* qr = Qs + (32 * qt + pi_row(li)) * C::kLd + 8 * hl;
      const T* dr = Ds + (32 * qt + pi_row(li)) * C::kLd + 8 * hl;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Frag<T> a, bq;
        a.load(qr + 16 * s);
        bq.load(dr + 16 * s);
        sacc[qt] = mma(a, kf[s], sacc[qt]);
        pacc[qt] = mma(bq, vf[s], pacc[qt]);
      }
    }
    // lane holds queries 32 qt + 16 hl + r
    Frag<T> pf[4], zf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int qt = s >> 1;
      const int q0 = 32 * qt + 16 * hl + 8 * (s & 1);
      float xp[8], xz[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * (s & 1) + e;
        const float pw = w * fast_exp2(__builtin_fmaf(sacc[qt][r], c2, -lse_s[q0 + e]));
        xp[e] = pw;
        xz[e] = pw * (pacc[qt][r] - del_s[q0 + e]);
      }
      pf[s].set(xp);
      zf[s].set(xz);
    }
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const T* dtr = Dt + (32 * dt + li) * C::kLd + 16 * hl;
      const T* qtr = Qt + (32 * dt + li) * C::kLd + 16 * hl;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Frag<T> a, bq;
        a.load(dtr + 32 * (s >> 1) + 8 * (s & 1));
        bq.load(qtr + 32 * (s >> 1) + 8 * (s & 1));
        dvacc[dt] = mma(a, pf[s], dvacc[dt]);
        dkacc[dt] = mma(bq, zf[s], dkacc[dt]);
      }
    }
    __syncthreads();
  }

  T* dk = static_cast<T*>(p.dk) + krow * kDim;
  T* dv = static_cast<T*>(p.dv) + krow * kDim;
  const float sc = p.attn_scale;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * dt + 8 * a + 4 * hl;
      store4(dk + d0, sc * dkacc[dt][4 * a], sc * dkacc[dt][4 * a + 1], sc * dkacc[dt][4 * a + 2],
             sc * dkacc[dt][4 * a + 3]);
      store4(dv + d0, dvacc[dt][4 * a], dvacc[dt][4 * a + 1], dvacc[dt][4 * a + 2], dvacc[dt][4 * a + 3]);
    }
}

// ------------------------------------------------------------- inverse retrieval index
// One workgroup per batch row b.  Entry e = (g * n_q + row) * K + slot; key = (j << 32) | e for
// retrievals that feed an existing query chunk (row + shift < n_q) and name a chunk j < n_kv,
// all ones otherwise.  A bitonic sort in LDS orders them by (j, e); segment offsets come from
// binary search.  The same pass writes the fusion weights of every row.
constexpr int kCsrThreads = 256;
constexpr int kCsrCap = 8192;

__global__ __launch_bounds__(kCsrThreads) void csr_build_kernel(AttendParams p) {
  __shared__ uint64_t keys[kCsrCap];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n_ent = p.pair_cap;
  int n2 = 1;
  while (n2 < n_ent) n2 <<= 1;
  for (int e = tid; e < n2; e += kCsrThreads) {
    uint64_t key = ~0ull;
    if (e < n_ent) {
      const int slot = e % p.K;
      const int64_t gr = e / p.K;
      const int64_t row = gr % p.n_q;
      const int g = static_cast<int>(gr / p.n_q);
      const int32_t jj = p.idx[((static_cast<int64_t>(g) * p.B + b) * p.n_q + row) * p.K + slot];
      if (row + p.shift < p.n_q && jj >= 0 && jj < p.n_kv)
        key = (static_cast<uint64_t>(jj) << 32) | static_cast<uint32_t>(e);
    }
    keys[e] = key;
  }
  // fusion weights of every (g, row) of this batch row
  for (int64_t gr = tid; gr < static_cast<int64_t>(p.G) * p.n_q; gr += kCsrThreads) {
    const int64_t row = gr % p.n_q;
    const int g = static_cast<int>(gr / p.n_q);
    const int64_t base = ((static_cast<int64_t>(g) * p.B + b) * p.n_q + row) * p.K;
    float w[kMaxTopk];
    bool valid[kMaxTopk];
    fusion_weights(p.idx + base, p.score + base, p.K, p.n_kv, w, valid);
    for (int k = 0; k < p.K; ++k) p.wts[base + k] = w[k];
  }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int e = tid; e < n2 / 2; e += kCsrThreads) {
        const int lo = 2 * e - (e & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = keys[lo], c = keys[hi];
        if ((a > c) == up) {
          keys[lo] = c;
          keys[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  int32_t* pairs = p.pairs + static_cast<int64_t>(b) * p.pair_cap;
  for (int e = tid; e < n_ent; e += kCsrThreads)
    pairs[e] = keys[e] == ~0ull ? -1 : static_cast<int32_t>(keys[e] & 0xffffffffu);
  int32_t* seg = p.seg + static_cast<int64_t>(b) * (p.n_kv + 1);
  for (int64_t jj = tid; jj <= p.n_kv; jj += kCsrThreads) {
    const uint64_t target = static_cast<uint64_t>(jj) << 32;
    int lo = 0, hi = n_ent;  // first position with key >= target
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (keys[mid] < target) lo = mid + 1;
      else hi = mid;
    }
    seg[jj] = lo;
  }
}

// ------------------------------------------------------------- d(score)
// dscore_k = w_k (dw_k - sum_k' w_k' dw_k'), dw_k = sum over heads (in order) of the per-head
// sums of e over the chunk's tokens.  One thread per (g, b, row).
__global__ __launch_bounds__(256) void score_grad_kernel(AttendParams p) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t rows = static_cast<int64_t>(p.G) * p.B * p.n_q;
  if (gid >= rows) return;
  const int64_t row = gid % p.n_q;
  float* ds = p.dscore + gid * p.K;
  const bool used = row + p.shift < p.n_q;
  float dw[kMaxTopk];
  float wdw = 0.f;
  for (int k = 0; k < p.K; ++k) {
    float acc = 0.f;
    const float w = p.wts[gid * p.K + k];
    const int32_t jj = p.idx[gid * p.K + k];
    if (used && jj >= 0 && jj < p.n_kv) {
      for (int h = 0; h < p.H; ++h) acc += p.dw_part[(gid * p.H + h) * p.K + k];
    }
    dw[k] = acc;
    wdw = __builtin_fmaf(w, acc, wdw);
  }
  for (int k = 0; k < p.K; ++k) {
    const int32_t jj = p.idx[gid * p.K + k];
    const bool valid = used && jj >= 0 && jj < p.n_kv;
    ds[k] = valid ? p.wts[gid * p.K + k] * (dw[k] - wdw) : 0.f;
  }
}

}  // namespace

hipError_t launch_attend_fwd(const AttendParams& p, bool f32, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.G) * p.B * p.H * p.n_q;
  if (f32)
    hipLaunchKernelGGL(attend_fwd_kernel<float>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(attend_fwd_kernel<bf16_t>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_csr_build(const AttendParams& p, hipStream_t s) {
  hipLaunchKernelGGL(csr_build_kernel, dim3(static_cast<uint32_t>(p.B)), dim3(kCsrThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_query(const AttendParams& p, bool f32, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.G) * p.B * p.H * p.n_q;
  if (f32)
    hipLaunchKernelGGL(bwd_query_kernel<float>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(bwd_query_kernel<bf16_t>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_key(const AttendParams& p, bool f32, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.B) * p.H * p.n_kv;
  if (f32)
    hipLaunchKernelGGL(bwd_key_kernel<float>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(bwd_key_kernel<bf16_t>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_score_grad(const AttendParams& p, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(p.G) * p.B * p.n_q;
  const int64_t blocks = (rows + 255) / 256;
  hipLaunchKernelGGL(score_grad_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace gca
