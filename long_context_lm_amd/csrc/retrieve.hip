// Causal chunk retrieval: exact landmark scores fused with a streaming top-k.
//
// [Notes, Key designs: causal retrieval]: the landmark of chunk i is scored against the
// landmark of every strictly earlier chunk j and the k best are kept.
// [Notes, Key designs: Gumbel top-k]: in training, Gumbel noise is added to the scores before
// the top-k; it only changes which chunks are selected.
//
// Each score is the float64 sequential sum over d of exact products lq[i,d] * lk[j,d]
// (bf16/fp32 products are exact in float64, so a fused multiply-add gives the same bits as a
// multiply followed by an add), rounded once to fp32 and multiplied by score_scale in fp32.
// The selection key packs the order-preserving image of the (possibly perturbed) fp32 score
// above the complement of j, so the largest key is the best score with the lowest j.  Key 0
// never occurs for a finite score and marks an empty slot.
//
// One workgroup scores one block of candidates of one row (cpt candidates per lane, 256 lanes);
// each lane keeps a sorted list of its best keys, each wave extracts its top K with K rounds of a
// wave-wide maximum, and the four wave lists are merged through LDS.  Rows with more candidates
// than one block are split over several workgroups whose partial top-K lists a second kernel
// merges (the 16M-token history: 262,144 candidates per row, 512 blocks of 512).
#include "gca_device.hpp"
#include "gca_internal.hpp"

namespace gca {
namespace {


// --------------------------------------------------------------- Philox4x64-10 (SC'11)
__device__ __forceinline__ uint64_t philox_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                                 uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t hi0 = __umul64hi(kM0, c0), lo0 = kM0 * c0;
    const uint64_t hi1 = __umul64hi(kM1, c2), lo1 = kM1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += kW0;
    k1 += kW1;
  }
  return c0;
}

// --------------------------------------------------------------- fixed-order logarithm
// ln(x) = e ln2 + 2 f (1 + z/3 + z^2/5 + ... + z^11/23), f = (m-1)/(m+1), z = f^2, with
// x = m 2^e and m in [sqrt(1/2), sqrt(2)).  Every operation is a single IEEE float64 rounding
// (no contraction into fused multiply-adds), so the result is a fixed function of x.
struct AtanhCoeffs {
  double c[12];
  constexpr AtanhCoeffs() : c() {
    for (int n = 0; n < 12; ++n) c[n] = 1.0 / static_cast<double>(2 * n + 1);
  }
};

__device__ __noinline__ double ln_fixed(double x) {
#pragma clang fp contract(off)
  constexpr AtanhCoeffs kC;
  constexpr double kSqrtHalf = 0x1.6a09e667f3bcdp-1;
  constexpr double kLn2 = 0x1.62e42fefa39efp-1;
  int e = 0;
  double m = frexp(x, &e);
  if (m < kSqrtHalf) {
    m = m * 2.0;
    e = e - 1;
  }
  const double f = (m - 1.0) / (m + 1.0);
  const double z = f * f;
  double p = kC.c[11];
#pragma unroll
  for (int n = 10; n >= 0; --n) p = p * z + kC.c[n];
  const double a = static_cast<double>(e) * kLn2;
  const double b = (2.0 * f) * p;
  return a + b;
}

__device__ float gumbel(uint64_t seed, int g, int b, int64_t i, int64_t j) {
  const uint64_t x = philox_word0(static_cast<uint64_t>(j), static_cast<uint64_t>(i),
                                  (static_cast<uint64_t>(g) << 32) | static_cast<uint32_t>(b), 0ull,
                                  seed, 0ull);
  const double u = (static_cast<double>(x >> 12) + 0.5) * 0x1.0p-52;
  const double y = -ln_fixed(-ln_fixed(u));
  return static_cast<float>(y);
}

__device__ __forceinline__ float canon_zero(float x) { return x == 0.f ? 0.f : x; }

__device__ __forceinline__ uint64_t make_key(float r, int64_t j) {
  const uint32_t u = __float_as_uint(r);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(j));
}

__device__ __forceinline__ int32_t key_index(uint64_t key) {
  return key == 0 ? -1 : static_cast<int32_t>(~static_cast<uint32_t>(key));
}

// --------------------------------------------------------------- per-lane sorted list
template <int KL>
struct TopList {
  uint64_t key[KL];
  float s[KL];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int e = 0; e < KL; ++e) {
      key[e] = 0;
      s[e] = 0.f;
    }
  }
  // Insert keeping key[] descending; the smallest entry falls off the end.
  __device__ __forceinline__ void insert(uint64_t k, float sv) {
    if (k <= key[KL - 1]) return;
#pragma unroll
    for (int e = 0; e < KL; ++e) {
      const bool take = k > key[e];
      const uint64_t tk = key[e];
      const float ts = s[e];
      key[e] = take ? k : key[e];
      s[e] = take ? sv : s[e];
      k = take ? tk : k;
      sv = take ? ts : sv;
    }
  }
  __device__ __forceinline__ void pop() {
#pragma unroll
    for (int e = 0; e + 1 < KL; ++e) {
      key[e] = key[e + 1];
      s[e] = s[e + 1];
    }
    key[KL - 1] = 0;
  }
};

// Wave-wide maximum of a 32-bit value, in every lane.  Within each 16-lane row the partners come
// from DPP lane permutations (xor 1, xor 2, then the half-row and row mirrors, which act as xor 4
// and xor 8 once the quads agree); across rows from v_permlane16_swap / v_permlane32_swap.  No
// LDS traffic, so the K selection rounds are not bound by LDS latency.
// (Every lane has a source lane under these permutations; the zero "old" value and bound_ctrl
// let the compiler fold the move into the max as one v_max_u32_dpp.)
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kCtrl, 0xf, 0xf, true));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // rows 0<->1, 2<->3
  v = max(r[0], r[1]);
  const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // halves
  return max(h[0], h[1]);
}

// Top K of the wave's lists; lane k (< K) returns the k-th best key and its clean score.  Each
// round finds the largest head key: first the largest high (score) word, then, only if several
// lanes share it, the largest low word (the lowest chunk index) among those lanes.  A finite score
// never has a zero high word and a chunk index never a zero low word, so zero marks an empty list.
template <int KL>
__device__ __forceinline__ void wave_topk(TopList<KL>& L, int K, uint64_t& my_key, float& my_s) {
  const int lane = threadIdx.x & 63;
  my_key = 0;
  my_s = 0.f;
  for (int k = 0; k < K; ++k) {
    const uint32_t hh = static_cast<uint32_t>(L.key[0] >> 32);
    const uint32_t hl = static_cast<uint32_t>(L.key[0]);
    const uint32_t mh = wave_max_u32(hh);
    if (mh == 0) break;  // wave-uniform: every list is empty
    const bool top = hh == mh;
    uint64_t hit = __ballot(top);
    if (__popcll(hit) > 1) {
      const uint32_t ml = wave_max_u32(top ? hl : 0u);
      hit = __ballot(top && hl == ml);
    }
    const int owner = __ffsll(static_cast<unsigned long long>(hit)) - 1;
    const uint32_t wl = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hl), owner));
    const float sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(L.s[0]), owner));
    if (lane == owner) L.pop();
    if (lane == k) {
      my_key = (static_cast<uint64_t>(mh) << 32) | wl;
      my_s = sw;
    }
  }
}

__device__ __forceinline__ double lmk_to_f64(const bf16_t* p, int d) { return static_cast<double>(to_f32(p[d])); }
__device__ __forceinline__ double lmk_to_f64(const float* p, int d) { return static_cast<double>(p[d]); }

// One key-landmark row held in registers, so that the next row's load can be in flight while
// this one is scored.
template <typename T>
struct LmkRow;

template <>
struct LmkRow<bf16_t> {
  u32x4_t c[8];
  __device__ __forceinline__ void load(const bf16_t* row) {
    const u32x4_t* r4 = reinterpret_cast<const u32x4_t*>(row);
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = r4[k];
  }
  // Exact sequential float64 dot product with the query landmark in LDS.
  __device__ __forceinline__ double dot(const double* lq_s) const {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t pair = c[k][w];
        const double lo = static_cast<double>(__uint_as_float(pair << 16));
        const double hi = static_cast<double>(__uint_as_float(pair & 0xffff0000u));
        acc = __builtin_fma(lq_s[8 * k + 2 * w], lo, acc);
        acc = __builtin_fma(lq_s[8 * k + 2 * w + 1], hi, acc);
      }
    }
    return acc;
  }
};

template <>
struct LmkRow<float> {
  f32x4_t c[16];
  __device__ __forceinline__ void load(const float* row) {
    const f32x4_t* r4 = reinterpret_cast<const f32x4_t*>(row);
#pragma unroll
    for (int k = 0; k < 16; ++k) c[k] = r4[k];
  }
  __device__ __forceinline__ double dot(const double* lq_s) const {
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int w = 0; w < 4; ++w) acc = __builtin_fma(lq_s[4 * k + w], static_cast<double>(c[k][w]), acc);
    return acc;
  }
};

constexpr int kMergeThreads = 1024;      // sixteen waves per merged row
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMergeBatch = 8;           // partial entries each merge thread loads at once

// Merge the K-best lists of `nw` waves (lane k < K of wave w holds entry k) through LDS; wave 0
// returns the top K of the union, lane k holding entry k.  Every thread of the workgroup calls it.
template <int KL>
__device__ __forceinline__ void workgroup_topk(int nw, int K, uint64_t key, float sv, uint64_t* lkey, float* ls,
                                               uint64_t& out_key, float& out_s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane < K) {
    lkey[wave * K + lane] = key;
    ls[wave * K + lane] = sv;
  }
  __syncthreads();
  out_key = 0;
  out_s = 0.f;
  if (wave == 0) {
    TopList<KL> L;
    L.clear();
    for (int e = lane; e < nw * K; e += 64)
      if (lkey[e] != 0) L.insert(lkey[e], ls[e]);
    wave_topk<KL>(L, K, out_key, out_s);
  }
}

// One workgroup of NW waves per (row, block of 64 NW cpt candidates).  Lane c of the workgroup
// scores the candidates j = block start + c + 64 NW n (n < cpt), so every pass reads 64 NW
// consecutive key-landmark rows; the next row's load is issued before the current one is scored.
// NW = 4 for a few long rows (a decode step over a long history: many blocks per row, their lists
// merged by the workgroup and then by topk_merge); NW = 1 for many short rows (training: one wave
// per row).  At most 128 VGPRs for bf16 landmarks and lists of 8 (four resident waves per SIMD,
// enough loads in flight to stream a long history); fp32 rows and lists of 16 keep two.
template <typename T, int KL, int NW>
__global__ __launch_bounds__(64 * NW, (sizeof(T) == 2 && KL <= 8) ? 4 : 2) void score_topk_kernel(RetrieveParams p) {
  constexpr int kBlockCand = 64 * NW;  // candidates of one block per pass (one per lane)
  __shared__ double lq_s[kDim];
  __shared__ uint64_t lkey[NW * kMaxTopk];
  __shared__ float ls[NW * kMaxTopk];
  const int lane = threadIdx.x & 63;
  const int64_t item = blockIdx.x;
  const int blk = static_cast<int>(item % p.nblk);
  const int64_t rowid = item / p.nblk;  // (g * B + b) * n_q + r
  const int64_t r = rowid % p.n_q;
  const int64_t gb = rowid / p.n_q;
  const int b = static_cast<int>(gb % p.B);
  const int g = static_cast<int>(gb / p.B);
  const int64_t i = p.base + r;
  const int64_t ncand = i < p.n_kv ? i : p.n_kv;

  TopList<KL> L;
  L.clear();
  const T* lk = static_cast<const T*>(p.lk) + gb * p.n_kv * kDim;
  const int64_t jb = static_cast<int64_t>(blk) * kBlockCand * p.cpt + threadIdx.x;
  int mine = 0;  // candidates of this lane
  if (jb < ncand) {
    const int64_t m = (ncand - jb + kBlockCand - 1) / kBlockCand;
    mine = m < p.cpt ? static_cast<int>(m) : p.cpt;
  }
  LmkRow<T> cur, nxt;
  if (mine > 0) cur.load(lk + jb * kDim);  // in flight while the query landmark is staged
  if (threadIdx.x < kDim) lq_s[threadIdx.x] = lmk_to_f64(static_cast<const T*>(p.lq) + rowid * kDim, threadIdx.x);
  __syncthreads();

  for (int n = 0; n < mine; ++n) {
    const int64_t j = jb + static_cast<int64_t>(n) * kBlockCand;
    if (n + 1 < mine) nxt.load(lk + (j + kBlockCand) * kDim);
    // an opaque zero offset keeps the query landmark in LDS (read per candidate) instead of in
    // 128 registers hoisted out of the loop
    int zero = 0;
    asm volatile("" : "+v"(zero));
    const double acc = cur.dot(lq_s + zero);
    const float s = canon_zero(static_cast<float>(acc) * p.score_scale);
    float rkey = s;
    if (p.use_gumbel) {
#pragma clang fp contract(off)
      const float noise = p.tau * gumbel(p.seed, g, b, i, j);
      rkey = canon_zero(s + noise);
    }
    L.insert(make_key(rkey, j), s);
    cur = nxt;
  }

  uint64_t key, bkey;
  float sv, bs;
  wave_topk<KL>(L, p.K, key, sv);
  if constexpr (NW > 1) {
    workgroup_topk<KL>(NW, p.K, key, sv, lkey, ls, bkey, bs);
  } else {
    bkey = key;
    bs = sv;
  }
  if (p.nblk == 1) {
    if (threadIdx.x < p.K) {
      p.idx[rowid * p.K + lane] = key_index(bkey);
      p.score[rowid * p.K + lane] = bkey == 0 ? -__builtin_inff() : bs;
    }
    return;
  }

  if (threadIdx.x < p.K) {
    const int64_t o = (rowid * p.nblk + blk) * p.K + lane;
    p.part_key[o] = bkey;
    p.part_s[o] = bs;
  }
}

// One workgroup of sixteen waves per long row merges the row's nblk partial top-K lists; each
// thread loads its share of the entries in batches whose loads are in flight together.
template <int KL>
__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(RetrieveParams p) {
  __shared__ uint64_t lkey[kMergeWaves * kMaxTopk];
  __shared__ float ls[kMergeWaves * kMaxTopk];
  const int64_t rowid = blockIdx.x;
  const int64_t n_in = static_cast<int64_t>(p.nblk) * p.K;
  const uint64_t* keys = p.part_key + rowid * n_in;
  const float* svals = p.part_s + rowid * n_in;
  TopList<KL> L;
  L.clear();
  for (int64_t c0 = threadIdx.x; c0 < n_in; c0 += static_cast<int64_t>(kMergeThreads) * kMergeBatch) {
    uint64_t kb[kMergeBatch];
    float sb[kMergeBatch];
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e) {
      const int64_t c = c0 + static_cast<int64_t>(e) * kMergeThreads;
      kb[e] = c < n_in ? keys[c] : 0;
      sb[e] = c < n_in ? svals[c] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < kMergeBatch; ++e)
      if (kb[e] != 0) L.insert(kb[e], sb[e]);
  }
  uint64_t key, bkey;
  float sv, bs;
  wave_topk<KL>(L, p.K, key, sv);
  workgroup_topk<KL>(kMergeWaves, p.K, key, sv, lkey, ls, bkey, bs);
  if (threadIdx.x < p.K) {
    p.idx[rowid * p.K + threadIdx.x] = key_index(bkey);
    p.score[rowid * p.K + threadIdx.x] = bkey == 0 ? -__builtin_inff() : bs;
  }
}

}  // namespace

template <int NW>
void launch_score_topk_nw(const RetrieveParams& p, bool f32, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.G) * p.B * p.n_q * p.nblk)), block(64 * NW);
  const bool small = p.K <= 8;
  if (f32) {
    if (small) hipLaunchKernelGGL((score_topk_kernel<float, 8, NW>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((score_topk_kernel<float, 16, NW>), grid, block, 0, s, p);
  } else {
    if (small) hipLaunchKernelGGL((score_topk_kernel<bf16_t, 8, NW>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((score_topk_kernel<bf16_t, 16, NW>), grid, block, 0, s, p);
  }
}

hipError_t launch_score_topk(const RetrieveParams& p, bool f32, hipStream_t s) {
  if (p.nw == 1) launch_score_topk_nw<1>(p, f32, s);
  else launch_score_topk_nw<4>(p, f32, s);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const RetrieveParams& p, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.G) * p.B * p.n_q));
  if (p.K <= 8) hipLaunchKernelGGL((topk_merge_kernel<8>), grid, dim3(kMergeThreads), 0, s, p);
  else hipLaunchKernelGGL((topk_merge_kernel<16>), grid, dim3(kMergeThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace gca
