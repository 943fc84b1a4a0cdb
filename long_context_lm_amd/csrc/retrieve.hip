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
// One 256-thread workgroup scores one block of candidates of one row; each thread keeps its
// own sorted top-K list, the block merges them with wave-wide max reductions.  Rows with more
// candidates than one block covers are split over several blocks whose partial top-K lists a
// second kernel merges (the 16M-token history: 262,144 candidates per row).
#include "gca_device.hpp"
#include "gca_internal.hpp"

namespace gca {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kList = kMaxTopk;  // per-thread list length (>= K)

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

// --------------------------------------------------------------- per-thread sorted list
struct TopList {
  uint64_t key[kList];
  float s[kList];
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int e = 0; e < kList; ++e) {
      key[e] = 0;
      s[e] = 0.f;
    }
  }
  // Insert keeping key[] descending; the smallest entry falls off the end.
  __device__ __forceinline__ void insert(uint64_t k, float sv) {
    if (k <= key[kList - 1]) return;
#pragma unroll
    for (int e = 0; e < kList; ++e) {
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
    for (int e = 0; e + 1 < kList; ++e) {
      key[e] = key[e + 1];
      s[e] = s[e + 1];
    }
    key[kList - 1] = 0;
  }
};

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Block-wide top-K of the threads' lists.  Results land in out_key/out_s (LDS, K entries).
__device__ void block_topk(TopList& L, int K, uint64_t* wave_key, float* wave_s, uint64_t* out_key,
                           float* out_s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int k = 0; k < K; ++k) {
    const uint64_t m = wave_max_u64(L.key[0]);
    float sw = 0.f;
    if (m != 0) {
      const uint64_t hit = __ballot(L.key[0] == m);
      const int owner = __ffsll(static_cast<unsigned long long>(hit)) - 1;
      sw = __shfl(L.s[0], owner, 64);
      if (lane == owner) L.pop();
    }
    if (lane == 0) {
      wave_key[wave * kMaxTopk + k] = m;
      wave_s[wave * kMaxTopk + k] = sw;
    }
  }
  __syncthreads();
  if (wave == 0) {
    uint64_t mine = 0;
    float ms = 0.f;
    if (lane < kWaves * K) {
      mine = wave_key[(lane / K) * kMaxTopk + lane % K];
      ms = wave_s[(lane / K) * kMaxTopk + lane % K];
    }
    for (int k = 0; k < K; ++k) {
      const uint64_t m = wave_max_u64(mine);
      float sw = 0.f;
      if (m != 0) {
        const uint64_t hit = __ballot(mine == m);
        const int owner = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        sw = __shfl(ms, owner, 64);
        if (lane == owner) mine = 0;
      }
      if (lane == 0) {
        out_key[k] = m;
        out_s[k] = sw;
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ double lmk_to_f64(const bf16_t* p, int d) { return static_cast<double>(to_f32(p[d])); }
__device__ __forceinline__ double lmk_to_f64(const float* p, int d) { return static_cast<double>(p[d]); }

// Exact sequential float64 dot product of one key landmark row with the query row in LDS.
template <typename T>
__device__ __forceinline__ double landmark_dot(const T* __restrict__ row, const double* lq_s);

template <>
__device__ __forceinline__ double landmark_dot<bf16_t>(const bf16_t* __restrict__ row, const double* lq_s) {
  const u32x4_t* r4 = reinterpret_cast<const u32x4_t*>(row);
  u32x4_t chunk[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) chunk[c] = r4[c];
  double acc = 0.0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t pair = chunk[c][w];
      const double lo = static_cast<double>(__uint_as_float(pair << 16));
      const double hi = static_cast<double>(__uint_as_float(pair & 0xffff0000u));
      acc = __builtin_fma(lq_s[8 * c + 2 * w], lo, acc);
      acc = __builtin_fma(lq_s[8 * c + 2 * w + 1], hi, acc);
    }
  }
  return acc;
}

template <>
__device__ __forceinline__ double landmark_dot<float>(const float* __restrict__ row, const double* lq_s) {
  const f32x4_t* r4 = reinterpret_cast<const f32x4_t*>(row);
  double acc = 0.0;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const f32x4_t x = r4[c];
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = __builtin_fma(lq_s[4 * c + w], static_cast<double>(x[w]), acc);
  }
  return acc;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void score_topk_kernel(RetrieveParams p) {
  __shared__ double lq_s[kDim];
  __shared__ uint64_t wave_key[kWaves * kMaxTopk];
  __shared__ float wave_s[kWaves * kMaxTopk];
  __shared__ uint64_t out_key[kMaxTopk];
  __shared__ float out_s[kMaxTopk];

  const int tid = threadIdx.x;
  const int64_t bid = blockIdx.x;
  const int blk = static_cast<int>(bid % p.nblk);
  const int64_t rowid = bid / p.nblk;  // (g * B + b) * n_q + r
  const int64_t r = rowid % p.n_q;
  const int64_t gb = rowid / p.n_q;
  const int b = static_cast<int>(gb % p.B);
  const int g = static_cast<int>(gb / p.B);
  const int64_t i = p.base + r;
  const int64_t ncand = i < p.n_kv ? i : p.n_kv;

  const T* lq = static_cast<const T*>(p.lq) + rowid * kDim;
  if (tid < kDim) lq_s[tid] = lmk_to_f64(lq, tid);
  __syncthreads();

  TopList L;
  L.clear();
  const T* lk = static_cast<const T*>(p.lk) + gb * p.n_kv * kDim;
  const int64_t j0 = static_cast<int64_t>(blk) * kThreads * p.cpt;
  for (int n = 0; n < p.cpt; ++n) {
    const int64_t j = j0 + static_cast<int64_t>(n) * kThreads + tid;
    if (j >= ncand) break;
    const double acc = landmark_dot<T>(lk + j * kDim, lq_s);
    const float s = canon_zero(static_cast<float>(acc) * p.score_scale);
    float rkey = s;
    if (p.use_gumbel) {
#pragma clang fp contract(off)
      const float noise = p.tau * gumbel(p.seed, g, b, i, j);
      rkey = canon_zero(s + noise);
    }
    L.insert(make_key(rkey, j), s);
  }

  block_topk(L, p.K, wave_key, wave_s, out_key, out_s);

  if (tid < p.K) {
    const uint64_t key = out_key[tid];
    if (p.nblk == 1) {
      p.idx[rowid * p.K + tid] = key_index(key);
      p.score[rowid * p.K + tid] = key == 0 ? -__builtin_inff() : out_s[tid];
    } else {
      const int64_t o = (rowid * p.nblk + blk) * p.K + tid;
      p.part_key[o] = key;
      p.part_s[o] = out_s[tid];
    }
  }
}

__global__ __launch_bounds__(kThreads) void topk_merge_kernel(RetrieveParams p) {
  __shared__ uint64_t wave_key[kWaves * kMaxTopk];
  __shared__ float wave_s[kWaves * kMaxTopk];
  __shared__ uint64_t out_key[kMaxTopk];
  __shared__ float out_s[kMaxTopk];
  const int tid = threadIdx.x;
  const int64_t rowid = blockIdx.x;
  const int64_t n_in = static_cast<int64_t>(p.nblk) * p.K;
  const uint64_t* keys = p.part_key + rowid * n_in;
  const float* svals = p.part_s + rowid * n_in;
  TopList L;
  L.clear();
  for (int64_t c = tid; c < n_in; c += kThreads) L.insert(keys[c], svals[c]);
  block_topk(L, p.K, wave_key, wave_s, out_key, out_s);
  if (tid < p.K) {
    const uint64_t key = out_key[tid];
    p.idx[rowid * p.K + tid] = key_index(key);
    p.score[rowid * p.K + tid] = key == 0 ? -__builtin_inff() : out_s[tid];
  }
}

}  // namespace

hipError_t launch_score_topk(const RetrieveParams& p, bool f32, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.G) * p.B * p.n_q * p.nblk;
  if (f32)
    hipLaunchKernelGGL(score_topk_kernel<float>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(score_topk_kernel<bf16_t>, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const RetrieveParams& p, hipStream_t s) {
  const int64_t blocks = static_cast<int64_t>(p.G) * p.B * p.n_q;
  hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace gca
