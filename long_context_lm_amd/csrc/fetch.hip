// Fetch of retrieved chunks: the K/V tiles a retrieval selected, gathered into a compact buffer.
//
// In inference the K/V of past chunks may be kept in host memory and the chunks a retrieval
// selects loaded back to the device before the next chunk attends to them [Notes, Key designs:
// memory-offload inference].  Retrieval slot (g, b, r, k) of a chunk j in range has its tiles
// k[b,h,j] and v[b,h,j] (every head h) copied to k_out[b,h,c] and v_out[b,h,c] with
// c = (g n_q + r) K + k, and idx_out[g,b,r,k] = c (-1 where j is out of range).  The sources are
// read with ordinary vector loads, so they may sit in device memory or in pinned host memory
// mapped into the device's address space (then every load crosses the host link).
#include "gca_device.hpp"
#include "gca_internal.hpp"

namespace gca {
namespace {

constexpr int kThreads = 256;

// One workgroup per (retrieval slot, head); heads are the fastest index, so the workgroups of one
// slot read the same chunk's tiles of consecutive heads.  Each thread issues all of its loads
// before its first store: the whole fetch is in flight at once.
template <typename T>
__global__ __launch_bounds__(kThreads) void fetch_chunks_kernel(FetchParams p) {
  constexpr int kTileBytes = kChunk * kDim * static_cast<int>(sizeof(T));
  constexpr int kPer = kTileBytes / (16 * kThreads);  // 16-byte pieces per thread per tile
  const int64_t item = blockIdx.x;
  const int h = static_cast<int>(item % p.H);
  const int64_t sl = item / p.H;  // ((g B + b) n_q + r) K + k
  const int k = static_cast<int>(sl % p.K);
  int64_t rest = sl / p.K;
  const int64_t r = rest % p.n_q;
  rest /= p.n_q;
  const int b = static_cast<int>(rest % p.B);
  const int g = static_cast<int>(rest / p.B);
  const int32_t j = p.idx[sl];
  const bool valid = j >= 0 && j < p.n_kv;
  const int64_t c = (static_cast<int64_t>(g) * p.n_q + r) * p.K + k;
  if (h == 0 && threadIdx.x == 0) p.idx_out[sl] = valid ? static_cast<int32_t>(c) : -1;
  if (!valid) return;
  const int64_t bh = static_cast<int64_t>(b) * p.H + h;
  const u32x4_t* ks = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.k) + (bh * p.n_kv + j) * kTileBytes);
  const u32x4_t* vs = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(p.v) + (bh * p.n_kv + j) * kTileBytes);
  u32x4_t* kd = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.k_out) + (bh * p.n_c + c) * kTileBytes);
  u32x4_t* vd = reinterpret_cast<u32x4_t*>(static_cast<char*>(p.v_out) + (bh * p.n_c + c) * kTileBytes);
  u32x4_t kb[kPer], vb[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    kb[e] = ks[threadIdx.x + e * kThreads];
    vb[e] = vs[threadIdx.x + e * kThreads];
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    kd[threadIdx.x + e * kThreads] = kb[e];
    vd[threadIdx.x + e * kThreads] = vb[e];
  }
}

}  // namespace

hipError_t launch_fetch_chunks(const FetchParams& p, bool f32, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.G) * p.B * p.n_q * p.K * p.H)), block(kThreads);
  if (f32) hipLaunchKernelGGL(fetch_chunks_kernel<float>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(fetch_chunks_kernel<bf16_t>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace gca
