// Host-side launch descriptors shared by the GCA kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gca {

// Which kernel a launch belongs to (names reported by the kernel timer).
enum KernelId {
  kScoreTopk = 0,
  kTopkMerge,
  kAttendFwd,
  kInverseIndex,
  kBwdQuery,
  kBwdKey,
  kScoreGrad,
  kLmkQueryGrad,
  kLmkKeyGrad,
  kFetchChunks,
  kDecodeTokens,
  kSwFwd,
  kSwBwdQuery,
  kSwBwdKey,
  kFusedFwd,
  kFusedBwdQuery,
  kNumKernels
};
const char* kernel_name(int id);

// Key-major backward: a key chunk's inverse-index list of more than kSplitMin entries is split
// into segments of at most kSegEntries entries that the key-major pass's helper workgroups walk
// in parallel (its other workgroups then walk at most kSplitMin entries per chunk).
constexpr int kSplitMin = 128;
constexpr int kSegEntries = 64;

struct RetrieveParams {
  const void* lq;
  const void* lk;
  int32_t* idx;
  float* score;
  uint64_t* part_key;   // [rows, nblk, K] partial keys (long rows only)
  float* part_s;        // [rows, nblk, K] partial clean scores
  int64_t n_q, base, n_kv;
  int32_t G, B, K;
  int32_t nblk;         // candidate blocks per row (1 = single stage)
  int32_t cpt;          // candidates per thread per block
  int32_t nw;           // waves per block (1 or 4): 64 nw cpt candidates per block
  float score_scale;
  int32_t use_gumbel;
  uint64_t seed;
  float tau;
};

struct AttendParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  const float* score;
  const float* lse_in;  // backward: forward log-sum-exp
  const void* dout;
  void* o;              // forward output
  float* lse;           // forward output (may be null)
  void* dq;
  void* dk;
  void* dv;
  float* dscore;
  float* delta;         // [G, B, H, n_q, K, 2, 64]: 64 biases log2 w_k - lse_{t,k} log2 e, then the
                        // 64 negated e_{t,k} = <dout_t, O_{t,k}>
  float* dw_part;       // [G, B, n_q, H, K] per-head sums of e over a chunk's tokens
  float* wts;           // [G, B, n_q, K] fusion weights (0 on invalid slots)
  int32_t* pairs;       // [B, n_kv, pair_cap, 2] one entry per retrieval of each key chunk, in
                        // (g, row, slot) order: {(g n_q + row) K + slot, value} (landmark
                        // gradients), or {row + shift, 16 g + slot} with entry_decoded
  int32_t* counts;      // [B, n_kv] list lengths
  int64_t n_q, n_kv, q_base;
  int32_t G, B, H, K, shift;
  int32_t pair_cap;     // G * n_q: most retrievals one key chunk can receive
  // fused layer attention (sliding window + GCA over the same queries, G = 1); unused otherwise
  const void* k_sw;     // [B, H, n_q * 64, 64] the window's keys and values
  const void* v_sw;
  float* lse_sw;        // forward output / backward input [B, H, n_q * 64] (may be null in the forward)
  float* sw_stats;      // backward: [B, H, n_q][2][64] per query tile: 64 biases -lse_sw log2 e,
                        // then the 64 negated D_sw, for the window's key pass
  int32_t m;            // window in chunks (W = 64 m); 0 = no window
  int32_t entry_decoded;  // inverse index entries for the key-major pass (see pairs)
  int32_t causal_rows;  // inverse index: 1 = list only rows whose global chunk lies after the key
                        // chunk (the landmark gradients' rule j < q_base + row); 0 = every row
                        // (the GCA backward, whose other passes count every 0 <= j < n_kv)
  // key-major pass with long lists split (null: no split): {long chunks, segment slots} counter,
  // long chunks [long_cap][4] {b, j, segments, first slot}, the long chunk of each segment slot
  // [seg_cap], float partials [seg_cap * H][2][64][64]; the first n_help (a multiple of 8)
  // workgroups of the key-major pass walk the segments
  uint64_t* long_ctl;
  int32_t* long_list;
  int32_t* long_seg;
  float* long_part;
  int32_t long_cap, seg_cap, n_help;
  float attn_scale;
};

struct LandmarkParams {
  const void* lq;
  const void* lk;
  const int32_t* idx;
  const float* dscore;
  void* dlq;
  void* dlk;
  const int32_t* pairs;   // inverse retrieval index with d(score) as the entry value
  const int32_t* counts;
  int64_t n_q, n_kv, q_base;
  int32_t G, B, K;
  int32_t pair_cap;       // G * n_q
  float score_scale;
};

struct FetchParams {
  const int32_t* idx;
  const void* k;        // [B, H, n_kv, 64, 64] device-visible address (device or pinned host memory)
  const void* v;
  void* k_out;          // [B, H, n_c, 64, 64], n_c = G n_q K
  void* v_out;
  int32_t* idx_out;     // [G, B, n_q, K]
  int64_t n_q, n_kv, n_c;
  int32_t G, B, H, K;
};

// Sliding-window attention over one sequence of n_c chunks: q, k, v, o, dout, dq, dk, dv are
// [B, H, n_c * 64, 64]; lse [B, H, n_c * 64] (natural log-sum-exp of attn_scale q.k over the window);
// stats [B, H, n_c][2][64] per query tile: 64 biases -lse log2 e, then the 64 negated
// D = <dout, o>, for the key-major pass.
struct SwParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o_in;
  const float* lse_in;
  const void* dout;
  void* o;
  float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* stats;
  int64_t n_c;
  int32_t B, H;
  int32_t m;            // window in chunks: W = 64 m keys per token, itself included
  float attn_scale;
};

// Launchers (return the hipError_t of the launch).
hipError_t launch_score_topk(const RetrieveParams& p, bool f32, hipStream_t s);
hipError_t launch_topk_merge(const RetrieveParams& p, hipStream_t s);
hipError_t launch_attend_fwd(const AttendParams& p, bool f32, hipStream_t s);
hipError_t launch_inverse_index(const AttendParams& p, hipStream_t s);
hipError_t launch_bwd_query(const AttendParams& p, bool f32, hipStream_t s);
hipError_t launch_bwd_key(const AttendParams& p, bool f32, hipStream_t s);
hipError_t launch_score_grad(const AttendParams& p, bool f32, hipStream_t s);
hipError_t launch_lmk_query_grad(const LandmarkParams& p, bool f32, hipStream_t s);
hipError_t launch_lmk_key_grad(const LandmarkParams& p, bool f32, hipStream_t s);
hipError_t launch_fetch_chunks(const FetchParams& p, bool f32, hipStream_t s);
hipError_t launch_decode_tokens(const AttendParams& p, int32_t n_tok, bool f32, hipStream_t s);
hipError_t launch_sw_fwd(const SwParams& p, bool f32, hipStream_t s);
hipError_t launch_sw_bwd_query(const SwParams& p, bool f32, hipStream_t s);
hipError_t launch_sw_bwd_key(const SwParams& p, bool f32, hipStream_t s);
hipError_t launch_fused_fwd(const AttendParams& p, bool f32, hipStream_t s);
hipError_t launch_fused_bwd_query(const AttendParams& p, bool f32, hipStream_t s);

}  // namespace gca
