/*
 * gca.h -- C ABI of the Grouped Cross-Attention (GCA) library for AMD Instinct MI355X (gfx950).
 *
 * The operation follows the pages on "Efficient Length-Generalizable Attention via Causal
 * Retrieval for Long-Context Language Modeling" (ICML 2025):
 *   [Notes]  zhaoyang97.github.io Paper-Notes page on the paper;
 *   [Forum]  openreview.net forum page (abstract).
 * A sequence is cut into chunks of S = 64 tokens [Notes, Overall framework].  The landmark of
 * chunk i is scored against the landmark of every strictly earlier chunk and the top-k are
 * kept, optionally after adding Gumbel noise [Notes, Key designs: causal retrieval; Gumbel
 * top-k].  Every token of the next chunk attends to each retrieved chunk with its own softmax,
 * and the k outputs are fused with a softmax of the retrieval scores, so the scores receive
 * gradients [Notes, Key designs: GCA; Background].  K/V are shared by all retrieval groups
 * [Notes, Key designs: GCA].
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major (last index fastest), in device memory, owned by the
 *     caller (the one exception: gca_fetch_chunks also reads its K/V sources from pinned host
 *     memory).  The library never allocates, frees or synchronises, keeps no state between
 *     calls, and enqueues all work on `stream` (a hipStream_t; NULL = the null stream).
 *     Calls that share a workspace must be ordered on one stream.
 *   - Floating tensors q, k, v, o, dout, dq, dk, dv, lq, lk use `problem->dtype`
 *     (bf16 or fp32).  idx is int32; score, lse and dscore are fp32.
 *   - Shapes (n_q = n_q_chunks, n_kv = n_kv_chunks, S = 64, d = d_head, dl = d_lmk):
 *       lq     [G, B, n_q,   dl]      query landmarks (one per retrieval row)
 *       lk     [G, B, n_kv,  dl]      key landmarks (one per history chunk)
 *       q, o, dout, dq  [G, B, H, n_q*S, d]
 *       k, v, dk, dv    [B, H, n_kv*S, d]      shared by all G groups
 *       idx, score, dscore [G, B, n_q, topk]
 *       lse    [G, B, H, n_q, topk, S]   (per query chunk and slot, the chunk's S tokens)
 *     Token-level decode: q, o [G, B, H, n_tokens, d].  Fetched chunks: k_out, v_out
 *     [B, H, G*n_q*topk*S, d].  Sliding-window attention (one sequence of L = n_q*S tokens per
 *     batch row and head): q, k, v, o, dout, dq, dk, dv [B, H, L, d] and lse [B, H, L].
 *   - Row r of a retrieval is global chunk i = q_chunk_base + r; its candidates are the
 *     chunks j < min(i, n_kv).  The valid slots of a row name distinct chunks (gca_retrieve
 *     guarantees it); idx rows given to gca_backward or gca_landmark_backward must keep to that,
 *     since their key-side sums count a row once per chunk.  Query chunk t uses row t - shift (shift = 1 in training, where
 *     the landmark of chunk t-1 retrieves for chunk t; shift = 0 when the caller passes the
 *     landmark of the chunk being generated).  Query chunks whose row is missing or has no
 *     valid slot get o = 0, lse = -inf, dq = 0.
 *   - Pointers to the floating tensors, lq, lk and the lse of gca_forward / gca_backward must be
 *     16-byte aligned; idx, score, dscore and the lse of gca_sw_forward / gca_sw_backward
 *     ([B, H, L] fp32) 4-byte aligned.  Otherwise GCA_ERR_MISALIGNED.
 *   - Every call validates all arguments on the host before touching the GPU and enqueues
 *     nothing when it returns an error.  A launch failure returns GCA_ERR_HIP; the HIP code
 *     is then available from gca_last_hip_error() (per calling thread).  Faults inside
 *     kernels surface at the caller's next synchronisation.
 *   - Outputs are fully overwritten (gca_fetch_chunks writes only the tiles of slots in range);
 *     inputs are read only.  Results are bit-identical from run to run (no floating-point
 *     atomics anywhere).
 *   - gca_retrieve and gca_forward with n_q_chunks = 0 validate and return GCA_OK without
 *     launching anything; gca_backward with n_q_chunks = 0 still writes zero dk and dv.
 */
#ifndef GCA_H
#define GCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GCA_OK = 0,
  GCA_ERR_INVALID_ARGUMENT = 1,    /* null pointer, negative size, bad enum, non-finite scale */
  GCA_ERR_UNSUPPORTED = 2,         /* S, d_head, d_lmk other than 64, topk > 16, size limits  */
  GCA_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes below gca_workspace_size()                     */
  GCA_ERR_MISALIGNED = 4,          /* a tensor pointer breaks the alignment rule above        */
  GCA_ERR_HIP = 5                  /* a HIP launch failed; see gca_last_hip_error()           */
} gca_status;

typedef enum { GCA_BF16 = 0, GCA_F32 = 1 } gca_dtype;

typedef enum {
  GCA_OP_RETRIEVE = 0,
  GCA_OP_FORWARD = 1,
  GCA_OP_BACKWARD = 2,
  GCA_OP_LANDMARK_BACKWARD = 3,
  GCA_OP_SW_BACKWARD = 4,
  GCA_OP_FUSED_BACKWARD = 5
} gca_op;

/* Sizes and options of one problem.  Fields are read, never written. */
typedef struct {
  int32_t B;              /* batch                                            >= 1 */
  int32_t G;              /* retrieval groups (independent landmark sets)     >= 1 */
  int32_t H;              /* attention heads                                  >= 1 */
  int32_t S;              /* chunk length: must be 64                              */
  int64_t n_q_chunks;     /* retrieval rows / query chunks in this call       >= 0 */
  int64_t q_chunk_base;   /* global chunk index of row 0                      >= 0 */
  int64_t n_kv_chunks;    /* chunks of K, V and key landmarks present         >= 0 */
  int32_t d_head;         /* must be 64                                            */
  int32_t d_lmk;          /* landmark dimension: must be 64                        */
  int32_t topk;           /* K, 1..16                                              */
  int32_t dtype;          /* gca_dtype of the floating tensors                     */
  float attn_scale;       /* z = attn_scale * <q, k>; usually 1/sqrt(d_head)       */
  float score_scale;      /* s = score_scale * <lq, lk>; usually 1/sqrt(d_lmk)     */
  int32_t use_gumbel;     /* 0 or 1: perturb the scores before the top-k           */
  int32_t shift;          /* 0 or 1: query chunk t uses retrieval row t - shift    */
  uint64_t seed;          /* Philox key word 0 for the Gumbel noise                */
  float gumbel_tau;       /* noise scale tau >= 0 (1 = standard Gumbel top-k)      */
  int32_t reserved;       /* must be 0                                             */
} gca_problem;

/*
 * Device workspace (bytes) that `op` needs for `problem`; 0 means ws may be NULL.
 * Pure host function.  Errors: GCA_ERR_INVALID_ARGUMENT (bad op, NULL pointers, invalid
 * problem), GCA_ERR_UNSUPPORTED.
 */
gca_status gca_workspace_size(int op, const gca_problem* problem, size_t* bytes);

/*
 * Causal retrieval [Notes, Key designs: causal retrieval; Gumbel top-k].
 * For every (g, b, row r) with i = q_chunk_base + r:
 *   s_ij = fl32(fl32(sum_{d=0}^{dl-1} lq[i,d] * lk[j,d]) * score_scale), the sum taken exactly
 *          as a float64 sequential sum over d (products of bf16/fp32 values are exact), -0
 *          canonicalised to +0;
 *   r_ij = s_ij, or with use_gumbel r_ij = fl32(s_ij + fl32(tau * g_ij)) where
 *          g_ij = fl32(-ln_s(-ln_s(u))), u = ((x >> 12) + 1/2) 2^-52, x = word 0 of
 *          Philox4x64-10(key = (seed, 0), counter = (j, i, (g << 32) | b, 0)) and ln_s the
 *          fixed atanh-series logarithm (float64, no fused multiply-add);
 *   the K candidates j < min(i, n_kv) with the largest r (ties toward lower j) are written to
 *   idx[g,b,r,:] in order (r descending, j ascending) with their clean s_ij in score[g,b,r,:];
 *   unused slots get idx = -1 and score = -inf.
 * lq, lk: inputs (see shapes).  idx, score: outputs.  ws: >= gca_workspace_size(RETRIEVE)
 * (partial top-k lists of rows longer than one block of the scan; contents need no setup).
 */
gca_status gca_retrieve(const gca_problem* problem, const void* lq, const void* lk,
                        int32_t* idx, float* score, void* ws, size_t ws_bytes, void* stream);

/*
 * gca_retrieve without a workspace argument, for callers that cannot allocate device memory:
 * code under HIP stream capture, serving loops that must not call hipMalloc, harnesses that
 * forbid allocation.  Same arguments (minus ws), same results bit for bit, same validation.
 * Rows longer than one scan block keep their partial top-k lists in a device array inside the
 * library (512 KiB per GPU, one copy per GPU, resident until the process ends; located with
 * hipGetSymbolAddress on the first call on each device) instead of a caller workspace.  Nothing
 * in it needs setup.  Every call on one GPU shares that array: calls that overlap on one GPU
 * (several streams or host threads) race and must be ordered on one stream.  Never allocates.
 * Errors: those of gca_retrieve; GCA_ERR_UNSUPPORTED if the problem needs more scratch than the
 * array holds (gca_workspace_size(RETRIEVE) > 512 KiB; the scan's grid cap keeps every problem
 * within 384 KiB); GCA_ERR_HIP if the device or the array's address cannot be obtained.
 */
gca_status gca_retrieve_static(const gca_problem* problem, const void* lq, const void* lk,
                               int32_t* idx, float* score, void* stream);

/*
 * GCA forward [Notes, Key designs: GCA].  For query chunk t with row = t - shift, valid slots
 * k (0 <= idx[k] < n_kv; gca_retrieve only produces j < min(i, n_kv)), w = softmax over the
 * valid slots of score[g,b,row,:]:
 *   O_{t,k} = softmax_u(attn_scale * q_t . K_u) V_u over the 64 keys u of chunk idx[k],
 *   o_t     = sum_k w_k O_{t,k},   lse[t,k] = logsumexp_u(attn_scale * q_t . K_u) (-inf if
 *   slot k is invalid).
 * q, k, v, idx, score: inputs; o: output; lse: output, or NULL when no backward will follow.
 * Arithmetic: bf16 inputs use bf16 matrix cores with fp32 accumulation and fp32 softmax; fp32
 * inputs use fp32 matrix cores.  ws: >= gca_workspace_size(FORWARD) (currently 0).
 */
gca_status gca_forward(const gca_problem* problem, const void* q, const void* k, const void* v,
                       const int32_t* idx, const float* score, void* o, float* lse, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * GCA backward: gradients of sum(dout * o) with the retrieved idx held fixed [Notes,
 * Background: the retrieval scores act as weights, so the loss gradient reaches them].
 *   e_{t,k}  = <dout_t, O_{t,k}>,  dw_k = sum over the chunk's 64 tokens and all heads of e,
 *   dscore_k = w_k (dw_k - sum_k' w_k' dw_k')  (0 on invalid slots and unused rows),
 *   dz_u     = w_k a_u (<dout_t, V_u> - e_{t,k}),
 *   dq_t     = attn_scale sum_{k,u} dz_u K_u,
 *   dk_u     = attn_scale sum dz_u q_t,   dv_u = sum w_k a_u dout_t, both summed over all
 *              groups and every (token, slot) that retrieved the chunk of u (zero if none).
 * Slots count exactly as in gca_forward: every slot with 0 <= idx < n_kv, whether or not
 * idx < q_chunk_base + row (so idx built by the caller, e.g. the compact buffers of
 * gca_fetch_chunks, is differentiated as the forward used it).
 * q, k, v, idx, score, lse (from gca_forward), dout: inputs; dq, dk, dv, dscore: outputs.
 * dk and dv are accumulated in fp32 in a fixed order and rounded once to dtype.  A chunk
 * retrieved by more than 128 (group, row) entries has its sums split into segments of 64
 * entries, each summed by its own workgroup; the segments' fp32 partials are then added in
 * segment order, so the result is the same on every run.
 * ws: >= gca_workspace_size(BACKWARD); it holds, among others, an inverse retrieval index of
 * B * n_kv * G * n_q int32 entries and room for the split chunks' partials (up to
 * B * (ceil(L / 64) + floor(L / 129)) segments of H * 32 KiB, L = G * n_q * topk).  Contents
 * need no setup.
 */
gca_status gca_backward(const gca_problem* problem, const void* q, const void* k, const void* v,
                        const int32_t* idx, const float* score, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, float* dscore, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * Sliding-window self-attention [Notes, Loss / training strategy: sliding-window self-attention
 * with W = 512 beside the top-k retrieval]: the local attention of the layers that also run GCA.
 * Token i of a sequence of L = 64 n_q_chunks tokens attends to tokens max(0, i - W + 1) .. i
 * (itself included) under one softmax:
 *   o[b,h,i,:] = sum_j softmax_j(attn_scale q[b,h,i,:] . k[b,h,j,:]) v[b,h,j,:]
 *   lse[b,h,i] = log sum_j exp(attn_scale q[b,h,i,:] . k[b,h,j,:])   (natural log)
 * window = W: a positive multiple of 64 (a window longer than the sequence is causal attention).
 * q, k, v, o [B,H,L,64] (problem->dtype); lse [B,H,L] fp32, may be NULL (the backward needs it).  Requires G = 1 and n_kv_chunks = n_q_chunks; uses B, H, n_q_chunks,
 * attn_scale of problem.  No workspace.
 */
gca_status gca_sw_forward(const gca_problem* problem, int32_t window, const void* q, const void* k,
                          const void* v, void* o, float* lse, void* stream);

/*
 * Backward of gca_sw_forward: with P the window softmax, dP = dout v^T and D = <dout, o> per
 * token,
 *   dS = P (dP - D),  dq = attn_scale dS k,  dk = attn_scale dS^T q,  dv = P^T dout,
 * in fp32 over fixed orders without atomics (bit-identical from run to run), rounded once to dtype.
 * q, k, v, o and lse (from gca_sw_forward), dout: inputs [B,H,L,64] (lse [B,H,L] fp32); dq, dk, dv:
 * outputs like q.  ws: >= gca_workspace_size(SW_BACKWARD) = B*H*L*8 bytes (per token
 * -lse log2 e and -D; contents need no setup).  Same problem rules as gca_sw_forward.
 */
gca_status gca_sw_backward(const gca_problem* problem, int32_t window, const void* q, const void* k,
                           const void* v, const void* o, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream);

/*
 * Fused layer attention [Notes, Loss / training strategy: the layers that run GCA also run
 * sliding-window self-attention, W = 512, beside the top-k retrieval].  Reading taken: both read
 * the layer's queries and their outputs are summed, with one retrieval group in the layer:
 *   o = SW(q, k_sw, v_sw; window) + GCA(q, k, v, idx, score)
 * SW as gca_sw_forward (token i attends to keys max(0, i - window + 1) .. i of k_sw, v_sw), GCA as
 * gca_forward with G = 1.  One kernel per query tile computes both on one Q tile and stores the
 * sum once.
 * problem: G must be 1; uses B, H, n_q_chunks (L = 64 n_q_chunks), n_kv_chunks, topk, shift,
 * dtype, attn_scale.  window: positive multiple of 64.
 * q, o [B, H, L, 64] (the same memory as [1, B, H, L, 64]); k_sw, v_sw [B, H, L, 64] (the layer's
 * own keys and values); k, v [B, H, n_kv * 64, 64] (the history GCA retrieves from; may alias
 * k_sw, v_sw); idx, score [1, B, n_q, K]: inputs.  o: output.  lse_sw [B, H, L] fp32 (the window's
 * natural log-sum-exp) and lse [1, B, H, n_q, K, 64] fp32 (as gca_forward): outputs, each may be
 * NULL (the backward needs both).  No workspace.  Alignment: lse_sw 4 bytes, the rest as above.
 */
gca_status gca_fused_forward(const gca_problem* problem, int32_t window, const void* q, const void* k_sw,
                             const void* v_sw, const void* k, const void* v, const int32_t* idx,
                             const float* score, void* o, float* lse_sw, float* lse, void* stream);

/*
 * Backward of gca_fused_forward, with dout the gradient of o:
 *   dq = dq_sw + dq_gca (one pass per query tile), dk_sw, dv_sw (the window's keys and values,
 *   as gca_sw_backward), dk, dv, dscore (the history's, as gca_backward with G = 1).
 * The window's D = <dout, o_sw> is taken as <dout, o> - sum_k w_k e_k with the e_k of the GCA
 * slots (o_gca = sum_k w_k O_k), so only the fused output o is needed.
 * Inputs: q, k_sw, v_sw, k, v, idx, score, o, lse_sw, lse (from gca_fused_forward), dout.
 * Outputs (overwritten): dq [B, H, L, 64], dk_sw, dv_sw [B, H, L, 64], dk, dv [B, H, n_kv*64, 64],
 * dscore [1, B, n_q, K].  k_sw and k are separate tensors here even when the caller aliases them:
 * then the gradient of that tensor is dk_sw + dk.  ws: >= gca_workspace_size(FUSED_BACKWARD)
 * (the GCA backward's workspace plus B * H * L * 8 bytes; contents need no setup).
 */
gca_status gca_fused_backward(const gca_problem* problem, int32_t window, const void* q, const void* k_sw,
                              const void* v_sw, const void* k, const void* v, const int32_t* idx,
                              const float* score, const void* o, const float* lse_sw, const float* lse,
                              const void* dout, void* dq, void* dk_sw, void* dv_sw, void* dk, void* dv,
                              float* dscore, void* ws, size_t ws_bytes, void* stream);

/*
 * Token-level decode [Notes, Key designs: GCA; Key designs: memory-offload inference]: while the
 * tokens of a query chunk are generated one at a time, every new token attends to the chunks
 * retrieved once for the chunk (one retrieval serves its S tokens).  For the call's single query
 * chunk (n_q_chunks must be 1; it uses retrieval row 0 - shift, so shift = 1 gives zeros) and its
 * first n_tokens tokens (1 <= n_tokens <= 64), o equals the first n_tokens rows of gca_forward's
 * output for that chunk:
 *   o[g,b,h,u,:] = sum_k w_k softmax_j(attn_scale q[g,b,h,u,:] . k_jk[j,:]) v_jk
 * with w the softmax over the valid slots of score[g,b,0,:].
 * q, o [G,B,H,n_tokens,64] (problem->dtype); k, v [B,H,n_kv,64,64]; idx, score [G,B,1,K]; all
 * device memory (k, v may also be the compact buffers of gca_fetch_chunks, with n_kv = G * K).
 * Arithmetic in fp32; no workspace.  Errors: GCA_ERR_INVALID_ARGUMENT if n_q_chunks != 1 or
 * n_tokens is out of range.
 */
gca_status gca_decode_tokens(const gca_problem* problem, int32_t n_tokens, const void* q,
                             const void* k, const void* v, const int32_t* idx, const float* score,
                             void* o, void* stream);

/*
 * Fetch of retrieved chunks [Notes, Key designs: memory-offload inference]: the K/V of past
 * chunks may be kept in host memory, and the chunks a retrieval selects are loaded back to the
 * device before the next chunk attends to them.  For every retrieval slot (g, b, r, k) whose
 * chunk j = idx[g,b,r,k] satisfies 0 <= j < n_kv, and every head h, the tiles k[b,h,j] and
 * v[b,h,j] are copied to k_out[b,h,c] and v_out[b,h,c] with c = (g * n_q + r) * K + k, and
 * idx_out[g,b,r,k] = c; idx_out is -1 for the other slots, whose output tiles are left as they
 * were.  gca_forward over (k_out, v_out, idx_out) with n_kv_chunks = G * n_q * K then computes
 * exactly what it computes over (k, v, idx).
 * k, v [B,H,n_kv,64,64] (problem->dtype): device memory, or pinned host memory from hipHostMalloc
 * (read through its device mapping, so every byte crosses the host link); pageable host memory
 * is refused with GCA_ERR_INVALID_ARGUMENT.  idx [G,B,n_q,K]: device input.  k_out, v_out
 * [B,H,G*n_q*K,64,64] and idx_out [G,B,n_q,K]: device outputs.
 * Uses n_q_chunks, n_kv_chunks, B, G, H, topk, dtype of problem.
 */
gca_status gca_fetch_chunks(const gca_problem* problem, const int32_t* idx, const void* k,
                            const void* v, void* k_out, void* v_out, int32_t* idx_out,
                            void* stream);

/*
 * Landmark gradients [Notes, Key designs: GCA; Key designs: causal retrieval]: the scores weight
 * the fused outputs, so the loss differentiates them, and a score relates the landmark of chunk i
 * to the landmark of an earlier chunk j; this carries d(score) on to both landmarks.  With
 * s_ij = score_scale <lq_i, lk_j> (the float32 roundings of the canonical score carry no
 * gradient) and the retrieved indices held fixed:
 *   dlq[g,b,r,:] = score_scale * sum over slots k of dscore[g,b,r,k] * lk[g,b,idx[g,b,r,k],:]
 *   dlk[g,b,j,:] = score_scale * sum over the (r, k) with idx[g,b,r,k] = j, in (r, k) order, of
 *                  dscore[g,b,r,k] * lq[g,b,r,:]
 * Slots count when 0 <= idx < min(q_chunk_base + r, n_kv) (every candidate gca_retrieve can
 * produce; pass dscore = 0 for slots that must not contribute).  Sums run in a fixed order,
 * without atomics, accumulated in fp32 and rounded once to the problem dtype: results are
 * bit-identical from run to run.
 * lq [G,B,n_q,dl], lk [G,B,n_kv,dl], idx, dscore [G,B,n_q,K]: inputs; dlq (like lq) and dlk
 * (like lk): outputs, fully overwritten (zero rows for chunks no slot selected).  dscore is fp32
 * (as gca_backward writes it); lq, lk, dlq, dlk use problem->dtype.  ws: >=
 * gca_workspace_size(LANDMARK_BACKWARD) (an inverse retrieval index; contents need no setup).
 * Uses only n_q_chunks, n_kv_chunks, q_chunk_base, B, G, topk, dtype, score_scale of problem.
 */
gca_status gca_landmark_backward(const gca_problem* problem, const void* lq, const void* lk,
                                 const int32_t* idx, const float* dscore, void* dlq, void* dlk,
                                 void* ws, size_t ws_bytes, void* stream);

/* Static English text for a status code ("unknown status" for values outside the enum). */
const char* gca_status_string(gca_status status);

/* hipError_t value of the last failed HIP call made by this thread inside the library
 * (0 if none). */
int gca_last_hip_error(void);

/*
 * Kernel timing, for measurement tools.  While enabled (on != 0), every kernel the library
 * launches from the calling thread is bracketed by HIP events recorded on its stream.
 * gca_profile_collect() waits for the recorded events, writes up to `cap` entries (static
 * kernel names, summed milliseconds and launch counts) and clears the record; *n receives the
 * number of distinct kernels.  Disabled by default; costs nothing when disabled.
 */
gca_status gca_profile_enable(int on);
gca_status gca_profile_collect(int cap, const char** names, double* total_ms, int64_t* counts,
                               int* n);

#ifdef __cplusplus
}
#endif

#endif /* GCA_H */
