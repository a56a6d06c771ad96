/*
 * hstu_attn.h -- C ABI of the MI355X (gfx950) jagged HSTU attention library.
 *
 * What it computes. HSTU's pointwise attention, named in the Abstract of
 * "Actions Speak Louder than Words: Trillion-Parameter Sequential Transducers
 * for Generative Recommendations" and, as target-aware full causal
 * self-attention with M-FALCON candidate scoring, in the Generative
 * Recommenders README ("HSTU Ultra attention benchmark"). The pages print no
 * equations; the definition implemented here, per jagged sequence b of length
 * L (tokens seq_offsets[b] .. seq_offsets[b+1]-1), head h and in-sequence
 * indices 0 <= i, j < L, is:
 *
 *   hist    = L - num_targets[b]            (num_targets NULL: hist = L)
 *   M[i,j]  = (j <= i && j < hist) || j == i          causal + candidate mask
 *   p_i     = min(i, hist)
 *   bp(i,j) = clamp(j - p_i, -(max_len-1), max_len-1) + (max_len-1)
 *   bt(i,j) = min(bitlen(|ts_i - ts_j| + 1) - 1, n_time_buckets - 1)
 *   S[i,j]  = sum_d Q[i,h,d] K[j,h,d] + rab_pos[hr,bp] + rab_time[hr,bt]
 *   A[i,h]  = (1/L) sum_j M[i,j] SiLU(S[i,j]) V[j,h],   SiLU(x) = x/(1+e^-x)
 *   O[i,h]  = A[i,h] * U[i,h]        (u == NULL: O = A)
 *
 * hr = 0 when rab_heads == 1 (one table shared by all heads), else hr = h.
 * The backward returns dQ, dK, dV, dU = dO*A and the rab-table gradients
 * (sums of dS = M * (dO*U . V_j) * SiLU'(S) / L over the pairs reading each
 * entry).
 *
 * Conventions for every call.
 *  - Pointers marked (device) are device memory; (host) are host memory.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream). Nothing synchronises with the host.
 *  - The caller allocates and owns every buffer, including the workspace;
 *    the library allocates nothing and keeps no state between calls (apart
 *    from the optional per-launch timing of hstu_profile_begin/end, off by
 *    default), so calls are reentrant. Calls that share a workspace must not
 *    overlap.
 *  - Every call validates its host-side arguments before it launches
 *    anything; on any error it returns a negative status without writing any
 *    output and hstu_last_error() describes the problem. Device-side data
 *    (offsets, timestamps) is not validated: offsets must be non-decreasing
 *    from 0 to total_tokens and 0 <= num_targets[b] <= L_b.
 *  - Token tensors are row-major [T, H, D]: element (t, h, d) is at
 *    t*stride + h*D + d, with `stride` (elements, >= H*D, <= 2^22; larger
 *    strides return HSTU_EUNSUPPORTED) given per input.
 *    Outputs and gradients are dense [T, H, D] (stride H*D).
 */
#ifndef HSTU_ATTN_H
#define HSTU_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define HSTU_API __attribute__((visibility("default")))
#else
#define HSTU_API
#endif

typedef enum {
  HSTU_OK = 0,
  HSTU_EINVAL = -1,        /* an argument is invalid (null, negative, bad stride) */
  HSTU_EUNSUPPORTED = -2,  /* valid but not supported by these kernels        */
  HSTU_EWORKSPACE = -3,    /* workspace missing or smaller than required       */
  HSTU_EHIP = -4           /* a HIP runtime call or kernel launch failed       */
} hstu_status;

typedef enum {
  HSTU_DTYPE_BF16 = 0,     /* bfloat16 storage, fp32 accumulation (MFMA)       */
  HSTU_DTYPE_FP32 = 1      /* float32 storage and arithmetic                   */
} hstu_dtype;

/* Shape and layout of one jagged attention call (host memory). */
typedef struct {
  int32_t batch;           /* B >= 0 sequences                                   */
  int32_t heads;           /* H >= 1                                             */
  int32_t d_qk;            /* head dim of Q, K: 32, 64 or 128                  */
  int32_t d_v;             /* head dim of V, U, O: must equal d_qk               */
  int32_t max_len;         /* >= 1; rab_pos holds 2*max_len-1 buckets            */
  int32_t n_time_buckets;  /* entries per rab_time row (0: no time bias), <= 1024 */
  int32_t rab_heads;       /* rows of each rab table: 1 (shared) or heads        */
  int32_t dtype;           /* hstu_dtype of Q,K,V,U,O,dO,dQ,dK,dV,dU             */
  int64_t total_tokens;    /* T = seq_offsets[B], 0 <= T < 2^31                  */
  int64_t stride_q, stride_k, stride_v, stride_u;  /* elements between tokens   */
  int32_t deterministic;   /* 0 or 1; backward only: 1 sums the rab gradients in
                              a fixed order (bitwise repeatable, see hstu_attn_bwd) */
} hstu_attn_desc;

/*
 * Bytes of workspace hstu_attn_fwd / hstu_attn_bwd need for this shape.
 *
 * The backward has two figures. hstu_attn_bwd_workspace_size_min is the
 * least it accepts: O(T * H * D) bytes (the dA' tensor, per-sequence
 * metadata and work lists), plus, when desc->deterministic is set, the
 * rab-gradient partials (768 bytes per (128-key block, 64-query tile) pair
 * and one row of n_time_buckets floats per (128-key block, head), sized like
 * the tiles below, at most 2 GiB).
 * hstu_attn_bwd_workspace_size is the preferred figure: for bf16 it adds
 * room for the dS tiles the key-block pass hands to the dQ pass, 16 KB per
 * (128-key block, 64-query tile) pair, sized for sequences no longer than
 * max_len: heads * (ceil(min(max_len, T) / 128) + 1) * (T / 128 + batch)
 * tiles, at most 4 GiB (about 1.5 GB for 8 sequences of up to 8192 rows, 4
 * heads). That room is O(sum of L^2) bytes.
 * hstu_attn_bwd uses the dS export when workspace_bytes reaches the preferred
 * figure, for the leading sequences whose tiles fit that room (all of them
 * when no sequence is longer than max_len and the 4 GiB cap is not reached);
 * for the others, and without the room, it computes dQ by recomputing dS per
 * query block (the same results; measured about 1.7x the dQ time at 8
 * sequences of 4096..8192 rows, 4 heads, head dim 128).
 * hstu_attn_bwd_report tells how many sequences took the export.
 */
HSTU_API hstu_status hstu_attn_fwd_workspace_size(const hstu_attn_desc* desc, size_t* bytes);
HSTU_API hstu_status hstu_attn_bwd_workspace_size(const hstu_attn_desc* desc, size_t* bytes);
HSTU_API hstu_status hstu_attn_bwd_workspace_size_min(const hstu_attn_desc* desc, size_t* bytes);

/*
 * Forward.
 *  seq_offsets  (device) int64 [B+1]
 *  num_targets  (device) int64 [B] or NULL (no candidates)
 *  timestamps   (device) int64 [T]; required when n_time_buckets > 0
 *  rab_pos      (device) fp32 [rab_heads, 2*max_len-1] or NULL (no position bias)
 *  rab_time     (device) fp32 [rab_heads, n_time_buckets] or NULL
 *  q, k         (device) dtype [T, H, d_qk], row strides stride_q / stride_k
 *  v, u         (device) dtype [T, H, d_v]; u NULL = no gate (O = A)
 *  o            (device) dtype [T, H, d_v], written
 *  a_saved      (device) fp32 [T, H, d_v] or NULL; receives A (needed by the
 *               backward when u != NULL, and by the layer's LayerNorm)
 *  workspace    (device) >= hstu_attn_fwd_workspace_size bytes, 256-aligned
 */
HSTU_API hstu_status hstu_attn_fwd(const hstu_attn_desc* desc, const int64_t* seq_offsets,
                          const int64_t* num_targets, const int64_t* timestamps,
                          const float* rab_pos, const float* rab_time,
                          const void* q, const void* k, const void* v, const void* u,
                          void* o, float* a_saved,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Arguments, results and errors as
 * in hstu_attn_fwd, without the workspace: the call uses a fixed 16 MiB
 * device array inside the library (enough for about 3.5 million tokens),
 * which each GPU the library runs on holds until the process ends. A shape
 * whose hstu_attn_fwd_workspace_size exceeds 16 MiB returns HSTU_EWORKSPACE
 * before any launch. All calls on one GPU share that array: calls on one GPU
 * that overlap in time (other streams or host threads) race and must not be
 * made. The first call on each device looks up the array's device address
 * (the device must be current).
 */
HSTU_API hstu_status hstu_attn_fwd_noalloc(const hstu_attn_desc* desc, const int64_t* seq_offsets,
                                           const int64_t* num_targets, const int64_t* timestamps,
                                           const float* rab_pos, const float* rab_time,
                                           const void* q, const void* k, const void* v,
                                           const void* u, void* o, float* a_saved, void* stream);

/*
 * Candidate scoring against a cached history (M-FALCON-style micro-batched
 * inference; the pages name M-FALCON for inference in the abstract of
 * "Actions Speak Louder than Words" and in the Generative Recommenders
 * README, whose "HSTU Ultra attention benchmark" defines the target-aware
 * mask used here and notes that cached incremental decoding is not yet
 * included there).
 *
 * Sequence b has h_b history rows, whose keys and values were computed once
 * (k_hist, v_hist), and n_b candidates, scored here in micro-batches: this
 * call takes m_b of them, the candidates cand_first[b] .. cand_first[b] +
 * m_b - 1. Each candidate attends to every history row and to itself. The
 * outputs equal those candidates' rows of hstu_attn_fwd on the whole
 * sequence [history, all n_b candidates] with num_targets = n_b: the same
 * normalisation 1 / (h_b + n_b), position buckets and time buckets.
 *
 *  desc          batch B; total_tokens = candidate rows of this call (sum of
 *                m_b); stride_q, stride_k, stride_v, stride_u as in
 *                hstu_attn_fwd, for q, k, v, u
 *  cand_offsets  (device) int64 [B+1]: sequence b's candidate rows of this
 *                call are cand_offsets[b] .. cand_offsets[b+1] - 1
 *  cand_first    (device) int64 [B]: index of the first of them among the
 *                sequence's n_b candidates (values < 0 count as 0)
 *  n_cands       (device) int64 [B]: n_b (at least cand_first[b] + m_b; a
 *                smaller value counts as cand_first[b] + m_b)
 *  hist_offsets  (device) int64 [B+1]: sequence b's history rows in
 *                k_hist / v_hist
 *  hist_tokens   rows of k_hist / v_hist; total_tokens + hist_tokens < 2^31
 *  ts_hist, ts_cand (device) int64 timestamps of the history rows and of
 *                this call's candidate rows; required when rab_time != NULL
 *  rab_pos, rab_time as in hstu_attn_fwd
 *  q, k, v, u    (device) dtype [total_tokens, H, d]: the candidates' rows
 *  k_hist, v_hist (device) dtype [hist_tokens, H, d], row strides
 *                stride_kh, stride_vh (>= H * d, multiples of 16 bytes)
 *  o, a_saved    (device) [total_tokens, H, d_v]: the candidates' O (dtype)
 *                and A (fp32, or NULL), written
 *  workspace     (device) >= hstu_attn_fwd_cached_workspace_size bytes,
 *                256-aligned
 * Errors as in hstu_attn_fwd. Offsets that index outside the given tensors
 * are the caller's error and are not checked on the device.
 */
HSTU_API hstu_status hstu_attn_fwd_cached_workspace_size(const hstu_attn_desc* desc,
                                                          int64_t hist_tokens, size_t* bytes);
HSTU_API hstu_status hstu_attn_fwd_cached(const hstu_attn_desc* desc, const int64_t* cand_offsets,
                                          const int64_t* cand_first, const int64_t* n_cands,
                                          const int64_t* hist_offsets, int64_t hist_tokens,
                                          const int64_t* ts_hist, const int64_t* ts_cand,
                                          const float* rab_pos, const float* rab_time,
                                          const void* q, const void* k, const void* v,
                                          const void* u, const void* k_hist, const void* v_hist,
                                          int64_t stride_kh, int64_t stride_vh, void* o,
                                          float* a_saved, void* workspace,
                                          size_t workspace_bytes, void* stream);

/*
 * Backward. Inputs as in hstu_attn_fwd, plus
 *  a_saved      (device) fp32 [T, H, d_v] from the forward; required if u != NULL
 *  d_o          (device) dtype [T, H, d_v] dense
 * Outputs (device, dense, all overwritten, never accumulated into):
 *  dq, dk       dtype [T, H, d_qk]
 *  dv           dtype [T, H, d_v]
 *  du           dtype [T, H, d_v]; required iff u != NULL
 *  d_rab_pos    fp32 [rab_heads, 2*max_len-1]; required iff rab_pos != NULL
 *  d_rab_time   fp32 [rab_heads, n_time_buckets]; required iff rab_time != NULL
 *  workspace    (device) >= hstu_attn_bwd_workspace_size_min bytes, 256-aligned
 * Reductions. dQ, dK, dV and dU are each written once by one workgroup, in a
 * fixed order of summation: they repeat bit for bit between runs. The rab
 * gradients are sums over many workgroups: with desc->deterministic = 0 each
 * workgroup adds its partial sums with floating-point atomics, so their last
 * bits may differ between runs; with desc->deterministic = 1 the partial
 * sums go to the workspace and one more kernel adds them in a fixed order,
 * so they repeat bit for bit (a batch whose tiles exceed the partials' room,
 * i.e. with sequences longer than max_len, falls back to the atomics;
 * hstu_attn_bwd_report tells).
 */
HSTU_API hstu_status hstu_attn_bwd(const hstu_attn_desc* desc, const int64_t* seq_offsets,
                          const int64_t* num_targets, const int64_t* timestamps,
                          const float* rab_pos, const float* rab_time,
                          const void* q, const void* k, const void* v, const void* u,
                          const float* a_saved, const void* d_o,
                          void* dq, void* dk, void* dv, void* du,
                          float* d_rab_pos, float* d_rab_time,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * What the last hstu_attn_bwd on this workspace did (for checking and
 * reporting; it waits for `stream`, then reads two flags the call left in the
 * workspace). desc, workspace and workspace_bytes as passed to that call.
 *  dq_from_ds         1: every sequence's dQ came from the exported dS
 *                     tiles; 0: at least one sequence's dQ came from the
 *                     pass that recomputes dS
 *  rab_deterministic  1: the rab gradients were summed in a fixed order
 *  ds_sequences       how many leading sequences (0 .. batch) took the dS
 *                     export: the tiles of sequences 0 .. n-1 fit the room
 *                     the workspace holds and the rest did not (sequences
 *                     longer than max_len, or a batch beyond the room's
 *                     4 GiB cap); 0 without room, or in fp32
 */
typedef struct {
  int32_t dq_from_ds;
  int32_t rab_deterministic;
  int32_t ds_sequences;
} hstu_attn_bwd_info;
HSTU_API hstu_status hstu_attn_bwd_report(const hstu_attn_desc* desc, const void* workspace,
                                          size_t workspace_bytes, hstu_attn_bwd_info* info,
                                          void* stream);

/*
 * rab bucket export (for checking and debugging): for every unmasked pair,
 * in sequence order, then query row i, then key j ascending, writes the
 * position bucket bp(i,j) and the time bucket bt(i,j) (the bucket
 * definitions at the top of this file, which the attention kernels apply to
 * each pair inside their tiles).
 *  pair_offsets (device) int64 [B+1]: first output slot of each sequence, as
 *               written by hstu_rab_pair_offsets; pair_offsets[B] = pairs
 *  bp_out       (device) uint16 [pairs] or NULL (requires max_len <= 32768)
 *  bt_out       (device) uint8 [pairs] or NULL (requires timestamps and
 *               1 <= n_time_buckets <= 256)
 * hstu_rab_pair_offsets writes pair_offsets (device, int64 [B+1]) from the
 * same seq_offsets / num_targets: sequence b has hist*(hist+1)/2 +
 * (L-hist)*(hist+1) unmasked pairs (hist = L - num_targets[b]). Only
 * desc->batch is read. A caller sizing bp_out / bt_out reads pair_offsets[B].
 */
HSTU_API hstu_status hstu_rab_pair_offsets(const hstu_attn_desc* desc, const int64_t* seq_offsets,
                                           const int64_t* num_targets, int64_t* pair_offsets,
                                           void* stream);
HSTU_API hstu_status hstu_rab_bucketize(const hstu_attn_desc* desc, const int64_t* seq_offsets,
                               const int64_t* num_targets, const int64_t* timestamps,
                               const int64_t* pair_offsets, uint16_t* bp_out,
                               uint8_t* bt_out, void* stream);

/*
 * HSTU layer pieces around the attention (Generative Recommenders README,
 * "HSTU Ultra attention benchmark": UVQK projection, attention, output
 * normalisation, gating and projection). bf16 storage, fp32 accumulation.
 *
 * hstu_linear: y[M,N] = act(x[M,K] @ w[K,N] + bias[N]); act = SiLU when
 *   apply_silu != 0, identity otherwise.
 *   x (device) bf16, row stride ldx >= K; w (device) bf16 [K, N] dense;
 *   bias (device) fp32 [N] or NULL; y (device) bf16 [M, N] dense.
 *   K must be a multiple of 32 and N a multiple of 128; M >= 0 any.
 */
HSTU_API hstu_status hstu_linear(int64_t M, int64_t K, int64_t N, const void* x, int64_t ldx,
                        const void* w, const float* bias, void* y, int32_t apply_silu,
                        void* stream);

/*
 * hstu_layernorm_gate: out[m, :] = LayerNorm(a[m, :]) * u[m, :] over N
 *   features, eps given, unit scale and zero shift.
 *   a (device) fp32 [M, N] dense; u (device) bf16, row stride ldu >= N;
 *   out (device) bf16 [M, N] dense. N must be a multiple of 64, <= 4096;
 *   ldu a multiple of 4.
 */
HSTU_API hstu_status hstu_layernorm_gate(int64_t M, int64_t N, const float* a, const void* u,
                                int64_t ldu, float eps, void* out, void* stream);

/*
 * FP8 projection path (Generative Recommenders README, "FP8 linear reference
 * and benchmark", and its description of the HSTU Ultra stack: row-wise E4M3
 * quantisation, FP8 addmm with weights quantised once and cached, and
 * normalisation steps fused with the quantisation of their output).
 * Codes are OCP E4M3FN bytes (sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; largest finite 448; 0x7F / 0xFF are NaN and never produced).
 * Row-wise quantisation: scale = amax(row) / 448 (1.0 for a row of zeros),
 * code = E4M3(x / scale) rounded to nearest even, both divisions IEEE fp32.
 * All pointers are device pointers; calls are asynchronous on `stream`.
 *
 * hstu_fp8_quantize_rows: x bf16 [M, K], row stride ldx (multiple of 8) ->
 *   q uint8 [M, K] dense, scale fp32 [M]. K a multiple of 16; x and q
 *   16-byte aligned.
 */
HSTU_API hstu_status hstu_fp8_quantize_rows(int64_t M, int64_t K, const void* x, int64_t ldx,
                                            void* q, float* scale, void* stream);

/*
 * hstu_fp8_prepare_weight: the weight w bf16 [K, N] (dense) of y = x w,
 *   quantised per output feature n -> q uint8 [N, K] (reduction index
 *   contiguous, the layout hstu_fp8_linear reads), scale fp32 [N]. A one-time
 *   step; the caller keeps q and scale. K a multiple of 16; q 16-byte aligned.
 */
HSTU_API hstu_status hstu_fp8_prepare_weight(int64_t K, int64_t N, const void* w, void* q,
                                             float* scale, void* stream);

/*
 * hstu_fp8_linear: y[m, n] = act(x_scale[m] * w_scale[n] * sum_k x[m, k] w[n, k]
 *   + bias[n]) with x, w the E4M3 values of xq uint8 [M, K] and wq uint8
 *   [N, K] (both dense, 16-byte aligned), fp32 accumulation; bias fp32 [N] or
 *   NULL; act = SiLU when apply_silu != 0; y bf16 [M, N] dense. K a multiple
 *   of 16; M, N >= 0 any.
 */
HSTU_API hstu_status hstu_fp8_linear(int64_t M, int64_t K, int64_t N, const void* xq,
                                     const float* x_scale, const void* wq, const float* w_scale,
                                     const float* bias, void* y, int32_t apply_silu, void* stream);

/*
 * hstu_layernorm_gate_fp8: row-wise quantisation of LayerNorm(a[m, :]) * u[m, :]
 *   (as hstu_layernorm_gate; u NULL: no gate, LayerNorm alone) -> q uint8
 *   [M, N] dense, scale fp32 [M]. a fp32 [M, N] dense; u bf16 with row stride
 *   ldu (multiple of 4). N a multiple of 64, <= 4096.
 */
HSTU_API hstu_status hstu_layernorm_gate_fp8(int64_t M, int64_t N, const float* a, const void* u,
                                             int64_t ldu, float eps, void* q, float* scale,
                                             void* stream);

/*
 * hstu_layer_bwd: gradients of one HSTU layer (the steps of hstu_linear,
 *   hstu_attn_fwd and hstu_layernorm_gate above, as the Generative
 *   Recommenders README's "HSTU Ultra attention benchmark" lists them:
 *   UVQK = SiLU(X W1 + b1), column blocks U, V, Q, K (head h at columns
 *   [h*head_dim, (h+1)*head_dim) of each block), A = attention(Q, K, V; no
 *   gate, no bias, num_targets candidates), Y = (LayerNorm(A) * U) W2 + b2)
 *   from dY, by the chain rule of those steps (the README gives no backward;
 *   this is the training of the layer it describes).
 *   M tokens in `batch` jagged sequences (seq_offsets, num_targets as in
 *   hstu_attn_fwd); d_model and heads*head_dim multiples of 128, head_dim in
 *   {32, 64, 128}; bf16 storage.
 *   x (device) bf16 [M, d_model]; w1 bf16 [d_model, 4*H*D]; b1 fp32 [4*H*D];
 *   w2 bf16 [H*D, d_model]; uvqk bf16 [M, 4*H*D] and a fp32 [M, H*D] as the
 *   forward produced them; eps the forward's LayerNorm epsilon; dy bf16
 *   [M, d_model]. Outputs (overwritten): dx bf16 [M, d_model]; dw1 fp32
 *   [d_model, 4*H*D]; db1 fp32 [4*H*D]; dw2 fp32 [H*D, d_model]; db2 fp32
 *   [d_model]. Pre = X W1 + b1 is recomputed (not saved by the forward).
 *   max_len: a bound on every sequence's length, or 0 for none. It sizes
 *   the attention backward's exported dS tiles (about
 *   H (ceil(max_len / 128) + 1) (M / 128 + batch) tiles of 16 KB, at most
 *   4 GiB); with 0 the attention backward recomputes dS for dQ instead
 *   (same results), and so it does for the sequences whose tiles do not fit
 *   the room after those of the sequences before them.
 *   workspace (device) >= hstu_layer_bwd_workspace_size bytes (same sizes
 *   and max_len), 256-aligned.
 *   Every reduction runs in a fixed order (no atomics: this attention has no
 *   bias tables), so results repeat exactly between runs.
 */
HSTU_API hstu_status hstu_layer_bwd_workspace_size(int64_t M, int32_t batch, int32_t d_model,
                                                   int32_t heads, int32_t head_dim, int32_t max_len,
                                                   size_t* bytes);
HSTU_API hstu_status hstu_layer_bwd(int64_t M, int32_t batch, int32_t d_model, int32_t heads,
                                    int32_t head_dim, int32_t max_len, const int64_t* seq_offsets,
                                    const int64_t* num_targets, const void* x, const void* w1,
                                    const float* b1, const void* w2, const void* uvqk,
                                    const float* a, float eps, const void* dy, void* dx,
                                    float* dw1, float* db1, float* dw2, float* db2,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Per-kernel timing for benchmarks (off by default). Between
 * hstu_profile_begin() and hstu_profile_end() every kernel launch of the
 * library is bracketed by two HIP events recorded on the caller's stream.
 * hstu_profile_end waits for the recorded events, writes for each kernel id
 * i < n the summed milliseconds total_ms[i] and launch count counts[i], and
 * turns recording off. Kernel ids: 0 .. hstu_kernel_count()-1, named by
 * hstu_kernel_name(id). Meant for one host thread at a time.
 */
HSTU_API hstu_status hstu_profile_begin(void);
HSTU_API hstu_status hstu_profile_end(int32_t n, double* total_ms, int32_t* counts);
HSTU_API const char* hstu_kernel_name(int32_t id);
HSTU_API int32_t hstu_kernel_count(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
HSTU_API const char* hstu_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_ATTN_H */
