// Host-side interface between the C ABI (api.hip) and the kernel sources.
#pragma once

#include "common.h"

namespace hstu {

// Everything one attention launch needs; filled and validated by api.hip.
struct AttnParams {
  int32_t B, H, D, max_len, n_time_buckets, rab_heads;
  int64_t T;
  int64_t sq, sk, sv, su;            // input row strides (elements)
  const int64_t* seq_offsets;
  const int64_t* num_targets;        // may be null
  const int64_t* timestamps;         // may be null
  const float* rab_pos;              // may be null
  const float* rab_time;             // may be null
  const void* q;
  const void* k;
  const void* v;
  const void* u;                     // may be null (no gate)
  // forward outputs
  void* o;
  float* a_saved;                    // may be null
  // backward inputs / outputs
  const float* a_in;
  const void* d_o;
  void* dq;
  void* dk;
  void* dv;
  void* du;
  float* d_rab_pos;
  float* d_rab_time;
  // workspace carve-up
  SeqInfo* seq;
  uint32_t* ts_rel;                  // [T] rebased timestamps
  WorkItem* items;                   // [max_items]
  WorkItem* items_q;                 // [max_items] query-block order (backward only)
  int32_t* n_items;                  // [1]: items of the work list
  int32_t* sched_scratch;            // schedule kernel scratch
  void* d_a;                         // [T, H, D] dtype: dO * U / L (backward)
  int64_t max_items;                 // T / 128 + B
  // candidate scoring against a cached history (null otherwise): T counts
  // history + candidate rows, seq_offsets / num_targets / timestamps are
  // unused by the kernels, which read the arrays below
  const SeqCand* cand;               // [B]
  const void* k_hist;
  const void* v_hist;
  int64_t skh, svh;                  // row strides of k_hist / v_hist
  // the history tiles of a candidate query block split over kv_splits
  // workgroups; with more than one, each writes its partial A to
  // part[split][row][head][d] (fp32, rows of q) and a finishing kernel sums
  // them into A and O
  int32_t kv_splits;
  int64_t m_rows;                    // candidate rows (rows of q)
  float* part;
  // Backward tile numbering: every (sequence, head, key block, 64-query
  // tile) a key-block workgroup visits has an index, each (sequence, head)'s
  // tiles from tile_base[b] + head * ds_seq_tiles(L), numbered row by row
  // (ds_row_start). The schedule kernel fills tile_base (when ds or det is
  // set) and blk_base (first key block of each sequence, when det is set).
  int64_t* tile_base;                // [B]
  int32_t* blk_base;                 // [B + 1]
  // dS export (bf16 backward; ds null: the dQ pass recomputes dS): storage
  // of ds_cap tiles. The schedule kernel sets *ds_on to the number of
  // leading sequences whose tiles fit (all B when the batch's do): those
  // export dS and take dq_ds_kernel, the rest take the recompute pass
  void* ds;
  int64_t ds_cap;
  int32_t* ds_on;
  // Deterministic rab gradients (det != 0): instead of adding into
  // d_rab_pos / d_rab_time with atomics, each key-block workgroup writes
  // its sums to part_pos (kPartW floats per tile: the tile's diagonal sums,
  // or its position-window sums when it holds candidate rows) and part_time
  // (n_time_buckets floats per (key block, head) slot, slot (blk_base[b] +
  // key block) * H + head); rab_reduce then sums them in a fixed order. The
  // schedule kernel sets *det_on to 1 when the batch's tiles fit part_cap,
  // else 0 (that call falls back to atomics).
  int32_t det;
  int32_t n_time_room;               // desc->n_time_buckets: sizes part_time whether
                                     // or not this call passes a time table
  float* part_pos;
  float* part_time;
  int64_t part_cap;
  int32_t* det_on;
  // rab_reduce's per-run sums: [rab_heads][kRedChunks][2 max_len - 1 +
  // n_time_room] floats (position buckets, then time buckets)
  float* part_red;
};

// Floats per tile of the position partials (>= the diagonals of a tile and
// the entries of a position window).
constexpr int kPartW = 192;

// Runs of units the deterministic reduction sums separately before adding
// the runs' sums in order.
constexpr int kRedChunks = 64;

// Records the message hstu_last_error() returns on this thread; returns status.
int set_error(int status, const char* fmt, ...);

// Workspace layout: returns total bytes and fills the pointers in p (when
// base != nullptr). ds_room: the bf16 backward's room for the dS export;
// p.det: the deterministic rab-gradient partials.
size_t carve_workspace(AttnParams& p, void* base, bool bwd, int elem_bytes, bool ds_room);

// Kernel identities for the optional per-launch timing (hstu_profile_*).
enum KernelId : int {
  kKPrep = 0, kKFwd, kKBwdPre, kKBwd, kKDq, kKFill, kKLinear, kKLayerNorm,
  kKBucketize, kKFp8Linear, kKFp8Quant, kKDqDs, kKRabReduce, kNumKernelIds
};
// Records a HIP event on `s` before / after a launch when timing is enabled.
void prof_before(int id, hipStream_t s);
void prof_after(int id, hipStream_t s);

hipError_t launch_bucketize(const AttnParams& p, const int64_t* pair_offsets, uint16_t* bp,
                            uint8_t* bt, hipStream_t s);
// out[b] = unmasked pairs of sequences 0..b-1; out[B] = all of them.
hipError_t launch_pair_offsets(const int64_t* seq_offsets, const int64_t* num_targets, int B,
                               int64_t* out, hipStream_t s);

template <typename T, int D> hipError_t launch_fwd(const AttnParams& p, hipStream_t s);
// Candidate scoring against a cached history (p.cand set): query blocks
// hold only candidate rows; launch_prep_cand builds p.seq, p.cand and the
// timestamp arrays of the joined row numbering first.
template <typename T, int D> hipError_t launch_fwd_cand(const AttnParams& p, hipStream_t s);
struct CandArgs {
  const int64_t* cand_offsets;
  const int64_t* cand_first;
  const int64_t* n_cands;
  const int64_t* hist_offsets;
  const int64_t* ts_hist;
  const int64_t* ts_cand;
  int64_t* ts_joined;                // [T] workspace (when timestamps are used)
  SeqCand* cand;                     // [B] workspace
};
hipError_t launch_prep_cand(const AttnParams& p, const CandArgs& c, hipStream_t s);
// p.T, p.B, p.H, p.D, p.m_rows and p.kv_splits set
size_t carve_workspace_cand(AttnParams& p, CandArgs& c, void* base);
// Splits of the history for a candidate call: enough workgroups to fill the
// chip, at least 8 history tiles (512 keys) per split on average.
int cand_kv_splits(int64_t m_rows, int64_t hist_rows, int B, int H);
// Backward: launch_bwd (fp32, bwd.hip) and launch_bwd_k16 (bf16,
// bwd_k16.hip) compute dK, dV and the rab gradients per key block;
// launch_dq computes dQ per query block (schedule mode 0, like the forward).
template <typename T, int D> hipError_t launch_bwd(const AttnParams& p, hipStream_t s);
template <int D> hipError_t launch_bwd_k16(const AttnParams& p, hipStream_t s);
template <typename T, int D> hipError_t launch_dq(const AttnParams& p, hipStream_t s);
// dQ from the exported dS tiles (dq_ds.hip) for the first *p.ds_on sequences.
template <int D> hipError_t launch_dq_ds(const AttnParams& p, hipStream_t s);
// Tiles of a batch of T tokens in B sequences of at most max_len rows each,
// H heads (an upper bound of the exact count), capped at max_tiles.
int64_t tile_capacity(int64_t T, int B, int H, int max_len, int64_t max_tiles);
// Capacity (tiles) of the dS export; 0 when the export is not used.
int64_t ds_capacity(int64_t T, int B, int H, int max_len);
// Fixed-order sums of the deterministic rab-gradient partials into
// d_rab_pos / d_rab_time (exits at once unless *p.det_on).
hipError_t launch_rab_reduce(const AttnParams& p, hipStream_t s);
// The forward's sequence prep and work list in one launch; the backward's
// sequence prep, work lists and dA' / dU pass in one launch.
hipError_t launch_fwd_prep(const AttnParams& p, hipStream_t s);
template <typename T> hipError_t launch_bwd_prep(const AttnParams& p, hipStream_t s);
hipError_t launch_fill_f32(float* x, int64_t n, float value, hipStream_t s);

hipError_t launch_linear(int64_t M, int64_t K, int64_t N, const void* x, int64_t ldx,
                         const void* w, const float* bias, void* y, int apply_silu,
                         hipStream_t s);
// Layer backward pieces (layer.hip).
// y[M,N] (bf16) = x[M,K] w^T, w stored [N][K] with row stride ldw.
hipError_t launch_linear_nt(int64_t M, int64_t K, int64_t N, const void* x, int64_t ldx,
                            const void* w, int64_t ldw, void* y, hipStream_t s);
// y[M,N] (fp32) = a^T b, a stored [K][M] (row stride lda), b stored [K][N]
// (row stride ldb); the reduction is split wgrad_splits(M, N, K) ways, the
// splits' partial sums kept in part ([splits][M][N] fp32) when more than one.
int wgrad_splits(int64_t M, int64_t N, int64_t K);
hipError_t launch_wgrad(int64_t M, int64_t N, int64_t K, const void* a, int64_t lda, const void* b,
                        int64_t ldb, float* y, float* part, hipStream_t s);
hipError_t launch_layernorm_gate_bwd(int64_t M, int64_t N, const float* a, const void* u,
                                     int64_t ldu, float eps, const void* dout, void* da, void* du,
                                     hipStream_t s);
// out[N] = column sums of x [M][N] (N a multiple of 8); part holds
// colsum_bands(M) x N floats of per-band sums.
int64_t colsum_bands(int64_t M);
hipError_t launch_colsum(int64_t M, int64_t N, const void* x, int64_t ldx, float* out, float* part,
                         hipStream_t s);
hipError_t launch_silu_bwd_uvqk(int64_t M, int64_t Mp, int64_t HD, const void* pre, const void* g0,
                                const void* g1, const void* g2, const void* g3, void* d_pre,
                                hipStream_t s);
hipError_t launch_layernorm_gate(int64_t M, int64_t N, const float* a, const void* u,
                                 int64_t ldu, float eps, void* out, hipStream_t s);

// FP8 (E4M3FN) projection pieces (fp8.hip).
hipError_t launch_fp8_quantize_rows(int64_t M, int64_t K, const void* x, int64_t ldx, void* q,
                                    float* scale, hipStream_t s);
hipError_t launch_fp8_prepare_weight(int64_t K, int64_t N, const void* w, void* q, float* scale,
                                     hipStream_t s);
hipError_t launch_fp8_linear(int64_t M, int64_t K, int64_t N, const void* xq, const float* x_scale,
                             const void* wq, const float* w_scale, const float* bias, void* y,
                             int apply_silu, hipStream_t s);
hipError_t launch_layernorm_gate_fp8(int64_t M, int64_t N, const float* a, const void* u,
                                     int64_t ldu, float eps, void* q, float* scale, hipStream_t s);

}  // namespace hstu
