// Fused forward of jagged HSTU pointwise attention for gfx950.
//
// One workgroup (4 waves) owns 128 query rows of one sequence and one head;
// wave w owns rows 32w..32w+31. It walks the key tiles (64 keys) that hold at
// least one unmasked pair for its rows, skipping the candidate-only tiles of
// M-FALCON-style batches. K and V tiles are staged row-major through LDS in
// two buffers so the global loads of tile t+1 overlap the math of tile t.
//
// Per tile and wave, with S^T = K Q^T computed as 32 x 32 MFMA blocks (keys on
// rows, the wave's queries on columns):
//   acc   = rab_pos window (read from LDS into the accumulator) + K Q^T
//   S'    = -log2(e) * (acc + rab_time[bt])         (one FMA per element)
//   p     = S' / (1 + 2^S')     = SiLU(S) / (-ln 2)
//   p     = 0 where masked (selection, never multiplication)
//   O^T  += V^T P^T            (V^T fragments by LDS transpose reads)
// and the epilogue applies the factor -ln(2)/L, stores A (fp32) and O = A*U.
// The accumulator layout of S^T is the B-operand layout of P^T, so P never
// leaves registers; the key order it implies is absorbed by the rows each
// transpose read starts from. The MFMAs of the next 32-key block are issued
// before the elementwise work of the current one so the two overlap.
#include "internal.h"

namespace hstu {

namespace {

// Row strides (elements) of the LDS tiles. The tile read by 16-byte row
// fragments (K forward, V gradient) runs at full LDS rate with a stride of
// D + 8. The tile read by transpose reads (V forward, K gradient, which
// also takes row fragments) does not at any plain stride near D (measured:
// about 110 B/clk per CU against 170-200 for the other patterns), so for
// D = 128 its rows are stored permuted (P) at stride D + 8, which serves
// both read patterns at 170-200 B/clk.
template <typename T, int D> struct FwdLd;
template <> struct FwdLd<bf16, 32> { static constexpr int K = 40, V = 56; static constexpr bool P = false; };
template <> struct FwdLd<bf16, 64> { static constexpr int K = 72, V = 72; static constexpr bool P = false; };
template <> struct FwdLd<bf16, 128> { static constexpr int K = 136, V = 136; static constexpr bool P = true; };
template <> struct FwdLd<float, 32> { static constexpr int K = 36, V = 36; static constexpr bool P = false; };
template <> struct FwdLd<float, 64> { static constexpr int K = 68, V = 68; static constexpr bool P = false; };
template <> struct FwdLd<float, 128> { static constexpr int K = 132, V = 132; static constexpr bool P = false; };

// Waves per SIMD the tile kernels are built for: two, except fp32 at head
// dim 128, whose resident Q (and dA') fragments and O (dQ) accumulators
// alone take 128 (256) registers, and whose K/V tiles fill the LDS of one
// workgroup per compute unit.
template <typename T, int D> struct FwdOcc { static constexpr int W = 2; };
template <> struct FwdOcc<float, 128> { static constexpr int W = 1; };

// P: the tile read by transposed reads (V forward, K gradient) stores row r
// at row_perm(r), which swaps the two 2-bit fields of r's low four bits.
__device__ __forceinline__ int row_perm(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

// ld_frag_kmajor of rows kr..kr+15 (kr a multiple of 16) stored permuted by
// row_perm: row kr + 4 g + s' sits at kr + 4 s' + g, row kr + 8 + 4 g + s'
// at kr + 4 s' + g + 2.
__device__ __forceinline__ bf16x8 ld_frag_kmajor_perm(const bf16* X, int ld, int n0, int kr) {
  const int l = threadIdx.x & 63, s = l & 15, g = l >> 5;
  const int col = n0 + 16 * ((l >> 4) & 1) + 4 * (s & 3);
  const bf16* p0 = X + (kr + 4 * (s >> 2) + g) * ld + col;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 2 * ld));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}

// GRAD: the query-block pass of the backward, which computes dQ with the
// same tiling (see the comment of fwd_body).
template <typename T, int D, bool GRAD = false>
struct FwdCfg {
  static constexpr int BM = 128;                 // query rows per workgroup
  static constexpr int BN = 64;                  // keys per tile
  static constexpr int NT = 256;                 // threads
  static constexpr int KC = D / 16;              // reduction chunks over head dim
  static constexpr int DB = D / 32;              // 32-wide blocks of head dim
  static constexpr int KB = BN / 32;             // 32-key blocks per tile
  static constexpr int ES = (int)sizeof(T);
  static constexpr int VPC = 16 / ES;            // elements per 16-byte chunk
  static constexpr int CPR = D / VPC;            // 16-byte chunks per row
  // The gradient pass reads K both ways (rows for K Q^T, transposed for
  // K^T dS^T) and V only by rows, so the two strides swap.
  static constexpr int K_LD = GRAD ? FwdLd<T, D>::V : FwdLd<T, D>::K;
  static constexpr int V_LD = GRAD ? FwdLd<T, D>::K : FwdLd<T, D>::V;
  static constexpr bool K_PERM = GRAD && FwdLd<T, D>::P;   // K rows stored permuted
  static constexpr bool V_PERM = !GRAD && FwdLd<T, D>::P;  // V rows stored permuted
  static constexpr int WIN = BN + BM;            // position-bias window (>= BN + BM - 1)
  static constexpr int CH = BN * CPR / NT;       // 16-byte chunks per thread per tile (K or V)
  static constexpr int MAX_TIME = 1024;
  static_assert(BN * CPR % NT == 0, "staging");
};

template <typename T, int D, bool GRAD>
struct FwdSmem {
  using C = FwdCfg<T, D, GRAD>;
  int64_t tsq[C::BM];            // query timestamps of the block
  float ttab[C::MAX_TIME];       // -log2(e) * rab_time[hr] (forward), rab_time[hr] (gradient)
};

// The two K and V tile buffers. Direct memory-to-LDS loads into one buffer
// run while the other is read; the compiler proves the two apart (and so
// adds no wait for the loads before the reads) only when they are distinct
// LDS variables named at compile time, so the kernels declare four arrays
// and the tile loop alternates between them in two unrolled steps.
template <typename T, int D, bool GRAD>
struct FwdKV {
  using C = FwdCfg<T, D, GRAD>;
  T k[2][C::BN * C::K_LD];
  T v[2][C::BN * C::V_LD];
  int64_t ts[2][C::BN];          // key timestamps: rebased (low 32 bits) or raw
  float win[2][C::WIN];          // rab_pos window for the tile
};
template <typename T>
struct KVBufs {
  T* k0; T* k1; T* v0; T* v1;
  int64_t* ts0; int64_t* ts1;
  float* w0; float* w1;
};
#define HSTU_FWD_TILE_BUFFERS(C)                                              \
  __shared__ __attribute__((aligned(16))) T k0[C::BN * C::K_LD];              \
  __shared__ __attribute__((aligned(16))) T k1[C::BN * C::K_LD];              \
  __shared__ __attribute__((aligned(16))) T v0[C::BN * C::V_LD];              \
  __shared__ __attribute__((aligned(16))) T v1[C::BN * C::V_LD];              \
  __shared__ int64_t ts0[C::BN], ts1[C::BN];                                  \
  __shared__ float w0[C::WIN], w1[C::WIN];                                    \
  const KVBufs<T> kvb{k0, k1, v0, v1, ts0, ts1, w0, w1};

// GRAD (the dQ pass of the backward): the same walk over key tiles with
// the same bias and mask, but per tile
//   S^T  = K Q^T + bias,  dP^T = V dA'^T        (dA' = dO*U/L resident like Q)
//   dS^T = dP^T * sigma(S)(1 + S(1 - sigma(S)))  (0 where masked)
//   dQ^T += K^T dS^T                             (K^T by LDS transpose reads)
// so dQ stays in registers and is written once, with no atomics.
// CAND (forward only): candidate scoring against a cached history. Rows are
// numbered as in the single-shot layout (history 0..hist-1, then this
// call's candidates); history keys and values come from p.k_hist /
// p.v_hist, candidate rows from q, k, v, u, and only candidate rows are
// queries. The self term's position bucket is shifted by the index of the
// call's first candidate among all of the sequence's candidates.
template <typename T, int D, bool WIDE, bool POS, bool TIME, bool GRAD, bool CAND = false>
__device__ __forceinline__ void fwd_body(const AttnParams& p, FwdSmem<T, D, GRAD>& sm,
                                         const KVBufs<T> kvb, const WorkItem wi, const SeqInfo si,
                                         const int head, const int split = 0) {
  using C = FwdCfg<T, D, GRAD>;
  using F = typename Frag<T>::type;
  const int H = p.H;
  const int L = si.len, hist = si.hist;
  const int64_t start = si.start;
  const SeqCand sc = CAND ? p.cand[wi.seq] : SeqCand{0, 0, 0, 0};
  const int i0 = (wi.blk + (CAND ? hist / C::BM : 0)) * C::BM;
  const int i_last = min(i0 + C::BM, L) - 1;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, g = lane >> 5;
  const int iw = i0 + 32 * wave;                 // first row of this wave
  const int i = iw + l32;                        // this lane's query row
  const bool row_ok = i < L && (!CAND || i >= hist);
  // row of this lane's query in q, u, o, a
  const int64_t qrow = CAND ? (int64_t)sc.cand_start + (i - hist) : start + i;
  const int hr = p.rab_heads == 1 ? 0 : head;
  // Which bias terms exist is a compile-time choice so the tile loop is
  // straight-line code the scheduler can interleave.
  constexpr bool has_pos = POS;
  constexpr bool has_time = TIME;
  const bool sorted_ts = (si.flags & kSeqSortedTs) != 0;
  // Sequences whose timestamp span needs 64-bit bucket arithmetic keep raw
  // timestamps and take this body with WIDE set (every tile in the general
  // time-bias mode).
  constexpr bool wide = WIDE;
  const int t_last = p.n_time_buckets - 1;

  const T* __restrict__ qg = reinterpret_cast<const T*>(p.q);
  const T* __restrict__ kg = reinterpret_cast<const T*>(p.k);
  const T* __restrict__ vg = reinterpret_cast<const T*>(p.v);

  if constexpr (has_time)
    for (int x = tid; x < p.n_time_buckets; x += C::NT)
      sm.ttab[x] = (GRAD ? 1.f : kNegLog2e) * p.rab_time[(int64_t)hr * p.n_time_buckets + x];

  // Q fragments of this lane's row (B operand of S^T = K Q^T).
  F qf[C::KC];
#pragma unroll
  for (int c = 0; c < C::KC; ++c) {
    if (row_ok) {
      qf[c] = ld_frag(qg + qrow * p.sq + (int64_t)head * D + 16 * c + 8 * g);
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) qf[c][m] = from_f32<T>(0.f);
    }
  }
  // dA' fragments of this lane's row (B operand of dP^T = V dA'^T).
  F daf[GRAD ? C::KC : 1];
  if constexpr (GRAD) {
    const T* dag = reinterpret_cast<const T*>(p.d_a);
#pragma unroll
    for (int c = 0; c < C::KC; ++c) {
      if (row_ok) {
        daf[c] = ld_frag(dag + ((start + i) * H + head) * (int64_t)D + 16 * c + 8 * g);
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) daf[c][m] = from_f32<T>(0.f);
      }
    }
  }
  // every row of the sequence has a timestamp (CAND: history rows too, which
  // are no queries but bound the wave's time-bucket range)
  int64_t ts_i = 0;
  if (has_time && i < L)
    ts_i = wide ? p.timestamps[start + i] : (int64_t)p.ts_rel[start + i];
  if constexpr (has_time) sm.tsq[32 * wave + l32] = ts_i;     // both lane halves hold the same row

  // Position-bias window: entry x holds the bias of offset j - p_i = j0 - p_max + x.
  const int p_max = min(i_last, hist);
  const int p_i = row_ok ? min(i, hist) : p_max;
  const int c_lane = p_max - p_i;                // >= 0, < BM

  // Key tiles: [0, t_end) minus the candidate-only tiles [skip_lo, skip_hi).
  const int t_end = i_last / C::BN + 1;
  const int skip_lo = (hist + C::BN - 1) / C::BN;
  const int skip_hi = max(i0, hist) / C::BN;
  const int n_a = min(skip_lo, t_end);
  const int b_start = max(skip_hi, n_a);
  // CAND with p.kv_splits > 1: this workgroup's share of the history tiles;
  // the last split also takes the candidate (diagonal) tiles
  int h_lo = 0, h_n = n_a, d_n = max(0, t_end - b_start);
  if constexpr (CAND) {
    const int S = p.kv_splits;
    if (S > 1) {
      h_lo = (int)((int64_t)n_a * split / S);
      h_n = (int)((int64_t)n_a * (split + 1) / S) - h_lo;
      if (split != S - 1) d_n = 0;
    }
  }
  const int n_tiles = h_n + d_n;

  // ---------------------------------------------------------------- staging
  u32x4 kreg[C::CH], vreg[C::CH];
  uint32_t tsreg = 0;                            // rebased timestamp (64-bit: tsreg64)
  int64_t tsreg64 = 0;
  float winreg = 0.f;

  auto tile_j0 = [&](int n) { return (n < h_n ? h_lo + n : b_start + (n - h_n)) * C::BN; };

  // Non-candidate tiles: K and V rows through buffer resources whose range
  // ends at the sequence's last row, so rows at or beyond L read as zero
  // without a branch; the lane's offsets within a tile are fixed.
  // Each LDS row of the K (V) tile is KROW (VROW) 16-byte chunks, of which
  // the first CPR hold the row and the rest are padding. The tile is written
  // straight from memory to LDS, 64 consecutive chunks per wave instruction:
  // instruction k' of a tile (k' = wave, wave + 4, ...) fills chunks 64 k' ..
  // 64 k' + 63, lane l chunk 64 k' + l, which it fetches from the row stored
  // there (rows permuted where the tile is) and, for padding, the row's last
  // chunk again.
  constexpr int KROW = C::K_LD * C::ES / 16, VROW = C::V_LD * C::ES / 16;
  constexpr int KI = (KROW + 3) / 4, VI = (VROW + 3) / 4;
  static_assert(KROW * 16 == C::K_LD * C::ES && VROW * 16 == C::V_LD * C::ES, "chunk rows");
  uint32_t koff[KI], voff[VI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int c = 64 * (wave + 4 * i) + lane;
    const int r = c / KROW, q = c % KROW;
    const int gr = C::K_PERM ? row_perm(r) : r;
    koff[i] = (uint32_t)((int64_t)gr * p.sk * C::ES + (q < C::CPR ? q : C::CPR - 1) * 16);
  }
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int c = 64 * (wave + 4 * i) + lane;
    const int r = c / VROW, q = c % VROW;
    const int gr = C::V_PERM ? row_perm(r) : r;
    voff[i] = (uint32_t)((int64_t)gr * p.sv * C::ES + (q < C::CPR ? q : C::CPR - 1) * 16);
  }
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto load_tile = [&](int j0, T* kn, T* vn) {
    if constexpr (!CAND) {
      const int rows = min(L - j0, C::BN);
      const T* kb = kg + (start + j0) * p.sk + (int64_t)head * D;
      const T* vb = vg + (start + j0) * p.sv + (int64_t)head * D;
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)kb, (short)0, rows * (int)p.sk * C::ES, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)vb, (short)0, rows * (int)p.sv * C::ES, 0x00020000);
      typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
      for (int i = 0; i < KI; ++i)
        if (wave_u + 4 * i < KROW)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rk, (lds_void*)((char*)kn + 1024 * (wave_u + 4 * i)), 16, koff[i], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < VI; ++i)
        if (wave_u + 4 * i < VROW)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rv, (lds_void*)((char*)vn + 1024 * (wave_u + 4 * i)), 16, voff[i], 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < (CAND ? C::CH : 0); ++m) {
      const int ch = tid + C::NT * m;
      const int row = ch / C::CPR, cc = ch % C::CPR;
      const int j = j0 + row;
      const int64_t off = (int64_t)head * D + cc * C::VPC;
      if constexpr (CAND) {
        const bool hj = j < hist;
        const int64_t r = hj ? (int64_t)sc.hist_start + j : (int64_t)sc.cand_start + (j - hist);
        const T* kr = hj ? reinterpret_cast<const T*>(p.k_hist) + r * p.skh : kg + r * p.sk;
        const T* vr = hj ? reinterpret_cast<const T*>(p.v_hist) + r * p.svh : vg + r * p.sv;
        kreg[m] = j < L ? ld16(kr + off) : u32x4{0, 0, 0, 0};
        vreg[m] = j < L ? ld16(vr + off) : u32x4{0, 0, 0, 0};
      } else {
        kreg[m] = j < L ? ld16(kg + (start + j) * p.sk + off) : u32x4{0, 0, 0, 0};
        vreg[m] = j < L ? ld16(vg + (start + j) * p.sv + off) : u32x4{0, 0, 0, 0};
      }
    }
    // wave-uniform conditions: no divergent branch around the loads, whose
    // results are not needed before the tile's end
    if (has_time && wave_u == 0) {
      const int j = j0 + tid;
      if constexpr (wide) tsreg64 = j < L ? p.timestamps[start + j] : 0;
      else tsreg = p.ts_rel[start + min(j, L - 1)];
    }
    if (has_pos && wave_u < C::WIN / kWave) {
      const int rel = j0 - p_max + tid;
      // CAND: offsets >= 0 are the self terms (candidates see no other candidate)
      const int relp = CAND && rel >= 0 ? rel + sc.pos_shift : rel;
      winreg = p.rab_pos[(int64_t)hr * (2 * p.max_len - 1) + pos_bucket(relp, p.max_len)];
    }
  };

  auto store_tile = [&](T* kn, T* vn, int64_t* tsn, float* wn) {
#pragma unroll
    for (int m = 0; m < (CAND ? C::CH : 0); ++m) {
      const int ch = tid + C::NT * m;
      const int row = ch / C::CPR, cc = ch % C::CPR;
      st16(kn + (C::K_PERM ? row_perm(row) : row) * C::K_LD + cc * C::VPC, kreg[m]);
      st16(vn + (C::V_PERM ? row_perm(row) : row) * C::V_LD + cc * C::VPC, vreg[m]);
    }
    if (has_time && wave_u == 0) tsn[tid] = wide ? tsreg64 : (int64_t)tsreg;
    if (has_pos && wave_u < C::WIN / kWave) wn[tid] = winreg;
  };

  f32x16 acc_o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;

  if (n_tiles > 0) {
    load_tile(tile_j0(0), kvb.k0, kvb.v0);
    store_tile(kvb.k0, kvb.v0, kvb.ts0, kvb.w0);
  }
  __syncthreads();

  // one tile: read ks / vs (buffer n & 1), load tile n + 1 into kn / vn
  auto step = [&](const int n, const T* ks, const T* vs, const int64_t* tss, const float* wins,
                  T* kn, T* vn, int64_t* tsn, float* wn) {
    const int j0 = tile_j0(n);
    const bool more = n + 1 < n_tiles;
    if (more) load_tile(tile_j0(n + 1), kn, vn);

    // Does this wave have any unmasked pair in the tile?
    const bool skip = iw >= L || j0 > iw + 31 || (j0 >= hist && j0 + C::BN - 1 < iw) ||
                      (CAND && iw + 31 < hist);   // CAND: no candidate row in this wave
    if (!skip) {
      const bool need_mask = j0 + C::BN - 1 > min(iw, hist - 1);
      // Time-bias mode of this wave's sub-tile (its 32 queries x the 64 keys):
      // with sorted timestamps and every key at or before every query, the
      // corners bound the bucket: one bucket (mode 0), two adjacent ones split
      // by a per-query threshold (mode 1), else per-element buckets (mode 2).
      auto s_block = [&](int kb, f32x16& acc, f32x16& pacc) {
        if constexpr (has_pos) {
          const float* w = wins + c_lane + 32 * kb + 4 * g;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = w[8 * (r >> 2) + (r & 3)];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        }
        if constexpr (GRAD)
#pragma unroll
          for (int r = 0; r < 16; ++r) pacc[r] = 0.f;
#pragma unroll
        for (int c = 0; c < C::KC; ++c) {
          const F a = ld_frag(ks + (32 * kb + (C::K_PERM ? row_perm(l32) : l32)) * C::K_LD + 16 * c + 8 * g);
          mfma_32x32x16(acc, a, qf[c]);
          if constexpr (GRAD) {
            const F b = ld_frag(vs + (32 * kb + l32) * C::V_LD + 16 * c + 8 * g);
            mfma_32x32x16(pacc, b, daf[c]);
          }
        }
      };
      // The first 32-key block's MFMAs do not depend on the time-bias mode:
      // issued before it is worked out, they run under its LDS round trips.
      f32x16 sacc_first, pacc_first;
      if constexpr (!GRAD) s_block(0, sacc_first, pacc_first);
      int tmode = 2, b_lo = 0, b_hi = 0;
      int jstar = 0;                               // keys jl < jstar of the tile are in b_hi
      if (has_time && !wide && !need_mask && sorted_ts && j0 + C::BN - 1 <= iw) {
        const int qi_hi = min(iw + 31, L - 1) - i0;
        const int kj_hi = min(j0 + C::BN - 1, L - 1) - j0;
        b_hi = time_bucket_rel((uint32_t)sm.tsq[qi_hi], (uint32_t)tss[0], t_last);
        b_lo = time_bucket_rel((uint32_t)sm.tsq[iw - i0], (uint32_t)tss[kj_hi], t_last);
        if (b_hi == b_lo) {
          tmode = 0;
        } else if (b_hi == b_lo + 1) {
          tmode = 1;
          // key j is in b_hi iff ts_j <= ts_i + 1 - 2^b_hi; the tile's 64 key
          // timestamps are valid (every key precedes the wave's queries) and
          // sorted, so those keys are a prefix: count them (binary search)
          const int32_t thr = (int32_t)ts_i + 1 - (1 << b_hi);
          int pos = 0;
#pragma unroll
          for (int step = C::BN / 2; step > 0; step >>= 1)
            if ((int32_t)tss[pos + step - 1] <= thr) pos += step;
          // the steps reach BN - 1 at most: the last key decides BN
          jstar = pos + ((int32_t)tss[pos] <= thr ? 1 : 0);
        }
      }
      // TM: time-bias mode (3: 64-bit timestamps); MASK: causal / candidate
      // masking (only tiles that cross the diagonal or hold candidates).
      auto tile_math = [&](auto tm, auto mk) {
        constexpr int TM = decltype(tm)::value;
        constexpr bool MASK = decltype(mk)::value;
        const float tb_lo = (TM < 2 && has_time) ? sm.ttab[b_lo] : 0.f;
        const float tb_hi = (TM == 1) ? sm.ttab[b_hi] : 0.f;
        // The next 32-key block's MFMAs are issued before this block's
        // elementwise work (PIPE) unless the gradient pass, which runs two
        // waves per SIMD, lacks the registers (measured: issuing them early
        // there spills).
        constexpr bool PIPE = !GRAD;
        f32x16 sacc[C::KB], pacc[GRAD ? C::KB : 1];
        if constexpr (PIPE) sacc[0] = sacc_first;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) {
          if constexpr (PIPE) {
            if (kb + 1 < C::KB) s_block(kb + 1, sacc[kb + 1], pacc[GRAD ? kb + 1 : 0]);
          } else {
            s_block(kb, sacc[kb], pacc[GRAD ? kb : 0]);
          }
          // time bias of element r (pre-scaled by -log2(e) in the forward)
          auto tbias = [&](const int r) {
            const int jl = 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
            float tb = 0.f;
            if constexpr (has_time) {
              if constexpr (TM == 0) {
                tb = tb_lo;
              } else if constexpr (TM == 1) {
                const bool hi = 32 * kb + 8 * (r >> 2) + (r & 3) < jstar - 4 * g;
                tb = hi ? tb_hi : tb_lo;
              } else if constexpr (TM == 2) {
                tb = sm.ttab[time_bucket_rel((uint32_t)ts_i, (uint32_t)tss[jl], t_last)];
              } else {
                tb = sm.ttab[time_bucket_wide(ts_i, tss[jl], t_last)];
              }
            }
            return tb;
          };
          auto mask = [&](const int r, float pr) {
            if constexpr (MASK) {
              // pr opaque first: left alone the compiler turns the select
              // into a branch around the whole element (bias lookups
              // included), and the elements then run one at a time
              asm volatile("" : "+v"(pr));
              const int j = j0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
              const bool ok = j <= i && (j < hist || j == i);
              pr = ok ? pr : 0.f;
            }
            return pr;
          };
          float pv[16];
          if constexpr (!GRAD) {
            // in stages over the block's 16 elements, so that independent
            // elements interleave (one element's chain of bias, exp,
            // reciprocal and product at a time leaves the SIMD waiting)
            float sv[16], sg[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) sv[r] = __builtin_fmaf(sacc[kb][r], kNegLog2e, tbias(r));
#pragma unroll
            for (int r = 0; r < 16; ++r) sg[r] = __builtin_amdgcn_exp2f(sv[r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) sg[r] = __builtin_amdgcn_rcpf(1.0f + sg[r]);
#pragma unroll
            for (int r = 0; r < 16; ++r) pv[r] = mask(r, sv[r] * sg[r]);
          } else {
            // the same in two groups of 8 (all 16 at once spills here)
#pragma unroll
            for (int r0 = 0; r0 < 16; r0 += 8) {
              float sv[8], sg[8];
#pragma unroll
              for (int r = 0; r < 8; ++r) sv[r] = sacc[kb][r0 + r] + tbias(r0 + r);
#pragma unroll
              for (int r = 0; r < 8; ++r) sg[r] = __builtin_amdgcn_exp2f(sv[r] * kNegLog2e);
#pragma unroll
              for (int r = 0; r < 8; ++r) sg[r] = __builtin_amdgcn_rcpf(1.0f + sg[r]);
#pragma unroll
              for (int r = 0; r < 8; ++r) {
                const float sl = sv[r] * sg[r];
                pv[r0 + r] = mask(r0 + r, pacc[kb][r0 + r] * (sg[r] + __builtin_fmaf(-sl, sg[r], sl)));
              }
            }
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const F pf = pack8<T>(&pv[8 * h]);
            const int kr = 32 * kb + 16 * h;
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
              // forward: O^T += V^T P^T; gradient: dQ^T += K^T dS^T
              F a;
              if constexpr (C::K_PERM)
                a = ld_frag_kmajor_perm(ks, C::K_LD, 32 * db, kr);
              else if constexpr (GRAD)
                a = ld_frag_kmajor(ks, C::K_LD, 32 * db, kr, kr + 8);
              else if constexpr (C::V_PERM)
                a = ld_frag_kmajor_perm(vs, C::V_LD, 32 * db, kr);
              else
                a = ld_frag_kmajor(vs, C::V_LD, 32 * db, kr, kr + 8);
              mfma_32x32x16(acc_o[db], a, pf);
            }
          }
        }
      };
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;   // 64-bit timestamps
      using NoMask = std::integral_constant<bool, false>;
      using Mask = std::integral_constant<bool, true>;
      if constexpr (WIDE) {
        tile_math(I3(), Mask());
      } else {
        if (need_mask)
          tile_math(I2(), Mask());
        else if (tmode == 0)
          tile_math(I0(), NoMask());
        else if (tmode == 1)
          tile_math(I1(), NoMask());
        else
          tile_math(I2(), NoMask());
      }
    }
    if (more) store_tile(kn, vn, tsn, wn);
    __syncthreads();
  };
  for (int n = 0; n < n_tiles; n += 2) {
    step(n, kvb.k0, kvb.v0, kvb.ts0, kvb.w0, kvb.k1, kvb.v1, kvb.ts1, kvb.w1);
    if (n + 1 < n_tiles) step(n + 1, kvb.k1, kvb.v1, kvb.ts1, kvb.w1, kvb.k0, kvb.v0, kvb.ts0, kvb.w0);
  }

  // ---------------------------------------------------------------- epilogue
  if (!row_ok) return;
  if constexpr (GRAD) {
    // dQ row of this lane: register 4 rq + m of block db is head dim
    // 32 db + 8 rq + 4 g + m (1/L is already in dA').
    T* dqg = reinterpret_cast<T*>(p.dq) + ((start + i) * H + head) * (int64_t)D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        f32x4 a;
#pragma unroll
        for (int m = 0; m < 4; ++m) a[m] = acc_o[db][4 * rq + m];
        st4_from_f32(dqg + 32 * db + 8 * rq + 4 * g, a);
      }
    return;
  }
  const float scale = kNegLn2 * si.inv_len;
  if constexpr (CAND) {
    if (p.kv_splits > 1) {                         // partial A of this split
      float* pg = p.part + (((int64_t)split * p.m_rows + qrow) * H + head) * (int64_t)D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          f32x4 a;
#pragma unroll
          for (int m = 0; m < 4; ++m) a[m] = acc_o[db][4 * rq + m] * scale;
          *reinterpret_cast<f32x4*>(pg + 32 * db + 8 * rq + 4 * g) = a;
        }
      return;
    }
  }
  const int64_t orow = (qrow * H + head) * (int64_t)D;
  T* og = reinterpret_cast<T*>(p.o) + orow;
  const T* ug = p.u ? reinterpret_cast<const T*>(p.u) + qrow * p.su + (int64_t)head * D
                    : nullptr;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d = 32 * db + 8 * rq + 4 * g;
      f32x4 a;
#pragma unroll
      for (int m = 0; m < 4; ++m) a[m] = acc_o[db][4 * rq + m] * scale;
      if (p.a_saved) *reinterpret_cast<f32x4*>(p.a_saved + orow + d) = a;
      if (ug) {
        const f32x4 uv = ld4_f32(ug + d);
#pragma unroll
        for (int m = 0; m < 4; ++m) a[m] *= uv[m];
      }
      st4_from_f32(og + d, a);
    }
  }
}

// One workgroup per (work item, head). A sequence whose timestamp span
// needs 64-bit bucket arithmetic (only possible with a time bias) takes the
// 64-bit body; both bodies are compiled into the one kernel, whose register
// count is that of the 32-bit body, so no second launch is needed for them.
template <typename T, int D, bool POS, bool TIME>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FwdOcc<T, D>::W, FwdOcc<T, D>::W)))
void hstu_fwd_kernel(AttnParams p) {
  __shared__ FwdSmem<T, D, false> sm;
  using C = FwdCfg<T, D, false>;
  HSTU_FWD_TILE_BUFFERS(C)
  const int item = blockIdx.x / p.H;
  const int head = blockIdx.x - item * p.H;
  if (item >= *p.n_items) return;
  const WorkItem wi = p.items[item];
  const SeqInfo si = p.seq[wi.seq];
  if (TIME && (si.flags & kSeqWideTs) != 0)
    fwd_body<T, D, true, POS, TIME, false>(p, sm, kvb, wi, si, head);
  else
    fwd_body<T, D, false, POS, TIME, false>(p, sm, kvb, wi, si, head);
}

template <typename T, int D, bool POS, bool TIME>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FwdOcc<T, D>::W, FwdOcc<T, D>::W)))
void hstu_fwd_cand_kernel(AttnParams p) {
  __shared__ FwdSmem<T, D, false> sm;
  __shared__ FwdKV<T, D, false> kv;
  const KVBufs<T> kvb{kv.k[0], kv.k[1], kv.v[0], kv.v[1], kv.ts[0], kv.ts[1], kv.win[0], kv.win[1]};
  const int S = p.kv_splits;                       // workgroups per (item, head)
  const int item = blockIdx.x / (p.H * S);
  const int rem = blockIdx.x - item * p.H * S;
  const int head = rem / S, split = rem - head * S;
  if (item >= *p.n_items) return;
  const WorkItem wi = p.items[item];
  const SeqInfo si = p.seq[wi.seq];
  if (TIME && (si.flags & kSeqWideTs) != 0)
    fwd_body<T, D, true, POS, TIME, false, true>(p, sm, kvb, wi, si, head, split);
  else
    fwd_body<T, D, false, POS, TIME, false, true>(p, sm, kvb, wi, si, head, split);
}

// Sum of the splits' partial A (candidate calls with p.kv_splits > 1), then
// A and O = A * U (or A), 4 elements per thread.
template <typename T>
__global__ __launch_bounds__(256) void cand_finish_kernel(AttnParams p) {
  const int64_t n4 = p.m_rows * p.H * p.D / 4;
  const int64_t plane = p.m_rows * p.H * p.D;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n4;
       x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = 4 * x;
    f32x4 a = *reinterpret_cast<const f32x4*>(p.part + e);
    for (int sp = 1; sp < p.kv_splits; ++sp) {
      const f32x4 b = *reinterpret_cast<const f32x4*>(p.part + sp * plane + e);
#pragma unroll
      for (int m = 0; m < 4; ++m) a[m] += b[m];
    }
    if (p.a_saved) *reinterpret_cast<f32x4*>(p.a_saved + e) = a;
    const int64_t row = e / ((int64_t)p.H * p.D), col = e - row * p.H * p.D;
    if (p.u) {
      const f32x4 uv = ld4_f32(reinterpret_cast<const T*>(p.u) + row * p.su + col);
#pragma unroll
      for (int m = 0; m < 4; ++m) a[m] *= uv[m];
    }
    st4_from_f32(reinterpret_cast<T*>(p.o) + e, a);
  }
}

template <typename T, int D, bool POS, bool TIME>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FwdOcc<T, D>::W, FwdOcc<T, D>::W)))
void hstu_dq_kernel(AttnParams p) {
  __shared__ FwdSmem<T, D, true> sm;
  using C = FwdCfg<T, D, true>;
  HSTU_FWD_TILE_BUFFERS(C)
  // sequences below n_ds take dQ from their exported dS tiles
  const int n_ds = p.ds_on != nullptr ? *p.ds_on : 0;
  if (n_ds >= p.B) return;
  const int item = blockIdx.x / p.H;
  const int head = blockIdx.x - item * p.H;
  if (item >= *p.n_items) return;
  const WorkItem wi = p.items[item];
  if (wi.seq < n_ds) return;
  const SeqInfo si = p.seq[wi.seq];
  if (TIME && (si.flags & kSeqWideTs) != 0)
    fwd_body<T, D, true, POS, TIME, true>(p, sm, kvb, wi, si, head);
  else
    fwd_body<T, D, false, POS, TIME, true>(p, sm, kvb, wi, si, head);
}

// KIND: 0 forward, 1 dQ pass, 2 candidate scoring against a cached history
template <int KIND, typename T, int D, bool POS, bool TIME>
void launch_one(const AttnParams& p, dim3 g, hipStream_t s) {
  if constexpr (KIND == 1)
    hipLaunchKernelGGL((hstu_dq_kernel<T, D, POS, TIME>), g, dim3(256), 0, s, p);
  else if constexpr (KIND == 2)
    hipLaunchKernelGGL((hstu_fwd_cand_kernel<T, D, POS, TIME>), g, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((hstu_fwd_kernel<T, D, POS, TIME>), g, dim3(256), 0, s, p);
}

template <int KIND, typename T, int D>
hipError_t launch_all(const AttnParams& p, int id, hipStream_t s) {
  const int64_t grid = p.max_items * p.H * (KIND == 2 ? p.kv_splits : 1);
  if (grid == 0) return hipSuccess;
  const dim3 g((unsigned)grid);
  const bool pos = p.rab_pos != nullptr, time = p.rab_time != nullptr;
  prof_before(id, s);
  if (pos && time) launch_one<KIND, T, D, true, true>(p, g, s);
  else if (pos) launch_one<KIND, T, D, true, false>(p, g, s);
  else if (time) launch_one<KIND, T, D, false, true>(p, g, s);
  else launch_one<KIND, T, D, false, false>(p, g, s);
  prof_after(id, s);
  return hipGetLastError();
}

}  // namespace

template <typename T, int D>
hipError_t launch_fwd(const AttnParams& p, hipStream_t s) {
  return launch_all<0, T, D>(p, kKFwd, s);
}

template <typename T, int D>
hipError_t launch_dq(const AttnParams& p, hipStream_t s) {
  return launch_all<1, T, D>(p, kKDq, s);
}

template <typename T, int D>
hipError_t launch_fwd_cand(const AttnParams& p, hipStream_t s) {
  hipError_t e = launch_all<2, T, D>(p, kKFwd, s);
  if (e != hipSuccess || p.kv_splits <= 1 || p.m_rows == 0) return e;
  const int64_t n4 = p.m_rows * p.H * p.D / 4;
  const int64_t blocks = (n4 + 255) / 256;
  hipLaunchKernelGGL(cand_finish_kernel<T>, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template hipError_t launch_fwd<bf16, 32>(const AttnParams&, hipStream_t);
template hipError_t launch_fwd<bf16, 64>(const AttnParams&, hipStream_t);
template hipError_t launch_fwd<bf16, 128>(const AttnParams&, hipStream_t);
template hipError_t launch_fwd<float, 32>(const AttnParams&, hipStream_t);
template hipError_t launch_fwd<float, 64>(const AttnParams&, hipStream_t);
template hipError_t launch_fwd<float, 128>(const AttnParams&, hipStream_t);
template hipError_t launch_fwd_cand<bf16, 32>(const AttnParams&, hipStream_t);
template hipError_t launch_fwd_cand<bf16, 64>(const AttnParams&, hipStream_t);
template hipError_t launch_fwd_cand<bf16, 128>(const AttnParams&, hipStream_t);
template hipError_t launch_fwd_cand<float, 32>(const AttnParams&, hipStream_t);
template hipError_t launch_fwd_cand<float, 64>(const AttnParams&, hipStream_t);
template hipError_t launch_fwd_cand<float, 128>(const AttnParams&, hipStream_t);
template hipError_t launch_dq<bf16, 32>(const AttnParams&, hipStream_t);
template hipError_t launch_dq<bf16, 64>(const AttnParams&, hipStream_t);
template hipError_t launch_dq<bf16, 128>(const AttnParams&, hipStream_t);
template hipError_t launch_dq<float, 32>(const AttnParams&, hipStream_t);
template hipError_t launch_dq<float, 64>(const AttnParams&, hipStream_t);
template hipError_t launch_dq<float, 128>(const AttnParams&, hipStream_t);

}  // namespace hstu
