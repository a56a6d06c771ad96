// Key-block backward of jagged HSTU pointwise attention for gfx950, fp32
// (the bf16 key-block kernel is bwd_k16.hip).
//
// One workgroup (4 waves) owns 128 keys of one sequence and one head; wave w
// owns keys 32w..32w+31 and keeps their K, V fragments and the dK, dV
// accumulators in registers for the whole loop over the 64-row query tiles
// that can see those keys. Per query tile (Q and dA' = dO*U/L staged
// row-major through LDS) and 32-query block:
//   S    = Q K^T + bias            (recomputed; bias read as in the forward)
//   dP   = dA' V^T
//   sg   = sigma(S), s = S*sg, s' = sg + s*(1 - sg)   (SiLU and its derivative)
//   dS   = dP * s'  (0 where masked)
//   dV  += s^T dA',  dK += dS^T Q   (Q, dA' fragments by LDS transpose reads)
// The accumulators hold S and dP with keys on lanes, which is the operand
// layout dV and dK need. dQ needs queries on lanes and a sum over all keys:
// adding per-block partials with fp32 atomics costs more than recomputing
// S and dP per query block, so dQ comes from a separate pass (the forward's
// tiling, in fwd.hip) and this kernel computes dK, dV and the rab gradients.
// The rab gradients are sums of dS over the pairs that read each table entry.
// Time buckets: with sorted timestamps a wave's sub-tile below the diagonal
// has one or two buckets, summed in registers; otherwise each element adds
// into an LDS histogram. Positions: a diagonal-major copy of the dS tile
// makes every diagonal a contiguous LDS row, summed after the tile; tiles
// with candidate rows (positions pinned to hist) add each element into a
// window instead.
#include "internal.h"

namespace hstu {

namespace {

// Row stride (elements) of the row-major Q / dA' tiles: 16-byte row reads
// need an odd multiple of 16 bytes, transpose reads need consecutive rows
// >= 8 banks apart.
template <typename T, int D> struct BwdLd;
template <> struct BwdLd<float, 32> { static constexpr int Q = 36; };
template <> struct BwdLd<float, 64> { static constexpr int Q = 68; };
template <> struct BwdLd<float, 128> { static constexpr int Q = 132; };

template <typename T, int D>
struct BwdCfg {
  static constexpr int BN = 128;                 // keys per workgroup
  static constexpr int BM = 64;                  // query rows per tile
  static constexpr int NT = 256;
  static constexpr int KC = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int QB = BM / 32;             // 32-row query blocks per tile
  static constexpr int ES = (int)sizeof(T);
  static constexpr int VPC = 16 / ES;
  static constexpr int CPR = D / VPC;
  static constexpr int Q_LD = BwdLd<T, D>::Q;    // row-major tiles [BM][D]
  static constexpr int NDIAG = BM + BN - 1;      // diagonals of a tile
  // Diagonal-major copy of dS, row dd = query - key + BN - 1 (so the
  // address of a lane's elements is a per-lane base plus constants), 64
  // queries (+8 padding: 16-byte aligned rows, at most 2-way write
  // conflicts).
  static constexpr int DG_LD = BM + 8;
  static constexpr int WIN = BN + BM;            // >= BN + BM - 1
  static constexpr int CH = BM * CPR / NT;       // 16-byte chunks per thread per tile
  static constexpr int MAX_TIME = 1024;
  // Time-gradient histogram: with up to HREP_NT buckets, HREP copies (lane
  // l adds into copy l % HREP, HREP_LD floats apart so a bucket's copies sit
  // in different banks) keep the per-element adds of one instruction from
  // piling onto one address; larger tables use a single copy.
  // Deterministic mode keeps one copy per wave instead (no two waves add
  // into one address, so the order of every sum is fixed by the program).
  static constexpr int HREP = 16, HREP_NT = 128, HREP_LD = HREP_NT + 1;
  static constexpr int NW = NT / kWave;
  static constexpr int THIST_DET = NW * (MAX_TIME + 1);
  static constexpr int THIST = HREP * HREP_LD > THIST_DET ? HREP * HREP_LD : THIST_DET;
  static_assert(BM * CPR % NT == 0, "staging");
};

// The arrays the tile loop touches per element come first, so their LDS
// addresses fit the 16-bit immediate offsets of the ds instructions.
template <typename T, int D>
struct BwdSmem {
  using C = BwdCfg<T, D>;
  T qs[C::BM * C::Q_LD];
  T das[C::BM * C::Q_LD];
  float win[C::WIN];
  float wing[C::NW * C::WIN];    // position window (one copy per wave in deterministic mode)
  int64_t tsq[C::BM];
  T dsd[C::NDIAG * C::DG_LD];
  int64_t tsk[C::BN];            // timestamps of the key block
  float ttab[C::MAX_TIME];
  float thist[C::THIST];
};

__device__ __forceinline__ float sum8(const f32x8& v) {
  return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

template <typename T, int D, bool WIDE, bool POS, bool TIME>
__device__ __forceinline__ void bwd_body(const AttnParams& p, BwdSmem<T, D>& sm, const WorkItem wi,
                                         const SeqInfo si, const int head) {
  using C = BwdCfg<T, D>;
  using F = typename Frag<T>::type;
  const int H = p.H;
  const int L = si.len, hist = si.hist;
  const int64_t start = si.start;
  const int k0 = wi.blk * C::BN;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, g = lane >> 5;
  const int jw = k0 + 32 * wave;                 // first key of this wave
  const int jl = 32 * wave + l32;                // this lane's key within the block
  const int j = k0 + jl;
  const bool key_ok = j < L;
  const int hr = p.rab_heads == 1 ? 0 : head;
  // Which bias terms exist is a compile-time choice so the tile loop is
  // straight-line code the scheduler can interleave.
  constexpr bool has_pos = POS;
  constexpr bool has_time = TIME;
  constexpr bool pos_grad = has_pos;
  constexpr bool time_grad = has_time;
  const bool sorted_ts = (si.flags & kSeqSortedTs) != 0;
  // Sequences whose timestamp span needs 64-bit bucket arithmetic keep raw
  // timestamps and take this body with WIDE set (every tile in the general
  // time-bias mode).
  constexpr bool wide = WIDE;
  const int n_pos = 2 * p.max_len - 1;
  const int t_last = p.n_time_buckets - 1;
  const int64_t HD = (int64_t)H * D;

  const T* __restrict__ qg = reinterpret_cast<const T*>(p.q);
  const T* __restrict__ kg = reinterpret_cast<const T*>(p.k);
  const T* __restrict__ vg = reinterpret_cast<const T*>(p.v);
  const T* __restrict__ dag = reinterpret_cast<const T*>(p.d_a);

  for (int x = tid; x < p.n_time_buckets; x += C::NT) sm.ttab[x] = p.rab_time[(int64_t)hr * p.n_time_buckets + x];
  // Deterministic mode: every sum has a fixed order (per-wave LDS copies,
  // partials in the workspace instead of global atomics).
  const bool det = p.det != 0 && *p.det_on != 0;
  const int nt_ld = p.n_time_buckets + 1;
  for (int x = tid; x < C::THIST; x += C::NT) sm.thist[x] = 0.f;
  const bool hrep = p.n_time_buckets <= C::HREP_NT;
  float* const thist_lane = det ? sm.thist + wave * nt_ld : sm.thist + (hrep ? (lane % C::HREP) * C::HREP_LD : 0);
  float* const thist_wave = det ? sm.thist + wave * nt_ld : sm.thist;
  for (int x = tid; x < C::NW * C::WIN; x += C::NT) sm.wing[x] = 0.f;
  float* const wing_w = sm.wing + (det ? wave * C::WIN : 0);
  float* const part_row =
      det ? p.part_pos + (p.tile_base[wi.seq] + (int64_t)head * ds_seq_tiles(L) + ds_row_start(L, wi.blk)) * kPartW
          : nullptr;
  // Diagonal-copy entries that no element maps to stay zero for the whole loop.
  if (pos_grad)
    for (int x = tid; x < C::NDIAG * C::DG_LD; x += C::NT) sm.dsd[x] = from_f32<T>(0.f);

  // Resident K, V fragments of this lane's key (B operands of Q K^T, dA' V^T).
  F kf[C::KC], vf[C::KC];
#pragma unroll
  for (int c = 0; c < C::KC; ++c) {
    if (key_ok) {
      kf[c] = ld_frag(kg + (start + j) * p.sk + (int64_t)head * D + 16 * c + 8 * g);
      vf[c] = ld_frag(vg + (start + j) * p.sv + (int64_t)head * D + 16 * c + 8 * g);
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        kf[c][m] = from_f32<T>(0.f);
        vf[c][m] = from_f32<T>(0.f);
      }
    }
  }
  int64_t ts_j = 0;
  if (has_time && key_ok) ts_j = wide ? p.timestamps[start + j] : (int64_t)p.ts_rel[start + j];
  if constexpr (has_time) sm.tsk[jl] = ts_j;

  // Query tiles that can see this key block.
  const int qt_first = k0 / C::BM;
  const int last_row = k0 < hist ? L - 1 : min(k0 + C::BN - 1, L - 1);
  const int n_qt = last_row / C::BM - qt_first + 1;

  // ---------------------------------------------------------------- staging
  u32x4 qreg[C::CH], dreg[C::CH];
  int64_t tsreg = 0;
  float winreg = 0.f;

  // Staging: thread tid moves 16-byte chunk tid % CPR of rows tid / CPR + m * RPM.
  constexpr int RPM = C::NT / C::CPR;
  static_assert(C::NT % C::CPR == 0, "staging rows");
  const int row0 = tid / C::CPR, cc0 = tid % C::CPR;
  const T* const q_lane = qg + (start + row0) * p.sq + (int64_t)head * D + cc0 * C::VPC;
  const T* const d_lane = dag + (start + row0) * HD + (int64_t)head * D + cc0 * C::VPC;
  auto load_tile = [&](int q0) {
    if (q0 + C::BM <= L) {
#pragma unroll
      for (int m = 0; m < C::CH; ++m) {
        qreg[m] = ld16(q_lane + (int64_t)(q0 + m * RPM) * p.sq);
        dreg[m] = ld16(d_lane + (int64_t)(q0 + m * RPM) * HD);
      }
    } else {
#pragma unroll
      for (int m = 0; m < C::CH; ++m) {
        const bool ok = q0 + row0 + m * RPM < L;
        qreg[m] = ok ? ld16(q_lane + (int64_t)(q0 + m * RPM) * p.sq) : u32x4{0, 0, 0, 0};
        dreg[m] = ok ? ld16(d_lane + (int64_t)(q0 + m * RPM) * HD) : u32x4{0, 0, 0, 0};
      }
    }
    if (has_time && tid < C::BM) {
      const int ii = q0 + tid;
      tsreg = ii < L ? (wide ? p.timestamps[start + ii] : (int64_t)p.ts_rel[start + ii]) : 0;
    }
    if (has_pos && tid < C::WIN) {
      // entry y: offset j - p_i = k0 + BN - 1 - p_min - y
      const int p_min = min(q0, hist);
      winreg = p.rab_pos[(int64_t)hr * n_pos + pos_bucket(k0 + C::BN - 1 - p_min - tid, p.max_len)];
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int m = 0; m < C::CH; ++m) {
      st16(sm.qs + (row0 + m * RPM) * C::Q_LD + cc0 * C::VPC, qreg[m]);
      st16(sm.das + (row0 + m * RPM) * C::Q_LD + cc0 * C::VPC, dreg[m]);
    }
    if (has_time && tid < C::BM) sm.tsq[tid] = tsreg;
    if (has_pos && tid < C::WIN) sm.win[tid] = winreg;
  };

  f32x16 acc_dk[C::DB], acc_dv[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc_dk[db][r] = 0.f;
      acc_dv[db][r] = 0.f;
    }

  // Per-lane base of this lane's entries in the diagonal copy.
  T* const dsd_lane = sm.dsd + (C::BN - 1 - jl) * C::DG_LD + 4 * g * (C::DG_LD + 1);

  load_tile(qt_first * C::BM);
  store_tile();
  // Nothing loaded before the loop is still in flight when it starts: the
  // memory counters inside the loop then only ever wait for the loop's own
  // loads, never behind the dQ atomics of the previous tile.
  __builtin_amdgcn_s_waitcnt(0);

  for (int n = 0; n < n_qt; ++n) {
    const int q0 = (qt_first + n) * C::BM;
    const bool more = n + 1 < n_qt;
    __syncthreads();                               // tile n staged; previous dQ done
    // Keep the loop-carried MFMA operands and accumulators in the
    // accumulation registers: left to itself the allocator parks them in
    // VGPRs between tiles and copies them back and forth every iteration.
#pragma unroll
    for (int db = 0; db < C::DB; ++db) asm volatile("" : "+a"(acc_dk[db]), "+a"(acc_dv[db]));
#pragma unroll
    for (int c = 0; c < C::KC; ++c) asm volatile("" : "+a"(kf[c]), "+a"(vf[c]));
    if (more) load_tile(q0 + C::BM);

    // Tiles of history rows only sum the position gradient along diagonals of
    // the dS tile after it is complete; tiles with candidate rows (whose
    // position is pinned to hist) add each element into a window instead.
    const bool pos_diag = has_pos && q0 + C::BM - 1 < hist;
    const bool skip = jw >= L || q0 + C::BM - 1 < jw ||
                      (jw >= hist && (q0 > jw + 31 || q0 + C::BM - 1 < jw));
    if (!skip) {
      const bool need_mask = !(q0 >= jw + 31 && jw + 31 < hist && q0 + C::BM - 1 < L);
      const int p_min = min(q0, hist);
      // Time-bias mode of this wave's sub-tile (its 32 keys x the 64 queries).
      // With sorted timestamps and every key at or before every query, the
      // bucket grows with the query and shrinks with the key, so the corners
      // bound it: at most two adjacent buckets, split by a per-key threshold
      // (mode 1; a single bucket is the case of a threshold no query
      // reaches). Everything else takes per-element buckets (mode 2).
      int tmode = has_time ? 2 : 1, b_lo = 0, b_hi = 0;   // no time bias: one "bucket"
      uint32_t thr = 0;
      if (has_time && !wide && !need_mask && sorted_ts) {
        const int qi_hi = min(q0 + C::BM - 1, L - 1) - q0;
        const int kj_hi = min(jw + 31, L - 1) - k0;
        b_hi = time_bucket_rel((uint32_t)sm.tsq[qi_hi], (uint32_t)sm.tsk[jw - k0], t_last);
        b_lo = time_bucket_rel((uint32_t)sm.tsq[0], (uint32_t)sm.tsk[kj_hi], t_last);
        if (b_hi == b_lo) {
          tmode = 1;
          thr = 0xffffffffu;                              // rebased timestamps stay below 2^31
        } else if (b_hi == b_lo + 1) {
          tmode = 1;
          thr = (uint32_t)ts_j + ((1u << b_hi) - 1u);   // hi iff ts_i - ts_j + 1 >= 2^b_hi
        }
      }
      // S = Q K^T + bias and dP = dA' V^T for one 32-query block. PD: the
      // tile holds history rows only (compile-time, so the element loop
      // below stays branch-free).
      auto sp_block = [&](auto pd, int qb, f32x16& acc_s, f32x16& acc_p) {
        constexpr bool PD = decltype(pd)::value;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_p[r] = 0.f;
        if constexpr (PD) {
          // history rows: entry y = (BN - 1 - jl) + ql, a per-lane base plus constants
          const float* w = sm.win + (C::BN - 1 - jl) + 32 * qb + 4 * g;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_s[r] = w[8 * (r >> 2) + (r & 3)];
        } else if constexpr (has_pos) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
            acc_s[r] = sm.win[(C::BN - 1 - jl) + min(q0 + ql, hist) - p_min];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc_s[r] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < C::KC; ++c) {
          const F a = ld_frag(sm.qs + (32 * qb + l32) * C::Q_LD + 16 * c + 8 * g);
          mfma_32x32x16(acc_s, a, kf[c]);
          {
            const F b = ld_frag(sm.das + (32 * qb + l32) * C::Q_LD + 16 * c + 8 * g);
            mfma_32x32x16(acc_p, b, vf[c]);
          }
        }
      };
      // Per 32-query block: elementwise (SiLU and dS), dV += s^T dA' and
      // dK += dS^T Q over the block's two 16-query chunks, then the
      // transposed dS block into the shared tile.
      auto tile_math = [&](auto tm, auto mk, auto pd) {
        constexpr int TM = decltype(tm)::value;
        constexpr bool MASK = decltype(mk)::value;
        constexpr bool PD = decltype(pd)::value;
        // TM 0: one bucket for the whole sub-tile; 1: two buckets split at a
        // per-key threshold; 2: per-element buckets of rebased timestamps; 3:
        // of raw 64-bit timestamps.
        const float tb_lo = (TM <= 1 && has_time) ? sm.ttab[b_lo] : 0.f;
        const float tb_hi = (TM == 1 && has_time) ? sm.ttab[b_hi] : 0.f;
        float g_all = 0.f, g_hi = 0.f;
        // Per-element buckets: the gradient of the lane's four largest
        // buckets in the tile (b_top - k, k < 4) is summed in registers and
        // added once per tile; only elements below that window add into the
        // LDS histogram one by one. With sorted timestamps the bucket grows
        // with the query, so nearly all elements land in the window.
        float gw[4] = {0.f, 0.f, 0.f, 0.f};
        int b_top = 0;
        if constexpr (time_grad && TM >= 2) {
          const int q_hi = min(q0 + C::BM - 1, L - 1) - q0;
          b_top = TM == 2 ? time_bucket_rel((uint32_t)sm.tsq[q_hi], (uint32_t)ts_j, t_last)
                          : time_bucket_wide(sm.tsq[q_hi], ts_j, t_last);
        }
        // The next block's S and dP MFMAs are issued before this block's
        // elementwise work so the two overlap.
        f32x16 acc_sb[C::QB], acc_pb[C::QB];
        constexpr bool PIPE = true;
        if constexpr (PIPE) sp_block(pd, 0, acc_sb[0], acc_pb[0]);
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) {
          if constexpr (PIPE) {
            if (qb + 1 < C::QB) sp_block(pd, qb + 1, acc_sb[qb + 1], acc_pb[qb + 1]);
          } else {
            sp_block(pd, qb, acc_sb[qb], acc_pb[qb]);
          }
          f32x16& acc_s = acc_sb[qb];
          f32x16& acc_p = acc_pb[qb];
          // B operands of the first 16-query chunk's dV / dK products, read
          // now so the elementwise work below covers the LDS latency.
          constexpr bool PREFETCH = true;
          F bv0[C::DB], bk0[C::DB];
          if constexpr (PREFETCH) {
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
              bv0[db] = ld_frag_kmajor(sm.das, C::Q_LD, 32 * db, 32 * qb, 32 * qb + 8);
              bk0[db] = ld_frag_kmajor(sm.qs, C::Q_LD, 32 * db, 32 * qb, 32 * qb + 8);
            }
          }
          int bts[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
            const int i = q0 + ql;
            float s = acc_s[r];
            int bt = 0;
            bool hi = false;
            if constexpr (has_time) {
              if constexpr (TM == 0) {
                s += tb_lo;
              } else if constexpr (TM == 1) {
                hi = (uint32_t)sm.tsq[ql] >= thr;
                s += hi ? tb_hi : tb_lo;
              } else if constexpr (TM == 2) {
                bt = time_bucket_rel((uint32_t)sm.tsq[ql], (uint32_t)ts_j, t_last);
                s += sm.ttab[bt];
              } else {
                bt = time_bucket_wide(sm.tsq[ql], ts_j, t_last);
                s += sm.ttab[bt];
              }
            }
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(s * kNegLog2e));
            float sl = s * sg;
            float ds = acc_p[r] * (sg + __builtin_fmaf(-sl, sg, sl));
            if constexpr (MASK) {
              const bool ok = j <= i && (j < hist || j == i) && i < L;
              sl = ok ? sl : 0.f;
              ds = ok ? ds : 0.f;
            }
            acc_s[r] = sl;
            acc_p[r] = ds;
            bts[r] = bt;
            if constexpr (TM <= 1 && time_grad) g_all += ds;
            if constexpr (TM == 1 && time_grad) g_hi += hi ? ds : 0.f;
          }
          // Side effects after all the block's LDS reads: the compiler cannot
          // move a table read above an LDS write it cannot disambiguate, so
          // interleaving them would serialize the elements.
          // The position gradient goes through the diagonal copy in history
          // tiles (plain stores) and through window adds only in tiles with
          // candidate rows; LDS float atomics cost far more than stores.
          const bool to_copy = pos_grad && (PD || pos_diag);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float ds = acc_p[r];
            if constexpr (pos_grad && !PD) {
              if (!pos_diag) {
                const int i = q0 + 32 * qb + 8 * (r >> 2) + 4 * g + (r & 3);
                atomicAdd(&wing_w[(C::BN - 1 - jl) + min(i, hist) - p_min], ds);
              }
            }
            if constexpr (time_grad && TM >= 2) {
              const int k = b_top - bts[r];
#pragma unroll
              for (int w = 0; w < 4; ++w) gw[w] += k == w ? ds : 0.f;
              if ((unsigned)k >= 4u && ds != 0.f) atomicAdd(thist_lane + bts[r], ds);
            }
            if (to_copy)
              dsd_lane[(32 * qb + 8 * (r >> 2) + (r & 3)) * (C::DG_LD + 1)] = from_f32<T>(ds);
          }
          F sf[2], df[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            sf[h] = pack8<T>(reinterpret_cast<const float*>(&acc_s) + 8 * h);
            df[h] = pack8<T>(reinterpret_cast<const float*>(&acc_p) + 8 * h);
          }
          if constexpr (PREFETCH) {
            // second chunk's operands in flight while the first chunk's MFMAs run
            F bv1[C::DB], bk1[C::DB];
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
              bv1[db] = ld_frag_kmajor(sm.das, C::Q_LD, 32 * db, 32 * qb + 16, 32 * qb + 24);
              bk1[db] = ld_frag_kmajor(sm.qs, C::Q_LD, 32 * db, 32 * qb + 16, 32 * qb + 24);
            }
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
              mfma_32x32x16(acc_dv[db], sf[0], bv0[db]);
              mfma_32x32x16(acc_dk[db], df[0], bk0[db]);
            }
#pragma unroll
            for (int db = 0; db < C::DB; ++db) {
              mfma_32x32x16(acc_dv[db], sf[1], bv1[db]);
              mfma_32x32x16(acc_dk[db], df[1], bk1[db]);
            }
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int db = 0; db < C::DB; ++db) {
                const int kr = 32 * qb + 16 * h;
                mfma_32x32x16(acc_dv[db], sf[h], ld_frag_kmajor(sm.das, C::Q_LD, 32 * db, kr, kr + 8));
                mfma_32x32x16(acc_dk[db], df[h], ld_frag_kmajor(sm.qs, C::Q_LD, 32 * db, kr, kr + 8));
              }
          }
        }
        if constexpr (time_grad && TM >= 2) {
#pragma unroll
          for (int w = 0; w < 4; ++w)
            if (gw[w] != 0.f) atomicAdd(thist_lane + (b_top - w), gw[w]);
        }
        if constexpr (TM < 2) {
          if constexpr (time_grad) {
            g_all = wave_sum(g_all);
            if constexpr (TM == 1) g_hi = wave_sum(g_hi);
            if (lane == 0) {
              atomicAdd(&thist_wave[b_lo], g_all - g_hi);
              if constexpr (TM == 1) atomicAdd(&thist_wave[b_hi], g_hi);
            }
          }
        }
      };
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;   // 64-bit timestamps
      using NoMask = std::integral_constant<bool, false>;
      using Mask = std::integral_constant<bool, true>;
      // Three bodies: every body of this size in the loop raises the register
      // pressure of the whole loop, so only shapes that pay for themselves
      // get one. The fast ones (no mask, history rows, position gradient
      // through the diagonal copy) take the bulk: one time bucket (most
      // tiles away from the diagonal: a constant bias, one gradient sum) or
      // two. The general one (masks, per-element buckets, position gradient
      // through the diagonal copy in history tiles and through the window in
      // tiles with candidate rows) takes the rest.
      using I0 = std::integral_constant<int, 0>;
      using IG = std::conditional_t<WIDE, I3, I2>;
      using PosDiag = std::integral_constant<bool, has_pos>;
      const bool fast = !WIDE && !need_mask && tmode == 1 && (!has_pos || pos_diag);
      if (fast && b_hi == b_lo)
        tile_math(I0(), NoMask(), PosDiag());
      else if (fast)
        tile_math(I1(), NoMask(), PosDiag());
      else
        tile_math(IG(), Mask(), std::false_type());
    } else {
      // This wave's entries of the diagonal copy are zero.
      if (pos_grad && pos_diag) {
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            dsd_lane[(32 * qb + 8 * (r >> 2) + (r & 3)) * (C::DG_LD + 1)] = from_f32<T>(0.f);
      }
    }
    // This wave's staging loads of the next tile complete before the
    // barrier, so the stores after it run back to back (measured: waiting
    // for them store by store after the barrier costs about 8%).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();                               // dS, rab partials complete
    // Every read of this tile's Q and dA' is done: stage the next tile.
    if (more) store_tile();

    if (pos_grad && pos_diag) {
      // Diagonal sums: diagonal dd (query - key + BN - 1 within the tile)
      // gathers the elements whose position bucket is that of offset
      // k0 - q0 + (BN - 1) - dd.
      if (tid < C::NDIAG) {
        const int dd = tid;
        float sum = 0.f;
        const T* row = sm.dsd + dd * C::DG_LD;
#pragma unroll
        for (int c = 0; c < C::BM / 8; ++c) sum += sum8(ld_frag(row + 8 * c));
        if (det)
          part_row[(int64_t)n * kPartW + dd] = sum;
        else if (sum != 0.f)
          atomicAdd(p.d_rab_pos + (int64_t)hr * n_pos +
                        pos_bucket(k0 - q0 + (C::BN - 1) - dd, p.max_len),
                    sum);
      }
    }
    if (pos_grad && !pos_diag && tid < C::WIN) {
      // Flush the position-gradient window of this tile.
      if (det) {
        float gsum = 0.f;
        for (int w = 0; w < C::NW; ++w) {
          gsum += sm.wing[w * C::WIN + tid];
          sm.wing[w * C::WIN + tid] = 0.f;
        }
        part_row[(int64_t)n * kPartW + tid] = gsum;
      } else {
        const float gsum = sm.wing[tid];
        if (gsum != 0.f) {
          const int p_min = min(q0, hist);
          atomicAdd(p.d_rab_pos + (int64_t)hr * n_pos +
                        pos_bucket(k0 + C::BN - 1 - p_min - tid, p.max_len),
                    gsum);
          sm.wing[tid] = 0.f;
        }
      }
    }
  }

  // Time-gradient histogram of this workgroup.
  if constexpr (time_grad) {
    __syncthreads();
    const int64_t slot = det ? ((int64_t)p.blk_base[wi.seq] + wi.blk) * H + head : 0;
    for (int x = tid; x < p.n_time_buckets; x += C::NT) {
      float gsum = 0.f;
      if (det) {
        for (int w = 0; w < C::NW; ++w) gsum += sm.thist[w * nt_ld + x];
        p.part_time[slot * p.n_time_buckets + x] = gsum;
      } else {
        for (int c = 0; c < (hrep ? C::HREP : 1); ++c) gsum += sm.thist[c * C::HREP_LD + x];
        if (gsum != 0.f) atomicAdd(p.d_rab_time + (int64_t)hr * p.n_time_buckets + x, gsum);
      }
    }
  }

  // dK, dV of this lane's keys: register r holds key 8(r/4) + 4g + r%4 of
  // the wave, column d = 32 db + l32.
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jj = jw + 8 * (r >> 2) + 4 * g + (r & 3);
      if (jj < L) {
        const int64_t o = ((start + jj) * H + head) * (int64_t)D + 32 * db + l32;
        reinterpret_cast<T*>(p.dk)[o] = from_f32<T>(acc_dk[db][r]);
        reinterpret_cast<T*>(p.dv)[o] = from_f32<T>(acc_dv[db][r]);
      }
    }
  }
}

// K, V, dK and dV stay in registers: one wave per SIMD. A sequence that
// needs 64-bit timestamp arithmetic takes the 64-bit body, compiled into the
// same kernel.
template <typename T, int D, bool POS, bool TIME>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void hstu_bwd_kernel(AttnParams p) {
  __shared__ BwdSmem<T, D> sm;
  const int item = blockIdx.x / p.H;
  const int head = blockIdx.x - item * p.H;
  if (item >= *p.n_items) return;
  const WorkItem wi = p.items[item];
  const SeqInfo si = p.seq[wi.seq];
  if (TIME && (si.flags & kSeqWideTs) != 0)
    bwd_body<T, D, true, POS, TIME>(p, sm, wi, si, head);
  else
    bwd_body<T, D, false, POS, TIME>(p, sm, wi, si, head);
}

}  // namespace

template <typename T, int D>
hipError_t launch_bwd(const AttnParams& p, hipStream_t s) {
  const int64_t grid = p.max_items * p.H;
  if (grid == 0) return hipSuccess;
  const dim3 g((unsigned)grid);
  const bool pos = p.rab_pos != nullptr, time = p.rab_time != nullptr;
  prof_before(kKBwd, s);
  if (pos && time) hipLaunchKernelGGL((hstu_bwd_kernel<T, D, true, true>), g, dim3(256), 0, s, p);
  else if (pos) hipLaunchKernelGGL((hstu_bwd_kernel<T, D, true, false>), g, dim3(256), 0, s, p);
  else if (time) hipLaunchKernelGGL((hstu_bwd_kernel<T, D, false, true>), g, dim3(256), 0, s, p);
  else hipLaunchKernelGGL((hstu_bwd_kernel<T, D, false, false>), g, dim3(256), 0, s, p);
  prof_after(kKBwd, s);
  return hipGetLastError();
}

template hipError_t launch_bwd<float, 32>(const AttnParams&, hipStream_t);
template hipError_t launch_bwd<float, 64>(const AttnParams&, hipStream_t);
template hipError_t launch_bwd<float, 128>(const AttnParams&, hipStream_t);

}  // namespace hstu
