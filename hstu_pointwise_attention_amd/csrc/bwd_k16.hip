// Key-block backward of jagged HSTU pointwise attention for gfx950, bf16:
// eight waves of 16 keys, two waves per SIMD.
//
// One workgroup owns 128 keys of one sequence and one head; wave w owns
// keys 16w..16w+15 and keeps their K, V fragments and dK, dV accumulators
// in registers (about 100 of them, so two waves share a SIMD: their
// elementwise work runs side by side, which one wave alone cannot issue
// fast enough, and one wave's MFMAs overlap the other's VALU work). Per
// 64-query tile (Q and dA' = dO*U/L staged row-major through LDS) and per
// 32-query chunk, with 16 x 16 x 32 MFMAs:
//   S  = Q K^T + bias, dP = dA' V^T     (four 16-query blocks, keys on lanes)
//   s  = SiLU(S), dS = dP * SiLU'(S)    (0 where masked)
//   dV += s^T dA', dK += dS^T Q         (Q, dA' as k-major fragments by
//                                        transposed LDS reads)
// and the rab gradients: a diagonal-major copy of dS whose rows are summed
// after the tile (position table), register sums or an LDS histogram (time
// table), a window of adds for tiles with candidate rows.
#include "internal.h"

namespace hstu {

namespace {

// Row stride (elements) of the staged Q and dA' tiles: D + 16 keeps both
// read patterns (16-row fragments of 16 bytes, and transposed reads of
// 4-row x 32-byte blocks per 16 lanes) free of bank conflicts; measured,
// strides of D + 8 or D + 24 take about 1.7x as long per byte.
template <int D> struct K16Ld { static constexpr int Q = D + 16; };

template <int D>
struct K16Cfg {
  static constexpr int BN = 128;                 // keys per workgroup
  static constexpr int BM = 64;                  // query rows per tile
  static constexpr int NT = 512;                 // 8 waves of 16 keys
  static constexpr int DK = D / 32;              // 32-wide reduction chunks of S, dP
  static constexpr int DB = D / 16;              // 16-wide column blocks of dK, dV
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int Q_LD = K16Ld<D>::Q;
  static constexpr int NDIAG = BM + BN - 1;
  static constexpr int DG_LD = BM + 8;
  static constexpr int WIN = BN + BM;
  static constexpr int SCH = BM * CPR;           // staging chunks per tensor per tile
  static constexpr int CH = SCH >= NT ? SCH / NT : 1;   // per staging thread
  static constexpr int NW = NT / kWave;          // waves
  static constexpr int MAX_TIME = 1024;
  // Time-gradient histogram: with up to HREP_NT buckets, HREP copies (lane l
  // adds into copy l % HREP) keep the adds of one instruction from piling
  // onto one address; larger tables use one copy. Deterministic mode keeps
  // one copy per wave instead (no two waves add into one address, so the
  // order of every sum is fixed by the program).
  static constexpr int HREP = 16, HREP_NT = 128, HREP_LD = HREP_NT + 1;
  static constexpr int THIST_DET = NW * (MAX_TIME + 1);
  static constexpr int THIST = HREP * HREP_LD > THIST_DET ? HREP * HREP_LD : THIST_DET;
  static_assert(SCH % NT == 0 || NT % SCH == 0, "staging");
};

template <int D>
struct K16Smem {
  using C = K16Cfg<D>;
  bf16 qs[C::BM * C::Q_LD];
  bf16 das[C::BM * C::Q_LD];
  float win[C::WIN];
  float wing[C::NW * C::WIN];    // position window (one copy per wave in deterministic mode)
  int64_t tsq[C::BM];
  bf16 dsd[C::NDIAG * C::DG_LD];
  int64_t tsk[C::BN];
  float ttab[C::MAX_TIME];
  float thist[C::THIST];
};

__device__ __forceinline__ void mfma16(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// B operand of a 16 x 16 x 32 MFMA gathered along the reduction dimension
// from a row-major LDS tile X (row = reduction index, ld elements per row):
// lane l = 16 q + s receives X[k][n0 + s] for k = kr0 + 4q + {0..3} (slots
// 0..3) and kr1 + 4q + {0..3} (slots 4..7): two ds_read_b64_tr_b16, lane s of
// each 16-lane group pointing at row s >> 2 of a 4-row block, columns
// 4(s & 3)..+3.
__device__ __forceinline__ bf16x8 ld_frag_kmajor16(const bf16* X, int ld, int n0, int kr0, int kr1) {
  const int l = threadIdx.x & 63, s = l & 15, q = l >> 4;
  const int col = n0 + 4 * (s & 3);
  const bf16* p0 = X + (kr0 + 4 * q + (s >> 2)) * ld + col;
  const bf16* p1 = X + (kr1 + 4 * q + (s >> 2)) * ld + col;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p1));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}

__device__ __forceinline__ float k16_sum8(const bf16x8& v) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const bf16x2 pr = {v[2 * m], v[2 * m + 1]};
    s = __builtin_amdgcn_fdot2_f32_bf16(pr, one, s, false);
  }
  return s;
}

template <int D, bool WIDE, bool POS, bool TIME>
__device__ __forceinline__ void k16_body(const AttnParams& p, K16Smem<D>& sm, const WorkItem wi,
                                         const SeqInfo si, const int head) {
  using C = K16Cfg<D>;
  using F = bf16x8;
  const int H = p.H;
  const int L = si.len, hist = si.hist;
  const int64_t start = si.start;
  const int k0 = wi.blk * C::BN;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int jw = k0 + 16 * wave;                 // first key of this wave
  const int jl = 16 * wave + l16;                // this lane's key within the block
  const int j = k0 + jl;
  const bool key_ok = j < L;
  const int hr = p.rab_heads == 1 ? 0 : head;
  constexpr bool has_pos = POS;
  constexpr bool has_time = TIME;
  constexpr bool wide = WIDE;
  const bool sorted_ts = (si.flags & kSeqSortedTs) != 0;
  const int n_pos = 2 * p.max_len - 1;
  const int t_last = p.n_time_buckets - 1;
  const int64_t HD = (int64_t)H * D;

  const bf16* __restrict__ qg = reinterpret_cast<const bf16*>(p.q);
  const bf16* __restrict__ kg = reinterpret_cast<const bf16*>(p.k);
  const bf16* __restrict__ vg = reinterpret_cast<const bf16*>(p.v);
  const bf16* __restrict__ dag = reinterpret_cast<const bf16*>(p.d_a);

  if constexpr (has_time)
    for (int x = tid; x < p.n_time_buckets; x += C::NT)
      sm.ttab[x] = kNegLog2e * p.rab_time[(int64_t)hr * p.n_time_buckets + x];
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
  if (has_pos)
    for (int x = tid; x < C::NDIAG * C::DG_LD; x += C::NT) sm.dsd[x] = (bf16)0.f;

  // K, V fragments of this lane's key: B operands of S = Q K^T, dP = dA' V^T
  // (lane l: key l % 16, head dims 32 c + 8 (l / 16) + 0..7).
  F kf[C::DK], vf[C::DK];
#pragma unroll
  for (int c = 0; c < C::DK; ++c) {
    if (key_ok) {
      kf[c] = ld_frag(kg + (start + j) * p.sk + (int64_t)head * D + 32 * c + 8 * q4);
      vf[c] = ld_frag(vg + (start + j) * p.sv + (int64_t)head * D + 32 * c + 8 * q4);
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) { kf[c][m] = (bf16)0.f; vf[c][m] = (bf16)0.f; }
    }
  }
  int64_t ts_j = 0;
  if (has_time && key_ok) ts_j = wide ? p.timestamps[start + j] : (int64_t)p.ts_rel[start + j];
  if (has_time && q4 == 0) sm.tsk[jl] = ts_j;

  const int qt_first = k0 / C::BM;
  const int last_row = k0 < hist ? L - 1 : min(k0 + C::BN - 1, L - 1);
  const int n_qt = last_row / C::BM - qt_first + 1;

  // dS export: this lane's 8 values of each 32-query chunk (queries
  // 16 h + 4 q4 + r of the chunk) sit together at positions 8 q4 + 4 h + r,
  // so each chunk is one 16-byte store per lane; tile (this key block, query
  // tile qt_first) of this head, query tile qt_first + n n tiles further.
  // A wave that skips a tile, or the first chunk of a tile that lies before
  // its keys, writes nothing there: the dQ pass applies the same rule and
  // reads zeros instead.
  static_assert(C::BN == kDsKeys && C::BM == kDsQueries, "dS tile shape");
  bf16* ds_row = nullptr;
  if (p.ds != nullptr && wi.seq < *p.ds_on)
    ds_row = reinterpret_cast<bf16*>(p.ds) +
             (p.tile_base[wi.seq] + (int64_t)head * ds_seq_tiles(L) + ds_row_start(L, wi.blk)) * kDsTile;
  const int ds_lane = jl * kDsQueries + 8 * q4;

  // ---------------------------------------------------------------- staging
  constexpr int RPM = C::NT / C::CPR;            // rows per staging step
  const bool stager = tid < C::SCH;              // all threads when D = 64, 128
  const int row0 = tid / C::CPR, cc0 = tid % C::CPR;
  u32x4 qreg[C::CH], dreg[C::CH];
  int64_t tsreg = 0;
  float winreg = 0.f;
  const bf16* const q_lane = qg + (start + row0) * p.sq + (int64_t)head * D + cc0 * 8;
  const bf16* const d_lane = dag + (start + row0) * HD + (int64_t)head * D + cc0 * 8;
  auto load_tile = [&](int q0) {
#pragma unroll
    for (int m = 0; m < C::CH; ++m) {
      const bool ok = stager && q0 + row0 + m * RPM < L;
      qreg[m] = ok ? ld16(q_lane + (int64_t)(q0 + m * RPM) * p.sq) : u32x4{0, 0, 0, 0};
      dreg[m] = ok ? ld16(d_lane + (int64_t)(q0 + m * RPM) * HD) : u32x4{0, 0, 0, 0};
    }
    if (has_time && tid < C::BM) {
      const int ii = q0 + tid;
      tsreg = ii < L ? (wide ? p.timestamps[start + ii] : (int64_t)p.ts_rel[start + ii]) : 0;
    }
    if (has_pos && tid < C::WIN) {
      const int p_min = min(q0, hist);
      winreg = p.rab_pos[(int64_t)hr * n_pos + pos_bucket(k0 + C::BN - 1 - p_min - tid, p.max_len)];
    }
  };
  auto store_tile = [&]() {
    if (stager) {
#pragma unroll
      for (int m = 0; m < C::CH; ++m) {
        st16(sm.qs + (row0 + m * RPM) * C::Q_LD + cc0 * 8, qreg[m]);
        st16(sm.das + (row0 + m * RPM) * C::Q_LD + cc0 * 8, dreg[m]);
      }
    }
    if (has_time && tid < C::BM) sm.tsq[tid] = tsreg;
    if (has_pos && tid < C::WIN) sm.win[tid] = winreg;
  };

  f32x4 acc_dk[C::DB], acc_dv[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) { acc_dk[db][r] = 0.f; acc_dv[db][r] = 0.f; }

  // element (block qb, register r) of this lane: query 16 qb + 4 q4 + r of the
  // tile; its diagonal-copy entry sits at a per-lane base plus a constant
  bf16* const dsd_lane = sm.dsd + (C::BN - 1 - jl) * C::DG_LD + 4 * q4 * (C::DG_LD + 1);

  load_tile(qt_first * C::BM);
  store_tile();
  __builtin_amdgcn_s_waitcnt(0);

  for (int n = 0; n < n_qt; ++n) {
    const int q0 = (qt_first + n) * C::BM;
    const bool more = n + 1 < n_qt;
    __syncthreads();                               // tile n staged
    if (more) load_tile(q0 + C::BM);
    const bool pos_diag = has_pos && q0 + C::BM - 1 < hist;
    bf16* const ds_w = ds_row ? ds_row + n * kDsTile : nullptr;
    const bool skip = jw >= L || q0 + C::BM - 1 < jw ||
                      (jw >= hist && (q0 > jw + 15 || q0 + C::BM - 1 < jw));
    if (!skip) {
      const bool need_mask = !(q0 >= jw + 15 && jw + 15 < hist && q0 + C::BM - 1 < L);
      const int p_min = min(q0, hist);
      int tmode = has_time ? 2 : 1, b_lo = 0, b_hi = 0;
      int istar = C::BM;                           // first query of the tile in bucket b_hi
      if (has_time && !wide && !need_mask && sorted_ts) {
        const int qi_hi = min(q0 + C::BM - 1, L - 1) - q0;
        const int kj_hi = min(jw + 15, L - 1) - k0;
        b_hi = time_bucket_rel((uint32_t)sm.tsq[qi_hi], (uint32_t)sm.tsk[jw - k0], t_last);
        b_lo = time_bucket_rel((uint32_t)sm.tsq[0], (uint32_t)sm.tsk[kj_hi], t_last);
        if (b_hi == b_lo) {
          tmode = 1;
        } else if (b_hi == b_lo + 1) {
          tmode = 1;
          // query i of this key's pairs is in b_hi iff ts_i - ts_j + 1 >= 2^b_hi;
          // the tile's 64 timestamps are valid and sorted, so those queries
          // are a suffix: count the ones below the threshold (binary search)
          const uint32_t thr = (uint32_t)ts_j + ((1u << b_hi) - 1u);
          int pos = 0;
#pragma unroll
          for (int step = C::BM / 2; step > 0; step >>= 1)
            if ((uint32_t)sm.tsq[pos + step - 1] < thr) pos += step;
          // the steps reach BM - 1 at most: the last query decides BM
          istar = pos + ((uint32_t)sm.tsq[pos] < thr ? 1 : 0);
        }
      }
      auto tile_math = [&](auto tm, auto mk, auto pd) {
        constexpr int TM = decltype(tm)::value;
        constexpr bool MASK = decltype(mk)::value;
        constexpr bool PD = decltype(pd)::value;
        const float tb_lo = (TM <= 1 && has_time) ? sm.ttab[b_lo] : 0.f;
        const float tb_hi = (TM == 1 && has_time) ? sm.ttab[b_hi] : 0.f;
        float g_all = 0.f, g_hi = 0.f;
        float gw[4] = {0.f, 0.f, 0.f, 0.f};
        int b_top = 0;
        if constexpr (has_time && TM >= 2) {
          const int q_hi = min(q0 + C::BM - 1, L - 1) - q0;
          b_top = TM == 2 ? time_bucket_rel((uint32_t)sm.tsq[q_hi], (uint32_t)ts_j, t_last)
                          : time_bucket_wide(sm.tsq[q_hi], ts_j, t_last);
        }
        const bool to_copy = has_pos && (PD || pos_diag);
        // per 32-query chunk: S, dP (sp), the elementwise step and the rab
        // gradient side effects (ew), dV, dK (kv)
        f32x4 acc_s[2][2], acc_p[2][2];              // [chunk][16-query block]
        auto sp = [&](const int kc) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int qb = 2 * kc + h;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc_p[kc][h][r] = 0.f;
            if constexpr (PD) {
              const float* w = sm.win + (C::BN - 1 - jl) + 16 * qb + 4 * q4;
#pragma unroll
              for (int r = 0; r < 4; ++r) acc_s[kc][h][r] = w[r];
            } else if constexpr (has_pos) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int ql = 16 * qb + 4 * q4 + r;
                acc_s[kc][h][r] = sm.win[(C::BN - 1 - jl) + min(q0 + ql, hist) - p_min];
              }
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) acc_s[kc][h][r] = 0.f;
            }
#pragma unroll
            for (int c = 0; c < C::DK; ++c) {
              const F a = ld_frag(sm.qs + (16 * qb + l16) * C::Q_LD + 32 * c + 8 * q4);
              mfma16(acc_s[kc][h], a, kf[c]);
              const F b = ld_frag(sm.das + (16 * qb + l16) * C::Q_LD + 32 * c + 8 * q4);
              mfma16(acc_p[kc][h], b, vf[c]);
            }
          }
        };
        auto ew = [&](const int kc, F& sf, F& df) {
          // in stages over the chunk's 8 elements (e = 4 h + r), so that
          // independent elements interleave
          int bts[8];
          bool his[8];
          float sv[8], sg[8];
#pragma unroll
          // sv = -log2(e) * S (the time table is stored scaled), so that
          // sigma(S) = 1 / (1 + 2^sv) and sl = sv * sigma(S) = -log2(e) SiLU(S)
          for (int e = 0; e < 8; ++e) {
            const int ql = 32 * kc + 16 * (e >> 2) + 4 * q4 + (e & 3);
            float tb = 0.f;
            int bt = 0;
            bool hi = false;
            if constexpr (has_time) {
              if constexpr (TM == 0) {
                tb = tb_lo;
              } else if constexpr (TM == 1) {
                hi = 32 * kc + 16 * (e >> 2) + (e & 3) >= istar - 4 * q4;
                tb = hi ? tb_hi : tb_lo;
              } else if constexpr (TM == 2) {
                bt = time_bucket_rel((uint32_t)sm.tsq[ql], (uint32_t)ts_j, t_last);
                tb = sm.ttab[bt];
              } else {
                bt = time_bucket_wide(sm.tsq[ql], ts_j, t_last);
                tb = sm.ttab[bt];
              }
            }
            sv[e] = __builtin_fmaf(acc_s[kc][e >> 2][e & 3], kNegLog2e, tb);
            bts[e] = bt;
            his[e] = hi;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) sg[e] = __builtin_amdgcn_exp2f(sv[e]);
#pragma unroll
          for (int e = 0; e < 8; ++e) sg[e] = __builtin_amdgcn_rcpf(1.0f + sg[e]);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int h = e >> 2, r = e & 3;
            const int i = q0 + 32 * kc + 16 * h + 4 * q4 + r;
            // SiLU'(S) = sigma + SiLU(S) (1 - sigma), SiLU(S) = -ln(2) sl
            float sl = sv[e] * sg[e];
            float ds = acc_p[kc][h][r] * __builtin_fmaf(__builtin_fmaf(-sl, sg[e], sl), kNegLn2, sg[e]);
            if constexpr (MASK) {
              const bool ok = j <= i && (j < hist || j == i) && i < L;
              sl = ok ? sl : 0.f;
              ds = ok ? ds : 0.f;
            }
            acc_s[kc][h][r] = sl;
            acc_p[kc][h][r] = ds;
            if constexpr (TM <= 1 && has_time) g_all += ds;
            if constexpr (TM == 1 && has_time) g_hi += his[e] ? ds : 0.f;
          }
          // s^T and dS^T as A operands: slots 0..3 the first block's
          // queries, 4..7 the second's (the k-major reads pair them alike)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sf[r] = (bf16)acc_s[kc][0][r];
            sf[4 + r] = (bf16)acc_s[kc][1][r];
            df[r] = (bf16)acc_p[kc][0][r];
            df[4 + r] = (bf16)acc_p[kc][1][r];
          }
          // side effects after the chunk's LDS reads; the dS copy stores the
          // halves of df's words (opaque, so that they are not converted again)
          asm volatile("" : "+v"(df));
          const u32x4 dfw = __builtin_bit_cast(u32x4, df);
          if (ds_w) st16(ds_w + (ds_lane + 32 * kc), dfw);   // dS^T row: the chunk's 8 values
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float ds = acc_p[kc][h][r];
              if constexpr (has_pos && !PD) {
                if (!pos_diag) {
                  const int i = q0 + 32 * kc + 16 * h + 4 * q4 + r;
                  atomicAdd(&wing_w[(C::BN - 1 - jl) + min(i, hist) - p_min], ds);
                }
              }
              if constexpr (has_time && TM >= 2) {
                const int k = b_top - bts[4 * h + r];
#pragma unroll
                for (int w = 0; w < 4; ++w) gw[w] += k == w ? ds : 0.f;
                if ((unsigned)k >= 4u && ds != 0.f) atomicAdd(thist_lane + bts[4 * h + r], ds);
              }
              if (to_copy) {
                const uint32_t w = dfw[2 * h + (r >> 1)];
                reinterpret_cast<uint16_t*>(dsd_lane)[(32 * kc + 16 * h + r) * (C::DG_LD + 1)] =
                    (uint16_t)((r & 1) ? (w >> 16) : w);
              }
            }
        };
        auto kv = [&](const int kc, const F& sf, const F& df) {
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            mfma16(acc_dv[db], sf, ld_frag_kmajor16(sm.das, C::Q_LD, 16 * db, 32 * kc, 32 * kc + 16));
            mfma16(acc_dk[db], df, ld_frag_kmajor16(sm.qs, C::Q_LD, 16 * db, 32 * kc, 32 * kc + 16));
          }
        };
        F sf0, df0, sf1, df1;
        if (MASK && q0 + 31 < jw) {
          // the first 32 queries lie before this wave's keys: all masked
          if (to_copy) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              dsd_lane[(16 * (e >> 2) + (e & 3)) * (C::DG_LD + 1)] = (bf16)0.f;
          }
        } else {
          sp(0);
          ew(0, sf0, df0);
          kv(0, sf0, df0);
        }
        sp(1);
        ew(1, sf1, df1);
        kv(1, sf1, df1);
        if constexpr (has_time && TM >= 2) {
#pragma unroll
          for (int w = 0; w < 4; ++w)
            if (gw[w] != 0.f) atomicAdd(thist_lane + (b_top - w), gw[w]);
        }
        if constexpr (has_time && TM < 2) {
          g_all = wave_sum(g_all);
          if constexpr (TM == 1) g_hi = wave_sum(g_hi);
          if (lane == 0) {
            atomicAdd(&thist_wave[b_lo], g_all - g_hi);
            if constexpr (TM == 1) atomicAdd(&thist_wave[b_hi], g_hi);
          }
        }
      };
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      using NoMask = std::integral_constant<bool, false>;
      using Mask = std::integral_constant<bool, true>;
      using IG = std::conditional_t<WIDE, I3, I2>;
      using PosDiag = std::integral_constant<bool, has_pos>;
      const bool fast = !WIDE && !need_mask && tmode == 1 && (!has_pos || pos_diag);
      if (fast && b_hi == b_lo)
        tile_math(I0(), NoMask(), PosDiag());
      else if (fast)
        tile_math(I1(), NoMask(), PosDiag());
      else
        tile_math(IG(), Mask(), std::false_type());
    } else if (has_pos && pos_diag) {
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dsd_lane[(16 * qb + r) * (C::DG_LD + 1)] = (bf16)0.f;
    }
    __syncthreads();                               // dS copy and window complete
    if (more) store_tile();
    if (has_pos && pos_diag) {
      if (tid < C::NDIAG) {
        const int dd = tid;
        float sum = 0.f;
        const bf16* row = sm.dsd + dd * C::DG_LD;
#pragma unroll
        for (int c = 0; c < C::BM / 8; ++c) sum += k16_sum8(ld_frag(row + 8 * c));
        if (det)
          part_row[(int64_t)n * kPartW + dd] = sum;
        else if (sum != 0.f)
          atomicAdd(p.d_rab_pos + (int64_t)hr * n_pos + pos_bucket(k0 - q0 + (C::BN - 1) - dd, p.max_len), sum);
      }
    } else if (has_pos && tid < C::WIN) {
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
          atomicAdd(p.d_rab_pos + (int64_t)hr * n_pos + pos_bucket(k0 + C::BN - 1 - p_min - tid, p.max_len), gsum);
          sm.wing[tid] = 0.f;
        }
      }
    }
  }

  if constexpr (has_time) {
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

  // dK, dV of this lane: register r of block db is key 4 (l / 16) + r of the
  // wave, head dim 16 db + l % 16.
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jj = jw + 4 * q4 + r;
      if (jj < L) {
        const int64_t o = ((start + jj) * H + head) * (int64_t)D + 16 * db + l16;
        reinterpret_cast<bf16*>(p.dk)[o] = (bf16)acc_dk[db][r];
        reinterpret_cast<bf16*>(p.dv)[o] = (bf16)(acc_dv[db][r] * kNegLn2);   // s was scaled by -log2(e)
      }
    }
  }
}

// One workgroup per (key block, head); a sequence that needs 64-bit
// timestamp arithmetic takes the 64-bit body, compiled into the same kernel
// (it needs no more registers than the 32-bit one).
template <int D, bool POS, bool TIME>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void hstu_bwd_k16_kernel(AttnParams p) {
  __shared__ K16Smem<D> sm;
  const int item = blockIdx.x / p.H;
  const int head = blockIdx.x - item * p.H;
  if (item >= *p.n_items) return;
  const WorkItem wi = p.items[item];
  const SeqInfo si = p.seq[wi.seq];
  if (TIME && (si.flags & kSeqWideTs) != 0)
    k16_body<D, true, POS, TIME>(p, sm, wi, si, head);
  else
    k16_body<D, false, POS, TIME>(p, sm, wi, si, head);
}

}  // namespace

template <int D>
hipError_t launch_bwd_k16(const AttnParams& p, hipStream_t s) {
  const int64_t grid = p.max_items * p.H;
  if (grid == 0) return hipSuccess;
  const dim3 g((unsigned)grid);
  const bool pos = p.rab_pos != nullptr, time = p.rab_time != nullptr;
  prof_before(kKBwd, s);
  if (pos && time) hipLaunchKernelGGL((hstu_bwd_k16_kernel<D, true, true>), g, dim3(512), 0, s, p);
  else if (pos) hipLaunchKernelGGL((hstu_bwd_k16_kernel<D, true, false>), g, dim3(512), 0, s, p);
  else if (time) hipLaunchKernelGGL((hstu_bwd_k16_kernel<D, false, true>), g, dim3(512), 0, s, p);
  else hipLaunchKernelGGL((hstu_bwd_k16_kernel<D, false, false>), g, dim3(512), 0, s, p);
  prof_after(kKBwd, s);
  return hipGetLastError();
}

template hipError_t launch_bwd_k16<32>(const AttnParams&, hipStream_t);
template hipError_t launch_bwd_k16<64>(const AttnParams&, hipStream_t);
template hipError_t launch_bwd_k16<128>(const AttnParams&, hipStream_t);

}  // namespace hstu
