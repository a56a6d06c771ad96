// dQ of the bf16 backward from the dS tiles the key-block kernel exported:
// for a query block of 128 rows, dQ[i][d] = sum_j dS[i][j] K[j][d] (the 1/L
// of the definition is already in dA', hence in dS). The key blocks whose
// tiles hold this block's queries are those the key-block kernel visited
// for them: every history key block up to the query block (key block kb
// visits all query tiles from 2 kb on when its first key is a history row)
// and the query block's own key block (a candidate key block visits only
// its own rows). The product is the (KS, KS) case of the layer GEMM: dS^T
// tiles [keys][queries] and K rows [keys][d], both read by transposing LDS
// loads, 64 keys per stage.
//
// Loads go through buffer resources set per stage (the stage's two dS tiles;
// its K rows, whose range ends at the sequence's last row), so a lane's
// offsets are the same in every stage. Only the query block's own key block
// and a key block holding candidate keys have rows the key-block kernel did
// not write (its waves of 16 keys that skipped a tile, or a first 32-query
// chunk before their keys): there the lane's offset for such a row is moved
// past the range, which reads zeros.
#include "internal.h"
#include "gemm_tile.h"

namespace hstu {

namespace {

constexpr uint32_t kOob = 0x80000000u;           // a buffer offset beyond every range: reads zero

// A pointer every lane holds, moved to scalar registers (a buffer resource
// built from it then needs no per-lane loop).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

template <int D>
__global__ __launch_bounds__(256) void dq_ds_kernel(AttnParams p) {
  const int n_ds = *p.ds_on;                     // leading sequences with exported tiles
  if (n_ds == 0) return;                         // the recompute pass runs instead
  __shared__ GemmSmem sm;
  const int item = blockIdx.x / p.H;
  const int head = blockIdx.x - item * p.H;
  if (item >= *p.n_items) return;
  const WorkItem wi = p.items[item];
  if (wi.seq >= n_ds) return;                    // its dS was not exported: recomputed
  const SeqInfo si = p.seq[wi.seq];
  const int L = si.len;
  const int64_t start = si.start;
  const int qb = wi.blk, i0 = qb * 128;
  const int nqt = (L + kDsQueries - 1) / kDsQueries;
  const int qt0 = 2 * qb;
  const bool has_qt1 = qt0 + 1 < nqt;
  const int kb_hist = (si.hist + kDsKeys - 1) / kDsKeys;   // key blocks starting in the history
  const int n_hist = qb + 1 < kb_hist ? qb + 1 : kb_hist;
  const int n_kb = n_hist + (qb >= kb_hist ? 1 : 0);
  const int64_t nk = 2 * (int64_t)n_kb;           // stages of 64 keys
  const bf16* const dsb = reinterpret_cast<const bf16*>(p.ds) +
                          (p.tile_base[wi.seq] + (int64_t)head * ds_seq_tiles(L)) * kDsTile;
  const bf16* const kg = reinterpret_cast<const bf16*>(p.k) + start * p.sk + (int64_t)head * D;

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  // This lane's chunks of a stage (i = 0..3): row kk = c >> 4 of the stage
  // (key 64 half + kk of the block), chunk cc = c & 15: A queries 8 (cc & 7)
  // .. + 7 of query tile qt0 + (cc >> 3); B head dims 8 cc .. + 7.
  uint32_t aoff[2][4], boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int kk = c >> 4, cc = c & 15;
#pragma unroll
    for (int half = 0; half < 2; ++half)
      aoff[half][i] = (cc >= 8 && !has_qt1) ? kOob
                      : (uint32_t)(((cc >> 3) * kDsTile + (64 * half + kk) * kDsQueries + 8 * (cc & 7)) * 2);
    boff[i] = 8 * cc < D ? (uint32_t)((int64_t)kk * p.sk * 2 + 16 * cc) : kOob;
  }

  // stage st: key block kb = (st / 2)-th of the list, keys kb*128 + 64 (st & 1) + kk
  auto load = [&](u32x4 (&va)[4], u32x4 (&vb)[4], int64_t st) {
    const int idx = (int)(st >> 1), half = (int)(st & 1);
    const int kb = idx < n_hist ? idx : qb;
    const int64_t row0 = ds_row_start(L, kb) + qt0 - 2 * kb;   // tile (kb, qt0)
    const int key0 = kb * kDsKeys + 64 * half;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(dsb + row0 * kDsTile), (short)0, 2 * (int)kDsTile * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(kg + (int64_t)key0 * p.sk), (short)0,
        __builtin_amdgcn_readfirstlane(max(0, min(64, L - key0)) * (int)p.sk * 2), 0x00020000);
    // rows the key-block kernel left unwritten: only in the query block's own
    // key block, and in a key block holding candidate keys (whose waves of
    // 16 candidate keys visit only their own rows)
    const bool own = kb == qb || (kb + 1) * kDsKeys > si.hist;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t ao = half ? aoff[1][i] : aoff[0][i];
      if (own) {
        const int c = tid + 256 * i;
        const int kk = c >> 4, cc = c & 15;
        const int jw = key0 + (kk & ~15);        // first key of the writer wave
        const int q0 = (qt0 + (cc >> 3)) * kDsQueries;
        const bool skipped = jw >= L || q0 + kDsQueries - 1 < jw ||
                             (jw >= si.hist && (q0 > jw + 15 || q0 + kDsQueries - 1 < jw));
        if (skipped || ((cc & 7) < 4 && q0 + 31 < jw)) ao = kOob;
      }
      va[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)ao, 0, 0);
      vb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, (int)boff[i], 0, 0);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  u32x4 ra[4], rb[4];
  load(ra, rb, 0);
  slab_store<KS>(sm.a[0], ra, tid);
  slab_store<KS>(sm.b[0], rb, tid);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    const bool more = kt + 1 < nk;
    if (more) load(ra, rb, kt + 1);
#pragma unroll
    for (int c = 0; c < TK / 16; ++c) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) af[a] = slab_frag<KS>(sm.a[buf], 64 * wm + 32 * a, 16 * c);
#pragma unroll
      for (int b = 0; b < 2; ++b) bfr[b] = slab_frag<KS>(sm.b[buf], 64 * wn + 32 * b, 16 * c);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) mfma_32x32x16(acc[a][b], af[a], bfr[b]);
    }
    if (more) {
      slab_store<KS>(sm.a[buf ^ 1], ra, tid);
      slab_store<KS>(sm.b[buf ^ 1], rb, tid);
    }
    __syncthreads();
  }

  // rows of the product are tile positions: position 8 q + 4 h + r of a
  // 32-query chunk holds query 16 h + 4 q + r; staged in query order
  bf16* ts = reinterpret_cast<bf16*>(&sm);
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pos = 8 * (r >> 2) + 4 * g + (r & 3);          // within the 32-row chunk
        const int qi = 64 * wm + 32 * a + 16 * ((pos >> 2) & 1) + 4 * (pos >> 3) + (pos & 3);
        ts[qi * tile_ld<bf16>() + 64 * wn + 32 * b + l32] = (bf16)acc[a][b][r];
      }
  __syncthreads();
  const int64_t HD = (int64_t)p.H * D;
  const int rows = L - i0 < 128 ? L - i0 : 128;
  copy_tile_out(ts, reinterpret_cast<bf16*>(p.dq) + (start + i0) * HD + (int64_t)head * D, HD, 0, 0, rows, D);
}

}  // namespace

template <int D>
hipError_t launch_dq_ds(const AttnParams& p, hipStream_t s) {
  const int64_t grid = p.max_items * p.H;
  if (grid == 0 || p.ds == nullptr) return hipSuccess;
  prof_before(kKDqDs, s);
  hipLaunchKernelGGL(dq_ds_kernel<D>, dim3((unsigned)grid), dim3(256), 0, s, p);
  prof_after(kKDqDs, s);
  return hipGetLastError();
}

template hipError_t launch_dq_ds<32>(const AttnParams&, hipStream_t);
template hipError_t launch_dq_ds<64>(const AttnParams&, hipStream_t);
template hipError_t launch_dq_ds<128>(const AttnParams&, hipStream_t);

}  // namespace hstu
