// Deterministic rab gradients: fixed-order sums of the partials the
// key-block kernels write when p.det is set.
//
// A key-block workgroup (sequence b, head h, 128 keys from k0 = 128 kb)
// visits the 64-query tiles q0 = 64 m, m = 2 kb .. 2 kb + n_qt - 1, and
// writes for tile m the kPartW floats
//   history rows only (q0 + 63 < hist): entry dd = sum of dS over the tile's
//     diagonal dd, whose pairs have offset j - i = k0 - q0 + 127 - dd;
//   otherwise (the tile holds candidate rows): entry y = sum of dS over the
//     tile's pairs of offset j - p_i = k0 + 127 - min(q0, hist) - y;
// and, per (key block, head) slot, the sums of dS per time bucket. Each
// rab_pos entry p receives the pairs whose clamped offset maps to p, so the
// sum over the partials below visits, for each output, the sequences, heads
// and key blocks in ascending order, the tiles in ascending order and the
// entries of a tile in ascending order; the waves of a workgroup take the
// (sequence, head, key block) units in turn and their sums are added
// in wave order. The result does not depend on timing.
#include "internal.h"

namespace hstu {

namespace {

constexpr int kRedWaves = 8;
constexpr int64_t kFar = (int64_t)1 << 40;

__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
__device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return -floor_div(-a, b); }

// Offsets j - p_i that map to position bucket pb: [lo, hi].
__device__ __forceinline__ void bucket_offsets(int pb, int max_len, int64_t& lo, int64_t& hi) {
  const int nb = 2 * max_len - 1;
  lo = pb == 0 ? -kFar : (int64_t)pb - (max_len - 1);
  hi = pb == nb - 1 ? kFar : (int64_t)pb - (max_len - 1);
}

__global__ __launch_bounds__(64 * kRedWaves) void rab_reduce_pos_kernel(AttnParams p) {
  __shared__ float red[kRedWaves][64];
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int n_pos = 2 * p.max_len - 1;
  const int pb = blockIdx.x * 64 + lane;
  const int hr = blockIdx.y;
  if (*p.det_on == 0) return;
  float acc = 0.f;
  int64_t lo = 0, hi = 0;
  if (pb < n_pos) bucket_offsets(pb, p.max_len, lo, hi);
  int unit = 0;
  for (int b = 0; b < p.B; ++b) {
    const SeqInfo si = p.seq[b];
    const int L = si.len, hist = si.hist;
    const int nkb = si.nblk;
    const int nqt = (L + kDsQueries - 1) / kDsQueries;
    for (int h = 0; h < p.H; ++h) {
      if (p.rab_heads != 1 && h != hr) continue;
      const int64_t seq_tiles = p.tile_base[b] + (int64_t)h * ds_seq_tiles(L);
      for (int kb = 0; kb < nkb; ++kb, ++unit) {
        if (unit % kRedWaves != wave || pb >= n_pos) continue;
        const int k0 = kb * kBlk;
        const int last_row = k0 < hist ? L - 1 : min(k0 + kBlk - 1, L - 1);
        const int m0 = 2 * kb, m1 = last_row / kDsQueries;   // tiles m0 .. m1
        const float* row = p.part_pos + (seq_tiles + ds_row_start(L, kb)) * kPartW;
        // history-row tiles whose diagonals reach [lo, hi]: c - dd in [lo, hi]
        // with c = k0 - q0 + 127 and 0 <= dd < 191
        int64_t ma = ceil_div((int64_t)k0 - 63 - hi, kDsQueries);
        int64_t mb = floor_div((int64_t)k0 + 127 - lo, kDsQueries);
        ma = ma < m0 ? m0 : ma;
        mb = mb > m1 ? m1 : mb;
        for (int64_t m = ma; m <= mb; ++m) {
          const int q0 = (int)m * kDsQueries;
          const float* t = row + (m - m0) * kPartW;
          if (q0 + kDsQueries - 1 < hist) {
            const int64_t c = (int64_t)k0 - q0 + 127;
            int64_t d0 = c - hi, d1 = c - lo;
            d0 = d0 < 0 ? 0 : d0;
            d1 = d1 > 190 ? 190 : d1;
            for (int64_t dd = d0; dd <= d1; ++dd) acc += t[dd];
          }
        }
        // tiles with candidate rows: entry y has offset c' - y, c' = k0 + 127 - min(q0, hist)
        const int mw = (int)ceil_div((int64_t)hist - (kDsQueries - 1), kDsQueries);
        for (int m = (mw > m0 ? mw : m0); m <= m1; ++m) {
          const int q0 = m * kDsQueries;
          const float* t = row + (m - m0) * kPartW;
          const int64_t c = (int64_t)k0 + 127 - (q0 < hist ? q0 : hist);
          int64_t y0 = c - hi, y1 = c - lo;
          y0 = y0 < 0 ? 0 : y0;
          y1 = y1 > kPartW - 1 ? kPartW - 1 : y1;
          for (int64_t y = y0; y <= y1; ++y) acc += t[y];
        }
      }
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && pb < n_pos) {
    float s = red[0][lane];
    for (int w = 1; w < kRedWaves; ++w) s += red[w][lane];
    p.d_rab_pos[(int64_t)hr * n_pos + pb] = s;
  }
}

__global__ __launch_bounds__(64 * kRedWaves) void rab_reduce_time_kernel(AttnParams p) {
  __shared__ float red[kRedWaves][64];
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int NT = p.n_time_buckets;
  const int x = blockIdx.x * 64 + lane;
  const int hr = blockIdx.y;
  if (*p.det_on == 0) return;
  float acc = 0.f;
  int unit = 0;
  for (int b = 0; b < p.B; ++b) {
    const int nkb = p.seq[b].nblk;
    for (int kb = 0; kb < nkb; ++kb) {
      for (int h = 0; h < p.H; ++h) {
        if (p.rab_heads != 1 && h != hr) continue;
        if (unit++ % kRedWaves != wave || x >= NT) continue;
        const int64_t slot = ((int64_t)p.blk_base[b] + kb) * p.H + h;
        acc += p.part_time[slot * NT + x];
      }
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && x < NT) {
    float s = red[0][lane];
    for (int w = 1; w < kRedWaves; ++w) s += red[w][lane];
    p.d_rab_time[(int64_t)hr * NT + x] = s;
  }
}

}  // namespace

hipError_t launch_rab_reduce(const AttnParams& p, hipStream_t s) {
  if (!p.det || p.det_on == nullptr) return hipSuccess;
  prof_before(kKRabReduce, s);
  if (p.d_rab_pos) {
    const int n_pos = 2 * p.max_len - 1;
    hipLaunchKernelGGL(rab_reduce_pos_kernel, dim3((n_pos + 63) / 64, p.rab_heads), dim3(64 * kRedWaves), 0, s, p);
  }
  if (p.d_rab_time && p.n_time_buckets > 0)
    hipLaunchKernelGGL(rab_reduce_time_kernel, dim3((p.n_time_buckets + 63) / 64, p.rab_heads),
                       dim3(64 * kRedWaves), 0, s, p);
  prof_after(kKRabReduce, s);
  return hipGetLastError();
}

}  // namespace hstu
