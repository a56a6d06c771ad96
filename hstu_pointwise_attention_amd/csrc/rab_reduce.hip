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
// rab_pos entry p receives the pairs whose clamped offset maps to p.
//
// The sum has a fixed order. The units (sequence, head, key block) of a
// table are numbered, sequences first; they are cut into kRedChunks equal
// runs. A workgroup takes one run for 256 outputs: its waves take the run's
// units in turn (wave w the units w, w + kRedWaves, ...), each unit's tiles
// in ascending order and a tile's entries in ascending order, and the wave
// sums are added in wave order. A second kernel adds the runs' sums in run
// order. The time table is the same with the (key block, head) slots as
// units. The result does not depend on timing.
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

// The last sequence b < B with blk_base[b] <= x (x below blk_base[B]: that
// sequence has key blocks).
__device__ __forceinline__ int seq_of_block(const int32_t* blk_base, int B, int64_t x) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (blk_base[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Run c of n units: [n c / kRedChunks, n (c + 1) / kRedChunks).
__device__ __forceinline__ void chunk_range(int64_t n, int c, int64_t& u0, int64_t& u1) {
  u0 = n * c / kRedChunks;
  u1 = n * (c + 1) / kRedChunks;
}

// Sum of the partials of table hr for kPosPer x 64 position buckets (lane
// l of workgroup x: buckets 64 (kPosPer x + o) + l, o < kPosPer) over one
// run of units; written
// to p.part_red[(hr * kRedChunks + run) * n_red + pb].
constexpr int kPosPer = 4;

__global__ __launch_bounds__(64 * kRedWaves) void rab_reduce_pos_kernel(AttnParams p) {
  __shared__ float red[kRedWaves][kPosPer * 64];
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int n_pos = 2 * p.max_len - 1;
  const int run = blockIdx.y;
  const int hr = blockIdx.z;
  if (*p.det_on == 0) return;
  int pb[kPosPer];
  int64_t lo[kPosPer], hi[kPosPer];
#pragma unroll
  for (int o = 0; o < kPosPer; ++o) {
    pb[o] = blockIdx.x * (kPosPer * 64) + 64 * o + lane;
    lo[o] = kFar;                                // beyond the table: no pair has this offset
    hi[o] = kFar;
    if (pb[o] < n_pos) bucket_offsets(pb[o], p.max_len, lo[o], hi[o]);
  }
  // units of table hr: (b, h, kb), h every head when the table is shared
  const int hn = p.rab_heads == 1 ? p.H : 1;
  const int64_t n_units = (int64_t)hn * p.blk_base[p.B];
  int64_t u0, u1;
  chunk_range(n_units, run, u0, u1);
  float acc[kPosPer];
#pragma unroll
  for (int o = 0; o < kPosPer; ++o) acc[o] = 0.f;
  for (int64_t u = u0 + wave; u < u1; u += kRedWaves) {
    const int b = seq_of_block(p.blk_base, p.B, u / hn);
    const SeqInfo si = p.seq[b];
    const int L = si.len, hist = si.hist;
    const int nkb = si.nblk;
    const int64_t r = u - (int64_t)hn * p.blk_base[b];
    const int h = p.rab_heads == 1 ? (int)(r / nkb) : hr;
    const int kb = (int)(r - (int64_t)(p.rab_heads == 1 ? h : 0) * nkb);
    const int64_t seq_tiles = p.tile_base[b] + (int64_t)h * ds_seq_tiles(L);
    const int k0 = kb * kBlk;
    const int last_row = k0 < hist ? L - 1 : min(k0 + kBlk - 1, L - 1);
    const int m0 = 2 * kb, m1 = last_row / kDsQueries;   // tiles m0 .. m1
    const float* row = p.part_pos + (seq_tiles + ds_row_start(L, kb)) * kPartW;
    // history-row tiles (q0 + 63 < hist, i.e. m < mh) whose diagonals reach
    // [lo, hi]: c - dd in [lo, hi] with c = k0 - q0 + 127 and 0 <= dd < 191
    const int mh = (int)floor_div((int64_t)hist - (kDsQueries - 1) - 1, kDsQueries) + 1;
    const int mhl = (mh - 1 < m1 ? mh - 1 : m1);   // last history-row tile
#pragma unroll
    for (int o = 0; o < kPosPer; ++o) {
      int64_t ma = ceil_div((int64_t)k0 - 63 - hi[o], kDsQueries);
      int64_t mb = floor_div((int64_t)k0 + 127 - lo[o], kDsQueries);
      ma = ma < m0 ? m0 : ma;
      mb = mb > mhl ? mhl : mb;
      for (int64_t m = ma; m <= mb; ++m) {
        const float* t = row + (m - m0) * kPartW;
        const int64_t c = (int64_t)k0 - m * kDsQueries + 127;
        int64_t d0 = c - hi[o], d1 = c - lo[o];
        d0 = d0 < 0 ? 0 : d0;
        d1 = d1 > 190 ? 190 : d1;
        for (int64_t dd = d0; dd <= d1; ++dd) acc[o] += t[dd];
      }
    }
    // tiles with candidate rows: entry y has offset c' - y, c' = k0 + 127 - min(q0, hist)
    for (int m = (mh > m0 ? mh : m0); m <= m1; ++m) {
      const int q0 = m * kDsQueries;
      const float* t = row + (m - m0) * kPartW;
      const int64_t c = (int64_t)k0 + 127 - (q0 < hist ? q0 : hist);
#pragma unroll
      for (int o = 0; o < kPosPer; ++o) {
        int64_t y0 = c - hi[o], y1 = c - lo[o];
        y0 = y0 < 0 ? 0 : y0;
        y1 = y1 > kPartW - 1 ? kPartW - 1 : y1;
        for (int64_t y = y0; y <= y1; ++y) acc[o] += t[y];
      }
    }
  }
#pragma unroll
  for (int o = 0; o < kPosPer; ++o) red[wave][64 * o + lane] = acc[o];
  __syncthreads();
  if (wave < kPosPer) {
    const int o = wave;
    const int q = blockIdx.x * (kPosPer * 64) + 64 * o + lane;
    if (q < n_pos) {
      float s = red[0][64 * o + lane];
      for (int w = 1; w < kRedWaves; ++w) s += red[w][64 * o + lane];
      const int n_red = n_pos + p.n_time_room;
      p.part_red[((int64_t)hr * kRedChunks + run) * n_red + q] = s;
    }
  }
}

// The same for 64 time buckets: units are the (key block, head) slots
// (blk_base[b] + kb) * H + h in ascending order, every head's slot when
// the table is shared, else head hr's.
__global__ __launch_bounds__(64 * kRedWaves) void rab_reduce_time_kernel(AttnParams p) {
  __shared__ float red[kRedWaves][64];
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int NT = p.n_time_buckets;
  const int x = blockIdx.x * 64 + lane;
  const int run = blockIdx.y;
  const int hr = blockIdx.z;
  if (*p.det_on == 0) return;
  const bool shared = p.rab_heads == 1;
  const int64_t n_units = (int64_t)p.blk_base[p.B] * (shared ? p.H : 1);
  int64_t u0, u1;
  chunk_range(n_units, run, u0, u1);
  float acc = 0.f;
  if (x < NT)
    for (int64_t u = u0 + wave; u < u1; u += kRedWaves) {
      const int64_t slot = shared ? u : u * p.H + hr;
      acc += p.part_time[slot * NT + x];
    }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && x < NT) {
    float s = red[0][lane];
    for (int w = 1; w < kRedWaves; ++w) s += red[w][lane];
    const int n_red = 2 * p.max_len - 1 + p.n_time_room;
    p.part_red[((int64_t)hr * kRedChunks + run) * n_red + (2 * p.max_len - 1) + x] = s;
  }
}

// Output e of table hr (position buckets, then time buckets): the runs'
// sums in run order.
__global__ __launch_bounds__(256) void rab_reduce_final_kernel(AttnParams p, int n_pos, int n_time) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int hr = blockIdx.y;
  if (*p.det_on == 0 || e >= n_pos + n_time) return;
  const int n_red = 2 * p.max_len - 1 + p.n_time_room;
  const int col = e < n_pos ? e : 2 * p.max_len - 1 + (e - n_pos);
  const float* src = p.part_red + (int64_t)hr * kRedChunks * n_red + col;
  float v[kRedChunks];
#pragma unroll
  for (int c = 0; c < kRedChunks; ++c) v[c] = src[(int64_t)c * n_red];
  float s = v[0];
#pragma unroll
  for (int c = 1; c < kRedChunks; ++c) s += v[c];
  if (e < n_pos)
    p.d_rab_pos[(int64_t)hr * n_pos + e] = s;
  else
    p.d_rab_time[(int64_t)hr * n_time + (e - n_pos)] = s;
}

}  // namespace

hipError_t launch_rab_reduce(const AttnParams& p, hipStream_t s) {
  if (!p.det || p.det_on == nullptr) return hipSuccess;
  const int n_pos = p.d_rab_pos ? 2 * p.max_len - 1 : 0;
  const int n_time = p.d_rab_time ? p.n_time_buckets : 0;
  if (n_pos + n_time == 0) return hipSuccess;
  prof_before(kKRabReduce, s);
  if (n_pos > 0)
    hipLaunchKernelGGL(rab_reduce_pos_kernel, dim3((n_pos + kPosPer * 64 - 1) / (kPosPer * 64), kRedChunks, p.rab_heads),
                       dim3(64 * kRedWaves), 0, s, p);
  if (n_time > 0)
    hipLaunchKernelGGL(rab_reduce_time_kernel, dim3((n_time + 63) / 64, kRedChunks, p.rab_heads),
                       dim3(64 * kRedWaves), 0, s, p);
  // the final sums read only the parts of each run's row written above
  hipLaunchKernelGGL(rab_reduce_final_kernel, dim3((n_pos + n_time + 255) / 256, p.rab_heads), dim3(256), 0, s,
                     p, n_pos, n_time);
  prof_after(kKRabReduce, s);
  return hipGetLastError();
}

}  // namespace hstu
