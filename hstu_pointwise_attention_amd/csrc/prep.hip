// Small kernels around the attention: per-sequence metadata and timestamp
// rebasing, the longest-first work schedule, the rab bucket export, and the
// elementwise passes before and after the fused backward.
#include "internal.h"

namespace hstu {

namespace {

constexpr int kSeqPrepThreads = 1024;
constexpr int kSchedThreads = 1024;

template <typename V, typename Op>
__device__ V block_reduce(V v, V* lds, Op op) {
  // wave64 butterfly, then across waves through LDS
  for (int off = 32; off > 0; off >>= 1) v = op(v, __shfl_xor(v, off));
  const int w = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  __syncthreads();
  if ((threadIdx.x % kWave) == 0) lds[w] = v;
  __syncthreads();
  v = lds[0];
  for (int i = 1; i < nw; ++i) v = op(v, lds[i]);
  return v;
}

struct MinOp { __device__ int64_t operator()(int64_t a, int64_t b) const { return a < b ? a : b; } };
struct MaxOp { __device__ int64_t operator()(int64_t a, int64_t b) const { return a > b ? a : b; } };
struct AndOp { __device__ int32_t operator()(int32_t a, int32_t b) const { return a & b; } };

// Metadata + rebased timestamps of sequence b, by one workgroup of any size
// up to kSeqPrepThreads; workgroup b of the n_groups doing this also clears
// its share of the rab gradient tables when they are set (the backward's
// overwritten outputs).
__device__ void seq_prep_body(const AttnParams& p, int b, int n_groups) {
  __shared__ int64_t lds64[kSeqPrepThreads / kWave];
  __shared__ int32_t lds32[kSeqPrepThreads / kWave];
  {
    const int64_t i0 = (int64_t)b * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)n_groups * blockDim.x;
    if (p.d_rab_pos) {
      const int64_t n = (int64_t)p.rab_heads * (2 * (int64_t)p.max_len - 1);
      for (int64_t i = i0; i < n; i += stride) p.d_rab_pos[i] = 0.f;
    }
    if (p.d_rab_time) {
      const int64_t n = (int64_t)p.rab_heads * p.n_time_buckets;
      for (int64_t i = i0; i < n; i += stride) p.d_rab_time[i] = 0.f;
    }
  }
  const int64_t s = p.seq_offsets[b];
  const int64_t e = p.seq_offsets[b + 1];
  const int L = (int)(e - s);
  int nt = p.num_targets ? (int)p.num_targets[b] : 0;
  nt = nt < 0 ? 0 : (nt > L ? L : nt);
  int flags = 0;
  int64_t origin = 0;
  if (p.timestamps != nullptr && L > 0) {
    // One pass: the timestamps relative to origin = first - 2^30 (known
    // before the pass, unlike the minimum), then min, max and sortedness.
    // The 32-bit form is exact when every relative value lies in
    // [0, 2^31 - 1), i.e. the sequence stays within 2^30 s before its first
    // timestamp and spans less than that range; otherwise the sequence is
    // flagged wide and the kernels use the 64-bit timestamps.
    origin = p.timestamps[s] - ((int64_t)1 << 30);
    int64_t lo = INT64_MAX, hi = INT64_MIN;
    int32_t sorted = 1;
    constexpr int U = 4;                         // loads in flight per step
    for (int64_t t0 = s + threadIdx.x; t0 < e; t0 += U * (int64_t)blockDim.x) {
      int64_t x[U], y[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t t = t0 + u * (int64_t)blockDim.x;
        x[u] = t < e ? p.timestamps[t] : 0;
        y[u] = (t < e && t > s) ? p.timestamps[t - 1] : INT64_MIN;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t t = t0 + u * (int64_t)blockDim.x;
        if (t < e) {
          lo = x[u] < lo ? x[u] : lo;
          hi = x[u] > hi ? x[u] : hi;
          if (y[u] > x[u]) sorted = 0;
          p.ts_rel[t] = (uint32_t)(x[u] - origin);
        }
      }
    }
    lo = block_reduce(lo, lds64, MinOp());
    hi = block_reduce(hi, lds64, MaxOp());
    sorted = block_reduce(sorted, lds32, AndOp());
    const bool narrow = lo >= origin && (uint64_t)hi - (uint64_t)origin < 0x7fffffffull;
    if (!narrow) flags |= kSeqWideTs;
    if (sorted) flags |= kSeqSortedTs;
  }
  if (threadIdx.x == 0) {
    SeqInfo si;
    si.start = (int32_t)s;
    si.len = L;
    si.hist = L - nt;
    si.flags = flags;
    si.inv_len = L > 0 ? 1.0f / (float)L : 0.0f;
    si.nblk = (L + kBlk - 1) / kBlk;
    si.ts_origin = origin;
    p.seq[b] = si;
  }
}

// Candidate scoring against a cached history: one workgroup per sequence.
// The sequence's rows are numbered as in the single-shot layout (history,
// then this call's candidates); the joined timestamps of that numbering go
// to c.ts_joined (64-bit) and p.ts_rel (rebased, as in seq_prep_body).
// Normalisation is 1 / (h + n) over all n candidates of the sequence, and
// only query blocks holding candidates are scheduled (nblk counts blocks
// from the one holding row h).
__device__ void seq_prep_cand_body(const AttnParams& p, const CandArgs& c, int b) {
  __shared__ int64_t lds64[kSeqPrepThreads / kWave];
  __shared__ int32_t lds32[kSeqPrepThreads / kWave];
  const int64_t hs = c.hist_offsets[b], cs = c.cand_offsets[b];
  const int h = (int)(c.hist_offsets[b + 1] - hs);
  const int m = (int)(c.cand_offsets[b + 1] - cs);
  const int L = h + m;
  const int64_t vs = (hs - c.hist_offsets[0]) + (cs - c.cand_offsets[0]);
  int64_t first = c.cand_first[b];
  first = first < 0 ? 0 : first;
  int64_t n_all = c.n_cands[b];
  n_all = n_all < first + m ? first + m : n_all;   // at least the candidates given
  auto ts_at = [&](int64_t j) { return j < h ? c.ts_hist[hs + j] : c.ts_cand[cs + (j - h)]; };
  int flags = 0;
  int64_t origin = 0;
  if (p.timestamps != nullptr && L > 0) {
    origin = ts_at(0) - ((int64_t)1 << 30);
    int64_t lo = INT64_MAX, hi = INT64_MIN;
    int32_t sorted = 1;
    for (int64_t j = threadIdx.x; j < L; j += blockDim.x) {
      const int64_t x = ts_at(j);
      lo = x < lo ? x : lo;
      hi = x > hi ? x : hi;
      if (j > 0 && ts_at(j - 1) > x) sorted = 0;
      c.ts_joined[vs + j] = x;
      p.ts_rel[vs + j] = (uint32_t)(x - origin);
    }
    lo = block_reduce(lo, lds64, MinOp());
    hi = block_reduce(hi, lds64, MaxOp());
    sorted = block_reduce(sorted, lds32, AndOp());
    const bool narrow = lo >= origin && (uint64_t)hi - (uint64_t)origin < 0x7fffffffull;
    if (!narrow) flags |= kSeqWideTs;
    if (sorted) flags |= kSeqSortedTs;
  }
  if (threadIdx.x == 0) {
    SeqInfo si;
    si.start = (int32_t)vs;
    si.len = L;
    si.hist = h;
    si.flags = flags;
    const int64_t n_norm = (int64_t)h + n_all;
    si.inv_len = n_norm > 0 ? 1.0f / (float)n_norm : 0.0f;
    si.nblk = m > 0 ? (L + kBlk - 1) / kBlk - h / kBlk : 0;
    si.ts_origin = origin;
    p.seq[b] = si;
    SeqCand sc;
    sc.hist_start = (int32_t)hs;
    sc.cand_start = (int32_t)cs;
    sc.pos_shift = first > (int64_t)1 << 30 ? 1 << 30 : (int32_t)first;
    sc.pad = 0;
    c.cand[b] = sc;
  }
}

// Inclusive prefix sum over the lanes of a wave (shuffles, no barrier).
template <typename V>
__device__ __forceinline__ V wave_scan_incl(V v) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const V t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

// Exclusive prefix sum of one value per thread over the workgroup (wave
// scans, then a scan of the wave totals by the first wave); lds holds at
// least blockDim.x / 64 + 1 values. Returns this thread's exclusive prefix
// and sets *total to the workgroup's sum. Ends with a barrier, so lds can
// be reused at once.
template <typename V>
__device__ V block_scan_one(V v, V* lds, V* total) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave, nw = blockDim.x / kWave;
  const V incl = wave_scan_incl(v);
  if (lane == kWave - 1) lds[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const V w = lane < nw ? lds[lane] : V(0);
    const V wi = wave_scan_incl(w);
    if (lane < nw) lds[lane] = wi - w;
    if (lane == kWave - 1) lds[nw] = wi;
  }
  __syncthreads();
  const V excl = lds[wave] + incl - v;
  *total = lds[nw];
  __syncthreads();
  return excl;
}

// Exclusive prefix sum over n ints in place (forward or from the end), one
// workgroup, chunks of blockDim.x with a running carry. Returns the total.
__device__ int block_scan_excl(int* data, int n, bool from_end, int* lds) {
  int carry = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int idx = base + threadIdx.x;
    const int pos = from_end ? n - 1 - idx : idx;
    const int v = idx < n ? data[pos] : 0;
    int total;
    const int excl = block_scan_one(v, lds, &total);
    if (idx < n) data[pos] = carry + excl;
    carry += total;
  }
  __syncthreads();
  return carry;
}

// Work list ordered longest first. A sequence with n blocks gives items
// x = 0..n-1 whose cost grows with x (forward: x is the query block index,
// the causal row block that sees the most keys; backward: x = n-1-key block,
// the key block that sees the most queries). Items are placed by x
// descending: start[x] = number of items with a larger x. Both orders hold
// the same multiset of x, so mode 2 places every item in both lists.
// Its arrays live in LDS when they fit (every access is then a short LDS
// round trip instead of a global one), else in the workspace scratch. One
// workgroup of any size up to kSchedThreads. Each sequence's block count and
// length come straight from the offsets (the values the sequence prep
// derives from them), so the schedule runs beside the prep in one launch.
// cand: candidate scoring against a cached history, whose rows are the
// history's and the call's candidates and whose scheduled blocks are those
// from the one holding the first candidate. mode 0: the forward order (query
// blocks, the last block first) into items; 2: the backward order (key
// blocks, the first block first) into items and the forward order into
// items_q, with the dS tile numbering and the export count.
constexpr int kSchedLds = 6144;

__device__ void schedule_body(const AttnParams& p, int mode, const CandArgs* cand) {
  __shared__ int lds[kSchedThreads];
  __shared__ int small[kSchedLds];
  const int B = p.B;
  auto len_of = [&](int b) {
    return cand ? (int)(cand->hist_offsets[b + 1] - cand->hist_offsets[b] +
                        cand->cand_offsets[b + 1] - cand->cand_offsets[b])
                : (int)(p.seq_offsets[b + 1] - p.seq_offsets[b]);
  };
  auto nblk_of = [&](int b) {
    if (!cand) return (len_of(b) + kBlk - 1) / kBlk;
    const int h = (int)(cand->hist_offsets[b + 1] - cand->hist_offsets[b]);
    const int m = (int)(cand->cand_offsets[b + 1] - cand->cand_offsets[b]);
    return m > 0 ? (h + m + kBlk - 1) / kBlk - h / kBlk : 0;
  };
  const int NB = (int)(p.T / kBlk) + 2;       // x ranges over [0, NB)
  int* seq_base = (B + 1 + 4 * NB <= kSchedLds) ? small : p.sched_scratch;   // [B + 1]
  int* hist = seq_base + (B + 1);               // [NB]: sequences with n blocks
  int* cnt = hist + NB;                         // [NB]: sequences with more than x blocks
  int* fill = cnt + NB;                         // [NB]
  int* fill_q = fill + NB;                      // [NB] (mode 2: forward-order list)
  for (int i = threadIdx.x; i < NB; i += blockDim.x) { hist[i] = 0; fill[i] = 0; fill_q[i] = 0; }
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int n = nblk_of(b);
    seq_base[b] = n;
    atomicAdd(&hist[n < NB ? n : NB - 1], 1);
  }
  __syncthreads();
  const int total = block_scan_excl(seq_base, B, false, lds);
  if (threadIdx.x == 0) seq_base[B] = total;
  // cnt[x] = sum_{n > x} hist[n]: exclusive scan from the end
  for (int i = threadIdx.x; i < NB; i += blockDim.x) cnt[i] = hist[i];
  __syncthreads();
  block_scan_excl(cnt, NB, true, lds);
  __syncthreads();
  // start[x] = sum_{x' > x} cnt[x'] (stored in hist)
  for (int i = threadIdx.x; i < NB; i += blockDim.x) hist[i] = cnt[i];
  __syncthreads();
  block_scan_excl(hist, NB, true, lds);
  __syncthreads();
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    int lo = 0, hi = B;                          // last b with seq_base[b] <= idx
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seq_base[mid] <= idx) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int blk = idx - seq_base[b];
    const int n = seq_base[b + 1] - seq_base[b];
    const int x = mode == 0 ? blk : n - 1 - blk;
    const int pos = hist[x] + atomicAdd(&fill[x], 1);
    WorkItem w;
    w.seq = b;
    w.blk = blk;
    p.items[pos] = w;
    if (mode == 2) p.items_q[hist[blk] + atomicAdd(&fill_q[blk], 1)] = w;
  }
  if (threadIdx.x == 0) *p.n_items = total;
  if (mode == 2 && p.blk_base != nullptr) {
    for (int b = threadIdx.x; b <= B; b += blockDim.x) p.blk_base[b] = seq_base[b];
  }
  if (mode == 2 && p.tile_base != nullptr) {
    // backward tile numbering: exclusive scan of H * ds_seq_tiles(L) over
    // the sequences, each thread a contiguous run of them
    __shared__ int64_t run[kSchedThreads / kWave + 1];
    __shared__ int cut;                          // first sequence whose tiles overflow ds_cap
    if (threadIdx.x == 0) cut = B;
    const int per = (B + (int)blockDim.x - 1) / (int)blockDim.x;
    const int b0 = threadIdx.x * per, b1 = b0 + per < B ? b0 + per : B;
    int64_t sum = 0;
    for (int b = b0; b < b1; ++b) sum += (int64_t)p.H * ds_seq_tiles(len_of(b));
    int64_t tiles;
    int64_t at = block_scan_one(sum, run, &tiles);   // (ends with a barrier)
    for (int b = b0; b < b1; ++b) {
      p.tile_base[b] = at;
      at += (int64_t)p.H * ds_seq_tiles(len_of(b));
      if (at > p.ds_cap) atomicMin(&cut, b);
    }
    __syncthreads();
    if (threadIdx.x == blockDim.x - 1) {
      if (p.ds_on) *p.ds_on = cut;
      if (p.det_on) *p.det_on = tiles <= p.part_cap ? 1 : 0;
    }
  }
}

// The forward's first launch: workgroup 0 builds the work list, workgroups
// 1..B prepare one sequence each; the two are independent.
__global__ __launch_bounds__(kSchedThreads) void fwd_prep_kernel(AttnParams p) {
  if (blockIdx.x == 0)
    schedule_body(p, 0, nullptr);
  else
    seq_prep_body(p, blockIdx.x - 1, p.B);
}

// The same for candidate scoring against a cached history.
__global__ __launch_bounds__(kSchedThreads) void cand_prep_kernel(AttnParams p, CandArgs c) {
  if (blockIdx.x == 0)
    schedule_body(p, 0, &c);
  else
    seq_prep_cand_body(p, c, blockIdx.x - 1);
}

// rab bucket export, laid out over the jagged lower triangle: sequence
// after sequence, query row i, then key j ascending (history rows i < hist
// see keys 0..i, candidate rows see the history and themselves).
//
// The kernel walks the export itself, not the rows. Each wave owns a run of
// up to kBktSteps steps of 512 consecutive slots (fewer for exports too
// small to give every wave of the grid a full run); lane l takes slots l, l + 64,
// ..., l + 448 of a step, so that the key-timestamp loads of a step are
// consecutive across the wave. The wave locates its run's first slot once
// (binary search over pair_offsets, staged in LDS for batches of up to
// kBktLdsSeqs sequences; the row in closed form, since history rows start
// at i (i + 1) / 2 and candidate rows follow with hist + 1 slots each) and
// then moves its position forward step by step in scalar registers. A step
// that lies within one row and holds no candidate's self term (nearly all
// of them for rows of a few thousand keys) is the fast path: position
// buckets from one base value, time buckets from 32-bit differences (a step
// where some |ts_i - ts_j| does not fit is redone in 64-bit arithmetic),
// the next step's key timestamps loaded before this step's arithmetic, and
// the step's buckets transposed through LDS so that each lane stores its 8
// consecutive slots with one 16-byte (bp) and one 8-byte (bt) store. Other
// steps (row ends, self terms, the export's last slots) and unaligned
// outputs go slot by slot, with 64-bit bucket arithmetic, exact for any
// int64 pair.
constexpr int kBktThreads = 256;
constexpr int kBktWaves = kBktThreads / kWave;
constexpr int kBktSlots = 8;                       // slots per lane and step
constexpr int kBktStep = kWave * kBktSlots;        // consecutive slots per step
constexpr int kBktSteps = 8;                       // most steps per wave run
constexpr int kBktGrid = 16384;
constexpr int kBktLdsSeqs = 2047;                  // pair_offsets in LDS up to this batch

__device__ __forceinline__ int64_t pairs_of(int L, int hist) {
  return (int64_t)hist * (hist + 1) / 2 + (int64_t)(L - hist) * (hist + 1);
}

__device__ __forceinline__ void seq_rows(const int64_t* seq_offsets, const int64_t* num_targets, int b,
                                         int64_t& s, int& L, int& hist) {
  s = seq_offsets[b];
  L = (int)(seq_offsets[b + 1] - s);
  int nt = num_targets ? (int)num_targets[b] : 0;
  nt = nt < 0 ? 0 : (nt > L ? L : nt);
  hist = L - nt;
}

// Row of local slot f of a sequence (0 <= f < its pairs) and the slot's key
// index within that row.
__device__ __forceinline__ void bkt_locate(int64_t f, int hist, int& i, int& k) {
  const int64_t h2 = (int64_t)hist * (hist + 1) / 2;
  if (f < h2) {
    // the largest i with i (i + 1) / 2 <= f, from the square root and then
    // corrected in integers
    int64_t r = (int64_t)((sqrt(8.0 * (double)f + 1.0) - 1.0) * 0.5);
    while (r * (r + 1) / 2 > f) --r;
    while ((r + 1) * (r + 2) / 2 <= f) ++r;
    i = (int)r;
    k = (int)(f - r * (r + 1) / 2);
  } else {
    const int64_t c = (f - h2) / (hist + 1);
    i = hist + (int)c;
    k = (int)(f - h2 - c * (hist + 1));
  }
}

// A position in the export: sequence b (first token s, L rows, hist history
// rows), query row i, key slot k of that row.
struct BktPos {
  int b, L, hist, i, k;
  int64_t s;
  bool cand;                 // i >= hist
  int n_r, p_i;              // slots of the row, position of its query
  int64_t ts_i;              // timestamp of the row's query (when timestamps are read)
};

__device__ __forceinline__ void bkt_row(BktPos& q, const int64_t* ts) {
  q.cand = q.i >= q.hist;
  q.n_r = q.cand ? q.hist + 1 : q.i + 1;
  q.p_i = q.cand ? q.hist : q.i;
  q.ts_i = ts ? ts[q.s + q.i] : 0;
}

// Moves q forward by n slots (into later rows and sequences as needed; the
// caller guarantees the target slot exists).
__device__ __forceinline__ void bkt_advance(BktPos& q, int n, const AttnParams& p) {
  q.k += n;
  while (q.k >= q.n_r) {
    q.k -= q.n_r;
    if (++q.i >= q.L) {
      do {
        ++q.b;
        seq_rows(p.seq_offsets, p.num_targets, q.b, q.s, q.L, q.hist);
      } while (q.L == 0);
      q.i = 0;
    }
    bkt_row(q, p.timestamps);
  }
}

// The kernel is bound by the latency of its steps, so it asks the compiler
// for a register budget that keeps many waves per SIMD in flight.
__global__ __launch_bounds__(kBktThreads) __attribute__((amdgpu_waves_per_eu(8)))
void bucketize_kernel(AttnParams p, const int64_t* pair_offsets, uint16_t* bp, uint8_t* bt, int vec) {
  __shared__ int64_t po_lds[kBktLdsSeqs + 1];
  __shared__ __attribute__((aligned(16))) uint16_t xp[kBktWaves][kBktStep];
  __shared__ __attribute__((aligned(16))) uint8_t xt[kBktWaves][kBktStep];
  const int B = p.B;
  const bool in_lds = B <= kBktLdsSeqs;
  if (in_lds)
    for (int x = threadIdx.x; x <= B; x += kBktThreads) po_lds[x] = pair_offsets[x];
  __syncthreads();
  const int64_t* const po = in_lds ? po_lds : pair_offsets;
  const int64_t P = po[B];
  const bool want_p = bp != nullptr, want_t = bt != nullptr;
  const int64_t* const tsg = want_t ? p.timestamps : nullptr;
  const int lim = p.max_len - 1;
  const int last = p.n_time_buckets - 1;
  const int lane = threadIdx.x % kWave;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  // steps per run: up to kBktSteps, fewer when the export is too small to
  // give every wave of the grid a run of that length
  const int64_t waves = (int64_t)gridDim.x * kBktWaves;
  const int64_t fill = (P + kBktStep * waves - 1) / (kBktStep * waves);
  const int steps = (int)(fill < kBktSteps ? (fill > 1 ? fill : 1) : kBktSteps);
  for (int64_t c = (int64_t)blockIdx.x * kBktWaves + wv; c * kBktStep * steps < P; c += waves) {
    int64_t F = c * kBktStep * steps;
    // the run's first slot: the last b with po[b] <= F (it has pairs, since
    // po[B] > F), then its row
    BktPos q;
    {
      int lo = 0, hi = B;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (po[mid] <= F) lo = mid; else hi = mid;
      }
      q.b = lo;
      seq_rows(p.seq_offsets, p.num_targets, q.b, q.s, q.L, q.hist);
      bkt_locate(F - po[q.b], q.hist, q.i, q.k);
      bkt_row(q, tsg);
    }
    int64_t tj[kBktSlots];
    bool have = false;                             // tj holds this step's key timestamps
    for (int st = 0; st < steps && F < P; ++st, F += kBktStep) {
      const int keys = q.cand ? q.hist : q.n_r;    // keys of the row before a self term
      if (vec && F + kBktStep <= P && q.k + kBktStep <= keys) {
        // the step's 512 slots are keys k .. k + 511 of one row
        int64_t cur[kBktSlots];
        if (want_t) {
          if (!have) {
            const int64_t* tk = tsg + q.s + q.k + lane;
#pragma unroll
            for (int m = 0; m < kBktSlots; ++m) tj[m] = tk[kWave * m];
          }
#pragma unroll
          for (int m = 0; m < kBktSlots; ++m) cur[m] = tj[m];
          // the next step's keys, when it stays in this row
          have = st + 1 < steps && F + 2 * kBktStep <= P && q.k + 2 * kBktStep <= keys;
          if (have) {
            const int64_t* tk = tsg + q.s + q.k + kBktStep + lane;
#pragma unroll
            for (int m = 0; m < kBktSlots; ++m) tj[m] = tk[kWave * m];
          }
          // d = ts_i - ts_j from 32-bit halves; it fits in 32 bits iff its
          // high word is the sign of its low word, and then |d| <= 2^31
          const uint32_t til = (uint32_t)q.ts_i, tih = (uint32_t)((uint64_t)q.ts_i >> 32);
          bool wide = false;
          uint32_t ev[kBktSlots];
#pragma unroll
          for (int m = 0; m < kBktSlots; ++m) {
            const uint32_t cl = (uint32_t)cur[m], chi = (uint32_t)((uint64_t)cur[m] >> 32);
            const uint32_t dl = til - cl;
            const uint32_t dh = tih - chi - (til < cl ? 1u : 0u);
            wide = wide || (int32_t)dh != ((int32_t)dl >> 31);
            const uint32_t a = ((int32_t)dl < 0 ? 0u - dl : dl) + 1u;
            const int e = 31 - __builtin_clz(a);
            ev[m] = (uint32_t)(e < last ? e : last);
          }
          if (__builtin_amdgcn_ballot_w64(wide) != 0) {
#pragma unroll
            for (int m = 0; m < kBktSlots; ++m) ev[m] = (uint32_t)time_bucket_wide(q.ts_i, cur[m], last);
          }
#pragma unroll
          for (int m = 0; m < kBktSlots; ++m) xt[wv][lane + kWave * m] = (uint8_t)ev[m];
        }
        if (want_p) {
          // keys k + o of the row sit at k + o - p_i <= 0: the bucket is
          // max(k + o - p_i + lim, 0)
          const int pbase = q.k - q.p_i + lim + lane;
#pragma unroll
          for (int m = 0; m < kBktSlots; ++m) xp[wv][lane + kWave * m] = (uint16_t)max(pbase + kWave * m, 0);
        }
        // lane l's slots 8 l .. 8 l + 7 of the step: one store each
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int64_t g = F + kBktSlots * lane;
        if (want_t) *reinterpret_cast<uint2*>(bt + g) = *reinterpret_cast<const uint2*>(&xt[wv][kBktSlots * lane]);
        if (want_p) st16(bp + g, *reinterpret_cast<const u32x4*>(&xp[wv][kBktSlots * lane]));
        __builtin_amdgcn_wave_barrier();
      } else {
        // slot by slot: lane l from slot F + l, then 64 slots on each time
        have = false;
        BktPos r = q;
        const int nv = (int)min((int64_t)kBktSlots, (P - F - lane + kWave - 1) / kWave);
        for (int m = 0; m < nv; ++m) {
          bkt_advance(r, m == 0 ? lane : kWave, p);
          const int j = (r.cand && r.k == r.hist) ? r.i : r.k;
          const int64_t f = F + lane + kWave * m;
          if (want_p) bp[f] = (uint16_t)pos_bucket(j - r.p_i, p.max_len);
          if (want_t) bt[f] = (uint8_t)time_bucket_wide(r.ts_i, tsg[r.s + j], last);
        }
      }
      if (F + kBktStep < P) bkt_advance(q, kBktStep, p);
    }
  }
}

// pair_offsets[b] = unmasked pairs of sequences 0..b-1, pair_offsets[B] = all
// of them (one workgroup, chunks of blockDim.x sequences with a running carry).
__global__ __launch_bounds__(kSchedThreads) void pair_offsets_kernel(const int64_t* seq_offsets,
                                                                     const int64_t* num_targets, int B,
                                                                     int64_t* out) {
  __shared__ int64_t lds[kSchedThreads / kWave + 1];
  int64_t carry = 0;
  for (int base = 0; base < B; base += blockDim.x) {
    const int idx = base + threadIdx.x;
    int64_t v = 0;
    if (idx < B) {
      int64_t s;
      int L, hist;
      seq_rows(seq_offsets, num_targets, idx, s, L, hist);
      v = pairs_of(L, hist);
    }
    int64_t total;
    const int64_t excl = block_scan_one(v, lds, &total);
    if (idx < B) out[idx] = carry + excl;
    carry += total;
  }
  if (threadIdx.x == 0) out[B] = carry;
}

__global__ void fill_f32_kernel(float* x, int64_t n, float value) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    x[i] = value;
}

// Sequence index of token t (last b with seq_offsets[b] <= t).
__device__ __forceinline__ int seq_of_token(const int64_t* offs, int B, int64_t t) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offs[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// dA' = dO * U / L (or dO / L without gate), dU = dO * A. Eight elements per
// thread, so every access is 16 bytes (bf16) or two of them (fp32). 1/L is
// formed from the offsets as the sequence prep forms it, so this needs none
// of the prep's outputs.
template <typename T> struct Vec8;
template <> struct Vec8<bf16> {
  static __device__ __forceinline__ void load(const bf16* p, float* f) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int m = 0; m < 8; ++m) f[m] = (float)v[m];
  }
  static __device__ __forceinline__ void store(bf16* p, const float* f) {
    bf16x8 v;
#pragma unroll
    for (int m = 0; m < 8; ++m) v[m] = (bf16)f[m];
    *reinterpret_cast<bf16x8*>(p) = v;
  }
};
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* f) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int m = 0; m < 4; ++m) { f[m] = a[m]; f[4 + m] = b[m]; }
  }
  static __device__ __forceinline__ void store(float* p, const float* f) {
    *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
  }
};

template <typename T>
__device__ void bwd_pre_body(const AttnParams& p, int blk, int n_blk) {
  const int HD = p.H * p.D;                      // a multiple of 32
  const int64_t n8 = p.T * HD / 8;
  for (int64_t q8 = (int64_t)blk * blockDim.x + threadIdx.x; q8 < n8;
       q8 += (int64_t)n_blk * blockDim.x) {
    const int64_t e0 = q8 * 8;
    const int64_t t = e0 / HD;
    const int hd = (int)(e0 - t * HD);
    const int b = seq_of_token(p.seq_offsets, p.B, t);
    const float inv = 1.0f / (float)(p.seq_offsets[b + 1] - p.seq_offsets[b]);
    float go[8], da[8];
    Vec8<T>::load(reinterpret_cast<const T*>(p.d_o) + e0, go);
    if (p.u != nullptr) {
      float uv[8], av[8], du[8];
      Vec8<T>::load(reinterpret_cast<const T*>(p.u) + t * p.su + hd, uv);
      Vec8<float>::load(p.a_in + e0, av);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        da[m] = go[m] * uv[m] * inv;
        du[m] = go[m] * av[m];
      }
      Vec8<T>::store(reinterpret_cast<T*>(p.du) + e0, du);
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) da[m] = go[m] * inv;
    }
    Vec8<T>::store(reinterpret_cast<T*>(p.d_a) + e0, da);
  }
}

// The backward's first launch: workgroup 0 builds both work lists and
// numbers the dS tiles, workgroups 1..B prepare one sequence each (and clear
// the rab gradient tables), the rest form dA' and dU. The three parts are
// independent, so the schedule's and the prep's latency run under the
// elementwise pass instead of in launches of their own.
template <typename T>
__global__ __launch_bounds__(kSchedThreads) void bwd_prep_kernel(AttnParams p) {
  if (blockIdx.x == 0)
    schedule_body(p, 2, nullptr);
  else if ((int)blockIdx.x <= p.B)
    seq_prep_body(p, blockIdx.x - 1, p.B);
  else
    bwd_pre_body<T>(p, blockIdx.x - 1 - p.B, gridDim.x - 1 - p.B);
}

int grid_for(int64_t n, int threads) {
  int64_t g = (n + threads - 1) / threads;
  if (g > 8192) g = 8192;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

size_t carve_workspace(AttnParams& p, void* base, bool bwd, int elem_bytes, bool ds_room) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return base ? (void*)((char*)base + at) : nullptr;
  };
  p.max_items = p.T / kBlk + p.B + 1;
  const int64_t NB = p.T / kBlk + 2;
  p.seq = (SeqInfo*)take(sizeof(SeqInfo) * (size_t)(p.B > 0 ? p.B : 1));
  p.ts_rel = (uint32_t*)take(sizeof(uint32_t) * (size_t)(p.T > 0 ? p.T : 1));
  p.items = (WorkItem*)take(sizeof(WorkItem) * (size_t)p.max_items);
  p.n_items = (int32_t*)take(sizeof(int32_t));
  p.sched_scratch = (int32_t*)take(sizeof(int32_t) * (size_t)(p.B + 1 + 4 * NB));
  p.items_q = nullptr;
  p.d_a = nullptr;
  p.tile_base = nullptr;
  p.blk_base = nullptr;
  p.ds = nullptr;
  p.ds_cap = 0;
  p.ds_on = nullptr;
  p.part_pos = nullptr;
  p.part_time = nullptr;
  p.part_cap = 0;
  p.det_on = nullptr;
  p.part_red = nullptr;
  if (bwd) {
    p.items_q = (WorkItem*)take(sizeof(WorkItem) * (size_t)p.max_items);
    p.d_a = take((size_t)elem_bytes * (size_t)p.T * p.H * p.D);
    const int64_t cap = (elem_bytes == 2 && ds_room) ? ds_capacity(p.T, p.B, p.H, p.max_len) : 0;
    const bool det = p.det != 0 && p.T > 0 && p.B > 0;
    if (cap > 0 || det) {
      p.tile_base = (int64_t*)take(sizeof(int64_t) * (size_t)p.B);
      int32_t* flags = (int32_t*)take(2 * sizeof(int32_t));
      p.ds_on = cap > 0 ? flags : nullptr;
      p.det_on = det && flags ? flags + 1 : nullptr;   // (no arithmetic on the sizing pass's null)
    }
    if (det) {
      p.blk_base = (int32_t*)take(sizeof(int32_t) * (size_t)(p.B + 1));
      p.part_cap = tile_capacity(p.T, p.B, p.H, p.max_len, ((int64_t)2 << 30) / (kPartW * 4));
      p.part_pos = (float*)take(sizeof(float) * kPartW * (size_t)p.part_cap);
      const int64_t slots = (p.T / kBlk + p.B) * (int64_t)p.H;
      p.part_time = (float*)take(sizeof(float) * (size_t)slots * (size_t)(p.n_time_room > 0 ? p.n_time_room : 1));
      const size_t n_red = 2 * (size_t)p.max_len - 1 + (size_t)(p.n_time_room > 0 ? p.n_time_room : 0);
      p.part_red = (float*)take(sizeof(float) * (size_t)kRedChunks * (size_t)p.H * n_red);
    }
    if (cap > 0) {
      p.ds_cap = cap;
      p.ds = take((size_t)cap * kDsTile * 2);
    }
  }
  return off;
}

// A sequence of L <= max_len rows holds ds_seq_tiles(L) <= nkb (nkb + 1)
// tiles per head, nkb = ceil(L / 128) <= ceil(max_len / 128); summed over
// the batch (sum of nkb <= T / 128 + B) that is at most
// (ceil(max_len / 128) + 1) (T / 128 + B) per head. The exact count is
// checked on the device, and a batch beyond the capacity (longer sequences
// than max_len, or beyond the 4 GiB cap) takes the recompute pass.
int64_t tile_capacity(int64_t T, int B, int H, int max_len, int64_t max_tiles) {
  if (T <= 0 || B <= 0) return 0;
  const int64_t len = max_len < T ? max_len : T;          // no sequence is longer than T
  const int64_t nkb = (len + kDsKeys - 1) / kDsKeys;
  const int64_t cap = (int64_t)H * (nkb + 1) * (T / kDsKeys + B);
  return cap < max_tiles ? cap : max_tiles;
}

int64_t ds_capacity(int64_t T, int B, int H, int max_len) {
  return tile_capacity(T, B, H, max_len, ((int64_t)4 << 30) / (kDsTile * 2));
}

// The forward's carve-up for the joined row count p.T, plus the per-sequence
// candidate records and, with a time bias, the joined 64-bit timestamps.
size_t carve_workspace_cand(AttnParams& p, CandArgs& c, void* base) {
  size_t off = carve_workspace(p, base, false, 2, false);
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return base ? (void*)((char*)base + at) : nullptr;
  };
  c.cand = (SeqCand*)take(sizeof(SeqCand) * (size_t)(p.B > 0 ? p.B : 1));
  c.ts_joined = (int64_t*)take(sizeof(int64_t) * (size_t)(p.T > 0 ? p.T : 1));
  p.part = nullptr;
  if (p.kv_splits > 1)
    p.part = (float*)take(sizeof(float) * (size_t)p.kv_splits * (size_t)p.m_rows * p.H * p.D);
  return off;
}

int cand_kv_splits(int64_t m_rows, int64_t hist_rows, int B, int H) {
  if (B <= 0 || m_rows <= 0) return 1;
  const int64_t blocks = (m_rows / kBlk + B) * H;          // query-block workgroups, at most
  const int64_t want = (2 * 256 + blocks - 1) / blocks;   // two workgroups per compute unit
  const int64_t by_len = hist_rows / ((int64_t)B * 512);  // >= 8 tiles of 64 keys per split
  int64_t s = want < by_len ? want : by_len;
  s = s < 1 ? 1 : (s > 16 ? 16 : s);
  return (int)s;
}

hipError_t launch_prep_cand(const AttnParams& p, const CandArgs& c, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  prof_before(kKPrep, s);
  hipLaunchKernelGGL(cand_prep_kernel, dim3(1 + p.B), dim3(kSchedThreads), 0, s, p, c);
  prof_after(kKPrep, s);
  return hipGetLastError();
}

hipError_t launch_bucketize(const AttnParams& p, const int64_t* pair_offsets, uint16_t* bp,
                            uint8_t* bt, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  prof_before(kKBucketize, s);
  // the fast path stores 8 slots per lane: 16 bytes of bp, 8 of bt
  const int vec = ((uintptr_t)bp % 16 == 0) && ((uintptr_t)bt % 8 == 0);
  hipLaunchKernelGGL(bucketize_kernel, dim3(kBktGrid), dim3(kBktThreads), 0, s, p, pair_offsets,
                     bp, bt, vec);
  prof_after(kKBucketize, s);
  return hipGetLastError();
}

hipError_t launch_pair_offsets(const int64_t* seq_offsets, const int64_t* num_targets, int B,
                               int64_t* out, hipStream_t s) {
  hipLaunchKernelGGL(pair_offsets_kernel, dim3(1), dim3(kSchedThreads), 0, s, seq_offsets,
                     num_targets, B, out);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* x, int64_t n, float value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  prof_before(kKFill, s);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, x, n, value);
  prof_after(kKFill, s);
  return hipGetLastError();
}

hipError_t launch_fwd_prep(const AttnParams& p, hipStream_t s) {
  prof_before(kKPrep, s);
  hipLaunchKernelGGL(fwd_prep_kernel, dim3(1 + p.B), dim3(kSchedThreads), 0, s, p);
  prof_after(kKPrep, s);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_prep(const AttnParams& p, hipStream_t s) {
  const int64_t n8 = p.T * p.H * p.D / 8;
  const int g = n8 > 0 ? grid_for(n8, kSchedThreads) : 1;
  prof_before(kKBwdPre, s);
  hipLaunchKernelGGL(bwd_prep_kernel<T>, dim3(1 + p.B + g), dim3(kSchedThreads), 0, s, p);
  prof_after(kKBwdPre, s);
  return hipGetLastError();
}

template hipError_t launch_bwd_prep<bf16>(const AttnParams&, hipStream_t);
template hipError_t launch_bwd_prep<float>(const AttnParams&, hipStream_t);

}  // namespace hstu
