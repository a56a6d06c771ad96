// Small kernels around the attention: per-sequence metadata and timestamp
// rebasing, the longest-first work schedule, the rab bucket export, and the
// elementwise passes before and after the fused backward.
#include "internal.h"

namespace hstu {

namespace {

constexpr int kPrepThreads = 256;
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

// Smallest / largest timestamp and sortedness of tokens [s, e).
struct TsStats { int64_t lo, hi; int32_t sorted; };

__device__ TsStats ts_stats(const int64_t* ts, int64_t s, int64_t e, int64_t* lds64, int32_t* lds32) {
  int64_t lo = INT64_MAX, hi = INT64_MIN;
  int32_t sorted = 1;
  // four rounds of loads in flight per step: the loop is latency-bound
  constexpr int U = 4;
  for (int64_t t0 = s + threadIdx.x; t0 < e; t0 += U * (int64_t)blockDim.x) {
    int64_t x[U], y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = t0 + u * (int64_t)blockDim.x;
      x[u] = t < e ? ts[t] : 0;
      y[u] = (t < e && t > s) ? ts[t - 1] : INT64_MIN;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t0 + u * (int64_t)blockDim.x < e) {
        lo = x[u] < lo ? x[u] : lo;
        hi = x[u] > hi ? x[u] : hi;
        if (y[u] > x[u]) sorted = 0;
      }
    }
  }
  TsStats r;
  r.lo = block_reduce(lo, lds64, MinOp());
  r.hi = block_reduce(hi, lds64, MaxOp());
  r.sorted = block_reduce(sorted, lds32, AndOp());
  return r;
}

// A sequence whose timestamp span reaches 2^31 - 1 uses 64-bit bucket math.
__device__ __forceinline__ bool span_is_wide(int64_t lo, int64_t hi) {
  return (uint64_t)hi - (uint64_t)lo >= 0x7fffffffull;
}

// One workgroup per sequence: metadata + rebased timestamps. In the backward
// the workgroups also clear the rab gradient tables (overwritten outputs).
__global__ __launch_bounds__(kSeqPrepThreads) void seq_prep_kernel(AttnParams p) {
  __shared__ int64_t lds64[kSeqPrepThreads / kWave];
  __shared__ int32_t lds32[kSeqPrepThreads / kWave];
  {
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if (p.d_rab_pos) {
      const int64_t n = (int64_t)p.rab_heads * (2 * (int64_t)p.max_len - 1);
      for (int64_t i = i0; i < n; i += stride) p.d_rab_pos[i] = 0.f;
    }
    if (p.d_rab_time) {
      const int64_t n = (int64_t)p.rab_heads * p.n_time_buckets;
      for (int64_t i = i0; i < n; i += stride) p.d_rab_time[i] = 0.f;
    }
  }
  const int b = blockIdx.x;
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
// to c.ts_joined (64-bit) and p.ts_rel (rebased, as in seq_prep_kernel).
// Normalisation is 1 / (h + n) over all n candidates of the sequence, and
// only query blocks holding candidates are scheduled (nblk counts blocks
// from the one holding row h).
__global__ __launch_bounds__(kSeqPrepThreads) void seq_prep_cand_kernel(AttnParams p, CandArgs c) {
  __shared__ int64_t lds64[kSeqPrepThreads / kWave];
  __shared__ int32_t lds32[kSeqPrepThreads / kWave];
  const int b = blockIdx.x;
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

// Exclusive prefix sum over n ints in place (forward or from the end), one
// workgroup, chunks of blockDim.x with a running carry. Returns the total.
__device__ int block_scan_excl(int* data, int n, bool from_end, int* lds) {
  int carry = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int idx = base + threadIdx.x;
    const int pos = from_end ? n - 1 - idx : idx;
    const int v = idx < n ? data[pos] : 0;
    lds[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < (int)blockDim.x; off <<= 1) {
      const int add = threadIdx.x >= (unsigned)off ? lds[threadIdx.x - off] : 0;
      __syncthreads();
      lds[threadIdx.x] += add;
      __syncthreads();
    }
    const int incl = lds[threadIdx.x];
    const int total = lds[blockDim.x - 1];
    if (idx < n) data[pos] = carry + incl - v;
    carry += total;
    __syncthreads();
  }
  return carry;
}

// Work list ordered longest first. A sequence with n blocks gives items
// x = 0..n-1 whose cost grows with x (forward: x is the query block index,
// the causal row block that sees the most keys; backward: x = n-1-key block,
// the key block that sees the most queries). Items are placed by x
// descending: start[x] = number of items with a larger x. Both orders hold
// the same multiset of x, so mode 2 places every item in both lists.
// Its arrays live in LDS when they fit (every access is then a short LDS
// round trip instead of a global one), else in the workspace scratch.
constexpr int kSchedLds = 6144;

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(AttnParams p, int mode) {
  __shared__ int lds[kSchedThreads];
  __shared__ int small[kSchedLds];
  const int B = p.B;
  const int NB = (int)(p.T / kBlk) + 2;       // x ranges over [0, NB)
  int* seq_base = (B + 1 + 4 * NB <= kSchedLds) ? small : p.sched_scratch;   // [B + 1]
  int* hist = seq_base + (B + 1);               // [NB]: sequences with n blocks
  int* cnt = hist + NB;                         // [NB]: sequences with more than x blocks
  int* fill = cnt + NB;                         // [NB]
  int* fill_q = fill + NB;                      // [NB] (mode 2: forward-order list)
  for (int i = threadIdx.x; i < NB; i += blockDim.x) { hist[i] = 0; fill[i] = 0; fill_q[i] = 0; }
  __syncthreads();
  if (threadIdx.x == 0) lds[0] = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const SeqInfo si = p.seq[b];
    const int n = si.nblk;
    seq_base[b] = n;
    atomicAdd(&hist[n < NB ? n : NB - 1], 1);
    if (si.flags & kSeqWideTs) atomicAdd(&lds[0], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) p.n_items[1] = lds[0];
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
  if (mode == 2 && p.ds != nullptr) {
    // dS tile numbering: exclusive scan of H * ds_seq_tiles(L) over the
    // sequences, each thread a contiguous run of them
    __shared__ int64_t run[kSchedThreads];
    const int per = (B + kSchedThreads - 1) / kSchedThreads;
    const int b0 = threadIdx.x * per, b1 = b0 + per < B ? b0 + per : B;
    int64_t sum = 0;
    for (int b = b0; b < b1; ++b) sum += (int64_t)p.H * ds_seq_tiles(p.seq[b].len);
    run[threadIdx.x] = sum;
    __syncthreads();
    for (int off = 1; off < kSchedThreads; off <<= 1) {
      const int64_t add = threadIdx.x >= off ? run[threadIdx.x - off] : 0;
      __syncthreads();
      run[threadIdx.x] += add;
      __syncthreads();
    }
    int64_t at = threadIdx.x > 0 ? run[threadIdx.x - 1] : 0;
    for (int b = b0; b < b1; ++b) {
      p.ds_base[b] = at;
      at += (int64_t)p.H * ds_seq_tiles(p.seq[b].len);
    }
    if (threadIdx.x == kSchedThreads - 1) *p.ds_on = run[kSchedThreads - 1] <= p.ds_cap ? 1 : 0;
  }
}

// rab bucket export: grid (64 row groups, B sequences).
__global__ __launch_bounds__(kPrepThreads) void bucketize_kernel(AttnParams p, const int64_t* pair_offsets,
                                                                  uint16_t* bp, uint8_t* bt) {
  __shared__ int64_t lds64[kPrepThreads / kWave];
  __shared__ int32_t lds32[kPrepThreads / kWave];
  const int b = blockIdx.y;
  const int64_t s = p.seq_offsets[b];
  const int64_t e = p.seq_offsets[b + 1];
  const int L = (int)(e - s);
  int nt = p.num_targets ? (int)p.num_targets[b] : 0;
  nt = nt < 0 ? 0 : (nt > L ? L : nt);
  const int hist = L - nt;
  bool wide = false;
  int64_t lo = 0;
  const bool want_t = bt != nullptr;
  if (want_t && L > 0) {
    TsStats st = ts_stats(p.timestamps, s, e, lds64, lds32);
    lo = st.lo;
    wide = span_is_wide(st.lo, st.hi);
  }
  const int last = p.n_time_buckets - 1;
  const int64_t base = pair_offsets[b];
  const int64_t hist_pairs = (int64_t)hist * (hist + 1) / 2;
  for (int i = blockIdx.x; i < L; i += gridDim.x) {
    const int64_t row = i < hist ? (int64_t)i * (i + 1) / 2
                                 : hist_pairs + (int64_t)(i - hist) * (hist + 1);
    const int n = i < hist ? i + 1 : hist + 1;
    const int pi = i < hist ? i : hist;
    for (int c = threadIdx.x; c < n; c += blockDim.x) {
      const int j = (i < hist || c < hist) ? c : i;
      const int64_t o = base + row + c;
      if (bp) bp[o] = (uint16_t)pos_bucket(j - pi, p.max_len);
      if (want_t) {
        const int64_t ti = p.timestamps[s + i], tj = p.timestamps[s + j];
        bt[o] = (uint8_t)(wide ? time_bucket_wide(ti, tj, last)
                               : time_bucket_rel((uint32_t)(ti - lo), (uint32_t)(tj - lo), last));
      }
    }
  }
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
// thread, so every access is 16 bytes (bf16) or two of them (fp32).
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
__global__ __launch_bounds__(256) void bwd_pre_kernel(AttnParams p) {
  const int HD = p.H * p.D;                      // a multiple of 32
  const int64_t n8 = p.T * HD / 8;
  for (int64_t q8 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q8 < n8;
       q8 += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = q8 * 8;
    const int64_t t = e0 / HD;
    const int hd = (int)(e0 - t * HD);
    const float inv = p.seq[seq_of_token(p.seq_offsets, p.B, t)].inv_len;
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


int grid_for(int64_t n, int threads) {
  int64_t g = (n + threads - 1) / threads;
  if (g > 8192) g = 8192;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

size_t carve_workspace(AttnParams& p, void* base, bool bwd, int elem_bytes) {
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
  p.n_items = (int32_t*)take(2 * sizeof(int32_t));
  p.sched_scratch = (int32_t*)take(sizeof(int32_t) * (size_t)(p.B + 1 + 4 * NB));
  p.items_q = nullptr;
  p.d_a = nullptr;
  p.ds = nullptr;
  p.ds_cap = 0;
  p.ds_base = nullptr;
  p.ds_on = nullptr;
  if (bwd) {
    p.items_q = (WorkItem*)take(sizeof(WorkItem) * (size_t)p.max_items);
    p.d_a = take((size_t)elem_bytes * (size_t)p.T * p.H * p.D);
    const int64_t cap = (elem_bytes == 2 && BWD_K16) ? ds_capacity(p.T, p.B, p.H, p.max_len) : 0;
    if (cap > 0) {
      p.ds_cap = cap;
      p.ds_base = (int64_t*)take(sizeof(int64_t) * (size_t)p.B);
      p.ds_on = (int32_t*)take(sizeof(int32_t));
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
int64_t ds_capacity(int64_t T, int B, int H, int max_len) {
  if (T <= 0 || B <= 0) return 0;
  const int64_t nkb = (max_len + kDsKeys - 1) / kDsKeys;
  int64_t cap = (int64_t)H * (nkb + 1) * (T / kDsKeys + B);
  const int64_t max_tiles = ((int64_t)4 << 30) / (kDsTile * 2);
  return cap < max_tiles ? cap : max_tiles;
}

// The forward's carve-up for the joined row count p.T, plus the per-sequence
// candidate records and, with a time bias, the joined 64-bit timestamps.
size_t carve_workspace_cand(AttnParams& p, CandArgs& c, void* base) {
  size_t off = carve_workspace(p, base, false, 2);
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
  hipLaunchKernelGGL(seq_prep_cand_kernel, dim3(p.B), dim3(kSeqPrepThreads), 0, s, p, c);
  prof_after(kKPrep, s);
  return hipGetLastError();
}

hipError_t launch_prep(const AttnParams& p, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  prof_before(kKPrep, s);
  hipLaunchKernelGGL(seq_prep_kernel, dim3(p.B), dim3(kSeqPrepThreads), 0, s, p);
  prof_after(kKPrep, s);
  return hipGetLastError();
}

hipError_t launch_schedule(const AttnParams& p, int mode, hipStream_t s) {
  prof_before(kKSchedule, s);
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, s, p, mode);
  prof_after(kKSchedule, s);
  return hipGetLastError();
}

hipError_t launch_bucketize(const AttnParams& p, const int64_t* pair_offsets, uint16_t* bp,
                            uint8_t* bt, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  prof_before(kKBucketize, s);
  hipLaunchKernelGGL(bucketize_kernel, dim3(64, p.B), dim3(kPrepThreads), 0, s, p, pair_offsets,
                     bp, bt);
  prof_after(kKBucketize, s);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* x, int64_t n, float value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  prof_before(kKFill, s);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, x, n, value);
  prof_after(kKFill, s);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_pre(const AttnParams& p, hipStream_t s) {
  const int64_t n8 = p.T * p.H * p.D / 8;
  if (n8 == 0) return hipSuccess;
  prof_before(kKBwdPre, s);
  hipLaunchKernelGGL(bwd_pre_kernel<T>, dim3(grid_for(n8, 256)), dim3(256), 0, s, p);
  prof_after(kKBwdPre, s);
  return hipGetLastError();
}

template hipError_t launch_bwd_pre<bf16>(const AttnParams&, hipStream_t);
template hipError_t launch_bwd_pre<float>(const AttnParams&, hipStream_t);

}  // namespace hstu
