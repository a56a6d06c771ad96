// Device-side building blocks shared by the gfx950 kernels of the jagged
// HSTU attention library: element types, MFMA fragment wrappers, rab bucket
// arithmetic and the per-sequence metadata the kernels read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace hstu {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kWave = 64;

// -log2(e) and -ln(2): SiLU(S) = S * sigma(S) with sigma(S) = 1 / (1 + 2^(S * -log2 e)).
constexpr float kNegLog2e = -1.4426950408889634f;
constexpr float kNegLn2 = -0.6931471805599453f;

// ---------------------------------------------------------------------------
// Fragments. Every MFMA operand in this library uses one register layout:
// lane l holds 8 consecutive reduction-dim elements k = 8*(l/32) + 0..7 of
// row (A) or column (B) l%32 of a 32 x 16 (or 16 x 32) operand block.
// For bf16 that is exactly the operand of v_mfma_f32_32x32x16_bf16. For fp32
// the same 8 values feed eight v_mfma_f32_32x32x2_f32, instruction m taking
// element m: its k-slot l/32 then stands for k = 8*(l/32) + m, the same
// pairing on both operands, so the sum over k is unchanged.
// Accumulator (32 x 32 fp32, 16 per lane): register r of lane l holds row
// 8*(r/4) + 4*(l/32) + (r%4), column l%32.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16> { typedef bf16x8 type; };
template <> struct Frag<float> { typedef f32x8 type; };

__device__ __forceinline__ void mfma_32x32x16(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ void mfma_32x32x16(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int m = 0; m < 8; ++m) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[m], b[m], acc, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }

// 8 accumulator values -> one fragment (bf16: round to nearest even).
template <typename T>
__device__ __forceinline__ typename Frag<T>::type pack8(const float* v) {
  typename Frag<T>::type f;
#pragma unroll
  for (int m = 0; m < 8; ++m) f[m] = from_f32<T>(v[m]);
  return f;
}

// Unaligned-free 16-byte global / LDS vector accesses.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

template <typename T>
__device__ __forceinline__ typename Frag<T>::type ld_frag(const T* p) {
  return *reinterpret_cast<const typename Frag<T>::type*>(p);
}

// Operand fragment gathered along the reduction dimension from a row-major
// LDS tile X (row = reduction index k, ld elements per row): lane l = 32g + c
// receives X[k][n0 + c] for the eight rows k = kr0 + 4g + {0..3} and
// kr1 + 4g + {0..3}. For bf16 this is two ds_read_b64_tr_b16: within each
// 16-lane group, lane s points at row (s >> 2) of a 4-row block and columns
// 4(s & 3)..4(s & 3)+3 of a 16-column block, and the transpose hands lane s
// column s of the block, rows 0..3. fp32 gathers element by element.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ bf16x8 ld_frag_kmajor(const bf16* X, int ld, int n0, int kr0, int kr1) {
  const int l = threadIdx.x & 63, s = l & 15, g = l >> 5;
  const int col = n0 + 16 * ((l >> 4) & 1) + 4 * (s & 3);
  const bf16* p0 = X + (kr0 + 4 * g + (s >> 2)) * ld + col;
  const bf16* p1 = X + (kr1 + 4 * g + (s >> 2)) * ld + col;
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p1));
  // joined as integers and cast once: element-wise bf16 casts of the
  // results were mis-compiled (every element became element 0)
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}

__device__ __forceinline__ f32x8 ld_frag_kmajor(const float* X, int ld, int n0, int kr0, int kr1) {
  const int l = threadIdx.x & 63, g = l >> 5, n = n0 + (l & 31);
  f32x8 f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    f[m] = X[(kr0 + 4 * g + m) * ld + n];
    f[4 + m] = X[(kr1 + 4 * g + m) * ld + n];
  }
  return f;
}

// Four consecutive elements <-> f32x4 (8-byte bf16 or 16-byte fp32 accesses).
__device__ __forceinline__ f32x4 ld4_f32(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 ld4_f32(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4_from_f32(bf16* p, f32x4 v) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
__device__ __forceinline__ void st4_from_f32(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Output tiles of the 128 x 128 GEMMs leave through LDS: the waves write
// their MFMA results at [row][col] with row stride tile_ld<T>() elements
// (rows 4 apart, written by the two lane halves, land 128 bytes apart in
// the banks), then the workgroup copies
// rows out as 16-byte chunks. Element-wise stores straight from the MFMA
// layout would write 2 or 4 bytes per lane, scattered over rows, and cost
// more than the whole reduction at short K.
template <typename T> __device__ __forceinline__ constexpr int tile_ld() { return 128 + 32 / (int)sizeof(T); }

// Copies rows [0, 128) x cols [0, 128) of the LDS tile t to y[m0 + r][n0 + c]
// (row stride ldy elements), skipping rows >= M and columns >= N; 256 threads.
template <typename T>
__device__ __forceinline__ void copy_tile_out(const T* t, T* __restrict__ y, int64_t ldy, int64_t m0,
                                              int64_t n0, int64_t M, int64_t N) {
  constexpr int EPC = 16 / (int)sizeof(T);       // elements per 16-byte chunk
  constexpr int CPR = 128 / EPC;                 // chunks per row
  const bool vec = ((uintptr_t)y % 16 == 0) && (ldy % EPC == 0);
  for (int c = (int)threadIdx.x; c < 128 * CPR; c += 256) {
    const int row = c / CPR, cc = c % CPR;
    const int64_t m = m0 + row, n = n0 + (int64_t)cc * EPC;
    if (m >= M || n >= N) continue;
    const T* src = t + row * tile_ld<T>() + cc * EPC;
    T* dst = y + m * ldy + n;
    if (vec && n + EPC <= N) {
      st16(dst, ld16(src));
    } else {
      for (int e = 0; e < EPC && n + e < N; ++e) dst[e] = src[e];
    }
  }
}

// Sum over the 64 lanes, returned to every lane. DPP adds within each 16-lane
// row (quad swaps, then half-row and row mirrors) stay in the VALU; the four
// row sums then come out through readlane. A shuffle ladder would instead make
// six LDS round trips, each waited on alone.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  int x = __builtin_bit_cast(int, v), y;
  switch (ctrl_sel) {
    case 0: y = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
    case 1: y = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
    case 2: y = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: y = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return v + __builtin_bit_cast(float, y);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int c = 0; c < 4; ++c) v = dpp_add(v, c);
  const int x = __builtin_bit_cast(int, v);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 48)));
}

// ---------------------------------------------------------------------------
// rab buckets. Position: clamp(j - p_i, -(max_len-1), max_len-1) + max_len-1.
// Time: min(bitlen(|dt| + 1) - 1, n_buckets - 1), exact in integers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int pos_bucket(int rel, int max_len) {
  const int lim = max_len - 1;
  rel = rel < -lim ? -lim : rel;
  rel = rel > lim ? lim : rel;
  return rel + lim;
}

// Rebased timestamps (offsets from a per-sequence origin) in [0, 2^31 - 1):
// |a - b| + 1 <= 2^31 - 1 cannot overflow.
__device__ __forceinline__ int time_bucket_rel(uint32_t a, uint32_t b, int last) {
  const uint32_t d = (a > b ? a - b : b - a) + 1u;
  const int bkt = 31 - __builtin_clz(d);
  return bkt < last ? bkt : last;
}

// Any pair of int64 timestamps (used for sequences whose span is too wide
// for the 32-bit form).
__device__ __forceinline__ int time_bucket_wide(int64_t a, int64_t b, int last) {
  const uint64_t d = a >= b ? (uint64_t)a - (uint64_t)b : (uint64_t)b - (uint64_t)a;
  const int bkt = (d == ~0ull) ? 64 : 63 - __builtin_clzll(d + 1ull);
  return bkt < last ? bkt : last;
}

// ---------------------------------------------------------------------------
// Per-sequence metadata (written by the prep kernel into the workspace).
// ---------------------------------------------------------------------------
enum : int32_t { kSeqWideTs = 1, kSeqSortedTs = 2 };

struct SeqInfo {
  int32_t start;    // first token of the sequence
  int32_t len;      // L
  int32_t hist;     // L - num_targets (history length)
  int32_t flags;    // kSeqWideTs | kSeqSortedTs
  float inv_len;    // 1 / L (0 for L == 0)
  int32_t nblk;     // ceil(L / 128): query blocks (forward) = key blocks (backward)
  int64_t ts_origin;  // rebasing origin of the 32-bit timestamps
};
static_assert(sizeof(SeqInfo) == 32, "SeqInfo layout");

// Candidate scoring against a cached history: where sequence b's rows live.
// Its rows are numbered as in the single-shot layout, history first
// (0..h-1, in k_hist / v_hist from hist_start) and then this call's
// candidates (h..h+m-1, in q / k / v / u from cand_start); pos_shift is the
// index of the first of them among all the sequence's candidates.
struct SeqCand {
  int32_t hist_start;
  int32_t cand_start;
  int32_t pos_shift;
  int32_t pad;
};

struct WorkItem {
  int32_t seq;
  int32_t blk;
};

// Both attention kernels tile a sequence in blocks of 128 tokens: 128 query
// rows per forward workgroup and 128 keys per backward workgroup.
constexpr int kBlk = 128;

// dS export of the bf16 backward: the key-block kernel writes, for every
// (key block kb, query tile qt) it visits, the tile dS^T [128 keys][64
// queries] (bf16); within each 32-query chunk of a key's row, position
// 8 q + 4 h + r holds query 16 h + 4 q + r (the key-block kernel's lane
// order, so that a lane's values are contiguous); the dQ pass reads them
// back and restores query order when it stages its output.
// Key block kb visits query tiles 2 kb .. nqt - 1 at most, so the tiles of
// one (sequence, head) are numbered row by row over that triangle.
constexpr int kDsKeys = 128, kDsQueries = 64;
constexpr int64_t kDsTile = (int64_t)kDsKeys * kDsQueries;    // elements per tile
__host__ __device__ inline int64_t ds_seq_tiles(int L) {
  const int64_t nkb = (L + kDsKeys - 1) / kDsKeys, nqt = (L + kDsQueries - 1) / kDsQueries;
  return nkb * nqt - nkb * (nkb - 1);
}
// index of tile (kb, 2 kb) within its (sequence, head)
__host__ __device__ inline int64_t ds_row_start(int L, int kb) {
  const int64_t nqt = (L + kDsQueries - 1) / kDsQueries;
  return (int64_t)kb * nqt - (int64_t)kb * (kb - 1);
}

}  // namespace hstu
