// Tile pieces of the 128 x 128 MFMA GEMMs (layer projections and their
// gradients, and the dQ pass over exported dS tiles).
#pragma once
#include "common.h"

namespace hstu {
namespace {

// GEMM tiles: a workgroup computes a TM x TN block of the output, its four
// waves 64 x 64 each as 2 x 2 blocks of 32 x 32 (MFMA 32x32x16 bf16), over
// TK reduction indices per double-buffered LDS stage.
constexpr int TM = 128, TN = 128, TK = 64;

// An operand is stored either with the reduction index contiguous (KC: A as
// [M][K], B as [N][K]) or strided (KS: A as [K][M], B as [K][N]). Its LDS tile
// keeps the memory layout (16-byte copies, no transposes): KC tiles are
// [128][TK] at row stride LDK, read as 16-byte row fragments; KS tiles are
// [TK][128] at row stride LDT, read by transposing LDS loads. Both strides
// keep the respective fragment reads free of bank conflicts.
enum { KC = 0, KS = 1 };
constexpr int LDK = TK + 8;
constexpr int LDT = 128 + 16;
constexpr int TILE = 128 * LDK;
static_assert(TILE == TK * LDT, "both tile shapes fill one buffer");

struct GemmSmem {
  bf16 a[2][TILE];
  bf16 b[2][TILE];
};

// The TK x 128 slab of one operand at reduction indices k0..k0+TK-1 and rows
// (m of A, n of B) r0..r0+127, as four 16-byte chunks per thread; elements at
// k >= k_end or row >= R read as 0.
template <int L>
__device__ __forceinline__ void slab_load(u32x4 (&v)[4], const bf16* __restrict__ p, int64_t ld,
                                          int64_t r0, int64_t R, int64_t k0, int64_t k_end,
                                          int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    if constexpr (L == KC) {                     // 8 chunks of 8 k per row
      const int64_t r = r0 + (c >> 3), k = k0 + 8 * (c & 7);
      v[i] = (r < R && k < k_end) ? ld16(p + r * ld + k) : u32x4{0, 0, 0, 0};
    } else {                                     // 16 chunks of 8 rows per k
      const int64_t k = k0 + (c >> 4), r = r0 + 8 * (c & 15);
      v[i] = (k < k_end && r < R) ? ld16(p + k * ld + r) : u32x4{0, 0, 0, 0};
    }
  }
}

template <int L>
__device__ __forceinline__ void slab_store(bf16* t, const u32x4 (&v)[4], int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    if constexpr (L == KC)
      st16(t + (c >> 3) * LDK + 8 * (c & 7), v[i]);
    else
      st16(t + (c >> 4) * LDT + 8 * (c & 15), v[i]);
  }
}

// MFMA operand of tile rows rb..rb+31 at reduction indices kr..kr+15: lane
// 32g + c holds row rb + c, indices kr + 8g .. kr + 8g + 7. For a KS tile
// these are two transposing reads: in each 16-lane group, lane s addresses
// row kr + 8g + (s >> 2) (then 4 rows further) at columns rb + 16((lane >> 4) & 1)
// + 4(s & 3) .. +3, and receives column rb + (lane & 31) of the four rows.
template <int L>
__device__ __forceinline__ bf16x8 slab_frag(const bf16* t, int rb, int kr) {
  const int l = threadIdx.x & 63, g = l >> 5;
  if constexpr (L == KC) {
    return ld_frag(t + (rb + (l & 31)) * LDK + kr + 8 * g);
  } else {
    const int s = l & 15;
    const bf16* p0 = t + (kr + 8 * g + (s >> 2)) * LDT + rb + 16 * ((l >> 4) & 1) + 4 * (s & 3);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 4 * LDT));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const v8i16 f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, f);
  }
}

}  // namespace
}  // namespace hstu
