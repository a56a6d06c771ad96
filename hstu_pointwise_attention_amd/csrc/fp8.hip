// FP8 projection pieces, OCP E4M3FN codes (sign, 4 exponent bits with bias 7,
// 3 mantissa bits, largest finite 448), as the Generative Recommenders README
// ("FP8 linear reference and benchmark", and the HSTU Ultra stack it
// describes) names them: row-wise quantisation of activations, weights
// quantised once per output feature and kept, LayerNorm-and-gate with its
// output quantised in the same pass, and the FP8 GEMM with the row and
// column scales applied in the epilogue.
//
// Quantisation of a row: s = amax / 448 (1 for a row of zeros), codes =
// E4M3(x / s) rounded to nearest even; the scale and the quotient are IEEE
// fp32 divisions, so the codes are a deterministic function of the fp32
// inputs.
#include "internal.h"

namespace hstu {

namespace {

constexpr float kE4M3Max = 448.f;

__device__ __forceinline__ float clamp_e4m3(float v) { return fminf(fmaxf(v, -kE4M3Max), kE4M3Max); }

// Four fp32 values -> four E4M3 codes, the first in the lowest byte.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(a), clamp_e4m3(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp_e4m3(c), clamp_e4m3(d), w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// One wave per row of x (bf16, row stride ldx): scale[row] and the row's
// codes q[row][0..K). 8 elements per lane per step (K a multiple of 8).
__global__ __launch_bounds__(256) void quantize_rows_kernel(int64_t M, int64_t K, const bf16* __restrict__ x,
                                                            int64_t ldx, uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= M) return;
  const bf16* xr = x + row * ldx;
  float amax = 0.f;
  for (int64_t c = 8 * lane; c < K; c += 8 * kWave) {
    const u32x4 v = ld16(xr + c);
    const bf16* e = reinterpret_cast<const bf16*>(&v);
#pragma unroll
    for (int m = 0; m < 8; ++m) amax = fmaxf(amax, fabsf((float)e[m]));
  }
  amax = wave_max(amax);
  const float s = amax > 0.f ? amax / kE4M3Max : 1.f;
  if (lane == 0) scale[row] = s;
  uint8_t* qr = q + row * K;
  for (int64_t c = 8 * lane; c < K; c += 8 * kWave) {
    const u32x4 v = ld16(xr + c);
    const bf16* e = reinterpret_cast<const bf16*>(&v);
    float f[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) f[m] = (float)e[m] / s;
    uint2 out;
    out.x = cvt4_e4m3(f[0], f[1], f[2], f[3]);
    out.y = cvt4_e4m3(f[4], f[5], f[6], f[7]);
    *reinterpret_cast<uint2*>(qr + c) = out;
  }
}

// Weight w [K][N] (bf16, dense) quantised per output feature n: scale[n] and
// codes q[n][0..K) (the layout the GEMM reads, reduction index contiguous).
// One thread per column; a one-time preparation, not on the hot path.
__global__ __launch_bounds__(256) void prepare_weight_kernel(int64_t K, int64_t N, const bf16* __restrict__ w,
                                                             uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  float amax = 0.f;
  for (int64_t k = 0; k < K; ++k) amax = fmaxf(amax, fabsf((float)w[k * N + n]));
  const float s = amax > 0.f ? amax / kE4M3Max : 1.f;
  scale[n] = s;
  for (int64_t k = 0; k < K; k += 4) {
    const float a = (float)w[k * N + n] / s, b = (float)w[(k + 1) * N + n] / s;
    const float c = (float)w[(k + 2) * N + n] / s, d = (float)w[(k + 3) * N + n] / s;
    *reinterpret_cast<uint32_t*>(q + n * K + k) = cvt4_e4m3(a, b, c, d);
  }
}

// LayerNorm(a) * u per row (u == nullptr: no gate), quantised row-wise: one
// wave per row, four features per lane per step. z is formed by the same
// expression in the amax pass and in the quantising pass.
__global__ __launch_bounds__(256) void layernorm_gate_fp8_kernel(int64_t M, int64_t N, const float* __restrict__ a,
                                                                 const bf16* __restrict__ u, int64_t ldu, float eps,
                                                                 uint8_t* __restrict__ q,
                                                                 float* __restrict__ scale) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= M) return;
  const float* ar = a + row * N;
  float sum = 0.f;
  for (int64_t c = 4 * lane; c < N; c += 4 * kWave) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ar + c);
    sum += (v[0] + v[1]) + (v[2] + v[3]);
  }
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  const float mean = sum / (float)N;
  float var = 0.f;
  for (int64_t c = 4 * lane; c < N; c += 4 * kWave) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ar + c);
#pragma unroll
    for (int m = 0; m < 4; ++m) var += (v[m] - mean) * (v[m] - mean);
  }
  for (int off = 32; off > 0; off >>= 1) var += __shfl_xor(var, off);
  const float rstd = __frsqrt_rn(var / (float)N + eps);
  auto z4 = [&](int64_t c) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ar + c);
    const f32x4 g = u ? ld4_f32(u + row * ldu + c) : f32x4{1.f, 1.f, 1.f, 1.f};
    f32x4 z;
#pragma unroll
    for (int m = 0; m < 4; ++m) z[m] = (v[m] - mean) * rstd * g[m];
    return z;
  };
  float amax = 0.f;
  for (int64_t c = 4 * lane; c < N; c += 4 * kWave) {
    const f32x4 z = z4(c);
#pragma unroll
    for (int m = 0; m < 4; ++m) amax = fmaxf(amax, fabsf(z[m]));
  }
  amax = wave_max(amax);
  const float s = amax > 0.f ? amax / kE4M3Max : 1.f;
  if (lane == 0) scale[row] = s;
  for (int64_t c = 4 * lane; c < N; c += 4 * kWave) {
    const f32x4 z = z4(c);
    *reinterpret_cast<uint32_t*>(q + row * N + c) = cvt4_e4m3(z[0] / s, z[1] / s, z[2] / s, z[3] / s);
  }
}

// FP8 GEMM: y[m][n] = act(s_x[m] s_w[n] sum_k xq[m][k] wq[n][k] + bias[n]),
// both operands with the reduction index contiguous (xq [M][K], wq [N][K],
// dense). A workgroup computes a 128 x 128 tile, its four waves 64 x 64 each
// as 2 x 2 MFMA 32x32x64 (E4M3 x E4M3, fp32 accumulation, unit block
// scales), over 128 codes of the reduction per double-buffered LDS stage.
// A lane's operand is 32 consecutive codes of its row (two 16-byte LDS
// reads); A and B take the same byte positions, so each MFMA sums over the
// same 64 reduction indices for both. Tiles are dealt to the 8 XCDs in
// contiguous runs (as in the bf16 GEMM).
constexpr int QM = 128, QN = 128, QK = 128;
constexpr int QLD = QK + 16;                     // LDS row stride (bytes)

struct Fp8Smem {
  uint8_t a[2][QM * QLD];
  uint8_t b[2][QN * QLD];
};

typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void q_slab_load(u32x4 (&v)[4], const uint8_t* __restrict__ p, int64_t r0, int64_t R,
                                            int64_t k0, int64_t K, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    const int64_t r = r0 + (c >> 3), k = k0 + 16 * (c & 7);
    v[i] = (r < R && k < K) ? ld16(p + r * K + k) : u32x4{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void q_slab_store(uint8_t* t, const u32x4 (&v)[4], int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i;
    st16(t + (c >> 3) * QLD + 16 * (c & 7), v[i]);
  }
}

__device__ __forceinline__ v8i q_frag(const uint8_t* t, int rb, int kc) {
  const int l = threadIdx.x & 63;
  const uint8_t* p = t + (rb + (l & 31)) * QLD + 64 * kc + 32 * (l >> 5);
  const u32x4 lo = ld16(p), hi = ld16(p + 16);
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ float silu_q(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * kNegLog2e));
}

__global__ __launch_bounds__(256) void fp8_gemm_kernel(int64_t M, int64_t N, int64_t K,
                                                       const uint8_t* __restrict__ xq,
                                                       const float* __restrict__ x_scale,
                                                       const uint8_t* __restrict__ wq,
                                                       const float* __restrict__ w_scale,
                                                       const float* __restrict__ bias,
                                                       bf16* __restrict__ y, int apply_silu) {
  __shared__ Fp8Smem sm;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (N + QN - 1) / QN;
  const int64_t tiles = ((M + QM - 1) / QM) * tiles_n;
  int64_t t = blockIdx.x;
  if (tiles % 8 == 0) t = (t % 8) * (tiles / 8) + t / 8;
  const int64_t m0 = (t / tiles_n) * QM, n0 = (t % tiles_n) * QN;
  const int64_t nk = (K + QK - 1) / QK;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  u32x4 ra[4], rb[4];
  if (nk > 0) {
    q_slab_load(ra, xq, m0, M, 0, K, tid);
    q_slab_load(rb, wq, n0, N, 0, K, tid);
    q_slab_store(sm.a[0], ra, tid);
    q_slab_store(sm.b[0], rb, tid);
  }
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    const bool more = kt + 1 < nk;
    if (more) {
      q_slab_load(ra, xq, m0, M, (kt + 1) * QK, K, tid);
      q_slab_load(rb, wq, n0, N, (kt + 1) * QK, K, tid);
    }
#pragma unroll
    for (int c = 0; c < QK / 64; ++c) {
      v8i af[2], bfr[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) af[a] = q_frag(sm.a[buf], 64 * wm + 32 * a, c);
#pragma unroll
      for (int b = 0; b < 2; ++b) bfr[b] = q_frag(sm.b[buf], 64 * wn + 32 * b, c);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[a], bfr[b], acc[a][b], 0, 0, 0,
                                                                      127, 0, 127);
    }
    if (more) {
      q_slab_store(sm.a[buf ^ 1], ra, tid);
      q_slab_store(sm.b[buf ^ 1], rb, tid);
    }
    __syncthreads();
  }

  static_assert(128 * tile_ld<bf16>() * sizeof(bf16) <= sizeof(Fp8Smem), "output tile fits");
  bf16* ts = reinterpret_cast<bf16*>(&sm);
  float sx[2][16];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + 64 * wm + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
      sx[a][r] = m < M ? x_scale[m] : 0.f;
    }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int nl = 64 * wn + 32 * b + l32;
    const bool n_ok = n0 + nl < N;
    const float sw = n_ok ? w_scale[n0 + nl] : 0.f;
    const float bv = (bias && n_ok) ? bias[n0 + nl] : 0.f;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ml = 64 * wm + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
        float z = acc[a][b][r] * sx[a][r] * sw + bv;
        if (apply_silu) z = silu_q(z);
        ts[ml * tile_ld<bf16>() + nl] = (bf16)z;
      }
    }
  }
  __syncthreads();
  copy_tile_out(ts, y, N, m0, n0, M, N);
}

}  // namespace

hipError_t launch_fp8_quantize_rows(int64_t M, int64_t K, const void* x, int64_t ldx, void* q,
                                    float* scale, hipStream_t s) {
  if (M == 0) return hipSuccess;
  prof_before(kKFp8Quant, s);
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, M, K,
                     reinterpret_cast<const bf16*>(x), ldx, reinterpret_cast<uint8_t*>(q), scale);
  prof_after(kKFp8Quant, s);
  return hipGetLastError();
}

hipError_t launch_fp8_prepare_weight(int64_t K, int64_t N, const void* w, void* q, float* scale,
                                     hipStream_t s) {
  if (N == 0) return hipSuccess;
  hipLaunchKernelGGL(prepare_weight_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s, K, N,
                     reinterpret_cast<const bf16*>(w), reinterpret_cast<uint8_t*>(q), scale);
  return hipGetLastError();
}

hipError_t launch_fp8_linear(int64_t M, int64_t K, int64_t N, const void* xq, const float* x_scale,
                             const void* wq, const float* w_scale, const float* bias, void* y,
                             int apply_silu, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles = ((M + QM - 1) / QM) * ((N + QN - 1) / QN);
  prof_before(kKFp8Linear, s);
  hipLaunchKernelGGL(fp8_gemm_kernel, dim3((unsigned)tiles), dim3(256), 0, s, M, N, K,
                     reinterpret_cast<const uint8_t*>(xq), x_scale, reinterpret_cast<const uint8_t*>(wq),
                     w_scale, bias, reinterpret_cast<bf16*>(y), apply_silu);
  prof_after(kKFp8Linear, s);
  return hipGetLastError();
}

hipError_t launch_layernorm_gate_fp8(int64_t M, int64_t N, const float* a, const void* u,
                                     int64_t ldu, float eps, void* q, float* scale, hipStream_t s) {
  if (M == 0) return hipSuccess;
  prof_before(kKFp8Quant, s);
  hipLaunchKernelGGL(layernorm_gate_fp8_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, M, N, a,
                     reinterpret_cast<const bf16*>(u), ldu, eps, reinterpret_cast<uint8_t*>(q), scale);
  prof_after(kKFp8Quant, s);
  return hipGetLastError();
}

}  // namespace hstu
