// HSTU layer pieces around the attention, bf16 storage with fp32 accumulation:
//  - linear: y = act(x W + b), act = SiLU or identity (the UVQK projection and
//    the output projection);
//  - layernorm_gate: LayerNorm(a) * u over each token's features (the output
//    normalisation and gating).
#include "internal.h"

namespace hstu {

namespace {

constexpr int GM = 128, GN = 128, GK = 32;       // workgroup tile
constexpr int G_LD = GK + 8;                     // LDS row stride (elements): 80 bytes

struct GemmSmem {
  bf16 a[2][GM * G_LD];                          // x tile, row-major [m][k]
  bf16 bt[2][GN * G_LD];                         // W tile, transposed [n][k]
};

__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * kNegLog2e));
}

// Wave (wm, wn) of the 2 x 2 arrangement computes a 64 x 64 sub-tile as
// 2 x 2 blocks of 32 x 32.
__global__ __launch_bounds__(256) void linear_kernel(int64_t M, int64_t K, int64_t N,
                                                     const bf16* __restrict__ x, int64_t ldx,
                                                     const bf16* __restrict__ w,
                                                     const float* __restrict__ bias,
                                                     bf16* __restrict__ y, int apply_silu) {
  __shared__ GemmSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t n_tiles_n = N / GN;
  const int64_t m0 = (blockIdx.x / n_tiles_n) * GM;
  const int64_t n0 = (blockIdx.x % n_tiles_n) * GN;

  // staging: A = 128 rows x 4 chunks of 16 B -> 2 per thread;
  //          W = 16 k-pairs x 16 n-chunks -> 1 unit (2 loads) per thread.
  u32x4 areg[2], breg[2];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int ch = tid + 256 * m;
      const int row = ch >> 2, cc = ch & 3;
      const int64_t gm = m0 + row;
      areg[m] = gm < M ? ld16(x + gm * ldx + k0 + 8 * cc) : u32x4{0, 0, 0, 0};
    }
    const int kp = tid >> 4, nc = tid & 15;
    const bf16* src = w + (k0 + 2 * kp) * N + n0 + 8 * nc;
    breg[0] = ld16(src);
    breg[1] = ld16(src + N);
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int ch = tid + 256 * m;
      const int row = ch >> 2, cc = ch & 3;
      st16(sm.a[buf] + row * G_LD + 8 * cc, areg[m]);
    }
    const int kp = tid >> 4, nc = tid & 15;
    const bf16* r0 = reinterpret_cast<const bf16*>(&breg[0]);
    const bf16* r1 = reinterpret_cast<const bf16*>(&breg[1]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16* dst = sm.bt[buf] + (8 * nc + e) * G_LD + 2 * kp;
      dst[0] = r0[e];
      dst[1] = r1[e];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int64_t nk = K / GK;
  load(0);
  store(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    const bool more = kt + 1 < nk;
    if (more) load((kt + 1) * GK);
#pragma unroll
    for (int c = 0; c < GK / 16; ++c) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = ld_frag(sm.a[buf] + (64 * wm + 32 * a + l32) * G_LD + 16 * c + 8 * g);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bfr[b] = ld_frag(sm.bt[buf] + (64 * wn + 32 * b + l32) * G_LD + 16 * c + 8 * g);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) mfma_32x32x16(acc[a][b], af[a], bfr[b]);
    }
    if (more) store(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t n = n0 + 64 * wn + 32 * b + l32;
    const float bv = bias ? bias[n] : 0.f;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + 64 * wm + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
        if (m < M) {
          float z = acc[a][b][r] + bv;
          if (apply_silu) z = silu_f(z);
          y[m * N + n] = (bf16)z;
        }
      }
    }
  }
}

// One wave per token row.
__global__ __launch_bounds__(256) void layernorm_gate_kernel(int64_t M, int64_t N, const float* __restrict__ a,
                                                             const bf16* __restrict__ u, int64_t ldu,
                                                             float eps, bf16* __restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (row >= M) return;
  const float* ar = a + row * N;
  float s = 0.f;
  for (int64_t c = 4 * lane; c < N; c += 4 * kWave) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ar + c);
    s += (v[0] + v[1]) + (v[2] + v[3]);
  }
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  const float mean = s / (float)N;
  float q = 0.f;
  for (int64_t c = 4 * lane; c < N; c += 4 * kWave) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ar + c);
#pragma unroll
    for (int m = 0; m < 4; ++m) q += (v[m] - mean) * (v[m] - mean);
  }
  for (int off = 32; off > 0; off >>= 1) q += __shfl_xor(q, off);
  const float rstd = __frsqrt_rn(q / (float)N + eps);
  for (int64_t c = 4 * lane; c < N; c += 4 * kWave) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ar + c);
    const f32x4 uv = ld4_f32(u + row * ldu + c);
    f32x4 o;
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] = (v[m] - mean) * rstd * uv[m];
    st4_from_f32(out + row * N + c, o);
  }
}

}  // namespace

hipError_t launch_linear(int64_t M, int64_t K, int64_t N, const void* x, int64_t ldx,
                         const void* w, const float* bias, void* y, int apply_silu,
                         hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t grid = ((M + GM - 1) / GM) * (N / GN);
  prof_before(kKLinear, s);
  hipLaunchKernelGGL(linear_kernel, dim3((unsigned)grid), dim3(256), 0, s, M, K, N,
                     reinterpret_cast<const bf16*>(x), ldx, reinterpret_cast<const bf16*>(w),
                     bias, reinterpret_cast<bf16*>(y), apply_silu);
  prof_after(kKLinear, s);
  return hipGetLastError();
}

hipError_t launch_layernorm_gate(int64_t M, int64_t N, const float* a, const void* u,
                                 int64_t ldu, float eps, void* out, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t grid = (M + 3) / 4;
  prof_before(kKLayerNorm, s);
  hipLaunchKernelGGL(layernorm_gate_kernel, dim3((unsigned)grid), dim3(256), 0, s, M, N, a,
                     reinterpret_cast<const bf16*>(u), ldu, eps, reinterpret_cast<bf16*>(out));
  prof_after(kKLayerNorm, s);
  return hipGetLastError();
}

}  // namespace hstu
