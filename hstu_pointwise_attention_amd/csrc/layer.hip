// HSTU layer pieces around the attention, bf16 storage with fp32 accumulation:
//  - linear: y = act(x W + b), act = SiLU or identity (the UVQK projection and
//    the output projection; in the backward, with fp32 output, the weight
//    gradients from transposed operands);
//  - layernorm_gate: LayerNorm(a) * u over each token's features (the output
//    normalisation and gating), and its backward;
//  - the backward's small pieces: transposes, row padding, column sums and
//    the SiLU derivative of the UVQK projection.
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
template <typename OutT>
__global__ __launch_bounds__(256) void linear_kernel(int64_t M, int64_t K, int64_t N,
                                                     const bf16* __restrict__ x, int64_t ldx,
                                                     const bf16* __restrict__ w,
                                                     const float* __restrict__ bias,
                                                     OutT* __restrict__ y, int apply_silu) {
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
          y[m * N + n] = (OutT)z;
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

// Backward of out = LayerNorm(a) * u, one wave per token row (unit scale,
// zero shift): with xh = (a - mean) * rstd,
//   du = dout * xh,  dln = dout * u,
//   da = rstd * (dln - mean(dln) - xh * mean(dln * xh)).
__global__ __launch_bounds__(256) void layernorm_gate_bwd_kernel(
    int64_t M, int64_t N, const float* __restrict__ a, const bf16* __restrict__ u, int64_t ldu,
    float eps, const bf16* __restrict__ dout, bf16* __restrict__ da, bf16* __restrict__ du) {
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
  float g1 = 0.f, g2 = 0.f;                      // sums of dln and dln * xh
  for (int64_t c = 4 * lane; c < N; c += 4 * kWave) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ar + c);
    const f32x4 uv = ld4_f32(u + row * ldu + c);
    const f32x4 dv = ld4_f32(dout + row * N + c);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float dln = dv[m] * uv[m];
      g1 += dln;
      g2 += dln * (v[m] - mean) * rstd;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    g1 += __shfl_xor(g1, off);
    g2 += __shfl_xor(g2, off);
  }
  g1 /= (float)N;
  g2 /= (float)N;
  for (int64_t c = 4 * lane; c < N; c += 4 * kWave) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(ar + c);
    const f32x4 uv = ld4_f32(u + row * ldu + c);
    const f32x4 dv = ld4_f32(dout + row * N + c);
    f32x4 oa, ou;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float xh = (v[m] - mean) * rstd;
      ou[m] = dv[m] * xh;
      oa[m] = rstd * (dv[m] * uv[m] - g1 - xh * g2);
    }
    st4_from_f32(da + row * N + c, oa);
    st4_from_f32(du + row * N + c, ou);
  }
}

// y[c][r] = x[r][c] for r < R, 0 for R <= r < ldy (columns of y padded to
// ldy); 64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void transpose_pad_kernel(int64_t R, int64_t C,
                                                           const bf16* __restrict__ x, int64_t ldx,
                                                           bf16* __restrict__ y, int64_t ldy) {
  __shared__ bf16 t[64][65];
  const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    t[i][tx] = (r < R && c < C) ? x[r * ldx + c] : (bf16)0.f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < C && r < ldy) y[c * ldy + r] = t[tx][i];
  }
}

// y[r][:] = x[r][:] for r < M, 0 for M <= r < Mp; N a multiple of 8.
__global__ __launch_bounds__(256) void copy_pad_rows_kernel(int64_t M, int64_t Mp, int64_t N,
                                                            const bf16* __restrict__ x, int64_t ldx,
                                                            bf16* __restrict__ y) {
  const int64_t n8 = N / 8;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < Mp * n8;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / n8, c = 8 * (e - r * n8);
    const u32x4 v = r < M ? ld16(x + r * ldx + c) : u32x4{0, 0, 0, 0};
    st16(y + r * N + c, v);
  }
}

// out[c] += sum over rows r of x[r][c] (fp32 atomics; out cleared by the
// caller): each thread one column of a 256-row chunk.
__global__ __launch_bounds__(256) void colsum_kernel(int64_t M, int64_t N, const bf16* __restrict__ x,
                                                     int64_t ldx, float* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= N) return;
  const int64_t r0 = (int64_t)blockIdx.y * 256, r1 = r0 + 256 < M ? r0 + 256 : M;
  float sum = 0.f;
  for (int64_t r = r0; r < r1; ++r) sum += (float)x[r * ldx + c];
  atomicAdd(out + c, sum);
}

// d_pre[m][c] = g[m][c] * SiLU'(pre[m][c]) over the 4 * HD columns of the
// UVQK projection, g taken from the column block's gradient (dU, dV, dQ, dK,
// each [M, HD] dense); rows M..Mp-1 of d_pre are 0. 8 columns per thread.
__global__ __launch_bounds__(256) void silu_bwd_uvqk_kernel(int64_t M, int64_t Mp, int64_t HD,
                                                            const bf16* __restrict__ pre,
                                                            const bf16* __restrict__ g0,
                                                            const bf16* __restrict__ g1,
                                                            const bf16* __restrict__ g2,
                                                            const bf16* __restrict__ g3,
                                                            bf16* __restrict__ d_pre) {
  const int64_t W = 4 * HD, n8 = W / 8;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < Mp * n8;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = e / n8, c = 8 * (e - r * n8);
    u32x4 outv = {0, 0, 0, 0};
    if (r < M) {
      const int64_t part = c / HD, cc = c - part * HD;
      const bf16* g = part == 0 ? g0 : part == 1 ? g1 : part == 2 ? g2 : g3;
      const u32x4 zv = ld16(pre + r * W + c), gv = ld16(g + r * HD + cc);
      const bf16* z8 = reinterpret_cast<const bf16*>(&zv);
      const bf16* g8 = reinterpret_cast<const bf16*>(&gv);
      bf16* o8 = reinterpret_cast<bf16*>(&outv);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float z = (float)z8[m];
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * kNegLog2e));
        o8[m] = (bf16)((float)g8[m] * sg * (1.0f + z * (1.0f - sg)));
      }
    }
    st16(d_pre + r * W + c, outv);
  }
}

}  // namespace

hipError_t launch_linear(int64_t M, int64_t K, int64_t N, const void* x, int64_t ldx,
                         const void* w, const float* bias, void* y, int apply_silu,
                         hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t grid = ((M + GM - 1) / GM) * (N / GN);
  prof_before(kKLinear, s);
  hipLaunchKernelGGL(linear_kernel<bf16>, dim3((unsigned)grid), dim3(256), 0, s, M, K, N,
                     reinterpret_cast<const bf16*>(x), ldx, reinterpret_cast<const bf16*>(w),
                     bias, reinterpret_cast<bf16*>(y), apply_silu);
  prof_after(kKLinear, s);
  return hipGetLastError();
}

hipError_t launch_linear_f32(int64_t M, int64_t K, int64_t N, const void* x, int64_t ldx,
                             const void* w, float* y, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const int64_t grid = ((M + GM - 1) / GM) * (N / GN);
  prof_before(kKLinear, s);
  hipLaunchKernelGGL(linear_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s, M, K, N,
                     reinterpret_cast<const bf16*>(x), ldx, reinterpret_cast<const bf16*>(w),
                     nullptr, y, 0);
  prof_after(kKLinear, s);
  return hipGetLastError();
}

hipError_t launch_layernorm_gate_bwd(int64_t M, int64_t N, const float* a, const void* u,
                                     int64_t ldu, float eps, const void* dout, void* da, void* du,
                                     hipStream_t s) {
  if (M == 0) return hipSuccess;
  prof_before(kKLayerNorm, s);
  hipLaunchKernelGGL(layernorm_gate_bwd_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, M, N, a,
                     reinterpret_cast<const bf16*>(u), ldu, eps, reinterpret_cast<const bf16*>(dout),
                     reinterpret_cast<bf16*>(da), reinterpret_cast<bf16*>(du));
  prof_after(kKLayerNorm, s);
  return hipGetLastError();
}

hipError_t launch_transpose_pad(int64_t R, int64_t C, const void* x, int64_t ldx, void* y,
                                int64_t ldy, hipStream_t s) {
  if (C == 0 || ldy == 0) return hipSuccess;
  const dim3 g((unsigned)((ldy + 63) / 64), (unsigned)((C + 63) / 64));
  hipLaunchKernelGGL(transpose_pad_kernel, g, dim3(256), 0, s, R, C, reinterpret_cast<const bf16*>(x),
                     ldx, reinterpret_cast<bf16*>(y), ldy);
  return hipGetLastError();
}

hipError_t launch_copy_pad_rows(int64_t M, int64_t Mp, int64_t N, const void* x, int64_t ldx,
                                void* y, hipStream_t s) {
  if (Mp == 0) return hipSuccess;
  const int64_t n = Mp * (N / 8), blocks = (n + 255) / 256;
  hipLaunchKernelGGL(copy_pad_rows_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, s,
                     M, Mp, N, reinterpret_cast<const bf16*>(x), ldx, reinterpret_cast<bf16*>(y));
  return hipGetLastError();
}

hipError_t launch_colsum(int64_t M, int64_t N, const void* x, int64_t ldx, float* out, hipStream_t s) {
  hipError_t e = launch_fill_f32(out, N, 0.f, s);
  if (e != hipSuccess || M == 0) return e;
  const dim3 g((unsigned)((N + 255) / 256), (unsigned)((M + 255) / 256));
  hipLaunchKernelGGL(colsum_kernel, g, dim3(256), 0, s, M, N, reinterpret_cast<const bf16*>(x), ldx, out);
  return hipGetLastError();
}

hipError_t launch_silu_bwd_uvqk(int64_t M, int64_t Mp, int64_t HD, const void* pre, const void* g0,
                                const void* g1, const void* g2, const void* g3, void* d_pre,
                                hipStream_t s) {
  if (Mp == 0) return hipSuccess;
  const int64_t n = Mp * (4 * HD / 8), blocks = (n + 255) / 256;
  hipLaunchKernelGGL(silu_bwd_uvqk_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, s,
                     M, Mp, HD, reinterpret_cast<const bf16*>(pre), reinterpret_cast<const bf16*>(g0),
                     reinterpret_cast<const bf16*>(g1), reinterpret_cast<const bf16*>(g2),
                     reinterpret_cast<const bf16*>(g3), reinterpret_cast<bf16*>(d_pre));
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
