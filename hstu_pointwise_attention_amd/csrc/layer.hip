// HSTU layer pieces around the attention, bf16 storage with fp32 accumulation:
//  - GEMM: y = act(x W + b), act = SiLU or identity (the UVQK projection and
//    the output projection); in the backward, x W^T (input gradients) and
//    x^T g with fp32 output split over the token axis (weight gradients);
//  - layernorm_gate: LayerNorm(a) * u over each token's features (the output
//    normalisation and gating), and its backward;
//  - the backward's small pieces: column sums (bias gradients) and the SiLU
//    derivative of the UVQK projection.
#include "internal.h"
#include "gemm_tile.h"

namespace hstu {

namespace {

__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * kNegLog2e));
}

struct GemmArgs {
  int64_t M, N, K;
  const bf16* a;                                 // A operand (rows m), layout LA
  int64_t lda;
  const bf16* b;                                 // B operand (columns n), layout LB
  int64_t ldb;
  const float* bias;                             // [N] or nullptr
  void* y;                                       // [M][N] dense; with a K split, fp32 partials [split][M][N]
  int64_t k_split;                               // reduction indices per split (multiple of TK)
  int apply_silu;
};

// y[m][n] = act(sum_k A(m, k) B(k, n) + bias[n]) over one TM x TN tile and one
// split of the reduction (blockIdx.y). Tiles are numbered row-major and, when
// their count is a multiple of 8, dealt out so that each of the 8 XCDs (which
// receive workgroups round-robin) takes a contiguous run of them: the tiles
// of one row band then share that XCD's L2.
template <int LA, int LB, typename OutT>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  __shared__ GemmSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t tiles_n = (p.N + TN - 1) / TN;
  const int64_t tiles = ((p.M + TM - 1) / TM) * tiles_n;
  int64_t t = blockIdx.x;
  if (tiles % 8 == 0) t = (t % 8) * (tiles / 8) + t / 8;
  const int64_t m0 = (t / tiles_n) * TM, n0 = (t % tiles_n) * TN;
  const int64_t kb = (int64_t)blockIdx.y * p.k_split;
  const int64_t ke = kb + p.k_split < p.K ? kb + p.k_split : p.K;
  const int64_t nk = ke > kb ? (ke - kb + TK - 1) / TK : 0;

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // Stage kt is in LDS buffer kt & 1 while stage kt + 1 arrives in registers.
  u32x4 ra[4], rb[4];
  if (nk > 0) {
    slab_load<LA>(ra, p.a, p.lda, m0, p.M, kb, ke, tid);
    slab_load<LB>(rb, p.b, p.ldb, n0, p.N, kb, ke, tid);
    slab_store<LA>(sm.a[0], ra, tid);
    slab_store<LB>(sm.b[0], rb, tid);
  }
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = (int)(kt & 1);
    const bool more = kt + 1 < nk;
    if (more) {
      slab_load<LA>(ra, p.a, p.lda, m0, p.M, kb + (kt + 1) * TK, ke, tid);
      slab_load<LB>(rb, p.b, p.ldb, n0, p.N, kb + (kt + 1) * TK, ke, tid);
    }
    const bf16* ta = sm.a[buf];
    const bf16* tb = sm.b[buf];
#pragma unroll
    for (int c = 0; c < TK / 16; ++c) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) af[a] = slab_frag<LA>(ta, 64 * wm + 32 * a, 16 * c);
#pragma unroll
      for (int b = 0; b < 2; ++b) bfr[b] = slab_frag<LB>(tb, 64 * wn + 32 * b, 16 * c);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) mfma_32x32x16(acc[a][b], af[a], bfr[b]);
    }
    if (more) {
      slab_store<LA>(sm.a[buf ^ 1], ra, tid);
      slab_store<LB>(sm.b[buf ^ 1], rb, tid);
    }
    __syncthreads();
  }

  // The loop's last barrier has retired every read of the stage buffers, so
  // the output tile is staged in their place.
  static_assert(128 * tile_ld<OutT>() * sizeof(OutT) <= sizeof(GemmSmem), "output tile fits");
  OutT* ts = reinterpret_cast<OutT*>(&sm);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int nl = 64 * wn + 32 * b + l32;
    const float bv = (p.bias && n0 + nl < p.N) ? p.bias[n0 + nl] : 0.f;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ml = 64 * wm + 32 * a + 8 * (r >> 2) + 4 * g + (r & 3);
        float z = acc[a][b][r] + bv;
        if (p.apply_silu) z = silu_f(z);
        ts[ml * tile_ld<OutT>() + nl] = (OutT)z;
      }
    }
  }
  __syncthreads();
  copy_tile_out(ts, reinterpret_cast<OutT*>(p.y) + (int64_t)blockIdx.y * p.M * p.N, p.N, m0, n0, p.M, p.N);
}

// out[e] = sum over s < splits of part[s * stride + e], four floats per thread.
__global__ __launch_bounds__(256) void split_sum_kernel(int64_t n4, int splits, int64_t stride,
                                                        const float* __restrict__ part,
                                                        float* __restrict__ out) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4;
       e += (int64_t)gridDim.x * blockDim.x) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(part + 4 * e);
    for (int sp = 1; sp < splits; ++sp) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(part + sp * stride + 4 * e);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] += v[m];
    }
    *reinterpret_cast<f32x4*>(out + 4 * e) = acc;
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

// Column sums in two deterministic passes. colsum_kernel: part[band][c] =
// sum of x[r][c] over the band's 128 rows; threads take 8 columns each
// (16-byte loads), cw threads across the column chunks of the block and
// 256 / cw rows at a time, the row groups then summed through LDS.
// rows_sum_kernel: out[c] = sum over bands of part[band][c], 32 float4
// column chunks x 8 band lanes per block.
constexpr int kColsumRows = 128;

__global__ __launch_bounds__(256) void colsum_kernel(int64_t M, int64_t N, const bf16* __restrict__ x,
                                                     int64_t ldx, float* __restrict__ part) {
  __shared__ float red[256 * 8];
  const int64_t n8 = N / 8;
  const int cw = n8 < 256 ? (int)n8 : 256, nr = 256 / cw;
  const int tid = threadIdx.x, cx = tid % cw, ry = tid / cw;
  const int64_t c = (int64_t)blockIdx.x * cw + cx;
  const int64_t r0 = (int64_t)blockIdx.y * kColsumRows;
  const int64_t r1 = r0 + kColsumRows < M ? r0 + kColsumRows : M;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (ry < nr && c < n8) {
#pragma unroll 4
    for (int64_t r = r0 + ry; r < r1; r += nr) {
      const u32x4 v = ld16(x + r * ldx + 8 * c);
      const bf16* e = reinterpret_cast<const bf16*>(&v);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] += (float)e[m];
    }
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) red[tid * 8 + m] = acc[m];
  __syncthreads();
  if (ry == 0 && c < n8) {
    for (int k = 1; k < nr; ++k)
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] += red[(k * cw + cx) * 8 + m];
    float* dst = part + (int64_t)blockIdx.y * N + 8 * c;
    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

__global__ __launch_bounds__(256) void rows_sum_kernel(int64_t R, int64_t N, const float* __restrict__ part,
                                                       float* __restrict__ out) {
  __shared__ f32x4 red[256];
  const int tid = threadIdx.x, cx = tid & 31, ry = tid >> 5;
  const int64_t c4 = (int64_t)blockIdx.x * 32 + cx;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (4 * c4 < N)
    for (int64_t r = ry; r < R; r += 8) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(part + r * N + 4 * c4);
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] += v[m];
    }
  red[tid] = acc;
  __syncthreads();
  if (ry == 0 && 4 * c4 < N) {
    for (int k = 1; k < 8; ++k)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[m] += red[32 * k + cx][m];
    *reinterpret_cast<f32x4*>(out + 4 * c4) = acc;
  }
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

namespace {

template <int LA, int LB, typename OutT>
hipError_t launch_gemm(const GemmArgs& g, int splits, hipStream_t s) {
  const int64_t tiles = ((g.M + TM - 1) / TM) * ((g.N + TN - 1) / TN);
  prof_before(kKLinear, s);
  hipLaunchKernelGGL((gemm_kernel<LA, LB, OutT>), dim3((unsigned)tiles, (unsigned)splits), dim3(256), 0, s, g);
  prof_after(kKLinear, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(int64_t M, int64_t K, int64_t N, const void* x, int64_t ldx,
                         const void* w, const float* bias, void* y, int apply_silu,
                         hipStream_t s) {
  if (M == 0) return hipSuccess;
  const GemmArgs g = {M, N, K, reinterpret_cast<const bf16*>(x), ldx,
                      reinterpret_cast<const bf16*>(w), N, bias, y, K, apply_silu};
  return launch_gemm<KC, KS, bf16>(g, 1, s);
}

hipError_t launch_linear_nt(int64_t M, int64_t K, int64_t N, const void* x, int64_t ldx,
                            const void* w, int64_t ldw, void* y, hipStream_t s) {
  if (M == 0) return hipSuccess;
  const GemmArgs g = {M, N, K, reinterpret_cast<const bf16*>(x), ldx,
                      reinterpret_cast<const bf16*>(w), ldw, nullptr, y, K, 0};
  return launch_gemm<KC, KC, bf16>(g, 1, s);
}

// Splits of the reduction for a weight gradient: enough workgroups to cover
// the chip about three times over, at least 8 stages of TK per split.
int wgrad_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
  int64_t sp = (768 + tiles - 1) / tiles;
  const int64_t by_k = K / (8 * TK);
  if (sp > by_k) sp = by_k;
  if (sp > 64) sp = 64;
  return sp < 1 ? 1 : (int)sp;
}

hipError_t launch_wgrad(int64_t M, int64_t N, int64_t K, const void* a, int64_t lda, const void* b,
                        int64_t ldb, float* y, float* part, hipStream_t s) {
  const int splits = wgrad_splits(M, N, K);
  int64_t k_split = (K + splits - 1) / splits;
  k_split = (k_split + TK - 1) / TK * TK;
  const GemmArgs g = {M, N, K, reinterpret_cast<const bf16*>(a), lda,
                      reinterpret_cast<const bf16*>(b), ldb, nullptr,
                      splits > 1 ? (void*)part : (void*)y, k_split, 0};
  hipError_t e = launch_gemm<KS, KS, float>(g, splits, s);
  if (e != hipSuccess || splits == 1) return e;
  const int64_t n4 = M * N / 4, blocks = (n4 + 255) / 256;
  hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                     n4, splits, M * N, part, y);
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

int64_t colsum_bands(int64_t M) { return (M + kColsumRows - 1) / kColsumRows; }

hipError_t launch_colsum(int64_t M, int64_t N, const void* x, int64_t ldx, float* out, float* part,
                         hipStream_t s) {
  if (M == 0) return launch_fill_f32(out, N, 0.f, s);
  const int64_t n8 = N / 8, cw = n8 < 256 ? n8 : 256, bands = colsum_bands(M);
  const dim3 g((unsigned)((n8 + cw - 1) / cw), (unsigned)bands);
  hipLaunchKernelGGL(colsum_kernel, g, dim3(256), 0, s, M, N, reinterpret_cast<const bf16*>(x), ldx, part);
  hipLaunchKernelGGL(rows_sum_kernel, dim3((unsigned)((N / 4 + 31) / 32)), dim3(256), 0, s, bands, N,
                     (const float*)part, out);
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
