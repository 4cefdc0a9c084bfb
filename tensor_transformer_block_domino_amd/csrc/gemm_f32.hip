// fp32 path of the MLP shard's products (vector-ALU FMA, LDS-tiled) and the elementwise
// activation kernels it pairs with, plus the GEMM entry that picks the bf16 MFMA path or
// this one. The fp32 path serves small fp32 layers; its activation steps run as separate
// elementwise passes (same formulas as the bf16 path's fused epilogues).
#include "common.hpp"
#include "kernels.hpp"

namespace domino {

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s, GemmSplit* split);
hipError_t launch_gemm_bf16_fixup(const GemmArgs& g, const GemmSplit& split, hipStream_t s);
int64_t gemm_bf16_ws_elems(const GemmArgs& g);

namespace {

constexpr int kTile = 64, kKt = 16;

struct F32Params {
  const float* A; int64_t lda;
  const float* B; int64_t ldb;
  float* C; int64_t ldc;
  int64_t M, N, K;
  int accumulate;
};

// C(m, n) (+)= Σ_k A(m, k)·B(k, n); 64×64 tile per 256 threads, 4×4 outputs per thread.
template <bool kAK, bool kBK>
__global__ __launch_bounds__(256) void gemm_f32_kernel(F32Params p) {
  __shared__ float As[kKt][kTile + 1];
  __shared__ float Bs[kKt][kTile + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = int64_t(blockIdx.y) * kTile, n0 = int64_t(blockIdx.x) * kTile;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < p.K; k0 += kKt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      // Walk the contiguous dimension fastest for coalescing.
      const int mm = kAK ? idx / kKt : idx % kTile, kk = kAK ? idx % kKt : idx / kTile;
      const int64_t gm = m0 + mm, gk = k0 + kk;
      As[kk][mm] = (gm < p.M && gk < p.K) ? (kAK ? p.A[gm * p.lda + gk] : p.A[gk * p.lda + gm]) : 0.0f;
      const int nn = kBK ? idx / kKt : idx % kTile, kb = kBK ? idx % kKt : idx / kTile;
      const int64_t gn = n0 + nn, gkb = k0 + kb;
      Bs[kb][nn] = (gn < p.N && gkb < p.K) ? (kBK ? p.B[gn * p.ldb + gkb] : p.B[gkb * p.ldb + gn]) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKt; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n >= p.N) continue;
      float* dst = p.C + m * p.ldc + n;
      *dst = p.accumulate ? *dst + acc[i][j] : acc[i][j];
    }
  }
}

hipError_t gemm_f32(const float* A, int64_t lda, bool ak, const float* B, int64_t ldb, bool bk, float* C,
                    int64_t ldc, int64_t M, int64_t N, int64_t K, int accumulate, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  F32Params p{A, lda, B, ldb, C, ldc, M, N, K, accumulate};
  dim3 grid(unsigned((N + kTile - 1) / kTile), unsigned((M + kTile - 1) / kTile));
  note_kernel("gemm_f32_kernel");
  if (ak && bk) DOMINO_LAUNCH((gemm_f32_kernel<true, true>), grid, dim3(256), 0, s, p);
  else if (ak && !bk) DOMINO_LAUNCH((gemm_f32_kernel<true, false>), grid, dim3(256), 0, s, p);
  else if (!ak && bk) DOMINO_LAUNCH((gemm_f32_kernel<false, true>), grid, dim3(256), 0, s, p);
  else DOMINO_LAUNCH((gemm_f32_kernel<false, false>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// H from Hpre: GeLU elementwise, or SwiGLU H[m, j] = silu(Hpre[m, j])·Hpre[m, f + j].
template <bool kSwiglu>
__global__ void act_fwd_f32_kernel(const float* __restrict__ hpre, int64_t ldp, float* __restrict__ h, int64_t ldh,
                                   int64_t rows, int64_t f) {
  const int64_t total = rows * f;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t m = i / f, j = i - m * f;
    const float x = hpre[m * ldp + j];
    h[m * ldh + j] = kSwiglu ? silu_f(x) * hpre[m * ldp + f + j] : gelu_tanh_f(x);
  }
}

// In place on dHpre: on entry columns [0, f) hold dH; on exit dHpre = act'(Hpre) ⊙ dH
// (SwiGLU: dgate in [0, f), dup in [f, 2f)).
template <bool kSwiglu>
__global__ void act_bwd_f32_kernel(const float* __restrict__ hpre, int64_t ldp, float* dhpre, int64_t ldd,
                                   int64_t rows, int64_t f) {
  const int64_t total = rows * f;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t m = i / f, j = i - m * f;
    const float dh = dhpre[m * ldd + j];
    if (kSwiglu) {
      const float g = hpre[m * ldp + j], u = hpre[m * ldp + f + j];
      const float sg = sigmoidf_(g);
      dhpre[m * ldd + j] = dh * u * sg * (1.0f + g * (1.0f - sg));
      dhpre[m * ldd + f + j] = dh * g * sg;
    } else {
      dhpre[m * ldd + j] = dh * gelu_tanh_grad_f(hpre[m * ldp + j]);
    }
  }
}

unsigned grid_for(int64_t total) {
  const int64_t b = (total + 255) / 256;
  return unsigned(b < 4096 ? (b ? b : 1) : 4096);
}

hipError_t launch_gemm_f32_path(const GemmArgs& g, hipStream_t s, int* launches) {
  const float* A = static_cast<const float*>(g.A);
  const float* B = static_cast<const float*>(g.B);
  float* C = static_cast<float*>(g.C);
  hipError_t e = hipSuccess;
  *launches = 0;
  switch (g.epi) {
    case Epi::kStore:
    case Epi::kF32:
      e = gemm_f32(A, g.lda, g.a_kcontig, B, g.ldb, g.b_kcontig, C, g.ldc, g.M, g.N, g.K,
                   g.epi == Epi::kF32 ? g.accumulate : 0, s);
      *launches = 1;
      return e;
    case Epi::kGelu:
    case Epi::kSwiglu: {
      const bool sw = g.epi == Epi::kSwiglu;
      e = gemm_f32(A, g.lda, g.a_kcontig, B, g.ldb, g.b_kcontig, C, g.ldc, g.M, sw ? 2 * g.f_s : g.N, g.K, 0, s);
      if (e != hipSuccess) return e;
      const int64_t f = sw ? g.f_s : g.N;
      note_kernel("gemm_f32_kernel + act_fwd_f32_kernel");
      if (sw)
        DOMINO_LAUNCH((act_fwd_f32_kernel<true>), dim3(grid_for(g.M * f)), dim3(256), 0, s, C, g.ldc,
                           static_cast<float*>(g.C2), g.ldc2, g.M, f);
      else
        DOMINO_LAUNCH((act_fwd_f32_kernel<false>), dim3(grid_for(g.M * f)), dim3(256), 0, s, C, g.ldc,
                           static_cast<float*>(g.C2), g.ldc2, g.M, f);
      *launches = 2;
      return hipGetLastError();
    }
    case Epi::kDGelu:
    case Epi::kDSwiglu: {
      e = gemm_f32(A, g.lda, g.a_kcontig, B, g.ldb, g.b_kcontig, C, g.ldc, g.M, g.N, g.K, 0, s);
      if (e != hipSuccess) return e;
      const float* hp = static_cast<const float*>(g.aux);
      note_kernel("gemm_f32_kernel + act_bwd_f32_kernel");
      if (g.epi == Epi::kDSwiglu)
        DOMINO_LAUNCH((act_bwd_f32_kernel<true>), dim3(grid_for(g.M * g.N)), dim3(256), 0, s, hp, g.ldaux, C,
                           g.ldc, g.M, g.N);
      else
        DOMINO_LAUNCH((act_bwd_f32_kernel<false>), dim3(grid_for(g.M * g.N)), dim3(256), 0, s, hp, g.ldaux, C,
                           g.ldc, g.M, g.N);
      *launches = 2;
      return hipGetLastError();
    }
  }
  return hipErrorInvalidValue;
}

__global__ void fill_zero_f32_kernel(float* out, int64_t ld, int64_t rows, int64_t cols) {
  const int64_t total = rows * cols;
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t m = i / cols;
    out[m * ld + (i - m * cols)] = 0.0f;
  }
}

}  // namespace

hipError_t launch_fill_zero_f32(float* out, int64_t ld, int64_t rows, int64_t cols, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  note_kernel("fill_zero_f32_kernel");
  DOMINO_LAUNCH(fill_zero_f32_kernel, dim3(grid_for(rows * cols)), dim3(256), 0, s, out, ld, rows, cols);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s, GemmSplit* split) {
  if (split) *split = GemmSplit{};
  int launches = 0;
  return g.bf16 ? launch_gemm_bf16(g, s, split) : launch_gemm_f32_path(g, s, &launches);
}

hipError_t launch_gemm_fixup(const GemmArgs& g, const GemmSplit& split, hipStream_t s) {
  return g.bf16 ? launch_gemm_bf16_fixup(g, split, s) : hipSuccess;
}

int64_t gemm_ws_elems(const GemmArgs& g) { return g.bf16 ? gemm_bf16_ws_elems(g) : 0; }

}  // namespace domino
