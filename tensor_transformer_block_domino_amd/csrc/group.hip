// The small-kernel group between the sublayers of a Domino transformer layer: dropout,
// residual add and LayerNorm, fused into one row pass (page "DeepSpeed-Domino 深度解析",
// section "前向：多个计算片段轮转重叠 AllReduce": the Dropout, Residual and LayerNorm kernels
// that hide an AllReduce; the layer excerpt under "μ-batch 流水").
//
//   forward:  r_out = resid + dropout(y + bias);  ln = (r_out − μ)·rstd·γ + β
//             (μ and σ² over the row, biased variance, rstd = 1/√(σ² + eps));
//   backward: d_resid = d_res + rstd·(g − mean(g) − x̂·mean(g·x̂)) with g = d_ln·γ,
//             d_y = dropout'(d_resid); dγ = Σ_rows d_ln·x̂, dβ = Σ_rows d_ln, dbias = Σ_rows d_y.
// Dropout is inverted dropout with a bit-packed keep mask (bit j % 32 of 32-bit word j / 32
// of the row; 8 elements of a 16-byte chunk are one byte of the mask). The LayerNorm reads
// the stored (bf16) r_out, so the backward sees the same x̂ as the forward. All arithmetic
// is fp32; every output is rounded once.
#include "common.hpp"
#include "kernels.hpp"

namespace domino {
namespace {

struct GroupFwdParams {
  const uint16_t* resid; const uint16_t* y; const uint16_t* bias; const uint8_t* keep;
  uint16_t* r_out; const uint16_t* gamma; const uint16_t* beta; uint16_t* ln; float* mean; float* rstd;
  int64_t rows; int h; int keep_row_bytes; float scale, eps;
};

struct GroupBwdParams {
  const uint16_t* d_ln; const uint16_t* d_res; const uint16_t* r_out; const float* mean; const float* rstd;
  const uint16_t* gamma; const uint8_t* keep;
  uint16_t* d_resid; uint16_t* d_y;
  float* part;           // [3][blocks][h]: dγ, dβ, dbias partial sums per row block
  int64_t rows; int h; int keep_row_bytes; int rows_per_block; float scale;
  bool want_ln, want_dy, want_bias;
};

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4_t*>(p); }
// Rows that are read once: non-temporal loads (measured 3.9 -> 4.4 TB/s for both kernels at
// 8192 x 4096, against 5.1 TB/s for a 1 GiB device copy).
__device__ __forceinline__ u32x4_t ld16_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void st16(uint16_t* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

__device__ __forceinline__ void unpack8(u32x4_t w, float (&f)[8]) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(a[i]);
    f[2 * i + 1] = bf16_hi(a[i]);
  }
}
__device__ __forceinline__ u32x4_t pack8(const float (&f)[8]) {
  return u32x4_t{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// One wave per row; lane l owns 16-byte chunks l, l + 64, … (CPL of them).
template <int CPL>
__global__ __launch_bounds__(256) void resid_ln_fwd_kernel(GroupFwdParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int nch = p.h >> 3;
  const int64_t base = row * p.h;
  float v[CPL][8];
  u32x4_t rw[CPL], yw[CPL], bw[CPL];
  uint32_t kb[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      rw[i] = ld16_stream(p.resid + base + 8 * c);
      if (p.y) {
        yw[i] = ld16_stream(p.y + base + 8 * c);
        bw[i] = p.bias ? ld16(p.bias + 8 * c) : u32x4_t{0u, 0u, 0u, 0u};
        kb[i] = p.keep ? p.keep[row * p.keep_row_bytes + c] : 0xffu;
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      unpack8(rw[i], v[i]);
      if (p.y) {
        float yv[8], bv[8];
        unpack8(yw[i], yv);
        unpack8(bw[i], bv);
        const float sc = p.keep ? p.scale : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] += (kb[i] >> e) & 1u ? (yv[e] + bv[e]) * sc : 0.f;
      }
      const u32x4_t o = pack8(v[i]);
      if (p.r_out) st16(p.r_out + base + 8 * c, o);
      unpack8(o, v[i]);  // the LayerNorm sees the stored value
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[i][e];
    }
  }
  if (!p.gamma) return;
  const float inv_h = 1.0f / float(p.h);
  const float mu = wave_sum(s) * inv_h;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i)
    if (lane + 64 * i < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[i][e] - mu;
        q = fmaf(d, d, q);
      }
    }
  const float rs = 1.0f / sqrtf(wave_sum(q) * inv_h + p.eps);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float g[8], b[8], o[8];
      unpack8(ld16(p.gamma + 8 * c), g);
      if (p.beta) unpack8(ld16(p.beta + 8 * c), b);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf((v[i][e] - mu) * rs, g[e], p.beta ? b[e] : 0.f);
      st16(p.ln + base + 8 * c, pack8(o));
    }
  }
  if (lane == 0) {
    p.mean[row] = mu;
    p.rstd[row] = rs;
  }
}

// One workgroup per block of consecutive rows, 256 threads across each row; thread t owns
// chunks t, t + 256, … (CPT of them) of every row, so its partial column sums stay in
// registers. The two row sums of the LayerNorm gradient go through LDS (one barrier per
// row, two alternating slots).
template <int CPT>
__global__ __launch_bounds__(256) void resid_ln_bwd_kernel(GroupBwdParams p) {
  __shared__ float red[2][4][2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nch = p.h >> 3;
  const int64_t r0 = int64_t(blockIdx.x) * p.rows_per_block;
  const int64_t r1 = r0 + p.rows_per_block < p.rows ? r0 + p.rows_per_block : p.rows;
  float gam[CPT][8], acc_g[CPT][8], acc_b[CPT][8], acc_y[CPT][8];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc_g[i][e] = acc_b[i][e] = acc_y[i][e] = 0.f;
    if (p.want_ln && c < nch) unpack8(ld16(p.gamma + 8 * c), gam[i]);
  }
  const float inv_h = 1.0f / float(p.h);
  // Raw 16-byte chunks of the current row; the next row's are loaded before this row's
  // reduction, so each workgroup keeps a row of loads in flight.
  u32x4_t cur_res[CPT], cur_ln[CPT], cur_r[CPT], nxt_res[CPT], nxt_ln[CPT], nxt_r[CPT];
  float cur_mu = 0.f, cur_rs = 0.f, nxt_mu = 0.f, nxt_rs = 0.f;
  auto load_row = [&](int64_t row, u32x4_t (&rs_)[CPT], u32x4_t (&ln_)[CPT], u32x4_t (&r_)[CPT], float& mu, float& rsd) {
    const int64_t base = row * p.h;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      if (c >= nch) continue;
      if (p.d_res) rs_[i] = ld16_stream(p.d_res + base + 8 * c);
      if (p.want_ln) {
        ln_[i] = ld16_stream(p.d_ln + base + 8 * c);
        r_[i] = ld16(p.r_out + base + 8 * c);
      }
    }
    if (p.want_ln) {
      mu = p.mean[row];
      rsd = p.rstd[row];
    }
  };
  if (r0 < r1) load_row(r0, cur_res, cur_ln, cur_r, cur_mu, cur_rs);
  int slot = 0;
  for (int64_t row = r0; row < r1; ++row, slot ^= 1) {
    if (row + 1 < r1) load_row(row + 1, nxt_res, nxt_ln, nxt_r, nxt_mu, nxt_rs);
    const int64_t base = row * p.h;
    float dl[CPT][8], xh[CPT][8], d[CPT][8];
    float sg = 0.f, sgx = 0.f;
    const float mu = cur_mu, rs = cur_rs;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      if (c >= nch) continue;
      if (p.d_res) unpack8(cur_res[i], d[i]);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) d[i][e] = 0.f;
      }
      if (p.want_ln) {
        float r[8];
        unpack8(cur_ln[i], dl[i]);
        unpack8(cur_r[i], r);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xh[i][e] = (r[e] - mu) * rs;
          const float g = dl[i][e] * gam[i][e];
          sg += g;
          sgx = fmaf(g, xh[i][e], sgx);
        }
      }
    }
    if (p.want_ln) {
      sg = wave_sum(sg);
      sgx = wave_sum(sgx);
      if (lane == 0) {
        red[slot][w][0] = sg;
        red[slot][w][1] = sgx;
      }
      __syncthreads();
      sg = ((red[slot][0][0] + red[slot][1][0]) + red[slot][2][0]) + red[slot][3][0];
      sgx = ((red[slot][0][1] + red[slot][1][1]) + red[slot][2][1]) + red[slot][3][1];
    }
    const float mg = sg * inv_h, mgx = sgx * inv_h;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      if (c >= nch) continue;
      if (p.want_ln) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float g = dl[i][e] * gam[i][e];
          d[i][e] += rs * (g - mg - xh[i][e] * mgx);
          acc_g[i][e] = fmaf(dl[i][e], xh[i][e], acc_g[i][e]);
          acc_b[i][e] += dl[i][e];
        }
      }
      if (p.d_resid) st16(p.d_resid + base + 8 * c, pack8(d[i]));
      if (p.want_dy || p.want_bias) {
        const uint32_t kb = p.keep ? p.keep[row * p.keep_row_bytes + c] : 0xffu;
        const float sc = p.keep ? p.scale : 1.0f;
        float dy[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          dy[e] = (kb >> e) & 1u ? d[i][e] * sc : 0.f;
          acc_y[i][e] += dy[e];
        }
        if (p.want_dy) st16(p.d_y + base + 8 * c, pack8(dy));
      }
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      cur_res[i] = nxt_res[i];
      cur_ln[i] = nxt_ln[i];
      cur_r[i] = nxt_r[i];
    }
    cur_mu = nxt_mu;
    cur_rs = nxt_rs;
  }
  const int64_t nb = gridDim.x;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + 256 * i;
    if (c >= nch) continue;
    float* pg = p.part + int64_t(blockIdx.x) * p.h + 8 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pg[e] = acc_g[i][e];
      pg[nb * p.h + e] = acc_b[i][e];
      pg[2 * nb * p.h + e] = acc_y[i][e];
    }
  }
}

// out_q[j] (+)= Σ_b part_q[b][j] for the quantities q = blockIdx.y whose output is non-null.
// A workgroup owns 32 columns; its 8 thread slices each sum a contiguous eighth of the
// partial rows (in order, 8 loads in flight), and the 8 slice sums are added in slice order,
// so the result is the same on every run.
struct ColsumParams {
  const float* part;   // [3][nb][h]
  float* out[3];
  int nb, h, accumulate;
};
__global__ __launch_bounds__(256) void colsum_kernel(ColsumParams p) {
  __shared__ float red[8][33];
  float* out = p.out[blockIdx.y];
  if (!out) return;
  const int c = threadIdx.x & 31, sl = threadIdx.x >> 5;
  const int j = blockIdx.x * 32 + c;
  const float* src = p.part + int64_t(blockIdx.y) * p.nb * p.h + j;
  const int per = (p.nb + 7) / 8, b0 = sl * per, b1 = b0 + per < p.nb ? b0 + per : p.nb;
  float s = 0.f;
  if (j < p.h) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[int64_t(b + u) * p.h];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < b1; ++b) s += src[int64_t(b) * p.h];
  }
  red[sl][c] = s;
  __syncthreads();
  if (sl == 0 && j < p.h) {
    float t = red[0][c];
#pragma unroll
    for (int k = 1; k < 8; ++k) t += red[k][c];
    out[j] = p.accumulate ? out[j] + t : t;
  }
}

// Stage one of a bias gradient: workgroup (column block, row block) sums 64 rows of 2048
// columns (8 per thread, 16-byte loads) into part[row block][col].
constexpr int kBiasRows = 64;
__global__ __launch_bounds__(256) void colpart_bf16_kernel(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                                           float* part) {
  const int64_t c = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (c >= cols) return;
  const int64_t r0 = int64_t(blockIdx.y) * kBiasRows;
  const int64_t r1 = r0 + kBiasRows < rows ? r0 + kBiasRows : rows;
  float s[8] = {};
  for (int64_t r = r0; r < r1; ++r) {
    float v[8];
    unpack8(ld16(x + r * ld + c), v);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += v[e];
  }
  float* dst = part + int64_t(blockIdx.y) * cols + c;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[e] = s[e];
}

constexpr int kBwdBlocks = 512;

template <int CPL>
hipError_t launch_fwd(const GroupFwdParams& p, hipStream_t s) {
  DOMINO_LAUNCH(resid_ln_fwd_kernel<CPL>, dim3(unsigned((p.rows + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}
template <int CPT>
hipError_t launch_bwd(const GroupBwdParams& p, int blocks, hipStream_t s) {
  DOMINO_LAUNCH(resid_ln_bwd_kernel<CPT>, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int64_t bias_grad_ws_floats(int64_t rows, int64_t cols) { return ((rows + kBiasRows - 1) / kBiasRows) * cols; }

hipError_t launch_bias_grad(const void* x, int64_t rows, int64_t cols, int64_t ld, float* out, int accumulate,
                            float* ws, hipStream_t s) {
  if (cols == 0) return hipSuccess;
  if (rows == 0) {
    if (accumulate) return hipSuccess;
    ColsumParams cp{};  // nb = 0: writes zeros
    cp.part = ws;
    cp.out[0] = out;
    cp.h = int(cols);
    DOMINO_LAUNCH(colsum_kernel, dim3(unsigned((cols + 31) / 32), 1), dim3(256), 0, s, cp);
    return hipGetLastError();
  }
  const unsigned rb = unsigned((rows + kBiasRows - 1) / kBiasRows);
  note_kernel("colpart_bf16_kernel");
  DOMINO_LAUNCH(colpart_bf16_kernel, dim3(unsigned((cols / 8 + 255) / 256), rb), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), rows, cols, ld, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ColsumParams cp{};
  cp.part = ws;
  cp.out[0] = out;
  cp.nb = int(rb);
  cp.h = int(cols);
  cp.accumulate = accumulate;
  DOMINO_LAUNCH(colsum_kernel, dim3(unsigned((cols + 31) / 32), 1), dim3(256), 0, s, cp);
  return hipGetLastError();
}

int64_t group_bwd_blocks(int64_t rows) {
  const int64_t b = (rows + 7) / 8;
  return b < kBwdBlocks ? (b > 0 ? b : 1) : kBwdBlocks;
}

hipError_t launch_resid_ln_fwd(const GroupFwdArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  GroupFwdParams p{};
  p.resid = static_cast<const uint16_t*>(a.resid);
  p.y = static_cast<const uint16_t*>(a.y);
  p.bias = static_cast<const uint16_t*>(a.bias);
  p.keep = reinterpret_cast<const uint8_t*>(a.keep);
  p.r_out = static_cast<uint16_t*>(a.r_out);
  p.gamma = static_cast<const uint16_t*>(a.gamma);
  p.beta = static_cast<const uint16_t*>(a.beta);
  p.ln = static_cast<uint16_t*>(a.ln);
  p.mean = a.mean;
  p.rstd = a.rstd;
  p.rows = a.rows;
  p.h = int(a.hidden);
  p.keep_row_bytes = int(4 * ((a.hidden + 31) / 32));
  p.scale = 1.0f / (1.0f - a.p_drop);
  p.eps = a.eps;
  note_kernel("resid_ln_fwd_kernel");
  switch ((a.hidden / 8 + 63) / 64) {
    case 1: return launch_fwd<1>(p, s);
    case 2: return launch_fwd<2>(p, s);
    case 3: return launch_fwd<3>(p, s);
    case 4: return launch_fwd<4>(p, s);
    case 5: return launch_fwd<5>(p, s);
    case 6: return launch_fwd<6>(p, s);
    case 7: case 8: return launch_fwd<8>(p, s);
    case 9: case 10: return launch_fwd<10>(p, s);
    case 11: case 12: return launch_fwd<12>(p, s);
    case 13: case 14: case 15: case 16: return launch_fwd<16>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_resid_ln_bwd(const GroupBwdArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  GroupBwdParams p{};
  p.d_ln = static_cast<const uint16_t*>(a.d_ln);
  p.d_res = static_cast<const uint16_t*>(a.d_res);
  p.r_out = static_cast<const uint16_t*>(a.r_out);
  p.mean = a.mean;
  p.rstd = a.rstd;
  p.gamma = static_cast<const uint16_t*>(a.gamma);
  p.keep = reinterpret_cast<const uint8_t*>(a.keep);
  p.d_resid = static_cast<uint16_t*>(a.d_resid);
  p.d_y = static_cast<uint16_t*>(a.d_y);
  p.part = a.workspace;
  p.rows = a.rows;
  p.h = int(a.hidden);
  p.keep_row_bytes = int(4 * ((a.hidden + 31) / 32));
  p.scale = 1.0f / (1.0f - a.p_drop);
  p.want_ln = a.d_ln != nullptr;
  p.want_dy = a.d_y != nullptr;
  p.want_bias = a.d_bias != nullptr;
  const int blocks = int(group_bwd_blocks(a.rows));
  p.rows_per_block = int((a.rows + blocks - 1) / blocks);
  note_kernel("resid_ln_bwd_kernel");
  hipError_t e;
  switch ((a.hidden / 8 + 255) / 256) {
    case 1: e = launch_bwd<1>(p, blocks, s); break;
    case 2: e = launch_bwd<2>(p, blocks, s); break;
    case 3: e = launch_bwd<3>(p, blocks, s); break;
    case 4: e = launch_bwd<4>(p, blocks, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  ColsumParams cp{};
  cp.part = a.workspace;
  cp.out[0] = a.d_ln ? a.d_gamma : nullptr;
  cp.out[1] = a.d_ln ? a.d_beta : nullptr;
  cp.out[2] = a.d_bias;
  cp.nb = blocks;
  cp.h = int(a.hidden);
  cp.accumulate = a.accumulate;
  if (cp.out[0] || cp.out[1] || cp.out[2])
    DOMINO_LAUNCH(colsum_kernel, dim3(unsigned((a.hidden + 31) / 32), 3), dim3(256), 0, s, cp);
  return hipGetLastError();
}

}  // namespace domino
