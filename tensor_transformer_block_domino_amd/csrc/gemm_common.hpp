// Building blocks shared by the bf16 GEMM kernels (gfx950): how an operand tile is copied
// into LDS and read back as MFMA fragments, the kernel parameters, the tile order, and the
// fused epilogues of the MLP shard's products (the forward's activation, the backward's
// activation gradient, fp32 weight gradients).
//
// The products are the "GeMM + GeLU + GeMM" kernel sequence of the MLP and the independent
// input-gradient / weight-gradient products of its backward (page "DeepSpeed-Domino 深度解析",
// sections "前向：多个计算片段轮转重叠 AllReduce" and "反向：扩展与权重梯度计算的重叠";
// page "04 · TP/SP 的通信-计算 overlap 与工程优化", §1).
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace domino {
namespace {

// Tile-row → global index of an operand's m (or n) dimension. For the SwiGLU forward's
// B operand, a tile of BN rows holds BN/2 FFN columns: each wave's BN/2 rows are
// [BN/4 gate columns | the same BN/4 up columns], so one lane holds gate and up of the
// same output element.
struct RowMap {
  int64_t base;   // first global index (or first FFN column j for SwiGLU)
  int64_t limit;  // valid indices are < limit (f_s for SwiGLU)
  int64_t f_s;    // offset of the up block (SwiGLU only)
};

template <bool kSw, int R>
__device__ __forceinline__ int64_t map_row(const RowMap& m, int r) {
  if constexpr (!kSw) {
    const int64_t g = m.base + r;
    return g < m.limit ? g : -1;
  } else {
    constexpr int kHalf = R / 4;
    const int wn = r / (R / 2), cc = r % (R / 2);
    const int64_t j = m.base + wn * kHalf + (cc % kHalf);
    if (j >= m.limit) return -1;
    return cc < kHalf ? j : m.f_s + j;
  }
}

// Operand contiguous along k (element (row, k) at p[row·ld + k]), staged as
// [R rows][BK k]: CPR 16-byte chunks per row, chunk c of row r stored at c ^ f(r), which
// keeps a fragment read (16 consecutive rows, same chunk) on distinct banks of the
// 64-bank LDS (and of a 32-bank one, 8 rows at a time).
template <int R, int BK, bool kSw = false>
struct OpK {
  static constexpr int CPR = BK / 8;
  static constexpr int kLoads = R * BK / 2048;  // 1 KB instructions per wave per stage
  static_assert(R * BK % 2048 == 0, "whole 1 KB copies per wave");
  static __device__ __forceinline__ int f(int row) {
    return CPR == 8 ? ((row & 7) ^ ((row >> 3) & 7)) : (((row >> 2) ^ (row >> 1)) & 3);
  }
  static __device__ __forceinline__ int off(int row, int c) { return row * BK + ((c ^ f(row)) << 3); }
  const uint16_t* base;
  int32_t voff[kLoads];
  int kc[kLoads];
  __device__ __forceinline__ void init(const uint16_t* p, int64_t ld, const RowMap& rm, int wave, int lane) {
    base = p + rm.base * ld;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int idx = (wave + 4 * q) * 64 + lane, row = idx / CPR, c = (idx % CPR) ^ f(row);
      kc[q] = c * 8;
      if constexpr (kSw) {
        // Tile row r holds the gate or up row of output column pair map_row<true>(r).
        const int64_t g = map_row<true, R>(rm, row);
        voff[q] = g >= 0 ? int32_t(((g - rm.base) * ld + c * 8) * 2) : kOOB;
      } else {
        voff[q] = map_row<false, R>(rm, row) >= 0 ? int32_t((row * ld + c * 8) * 2) : kOOB;
      }
    }
  }
  // The copies of one stage: a buffer resource at k0 and the k left, then kLoads 1 KB
  // copies per wave.
  struct Src {
    __amdgpu_buffer_rsrc_t rs;
    int krem;
  };
  __device__ __forceinline__ Src src(int64_t k0, int64_t K) const {
    return Src{make_rsrc(base + k0), K - k0 > BK ? BK : int(K - k0)};
  }
  __device__ __forceinline__ void issue_one(const Src& sr, uint16_t* stage, int wave, int q) const {
    dma16(sr.rs, stage + (wave + 4 * q) * 512, kc[q] < sr.krem ? voff[q] : kOOB);
  }
  // MFMA fragment: row `row0 + lane%32`, k = 16·s + 8·(lane/32) .. +7, one 16-byte read.
  static constexpr int kRd = 1;
  static __device__ __forceinline__ void read(const uint16_t* stage, int row0, int s, int lane, int,
                                              u32x4_t& dst) {
    asm volatile("ds_read_b128 %0, %1" : "=v"(dst) : "v"(lds_addr(stage + off(row0 + (lane & 31), s * 2 + (lane >> 5)))));
  }
};

// Operand contiguous along m/n (element (row, k) at p[k·ld + row]), staged as it lies in
// memory: [BK k-rows][R] with chunk c of k-row r stored at c ^ h(r). Fragments come out
// transposed through ds_read_b64_tr_b16: within each 16-lane group, lane i receives
// element i%4 of the 4-element blocks addressed by lanes 4e + i/4 (e = 0..3). With lane
// j of the group addressing k-row k0 + j/4 at columns n0 + 4·(j%4), lane i receives
// column n0 + i at k-rows k0 .. k0+3. h(r) spreads the 4 k-rows × 4 chunks that 32
// lanes read at once over distinct banks. With R = 160 a k-row is 80 banks long, so
// k-rows k0 .. k0+3 (k0 a multiple of 4) already start 16 banks apart and need no swizzle.
template <int R, int BK, bool kSw>
struct OpMN {
  static constexpr int CPR = R / 8;
  static constexpr int kLoads = R * BK / 2048;
  static_assert(R * BK % 2048 == 0, "whole 1 KB copies per wave");
  static constexpr bool kSwz = R % 128 == 0;
  static __device__ __forceinline__ int h(int krow) {
    return kSwz ? ((krow & 3) << 2) ^ (((krow >> 1) & 1) << 1) : 0;
  }
  static __device__ __forceinline__ int off(int krow, int c) { return krow * R + ((c ^ h(krow)) << 3); }
  const uint16_t* base;
  int64_t ld;
  int32_t voff[kLoads];
  int kr[kLoads];
  __device__ __forceinline__ void init(const uint16_t* p, int64_t ld_, const RowMap& rm, int wave, int lane) {
    ld = ld_;
    base = p + rm.base;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
      const int idx = (wave + 4 * q) * 64 + lane, krow = idx / CPR, c = (idx % CPR) ^ h(krow);
      kr[q] = krow;
      const int64_t g = map_row<kSw, R>(rm, c * 8);
      voff[q] = g >= 0 ? int32_t((krow * ld_ + (g - rm.base)) * 2) : kOOB;
    }
  }
  struct Src {
    __amdgpu_buffer_rsrc_t rs;
    int krem;
  };
  __device__ __forceinline__ Src src(int64_t k0, int64_t K) const {
    return Src{make_rsrc(base + k0 * ld), K - k0 > BK ? BK : int(K - k0)};
  }
  __device__ __forceinline__ void issue_one(const Src& sr, uint16_t* stage, int wave, int q) const {
    dma16(sr.rs, stage + (wave + 4 * q) * 512, kr[q] < sr.krem ? voff[q] : kOOB);
  }
  // MFMA fragment in two transposed reads: part 0 = k-rows k0 .. k0+3, part 1 = k0+4 .. k0+7.
  static constexpr int kRd = 2;
  static __device__ __forceinline__ void read(const uint16_t* stage, int row0, int s, int lane, int part,
                                              u32x4_t& dst) {
    const int g = lane >> 4, j = lane & 15;
    const int k0 = s * 16 + 8 * (g >> 1) + (j >> 2) + 4 * part;
    const int mn = row0 + 16 * (g & 1) + 4 * (j & 3);
    const int c = mn >> 3, e = mn & 7;
    u32x2_t v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(lds_addr(stage + off(k0, c) + e)));
    if (part == 0) {
      dst.x = v.x;
      dst.y = v.y;
    } else {
      dst.z = v.x;
      dst.w = v.y;
    }
  }
};

struct KParams {
  const uint16_t* A; int64_t lda;
  const uint16_t* B; int64_t ldb;
  void* C; int64_t ldc;
  uint16_t* C2; int64_t ldc2;
  const uint16_t* aux; int64_t ldaux;
  const uint16_t* bias;  // column bias added before the forward epilogues, or null
  float* ws;             // k-split tiles' fp32 slices: [tile − dp_tiles][split][BM][BN]
  int64_t M, N, K, f_s;
  int tiles_m, tiles_n;
  int dp_tiles;          // tiles 0 .. dp_tiles−1 run whole, with the fused epilogue
  int splits;            // k-slices of each remaining tile
  int kt_per_split;      // k-steps (of BK) per slice
  int accumulate;
};

// Tile t → (tile row, tile column): groups of 8 tile rows, column-major inside a group, so
// consecutive tiles share rows of A.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int kGroup = 8;
  const int per_group = kGroup * tiles_n;
  const int first_m = (t / per_group) * kGroup;
  const int gsize = min(tiles_m - first_m, kGroup);
  tm = first_m + (t % per_group) % gsize;
  tn = (t % per_group) / gsize;
}

__device__ __forceinline__ void store_bf16x4(uint16_t* dst, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// The saved activation input the backward epilogues read for outputs (m, n..n+3): Hpre
// (tanh-GeLU), or its gate and up columns (SwiGLU). Loaded for a whole row block before
// any is used, so the loads overlap.
struct AuxQuad {
  u32x2_t g, u;
};
template <Epi kEpi>
__device__ __forceinline__ AuxQuad load_aux4(const KParams& p, int64_t m, int64_t n) {
  AuxQuad a{};
  if constexpr (kEpi == Epi::kDGelu || kEpi == Epi::kDSwiglu)
    a.g = *reinterpret_cast<const u32x2_t*>(p.aux + m * p.ldaux + n);
  if constexpr (kEpi == Epi::kDSwiglu)
    a.u = *reinterpret_cast<const u32x2_t*>(p.aux + m * p.ldaux + p.f_s + n);
  return a;
}

// The column bias of outputs n..n+3 (a wave-uniform branch; no bias, no load).
__device__ __forceinline__ f32x4_t add_bias4(const KParams& p, int64_t n, f32x4_t v) {
  if (p.bias) {
    const u32x2_t b = *reinterpret_cast<const u32x2_t*>(p.bias + n);
    v.x += bf16_lo(b.x);
    v.y += bf16_hi(b.x);
    v.z += bf16_lo(b.y);
    v.w += bf16_hi(b.y);
  }
  return v;
}

// Epilogue for 4 consecutive output columns n..n+3 of row m (n < N, all four in range).
template <Epi kEpi>
__device__ __forceinline__ void epilogue4(const KParams& p, int64_t m, int64_t n, f32x4_t v,
                                          const AuxQuad& ax) {
  if constexpr (kEpi == Epi::kStore || kEpi == Epi::kGelu) v = add_bias4(p, n, v);
  if constexpr (kEpi == Epi::kStore) {
    store_bf16x4(static_cast<uint16_t*>(p.C) + m * p.ldc + n, v.x, v.y, v.z, v.w);
  } else if constexpr (kEpi == Epi::kGelu) {
    store_bf16x4(static_cast<uint16_t*>(p.C) + m * p.ldc + n, v.x, v.y, v.z, v.w);
    store_bf16x4(p.C2 + m * p.ldc2 + n, gelu_tanh_f(v.x), gelu_tanh_f(v.y), gelu_tanh_f(v.z), gelu_tanh_f(v.w));
  } else if constexpr (kEpi == Epi::kDGelu) {
    const u32x2_t x = ax.g;
    store_bf16x4(static_cast<uint16_t*>(p.C) + m * p.ldc + n, v.x * gelu_tanh_grad_f(bf16_lo(x.x)),
                 v.y * gelu_tanh_grad_f(bf16_hi(x.x)), v.z * gelu_tanh_grad_f(bf16_lo(x.y)),
                 v.w * gelu_tanh_grad_f(bf16_hi(x.y)));
  } else if constexpr (kEpi == Epi::kDSwiglu) {
    const u32x2_t gw = ax.g, uw = ax.u;
    const float g[4] = {bf16_lo(gw.x), bf16_hi(gw.x), bf16_lo(gw.y), bf16_hi(gw.y)};
    const float u[4] = {bf16_lo(uw.x), bf16_hi(uw.x), bf16_lo(uw.y), bf16_hi(uw.y)};
    const float dh[4] = {v.x, v.y, v.z, v.w};
    float dg[4], du[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float sg = sigmoidf_(g[e]);
      dg[e] = dh[e] * u[e] * sg * (1.0f + g[e] * (1.0f - sg));
      du[e] = dh[e] * g[e] * sg;
    }
    uint16_t* dp = static_cast<uint16_t*>(p.C) + m * p.ldc;
    store_bf16x4(dp + n, dg[0], dg[1], dg[2], dg[3]);
    store_bf16x4(dp + p.f_s + n, du[0], du[1], du[2], du[3]);
  } else if constexpr (kEpi == Epi::kF32) {
    f32x4_t* dst = reinterpret_cast<f32x4_t*>(static_cast<float*>(p.C) + m * p.ldc + n);
    *dst = p.accumulate ? (*dst + v) : v;
  }
}

// SwiGLU epilogue for FFN columns j..j+3 of row m: gate g and up u from the same lane.
__device__ __forceinline__ void epilogue_swiglu4(const KParams& p, int64_t m, int64_t j, f32x4_t g, f32x4_t u) {
  g = add_bias4(p, j, g);
  u = add_bias4(p, p.f_s + j, u);
  uint16_t* hp = static_cast<uint16_t*>(p.C) + m * p.ldc;
  store_bf16x4(hp + j, g.x, g.y, g.z, g.w);
  store_bf16x4(hp + p.f_s + j, u.x, u.y, u.z, u.w);
  store_bf16x4(p.C2 + m * p.ldc2 + j, silu_f(g.x) * u.x, silu_f(g.y) * u.y, silu_f(g.z) * u.z, silu_f(g.w) * u.w);
}


}  // namespace
}  // namespace domino
