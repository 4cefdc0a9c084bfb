// shard_reduce kernels: the sum an AllReduce of the tensor-parallel partials produces,
// done on one GPU over partials resident in HBM.
// (Page "DeepSpeed-Domino 深度解析", section "TP 的数据依赖：通信为何难以隐藏": each TP
// layer ends with AllReduce(Y); primer "从单卡到集群…" §3.1: row-parallel outputs are
// partial sums that the reduce adds.)
//
// HBM-bound streaming kernel: every partial is read once and the result written once,
// (P+1)·rows·cols·elem bytes. Each thread owns 16-byte column groups of a row; all P
// loads of a group are issued before the fp32 accumulation in the fixed order p = 0..P−1,
// so a wave keeps 2·P 16-byte loads in flight. No LDS, no MFMA.
#include <cstdio>

#include "common.hpp"
#include "kernels.hpp"

namespace domino {

struct PartialPtrs {
  const void* p[kMaxPartials];
};

template <typename T, int P>
__global__ __launch_bounds__(256) void shard_reduce_kernel(void* __restrict__ out, int64_t ld_out,
                                                           PartialPtrs parts, int64_t ld_in,
                                                           uint32_t rows, uint32_t groups_per_row,
                                                           uint32_t total_groups) {
  constexpr int kElems = 16 / sizeof(T);  // elements per 16-byte group
  constexpr int kUnroll = 2;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t g0 = blockIdx.x * blockDim.x + threadIdx.x; g0 < total_groups; g0 += stride * kUnroll) {
    u32x4_t v[kUnroll][P];
    uint32_t row[kUnroll], grp[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t g = g0 + u * stride;
      ok[u] = g < total_groups;
      row[u] = ok[u] ? g / groups_per_row : 0;
      grp[u] = ok[u] ? g - row[u] * groups_per_row : 0;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const T* src = static_cast<const T*>(parts.p[p]) + int64_t(row[u]) * ld_in + int64_t(grp[u]) * kElems;
        v[u][p] = ok[u] ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src)) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (!ok[u]) continue;
      T* dst = static_cast<T*>(out) + int64_t(row[u]) * ld_out + int64_t(grp[u]) * kElems;
      if constexpr (sizeof(T) == 2) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const uint32_t w[4] = {v[u][p].x, v[u][p].y, v[u][p].z, v[u][p].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] += bf16_lo(w[q]);
            acc[2 * q + 1] += bf16_hi(w[q]);
          }
        }
        const u32x4_t r = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                           pack_bf16x2(acc[6], acc[7])};
        __builtin_nontemporal_store(r, reinterpret_cast<u32x4_t*>(dst));
      } else {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int p = 0; p < P; ++p) {
          acc[0] += __uint_as_float(v[u][p].x);
          acc[1] += __uint_as_float(v[u][p].y);
          acc[2] += __uint_as_float(v[u][p].z);
          acc[3] += __uint_as_float(v[u][p].w);
        }
        const f32x4_t r = {acc[0], acc[1], acc[2], acc[3]};
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4_t*>(dst));
      }
    }
  }
}

// The same sum with buffer loads: one 32-bit byte offset per group, shared by the P
// partials (each a scalar buffer resource), instead of a 64-bit address per load: 66
// VGPRs instead of 82, so a reduction wave (72 allocated) fits on a SIMD beside two waves
// of the eight-wave GEMM (216 each of the 512) and runs beside it instead of waiting for
// a CU to empty. Used for large reductions whose byte offsets fit the buffer range;
// measured, it made the Llama-2 steps 0.8% (13B, 2D) and 3% (7B, columns) faster and the
// attention block 1.3%, while for the GPT-3 2.7B chunks (4096×2560, beside one-wave
// 256×160 GEMMs that leave room for either kernel) the 64-bit form stayed 2% faster.
template <typename T, int P>
__global__ __launch_bounds__(256) void shard_reduce_buf_kernel(void* __restrict__ out, int64_t ld_out,
                                                               PartialPtrs parts, int64_t ld_in,
                                                               uint32_t rows, uint32_t groups_per_row,
                                                               uint32_t total_groups) {
  constexpr int kElems = 16 / sizeof(T);
  constexpr int kUnroll = 2;
  constexpr int kNt = 2;  // non-temporal
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t g0 = blockIdx.x * blockDim.x + threadIdx.x; g0 < total_groups; g0 += stride * kUnroll) {
    u32x4_t v[kUnroll][P];
    uint32_t row[kUnroll], grp[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t g = g0 + u * stride;
      ok[u] = g < total_groups;
      row[u] = ok[u] ? g / groups_per_row : 0;
      grp[u] = ok[u] ? g - row[u] * groups_per_row : 0;
      const int32_t off = ok[u] ? int32_t((int64_t(row[u]) * ld_in + int64_t(grp[u]) * kElems) * int64_t(sizeof(T))) : kOOB;
#pragma unroll
      for (int p = 0; p < P; ++p)
        v[u][p] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                  make_rsrc(static_cast<const uint16_t*>(parts.p[p])), off, 0, kNt));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (!ok[u]) continue;
      T* dst = static_cast<T*>(out) + int64_t(row[u]) * ld_out + int64_t(grp[u]) * kElems;
      if constexpr (sizeof(T) == 2) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const uint32_t w[4] = {v[u][p].x, v[u][p].y, v[u][p].z, v[u][p].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] += bf16_lo(w[q]);
            acc[2 * q + 1] += bf16_hi(w[q]);
          }
        }
        const u32x4_t r = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                           pack_bf16x2(acc[6], acc[7])};
        __builtin_nontemporal_store(r, reinterpret_cast<u32x4_t*>(dst));
      } else {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int p = 0; p < P; ++p) {
          acc[0] += __uint_as_float(v[u][p].x);
          acc[1] += __uint_as_float(v[u][p].y);
          acc[2] += __uint_as_float(v[u][p].z);
          acc[3] += __uint_as_float(v[u][p].w);
        }
        const f32x4_t r = {acc[0], acc[1], acc[2], acc[3]};
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4_t*>(dst));
      }
    }
  }
}

template <typename T, int P>
static hipError_t launch_reduce_p(const ReduceArgs& a, hipStream_t s) {
  constexpr int kElems = 16 / sizeof(T);
  PartialPtrs parts{};
  for (int p = 0; p < P; ++p) parts.p[p] = a.partials[p];
  const uint32_t groups_per_row = uint32_t(a.cols / kElems);
  const uint32_t total = uint32_t(a.rows) * groups_per_row;
  // One workgroup of 256 threads per CU at most (kReduceMaxBlocks).
  const uint32_t want = (total + 2 * 256 - 1) / (2 * 256);
  static_assert(int64_t(kReduceMaxBlocks) * 256 * 2 <= (int64_t(1) << 21), "grid stride within the group limit");
  const uint32_t blocks = want < uint32_t(kReduceMaxBlocks) ? (want ? want : 1u) : uint32_t(kReduceMaxBlocks);
  char name[64];
  // Every input byte offset within the buffer range (the partials share ld_in).
  const bool buf = a.rows * a.cols >= (int64_t(1) << 25) &&
                   ((a.rows - 1) * a.ld_in + a.cols) * int64_t(sizeof(T)) <= int64_t(kRangeBytes) - 16;
  snprintf(name, sizeof name, "%s<%s, %d>", buf ? "shard_reduce_buf_kernel" : "shard_reduce_kernel",
           sizeof(T) == 2 ? "bf16" : "f32", P);
  note_kernel(name);
  if (buf)
    DOMINO_LAUNCH((shard_reduce_buf_kernel<T, P>), dim3(blocks), dim3(256), 0, s, a.out, a.ld_out, parts,
                  a.ld_in, uint32_t(a.rows), groups_per_row, total);
  else
    DOMINO_LAUNCH((shard_reduce_kernel<T, P>), dim3(blocks), dim3(256), 0, s, a.out, a.ld_out, parts,
                  a.ld_in, uint32_t(a.rows), groups_per_row, total);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_reduce_t(const ReduceArgs& a, hipStream_t s) {
  switch (a.n_partials) {
    case 1: return launch_reduce_p<T, 1>(a, s);
    case 2: return launch_reduce_p<T, 2>(a, s);
    case 3: return launch_reduce_p<T, 3>(a, s);
    case 4: return launch_reduce_p<T, 4>(a, s);
    case 5: return launch_reduce_p<T, 5>(a, s);
    case 6: return launch_reduce_p<T, 6>(a, s);
    case 7: return launch_reduce_p<T, 7>(a, s);
    case 8: return launch_reduce_p<T, 8>(a, s);
    case 9: return launch_reduce_p<T, 9>(a, s);
    case 10: return launch_reduce_p<T, 10>(a, s);
    case 11: return launch_reduce_p<T, 11>(a, s);
    case 12: return launch_reduce_p<T, 12>(a, s);
    case 13: return launch_reduce_p<T, 13>(a, s);
    case 14: return launch_reduce_p<T, 14>(a, s);
    case 15: return launch_reduce_p<T, 15>(a, s);
    case 16: return launch_reduce_p<T, 16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_shard_reduce(const ReduceArgs& a, hipStream_t s) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  return a.bf16 ? launch_reduce_t<uint16_t>(a, s) : launch_reduce_t<float>(a, s);
}

}  // namespace domino
