// Transposed bf16 copy of a weight shard: dst[c][r] = src[r][c]. The forward products of
// the MLP shard read their weight operand contiguous along k when it is given that way
// ([out][in] instead of the shard's [in][out]): measured on the Llama-2-13B shapes, the
// first product 986 vs 1042 µs and the second product's chunks 511 vs 583–609 µs per step
// (plain stores, products alone), for 18–26 µs of copying per step.
//
// HBM-bound: rows·cols·2 bytes read and written once. A workgroup moves a 64×64 tile
// through LDS: 16-byte loads along the source rows, 16-byte stores along the destination
// rows, the LDS rows padded so the column reads spread over the banks. Rows and columns
// are multiples of 8 (the library's shape rules).
#include "common.hpp"
#include "kernels.hpp"

namespace domino {
namespace {

constexpr int kTile = 64;
// LDS row length in elements: 132 bytes, so the 8 rows 8 apart that a wave's column reads
// touch start 8 banks apart (264 words) instead of sharing two banks.
constexpr int kPad = 66;
constexpr int kRowTiles = 4;

__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                                             uint16_t* __restrict__ dst, int64_t ld_dst, int rows,
                                                             int cols) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTile][kPad];
  uint32_t* const tile32 = reinterpret_cast<uint32_t*>(&tile[0][0]);
  const int c0 = blockIdx.x * kTile, t = threadIdx.x;
  // kRowTiles tiles down the source rows per workgroup.
  for (int rt = 0; rt < kRowTiles; ++rt) {
  const int r0 = (blockIdx.y * kRowTiles + rt) * kTile;
  if (r0 >= rows) break;
  if (rt) __syncthreads();  // the previous tile's reads are done before it is overwritten
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = t + 256 * k, rr = idx >> 3, cc = (idx & 7) * 8;
    const int r = r0 + rr, c = c0 + cc;
    const u32x4_t v = r < rows && c < cols ? *reinterpret_cast<const u32x4_t*>(src + int64_t(r) * ld_src + c)
                                           : u32x4_t{0u, 0u, 0u, 0u};
    uint32_t* t4 = tile32 + (rr * kPad + cc) / 2;  // 4-byte aligned (kPad, cc even)
    t4[0] = v.x;
    t4[1] = v.y;
    t4[2] = v.z;
    t4[3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = t + 256 * k, cr = idx >> 3, rc = (idx & 7) * 8;
    const int c = c0 + cr, r = r0 + rc;
    if (c >= cols || r >= rows) continue;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = uint32_t(tile[rc + 2 * e][cr]) | (uint32_t(tile[rc + 2 * e + 1][cr]) << 16);
    *reinterpret_cast<u32x4_t*>(dst + int64_t(c) * ld_dst + r) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
  }
}

}  // namespace

hipError_t launch_transpose_bf16(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t rows,
                                 int64_t cols, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (rows % 8 || cols % 8) return hipErrorInvalidValue;
  note_kernel("transpose_bf16_kernel");
  const dim3 grid(unsigned((cols + kTile - 1) / kTile), unsigned((rows + kTile * kRowTiles - 1) / (kTile * kRowTiles)));
  DOMINO_LAUNCH(transpose_bf16_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src), ld_src,
                static_cast<uint16_t*>(dst), ld_dst, int(rows), int(cols));
  return hipGetLastError();
}

}  // namespace domino
