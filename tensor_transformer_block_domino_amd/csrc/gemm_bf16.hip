// bf16 GEMMs on the CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation,
// with the fused epilogues of the MLP shard: the forward's activation (tanh-GeLU or
// SwiGLU) and the backward's activation gradient, and fp32 weight-gradient output.
//
// The products are the "GeMM + GeLU + GeMM" kernel sequence of the MLP and the
// independent input-gradient / weight-gradient products of its backward (page
// "DeepSpeed-Domino 深度解析", sections "前向：多个计算片段轮转重叠 AllReduce" and
// "反向：扩展与权重梯度计算的重叠"; page "04 · TP/SP 的通信-计算 overlap 与工程优化", §1).
//
// Design (gfx950, 64-wide waves, 160 KB LDS per CU):
//  * 256 threads = 4 waves in a 2×2 grid; block tile BM×BN with BM, BN ∈ {128, 256};
//    each wave owns (BM/2)×(BN/2) as 16×16 MFMA sub-tiles.
//  * K advances 64 at a time through two LDS stages (double buffer, one barrier per
//    step); the next stage's global loads are in flight while the current stage feeds
//    the MFMAs.
//  * Both operands sit in LDS as [tile row][64 k] bf16 (128 B per row, 8 chunks of
//    16 B), so every MFMA fragment is one 16-byte LDS read. Chunk c of row r is stored at
//    chunk c ^ (r & 7) ^ ((r >> 3) & 7): conflict-free for fragment reads (8 rows, same
//    chunk) and for both store patterns below.
//  * An operand contiguous along k is copied 16 B at a time. An operand contiguous
//    along m (or n) — the transposed operands of the weight gradients and the [in, out]
//    weights of the forward — is read as 8 k-rows × 4..8 elements per thread and
//    transposed in registers before the LDS store.
//  * The MFMA is issued with the operands swapped (B fragment as the matrix-core's A),
//    so each lane ends up with 4 consecutive output columns of one row: 8-byte bf16
//    stores and 16-byte fp32 stores in the epilogue.
//  * Workgroups are dispatched round-robin over the 8 XCDs; the tile index is remapped
//    so each XCD gets a contiguous, M-grouped range of tiles that share operand rows in
//    its L2.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace domino {
namespace {

constexpr int kKStep = 64;
constexpr int kThreads = 256;

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 7); }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * kKStep + ((chunk ^ swz(row)) << 3); }

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

// Global loads go through buffer instructions: a lane whose element is outside the
// matrix gets byte offset kOOB, which the buffer range check turns into zeros without a
// branch. Each k-step rebuilds the resource from a base pointer so offsets stay small.
constexpr int32_t kOOB = int32_t(0x80000000u);
constexpr int32_t kRangeBytes = 0x7fffffff;
constexpr int32_t kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint16_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, kRangeBytes, kRsrcWord3);
}

// Operand contiguous along k: element (row, k) at p[row·ld + k].
template <int R, bool kSw>
struct TileKContig {
  static constexpr int kPer = R / 32;  // 16-byte chunks per thread
  u32x4_t v[kPer];
  const uint16_t* base;
  int32_t off[kPer];
  int c8;
  __device__ __forceinline__ void init(const uint16_t* p, int64_t ld, const RowMap& rm, int tid) {
    static_assert(!kSw, "the SwiGLU column map applies to the m/n-contiguous forward operand only");
    c8 = (tid & 7) * 8;
    base = p + rm.base * ld;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int r = (tid >> 3) + 32 * j;
      off[j] = map_row<false, R>(rm, r) >= 0 ? int32_t((r * ld + c8) * 2) : kOOB;
    }
  }
  __device__ __forceinline__ void load(int64_t k0, int64_t K) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0);
    const bool kok = k0 + c8 < K;
#pragma unroll
    for (int j = 0; j < kPer; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, kok ? off[j] : kOOB, 0, 0);
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
    const int c = tid & 7;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int r = (tid >> 3) + 32 * j;
      *reinterpret_cast<u32x4_t*>(lds + lds_off(r, c)) = v[j];
    }
  }
  static constexpr int kStores = kPer;
  static constexpr int kLoads = kPer;
};

// Operand contiguous along m/n: element (row, k) at p[k·ld + row]. Thread t reads
// k-rows 8·(t/32) .. +7 of tile rows W·(t%32) .. +W−1 and transposes the 8×W block.
template <int R, bool kSw>
struct TileMNContig {
  static constexpr int kW = R / 32;  // tile rows per thread: 8 (R = 256) or 4 (R = 128)
  uint32_t v[8][kW / 2];
  const uint16_t* base;
  int64_t ld;
  int32_t moff;
  int kb;
  __device__ __forceinline__ void init(const uint16_t* p, int64_t ld_, const RowMap& rm, int tid) {
    ld = ld_;
    kb = tid >> 5;
    base = p + rm.base;
    const int64_t g = map_row<kSw, R>(rm, (tid & 31) * kW);
    moff = g >= 0 ? int32_t((g - rm.base) * 2) : kOOB;
  }
  __device__ __forceinline__ void load(int64_t k0, int64_t K) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + k0 * ld);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int kr = kb * 8 + kk;
      const int32_t o = (moff != kOOB && k0 + kr < K) ? moff + int32_t(kr * ld * 2) : kOOB;
      if constexpr (kW == 8) {
        const u32x4_t t = __builtin_amdgcn_raw_buffer_load_b128(rs, o, 0, 0);
        v[kk][0] = t.x; v[kk][1] = t.y; v[kk][2] = t.z; v[kk][3] = t.w;
      } else {
        const u32x2_t t = __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, 0);
        v[kk][0] = t.x; v[kk][1] = t.y;
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
    const int b = tid & 31;
#pragma unroll
    for (int e = 0; e < kW; ++e) {
      uint32_t d[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = v[2 * q][e >> 1], hi = v[2 * q + 1][e >> 1];
        d[q] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      const int r = b * kW + e;
      *reinterpret_cast<u32x4_t*>(lds + lds_off(r, kb)) = u32x4_t{d[0], d[1], d[2], d[3]};
    }
  }
  static constexpr int kStores = kW;
  static constexpr int kLoads = 8;
};

template <int R, bool kKContig, bool kSw>
using Tile = typename std::conditional<kKContig, TileKContig<R, kSw>, TileMNContig<R, kSw>>::type;

struct KParams {
  const uint16_t* A; int64_t lda;
  const uint16_t* B; int64_t ldb;
  void* C; int64_t ldc;
  uint16_t* C2; int64_t ldc2;
  const uint16_t* aux; int64_t ldaux;
  float* ws;
  int64_t M, N, K, f_s;
  int tiles_m, tiles_n, splits, kt_per_split;
  int accumulate;
};

__device__ __forceinline__ void store_bf16x4(uint16_t* dst, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// Interleave hints for the scheduler: `n` groups of {one instruction of class `mask`,
// then `mfma` MFMAs}. Masks: 0x008 MFMA, 0x020 VMEM read, 0x100 DS read, 0x200 DS write.
template <int kMask, int kN, int kMfma>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < kN; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMask, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma, 0);
  }
}

template <int BM, int BN, bool kAK, bool kBKc, Epi kEpi>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(KParams p) {
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 16, TN = WN / 16;
  constexpr bool kSw = kEpi == Epi::kSwiglu;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * kKStep];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Tile index: XCD-contiguous remap, then M-grouped order within the range.
  int bid = blockIdx.x;
  const int nwg = gridDim.x, full = (nwg / 8) * 8;
  if (bid < full) bid = (bid % 8) * (full / 8) + bid / 8;
  const int tiles = p.tiles_m * p.tiles_n;
  const int split = bid / tiles;
  const int t = bid - split * tiles;
  constexpr int kGroup = 8;
  const int per_group = kGroup * p.tiles_n;
  const int first_m = (t / per_group) * kGroup;
  const int gsize = min(p.tiles_m - first_m, kGroup);
  const int tm = first_m + (t % per_group) % gsize;
  const int tn = (t % per_group) / gsize;

  const int64_t m0 = int64_t(tm) * BM;
  const int64_t n0 = kSw ? int64_t(tn) * (BN / 2) : int64_t(tn) * BN;
  const RowMap rmA{m0, p.M, 0};
  const RowMap rmB{n0, kSw ? p.f_s : p.N, p.f_s};

  const int kt_total = int((p.K + kKStep - 1) / kKStep);
  const int kt_begin = split * p.kt_per_split;
  const int kt_end = min(kt_total, kt_begin + p.kt_per_split);

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Tile<BM, kAK, false> ta;
  Tile<BN, kBKc, kSw> tb;
  ta.init(p.A, p.lda, rmA, tid);
  tb.init(p.B, p.ldb, rmB, tid);

  // MFMA fragments of one 32-wide k sub-step, double-buffered in registers: the LDS
  // reads of sub-step s+1 are in flight while sub-step s feeds the matrix cores.
  struct Frag {
    u32x4_t a[TM], b[TN];
  };
  Frag f0, f1;
  const int frow_a = wm * WM + (lane & 15), frow_b = wn * WN + (lane & 15);
  auto read_frags = [&](Frag& f, const uint16_t* sA, const uint16_t* sB, int s) {
    const int chunk = s * 4 + (lane >> 4);
#pragma unroll
    for (int j = 0; j < TN; ++j) f.b[j] = *reinterpret_cast<const u32x4_t*>(sB + lds_off(frow_b + j * 16, chunk));
#pragma unroll
    for (int i = 0; i < TM; ++i) f.a[i] = *reinterpret_cast<const u32x4_t*>(sA + lds_off(frow_a + i * 16, chunk));
  };
  auto mma = [&](const Frag& f, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f.b[j]),
                                                           __builtin_bit_cast(bf16x8_t, f.a[i]), acc[i][j], 0, 0, 0);
  };

  uint16_t* const sA0 = smem;
  uint16_t* const sB0 = smem + BM * kKStep;
  uint16_t* const sA1 = smem + (BM + BN) * kKStep;
  uint16_t* const sB1 = sA1 + BM * kKStep;

  if (kt_begin < kt_end) {
    ta.load(int64_t(kt_begin) * kKStep, p.K);
    tb.load(int64_t(kt_begin) * kKStep, p.K);
    ta.store(sA0, tid);
    tb.store(sB0, tid);
    __syncthreads();
    ta.load(int64_t(kt_begin + 1) * kKStep, p.K);
    tb.load(int64_t(kt_begin + 1) * kKStep, p.K);
    read_frags(f0, sA0, sB0, 0);
  }
  // One k-step per iteration, a single basic block: loads past the end of the k range
  // read zeros (or another split's data) and their LDS stores are never read.
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const bool odd = (kt - kt_begin) & 1;
    const uint16_t* cA = odd ? sA1 : sA0;
    const uint16_t* cB = odd ? sB1 : sB0;
    uint16_t* nA = odd ? sA0 : sA1;
    uint16_t* nB = odd ? sB0 : sB1;
    // Sub-step 0 on the matrix cores; sub-step 1's fragments come in from LDS.
    read_frags(f1, cA, cB, 1);
    mma(f0, 0, TM);
    interleave<0x100, TM + TN, (TM * TN) / (TM + TN)>();
    __builtin_amdgcn_sched_barrier(0);
    // First half of sub-step 1; the next k-step's tile goes from registers to LDS.
    ta.store(nA, tid);
    tb.store(nB, tid);
    mma(f1, 0, TM / 2);
    interleave<0x200, decltype(ta)::kStores + decltype(tb)::kStores,
               (TM / 2 * TN) / (decltype(ta)::kStores + decltype(tb)::kStores)>();
    __syncthreads();
    // Second half of sub-step 1; the k-step after next is requested from memory and the
    // next k-step's first fragments are read.
    ta.load(int64_t(kt + 2) * kKStep, p.K);
    tb.load(int64_t(kt + 2) * kKStep, p.K);
    read_frags(f0, nA, nB, 0);
    mma(f1, TM / 2, TM);
    interleave<0x100, TM + TN, (TM / 2 * TN) / (TM + TN) ? (TM / 2 * TN) / (TM + TN) : 1>();
    __builtin_amdgcn_sched_barrier(0);
  }

  // Epilogue: lane holds C[m][n .. n+3] of each sub-tile.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + wm * WM + i * 16 + (lane & 15);
    if (m >= p.M) continue;
    if constexpr (kSw) {
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) {
        const int64_t jj = n0 + wn * (BN / 4) + j * 16 + 4 * (lane >> 4);
        if (jj >= p.f_s) continue;
        const f32x4_t g = acc[i][j], u = acc[i][j + TN / 2];
        uint16_t* hp = static_cast<uint16_t*>(p.C) + m * p.ldc;
        store_bf16x4(hp + jj, g.x, g.y, g.z, g.w);
        store_bf16x4(hp + p.f_s + jj, u.x, u.y, u.z, u.w);
        store_bf16x4(p.C2 + m * p.ldc2 + jj, silu_f(g.x) * u.x, silu_f(g.y) * u.y, silu_f(g.z) * u.z,
                     silu_f(g.w) * u.w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WN + j * 16 + 4 * (lane >> 4);
        if (n >= p.N) continue;
        const f32x4_t v = acc[i][j];
        if constexpr (kEpi == Epi::kStore) {
          store_bf16x4(static_cast<uint16_t*>(p.C) + m * p.ldc + n, v.x, v.y, v.z, v.w);
        } else if constexpr (kEpi == Epi::kGelu) {
          store_bf16x4(static_cast<uint16_t*>(p.C) + m * p.ldc + n, v.x, v.y, v.z, v.w);
          store_bf16x4(p.C2 + m * p.ldc2 + n, gelu_tanh_f(v.x), gelu_tanh_f(v.y), gelu_tanh_f(v.z),
                       gelu_tanh_f(v.w));
        } else if constexpr (kEpi == Epi::kDGelu) {
          const u32x2_t x = *reinterpret_cast<const u32x2_t*>(p.aux + m * p.ldaux + n);
          store_bf16x4(static_cast<uint16_t*>(p.C) + m * p.ldc + n, v.x * gelu_tanh_grad_f(bf16_lo(x.x)),
                       v.y * gelu_tanh_grad_f(bf16_hi(x.x)), v.z * gelu_tanh_grad_f(bf16_lo(x.y)),
                       v.w * gelu_tanh_grad_f(bf16_hi(x.y)));
        } else if constexpr (kEpi == Epi::kDSwiglu) {
          const u32x2_t gw = *reinterpret_cast<const u32x2_t*>(p.aux + m * p.ldaux + n);
          const u32x2_t uw = *reinterpret_cast<const u32x2_t*>(p.aux + m * p.ldaux + p.f_s + n);
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
        } else {  // kF32
          if (p.splits > 1) {
            *reinterpret_cast<f32x4_t*>(p.ws + int64_t(split) * p.M * p.N + m * p.N + n) = v;
          } else {
            f32x4_t* dst = reinterpret_cast<f32x4_t*>(static_cast<float*>(p.C) + m * p.ldc + n);
            *dst = p.accumulate ? (*dst + v) : v;
          }
        }
      }
    }
  }
}

struct TileCfg {
  int bm, bn;
};

template <bool kAK, bool kBKc, Epi kEpi>
hipError_t dispatch_tile(const TileCfg& tc, const KParams& kp, int blocks, hipStream_t s) {
  if (tc.bm == 256 && tc.bn == 128)
    hipLaunchKernelGGL((gemm_bf16_kernel<256, 128, kAK, kBKc, kEpi>), dim3(blocks), dim3(kThreads), 0, s, kp);
  else if (tc.bm == 128 && tc.bn == 256)
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 256, kAK, kBKc, kEpi>), dim3(blocks), dim3(kThreads), 0, s, kp);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, kAK, kBKc, kEpi>), dim3(blocks), dim3(kThreads), 0, s, kp);
  return hipGetLastError();
}

// Choose the tile that minimises (waves of workgroups) × (work per workgroup ÷ its
// relative efficiency) on 256 CUs, one workgroup per CU.
TileCfg choose_tile(int64_t M, int64_t Neff, bool swiglu) {
  const TileCfg cands[3] = {{256, 128}, {128, 256}, {128, 128}};
  const double eff[3] = {1.0, 1.0, 0.8};
  double best = 1e300;
  TileCfg bt = cands[0];
  for (int c = 0; c < 3; ++c) {
    const int64_t bn_cols = swiglu ? cands[c].bn / 2 : cands[c].bn;
    const int64_t tiles = ((M + cands[c].bm - 1) / cands[c].bm) * ((Neff + bn_cols - 1) / bn_cols);
    const int64_t waves = (tiles + 255) / 256;
    const double est = double(waves) * double(cands[c].bm) * double(cands[c].bn) / eff[c];
    if (est < best) {
      best = est;
      bt = cands[c];
    }
  }
  return bt;
}

}  // namespace

int64_t gemm_splitk_ws_elems(int64_t M, int64_t N, int64_t K) {
  const TileCfg tc = choose_tile(M, N, false);
  const int64_t tiles = ((M + tc.bm - 1) / tc.bm) * ((N + tc.bn - 1) / tc.bn);
  if (tiles >= 192 || K < 2048) return 0;
  int64_t splits = 1;
  while (tiles * splits * 2 <= 320 && K / (splits * 2) >= 1024) splits *= 2;
  return splits > 1 ? splits * M * N : 0;
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s, int* launches_out) {
  const bool sw = g.epi == Epi::kSwiglu;
  const TileCfg tc = choose_tile(g.M, g.N, sw);
  KParams kp{};
  kp.A = static_cast<const uint16_t*>(g.A); kp.lda = g.lda;
  kp.B = static_cast<const uint16_t*>(g.B); kp.ldb = g.ldb;
  kp.C = g.C; kp.ldc = g.ldc;
  kp.C2 = static_cast<uint16_t*>(g.C2); kp.ldc2 = g.ldc2;
  kp.aux = static_cast<const uint16_t*>(g.aux); kp.ldaux = g.ldaux;
  kp.M = g.M; kp.N = g.N; kp.K = g.K; kp.f_s = g.f_s;
  kp.accumulate = g.accumulate;
  const int64_t bn_cols = sw ? tc.bn / 2 : tc.bn;
  kp.tiles_m = int((g.M + tc.bm - 1) / tc.bm);
  kp.tiles_n = int((g.N + bn_cols - 1) / bn_cols);
  const int kt_total = int((g.K + kKStep - 1) / kKStep);
  int splits = 1;
  if (g.epi == Epi::kF32 && g.ws) {
    const int64_t need = gemm_splitk_ws_elems(g.M, g.N, g.K);
    if (need && need <= g.ws_elems) splits = int(need / (g.M * g.N));
  }
  kp.splits = splits;
  kp.kt_per_split = (kt_total + splits - 1) / splits;
  kp.ws = g.ws;
  const int blocks = kp.tiles_m * kp.tiles_n * splits;
  int launches = 0;
  if (blocks == 0) {
    if (launches_out) *launches_out = 0;
    return hipSuccess;
  }
  hipError_t e = hipSuccess;
  const bool ak = g.a_kcontig, bk = g.b_kcontig;
  switch (g.epi) {
    case Epi::kStore:
      if (ak && !bk) e = dispatch_tile<true, false, Epi::kStore>(tc, kp, blocks, s);
      else if (ak && bk) e = dispatch_tile<true, true, Epi::kStore>(tc, kp, blocks, s);
      else e = hipErrorInvalidValue;
      break;
    case Epi::kGelu:
      e = (ak && !bk) ? dispatch_tile<true, false, Epi::kGelu>(tc, kp, blocks, s) : hipErrorInvalidValue;
      break;
    case Epi::kSwiglu:
      e = (ak && !bk) ? dispatch_tile<true, false, Epi::kSwiglu>(tc, kp, blocks, s) : hipErrorInvalidValue;
      break;
    case Epi::kDGelu:
      e = (ak && bk) ? dispatch_tile<true, true, Epi::kDGelu>(tc, kp, blocks, s) : hipErrorInvalidValue;
      break;
    case Epi::kDSwiglu:
      e = (ak && bk) ? dispatch_tile<true, true, Epi::kDSwiglu>(tc, kp, blocks, s) : hipErrorInvalidValue;
      break;
    case Epi::kF32:
      e = (!ak && !bk) ? dispatch_tile<false, false, Epi::kF32>(tc, kp, blocks, s) : hipErrorInvalidValue;
      break;
  }
  ++launches;
  if (e == hipSuccess && splits > 1) {
    e = launch_splitk_sum(static_cast<float*>(g.C), g.ldc, g.ws, splits, g.M, g.N, g.accumulate, s);
    ++launches;
  }
  if (launches_out) *launches_out = launches;
  return e;
}

}  // namespace domino
