// bf16 GEMM with eight waves per workgroup in two ping-pong groups (gfx950), for the large
// products of the MLP shard: 256×256 output tiles, one workgroup per CU, two waves per SIMD.
//
// The products are the "GeMM + GeLU + GeMM" kernel sequence of the MLP and the independent
// input-gradient / weight-gradient products of its backward (page "DeepSpeed-Domino 深度解析",
// sections "前向：多个计算片段轮转重叠 AllReduce" and "反向：扩展与权重梯度计算的重叠";
// page "04 · TP/SP 的通信-计算 overlap 与工程优化", §1).
//
// Design:
//  * 512 threads = 8 waves; the hardware places waves w and w + 4 on the same SIMD. Waves
//    0–3 form group 0 and waves 4–7 group 1, so every SIMD holds one wave of each group.
//    Wave (g, i) owns the 64×128 output block at rows 64·i, columns 128·g of the tile:
//    2×4 blocks of v_mfma_f32_32x32x16_bf16, 128 fp32 accumulators held in AGPRs.
//  * k advances 32 at a time. A step has a memory phase (the wave reads all its fragments
//    of the step from LDS — 4 A and 8 B 16-byte fragments — and issues its share of a later
//    step's global→LDS copies) and a compute phase (its 16 MFMAs on those fragments). The
//    two groups run the phases offset by one: while group 0 computes step k, group 1 reads
//    step k, and the other way round, separated by workgroup barriers. Each SIMD's matrix
//    core is then fed by one wave while the other wave's LDS reads and copies go on, which
//    a single wave per SIMD can only approximate by interleaving (the four-wave kernel's
//    matrix cores were busy 24–38% of cycles).
//  * The operand tiles of a step (A 256×32 and B 256×32, 16 KB each) reach LDS through
//    buffer loads that write LDS directly, in a ring of four stages (128 KB). Group 0
//    copies A and group 1 copies B, each during its memory phase, three steps ahead of
//    the group's next read; each group waits for its own copies of the next step before
//    the barrier that precedes that step's first read.
//  * LDS layouts and fragment reads are those of the four-wave kernel (gemm_common.hpp):
//    k-contiguous operands [row][k] with an XOR chunk swizzle (one ds_read_b128 per
//    fragment), m/n-contiguous ones [k][mn] read transposed (ds_read_b64_tr_b16).
//  * The epilogue stages each wave's 32-row bands in fp32 through LDS and writes whole rows,
//    applying the product's fused epilogue.
#include <algorithm>
#include <cstdio>
#include <type_traits>

#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace domino {
namespace {

constexpr int k8Threads = 512;

constexpr int kBK8 = 32, kNS8 = 4;
constexpr int kStage8 = (256 + 256) * kBK8;  // bf16 elements per stage (32 KB)
constexpr int kRS8 = 128 + 4;                // floats per staged epilogue row: rows 4 banks apart
constexpr int kRegion8 = 32 * kRS8;          // floats staged per wave
constexpr int kSmem8 = kNS8 * kStage8 > 8 * kRegion8 * 2 ? kNS8 * kStage8 : 8 * kRegion8 * 2;

// One output tile of 128·TM rows × 256 columns at (m0, n0): TM = 2 is the whole 256×256
// tile, TM = 1 the half tile (each wave then owns 32 rows instead of 64).
template <bool kAK, bool kBKc, Epi kEpi, int TM>
__device__ __forceinline__ void gemm8_tile(const KParams& p, uint16_t* smem, int64_t m0, int64_t n0) {
  constexpr int BM = 128 * TM, BN = 256, BK = kBK8, NS = kNS8;
  constexpr int TN = 4;  // 32×32 blocks per wave
  constexpr int WM = 32 * TM;  // rows per wave
  constexpr bool kSw = kEpi == Epi::kSwiglu;
  using OA = typename std::conditional<kAK, OpK<BM, BK>, OpMN<BM, BK, false>>::type;
  using OB = typename std::conditional<kBKc, OpK<BN, BK, kSw>, OpMN<BN, BK, kSw>>::type;
  constexpr int kLoadsA = OA::kLoads, kLoadsB = OB::kLoads;  // 1 KB copies per wave per step
  static_assert(kLoadsA == 2 * TM && kLoadsB == 4, "copies per wave per step");
  constexpr int kStage = kStage8;
  constexpr int RS = kRS8;
  constexpr int kRegion = kRegion8;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2, wi = wave & 3;
  const RowMap rmA{m0, p.M, 0};
  const RowMap rmB{n0, kSw ? p.f_s : p.N, p.f_s};

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Group 0 copies the A tile of each step, group 1 the B tile.
  OA oa;
  OB ob;
  if (g == 0) oa.init(p.A, p.lda, rmA, wi, lane);
  else ob.init(p.B, p.ldb, rmB, wi, lane);
  auto issue = [&](int kt) {
    uint16_t* st = smem + (kt % NS) * kStage;
    if (g == 0) {
      const typename OA::Src sr = oa.src(int64_t(kt) * BK, p.K);
#pragma unroll
      for (int q = 0; q < kLoadsA; ++q) oa.issue_one(sr, st, wi, q);
    } else {
      const typename OB::Src sr = ob.src(int64_t(kt) * BK, p.K);
#pragma unroll
      for (int q = 0; q < kLoadsB; ++q) ob.issue_one(sr, st + BM * BK, wi, q);
    }
  };

  // The step's fragments: [k16 sub-step][block].
  u32x4_t fa[2][TM], fb[2][TN];
  auto read_frags = [&](int kt) {
    const uint16_t* sa = smem + (kt % NS) * kStage;
    const uint16_t* sb = sa + BM * BK;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < OA::kRd; ++r) OA::read(sa, wi * WM + i * 32, s, lane, r, fa[s][i]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < OB::kRd; ++r) OB::read(sb, g * 128 + j * 32, s, lane, r, fb[s][j]);
    }
  };
  // All fragment reads landed; tying the registers keeps the MFMAs after the wait.
  auto wait_frags = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int i = 0; i < TM; ++i) asm volatile("" : "+v"(fa[s][i]));
#pragma unroll
      for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(fb[s][j]));
    }
  };
  auto compute = [&]() {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fb[s][j]),
                                                              __builtin_bit_cast(bf16x8_t, fa[s][i]), acc[i][j], 0,
                                                              0, 0);
  };
  auto pin_acc = [&]() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) asm volatile("" : "+a"(acc[i][j]));
  };

  const int kt_total = int((p.K + BK - 1) / BK);
  // Fill the ring: steps 0 .. NS−2 (steps past the k range load zeros and are never read).
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) issue(st);
  // Step 0 of this group's operand landed (the later two may be in flight), then the
  // barrier publishes it to the other group.
  if (g == 0) wait_vm_barrier<(NS - 2) * kLoadsA>();
  else wait_vm_barrier<(NS - 2) * kLoadsB>();
  // Phases are separated by workgroup barriers; group 1 runs one phase behind group 0.
  if (g == 1) asm volatile("s_barrier" ::: "memory");
  for (int kt = 0; kt < kt_total; ++kt) {
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
    // Memory phase: this step's fragments, and the copies of step kt + NS − 1 into the
    // slot of step kt − 1 (both groups finished reading it before the last barrier).
    read_frags(kt);
    issue(kt + NS - 1);
    wait_frags();
    // Group 1's copies of step kt + 1 must have landed before group 0 reads that step,
    // which follows this barrier.
    if (g == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * kLoadsB) : "memory");
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // Compute phase.
    compute();
    __builtin_amdgcn_sched_barrier(0);
    // Group 0's copies of step kt + 1 must have landed before it reads that step next.
    if (g == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * kLoadsA) : "memory");
    asm volatile("s_barrier" ::: "memory");
  }
  pin_acc();
  // Copies past the k range may still be in flight in either group; every wave drains its
  // own, and the barrier after group 0's closing one (which pairs with group 1's last loop
  // barrier) keeps all waves out of the epilogue until both groups have: the epilogue
  // stages through the ring, and a late copy landing there would overwrite staged sums.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (g == 0) asm volatile("s_barrier" ::: "memory");
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // Epilogue. With the operands swapped in the MFMA, lane l holds, for block (i, j) and
  // q = 0..3, C[m][n .. n+3] with m = row0 + l%32 and n = col0 + 8q + 4·(l/32). Each 32-row
  // band of the wave's block is staged in fp32 through a wave-private LDS region and read
  // back so that consecutive lanes cover whole rows: item = 64u + lane of the band is row
  // item / QPR, output quad item % QPR (for SwiGLU, of the 64 FFN columns whose gate and up
  // values the wave holds).
  constexpr int WN = 128;
  constexpr int QPR = (kSw ? WN / 2 : WN) / 4;
  constexpr int kPasses = 32 * QPR / 64;
  constexpr bool kAux = kEpi == Epi::kDGelu || kEpi == Epi::kDSwiglu;
  float* const stg = reinterpret_cast<float*>(smem) + wave * kRegion;
  // Four passes at a time: their staged values (and saved-activation loads) are issued
  // before any is used, so the loads overlap, within the registers the loop leaves free.
  constexpr int kGrp = 4;
  static_assert(kPasses % kGrp == 0, "whole groups of passes");
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int band = wi * WM + i * 32;  // tile-local first row
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4_t*>(stg + (lane & 31) * RS + j * 32 + 8 * q + 4 * (lane >> 5)) =
            f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
#pragma unroll
    for (int u0 = 0; u0 < kPasses; u0 += kGrp) {
      AuxQuad ax[kAux ? kGrp : 1];
      f32x4_t v[kGrp], v2[kSw ? kGrp : 1];
#pragma unroll
      for (int u = 0; u < kGrp; ++u) {
        const int item = 64 * (u0 + u) + lane;
        if constexpr (kAux) {
          const int64_t m = m0 + band + item / QPR;
          const int64_t n = n0 + g * WN + 4 * (item % QPR);
          ax[u] = m < p.M && n < p.N ? load_aux4<kEpi>(p, m, n) : AuxQuad{};
        }
        const float* src = stg + (item / QPR) * RS + 4 * (item % QPR);
        v[u] = *reinterpret_cast<const f32x4_t*>(src);
        if constexpr (kSw) v2[u] = *reinterpret_cast<const f32x4_t*>(src + WN / 2);
      }
#pragma unroll
      for (int u = 0; u < kGrp; ++u) {
        const int item = 64 * (u0 + u) + lane, c = 4 * (item % QPR);
        const int64_t m = m0 + band + item / QPR;
        if constexpr (kSw) {
          const int64_t jj = n0 + g * (WN / 2) + c;
          if (m < p.M && jj < p.f_s) epilogue_swiglu4(p, m, jj, v[u], v2[kSw ? u : 0]);
        } else {
          const int64_t n = n0 + g * WN + c;
          if (m < p.M && n < p.N) epilogue4<kEpi>(p, m, n, v[u], ax[kAux ? u : 0]);
        }
      }
    }
  }
}

// Workgroups 0 .. dp_tiles−1 compute whole 256×256 tiles; when the tiles do not fill their
// last round of the CUs, the remaining ones (dp_tiles .. tiles−1) are computed as two
// 128-row halves each by the workgroups after those, so the partial round takes about half
// the time. Workgroups are dispatched round-robin over the 8 XCDs; each range is remapped
// so every XCD gets a contiguous, M-grouped run of tiles (and both halves of a tile).
template <bool kAK, bool kBKc, Epi kEpi>
__global__ __launch_bounds__(k8Threads, 1) void gemm8_kernel(KParams p) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[kSmem8];
  constexpr bool kSw = kEpi == Epi::kSwiglu;
  const int b = blockIdx.x;
  int t, half = -1;
  if (b < p.dp_tiles) {
    const int full = (p.dp_tiles / 8) * 8;
    t = b < full ? (b % 8) * (full / 8) + b / 8 : b;
  } else {
    const int items = 2 * (p.tiles_m * p.tiles_n - p.dp_tiles), full = (items / 8) * 8;
    const int hb = b - p.dp_tiles;
    const int u = hb < full ? (hb % 8) * (full / 8) + hb / 8 : hb;
    t = p.dp_tiles + u / 2;
    half = u % 2;
  }
  int tm, tn;
  tile_coords(t, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t n0 = kSw ? int64_t(tn) * 128 : int64_t(tn) * 256;
  if (half < 0) gemm8_tile<kAK, kBKc, kEpi, 2>(p, smem, int64_t(tm) * 256, n0);
  else gemm8_tile<kAK, kBKc, kEpi, 1>(p, smem, int64_t(tm) * 256 + half * 128, n0);
}

template <bool kAK, bool kBKc, Epi kEpi>
hipError_t launch8(const KParams& kp, int blocks, hipStream_t s) {
  char name[96];
  snprintf(name, sizeof name, "gemm8_kernel<%s, %s, (domino::Epi)%d>", kAK ? "true" : "false",
           kBKc ? "true" : "false", int(kEpi));
  note_kernel(name);
  DOMINO_LAUNCH((gemm8_kernel<kAK, kBKc, kEpi>), dim3(blocks), dim3(k8Threads), 0, s, kp);
  return hipGetLastError();
}

}  // namespace

bool gemm8_supports(const GemmArgs& g) {
  const bool ak = g.a_kcontig, bk = g.b_kcontig;
  switch (g.epi) {
    case Epi::kStore: return ak;
    case Epi::kGelu:
    case Epi::kSwiglu: return ak;
    case Epi::kDGelu:
    case Epi::kDSwiglu: return ak && bk;
    case Epi::kF32: return !ak && !bk;
  }
  return false;
}

// Whole 256×256 tiles, one workgroup each (no workspace).
hipError_t launch_gemm8(const GemmArgs& g, hipStream_t s) {
  KParams kp{};
  kp.A = static_cast<const uint16_t*>(g.A); kp.lda = g.lda;
  kp.B = static_cast<const uint16_t*>(g.B); kp.ldb = g.ldb;
  kp.C = g.C; kp.ldc = g.ldc;
  kp.C2 = static_cast<uint16_t*>(g.C2); kp.ldc2 = g.ldc2;
  kp.aux = static_cast<const uint16_t*>(g.aux); kp.ldaux = g.ldaux;
  kp.bias = static_cast<const uint16_t*>(g.bias);
  kp.M = g.M; kp.N = g.N; kp.K = g.K; kp.f_s = g.f_s;
  const int64_t bn = g.epi == Epi::kSwiglu ? 128 : 256;
  kp.tiles_m = int((g.M + 255) / 256);
  kp.tiles_n = int((g.N + bn - 1) / bn);
  const int tiles = kp.tiles_m * kp.tiles_n;
  // A last round filling at most half the CUs runs as half tiles (twice the workgroups).
  constexpr int kCUs8 = 256;
  const int rest = tiles % kCUs8;
  kp.dp_tiles = tiles > kCUs8 && rest > 0 && 2 * rest <= kCUs8 ? tiles - rest : tiles;
  kp.splits = 1;
  kp.kt_per_split = int((g.K + 31) / 32);
  kp.accumulate = g.accumulate;
  const int blocks = kp.dp_tiles + 2 * (tiles - kp.dp_tiles);
  if (blocks == 0) return hipSuccess;
  const bool ak = g.a_kcontig, bk = g.b_kcontig;
  switch (g.epi) {
    case Epi::kStore:
      if (ak && !bk) return launch8<true, false, Epi::kStore>(kp, blocks, s);
      if (ak && bk) return launch8<true, true, Epi::kStore>(kp, blocks, s);
      break;
    case Epi::kGelu:
      if (ak && !bk) return launch8<true, false, Epi::kGelu>(kp, blocks, s);
      if (ak && bk) return launch8<true, true, Epi::kGelu>(kp, blocks, s);
      break;
    case Epi::kSwiglu:
      if (ak && !bk) return launch8<true, false, Epi::kSwiglu>(kp, blocks, s);
      if (ak && bk) return launch8<true, true, Epi::kSwiglu>(kp, blocks, s);
      break;
    case Epi::kDGelu:
      if (ak && bk) return launch8<true, true, Epi::kDGelu>(kp, blocks, s);
      break;
    case Epi::kDSwiglu:
      if (ak && bk) return launch8<true, true, Epi::kDSwiglu>(kp, blocks, s);
      break;
    case Epi::kF32:
      if (!ak && !bk) return launch8<false, false, Epi::kF32>(kp, blocks, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace domino
