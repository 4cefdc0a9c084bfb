// bf16 GEMMs on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation,
// with the fused epilogues of the MLP shard: the forward's activation (tanh-GeLU or
// SwiGLU) and the backward's activation gradient, and fp32 weight-gradient output.
//
// The products are the "GeMM + GeLU + GeMM" kernel sequence of the MLP and the
// independent input-gradient / weight-gradient products of its backward (page
// "DeepSpeed-Domino 深度解析", sections "前向：多个计算片段轮转重叠 AllReduce" and
// "反向：扩展与权重梯度计算的重叠"; page "04 · TP/SP 的通信-计算 overlap 与工程优化", §1).
//
// Design (gfx950, 64-wide waves, 160 KB LDS per CU):
//  * 256 threads = 4 waves; block tile BM×BN with BM ∈ {128, 256}, BN ∈ {128, 160, 256}.
//    The waves form a 2×2 grid, or a 4×1 stack along M when BN/2 is not a whole number
//    of 32-column blocks (BN = 160); each wave owns its part as 32×32 MFMA blocks (the
//    32×32×16 shape sustains a higher issue rate than 16×16×32 with one wave per SIMD).
//  * K advances through a ring of NS LDS stages of BK k each. Stages are filled by
//    buffer loads that write LDS directly (no staging registers), NS−1 stages ahead of
//    the one being consumed; one barrier per stage.
//  * Within a stage, k advances 16 at a time; the fragments of sub-step s+1 (s+2 with one
//    workgroup per CU) are read from LDS while sub-step s runs on the matrix cores, one
//    read between consecutive MFMAs (MFMA issue blocks the wave, so the reads must not
//    form a run).
//  * An operand contiguous along k is staged [row][k] with an XOR chunk swizzle, and
//    each MFMA fragment (8 consecutive k of one row) is one 16-byte LDS read. An
//    operand contiguous along m (or n) — the [in, out] weights of the forward and both
//    operands of the weight gradients — is staged as it lies in memory, [k][m], and its
//    fragments are read transposed with ds_read_b64_tr_b16.
//  * The MFMA is issued with the operands swapped (B fragment as the matrix-core's A),
//    so each lane ends up with runs of 4 consecutive output columns of one row: 8-byte
//    bf16 stores and 16-byte fp32 stores in the epilogue.
//  * Workgroups are dispatched round-robin over the 8 XCDs; the tile index is remapped
//    so each XCD gets a contiguous, M-grouped range of tiles that share operand rows in
//    its L2.
#include <algorithm>
#include <cstdio>
#include <type_traits>

#include "common.hpp"
#include "gemm_common.hpp"
#include "kernels.hpp"

namespace domino {
namespace {

constexpr int kThreads = 256;

template <int BM, int BN, int BK, int NS, int kOcc, bool kAK, bool kBKc, Epi kEpi>
__global__ __launch_bounds__(kThreads, kOcc) void gemm_bf16_kernel(KParams p) {
  // Wave tile WM×WN as 32×32 blocks of v_mfma_f32_32x32x16_bf16 (k = 16 per MFMA); the
  // waves form WGM rows × WGN columns over the block tile.
  constexpr int WGM = (BN / 2) % 32 == 0 ? 2 : 4, WGN = 4 / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN, TM = WM / 32, TN = WN / 32, NSUB = BK / 16;
  constexpr bool kSw = kEpi == Epi::kSwiglu;
  static_assert(WM % 32 == 0 && WN % 32 == 0, "whole 32×32 blocks per wave");
  static_assert(!kSw || (WGM == 2 && TN % 2 == 0), "SwiGLU pairs gate and up blocks within a wave");
  static_assert(NSUB % 2 == 0, "sub-steps alternate between two fragment sets");
  using OA = typename std::conditional<kAK, OpK<BM, BK>, OpMN<BM, BK, false>>::type;
  using OB = typename std::conditional<kBKc, OpK<BN, BK>, OpMN<BN, BK, kSw>>::type;
  constexpr int kStage = (BM + BN) * BK;                // elements per stage
  constexpr int kLPS = OA::kLoads + OB::kLoads;         // DMA instructions per wave per stage
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS bases go to M0
  const int wm = wave / WGN, wn = wave % WGN;

  // Work item. Blocks 0 .. dp_tiles−1 compute whole tiles; the rest compute one k-slice of
  // one of the remaining tiles, slice-major. Workgroups are dispatched round-robin over
  // the 8 XCDs, so each range is remapped to give every XCD a contiguous run of items
  // (neighbouring tiles share operand rows in that XCD's L2).
  const int kt_total = int((p.K + BK - 1) / BK);
  const int tiles = p.tiles_m * p.tiles_n;
  const bool part = int(blockIdx.x) >= p.dp_tiles;
  int t, split = 0, kt_begin = 0, kt_end = kt_total;
  if (!part) {
    const int full = (p.dp_tiles / 8) * 8;
    const int b = blockIdx.x;
    t = b < full ? (b % 8) * (full / 8) + b / 8 : b;
  } else {
    const int rest = tiles - p.dp_tiles, items = rest * p.splits, full = (items / 8) * 8;
    const int b = blockIdx.x - p.dp_tiles;
    const int u = b < full ? (b % 8) * (full / 8) + b / 8 : b;
    split = u / rest;
    t = p.dp_tiles + (u - split * rest);
    kt_begin = split * p.kt_per_split;
    kt_end = min(kt_total, kt_begin + p.kt_per_split);
  }
  int tm, tn;
  tile_coords(t, p.tiles_m, p.tiles_n, tm, tn);

  const int64_t m0 = int64_t(tm) * BM;
  const int64_t n0 = kSw ? int64_t(tn) * (BN / 2) : int64_t(tn) * BN;
  const RowMap rmA{m0, p.M, 0};
  const RowMap rmB{n0, kSw ? p.f_s : p.N, p.f_s};

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  OA oa;
  OB ob;
  oa.init(p.A, p.lda, rmA, wave, lane);
  ob.init(p.B, p.ldb, rmB, wave, lane);

  struct Frag {
    u32x4_t a[TM], b[TN];
  };
  // Fragments are read kAhead sub-steps before their MFMAs: two with one workgroup per CU
  // (its four waves are the only ones to hide the LDS latency), else one. NF fragment sets
  // rotate with the sub-step.
  constexpr int kAhead = kOcc == 1 && NS >= 3 && NSUB % 4 == 0 ? 2 : 1;
  constexpr int NF = kAhead == 2 ? 4 : 2;
  Frag f[NF];
  // Fragment reads are inline assembly, so their order against the MFMAs is the order
  // written here and the compiler adds no waits of its own: through the builtins, each
  // transposed read would wait for every global→LDS copy in flight (the compiler cannot
  // tell which LDS they write), stalling every k-step on the copies it has just issued.
  // Read order of a sub-step: A0, B0 .. B(TN−1), A1 .. A(TM−1) (each fragment one 16-byte
  // read, or two transposed ones), the order in which the MFMAs (i outer, j inner) first
  // need them.
  constexpr int kRA = OA::kRd, kRB = OB::kRd;
  constexpr int kReads = TN * kRB + TM * kRA;
  auto read_op = [&](Frag& f, int slot, int s, int r) {
    const uint16_t* sa = smem + slot * kStage;
    const uint16_t* sb = sa + BM * BK;
    if (r < kRA) {
      OA::read(sa, wm * WM, s, lane, r, f.a[0]);
    } else if (r < kRA + TN * kRB) {
      const int q = r - kRA;
      OB::read(sb, wn * WN + (q / kRB) * 32, s, lane, q % kRB, f.b[q / kRB]);
    } else {
      const int q = r - kRA - TN * kRB + kRA;  // ≥ kRA: fragments A1 ..
      OA::read(sa, wm * WM + (q / kRA) * 32, s, lane, q % kRA, f.a[q / kRA]);
    }
  };
  // Last read (in the order above) that MFMA (i, j) needs.
  auto need = [&](int i, int j) { return i == 0 ? kRA + (j + 1) * kRB - 1 : kRA + TN * kRB + i * kRA - 1; };
  // Waits until this wave's fragment reads have all landed; tying the fragments keeps
  // their MFMAs after the wait.
  auto wait_frags = [&](Frag& f) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < TN; ++j) asm volatile("" : "+v"(f.b[j]));
#pragma unroll
    for (int i = 0; i < TM; ++i) asm volatile("" : "+v"(f.a[i]));
  };
  // One sub-step: the TM·TN MFMAs of `cur`, with the reads of the next sub-step's
  // fragments spread over the first kSpread MFMAs (MFMA issue blocks the wave, so the
  // reads must not form a run). Before each MFMA the wave waits only for the reads that
  // MFMA uses: LDS reads complete in order, so "at most n in flight" with n = the reads
  // issued after them covers exactly those.
  constexpr int NQ = TM * TN;
  constexpr int kLead = NQ >= 8 ? 3 : 1;
  constexpr int kSpread = NQ - kLead;
  auto issued_after = [&](int q) { return q < kSpread ? (q + 1) * kReads / kSpread : kReads; };
  // The refill of a freed slot. With one workgroup per CU and at least three stages, its
  // copies (kLPS per wave) are spread over the MFMAs of NSUB sub-steps, window position
  // w = 0 being the sub-step of the barrier that frees the slot and w = NSUB−1 the one
  // before the next barrier (whose stage wait counts them): issued all at once, the four
  // waves' copies queue behind each other in the CU's address unit while no wave issues
  // MFMAs. With two stages the spread copies would land just before they are waited for,
  // and with more workgroups per CU the others' MFMAs cover the burst, so there all of a
  // stage's copies are issued at the barrier.
  constexpr bool kSpreadCopies = kOcc == 1 && NS >= 3;
  // The refill's k-step and slot are kept as plain integers and the buffer resources
  // rebuilt per sub-step from them, which keeps them in scalar registers.
  int dkt = 0, dslot = 0;
  auto dma_at = [&](int w, int q) { return (w * NQ + q) * kLPS / (NSUB * NQ); };
  auto step = [&](Frag& cur, Frag& nxt, int rslot, int rs, int w, bool dma) {
    const typename OA::Src ra = kSpreadCopies ? oa.src(int64_t(dkt) * BK, p.K) : typename OA::Src{};
    const typename OB::Src rb = kSpreadCopies ? ob.src(int64_t(dkt) * BK, p.K) : typename OB::Src{};
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int i = q / TN, j = q % TN;
      const int before = q == 0 ? 0 : issued_after(q - 1);
      lgkm_wait_tied(min(15, kReads - 1 - need(i, j) + (kAhead - 1) * kReads + before), cur.a[i], cur.b[j]);
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, cur.b[j]),
                                                         __builtin_bit_cast(bf16x8_t, cur.a[i]), acc[i][j], 0, 0, 0);
#pragma unroll
      for (int r = before; r < issued_after(q); ++r) read_op(nxt, rslot, rs, r);
      if (kSpreadCopies && dma) {
        uint16_t* const dst = smem + dslot * kStage;
#pragma unroll
        for (int d = dma_at(w, q); d < dma_at(w, q + 1); ++d) {
          if (d < OA::kLoads) oa.issue_one(ra, dst, wave, d);
          else ob.issue_one(rb, dst + BM * BK, wave, d - OA::kLoads);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto issue = [&](int kt, int slot) {
    uint16_t* sa = smem + slot * kStage;
    const typename OA::Src ra = oa.src(int64_t(kt) * BK, p.K);
    const typename OB::Src rb = ob.src(int64_t(kt) * BK, p.K);
#pragma unroll
    for (int q = 0; q < OA::kLoads; ++q) oa.issue_one(ra, sa, wave, q);
#pragma unroll
    for (int q = 0; q < OB::kLoads; ++q) ob.issue_one(rb, sa + BM * BK, wave, q);
  };

  // Epilogue layout: each 32-row band i of the wave tile is handled in kPasses passes of
  // the wave, pass u covering output quad item = 64u + lane of the band, i.e. band row
  // item / QPR, columns 4·(item % QPR) .. +3 of the wave's WN columns (for SwiGLU: of its
  // WN/2 FFN columns), so consecutive lanes cover whole contiguous rows.
  constexpr int QPR = (kSw ? WN / 2 : WN) / 4;
  constexpr int kPasses = 32 * QPR / 64;
  static_assert(32 * QPR % 64 == 0, "whole passes");
  // The saved activation the backward epilogues read, in that layout. Loaded before the
  // stage ring is filled, so the loads overlap the whole k loop; being older than every
  // copy, they never delay a stage wait.
  constexpr bool kAux = kEpi == Epi::kDGelu || kEpi == Epi::kDSwiglu;
  AuxQuad ax[kAux ? TM : 1][kAux ? kPasses : 1];
  if constexpr (kAux) {
    if (!part) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int u = 0; u < kPasses; ++u) {
          const int item = 64 * u + lane;
          const int64_t m = m0 + wm * WM + i * 32 + item / QPR;
          const int64_t n = n0 + wn * WN + 4 * (item % QPR);
          ax[i][u] = m < p.M && n < p.N ? load_aux4<kEpi>(p, m, n) : AuxQuad{};
        }
    }
  }

  if (kt_begin < kt_end) {
    // Fill the ring: stages kt_begin .. kt_begin+NS-1 (stages past the k range load
    // zeros, or another split's data, and are never read).
#pragma unroll
    for (int st = 0; st < NS; ++st) issue(kt_begin + st, st);
    wait_vm_barrier<(NS - 1) * kLPS>();
#pragma unroll
    for (int r = 0; r < kReads; ++r) read_op(f[0], 0, 0, r);
    if constexpr (kAhead == 2) {
#pragma unroll
      for (int r = 0; r < kReads; ++r) read_op(f[1], 0, 1, r);
    }
    int slot = 0;
    for (int kt = kt_begin; kt < kt_end; ++kt) {
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        Frag& cur = f[s % NF];
        Frag& nxt = f[(s + kAhead) % NF];
        constexpr int sb = NSUB - kAhead;  // the sub-step that starts with the stage barrier
        if (s < sb) {
          step(cur, nxt, slot, s + kAhead, s + kAhead, kSpreadCopies && kt > kt_begin);
        } else {
          if (s == sb) {
            // Every wave has issued all reads of this stage (the barrier waits for them):
            // wait for the next stage, start refilling this slot NS stages ahead, and read
            // the next stage's first fragments from this sub-step on.
            wait_vm_barrier<(NS - 2) * kLPS>();
            if constexpr (kSpreadCopies) {
              dkt = __builtin_amdgcn_readfirstlane(kt + NS);
              dslot = __builtin_amdgcn_readfirstlane(slot);
            } else {
              issue(kt + NS, slot);
            }
            slot = slot + 1 == NS ? 0 : slot + 1;
          }
          step(cur, nxt, slot, s + kAhead - NSUB, s - sb, kSpreadCopies);
        }
      }
    }
    // The reads of the sub-step after the last are never used; they must land before their
    // registers are reused, and no LDS write may land after the workgroup ends.
#pragma unroll
    for (int q = 0; q < NF; ++q) wait_frags(f[q]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // Epilogue. With the operands swapped, lane l holds, for block (i, j) and q = 0..3,
  // C[m][n .. n+3] with m = row0 + l%32 and n = col0 + 8q + 4·(l/32): written from there,
  // one store instruction would touch 32 rows 16 bytes each. Each 32-row band of the wave
  // tile is staged in fp32 through a wave-private LDS region instead and read back in the
  // epilogue layout above, so stores (and the saved-activation loads) run along whole
  // rows; the epilogue still sees the fp32 sums.
  // Every wave has to be done with the stage ring before any overwrites it.
  __syncthreads();
  constexpr int RS = WN + 4;          // floats per staged row: rows 4 or 36 banks apart
  constexpr int kRegion = 32 * RS;    // floats per wave
  static_assert(4 * kRegion * 4 <= NS * kStage * 2, "staging fits in the stage ring");
  float* const stg = reinterpret_cast<float*>(smem) + wave * kRegion;
  float* const slot = part ? p.ws + (int64_t(t - p.dp_tiles) * p.splits + split) * (BM * BN) : nullptr;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4_t*>(stg + (lane & 31) * RS + j * 32 + 8 * q + 4 * (lane >> 5)) =
            f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    const int band = wm * WM + i * 32;  // tile-local first row
    // All of the band's values are read back before any is stored, so the LDS reads
    // overlap each other instead of each store waiting for its own.
    f32x4_t v[kPasses], v2[kSw ? kPasses : 1];
#pragma unroll
    for (int u = 0; u < kPasses; ++u) {
      const int item = 64 * u + lane;
      const float* src = stg + (item / QPR) * RS + 4 * (item % QPR);
      v[u] = *reinterpret_cast<const f32x4_t*>(src);
      if constexpr (kSw) v2[u] = *reinterpret_cast<const f32x4_t*>(src + WN / 2);
    }
    if (part) {
      // A k-slice: raw fp32 sums into this slice's [BM][BN] slot, by tile-local output
      // column (for SwiGLU: FFN columns 0..BN/2−1 hold gate, BN/2.. the matching up).
#pragma unroll
      for (int u = 0; u < kPasses; ++u) {
        const int item = 64 * u + lane, c = 4 * (item % QPR);
        float* row = slot + (band + item / QPR) * BN;
        if constexpr (kSw) {
          *reinterpret_cast<f32x4_t*>(row + wn * (BN / 4) + c) = v[u];
          *reinterpret_cast<f32x4_t*>(row + BN / 2 + wn * (BN / 4) + c) = v2[kSw ? u : 0];
        } else {
          *reinterpret_cast<f32x4_t*>(row + wn * WN + c) = v[u];
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kPasses; ++u) {
        const int item = 64 * u + lane, c = 4 * (item % QPR);
        const int64_t m = m0 + band + item / QPR;
        if constexpr (kSw) {
          const int64_t jj = n0 + wn * (BN / 4) + c;
          if (m < p.M && jj < p.f_s) epilogue_swiglu4(p, m, jj, v[u], v2[kSw ? u : 0]);
        } else {
          const int64_t n = n0 + wn * WN + c;
          if (m < p.M && n < p.N) epilogue4<kEpi>(p, m, n, v[u], ax[kAux ? i : 0][kAux ? u : 0]);
        }
      }
    }
  }
}

// Finishes the k-split tiles: sums each tile's slices in slice order (a fixed order, so the
// result does not depend on which workgroup ran first) and applies the product's epilogue.
// One thread per output quad: item = 256·block + thread over the split tiles' BM rows ×
// kQuads quads.
template <int BM, int BN, Epi kEpi>
__global__ __launch_bounds__(256) void gemm_fixup_kernel(KParams p) {
  constexpr bool kSw = kEpi == Epi::kSwiglu;
  constexpr int kCols = kSw ? BN / 2 : BN;  // output columns of a tile (FFN columns for SwiGLU)
  constexpr int kQuads = kCols / 4;
  const int64_t item = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int tt = int(item / (BM * kQuads));
  if (tt >= p.tiles_m * p.tiles_n - p.dp_tiles) return;
  const int r = int(item % (BM * kQuads)) / kQuads;
  const int c = int(item % kQuads) * 4;
  int tm, tn;
  tile_coords(p.dp_tiles + tt, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m = int64_t(tm) * BM + r;
  if (m >= p.M) return;
  const float* src = p.ws + int64_t(tt) * p.splits * (BM * BN) + r * BN + c;
  f32x4_t v = *reinterpret_cast<const f32x4_t*>(src);
  for (int z = 1; z < p.splits; ++z) v += *reinterpret_cast<const f32x4_t*>(src + int64_t(z) * (BM * BN));
  if constexpr (kSw) {
    f32x4_t u = *reinterpret_cast<const f32x4_t*>(src + BN / 2);
    for (int z = 1; z < p.splits; ++z) u += *reinterpret_cast<const f32x4_t*>(src + int64_t(z) * (BM * BN) + BN / 2);
    const int64_t j = int64_t(tn) * (BN / 2) + c;
    if (j < p.f_s) epilogue_swiglu4(p, m, j, v, u);
  } else {
    const int64_t n = int64_t(tn) * BN + c;
    if (n < p.N) epilogue4<kEpi>(p, m, n, v, load_aux4<kEpi>(p, m, n));
  }
}

// A block-tile configuration: BM×BN outputs, BK k per LDS stage, NS stages, and the
// workgroups per CU it is sized for (LDS NS·(BM+BN)·BK·2 bytes; registers per lane).
struct TileCfg {
  int bm, bn, bk, ns, occ;
};
// Per-CU rates on gfx950, measured in shader cycles: global→LDS copies 64 B/clk, LDS
// ds_read_b128 ~158 B/clk, ds_read_b64_tr_b16 ~103 B/clk, LDS writes ~75 B/clk, one
// 32×32×16 MFMA per 32 cycles per SIMD. At the MFMA rate a 128×128 tile needs all 64 B/clk
// of copies and more LDS time than there is; 256-wide tiles halve both per FLOP but cut
// the number of tiles, which small products need to fill 256 CUs.
enum TileId { kT128 = 0, kT128o3 = 1, kT256 = 2, kT256x128 = 3, kT128x256 = 4, kT256x160 = 5 };
constexpr TileCfg kTiles[] = {
    {128, 128, 64, 2, 2},  // 64 KB LDS, 2 workgroups per CU
    {128, 128, 32, 3, 3},  // 48 KB LDS, 3 per CU
    {256, 256, 64, 2, 1},  // 128 KB LDS, 1 per CU
    {256, 128, 32, 3, 2},  // 72 KB LDS, 2 per CU
    {128, 256, 32, 3, 2},  // 72 KB LDS, 2 per CU
    {256, 160, 64, 3, 1},  // 156 KB LDS, 1 per CU; waves stacked along M (64×160 each)
};

template <int BM, int BN, int BK, int NS, int kOcc, bool kAK, bool kBKc, Epi kEpi>
void launch_tile(const KParams& kp, int blocks, hipStream_t s) {
  DOMINO_LAUNCH((gemm_bf16_kernel<BM, BN, BK, NS, kOcc, kAK, kBKc, kEpi>), dim3(blocks), dim3(kThreads), 0, s, kp);
}

// Each operand layout is built only with the tiles make_plan can choose for it.
template <bool kAK, bool kBKc, Epi kEpi>
hipError_t dispatch_tile(int ti, const KParams& kp, int blocks, hipStream_t s) {
  const TileCfg& tc = kTiles[ti];
  char name[96];
  snprintf(name, sizeof name, "gemm_bf16_kernel<%d, %d, %d, %d, %d, %s, %s, (domino::Epi)%d>", tc.bm, tc.bn, tc.bk,
           tc.ns, tc.occ, kAK ? "true" : "false", kBKc ? "true" : "false", int(kEpi));
  note_kernel(name);
  if constexpr (kAK && !kBKc) {  // forward products: the [in, out] weight is n-major
    if (ti == kT128x256) {
      launch_tile<128, 256, 32, 3, 2, kAK, kBKc, kEpi>(kp, blocks, s);
    } else if (ti == kT128o3) {
      launch_tile<128, 128, 32, 3, 3, kAK, kBKc, kEpi>(kp, blocks, s);
    } else {
      if constexpr (kEpi == Epi::kSwiglu) {
        return hipErrorInvalidValue;  // gate/up pairing needs two waves along N
      } else {
        if (ti != kT256x160) return hipErrorInvalidValue;
        launch_tile<256, 160, 64, 3, 1, kAK, kBKc, kEpi>(kp, blocks, s);
      }
    }
  } else if constexpr (kAK && kBKc) {  // input gradients: both operands k-contiguous
    if (ti == kT128) {
      launch_tile<128, 128, 64, 2, 2, kAK, kBKc, kEpi>(kp, blocks, s);
    } else if (ti == kT256x160) {
      launch_tile<256, 160, 64, 3, 1, kAK, kBKc, kEpi>(kp, blocks, s);
    } else {
      if constexpr (kEpi == Epi::kDGelu || kEpi == Epi::kDSwiglu) {
        return hipErrorInvalidValue;  // epilogues reading the saved activation: 128×128 only
      } else {
        if (ti != kT256) return hipErrorInvalidValue;
        launch_tile<256, 256, 64, 2, 1, kAK, kBKc, kEpi>(kp, blocks, s);
      }
    }
  } else {  // weight gradients: both operands m/n-major
    switch (ti) {
      case kT128: launch_tile<128, 128, 64, 2, 2, kAK, kBKc, kEpi>(kp, blocks, s); break;
      case kT128o3: launch_tile<128, 128, 32, 3, 3, kAK, kBKc, kEpi>(kp, blocks, s); break;
      case kT256: launch_tile<256, 256, 64, 2, 1, kAK, kBKc, kEpi>(kp, blocks, s); break;
      case kT256x128: launch_tile<256, 128, 32, 3, 2, kAK, kBKc, kEpi>(kp, blocks, s); break;
      case kT128x256: launch_tile<128, 256, 32, 3, 2, kAK, kBKc, kEpi>(kp, blocks, s); break;
      case kT256x160: launch_tile<256, 160, 64, 3, 1, kAK, kBKc, kEpi>(kp, blocks, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <int BM, int BN, Epi kEpi>
void launch_fixup(const KParams& kp, int rest, hipStream_t s) {
  constexpr int kCols = kEpi == Epi::kSwiglu ? BN / 2 : BN;
  const int64_t items = int64_t(rest) * BM * (kCols / 4);
  DOMINO_LAUNCH((gemm_fixup_kernel<BM, BN, kEpi>), dim3(unsigned((items + 255) / 256)), dim3(256), 0, s, kp);
}

// k-split tiles occur for input gradients (tiles kT128, kT256) and weight gradients (any
// tile); forward products never split.
template <Epi kEpi>
hipError_t dispatch_fixup(int ti, const KParams& kp, int rest, hipStream_t s) {
  const TileCfg& tc = kTiles[ti];
  char name[64];
  snprintf(name, sizeof name, "gemm_fixup_kernel<%d, %d, (domino::Epi)%d>", tc.bm, tc.bn, int(kEpi));
  note_kernel(name);
  if constexpr (kEpi == Epi::kF32) {
    if (tc.bm == 128 && tc.bn == 128) launch_fixup<128, 128, kEpi>(kp, rest, s);
    else if (tc.bm == 256 && tc.bn == 256) launch_fixup<256, 256, kEpi>(kp, rest, s);
    else if (tc.bm == 256 && tc.bn == 128) launch_fixup<256, 128, kEpi>(kp, rest, s);
    else if (tc.bm == 256 && tc.bn == 160) launch_fixup<256, 160, kEpi>(kp, rest, s);
    else launch_fixup<128, 256, kEpi>(kp, rest, s);
  } else if constexpr (kEpi == Epi::kStore) {
    if (ti == kT256) launch_fixup<256, 256, kEpi>(kp, rest, s);
    else if (ti == kT128) launch_fixup<128, 128, kEpi>(kp, rest, s);
    else return hipErrorInvalidValue;
  } else if constexpr (kEpi == Epi::kDGelu || kEpi == Epi::kDSwiglu) {
    if (ti == kT128) launch_fixup<128, 128, kEpi>(kp, rest, s);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The launch plan of one product: its tile configuration, the tiles computed whole, and
// the k-split of the rest.
struct Plan {
  int ti, tiles_m, tiles_n, dp_tiles, splits, kt_per_split;
  int64_t ws_elems;  // fp32 slots the k-split tiles need
};

constexpr int kCUs = 256;
constexpr int64_t kMinSliceK = 512;  // k per slice of a split tile, at least

int tile_count(const TileCfg& tc, int64_t M, int64_t N, bool sw) {
  const int64_t bn = sw ? tc.bn / 2 : tc.bn;
  return int(((M + tc.bm - 1) / tc.bm) * ((N + bn - 1) / bn));
}

// Slices per leftover tile when the tiles beyond whole rounds of the 256·occ resident
// workgroups would fill at most 3/4 of a last round: enough to fill that round, each
// slice keeping at least kMinSliceK of k (1: no split).
int fill_split(int tiles, const TileCfg& tc, int64_t K) {
  const int slots = kCUs * tc.occ, rest = tiles % slots;
  if (rest == 0 || rest * 4 > slots * 3) return 1;
  const int64_t sp = std::min<int64_t>(std::min<int64_t>(slots / rest, 16), K / kMinSliceK);
  return sp >= 2 ? int(sp) : 1;
}

// Mean work per CU over the largest (1 = every CU equally busy), in tiles: the whole tiles
// spread over the CUs, then the leftover tiles' slices.
double cu_fill(int tiles, const TileCfg& tc, int sp) {
  const int slots = kCUs * tc.occ, rest = sp > 1 ? tiles % slots : 0, whole = tiles - rest;
  const double most = double((whole + kCUs - 1) / kCUs) + double((rest * sp + kCUs - 1) / kCUs) / sp;
  return most > 0 ? (double(tiles) / kCUs) / most : 1.0;
}

// A product whose 256×160 tiles make one round of at least 3/4 of the CUs runs them:
// one workgroup per CU with the LDS and copy traffic per MFMA of the large tiles.
bool one_round_256x160(const GemmArgs& g, bool sw) {
  if (sw) return false;
  const int t = tile_count(kTiles[kT256x160], g.M, g.N, false);
  return t <= kCUs && 4 * t >= 3 * kCUs;
}

// Products that run on the eight-wave 256×256 kernel (gemm8.hip): the first product of
// each direction (forward with its activation, activation gradient) and the input
// gradient, when their 256×256 tiles fill at least one round of the CUs. Measured on the
// Llama-2-13B shard (products alone): GEMM1 1040–1080 vs 1029 TFLOP/s, activation
// gradient 890–905 vs ~710, input gradient 1180–1200 vs ~1100 for the four-wave kernels.
// Products with a plain store and an n-major B (the second MLP product, the attention's
// output projection) take it when at least 2048 wide: alone they run 5–10% faster on the
// four-wave 128×256 tiles, but those leave no room on a CU for a reduction wave beside
// them (2·224 of 512 VGPRs), and in the step they run beside reductions (Llama-2-13B GEMM2
// chunks 0.86 vs 0.89 ms per step, the attention's output projection 137 vs 191 µs).
// Narrower ones stay on the four-wave tiles, except with a long k loop (k ≥ 4096) when the
// 256×256 tiles make one round on at least 3/4 of the CUs, or more rounds whose last one
// runs as half tiles: the QKV product of the GPT-3 6.7B layer stack per μ-batch (192
// tiles; stack 8.77 -> 8.69 ms) and of its attention block over 16384 rows (384 tiles;
// 228 -> 222 µs). The weight gradients (both operands m/n-major, read transposed) run
// 20–50% faster on the four-wave kernels' k-split.
bool pick_gemm8(const GemmArgs& g) {
  if (g.epi == Epi::kF32 || !gemm8_supports(g)) return false;
  const int64_t bn = g.epi == Epi::kSwiglu ? 128 : 256;
  const int64_t tiles = ((g.M + 255) / 256) * ((g.N + bn - 1) / bn);
  if (g.epi == Epi::kStore && !g.b_kcontig && g.N < 2048)
    return g.K >= 4096 && tiles >= kCUs * 3 / 4 && (tiles <= kCUs || 2 * (tiles % kCUs) <= kCUs);
  return tiles >= kCUs;
}

Plan make_plan(const GemmArgs& g) {
  const bool sw = g.epi == Epi::kSwiglu;
  Plan pl{};
  int sp = 1;
  if (g.a_kcontig && one_round_256x160(g, sw)) {
    pl.ti = kT256x160;
  } else if (g.a_kcontig && !g.b_kcontig) {
    // Forward products: 128×256 tiles when there are at least two per CU, else 128×128 at
    // three workgroups per CU; they are not split (the fixed-order slice sum costs more
    // than the idle tail it saves at these k).
    pl.ti = tile_count(kTiles[kT128x256], g.M, g.N, sw) >= 2 * kCUs ? kT128x256 : kT128o3;
  } else if (g.a_kcontig && g.b_kcontig) {
    // Input gradients: 256×256 for large grids with k ≥ 2048, unless the epilogue reads the
    // saved activation (its loads then overlap other workgroups' loops only with two
    // workgroups per CU); a half-empty last round splits in two when k ≥ 2048.
    const bool aux = g.epi == Epi::kDGelu || g.epi == Epi::kDSwiglu;
    pl.ti = !aux && g.K >= 2048 && tile_count(kTiles[kT256], g.M, g.N, false) >= 2 * kCUs ? kT256 : kT128;
    const TileCfg& tc = kTiles[pl.ti];
    const int slots = kCUs * tc.occ, rest = tile_count(tc, g.M, g.N, false) % slots;
    if (rest > 0 && rest * 2 <= slots && g.K >= 2048) sp = 2;
  } else {
    // Weight gradients (k = tokens, long): the tile whose k-split fills the CUs best,
    // weighted by its measured relative rate on these operands.
    constexpr TileId kCand[] = {kT256x160, kT256x128, kT128x256, kT128o3, kT128, kT256};
    constexpr double kRate[] = {0.84, 1.00, 0.98, 0.96, 0.93, 0.90};
    double best = -1.0;
    for (int c = 0; c < 6; ++c) {
      const TileCfg& tc = kTiles[kCand[c]];
      const int tiles = tile_count(tc, g.M, g.N, false), s = fill_split(tiles, tc, g.K);
      const double score = cu_fill(tiles, tc, s) * kRate[c];
      if (score > best) {
        best = score;
        pl.ti = kCand[c];
        sp = s;
      }
    }
  }
  const TileCfg& tc = kTiles[pl.ti];
  const int64_t bn_cols = sw ? tc.bn / 2 : tc.bn;
  pl.tiles_m = int((g.M + tc.bm - 1) / tc.bm);
  pl.tiles_n = int((g.N + bn_cols - 1) / bn_cols);
  const int tiles = pl.tiles_m * pl.tiles_n;
  const int kt_total = int((g.K + tc.bk - 1) / tc.bk);
  pl.dp_tiles = tiles;
  pl.splits = 1;
  pl.kt_per_split = kt_total;
  pl.ws_elems = 0;
  if (sp < 2 || tiles == 0) return pl;
  const int rest = tiles % (kCUs * tc.occ);
  pl.kt_per_split = (kt_total + sp - 1) / sp;
  pl.splits = (kt_total + pl.kt_per_split - 1) / pl.kt_per_split;  // no empty slice
  if (pl.splits < 2 || rest == 0) {
    pl.kt_per_split = kt_total;
    pl.splits = 1;
    return pl;
  }
  pl.dp_tiles = tiles - rest;
  pl.ws_elems = int64_t(rest) * pl.splits * tc.bm * tc.bn;
  return pl;
}

KParams make_params(const GemmArgs& g, const Plan& pl) {
  KParams kp{};
  kp.A = static_cast<const uint16_t*>(g.A); kp.lda = g.lda;
  kp.B = static_cast<const uint16_t*>(g.B); kp.ldb = g.ldb;
  kp.C = g.C; kp.ldc = g.ldc;
  kp.C2 = static_cast<uint16_t*>(g.C2); kp.ldc2 = g.ldc2;
  kp.aux = static_cast<const uint16_t*>(g.aux); kp.ldaux = g.ldaux;
  kp.bias = static_cast<const uint16_t*>(g.bias);
  kp.ws = g.ws;
  kp.M = g.M; kp.N = g.N; kp.K = g.K; kp.f_s = g.f_s;
  kp.tiles_m = pl.tiles_m; kp.tiles_n = pl.tiles_n;
  kp.dp_tiles = pl.dp_tiles; kp.splits = pl.splits; kp.kt_per_split = pl.kt_per_split;
  kp.accumulate = g.accumulate;
  return kp;
}

// The plan a launch with this workspace uses: without room for the slices, every tile
// runs whole.
Plan plan_for(const GemmArgs& g) {
  Plan pl = make_plan(g);
  if (pl.splits > 1 && (!g.ws || g.ws_elems < pl.ws_elems)) {
    pl.dp_tiles = pl.tiles_m * pl.tiles_n;
    pl.splits = 1;
    pl.kt_per_split = int((g.K + kTiles[pl.ti].bk - 1) / kTiles[pl.ti].bk);
    pl.ws_elems = 0;
  }
  return pl;
}

}  // namespace

bool use_gemm8(const GemmArgs& g) { return pick_gemm8(g); }

int64_t gemm_bf16_ws_elems(const GemmArgs& g) { return use_gemm8(g) ? 0 : make_plan(g).ws_elems; }

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s, GemmSplit* split) {
  if (split) *split = GemmSplit{};
  if (pick_gemm8(g)) return launch_gemm8(g, s);
  const Plan pl = plan_for(g);
  const KParams kp = make_params(g, pl);
  const int tiles = pl.tiles_m * pl.tiles_n;
  const int blocks = pl.dp_tiles + (tiles - pl.dp_tiles) * pl.splits;
  if (split) *split = GemmSplit{};
  if (blocks == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  const bool ak = g.a_kcontig, bk = g.b_kcontig;
  const int ti = pl.ti;
  switch (g.epi) {
    case Epi::kStore:
      if (ak && !bk) e = dispatch_tile<true, false, Epi::kStore>(ti, kp, blocks, s);
      else if (ak && bk) e = dispatch_tile<true, true, Epi::kStore>(ti, kp, blocks, s);
      else e = hipErrorInvalidValue;
      break;
    case Epi::kGelu:
      e = (ak && !bk) ? dispatch_tile<true, false, Epi::kGelu>(ti, kp, blocks, s) : hipErrorInvalidValue;
      break;
    case Epi::kSwiglu:
      e = (ak && !bk) ? dispatch_tile<true, false, Epi::kSwiglu>(ti, kp, blocks, s) : hipErrorInvalidValue;
      break;
    case Epi::kDGelu:
      e = (ak && bk) ? dispatch_tile<true, true, Epi::kDGelu>(ti, kp, blocks, s) : hipErrorInvalidValue;
      break;
    case Epi::kDSwiglu:
      e = (ak && bk) ? dispatch_tile<true, true, Epi::kDSwiglu>(ti, kp, blocks, s) : hipErrorInvalidValue;
      break;
    case Epi::kF32:
      e = (!ak && !bk) ? dispatch_tile<false, false, Epi::kF32>(ti, kp, blocks, s) : hipErrorInvalidValue;
      break;
  }
  if (e == hipSuccess && split && pl.splits > 1) {
    split->pending = 1;
    split->tile = pl.ti;
    split->tiles_m = pl.tiles_m;
    split->tiles_n = pl.tiles_n;
    split->dp_tiles = pl.dp_tiles;
    split->splits = pl.splits;
  }
  return e;
}

hipError_t launch_gemm_bf16_fixup(const GemmArgs& g, const GemmSplit& sp, hipStream_t s) {
  if (!sp.pending) return hipSuccess;
  Plan pl{};
  pl.ti = sp.tile;
  pl.tiles_m = sp.tiles_m;
  pl.tiles_n = sp.tiles_n;
  pl.dp_tiles = sp.dp_tiles;
  pl.splits = sp.splits;
  const KParams kp = make_params(g, pl);
  const int rest = sp.tiles_m * sp.tiles_n - sp.dp_tiles;
  switch (g.epi) {
    case Epi::kStore: return dispatch_fixup<Epi::kStore>(sp.tile, kp, rest, s);
    case Epi::kGelu: return dispatch_fixup<Epi::kGelu>(sp.tile, kp, rest, s);
    case Epi::kSwiglu: return dispatch_fixup<Epi::kSwiglu>(sp.tile, kp, rest, s);
    case Epi::kDGelu: return dispatch_fixup<Epi::kDGelu>(sp.tile, kp, rest, s);
    case Epi::kDSwiglu: return dispatch_fixup<Epi::kDSwiglu>(sp.tile, kp, rest, s);
    case Epi::kF32: return dispatch_fixup<Epi::kF32>(sp.tile, kp, rest, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace domino
