// Causal self-attention backward for one rank's head slice (bf16, head_dim 128): dQ, dK and
// dV from Q, K, V (the saved QKV), O, dO and the forward's per-row log-sum-exp. The
// attention is the layer's A on the rank's heads (page "DeepSpeed-Domino 深度解析",
// sections "TP 的数据依赖：通信为何难以隐藏" and "反向：扩展与权重梯度计算的重叠"); causal
// self-attention only (section "如何尝试 DeepSpeed-Domino").
//
// With P rebuilt from the LSE (P = exp(scale·s − LSE), no renormalising):
//   dV = Pᵀ·dO,  dP = dO·Vᵀ,  dS = P ⊙ (dP − Δ) with Δ_q = Σ_d dO_qd·O_qd (= Σ_k P_qk·dP_qk),
//   dQ = scale·dS·K,  dK = scale·dSᵀ·Q.
// Three launches and no atomics, so results do not depend on timing:
//  * prep: Δ per (token, head), and LSE·log2 e, stored head-major so the values of a block
//    of queries are one contiguous run;
//  * dK/dV: one workgroup per (sequence, head, 128 keys), each wave 32 keys whose K and V
//    fragments stay in registers; blocks of 64 queries (from the diagonal on) stream
//    through LDS. S and dP come out of the MFMAs with one key per lane (16 queries in its
//    registers), so P and dS are already the B operand of dVᵀ += dOᵀ·P and dKᵀ += Qᵀ·dS,
//    whose A operand is dO or Q read transposed out of LDS (ds_read_b64_tr_b16);
//  * dQ: one workgroup per (sequence, head, 128 queries), as in the forward: blocks of 64
//    keys stream through LDS, S and dP come out with one query per lane, and
//    dQᵀ += Kᵀ·dSᵀ reads K transposed.
// Every LDS tile is [row][d] with the 16-byte chunk c of row r at c ^ sw(r), sw(r) the low
// four bits of r with their two halves swapped: a row read (16 consecutive rows × one chunk)
// and a transposed read (4 consecutive rows × 4 consecutive chunks per 32 lanes) both hit
// every bank once. (With c ^ (r & 15) the transposed reads hit half the banks twice.) LDS reads are inline assembly with explicit waits (through the builtins
// the compiler would make them wait for the global→LDS copies of the next block).
#include "common.hpp"
#include "kernels.hpp"

namespace domino {
namespace {

constexpr int kD = 128;    // head_dim
constexpr int kWG = 128;   // keys (dK/dV) or queries (dQ) per workgroup
constexpr int kBlk = 64;   // queries (dK/dV) or keys (dQ) per streamed block
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int sw(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int t_off(int row, int chunk) { return row * kD + ((chunk ^ sw(row)) << 3); }

struct BwdParams {
  const uint16_t* qkv; int64_t ld_qkv;
  const uint16_t* o; const uint16_t* dout; int64_t ld_o;
  const float* lse; int64_t ld_lse;
  uint16_t* dqkv; int64_t ld_dqkv;
  uint16_t* stx;         // [heads][T][8] bf16 stats entries (L = LSE/scale and Δ, three parts each)
  float* stats;          // [heads][T] LSE·log2 e, then [heads][T] Δ
  int64_t T, hd;
  int seq, heads, batch;
  float scale, scale_log2;
};

// One 16-byte fragment of d-chunk `chunk` (8 values) for the MFMA: row = the lane's row.
__device__ __forceinline__ u32x4_t ld_frag(const uint16_t* g) { return *reinterpret_cast<const u32x4_t*>(g); }

// Copy offsets (bytes) of a [64][128] tile in the swizzled layout: wave w fills 1 KB pieces
// w, w+4, w+8, w+12; lane byte 16·(64·piece + lane) holds row (64·piece + lane)/16 and
// logical chunk (lane & 15) ^ sw(row).
struct TileCopy {
  int32_t off[4];
  int row[4];
  __device__ __forceinline__ void init(int64_t ld, int w, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = (w + 4 * i) * 64 + lane, r = pos >> 4, c16 = pos & 15;
      row[i] = r;
      off[i] = int32_t((int64_t(r) * ld + ((c16 ^ sw(r)) << 3)) * 2);
    }
  }
  // Rows at or beyond `valid` load zeros.
  __device__ __forceinline__ void issue(const uint16_t* src, uint16_t* tile, int valid, int w) const {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16(rs, tile + (w + 4 * i) * 512, row[i] < valid ? off[i] : kOOB);
  }
};

// Transposed fragment for the A operand of an MFMA whose k runs over the tile's rows: the
// lane's column d = 32·db + lane%32 at rows 16t + 4·(lane/32) + (0..3) and the same + 8.
__device__ __forceinline__ void read_tr_frag(u32x4_t& f, const uint16_t* tile, int t, int db, int lane) {
  const int g = lane >> 4, i16 = lane & 15, h = lane >> 5;
  const int r = 16 * t + 4 * h + (i16 >> 2);
  const int d = db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
  u32x2_t lo, hi;
  lds_read_tr16_b64(lo, tile + t_off(r, d >> 3) + (d & 7));
  lds_read_tr16_b64(hi, tile + t_off(r + 8, d >> 3) + (d & 7));
  f = u32x4_t{lo.x, lo.y, hi.x, hi.y};
}

__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// An accumulation-register operand anywhere in a kernel makes the compiler give its MFMAs
// their accumulators in AGPRs, which leaves the VGPRs to the operands and the softmax.
__device__ __forceinline__ void agpr_accumulators() {
  float z = 0.f;
  asm volatile("" ::"a"(z));
}

// x as three bf16 parts whose fp32 sum is x exactly (each part takes the next 8 bits).
__device__ __forceinline__ void split3(float x, uint32_t& a, uint32_t& b, uint32_t& c) {
  a = f32_to_bf16_bits(x);
  const float r = x - bf16_to_f32(uint16_t(a));
  b = f32_to_bf16_bits(r);
  c = f32_to_bf16_bits(r - bf16_to_f32(uint16_t(b)));
}
__device__ __forceinline__ void tie(u32x4_t& v) { asm volatile("" : "+v"(v)); }

// Scores j = 2tt, 2tt+1 of a 32-row block (16 values) as the 8 bf16 B-operand values of
// 16-row step tt: rows 4h + (0..3) and 8 + 4h + (0..3) of the step.
__device__ __forceinline__ u32x4_t pack_step(const f32x16_t& v, int tt) {
  return u32x4_t{pack_bf16x2(v[8 * tt + 0], v[8 * tt + 1]), pack_bf16x2(v[8 * tt + 2], v[8 * tt + 3]),
                 pack_bf16x2(v[8 * tt + 4], v[8 * tt + 5]), pack_bf16x2(v[8 * tt + 6], v[8 * tt + 7])};
}

// Δ and LSE·log2 e per (token, head): 16 threads per pair, 8 d each, a fixed xor tree; and
// the pair's stats entry (L_hi, L_mid, L_lo, Δ_hi, Δ_mid, Δ_lo, 0, 0) in bf16, L = LSE/scale.
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(BwdParams p) {
  const int64_t item = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int j = threadIdx.x & 15;
  const bool ok = item < p.T * p.heads;
  const int64_t tok = ok ? item / p.heads : 0;
  const int head = ok ? int(item % p.heads) : 0;
  float acc = 0.f;
  if (ok) {
    const u32x4_t a = ld_frag(p.o + tok * p.ld_o + head * kD + 8 * j);
    const u32x4_t b = ld_frag(p.dout + tok * p.ld_o + head * kD + 8 * j);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(bf16_lo(aw[e]), bf16_lo(bw[e]), acc);
      acc = fmaf(bf16_hi(aw[e]), bf16_hi(bw[e]), acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 8);
  if (ok && j == 0) {
    const float lse = p.lse[tok * p.ld_lse + head];
    p.stats[head * p.T + tok] = lse * kLog2e;
    p.stats[(int64_t(p.heads) + head) * p.T + tok] = acc;
    uint32_t l0, l1, l2, d0, d1, d2;
    split3(lse / p.scale, l0, l1, l2);
    split3(acc, d0, d1, d2);
    *reinterpret_cast<u32x4_t*>(p.stx + (int64_t(head) * p.T + tok) * 8) =
        u32x4_t{l0 | (l1 << 16), l2 | (d0 << 16), d1 | (d2 << 16), 0u};
  }
}

// dK and dV of 128 keys of one (sequence, head).
//
// Each wave owns 32 keys; per 32-query half of a block it computes S − L and dP − Δ (the
// row terms enter as one more MFMA k-step: the query's stats entry times a constant −1
// column), P = 2^(c·(S − L)) and dS = P·(dP − Δ), then dVᵀ += dOᵀ·P and dKᵀ += Qᵀ·dS.
// The first two query blocks hold each wave's diagonal half (masked) and the halves that
// precede its keys (skipped); after them every half is whole, so the main loop has no
// branches and no masks. Query rows past the sequence are copied as zeros (Q, dO and the
// stats entry), which makes their contributions zero without a mask.
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint16_t sQ[2][kBlk * kD];
  __shared__ __attribute__((aligned(1024))) uint16_t sO[2][kBlk * kD];
  __shared__ __attribute__((aligned(1024))) uint16_t sX[2][kBlk * 8];  // stats entries of the block's queries
  agpr_accumulators();

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;

  // Longest work first (key block 0 sees every query block): with one workgroup per CU, a
  // CU that finishes a long block early picks up the next longest, which balances the CUs.
  const int nkb = (p.seq + kWG - 1) / kWG, nqb = (p.seq + kBlk - 1) / kBlk;
  const int hb = p.heads * p.batch;
  const int srt = blockIdx.x;
  const int kb = srt / hb;
  const int head = (srt % hb) % p.heads;
  const int b = (srt % hb) / p.heads;
  (void)nkb;

  const int64_t row0 = int64_t(b) * p.seq;
  const uint16_t* Qg = p.qkv + head * kD;
  const uint16_t* Kg = p.qkv + p.hd + head * kD;
  const uint16_t* Vg = p.qkv + 2 * p.hd + head * kD;
  const uint16_t* dOg = p.dout + head * kD;
  const uint16_t* Xg = p.stx + (int64_t(head) * p.T + row0) * 8;

  const int k0 = kb * kWG;
  const int kw = k0 + w * 32;   // this wave's first key
  const int key = kw + l32;     // this lane's key

  // K and V of the lane's key as B operands (d = 16s + 8h .. +7).
  u32x4_t kf[8], vf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    kf[s] = key < p.seq ? ld_frag(Kg + (row0 + key) * p.ld_qkv + s * 16 + h * 8) : u32x4_t{0u, 0u, 0u, 0u};
    vf[s] = key < p.seq ? ld_frag(Vg + (row0 + key) * p.ld_qkv + s * 16 + h * 8) : u32x4_t{0u, 0u, 0u, 0u};
  }
  // B operands of the stats step: −1 at k = 0..2 (L) or k = 3..5 (Δ) for lanes 0–31; the
  // lanes 32–63 hold k = 8..15, which are zero.
  const u32x4_t ys = h == 0 ? u32x4_t{0xBF80BF80u, 0x0000BF80u, 0u, 0u} : u32x4_t{0u, 0u, 0u, 0u};
  const u32x4_t yd = h == 0 ? u32x4_t{0u, 0xBF800000u, 0xBF80BF80u, 0u} : u32x4_t{0u, 0u, 0u, 0u};
  f32x16_t dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[i][r] = dv[i][r] = 0.f;

  TileCopy cq, co;
  cq.init(p.ld_qkv, w, lane);
  co.init(p.ld_o, w, lane);
  const int qb0 = k0 / kBlk;  // first query block that reaches these keys
  auto issue = [&](int qb, int st) {
    const int q0 = qb * kBlk;
    cq.issue(Qg + (row0 + q0) * p.ld_qkv, sQ[st], p.seq - q0, w);
    co.issue(dOg + (row0 + q0) * p.ld_o, sO[st], p.seq - q0, w);
    if (w == 0) dma16(make_rsrc(Xg + int64_t(q0) * 8), sX[st], lane < p.seq - q0 ? 16 * lane : kOOB);
  };

  const float c = p.scale_log2;
  // One 32-query half of stage st. diag: the half whose first query is this wave's first
  // key; query 8j + 4h + r of the half sees the lane's key iff l32 ≤ 8j + 4h + r.
  auto half = [&](int st, int nb, bool diag) {
    u32x4_t sx, qr[8], dr[8];
    lds_read_b128(sx, &sX[st][(nb * 32 + l32) * 8]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      lds_read_b128(qr[s], &sQ[st][t_off(nb * 32 + l32, 2 * s + h)]);
      lds_read_b128(dr[s], &sO[st][t_off(nb * 32 + l32, 2 * s + h)]);
    }
    const f32x16_t zero = {};
    lgkm_wait_tied1(8, sx);
    f32x16_t sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, sx),
                                                           __builtin_bit_cast(bf16x8_t, ys), zero, 0, 0, 0);
    f32x16_t pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, sx),
                                                           __builtin_bit_cast(bf16x8_t, yd), zero, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      // Issued so far: sx, then the pairs 0..min(s, 4) + 3; pair s is 2s+1, 2s+2.
      lgkm_wait_tied(6 + 2 * (s < 4 ? s : 4) - 2 * s, qr[s], dr[s]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, qr[s]),
                                                    __builtin_bit_cast(bf16x8_t, kf[s]), sacc, 0, 0, 0);
      pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, dr[s]),
                                                    __builtin_bit_cast(bf16x8_t, vf[s]), pacc, 0, 0, 0);
      if (s + 4 < 8) {
        lds_read_b128(qr[s + 4], &sQ[st][t_off(nb * 32 + l32, 2 * (s + 4) + h)]);
        lds_read_b128(dr[s + 4], &sO[st][t_off(nb * 32 + l32, 2 * (s + 4) + h)]);
      }
    }
    // Transposed dO and Q for the half's two 16-query steps (4 reads per (tt, db)).
    u32x4_t dot[2][4], qt[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        read_tr_frag(dot[tt][db], sO[st], 2 * nb + tt, db, lane);
        read_tr_frag(qt[tt][db], sQ[st], 2 * nb + tt, db, lane);
      }
    f32x16_t pm, ds;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float pe = __builtin_amdgcn_exp2f(sacc[e] * c);
      if (diag) pe = l32 <= 8 * (e >> 2) + 4 * h + (e & 3) ? pe : 0.f;
      pm[e] = pe;
      ds[e] = pe * pacc[e];
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const u32x4_t pf = pack_step(pm, tt), sf = pack_step(ds, tt);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int i = 4 * tt + db;
        lgkm_wait_tied(28 - 4 * i < 15 ? 28 - 4 * i : 15, dot[tt][db], qt[tt][db]);
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, dot[tt][db]),
                                                        __builtin_bit_cast(bf16x8_t, pf), dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, qt[tt][db]),
                                                        __builtin_bit_cast(bf16x8_t, sf), dk[db], 0, 0, 0);
      }
    }
  };

  // The first two blocks: half i (= 2·block + nb) is wave i's diagonal, earlier ones are
  // skipped by it.
  issue(qb0, 0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int qb = qb0 + i;
    if (qb >= nqb) break;
    wait_vm_barrier<0>();
    if (qb + 1 < nqb) issue(qb + 1, (i + 1) & 1);
    if (kw < p.seq) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int hx = 2 * i + nb;
        if (hx == w) half(i, nb, true);
        else if (hx > w) half(i, nb, false);
      }
    }
  }
  for (int qb = qb0 + 2; qb < nqb; ++qb) {
    const int st = (qb - qb0) & 1;
    wait_vm_barrier<0>();
    if (qb + 1 < nqb) issue(qb + 1, st ^ 1);
    half(st, 0, false);
    half(st, 1, false);
  }
  // No LDS write may land after the workgroup ends.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // The lane holds d = 32·db + 8j + 4h + (0..3) of its key.
  if (key < p.seq) {
    uint16_t* dK = p.dqkv + (row0 + key) * p.ld_dqkv + p.hd + head * kD;
    uint16_t* dV = dK + p.hd;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = db * 32 + 8 * j + 4 * h;
        *reinterpret_cast<u32x2_t*>(dK + d) =
            u32x2_t{pack_bf16x2(dk[db][4 * j] * p.scale, dk[db][4 * j + 1] * p.scale),
                    pack_bf16x2(dk[db][4 * j + 2] * p.scale, dk[db][4 * j + 3] * p.scale)};
        *reinterpret_cast<u32x2_t*>(dV + d) =
            u32x2_t{pack_bf16x2(dv[db][4 * j], dv[db][4 * j + 1]), pack_bf16x2(dv[db][4 * j + 2], dv[db][4 * j + 3])};
      }
  }
}

// dQ of 128 queries of one (sequence, head).
//
// Each wave owns 32 queries (Q, dO fragments, LSE and Δ in registers); blocks of 64 keys
// stream through LDS. Per block: S and dP for the two 32-key halves with one query per lane
// (K and V fragments read four k-steps ahead), dS = P·(dP − Δ), then dQᵀ += Kᵀ·dSᵀ with K
// read transposed. Key blocks that end before the workgroup's first query are whole for
// every wave (main loop, no mask); the last two blocks hold the diagonals and are peeled.
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) uint16_t sK[2][kBlk * kD];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[2][kBlk * kD];
  agpr_accumulators();

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;

  // Longest work first (the last query block sees every key block), as for dK/dV.
  const int nqb = (p.seq + kWG - 1) / kWG;
  const int hb = p.heads * p.batch;
  const int srt = blockIdx.x;
  const int qb = nqb - 1 - srt / hb;
  const int head = (srt % hb) % p.heads;
  const int b = (srt % hb) / p.heads;

  const int64_t row0 = int64_t(b) * p.seq;
  const uint16_t* Qg = p.qkv + head * kD;
  const uint16_t* Kg = p.qkv + p.hd + head * kD;
  const uint16_t* Vg = p.qkv + 2 * p.hd + head * kD;
  const uint16_t* dOg = p.dout + head * kD;

  const int q0 = qb * kWG;
  const int qw = q0 + w * 32;   // this wave's first query
  const int q = qw + l32;       // this lane's query

  // Q and dO of the lane's query as B operands (d = 16s + 8h .. +7), its LSE·log2 e and Δ.
  u32x4_t qf[8], df[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qf[s] = q < p.seq ? ld_frag(Qg + (row0 + q) * p.ld_qkv + s * 16 + h * 8) : u32x4_t{0u, 0u, 0u, 0u};
    df[s] = q < p.seq ? ld_frag(dOg + (row0 + q) * p.ld_o + s * 16 + h * 8) : u32x4_t{0u, 0u, 0u, 0u};
  }
  const float l2 = q < p.seq ? p.stats[head * p.T + row0 + q] : 0.f;
  const float dl = q < p.seq ? p.stats[(int64_t(p.heads) + head) * p.T + row0 + q] : 0.f;

  f32x16_t dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[i][r] = 0.f;

  TileCopy ck;
  ck.init(p.ld_qkv, w, lane);
  const int q_hi = min(q0 + kWG, p.seq);
  const int nkb = (q_hi + kBlk - 1) / kBlk;  // key blocks these queries see
  auto issue = [&](int kb, int st) {
    const int k0 = kb * kBlk;
    ck.issue(Kg + (row0 + k0) * p.ld_qkv, sK[st], p.seq - k0, w);
    ck.issue(Vg + (row0 + k0) * p.ld_qkv, sV[st], p.seq - k0, w);
  };

  const float c = p.scale_log2;
  // One block of 64 keys from stage st. lim: the lane's query sees key k0 + 4h + off
  // (off = 32nb + 8j + r) iff off ≤ lim; masked only on the blocks that reach the diagonal.
  auto block = [&](int st, bool masked, int lim) {
    // Pin the dQ accumulators to AGPRs across blocks (else the allocator moves them through
    // VGPRs at every loop boundary).
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+a"(dq[i]));
    // K and V fragments in the order (s, nb), four pairs ahead; pair i = 2s + nb.
    u32x4_t kr[16], vr[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lds_read_b128(kr[i], &sK[st][t_off((i & 1) * 32 + l32, 2 * (i >> 1) + h)]);
      lds_read_b128(vr[i], &sV[st][t_off((i & 1) * 32 + l32, 2 * (i >> 1) + h)]);
    }
    const f32x16_t zero = {};
    f32x16_t sacc[2] = {zero, zero}, pacc[2] = {zero, zero};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int s = i >> 1, nb = i & 1;
      // Issued so far: pairs 0 .. min(i, 12) + 3; pair i is reads 2i, 2i + 1.
      lgkm_wait_tied(2 * ((i < 12 ? i : 12) + 4) - 2 * i - 2, kr[i], vr[i]);
      sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kr[i]),
                                                        __builtin_bit_cast(bf16x8_t, qf[s]), sacc[nb], 0, 0, 0);
      pacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vr[i]),
                                                        __builtin_bit_cast(bf16x8_t, df[s]), pacc[nb], 0, 0, 0);
      if (i + 4 < 16) {
        const int j = i + 4;
        lds_read_b128(kr[j], &sK[st][t_off((j & 1) * 32 + l32, 2 * (j >> 1) + h)]);
        lds_read_b128(vr[j], &sV[st][t_off((j & 1) * 32 + l32, 2 * (j >> 1) + h)]);
      }
    }
    // dS, packed to the bf16 B operands of the four 16-key steps.
    u32x4_t sf[4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      f32x16_t ds;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int off = nb * 32 + 8 * (e >> 2) + (e & 3);
        float pe = __builtin_amdgcn_exp2f(fmaf(sacc[nb][e], c, -l2));
        if (masked) pe = off <= lim ? pe : 0.f;
        ds[e] = pe * (pacc[nb][e] - dl);
      }
      sf[2 * nb] = pack_step(ds, 0);
      sf[2 * nb + 1] = pack_step(ds, 1);
    }
    // dQᵀ += Kᵀ·dSᵀ: K read transposed, one 16-key step ahead (8 reads per step).
    u32x4_t kt[2][4];
#pragma unroll
    for (int db = 0; db < 4; ++db) read_tr_frag(kt[0][db], sK[st], 0, db, lane);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t + 1 < 4) {
#pragma unroll
        for (int db = 0; db < 4; ++db) read_tr_frag(kt[(t + 1) & 1][db], sK[st], t + 1, db, lane);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        lgkm_wait_tied1((t + 1 < 4 ? 8 : 0) + 2 * (3 - db), kt[t & 1][db]);
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kt[t & 1][db]),
                                                        __builtin_bit_cast(bf16x8_t, sf[t]), dq[db], 0, 0, 0);
      }
    }
  };

  // Blocks before the workgroup's first query: whole for every wave.
  const int kfull = min(q0 / kBlk, nkb);
  issue(0, 0);
  for (int kb = 0; kb < kfull; ++kb) {
    const int st = kb & 1;
    wait_vm_barrier<0>();
    if (kb + 1 < nkb) issue(kb + 1, st ^ 1);
    block(st, false, 0);
  }
  // The last (at most two) blocks: each wave's diagonal, masked; blocks wholly after a
  // wave's queries are skipped by it.
  for (int kb = kfull; kb < nkb; ++kb) {
    const int st = kb & 1;
    wait_vm_barrier<0>();
    if (kb + 1 < nkb) issue(kb + 1, st ^ 1);
    const int k0 = kb * kBlk;
    if (k0 <= qw + 31 && qw < p.seq) block(st, true, min(q, p.seq - 1) - k0 - 4 * h);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // The lane holds d = 32·db + 8j + 4h + (0..3) of its query.
  if (q < p.seq) {
    uint16_t* dst = p.dqkv + (row0 + q) * p.ld_dqkv + head * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x2_t*>(dst + db * 32 + 8 * j + 4 * h) =
            u32x2_t{pack_bf16x2(dq[db][4 * j] * p.scale, dq[db][4 * j + 1] * p.scale),
                    pack_bf16x2(dq[db][4 * j + 2] * p.scale, dq[db][4 * j + 3] * p.scale)};
  }
}

}  // namespace

// Stats entries first (16 bytes per (token, head), so they stay 16-byte aligned), then the
// two fp32 arrays.
int64_t attn_bwd_stats_floats(int64_t tokens, int64_t heads) { return 6 * heads * tokens; }

namespace {
BwdParams bwd_params(const AttnBwdArgs& a) {
  BwdParams p{};
  p.qkv = static_cast<const uint16_t*>(a.qkv);
  p.ld_qkv = a.ld_qkv;
  p.o = static_cast<const uint16_t*>(a.o);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.ld_o = a.ld_o;
  p.lse = a.lse;
  p.ld_lse = a.ld_lse;
  p.dqkv = static_cast<uint16_t*>(a.dqkv);
  p.ld_dqkv = a.ld_dqkv;
  p.T = a.batch * a.seq;
  p.stx = reinterpret_cast<uint16_t*>(a.stats);
  p.stats = a.stats + 4 * p.T * a.heads;
  p.hd = a.heads * a.head_dim;
  p.seq = int(a.seq);
  p.heads = int(a.heads);
  p.batch = int(a.batch);
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  return p;
}
}  // namespace

hipError_t launch_attention_bwd_prep(const AttnBwdArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.seq == 0 || a.heads == 0) return hipSuccess;
  const BwdParams p = bwd_params(a);
  note_kernel("attn_bwd_prep_kernel");
  DOMINO_LAUNCH(attn_bwd_prep_kernel, dim3(unsigned((p.T * p.heads + 15) / 16)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attention_bwd_dkdv(const AttnBwdArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.seq == 0 || a.heads == 0) return hipSuccess;
  const BwdParams p = bwd_params(a);
  const int nkb = int((a.seq + kWG - 1) / kWG);
  note_kernel("attn_bwd_dkdv_kernel");
  DOMINO_LAUNCH(attn_bwd_dkdv_kernel, dim3(nkb * p.heads * p.batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attention_bwd_dq(const AttnBwdArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.seq == 0 || a.heads == 0) return hipSuccess;
  const BwdParams p = bwd_params(a);
  const int nqb = int((a.seq + kWG - 1) / kWG);
  note_kernel("attn_bwd_dq_kernel");
  DOMINO_LAUNCH(attn_bwd_dq_kernel, dim3(nqb * p.heads * p.batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace domino
