// Fused causal self-attention forward for one rank's head slice (bf16, head_dim 128).
// For attention the TP layer X·A·B = Y has A = multi-head attention on the rank's heads
// (page "DeepSpeed-Domino 深度解析", section "TP 的数据依赖：通信为何难以隐藏"); only causal
// self-attention is supported (section "如何尝试 DeepSpeed-Domino").
//
// O[q] = Σ_{k ≤ q} softmax_k(Q[q]·K[k]·scale)·V[k] per (sequence, head), computed block by
// block with a running maximum and running sum (online softmax), so the seq×seq score
// matrix never leaves registers.
//
// Design (gfx950): one workgroup = 4 waves = 128 query rows of one (sequence, head); each
// wave owns 32 query rows. Keys advance 64 at a time; K and V blocks reach LDS through
// buffer loads that write LDS directly, two stages deep, one barrier per block.
//  * S = Q·Kᵀ on 32×32×16 MFMAs with the operands swapped, so lane l holds the scores of
//    query l%32 for keys 8j + 4·(l/32) + r (j, r = 0..3) of each 32-key block: a query's
//    row lives in two lanes (l, l^32), and its running max and sum need one cross-lane
//    exchange each.
//  * The exponentiated scores of a 16-key step are then already the A operand of O += P·V
//    (keys 4·(l/32) + r and 8 + 4·(l/32) + r of the step, in that k order); the V operand
//    reads the same keys, transposed out of LDS with ds_read_b64_tr_b16, so P never leaves
//    registers.
//  * Q stays in registers (read once). K is staged [key][d] with a 16-byte-chunk XOR
//    swizzle (a fragment read, 16 keys × one chunk, hits distinct banks); V is staged
//    [key][d] with a 32-byte-chunk swizzle for the transposed reads.
//  * Causal balance: the first half of the grid takes query blocks longest first, the
//    second half shortest first, so the two workgroups a CU holds at once carry the same
//    total work.
#include "common.hpp"
#include "kernels.hpp"

namespace domino {
namespace {

constexpr int kD = 128;   // head_dim
constexpr int kQB = 128;  // query rows per workgroup
constexpr int kKB = 64;   // keys per block

// K tile [64 keys][128 d]: 16-byte chunk c of key k at c ^ (k & 15).
__device__ __forceinline__ int k_off(int key, int chunk) { return key * kD + ((chunk ^ (key & 15)) << 3); }
// V tile [64 keys][128 d]: 32-byte chunk c of key k at c ^ 2·(k & 3).
__device__ __forceinline__ int v_off(int key, int d) { return key * kD + (((d >> 4) ^ ((key & 3) << 1)) << 4) + (d & 15); }

struct AttnParams {
  const uint16_t* qkv; int64_t ld_qkv;
  uint16_t* o; int64_t ld_o;
  float* lse; int64_t ld_lse;  // optional [T, heads]: natural log of each row's softmax sum
  int seq, heads, batch, nqb;
  int64_t hd;          // heads · head_dim (width of each of the Q, K, V blocks)
  float scale_log2;    // scale · log2(e)
};

__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint16_t sK[2][kKB * kD];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[2][kKB * kD];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;

  // Grid order: positions 0 .. G/2−1 longest query block first, the rest shortest first.
  const int hb = p.heads * p.batch, G = p.nqb * hb, half = (G + 1) / 2;
  const int lin = blockIdx.x;
  const int srt = lin < half ? lin : G - 1 - (lin - half);
  const int qb = p.nqb - 1 - srt / hb;
  const int head = (srt % hb) % p.heads;
  const int b = (srt % hb) / p.heads;

  const int64_t row0 = int64_t(b) * p.seq;  // first token of this sequence
  const uint16_t* Qg = p.qkv + head * kD;
  const uint16_t* Kg = p.qkv + p.hd + head * kD;
  const uint16_t* Vg = p.qkv + 2 * p.hd + head * kD;

  const int q0 = qb * kQB;
  const int qw = q0 + w * 32;     // this wave's first query
  const int q = qw + l32;         // this lane's query

  // Q fragments (A operand of S): d = 16s + 8h .. +7 of query q.
  u32x4_t qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = q < p.seq ? *reinterpret_cast<const u32x4_t*>(Qg + (row0 + q) * p.ld_qkv + s * 16 + h * 8)
                      : u32x4_t{0u, 0u, 0u, 0u};

  f32x16_t oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mrun = -1e30f, lrun = 0.f;

  const int q_hi = min(q0 + kQB, p.seq);   // exclusive
  const int nkb = (q_hi + kKB - 1) / kKB;  // key blocks this workgroup needs

  // Copies of one key block: wave w fills 1 KB pieces w, w+4, w+8, w+12 of each tile.
  // Piece byte offset 16·(64·piece + lane) holds key (64·piece + lane)/16 and, for K,
  // 16-byte chunk (lane & 15) ^ (key & 15); for V, 32-byte chunk ((lane & 15) >> 1) ^ 2·(key & 3).
  int32_t koff[4], voff[4];
  int kkey[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pos = (w + 4 * i) * 64 + lane, key = pos >> 4, c16 = pos & 15;
    kkey[i] = key;
    koff[i] = int32_t((int64_t(key) * p.ld_qkv + ((c16 ^ (key & 15)) << 3)) * 2);
    const int c32 = (c16 >> 1) ^ ((key & 3) << 1);
    voff[i] = int32_t((int64_t(key) * p.ld_qkv + (c32 << 4) + ((c16 & 1) << 3)) * 2);
  }
  auto issue = [&](int kb, int st) {
    const int key0 = kb * kKB;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (row0 + key0) * p.ld_qkv);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (row0 + key0) * p.ld_qkv);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = key0 + kkey[i] < p.seq;
      dma16(rk, &sK[st][(w + 4 * i) * 512], in ? koff[i] : kOOB);
      dma16(rv, &sV[st][(w + 4 * i) * 512], in ? voff[i] : kOOB);
    }
  };

  issue(0, 0);
  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb & 1;
    // Block kb has landed (the only copies in flight) and every wave is done with kb−1,
    // whose stage the next copies overwrite.
    wait_vm_barrier<0>();
    if (kb + 1 < nkb) issue(kb + 1, st ^ 1);

    const int key0 = kb * kKB;
    if (key0 > qw + 31 || qw >= p.seq) continue;  // every key of this block is in this wave's future

    // S = Q·Kᵀ for 32 queries × 64 keys (two 32-key blocks).
    f32x16_t sacc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[nb][r] = 0.f;
    // LDS reads are inline assembly with explicit waits: through the builtins the
    // compiler makes them wait for every global→LDS copy in flight (it cannot tell which
    // LDS they write), which would serialise the next block's copies with this block.
    // All K fragments are read before the first MFMA; the MFMAs of sub-step s wait only
    // for the reads of fragments s (LDS reads complete in order).
    u32x4_t kf[8][2];
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) lds_read_b128(kf[s][nb], &sK[st][k_off(nb * 32 + l32, 2 * s + h)]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      lgkm_wait_tied(14 - 2 * s, kf[s][0], kf[s][1]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[s][nb]),
                                                          __builtin_bit_cast(bf16x8_t, qf[s]), sacc[nb], 0, 0, 0);
    }

    // The V fragments do not depend on the softmax: read them now, behind it. Lane keys
    // of step t: 16t + 4h + (0..3) and 16t + 8 + 4h + (0..3); the transposed read gives
    // lane i of each 16-lane group column n0 + i of 4 rows.
    u32x4_t vf[4][4];
    {
      const int g = lane >> 4, i16 = lane & 15;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int krow = 16 * t + 4 * h + (i16 >> 2);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int d = db * 32 + 16 * (g & 1) + 4 * (i16 & 3);
          u32x2_t lo, hi;
          lds_read_tr16_b64(lo, &sV[st][v_off(krow, d)]);
          lds_read_tr16_b64(hi, &sV[st][v_off(krow + 8, d)]);
          vf[t][db] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        }
      }
    }

    // Online softmax over this block in the log2 domain, with scores scaled inside the
    // exponent (c = scale·log2 e > 0, so max(c·s) = c·max(s)). Key key0 + 4h + off
    // (off = 32·nb + 8j + r) is visible iff off ≤ lim; only blocks that reach the wave's
    // diagonal (or the sequence end) are masked.
    float mx = -1e30f;
    if (key0 + kKB - 1 > qw || key0 + kKB > p.seq) {  // wave-uniform
      const int lim = min(q, p.seq - 1) - key0 - 4 * h;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int off = nb * 32 + 8 * (e >> 2) + (e & 3);
          sacc[nb][e] = off <= lim ? sacc[nb][e] : -INFINITY;
        }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[nb][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float c = p.scale_log2;
    const float mnew = fmaxf(mrun, mx * c);
    float rs = 0.f;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[nb][e], c, -mnew));
        sacc[nb][e] = pe;
        rs += pe;
      }
    rs += __shfl_xor(rs, 32);
    // Rescale O and l only when some row's maximum grew (after the first blocks it
    // rarely does).
    if (__ballot(mnew > mrun)) {
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      lrun *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
    }
    lrun += rs;
    mrun = mnew;

    // O += P·V over the block's 64 keys: four 16-key steps; step t = 2·nb + tt uses the
    // scores j = 2tt, 2tt+1 of 32-key block nb. The V reads have landed behind the softmax.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int db = 0; db < 4; ++db) asm volatile("" : "+v"(vf[t][db]));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int nb = t >> 1, tt = t & 1;
      const u32x4_t pf = {pack_bf16x2(sacc[nb][8 * tt + 0], sacc[nb][8 * tt + 1]),
                          pack_bf16x2(sacc[nb][8 * tt + 2], sacc[nb][8 * tt + 3]),
                          pack_bf16x2(sacc[nb][8 * tt + 4], sacc[nb][8 * tt + 5]),
                          pack_bf16x2(sacc[nb][8 * tt + 6], sacc[nb][8 * tt + 7])};
#pragma unroll
      for (int db = 0; db < 4; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[t][db]),
                                                          __builtin_bit_cast(bf16x8_t, pf), oacc[db], 0, 0, 0);
    }
  }
  // No LDS write may land after the workgroup ends.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // O[q][d .. d+3] = O / l; lane holds d = 32·db + 8j + 4h + (0..3).
  if (q < p.seq) {
    // ln Σ_k exp(scale·s_k) = (m + log2 l)·ln 2 with m, l the running max and sum (log2 units).
    if (p.lse && h == 0) p.lse[(row0 + q) * p.ld_lse + head] = (mrun + log2f(lrun)) * 0.69314718055994531f;
    const float inv = 1.0f / lrun;
    uint16_t* dst = p.o + (row0 + q) * p.ld_o + head * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4_t v = {oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv, oacc[db][4 * j + 2] * inv,
                           oacc[db][4 * j + 3] * inv};
        *reinterpret_cast<u32x2_t*>(dst + db * 32 + 8 * j + 4 * h) = u32x2_t{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
      }
  }
}

}  // namespace

hipError_t launch_attention_fwd(const AttnArgs& a, hipStream_t s) {
  if (a.batch == 0 || a.seq == 0 || a.heads == 0) return hipSuccess;
  AttnParams p{};
  p.qkv = static_cast<const uint16_t*>(a.qkv);
  p.ld_qkv = a.ld_qkv;
  p.o = static_cast<uint16_t*>(a.o);
  p.ld_o = a.ld_o;
  p.lse = a.lse;
  p.ld_lse = a.ld_lse;
  p.seq = int(a.seq);
  p.heads = int(a.heads);
  p.batch = int(a.batch);
  p.nqb = int((a.seq + kQB - 1) / kQB);
  p.hd = a.heads * a.head_dim;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  const int blocks = p.nqb * p.heads * p.batch;
  note_kernel("attn_fwd_kernel");
  DOMINO_LAUNCH(attn_fwd_kernel, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace domino
