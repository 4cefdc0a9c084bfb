// Fused causal self-attention forward for one rank's head slice (bf16, head_dim 128).
// For attention the TP layer X·A·B = Y has A = multi-head attention on the rank's heads
// (page "DeepSpeed-Domino 深度解析", section "TP 的数据依赖：通信为何难以隐藏"); only causal
// self-attention is supported (section "如何尝试 DeepSpeed-Domino").
//
// O[q] = Σ_{k ≤ q} softmax_k(Q[q]·K[k]·scale)·V[k] per (sequence, head), computed block by
// block with a running maximum and running sum (online softmax), so the seq×seq score
// matrix never leaves registers.
//
// Design (gfx950): one workgroup = 8 waves = 128 query rows of one (sequence, head),
// computed twice over: wave group 0 (waves 0-3) takes the even 64-key blocks, group 1
// (waves 4-7) the odd ones, and each wave of a group owns 32 query rows. The two partial
// results (O, running max, running sum) are merged at the end, through LDS. Splitting
// the keys rather than the queries gives both groups the same number of blocks, so they
// stay paired to the end.
//  * Ping-pong: time step t is key block t. The group that owns block t runs its MFMAs
//    (S_t = Q·K_tᵀ, and O += P·V of its previous block t − 2) while the other group runs
//    the online softmax of its block t − 1 (VALU and transcendental work) and issues the
//    copies of later blocks; a workgroup barrier ends each step. Waves w and w + 4 share a
//    SIMD, so each SIMD always pairs one wave's MFMAs with the other wave's softmax.
//  * K blocks sit in a ring of 4 stages and V blocks in a ring of 5 (144 KB): at the start
//    of step t the softmax group copies K_{t+3} and V_{t+2} over K_{t−1} and V_{t−3} (which
//    it read in its previous step) and waits for them at the end of its next softmax step,
//    three steps ahead of their first reads. Copies issued between the MFMAs measured
//    slower: they stall the MFMA group more than the softmax group.
//  * S = Q·Kᵀ on 32×32×16 MFMAs with the operands swapped, so lane l holds the scores of
//    query l%32 for keys 8j + 4·(l/32) + r (j, r = 0..3) of each 32-key block: a query's
//    row lives in two lanes (l, l^32), and its running max and sum need one cross-lane
//    exchange each (v_permlane32_swap).
//  * The exponentiated scores of a 16-key step are then already the A operand of O += P·V
//    (keys 4·(l/32) + r and 8 + 4·(l/32) + r of the step, in that k order); the V operand
//    reads the same keys, transposed out of LDS with ds_read_b64_tr_b16, so P never goes
//    through LDS.
//  * Q stays in registers (read once). K is staged [key][d] with a 16-byte-chunk XOR
//    swizzle (a fragment read, 16 keys × one chunk, hits distinct banks); V is staged
//    [key][d] with a 32-byte-chunk swizzle for the transposed reads.
//  * Causal balance: a workgroup (one per CU) takes the k-th longest and then the k-th
//    shortest query block of one (sequence, head), so all carry about the same work and
//    no CU waits between two workgroups.
//  * The running maximum moves only when a block's exceeds it by more than 2^8, so O and
//    l are rescaled rarely; fragment addresses are one XOR of a per-lane base with the
//    fragment's index, the rest instruction immediates.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace domino {
namespace {

constexpr int kD = 128;   // head_dim
constexpr int kQB = 128;  // query rows per workgroup
constexpr int kKB = 64;   // keys per block
constexpr int kTile = kKB * kD;          // elements of one K or V block (16 KB)
constexpr int kKRing = 4, kVRing = 5;    // stages of the K and V rings


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

// The value of lane l ^ 32 combined with lane l's: both halves of the wave get op(x[l], x[l ^ 32]).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__global__ __launch_bounds__(512, 1) void attn_fwd_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint16_t smem[(kKRing + kVRing) * kTile];
  uint16_t* const sK = smem;
  uint16_t* const sV = smem + kKRing * kTile;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = wave >> 2, w = wave & 3;
  const int h = lane >> 5, l32 = lane & 31;

  // Two query blocks of one (sequence, head) per workgroup in turn, the k-th longest and
  // the k-th shortest (only the middle one when they meet), so every workgroup carries
  // about the same work and no CU waits for a second workgroup to be dispatched.
  const int hb = p.heads * p.batch;
  const int lin = blockIdx.x;
  const int kpair = lin / hb;
  const int head = (lin % hb) % p.heads;
  const int b = (lin % hb) / p.heads;

  const int64_t row0 = int64_t(b) * p.seq;  // first token of this sequence
  const uint16_t* Qg = p.qkv + head * kD;
  const uint16_t* Kg = p.qkv + p.hd + head * kD;
  const uint16_t* Vg = p.qkv + 2 * p.hd + head * kD;

  // One query block, start to finish (inlined once per block of the pair).
  auto run_block = [&](const int qb) {
  const int q0 = qb * kQB;
  const int qw = q0 + w * 32;     // this wave's first query
  const int q = qw + l32;         // this lane's query

  // Q fragments (B operand of S): d = 16s + 8h .. +7 of query q.
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

  const int q_hi = min(q0 + kQB, p.seq);    // exclusive
  const int nkb = (q_hi + kKB - 1) / kKB;   // key blocks of this query block
  // The last key block holding a key this wave's queries see (key blocks start at multiples
  // of 64 and waves at multiples of 32, so every query of the wave sees the first key of
  // each block up to this one).
  const int wlast = qw < p.seq ? min(qw + 31, p.seq - 1) / kKB : -1;

  // Copies of one key block by the four waves of a group: wave w fills 1 KB pieces w, w+4,
  // w+8, w+12 of each tile. Piece byte offset 16·(64·piece + lane) holds key
  // (64·piece + lane)/16 and, for K, 16-byte chunk (lane & 15) ^ (key & 15); for V, 32-byte
  // chunk ((lane & 15) >> 1) ^ 2·(key & 3).
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
  // Copy i (1 KB) of K or V block kb; a block past this query block's range (kb ≥ nkb)
  // loads zeros without touching memory, so every step issues the same number of copies.
  struct Copy {
    __amdgpu_buffer_rsrc_t rs;
    uint16_t* dst;
    bool in;
  };
  auto copy_k = [&](int kb) {
    return Copy{make_rsrc(Kg + (row0 + int64_t(kb) * kKB) * p.ld_qkv), sK + (kb % kKRing) * kTile, kb < nkb};
  };
  auto copy_v = [&](int kb) {
    return Copy{make_rsrc(Vg + (row0 + int64_t(kb) * kKB) * p.ld_qkv), sV + (kb % kVRing) * kTile, kb < nkb};
  };
  auto issue_k = [&](const Copy& cp, int kb, int i) {
    dma16(cp.rs, cp.dst + (w + 4 * i) * 512, cp.in && kb * kKB + kkey[i] < p.seq ? koff[i] : kOOB);
  };
  auto issue_v = [&](const Copy& cp, int kb, int i) {
    dma16(cp.rs, cp.dst + (w + 4 * i) * 512, cp.in && kb * kKB + kkey[i] < p.seq ? voff[i] : kOOB);
  };

  // LDS byte addresses of the fragment reads. A K fragment (key nb·32 + l, 16-byte chunk
  // 2s + h) sits at key·256 + 16·((2s + h) ^ (key & 15)) = kbase ^ 32s, plus 8192·nb: kbase
  // holds the lane's key row and, in bits 5-7 and 4, the swizzle's lane part. A V
  // fragment (key 16u + 8·hi + 4h + k3 with k3 = (l & 15) >> 2, 32-byte chunk
  // 2·(db ^ k3) + ((l >> 4) & 1), column 4·(l & 3) of it) sits at vbase ^ 64db, plus
  // 4096u + 2048·hi. The per-block offsets are instruction immediates.
  const int x15 = l32 & 15, k3 = x15 >> 2;
  const uint32_t kbase = lds_addr(sK) + l32 * 256 + ((x15 >> 1) << 5) + (((h ^ x15) & 1) << 4);
  const uint32_t vbase = lds_addr(sV) + (4 * h + k3) * 256 + (k3 << 6) + (((l32 >> 4) & 1) << 5) + ((x15 & 3) << 3);

  f32x16_t sacc[2];   // S of this group's current block
  u32x4_t pf[4];      // P of this group's previous block, bf16: four 16-key steps
  bool p_live = false;
  const float c = p.scale_log2;

  // Prologue: K_0 .. K_2 and V_0, V_1, each group first the K block it reads first.
  // Group 0 reads K_0 in step 0: its copies land once at most the eight later ones are in
  // flight. Everything else lands by the end of the issuing group's first softmax step
  // (all but that step's own eight copies), before anything reads it.
  {
    const int k0 = g == 0 ? 0 : 1;
    const Copy a = copy_k(k0), bk = copy_k(2), v = copy_v(k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_k(a, k0, i);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      issue_v(v, k0, i);
      if (g == 0) issue_k(bk, 2, i);
    }
  }
  if (g == 0) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  asm volatile("s_barrier" ::: "memory");

  // Step t: the group owning block t runs mma_step(t), the other softmax_step(t). Each
  // group's steps alternate, so each group's loop is written with its two kinds of step in
  // order (the compiler then sees that S and P are never live at once), and every wave
  // passes the same barriers.
  auto mma_step = [&](int t) {
    // MFMA step of block t (this group's): O += P·V of block t − 2 (P dies before S_t
    // is born, so the two never hold registers at once), then S_t.
    if (p_live) {
      const uint32_t vb = vbase + uint32_t(((t - 2) % kVRing) * kTile * 2);
      uint32_t va[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) va[db] = vb ^ uint32_t(db << 6);
      // V fragments two 16-key steps ahead (eight reads per step).
      u32x4_t vf[4][4];
      auto read_v = [&](auto uc) {
        constexpr int u = decltype(uc)::value;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          u32x2_t lo, hi;
          asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(va[db]), "n"(4096 * u));
          asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(va[db]), "n"(4096 * u + 2048));
          vf[u][db] = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        }
      };
      read_v(std::integral_constant<int, 0>{});
      read_v(std::integral_constant<int, 1>{});
      auto pv = [&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if constexpr (u < 3) asm volatile("s_waitcnt lgkmcnt(8)" ::: "memory");
        else asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int db = 0; db < 4; ++db) asm volatile("" : "+v"(vf[u][db]));
#pragma unroll
        for (int db = 0; db < 4; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vf[u][db]),
                                                            __builtin_bit_cast(bf16x8_t, pf[u]), oacc[db], 0, 0, 0);
        if constexpr (u < 2) read_v(std::integral_constant<int, u + 2>{});
      };
      pv(std::integral_constant<int, 0>{});
      pv(std::integral_constant<int, 1>{});
      pv(std::integral_constant<int, 2>{});
      pv(std::integral_constant<int, 3>{});
    }
    if (t < nkb && t <= wlast) {
      const uint32_t kb0 = kbase + uint32_t((t % kKRing) * kTile * 2);
      // K fragments four sub-steps ahead: sub-step s + 4 is read once the MFMAs of s are
      // issued, so at most four sub-steps' registers are live.
      u32x4_t kf[8][2];
      auto read_k = [&](auto sc) {
        constexpr int s = decltype(sc)::value;
        const uint32_t a = kb0 ^ uint32_t(s << 5);
        u32x4_t r0, r1;
        asm volatile("ds_read_b128 %0, %1" : "=v"(r0) : "v"(a));
        asm volatile("ds_read_b128 %0, %1 offset:8192" : "=v"(r1) : "v"(a));
        kf[s][0] = r0;
        kf[s][1] = r1;
      };
      read_k(std::integral_constant<int, 0>{});
      read_k(std::integral_constant<int, 1>{});
      read_k(std::integral_constant<int, 2>{});
      read_k(std::integral_constant<int, 3>{});
      auto qk = [&](auto sc) {
        constexpr int s = decltype(sc)::value;
        lgkm_wait_tied(s < 4 ? 6 : 14 - 2 * s, kf[s][0], kf[s][1]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          sacc[nb] = s == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[s][nb]),
                                                                     __builtin_bit_cast(bf16x8_t, qf[s]),
                                                                     f32x16_t{}, 0, 0, 0)
                            : __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[s][nb]),
                                                                     __builtin_bit_cast(bf16x8_t, qf[s]), sacc[nb],
                                                                     0, 0, 0);
        if constexpr (s < 4) read_k(std::integral_constant<int, s + 4>{});
      };
      qk(std::integral_constant<int, 0>{});
      qk(std::integral_constant<int, 1>{});
      qk(std::integral_constant<int, 2>{});
      qk(std::integral_constant<int, 3>{});
      qk(std::integral_constant<int, 4>{});
      qk(std::integral_constant<int, 5>{});
      qk(std::integral_constant<int, 6>{});
      qk(std::integral_constant<int, 7>{});
    }
  };
  auto softmax_step = [&](int t) {
    // Softmax step of block j = t − 1 (this group's). First the copies of K_{t+3} and
    // V_{t+2} (over K_{t−1} and V_{t−3}, which this group read in its previous step); this
    // group waits for them at the end of its next softmax step, before K_{t+3} is read.
    {
      const Copy ck = copy_k(t + 3), cv = copy_v(t + 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        issue_k(ck, t + 3, i);
        issue_v(cv, t + 2, i);
      }
    }
    const int j = t - 1;
    p_live = j >= 0 && j < nkb && j <= wlast;
    if (p_live) {
      // Online softmax in the log2 domain, scores scaled inside the exponent (c > 0, so
      // max(c·s) = c·max(s)). Key key0 + 4h + off (off = 32·nb + 8e' + r) is visible iff
      // off ≤ lim; only blocks that reach the wave's diagonal (or the sequence end) are
      // masked.
      const int key0 = j * kKB;
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
      float mx0 = -1e30f, mx1 = -1e30f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        mx0 = fmaxf(mx0, sacc[0][e]);
        mx1 = fmaxf(mx1, sacc[1][e]);
      }
      const float bmax = xor32_max(fmaxf(mx0, mx1)) * c;
      // The running maximum moves only when the block's exceeds it by more than 2^8 (the
      // exponentials stay ≤ 256, exact in fp32 and as precise in bf16); O and l are
      // rescaled only then. The group's first block sets it.
      const bool first = j == g;
      const float mnew = first || bmax > mrun + 8.0f ? fmaxf(mrun, bmax) : mrun;
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int nb = qq >> 1;
#pragma unroll
        for (int e = 8 * (qq & 1); e < 8 * (qq & 1) + 8; ++e) {
          const float pe = __builtin_amdgcn_exp2f(fmaf(sacc[nb][e], c, -mnew));
          sacc[nb][e] = pe;
          rs[e & 3] += pe;
        }
      }
      const float bsum = xor32_sum((rs[0] + rs[1]) + (rs[2] + rs[3]));
      if (!first && __ballot(mnew != mrun)) {
        const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
        lrun *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      }
      lrun += bsum;
      mrun = mnew;
      // 16-key step u = 2·nb + uu uses the scores e = 8uu .. 8uu + 7 of 32-key block nb.
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int nb = u >> 1, uu = u & 1;
        pf[u] = u32x4_t{pack_bf16x2(sacc[nb][8 * uu + 0], sacc[nb][8 * uu + 1]),
                        pack_bf16x2(sacc[nb][8 * uu + 2], sacc[nb][8 * uu + 3]),
                        pack_bf16x2(sacc[nb][8 * uu + 4], sacc[nb][8 * uu + 5]),
                        pack_bf16x2(sacc[nb][8 * uu + 6], sacc[nb][8 * uu + 7])};
      }
    }
    // The copies of step t − 2 have landed (this step's eight are the only ones newer).
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  };
  const int pairs = (nkb + 3) / 2;   // steps 0 .. nkb + 1, two per iteration
  if (g == 0) {
    for (int i = 0; i < pairs; ++i) {
      mma_step(2 * i);
      asm volatile("s_barrier" ::: "memory");
      softmax_step(2 * i + 1);
      asm volatile("s_barrier" ::: "memory");
    }
  } else {
    for (int i = 0; i < pairs; ++i) {
      softmax_step(2 * i);
      asm volatile("s_barrier" ::: "memory");
      mma_step(2 * i + 1);
      asm volatile("s_barrier" ::: "memory");
    }
  }
  // The last copies (zeros past the range) land before the rings are reused below.
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");

  // Merge the two groups' partial results (every copy has landed and every LDS read of
  // the rings is done). Group 1 stages O (fp32, lane-major 16-byte pieces), m and l.
  float* const stO = reinterpret_cast<float*>(smem) + w * (64 * 64);
  float* const stM = reinterpret_cast<float*>(smem) + 4 * 64 * 64 + w * 128;
  if (g == 1) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        *reinterpret_cast<f32x4_t*>(stO + ((db * 4 + jj) * 64 + lane) * 4) =
            f32x4_t{oacc[db][4 * jj], oacc[db][4 * jj + 1], oacc[db][4 * jj + 2], oacc[db][4 * jj + 3]};
    stM[lane] = mrun;
    stM[64 + lane] = lrun;
  }
  __syncthreads();
  if (g == 0 && q < p.seq) {
  const float m1 = stM[lane], l1 = stM[64 + lane];
  const float m = fmaxf(mrun, m1);
  const float a0 = __builtin_amdgcn_exp2f(mrun - m), a1 = __builtin_amdgcn_exp2f(m1 - m);
  const float l = a0 * lrun + a1 * l1;
  // ln Σ_k exp(scale·s_k) = (m + log2 l)·ln 2 with m, l the merged max and sum (log2 units).
  if (p.lse && h == 0) p.lse[(row0 + q) * p.ld_lse + head] = (m + log2f(l)) * 0.69314718055994531f;
  const float inv = 1.0f / l, b0 = a0 * inv, b1 = a1 * inv;
  // O[q][d .. d+3]; lane holds d = 32·db + 8·jj + 4h + (0..3).
  uint16_t* dst = p.o + (row0 + q) * p.ld_o + head * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4_t o1 = *reinterpret_cast<const f32x4_t*>(stO + ((db * 4 + jj) * 64 + lane) * 4);
      const float v0 = oacc[db][4 * jj] * b0 + o1.x * b1, v1 = oacc[db][4 * jj + 1] * b0 + o1.y * b1;
      const float v2 = oacc[db][4 * jj + 2] * b0 + o1.z * b1, v3 = oacc[db][4 * jj + 3] * b0 + o1.w * b1;
      *reinterpret_cast<u32x2_t*>(dst + db * 32 + 8 * jj + 4 * h) = u32x2_t{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
    }
  }
  };
  run_block(p.nqb - 1 - kpair);
  if (p.nqb - 1 - kpair != kpair) {
    // The staged partials are read before the next block's copies overwrite them.
    __syncthreads();
    run_block(kpair);
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
  const int blocks = (p.nqb + 1) / 2 * p.heads * p.batch;
  note_kernel("attn_fwd_kernel");
  DOMINO_LAUNCH(attn_fwd_kernel, dim3(blocks), dim3(512), 0, s, p);
  return hipGetLastError();
}

}  // namespace domino
