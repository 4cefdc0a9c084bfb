// Fused causal self-attention forward for one rank's head slice (bf16, head_dim 128).
// For attention the TP layer X·A·B = Y has A = multi-head attention on the rank's heads
// (page "DeepSpeed-Domino 深度解析", section "TP 的数据依赖：通信为何难以隐藏"); only causal
// self-attention is supported (section "如何尝试 DeepSpeed-Domino").
//
// O[q] = Σ_{k ≤ q} softmax_k(Q[q]·K[k]·scale)·V[k] per (sequence, head), computed block by
// block with a running maximum and running sum (online softmax), so the seq×seq score
// matrix never leaves registers.
//
// Design (gfx950): one workgroup = 4 waves = 128 query rows of one (sequence, head);
// each wave owns 32 query rows. Keys advance 64 at a time through two LDS stages.
//  * Scores are computed transposed, Sᵀ = K·Qᵀ (K fragment as the matrix-core's A), so a
//    lane holds 4 keys of one query: the softmax statistics of a query live in one lane
//    column (reduced over 4 lanes with cross-lane shuffles), and the probabilities are
//    already laid out as the B operand of Oᵀ += Vᵀ·Pᵀ.
//  * The 8 keys a lane feeds to one 16x16x32 MFMA are {4g..4g+3} ∪ {16+4g..16+4g+3} of the
//    32-key step (g = lane/16); the V fragment reads the same keys, so the contraction is
//    exact whatever order the matrix core sums them in.
//  * Q stays in registers (read once from global memory); K is staged as [key][d], V as
//    Vᵀ [d][key] (transposed in registers on the way into LDS).
//  * Workgroups are issued longest-first (last query block of every sequence and head
//    first) to balance the causal triangle.
#include "common.hpp"
#include "kernels.hpp"

namespace domino {
namespace {

constexpr int kD = 128;   // head_dim
constexpr int kQB = 128;  // query rows per workgroup
constexpr int kKB = 64;   // keys per stage

// K tile: [64 keys][128 d], 16 chunks of 16 B per row; chunk c stored at c ^ (row & 7).
__device__ __forceinline__ int k_off(int key, int chunk) { return key * kD + ((chunk ^ (key & 7)) << 3); }
// Vᵀ tile: [128 d][64 keys], 8 chunks per row; chunk c stored at c ^ (row&7) ^ ((row>>3)&7).
__device__ __forceinline__ int v_off(int d, int chunk) {
  return d * kKB + ((chunk ^ ((d & 7) ^ ((d >> 3) & 7))) << 3);
}

struct AttnParams {
  const uint16_t* qkv; int64_t ld_qkv;
  uint16_t* o; int64_t ld_o;
  int seq, heads, batch, nqb;
  int64_t hd;          // heads · head_dim (width of each of the Q, K, V blocks)
  float scale_log2;    // scale · log2(e)
};

__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kKB * kD];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kD * kKB];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, lq = lane & 15;
  // Longest-first order: the first heads·batch workgroups take the last query block.
  const int lin = blockIdx.x;
  const int hb = p.heads * p.batch;
  const int qb = p.nqb - 1 - lin / hb;
  const int head = (lin % hb) % p.heads;
  const int b = (lin % hb) / p.heads;

  const int64_t row0 = int64_t(b) * p.seq;  // first token of this sequence
  const uint16_t* Qg = p.qkv + head * kD;
  const uint16_t* Kg = p.qkv + p.hd + head * kD;
  const uint16_t* Vg = p.qkv + 2 * p.hd + head * kD;

  const int q0 = qb * kQB;
  const int qw = q0 + w * 32;  // this wave's first query

  // Q fragments: B operand of Sᵀ = K·Qᵀ; lane (q = qw + nq·16 + lq) holds d = 32s + 8g .. +7.
  u32x4_t qf[2][4];
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    const int q = qw + nq * 16 + lq;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[nq][s] = q < p.seq ? *reinterpret_cast<const u32x4_t*>(Qg + (row0 + q) * p.ld_qkv + s * 32 + g * 8)
                            : u32x4_t{0u, 0u, 0u, 0u};
  }

  f32x4_t oacc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i][0] = oacc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrun[2] = {-1e30f, -1e30f}, lrun[2] = {0.f, 0.f};

  const int q_hi = min(q0 + kQB, p.seq);               // exclusive
  const int nkb = (q_hi + kKB - 1) / kKB;              // key blocks this workgroup needs

  // Global → register staging for one key block.
  u32x4_t kst[4];
  uint32_t vst[8][2];
  auto load_kv = [&](int kb) {
    const int key0 = kb * kKB;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = (tid >> 4) + 16 * j, c = tid & 15;
      kst[j] = key0 + key < p.seq ? *reinterpret_cast<const u32x4_t*>(Kg + (row0 + key0 + key) * p.ld_qkv + c * 8)
                                  : u32x4_t{0u, 0u, 0u, 0u};
    }
    const int db = tid & 31, kb8 = tid >> 5;  // d block of 4, key block of 8
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int key = key0 + kb8 * 8 + kk;
      const u32x2_t t = key < p.seq ? *reinterpret_cast<const u32x2_t*>(Vg + (row0 + key) * p.ld_qkv + db * 4)
                                    : u32x2_t{0u, 0u};
      vst[kk][0] = t.x;
      vst[kk][1] = t.y;
    }
  };
  auto store_kv = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = (tid >> 4) + 16 * j, c = tid & 15;
      *reinterpret_cast<u32x4_t*>(&sK[buf][k_off(key, c)]) = kst[j];
    }
    const int db = tid & 31, kb8 = tid >> 5;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t d4[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = vst[2 * q][e >> 1], hi = vst[2 * q + 1][e >> 1];
        d4[q] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      *reinterpret_cast<u32x4_t*>(&sV[buf][v_off(db * 4 + e, kb8)]) = u32x4_t{d4[0], d4[1], d4[2], d4[3]};
    }
  };

  load_kv(0);
  store_kv(0);
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const bool has_next = kb + 1 < nkb;
    if (has_next) load_kv(kb + 1);

    const int key0 = kb * kKB;
    if (key0 <= qw + 31 && qw < p.seq) {  // some key of this block is visible to this wave
      // Sᵀ = K·Qᵀ for 64 keys × 32 queries.
      f32x4_t sacc[4][2];
#pragma unroll
      for (int mk = 0; mk < 4; ++mk) sacc[mk][0] = sacc[mk][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int mk = 0; mk < 4; ++mk) {
          const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(&sK[buf][k_off(mk * 16 + lq, s * 4 + g)]);
#pragma unroll
          for (int nq = 0; nq < 2; ++nq)
            sacc[mk][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf),
                                                                  __builtin_bit_cast(bf16x8_t, qf[nq][s]),
                                                                  sacc[mk][nq], 0, 0, 0);
        }
      }
      // Online softmax per query (lane column); scores in the log2 domain.
      uint32_t pf[2][2][4];  // [nq][key step t][packed bf16 pairs]
#pragma unroll
      for (int nq = 0; nq < 2; ++nq) {
        const int q = qw + nq * 16 + lq;
        float sv[4][4];
        float mx = -1e30f;
#pragma unroll
        for (int mk = 0; mk < 4; ++mk)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = key0 + mk * 16 + 4 * g + r;
            const float v = (key <= q && key < p.seq) ? sacc[mk][nq][r] * p.scale_log2 : -INFINITY;
            sv[mk][r] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrun[nq], mx);
        const float alpha = exp2f(mrun[nq] - mnew);
        float rs = 0.f;
        float pv[4][4];
#pragma unroll
        for (int mk = 0; mk < 4; ++mk)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            pv[mk][r] = exp2f(sv[mk][r] - mnew);
            rs += pv[mk][r];
          }
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
        lrun[nq] = lrun[nq] * alpha + rs;
        mrun[nq] = mnew;
#pragma unroll
        for (int md = 0; md < 8; ++md) oacc[md][nq] *= alpha;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          pf[nq][t][0] = pack_bf16x2(pv[2 * t][0], pv[2 * t][1]);
          pf[nq][t][1] = pack_bf16x2(pv[2 * t][2], pv[2 * t][3]);
          pf[nq][t][2] = pack_bf16x2(pv[2 * t + 1][0], pv[2 * t + 1][1]);
          pf[nq][t][3] = pack_bf16x2(pv[2 * t + 1][2], pv[2 * t + 1][3]);
        }
      }
      // Oᵀ += Vᵀ·Pᵀ over the block's 64 keys (two 32-key steps).
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int md = 0; md < 8; ++md) {
          const int d = md * 16 + lq;
          const int c0 = 4 * t + (g >> 1), c1 = 4 * t + 2 + (g >> 1), half = (g & 1) * 4;
          const u32x2_t v0 = *reinterpret_cast<const u32x2_t*>(&sV[buf][v_off(d, c0) + half]);
          const u32x2_t v1 = *reinterpret_cast<const u32x2_t*>(&sV[buf][v_off(d, c1) + half]);
          const u32x4_t vf = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
          for (int nq = 0; nq < 2; ++nq) {
            const u32x4_t pfr = {pf[nq][t][0], pf[nq][t][1], pf[nq][t][2], pf[nq][t][3]};
            oacc[md][nq] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vf),
                                                                  __builtin_bit_cast(bf16x8_t, pfr), oacc[md][nq],
                                                                  0, 0, 0);
          }
        }
      }
    }
    if (has_next) store_kv(buf ^ 1);
    __syncthreads();
  }

  // O[q][d .. d+3] = Oᵀ / l.
#pragma unroll
  for (int nq = 0; nq < 2; ++nq) {
    const int q = qw + nq * 16 + lq;
    if (q >= p.seq) continue;
    const float inv = 1.0f / lrun[nq];
    uint16_t* dst = p.o + (row0 + q) * p.ld_o + head * kD;
#pragma unroll
    for (int md = 0; md < 8; ++md) {
      const f32x4_t v = oacc[md][nq] * inv;
      *reinterpret_cast<u32x2_t*>(dst + md * 16 + 4 * g) = u32x2_t{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
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
  p.seq = int(a.seq);
  p.heads = int(a.heads);
  p.batch = int(a.batch);
  p.nqb = int((a.seq + kQB - 1) / kQB);
  p.hd = a.heads * a.head_dim;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  const int blocks = p.nqb * p.heads * p.batch;
  note_kernel("attn_fwd_kernel");
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace domino
