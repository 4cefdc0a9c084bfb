// Host-side launchers of the library's HIP kernels (internal interface; no checks here —
// the C ABI validates every argument before any launcher runs).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace domino {

// Events of a timed call. While the library's kernel timing is on, its timing wrapper hands
// the launches of the call it times (on the calling thread) a start and a stop event, which
// the dispatch itself records: the start at the first kernel's start, the stop at the end of
// every kernel, so that it ends up at the last one's end. Null otherwise.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

constexpr int kMaxPartials = 16;

// Size limits of the kernels' 32-bit index arithmetic, which the C ABI checks.
//  * GEMM operands are copied by buffer loads whose per-lane byte offset from the tile's
//    first row is an int32: row·ld·2 + k-chunk with row < 256, so every leading dimension
//    of a product operand must stay at or below 2^22 elements (255·2^22·2 + 112 < 2^31).
//    The attention kernels' copy offsets (64 rows of the QKV leading dimension) fit
//    within the same bound.
//  * shard_reduce walks its 16-byte groups with a uint32 grid stride (at most
//    kReduceMaxBlocks workgroups × 256 threads, two groups per thread per pass), so a
//    region may hold at most 2^32 − 2^21 groups: the index then never wraps past the end.
constexpr int64_t kMaxLd = int64_t(1) << 22;
constexpr int64_t kReduceMaxGroups = (int64_t(1) << 32) - (int64_t(1) << 21);
// One workgroup per CU: on the Llama-2-13B reductions (8 partials of 16384 × 2560) 256
// workgroups stream 5.7 TB/s alone against 4.9 TB/s for 2048, and leave more of each CU's
// memory pipeline to the products running beside them (Domino step 5.81 vs 5.97 ms).
constexpr int kReduceMaxBlocks = 256;

// Records the kernel (symbol and template arguments) a launcher is about to launch on the
// calling thread; the timing facility attaches it to the launch it brackets.
void note_kernel(const char* name);

struct ReduceArgs {
  void* out;
  int64_t ld_out;
  const void* partials[kMaxPartials];
  int n_partials;
  int64_t ld_in;
  int64_t rows, cols;
  bool bf16;
};
hipError_t launch_shard_reduce(const ReduceArgs& a, hipStream_t s);
hipError_t launch_fill_zero_f32(float* out, int64_t ld, int64_t rows, int64_t cols, hipStream_t s);

// GEMM epilogues. C(m, n) = Σ_k A(m, k)·B(k, n), accumulated in fp32.
enum class Epi : int {
  kStore = 0,        // C[m, n] = acc                                  (C in the input dtype)
  kGelu = 1,         // C[m, n] = acc (Hpre); C2[m, n] = gelu(acc) (H)
  kSwiglu = 2,       // N = f_s pairs: C[m, j] = g, C[m, f_s + j] = u, C2[m, j] = silu(g)·u
  kDGelu = 3,        // C[m, n] = acc · gelu'(aux[m, n])               (aux = Hpre)
  kDSwiglu = 4,      // C[m, j] = acc·u·σ(g)(1 + g(1 − σ(g))), C[m, f_s + j] = acc·silu(g)
  kF32 = 5,          // fp32 C: C = acc, or C += acc when accumulate; split-K writes slices
};

struct GemmArgs {
  int64_t M, N, K;            // for kSwiglu N is f_s (each column yields a gate/up pair)
  const void* A; int64_t lda; bool a_kcontig;   // A(m,k) = a_kcontig ? A[m·lda + k] : A[k·lda + m]
  const void* B; int64_t ldb; bool b_kcontig;   // B(k,n) = b_kcontig ? B[n·ldb + k] : B[k·ldb + n]
  void* C; int64_t ldc;
  void* C2; int64_t ldc2;
  const void* aux; int64_t ldaux;
  int64_t f_s;                // gate/up offset for kSwiglu / kDSwiglu
  Epi epi;
  int accumulate;             // kF32
  float* ws;                  // fp32 slices of k-split tiles; null: every tile runs whole
  int64_t ws_elems;           // capacity of ws in floats
  bool bf16;                  // operand dtype: bf16 (MFMA path) or fp32 (vector-ALU path)
  const void* bias = nullptr; // bf16 [N] (kSwiglu: [gate | up], 2·f_s) added before the epilogue's
                              // activation (kStore, kGelu, kSwiglu; bf16 path only)
};

// Set by launch_gemm when the product left k-split tiles for launch_gemm_fixup, which the
// caller launches next on the same stream (it sums their slices and applies the epilogue).
struct GemmSplit {
  int pending = 0;
  int tile = 0, tiles_m = 0, tiles_n = 0, dp_tiles = 0, splits = 1;
};
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s, GemmSplit* split);
// The eight-wave 256×256 kernel on whole tiles (gemm8.hip); launch_gemm picks it for the
// products it supports and that are large enough.
bool gemm8_supports(const GemmArgs& g);
// Whether launch_gemm_bf16 runs this product on the eight-wave kernel.
bool use_gemm8(const GemmArgs& g);
// dst[c][r] = src[r][c] for a bf16 [rows, cols] matrix (rows, cols multiples of 8).
hipError_t launch_transpose_bf16(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t rows,
                                 int64_t cols, hipStream_t s);
hipError_t launch_gemm8(const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_fixup(const GemmArgs& g, const GemmSplit& split, hipStream_t s);
// Floats of workspace the product's k-split tiles use (0: it splits none); shapes, layouts
// and epilogue of g are read, its pointers are not.
int64_t gemm_ws_elems(const GemmArgs& g);

struct AttnArgs {
  const void* qkv; int64_t ld_qkv;   // [T, 3·H·d] = [Q | K | V]
  void* o; int64_t ld_o;             // [T, H·d]
  float* lse; int64_t ld_lse;        // optional [T, H]: ln Σ_k exp(scale·q·k) per row
  int64_t batch, seq, heads, head_dim;
  float scale;
};
hipError_t launch_attention_fwd(const AttnArgs& a, hipStream_t s);

// Attention backward for one head slice: dQKV [T, 3·H·d] = [dQ | dK | dV] from QKV, O, dO
// and the forward's LSE. `stats` is scratch of attn_bwd_stats_floats() floats.
struct AttnBwdArgs {
  const void* qkv; int64_t ld_qkv;
  const void* o; const void* dout; int64_t ld_o;
  const float* lse; int64_t ld_lse;
  void* dqkv; int64_t ld_dqkv;
  float* stats;
  int64_t batch, seq, heads, head_dim;
  float scale;
};
int64_t attn_bwd_stats_floats(int64_t tokens, int64_t heads);
// The three launches in order: Δ and the stats entries; dK, dV; dQ.
hipError_t launch_attention_bwd_prep(const AttnBwdArgs& a, hipStream_t s);
hipError_t launch_attention_bwd_dkdv(const AttnBwdArgs& a, hipStream_t s);
hipError_t launch_attention_bwd_dq(const AttnBwdArgs& a, hipStream_t s);

// The dropout + residual + LayerNorm group and its backward (bf16 rows × hidden,
// contiguous). Null pointers select the variants the ABI documents.
struct GroupFwdArgs {
  const void* resid; const void* y; const void* bias; const int32_t* keep;
  void* r_out; const void* gamma; const void* beta; void* ln; float* mean; float* rstd;
  int64_t rows, hidden;
  float eps, p_drop;
};
hipError_t launch_resid_ln_fwd(const GroupFwdArgs& a, hipStream_t s);

struct GroupBwdArgs {
  const void* d_ln; const void* d_res; const void* r_out; const float* mean; const float* rstd;
  const void* gamma; const int32_t* keep;
  void* d_resid; void* d_y; float* d_gamma; float* d_beta; float* d_bias;
  int accumulate;
  float* workspace;    // 3 · group_bwd_blocks(rows) · hidden floats
  int64_t rows, hidden;
  float p_drop;
};
int64_t group_bwd_blocks(int64_t rows);

// Column sums of a bf16 [rows, cols] matrix (leading dimension ld), out (+)= Σ_rows, in a
// fixed order; ws holds bias_grad_ws_floats(rows, cols) floats.
int64_t bias_grad_ws_floats(int64_t rows, int64_t cols);
hipError_t launch_bias_grad(const void* x, int64_t rows, int64_t cols, int64_t ld, float* out, int accumulate,
                            float* ws, hipStream_t s);
hipError_t launch_resid_ln_bwd(const GroupBwdArgs& a, hipStream_t s);

}  // namespace domino
