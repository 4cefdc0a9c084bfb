/*
 * domino.h — C ABI of the MI355X (gfx950) Domino tensor-parallel shard library.
 *
 * One tensor-parallel (TP) rank's share of a transformer layer, X·A·B = Y, computed in
 * Domino's independent chunks, with the TP AllReduce's reduction done on one GPU by
 * summing the rank's own partial with the other ranks' partials held in local HBM.
 *
 * Sources (web pages, by title and section):
 *   "DeepSpeed-Domino 深度解析：通过通用张量切分与计算通信重叠实现单机与多节点统一的 LLM 张量并行训练"
 *     — "TP 的数据依赖：通信为何难以隐藏": a TP layer is X·A·B = Y followed by AllReduce(Y);
 *       for the MLP A and B are linear layers, for attention A is multi-head attention
 *       and B the output projection.
 *     — "按行切分输入 X" / "按列切分权重 B" / "2D 切分（同时切 X 与 B）": the three splits
 *       (rows of X along batch; columns of B, its last dimension; both).
 *     — "反向：扩展与权重梯度计算的重叠": each grad matmul is two independent products
 *       (input gradient, weight gradient); the input-gradient reduce hides behind the
 *       weight-gradient products.
 *     — "异步 AllReduce 的发起" / "μ-batch 流水": the reduce is issued asynchronously per
 *       chunk and waited before its consumer.
 *     — "如何尝试 DeepSpeed-Domino": causal self-attention only; the config fields
 *       hidden_size, num_attention_heads, ffn_hidden_size, params_dtype.
 *   "从单卡到集群…" (parallel-training primer), §3.1 "TP的切分方式与计算模式": column-parallel
 *     first FFN layer, row-parallel second layer, partial sums reduced.
 *   "04 · TP/SP 的通信-计算 overlap 与工程优化", §1: grad_input = grad_output·Wᵀ needs the
 *     reduce, grad_weight = grad_outputᵀ·input is local and accumulates in fp32.
 *
 * Conventions shared by every call
 *   Layout     Row-major, explicit sizes. Tokens are T = batch·seq rows, token = b·seq + i,
 *              so a batch chunk is a contiguous row range. Weights are [in, out] (the X·A
 *              convention). SwiGLU's A_s is [hidden, 2·ffn_shard] = [gate | up].
 *   Dtypes     DOMINO_BF16: bf16 storage, fp32 accumulation, fp32 weight gradients.
 *              DOMINO_F32: fp32 everywhere (MLP calls and shard_reduce only).
 *   Pointers   Device pointers from hipMalloc (or torch), 16-byte aligned. Leading
 *              dimensions are in elements. bf16 matrix widths must be multiples of 8.
 *   Ownership  The caller owns every buffer and both streams. The library keeps no
 *              per-call state; it creates its hipEvent_t objects once per device, lazily.
 *   Streams    Work is enqueued on `compute`; the reductions run on `comm` after an event
 *              wait on the chunk they reduce. Before returning, `compute` is made to wait
 *              on every reduction (the handle wait of the asynchronous AllReduce), unless
 *              the descriptor's `no_join` is set, in which case the reduced output is
 *              valid only in `comm` order. comm == NULL or comm == compute runs the
 *              reductions inline on `compute` (plain, un-overlapped tensor parallelism).
 *              Peer partials must be ready in `compute` order when the call is made.
 *              The overlap needs the two streams on different hardware queues: HIP
 *              spreads streams over a few queues (4 by default) in creation order, so a
 *              process that makes many streams should make these two early and keep them.
 *   Workspace  The block calls take an optional device workspace (`workspace`,
 *              `workspace_bytes`; its size from the matching *_workspace_size query).
 *              With it, a product whose last round of tiles would leave most of the GPU
 *              idle splits those tiles along k into fp32 slices and finishes them with a
 *              fixed-order sum (results do not depend on timing); without it (NULL, or
 *              too small) every tile is computed whole. Its contents need no
 *              initialisation and are scratch between calls; calls sharing one workspace
 *              must be ordered by the caller.
 *   Errors     Every argument is checked before anything is enqueued; on an error
 *              nothing runs and the status says why. A failed HIP launch returns
 *              DOMINO_ERR_HIP (work enqueued before it may have run).
 *   Limits     (DOMINO_ERR_UNSUPPORTED beyond them; the kernels index with 32-bit
 *              offsets) every leading dimension of a product operand — hidden, n1,
 *              ffn_shard, 3·heads·head_dim — at most 2^22 elements; at most 2^31 tokens;
 *              a reduced region (shard_reduce, or T × hidden of a block call) at most
 *              2^32 − 2^21 groups of 8 bf16 (4 fp32) elements.
 *   Threads    Calls may come from any host thread; calls that share output buffers
 *              must be ordered by the caller.
 */
#ifndef DOMINO_H
#define DOMINO_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DOMINO_OK = 0,
  DOMINO_ERR_INVALID_ARG = 1,  /* null pointer, bad enum, n_partials out of range */
  DOMINO_ERR_SHAPE = 2,        /* sizes inconsistent or not divisible as required */
  DOMINO_ERR_ALIGN = 3,        /* pointer not 16-byte aligned or width / ld not a multiple of 8 */
  DOMINO_ERR_UNSUPPORTED = 4,  /* a valid combination the library does not implement */
  DOMINO_ERR_HIP = 5           /* a HIP runtime call or kernel launch failed */
} domino_status;

typedef enum { DOMINO_F32 = 0, DOMINO_BF16 = 1 } domino_dtype;
typedef enum { DOMINO_ACT_GELU_TANH = 0, DOMINO_ACT_SWIGLU = 1 } domino_act;

/* Maximum number of partials one reduction sums (own partial included). */
#define DOMINO_MAX_PARTIALS 16

/* MLP shard: Y_s = act(X·A_s)·B_s with A_s [hidden, n1], B_s [ffn_shard, hidden],
 * n1 = ffn_shard (GeLU) or 2·ffn_shard (SwiGLU). Chunks: (row_chunks, col_chunks) =
 * (1,1) unsplit, (r,1) rows of X split along batch into r chunks, (1,c) columns of B_s
 * into c chunks, (r,c) the 2D split, chunk order r0c0, r0c1, r1c0, ... */
typedef struct {
  int64_t batch, seq, hidden, ffn_shard;
  int32_t act;          /* domino_act */
  int32_t dtype;        /* domino_dtype */
  int32_t row_chunks;   /* >= 1, divides batch */
  int32_t col_chunks;   /* >= 1, hidden % (8·col_chunks) == 0 */
  int32_t n_partials;   /* P = TP degree: own partial + P-1 peer partials; 1..DOMINO_MAX_PARTIALS */
  int32_t no_join;      /* 0: compute waits on the reductions before return; 1: it does not */
} domino_mlp_desc;

/* Attention shard: heads · head_dim columns each of Q, K, V; causal self-attention. */
typedef struct {
  int64_t batch, seq, hidden, heads, head_dim;
  float scale;          /* softmax scale; 0 means 1/sqrt(head_dim) */
  int32_t dtype;        /* DOMINO_BF16 only */
  int32_t row_chunks;   /* >= 1, divides batch (a chunk holds whole sequences) */
  int32_t n_partials;
  int32_t no_join;
} domino_attn_desc;

/*
 * shard_reduce — the AllReduce's reduction on one GPU ("TP 的数据依赖：通信为何难以隐藏":
 * AllReduce(Y) sums the ranks' partials; primer §3.1: row-parallel outputs are partial
 * sums). out[r, c] = Σ_{p=0}^{n_partials-1} partials[p][r·ld_in + c] for r < rows,
 * c < cols, accumulated in fp32 in the order p = 0, 1, ..., rounded once to the dtype
 * (round to nearest even for bf16).
 *   out        device, [rows, ld_out]; may alias partials[p] only if ld_out == ld_in
 *   partials   HOST array of n_partials device pointers, each [rows, ld_in]
 *   cols       multiple of 8 (bf16) or 4 (fp32); ld_* >= cols and multiples of 8 / 4
 * rows == 0 or cols == 0 enqueues nothing and returns DOMINO_OK.
 */
domino_status shard_reduce(void* out, int64_t ld_out, const void* const* partials, int32_t n_partials,
                           int64_t ld_in, int64_t rows, int64_t cols, int32_t dtype, hipStream_t stream);

/*
 * domino_block_fwd — MLP shard forward in Domino chunks ("按行切分输入 X", "按列切分权重 B",
 * "2D 切分"; primer §3.1 for the column→row pairing).
 * Hpre = X·A_s and H = act(Hpre) (one GEMM over all rows with a fused activation
 * epilogue; it feeds no reduction); then for each chunk (R_i, C_j): Y_own[R_i, C_j] =
 * H[R_i]·B_s[:, C_j], and the chunk's reduction Y[R_i, C_j] = Y_own + Σ peer_Y runs on
 * `comm` while the next chunk's GEMM runs on `compute`.
 *   X [T, hidden]; A_s [hidden, n1]; B_s [ffn_shard, hidden]            (inputs)
 *   b1_s [n1] or NULL                  the column-parallel bias (deep-dive, "如何尝试
 *                                      DeepSpeed-Domino": add_bias_linear), added before the
 *                                      activation: Hpre = X·A_s + b1_s (bf16 only)
 *   Hpre [T, n1], H [T, ffn_shard]     saved for the backward           (outputs)
 *   Y_own [T, hidden]                  this rank's partial              (output)
 *   peer_Y  HOST array of n_partials-1 device pointers [T, hidden]      (inputs; NULL if P==1)
 *   Y [T, hidden]                      reduced output; NULL or Y_own reduces in place into
 *                                      Y_own (with P == 1 that means no reduction runs)
 *   workspace, workspace_bytes         optional device scratch (see Workspace above). In bf16,
 *                                      when the first product runs on the large-tile kernel
 *                                      and the workspace holds domino_block_fwd_workspace_size
 *                                      bytes, its front first receives transposed copies of A_s
 *                                      and B_s, which both products then read contiguous along
 *                                      k (the same values in the same order: the outputs equal
 *                                      those without a workspace bit for bit).
 */
domino_status domino_block_fwd(const domino_mlp_desc* desc, const void* X, const void* A_s, const void* B_s,
                               const void* b1_s, void* Hpre, void* H, void* Y_own, const void* const* peer_Y, void* Y,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t compute, hipStream_t comm);

/* Bytes of workspace the block calls with this descriptor can use (0 for an invalid
 * descriptor or when no product splits; any size, including 0, is valid to pass). */
size_t domino_block_fwd_workspace_size(const domino_mlp_desc* desc);
size_t domino_block_bwd_workspace_size(const domino_mlp_desc* desc);

/*
 * domino_block_bwd — MLP shard backward ("反向：扩展与权重梯度计算的重叠"; overlap page §1).
 *   dHpre = act'(Hpre) ⊙ (dY·B_sᵀ)      (one GEMM over all rows, activation gradient fused)
 * then per dX chunk (row chunks; for a column-only split, column chunks of dX, the mirror
 * of the forward's column split; the 2D split reduces dX by row chunks):
 *   dX_own[chunk] = dHpre·A_s[chunk]ᵀ   (this rank's partial input gradient)
 *   dX[chunk] = dX_own + Σ peer_dX      (reduction on `comm`)
 * then the independent weight gradients, which hide the last reduction:
 *   dB_s (+)= Hᵀ·dY,  dA_s (+)= Xᵀ·dHpre     (fp32; accumulate != 0 adds to their contents)
 *   X, A_s, B_s, Hpre, H as in the forward; dY [T, hidden]                (inputs)
 *   dHpre [T, n1]                       caller-provided scratch/output (bf16 or fp32)
 *   dX_own, dX [T, hidden]; peer_dX HOST array of n_partials-1 device pointers; dX NULL or
 *                                       dX_own reduces in place into dX_own
 *   dA_s [hidden, n1], dB_s [ffn_shard, hidden]  fp32
 *   d_b1_s [n1] fp32 or NULL            (+)= Σ_rows dHpre, the bias gradient (bf16 only; needs
 *                                       the workspace)
 *   workspace, workspace_bytes          optional device scratch (see Workspace above)
 * Weight gradients are deterministic; the reduction order is fixed.
 */
domino_status domino_block_bwd(const domino_mlp_desc* desc, const void* X, const void* A_s, const void* B_s,
                               const void* Hpre, const void* H, const void* dY, void* dHpre,
                               void* dX_own, const void* const* peer_dX, void* dX,
                               float* dA_s, float* dB_s, float* d_b1_s, int32_t accumulate,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t compute, hipStream_t comm);

/*
 * domino_block_bwd_noalloc — domino_block_bwd without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The arguments and results are those of
 * domino_block_bwd; the k-split workspace is a static device array of
 * DOMINO_NOALLOC_SCRATCH_BYTES bytes that each GPU holds until the process ends.
 *   - Shapes whose domino_block_bwd_workspace_size exceeds that size are rejected with
 *     DOMINO_ERR_UNSUPPORTED before anything is enqueued (domino_last_error says why).
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents:
 *     calls that overlap on one GPU (different streams, or host threads) race on it and
 *     must be ordered by the caller.
 *   - No hipMalloc, hipFree or other allocating routine is called. The first call on a
 *     device looks up the array's device address; the library's events are created once
 *     per device and host thread, on its first call there (as for every entry point).
 */
#define DOMINO_NOALLOC_SCRATCH_BYTES (64u << 20)
domino_status domino_block_bwd_noalloc(const domino_mlp_desc* desc, const void* X, const void* A_s,
                                       const void* B_s, const void* Hpre, const void* H, const void* dY,
                                       void* dHpre, void* dX_own, const void* const* peer_dX, void* dX,
                                       float* dA_s, float* dB_s, float* d_b1_s, int32_t accumulate,
                                       hipStream_t compute, hipStream_t comm);

/*
 * domino_attn_block_fwd — attention shard forward by row chunks (whole sequences)
 * ("TP 的数据依赖…": A = multi-head attention on the rank's heads, B = output projection;
 * "前向：多个计算片段轮转重叠 AllReduce": AllReduce(attn0) overlaps μ-batch 1's attention).
 * QKV = X·A_qkv_s and O = causal softmax(Q·Kᵀ·scale)·V per (sequence, head), each one
 * launch over all sequences; then per chunk: Y_own = O·B_o_s; Y = Y_own + Σ peer_Y on `comm`.
 *   X [T, hidden]; A_qkv_s [hidden, 3·heads·head_dim] = [Q | K | V] blocks, head j at
 *   columns j·head_dim within each block; B_o_s [heads·head_dim, hidden]   (inputs)
 *   b_qkv_s [3·heads·head_dim] or NULL  column-parallel bias: QKV = X·A_qkv_s + b_qkv_s
 *   QKV [T, 3·heads·head_dim], O [T, heads·head_dim]   saved activations   (outputs)
 *   lse [T, heads] fp32 or NULL: per query row and head, ln Σ_{k ≤ q} exp(scale·q·k), the
 *                                       statistic the backward needs (output)
 *   Y_own, Y [T, hidden]; peer_Y HOST array of n_partials-1 device pointers
 *   workspace, workspace_bytes          optional device scratch (see Workspace above)
 * head_dim must be 128; bf16 only.
 */
domino_status domino_attn_block_fwd(const domino_attn_desc* desc, const void* X, const void* A_qkv_s,
                                    const void* B_o_s, const void* b_qkv_s, void* QKV, void* O, float* lse, void* Y_own,
                                    const void* const* peer_Y, void* Y, void* workspace, size_t workspace_bytes,
                                    hipStream_t compute, hipStream_t comm);
size_t domino_attn_block_fwd_workspace_size(const domino_attn_desc* desc);

/*
 * domino_attn_block_bwd — attention shard backward ("反向：扩展与权重梯度计算的重叠";
 * overlap page §1: input gradients need the reduction, weight gradients are local).
 *   dO = dY·B_o_sᵀ                            (one GEMM over all rows)
 *   dQKV = [dQ | dK | dV] of causal attention per (sequence, head), from QKV, O, dO and
 *          lse: with P = exp(scale·Q·Kᵀ − lse) (causal), dV = Pᵀ·dO, dS = P ⊙ (dO·Vᵀ − Δ),
 *          Δ = rowsum(dO ⊙ O), dQ = scale·dS·K, dK = scale·dSᵀ·Q    (one pass over all rows)
 * then per row chunk (whole sequences):
 *   dX_own[chunk] = dQKV·A_qkv_sᵀ            (this rank's partial input gradient)
 *   dX[chunk] = dX_own + Σ peer_dX            (reduction on `comm`)
 * then the independent weight gradients, which hide the last reduction:
 *   dA_qkv_s (+)= Xᵀ·dQKV,  dB_o_s (+)= Oᵀ·dY  (fp32; accumulate != 0 adds to their contents)
 *   X, A_qkv_s, B_o_s, QKV, O as in the forward; lse from the forward (required);
 *   dY [T, hidden]                                                         (inputs)
 *   dO [T, heads·head_dim], dQKV [T, 3·heads·head_dim]   caller-provided scratch/outputs
 *   dX_own, dX [T, hidden]; peer_dX HOST array of n_partials-1 device pointers
 *   dA_qkv_s [hidden, 3·heads·head_dim], dB_o_s [heads·head_dim, hidden]   fp32
 *   d_b_qkv_s [3·heads·head_dim] fp32 or NULL  (+)= Σ_rows dQKV, the bias gradient
 *   workspace, workspace_bytes          device scratch of at least
 *                                       domino_attn_block_bwd_workspace_size bytes (required:
 *                                       it also holds the attention statistics)
 * Deterministic: no atomics; the reduction order is fixed.
 */
domino_status domino_attn_block_bwd(const domino_attn_desc* desc, const void* X, const void* A_qkv_s,
                                    const void* B_o_s, const void* QKV, const void* O, const float* lse,
                                    const void* dY, void* dO, void* dQKV, void* dX_own,
                                    const void* const* peer_dX, void* dX, float* dA_qkv_s, float* dB_o_s,
                                    float* d_b_qkv_s, int32_t accumulate, void* workspace, size_t workspace_bytes,
                                    hipStream_t compute, hipStream_t comm);
size_t domino_attn_block_bwd_workspace_size(const domino_attn_desc* desc);

/*
 * The small-kernel group between sublayers (deep-dive, "前向：多个计算片段轮转重叠 AllReduce":
 * the Dropout, Residual and LayerNorm kernels that hide an AllReduce; the layer excerpt
 * under "μ-batch 流水"), fused into one pass over the rows. bf16, rows × hidden contiguous;
 * hidden a multiple of 8, at most 8192; 0 <= p_drop < 1; eps > 0.
 */
typedef struct {
  int64_t rows, hidden;
  float eps;        /* LayerNorm epsilon, inside the root */
  float p_drop;     /* dropout probability; kept values are scaled by 1/(1 − p_drop) */
} domino_group_desc;

/*
 * domino_resid_ln_fwd:
 *   resid_out = resid + dropout(y + bias)     (y NULL: resid_out = resid; bias NULL: 0;
 *                                              keep NULL: no dropout)
 *   ln_out = (resid_out − μ)·rstd·gamma + beta, μ and σ² over the row (biased variance),
 *   rstd = 1/√(σ² + eps), computed from the stored bf16 resid_out; mean, rstd [rows] fp32
 *   saved for the backward. gamma NULL: no LayerNorm (ln_out, beta, mean, rstd unused);
 *   beta NULL: 0.
 *   keep: bit-packed [rows][ceil(hidden/32)] int32 words, element j of a row kept iff bit
 *   j % 32 of word j / 32 is set. resid_out may alias resid. Fp32 arithmetic, one rounding
 *   per output.
 */
domino_status domino_resid_ln_fwd(const domino_group_desc* desc, const void* resid, const void* y,
                                  const void* bias, const int32_t* keep, void* resid_out, const void* gamma,
                                  const void* beta, void* ln_out, float* mean, float* rstd, hipStream_t stream);

/*
 * domino_resid_ln_bwd: the backward of domino_resid_ln_fwd.
 *   d_resid = d_res + LayerNorm'(d_ln)  (d_res NULL: 0; d_ln NULL: no LayerNorm term)
 *     with g = d_ln·gamma, x̂ = (resid_out − mean)·rstd:
 *     LayerNorm'(d_ln) = rstd·(g − mean_row(g) − x̂·mean_row(g·x̂))
 *   d_y = dropout'(d_resid) = keep ? d_resid/(1 − p_drop) : 0   (NULL: not stored)
 *   d_gamma (+)= Σ_rows d_ln·x̂, d_beta (+)= Σ_rows d_ln, d_bias (+)= Σ_rows d_y   [hidden] fp32,
 *   each NULL to skip; accumulate != 0 adds to their contents. Column sums are per-block
 *   partials in the workspace, summed in a fixed order (deterministic).
 *   resid_out, mean, rstd, gamma: from the forward (needed when d_ln is given).
 *   d_resid may alias d_res. workspace: at least domino_resid_ln_bwd_workspace_size bytes.
 */
domino_status domino_resid_ln_bwd(const domino_group_desc* desc, const void* d_ln, const void* d_res,
                                  const void* resid_out, const float* mean, const float* rstd, const void* gamma,
                                  const int32_t* keep, void* d_resid, void* d_y, float* d_gamma, float* d_beta,
                                  float* d_bias, int32_t accumulate, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);
size_t domino_resid_ln_bwd_workspace_size(const domino_group_desc* desc);

/*
 * A stack of Domino transformer layers on one tensor-parallel rank (deep-dive, "前向：多个计算
 * 片段轮转重叠 AllReduce" and the DominoTransformerLayer excerpt under "μ-batch 流水"). Per
 * layer, with x the residual stream entering it:
 *   a = LN1(x);  y_attn = Σ_ranks Attn_s(a);  h = x + dropout(y_attn + b_o);  m = LN2(h);
 *   y_mlp = Σ_ranks MLP_s(m);  x_next = h + dropout(y_mlp + b_2)
 * (Attn_s: QKV product, causal attention over the rank's heads, out-projection; MLP_s: GEMM
 * with the activation epilogue, GEMM; Σ_ranks: the own partial plus the P-1 peer partials,
 * the AllReduce's sum). The rows are split into row_chunks μ-batches of whole sequences. Per
 * layer the work forms blocks: the attention block of each μ, then the MLP block of each μ;
 * a block is its group kernel (the closing group of the previous layer fused with LN1, which
 * waits for that layer's MLP reduction of μ; or dropout + residual + LN2, which waits for the
 * attention reduction of μ), its products (QKV product, attention, out-projection; or GEMM1,
 * GEMM2) and the reduction its last product starts on `comm`. So the reduction of one
 * μ-batch's attention hides behind the next μ-batch's attention, an MLP reduction behind the
 * next μ-batch's MLP, and a layer's last MLP reduction behind the next layer's first
 * attention. With row_chunks >= 2 each block's group kernel is issued on `compute` before the
 * previous block's last product (the reduction it waits for was started one block earlier),
 * so the HBM-bound group does not run beside the reduction that product starts; with one
 * μ-batch it follows that product. After the last layer the closing group writes `out` per
 * μ. comm NULL (or == compute): everything in order on `compute`.
 */
typedef struct {
  int64_t batch, seq, hidden;
  int64_t heads, head_dim;    /* this rank's heads; head_dim 128 */
  int64_t ffn_shard;          /* this rank's FFN columns (per half for SwiGLU) */
  int32_t act;                /* domino_act */
  float eps;                  /* LayerNorm epsilon (inside the root), > 0 */
  float p_drop;               /* dropout probability of both residual branches, [0, 1) */
  float scale;                /* softmax scale; 0 means 1/sqrt(head_dim) */
  int32_t row_chunks;         /* μ-batches, >= 1, divides batch */
  int32_t n_partials;         /* P: own partial + P-1 peer partials */
  int32_t layers;             /* >= 1 */
  int32_t reserved;           /* 0 */
} domino_layer_desc;

/* One layer's parameters on this rank (device pointers, bf16; T = batch·seq). */
typedef struct {
  const void* ln1_gamma; const void* ln1_beta;    /* [hidden]; beta may be NULL (0) */
  const void* A_qkv_s;                            /* [hidden, 3·heads·head_dim] = [Q | K | V] */
  const void* B_o_s;                              /* [heads·head_dim, hidden] */
  const void* b_o;                                /* [hidden] or NULL */
  const void* ln2_gamma; const void* ln2_beta;
  const void* A_s;                                /* [hidden, n1] ([gate | up] for SwiGLU) */
  const void* B_s;                                /* [ffn_shard, hidden] */
  const void* b_2;                                /* [hidden] or NULL */
  const int32_t* keep_attn;                       /* keep masks [T][ceil(hidden/32)] (bit j % 32 of */
  const int32_t* keep_mlp;                        /* word j / 32) or NULL: no dropout there */
  const void* b_qkv;                              /* [3·heads·head_dim] column-parallel bias or NULL */
  const void* b_1;                                /* [n1] column-parallel bias or NULL */
} domino_layer_params;

/* One layer's activations: written by the forward and kept for the backward. All
 * [T, hidden] bf16 unless stated. */
typedef struct {
  void* x_in;                                     /* the residual stream entering the layer; for layer 0
                                                     NULL means X itself (else a copy of X is written) */
  void* ln1; float* mean1; float* rstd1;          /* LN1 output; its row mean and 1/σ [T] fp32 */
  void* QKV;                                      /* [T, 3·heads·head_dim] */
  void* O;                                        /* [T, heads·head_dim] */
  float* lse;                                     /* [T, heads] fp32 or NULL */
  void* y_attn_own;                               /* this rank's attention partial */
  const void* const* peer_y_attn;                 /* HOST array of P-1 device pointers */
  void* y_attn;                                   /* reduced attention output (may be y_attn_own if P = 1) */
  void* h; void* ln2; float* mean2; float* rstd2; /* mid residual, LN2 output and its statistics */
  void* Hpre; void* H;                            /* [T, n1], [T, ffn_shard] */
  void* y_mlp_own; const void* const* peer_y_mlp; void* y_mlp;
} domino_layer_acts;

/* params and acts: arrays of desc->layers entries. out [T, hidden]: the last layer's output.
 * workspace: optional device scratch (k-split slices). */
domino_status domino_stack_fwd(const domino_layer_desc* desc, const void* X, const domino_layer_params* params,
                               const domino_layer_acts* acts, void* out, void* workspace, size_t workspace_bytes,
                               hipStream_t compute, hipStream_t comm);

/*
 * One layer's gradients and backward scratch on this rank (device pointers). Parameter
 * gradients are fp32 (NULL skips the bias ones); the rest is bf16 [T, hidden] unless stated.
 */
typedef struct {
  float* d_ln1_gamma; float* d_ln1_beta;          /* [hidden] */
  float* dA_qkv_s; float* dB_o_s; float* d_b_o;   /* as A_qkv_s, B_o_s; [hidden] or NULL */
  float* d_ln2_gamma; float* d_ln2_beta;
  float* dA_s; float* dB_s; float* d_b_2;
  void* d_x_in;        /* gradient of the residual stream entering the layer (layer 0: NULL, dX is used) */
  void* d_ym;          /* gradient of y_mlp: the MLP's dY */
  void* dHpre;         /* [T, n1] */
  void* dx_mlp_own; const void* const* peer_dx_mlp; void* dx_mlp;     /* MLP input-gradient partials, their sum */
  void* d_h;           /* gradient of the middle residual h */
  void* d_ya;          /* gradient of y_attn: the attention's dY */
  void* dO;            /* [T, heads·head_dim] */
  void* dQKV;          /* [T, 3·heads·head_dim] */
  void* dx_attn_own; const void* const* peer_dx_attn; void* dx_attn;  /* attention input-gradient partials, sum */
  float* d_b_qkv; float* d_b_1;                                       /* [3·heads·head_dim], [n1] or NULL */
} domino_layer_grads;

/*
 * domino_stack_bwd — the backward of domino_stack_fwd, in reverse order of its steps
 * (deep-dive, "反向：扩展与权重梯度计算的重叠"; overlap page §1: input gradients need the
 * reduction, weight gradients are local). Given d_out, the gradient of `out`:
 *   the last layer's closing group: d_ym = dropout'(d_out);
 *   per layer, top down (in each "for each μ" below, the group kernel of μ+1 is issued
 *   before the last product of μ, so it does not run beside the reduction that product starts;
 *   with two or more μ-batches the first LN2 backward is issued before the MLP's last product):
 *     for each μ: MLP input gradient (dHpre = act'(Hpre) ⊙ d_ym·B_sᵀ, dx_mlp_own =
 *                 dHpre·A_sᵀ), then its reduction on `comm`;
 *     for each μ: wait for the MLP reduction of μ; LN2's backward with the residual
 *                 gradient (d_h) and dropout'(d_h) = d_ya; attention input gradient (dO,
 *                 attention backward, dx_attn_own = dQKV·A_qkv_sᵀ), then its reduction
 *                 (the MLP's last reduction hides behind the first μ-batch's work here);
 *     dA_qkv_s (+)= ln1ᵀ·dQKV, dB_o_s (+)= Oᵀ·d_ya, dB_s (+)= Hᵀ·d_ym,
 *     dA_s (+)= ln2ᵀ·dHpre                          (hide the attention's last reduction);
 *     for each μ: wait for the attention reduction of μ; LN1's backward with the residual
 *                 gradient gives d_x_in, fused with the layer below's closing group
 *                 (d_ym of that layer = dropout'(d_x_in)) — issued at the start of the layer
 *                 below, so a layer's last attention reduction hides behind the next
 *                 layer's first MLP input gradient;
 *   layer 0's LN1 backward writes dX.
 * LayerNorm and bias gradients are sums over rows (fixed order). accumulate != 0 adds every
 * parameter gradient to its contents. workspace: at least domino_stack_bwd_workspace_size
 * bytes (required: it holds the attention statistics and the column partial sums).
 * params and acts: those of the forward; grads: desc->layers entries.
 */
domino_status domino_stack_bwd(const domino_layer_desc* desc, const void* X, const domino_layer_params* params,
                               const domino_layer_acts* acts, const domino_layer_grads* grads, const void* d_out,
                               void* dX, int32_t accumulate, void* workspace, size_t workspace_bytes,
                               hipStream_t compute, hipStream_t comm);
size_t domino_stack_bwd_workspace_size(const domino_layer_desc* desc);

/* Human-readable name of a status code (static storage). */
const char* domino_status_string(domino_status status);

/* Text of the most recent error on the calling thread (static thread-local storage). */
const char* domino_last_error(void);

/*
 * Kernel timing for measurement: while enabled, each timed launch (one kernel, or a kernel
 * and its small companion such as a column sum) is dispatched with a pair of hipEvents
 * that the dispatch itself records at the first kernel's start and the last kernel's end
 * (hipExtLaunchKernel), on the stream it runs on. domino_timing_read waits for those events
 * and returns, for kernel class `kind`, the number of launches and their summed duration
 * in milliseconds since the last reset. Keep timing off outside measurement and graph
 * capture.
 */
typedef enum {
  DOMINO_K_REDUCE = 0,
  DOMINO_K_FWD_GEMM1 = 1,   /* X·A_s + activation epilogue */
  DOMINO_K_FWD_GEMM2 = 2,   /* H·B_s[:, C_j] */
  DOMINO_K_DGRAD_B = 3,     /* dY·B_sᵀ + activation-gradient epilogue */
  DOMINO_K_DGRAD_A = 4,     /* dHpre·A_sᵀ */
  DOMINO_K_WGRAD_B = 5,     /* Hᵀ·dY */
  DOMINO_K_WGRAD_A = 6,     /* Xᵀ·dHpre */
  DOMINO_K_QKV = 7,
  DOMINO_K_ATTN = 8,
  DOMINO_K_OUTPROJ = 9,
  DOMINO_K_AUX = 10,        /* k-split tiles' fixed-order slice sums with their epilogues; the
                               MLP forward's transposed weight copies */
  DOMINO_K_ATTN_BWD = 11,   /* attention backward: the dK/dV kernel */
  DOMINO_K_OUTPROJ_DGRAD = 12,  /* dY·B_o_sᵀ */
  DOMINO_K_QKV_DGRAD = 13,  /* dQKV·A_qkv_sᵀ */
  DOMINO_K_OUTPROJ_WGRAD = 14,  /* Oᵀ·dY */
  DOMINO_K_QKV_WGRAD = 15,  /* Xᵀ·dQKV */
  DOMINO_K_ATTN_BWD_DQ = 16,    /* attention backward: the dQ kernel */
  DOMINO_K_ATTN_BWD_PREP = 17,  /* attention backward: Δ and the per-row statistics */
  DOMINO_K_GROUP_FWD = 18,      /* dropout + residual + LayerNorm */
  DOMINO_K_GROUP_BWD = 19,      /* its backward (with the fixed-order column sums) */
  DOMINO_K_BIAS_GRAD = 20,      /* column sums of dHpre or dQKV (column-parallel bias gradients) */
  DOMINO_K_COUNT = 21
} domino_kernel_kind;

domino_status domino_timing_enable(int32_t enable);   /* enabling also resets */
domino_status domino_timing_read(int32_t kind, int64_t* launches, double* total_ms);
/*
 * Writes into `name` (capacity bytes, NUL-terminated) the kernel that the most recent
 * timed launch of class `kind` ran: its symbol and template arguments as a profiler
 * prints them, e.g. "gemm_bf16_kernel<128, 128, 32, 3, 3, false, false, (domino::Epi)5>", or
 * "" if none was timed since the last reset. Launches of one class with the same shapes
 * run the same kernel, so classes can be grouped by it. DOMINO_ERR_INVALID_ARG for a bad
 * kind, a NULL name or a buffer too small for the text.
 */
domino_status domino_timing_kernel(int32_t kind, char* name, size_t capacity);

#ifdef __cplusplus
}
#endif
#endif /* DOMINO_H */
