// C ABI of the Domino shard library: argument validation and the two-stream chunk
// scheduler that turns one call into the chunked kernel sequence.
//
// The scheduler follows the pages' Domino schedule (page "DeepSpeed-Domino 深度解析"):
//  * the layer's input rows are split along batch ("按行切分输入 X"), the second weight
//    along its last dimension ("按列切分权重 B"), or both ("2D 切分"); each chunk's output is
//    independent, so its reduction can start as soon as that chunk's products end;
//  * the layer's first product (and, for attention, the attention itself) feeds no
//    reduction, so it is launched once over all rows; only the product whose output is
//    reduced is launched per chunk. Row-splitting makes tensors narrower and hurts kernel
//    efficiency ("按行切分输入 X"), and here that cost buys nothing;
//  * the reductions are issued asynchronously on a second stream and waited only by the
//    consumer ("异步 AllReduce 的发起", "μ-batch 流水"): here `compute` records an event after
//    a chunk's last product, `comm` waits on it and reduces, and `compute` finally waits
//    on `comm` (the handle wait);
//  * in the backward, the input-gradient chunks and their reductions come first and the
//    independent weight-gradient products follow, hiding the last reduction
//    ("反向：扩展与权重梯度计算的重叠"; page "04 · TP/SP 的通信-计算 overlap 与工程优化", §1).
// One hipEvent_t pair per chunk stands in for the pages' communication handles.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/domino.h"
#include "kernels.hpp"

using namespace domino;

namespace {

thread_local std::string t_last_error;

domino_status fail(domino_status st, const std::string& msg) {
  t_last_error = msg;
  return st;
}

// ---------------------------------------------------------------------------------------
// Events: a per-thread, per-device set, created once and reused by every call.
// ---------------------------------------------------------------------------------------
constexpr int kMaxChunks = 64;
struct EventSet {
  bool ready = false;
  hipEvent_t done[kMaxChunks];  // compute: chunk's products finished
  hipEvent_t reduced;           // comm: last reduction finished
  hipEvent_t sub[2][kMaxChunks];  // comm: a layer's attention (0) or MLP (1) reduction of a μ-batch finished
};
constexpr int kMaxDevices = 64;
thread_local EventSet t_events[kMaxDevices];

hipError_t events_for_current_device(EventSet** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  EventSet& es = t_events[dev];
  if (!es.ready) {
    // The events only order kernels of this device's two streams: each kernel's own
    // completion already makes its writes visible device-wide, so the record skips the
    // system-scope fence (host visibility), which leaves the compute stream idle for
    // ~2 us more at every chunk boundary (measured: 5.1 vs 7.1 us between two kernels).
    for (int i = 0; i < kMaxChunks; ++i) {
      e = hipEventCreateWithFlags(&es.done[i], hipEventDisableTiming | hipEventDisableSystemFence);
      if (e != hipSuccess) return e;
    }
    e = hipEventCreateWithFlags(&es.reduced, hipEventDisableTiming | hipEventDisableSystemFence);
    if (e != hipSuccess) return e;
    for (int k = 0; k < 2; ++k)
      for (int i = 0; i < kMaxChunks; ++i) {
        e = hipEventCreateWithFlags(&es.sub[k][i], hipEventDisableTiming | hipEventDisableSystemFence);
        if (e != hipSuccess) return e;
      }
    es.ready = true;
  }
  *out = &es;
  return hipSuccess;
}

// ---------------------------------------------------------------------------------------
// Kernel timing (measurement only).
// ---------------------------------------------------------------------------------------
struct TimingRec {
  int kind;
  hipEvent_t a, b;
  std::string kernel;
};
std::mutex g_timing_mu;
bool g_timing = false;
std::vector<TimingRec> g_timing_recs;
std::vector<hipEvent_t> g_timing_free;
double g_timing_ms[DOMINO_K_COUNT];
int64_t g_timing_n[DOMINO_K_COUNT];
std::string g_timing_kernel[DOMINO_K_COUNT];
thread_local std::string t_kernel;  // the kernel the calling thread's launcher last noted

}  // namespace

LaunchEvents& domino::launch_events() {
  thread_local LaunchEvents ev;
  return ev;
}

namespace {

hipEvent_t timing_event() {
  if (!g_timing_free.empty()) {
    hipEvent_t e = g_timing_free.back();
    g_timing_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventReleaseToDevice) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t timed(int kind, hipStream_t s, F&& f) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    on = g_timing;
  }
  if (!on) return f();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    a = timing_event();
    b = timing_event();
  }
  if (!a || !b) return hipErrorOutOfMemory;
  t_kernel.clear();
  // The launches inside f record a at the first kernel's start and b at the last one's end.
  LaunchEvents& ev = launch_events();
  ev.start = a;
  ev.stop = b;
  hipError_t e = f();
  const bool launched = ev.start == nullptr;
  ev.start = ev.stop = nullptr;
  if (e == hipSuccess && !launched) {  // nothing launched: an empty interval
    e = hipEventRecord(a, s);
    if (e == hipSuccess) e = hipEventRecord(b, s);
  }
  if (e == hipSuccess) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    g_timing_recs.push_back({kind, a, b, t_kernel});
  }
  return e;
}

// ---------------------------------------------------------------------------------------
// Validation helpers.
// ---------------------------------------------------------------------------------------
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

domino_status check_ptr(const void* p, const char* name, bool needed) {
  if (!needed) return DOMINO_OK;
  if (!p) return fail(DOMINO_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(DOMINO_ERR_ALIGN, std::string(name) + " is not 16-byte aligned");
  return DOMINO_OK;
}

domino_status check_peers(const void* const* peers, int n_partials, const char* name, bool needed) {
  if (!needed || n_partials <= 1) return DOMINO_OK;
  if (!peers) return fail(DOMINO_ERR_INVALID_ARG, std::string(name) + " is NULL but n_partials > 1");
  for (int p = 0; p < n_partials - 1; ++p) {
    const std::string nm = std::string(name) + "[" + std::to_string(p) + "]";
    const domino_status st = check_ptr(peers[p], nm.c_str(), true);
    if (st != DOMINO_OK) return st;
  }
  return DOMINO_OK;
}

domino_status check_group_desc(const domino_group_desc* d) {
  if (!d) return fail(DOMINO_ERR_INVALID_ARG, "desc is NULL");
  if (d->rows < 0 || d->hidden < 0) return fail(DOMINO_ERR_SHAPE, "negative size");
  if (d->hidden % 8) return fail(DOMINO_ERR_ALIGN, "hidden must be a multiple of 8");
  if (d->hidden > 8192) return fail(DOMINO_ERR_UNSUPPORTED, "hidden above 8192");
  if (!(d->p_drop >= 0.0f && d->p_drop < 1.0f)) return fail(DOMINO_ERR_INVALID_ARG, "p_drop must be in [0, 1)");
  if (!(d->eps > 0.0f)) return fail(DOMINO_ERR_INVALID_ARG, "eps must be > 0");
  return DOMINO_OK;
}

domino_status check_keep(const int32_t* keep) {
  if (keep && (reinterpret_cast<uintptr_t>(keep) & 3u)) return fail(DOMINO_ERR_ALIGN, "keep is not 4-byte aligned");
  return DOMINO_OK;
}

domino_status check_layer_desc(const domino_layer_desc* d) {
  if (!d) return fail(DOMINO_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 0 || d->seq < 0 || d->hidden < 0 || d->heads < 0 || d->ffn_shard < 0)
    return fail(DOMINO_ERR_SHAPE, "negative size");
  if (d->act != DOMINO_ACT_GELU_TANH && d->act != DOMINO_ACT_SWIGLU) return fail(DOMINO_ERR_INVALID_ARG, "bad act");
  if (d->head_dim != 128) return fail(DOMINO_ERR_UNSUPPORTED, "head_dim must be 128");
  if (d->row_chunks < 1 || d->row_chunks > kMaxChunks) return fail(DOMINO_ERR_SHAPE, "bad row_chunks");
  if (d->batch % d->row_chunks) return fail(DOMINO_ERR_SHAPE, "batch % row_chunks != 0");
  if (d->n_partials < 1 || d->n_partials > DOMINO_MAX_PARTIALS) return fail(DOMINO_ERR_INVALID_ARG, "bad n_partials");
  if (d->layers < 1) return fail(DOMINO_ERR_INVALID_ARG, "layers must be >= 1");
  if (d->hidden % 8 || d->ffn_shard % 8) return fail(DOMINO_ERR_ALIGN, "hidden and ffn_shard must be multiples of 8");
  if (d->hidden > 8192) return fail(DOMINO_ERR_UNSUPPORTED, "hidden above 8192");
  if (!(d->p_drop >= 0.0f && d->p_drop < 1.0f)) return fail(DOMINO_ERR_INVALID_ARG, "p_drop must be in [0, 1)");
  if (!(d->eps > 0.0f)) return fail(DOMINO_ERR_INVALID_ARG, "eps must be > 0");
  if (d->reserved != 0) return fail(DOMINO_ERR_INVALID_ARG, "reserved must be 0");
  return DOMINO_OK;
}

domino_status check_layer_ptrs(const domino_layer_desc* d, const domino_layer_params* prm, const domino_layer_acts* act,
                               const void* X, const void* out) {
  if (!prm || !act) return fail(DOMINO_ERR_INVALID_ARG, "params or acts is NULL");
  domino_status st;
  if ((st = check_ptr(X, "X", true)) || (st = check_ptr(out, "out", true))) return st;
  for (int l = 0; l < d->layers; ++l) {
    const domino_layer_params& p = prm[l];
    const domino_layer_acts& a = act[l];
    const std::string L = "layer " + std::to_string(l) + ": ";
    auto need = [&](const void* q, const char* n, bool req) { return check_ptr(q, (L + n).c_str(), req); };
    const bool P = d->n_partials > 1;
    if ((st = need(p.ln1_gamma, "ln1_gamma", true)) || (st = need(p.ln1_beta, "ln1_beta", p.ln1_beta)) ||
        (st = need(p.A_qkv_s, "A_qkv_s", true)) || (st = need(p.B_o_s, "B_o_s", true)) ||
        (st = need(p.b_o, "b_o", p.b_o)) || (st = need(p.ln2_gamma, "ln2_gamma", true)) ||
        (st = need(p.ln2_beta, "ln2_beta", p.ln2_beta)) || (st = need(p.A_s, "A_s", true)) ||
        (st = need(p.B_s, "B_s", true)) || (st = need(p.b_2, "b_2", p.b_2)) || (st = check_keep(p.keep_attn)) ||
        (st = need(p.b_qkv, "b_qkv", p.b_qkv)) || (st = need(p.b_1, "b_1", p.b_1)) ||
        (st = check_keep(p.keep_mlp)) || (st = need(a.x_in, "x_in", l > 0)) || (st = need(a.ln1, "ln1", true)) ||
        (st = need(a.mean1, "mean1", true)) || (st = need(a.rstd1, "rstd1", true)) || (st = need(a.QKV, "QKV", true)) ||
        (st = need(a.O, "O", true)) || (st = need(a.lse, "lse", a.lse)) ||
        (st = need(a.y_attn_own, "y_attn_own", true)) || (st = need(a.y_attn, "y_attn", true)) ||
        (st = check_peers(a.peer_y_attn, d->n_partials, (L + "peer_y_attn").c_str(), P)) ||
        (st = need(a.h, "h", true)) || (st = need(a.ln2, "ln2", true)) || (st = need(a.mean2, "mean2", true)) ||
        (st = need(a.rstd2, "rstd2", true)) || (st = need(a.Hpre, "Hpre", true)) || (st = need(a.H, "H", true)) ||
        (st = need(a.y_mlp_own, "y_mlp_own", true)) || (st = need(a.y_mlp, "y_mlp", true)) ||
        (st = check_peers(a.peer_y_mlp, d->n_partials, (L + "peer_y_mlp").c_str(), P)))
      return st;
  }
  return DOMINO_OK;
}

hipError_t hip_ok(hipError_t e, std::string* msg, const char* what) {
  if (e != hipSuccess) *msg = std::string(what) + ": " + hipGetErrorString(e);
  return e;
}

size_t esize(int dtype) { return dtype == DOMINO_BF16 ? 2 : 4; }

// Reduction of one chunk [rows × cols] at element offset `off` of [·, ld] buffers.
hipError_t reduce_chunk(void* out, const void* own, const void* const* peers, int n_partials, int64_t ld, int64_t off,
                        int64_t rows, int64_t cols, int dtype, hipStream_t s) {
  ReduceArgs ra{};
  const size_t es = esize(dtype);
  ra.out = static_cast<char*>(out) + off * es;
  ra.ld_out = ld;
  ra.partials[0] = static_cast<const char*>(own) + off * es;
  for (int p = 1; p < n_partials; ++p) ra.partials[p] = static_cast<const char*>(peers[p - 1]) + off * es;
  ra.n_partials = n_partials;
  ra.ld_in = ld;
  ra.rows = rows;
  ra.cols = cols;
  ra.bf16 = dtype == DOMINO_BF16;
  return timed(DOMINO_K_REDUCE, s, [&] { return launch_shard_reduce(ra, s); });
}

// The reduction step of the schedule: after the chunk's products on `cs`, reduce it on
// `rs` (inline if rs == cs).
struct Sched {
  hipStream_t cs, rs;
  bool overlap;
  EventSet* ev;
  int next_event = 0;
  bool any_reduce = false;
  hipError_t reduce(void* out, const void* own, const void* const* peers, int n_partials, int64_t ld, int64_t off,
                    int64_t rows, int64_t cols, int dtype) {
    hipError_t e = hipSuccess;
    if (overlap) {
      hipEvent_t done = ev->done[next_event++ % kMaxChunks];
      e = hipEventRecord(done, cs);
      if (e == hipSuccess) e = hipStreamWaitEvent(rs, done, 0);
    }
    if (e == hipSuccess) e = reduce_chunk(out, own, peers, n_partials, ld, off, rows, cols, dtype, rs);
    any_reduce = true;
    return e;
  }
  hipError_t join() {
    if (!overlap || !any_reduce) return hipSuccess;
    hipError_t e = hipEventRecord(ev->reduced, rs);
    if (e == hipSuccess) e = hipStreamWaitEvent(cs, ev->reduced, 0);
    return e;
  }
};

domino_status make_sched(hipStream_t compute, hipStream_t comm, Sched* s) {
  s->cs = compute;
  s->rs = (comm && comm != compute) ? comm : compute;
  s->overlap = s->rs != s->cs;
  s->ev = nullptr;
  if (s->overlap) {
    std::string msg;
    if (hip_ok(events_for_current_device(&s->ev), &msg, "event setup") != hipSuccess)
      return fail(DOMINO_ERR_HIP, msg);
  }
  return DOMINO_OK;
}

int64_t mlp_n1(const domino_mlp_desc* d) { return d->act == DOMINO_ACT_SWIGLU ? 2 * d->ffn_shard : d->ffn_shard; }

domino_status check_mlp_desc(const domino_mlp_desc* d) {
  if (!d) return fail(DOMINO_ERR_INVALID_ARG, "desc is NULL");
  if (d->act != DOMINO_ACT_GELU_TANH && d->act != DOMINO_ACT_SWIGLU) return fail(DOMINO_ERR_INVALID_ARG, "bad act");
  if (d->dtype != DOMINO_BF16 && d->dtype != DOMINO_F32) return fail(DOMINO_ERR_INVALID_ARG, "bad dtype");
  if (d->batch < 0 || d->seq < 0 || d->hidden < 0 || d->ffn_shard < 0)
    return fail(DOMINO_ERR_SHAPE, "negative size");
  if (d->row_chunks < 1 || d->col_chunks < 1) return fail(DOMINO_ERR_SHAPE, "row_chunks and col_chunks must be >= 1");
  if (int64_t(d->row_chunks) * d->col_chunks > kMaxChunks) return fail(DOMINO_ERR_UNSUPPORTED, "too many chunks");
  if (d->n_partials < 1 || d->n_partials > DOMINO_MAX_PARTIALS)
    return fail(DOMINO_ERR_INVALID_ARG, "n_partials must be in 1..DOMINO_MAX_PARTIALS");
  if (d->batch % d->row_chunks) return fail(DOMINO_ERR_SHAPE, "batch % row_chunks != 0");
  const int64_t al = d->dtype == DOMINO_BF16 ? 8 : 4;
  if (d->hidden % (al * d->col_chunks))
    return fail(DOMINO_ERR_ALIGN, "hidden must be a multiple of col_chunks * (8 for bf16, 4 for fp32)");
  if (d->ffn_shard % al) return fail(DOMINO_ERR_ALIGN, "ffn_shard must be a multiple of 8 (bf16) or 4 (fp32)");
  const int64_t T = d->batch * d->seq;
  if (T > (int64_t(1) << 31)) return fail(DOMINO_ERR_UNSUPPORTED, "more than 2^31 tokens");
  if (d->hidden > kMaxLd || mlp_n1(d) > kMaxLd)
    return fail(DOMINO_ERR_UNSUPPORTED, "hidden and the first product's width (ffn_shard, 2*ffn_shard for SwiGLU) "
                                        "must be at most 2^22 (32-bit operand offsets)");
  if (T / 128 * (std::max(d->hidden, mlp_n1(d)) / 128 + 1) >= (int64_t(1) << 30))
    return fail(DOMINO_ERR_UNSUPPORTED, "too many output tiles for one launch");
  if (T * (d->hidden / al) > kReduceMaxGroups)
    return fail(DOMINO_ERR_UNSUPPORTED, "tokens * hidden beyond the reduction's 32-bit range");
  return DOMINO_OK;
}

domino_status check_attn_desc(const domino_attn_desc* d) {
  if (!d) return fail(DOMINO_ERR_INVALID_ARG, "desc is NULL");
  if (d->dtype != DOMINO_BF16) {
    if (d->dtype == DOMINO_F32) return fail(DOMINO_ERR_UNSUPPORTED, "attention is bf16 only");
    return fail(DOMINO_ERR_INVALID_ARG, "bad dtype");
  }
  if (d->batch < 0 || d->seq < 0 || d->hidden < 0 || d->heads < 0) return fail(DOMINO_ERR_SHAPE, "negative size");
  if (d->head_dim != 128) return fail(DOMINO_ERR_UNSUPPORTED, "head_dim must be 128");
  if (d->row_chunks < 1 || d->row_chunks > kMaxChunks) return fail(DOMINO_ERR_SHAPE, "bad row_chunks");
  if (d->batch % d->row_chunks) return fail(DOMINO_ERR_SHAPE, "batch % row_chunks != 0");
  if (d->n_partials < 1 || d->n_partials > DOMINO_MAX_PARTIALS)
    return fail(DOMINO_ERR_INVALID_ARG, "n_partials must be in 1..DOMINO_MAX_PARTIALS");
  if (d->hidden % 8) return fail(DOMINO_ERR_ALIGN, "hidden must be a multiple of 8");
  if (!(d->scale >= 0.0f)) return fail(DOMINO_ERR_INVALID_ARG, "scale must be >= 0 (0 selects 1/sqrt(head_dim))");
  const int64_t T = d->batch * d->seq;
  if (T > (int64_t(1) << 31) || d->seq > (int64_t(1) << 30)) return fail(DOMINO_ERR_UNSUPPORTED, "too many tokens");
  if (d->hidden > kMaxLd || 3 * d->heads * d->head_dim > kMaxLd)
    return fail(DOMINO_ERR_UNSUPPORTED, "hidden and 3*heads*head_dim must be at most 2^22 (32-bit operand offsets)");
  if (T / 128 * (std::max(d->hidden, 3 * d->heads * d->head_dim) / 128 + 1) >= (int64_t(1) << 30))
    return fail(DOMINO_ERR_UNSUPPORTED, "too many output tiles for one launch");
  if (T * (d->hidden / 8) > kReduceMaxGroups)
    return fail(DOMINO_ERR_UNSUPPORTED, "tokens * hidden beyond the reduction's 32-bit range");
  return DOMINO_OK;
}

bool needs_reduce(int n_partials, const void* own, const void* out) { return n_partials > 1 || (out && out != own); }

// The products of each call, built from the descriptor and the caller's buffers (null
// buffers give the shapes alone, as the workspace-size queries need). Row-major buffers;
// B(k, n) of a product reads an [in, out] weight as stored, or its transpose.
GemmArgs gemm_base(int64_t M, int64_t N, int64_t K, bool bf16) {
  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.bf16 = bf16;
  return g;
}
const char* at(const void* p, int64_t elems, size_t es) { return p ? static_cast<const char*>(p) + elems * es : nullptr; }
char* at(void* p, int64_t elems, size_t es) { return p ? static_cast<char*>(p) + elems * es : nullptr; }

// Hpre = X·A_s with the activation epilogue (H = act(Hpre)), over all T rows.
GemmArgs mlp_gemm1(const domino_mlp_desc* d, const void* X, const void* A_s, void* Hpre, void* H) {
  const int64_t T = d->batch * d->seq, h = d->hidden, f = d->ffn_shard, n1 = mlp_n1(d);
  GemmArgs g = gemm_base(T, f, h, d->dtype == DOMINO_BF16);
  g.A = X; g.lda = h; g.a_kcontig = true;
  g.B = A_s; g.ldb = n1; g.b_kcontig = false;
  g.C = Hpre; g.ldc = n1;
  g.C2 = H; g.ldc2 = f;
  g.f_s = f;
  g.epi = d->act == DOMINO_ACT_SWIGLU ? Epi::kSwiglu : Epi::kGelu;
  return g;
}
// The same two products reading transposed weight copies (A_sT [n1, h], B_sT [h, f_s]),
// contiguous along k.
GemmArgs mlp_gemm1_t(const domino_mlp_desc* d, const void* X, const void* A_sT, void* Hpre, void* H) {
  GemmArgs g = mlp_gemm1(d, X, A_sT, Hpre, H);
  g.ldb = d->hidden; g.b_kcontig = true;
  return g;
}
GemmArgs mlp_gemm2_t(const domino_mlp_desc* d, const void* H, const void* B_sT, void* Y_own, int i, int j) {
  const int64_t h = d->hidden, f = d->ffn_shard, Tc = (d->batch / d->row_chunks) * d->seq, hc = h / d->col_chunks;
  GemmArgs g = gemm_base(Tc, hc, f, true);
  g.A = at(H, i * Tc * f, 2); g.lda = f; g.a_kcontig = true;
  g.B = at(B_sT, j * hc * f, 2); g.ldb = f; g.b_kcontig = true;
  g.C = at(Y_own, i * Tc * h + j * hc, 2); g.ldc = h;
  g.epi = Epi::kStore;
  return g;
}
// Bytes of the transposed weight copies at the front of the forward's workspace.
size_t mlp_wt_bytes(const domino_mlp_desc* d) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  return up(size_t(mlp_n1(d)) * d->hidden * 2) + up(size_t(d->ffn_shard) * d->hidden * 2);
}
// Y_own chunk (i, j) = H[rows_i]·B_s[:, cols_j].
GemmArgs mlp_gemm2(const domino_mlp_desc* d, const void* H, const void* B_s, void* Y_own, int i, int j) {
  const int64_t h = d->hidden, f = d->ffn_shard, Tc = (d->batch / d->row_chunks) * d->seq, hc = h / d->col_chunks;
  const size_t es = esize(d->dtype);
  GemmArgs g = gemm_base(Tc, hc, f, d->dtype == DOMINO_BF16);
  g.A = at(H, i * Tc * f, es); g.lda = f; g.a_kcontig = true;
  g.B = at(B_s, j * hc, es); g.ldb = h; g.b_kcontig = false;
  g.C = at(Y_own, i * Tc * h + j * hc, es); g.ldc = h;
  g.epi = Epi::kStore;
  return g;
}
// dX chunks: row chunks when rows are split (row or 2D split), else the column chunks.
void mlp_dx_chunks(const domino_mlp_desc* d, int* rch, int* cch) {
  *rch = d->row_chunks;
  *cch = d->row_chunks > 1 ? 1 : d->col_chunks;
}
// dHpre = (dY·B_sᵀ) ⊙ act'(Hpre), over all T rows.
GemmArgs mlp_dgrad_b(const domino_mlp_desc* d, const void* dY, const void* B_s, void* dHpre, const void* Hpre) {
  const int64_t T = d->batch * d->seq, h = d->hidden, f = d->ffn_shard, n1 = mlp_n1(d);
  GemmArgs g = gemm_base(T, f, h, d->dtype == DOMINO_BF16);
  g.A = dY; g.lda = h; g.a_kcontig = true;
  g.B = B_s; g.ldb = h; g.b_kcontig = true;  // B(k, n) = B_s[n][k]
  g.C = dHpre; g.ldc = n1;
  g.aux = Hpre; g.ldaux = n1;
  g.f_s = f;
  g.epi = d->act == DOMINO_ACT_SWIGLU ? Epi::kDSwiglu : Epi::kDGelu;
  return g;
}
// dX_own chunk (i, j) = dHpre[rows_i]·A_s[cols_j, :]ᵀ.
GemmArgs mlp_dgrad_a(const domino_mlp_desc* d, const void* dHpre, const void* A_s, void* dX_own, int i, int j) {
  int rch, cch;
  mlp_dx_chunks(d, &rch, &cch);
  const int64_t h = d->hidden, n1 = mlp_n1(d), Tc = (d->batch / rch) * d->seq, hc = h / cch;
  const size_t es = esize(d->dtype);
  GemmArgs g = gemm_base(Tc, hc, n1, d->dtype == DOMINO_BF16);
  g.A = at(dHpre, i * Tc * n1, es); g.lda = n1; g.a_kcontig = true;
  g.B = at(A_s, j * hc * n1, es); g.ldb = n1; g.b_kcontig = true;  // B(k, n) = A_s[n][k]
  g.C = at(dX_own, i * Tc * h + j * hc, es); g.ldc = h;
  g.epi = Epi::kStore;
  return g;
}
// dB_s (+)= Hᵀ·dY in fp32.
GemmArgs mlp_wgrad_b(const domino_mlp_desc* d, const void* H, const void* dY, float* dB_s, int accumulate) {
  const int64_t T = d->batch * d->seq, h = d->hidden, f = d->ffn_shard;
  GemmArgs g = gemm_base(f, h, T, d->dtype == DOMINO_BF16);
  g.A = H; g.lda = f; g.a_kcontig = false;   // A(m, k) = H[k][m]
  g.B = dY; g.ldb = h; g.b_kcontig = false;  // B(k, n) = dY[k][n]
  g.C = dB_s; g.ldc = h;
  g.epi = Epi::kF32;
  g.accumulate = accumulate;
  return g;
}
// dA_s (+)= Xᵀ·dHpre in fp32.
GemmArgs mlp_wgrad_a(const domino_mlp_desc* d, const void* X, const void* dHpre, float* dA_s, int accumulate) {
  const int64_t T = d->batch * d->seq, h = d->hidden, n1 = mlp_n1(d);
  GemmArgs g = gemm_base(h, n1, T, d->dtype == DOMINO_BF16);
  g.A = X; g.lda = h; g.a_kcontig = false;      // A(m, k) = X[k][m]
  g.B = dHpre; g.ldb = n1; g.b_kcontig = false;  // B(k, n) = dHpre[k][n]
  g.C = dA_s; g.ldc = n1;
  g.epi = Epi::kF32;
  g.accumulate = accumulate;
  return g;
}
// QKV = X·A_qkv_s over all T rows.
GemmArgs attn_qkv(const domino_attn_desc* d, const void* X, const void* A_qkv_s, void* QKV) {
  const int64_t T = d->batch * d->seq, h = d->hidden, hd = d->heads * d->head_dim;
  GemmArgs g = gemm_base(T, 3 * hd, h, true);
  g.A = X; g.lda = h; g.a_kcontig = true;
  g.B = A_qkv_s; g.ldb = 3 * hd; g.b_kcontig = false;
  g.C = QKV; g.ldc = 3 * hd;
  g.epi = Epi::kStore;
  return g;
}
// Y_own chunk i = O[rows_i]·B_o_s.
GemmArgs attn_out(const domino_attn_desc* d, const void* O, const void* B_o_s, void* Y_own, int i) {
  const int64_t h = d->hidden, hd = d->heads * d->head_dim, Tc = (d->batch / d->row_chunks) * d->seq;
  GemmArgs g = gemm_base(Tc, h, hd, true);
  g.A = at(O, i * Tc * hd, 2); g.lda = hd; g.a_kcontig = true;
  g.B = B_o_s; g.ldb = h; g.b_kcontig = false;
  g.C = at(Y_own, i * Tc * h, 2); g.ldc = h;
  g.epi = Epi::kStore;
  return g;
}

// dO = dY·B_o_sᵀ over all rows (B_o_s [hd, h] read as [n = hd][k = h]).
GemmArgs attn_dout(const domino_attn_desc* d, const void* dY, const void* B_o_s, void* dO) {
  const int64_t T = d->batch * d->seq, h = d->hidden, hd = d->heads * d->head_dim;
  GemmArgs g = gemm_base(T, hd, h, true);
  g.A = dY; g.lda = h; g.a_kcontig = true;
  g.B = B_o_s; g.ldb = h; g.b_kcontig = true;
  g.C = dO; g.ldc = hd;
  g.epi = Epi::kStore;
  return g;
}
// dX_own chunk i = dQKV[rows_i]·A_qkv_sᵀ (A_qkv_s [h, 3hd] read as [n = h][k = 3hd]).
GemmArgs attn_dx(const domino_attn_desc* d, const void* dQKV, const void* A_qkv_s, void* dX_own, int i) {
  const int64_t h = d->hidden, hd = d->heads * d->head_dim, Tc = (d->batch / d->row_chunks) * d->seq;
  GemmArgs g = gemm_base(Tc, h, 3 * hd, true);
  g.A = at(dQKV, i * Tc * 3 * hd, 2); g.lda = 3 * hd; g.a_kcontig = true;
  g.B = A_qkv_s; g.ldb = 3 * hd; g.b_kcontig = true;
  g.C = at(dX_own, i * Tc * h, 2); g.ldc = h;
  g.epi = Epi::kStore;
  return g;
}
// dB_o_s (+)= Oᵀ·dY: [hd, h], k = tokens.
GemmArgs attn_wgrad_o(const domino_attn_desc* d, const void* O, const void* dY, float* dB_o_s, int accumulate) {
  const int64_t T = d->batch * d->seq, h = d->hidden, hd = d->heads * d->head_dim;
  GemmArgs g = gemm_base(hd, h, T, true);
  g.A = O; g.lda = hd; g.a_kcontig = false;
  g.B = dY; g.ldb = h; g.b_kcontig = false;
  g.C = dB_o_s; g.ldc = h;
  g.epi = Epi::kF32;
  g.accumulate = accumulate;
  return g;
}
// dA_qkv_s (+)= Xᵀ·dQKV: [h, 3hd], k = tokens.
GemmArgs attn_wgrad_qkv(const domino_attn_desc* d, const void* X, const void* dQKV, float* dA_qkv_s, int accumulate) {
  const int64_t T = d->batch * d->seq, h = d->hidden, hd = d->heads * d->head_dim;
  GemmArgs g = gemm_base(h, 3 * hd, T, true);
  g.A = X; g.lda = h; g.a_kcontig = false;
  g.B = dQKV; g.ldb = 3 * hd; g.b_kcontig = false;
  g.C = dA_qkv_s; g.ldc = 3 * hd;
  g.epi = Epi::kF32;
  g.accumulate = accumulate;
  return g;
}

// One product on stream s: the GEMM (timed as `kind`), then, if it split tiles along k,
// the fixed-order sum of their slices with the epilogue (timed as auxiliary work).
hipError_t run_gemm(int kind, GemmArgs g, void* ws, size_t ws_bytes, hipStream_t s) {
  g.ws = static_cast<float*>(ws);
  g.ws_elems = ws ? int64_t(ws_bytes / sizeof(float)) : 0;
  GemmSplit sp;
  hipError_t e = timed(kind, s, [&] { return launch_gemm(g, s, &sp); });
  if (e == hipSuccess && sp.pending) e = timed(DOMINO_K_AUX, s, [&] { return launch_gemm_fixup(g, sp, s); });
  return e;
}

size_t ws_bytes_of(std::initializer_list<GemmArgs> gs) {
  int64_t n = 0;
  for (const GemmArgs& g : gs) n = std::max(n, gemm_ws_elems(g));
  return size_t(n) * sizeof(float);
}

// Folds the pending event pairs into the per-kind sums (caller holds g_timing_mu).
domino_status timing_collect() {
  for (auto& r : g_timing_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      return fail(DOMINO_ERR_HIP, "timing event query failed");
    g_timing_ms[r.kind] += ms;
    g_timing_n[r.kind] += 1;
    if (!r.kernel.empty()) g_timing_kernel[r.kind] = r.kernel;
    g_timing_free.push_back(r.a);
    g_timing_free.push_back(r.b);
  }
  g_timing_recs.clear();
  return DOMINO_OK;
}

}  // namespace

void domino::note_kernel(const char* name) { t_kernel = name; }

extern "C" {

const char* domino_status_string(domino_status st) {
  switch (st) {
    case DOMINO_OK: return "DOMINO_OK";
    case DOMINO_ERR_INVALID_ARG: return "DOMINO_ERR_INVALID_ARG";
    case DOMINO_ERR_SHAPE: return "DOMINO_ERR_SHAPE";
    case DOMINO_ERR_ALIGN: return "DOMINO_ERR_ALIGN";
    case DOMINO_ERR_UNSUPPORTED: return "DOMINO_ERR_UNSUPPORTED";
    case DOMINO_ERR_HIP: return "DOMINO_ERR_HIP";
  }
  return "DOMINO_ERR_UNKNOWN";
}

const char* domino_last_error(void) { return t_last_error.c_str(); }

domino_status shard_reduce(void* out, int64_t ld_out, const void* const* partials, int32_t n_partials, int64_t ld_in,
                           int64_t rows, int64_t cols, int32_t dtype, hipStream_t stream) {
  t_last_error.clear();
  if (dtype != DOMINO_BF16 && dtype != DOMINO_F32) return fail(DOMINO_ERR_INVALID_ARG, "bad dtype");
  if (n_partials < 1 || n_partials > DOMINO_MAX_PARTIALS)
    return fail(DOMINO_ERR_INVALID_ARG, "n_partials must be in 1..DOMINO_MAX_PARTIALS");
  if (rows < 0 || cols < 0) return fail(DOMINO_ERR_SHAPE, "negative size");
  if (rows == 0 || cols == 0) return DOMINO_OK;
  if (!partials) return fail(DOMINO_ERR_INVALID_ARG, "partials is NULL");
  const int64_t al = dtype == DOMINO_BF16 ? 8 : 4;
  if (cols % al || ld_in % al || ld_out % al)
    return fail(DOMINO_ERR_ALIGN, "cols and leading dimensions must be multiples of 8 (bf16) / 4 (fp32)");
  if (ld_in < cols || ld_out < cols) return fail(DOMINO_ERR_SHAPE, "leading dimension smaller than cols");
  if (rows > kReduceMaxGroups || rows * (cols / al) > kReduceMaxGroups)
    return fail(DOMINO_ERR_UNSUPPORTED, "region too large: rows * cols / (8 bf16, 4 fp32) must be at most 2^32 - 2^21");
  domino_status st = check_ptr(out, "out", true);
  if (st != DOMINO_OK) return st;
  for (int p = 0; p < n_partials; ++p) {
    const std::string nm = "partials[" + std::to_string(p) + "]";
    st = check_ptr(partials[p], nm.c_str(), true);
    if (st != DOMINO_OK) return st;
    if (partials[p] == out && ld_in != ld_out)
      return fail(DOMINO_ERR_INVALID_ARG, "out aliases a partial with a different leading dimension");
  }
  ReduceArgs ra{};
  ra.out = out;
  ra.ld_out = ld_out;
  for (int p = 0; p < n_partials; ++p) ra.partials[p] = partials[p];
  ra.n_partials = n_partials;
  ra.ld_in = ld_in;
  ra.rows = rows;
  ra.cols = cols;
  ra.bf16 = dtype == DOMINO_BF16;
  std::string msg;
  if (hip_ok(timed(DOMINO_K_REDUCE, stream, [&] { return launch_shard_reduce(ra, stream); }), &msg, "shard_reduce") !=
      hipSuccess)
    return fail(DOMINO_ERR_HIP, msg);
  return DOMINO_OK;
}

}  // extern "C"
namespace {
// Whether the forward transposes the weights (bf16, and the first product then runs on
// the eight-wave kernel, which takes the activations' k-contiguous weight operand).
bool mlp_fwd_transposed(const domino_mlp_desc* d) {
  return d->dtype == DOMINO_BF16 && d->ffn_shard > 0 && d->batch * d->seq > 0 &&
         use_gemm8(mlp_gemm1_t(d, nullptr, nullptr, nullptr, nullptr));
}
size_t mlp_fwd_ws_plain(const domino_mlp_desc* d) {
  return ws_bytes_of({mlp_gemm1(d, nullptr, nullptr, nullptr, nullptr), mlp_gemm2(d, nullptr, nullptr, nullptr, 0, 0)});
}
size_t mlp_fwd_ws_transposed(const domino_mlp_desc* d) {
  return mlp_wt_bytes(d) + ws_bytes_of({mlp_gemm1_t(d, nullptr, nullptr, nullptr, nullptr),
                                        mlp_gemm2_t(d, nullptr, nullptr, nullptr, 0, 0)});
}
}  // namespace
extern "C" {

size_t domino_block_fwd_workspace_size(const domino_mlp_desc* d) {
  if (check_mlp_desc(d) != DOMINO_OK) return 0;
  const size_t plain = mlp_fwd_ws_plain(d);
  return mlp_fwd_transposed(d) ? std::max(plain, mlp_fwd_ws_transposed(d)) : plain;
}

domino_status domino_block_fwd(const domino_mlp_desc* d, const void* X, const void* A_s, const void* B_s,
                               const void* b1_s, void* Hpre, void* H, void* Y_own, const void* const* peer_Y, void* Y,
                               void* workspace, size_t workspace_bytes, hipStream_t compute, hipStream_t comm) {
  t_last_error.clear();
  domino_status st = check_mlp_desc(d);
  if (st != DOMINO_OK) return st;
  const int64_t T = d->batch * d->seq, h = d->hidden, f = d->ffn_shard;
  if (T == 0 || h == 0) return DOMINO_OK;
  const bool red = needs_reduce(d->n_partials, Y_own, Y);
  if ((st = check_ptr(X, "X", true)) || (st = check_ptr(A_s, "A_s", f > 0)) || (st = check_ptr(B_s, "B_s", f > 0)) ||
      (st = check_ptr(b1_s, "b1_s", f > 0 && b1_s)) ||
      (st = check_ptr(Hpre, "Hpre", f > 0)) || (st = check_ptr(H, "H", f > 0)) || (st = check_ptr(Y_own, "Y_own", true)) ||
      (st = check_peers(peer_Y, d->n_partials, "peer_Y", red)) || (st = check_ptr(Y ? Y : Y_own, "Y", red)))
    return st;
  if (b1_s && d->dtype != DOMINO_BF16) return fail(DOMINO_ERR_UNSUPPORTED, "b1_s needs bf16");
  if (workspace && !aligned16(workspace)) return fail(DOMINO_ERR_ALIGN, "workspace is not 16-byte aligned");
  Sched sc;
  if ((st = make_sched(compute, comm, &sc)) != DOMINO_OK) return st;

  const int64_t Tc = (d->batch / d->row_chunks) * d->seq, hc = h / d->col_chunks;
  std::string msg;
  // With room in the workspace (bf16), the weights are first copied transposed to its
  // front, so both products read them contiguous along k; the rest of the workspace serves
  // the products' k-split slices.
  const bool tw = workspace && mlp_fwd_transposed(d) && workspace_bytes >= mlp_fwd_ws_transposed(d);
  const size_t wt = tw ? mlp_wt_bytes(d) : 0;
  void* const A_sT = workspace;
  void* const B_sT = tw ? at(workspace, int64_t((size_t(mlp_n1(d)) * h * 2 + 255) / 256 * 256), 1) : nullptr;
  void* const ws = tw ? at(workspace, int64_t(wt), 1) : workspace;
  const size_t ws_bytes = workspace_bytes - wt;
  if (tw && hip_ok(timed(DOMINO_K_AUX, sc.cs, [&] {
                     hipError_t e = launch_transpose_bf16(A_s, mlp_n1(d), A_sT, h, h, mlp_n1(d), sc.cs);
                     return e == hipSuccess ? launch_transpose_bf16(B_s, h, B_sT, f, f, h, sc.cs) : e;
                   }), &msg, "weight transposes"))
    return fail(DOMINO_ERR_HIP, msg);
  GemmArgs g1 = tw ? mlp_gemm1_t(d, X, A_sT, Hpre, H) : mlp_gemm1(d, X, A_s, Hpre, H);
  g1.bias = b1_s;
  // The first product (column-parallel, activation fused) feeds no reduction, so it runs
  // once over all rows: chunking it would only narrow the GEMM. The second product is
  // launched per Domino chunk, and each chunk's reduction starts as soon as it ends.
  if (f > 0 && hip_ok(run_gemm(DOMINO_K_FWD_GEMM1, g1, ws, ws_bytes, sc.cs), &msg, "GEMM1"))
    return fail(DOMINO_ERR_HIP, msg);
  for (int i = 0; i < d->row_chunks; ++i) {
    for (int j = 0; j < d->col_chunks; ++j) {
      const GemmArgs g2 = tw ? mlp_gemm2_t(d, H, B_sT, Y_own, i, j) : mlp_gemm2(d, H, B_s, Y_own, i, j);
      if (hip_ok(run_gemm(DOMINO_K_FWD_GEMM2, g2, ws, ws_bytes, sc.cs), &msg, "GEMM2"))
        return fail(DOMINO_ERR_HIP, msg);
      if (red && hip_ok(sc.reduce(Y ? Y : Y_own, Y_own, peer_Y, d->n_partials, h, i * Tc * h + j * hc, Tc, hc, d->dtype),
                        &msg, "reduce Y"))
        return fail(DOMINO_ERR_HIP, msg);
    }
  }
  if (!d->no_join && hip_ok(sc.join(), &msg, "join")) return fail(DOMINO_ERR_HIP, msg);
  return DOMINO_OK;
}

size_t domino_block_bwd_workspace_size(const domino_mlp_desc* d) {
  if (check_mlp_desc(d) != DOMINO_OK) return 0;
  const size_t bias =  // the bias gradient (bf16 only)
      d->dtype == DOMINO_BF16 ? size_t(bias_grad_ws_floats(d->batch * d->seq, mlp_n1(d))) * sizeof(float) : 0;
  return std::max(bias, ws_bytes_of({mlp_dgrad_b(d, nullptr, nullptr, nullptr, nullptr),
                                     mlp_dgrad_a(d, nullptr, nullptr, nullptr, 0, 0),
                                     mlp_wgrad_b(d, nullptr, nullptr, nullptr, 0),
                                     mlp_wgrad_a(d, nullptr, nullptr, nullptr, 0)}));
}

domino_status domino_block_bwd(const domino_mlp_desc* d, const void* X, const void* A_s, const void* B_s,
                               const void* Hpre, const void* H, const void* dY, void* dHpre, void* dX_own,
                               const void* const* peer_dX, void* dX, float* dA_s, float* dB_s, float* d_b1_s,
                               int32_t accumulate, void* workspace, size_t workspace_bytes, hipStream_t compute,
                               hipStream_t comm) {
  t_last_error.clear();
  domino_status st = check_mlp_desc(d);
  if (st != DOMINO_OK) return st;
  const int64_t T = d->batch * d->seq, h = d->hidden, f = d->ffn_shard;
  if (h == 0) return DOMINO_OK;
  const bool red = T > 0 && needs_reduce(d->n_partials, dX_own, dX);
  const bool tok = T > 0, ffn = f > 0;
  if ((st = check_ptr(X, "X", tok && ffn)) || (st = check_ptr(A_s, "A_s", tok && ffn)) ||
      (st = check_ptr(B_s, "B_s", tok && ffn)) || (st = check_ptr(Hpre, "Hpre", tok && ffn)) ||
      (st = check_ptr(H, "H", tok && ffn)) || (st = check_ptr(dY, "dY", tok && ffn)) ||
      (st = check_ptr(dHpre, "dHpre", tok && ffn)) || (st = check_ptr(dX_own, "dX_own", tok)) ||
      (st = check_peers(peer_dX, d->n_partials, "peer_dX", red)) || (st = check_ptr(dX ? dX : dX_own, "dX", red)) ||
      (st = check_ptr(dA_s, "dA_s", ffn)) || (st = check_ptr(dB_s, "dB_s", ffn)) ||
      (st = check_ptr(d_b1_s, "d_b1_s", ffn && d_b1_s)))
    return st;
  if (workspace && !aligned16(workspace)) return fail(DOMINO_ERR_ALIGN, "workspace is not 16-byte aligned");
  if (d_b1_s && ffn) {
    if (d->dtype != DOMINO_BF16) return fail(DOMINO_ERR_UNSUPPORTED, "d_b1_s needs bf16");
    if (!workspace || workspace_bytes < size_t(bias_grad_ws_floats(T, mlp_n1(d))) * sizeof(float))
      return fail(DOMINO_ERR_INVALID_ARG, "d_b1_s needs a workspace of domino_block_bwd_workspace_size bytes");
  }
  Sched sc;
  if ((st = make_sched(compute, comm, &sc)) != DOMINO_OK) return st;

  int rch, cch;
  mlp_dx_chunks(d, &rch, &cch);
  const int64_t Tc = (d->batch / rch) * d->seq, hc = h / cch;
  std::string msg;
  // dgrad of the second layer (activation gradient fused) feeds no reduction: one launch
  // over all rows. dgrad of the first layer is launched per dX chunk, each followed by
  // its reduction; the weight gradients follow, behind the last reduction.
  if (tok && ffn &&
      hip_ok(run_gemm(DOMINO_K_DGRAD_B, mlp_dgrad_b(d, dY, B_s, dHpre, Hpre), workspace, workspace_bytes, sc.cs), &msg,
             "dgrad B"))
    return fail(DOMINO_ERR_HIP, msg);
  for (int i = 0; i < rch && tok; ++i) {
    for (int j = 0; j < cch; ++j) {
      if (hip_ok(run_gemm(DOMINO_K_DGRAD_A, mlp_dgrad_a(d, dHpre, A_s, dX_own, i, j), workspace, workspace_bytes, sc.cs),
                 &msg, "dgrad A"))
        return fail(DOMINO_ERR_HIP, msg);
      if (red && hip_ok(sc.reduce(dX ? dX : dX_own, dX_own, peer_dX, d->n_partials, h, i * Tc * h + j * hc, Tc, hc,
                                  d->dtype),
                        &msg, "reduce dX"))
        return fail(DOMINO_ERR_HIP, msg);
    }
  }
  if (ffn) {
    if (hip_ok(run_gemm(DOMINO_K_WGRAD_B, mlp_wgrad_b(d, H, dY, dB_s, accumulate), workspace, workspace_bytes, sc.cs),
               &msg, "wgrad B") ||
        hip_ok(run_gemm(DOMINO_K_WGRAD_A, mlp_wgrad_a(d, X, dHpre, dA_s, accumulate), workspace, workspace_bytes, sc.cs),
               &msg, "wgrad A"))
      return fail(DOMINO_ERR_HIP, msg);
    if (d_b1_s && hip_ok(timed(DOMINO_K_BIAS_GRAD, sc.cs, [&] {
                           return launch_bias_grad(dHpre, T, mlp_n1(d), mlp_n1(d), d_b1_s, accumulate,
                                                   static_cast<float*>(workspace), sc.cs);
                         }), &msg, "bias gradient"))
      return fail(DOMINO_ERR_HIP, msg);
  }
  if (!d->no_join && hip_ok(sc.join(), &msg, "join")) return fail(DOMINO_ERR_HIP, msg);
  return DOMINO_OK;
}

size_t domino_attn_block_fwd_workspace_size(const domino_attn_desc* d) {
  if (check_attn_desc(d) != DOMINO_OK) return 0;
  return ws_bytes_of({attn_qkv(d, nullptr, nullptr, nullptr), attn_out(d, nullptr, nullptr, nullptr, 0)});
}

domino_status domino_attn_block_fwd(const domino_attn_desc* d, const void* X, const void* A_qkv_s, const void* B_o_s,
                                    const void* b_qkv_s, void* QKV, void* O, float* lse, void* Y_own, const void* const* peer_Y, void* Y,
                                    void* workspace, size_t workspace_bytes, hipStream_t compute, hipStream_t comm) {
  t_last_error.clear();
  domino_status st = check_attn_desc(d);
  if (st != DOMINO_OK) return st;
  const int64_t T = d->batch * d->seq, h = d->hidden, hd = d->heads * d->head_dim;
  if (T == 0 || h == 0) return DOMINO_OK;
  const bool red = needs_reduce(d->n_partials, Y_own, Y);
  const bool heads = d->heads > 0;
  if ((st = check_ptr(X, "X", heads)) || (st = check_ptr(A_qkv_s, "A_qkv_s", heads)) ||
      (st = check_ptr(B_o_s, "B_o_s", heads)) || (st = check_ptr(QKV, "QKV", heads)) || (st = check_ptr(O, "O", heads)) ||
      (st = check_ptr(lse, "lse", heads && lse)) || (st = check_ptr(b_qkv_s, "b_qkv_s", heads && b_qkv_s)) ||
      (st = check_ptr(Y_own, "Y_own", true)) || (st = check_peers(peer_Y, d->n_partials, "peer_Y", red)) ||
      (st = check_ptr(Y ? Y : Y_own, "Y", red)))
    return st;
  if (workspace && !aligned16(workspace)) return fail(DOMINO_ERR_ALIGN, "workspace is not 16-byte aligned");
  Sched sc;
  if ((st = make_sched(compute, comm, &sc)) != DOMINO_OK) return st;
  const float scale = d->scale > 0.0f ? d->scale : 1.0f / sqrtf(float(d->head_dim));
  const int64_t Tc = (d->batch / d->row_chunks) * d->seq;
  std::string msg;
  // QKV projection and attention feed no reduction: one launch each over all sequences.
  // The output projection runs per chunk (whole sequences) and each chunk's reduction
  // starts as soon as it ends.
  if (heads) {
    AttnArgs aa{};
    aa.qkv = QKV; aa.ld_qkv = 3 * hd;
    aa.o = O; aa.ld_o = hd;
    aa.lse = lse; aa.ld_lse = d->heads;
    aa.batch = d->batch; aa.seq = d->seq; aa.heads = d->heads; aa.head_dim = d->head_dim;
    aa.scale = scale;
    GemmArgs gq = attn_qkv(d, X, A_qkv_s, QKV);
    gq.bias = b_qkv_s;
    if (hip_ok(run_gemm(DOMINO_K_QKV, gq, workspace, workspace_bytes, sc.cs), &msg, "QKV GEMM") ||
        hip_ok(timed(DOMINO_K_ATTN, sc.cs, [&] { return launch_attention_fwd(aa, sc.cs); }), &msg, "attention"))
      return fail(DOMINO_ERR_HIP, msg);
  }
  for (int i = 0; i < d->row_chunks; ++i) {
    if (hip_ok(run_gemm(DOMINO_K_OUTPROJ, attn_out(d, O, B_o_s, Y_own, i), workspace, workspace_bytes, sc.cs), &msg,
               "out-projection"))
      return fail(DOMINO_ERR_HIP, msg);
    if (red && hip_ok(sc.reduce(Y ? Y : Y_own, Y_own, peer_Y, d->n_partials, h, i * Tc * h, Tc, h, DOMINO_BF16), &msg,
                      "reduce Y"))
      return fail(DOMINO_ERR_HIP, msg);
  }
  if (!d->no_join && hip_ok(sc.join(), &msg, "join")) return fail(DOMINO_ERR_HIP, msg);
  return DOMINO_OK;
}

size_t domino_attn_block_bwd_workspace_size(const domino_attn_desc* d) {
  if (check_attn_desc(d) != DOMINO_OK) return 0;
  const size_t stats = size_t(attn_bwd_stats_floats(d->batch * d->seq, d->heads)) * sizeof(float);
  const size_t bias = size_t(bias_grad_ws_floats(d->batch * d->seq, 3 * d->heads * d->head_dim)) * sizeof(float);
  return std::max(std::max(stats, bias),
                  ws_bytes_of({attn_dout(d, nullptr, nullptr, nullptr), attn_dx(d, nullptr, nullptr, nullptr, 0),
                               attn_wgrad_o(d, nullptr, nullptr, nullptr, 0),
                               attn_wgrad_qkv(d, nullptr, nullptr, nullptr, 0)}));
}

domino_status domino_attn_block_bwd(const domino_attn_desc* d, const void* X, const void* A_qkv_s, const void* B_o_s,
                                    const void* QKV, const void* O, const float* lse, const void* dY, void* dO,
                                    void* dQKV, void* dX_own, const void* const* peer_dX, void* dX, float* dA_qkv_s,
                                    float* dB_o_s, float* d_b_qkv_s, int32_t accumulate, void* workspace,
                                    size_t workspace_bytes, hipStream_t compute, hipStream_t comm) {
  t_last_error.clear();
  domino_status st = check_attn_desc(d);
  if (st != DOMINO_OK) return st;
  const int64_t T = d->batch * d->seq, h = d->hidden, hd = d->heads * d->head_dim;
  if (h == 0) return DOMINO_OK;
  const bool red = T > 0 && needs_reduce(d->n_partials, dX_own, dX);
  const bool tok = T > 0, heads = d->heads > 0;
  if ((st = check_ptr(X, "X", tok && heads)) || (st = check_ptr(A_qkv_s, "A_qkv_s", tok && heads)) ||
      (st = check_ptr(B_o_s, "B_o_s", tok && heads)) || (st = check_ptr(QKV, "QKV", tok && heads)) ||
      (st = check_ptr(O, "O", tok && heads)) || (st = check_ptr(lse, "lse", tok && heads)) ||
      (st = check_ptr(dY, "dY", tok && heads)) || (st = check_ptr(dO, "dO", tok && heads)) ||
      (st = check_ptr(dQKV, "dQKV", tok && heads)) || (st = check_ptr(dX_own, "dX_own", tok)) ||
      (st = check_peers(peer_dX, d->n_partials, "peer_dX", red)) || (st = check_ptr(dX ? dX : dX_own, "dX", red)) ||
      (st = check_ptr(dA_qkv_s, "dA_qkv_s", heads)) || (st = check_ptr(dB_o_s, "dB_o_s", heads)) ||
      (st = check_ptr(d_b_qkv_s, "d_b_qkv_s", heads && d_b_qkv_s)))
    return st;
  if (((tok && heads) || d_b_qkv_s) && (!workspace || workspace_bytes < domino_attn_block_bwd_workspace_size(d)))
    return fail(DOMINO_ERR_INVALID_ARG, "workspace smaller than domino_attn_block_bwd_workspace_size");
  if (workspace && !aligned16(workspace)) return fail(DOMINO_ERR_ALIGN, "workspace is not 16-byte aligned");
  Sched sc;
  if ((st = make_sched(compute, comm, &sc)) != DOMINO_OK) return st;
  const float scale = d->scale > 0.0f ? d->scale : 1.0f / sqrtf(float(d->head_dim));
  const int64_t Tc = (d->batch / d->row_chunks) * d->seq;
  std::string msg;
  // dO and the attention backward feed no reduction: one launch each over all sequences
  // (the attention statistics live in the workspace until the products after it reuse it).
  // The input gradient runs per chunk (whole sequences), each followed by its reduction;
  // the weight gradients follow, behind the last reduction.
  if (tok && heads) {
    AttnBwdArgs ab{};
    ab.qkv = QKV; ab.ld_qkv = 3 * hd;
    ab.o = O; ab.dout = dO; ab.ld_o = hd;
    ab.lse = lse; ab.ld_lse = d->heads;
    ab.dqkv = dQKV; ab.ld_dqkv = 3 * hd;
    ab.stats = static_cast<float*>(workspace);
    ab.batch = d->batch; ab.seq = d->seq; ab.heads = d->heads; ab.head_dim = d->head_dim;
    ab.scale = scale;
    if (hip_ok(run_gemm(DOMINO_K_OUTPROJ_DGRAD, attn_dout(d, dY, B_o_s, dO), workspace, workspace_bytes, sc.cs), &msg,
               "dO GEMM") ||
        hip_ok(timed(DOMINO_K_ATTN_BWD_PREP, sc.cs, [&] { return launch_attention_bwd_prep(ab, sc.cs); }), &msg,
               "attention backward statistics") ||
        hip_ok(timed(DOMINO_K_ATTN_BWD, sc.cs, [&] { return launch_attention_bwd_dkdv(ab, sc.cs); }), &msg,
               "attention backward dK/dV") ||
        hip_ok(timed(DOMINO_K_ATTN_BWD_DQ, sc.cs, [&] { return launch_attention_bwd_dq(ab, sc.cs); }), &msg,
               "attention backward dQ"))
      return fail(DOMINO_ERR_HIP, msg);
  }
  for (int i = 0; i < d->row_chunks && tok; ++i) {
    // (no heads: k = 0 and the product writes zeros)
    if (hip_ok(run_gemm(DOMINO_K_QKV_DGRAD, attn_dx(d, dQKV, A_qkv_s, dX_own, i), workspace, workspace_bytes, sc.cs),
               &msg, "dX GEMM"))
      return fail(DOMINO_ERR_HIP, msg);
    if (red && hip_ok(sc.reduce(dX ? dX : dX_own, dX_own, peer_dX, d->n_partials, h, i * Tc * h, Tc, h, DOMINO_BF16),
                      &msg, "reduce dX"))
      return fail(DOMINO_ERR_HIP, msg);
  }
  // (no tokens: k = 0 and the products write zeros, or add nothing when accumulating)
  // The QKV weight gradient first: with the out-projection's first, that product's k-slice
  // sum ran beside the last reduction, ~90 instead of ~25 µs (GPT-3 6.7B block fwd+bwd 1.55
  // vs 1.47 ms).
  if (heads && (hip_ok(run_gemm(DOMINO_K_QKV_WGRAD, attn_wgrad_qkv(d, X, dQKV, dA_qkv_s, accumulate), workspace,
                                workspace_bytes, sc.cs), &msg, "dA_qkv GEMM") ||
                hip_ok(run_gemm(DOMINO_K_OUTPROJ_WGRAD, attn_wgrad_o(d, O, dY, dB_o_s, accumulate), workspace,
                                workspace_bytes, sc.cs), &msg, "dB_o GEMM")))
    return fail(DOMINO_ERR_HIP, msg);
  if (heads && d_b_qkv_s && hip_ok(timed(DOMINO_K_BIAS_GRAD, sc.cs, [&] {
                                     return launch_bias_grad(dQKV, T, 3 * hd, 3 * hd, d_b_qkv_s, accumulate,
                                                             static_cast<float*>(workspace), sc.cs);
                                   }), &msg, "bias gradient"))
    return fail(DOMINO_ERR_HIP, msg);
  if (!d->no_join && hip_ok(sc.join(), &msg, "join")) return fail(DOMINO_ERR_HIP, msg);
  return DOMINO_OK;
}

domino_status domino_resid_ln_fwd(const domino_group_desc* d, const void* resid, const void* y, const void* bias,
                                  const int32_t* keep, void* resid_out, const void* gamma, const void* beta,
                                  void* ln_out, float* mean, float* rstd, hipStream_t stream) {
  domino_status st = check_group_desc(d);
  if (st != DOMINO_OK) return st;
  const bool any = d->rows > 0 && d->hidden > 0;
  if ((st = check_ptr(resid, "resid", any)) || (st = check_ptr(resid_out, "resid_out", any)) ||
      (st = check_ptr(y, "y", any && y)) || (st = check_ptr(bias, "bias", any && bias)) || (st = check_keep(keep)) ||
      (st = check_ptr(gamma, "gamma", any && gamma)) || (st = check_ptr(beta, "beta", any && beta)) ||
      (st = check_ptr(ln_out, "ln_out", any && gamma)) || (st = check_ptr(mean, "mean", any && gamma)) ||
      (st = check_ptr(rstd, "rstd", any && gamma)))
    return st;
  if (!any) return DOMINO_OK;
  GroupFwdArgs a{resid, y, bias, keep, resid_out, gamma, beta, ln_out, mean, rstd, d->rows, d->hidden, d->eps,
                 d->p_drop};
  std::string msg;
  if (hip_ok(timed(DOMINO_K_GROUP_FWD, stream, [&] { return launch_resid_ln_fwd(a, stream); }), &msg, "group"))
    return fail(DOMINO_ERR_HIP, msg);
  return DOMINO_OK;
}

size_t domino_resid_ln_bwd_workspace_size(const domino_group_desc* d) {
  if (!d || d->rows <= 0 || d->hidden <= 0) return 0;
  return size_t(3 * group_bwd_blocks(d->rows) * d->hidden) * sizeof(float);
}

domino_status domino_resid_ln_bwd(const domino_group_desc* d, const void* d_ln, const void* d_res,
                                  const void* resid_out, const float* mean, const float* rstd, const void* gamma,
                                  const int32_t* keep, void* d_resid, void* d_y, float* d_gamma, float* d_beta,
                                  float* d_bias, int32_t accumulate, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  domino_status st = check_group_desc(d);
  if (st != DOMINO_OK) return st;
  const bool any = d->rows > 0 && d->hidden > 0, ln = d_ln != nullptr;
  if ((st = check_ptr(d_ln, "d_ln", any && ln)) || (st = check_ptr(d_res, "d_res", any && d_res)) ||
      (st = check_ptr(resid_out, "resid_out", any && ln)) || (st = check_ptr(mean, "mean", any && ln)) ||
      (st = check_ptr(rstd, "rstd", any && ln)) || (st = check_ptr(gamma, "gamma", any && ln)) ||
      (st = check_keep(keep)) || (st = check_ptr(d_resid, "d_resid", any)) ||
      (st = check_ptr(d_y, "d_y", any && d_y)) || (st = check_ptr(d_gamma, "d_gamma", d->hidden > 0 && d_gamma)) ||
      (st = check_ptr(d_beta, "d_beta", d->hidden > 0 && d_beta)) ||
      (st = check_ptr(d_bias, "d_bias", d->hidden > 0 && d_bias)))
    return st;
  if (!ln && (d_gamma || d_beta)) return fail(DOMINO_ERR_INVALID_ARG, "d_gamma/d_beta need d_ln");
  if (!any) return DOMINO_OK;
  if (!workspace || workspace_bytes < domino_resid_ln_bwd_workspace_size(d))
    return fail(DOMINO_ERR_INVALID_ARG, "workspace smaller than domino_resid_ln_bwd_workspace_size");
  if (!aligned16(workspace)) return fail(DOMINO_ERR_ALIGN, "workspace is not 16-byte aligned");
  GroupBwdArgs a{d_ln, d_res, resid_out, mean, rstd, gamma, keep, d_resid, d_y, d_gamma, d_beta, d_bias,
                 accumulate ? 1 : 0, static_cast<float*>(workspace), d->rows, d->hidden, d->p_drop};
  std::string msg;
  if (hip_ok(timed(DOMINO_K_GROUP_BWD, stream, [&] { return launch_resid_ln_bwd(a, stream); }), &msg, "group backward"))
    return fail(DOMINO_ERR_HIP, msg);
  return DOMINO_OK;
}

domino_status domino_stack_fwd(const domino_layer_desc* d, const void* X, const domino_layer_params* prm,
                               const domino_layer_acts* act, void* out, void* workspace, size_t workspace_bytes,
                               hipStream_t compute, hipStream_t comm) {
  t_last_error.clear();
  domino_status st = check_layer_desc(d);
  if (st != DOMINO_OK) return st;
  const int64_t T = d->batch * d->seq, h = d->hidden, hd = d->heads * d->head_dim, f = d->ffn_shard;
  const int64_t n1 = d->act == DOMINO_ACT_SWIGLU ? 2 * f : f;
  if (T == 0 || h == 0) return DOMINO_OK;
  if (d->heads == 0 || f == 0) return fail(DOMINO_ERR_UNSUPPORTED, "a layer needs heads > 0 and ffn_shard > 0");
  if ((st = check_layer_ptrs(d, prm, act, X, out))) return st;
  if (workspace && !aligned16(workspace)) return fail(DOMINO_ERR_ALIGN, "workspace is not 16-byte aligned");
  Sched sc;
  if ((st = make_sched(compute, comm, &sc)) != DOMINO_OK) return st;
  const int rc = d->row_chunks, P = d->n_partials;
  const int64_t Tc = (d->batch / rc) * d->seq, kw = (h + 31) / 32;
  const float scale = d->scale > 0.0f ? d->scale : 1.0f / sqrtf(float(d->head_dim));
  // One μ-batch as a problem of its own: batch / row_chunks whole sequences.
  domino_attn_desc ad{d->batch / rc, d->seq, h, d->heads, d->head_dim, scale, DOMINO_BF16, 1, P, 1};
  domino_mlp_desc md{d->batch / rc, d->seq, h, f, d->act, DOMINO_BF16, 1, 1, P, 1};
  std::string msg;
  hipError_t e = hipSuccess;
  auto ok = [&](hipError_t r, const char* what) {
    if (e == hipSuccess && r != hipSuccess) e = hip_ok(r, &msg, what);
    return e == hipSuccess;
  };
  auto group = [&](const void* resid, const void* y, const void* bias, const int32_t* keep, void* r_out,
                   const void* g, const void* b, void* ln, float* mean, float* rstd, int64_t r0) {
    GroupFwdArgs ga{at(resid, r0 * h, 2), at(y, r0 * h, 2), bias, keep ? keep + r0 * kw : nullptr, at(r_out, r0 * h, 2),
                    g, b, at(ln, r0 * h, 2), mean ? mean + r0 : nullptr, rstd ? rstd + r0 : nullptr, Tc, h, d->eps,
                    d->p_drop};
    return timed(DOMINO_K_GROUP_FWD, sc.cs, [&] { return launch_resid_ln_fwd(ga, sc.cs); });
  };
  // The μ-batch's reduction on the second stream, and an event the compute stream waits on
  // (nothing when P = 1 and the reduced buffer is the own partial).
  auto reduce = [&](void* y, const void* own, const void* const* peers, int kind, int mu) {
    if (!needs_reduce(P, own, y)) return hipSuccess;
    hipError_t r = sc.reduce(y, own, peers, P, h, mu * Tc * h, Tc, h, DOMINO_BF16);
    if (r == hipSuccess && sc.overlap) r = hipEventRecord(sc.ev->sub[kind][mu], sc.rs);
    return r;
  };
  auto wait = [&](const void* y, const void* own, int kind, int mu) {
    return sc.overlap && needs_reduce(P, own, y) ? hipStreamWaitEvent(sc.cs, sc.ev->sub[kind][mu], 0) : hipSuccess;
  };
  // The schedule as a sequence of blocks: per layer the attention block of each μ-batch,
  // then the MLP block of each, and after the last layer each μ-batch's closing group.
  // A block opens with its group kernel (dropout + residual + LayerNorm), which needs the
  // reduction of the block rc places earlier, then runs its products; its last product
  // (out-projection or GEMM2) starts the block's reduction. With two or more μ-batches the
  // next block's group is issued before that last product: the group is HBM-bound like
  // the reduction, and issued after it would run beside it, while the products before it
  // already gave the reduction it waits for a GEMM to hide behind.
  const int nreal = d->layers * 2 * rc, nblk = nreal + rc;
  auto open = [&](int i) {
    const int mu = i % rc;
    const int64_t r0 = mu * Tc;
    if (i >= nreal) {  // closing group of the last layer
      const domino_layer_params& q = prm[d->layers - 1];
      const domino_layer_acts& b = act[d->layers - 1];
      ok(wait(b.y_mlp, b.y_mlp_own, 1, mu), "wait for the MLP reduction") &&
          ok(group(b.h, b.y_mlp, q.b_2, q.keep_mlp, out, nullptr, nullptr, nullptr, nullptr, nullptr, r0),
             "closing group");
      return;
    }
    const int l = i / (2 * rc);
    const domino_layer_params& p = prm[l];
    const domino_layer_acts& a = act[l];
    if ((i / rc) % 2 == 0) {  // LN1, fused with the previous layer's closing group
      if (l == 0) {
        ok(group(X, nullptr, nullptr, nullptr, a.x_in && a.x_in != X ? a.x_in : nullptr, p.ln1_gamma, p.ln1_beta,
                 a.ln1, a.mean1, a.rstd1, r0), "LN1");
      } else {
        const domino_layer_params& q = prm[l - 1];
        const domino_layer_acts& b = act[l - 1];
        ok(wait(b.y_mlp, b.y_mlp_own, 1, mu), "wait for the MLP reduction") &&
            ok(group(b.h, b.y_mlp, q.b_2, q.keep_mlp, a.x_in, p.ln1_gamma, p.ln1_beta, a.ln1, a.mean1, a.rstd1, r0),
               "closing group + LN1");
      }
    } else {  // dropout + residual + LN2
      const void* x = l == 0 && !a.x_in ? X : a.x_in;
      ok(wait(a.y_attn, a.y_attn_own, 0, mu), "wait for the attention reduction") &&
          ok(group(x, a.y_attn, p.b_o, p.keep_attn, a.h, p.ln2_gamma, p.ln2_beta, a.ln2, a.mean2, a.rstd2, r0),
             "middle group");
    }
  };
  // The block's products up to (head) and from (tail) its last one.
  auto products = [&](int i, bool tail) {
    if (i >= nreal) return;
    const int l = i / (2 * rc), mu = i % rc;
    const int64_t r0 = mu * Tc;
    const domino_layer_params& p = prm[l];
    const domino_layer_acts& a = act[l];
    if ((i / rc) % 2 == 0) {
      if (!tail) {
        AttnArgs aa{};
        aa.qkv = at(a.QKV, r0 * 3 * hd, 2); aa.ld_qkv = 3 * hd;
        aa.o = at(a.O, r0 * hd, 2); aa.ld_o = hd;
        aa.lse = a.lse ? a.lse + r0 * d->heads : nullptr; aa.ld_lse = d->heads;
        aa.batch = d->batch / rc; aa.seq = d->seq; aa.heads = d->heads; aa.head_dim = d->head_dim;
        aa.scale = scale;
        GemmArgs gq = attn_qkv(&ad, at(a.ln1, r0 * h, 2), p.A_qkv_s, at(a.QKV, r0 * 3 * hd, 2));
        gq.bias = p.b_qkv;
        ok(run_gemm(DOMINO_K_QKV, gq, workspace, workspace_bytes, sc.cs), "QKV GEMM") &&
            ok(timed(DOMINO_K_ATTN, sc.cs, [&] { return launch_attention_fwd(aa, sc.cs); }), "attention");
      } else {
        ok(run_gemm(DOMINO_K_OUTPROJ, attn_out(&ad, at(a.O, r0 * hd, 2), p.B_o_s, at(a.y_attn_own, r0 * h, 2), 0),
                    workspace, workspace_bytes, sc.cs), "out-projection") &&
            ok(reduce(a.y_attn, a.y_attn_own, a.peer_y_attn, 0, mu), "reduce attention");
      }
    } else {
      if (!tail) {
        GemmArgs g1 = mlp_gemm1(&md, at(a.ln2, r0 * h, 2), p.A_s, at(a.Hpre, r0 * n1, 2), at(a.H, r0 * f, 2));
        g1.bias = p.b_1;
        ok(run_gemm(DOMINO_K_FWD_GEMM1, g1, workspace, workspace_bytes, sc.cs), "GEMM1");
      } else {
        ok(run_gemm(DOMINO_K_FWD_GEMM2, mlp_gemm2(&md, at(a.H, r0 * f, 2), p.B_s, at(a.y_mlp_own, r0 * h, 2), 0, 0),
                    workspace, workspace_bytes, sc.cs), "GEMM2") &&
            ok(reduce(a.y_mlp, a.y_mlp_own, a.peer_y_mlp, 1, mu), "reduce MLP");
      }
    }
  };
  // With one μ-batch a block's group needs the reduction the previous block just started,
  // so it is issued after that block's tail.
  const bool early = rc >= 2;
  open(0);
  for (int i = 0; i < nblk && e == hipSuccess; ++i) {
    products(i, false);
    if (early && i + 1 < nblk) open(i + 1);
    products(i, true);
    if (!early && i + 1 < nblk) open(i + 1);
  }
  if (e != hipSuccess) return fail(DOMINO_ERR_HIP, msg);
  return DOMINO_OK;
}

}  // extern "C"
namespace {
// The sub-problems of the layer schedule: one μ-batch (batch / row_chunks sequences) and
// all rows (for the weight gradients).
struct LayerShapes {
  domino_attn_desc ad, ad_all;
  domino_mlp_desc md, md_all;
  float scale;
};
LayerShapes layer_shapes(const domino_layer_desc* d) {
  LayerShapes s{};
  s.scale = d->scale > 0.0f ? d->scale : 1.0f / sqrtf(float(d->head_dim));
  const int64_t b = d->batch / d->row_chunks;
  s.ad = domino_attn_desc{b, d->seq, d->hidden, d->heads, d->head_dim, s.scale, DOMINO_BF16, 1, d->n_partials, 1};
  s.ad_all = s.ad;
  s.ad_all.batch = d->batch;
  s.md = domino_mlp_desc{b, d->seq, d->hidden, d->ffn_shard, d->act, DOMINO_BF16, 1, 1, d->n_partials, 1};
  s.md_all = s.md;
  s.md_all.batch = d->batch;
  return s;
}
}  // namespace
extern "C" {

size_t domino_stack_bwd_workspace_size(const domino_layer_desc* d) {
  if (check_layer_desc(d) != DOMINO_OK || d->heads == 0 || d->ffn_shard == 0) return 0;
  const LayerShapes s = layer_shapes(d);
  const int64_t Tc = s.md.batch * d->seq;
  if (Tc == 0 || d->hidden == 0) return 0;
  const size_t stats = size_t(attn_bwd_stats_floats(Tc, d->heads)) * sizeof(float);
  const size_t part = std::max(size_t(3 * group_bwd_blocks(Tc) * d->hidden),
                               size_t(bias_grad_ws_floats(d->batch * d->seq,
                                                          std::max(3 * d->heads * d->head_dim,
                                                                   (d->act == DOMINO_ACT_SWIGLU ? 2 : 1) * d->ffn_shard)))) *
                      sizeof(float);
  const size_t gemm = ws_bytes_of({mlp_dgrad_b(&s.md, nullptr, nullptr, nullptr, nullptr),
                                   mlp_dgrad_a(&s.md, nullptr, nullptr, nullptr, 0, 0),
                                   mlp_wgrad_b(&s.md_all, nullptr, nullptr, nullptr, 0),
                                   mlp_wgrad_a(&s.md_all, nullptr, nullptr, nullptr, 0),
                                   attn_dout(&s.ad, nullptr, nullptr, nullptr), attn_dx(&s.ad, nullptr, nullptr, nullptr, 0),
                                   attn_wgrad_o(&s.ad_all, nullptr, nullptr, nullptr, 0),
                                   attn_wgrad_qkv(&s.ad_all, nullptr, nullptr, nullptr, 0)});
  return std::max(std::max(stats, part), gemm);
}

domino_status domino_stack_bwd(const domino_layer_desc* d, const void* X, const domino_layer_params* prm,
                               const domino_layer_acts* act, const domino_layer_grads* grd, const void* d_out, void* dX,
                               int32_t accumulate, void* workspace, size_t workspace_bytes, hipStream_t compute,
                               hipStream_t comm) {
  t_last_error.clear();
  domino_status st = check_layer_desc(d);
  if (st != DOMINO_OK) return st;
  const int64_t T = d->batch * d->seq, h = d->hidden, hd = d->heads * d->head_dim, f = d->ffn_shard;
  const int64_t n1 = d->act == DOMINO_ACT_SWIGLU ? 2 * f : f;
  if (T == 0 || h == 0) return DOMINO_OK;
  if (d->heads == 0 || f == 0) return fail(DOMINO_ERR_UNSUPPORTED, "a layer needs heads > 0 and ffn_shard > 0");
  if ((st = check_layer_ptrs(d, prm, act, X, d_out))) return st;
  if (!grd) return fail(DOMINO_ERR_INVALID_ARG, "grads is NULL");
  if ((st = check_ptr(dX, "dX", true))) return st;
  const bool P = d->n_partials > 1;
  for (int l = 0; l < d->layers; ++l) {
    const domino_layer_grads& g = grd[l];
    const std::string L = "layer " + std::to_string(l) + ": ";
    auto need = [&](const void* q, const char* n, bool req) { return check_ptr(q, (L + n).c_str(), req); };
    if ((st = need(g.d_ln1_gamma, "d_ln1_gamma", true)) || (st = need(g.d_ln1_beta, "d_ln1_beta", true)) ||
        (st = need(g.dA_qkv_s, "dA_qkv_s", true)) || (st = need(g.dB_o_s, "dB_o_s", true)) ||
        (st = need(g.d_b_o, "d_b_o", g.d_b_o)) || (st = need(g.d_ln2_gamma, "d_ln2_gamma", true)) ||
        (st = need(g.d_ln2_beta, "d_ln2_beta", true)) || (st = need(g.dA_s, "dA_s", true)) ||
        (st = need(g.dB_s, "dB_s", true)) || (st = need(g.d_b_2, "d_b_2", g.d_b_2)) ||
        (st = need(g.d_x_in, "d_x_in", l > 0)) || (st = need(g.d_ym, "d_ym", true)) ||
        (st = need(g.dHpre, "dHpre", true)) || (st = need(g.dx_mlp_own, "dx_mlp_own", true)) ||
        (st = check_peers(g.peer_dx_mlp, d->n_partials, (L + "peer_dx_mlp").c_str(), P)) ||
        (st = need(g.dx_mlp, "dx_mlp", true)) || (st = need(g.d_h, "d_h", true)) || (st = need(g.d_ya, "d_ya", true)) ||
        (st = need(g.dO, "dO", true)) || (st = need(g.dQKV, "dQKV", true)) ||
        (st = need(g.dx_attn_own, "dx_attn_own", true)) ||
        (st = check_peers(g.peer_dx_attn, d->n_partials, (L + "peer_dx_attn").c_str(), P)) ||
        (st = need(g.dx_attn, "dx_attn", true)) || (st = need(act[l].lse, "lse", true)) ||
        (st = need(g.d_b_qkv, "d_b_qkv", g.d_b_qkv)) || (st = need(g.d_b_1, "d_b_1", g.d_b_1)))
      return st;
  }
  if (!workspace || workspace_bytes < domino_stack_bwd_workspace_size(d))
    return fail(DOMINO_ERR_INVALID_ARG, "workspace smaller than domino_stack_bwd_workspace_size");
  if (!aligned16(workspace)) return fail(DOMINO_ERR_ALIGN, "workspace is not 16-byte aligned");
  Sched sc;
  if ((st = make_sched(compute, comm, &sc)) != DOMINO_OK) return st;
  const int rc = d->row_chunks, Pn = d->n_partials, Lk = d->layers;
  const int64_t Tc = (d->batch / rc) * d->seq, kw = (h + 31) / 32;
  const LayerShapes s = layer_shapes(d);
  std::string msg;
  hipError_t e = hipSuccess;
  auto ok = [&](hipError_t r, const char* what) {
    if (e == hipSuccess && r != hipSuccess) e = hip_ok(r, &msg, what);
    return e == hipSuccess;
  };
  // Group backward over the rows of μ-batch mu; parameter gradients accumulate over μ-batches.
  auto group = [&](const void* d_ln, const void* d_res, const void* r_out, const float* mean, const float* rstd,
                   const void* gamma, const int32_t* keep, void* d_resid, void* d_y, float* dg, float* db, float* dbias,
                   int mu) {
    const int64_t r0 = mu * Tc;
    GroupBwdArgs ga{at(d_ln, r0 * h, 2), at(d_res, r0 * h, 2), at(r_out, r0 * h, 2), mean ? mean + r0 : nullptr,
                    rstd ? rstd + r0 : nullptr, gamma, keep ? keep + r0 * kw : nullptr, at(d_resid, r0 * h, 2),
                    at(d_y, r0 * h, 2), dg, db, dbias, (accumulate || mu > 0) ? 1 : 0, static_cast<float*>(workspace),
                    Tc, h, d->p_drop};
    return timed(DOMINO_K_GROUP_BWD, sc.cs, [&] { return launch_resid_ln_bwd(ga, sc.cs); });
  };
  auto reduce = [&](void* y, const void* own, const void* const* peers, int kind, int mu) {
    if (!needs_reduce(Pn, own, y)) return hipSuccess;
    hipError_t r = sc.reduce(y, own, peers, Pn, h, mu * Tc * h, Tc, h, DOMINO_BF16);
    if (r == hipSuccess && sc.overlap) r = hipEventRecord(sc.ev->sub[kind][mu], sc.rs);
    return r;
  };
  auto wait = [&](const void* y, const void* own, int kind, int mu) {
    return sc.overlap && needs_reduce(Pn, own, y) ? hipStreamWaitEvent(sc.cs, sc.ev->sub[kind][mu], 0) : hipSuccess;
  };
  // The residual stream entering layer l and the gradient that flows out of it.
  auto x_in = [&](int l) { return l == 0 && !act[0].x_in ? X : static_cast<const void*>(act[l].x_in); };
  auto d_xin = [&](int l) { return l == 0 ? dX : grd[l].d_x_in; };
  for (int l = Lk - 1; l >= 0 && e == hipSuccess; --l) {
    const domino_layer_params& p = prm[l];
    const domino_layer_acts& a = act[l];
    const domino_layer_grads& g = grd[l];
    // Gradient of the layer's output residual: d_out, or what the layer above wrote.
    const void* d_r = l == Lk - 1 ? d_out : grd[l + 1].d_x_in;
    // Each section below issues the group kernel of μ-batch μ+1 before the last product of
    // μ-batch μ: the group is HBM-bound like the reduction that product starts, and the
    // reduction it needs was started in the previous section. With two or more μ-batches the
    // MLP section does the same with the attention section's first group (LN2 backward of
    // μ-batch 0), so the MLP's last reduction runs beside the attention backward of μ-batch 0.
    auto open_mlp = [&](int mu) {
      if (l == Lk - 1) {
        ok(group(nullptr, d_out, nullptr, nullptr, nullptr, nullptr, p.keep_mlp, nullptr, g.d_ym, nullptr, nullptr,
                 g.d_b_2, mu), "closing group backward");
      } else {
        // LN1 backward of the layer above, fused with this layer's closing dropout.
        const domino_layer_params& q = prm[l + 1];
        const domino_layer_acts& b = act[l + 1];
        const domino_layer_grads& u = grd[l + 1];
        ok(wait(u.dx_attn, u.dx_attn_own, 0, mu), "wait for the attention reduction") &&
            ok(group(u.dx_attn, u.d_h, x_in(l + 1), b.mean1, b.rstd1, q.ln1_gamma, p.keep_mlp, u.d_x_in, g.d_ym,
                     u.d_ln1_gamma, u.d_ln1_beta, g.d_b_2, mu), "LN1 backward + closing group backward");
      }
    };
    auto open_attn = [&](int mu) {
      ok(wait(g.dx_mlp, g.dx_mlp_own, 1, mu), "wait for the MLP reduction") &&
          ok(group(g.dx_mlp, d_r, a.h, a.mean2, a.rstd2, p.ln2_gamma, p.keep_attn, g.d_h, g.d_ya, g.d_ln2_gamma,
                   g.d_ln2_beta, g.d_b_o, mu), "middle group backward");
    };
    open_mlp(0);
    for (int mu = 0; mu < rc && e == hipSuccess; ++mu) {
      const int64_t r0 = mu * Tc;
      ok(run_gemm(DOMINO_K_DGRAD_B, mlp_dgrad_b(&s.md, at(g.d_ym, r0 * h, 2), p.B_s, at(g.dHpre, r0 * n1, 2),
                                                at(a.Hpre, r0 * n1, 2)), workspace, workspace_bytes, sc.cs),
         "MLP dgrad-B");
      if (mu + 1 < rc) open_mlp(mu + 1);
      else if (rc >= 2) open_attn(0);  // its reduction (μ-batch 0) was started above
      ok(run_gemm(DOMINO_K_DGRAD_A, mlp_dgrad_a(&s.md, at(g.dHpre, r0 * n1, 2), p.A_s, at(g.dx_mlp_own, r0 * h, 2), 0,
                                                0), workspace, workspace_bytes, sc.cs), "MLP dgrad-A") &&
          ok(reduce(g.dx_mlp, g.dx_mlp_own, g.peer_dx_mlp, 1, mu), "reduce MLP dX");
    }
    if (rc < 2) open_attn(0);
    for (int mu = 0; mu < rc && e == hipSuccess; ++mu) {
      const int64_t r0 = mu * Tc;
      AttnBwdArgs ab{};
      ab.qkv = at(a.QKV, r0 * 3 * hd, 2); ab.ld_qkv = 3 * hd;
      ab.o = at(a.O, r0 * hd, 2); ab.dout = at(g.dO, r0 * hd, 2); ab.ld_o = hd;
      ab.lse = a.lse + r0 * d->heads; ab.ld_lse = d->heads;
      ab.dqkv = at(g.dQKV, r0 * 3 * hd, 2); ab.ld_dqkv = 3 * hd;
      ab.stats = static_cast<float*>(workspace);
      ab.batch = s.ad.batch; ab.seq = d->seq; ab.heads = d->heads; ab.head_dim = d->head_dim;
      ab.scale = s.scale;
      ok(run_gemm(DOMINO_K_OUTPROJ_DGRAD, attn_dout(&s.ad, at(g.d_ya, r0 * h, 2), p.B_o_s, at(g.dO, r0 * hd, 2)),
                  workspace, workspace_bytes, sc.cs), "dO GEMM") &&
          ok(timed(DOMINO_K_ATTN_BWD_PREP, sc.cs, [&] { return launch_attention_bwd_prep(ab, sc.cs); }),
             "attention backward statistics") &&
          ok(timed(DOMINO_K_ATTN_BWD, sc.cs, [&] { return launch_attention_bwd_dkdv(ab, sc.cs); }),
             "attention backward dK/dV") &&
          ok(timed(DOMINO_K_ATTN_BWD_DQ, sc.cs, [&] { return launch_attention_bwd_dq(ab, sc.cs); }),
             "attention backward dQ");
      if (mu + 1 < rc) open_attn(mu + 1);
      ok(run_gemm(DOMINO_K_QKV_DGRAD, attn_dx(&s.ad, at(g.dQKV, r0 * 3 * hd, 2), p.A_qkv_s,
                                              at(g.dx_attn_own, r0 * h, 2), 0), workspace, workspace_bytes, sc.cs),
         "QKV dgrad") &&
          ok(reduce(g.dx_attn, g.dx_attn_own, g.peer_dx_attn, 0, mu), "reduce attention dX");
    }
    // The weight gradients, beside the attention's last reduction: the QKV one first (with
    // the out-projection's first, that product's k-slice sum ran beside the reduction at a
    // sixth of its speed, ~65 instead of ~10 µs: GPT-3 6.7B two-layer step 8.44 vs 8.33 ms).
    ok(run_gemm(DOMINO_K_QKV_WGRAD, attn_wgrad_qkv(&s.ad_all, a.ln1, g.dQKV, g.dA_qkv_s, accumulate), workspace,
                workspace_bytes, sc.cs), "dA_qkv GEMM") &&
        ok(run_gemm(DOMINO_K_OUTPROJ_WGRAD, attn_wgrad_o(&s.ad_all, a.O, g.d_ya, g.dB_o_s, accumulate), workspace,
                    workspace_bytes, sc.cs), "dB_o GEMM");
    if (g.d_b_qkv)
      ok(timed(DOMINO_K_BIAS_GRAD, sc.cs, [&] {
           return launch_bias_grad(g.dQKV, T, 3 * hd, 3 * hd, g.d_b_qkv, accumulate, static_cast<float*>(workspace),
                                   sc.cs);
         }), "QKV bias gradient");
    // The MLP weight gradients come last, with the attention's. Run straight after the MLP
    // input gradients, with the MLP's last reduction beside them, the second of them took
    // half as long again (a k-split product beside a reduction fares badly); beside the
    // attention backward of μ-batch 0 that reduction costs less. GPT-3 6.7B two-layer step:
    // 8.66 -> 8.44 ms, serial 8.65-8.68.
    ok(run_gemm(DOMINO_K_WGRAD_B, mlp_wgrad_b(&s.md_all, a.H, g.d_ym, g.dB_s, accumulate), workspace, workspace_bytes,
                sc.cs), "MLP dB") &&
        ok(run_gemm(DOMINO_K_WGRAD_A, mlp_wgrad_a(&s.md_all, a.ln2, g.dHpre, g.dA_s, accumulate), workspace,
                    workspace_bytes, sc.cs), "MLP dA");
    if (g.d_b_1)
      ok(timed(DOMINO_K_BIAS_GRAD, sc.cs, [&] {
           return launch_bias_grad(g.dHpre, T, n1, n1, g.d_b_1, accumulate, static_cast<float*>(workspace), sc.cs);
         }), "MLP bias gradient");
  }
  // Layer 0's LN1 backward with its residual gradient: dX.
  const domino_layer_params& p0 = prm[0];
  const domino_layer_acts& a0 = act[0];
  const domino_layer_grads& g0 = grd[0];
  for (int mu = 0; mu < rc && e == hipSuccess; ++mu)
    ok(wait(g0.dx_attn, g0.dx_attn_own, 0, mu), "wait for the attention reduction") &&
        ok(group(g0.dx_attn, g0.d_h, x_in(0), a0.mean1, a0.rstd1, p0.ln1_gamma, nullptr, d_xin(0), nullptr,
                 g0.d_ln1_gamma, g0.d_ln1_beta, nullptr, mu), "LN1 backward");
  if (e != hipSuccess) return fail(DOMINO_ERR_HIP, msg);
  return DOMINO_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------
// The allocation-free variant of domino_block_bwd, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): the workspace of the backward's k-split products is a file-scope device
// array instead of a caller buffer. Each GPU the library runs on holds its own copy of
// `scratch` until the process ends. Its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) on the first call there, and only that
// address is handed to kernels: in host code the array's name is a host-side stand-in,
// not a device pointer. Every call on a GPU shares that GPU's array; nothing in it needs
// to start at zero (the split products write every slot they read), and calls that
// overlap on one GPU race on it.
// ---------------------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = size_t(DOMINO_NOALLOC_SCRATCH_BYTES);

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of the current device's scratch array (looked up on first use).
domino_status scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DOMINO_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DOMINO_ERR_UNSUPPORTED, "device index beyond the library's table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DOMINO_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DOMINO_OK;
}

}  // namespace

extern "C" {

domino_status domino_block_bwd_noalloc(const domino_mlp_desc* d, const void* X, const void* A_s, const void* B_s,
                                       const void* Hpre, const void* H, const void* dY, void* dHpre, void* dX_own,
                                       const void* const* peer_dX, void* dX, float* dA_s, float* dB_s,
                                       float* d_b1_s, int32_t accumulate, hipStream_t compute, hipStream_t comm) {
  t_last_error.clear();
  domino_status st = check_mlp_desc(d);
  if (st != DOMINO_OK) return st;
  const size_t need = domino_block_bwd_workspace_size(d);
  if (need > kScratchBytes)
    return fail(DOMINO_ERR_UNSUPPORTED, "this shape's backward needs " + std::to_string(need) +
                                            " bytes of workspace; the static scratch holds " +
                                            std::to_string(kScratchBytes) +
                                            " (domino_block_bwd takes a caller workspace of any size)");
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != DOMINO_OK) return st;
  return domino_block_bwd(d, X, A_s, B_s, Hpre, H, dY, dHpre, dX_own, peer_dX, dX, dA_s, dB_s, d_b1_s, accumulate, ws,
                          kScratchBytes, compute, comm);
}

domino_status domino_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (auto& r : g_timing_recs) {
    g_timing_free.push_back(r.a);
    g_timing_free.push_back(r.b);
  }
  g_timing_recs.clear();
  for (int k = 0; k < DOMINO_K_COUNT; ++k) {
    g_timing_ms[k] = 0.0;
    g_timing_n[k] = 0;
    g_timing_kernel[k].clear();
  }
  g_timing = enable != 0;
  return DOMINO_OK;
}

domino_status domino_timing_read(int32_t kind, int64_t* launches, double* total_ms) {
  t_last_error.clear();
  if (kind < 0 || kind >= DOMINO_K_COUNT || !launches || !total_ms) return fail(DOMINO_ERR_INVALID_ARG, "bad argument");
  std::lock_guard<std::mutex> lk(g_timing_mu);
  domino_status st = timing_collect();
  if (st != DOMINO_OK) return st;
  *launches = g_timing_n[kind];
  *total_ms = g_timing_ms[kind];
  return DOMINO_OK;
}

domino_status domino_timing_kernel(int32_t kind, char* name, size_t capacity) {
  t_last_error.clear();
  if (kind < 0 || kind >= DOMINO_K_COUNT || !name || capacity == 0) return fail(DOMINO_ERR_INVALID_ARG, "bad argument");
  std::lock_guard<std::mutex> lk(g_timing_mu);
  domino_status st = timing_collect();
  if (st != DOMINO_OK) return st;
  const std::string& k = g_timing_kernel[kind];
  if (k.size() + 1 > capacity) return fail(DOMINO_ERR_INVALID_ARG, "name buffer too small");
  std::copy(k.c_str(), k.c_str() + k.size() + 1, name);
  return DOMINO_OK;
}

}  // extern "C"
