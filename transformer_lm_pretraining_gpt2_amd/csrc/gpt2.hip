// gpt2.hip -- host side of the library: shape checks, flat parameter layout,
// workspace plan, the kernel sequence of one training step, and the C ABI
// declared in include/gpt2.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "gpt2.h"
#include "kernels.h"

using namespace gpt2k;

namespace {

// ---------------------------------------------------------------------------
// Parameter layout.  The GPT-2 tensors ("Karpathy's four-hour GPT-2
// reproduction in one post", part 1: HF-compatible names, embedding tied to
// the output layer), 2-D tensors first so weight decay covers one prefix.
// ---------------------------------------------------------------------------
enum TensorKind { T_WTE, T_WPE, T_QKVW, T_PROJW, T_FCW, T_FCPW, T_LN1G, T_LN1B, T_QKVB, T_PROJB, T_LN2G, T_LN2B,
                  T_FCB, T_FCPB, T_LNFG, T_LNFB };

struct Tensor {
  std::string name;
  int kind, layer;
  int64_t offset;
  int rows, cols;
  int decay;
};

struct Layout {
  std::vector<Tensor> t;
  int64_t total = 0, n_decay = 0;
};

Layout make_layout(const gpt2_config_t& c) {
  Layout L;
  const int C = c.n_embd;
  auto add = [&](const char* nm, int kind, int layer, int rows, int cols) {
    Tensor x;
    x.name = layer >= 0 ? "h." + std::to_string(layer) + "." + nm : nm;
    x.kind = kind;
    x.layer = layer;
    x.offset = L.total;
    x.rows = rows;
    x.cols = cols;
    x.decay = cols > 0;
    L.total += (int64_t)rows * (cols > 0 ? cols : 1);
    if (x.decay) L.n_decay = L.total;
    L.t.push_back(x);
  };
  add("wte", T_WTE, -1, c.padded_vocab_size, C);
  add("wpe", T_WPE, -1, c.max_seq_len, C);
  for (int l = 0; l < c.n_layer; l++) {
    add("attn.c_attn.weight", T_QKVW, l, 3 * C, C);
    add("attn.c_proj.weight", T_PROJW, l, C, C);
    add("mlp.c_fc.weight", T_FCW, l, 4 * C, C);
    add("mlp.c_proj.weight", T_FCPW, l, C, 4 * C);
  }
  for (int l = 0; l < c.n_layer; l++) {
    add("ln_1.weight", T_LN1G, l, C, 0);
    add("ln_1.bias", T_LN1B, l, C, 0);
    add("attn.c_attn.bias", T_QKVB, l, 3 * C, 0);
    add("attn.c_proj.bias", T_PROJB, l, C, 0);
    add("ln_2.weight", T_LN2G, l, C, 0);
    add("ln_2.bias", T_LN2B, l, C, 0);
    add("mlp.c_fc.bias", T_FCB, l, 4 * C, 0);
    add("mlp.c_proj.bias", T_FCPB, l, C, 0);
  }
  add("ln_f.weight", T_LNFG, -1, C, 0);
  add("ln_f.bias", T_LNFB, -1, C, 0);
  return L;
}

// Widths the row kernels are instantiated for: LayerNorm keeps a row in
// registers as n_embd / 128 chunks per lane (1, 2, 3, 4, 6, 8, 12 or 16), and
// the cross-entropy row as at most 8 vectors of 8 logits per thread of a
// 1024-thread block (padded vocabulary <= 65536).
bool ln_width_ok(int C) {
  if (C <= 0 || C % 128 != 0) return false;
  switch (C / 128) {
    case 1: case 2: case 3: case 4: case 6: case 8: case 12: case 16: return true;
    default: return false;
  }
}
constexpr int kMaxPaddedVocab = 65536;

int check_config(const gpt2_config_t* c) {
  if (!c) return GPT2_ERR_ARG;
  if (c->vocab_size <= 0 || c->padded_vocab_size < c->vocab_size || c->padded_vocab_size > kMaxPaddedVocab ||
      c->padded_vocab_size % 128 != 0 || c->n_layer <= 0 || c->n_head <= 0 || c->n_embd <= 0 ||
      c->n_embd % c->n_head != 0 || !ln_width_ok(c->n_embd) || c->max_seq_len <= 0)
    return GPT2_ERR_CONFIG;
  const int hd = c->n_embd / c->n_head;
  if (hd != 32 && hd != 64) return GPT2_ERR_CONFIG;
  return GPT2_OK;
}

// FP8 forward products: bf16 base precision; the LayerNorm's fused FP8 copy
// needs a width that is a multiple of 256, and the row quantizer holds rows of
// at most 4096 values (the MLP's 4 * n_embd), so n_embd <= 1024.
bool fp8_ok(const gpt2_config_t* c, int base) {
  return base == GPT2_BF16 && c->n_embd % 256 == 0 && 4 * c->n_embd <= 4096;
}

int check_bt(const gpt2_config_t* c, int B, int T) {
  if (B <= 0 || T <= 0 || T % 64 != 0 || T > c->max_seq_len || ((int64_t)B * T) % 128 != 0 ||
      (int64_t)B * T > (1 << 26))
    return GPT2_ERR_SHAPE;
  return GPT2_OK;
}

// ---------------------------------------------------------------------------
// Workspace plan: byte offsets (256-aligned) of every device scratch array.
// ---------------------------------------------------------------------------
struct Plan {
  int64_t bytes = 0;
  // per layer
  std::vector<int64_t> x_in, x_mid, h1, h2, mean1, rstd1, mean2, rstd2, qkv, atty, lse, u, g;
  int64_t hf, meanf, rstdf, logits, loss_rows, loss_tmp;
  int64_t dres, dres_lp, dh, datty, dqkv, du, dsum, piece;
  // bf16: odd layers' du and dqkv, and LayerNorm 2's matmul copies of dres
  // (even, odd layers); fp32: aliases of du, dqkv and dres
  int64_t du2, dqkv2, lp2[2];
  // reduction partials, one buffer per producer so a whole layer's partial
  // sums can be reduced by one launch: weight kinds (qkv, proj, fc, fcproj)
  // for the split-K products and their bias column sums; LayerNorm slots
  // (final, ln_2, ln_1) for the gain/bias partials
  int64_t wpart[4], cspart[4];
  // LayerNorm partials: final, LN2 (even, odd layers), LN1 (even, odd layers)
  int64_t lnpart[5];
  // bf16: the second matmul copy of dres (odd layers' block-output gradient
  // when the weight gradients of a layer run as one grouped launch)
  int64_t dres_lp2 = -1;
  // grouped weight gradients (bf16): the split-K partials and column-sum
  // partials of a layer's four products (qkv, fc, proj, fcproj), and their
  // split counts
  int64_t gpart = -1, gcs = -1;
  int gsplit[4] = {1, 1, 1, 1};
  int64_t normpart;
  int64_t ska, sva, skb, svb, seg, nseg;
  int64_t flags, scale, norm;
  // FP8 forward products: per-output-channel FP8 copy of the weights (laid out
  // like the flat parameters) with its row scales, and one FP8 activation
  // buffer with per-row scales shared by the forward's products
  int64_t w8 = -1, wsc = -1, a8 = -1, asc = -1;
  // bf16: each layer's MLP down-projection weight transposed, [4C][C] per
  // layer, rebuilt by every training forward for the backward's GELU' product
  int64_t wt = -1;
  std::vector<int> split;  // split-K factor per layer weight kind (qkv, proj, fc, fcproj)
};


Plan make_plan(const gpt2_config_t& c, int B, int T, int prec) {
  Plan P;
  const int64_t M = (int64_t)B * T, C = c.n_embd, L = c.n_layer, NH = c.n_head;
  const bool recompute = (prec & GPT2_RECOMPUTE_GELU) != 0;
  const bool fp8 = (prec & GPT2_FP8_FWD) != 0;
  prec &= ~(GPT2_RECOMPUTE_GELU | GPT2_FP8_FWD);
  const int64_t a = prec == GPT2_BF16 ? 2 : 4;
  auto take = [&](int64_t bytes) {
    const int64_t off = P.bytes;
    P.bytes += (bytes + 255) / 256 * 256;
    return off;
  };
  for (int64_t l = 0; l <= L; l++) P.x_in.push_back(take(4 * M * C));
  for (int64_t l = 0; l < L; l++) {
    P.x_mid.push_back(take(4 * M * C));
    P.h1.push_back(take(a * M * C));
    P.h2.push_back(take(a * M * C));
    P.mean1.push_back(take(4 * M));
    P.rstd1.push_back(take(4 * M));
    P.mean2.push_back(take(4 * M));
    P.rstd2.push_back(take(4 * M));
    P.qkv.push_back(take(a * M * 3 * C));
    P.atty.push_back(take(a * M * C));
    P.lse.push_back(take(4 * M * NH));
    P.u.push_back(take(a * M * 4 * C));
    // with activation recompute the layers' GELU outputs share two buffers,
    // by layer parity (a layer's weight gradients may still read one while
    // the next layer down rebuilds the other)
    P.g.push_back(recompute && l > 1 ? P.g[l & 1] : take(a * M * 4 * C));
  }
  P.hf = take(a * M * C);
  P.meanf = take(4 * M);
  P.rstdf = take(4 * M);
  P.logits = take(a * M * c.padded_vocab_size);
  P.loss_rows = take(4 * M);
  P.loss_tmp = take(4);
  P.dres = take(4 * M * C);
  P.dres_lp = prec == GPT2_BF16 ? take(a * M * C) : P.dres;
  if (prec == GPT2_BF16) P.dres_lp2 = take(a * M * C);
  P.dh = take(a * M * C);
  P.datty = take(a * M * C);
  P.dqkv = take(a * M * 3 * C);
  P.du = take(a * M * 4 * C);
  if (prec == GPT2_BF16) {
    P.du2 = take(a * M * 4 * C);
    P.dqkv2 = take(a * M * 3 * C);
    P.lp2[0] = take(a * M * C);
    P.lp2[1] = take(a * M * C);
  } else {
    P.du2 = P.du;
    P.dqkv2 = P.dqkv;
    P.lp2[0] = P.lp2[1] = P.dres;
  }
  P.dsum = take(4 * M * NH);
  P.piece = take(4 * M * C);
  const Prec pr = prec == GPT2_BF16 ? BF16 : F32;
  const int Mi = (int)M, Ci = (int)C;
  P.split = {gemm_split_hint(pr, 1, 1, 3 * Ci, Ci, Mi), gemm_split_hint(pr, 1, 1, Ci, Ci, Mi),
             gemm_split_hint(pr, 1, 1, 4 * Ci, Ci, Mi), gemm_split_hint(pr, 1, 1, Ci, 4 * Ci, Mi)};
  const int64_t wsz[4] = {3 * C * C, C * C, 4 * C * C, 4 * C * C}, wout[4] = {3 * C, C, 4 * C, C};
  for (int k = 0; k < 4; k++) {
    P.wpart[k] = P.split[k] > 1 ? take(4 * (int64_t)P.split[k] * wsz[k]) : 0;
    P.cspart[k] = take(4 * (int64_t)P.split[k] * wout[k]);
  }
  for (int k = 0; k < 5; k++) P.lnpart[k] = take(4 * (int64_t)layernorm_bwd_parts((int)M) * 2 * C);
  if (prec == GPT2_BF16) {
    const int gt = gemm_group_tiles(3 * Ci, Ci) + gemm_group_tiles(Ci, Ci) + gemm_group_tiles(4 * Ci, Ci) +
                   gemm_group_tiles(Ci, 4 * Ci);
    // the grouped launch's problem order: qkv, fc, proj, fcproj
    const int64_t gsz[4] = {3 * C * C, 4 * C * C, C * C, 4 * C * C}, gout[4] = {3 * C, 4 * C, C, C};
    int64_t wp = 0, cp = 0;
    for (int k = 0; k < 4; k++) {
      P.gsplit[k] = gemm_group_split_hint((int)gout[k], (int)(gsz[k] / gout[k]), Mi, gt);
      if (P.gsplit[k] > 1) wp += (int64_t)P.gsplit[k] * gsz[k];
      cp += (int64_t)P.gsplit[k] * gout[k];
    }
    P.gpart = take(4 * std::max<int64_t>(wp, 1));
    P.gcs = take(4 * cp);
    P.wt = take(2 * L * 4 * C * C);
  }
  if (fp8) {
    P.w8 = take(make_layout(c).total);
    P.wsc = take(4 * ((int64_t)c.padded_vocab_size + L * 9 * C));  // rows of wte and the four per-layer matrices
    P.a8 = take(M * 4 * C);
    P.asc = take(4 * M);
  }
  P.normpart = take(8 * (int64_t)grad_norm_parts());
  P.ska = take(4 * M);
  P.sva = take(4 * M);
  P.skb = take(4 * M);
  P.svb = take(4 * M);
  P.seg = take(4 * (M + 1));
  P.nseg = take(4);
  P.flags = take(16);
  P.scale = take(4);
  P.norm = take(4);
  return P;
}

// ---------------------------------------------------------------------------
// Kernel timing (HIP events on the library's stream around selected launches)
// ---------------------------------------------------------------------------
struct TimedLaunch {
  hipEvent_t a, b;
  double flops;
};

}  // namespace

struct gpt2_handle {
  gpt2_config_t cfg;
  Prec prec;
  int B, T;
  int64_t M;
  float *params, *grads, *m, *v;
  void* params_lp;
  char* ws;
  hipStream_t st;
  // The per-layer weight-gradient products run on a second stream owned by
  // the library, overlapping the rest of the layer's backward; events order
  // them after their inputs and before anything that overwrites those inputs
  // or reads their partial sums.
  hipStream_t side = nullptr;
  bool overlap = true;
  bool recompute = false;  // GPT2_RECOMPUTE_GELU: the layers share two GELU-output buffers
  bool fp8 = false;        // GPT2_FP8_FWD: forward products on FP8 copies
  std::vector<QuantJob> wquant;     // the weights' FP8 copies, one job per matrix
  std::vector<int64_t> wsc_off;     // [kind * (L+1) + layer+1]: row-scale offset (floats) in plan.wsc
  // ev_done[0..3]: a layer's weight-gradient products (qkv, proj, fc, fcproj)
  // on the second stream; ev_done[4]: the forward's embedding sort there;
  // ev_done[5]: the tied head's weight gradient there; ev_done[6]: a layer's
  // batched reduction of partial sums there
  hipEvent_t ev_fork = nullptr, ev_done[7] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  // grouped weight gradients (bf16): a layer's section on the second stream,
  // one event per layer parity (the main stream waits for the layer above's
  // while the current layer's may still be running)
  hipEvent_t ev_layer[2] = {nullptr, nullptr};
  Layout lay;
  Plan plan;
  std::vector<const Tensor*> by_kind_layer;  // [kind * (L+1) + layer+1]
  bool have_fwd = false, fwd_has_targets = false;
  std::vector<ReduceJob> pending;  // partial sums not yet reduced (backward only)
  std::string err;
  int timed = -1;
  std::vector<TimedLaunch> timings;

  template <typename X> X* w(int64_t off) { return reinterpret_cast<X*>(ws + off); }
  const Tensor& tensor(int kind, int layer) const { return *by_kind_layer[kind * (cfg.n_layer + 1) + layer + 1]; }
  float* P32(int kind, int layer = -1) { return params + tensor(kind, layer).offset; }
  float* G32(int kind, int layer = -1) { return grads + tensor(kind, layer).offset; }
  // matmul operand copy of a weight: bf16 copy in BF16, the master in FP32
  const void* W(int kind, int layer = -1) {
    const int64_t off = tensor(kind, layer).offset;
    return prec == BF16 ? static_cast<const void*>(static_cast<const uint16_t*>(params_lp) + off)
                        : static_cast<const void*>(params + off);
  }
  int64_t act_bytes() const { return prec == BF16 ? 2 : 4; }
  // FP8 copy of a weight matrix and its row scales
  const unsigned char* W8(int kind, int layer = -1) {
    return reinterpret_cast<const unsigned char*>(ws + plan.w8) + tensor(kind, layer).offset;
  }
  const float* WS(int kind, int layer = -1) {
    return reinterpret_cast<const float*>(ws + plan.wsc) + wsc_off[kind * (cfg.n_layer + 1) + layer + 1];
  }
};

namespace {

int fail(gpt2_t* h, int code, const std::string& msg) {
  if (h) h->err = msg;
  return code;
}

int hip_check(gpt2_t* h, hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(h, GPT2_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return GPT2_OK;
}

// Brackets one launch with events when its kernel id is being timed.
struct Timer {
  gpt2_t* h;
  bool on;
  TimedLaunch tl;
  Timer(gpt2_t* h_, int id, double flops) : h(h_), on(h_->timed == id) {
    if (on) {
      tl.flops = flops;
      (void)hipEventCreateWithFlags(&tl.a, hipEventDisableSystemFence);
      (void)hipEventCreateWithFlags(&tl.b, hipEventDisableSystemFence);
      (void)hipEventRecord(tl.a, h->st);
    }
  }
  void done() {
    if (on) {
      (void)hipEventRecord(tl.b, h->st);
      h->timings.push_back(tl);
      on = false;
    }
  }
  ~Timer() { done(); }
};

}  // namespace

// Kernel ids for timing (one per kernel function).
enum {
  K_GEMM_NT_STORE = 0,
  K_GEMM_NT_GELU,
  K_GEMM_NT_RESID,
  K_GEMM_NN_STORE,
  K_GEMM_NN_GELU_BWD,
  K_GEMM_TN_F32,
  K_GEMM_TN_LMHEAD,
  K_ATTN_FWD,
  K_ATTN_DKV,
  K_ATTN_DQ,
  K_CE,
  K_LN_FWD,
  K_LN_BWD,
  K_ADAMW,
  K_COUNT
};
static const char* const kKernelNames[K_COUNT] = {
    "gemm_nt_store", "gemm_nt_gelu", "gemm_nt_resid", "gemm_nn_store", "gemm_nn_gelu_bwd", "gemm_tn_f32",
    "gemm_tn_lmhead", "attn_fwd",      "attn_bwd_dkv", "attn_bwd_dq",   "cross_entropy", "layernorm_fwd",     "layernorm_bwd",
    "adamw"};

namespace {

int run_gemm(gpt2_t* h, int kid, int a_t, int b_t, int epi, const GemmArgs& g, const char* what) {
  Timer t(h, kid, 2.0 * g.M * g.N * g.K);
  hipError_t e = gemm(h->st, h->prec, a_t, b_t, epi, g);
  t.done();
  return hip_check(h, e, what);
}

// Forward matmul on FP8 copies: A = the shared FP8 activation buffer (rows
// scaled by plan.asc), B = the weight's FP8 copy with its row scales.
int run_gemm8(gpt2_t* h, int kid, int epi, GemmArgs g, int wkind, int layer, const char* what) {
  g.A = h->w<unsigned char>(h->plan.a8);
  g.scale_a = h->w<float>(h->plan.asc);
  g.B = h->W8(wkind, layer);
  g.scale_b = h->WS(wkind, layer);
  Timer t(h, kid, 2.0 * g.M * g.N * g.K);
  hipError_t e = gemm_fp8(h->st, epi, g);
  t.done();
  return hip_check(h, e, what);
}

// The weights' FP8 copies (after every update of the bf16 copy)
int quantize_weights(gpt2_t* h) {
  for (size_t i = 0; i < h->wquant.size(); i += kMaxQuantJobs) {
    const int n = (int)std::min<size_t>(kMaxQuantJobs, h->wquant.size() - i);
    int rc = hip_check(h, quant_jobs(h->st, h->wquant.data() + i, n), "weight fp8 copy");
    if (rc) return rc;
  }
  return GPT2_OK;
}

// Forward-layer matmul: out = X W^T (+ epilogue); X [M, K] row-major, W [N, K].
GemmArgs fwd_args(gpt2_t* h, const void* X, const void* W, int N, int K, void* out, const float* bias) {
  GemmArgs g;
  g.A = X;
  g.lda = K;
  g.B = W;
  g.ldb = K;
  g.M = (int)h->M;
  g.N = N;
  g.K = K;
  g.C = out;
  g.ldc = N;
  g.bias = bias;
  return g;
}

// Input gradient: out [M, K] = dY [M, N] W [N, K].
GemmArgs dx_args(gpt2_t* h, const void* dY, const void* W, int N, int K, void* out) {
  GemmArgs g;
  g.A = dY;
  g.lda = N;
  g.B = W;
  g.ldb = K;
  g.M = (int)h->M;
  g.N = K;
  g.K = N;
  g.C = out;
  g.ldc = K;
  return g;
}

// The MLP down-projection's input gradient times GELU'(u) of the forward:
// du [M, 4C] = (dres [M, C] W [C, 4C]) * gelu'.  bf16 reads the transposed
// weight copy the training forward made ([4C, C], so both operands are
// reduction-contiguous, which selects the direct-to-LDS 256x256 tile at
// the model widths); fp32 reads W.
int fcproj_dx(gpt2_t* h, const void* dres, int l, void* du) {
  const int C = h->cfg.n_embd;
  const bool tr = h->prec == BF16;
  GemmArgs g = tr ? fwd_args(h, dres, h->w<__bf16>(h->plan.wt) + (int64_t)l * 4 * C * C, 4 * C, C, du, nullptr)
                  : dx_args(h, dres, h->W(T_FCPW, l), C, 4 * C, du);
  g.aux = h->w<void>(h->plan.u[l]);
  g.ldaux = 4 * C;
  g.preact = h->recompute;
  return run_gemm(h, K_GEMM_NN_GELU_BWD, 0, tr ? 0 : 1, EPI_GELU_BWD, g, "fcproj dx");
}

// Partial sums wait in a queue until the layer's backward is done; then one
// launch reduces them all (each into its own gradient, in a fixed order).
void queue_reduction(gpt2_t* h, const float* part, int nparts, int64_t ld, float* out, int n, int accumulate) {
  ReduceJob j;
  j.part = part;
  j.ld = ld;
  j.out = out;
  j.n = n;
  j.nparts = nparts;
  j.accumulate = accumulate;
  h->pending.push_back(j);
}

int flush_reductions(gpt2_t* h) {
  int rc = GPT2_OK;
  for (size_t k = 0; k < h->pending.size() && !rc; k += kMaxReduceJobs) {
    const int n = (int)std::min<size_t>(kMaxReduceJobs, h->pending.size() - k);
    rc = hip_check(h, reduce_jobs(h->st, h->pending.data() + k, n), "reduce partials");
  }
  h->pending.clear();
  return rc;
}

// Weight gradient of W [N, K]: dW (+)= dY^T X, dY [M, N], X [M, K], and the
// bias gradient db (+)= sum_rows dY (column sums fused into the same product);
// split-K partials are reduced in order into the gradient buffers.
int weight_grad(gpt2_t* h, const void* dY, const void* X, int N, int K, float* dW, float* db, int wkind,
                int accumulate, const char* what) {
  const int splits = h->plan.split[wkind];
  GemmArgs g;
  g.A = dY;
  g.lda = N;
  g.B = X;
  g.ldb = K;
  g.M = N;
  g.N = K;
  g.K = (int)h->M;
  g.splits = splits;
  float* cpart = h->w<float>(h->plan.cspart[wkind]);
  if (db) {
    g.colsum = cpart;
    g.colsum_stride = N;
  }
  int rc;
  if (splits == 1) {
    g.C = dW;
    g.ldc = K;
    g.accumulate = accumulate;
    rc = run_gemm(h, K_GEMM_TN_F32, 1, 1, EPI_F32, g, what);
  } else {
    float* part = h->w<float>(h->plan.wpart[wkind]);
    g.C = part;
    g.ldc = K;
    g.split_stride = (int64_t)N * K;
    rc = run_gemm(h, K_GEMM_TN_F32, 1, 1, EPI_F32, g, what);
    if (!rc) queue_reduction(h, part, splits, (int64_t)N * K, dW, N * K, accumulate);
  }
  if (!rc && db) queue_reduction(h, cpart, splits, N, db, N, accumulate);
  return rc;
}

// A layer's four weight gradients (qkv, attention projection, MLP up and
// down; each dW (+)= dY^T X with its bias gradient as fused column sums) in
// one grouped launch.  Products with more than one split leave fp32 partials
// that are reduced in order into the gradients with the layer's other
// partial sums.
struct WGrad {
  const void* dY;
  const void* X;
  int N, K;  // dW is [N, K]
  float *dW, *db;
};

int weight_grad_group(gpt2_t* h, const WGrad (&w)[4], int accumulate) {
  const Plan& P = h->plan;
  GemmArgs g[4];
  int64_t wp = 0, cp = 0;
  for (int k = 0; k < 4; k++) {
    GemmArgs& a = g[k];
    a.A = w[k].dY;
    a.lda = w[k].N;
    a.B = w[k].X;
    a.ldb = w[k].K;
    a.M = w[k].N;
    a.N = w[k].K;
    a.K = (int)h->M;
    a.splits = P.gsplit[k];
    a.ldc = w[k].K;
    a.colsum = h->w<float>(P.gcs) + cp;
    a.colsum_stride = w[k].N;
    cp += (int64_t)a.splits * w[k].N;
    if (a.splits == 1) {
      a.C = w[k].dW;
      a.accumulate = accumulate;
    } else {
      a.C = h->w<float>(P.gpart) + wp;
      a.split_stride = (int64_t)w[k].N * w[k].K;
      wp += (int64_t)a.splits * w[k].N * w[k].K;
    }
  }
  double fl = 0;
  for (auto& a : g) fl += 2.0 * a.M * a.N * a.K;
  Timer t(h, K_GEMM_TN_F32, fl);
  hipError_t e = gemm_group(h->st, g, 4);
  t.done();
  int rc = hip_check(h, e, "weight gradients");
  if (rc) return rc;
  for (int k = 0; k < 4; k++) {
    if (g[k].splits > 1)
      queue_reduction(h, static_cast<const float*>(g[k].C), g[k].splits, g[k].split_stride, w[k].dW, w[k].N * w[k].K,
                      accumulate);
    queue_reduction(h, g[k].colsum, g[k].splits, w[k].N, w[k].db, w[k].N, accumulate);
  }
  return GPT2_OK;
}

// The main stream waits for the second-stream work that recorded ev_done[ev]
// (and, by that stream's order, for everything enqueued there before it).
int join_side(gpt2_t* h, int ev) {
  if (!h->overlap) return GPT2_OK;
  return hip_check(h, hipStreamWaitEvent(h->st, h->ev_done[ev], 0), "join wait");
}

// Work enqueued while a SideSection is open goes to the second stream, after
// everything enqueued so far on the main stream; close(ev) records ev_done[ev]
// there.  Without overlap both are no-ops (the main stream).  The caller's
// stream is put back when the section closes or goes out of scope, so an error
// inside a section never leaves later calls enqueueing on the second stream.
class SideSection {
 public:
  explicit SideSection(gpt2_t* h) : h_(h), saved_(h->st) {}
  ~SideSection() { h_->st = saved_; }
  SideSection(const SideSection&) = delete;
  SideSection& operator=(const SideSection&) = delete;
  int open() {
    if (!h_->overlap) return GPT2_OK;
    int rc = hip_check(h_, hipEventRecord(h_->ev_fork, h_->st), "fork");
    if (!rc) rc = hip_check(h_, hipStreamWaitEvent(h_->side, h_->ev_fork, 0), "fork wait");
    if (!rc) h_->st = h_->side;
    return rc;
  }
  int close(int ev) { return close_event(h_->ev_done[ev]); }
  int close_event(hipEvent_t e) {
    h_->st = saved_;
    if (!h_->overlap) return GPT2_OK;
    return hip_check(h_, hipEventRecord(e, h_->side), "side done");
  }

 private:
  gpt2_t* h_;
  hipStream_t saved_;
};

// lp_off: workspace offset of the bf16 copy of dres it writes (bf16 only)
int ln_backward(gpt2_t* h, const void* dy, const float* x, const float* mean, const float* rstd, int kind_g, int layer,
                int slot, int64_t lp_off, int accumulate_dres, int accumulate_grads) {
  const int C = h->cfg.n_embd, M = (int)h->M;
  float* part = h->w<float>(h->plan.lnpart[slot]);
  int nparts = 0;
  void* dres_lp = h->prec == BF16 ? h->w<void>(lp_off) : nullptr;
  Timer t(h, K_LN_BWD, 0);
  hipError_t e = layernorm_bwd(h->st, h->prec, dy, x, mean, rstd, h->P32(kind_g, layer), h->w<float>(h->plan.dres),
                               dres_lp, accumulate_dres, part, M, C, &nparts);
  t.done();
  int rc = hip_check(h, e, "layernorm_bwd");
  if (rc) return rc;
  // gain and bias gradients are adjacent in the layout: one reduction covers both
  queue_reduction(h, part, nparts, 2 * C, h->G32(kind_g, layer), 2 * C, accumulate_grads);
  return GPT2_OK;
}

}  // namespace

extern "C" {

int64_t gpt2_num_params(const gpt2_config_t* cfg) {
  int rc = check_config(cfg);
  if (rc) return rc;
  return make_layout(*cfg).total;
}

int64_t gpt2_num_decay_params(const gpt2_config_t* cfg) {
  int rc = check_config(cfg);
  if (rc) return rc;
  return make_layout(*cfg).n_decay;
}

int gpt2_param_layout(const gpt2_config_t* cfg, gpt2_tensor_desc_t* out, int cap) {
  int rc = check_config(cfg);
  if (rc) return rc;
  Layout L = make_layout(*cfg);
  if (out)
    for (int i = 0; i < (int)L.t.size() && i < cap; i++) {
      memset(&out[i], 0, sizeof(out[i]));
      snprintf(out[i].name, sizeof(out[i].name), "%s", L.t[i].name.c_str());
      out[i].offset = L.t[i].offset;
      out[i].rows = L.t[i].rows;
      out[i].cols = L.t[i].cols;
      out[i].decay = L.t[i].decay;
    }
  return (int)L.t.size();
}

int gpt2_check_shapes(const gpt2_config_t* cfg, int B, int T) {
  int rc = check_config(cfg);
  if (rc) return rc;
  return check_bt(cfg, B, T);
}

int64_t gpt2_workspace_bytes(const gpt2_config_t* cfg, int B, int T, int precision) {
  int rc = gpt2_check_shapes(cfg, B, T);
  if (rc) return rc;
  const int base = precision & ~(GPT2_RECOMPUTE_GELU | GPT2_FP8_FWD);
  if (base != GPT2_FP32 && base != GPT2_BF16) return GPT2_ERR_ARG;
  if ((precision & GPT2_FP8_FWD) && !fp8_ok(cfg, base)) return GPT2_ERR_ARG;
  return make_plan(*cfg, B, T, precision).bytes;
}

int gpt2_init(gpt2_t** out, const gpt2_config_t* cfg, int precision, int B, int T, float* params, void* params_lp,
              float* grads, float* adam_m, float* adam_v, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!out) return GPT2_ERR_ARG;
  *out = nullptr;
  int rc = gpt2_check_shapes(cfg, B, T);
  if (rc) return rc;
  const bool recompute = (precision & GPT2_RECOMPUTE_GELU) != 0;
  const bool fp8 = (precision & GPT2_FP8_FWD) != 0;
  const int base = precision & ~(GPT2_RECOMPUTE_GELU | GPT2_FP8_FWD);
  if (base != GPT2_FP32 && base != GPT2_BF16) return GPT2_ERR_ARG;
  if (fp8 && !fp8_ok(cfg, base)) return GPT2_ERR_ARG;
  auto aligned = [](const void* p) { return p && (reinterpret_cast<uintptr_t>(p) % 256) == 0; };
  if (!aligned(params) || !aligned(grads) || !aligned(adam_m) || !aligned(adam_v) || !aligned(workspace))
    return GPT2_ERR_ARG;
  if (base == GPT2_BF16 && !aligned(params_lp)) return GPT2_ERR_ARG;
  Plan plan = make_plan(*cfg, B, T, precision);
  if (workspace_bytes < plan.bytes) return GPT2_ERR_WORKSPACE;
  gpt2_t* h = new (std::nothrow) gpt2_handle();
  if (!h) return GPT2_ERR_ARG;
  h->cfg = *cfg;
  h->prec = base == GPT2_BF16 ? BF16 : F32;
  h->recompute = recompute;
  h->fp8 = fp8;
  h->B = B;
  h->T = T;
  h->M = (int64_t)B * T;
  h->params = params;
  h->params_lp = base == GPT2_BF16 ? params_lp : nullptr;
  h->grads = grads;
  h->m = adam_m;
  h->v = adam_v;
  h->ws = static_cast<char*>(workspace);
  h->st = static_cast<hipStream_t>(stream);
  h->lay = make_layout(*cfg);
  h->plan = plan;
  h->by_kind_layer.assign(16 * (cfg->n_layer + 1), nullptr);
  for (auto& t : h->lay.t) h->by_kind_layer[t.kind * (cfg->n_layer + 1) + t.layer + 1] = &t;
  if (fp8) {
    // one quantization job per forward matrix, scales packed in plan.wsc
    h->wsc_off.assign(16 * (cfg->n_layer + 1), -1);
    int64_t rows = 0;
    auto job = [&](int kind, int layer) {
      const Tensor& t = h->tensor(kind, layer);
      QuantJob q;
      q.in = static_cast<const __bf16*>(params_lp) + t.offset;
      q.out = reinterpret_cast<unsigned char*>(h->ws + plan.w8) + t.offset;
      q.scale = reinterpret_cast<float*>(h->ws + plan.wsc) + rows;
      q.rows = t.rows;
      q.cols = t.cols;
      h->wsc_off[kind * (cfg->n_layer + 1) + layer + 1] = rows;
      rows += t.rows;
      h->wquant.push_back(q);
    };
    job(T_WTE, -1);
    for (int l = 0; l < cfg->n_layer; l++) {
      job(T_QKVW, l);
      job(T_PROJW, l);
      job(T_FCW, l);
      job(T_FCPW, l);
    }
  }
  // the deferred status flags live in the caller's workspace: start them at zero
  if (hipMemsetAsync(h->w<int>(plan.flags), 0, 16, h->st) != hipSuccess) {
    delete h;
    return GPT2_ERR_HIP;
  }
  if (hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess) {
    gpt2_destroy(h);
    return GPT2_ERR_HIP;
  }
  for (auto& e : h->ev_done)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess) {
      gpt2_destroy(h);
      return GPT2_ERR_HIP;
    }
  for (auto& e : h->ev_layer)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess) {
      gpt2_destroy(h);
      return GPT2_ERR_HIP;
    }
  *out = h;
  return GPT2_OK;
}

void gpt2_destroy(gpt2_t* h) {
  if (!h) return;
  for (auto& t : h->timings) {
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  if (h->side) {
    (void)hipStreamSynchronize(h->side);
    (void)hipStreamDestroy(h->side);
  }
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  for (auto& e : h->ev_done)
    if (e) (void)hipEventDestroy(e);
  for (auto& e : h->ev_layer)
    if (e) (void)hipEventDestroy(e);
  delete h;
}

int gpt2_set_stream(gpt2_t* h, void* stream) {
  if (!h) return GPT2_ERR_ARG;
  h->st = static_cast<hipStream_t>(stream);
  return GPT2_OK;
}

int gpt2_set_overlap(gpt2_t* h, int enable) {
  if (!h) return GPT2_ERR_ARG;
  h->overlap = enable != 0;
  return GPT2_OK;
}

int gpt2_refresh_params(gpt2_t* h) {
  if (!h) return GPT2_ERR_ARG;
  if (h->prec != BF16) return GPT2_OK;
  int rc = hip_check(h, to_bf16(h->st, h->params, h->params_lp, h->lay.total), "to_bf16");
  if (!rc && h->fp8) rc = quantize_weights(h);
  return rc;
}

// The forward of training (train = 1: keeps what the backward needs, gelu'
// and the embedding sort, and leaves dlogits in place of the logits) or of
// evaluation (train = 0: loss only).
static int forward_impl(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, float* d_loss, float* d_loss_rows,
                        bool train) {
  if (!h || !d_idx) return fail(h, GPT2_ERR_ARG, "null handle or ids");
  const gpt2_config_t& c = h->cfg;
  const int C = c.n_embd, L = c.n_layer, NH = c.n_head, hd = C / NH, Mi = (int)h->M;
  const Plan& P = h->plan;
  const int64_t Mx = h->M;
  int rc;
  int* flags = h->w<int>(P.flags);
  h->have_fwd = false;
  // FP8 forward products: the layer norms also write FP8 rows here
  unsigned char* a8 = h->fp8 ? h->w<unsigned char>(P.a8) : nullptr;
  float* asc = h->fp8 ? h->w<float>(P.asc) : nullptr;

  rc = hip_check(h, embed_fwd(h->st, d_idx, d_targets, h->P32(T_WTE), h->P32(T_WPE), h->w<float>(P.x_in[0]), h->B, h->T, C,
                              c.vocab_size, flags),
                 "embed_fwd");
  if (rc) return rc;
  if (d_targets && train) {
    // the sort of the ids (for the embedding backward) needs only the ids: with
    // overlap on it runs on the second stream beside the layers, joined back at
    // the end of the forward
    hipStream_t sst = h->st;
    if (h->overlap) {
      rc = hip_check(h, hipEventRecord(h->ev_fork, h->st), "fork");
      if (!rc) rc = hip_check(h, hipStreamWaitEvent(h->side, h->ev_fork, 0), "fork wait");
      if (rc) return rc;
      sst = h->side;
    }
    rc = hip_check(h, embed_sort(sst, d_idx, Mi, c.vocab_size, h->w<int32_t>(P.ska), h->w<int32_t>(P.sva),
                                 h->w<int32_t>(P.skb), h->w<int32_t>(P.svb), h->w<int32_t>(P.seg), h->w<int32_t>(P.nseg)),
                   "embed_sort");
    // (bf16) the transposed MLP down-projection weights the backward's GELU'
    // product reads, from the current bf16 copy
    if (!rc && h->prec == BF16)
      rc = hip_check(h, transpose_bf16(sst, h->W(T_FCPW, 0), 12 * (int64_t)C * C, h->w<void>(P.wt), C, 4 * C, L),
                     "fcproj transpose");
    if (!rc && h->overlap) rc = hip_check(h, hipEventRecord(h->ev_done[4], h->side), "sort done");
    if (rc) return rc;
  }
  for (int l = 0; l < L; l++) {
    {
      Timer t(h, K_LN_FWD, 0);
      rc = hip_check(h, layernorm_fwd(h->st, h->prec, h->w<float>(P.x_in[l]), h->P32(T_LN1G, l), h->P32(T_LN1B, l),
                                      h->w<void>(P.h1[l]), h->w<float>(P.mean1[l]), h->w<float>(P.rstd1[l]), Mi, C,
                                      a8, asc),
                     "ln1");
    }
    if (rc) return rc;
    GemmArgs g = fwd_args(h, h->w<void>(P.h1[l]), h->W(T_QKVW, l), 3 * C, C, h->w<void>(P.qkv[l]), h->P32(T_QKVB, l));
    if ((rc = h->fp8 ? run_gemm8(h, K_GEMM_NT_STORE, EPI_STORE, g, T_QKVW, l, "qkv")
                     : run_gemm(h, K_GEMM_NT_STORE, 0, 0, EPI_STORE, g, "qkv")))
      return rc;
    {
      const double pairs = (double)h->B * NH * ((double)h->T * (h->T + 1) / 2);
      Timer t(h, K_ATTN_FWD, 4.0 * hd * pairs);
      rc = hip_check(h, attn_fwd(h->st, h->prec, h->w<void>(P.qkv[l]), h->w<void>(P.atty[l]), h->w<float>(P.lse[l]),
                                 h->B, h->T, NH, hd),
                     "attn_fwd");
    }
    if (rc) return rc;
    if (h->fp8 && (rc = hip_check(h, quant_rows(h->st, h->w<void>(P.atty[l]), a8, asc, Mi, C), "attn out fp8")))
      return rc;
    g = fwd_args(h, h->w<void>(P.atty[l]), h->W(T_PROJW, l), C, C, h->w<void>(P.x_mid[l]), h->P32(T_PROJB, l));
    g.resid = h->w<float>(P.x_in[l]);
    g.ldr = C;
    if ((rc = h->fp8 ? run_gemm8(h, K_GEMM_NT_RESID, EPI_RESID, g, T_PROJW, l, "proj")
                     : run_gemm(h, K_GEMM_NT_RESID, 0, 0, EPI_RESID, g, "proj")))
      return rc;
    {
      Timer t(h, K_LN_FWD, 0);
      rc = hip_check(h, layernorm_fwd(h->st, h->prec, h->w<float>(P.x_mid[l]), h->P32(T_LN2G, l), h->P32(T_LN2B, l),
                                      h->w<void>(P.h2[l]), h->w<float>(P.mean2[l]), h->w<float>(P.rstd2[l]), Mi, C,
                                      a8, asc),
                     "ln2");
    }
    if (rc) return rc;
    g = fwd_args(h, h->w<void>(P.h2[l]), h->W(T_FCW, l), 4 * C, C, h->w<void>(P.g[l]), h->P32(T_FCB, l));
    g.aux = train ? h->w<void>(P.u[l]) : nullptr;
    g.ldaux = 4 * C;
    g.preact = h->recompute;  // (in evaluation too, so its loss equals the training forward's)
    if ((rc = h->fp8 ? run_gemm8(h, K_GEMM_NT_GELU, EPI_GELU, g, T_FCW, l, "fc")
                     : run_gemm(h, K_GEMM_NT_GELU, 0, 0, EPI_GELU, g, "fc")))
      return rc;
    if (h->fp8 && (rc = hip_check(h, quant_rows(h->st, h->w<void>(P.g[l]), a8, asc, Mi, 4 * C), "gelu out fp8")))
      return rc;
    g = fwd_args(h, h->w<void>(P.g[l]), h->W(T_FCPW, l), C, 4 * C, h->w<void>(P.x_in[l + 1]), h->P32(T_FCPB, l));
    g.resid = h->w<float>(P.x_mid[l]);
    g.ldr = C;
    if ((rc = h->fp8 ? run_gemm8(h, K_GEMM_NT_RESID, EPI_RESID, g, T_FCPW, l, "fcproj")
                     : run_gemm(h, K_GEMM_NT_RESID, 0, 0, EPI_RESID, g, "fcproj")))
      return rc;
  }
  {
    Timer t(h, K_LN_FWD, 0);
    rc = hip_check(h, layernorm_fwd(h->st, h->prec, h->w<float>(P.x_in[L]), h->P32(T_LNFG), h->P32(T_LNFB),
                                    h->w<void>(P.hf), h->w<float>(P.meanf), h->w<float>(P.rstdf), Mi, C, a8, asc),
                   "lnf");
  }
  if (rc) return rc;
  // tied output layer over the padded vocabulary
  GemmArgs g = fwd_args(h, h->w<void>(P.hf), h->W(T_WTE), c.padded_vocab_size, C, h->w<void>(P.logits), nullptr);
  if ((rc = h->fp8 ? run_gemm8(h, K_GEMM_NT_STORE, EPI_STORE, g, T_WTE, -1, "lm_head")
                   : run_gemm(h, K_GEMM_NT_STORE, 0, 0, EPI_STORE, g, "lm_head")))
    return rc;
  if (d_targets) {
    float* rows = d_loss_rows ? d_loss_rows : h->w<float>(P.loss_rows);
    {
      Timer t(h, K_CE, 0);
      // dlogits of the mean loss; the 1/K of gradient accumulation is applied in backward
      rc = hip_check(h, cross_entropy(h->st, h->prec, h->w<void>(P.logits), d_targets, rows, Mi, c.vocab_size,
                                      c.padded_vocab_size, 1.0f / (float)Mx, train ? 1 : 0),
                     "cross_entropy");
    }
    if (rc) return rc;
    if (d_loss) {
      rc = hip_check(h, mean_loss(h->st, rows, Mi, d_loss), "mean_loss");
      if (rc) return rc;
    }
  }
  if (d_targets && train && h->overlap) {
    rc = hip_check(h, hipStreamWaitEvent(h->st, h->ev_done[4], 0), "sort join");
    if (rc) return rc;
  }
  h->have_fwd = train;
  h->fwd_has_targets = d_targets != nullptr;
  return GPT2_OK;
}

int gpt2_forward(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, float* d_loss, float* d_loss_rows) {
  return forward_impl(h, d_idx, d_targets, d_loss, d_loss_rows, true);
}

int gpt2_eval(gpt2_t* h, const int32_t* d_idx, const int32_t* d_targets, float* d_loss, float* d_loss_rows) {
  if (!h || !d_targets) return fail(h, GPT2_ERR_ARG, "evaluation needs targets");
  return forward_impl(h, d_idx, d_targets, d_loss, d_loss_rows, false);
}

int gpt2_residual(gpt2_t* h, int layer, const float** out) {
  if (!h || !out) return GPT2_ERR_ARG;
  if (layer < 0 || layer > h->cfg.n_layer) return fail(h, GPT2_ERR_ARG, "layer outside [0, n_layer]");
  *out = h->w<float>(h->plan.x_in[layer]);
  return GPT2_OK;
}

int gpt2_backward(gpt2_t* h, int micro_step, int grad_accum_steps) {
  if (!h) return GPT2_ERR_ARG;
  if (grad_accum_steps < 1 || micro_step < 0 || micro_step >= grad_accum_steps)
    return fail(h, GPT2_ERR_ARG, "bad micro_step / grad_accum_steps");
  if (!h->have_fwd || !h->fwd_has_targets) return fail(h, GPT2_ERR_ARG, "backward needs a forward with targets");
  const gpt2_config_t& c = h->cfg;
  const int C = c.n_embd, L = c.n_layer, NH = c.n_head, hd = C / NH, Vp = c.padded_vocab_size;
  const Plan& P = h->plan;
  h->pending.clear();
  const int acc = micro_step > 0;
  const float alpha = 1.0f / (float)grad_accum_steps;
  const bool lp = h->prec == BF16;
  void* dres_op = lp ? h->w<void>(P.dres_lp) : h->w<void>(P.dres);  // matmul operand view of dres
  float* dres = h->w<float>(P.dres);
  int rc;

  // tied output layer: dhf = dlogits wte ; dwte (+)= dlogits^T hf   (both scaled by 1/K).
  // With overlap the weight gradient runs on the second stream beside the
  // input gradient (both only read dlogits); the embedding backward, which
  // adds the token rows' gradient into the same dwte, waits for it.
  {
    hipStream_t main_st = h->st;
    if (h->overlap) {
      rc = hip_check(h, hipEventRecord(h->ev_fork, h->st), "fork");
      if (!rc) rc = hip_check(h, hipStreamWaitEvent(h->side, h->ev_fork, 0), "fork wait");
      if (rc) return rc;
      h->st = h->side;
    }
    GemmArgs w;
    w.A = h->w<void>(P.logits);
    w.lda = Vp;
    w.B = h->w<void>(P.hf);
    w.ldb = C;
    w.M = Vp;
    w.N = C;
    w.K = (int)h->M;
    w.C = h->G32(T_WTE);
    w.ldc = C;
    w.accumulate = acc;
    w.alpha = alpha;
    rc = run_gemm(h, K_GEMM_TN_LMHEAD, 1, 1, EPI_F32, w, "lm_head dw");
    h->st = main_st;
    if (!rc && h->overlap) rc = hip_check(h, hipEventRecord(h->ev_done[5], h->side), "join");
    if (rc) return rc;
  }
  GemmArgs g = dx_args(h, h->w<void>(P.logits), h->W(T_WTE), Vp, C, h->w<void>(P.dh));
  g.alpha = alpha;
  if ((rc = run_gemm(h, K_GEMM_NN_STORE, 0, 1, EPI_STORE, g, "lm_head dx"))) return rc;
  // grouped weight gradients (bf16): the matmul copy of a layer's
  // block-output gradient alternates between two buffers
  const bool grouped = lp;
  auto dres_lp_slot = [&](int layer) { return grouped && (layer & 1) ? P.dres_lp2 : P.dres_lp; };
  if ((rc = ln_backward(h, h->w<void>(P.dh), h->w<float>(P.x_in[L]), h->w<float>(P.meanf), h->w<float>(P.rstdf), T_LNFG,
                        -1, 0, dres_lp_slot(L - 1), 0, acc)))
    return rc;

  if (grouped) {
    // Per layer, on the main stream: the input gradients, LayerNorm and
    // attention backward.  After the attention backward the layer's four
    // weight gradients go to the second stream as one grouped launch, behind
    // the queued reductions of the layer above.  Everything such a launch
    // reads alternates between two buffers by layer (the block-output
    // gradient's matmul copy, du, LayerNorm 2's copy, dqkv; also the
    // LayerNorm partial sums its section reduces), so the main stream waits
    // for layer l+1's section only before LayerNorm 1 of layer l rewrites the
    // buffer that section read.
    for (int l = L - 1; l >= 0; l--) {
      // activation recompute: rebuild this layer's GELU output (the last
      // two layers' are still in their buffers from the forward); the
      // buffer's previous reader, layer l+2's weight gradients, was joined
      // before LayerNorm 1 of layer l+1
      if (h->recompute && l < L - 2) {
        rc = hip_check(h, gelu_fwd(h->st, h->prec, h->w<void>(P.u[l]), h->w<void>(P.g[l]), h->M * 4 * C),
                       "gelu recompute");
        if (rc) return rc;
      }
      void* dres_op_l = h->w<void>(dres_lp_slot(l));
      void* du = h->w<void>((l & 1) ? P.du2 : P.du);
      void* dqkv = h->w<void>((l & 1) ? P.dqkv2 : P.dqkv);
      const int64_t lp2_off = P.lp2[l & 1];
      void* ln2_op = h->w<void>(lp2_off);
      if ((rc = fcproj_dx(h, dres_op_l, l, du))) return rc;
      g = dx_args(h, du, h->W(T_FCW, l), 4 * C, C, h->w<void>(P.dh));
      if ((rc = run_gemm(h, K_GEMM_NN_STORE, 0, 1, EPI_STORE, g, "fc dx"))) return rc;
      if ((rc = ln_backward(h, h->w<void>(P.dh), h->w<float>(P.x_mid[l]), h->w<float>(P.mean2[l]),
                            h->w<float>(P.rstd2[l]), T_LN2G, l, 1 + (l & 1), lp2_off, 1, acc)))
        return rc;
      g = dx_args(h, ln2_op, h->W(T_PROJW, l), C, C, h->w<void>(P.datty));
      if ((rc = run_gemm(h, K_GEMM_NN_STORE, 0, 1, EPI_STORE, g, "proj dx"))) return rc;
      {
        const double pairs = (double)h->B * NH * ((double)h->T * (h->T + 1) / 2);
        {
          Timer t(h, K_ATTN_DQ, 4.0 * hd * pairs);
          rc = hip_check(h, attn_bwd_dq(h->st, h->prec, h->w<void>(P.qkv[l]), h->w<void>(P.atty[l]),
                                        h->w<void>(P.datty), h->w<float>(P.lse[l]), h->w<float>(P.dsum), dqkv, h->B,
                                        h->T, NH, hd),
                         "attn dq");
        }
        if (rc) return rc;
        {
          Timer t(h, K_ATTN_DKV, 4.0 * hd * pairs);
          rc = hip_check(h, attn_bwd_dkv(h->st, h->prec, h->w<void>(P.qkv[l]), h->w<void>(P.datty),
                                         h->w<float>(P.lse[l]), h->w<float>(P.dsum), dqkv, h->B, h->T, NH, hd),
                         "attn dkv");
        }
        if (rc) return rc;
      }
      {
        SideSection side(h);
        if ((rc = side.open())) return rc;
        rc = flush_reductions(h);  // the layer above's partial sums (and this layer's LayerNorm 2's)
        // (order: at 124M each XCD's range of the launch then holds whole
        // splits of the qkv product and cuts the others between row or
        // column tiles only)
        const WGrad w[4] = {{dqkv, h->w<void>(P.h1[l]), 3 * C, C, h->G32(T_QKVW, l), h->G32(T_QKVB, l)},
                            {du, h->w<void>(P.h2[l]), 4 * C, C, h->G32(T_FCW, l), h->G32(T_FCB, l)},
                            {ln2_op, h->w<void>(P.atty[l]), C, C, h->G32(T_PROJW, l), h->G32(T_PROJB, l)},
                            {dres_op_l, h->w<void>(P.g[l]), C, 4 * C, h->G32(T_FCPW, l), h->G32(T_FCPB, l)}};
        if (!rc) rc = weight_grad_group(h, w, acc);
        if (rc || (rc = side.close_event(h->ev_layer[l & 1]))) return rc;
      }
      g = dx_args(h, dqkv, h->W(T_QKVW, l), 3 * C, C, h->w<void>(P.dh));
      if ((rc = run_gemm(h, K_GEMM_NN_STORE, 0, 1, EPI_STORE, g, "qkv dx"))) return rc;
      // LayerNorm 1 writes the block-output gradient's copy for layer l-1,
      // the buffer layer l+1's weight gradients read
      if (l < L - 1 && h->overlap &&
          (rc = hip_check(h, hipStreamWaitEvent(h->st, h->ev_layer[(l + 1) & 1], 0), "join wait")))
        return rc;
      if ((rc = ln_backward(h, h->w<void>(P.dh), h->w<float>(P.x_in[l]), h->w<float>(P.mean1[l]),
                            h->w<float>(P.rstd1[l]), T_LN1G, l, 3 + (l & 1), dres_lp_slot(l - 1), 1, acc)))
        return rc;
    }
  } else {

  // Second stream, per layer: one section before the MLP down-projection's
  // input gradient (the layer above's queued reductions, then this
  // layer's fcproj weight gradient), one after it (fc), and one after the
  // attention backward (proj, qkv).  The main stream joins it once per layer,
  // before LayerNorm 1, which rewrites the matmul copy of dres that the fcproj
  // weight gradient reads (and so, by stream order, after everything the
  // second stream did for the layer above).  With bf16, du, dqkv and LayerNorm
  // 2's copy of dres alternate between two buffers by layer, so their readers
  // (two layers back) are covered by that join.  fp32 matmuls read dres itself,
  // which every LayerNorm backward rewrites: there each rewrite waits for its
  // readers, as does each single du / dqkv buffer.
  const bool strict = !lp;
  for (int l = L - 1; l >= 0; l--) {
    void* du = h->w<void>((l & 1) ? P.du2 : P.du);
    void* dqkv = h->w<void>((l & 1) ? P.dqkv2 : P.dqkv);
    const int64_t lp2_off = P.lp2[l & 1];
    void* ln2_op = lp ? h->w<void>(lp2_off) : dres;  // matmul view of dres after LayerNorm 2
    // activation recompute: rebuild this layer's GELU output in its shared
    // buffer (the last two layers' are still there from the forward); its
    // reader two layers above (the fcproj weight gradient) was joined before
    // the layer above's LayerNorm 1 backward
    if (h->recompute && l < L - 2) {
      rc = hip_check(h, gelu_fwd(h->st, h->prec, h->w<void>(P.u[l]), h->w<void>(P.g[l]), h->M * 4 * C), "gelu recompute");
      if (rc) return rc;
    }
    // MLP down-projection: dres is the gradient of the block output
    {
      SideSection side(h);
      if ((rc = side.open())) return rc;
      rc = flush_reductions(h);  // the layer above's partial sums (and the final LayerNorm's)
      if (!rc) rc = weight_grad(h, dres_op, h->w<void>(P.g[l]), C, 4 * C, h->G32(T_FCPW, l), h->G32(T_FCPB, l), 3, acc,
                                "fcproj dw");
      if (rc || (rc = side.close(3))) return rc;
    }
    if (strict && l < L - 1 && (rc = join_side(h, 2))) return rc;  // the layer above's fc weight gradient read du
    if ((rc = fcproj_dx(h, dres_op, l, du))) return rc;
    // MLP up-projection
    {
      SideSection side(h);
      if ((rc = side.open())) return rc;
      rc = weight_grad(h, du, h->w<void>(P.h2[l]), 4 * C, C, h->G32(T_FCW, l), h->G32(T_FCB, l), 2, acc, "fc dw");
      if (rc || (rc = side.close(2))) return rc;
    }
    g = dx_args(h, du, h->W(T_FCW, l), 4 * C, C, h->w<void>(P.dh));
    if ((rc = run_gemm(h, K_GEMM_NN_STORE, 0, 1, EPI_STORE, g, "fc dx"))) return rc;
    if (strict && (rc = join_side(h, 3))) return rc;  // the fcproj weight gradient reads dres
    if ((rc = ln_backward(h, h->w<void>(P.dh), h->w<float>(P.x_mid[l]), h->w<float>(P.mean2[l]), h->w<float>(P.rstd2[l]),
                          T_LN2G, l, 1 + (l & 1), lp2_off, 1, acc)))
      return rc;
    if (strict) {  // the projection's weight gradient now, before LayerNorm 1 rewrites dres
      SideSection side(h);
      if ((rc = side.open())) return rc;
      rc = weight_grad(h, ln2_op, h->w<void>(P.atty[l]), C, C, h->G32(T_PROJW, l), h->G32(T_PROJB, l), 1, acc, "proj dw");
      if (rc || (rc = side.close(1))) return rc;
    }
    // attention output projection
    g = dx_args(h, ln2_op, h->W(T_PROJW, l), C, C, h->w<void>(P.datty));
    if ((rc = run_gemm(h, K_GEMM_NN_STORE, 0, 1, EPI_STORE, g, "proj dx"))) return rc;
    if (strict && l < L - 1 && (rc = join_side(h, 0))) return rc;  // the layer above's qkv weight gradient read dqkv
    // attention
    {
      // dQ first: it also stores D = rowsum(dO * O), which dK/dV reads
      const double pairs = (double)h->B * NH * ((double)h->T * (h->T + 1) / 2);
      {
        Timer t(h, K_ATTN_DQ, 4.0 * hd * pairs);
        rc = hip_check(h, attn_bwd_dq(h->st, h->prec, h->w<void>(P.qkv[l]), h->w<void>(P.atty[l]), h->w<void>(P.datty),
                                      h->w<float>(P.lse[l]), h->w<float>(P.dsum), dqkv, h->B, h->T, NH, hd),
                       "attn dq");
      }
      if (rc) return rc;
      {
        Timer t(h, K_ATTN_DKV, 4.0 * hd * pairs);
        rc = hip_check(h, attn_bwd_dkv(h->st, h->prec, h->w<void>(P.qkv[l]), h->w<void>(P.datty), h->w<float>(P.lse[l]),
                                       h->w<float>(P.dsum), dqkv, h->B, h->T, NH, hd),
                       "attn dkv");
      }
      if (rc) return rc;
    }
    // qkv projection (and, with bf16, the output projection's weight gradient)
    {
      SideSection side(h);
      if ((rc = side.open())) return rc;
      if (!strict)
        rc = weight_grad(h, ln2_op, h->w<void>(P.atty[l]), C, C, h->G32(T_PROJW, l), h->G32(T_PROJB, l), 1, acc,
                         "proj dw");
      if (!rc) rc = weight_grad(h, dqkv, h->w<void>(P.h1[l]), 3 * C, C, h->G32(T_QKVW, l), h->G32(T_QKVB, l), 0, acc,
                                "qkv dw");
      if (rc || (rc = side.close(0))) return rc;
    }
    g = dx_args(h, dqkv, h->W(T_QKVW, l), 3 * C, C, h->w<void>(P.dh));
    if ((rc = run_gemm(h, K_GEMM_NN_STORE, 0, 1, EPI_STORE, g, "qkv dx"))) return rc;
    // LayerNorm 1 rewrites the copy of dres the fcproj weight gradient read
    // (fp32: dres itself, which the projection's weight gradient also reads)
    if ((rc = join_side(h, strict ? 1 : 3))) return rc;
    if ((rc = ln_backward(h, h->w<void>(P.dh), h->w<float>(P.x_in[l]), h->w<float>(P.mean1[l]), h->w<float>(P.rstd1[l]),
                          T_LN1G, l, 3, P.dres_lp, 1, acc)))
      return rc;
  }
  }  // grouped
  // layer 0's partial sums (the last layer processed), on the second stream
  // behind its products
  {
    SideSection side(h);
    if ((rc = side.open())) return rc;
    rc = flush_reductions(h);
    if (rc || (rc = side.close(6))) return rc;
  }
  // embeddings: position rows and the (tied) token rows, in a fixed order,
  // after the tied head's weight gradient (which wrote dwte first) and beside
  // layer 0's weight gradients and reductions, which touch neither
  if ((rc = join_side(h, 5))) return rc;
  rc = hip_check(h, embed_bwd(h->st, dres, h->w<int32_t>(P.ska), h->w<int32_t>(P.sva), h->w<int32_t>(P.seg),
                              h->w<int32_t>(P.nseg), h->G32(T_WTE), h->G32(T_WPE), h->w<float>(P.piece), h->B, h->T,
                              c.max_seq_len, C, c.vocab_size, acc),
                 "embed_bwd");
  if (rc) return rc;
  return join_side(h, 6);  // everything else on the second stream
}

int gpt2_adamw_step(gpt2_t* h, int step, float lr, float beta1, float beta2, float eps, float weight_decay,
                    float grad_clip, float* d_grad_norm) {
  if (!h) return GPT2_ERR_ARG;
  if (step < 1) return fail(h, GPT2_ERR_ARG, "step must be >= 1");
  const Plan& P = h->plan;
  int* flags = h->w<int>(P.flags);
  float* scale = h->w<float>(P.scale);
  float* norm = d_grad_norm ? d_grad_norm : h->w<float>(P.norm);
  int rc = hip_check(h, grad_norm(h->st, h->grads, h->lay.total, h->w<double>(P.normpart), grad_clip, norm, scale, flags),
                     "grad_norm");
  if (rc) return rc;
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
  Timer t(h, K_ADAMW, 0);
  rc = hip_check(h, adamw(h->st, h->params, h->grads, h->m, h->v, h->params_lp, h->lay.total, h->lay.n_decay, lr, beta1,
                          beta2, eps, weight_decay, (float)bc1, (float)bc2, scale, flags),
                 "adamw");
  t.done();
  if (!rc && h->fp8) rc = quantize_weights(h);
  return rc;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Clip + AdamW without allocation.  The scratch of gpt2_adamw_step_noalloc
// (the global norm's fp64 partial sums, the clip factor and the skip flag) is
// this file-scope device array instead of a workspace: each GPU the library
// runs on holds its own copy until the process ends.  Every word a call reads
// is written earlier in the same call (all partials by the first norm kernel,
// the clip factor and the skip flag by the second), so nothing needs clearing
// between calls; calls that overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------
namespace {
constexpr int64_t kNoAllocPartOff = 0;                                  // double[kGradNormParts]
constexpr int64_t kNoAllocScaleOff = 8 * (int64_t)kGradNormParts;      // float: clip factor
constexpr int64_t kNoAllocFlagsOff = kNoAllocScaleOff + 16;             // int[4]: [1] non-finite, [2] skip
constexpr int64_t kNoAllocScratchBytes = (kNoAllocFlagsOff + 16 + 255) / 256 * 256;
constexpr int64_t kNoAllocMaxParams = (int64_t)1 << 36;                 // 64 Gi parameters
constexpr int kNoAllocMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices] = {};

// Device address of the current device's copy of the scratch array, looked up
// once per device (the host-side name of the array is not a device address).
hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

int gpt2_adamw_step_noalloc(float* params, void* params_lp, const float* grads, float* adam_m, float* adam_v,
                            int64_t n, int64_t n_decay, int step, float lr, float beta1, float beta2, float eps,
                            float weight_decay, float grad_clip, float* d_grad_norm, void* stream) {
  if (!params || !grads || !adam_m || !adam_v || !d_grad_norm) return GPT2_ERR_ARG;
  auto aligned16 = [](const void* p) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % 16 == 0; };
  if (!aligned16(params) || !aligned16(grads) || !aligned16(adam_m) || !aligned16(adam_v) ||
      reinterpret_cast<uintptr_t>(params_lp) % 8 != 0)
    return GPT2_ERR_ARG;
  if (n <= 0 || n % 4 != 0 || n > kNoAllocMaxParams || n_decay < 0 || n_decay > n || n_decay % 4 != 0 || step < 1)
    return GPT2_ERR_ARG;
  void* ptr = nullptr;
  if (noalloc_scratch(&ptr) != hipSuccess) return GPT2_ERR_HIP;
  char* base = static_cast<char*>(ptr);
  double* part = reinterpret_cast<double*>(base + kNoAllocPartOff);
  float* scale = reinterpret_cast<float*>(base + kNoAllocScaleOff);
  int* flags = reinterpret_cast<int*>(base + kNoAllocFlagsOff);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (grad_norm(st, grads, n, part, grad_clip, d_grad_norm, scale, flags) != hipSuccess) return GPT2_ERR_HIP;
  const double bc1 = 1.0 - std::pow((double)beta1, (double)step);
  const double bc2 = 1.0 - std::pow((double)beta2, (double)step);
  if (adamw(st, params, grads, adam_m, adam_v, params_lp, n, n_decay, lr, beta1, beta2, eps, weight_decay, (float)bc1,
            (float)bc2, scale, flags) != hipSuccess)
    return GPT2_ERR_HIP;
  return GPT2_OK;
}

int gpt2_sync_status(gpt2_t* h) {
  if (!h) return GPT2_ERR_ARG;
  int rc = hip_check(h, hipStreamSynchronize(h->st), "sync");
  if (rc) return rc;
  int f[4] = {0, 0, 0, 0};
  int* flags = h->w<int>(h->plan.flags);
  rc = hip_check(h, hipMemcpy(f, flags, sizeof(f), hipMemcpyDeviceToHost), "read flags");
  if (rc) return rc;
  const int zero[2] = {0, 0};
  rc = hip_check(h, hipMemcpy(flags, zero, sizeof(zero), hipMemcpyHostToDevice), "clear flags");
  if (rc) return rc;
  if (f[0]) return fail(h, GPT2_ERR_TOKEN_RANGE, "token id or target outside [0, vocab_size)");
  if (f[1]) return fail(h, GPT2_ERR_NONFINITE, "non-finite gradient norm; the update was skipped");
  return GPT2_OK;
}

const char* gpt2_last_error(gpt2_t* h) { return h ? h->err.c_str() : "null handle"; }

const char* gpt2_strerror(int code) {
  switch (code) {
    case GPT2_OK: return "ok";
    case GPT2_ERR_CONFIG: return "invalid model configuration";
    case GPT2_ERR_SHAPE: return "invalid batch shape";
    case GPT2_ERR_ARG: return "invalid argument";
    case GPT2_ERR_HIP: return "HIP runtime error";
    case GPT2_ERR_TOKEN_RANGE: return "token id or target out of range";
    case GPT2_ERR_NONFINITE: return "non-finite gradient norm";
    case GPT2_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown error";
  }
}

int gpt2_kernel_count(void) { return K_COUNT; }

const char* gpt2_kernel_name(int id) { return id >= 0 && id < K_COUNT ? kKernelNames[id] : nullptr; }

int gpt2_timing_enable(gpt2_t* h, int kernel_id, int enable) {
  if (!h || kernel_id < 0 || kernel_id >= K_COUNT) return GPT2_ERR_ARG;
  h->timed = enable ? kernel_id : -1;
  return GPT2_OK;
}

int gpt2_timing_read(gpt2_t* h, double* total_ms, int64_t* launches, double* flops) {
  if (!h) return GPT2_ERR_ARG;
  int rc = hip_check(h, hipStreamSynchronize(h->st), "sync");
  if (rc) return rc;
  double ms = 0, fl = 0;
  for (auto& t : h->timings) {
    float e = 0;
    (void)hipEventElapsedTime(&e, t.a, t.b);
    ms += e;
    fl += t.flops;
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  if (total_ms) *total_ms = ms;
  if (launches) *launches = (int64_t)h->timings.size();
  if (flops) *flops = fl;
  h->timings.clear();
  return GPT2_OK;
}

}  // extern "C"
