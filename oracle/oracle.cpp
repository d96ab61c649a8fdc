/*
 * oracle.cpp -- a plain, slow CPU implementation of one GPT-2 training step:
 * forward pass, mean cross-entropy loss, analytic backward pass, global
 * gradient-norm clipping and AdamW.
 *
 * TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the benchmark's CPU
 * baseline use it to check the HIP library against a definition that a reader
 * can verify by eye.  It shares no code, header or table with the HIP library
 * and the product path never loads it.
 *
 * Every routine is a template on the real type R: double is the parity
 * reference and serves the finite-difference tests, float is the plain fp32
 * variant timed as the CPU baseline.  Loops follow the textbook definitions.
 * OpenMP only splits independent output elements; each output is summed
 * serially in a fixed order, so results do not depend on the thread count.
 *
 * Pages this follows (cited by title and section):
 *  [llm.c]    "Reproducing GPT-2 (124M) cheaply with llm.c" (GeekNews topic 15065)
 *  [story]    "A small GPT that writes fairy tales" (lm-book, TinyStories training chapter)
 *  [video]    "Karpathy's four-hour GPT-2 reproduction in one post" (sotaaz.com)
 *
 * Readings where the pages are silent (each one is also listed in the design
 * notes): pre-LN blocks plus a final LN; LayerNorm eps 1e-5 with the biased
 * variance; attention scale 1/sqrt(head_dim) with key j visible to query i iff
 * j <= i; tanh-approximate GELU with the published constants sqrt(2/pi) and
 * 0.044715; softmax over the real vocabulary [0, V) only (padded rows of the
 * tied matrix never reach the loss); loss = mean over all B*T positions;
 * clipping scales by clip/norm when norm > clip; AdamW with bias correction,
 * eps outside the square root and decoupled, lr-scaled weight decay applied to
 * the pre-update parameter.
 *
 * Every function here is pinned by a CPU test; no function is "parity unpinned".
 */
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <vector>
#include <algorithm>

namespace {

struct Cfg {
  int V, Vp, L, NH, C, Tmax;
};

Cfg cfg_from(const int32_t* c) { return Cfg{c[0], c[1], c[2], c[3], c[4], c[5]}; }

bool cfg_ok(const Cfg& c) {
  return c.V > 0 && c.Vp >= c.V && c.L > 0 && c.NH > 0 && c.C > 0 && c.C % c.NH == 0 && c.Tmax > 0;
}

/* ---------------------------------------------------------------------------
 * Parameter set and its flat order.
 * The tensors are those of GPT-2 ([video] part 1: HF-compatible names, the
 * token embedding shared with the output layer): token embedding wte [Vp, C],
 * learned positions wpe [Tmax, C], per block ln_1 (gain, bias), qkv [3C, C] +
 * bias, attention output projection [C, C] + bias, ln_2, MLP up [4C, C] + bias,
 * MLP down [C, 4C] + bias, and a final ln_f.  The count closed form
 * Vp*C + Tmax*C + L*(12C^2 + 13C) + 2C matches the counts the [story] log
 * prints.  Linear weights are stored [out, in].
 * The 2-D tensors (which take weight decay, [video] part 3) come first so the
 * decayed set is one contiguous prefix.
 * ------------------------------------------------------------------------- */
enum Kind { WTE, WPE, QKV_W, PROJ_W, FC_W, FCPROJ_W, LN1_G, LN1_B, QKV_B, PROJ_B, LN2_G, LN2_B, FC_B, FCPROJ_B, LNF_G, LNF_B };

struct Entry {
  char name[32];
  int kind, layer;
  int64_t offset;
  int rows, cols;  // cols == 0 for 1-D tensors
  int decay;
};

std::vector<Entry> layout(const Cfg& c) {
  std::vector<Entry> e;
  int64_t off = 0;
  auto add = [&](const char* base, int kind, int layer, int rows, int cols, int decay) {
    Entry x{};
    if (layer >= 0) snprintf(x.name, sizeof x.name, "h.%d.%s", layer, base);
    else snprintf(x.name, sizeof x.name, "%s", base);
    x.kind = kind; x.layer = layer; x.offset = off; x.rows = rows; x.cols = cols; x.decay = decay;
    off += (int64_t)rows * (cols ? cols : 1);
    e.push_back(x);
  };
  const int C = c.C;
  add("wte", WTE, -1, c.Vp, C, 1);
  add("wpe", WPE, -1, c.Tmax, C, 1);
  for (int l = 0; l < c.L; l++) {
    add("attn.c_attn.weight", QKV_W, l, 3 * C, C, 1);
    add("attn.c_proj.weight", PROJ_W, l, C, C, 1);
    add("mlp.c_fc.weight", FC_W, l, 4 * C, C, 1);
    add("mlp.c_proj.weight", FCPROJ_W, l, C, 4 * C, 1);
  }
  for (int l = 0; l < c.L; l++) {
    add("ln_1.weight", LN1_G, l, C, 0, 0);
    add("ln_1.bias", LN1_B, l, C, 0, 0);
    add("attn.c_attn.bias", QKV_B, l, 3 * C, 0, 0);
    add("attn.c_proj.bias", PROJ_B, l, C, 0, 0);
    add("ln_2.weight", LN2_G, l, C, 0, 0);
    add("ln_2.bias", LN2_B, l, C, 0, 0);
    add("mlp.c_fc.bias", FC_B, l, 4 * C, 0, 0);
    add("mlp.c_proj.bias", FCPROJ_B, l, C, 0, 0);
  }
  add("ln_f.weight", LNF_G, -1, C, 0, 0);
  add("ln_f.bias", LNF_B, -1, C, 0, 0);
  return e;
}

int64_t total_params(const Cfg& c) {
  auto e = layout(c);
  const Entry& last = e.back();
  return last.offset + last.rows;
}

/* Pointers into a flat parameter (or gradient) array. */
template <typename R>
struct Params {
  R *wte, *wpe, *lnf_g, *lnf_b;
  std::vector<R*> qkv_w, proj_w, fc_w, fcproj_w, ln1_g, ln1_b, qkv_b, proj_b, ln2_g, ln2_b, fc_b, fcproj_b;
  Params(const Cfg& c, R* base) {
    auto e = layout(c);
    int L = c.L;
    for (auto* v : {&qkv_w, &proj_w, &fc_w, &fcproj_w, &ln1_g, &ln1_b, &qkv_b, &proj_b, &ln2_g, &ln2_b, &fc_b, &fcproj_b})
      v->assign(L, nullptr);
    for (auto& x : e) {
      R* p = base + x.offset;
      switch (x.kind) {
        case WTE: wte = p; break;
        case WPE: wpe = p; break;
        case QKV_W: qkv_w[x.layer] = p; break;
        case PROJ_W: proj_w[x.layer] = p; break;
        case FC_W: fc_w[x.layer] = p; break;
        case FCPROJ_W: fcproj_w[x.layer] = p; break;
        case LN1_G: ln1_g[x.layer] = p; break;
        case LN1_B: ln1_b[x.layer] = p; break;
        case QKV_B: qkv_b[x.layer] = p; break;
        case PROJ_B: proj_b[x.layer] = p; break;
        case LN2_G: ln2_g[x.layer] = p; break;
        case LN2_B: ln2_b[x.layer] = p; break;
        case FC_B: fc_b[x.layer] = p; break;
        case FCPROJ_B: fcproj_b[x.layer] = p; break;
        case LNF_G: lnf_g = p; break;
        case LNF_B: lnf_b = p; break;
      }
    }
  }
};

/* ---------------------------------------------------------------------------
 * Building blocks.
 * ------------------------------------------------------------------------- */

/* Linear layer y[m][n] = b[n] + sum_k x[m][k] * W[n][k]  (W stored [N, K]).
 * W is first copied to [K, N] so the loop over independent outputs n is
 * contiguous; each output is still summed over k = 0..K-1 in order. */
template <typename R>
void linear_fwd(R* y, const R* x, const R* W, const R* b, int M, int N, int K) {
  std::vector<R> Wt((size_t)K * N);
#pragma omp parallel for schedule(static)
  for (int k = 0; k < K; k++)
    for (int n = 0; n < N; n++) Wt[(size_t)k * N + n] = W[(size_t)n * K + k];
#pragma omp parallel for schedule(static)
  for (int m = 0; m < M; m++) {
    R* yr = y + (size_t)m * N;
    for (int n = 0; n < N; n++) yr[n] = b ? b[n] : R(0);
    const R* xr = x + (size_t)m * K;
    for (int k = 0; k < K; k++) {
      const R a = xr[k];
      const R* wr = &Wt[(size_t)k * N];
      for (int n = 0; n < N; n++) yr[n] += a * wr[n];
    }
  }
}

/* Backward of linear_fwd: dx[m][k] = sum_n dy[m][n] W[n][k] (overwrites dx),
 * dW[n][k] += sum_m dy[m][n] x[m][k], db[n] += sum_m dy[m][n]. */
template <typename R>
void linear_bwd(R* dx, R* dW, R* db, const R* dy, const R* x, const R* W, int M, int N, int K) {
  if (dx) {
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; m++) {
      R* dxr = dx + (size_t)m * K;
      for (int k = 0; k < K; k++) dxr[k] = R(0);
      const R* dyr = dy + (size_t)m * N;
      for (int n = 0; n < N; n++) {
        const R a = dyr[n];
        const R* wr = W + (size_t)n * K;
        for (int k = 0; k < K; k++) dxr[k] += a * wr[k];
      }
    }
  }
  if (dW) {
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
      std::vector<R> acc(K, R(0));
      for (int m = 0; m < M; m++) {
        const R a = dy[(size_t)m * N + n];
        const R* xr = x + (size_t)m * K;
        for (int k = 0; k < K; k++) acc[k] += a * xr[k];
      }
      R* dwr = dW + (size_t)n * K;
      for (int k = 0; k < K; k++) dwr[k] += acc[k];
    }
  }
  if (db) {
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++) {
      R s = 0;
      for (int m = 0; m < M; m++) s += dy[(size_t)m * N + n];
      db[n] += s;
    }
  }
}

/* LayerNorm over the last dimension: mean and biased variance over C,
 * y = (x - mean) / sqrt(var + eps) * g + b. */
template <typename R>
void layernorm_fwd(R* y, R* mean, R* rstd, const R* x, const R* g, const R* b, int M, int C, R eps) {
#pragma omp parallel for schedule(static)
  for (int m = 0; m < M; m++) {
    const R* xr = x + (size_t)m * C;
    R s = 0;
    for (int c = 0; c < C; c++) s += xr[c];
    const R mu = s / C;
    R v = 0;
    for (int c = 0; c < C; c++) v += (xr[c] - mu) * (xr[c] - mu);
    v /= C;
    const R rs = R(1) / std::sqrt(v + eps);
    R* yr = y + (size_t)m * C;
    for (int c = 0; c < C; c++) yr[c] = (xr[c] - mu) * rs * g[c] + b[c];
    if (mean) mean[m] = mu;
    if (rstd) rstd[m] = rs;
  }
}

/* Backward of layernorm_fwd.  With xhat = (x-mean)*rstd and d = dy*g:
 * dx = rstd * (d - mean_c(d) - xhat * mean_c(d*xhat)), added into dx;
 * dg += sum_m dy*xhat, db += sum_m dy. */
template <typename R>
void layernorm_bwd(R* dx, R* dg, R* db, const R* dy, const R* x, const R* mean, const R* rstd, const R* g, int M, int C) {
#pragma omp parallel for schedule(static)
  for (int m = 0; m < M; m++) {
    const R* xr = x + (size_t)m * C;
    const R* dyr = dy + (size_t)m * C;
    const R mu = mean[m], rs = rstd[m];
    R sd = 0, sdx = 0;
    for (int c = 0; c < C; c++) {
      const R xh = (xr[c] - mu) * rs;
      const R d = dyr[c] * g[c];
      sd += d;
      sdx += d * xh;
    }
    sd /= C;
    sdx /= C;
    R* dxr = dx + (size_t)m * C;
    for (int c = 0; c < C; c++) {
      const R xh = (xr[c] - mu) * rs;
      const R d = dyr[c] * g[c];
      dxr[c] += rs * (d - sd - xh * sdx);
    }
  }
#pragma omp parallel for schedule(static)
  for (int c = 0; c < C; c++) {
    R sg = 0, sb = 0;
    for (int m = 0; m < M; m++) {
      const R xh = (x[(size_t)m * C + c] - mean[m]) * rstd[m];
      sg += dy[(size_t)m * C + c] * xh;
      sb += dy[(size_t)m * C + c];
    }
    dg[c] += sg;
    db[c] += sb;
  }
}

/* tanh-approximate GELU ([video], "what I checked myself": GPT-2 uses the tanh
 * approximation, not the exact erf form):
 * gelu(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). */
template <typename R>
R gelu(R x) {
  const R k = std::sqrt(R(2) / R(M_PI));
  return R(0.5) * x * (R(1) + std::tanh(k * (x + R(0.044715) * x * x * x)));
}

/* d gelu / dx = 0.5 (1 + t) + 0.5 x (1 - t^2) sqrt(2/pi) (1 + 3*0.044715 x^2), t = tanh(...). */
template <typename R>
R gelu_grad(R x) {
  const R k = std::sqrt(R(2) / R(M_PI));
  const R t = std::tanh(k * (x + R(0.044715) * x * x * x));
  return R(0.5) * (R(1) + t) + R(0.5) * x * (R(1) - t * t) * k * (R(1) + R(3) * R(0.044715) * x * x);
}

/* Causal softmax probabilities of query i of one head: p[j] for j <= i.
 * q, k rows are hd long; rows of k are `stride` apart. */
template <typename R>
void attn_probs_row(R* p, const R* q, const R* k, int i, int hd, int stride, R scale) {
  R mx = -INFINITY;
  for (int j = 0; j <= i; j++) {
    R s = 0;
    const R* kj = k + (size_t)j * stride;
    for (int d = 0; d < hd; d++) s += q[d] * kj[d];
    p[j] = s * scale;
    mx = std::max(mx, p[j]);
  }
  R sum = 0;
  for (int j = 0; j <= i; j++) {
    p[j] = std::exp(p[j] - mx);
    sum += p[j];
  }
  for (int j = 0; j <= i; j++) p[j] /= sum;
}

/* Causal multi-head self-attention on packed qkv [B*T, 3C] (q heads, then k
 * heads, then v heads): y[b,i,h,:] = sum_{j<=i} softmax_j(q.k/sqrt(hd)) v_j.
 * probs, if given, is [B, NH, T, T] with zeros above the diagonal. */
template <typename R>
void attention_fwd(R* y, R* probs, const R* qkv, int B, int T, int NH, int hd) {
  const int C = NH * hd, S = 3 * C;
  const R scale = R(1) / std::sqrt(R(hd));
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; b++)
    for (int h = 0; h < NH; h++) {
      std::vector<R> p(T);
      const R* base = qkv + (size_t)b * T * S;
      for (int i = 0; i < T; i++) {
        attn_probs_row(p.data(), base + (size_t)i * S + h * hd, base + C + h * hd, i, hd, S, scale);
        R* yr = y + ((size_t)b * T + i) * C + h * hd;
        for (int d = 0; d < hd; d++) {
          R s = 0;
          for (int j = 0; j <= i; j++) s += p[j] * base[(size_t)j * S + 2 * C + h * hd + d];
          yr[d] = s;
        }
        if (probs) {
          R* pr = probs + (((size_t)b * NH + h) * T + i) * T;
          for (int j = 0; j < T; j++) pr[j] = j <= i ? p[j] : R(0);
        }
      }
    }
}

/* Backward of attention_fwd (probabilities recomputed with the same routine):
 * dv_j += p_j dy_i;  dp_j = dy_i . v_j;  ds_j = p_j (dp_j - sum_k p_k dp_k);
 * dq_i = scale sum_j ds_j k_j;  dk_j += scale ds_j q_i.  dqkv is overwritten. */
template <typename R>
void attention_bwd(R* dqkv, const R* dy, const R* qkv, int B, int T, int NH, int hd) {
  const int C = NH * hd, S = 3 * C;
  const R scale = R(1) / std::sqrt(R(hd));
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; b++)
    for (int h = 0; h < NH; h++) {
      std::vector<R> p(T), dp(T);
      const R* base = qkv + (size_t)b * T * S;
      R* dbase = dqkv + (size_t)b * T * S;
      for (int i = 0; i < T; i++)
        for (int d = 0; d < hd; d++) {
          dbase[(size_t)i * S + h * hd + d] = 0;
          dbase[(size_t)i * S + C + h * hd + d] = 0;
          dbase[(size_t)i * S + 2 * C + h * hd + d] = 0;
        }
      for (int i = 0; i < T; i++) {
        const R* qi = base + (size_t)i * S + h * hd;
        attn_probs_row(p.data(), qi, base + C + h * hd, i, hd, S, scale);
        const R* dyi = dy + ((size_t)b * T + i) * C + h * hd;
        R pdp = 0;
        for (int j = 0; j <= i; j++) {
          const R* vj = base + (size_t)j * S + 2 * C + h * hd;
          R s = 0;
          for (int d = 0; d < hd; d++) s += dyi[d] * vj[d];
          dp[j] = s;
          pdp += p[j] * s;
          R* dvj = dbase + (size_t)j * S + 2 * C + h * hd;
          for (int d = 0; d < hd; d++) dvj[d] += p[j] * dyi[d];
        }
        R* dqi = dbase + (size_t)i * S + h * hd;
        for (int j = 0; j <= i; j++) {
          const R ds = p[j] * (dp[j] - pdp) * scale;
          const R* kj = base + (size_t)j * S + C + h * hd;
          R* dkj = dbase + (size_t)j * S + C + h * hd;
          for (int d = 0; d < hd; d++) {
            dqi[d] += ds * kj[d];
            dkj[d] += ds * qi[d];
          }
        }
      }
    }
}

/* Softmax cross-entropy over the real vocabulary [0, V) of rows `ld` apart
 * ([story] problem 3: the loss is nats per token):
 * loss_m = logsumexp(z_m[0:V]) - z_m[y_m];  dz_m[j] = scale * (softmax_j - [j == y_m]).
 * dlogits may be null. */
template <typename R>
void cross_entropy(R* row_loss, R* dlogits, const R* logits, const int32_t* tgt, int M, int V, int ld, R scale) {
#pragma omp parallel for schedule(static)
  for (int m = 0; m < M; m++) {
    const R* z = logits + (size_t)m * ld;
    R mx = -INFINITY;
    for (int j = 0; j < V; j++) mx = std::max(mx, z[j]);
    R s = 0;
    for (int j = 0; j < V; j++) s += std::exp(z[j] - mx);
    const R lse = mx + std::log(s);
    row_loss[m] = lse - z[tgt[m]];
    if (dlogits) {
      R* dz = dlogits + (size_t)m * ld;
      for (int j = 0; j < V; j++) dz[j] = scale * (std::exp(z[j] - lse) - (j == tgt[m] ? R(1) : R(0)));
    }
  }
}

/* ---------------------------------------------------------------------------
 * The whole model.
 * ------------------------------------------------------------------------- */
template <typename R>
struct Acts {
  int B, T, C, L, V;
  std::vector<std::vector<R>> x_in, h1, mean1, rstd1, qkv, atty, x_mid, h2, mean2, rstd2, u, g;
  std::vector<R> x_out, hf, meanf, rstdf, logits;
  Acts(const Cfg& c, int B_, int T_) : B(B_), T(T_), C(c.C), L(c.L), V(c.V) {
    const size_t M = (size_t)B * T;
    auto mk = [&](std::vector<std::vector<R>>& v, size_t n) { v.assign(L, std::vector<R>(n)); };
    mk(x_in, M * C); mk(h1, M * C); mk(mean1, M); mk(rstd1, M); mk(qkv, M * 3 * C); mk(atty, M * C);
    mk(x_mid, M * C); mk(h2, M * C); mk(mean2, M); mk(rstd2, M); mk(u, M * 4 * C); mk(g, M * 4 * C);
    x_out.resize(M * C); hf.resize(M * C); meanf.resize(M); rstdf.resize(M); logits.resize(M * (size_t)V);
  }
};

const double LN_EPS = 1e-5;

/* Forward pass ([video] part 1 for the tied embedding/head; pre-LN blocks).
 * Returns the mean loss; row_loss gets the per-position losses. */
template <typename R>
R forward(Acts<R>& a, const Cfg& c, const Params<R>& P, const int32_t* ids, const int32_t* tgt, R* row_loss) {
  const int B = a.B, T = a.T, C = c.C, M = B * T;
  const int hd = C / c.NH;
  // token + position embedding
  {
    R* x = a.x_in[0].data();
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; m++) {
      const int t = m % T;
      for (int ch = 0; ch < C; ch++) x[(size_t)m * C + ch] = P.wte[(size_t)ids[m] * C + ch] + P.wpe[(size_t)t * C + ch];
    }
  }
  for (int l = 0; l < c.L; l++) {
    const R* x = a.x_in[l].data();
    layernorm_fwd(a.h1[l].data(), a.mean1[l].data(), a.rstd1[l].data(), x, P.ln1_g[l], P.ln1_b[l], M, C, R(LN_EPS));
    linear_fwd(a.qkv[l].data(), a.h1[l].data(), P.qkv_w[l], P.qkv_b[l], M, 3 * C, C);
    attention_fwd(a.atty[l].data(), (R*)nullptr, a.qkv[l].data(), B, T, c.NH, hd);
    std::vector<R> tmp((size_t)M * C);
    linear_fwd(tmp.data(), a.atty[l].data(), P.proj_w[l], P.proj_b[l], M, C, C);
    R* xm = a.x_mid[l].data();
    for (size_t i = 0; i < (size_t)M * C; i++) xm[i] = x[i] + tmp[i];
    layernorm_fwd(a.h2[l].data(), a.mean2[l].data(), a.rstd2[l].data(), xm, P.ln2_g[l], P.ln2_b[l], M, C, R(LN_EPS));
    linear_fwd(a.u[l].data(), a.h2[l].data(), P.fc_w[l], P.fc_b[l], M, 4 * C, C);
    R* u = a.u[l].data();
    R* g = a.g[l].data();
    for (size_t i = 0; i < (size_t)M * 4 * C; i++) g[i] = gelu(u[i]);
    linear_fwd(tmp.data(), g, P.fcproj_w[l], P.fcproj_b[l], M, C, 4 * C);
    R* xo = (l + 1 < c.L) ? a.x_in[l + 1].data() : a.x_out.data();
    for (size_t i = 0; i < (size_t)M * C; i++) xo[i] = xm[i] + tmp[i];
  }
  layernorm_fwd(a.hf.data(), a.meanf.data(), a.rstdf.data(), a.x_out.data(), P.lnf_g, P.lnf_b, M, C, R(LN_EPS));
  // tied head over the real vocabulary rows of wte
  linear_fwd(a.logits.data(), a.hf.data(), P.wte, (const R*)nullptr, M, c.V, C);
  std::vector<R> rl(M);
  cross_entropy(rl.data(), (R*)nullptr, a.logits.data(), tgt, M, c.V, c.V, R(0));
  R s = 0;
  for (int m = 0; m < M; m++) s += rl[m];
  if (row_loss)
    for (int m = 0; m < M; m++) row_loss[m] = rl[m];
  return s / M;
}

/* Backward pass: adds grad_scale * d(mean loss)/d(theta) into G.  With
 * grad_scale = 1/K for each of K micro-batches the sum is the gradient of the
 * mean loss over all K*B*T positions ([video] part 3: each micro-batch loss is
 * divided by the number of micro-batches). */
template <typename R>
void backward(Acts<R>& a, const Cfg& c, const Params<R>& P, Params<R>& G, const int32_t* ids, const int32_t* tgt, R grad_scale) {
  const int B = a.B, T = a.T, C = c.C, M = B * T;
  const int hd = C / c.NH;
  std::vector<R> rl(M), dz((size_t)M * c.V);
  cross_entropy(rl.data(), dz.data(), a.logits.data(), tgt, M, c.V, c.V, grad_scale / R(M));
  std::vector<R> dhf((size_t)M * C), dx((size_t)M * C, R(0));
  // tied head: the LM-head contribution to wte's gradient
  linear_bwd(dhf.data(), G.wte, (R*)nullptr, dz.data(), a.hf.data(), P.wte, M, c.V, C);
  dz.clear();
  dz.shrink_to_fit();
  layernorm_bwd(dx.data(), G.lnf_g, G.lnf_b, dhf.data(), a.x_out.data(), a.meanf.data(), a.rstdf.data(), P.lnf_g, M, C);
  std::vector<R> dg((size_t)M * 4 * C), dh((size_t)M * C), datty((size_t)M * C), dqkv((size_t)M * 3 * C);
  for (int l = c.L - 1; l >= 0; l--) {
    // dx holds dL/d(block output).  MLP branch: out = x_mid + fcproj(gelu(fc(ln2(x_mid))))
    linear_bwd(dg.data(), G.fcproj_w[l], G.fcproj_b[l], dx.data(), a.g[l].data(), P.fcproj_w[l], M, C, 4 * C);
    const R* u = a.u[l].data();
    for (size_t i = 0; i < (size_t)M * 4 * C; i++) dg[i] *= gelu_grad(u[i]);
    linear_bwd(dh.data(), G.fc_w[l], G.fc_b[l], dg.data(), a.h2[l].data(), P.fc_w[l], M, 4 * C, C);
    layernorm_bwd(dx.data(), G.ln2_g[l], G.ln2_b[l], dh.data(), a.x_mid[l].data(), a.mean2[l].data(), a.rstd2[l].data(), P.ln2_g[l], M, C);
    // attention branch: x_mid = x_in + proj(attn(ln1(x_in)))
    linear_bwd(datty.data(), G.proj_w[l], G.proj_b[l], dx.data(), a.atty[l].data(), P.proj_w[l], M, C, C);
    attention_bwd(dqkv.data(), datty.data(), a.qkv[l].data(), B, T, c.NH, hd);
    linear_bwd(dh.data(), G.qkv_w[l], G.qkv_b[l], dqkv.data(), a.h1[l].data(), P.qkv_w[l], M, 3 * C, C);
    layernorm_bwd(dx.data(), G.ln1_g[l], G.ln1_b[l], dh.data(), a.x_in[l].data(), a.mean1[l].data(), a.rstd1[l].data(), P.ln1_g[l], M, C);
  }
  // embeddings: dwpe[t] += sum_b dx[b,t]; dwte[id] += dx (positions in order)
#pragma omp parallel for schedule(static)
  for (int ch = 0; ch < C; ch++) {
    for (int m = 0; m < M; m++) {
      G.wpe[(size_t)(m % T) * C + ch] += dx[(size_t)m * C + ch];
      G.wte[(size_t)ids[m] * C + ch] += dx[(size_t)m * C + ch];
    }
  }
}

/* Global L2 norm over all gradients, summed in index order. */
template <typename R>
R grad_norm(const R* g, int64_t n) {
  R s = 0;
  for (int64_t i = 0; i < n; i++) s += g[i] * g[i];
  return std::sqrt(s);
}

/* Gradient clipping by global norm ([video] part 3: norm clipped to 1.0;
 * [llm.c] training progress: clipping tames the early gradient blow-ups).
 * Returns the pre-clip norm. */
template <typename R>
R clip_grads(R* g, int64_t n, R clip) {
  const R norm = grad_norm(g, n);
  if (norm > clip) {
    const R s = clip / norm;
    for (int64_t i = 0; i < n; i++) g[i] *= s;
  }
  return norm;
}

/* AdamW ([video] part 3: betas (0.9, 0.95), eps 1e-8, weight decay 0.1 on 2-D
 * tensors only -- matmul weights and embeddings -- and never on biases or
 * LayerNorm gains).  Step t >= 1:
 * m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 * p -= lr * ( (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps) + wd * [2-D] * p ). */
template <typename R>
void adamw(const Cfg& c, R* p, const R* g, R* m, R* v, int t, R lr, R b1, R b2, R eps, R wd) {
  const R bc1 = R(1) - std::pow(b1, R(t));
  const R bc2 = R(1) - std::pow(b2, R(t));
  for (auto& e : layout(c)) {
    const int64_t n = (int64_t)e.rows * (e.cols ? e.cols : 1);
    const R w = e.decay ? wd : R(0);
#pragma omp parallel for schedule(static)
    for (int64_t i = e.offset; i < e.offset + n; i++) {
      m[i] = b1 * m[i] + (R(1) - b1) * g[i];
      v[i] = b2 * v[i] + (R(1) - b2) * g[i] * g[i];
      const R mh = m[i] / bc1;
      const R vh = v[i] / bc2;
      p[i] -= lr * (mh / (std::sqrt(vh) + eps) + w * p[i]);
    }
  }
}

template <typename R>
int check_ids(const Cfg& c, int B, int T, const int32_t* ids, const int32_t* tgt) {
  if (B <= 0 || T <= 0 || T > c.Tmax) return -2;
  for (int64_t i = 0; i < (int64_t)B * T; i++) {
    if (ids[i] < 0 || ids[i] >= c.V) return -3;
    if (tgt && (tgt[i] < 0 || tgt[i] >= c.V)) return -3;
  }
  return 0;
}

template <typename R>
R fwd_bwd(const int32_t* cfg, int B, int T, const R* params, const int32_t* ids, const int32_t* tgt, R grad_scale, R* grads, R* row_loss) {
  const Cfg c = cfg_from(cfg);
  if (!cfg_ok(c) || check_ids<R>(c, B, T, ids, tgt) != 0) return R(NAN);
  Acts<R> a(c, B, T);
  Params<R> P(c, const_cast<R*>(params));
  R loss = forward(a, c, P, ids, tgt, row_loss);
  if (grads) {
    Params<R> G(c, grads);
    backward(a, c, P, G, ids, tgt, grad_scale);
  }
  return loss;
}

}  // namespace

/* ---------------------------------------------------------------------------
 * C API (used from Python through ctypes).  cfg is int32[6]:
 * {vocab_size, padded_vocab_size, n_layer, n_head, n_embd, max_seq_len}.
 * ------------------------------------------------------------------------- */
extern "C" {

int64_t oracle_num_params(const int32_t* cfg) {
  Cfg c = cfg_from(cfg);
  return cfg_ok(c) ? total_params(c) : -1;
}

int oracle_num_tensors(const int32_t* cfg) {
  Cfg c = cfg_from(cfg);
  return cfg_ok(c) ? (int)layout(c).size() : -1;
}

/* Tensor i of the flat layout: name (NUL-terminated, <= 31 chars), offset,
 * rows, cols (0 for 1-D), decay flag. */
int oracle_tensor(const int32_t* cfg, int i, char* name, int64_t* offset, int32_t* rows, int32_t* cols, int32_t* decay) {
  Cfg c = cfg_from(cfg);
  if (!cfg_ok(c)) return -1;
  auto e = layout(c);
  if (i < 0 || i >= (int)e.size()) return -1;
  memcpy(name, e[i].name, 32);
  *offset = e[i].offset;
  *rows = e[i].rows;
  *cols = e[i].cols;
  *decay = e[i].decay;
  return 0;
}

#define ORACLE_API(R, SFX)                                                                                          \
  R oracle_##SFX##_fwd_bwd(const int32_t* cfg, int B, int T, const R* params, const int32_t* ids, const int32_t* tgt, \
                           R grad_scale, R* grads, R* row_loss) {                                                   \
    return fwd_bwd<R>(cfg, B, T, params, ids, tgt, grad_scale, grads, row_loss);                                    \
  }                                                                                                                  \
  R oracle_##SFX##_grad_norm(const R* g, int64_t n) { return grad_norm<R>(g, n); }                                   \
  R oracle_##SFX##_clip_grads(R* g, int64_t n, R clip) { return clip_grads<R>(g, n, clip); }                        \
  int oracle_##SFX##_adamw(const int32_t* cfg, R* p, const R* g, R* m, R* v, int t, R lr, R b1, R b2, R eps, R wd) { \
    Cfg c = cfg_from(cfg);                                                                                           \
    if (!cfg_ok(c) || t < 1) return -1;                                                                              \
    adamw<R>(c, p, g, m, v, t, lr, b1, b2, eps, wd);                                                                 \
    return 0;                                                                                                        \
  }                                                                                                                  \
  void oracle_##SFX##_linear(R* y, const R* x, const R* W, const R* b, int M, int N, int K) {                        \
    linear_fwd<R>(y, x, W, b, M, N, K);                                                                              \
  }                                                                                                                  \
  void oracle_##SFX##_linear_bwd(R* dx, R* dW, R* db, const R* dy, const R* x, const R* W, int M, int N, int K) {    \
    linear_bwd<R>(dx, dW, db, dy, x, W, M, N, K);                                                                    \
  }                                                                                                                  \
  void oracle_##SFX##_layernorm(R* y, R* mean, R* rstd, const R* x, const R* g, const R* b, int M, int C, R eps) {   \
    layernorm_fwd<R>(y, mean, rstd, x, g, b, M, C, eps);                                                             \
  }                                                                                                                  \
  void oracle_##SFX##_layernorm_bwd(R* dx, R* dg, R* db, const R* dy, const R* x, const R* mean, const R* rstd,      \
                                    const R* g, int M, int C) {                                                      \
    layernorm_bwd<R>(dx, dg, db, dy, x, mean, rstd, g, M, C);                                                        \
  }                                                                                                                  \
  void oracle_##SFX##_gelu(R* y, R* dydx, const R* x, int64_t n) {                                                   \
    for (int64_t i = 0; i < n; i++) {                                                                                \
      if (y) y[i] = gelu<R>(x[i]);                                                                                   \
      if (dydx) dydx[i] = gelu_grad<R>(x[i]);                                                                        \
    }                                                                                                                \
  }                                                                                                                  \
  void oracle_##SFX##_attention(R* y, R* probs, const R* qkv, int B, int T, int NH, int hd) {                        \
    attention_fwd<R>(y, probs, qkv, B, T, NH, hd);                                                                   \
  }                                                                                                                  \
  void oracle_##SFX##_attention_bwd(R* dqkv, const R* dy, const R* qkv, int B, int T, int NH, int hd) {              \
    attention_bwd<R>(dqkv, dy, qkv, B, T, NH, hd);                                                                   \
  }                                                                                                                  \
  void oracle_##SFX##_cross_entropy(R* row_loss, R* dlogits, const R* logits, const int32_t* tgt, int M, int V,      \
                                    int ld, R scale) {                                                               \
    cross_entropy<R>(row_loss, dlogits, logits, tgt, M, V, ld, scale);                                               \
  }

ORACLE_API(double, f64)
ORACLE_API(float, f32)

}  // extern "C"
