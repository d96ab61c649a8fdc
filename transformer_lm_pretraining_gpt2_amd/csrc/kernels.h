// kernels.h -- host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt2k {

enum Prec { F32 = 0, BF16 = 1 };

// ---- matmul: out[i][j] = sum_r A(i, r) * B(j, r), i < M, j < N, r < K ------
// A(i, r) = A[i*lda + r] (a_t = 0) or A[r*lda + i] (a_t = 1); same for B.
enum Epi {
  EPI_STORE = 0,    // out (act type) = acc + bias[j]
  EPI_GELU = 1,     // u = acc + bias[j]; out = gelu_tanh(u), aux = gelu_tanh'(u)   (act type; no aux if null)
                    //   preact: aux = u rounded to the act type, out = gelu_tanh(that rounded u)
  EPI_RESID = 2,    // out (fp32) = resid (fp32) + acc + bias[j]
  EPI_GELU_BWD = 3, // out (act type) = acc * aux   (aux = gelu_tanh' at the pre-activation)
                    //   preact: aux = the pre-activation u, out = acc * gelu_tanh'(u)
  EPI_F32 = 4       // out (fp32) = (accumulate ? out : 0) + acc; split s writes out + s*split_stride
};

struct GemmArgs {
  const void* A = nullptr;
  int64_t lda = 0;
  const void* B = nullptr;
  int64_t ldb = 0;
  int M = 0, N = 0, K = 0;
  void* C = nullptr;
  int64_t ldc = 0;
  const float* bias = nullptr;
  const float* resid = nullptr;
  int64_t ldr = 0;
  void* aux = nullptr;
  int64_t ldaux = 0;
  int accumulate = 0;
  int splits = 1;
  int64_t split_stride = 0;
  float alpha = 1.f;  // EPI_STORE / EPI_F32: acc is scaled by alpha before the bias / accumulation
  int preact = 0;     // EPI_GELU / EPI_GELU_BWD: aux holds the pre-activation (activation recompute)
  // gemm_fp8: per-row scales of the FP8 operands, A(i, .) ~= A8(i, .) * scale_a[i]
  // and B(j, .) ~= B8(j, .) * scale_b[j] (device [M] and [N])
  const float* scale_a = nullptr;
  const float* scale_b = nullptr;
  // EPI_F32 with a_t = 1 only: when set, the blocks of the first column tile also
  // write sum_r A(i, r) over their reduction range to colsum[split*colsum_stride + i]
  // (the bias gradient of a weight-gradient product, before the split reduction)
  float* colsum = nullptr;
  int64_t colsum_stride = 0;
};

hipError_t gemm(hipStream_t st, Prec p, int a_t, int b_t, int epi, const GemmArgs& g);
// Up to kMaxGemmGroup weight-gradient products (a_t = b_t = 1, EPI_F32, bf16,
// each with its own splits and optional column sums) in one launch.
constexpr int kMaxGemmGroup = 4;
struct GemmGroup {
  GemmArgs p[kMaxGemmGroup];
  int block0[kMaxGemmGroup + 1];  // filled in by gemm_group
  int count;
};
hipError_t gemm_group(hipStream_t st, const GemmArgs* probs, int count);
// split-K factor of a product inside a group of products whose output tiles
// total `group_tiles` (one round of blocks over the chip)
int gemm_group_split_hint(int M, int N, int K, int group_tiles);
int gemm_group_tiles(int M, int N);
// forward product (a_t = b_t = 0) with FP8 E4M3 operands A, B (bytes) and
// bf16 / fp32 outputs as in gemm; acc(i, j) is multiplied by scale_a[i] * scale_b[j]
hipError_t gemm_fp8(hipStream_t st, int epi, const GemmArgs& g);
// split-K factor that fills the chip for an M x N x K weight-gradient product
int gemm_split_hint(Prec p, int a_t, int b_t, int M, int N, int K);

// ---- attention (causal, packed qkv [B*T, 3C]: q heads | k heads | v heads) ----
hipError_t attn_fwd(hipStream_t st, Prec p, const void* qkv, void* out, float* lse, int B, int T, int NH, int hd);
// backward in two launches: dQ (which also stores D = rowsum(dout * out) in
// dsum [B, NH, T]), then dK,dV (which reads D)
hipError_t attn_bwd_dq(hipStream_t st, Prec p, const void* qkv, const void* out, const void* dout, const float* lse,
                       float* dsum, void* dqkv, int B, int T, int NH, int hd);
hipError_t attn_bwd_dkv(hipStream_t st, Prec p, const void* qkv, const void* dout, const float* lse, const float* dsum,
                        void* dqkv, int B, int T, int NH, int hd);

// ---- LayerNorm ----
// y8/s8 (optional, C a multiple of 256): FP8 E4M3 copy of the output rows with
// one scale per row (y ~= y8 * s8[row])
hipError_t layernorm_fwd(hipStream_t st, Prec p, const float* x, const float* g, const float* b, void* y, float* mean,
                         float* rstd, int M, int C, unsigned char* y8 = nullptr, float* s8 = nullptr);
// dres (+)= LN backward(dy); also writes dres_lp (act-type copy of dres) when p == BF16,
// and per-block partials of dgamma/dbeta into part [nblk][2C].
hipError_t layernorm_bwd(hipStream_t st, Prec p, const void* dy, const float* x, const float* mean, const float* rstd,
                         const float* g, float* dres, void* dres_lp, int accumulate, float* part, int M, int C,
                         int* nparts);
int layernorm_bwd_parts(int M);

// out[j] = [out[j] +] sum_{p < nparts} part[p*ld + j] for j < n (n, ld multiples
// of 4), partials added in order; up to kMaxReduceJobs independent jobs per launch.
constexpr int kMaxReduceJobs = 16;
struct ReduceJob {
  const float* part = nullptr;
  int64_t ld = 0;
  float* out = nullptr;
  int n = 0, nparts = 0, accumulate = 0;
  int block0 = 0;  // filled in by reduce_jobs
};
struct ReduceJobs {
  ReduceJob j[kMaxReduceJobs];
  int count;
};
hipError_t reduce_jobs(hipStream_t st, const ReduceJob* jobs, int count);

// ---- embeddings ----
hipError_t embed_fwd(hipStream_t st, const int32_t* idx, const int32_t* tgt, const float* wte, const float* wpe,
                     float* x, int B, int T, int C, int V, int* err_flag);
// stable sort of ids with their positions; segment starts of equal ids
hipError_t embed_sort(hipStream_t st, const int32_t* idx, int M, int V, int32_t* keys_a, int32_t* vals_a,
                      int32_t* keys_b, int32_t* vals_b, int32_t* seg_start, int32_t* nseg);
// piece: fp32 scratch [B*T, C]
hipError_t embed_bwd(hipStream_t st, const float* dx, const int32_t* sorted_ids, const int32_t* sorted_pos,
                     const int32_t* seg_start, const int32_t* nseg, float* dwte, float* dwpe, float* piece, int B,
                     int T, int Tmax, int C, int V, int accumulate_wpe);

// ---- softmax cross-entropy over the real vocabulary, dlogits in place ----
hipError_t cross_entropy(hipStream_t st, Prec p, void* logits, const int32_t* tgt, float* row_loss, int M, int V, int Vp,
                         float dscale, int write_grad);
hipError_t mean_loss(hipStream_t st, const float* row_loss, int M, float* out);

// ---- optimizer ----
// fp64 partial sums of the gradient norm: one per block of the first pass,
// every one written by each call (so a reused buffer needs no clearing)
constexpr int kGradNormParts = 1024;
inline int grad_norm_parts() { return kGradNormParts; }
hipError_t grad_norm(hipStream_t st, const float* g, int64_t n, double* part, float clip, float* norm_out,
                     float* scale_out, int* err_flag);
// AdamW over the flat buffer; indices < n_decay take weight decay.  g is
// multiplied by *scale (clip factor); nothing is written when *skip != 0.
hipError_t adamw(hipStream_t st, float* p, const float* g, float* m, float* v, void* p_lp, int64_t n, int64_t n_decay,
                 float lr, float b1, float b2, float eps, float wd, float bc1, float bc2, const float* scale,
                 const int* skip);
// bf16 copy of fp32 values
hipError_t to_bf16(hipStream_t st, const float* src, void* dst, int64_t n);
// Transposed copies of `count` bf16 matrices [rows][cols], the z-th at
// in + z * in_stride (elements), into out[z][cols][rows] (contiguous).
// rows and cols multiples of 64.
hipError_t transpose_bf16(hipStream_t st, const void* in, int64_t in_stride, void* out, int rows, int cols, int count);
// FP8 E4M3 copies of bf16 rows with one scale per row (x ~= q * scale[row]):
// scale = max|row| / 448, q = round(x / scale).  K a multiple of 8, <= 4096.
hipError_t quant_rows(hipStream_t st, const void* x, unsigned char* q, float* scale, int rows, int K);
constexpr int kMaxQuantJobs = 64;
struct QuantJob {
  const __bf16* in = nullptr;
  unsigned char* out = nullptr;
  float* scale = nullptr;
  int rows = 0, cols = 0;
  int row0 = 0;  // filled in by quant_jobs
};
struct QuantJobs {
  QuantJob j[kMaxQuantJobs];
  int count;
};
// several matrices in one launch (the weights' per-output-channel copies)
hipError_t quant_jobs(hipStream_t st, const QuantJob* jobs, int count);
// out = gelu_tanh(u) elementwise in the act type (n a multiple of 8)
hipError_t gelu_fwd(hipStream_t st, Prec p, const void* u, void* out, int64_t n);

}  // namespace gpt2k
