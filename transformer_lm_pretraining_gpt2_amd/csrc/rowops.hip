// rowops.hip -- the memory-bound kernels of the GPT-2 step on gfx950:
// LayerNorm forward/backward, column sums, embeddings (forward gather and a
// deterministic sorted scatter-add backward), the fused softmax
// cross-entropy, the global gradient norm and AdamW.
//
// Every reduction runs in a fixed order (wave butterflies, then wave partials
// summed in index order, then block partials summed in index order by a
// second kernel), so results are bitwise reproducible; no kernel uses
// floating-point atomics.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace gpt2k {
namespace {

template <typename T> struct Pair;
template <> struct Pair<bf16> { typedef bf16 __attribute__((ext_vector_type(2))) type; };
template <> struct Pair<float> { typedef float __attribute__((ext_vector_type(2))) type; };
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// LayerNorm forward: one wave per row; mean and biased variance over C,
// y = (x - mean) * rstd * g + b, rstd = 1/sqrt(var + 1e-5).
// Lane l holds elements VE*l + 64*VE*k .. +VE-1 (k < C / (64*VE)): 16-byte
// loads (VE = 4) when C is a multiple of 256, else VE = 2.
// ---------------------------------------------------------------------------
// FP8 E4M3 quantization of one row held by a wave: scale = amax / 448 (the
// largest finite E4M3 value), q = round(v / scale) clamped to +-448 (the
// conversion does not saturate).  A zero row gets scale 1.
__device__ __forceinline__ float fp8_row_scale(float amax) { return amax > 0.f ? amax * (1.f / 448.f) : 1.f; }
__device__ __forceinline__ unsigned fp8_pack4(float a, float b, float c, float d, float inv) {
  auto cl = [](float t) { return fminf(fmaxf(t, -448.f), 448.f); };
  unsigned p = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a * inv), cl(b * inv), 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(cl(c * inv), cl(d * inv), p, true);
}

template <typename T, int NP>
__global__ void __launch_bounds__(256) ln_fwd_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                     const float* __restrict__ b, T* __restrict__ y,
                                                     float* __restrict__ mean, float* __restrict__ rstd, int M,
                                                     fp8e4* __restrict__ y8, float* __restrict__ s8) {
  constexpr int C = NP * 128;
  constexpr int VE = C % 256 == 0 ? 4 : 2, NC = C / (64 * VE);
  typedef float fv __attribute__((ext_vector_type(VE)));
  typedef T tv __attribute__((ext_vector_type(VE)));
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* xr = x + (int64_t)row * C;
  fv v[NC];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NC; k++) {
    v[k] = *reinterpret_cast<const fv*>(xr + VE * lane + 64 * VE * k);
#pragma unroll
    for (int e = 0; e < VE; e++) s += v[k][e];
  }
  const float mu = wave_sum(s) * (1.f / C);
  float q = 0.f;
#pragma unroll
  for (int k = 0; k < NC; k++)
#pragma unroll
    for (int e = 0; e < VE; e++) {
      const float a = v[k][e] - mu;
      q += a * a;
    }
  const float rs = 1.f / sqrtf(wave_sum(q) * (1.f / C) + 1e-5f);
  T* yr = y + (int64_t)row * C;
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < NC; k++) {
    const int c0 = VE * lane + 64 * VE * k;
    const fv gg = *reinterpret_cast<const fv*>(g + c0);
    const fv bb = *reinterpret_cast<const fv*>(b + c0);
    tv o;
#pragma unroll
    for (int e = 0; e < VE; e++) {
      v[k][e] = (v[k][e] - mu) * rs * gg[e] + bb[e];
      o[e] = from_f<T>(v[k][e]);
      amax = fmaxf(amax, fabsf(v[k][e]));
    }
    *reinterpret_cast<tv*>(yr + c0) = o;
  }
  if (y8) {  // FP8 copy of the output row with its own scale (forward products in FP8)
    if constexpr (VE == 4) {
      amax = wave_max(amax);
      const float sc = fp8_row_scale(amax), inv = 1.f / sc;
#pragma unroll
      for (int k = 0; k < NC; k++) {
        const int c0 = VE * lane + 64 * VE * k;
        *reinterpret_cast<unsigned*>(y8 + (int64_t)row * C + c0) = fp8_pack4(v[k][0], v[k][1], v[k][2], v[k][3], inv);
      }
      if (lane == 0) s8[row] = sc;
    }
  }
  if (lane == 0) {
    mean[row] = mu;
    rstd[row] = rs;
  }
}

// ---------------------------------------------------------------------------
// LayerNorm backward fused with the residual-gradient add.  With
// xhat = (x - mean) rstd and d = dy g:
//   dx = rstd (d - mean_c(d) - xhat mean_c(d xhat));  dres = [dres +] dx
// dgamma = sum_rows dy xhat, dbeta = sum_rows dy: each block writes its
// partial sums (rows visited in a fixed order) to part[block][0:C | C:2C].
// Each wave walks its rows with the next row's inputs already in flight.
// ---------------------------------------------------------------------------
constexpr int LNB_BLOCKS = 512;

template <typename T, int NP>
struct LnRow {
  typedef typename Pair<T>::type P;
  P dy[NP];
  f32x2 x[NP], r[NP];
  float mu, rs;
  __device__ __forceinline__ void load(const T* dyp, const float* xp, const float* rp, const float* mean,
                                       const float* rstd, int row, int lane, int accumulate) {
    constexpr int C = NP * 128;
#pragma unroll
    for (int k = 0; k < NP; k++) {
      const int c0 = 2 * lane + 128 * k;
      dy[k] = *reinterpret_cast<const P*>(dyp + (int64_t)row * C + c0);
      x[k] = *reinterpret_cast<const f32x2*>(xp + (int64_t)row * C + c0);
      if (accumulate) r[k] = *reinterpret_cast<const f32x2*>(rp + (int64_t)row * C + c0);
    }
    mu = mean[row];
    rs = rstd[row];
  }
};

template <typename T, int NP>
__global__ void __launch_bounds__(256) ln_bwd_kernel(const T* __restrict__ dy, const float* __restrict__ x,
                                                     const float* __restrict__ mean, const float* __restrict__ rstd,
                                                     const float* __restrict__ g, float* __restrict__ dres,
                                                     T* __restrict__ dres_lp, int accumulate, float* __restrict__ part,
                                                     int M) {
  typedef typename Pair<T>::type P;
  constexpr int C = NP * 128;
  __shared__ float sh[4][2 * C];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  f32x2 gg[NP], ag[NP], ab[NP];
#pragma unroll
  for (int k = 0; k < NP; k++) {
    gg[k] = *reinterpret_cast<const f32x2*>(g + 2 * lane + 128 * k);
    ag[k] = f32x2{0.f, 0.f};
    ab[k] = f32x2{0.f, 0.f};
  }
  const int stride = gridDim.x * 4;
  int row = blockIdx.x * 4 + w;
  LnRow<T, NP> cur;
  if (row < M) cur.load(dy, x, dres, mean, rstd, row, lane, accumulate);
  while (row < M) {
    const int next = row + stride;
    LnRow<T, NP> nxt;
    if (next < M) nxt.load(dy, x, dres, mean, rstd, next, lane, accumulate);
    f32x2 xh[NP], d[NP];
    float sd = 0.f, sdx = 0.f;
#pragma unroll
    for (int k = 0; k < NP; k++) {
      const float d0 = to_f<T>(cur.dy[k][0]), d1 = to_f<T>(cur.dy[k][1]);
      xh[k] = f32x2{(cur.x[k][0] - cur.mu) * cur.rs, (cur.x[k][1] - cur.mu) * cur.rs};
      ag[k][0] += d0 * xh[k][0];
      ag[k][1] += d1 * xh[k][1];
      ab[k][0] += d0;
      ab[k][1] += d1;
      d[k] = f32x2{d0 * gg[k][0], d1 * gg[k][1]};
      sd += d[k][0] + d[k][1];
      sdx += d[k][0] * xh[k][0] + d[k][1] * xh[k][1];
    }
    sd = wave_sum(sd) * (1.f / C);
    sdx = wave_sum(sdx) * (1.f / C);
    float* rr = dres + (int64_t)row * C;
#pragma unroll
    for (int k = 0; k < NP; k++) {
      const int c0 = 2 * lane + 128 * k;
      f32x2 o{cur.rs * (d[k][0] - sd - xh[k][0] * sdx), cur.rs * (d[k][1] - sd - xh[k][1] * sdx)};
      if (accumulate) {
        o[0] += cur.r[k][0];
        o[1] += cur.r[k][1];
      }
      *reinterpret_cast<f32x2*>(rr + c0) = o;
      if (dres_lp) {
        P lp;
        lp[0] = from_f<T>(o[0]);
        lp[1] = from_f<T>(o[1]);
        *reinterpret_cast<P*>(dres_lp + (int64_t)row * C + c0) = lp;
      }
    }
    cur = nxt;
    row = next;
  }
  // block partials: waves combined in index order
#pragma unroll
  for (int k = 0; k < NP; k++) {
    const int c0 = 2 * lane + 128 * k;
    sh[w][c0] = ag[k][0];
    sh[w][c0 + 1] = ag[k][1];
    sh[w][C + c0] = ab[k][0];
    sh[w][C + c0 + 1] = ab[k][1];
  }
  __syncthreads();
  for (int j = threadIdx.x; j < 2 * C; j += 256)
    part[(int64_t)blockIdx.x * 2 * C + j] = ((sh[0][j] + sh[1][j]) + sh[2][j]) + sh[3][j];
}

// Batched partial-sum reduction: for every job, out[j] = [out[j] +]
// sum_p part[p*ld + j], p in order.  One launch serves up to
// kMaxReduceJobs jobs (all split-K, bias and LayerNorm partials of a layer).
// A job with at most RED_SLICES partials gives each thread one 4-float output
// chunk and adds its partials in order; a job with more splits the partials
// into RED_SLICES contiguous ranges (summed in order by separate threads) and
// adds the range sums in range order.  Either way the summation order is
// fixed, so results are deterministic.
constexpr int RED_SLICES = 16;
constexpr int RED_THREADS = 256;

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

__global__ void __launch_bounds__(RED_THREADS) reduce_jobs_kernel(ReduceJobs jobs) {
  __shared__ f32x4 sh[RED_THREADS];
  int jb = 0;
  while (jb + 1 < jobs.count && (int)blockIdx.x >= jobs.j[jb + 1].block0) jb++;
  const ReduceJob& J = jobs.j[jb];
  const int blk = blockIdx.x - J.block0, tid = threadIdx.x;
  if (J.nparts <= RED_SLICES) {
    const int64_t j = ((int64_t)blk * RED_THREADS + tid) * 4;
    if (j >= J.n) return;
    const float* src = J.part + j;
    f32x4 v[RED_SLICES];
#pragma unroll
    for (int p = 0; p < RED_SLICES; p++)
      if (p < J.nparts) v[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + p * J.ld));
    f32x4 t = v[0];
#pragma unroll
    for (int p = 1; p < RED_SLICES; p++)
      if (p < J.nparts) t += v[p];
    if (J.accumulate) t += ld4(J.out + j);
    *reinterpret_cast<f32x4*>(J.out + j) = t;
  } else {
    constexpr int CH = RED_THREADS / RED_SLICES;  // output chunks per block
    const int slice = tid / CH, c = tid % CH;
    const int64_t j = ((int64_t)blk * CH + c) * 4;
    const int p0 = (int)((int64_t)J.nparts * slice / RED_SLICES), p1 = (int)((int64_t)J.nparts * (slice + 1) / RED_SLICES);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    // (unrolled so eight loads are in flight; the additions keep their order)
    if (j < J.n) {
#pragma unroll 8
      for (int p = p0; p < p1; p++) t += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(J.part + (int64_t)p * J.ld + j));
    }
    sh[tid] = t;
    __syncthreads();
    if (slice == 0 && j < J.n) {
      f32x4 u = sh[c];
#pragma unroll
      for (int k = 1; k < RED_SLICES; k++) u += sh[k * CH + c];
      if (J.accumulate) u += ld4(J.out + j);
      *reinterpret_cast<f32x4*>(J.out + j) = u;
    }
  }
}


// ---------------------------------------------------------------------------
// Embedding forward: x[b,t] = wte[id[b,t]] + wpe[t]  (one wave per row).
// Ids or targets outside [0, V) set *err (the gather then reads row 0).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) embed_fwd_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ tgt,
                                                        const float* __restrict__ wte, const float* __restrict__ wpe,
                                                        float* __restrict__ x, int M, int T_, int C, int V,
                                                        int* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  int id = idx[row];
  bool bad = id < 0 || id >= V;
  if (tgt) {
    const int tg = tgt[row];
    bad = bad || tg < 0 || tg >= V;
  }
  if (bad) {
    if (lane == 0) atomicOr(err, 1);
    if (id < 0 || id >= V) id = 0;
  }
  const int t = row % T_;
  const float* a = wte + (int64_t)id * C;
  const float* p = wpe + (int64_t)t * C;
  float* o = x + (int64_t)row * C;
  for (int c = 2 * lane; c < C; c += 128) {
    const f32x2 u = *reinterpret_cast<const f32x2*>(a + c);
    const f32x2 v = *reinterpret_cast<const f32x2*>(p + c);
    *reinterpret_cast<f32x2*>(o + c) = f32x2{u[0] + v[0], u[1] + v[1]};
  }
}

// ---------------------------------------------------------------------------
// Stable LSD radix sort of (id, position) pairs in one workgroup of 1024
// threads (8-bit digits), then the start index of every run of equal ids.
// The result depends only on the ids: positions with equal id stay in
// increasing order, so every later sum over a run has a fixed order.
// ---------------------------------------------------------------------------
constexpr int SORT_T = 1024;

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return lane == 0 ? 0ull : (~0ull >> (64 - lane)); }

__global__ void __launch_bounds__(SORT_T) embed_sort_kernel(const int32_t* __restrict__ idx, int M, int passes,
                                                            int32_t* ka, int32_t* va, int32_t* kb, int32_t* vb,
                                                            int32_t* __restrict__ seg_start, int32_t* __restrict__ nseg) {
  __shared__ int hist[256];
  __shared__ int base[256];
  __shared__ int wcnt[SORT_T / 64][257];
  __shared__ int wtot[SORT_T / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int32_t* kin = idx;
  const int32_t* vin = nullptr;
  int32_t *kout = ka, *vout = va;
  for (int pass = 0; pass < passes; pass++) {
    const int shift = 8 * pass;
    if (tid < 256) {
      hist[tid] = 0;
    }
    __syncthreads();
    for (int i = tid; i < M; i += SORT_T) atomicAdd(&hist[(kin[i] >> shift) & 255], 1);
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int d = 0; d < 256; d++) {
        base[d] = run;
        run += hist[d];
      }
    }
    __syncthreads();
    for (int t0 = 0; t0 < M; t0 += SORT_T) {
      const int i = t0 + tid;
      const bool valid = i < M;
      const int key = valid ? kin[i] : 0;
      const int val = valid ? (vin ? vin[i] : i) : 0;
      const int d = (key >> shift) & 255;
      uint64_t mask = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 8; bit++) {
        const uint64_t bb = __ballot((d >> bit) & 1);
        mask &= ((d >> bit) & 1) ? bb : ~bb;
      }
      const int rank = __popcll(mask & lanemask_lt(lane));
      for (int j = tid; j < (SORT_T / 64) * 257; j += SORT_T) (&wcnt[0][0])[j] = 0;
      __syncthreads();
      if (valid && rank == 0) wcnt[w][d] = __popcll(mask);
      __syncthreads();
      if (valid) {
        int off = base[d] + rank;
        for (int ww = 0; ww < w; ww++) off += wcnt[ww][d];
        kout[off] = key;
        vout[off] = val;
      }
      __syncthreads();
      if (tid < 256) {
        int add = 0;
        for (int ww = 0; ww < SORT_T / 64; ww++) add += wcnt[ww][tid];
        base[tid] += add;
      }
      __syncthreads();
    }
    // next pass reads what this one wrote
    __threadfence_block();
    kin = kout;
    vin = vout;
    kout = (kout == ka) ? kb : ka;
    vout = (vout == va) ? vb : va;
    __syncthreads();
  }
  // kin/vin hold the sorted result; make sure it sits in (ka, va)
  if (kin != ka) {
    for (int i = tid; i < M; i += SORT_T) {
      ka[i] = kin[i];
      va[i] = vin[i];
    }
    __syncthreads();
  }
  // run starts: flag[i] = (i == 0 || key[i] != key[i-1]); exclusive scan of flags
  int running = 0;
  for (int t0 = 0; t0 < M; t0 += SORT_T) {
    const int i = t0 + tid;
    const bool f = i < M && (i == 0 || ka[i] != ka[i - 1]);
    const uint64_t bal = __ballot(f);
    const int wr = __popcll(bal & lanemask_lt(lane));
    if (lane == 0) wtot[w] = __popcll(bal);
    __syncthreads();
    int off = running + wr;
    for (int ww = 0; ww < w; ww++) off += wtot[ww];
    if (f) seg_start[off] = i;
    int tot = 0;
    for (int ww = 0; ww < SORT_T / 64; ww++) tot += wtot[ww];
    running += tot;
    __syncthreads();
  }
  if (tid == 0) {
    seg_start[running] = M;
    *nseg = running;
  }
}

// ---------------------------------------------------------------------------
// Embedding backward.
// dwpe[t] = [dwpe[t] +] sum_b dx[b, t]  (b in order; rows t >= T are zeroed
// when not accumulating).  dwte[id] += sum over the positions with that id,
// in sorted (= increasing position) order, computed in two steps so a very
// frequent id does not serialise: pieces of at most EMB_P sorted positions
// are summed in parallel, then each run adds up its pieces in order.
// ---------------------------------------------------------------------------
constexpr int EMB_P = 64;

__global__ void dwpe_kernel(const float* __restrict__ dx, float* __restrict__ dwpe, int B, int T_, int Tmax, int C,
                            int accumulate) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)Tmax * C) return;
  const int t = e / C, c = e % C;
  float s = 0.f;
  if (t < T_)
    for (int b = 0; b < B; b++) s += dx[((int64_t)b * T_ + t) * C + c];
  dwpe[e] = accumulate ? dwpe[e] + s : s;
}

// grid (ceil(M/EMB_P), C/64), one wave: lane = channel within a 64-wide slice.
__global__ void __launch_bounds__(64) dwte_piece_kernel(const float* __restrict__ dx, const int32_t* __restrict__ skey,
                                                        const int32_t* __restrict__ spos, float* __restrict__ piece,
                                                        int M, int C) {
  const int c = blockIdx.y * 64 + threadIdx.x;
  const int i0 = blockIdx.x * EMB_P, i1 = min(M, i0 + EMB_P);
  float acc = 0.f;
  int start = i0;
  for (int i = i0; i < i1; i++) {
    if (i > start && skey[i] != skey[i - 1]) {
      piece[(int64_t)start * C + c] = acc;
      acc = 0.f;
      start = i;
    }
    acc += dx[(int64_t)spos[i] * C + c];
  }
  if (i1 > i0) piece[(int64_t)start * C + c] = acc;
}

// grid (G, C/64), one wave: runs s = blockIdx.x, blockIdx.x + G, ...
__global__ void __launch_bounds__(64) dwte_run_kernel(const float* __restrict__ piece, const int32_t* __restrict__ skey,
                                                      const int32_t* __restrict__ seg_start,
                                                      const int32_t* __restrict__ nseg, float* __restrict__ dwte, int C,
                                                      int V) {
  const int c = blockIdx.y * 64 + threadIdx.x;
  const int ns = *nseg;
  for (int s = blockIdx.x; s < ns; s += gridDim.x) {
    const int a = seg_start[s], e = seg_start[s + 1];
    float acc = piece[(int64_t)a * C + c];
    for (int p = (a / EMB_P + 1) * EMB_P; p < e; p += EMB_P) acc += piece[(int64_t)p * C + c];
    const int id = skey[a];
    if (id >= 0 && id < V) dwte[(int64_t)id * C + c] += acc;  // bad ids were flagged in the forward pass
  }
}

// ---------------------------------------------------------------------------
// Fused softmax cross-entropy, one block (1024 threads) per row, one pass over
// the logits in memory.  Each thread holds its share of the row in registers
// as loaded (act type, so two rows fit per CU and one row's reductions overlap
// another's memory traffic), takes its own maximum m_t and sum of
// e = exp(z - m_t); one block reduction combines the (m_t, sum e) pairs into
// logsumexp over the real vocabulary [0, V).  loss = logsumexp - z[target];
// the logits are overwritten in place with dscale * (softmax - onehot), where
// softmax = exp(z - m_t) * exp(m_t - logsumexp) (the exponential taken again
// from the held logits), and 0 on the padded columns.
// ---------------------------------------------------------------------------
constexpr int CE_T = 1024;

template <typename T, int NV>
__global__ void __launch_bounds__(CE_T) ce_kernel(T* __restrict__ logits, const int32_t* __restrict__ tgt,
                                                  float* __restrict__ row_loss, int V, int Vp, float dscale,
                                                  int write_grad) {
  typedef typename Frag<T>::type F;
  __shared__ float rm[CE_T / 64], rs[CE_T / 64];
  __shared__ float zt;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t row = blockIdx.x;
  T* z = logits + row * Vp;
  const int nvec = Vp / 8;
  const int y = min(max(tgt[row], 0), V - 1);  // out-of-range targets were flagged by the embedding pass
  if (tid == 0) zt = to_f<T>(z[y]);
  constexpr float L2E = 1.4426950408889634f;
  // load this thread's vectors (held as loaded); columns >= V count as -inf.
  // Only vectors k >= kfull can reach past V (a block-wide bound): the others
  // take a copy of each pass without the column test (a scalar branch per k).
  F zv[NV];
  float mt = -INFINITY;
  const int kfull = V / (CE_T * 8);
  auto val = [&](int k, int q, auto check) {
    const int vi = tid + k * CE_T;
    return !decltype(check)::value || vi * 8 + q < V ? to_f<T>(zv[k][q]) : -INFINITY;
  };
#pragma unroll
  for (int k = 0; k < NV; k++) {
    const int vi = tid + k * CE_T;
    if (vi < nvec) {
      zv[k] = __builtin_nontemporal_load(reinterpret_cast<const F*>(z + vi * 8));
      if (k < kfull) {
#pragma unroll
        for (int q = 0; q < 8; q++) mt = fmaxf(mt, val(k, q, std::false_type{}));
      } else {
#pragma unroll
        for (int q = 0; q < 8; q++) mt = fmaxf(mt, val(k, q, std::true_type{}));
      }
    }
  }
  // sum of e = exp(z - m_t) (a thread without real columns keeps m_t = -inf, st = 0)
  float st = 0.f;
  const float mtl = mt == -INFINITY ? 0.f : mt * L2E;
#pragma unroll
  for (int k = 0; k < NV; k++) {
    const int vi = tid + k * CE_T;
    if (vi < nvec) {
      if (k < kfull) {
#pragma unroll
        for (int q = 0; q < 8; q++) st += __builtin_amdgcn_exp2f(fmaf(val(k, q, std::false_type{}), L2E, -mtl));
      } else {
#pragma unroll
        for (int q = 0; q < 8; q++) st += __builtin_amdgcn_exp2f(fmaf(val(k, q, std::true_type{}), L2E, -mtl));
      }
    }
  }
  // combine (m_t, st) over the block: M = max m_t, S = sum st * exp(m_t - M)
  float M = wave_max(mt);
  if (lane == 0) rm[w] = M;
  __syncthreads();
  M = rm[0];
#pragma unroll
  for (int i = 1; i < CE_T / 64; i++) M = fmaxf(M, rm[i]);
  float sc = st > 0.f ? st * __builtin_amdgcn_exp2f((mt - M) * L2E) : 0.f;
  sc = wave_sum(sc);
  if (lane == 0) rs[w] = sc;
  __syncthreads();
  float S = rs[0];
#pragma unroll
  for (int i = 1; i < CE_T / 64; i++) S += rs[i];
  const float lse = M + __logf(S);
  if (tid == 0) row_loss[row] = lse - zt;
  if (!write_grad) return;
  const float f = st > 0.f ? __builtin_amdgcn_exp2f((mt - lse) * L2E) * dscale : 0.f;
  // the target's column gets softmax - 1: its thread rewrites that one value
  // after the vector stores (the same thread, so in program order)
  const bool owns_y = (y / 8) % CE_T == tid;
  auto grad = [&](int k, auto check) {
    const int vi = tid + k * CE_T;
    F o;
#pragma unroll
    for (int q = 0; q < 8; q++) o[q] = from_f<T>(__builtin_amdgcn_exp2f(fmaf(val(k, q, check), L2E, -mtl)) * f);
    __builtin_nontemporal_store(o, reinterpret_cast<F*>(z + vi * 8));
  };
#pragma unroll
  for (int k = 0; k < NV; k++) {
    if (tid + k * CE_T < nvec) {
      if (k < kfull) grad(k, std::false_type{});
      else grad(k, std::true_type{});
    }
  }
  if (owns_y) {
    // the same exponential as in its vector (zt is that logit), less 1, in one
    // rounding (a fused multiply-add)
    const float e = __builtin_amdgcn_exp2f(fmaf(zt, L2E, -mtl));
    z[y] = from_f<T>(fmaf(e, f, -dscale));
  }
}

__global__ void __launch_bounds__(1024) mean_loss_kernel(const float* __restrict__ row_loss, int M,
                                                         float* __restrict__ out) {
  __shared__ double red[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  double s = 0.0;
  for (int i = tid; i < M; i += 1024) s += row_loss[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) red[w] = s;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int i = 0; i < 16; i++) t += red[i];
    *out = (float)(t / M);
  }
}

// ---------------------------------------------------------------------------
// Global gradient norm: block b sums g^2 over its contiguous chunk (fixed
// order), then one block adds the partials in order and derives the clip
// factor min(1, clip / norm); a non-finite norm sets the error and skip flags.
// ---------------------------------------------------------------------------
constexpr int NORM_BLOCKS = kGradNormParts;

__global__ void __launch_bounds__(256) norm_part_kernel(const float* __restrict__ g, int64_t n,
                                                        double* __restrict__ part) {
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t nq = n / 4;
  const int64_t per = (nq + gridDim.x - 1) / gridDim.x;
  const int64_t q0 = blockIdx.x * per, q1 = min(nq, q0 + per);
  // four loads in flight per thread, into four partial sums combined in a
  // fixed order (the sum of squares is deterministic for a given n)
  double s4[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t q = q0 + tid;
  for (; q + 3 * 256 < q1; q += 4 * 256) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; u++) v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + 4 * (q + u * 256)));
#pragma unroll
    for (int u = 0; u < 4; u++)
      s4[u] += (double)v[u][0] * v[u][0] + (double)v[u][1] * v[u][1] + (double)v[u][2] * v[u][2] +
               (double)v[u][3] * v[u][3];
  }
  for (; q < q1; q += 256) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + 4 * q));
    s4[0] += (double)v[0] * v[0] + (double)v[1] * v[1] + (double)v[2] * v[2] + (double)v[3] * v[3];
  }
  double s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  if (blockIdx.x == gridDim.x - 1)
    for (int64_t i = 4 * nq + tid; i < n; i += 256) s += (double)g[i] * g[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) red[w] = s;
  __syncthreads();
  if (tid == 0) part[blockIdx.x] = ((red[0] + red[1]) + red[2]) + red[3];
}

__global__ void __launch_bounds__(256) norm_final_kernel(const double* __restrict__ part, int nparts, float clip,
                                                         float* __restrict__ norm_out, float* __restrict__ scale_out,
                                                         int* __restrict__ flags) {
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  double s = 0.0;
  for (int i = tid; i < nparts; i += 256) s += part[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) red[w] = s;
  __syncthreads();
  if (tid == 0) {
    const double tot = ((red[0] + red[1]) + red[2]) + red[3];
    const float nrm = (float)sqrt(tot);
    if (norm_out) *norm_out = nrm;
    const bool finite = isfinite(nrm);
    *scale_out = finite && nrm > clip ? clip / nrm : 1.f;
    flags[2] = finite ? 0 : 1;  // skip this update
    if (!finite) flags[1] = 1;  // reported by the next status check
  }
}

// AdamW with bias correction and decoupled weight decay on indices < n_decay.
// One 4-element quad per thread; parameters, gradients and moments stream
// through once, so their loads and stores are marked non-temporal.
__global__ void __launch_bounds__(256) adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    bf16* __restrict__ p_lp, int64_t nq, int64_t n_decay, float lr,
                                                    float b1, float b2, float eps, float wd, float rbc1, float rbc2,
                                                    const float* __restrict__ scale, const int* __restrict__ flags) {
  if (flags[2]) return;
  const float sc = *scale;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nq; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = 4 * q;
    f32x4 pp = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + i));
    const f32x4 gg = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + i));
    f32x4 mm = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(m + i));
    f32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(v + i));
    const float d = i < n_decay ? wd : 0.f;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float gr = gg[e] * sc;
      mm[e] = b1 * mm[e] + (1.f - b1) * gr;
      vv[e] = b2 * vv[e] + (1.f - b2) * gr * gr;
      const float mh = mm[e] * rbc1, vh = vv[e] * rbc2;
      pp[e] -= lr * (mh / (sqrtf(vh) + eps) + d * pp[e]);
    }
    __builtin_nontemporal_store(pp, reinterpret_cast<f32x4*>(p + i));
    __builtin_nontemporal_store(mm, reinterpret_cast<f32x4*>(m + i));
    __builtin_nontemporal_store(vv, reinterpret_cast<f32x4*>(v + i));
    if (p_lp) {
      bf16x4 o;
#pragma unroll
      for (int e = 0; e < 4; e++) o[e] = (bf16)pp[e];
      *reinterpret_cast<bf16x4*>(p_lp + i) = o;
    }
  }
}

// FP8 copy of bf16 rows [rows][K] with one scale per row; one wave per row,
// the row kept in registers between the amax and the conversion.  CPL: 16-byte
// chunks per lane (K <= 512 * CPL, K a multiple of 8).
template <int CPL>
__device__ __forceinline__ void quant_row(const bf16* __restrict__ xr, fp8e4* __restrict__ qr, float* __restrict__ sc,
                                          int K, int lane) {
  const int nch = K / 8;
  bf16x8 v[CPL];
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; c++) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      v[c] = ld8(xr + ch * 8);
#pragma unroll
      for (int e = 0; e < 8; e++) amax = fmaxf(amax, fabsf((float)v[c][e]));
    }
  }
  amax = wave_max(amax);
  const float s = fp8_row_scale(amax), inv = 1.f / s;
#pragma unroll
  for (int c = 0; c < CPL; c++) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      uint2 o;
      o.x = fp8_pack4((float)v[c][0], (float)v[c][1], (float)v[c][2], (float)v[c][3], inv);
      o.y = fp8_pack4((float)v[c][4], (float)v[c][5], (float)v[c][6], (float)v[c][7], inv);
      *reinterpret_cast<uint2*>(qr + ch * 8) = o;
    }
  }
  if (lane == 0) *sc = s;
}

template <int CPL>
__global__ void __launch_bounds__(256) quant_rows_kernel(const bf16* __restrict__ x, fp8e4* __restrict__ q,
                                                         float* __restrict__ sc, int rows, int K) {
  const int lane = threadIdx.x & 63, row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  quant_row<CPL>(x + (int64_t)row * K, q + (int64_t)row * K, sc + row, K, lane);
}

template <int CPL>
__global__ void __launch_bounds__(256) quant_jobs_kernel(QuantJobs jobs) {
  const int lane = threadIdx.x & 63, grow = blockIdx.x * 4 + (threadIdx.x >> 6);
  int j = 0;
  while (j + 1 < jobs.count && grow >= jobs.j[j + 1].row0) j++;
  const QuantJob& jb = jobs.j[j];
  const int row = grow - jb.row0;
  if (row < 0 || row >= jb.rows) return;
  quant_row<CPL>(jb.in + (int64_t)row * jb.cols, jb.out + (int64_t)row * jb.cols, jb.scale + row, jb.cols, lane);
}

// gelu of a stored pre-activation (activation recompute): the same function of
// the same rounded values as the forward's GELU epilogue, so the result is the
// forward's activation bit for bit
template <typename T>
__global__ void __launch_bounds__(256) gelu_fwd_kernel(const T* __restrict__ u, T* __restrict__ out, int64_t n8) {
  typedef typename Frag<T>::type F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const F x = ld8(u + i * 8);
    F o;
#pragma unroll
    for (int e = 0; e < 8; e++) o[e] = from_f<T>(gelu_tanh(to_f<T>(x[e])));
    st8(out + i * 8, o);
  }
}

__global__ void to_bf16_kernel(const float* __restrict__ src, bf16* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = (bf16)src[i];
}

// One 64 x 64 tile of a bf16 matrix transposed through LDS: rows read and
// columns written as 16-byte runs (each of the 256 threads moves two runs of
// eight values each way).  Grid (cols/64, rows/64, matrices).
__global__ void __launch_bounds__(256) transpose_bf16_kernel(const bf16* __restrict__ in, int64_t in_stride,
                                                             bf16* __restrict__ out, int rows, int cols) {
  __shared__ bf16 t[64][64 + 2];  // odd word pitch: the column reads fall in distinct banks
  const bf16* src = in + (int64_t)blockIdx.z * in_stride;
  bf16* dst = out + (int64_t)blockIdx.z * rows * cols;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const int idx = threadIdx.x + 256 * k, r = idx / 8, c = (idx % 8) * 8;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + (int64_t)(r0 + r) * cols + c0 + c);
#pragma unroll
    for (int e = 0; e < 8; e++) t[r][c + e] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const int idx = threadIdx.x + 256 * k, c = idx / 8, r = (idx % 8) * 8;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; e++) v[e] = t[r + e][c];
    *reinterpret_cast<bf16x8*>(dst + (int64_t)(c0 + c) * rows + r0 + r) = v;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define LN_NP_DISPATCH(C, F)       \
  switch ((C) / 128) {              \
    case 1: F(1); break;            \
    case 2: F(2); break;            \
    case 3: F(3); break;            \
    case 4: F(4); break;            \
    case 6: F(6); break;            \
    case 8: F(8); break;            \
    case 12: F(12); break;          \
    case 16: F(16); break;          \
    default: return hipErrorInvalidValue; \
  }

hipError_t layernorm_fwd(hipStream_t st, Prec p, const float* x, const float* g, const float* b, void* y, float* mean,
                         float* rstd, int M, int C, fp8e4* y8, float* s8) {
  if (C % 128 != 0 || (y8 && C % 256 != 0)) return hipErrorInvalidValue;
  dim3 grid((M + 3) / 4);
#define LNF(NP)                                                                                                    \
  if (p == BF16)                                                                                                   \
    hipLaunchKernelGGL((ln_fwd_kernel<bf16, NP>), grid, dim3(256), 0, st, x, g, b, static_cast<bf16*>(y), mean, rstd, M, \
                       y8, s8);                                                                                    \
  else                                                                                                             \
    hipLaunchKernelGGL((ln_fwd_kernel<float, NP>), grid, dim3(256), 0, st, x, g, b, static_cast<float*>(y), mean, rstd, M, \
                       y8, s8);
  LN_NP_DISPATCH(C, LNF)
#undef LNF
  return hipGetLastError();
}

int layernorm_bwd_parts(int M) { return std::min(LNB_BLOCKS, (M + 3) / 4); }

hipError_t layernorm_bwd(hipStream_t st, Prec p, const void* dy, const float* x, const float* mean, const float* rstd,
                         const float* g, float* dres, void* dres_lp, int accumulate, float* part, int M, int C,
                         int* nparts) {
  if (C % 128 != 0) return hipErrorInvalidValue;
  const int nb = layernorm_bwd_parts(M);
  *nparts = nb;
#define LNB(NP)                                                                                                     \
  if (p == BF16)                                                                                                    \
    hipLaunchKernelGGL((ln_bwd_kernel<bf16, NP>), dim3(nb), dim3(256), 0, st, static_cast<const bf16*>(dy), x, mean, \
                       rstd, g, dres, static_cast<bf16*>(dres_lp), accumulate, part, M);                            \
  else                                                                                                              \
    hipLaunchKernelGGL((ln_bwd_kernel<float, NP>), dim3(nb), dim3(256), 0, st, static_cast<const float*>(dy), x,    \
                       mean, rstd, g, dres, static_cast<float*>(dres_lp), accumulate, part, M);
  LN_NP_DISPATCH(C, LNB)
#undef LNB
  return hipGetLastError();
}

hipError_t reduce_jobs(hipStream_t st, const ReduceJob* jobs, int count) {
  if (count <= 0) return hipSuccess;
  if (count > kMaxReduceJobs) return hipErrorInvalidValue;
  ReduceJobs J;
  J.count = count;
  int blocks = 0;
  for (int k = 0; k < count; k++) {
    J.j[k] = jobs[k];
    const ReduceJob& q = jobs[k];
    if (q.n % 4 != 0 || q.ld % 4 != 0 || q.nparts < 1 || q.part == nullptr || q.out == nullptr)
      return hipErrorInvalidValue;
    J.j[k].block0 = blocks;
    const int per = q.nparts <= RED_SLICES ? RED_THREADS * 4 : (RED_THREADS / RED_SLICES) * 4;
    blocks += (q.n + per - 1) / per;
  }
  hipLaunchKernelGGL(reduce_jobs_kernel, dim3(blocks), dim3(RED_THREADS), 0, st, J);
  return hipGetLastError();
}

hipError_t embed_fwd(hipStream_t st, const int32_t* idx, const int32_t* tgt, const float* wte, const float* wpe,
                     float* x, int B, int T_, int C, int V, int* err_flag) {
  const int M = B * T_;
  hipLaunchKernelGGL(embed_fwd_kernel, dim3((M + 3) / 4), dim3(256), 0, st, idx, tgt, wte, wpe, x, M, T_, C, V,
                     err_flag);
  return hipGetLastError();
}

hipError_t embed_sort(hipStream_t st, const int32_t* idx, int M, int V, int32_t* keys_a, int32_t* vals_a,
                      int32_t* keys_b, int32_t* vals_b, int32_t* seg_start, int32_t* nseg) {
  int passes = 1;
  while (passes < 4 && (int64_t)(V - 1) >> (8 * passes)) passes++;
  hipLaunchKernelGGL(embed_sort_kernel, dim3(1), dim3(SORT_T), 0, st, idx, M, passes, keys_a, vals_a, keys_b, vals_b,
                     seg_start, nseg);
  return hipGetLastError();
}

hipError_t embed_bwd(hipStream_t st, const float* dx, const int32_t* sorted_ids, const int32_t* sorted_pos,
                     const int32_t* seg_start, const int32_t* nseg, float* dwte, float* dwpe, float* piece, int B,
                     int T_, int Tmax, int C, int V, int accumulate_wpe) {
  const int M = B * T_;
  const int64_t nw = (int64_t)Tmax * C;
  hipLaunchKernelGGL(dwpe_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, st, dx, dwpe, B, T_, Tmax, C,
                     accumulate_wpe);
  hipLaunchKernelGGL(dwte_piece_kernel, dim3((M + EMB_P - 1) / EMB_P, C / 64), dim3(64), 0, st, dx, sorted_ids,
                     sorted_pos, piece, M, C);
  hipLaunchKernelGGL(dwte_run_kernel, dim3(std::min(M, 2048), C / 64), dim3(64), 0, st, piece, sorted_ids, seg_start,
                     nseg, dwte, C, V);
  return hipGetLastError();
}

hipError_t cross_entropy(hipStream_t st, Prec p, void* logits, const int32_t* tgt, float* row_loss, int M, int V, int Vp,
                         float dscale, int write_grad) {
  if (Vp % 8 != 0) return hipErrorInvalidValue;
  const int nvec = Vp / 8;
  const int nv = (nvec + CE_T - 1) / CE_T;
#define CE_LAUNCH(TT, NV)                                                                                            \
  hipLaunchKernelGGL((ce_kernel<TT, NV>), dim3(M), dim3(CE_T), 0, st, static_cast<TT*>(logits), tgt, row_loss, V, Vp, \
                     dscale, write_grad)
#define CE_DISPATCH(TT)     \
  if (nv <= 1)              \
    CE_LAUNCH(TT, 1);       \
  else if (nv <= 2)         \
    CE_LAUNCH(TT, 2);       \
  else if (nv <= 4)         \
    CE_LAUNCH(TT, 4);       \
  else if (nv <= 7)         \
    CE_LAUNCH(TT, 7);       \
  else if (nv <= 8)         \
    CE_LAUNCH(TT, 8);       \
  else                      \
    return hipErrorInvalidValue;
  if (p == BF16) {
    CE_DISPATCH(bf16)
  } else {
    CE_DISPATCH(float)
  }
#undef CE_DISPATCH
#undef CE_LAUNCH
  return hipGetLastError();
}

hipError_t mean_loss(hipStream_t st, const float* row_loss, int M, float* out) {
  hipLaunchKernelGGL(mean_loss_kernel, dim3(1), dim3(1024), 0, st, row_loss, M, out);
  return hipGetLastError();
}

hipError_t grad_norm(hipStream_t st, const float* g, int64_t n, double* part, float clip, float* norm_out,
                     float* scale_out, int* flags) {
  hipLaunchKernelGGL(norm_part_kernel, dim3(NORM_BLOCKS), dim3(256), 0, st, g, n, part);
  hipLaunchKernelGGL(norm_final_kernel, dim3(1), dim3(256), 0, st, part, NORM_BLOCKS, clip, norm_out, scale_out, flags);
  return hipGetLastError();
}

hipError_t adamw(hipStream_t st, float* p, const float* g, float* m, float* v, void* p_lp, int64_t n, int64_t n_decay,
                 float lr, float b1, float b2, float eps, float wd, float bc1, float bc2, const float* scale,
                 const int* flags) {
  if (n % 4 != 0 || n_decay % 4 != 0) return hipErrorInvalidValue;
  const int64_t nq = n / 4;
  const unsigned blocks = (unsigned)std::min<int64_t>((nq + 255) / 256, 1 << 30);
  hipLaunchKernelGGL(adamw_kernel, dim3(blocks), dim3(256), 0, st, p, g, m, v, static_cast<bf16*>(p_lp), nq, n_decay, lr,
                     b1, b2, eps, wd, 1.f / bc1, 1.f / bc2, scale, flags);
  return hipGetLastError();
}

hipError_t quant_rows(hipStream_t st, const void* x, fp8e4* q, float* scale, int rows, int K) {
  if (K % 8 != 0 || K > 512 * 8) return hipErrorInvalidValue;
  const dim3 grid((rows + 3) / 4);
  const bf16* xb = static_cast<const bf16*>(x);
  if (K <= 512 * 2)
    hipLaunchKernelGGL(quant_rows_kernel<2>, grid, dim3(256), 0, st, xb, q, scale, rows, K);
  else if (K <= 512 * 6)
    hipLaunchKernelGGL(quant_rows_kernel<6>, grid, dim3(256), 0, st, xb, q, scale, rows, K);
  else
    hipLaunchKernelGGL(quant_rows_kernel<8>, grid, dim3(256), 0, st, xb, q, scale, rows, K);
  return hipGetLastError();
}

hipError_t quant_jobs(hipStream_t st, const QuantJob* jobs, int count) {
  if (count <= 0) return hipSuccess;
  if (count > kMaxQuantJobs) return hipErrorInvalidValue;
  QuantJobs J;
  J.count = count;
  int rows = 0, kmax = 0;
  for (int i = 0; i < count; i++) {
    J.j[i] = jobs[i];
    J.j[i].row0 = rows;
    rows += jobs[i].rows;
    kmax = std::max(kmax, jobs[i].cols);
    if (jobs[i].cols % 8 != 0) return hipErrorInvalidValue;
  }
  if (kmax > 512 * 8) return hipErrorInvalidValue;
  const dim3 grid((rows + 3) / 4);
  if (kmax <= 512 * 2)
    hipLaunchKernelGGL(quant_jobs_kernel<2>, grid, dim3(256), 0, st, J);
  else if (kmax <= 512 * 6)
    hipLaunchKernelGGL(quant_jobs_kernel<6>, grid, dim3(256), 0, st, J);
  else
    hipLaunchKernelGGL(quant_jobs_kernel<8>, grid, dim3(256), 0, st, J);
  return hipGetLastError();
}

hipError_t gelu_fwd(hipStream_t st, Prec p, const void* u, void* out, int64_t n) {
  if (n % 8 != 0) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  const unsigned blocks = (unsigned)std::min<int64_t>((n8 + 255) / 256, 4096);
  if (p == BF16)
    hipLaunchKernelGGL(gelu_fwd_kernel<bf16>, dim3(blocks), dim3(256), 0, st, static_cast<const bf16*>(u),
                       static_cast<bf16*>(out), n8);
  else
    hipLaunchKernelGGL(gelu_fwd_kernel<float>, dim3(blocks), dim3(256), 0, st, static_cast<const float*>(u),
                       static_cast<float*>(out), n8);
  return hipGetLastError();
}

hipError_t transpose_bf16(hipStream_t st, const void* in, int64_t in_stride, void* out, int rows, int cols, int count) {
  if (rows <= 0 || cols <= 0 || rows % 64 != 0 || cols % 64 != 0 || count < 1 || count > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(cols / 64, rows / 64, count), dim3(256), 0, st,
                     static_cast<const bf16*>(in), in_stride, static_cast<bf16*>(out), rows, cols);
  return hipGetLastError();
}

hipError_t to_bf16(hipStream_t st, const float* src, void* dst, int64_t n) {
  const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(to_bf16_kernel, dim3(blocks), dim3(256), 0, st, src, static_cast<bf16*>(dst), n);
  return hipGetLastError();
}

}  // namespace gpt2k
