// attention.hip -- causal multi-head self-attention on MFMA for gfx950.
//
// Per head: y_i = sum_{j<=i} softmax_j(q_i . k_j / sqrt(hd)) v_j, computed
// tile by tile with an online softmax so the T x T score matrix never leaves
// registers ("Karpathy's four-hour GPT-2 reproduction in one post", part 2:
// Flash Attention; "Reproducing GPT-2 (124M) cheaply with llm.c", setup:
// FlashAttention).  The forward pass saves the per-row log-sum-exp; the
// backward pass recomputes probabilities from it.
//
// Layout: qkv is [B*T, 3C] with q heads, then k heads, then v heads
// (head h at column offset h*hd inside each third); out / dout are [B*T, C].
// Each wave owns 32 query (or key) rows; a block of 4 waves shares K/V (or
// Q/dO) tiles of 64 rows through LDS.
//
// Orientation: scores are produced as S^T (keys x queries) in the forward and
// dQ kernels, so every lane owns one query column and its softmax statistics
// (max, sum, LSE, D) are per-lane scalars shared with the partner lane l^32.
// The dK/dV kernel produces S (queries x keys) so each lane owns one key.
// The second product of each pair consumes the accumulator directly as its
// k-operand: the 16 reduction slots of a (virtual) 32x32x16 MFMA may be any
// 16 keys as long as both operands use the same assignment, here
// key(c, g, s) = 16c + 8(s/4) + 4g + s%4 for chunk c, lane group g, slot s.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gpt2k {
namespace {

constexpr int KT = 64;   // rows per K/V (or Q/dO) LDS tile
constexpr int WQ = 32;   // rows per wave
constexpr int NW = 4;    // waves per block
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <typename T> struct V16;
template <> struct V16<bf16> { typedef bf16x8 type; static constexpr int n = 8; };
template <> struct V16<float> { typedef f32x4 type; static constexpr int n = 4; };

// One KT x HD row tile (rows `ld` apart in global memory) held in registers,
// spread over all threads of the block as 16-byte chunks; stored to LDS
// row-major [KT][HD + VE].  Loading the next tile while the current one is
// consumed hides the memory latency.
template <typename T, int HD>
struct RowTile {
  static constexpr int VE = V16<T>::n, LD = HD + VE, CPR = HD / VE, PER = KT * CPR / (NW * 64);
  static_assert(KT * CPR % (NW * 64) == 0, "tile must split evenly over the block");
  f32x4 v[PER];
  __device__ __forceinline__ void load(const T* g, int64_t ld, int tid) {
#pragma unroll
    for (int c = 0; c < PER; c++) {
      const int idx = tid + c * NW * 64, r = idx / CPR, k = idx % CPR;
      v[c] = *reinterpret_cast<const f32x4*>(g + (int64_t)r * ld + k * VE);
    }
  }
  __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
    for (int c = 0; c < PER; c++) {
      const int idx = tid + c * NW * 64, r = idx / CPR, k = idx % CPR;
      *reinterpret_cast<f32x4*>(s + r * LD + k * VE) = v[c];
    }
  }
};

// k-operand fragment of X^T read from a row-major tile X [KT][LD]: lane l
// gets column d = dbase + l%32 and the 8 rows key(c, g, s) = 16c + 8(s/4) +
// 4g + s%4 (g = l/32).  bf16 uses the transposing LDS read: within each
// 16-lane group, lane j points at row r0 + j/4, columns c0 + 4*(j%4) .. +3
// and receives rows r0 .. r0+3 of column c0 + j.
template <typename T, int LD>
__device__ __forceinline__ typename Frag<T>::type ld_tsplit(const T* s, int dbase, int c, int lane) {
  typename Frag<T>::type f;
  if constexpr (sizeof(T) == 2) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int j = lane & 15, G = lane >> 4;
    const int r0 = 16 * c + 4 * (G >> 1) + (j >> 2);
    const int col = dbase + 16 * (G & 1) + 4 * (j & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(s + r0 * LD + col));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(s + (r0 + 8) * LD + col));
    const bf16x4 a = __builtin_bit_cast(bf16x4, lo), b = __builtin_bit_cast(bf16x4, hi);
    f = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
    const int d = dbase + (lane & 31), g = lane >> 5;
#pragma unroll
    for (int e = 0; e < 8; e++) f[e] = s[(16 * c + 8 * (e / 4) + 4 * g + (e % 4)) * LD + d];
  }
  return f;
}

// Slots 8h..8h+7 of a 32x32 accumulator as a k-operand fragment.
template <typename T>
__device__ __forceinline__ typename Frag<T>::type acc_frag(const f32x16& a, int h) {
  typename Frag<T>::type f;
#pragma unroll
  for (int e = 0; e < 8; e++) f[e] = from_f<T>(a[8 * h + e]);
  return f;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------------
// Forward.  grid (NH*B, ceil(T/128)); heavy (late) query blocks first.
// Per key tile: K and V rows (next tile prefetched into registers).
// ------------------------------------------------------------------------
template <typename T, int HD>
__global__ void __launch_bounds__(NW * 64, 3) attn_fwd_kernel(const T* __restrict__ qkv, T* __restrict__ out,
                                                              float* __restrict__ lse, int T_, int NH, float sl2) {
  typedef RowTile<T, HD> RT;
  constexpr int LD = RT::LD, ND = HD / 16, NDT = HD / 32;
  typedef typename Frag<T>::type F;
  typedef typename Quad<T>::type Q;
  __shared__ __attribute__((aligned(16))) T Ks[2][KT * LD];
  __shared__ __attribute__((aligned(16))) T Vs[2][KT * LD];

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), lr = lane & 31, lg = lane >> 5;
  const int qblk = gridDim.y - 1 - blockIdx.y;  // heaviest (latest) query blocks dispatch first
  const int h = blockIdx.x % NH, b = blockIdx.x / NH;
  const int C = NH * HD, S3 = 3 * C;
  const int q0 = qblk * NW * WQ + w * WQ;
  const bool active = q0 < T_;
  const T* base = qkv + (int64_t)b * T_ * S3;
  const T* kbase = base + C + h * HD;
  const T* vbase = base + 2 * C + h * HD;

  F qf[ND];
  if (active) {
#pragma unroll
    for (int ds = 0; ds < ND; ds++) qf[ds] = ld8(base + (int64_t)(q0 + lr) * S3 + h * HD + ds * 16 + 8 * lg);
  }
  f32x16 o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; dt++) o[dt] = f32x16{};
  // Running max m (log2 domain) and running sum: the sum is accumulated by
  // the matrix core as (ones x P), so every entry of lsum holds this lane's
  // query's sum of the very (rounded) P values that multiply V.
  f32x16 lsum = f32x16{};
  float m = -INFINITY;
  F ones;
#pragma unroll
  for (int e = 0; e < 8; e++) ones[e] = from_f<T>(1.f);
  const int q = q0 + lr;

  const int ntiles = min(T_, (qblk + 1) * NW * WQ) / KT;
  RT kt, vt;
  kt.load(kbase, S3, tid);
  vt.load(vbase, S3, tid);
  kt.store(Ks[0], tid);
  vt.store(Vs[0], tid);
  __syncthreads();
  // One 64-key tile: prefetch the next tile, compute, stage the prefetch.
  // Only the last two tiles can straddle one of the block's queries, so they
  // run a copy with the causal mask and the rest a copy without it.
  auto iteration = [&](int it, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int cur = it & 1, kv0 = it * KT;
    const bool more = it + 1 < ntiles;
    if (more) {
      kt.load(kbase + (int64_t)(kv0 + KT) * S3, S3, tid);
      vt.load(vbase + (int64_t)(kv0 + KT) * S3, S3, tid);
    }
    if (active && kv0 <= q0 + WQ - 1) {
      f32x16 s[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; c2++) {
        s[c2] = f32x16{};
#pragma unroll
        for (int ds = 0; ds < ND; ds++) mma16(s[c2], ld8(Ks[cur] + (c2 * 32 + lr) * LD + ds * 16 + 8 * lg), qf[ds]);
      }
      if (MASK) {  // hide keys after the query: key kl of the tile when kl > lim
        const int lim = q - kv0 - 4 * lg;
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++)
#pragma unroll
          for (int r = 0; r < 16; r++)
            if (c2 * 32 + 8 * (r / 4) + (r % 4) > lim) s[c2][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int c2 = 0; c2 < 2; c2++)
#pragma unroll
        for (int r = 0; r < 16; r++) mx = fmaxf(mx, s[c2][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
      // Lazy rescaling: the reference max moves only when this tile's max
      // exceeds it by more than 8 (so P <= 2^8, exact in range for bf16 and
      // fp32); then o and the sum are rescaled, in a branch the wave takes
      // only if one of its queries needs it (the first tile, then rarely).
      const bool grow = mx > m + 8.f;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mn = grow ? mx : m;
        const float alpha = fast_exp2(m - mn);
#pragma unroll
        for (int dt = 0; dt < NDT; dt++) o[dt] *= alpha;
        lsum *= alpha;
        m = mn;
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; c2++)
#pragma unroll
        for (int r = 0; r < 16; r++) s[c2][r] = fast_exp2(fmaf(s[c2][r], sl2, -m));
#pragma unroll
      for (int c = 0; c < KT / 16; c++) {
        const F pf = acc_frag<T>(s[c / 2], c % 2);
        mma16(lsum, ones, pf);
#pragma unroll
        for (int dt = 0; dt < NDT; dt++) mma16(o[dt], ld_tsplit<T, LD>(Vs[cur], dt * 32, c, lane), pf);
      }
    }
    if (more) {
      kt.store(Ks[cur ^ 1], tid);
      vt.store(Vs[cur ^ 1], tid);
    }
    __syncthreads();
  };
  static_assert(NW * WQ == 2 * KT, "a block's queries span two key tiles");
  const int nplain = max(0, ntiles - 2);
  for (int it = 0; it < nplain; it++) iteration(it, std::false_type{});
  for (int it = nplain; it < ntiles; it++) iteration(it, std::true_type{});
  if (!active) return;
  const float l = lsum[0];
  const float inv = 1.f / l;
  T* orow = out + ((int64_t)b * T_ + q) * C + h * HD;
#pragma unroll
  for (int dt = 0; dt < NDT; dt++)
#pragma unroll
    for (int qq = 0; qq < 4; qq++) {
      Q v;
#pragma unroll
      for (int e = 0; e < 4; e++) v[e] = from_f<T>(o[dt][4 * qq + e] * inv);
      *reinterpret_cast<Q*>(orow + dt * 32 + 8 * qq + 4 * lg) = v;
    }
  if (lg == 0) lse[((int64_t)b * NH + h) * T_ + q] = (m + log2f(l)) * LN2;
}

// x as the sum of three bf16 values (x = h + m + l to about 2^-24 relative):
// each remainder is exact in fp32, so the split loses only the last rounding.
__device__ __forceinline__ void split3_bf16(float x, bf16x8& v, int at) {
  const bf16 h = (bf16)x;
  const float r = x - (float)h;
  const bf16 m = (bf16)r;
  v[at] = h;
  v[at + 1] = m;
  v[at + 2] = (bf16)(r - (float)m);
  v[at + 3] = (bf16)0.f;
}

// ------------------------------------------------------------------------
// dQ.  grid (NH*B, ceil(T/128)), heavy blocks first.  Per query column (one per lane):
// D = rowsum(dO * O) (stored for the dK/dV kernel, which runs after this one),
// P^T = exp(S^T - LSE), dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ = scale dS K.
// Per key tile: K and V rows; K^T fragments come from transposing reads.
// ------------------------------------------------------------------------
template <typename T, int HD>
__global__ void __launch_bounds__(NW * 64, 2) attn_dq_kernel(const T* __restrict__ qkv, const T* __restrict__ out,
                                                             const T* __restrict__ dout, const float* __restrict__ lse,
                                                             float* __restrict__ dsum, T* __restrict__ dqkv,
                                                             int T_, int NH, float sl2, float scale) {
  typedef RowTile<T, HD> RT;
  constexpr int LD = RT::LD, ND = HD / 16, NDT = HD / 32;
  typedef typename Frag<T>::type F;
  typedef typename Quad<T>::type Q;
  __shared__ __attribute__((aligned(16))) T Ks[2][KT * LD];
  __shared__ __attribute__((aligned(16))) T Vs[2][KT * LD];

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), lr = lane & 31, lg = lane >> 5;
  const int qblk = gridDim.y - 1 - blockIdx.y;  // heaviest (latest) query blocks dispatch first
  const int h = blockIdx.x % NH, b = blockIdx.x / NH;
  const int C = NH * HD, S3 = 3 * C;
  const int q0 = qblk * NW * WQ + w * WQ;
  const bool active = q0 < T_;
  const T* base = qkv + (int64_t)b * T_ * S3;
  const T* kbase = base + C + h * HD;
  const T* vbase = base + 2 * C + h * HD;
  const int q = q0 + lr;

  F qf[ND], df[ND];
  float lse2 = 0.f, dq_d = 0.f;
  if (active) {
    // the lane pair (l, l^32) holds the query's dO row: each half dots its
    // 8-element slices with O, in slice order, then the halves are added
    float part = 0.f;
#pragma unroll
    for (int ds = 0; ds < ND; ds++) {
      qf[ds] = ld8(base + (int64_t)q * S3 + h * HD + ds * 16 + 8 * lg);
      df[ds] = ld8(dout + ((int64_t)b * T_ + q) * C + h * HD + ds * 16 + 8 * lg);
      const F of = ld8(out + ((int64_t)b * T_ + q) * C + h * HD + ds * 16 + 8 * lg);
#pragma unroll
      for (int e = 0; e < 8; e++) part = fmaf(to_f<T>(df[ds][e]), to_f<T>(of[e]), part);
    }
    const float other = __shfl_xor(part, 32, 64);
    dq_d = lg == 0 ? part + other : other + part;
    lse2 = lse[((int64_t)b * NH + h) * T_ + q] * LOG2E;
    if (lg == 0) dsum[((int64_t)b * NH + h) * T_ + q] = dq_d;
  }
  f32x16 dq[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; dt++) dq[dt] = f32x16{};

  const int ntiles = min(T_, (qblk + 1) * NW * WQ) / KT;
  RT kt, vt;
  kt.load(kbase, S3, tid);
  vt.load(vbase, S3, tid);
  kt.store(Ks[0], tid);
  vt.store(Vs[0], tid);
  __syncthreads();
  // One 64-key tile: prefetch the next tile, compute, stage the prefetch.
  // Only the last two tiles can straddle one of the block's queries, so they
  // run a copy with the causal mask and the rest a copy without it.
  auto iteration = [&](int it, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int cur = it & 1, kv0 = it * KT;
    const bool more = it + 1 < ntiles;
    if (more) {
      kt.load(kbase + (int64_t)(kv0 + KT) * S3, S3, tid);
      vt.load(vbase + (int64_t)(kv0 + KT) * S3, S3, tid);
    }
    if (active && kv0 <= q0 + WQ - 1) {
      // key kl of the tile is masked for this lane's query when kl > lim
      const int lim = q - kv0 - 4 * lg;
      // the tile's two 32-key halves one after the other: one S^T and one
      // dP^T accumulator live at a time
#pragma unroll
      for (int c2 = 0; c2 < 2; c2++) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ds = 0; ds < ND; ds++) {
          mma16(s, ld8(Ks[cur] + (c2 * 32 + lr) * LD + ds * 16 + 8 * lg), qf[ds]);
          mma16(dp, ld8(Vs[cur] + (c2 * 32 + lr) * LD + ds * 16 + 8 * lg), df[ds]);
        }
#pragma unroll
        for (int r = 0; r < 16; r++) {
          s[r] = fast_exp2(fmaf(s[r], sl2, -lse2));
          if (MASK && c2 * 32 + 8 * (r / 4) + (r % 4) > lim) s[r] = 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; r++) s[r] = s[r] * (dp[r] - dq_d);  // dS^T
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
          const F sf = acc_frag<T>(s, h2);
#pragma unroll
          for (int dt = 0; dt < NDT; dt++) mma16(dq[dt], ld_tsplit<T, LD>(Ks[cur], dt * 32, 2 * c2 + h2, lane), sf);
        }
      }
    }
    if (more) {
      kt.store(Ks[cur ^ 1], tid);
      vt.store(Vs[cur ^ 1], tid);
    }
    __syncthreads();
  };
  static_assert(NW * WQ == 2 * KT, "a block's queries span two key tiles");
  const int nplain = max(0, ntiles - 2);
  for (int it = 0; it < nplain; it++) iteration(it, std::false_type{});
  for (int it = nplain; it < ntiles; it++) iteration(it, std::true_type{});
  if (!active) return;
  T* row = dqkv + ((int64_t)b * T_ + q) * S3 + h * HD;
#pragma unroll
  for (int dt = 0; dt < NDT; dt++)
#pragma unroll
    for (int qq = 0; qq < 4; qq++) {
      Q v;
#pragma unroll
      for (int e = 0; e < 4; e++) v[e] = from_f<T>(dq[dt][4 * qq + e] * scale);
      *reinterpret_cast<Q*>(row + dt * 32 + 8 * qq + 4 * lg) = v;
    }
}

// ------------------------------------------------------------------------
// dK, dV.  grid (NH*B, ceil(T/128)), heavy blocks first; each wave owns 32 keys and walks the
// query tiles at or after them.  Per key column (one per lane):
// P = exp(S - LSE), dV += dO^T P, dP = dO V^T, dS = P (dP - D), dK += scale Q^T dS.
// Per query tile: Q and dO rows (their transposes come from transposing
// reads), and the tile's LSE and D values.
//
// bf16: the per-query terms enter through the matrix core.  S and dP are
// laid out query x key, so LSE and D vary along the slots of each lane's
// accumulator, and reading them per element would cost as many LDS bytes as
// the S operand.  Instead each query row of the tile carries eight bf16
// values [-LSE*sqrt(hd) as three terms, 0, -D as three terms, 0]: one more
// MFMA per accumulator, against a ones fragment that picks the first or the
// second triple, starts S at S - LSE*sqrt(hd) (so P = exp2(S * log2(e) /
// sqrt(hd))) and dP at dP - D.
// ------------------------------------------------------------------------
template <typename T, int HD>
__global__ void __launch_bounds__(NW * 64, 2) attn_dkv_kernel(const T* __restrict__ qkv, const T* __restrict__ dout,
                                                           const float* __restrict__ lse, const float* __restrict__ dsum,
                                                           T* __restrict__ dqkv, int T_, int NH, float sl2,
                                                           float scale, float rs) {
  typedef RowTile<T, HD> RT;
  constexpr int LD = RT::LD, ND = HD / 16, NDT = HD / 32;
  typedef typename Frag<T>::type F;
  typedef typename Quad<T>::type Q;
  constexpr bool AUG = sizeof(T) == 2;  // per-query terms through the matrix core (bf16)
  __shared__ __attribute__((aligned(16))) T Qs[2][KT * LD];
  __shared__ __attribute__((aligned(16))) T Ds[2][KT * LD];
  __shared__ float Ls[AUG ? 1 : 2][AUG ? 1 : KT], Dd[AUG ? 1 : 2][AUG ? 1 : KT];
  __shared__ __attribute__((aligned(16))) bf16 Aug[AUG ? 2 : 1][AUG ? KT * 8 : 8];

  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), lr = lane & 31, lg = lane >> 5;
  const int kblk = blockIdx.y;  // early key blocks see the most queries: they dispatch first
  const int h = blockIdx.x % NH, b = blockIdx.x / NH;
  const int C = NH * HD, S3 = 3 * C;
  const int k0 = kblk * NW * WQ + w * WQ;
  const bool active = k0 < T_;
  const T* base = qkv + (int64_t)b * T_ * S3;
  const T* qbase = base + h * HD;
  const T* obase = dout + (int64_t)b * T_ * C + h * HD;
  const bool ldl = tid < KT;  // these threads also bring the tile's LSE and D values
  const int kv = k0 + lr;

  F kf[ND], vf[ND];
  if (active) {
#pragma unroll
    for (int ds = 0; ds < ND; ds++) {
      kf[ds] = ld8(base + (int64_t)kv * S3 + C + h * HD + ds * 16 + 8 * lg);
      vf[ds] = ld8(base + (int64_t)kv * S3 + 2 * C + h * HD + ds * 16 + 8 * lg);
    }
  }
  f32x16 dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; dt++) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }
  const float* lrow = lse + ((int64_t)b * NH + h) * T_;
  const float* drow = dsum + ((int64_t)b * NH + h) * T_;
  // ones fragments (key side) that pick the LSE triple or the D triple of a
  // query's eight augmentation values; lanes of the upper group add zeros
  F onesL, onesD;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    onesL[e] = from_f<T>(lg == 0 && e < 3 ? 1.f : 0.f);
    onesD[e] = from_f<T>(lg == 0 && e >= 4 && e < 7 ? 1.f : 0.f);
  }
  // a query's values as staged: LSE in log2 units (fp32), or the bf16
  // augmentation row [-LSE*sqrt(hd) x3, 0, -D x3, 0]
  auto stage_rowvals = [&](int buf, float l_nat, float d) {
    if constexpr (AUG) {
      bf16x8 a;
      split3_bf16(-l_nat * rs, a, 0);
      split3_bf16(-d, a, 4);
      *reinterpret_cast<bf16x8*>(&Aug[buf][tid * 8]) = a;
    } else {
      Ls[buf][tid] = l_nat * LOG2E;
      Dd[buf][tid] = d;
    }
  };

  const int qt_begin = (kblk * NW * WQ / KT) * KT;
  const int ntiles = (T_ - qt_begin) / KT;
  RT qt, ot;
  float sl = 0.f, sd = 0.f;
  qt.load(qbase + (int64_t)qt_begin * S3, S3, tid);
  ot.load(obase + (int64_t)qt_begin * C, C, tid);
  if (ldl) {
    sl = lrow[qt_begin + tid];
    sd = drow[qt_begin + tid];
  }
  qt.store(Qs[0], tid);
  ot.store(Ds[0], tid);
  if (ldl) stage_rowvals(0, sl, sd);
  __syncthreads();
  // One 64-query tile: prefetch the next tile, compute, stage the prefetch.
  // Only the first two tiles of a block can straddle one of its waves' keys,
  // so they run a copy with the causal mask and the rest a copy without it,
  // each one branch-free block the compiler schedules across both halves.
  auto iteration = [&](int it, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int cur = it & 1, qt0 = qt_begin + it * KT;
    const bool more = it + 1 < ntiles;
    if (more) {
      qt.load(qbase + (int64_t)(qt0 + KT) * S3, S3, tid);
      ot.load(obase + (int64_t)(qt0 + KT) * C, C, tid);
      if (ldl) {
        sl = lrow[qt0 + KT + tid];
        sd = drow[qt0 + KT + tid];
      }
    }
    if (active && qt0 + KT - 1 >= k0) {
      // query ql of the tile is masked for this lane's key when ql < lim
      const int lim = kv - qt0 - 4 * lg;
      // S and dP of both 32-query halves first, so the exponentials of the
      // first half overlap the matrix products of the second
      f32x16 s[2], dp[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; c2++) {
        s[c2] = f32x16{};
        dp[c2] = f32x16{};
        if constexpr (AUG) {
          const F av = *reinterpret_cast<const F*>(&Aug[cur][(c2 * 32 + lr) * 8]);
          mma16(s[c2], av, onesL);
          mma16(dp[c2], av, onesD);
        }
#pragma unroll
        for (int ds = 0; ds < ND; ds++) {
          mma16(s[c2], ld8(Qs[cur] + (c2 * 32 + lr) * LD + ds * 16 + 8 * lg), kf[ds]);
          mma16(dp[c2], ld8(Ds[cur] + (c2 * 32 + lr) * LD + ds * 16 + 8 * lg), vf[ds]);
        }
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; c2++) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int ql = c2 * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
          if constexpr (AUG) {
            s[c2][r] = fast_exp2(s[c2][r] * sl2);
          } else {
            s[c2][r] = fast_exp2(fmaf(s[c2][r], sl2, -Ls[cur][ql]));
          }
          if (MASK && c2 * 32 + 8 * (r / 4) + (r % 4) < lim) s[c2][r] = 0.f;
          if constexpr (AUG) {
            dp[c2][r] = s[c2][r] * dp[c2][r];
          } else {
            dp[c2][r] = s[c2][r] * (dp[c2][r] - Dd[cur][ql]);
          }
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
          const int c = 2 * c2 + h2;
          const F pf = acc_frag<T>(s[c2], h2);
          const F sf = acc_frag<T>(dp[c2], h2);
#pragma unroll
          for (int dt = 0; dt < NDT; dt++) {
            mma16(dv[dt], ld_tsplit<T, LD>(Ds[cur], dt * 32, c, lane), pf);
            mma16(dk[dt], ld_tsplit<T, LD>(Qs[cur], dt * 32, c, lane), sf);
          }
        }
      }
    }
    if (more) {
      qt.store(Qs[cur ^ 1], tid);
      ot.store(Ds[cur ^ 1], tid);
      if (ldl) stage_rowvals(cur ^ 1, sl, sd);
    }
    __syncthreads();
  };
  static_assert(NW * WQ == 2 * KT, "a block's keys span two query tiles");
  const int nmask = min(2, ntiles);
  for (int it = 0; it < nmask; it++) iteration(it, std::true_type{});
  for (int it = nmask; it < ntiles; it++) iteration(it, std::false_type{});
  if (!active) return;
  T* row = dqkv + ((int64_t)b * T_ + kv) * S3 + h * HD;
#pragma unroll
  for (int dt = 0; dt < NDT; dt++)
#pragma unroll
    for (int qq = 0; qq < 4; qq++) {
      Q vk, vv;
#pragma unroll
      for (int e = 0; e < 4; e++) {
        vk[e] = from_f<T>(dk[dt][4 * qq + e] * scale);
        vv[e] = from_f<T>(dv[dt][4 * qq + e]);
      }
      *reinterpret_cast<Q*>(row + C + dt * 32 + 8 * qq + 4 * lg) = vk;
      *reinterpret_cast<Q*>(row + 2 * C + dt * 32 + 8 * qq + 4 * lg) = vv;
    }
}

template <typename T, int HD>
hipError_t fwd_t(hipStream_t st, const void* qkv, void* out, float* lse, int B, int T_, int NH) {
  // blockIdx.x (dispatched fastest) walks the heads, blockIdx.y the row
  // blocks from the most work to the least, so the long blocks start first
  dim3 grid(NH * B, (T_ + NW * WQ - 1) / (NW * WQ));
  const float sl2 = LOG2E / sqrtf((float)HD);
  hipLaunchKernelGGL((attn_fwd_kernel<T, HD>), grid, dim3(NW * 64), 0, st, static_cast<const T*>(qkv),
                     static_cast<T*>(out), lse, T_, NH, sl2);
  return hipGetLastError();
}

template <typename T, int HD>
hipError_t dq_t(hipStream_t st, const void* qkv, const void* out, const void* dout, const float* lse, float* dsum,
                void* dqkv, int B, int T_, int NH) {
  // blockIdx.x (dispatched fastest) walks the heads, blockIdx.y the row
  // blocks from the most work to the least, so the long blocks start first
  dim3 grid(NH * B, (T_ + NW * WQ - 1) / (NW * WQ));
  const float scale = 1.f / sqrtf((float)HD), sl2 = LOG2E * scale;
  hipLaunchKernelGGL((attn_dq_kernel<T, HD>), grid, dim3(NW * 64), 0, st, static_cast<const T*>(qkv),
                     static_cast<const T*>(out), static_cast<const T*>(dout), lse, dsum, static_cast<T*>(dqkv), T_, NH,
                     sl2, scale);
  return hipGetLastError();
}

template <typename T, int HD>
hipError_t dkv_t(hipStream_t st, const void* qkv, const void* dout, const float* lse, const float* dsum, void* dqkv,
                 int B, int T_, int NH) {
  // blockIdx.x (dispatched fastest) walks the heads, blockIdx.y the row
  // blocks from the most work to the least, so the long blocks start first
  dim3 grid(NH * B, (T_ + NW * WQ - 1) / (NW * WQ));
  const float rs = sqrtf((float)HD), scale = 1.f / rs, sl2 = LOG2E * scale;
  hipLaunchKernelGGL((attn_dkv_kernel<T, HD>), grid, dim3(NW * 64), 0, st, static_cast<const T*>(qkv),
                     static_cast<const T*>(dout), lse, dsum, static_cast<T*>(dqkv), T_, NH, sl2, scale, rs);
  return hipGetLastError();
}

}  // namespace

hipError_t attn_fwd(hipStream_t st, Prec p, const void* qkv, void* out, float* lse, int B, int T_, int NH, int hd) {
  if (T_ % KT != 0) return hipErrorInvalidValue;
  if (p == BF16) {
    if (hd == 64) return fwd_t<bf16, 64>(st, qkv, out, lse, B, T_, NH);
    if (hd == 32) return fwd_t<bf16, 32>(st, qkv, out, lse, B, T_, NH);
  } else {
    if (hd == 64) return fwd_t<float, 64>(st, qkv, out, lse, B, T_, NH);
    if (hd == 32) return fwd_t<float, 32>(st, qkv, out, lse, B, T_, NH);
  }
  return hipErrorInvalidValue;
}

#define ATTN_HD_DISPATCH(CALL)                            \
  if (T_ % KT != 0) return hipErrorInvalidValue;           \
  if (p == BF16) {                                         \
    if (hd == 64) return CALL(bf16, 64);                   \
    if (hd == 32) return CALL(bf16, 32);                   \
  } else {                                                 \
    if (hd == 64) return CALL(float, 64);                  \
    if (hd == 32) return CALL(float, 32);                  \
  }                                                        \
  return hipErrorInvalidValue;

hipError_t attn_bwd_dq(hipStream_t st, Prec p, const void* qkv, const void* out, const void* dout, const float* lse,
                       float* dsum, void* dqkv, int B, int T_, int NH, int hd) {
#define DQ_CALL(TT, H) dq_t<TT, H>(st, qkv, out, dout, lse, dsum, dqkv, B, T_, NH)
  ATTN_HD_DISPATCH(DQ_CALL)
#undef DQ_CALL
}

hipError_t attn_bwd_dkv(hipStream_t st, Prec p, const void* qkv, const void* dout, const float* lse, const float* dsum,
                        void* dqkv, int B, int T_, int NH, int hd) {
#define DKV_CALL(TT, H) dkv_t<TT, H>(st, qkv, dout, lse, dsum, dqkv, B, T_, NH)
  ATTN_HD_DISPATCH(DKV_CALL)
#undef DKV_CALL
}
#undef ATTN_HD_DISPATCH

}  // namespace gpt2k
