// gemm.hip -- MFMA matmul for gfx950 with fused epilogues.
//
// out[i][j] = sum_r A(i, r) * B(j, r): every linear layer of the GPT-2 step,
// forward (x W^T), input gradient (dy W) and weight gradient (dy^T x), and
// the tied output layer ("Karpathy's four-hour GPT-2 reproduction in one
// post", part 1).  Either operand may be stored with the reduction index
// contiguous (A(i, r) = A[i*lda + r]) or strided (A[r*lda + i]); strided
// tiles are transposed in registers (8x8 blocks) on their way into LDS so the
// MFMA fragments are always 16-byte LDS reads.
//
// Block tile BM x BN, reduction step BK, double-buffered LDS with register
// prefetch of the next tile; WI x WJ waves, each owning a (BM/WI) x (BN/WJ)
// tile of 32x32 accumulators.  The MFMA row operand is the B side, so each
// lane ends with runs of four consecutive output columns (vector stores).
#include "common.h"
#include "kernels.h"

namespace gpt2k {
namespace {

template <typename T> struct Vec16;  // 16 bytes of T
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int n = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int n = 4; };

// Global -> LDS loader of one R x BK operand tile, LDS layout [R][LDK] with
// the reduction index contiguous.
template <typename T, int R, int BK, int LDK, int NT, int TRANS>
struct TileLoader;

// Reduction index contiguous in memory: X(row, r) = X[row*ld + r].
template <typename T, int R, int BK, int LDK, int NT>
struct TileLoader<T, R, BK, LDK, NT, 0> {
  static constexpr int VE = Vec16<T>::n;
  static constexpr int CPR = BK / VE;
  static constexpr int TOTAL = R * CPR;
  static constexpr int PER = TOTAL / NT;
  static_assert(TOTAL % NT == 0, "tile does not split evenly over threads");
  f32x4 reg[PER];
  __device__ __forceinline__ void load(const T* X, int64_t ld, int row0, int nrows, int k0, int tid) {
#pragma unroll
    for (int c = 0; c < PER; c++) {
      const int idx = tid + c * NT;
      const int row = idx / CPR, kc = idx % CPR;
      // rows past the edge read the last row: they only feed outputs the epilogue drops
      const int r = min(row0 + row, nrows - 1);
      reg[c] = *reinterpret_cast<const f32x4*>(X + (int64_t)r * ld + k0 + kc * VE);
    }
  }
  __device__ __forceinline__ void store(T* s, int tid) {
#pragma unroll
    for (int c = 0; c < PER; c++) {
      const int idx = tid + c * NT;
      const int row = idx / CPR, kc = idx % CPR;
      *reinterpret_cast<f32x4*>(s + row * LDK + kc * VE) = reg[c];
    }
  }
};

// Reduction index strided: X(row, r) = X[r*ld + row].  Each thread moves an
// 8 (r) x VE (rows) block: eight 16-byte loads along rows, an in-register
// transpose, then VE stores of 8 consecutive r values.
template <typename T, int R, int BK, int LDK, int NT>
struct TileLoader<T, R, BK, LDK, NT, 1> {
  typedef typename Vec16<T>::type V;
  typedef typename Frag<T>::type F;
  static constexpr int VE = Vec16<T>::n;
  static constexpr int NCB = R / VE;
  static constexpr int TOTAL = (BK / 8) * NCB;
  static constexpr int PER = (TOTAL + NT - 1) / NT;
  V reg[PER][8];
  __device__ __forceinline__ void load(const T* X, int64_t ld, int row0, int nrows, int k0, int tid) {
#pragma unroll
    for (int c = 0; c < PER; c++) {
      const int blk = tid + c * NT;
      if (TOTAL % NT != 0 && blk >= TOTAL) continue;
      const int rb = blk / NCB, cb = blk % NCB;
      // column blocks past the edge re-read the last one (their outputs are dropped)
      const int col = min(row0 + cb * VE, nrows - VE);
#pragma unroll
      for (int a = 0; a < 8; a++) reg[c][a] = *reinterpret_cast<const V*>(X + (int64_t)(k0 + rb * 8 + a) * ld + col);
    }
  }
  __device__ __forceinline__ void store(T* s, int tid) {
#pragma unroll
    for (int c = 0; c < PER; c++) {
      const int blk = tid + c * NT;
      if (TOTAL % NT != 0 && blk >= TOTAL) continue;
      const int rb = blk / NCB, cb = blk % NCB;
#pragma unroll
      for (int b = 0; b < VE; b++) {
        F w;
#pragma unroll
        for (int a = 0; a < 8; a++) w[a] = reg[c][a][b];
        st8(s + (cb * VE + b) * LDK + rb * 8, w);
      }
    }
  }
};

template <typename T, int BM, int BN, int BK, int WI, int WJ, int AT, int BT, int EPI>
__global__ void __launch_bounds__(WI * WJ * 64) gemm_kernel(GemmArgs g) {
  constexpr int NT = WI * WJ * 64;
  constexpr int VE = Vec16<T>::n;
  constexpr int LDK = BK + VE;  // 16 bytes of row padding against LDS bank conflicts
  constexpr int WTI = BM / WI, WTJ = BN / WJ;
  constexpr int TI = WTI / 32, TJ = WTJ / 32;
  typedef typename Frag<T>::type F;
  typedef typename Quad<T>::type Q;
  __shared__ __attribute__((aligned(16))) T sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) T sB[2][BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave / WJ, wj = wave % WJ;
  const int nbi = (g.M + BM - 1) / BM, nbj = (g.N + BN - 1) / BN;
  const int tile = xcd_remap(blockIdx.x, nbi * nbj);
  // Grouped tile order: GM consecutive row-tiles sweep the columns together.
  constexpr int GM = 8;
  const int group = tile / (GM * nbj);
  const int first_i = group * GM;
  const int gsize = min(nbi - first_i, GM);
  const int tig = tile - group * GM * nbj;
  const int bi = first_i + tig % gsize, bj = tig / gsize;
  const int i0 = bi * BM, j0 = bj * BN;

  const int kchunk = g.K / g.splits;
  const int kbeg = blockIdx.y * kchunk;
  const int nk = kchunk / BK;
  const T* A = static_cast<const T*>(g.A);
  const T* Bm = static_cast<const T*>(g.B);

  TileLoader<T, BM, BK, LDK, NT, AT> la;
  TileLoader<T, BN, BK, LDK, NT, BT> lb;
  f32x16 acc[TI][TJ];
#pragma unroll
  for (int ti = 0; ti < TI; ti++)
#pragma unroll
    for (int tj = 0; tj < TJ; tj++) acc[ti][tj] = f32x16{};

  la.load(A, g.lda, i0, g.M, kbeg, tid);
  lb.load(Bm, g.ldb, j0, g.N, kbeg, tid);
  la.store(sA[0], tid);
  lb.store(sB[0], tid);
  __syncthreads();

  const int lr = lane & 31, lg = lane >> 5;
  for (int kt = 0; kt < nk; kt++) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      la.load(A, g.lda, i0, g.M, kbeg + (kt + 1) * BK, tid);
      lb.load(Bm, g.ldb, j0, g.N, kbeg + (kt + 1) * BK, tid);
    }
    const T* as = sA[cur];
    const T* bs = sB[cur];
#pragma unroll
    for (int s = 0; s < BK / 16; s++) {
      F fa[TI], fb[TJ];
#pragma unroll
      for (int ti = 0; ti < TI; ti++) fa[ti] = ld8(as + (wi * WTI + ti * 32 + lr) * LDK + s * 16 + 8 * lg);
#pragma unroll
      for (int tj = 0; tj < TJ; tj++) fb[tj] = ld8(bs + (wj * WTJ + tj * 32 + lr) * LDK + s * 16 + 8 * lg);
#pragma unroll
      for (int ti = 0; ti < TI; ti++)
#pragma unroll
        for (int tj = 0; tj < TJ; tj++) mma16(acc[ti][tj], fb[tj], fa[ti]);
    }
    if (kt + 1 < nk) {
      la.store(sA[cur ^ 1], tid);
      lb.store(sB[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // Epilogue: accumulator r of lane l holds out[i][j] with
  // i = tile row base + l%32, j = tile col base + 8*(r/4) + 4*(l/32) + r%4.
#pragma unroll
  for (int ti = 0; ti < TI; ti++) {
    const int i = i0 + wi * WTI + ti * 32 + lr;
    if (i >= g.M) continue;
#pragma unroll
    for (int tj = 0; tj < TJ; tj++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int j = j0 + wj * WTJ + tj * 32 + 8 * q + 4 * lg;
        if (j >= g.N) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; e++) v[e] = acc[ti][tj][4 * q + e];
        if constexpr (EPI == EPI_STORE || EPI == EPI_F32) {
#pragma unroll
          for (int e = 0; e < 4; e++) v[e] *= g.alpha;
        }
        if constexpr (EPI == EPI_STORE) {
          if (g.bias) {
            const f32x4 b = *reinterpret_cast<const f32x4*>(g.bias + j);
#pragma unroll
            for (int e = 0; e < 4; e++) v[e] += b[e];
          }
          Q o;
#pragma unroll
          for (int e = 0; e < 4; e++) o[e] = from_f<T>(v[e]);
          *reinterpret_cast<Q*>(static_cast<T*>(g.C) + (int64_t)i * g.ldc + j) = o;
        } else if constexpr (EPI == EPI_GELU) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(g.bias + j);
          Q u, o;
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const float x = v[e] + b[e];
            u[e] = from_f<T>(x);
            o[e] = from_f<T>(gelu_tanh(x));
          }
          *reinterpret_cast<Q*>(static_cast<T*>(g.aux) + (int64_t)i * g.ldaux + j) = u;
          *reinterpret_cast<Q*>(static_cast<T*>(g.C) + (int64_t)i * g.ldc + j) = o;
        } else if constexpr (EPI == EPI_RESID) {
          const f32x4 b = *reinterpret_cast<const f32x4*>(g.bias + j);
          const f32x4 r = *reinterpret_cast<const f32x4*>(g.resid + (int64_t)i * g.ldr + j);
          f32x4 o;
#pragma unroll
          for (int e = 0; e < 4; e++) o[e] = r[e] + (v[e] + b[e]);
          *reinterpret_cast<f32x4*>(static_cast<float*>(g.C) + (int64_t)i * g.ldc + j) = o;
        } else if constexpr (EPI == EPI_GELU_BWD) {
          const Q u = *reinterpret_cast<const Q*>(static_cast<const T*>(g.aux) + (int64_t)i * g.ldaux + j);
          Q o;
#pragma unroll
          for (int e = 0; e < 4; e++) o[e] = from_f<T>(v[e] * gelu_tanh_grad(to_f<T>(u[e])));
          *reinterpret_cast<Q*>(static_cast<T*>(g.C) + (int64_t)i * g.ldc + j) = o;
        } else {  // EPI_F32
          float* C = static_cast<float*>(g.C) + (int64_t)blockIdx.y * g.split_stride + (int64_t)i * g.ldc + j;
          f32x4 o;
          if (g.accumulate) {
            const f32x4 c = *reinterpret_cast<const f32x4*>(C);
#pragma unroll
            for (int e = 0; e < 4; e++) o[e] = c[e] + v[e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; e++) o[e] = v[e];
          }
          *reinterpret_cast<f32x4*>(C) = o;
        }
      }
    }
  }
}

template <typename T, int BM, int BN, int WI, int WJ, int AT, int BT, int EPI>
hipError_t launch(hipStream_t st, const GemmArgs& g) {
  constexpr int BK = sizeof(T) == 2 ? 64 : 32;
  constexpr int VE = Vec16<T>::n;
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.splits < 1 || g.K % (g.splits * BK) != 0 || g.M % VE != 0 || g.N % 8 != 0 || g.lda % VE != 0 ||
      g.ldb % VE != 0 || (EPI != EPI_F32 && g.splits != 1))
    return hipErrorInvalidValue;
  const int nbi = (g.M + BM - 1) / BM, nbj = (g.N + BN - 1) / BN;
  dim3 grid(nbi * nbj, g.splits);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WI, WJ, AT, BT, EPI>), grid, dim3(WI * WJ * 64), 0, st, g);
  return hipGetLastError();
}

// Tile shape per operand layout and output shape (bf16), from a sweep of the
// step's matmuls on MI355X: 256x192 where the output width is a multiple of
// 192 up to 1536 (one wave of 256 CUs for 16384 x 768), 256x256 with eight
// waves for wide outputs, 128x128 otherwise.
enum TileKind { TILE_128 = 0, TILE_256x192 = 1, TILE_256_W8 = 2 };

TileKind choose_tile(Prec p, int a_t, int b_t, int M, int N) {
  if (p != BF16 || M < 256) return TILE_128;
  const bool narrow = N % 192 == 0 && N <= 1536;
  if (a_t && b_t) return (int64_t)M * N >= 8000000 ? TILE_256_W8 : narrow ? TILE_256x192 : TILE_256_W8;
  if (N >= 3072) return TILE_256_W8;
  if (narrow) return TILE_256x192;
  return TILE_128;
}

template <typename T, int AT, int BT, int EPI>
hipError_t launch_tiled(hipStream_t st, const GemmArgs& g, TileKind k) {
  if constexpr (sizeof(T) == 2) {
    if (k == TILE_256x192) return launch<T, 256, 192, 2, 2, AT, BT, EPI>(st, g);
    if (k == TILE_256_W8) {
      if (AT || BT) return launch<T, 256, 256, 2, 4, AT, BT, EPI>(st, g);
      return launch<T, 256, 256, 4, 2, AT, BT, EPI>(st, g);
    }
  }
  return launch<T, 128, 128, 2, 2, AT, BT, EPI>(st, g);
}

template <typename T>
hipError_t dispatch(hipStream_t st, int a_t, int b_t, int epi, const GemmArgs& g, TileKind k) {
  if (!a_t && !b_t) {
    if (epi == EPI_STORE) return launch_tiled<T, 0, 0, EPI_STORE>(st, g, k);
    if (epi == EPI_GELU) return launch_tiled<T, 0, 0, EPI_GELU>(st, g, k);
    if (epi == EPI_RESID) return launch_tiled<T, 0, 0, EPI_RESID>(st, g, k);
  } else if (!a_t && b_t) {
    if (epi == EPI_STORE) return launch_tiled<T, 0, 1, EPI_STORE>(st, g, k);
    if (epi == EPI_GELU_BWD) return launch_tiled<T, 0, 1, EPI_GELU_BWD>(st, g, k);
  } else if (a_t && b_t) {
    if (epi == EPI_F32) return launch_tiled<T, 1, 1, EPI_F32>(st, g, k);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t gemm(hipStream_t st, Prec p, int a_t, int b_t, int epi, const GemmArgs& g) {
  const TileKind k = choose_tile(p, a_t, b_t, g.M, g.N);
  return p == BF16 ? dispatch<bf16>(st, a_t, b_t, epi, g, k) : dispatch<float>(st, a_t, b_t, epi, g, k);
}

int gemm_split_hint(Prec p, int a_t, int b_t, int M, int N, int K) {
  const TileKind k = choose_tile(p, a_t, b_t, M, N);
  const int bm = k == TILE_128 ? 128 : 256, bn = k == TILE_256x192 ? 192 : (k == TILE_256_W8 ? 256 : 128);
  const int bk = p == BF16 ? 64 : 32;
  const int tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  // one block per CU for the large tiles, two for 128x128; the reduction must
  // split into equal multiples of the K step
  const int target = k == TILE_128 ? 512 : 256;
  int s = 1;
  while (s < 16 && tiles * s < target && K % (2 * s * bk) == 0) s *= 2;
  return s;
}

}  // namespace gpt2k
