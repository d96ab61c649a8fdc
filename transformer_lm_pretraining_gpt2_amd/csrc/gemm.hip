// gemm.hip -- MFMA matmul for gfx950 with fused epilogues.
//
// out[i][j] = sum_r A(i, r) * B(j, r): every linear layer of the GPT-2 step,
// forward (x W^T), input gradient (dy W) and weight gradient (dy^T x), and
// the tied output layer ("Karpathy's four-hour GPT-2 reproduction in one
// post", part 1).  Either operand may be stored with the reduction index
// contiguous (A(i, r) = A[i*lda + r]) or strided (A[r*lda + i]); strided
// tiles keep their global layout in LDS and their MFMA fragments come from the
// transposing LDS read.
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
template <> struct Vec16<fp8e4> { typedef f32x4 type; static constexpr int n = 16; };

// One operand tile (R output rows x BK reduction) on its way global ->
// registers -> LDS, and the MFMA fragments read back from LDS.
//  TRANS = 0: X(row, r) = X[row*ld + r]; LDS [R][BK + VE]  (reduction contiguous,
//             16-byte row pad keeps the fragment reads free of bank conflicts)
//  TRANS = 1: X(row, r) = X[r*ld + row]; LDS [BK][R + PADR] (kept in the global
//             layout; bf16 fragments come from the transposing LDS read
//             ds_read_b64_tr_b16, fp32 fragments from scalar reads)
// Both layouts are filled with plain 16-byte copies.
constexpr int PADR = 32;  // elements; a 64-byte pad puts the 4 rows one transposing read touches in distinct banks

template <typename T, int R, int BK, int NT, int TRANS>
struct Operand {
  static constexpr int VE = Vec16<T>::n;
  static constexpr int LD = TRANS ? R + PADR : BK + VE;         // LDS row length (elements)
  static constexpr int ELEMS = TRANS ? BK * LD : R * LD;        // LDS tile size (elements)
  static constexpr int CPR = TRANS ? R / VE : BK / VE;          // 16-byte chunks per global row
  static constexpr int PER = R * BK / VE / NT;                  // chunks per thread
  static_assert((R * BK / VE) % NT == 0, "tile does not split evenly over threads");
  typedef typename Frag<T>::type F;
  f32x4 reg[PER];
  // Global loads go through a buffer descriptor (base address in scalar
  // registers) whose base sits at the block's first row (reduction-contiguous
  // operands) or at the current reduction step (strided operands), so each
  // chunk's 32-bit byte offset stays inside one tile however large the
  // operand is; it is loop-invariant, and the reduction step is a uniform
  // scalar offset (contiguous operands) or a new base (strided operands).
  const T* base;
  int64_t ld_;
  uint32_t voff[PER];

  __device__ __forceinline__ void init(const T* X, int64_t ld, int row0, int nrows, int tid) {
    ld_ = ld;
    base = TRANS ? X : X + (int64_t)row0 * ld;  // row0 < nrows: every tile starts inside the operand
#pragma unroll
    for (int c = 0; c < PER; c++) {
      const int idx = tid + c * NT;
      const int gr = idx / CPR, gc = idx % CPR;
      if constexpr (TRANS == 0) {
        // rows past the edge re-read the last row: they only feed outputs the epilogue drops
        const int r = min(row0 + gr, nrows - 1);
        voff[c] = (uint32_t)(((int64_t)(r - row0) * ld + gc * VE) * (int64_t)sizeof(T));
      } else {
        const int col = min(row0 + gc * VE, nrows - VE);
        voff[c] = (uint32_t)(((int64_t)gr * ld + col) * (int64_t)sizeof(T));
      }
    }
  }
  __device__ __forceinline__ void load(int k0) {
    __amdgpu_buffer_rsrc_t rsrc;
    int soff = 0;
    if constexpr (TRANS == 0) {
      rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), 0, -1, 0x00020000);
      soff = k0 * (int)sizeof(T);
    } else {
      rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base + (int64_t)k0 * ld_), 0, -1, 0x00020000);
    }
#pragma unroll
    for (int c = 0; c < PER; c++)
      reg[c] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff[c], soff, 0));
  }
  __device__ __forceinline__ void store(T* s, int tid) const {
#pragma unroll
    for (int c = 0; c < PER; c++) {
      const int idx = tid + c * NT;
      const int gr = idx / CPR, gc = idx % CPR;
      *reinterpret_cast<f32x4*>(s + gr * LD + gc * VE) = reg[c];
    }
  }
  // Strided operands (TRANS = 1): every chunk a thread stages covers the same
  // VE operand rows (NT is a multiple of the chunks per reduction row), so
  // the thread can keep per-row sums of the reduction values it stages,
  // chunk by chunk in reduction order.  w is 1 (or 0 for a staged re-read
  // past the last step: a multiply, not a branch, which would split the main
  // loop and cost register copies).
  __device__ __forceinline__ void row_sums(float (&acc)[VE], float w) const {
    static_assert(TRANS == 1 && NT % CPR == 0, "row sums need a fixed row range per thread");
#pragma unroll
    for (int c = 0; c < PER; c++) {
      if constexpr (sizeof(T) == 2) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, reg[c]);
#pragma unroll
        for (int e = 0; e < VE; e++) acc[e] = __builtin_fmaf((float)v[e], w, acc[e]);
      } else {
#pragma unroll
        for (int e = 0; e < VE; e++) acc[e] = __builtin_fmaf(reg[c][e], w, acc[e]);
      }
    }
  }
  // part p of NP of the store (chunks spread over the substeps of a tile)
  template <int NP>
  __device__ __forceinline__ void store_part(T* s, int tid, int p) const {
#pragma unroll
    for (int c = 0; c < PER; c++) {
      if (c * NP / PER != p) continue;
      const int idx = tid + c * NT;
      const int gr = idx / CPR, gc = idx % CPR;
      *reinterpret_cast<f32x4*>(s + gr * LD + gc * VE) = reg[c];
    }
  }
  // Fragment of substep ks for rows rb .. rb+31: lane l gets row rb + l%32 and
  // reduction values 16*ks + 8*(l/32) + 0..7.
  static __device__ __forceinline__ F frag(const T* s, int rb, int ks, int lane) {
    if constexpr (sizeof(T) == 1) {
      // FP8: 32 values (two 16-byte reads) at reduction offset 64*ks + 32*(l/32)
      static_assert(TRANS == 0, "FP8 operands must be reduction-contiguous");
      const T* p = s + (rb + (lane & 31)) * LD + ks * 64 + 32 * (lane >> 5);
      const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 16);
      return __builtin_bit_cast(F, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else if constexpr (TRANS == 0) {
      return ld8(s + (rb + (lane & 31)) * LD + ks * 16 + 8 * (lane >> 5));
    } else if constexpr (sizeof(T) == 2) {
      // within each 16-lane group, lane j points at row r0 + j/4, columns
      // c0 + 4*(j%4) .. +3; the transposing read hands lane i the four rows at
      // column c0 + i
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const int j = lane & 15;
      const int kr = ks * 16 + 8 * (lane >> 5) + (j >> 2);
      const int col = rb + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      const T* p = s + kr * LD + col;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * LD));
      // whole-vector bit casts (element-wise casts of these vectors miscompile)
      const bf16x4 a = __builtin_bit_cast(bf16x4, lo), b = __builtin_bit_cast(bf16x4, hi);
      return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      F f;
      const T* p = s + (ks * 16 + 8 * (lane >> 5)) * LD + rb + (lane & 31);
#pragma unroll
      for (int e = 0; e < 8; e++) f[e] = p[e * LD];
      return f;
    }
  }
};

// acc + the sum of a fragment's 8 values, in slot order
__device__ __forceinline__ float frag_sum(bf16x8 f, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
#pragma unroll
  for (int e = 0; e < 8; e += 2) acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[e], f[e + 1]}, one, acc, false);
  return acc;
}

// Direct-to-LDS operand tile (bf16): buffer_load ... lds moves each lane's 16
// bytes from global memory straight into LDS, with no staging registers.  One
// such load writes 64 lanes x 16 bytes contiguously at a wave-uniform LDS
// address, so the tile has no row padding; instead the 16-byte chunks of each
// LDS row are permuted (XOR with a function of the row), which the loads apply
// by choosing which global chunk each lane fetches and the fragment reads undo.
//  TRANS = 0: LDS row q = operand row row0 + q, BK reduction values
//  TRANS = 1: LDS row q = reduction index k0 + q, R operand rows (R = 128 or
//             256, so every LDS row starts on the same bank)
// The permutations keep each fragment read conflict-free for 32 or 64 banks:
// the 16 (or 8) rows one pass of a 16-byte read touches land on distinct
// 16-byte bank groups; the transposing reads spread their 8 rows over all
// four 64-byte groups of a 256-byte bank line.
template <int R, int BK, int NW, int TRANS>
struct DtlOperand {
  static constexpr int ROWB = TRANS ? R * 2 : BK * 2;  // bytes per LDS row
  static constexpr int CPR = ROWB / 16;                // 16-byte chunks per LDS row
  static constexpr int BYTES = R * BK * 2;
  static constexpr int PER = BYTES / 1024 / NW;        // loads per wave per tile
  static_assert(BYTES % (1024 * NW) == 0, "tile does not split evenly over the waves");
  static_assert(TRANS ? (R == 128 || R == 256) : (CPR == 4 || CPR == 8), "unsupported tile for direct loads");
  const bf16* base;
  int64_t ld_;
  uint32_t voff[PER];

  // LDS position of logical chunk c in LDS row q (an involution: also the inverse)
  static __device__ __forceinline__ int swz(int q, int c) {
    if constexpr (TRANS) return c ^ ((q & 3) << 2);
    else if constexpr (CPR == 8) return c ^ (((q >> 1) ^ ((q & 1) << 2)) & 7);
    else return c ^ (((q >> 2) ^ (q & 2)) & 3);
  }
  __device__ __forceinline__ void init(const bf16* X, int64_t ld, int row0, int nrows, int wave, int lane) {
    ld_ = ld;
    base = TRANS ? X : X + (int64_t)row0 * ld;  // row0 < nrows: every tile starts inside the operand
#pragma unroll
    for (int c = 0; c < PER; c++) {
      const int slot = (c * NW + wave) * 64 + lane;  // LDS chunk this lane fills
      const int q = slot / CPR, lc = swz(q, slot % CPR);
      if constexpr (TRANS == 0) {
        // rows past the edge re-read the last row: they only feed outputs the epilogue drops
        const int r = min(row0 + q, nrows - 1);
        voff[c] = (uint32_t)(((int64_t)(r - row0) * ld + lc * 8) * 2);
      } else {
        const int col = min(row0 + lc * 8, nrows - 8);
        voff[c] = (uint32_t)(((int64_t)q * ld + col) * 2);
      }
    }
  }
  // start the loads of the tile at reduction offset k0 into LDS at tile
  __device__ __forceinline__ void issue(char* tile, int k0, int wave) const {
    __amdgpu_buffer_rsrc_t rsrc;
    int soff = 0;
    if constexpr (TRANS == 0) {
      rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), 0, -1, 0x00020000);
      soff = k0 * 2;
    } else {
      rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base + (int64_t)k0 * ld_), 0, -1, 0x00020000);
    }
    // (device pass only: with the builtin in the host pass, clang omits the
    // launch stubs of all but the first kernel instantiation using it)
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int c = 0; c < PER; c++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(tile + (c * NW + wave) * 1024),
                                               16, voff[c], soff, 0, 0);
#endif
  }
  // same fragment as Operand::frag (lane l: row rb + l%32, reduction values
  // 16*ks + 8*(l/32) + 0..7)
  static __device__ __forceinline__ bf16x8 frag(const char* tile, int rb, int ks, int lane) {
    if constexpr (TRANS == 0) {
      const int q = rb + (lane & 31);
      return *reinterpret_cast<const bf16x8*>(tile + q * ROWB + swz(q, 2 * ks + (lane >> 5)) * 16);
    } else {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const int j = lane & 15;
      const int kr = ks * 16 + 8 * (lane >> 5) + (j >> 2);
      const int col = rb + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      // rows kr and kr + 4 share the permutation
      const char* p = tile + kr * ROWB + swz(kr, col >> 3) * 16 + (col & 7) * 2;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * ROWB));
      const bf16x4 a = __builtin_bit_cast(bf16x4, lo), b = __builtin_bit_cast(bf16x4, hi);
      return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
};

// Wait until at most N of this wave's vector-memory loads are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  asm volatile("" ::: "memory");
}
// Wait until the tiles issued after the one needed are the only ones in
// flight: n tiles (of P loads each) were issued after it, at most MAX of them
// may stay outstanding.  n is the same for the whole wave (scalar branches).
template <int P, int MAX>
__device__ __forceinline__ void wait_tiles_after(int n) {
  if constexpr (MAX <= 0) {
    wait_vm<0>();
  } else {
    if (n >= MAX) wait_vm<MAX * P>();
    else wait_tiles_after<P, MAX - 1>(n);
  }
}
// Workgroup barrier without the memory fence of __syncthreads (whose release
// would wait for every load in flight, the next tiles' included); LDS
// ordering is by the explicit waits around it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Instruction order of one substep (its MFMAs and the next fragments' LDS
// reads): the reads go out two at a time between the first MFMAs, so their
// latency hides behind the remaining MFMAs instead of stalling the next
// substep (left alone, the scheduler sinks them to just before their use).
template <int NM, int NR>
__device__ __forceinline__ void dtl_schedule() {
#pragma unroll
  for (int r = 0; r < NR; r += 2) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - (NR + 1) / 2, 0);  // the remaining MFMAs
}

// Register-path substep order (with the next substep's fragment reads issued
// in this one): each of the first MFMAs is followed by two of those LDS
// reads, then by one of the next tile's LDS stores, the rest of the MFMAs
// last, so the reads' latency hides behind the matrix core.
template <int NM, int NR, int NW>
__device__ __forceinline__ void reg_schedule() {
  constexpr int GR = (NR + 1) / 2, GW = NW, REST = NM - GR - GW > 0 ? NM - GR - GW : 0;
#pragma unroll
  for (int r = 0; r < GR; r++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
  }
#pragma unroll
  for (int w = 0; w < GW; w++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // one LDS write
  }
  __builtin_amdgcn_sched_group_barrier(0x008, REST, 0);
}

// Which instantiations can produce the bias gradient: weight-gradient products
// (strided A, fp32 output) on 4-wave tiles.  The 8-wave tile serves only the
// bias-free tied output layer; a second copy of its main loop would not fit
// its 256 registers.
constexpr bool gemm_has_colsum(int at, int epi, int waves) { return at == 1 && epi == EPI_F32 && (waves == 4 || waves == 8); }

// Epilogue of one output tile: acc holds this wave's (BM/WI) x (BN/WJ) block of
// accumulators; smem is the block's LDS (free of operand tiles: the first
// barrier below waits for every wave's last fragment reads).  UNROLL unrolls
// the loops over passes and chunks (straight-line code lets the compiler count
// the memory operations still in flight exactly, so a persistent block can
// leave the stores outstanding while it moves on to the next tile).
template <typename T, int BM, int BN, int WI, int WJ, int EPI, bool FP8, bool UNROLL>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, const f32x16 (&acc)[BM / WI / 32][BN / WJ / 32],
                                              char* smem, int i0, int j0, int split, int tid, int lane, int wi,
                                              int wj) {
  constexpr int NT = WI * WJ * 64;
  constexpr int WTJ = BN / WJ;
  constexpr int TI = BM / WI / 32, TJ = WTJ / 32;
  constexpr int RP = BM / WI;  // output rows staged per pass (one row of waves)
  constexpr int SLD = BN + 4;  // staging row length (floats)
  typedef typename Frag<T>::type F;
  const int lr = lane & 31, lg = lane >> 5;
  // Epilogue, staged through LDS one row of waves at a time so every global
  // access is a coalesced 16-byte run along an output row.  Accumulator r of
  // lane l holds out[i][j] with i = tile row base + l%32 and
  // j = tile col base + 8*(r/4) + 4*(l/32) + r%4.
  float* stage = reinterpret_cast<float*>(smem);
  constexpr int CPRW = BN / 8;  // 8-column chunks per staged row
  // Each thread takes NCH 8-column chunks of the staged rows per pass.  Their
  // columns are the same in every pass, so the bias is loaded once, before
  // the passes; the inputs that depend on the row (residual, gelu', the
  // accumulated partial) are loaded a batch at a time, every load of a batch
  // issued before its first store, so a batch pays one memory latency rather
  // than one per chunk (the stores might alias the inputs, so the compiler
  // would not hoist the loads above them by itself).
  constexpr int NCH = (RP * CPRW + NT - 1) / NT;
  constexpr bool HAS_BIAS = EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_RESID;
  constexpr int NBV0 = NT % CPRW == 0 ? 1 : NCH;  // distinct bias chunks per thread
  constexpr bool HOIST = HAS_BIAS && NBV0 <= 4;    // (else the bias is loaded with each chunk)
  constexpr int NBV = HOIST ? NBV0 : 1;
  // (batches measured: one chunk at a time is as fast or faster for gelu',
  // the plain store and the fp32 partials, whose 8-wave kernels spill)
  // (and a thread with several bias chunks takes all its chunks at once, so
  // the bias array is indexed with constants)
  constexpr int BATCH = NBV > 1 ? NCH : EPI == EPI_RESID ? (NCH < 3 ? NCH : 3) : EPI == EPI_GELU_BWD ? NCH : 1;
  static_assert(NBV == 1 || BATCH == NCH, "bias chunk index must be a constant");
  const bool use_bias = HAS_BIAS && (EPI != EPI_STORE || g.bias != nullptr);
  // FP8 operands: the column scales of a thread's chunks (fixed columns, as the bias)
  f32x8 sbv[FP8 ? NBV : 1];
  if constexpr (FP8) {
#pragma unroll
    for (int k = 0; k < NBV; k++) {
      const int j = j0 + ((tid + k * NT) % CPRW) * 8;
      sbv[k] = j < g.N ? ld8(g.scale_b + j) : f32x8{};
    }
  }
  f32x8 bv[NBV];
#pragma unroll
  for (int k = 0; k < NBV; k++) bv[k] = f32x8{};
  if (HOIST && use_bias) {
    // (a uniform branch, with its own wait: a product without a bias waits
    // for nothing here, and the chunks below wait for no load, so the
    // stores of one chunk never wait on those of the chunk before it)
#pragma unroll
    for (int k = 0; k < NBV; k++) {
      const int j = j0 + ((tid + k * NT) % CPRW) * 8;
      if (j < g.N) bv[k] = ld8(g.bias + j);
    }
    wait_vm<0>();
  }
  constexpr int PASS_UNROLL = UNROLL ? WI : 1;
#pragma unroll PASS_UNROLL
  for (int pass = 0; pass < WI; pass++) {
    // the row-dependent inputs (residual, gelu', accumulated partial) of a
    // batch of chunks: the first batch's loads are issued before the staging
    // barrier, so their latency overlaps the accumulators' trip through LDS
    auto load_batch = [&](const int b0, f32x8 (&x)[BATCH], F (&u)[BATCH]) {
#pragma unroll
      for (int k = 0; k < BATCH; k++) {
        const int c = tid + (b0 + k) * NT;
        const int il = c / CPRW, jl = (c % CPRW) * 8;
        const int i = i0 + pass * RP + il, j = j0 + jl;
        if (b0 + k < NCH && c < RP * CPRW && i < g.M && j < g.N) {
          if constexpr (EPI == EPI_RESID) x[k] = ld8(g.resid + (int64_t)i * g.ldr + j);
          if constexpr (EPI == EPI_GELU_BWD) u[k] = ld8(static_cast<const T*>(g.aux) + (int64_t)i * g.ldaux + j);
          if constexpr (EPI == EPI_F32) {
            if (g.accumulate)
              x[k] = ld8(static_cast<const float*>(g.C) + (int64_t)split * g.split_stride + (int64_t)i * g.ldc + j);
          }
        }
      }
    };
    f32x8 x0[BATCH];
    F u0[BATCH];
    load_batch(0, x0, u0);
    __syncthreads();  // operand tiles (or the previous pass) are no longer read
    if (wi == pass) {
#pragma unroll
      for (int ti = 0; ti < TI; ti++)
#pragma unroll
        for (int tj = 0; tj < TJ; tj++)
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int il = ti * 32 + lr, jl = wj * WTJ + tj * 32 + 8 * q + 4 * lg;
            *reinterpret_cast<f32x4*>(stage + il * SLD + jl) =
                f32x4{acc[ti][tj][4 * q], acc[ti][tj][4 * q + 1], acc[ti][tj][4 * q + 2], acc[ti][tj][4 * q + 3]};
          }
    }
    __syncthreads();
    auto chunk_batch = [&](const int b0) {
      f32x8 x[BATCH];
      F u[BATCH];
      if (b0 == 0) {
#pragma unroll
        for (int k = 0; k < BATCH; k++) {
          x[k] = x0[k];
          u[k] = u0[k];
        }
      } else {
        load_batch(b0, x, u);
      }
#pragma unroll
      for (int k = 0; k < BATCH; k++) {
        const int c = tid + (b0 + k) * NT;
        const int il = c / CPRW, jl = (c % CPRW) * 8;
        const int i = i0 + pass * RP + il, j = j0 + jl;
        if (!(b0 + k < NCH && c < RP * CPRW && i < g.M && j < g.N)) continue;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(stage + il * SLD + jl);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(stage + il * SLD + jl + 4);
        f32x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const f32x8 bias = HOIST ? bv[NBV == 1 ? 0 : (b0 + k) % NBV] : (use_bias ? ld8(g.bias + j) : f32x8{});
        if constexpr (FP8) {
          static_assert(!FP8 || HOIST, "FP8 tiles keep their column scales in registers");
          v *= sbv[NBV == 1 ? 0 : (b0 + k) % NBV] * g.scale_a[i];
        }
        if constexpr (EPI == EPI_STORE || EPI == EPI_F32) v *= g.alpha;
        if constexpr (EPI == EPI_STORE) {
          if (use_bias) v += bias;
          F o;
#pragma unroll
          for (int e = 0; e < 8; e++) o[e] = from_f<T>(v[e]);
          st8(static_cast<T*>(g.C) + (int64_t)i * g.ldc + j, o);
        } else if constexpr (EPI == EPI_GELU) {
          // the backward needs only gelu' at the pre-activation: store that
          // (from the fp32 value) next to the activation
          v += bias;
          F gu, o;
          if (g.preact) {
            // keep the rounded pre-activation; the activation comes from that
            // same rounded value, so recomputing it later reproduces it exactly
#pragma unroll
            for (int e = 0; e < 8; e++) {
              gu[e] = from_f<T>(v[e]);
              o[e] = from_f<T>(gelu_tanh(to_f<T>(gu[e])));
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; e++) {
              const float sg = gelu_sigmoid(v[e]);
              gu[e] = from_f<T>(gelu_tanh_grad_s(v[e], sg));
              o[e] = from_f<T>(v[e] * sg);
            }
          }
          if (g.aux) st8(static_cast<T*>(g.aux) + (int64_t)i * g.ldaux + j, gu);  // (none when evaluating)
          st8(static_cast<T*>(g.C) + (int64_t)i * g.ldc + j, o);
        } else if constexpr (EPI == EPI_RESID) {
          v += bias;
          v += x[k];
          st8(static_cast<float*>(g.C) + (int64_t)i * g.ldc + j, v);
        } else if constexpr (EPI == EPI_GELU_BWD) {
          F o;
          if (g.preact) {
#pragma unroll
            for (int e = 0; e < 8; e++) {
              const float x = to_f<T>(u[k][e]);
              o[e] = from_f<T>(v[e] * gelu_tanh_grad_s(x, gelu_sigmoid(x)));
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; e++) o[e] = from_f<T>(v[e] * to_f<T>(u[k][e]));
          }
          st8(static_cast<T*>(g.C) + (int64_t)i * g.ldc + j, o);
        } else {  // EPI_F32
          float* Cp = static_cast<float*>(g.C) + (int64_t)split * g.split_stride + (int64_t)i * g.ldc + j;
          if (g.accumulate) v += x[k];
          st8(Cp, v);
        }
      }
    };
    if constexpr (BATCH == 1 && !UNROLL) {
#pragma unroll 1
      for (int b0 = 0; b0 < NCH; b0++) chunk_batch(b0);
    } else {
#pragma unroll
      for (int b0 = 0; b0 < NCH; b0 += BATCH) chunk_batch(b0);
    }
  }
}

// NBUF = 0: operands staged through registers (two register stages, two LDS
// buffers).  NBUF >= 2 (bf16): direct-to-LDS loads into a ring of NBUF LDS
// buffers, the tile NBUF steps ahead loading while the current one is used.
// TIn: operand type (T, or FP8 E4M3 with T = bf16 outputs: reduction-
// contiguous operands, register staging, acc(i, j) scaled by scale_a[i] *
// scale_b[j] before the epilogue).
template <typename T, int BM, int BN, int BK, int WI, int WJ, int AT, int BT, int EPI, int NBUF, typename TIn,
          int GM = 4>
__device__ __forceinline__ void gemm_body(const GemmArgs& g, int tile, int split) {
  constexpr int NT = WI * WJ * 64;
  constexpr int WTI = BM / WI, WTJ = BN / WJ;
  constexpr int TI = WTI / 32, TJ = WTJ / 32;
  constexpr bool FP8 = sizeof(TIn) == 1;
  constexpr int KS = KStep<TIn>::k;  // reduction depth of one MFMA step
  constexpr int NSUB = BK / KS;      // MFMA steps per LDS tile
  static_assert(!FP8 || (AT == 0 && BT == 0 && NBUF == 0), "FP8: reduction-contiguous operands, register staging");
  typedef Operand<TIn, BM, BK, NT, AT> OA;
  typedef Operand<TIn, BN, BK, NT, BT> OB;
  typedef typename Frag<TIn>::type FI;  // operand fragments
  typedef typename Frag<T>::type F;     // eight output values
  // Operand tiles (two buffers each) and, after the main loop, the epilogue's
  // staging area for half of the output tile (fp32) share one LDS block.
  constexpr int RP = BM / WI;                 // output rows staged per pass (one row of waves)
  constexpr int SLD = BN + 4;                 // staging row length (floats)
  typedef DtlOperand<BM, BK, WI * WJ, AT> DA;
  typedef DtlOperand<BN, BK, WI * WJ, BT> DB;
  constexpr int DSTAGE = (BM + BN) * BK * 2;  // one ring buffer (both operands)
  constexpr int OPER_BYTES = NBUF ? NBUF * DSTAGE : 2 * (OA::ELEMS + OB::ELEMS) * (int)sizeof(TIn);
  constexpr int STAGE_BYTES = RP * SLD * 4;
  __shared__ __attribute__((aligned(16))) char smem[OPER_BYTES > STAGE_BYTES ? OPER_BYTES : STAGE_BYTES];
  TIn (*sA)[OA::ELEMS] = reinterpret_cast<TIn (*)[OA::ELEMS]>(smem);
  TIn (*sB)[OB::ELEMS] = reinterpret_cast<TIn (*)[OB::ELEMS]>(smem + 2 * OA::ELEMS * sizeof(TIn));

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wi = wave / WJ, wj = wave % WJ;
  const int nbi = (g.M + BM - 1) / BM, nbj = (g.N + BN - 1) / BN;
  // Grouped tile order: GM consecutive row-tiles sweep the columns together.
  const int group = tile / (GM * nbj);
  const int first_i = group * GM;
  const int gsize = min(nbi - first_i, GM);
  const int tig = tile - group * GM * nbj;
  const int bi = first_i + tig % gsize, bj = tig / gsize;
  const int i0 = bi * BM, j0 = bj * BN;

  // split s of S takes reduction steps [s*nkt/S, (s+1)*nkt/S): the splits
  // differ by at most one step, so any S fills the chip evenly
  const int nkt = g.K / BK;
  const int ks0 = (int)((int64_t)split * nkt / g.splits);
  const int kbeg = ks0 * BK;
  const int nk = (int)((int64_t)(split + 1) * nkt / g.splits) - ks0;
  const TIn* A = static_cast<const TIn*>(g.A);
  const TIn* Bm = static_cast<const TIn*>(g.B);

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int ti = 0; ti < TI; ti++)
#pragma unroll
    for (int tj = 0; tj < TJ; tj++) acc[ti][tj] = f32x16{};

  // One LDS tile: BK/16 substeps of TI x TJ MFMAs.  With PIPE the fragments
  // of substep ks+1 are read before the MFMAs of substep ks are issued, so LDS
  // latency overlaps the matrix core (a gain when both operands come from
  // plain LDS rows; with two transposed operands the extra registers cost
  // more than the overlap wins).  GEMM_MAINLOOP(1) also accumulates the bias
  // gradient sum_r A(i, r) from the staged A chunks (Operand::row_sums).
  constexpr bool PIPE = AT == 0 && !FP8;  // (FP8 fragments are twice as wide: no room for a second set)
  // With BK = 64 (four substeps per tile) the next tile's LDS stores are
  // spread over the substeps, overlapping them with the MFMAs (they fill the
  // other buffer, which the barrier after the tile protects); with two
  // substeps the spread costs more than it hides.
  constexpr bool ILV = NSUB >= 4;
  constexpr bool SCH_ON = true;
  constexpr int SCH_READS = TI * (AT ? 2 : 1) + TJ * (BT ? 2 : 1);
  constexpr int SCH_WRITES = ILV ? (OA::PER + NSUB - 1) / NSUB + (OB::PER + NSUB - 1) / NSUB : 0;
  constexpr bool HAS_CS = gemm_has_colsum(AT, EPI, WI * WJ);
#define GEMM_FRAGS(AS, BS, KS, FA, FB)                                                            \
  _Pragma("unroll") for (int ti = 0; ti < TI; ti++) FA[ti] = OA::frag(AS, wi * WTI + ti * 32, KS, lane); \
  _Pragma("unroll") for (int tj = 0; tj < TJ; tj++) FB[tj] = OB::frag(BS, wj * WTJ + tj * 32, KS, lane);
#define GEMM_COMPUTE(AS, BS, PP) GEMM_COMPUTE_ST(AS, BS, PP, (void)0)
  // ST(ks): work interleaved with substep ks (the next tile's LDS stores)
#define GEMM_COMPUTE_ST(AS, BS, PP, ST)                                                           \
  {                                                                                               \
    FI fa[2][TI], fb[2][TJ];                                                                      \
    if constexpr (PP) { GEMM_FRAGS(AS, BS, 0, fa[0], fb[0]) }                                     \
    _Pragma("unroll") for (int ks = 0; ks < NSUB; ks++) {                                      \
      ST;                                                                                         \
      const int cur = PP ? ks & 1 : 0;                                                            \
      if constexpr (PP) {                                                                         \
        if (ks + 1 < NSUB) { GEMM_FRAGS(AS, BS, ks + 1, fa[cur ^ 1], fb[cur ^ 1]) }            \
      } else {                                                                                    \
        GEMM_FRAGS(AS, BS, ks, fa[0], fb[0])                                                      \
      }                                                                                           \
      _Pragma("unroll") for (int ti = 0; ti < TI; ti++)                                           \
        _Pragma("unroll") for (int tj = 0; tj < TJ; tj++) mma16(acc[ti][tj], fb[cur][tj], fa[cur][ti]); \
      if constexpr (PP && SCH_ON && sizeof(T) == 2) reg_schedule<TI * TJ, SCH_READS, SCH_WRITES>();          \
    }                                                                                             \
  }

  // Two register stages: the tile two steps ahead is loaded while the current
  // one is consumed from LDS and the next one is stored to the other buffer.
  // Loads and stores are unconditional (tile indices past the end re-read the
  // last tile, which is then never consumed): with no branch around them the
  // compiler can leave the newest loads in flight at every LDS store instead
  // of draining the whole load queue.
#define GEMM_MAINLOOP(CSV)                                                                        \
  {                                                                                               \
    OA a0, a1;                                                                                    \
    OB b0, b1;                                                                                    \
    a0.init(A, g.lda, i0, g.M, tid);                                                              \
    b0.init(Bm, g.ldb, j0, g.N, tid);                                                             \
    a1.init(A, g.lda, i0, g.M, tid);                                                              \
    b1.init(Bm, g.ldb, j0, g.N, tid);                                                             \
    const int klast = kbeg + (nk - 1) * BK;                                                       \
    a0.load(kbeg);                                                                                \
    b0.load(kbeg);                                                                                \
    a1.load(min(kbeg + BK, klast));                                                               \
    b1.load(min(kbeg + BK, klast));                                                               \
    a0.store(sA[0], tid);                                                                         \
    b0.store(sB[0], tid);                                                                         \
    if constexpr (CSV) a0.row_sums(rs, 1.f);                                                      \
    __syncthreads();                                                                              \
    for (int kt = 0; kt + 2 <= nk; kt += 2) {                                                     \
      /* buffer 0 holds tile kt, registers 1 hold tile kt+1 */                                    \
      const int k2 = min(kbeg + (kt + 2) * BK, klast), k3 = min(kbeg + (kt + 3) * BK, klast);     \
      a0.load(k2);                                                                                \
      b0.load(k2);                                                                                \
      if constexpr (ILV) {                                                                        \
        GEMM_COMPUTE_ST(sA[0], sB[0], PIPE,                                                  \
                        (a1.template store_part<NSUB>(sA[1], tid, ks),                         \
                         b1.template store_part<NSUB>(sB[1], tid, ks)))                        \
      } else {                                                                                    \
        GEMM_COMPUTE(sA[0], sB[0], PIPE)                                                     \
        a1.store(sA[1], tid);                                                                     \
        b1.store(sB[1], tid);                                                                     \
      }                                                                                           \
      if constexpr (CSV) a1.row_sums(rs, 1.f); /* tile kt+1 (kt + 2 <= nk) */                    \
      __syncthreads();                                                                            \
      /* buffer 1 holds tile kt+1, registers 0 hold tile kt+2 */                                  \
      a1.load(k3);                                                                                \
      b1.load(k3);                                                                                \
      if constexpr (ILV) {                                                                        \
        GEMM_COMPUTE_ST(sA[1], sB[1], PIPE,                                                  \
                        (a0.template store_part<NSUB>(sA[0], tid, ks),                         \
                         b0.template store_part<NSUB>(sB[0], tid, ks)))                        \
      } else {                                                                                    \
        GEMM_COMPUTE(sA[1], sB[1], PIPE)                                                     \
        a0.store(sA[0], tid);                                                                     \
        b0.store(sB[0], tid);                                                                     \
      }                                                                                           \
      if constexpr (CSV) a0.row_sums(rs, kt + 2 < nk ? 1.f : 0.f); /* tile kt+2, if any */       \
      __syncthreads();                                                                            \
    }                                                                                             \
    if (nk & 1) { /* the last tile sits in buffer 0 (no read-ahead: registers are tight here) */  \
      GEMM_COMPUTE(sA[0], sB[0], false)                                                      \
    }                                                                                             \
  }

  // Direct-to-LDS main loop.  At the last substep of tile kt the wave waits
  // for its own loads of tile kt+1 and for its reads of tile kt, then one
  // barrier makes tile kt+1 visible and frees tile kt's buffer, which takes
  // tile kt+NBUF; the first fragments of tile kt+1 are read while the last
  // MFMAs of tile kt run.  Tiles past the last are never loaded (the waits
  // count only the loads actually issued).
#define GEMM_DFRAGS(TILE, KS, FA, FB)                                                                     \
  _Pragma("unroll") for (int ti = 0; ti < TI; ti++) FA[ti] = DA::frag(TILE, wi * WTI + ti * 32, KS, lane); \
  _Pragma("unroll") for (int tj = 0; tj < TJ; tj++) FB[tj] = DB::frag(TILE + DA::BYTES, wj * WTJ + tj * 32, KS, lane);
// One tile from LDS buffer CUR; unless LAST, its last substep also moves to
// tile kt+1 (kept out of a runtime branch so the substep's MFMAs never wait
// for the next tile's fragment reads)
#define GEMM_DTL_TILE(CSV, LAST)                                                                          \
  {                                                                                                       \
    const char* cur = smem + (kt % NBUF) * DSTAGE;                                                        \
    _Pragma("unroll") for (int ks = 0; ks < BK / 16; ks++) {                                              \
      const int c = ks & 1;                                                                               \
      if (ks + 1 < BK / 16) {                                                                             \
        GEMM_DFRAGS(cur, ks + 1, fa[c ^ 1], fb[c ^ 1])                                                    \
      } else if constexpr (!LAST) {                                                                       \
        wait_tiles_after<P, NBUF - 2>(nk - 2 - kt);                                                       \
        lds_barrier();                                                                                    \
        if (kt + NBUF < nk) {                                                                             \
          da.issue(smem + (kt % NBUF) * DSTAGE, kbeg + (kt + NBUF) * BK, wave);                           \
          db.issue(smem + (kt % NBUF) * DSTAGE + DA::BYTES, kbeg + (kt + NBUF) * BK, wave);               \
        }                                                                                                 \
        const char* nxt = smem + ((kt + 1) % NBUF) * DSTAGE;                                              \
        GEMM_DFRAGS(nxt, 0, fa[c ^ 1], fb[c ^ 1])                                                         \
      }                                                                                                   \
      if constexpr (CSV) {                                                                                \
        _Pragma("unroll") for (int ti = 0; ti < TI; ti++)                                                 \
          if (ti % WJ == wj) cs[ti] = frag_sum(fa[c][ti], cs[ti]);                                        \
      }                                                                                                   \
      _Pragma("unroll") for (int ti = 0; ti < TI; ti++)                                                   \
        _Pragma("unroll") for (int tj = 0; tj < TJ; tj++) mma16(acc[ti][tj], fb[c][tj], fa[c][ti]);       \
      if (ks + 1 < BK / 16 || !LAST) dtl_schedule<TI * TJ, NREAD>();                                      \
    }                                                                                                     \
  }
#define GEMM_DTL_LOOP(CSV)                                                                                \
  {                                                                                                       \
    constexpr int P = DA::PER + DB::PER;                                                                  \
    constexpr int NREAD = TI * (AT ? 2 : 1) + TJ * (BT ? 2 : 1);                                          \
    DA da;                                                                                                \
    DB db;                                                                                                \
    da.init(static_cast<const bf16*>(g.A), g.lda, i0, g.M, wave, lane);                                   \
    db.init(static_cast<const bf16*>(g.B), g.ldb, j0, g.N, wave, lane);                                   \
    _Pragma("unroll") for (int s = 0; s < NBUF; s++) {                                                    \
      if (s < nk) {                                                                                       \
        da.issue(smem + s * DSTAGE, kbeg + s * BK, wave);                                                 \
        db.issue(smem + s * DSTAGE + DA::BYTES, kbeg + s * BK, wave);                                     \
      }                                                                                                   \
    }                                                                                                     \
    wait_tiles_after<P, NBUF - 1>(nk - 1);                                                                \
    lds_barrier();                                                                                        \
    bf16x8 fa[2][TI], fb[2][TJ];                                                                          \
    GEMM_DFRAGS(smem, 0, fa[0], fb[0])                                                                    \
    int kt = 0;                                                                                           \
    _Pragma("unroll 1") for (; kt < nk - 1; kt++) GEMM_DTL_TILE(CSV, false)                               \
    GEMM_DTL_TILE(CSV, true)                                                                              \
  }

  // Only the blocks of the first column tile (bj == 0) sum the bias gradient.
  // The choice is made once per block, outside the main loop, so the loop
  // itself stays one branch-free block and every wave passes the same
  // barriers.  On the register path each thread sums the A chunks it stages
  // (no dependence on the LDS fragment reads, which the MFMAs wait for; sums
  // of the fragments held the MFMAs back and made the summing blocks a fifth
  // slower than the others, which set the time of a weight-gradient launch);
  // the direct-to-LDS path sums fragments, each wave column a share of the
  // rows.
  const bool do_cs = HAS_CS && g.colsum != nullptr && bj == 0;
  float cs[TI];  // direct-to-LDS path: sums of the A fragments
#pragma unroll
  for (int ti = 0; ti < TI; ti++) cs[ti] = 0.f;
  float rs[OA::VE];  // register path: sums of the staged A chunks
#pragma unroll
  for (int e = 0; e < OA::VE; e++) rs[e] = 0.f;
  if constexpr (NBUF > 0) {
    static_assert(sizeof(T) == 2 && BK % 32 == 0, "direct-to-LDS loads: bf16, even substep count");
    if constexpr (HAS_CS) {
      if (do_cs) GEMM_DTL_LOOP(1) else GEMM_DTL_LOOP(0)
    } else {
      GEMM_DTL_LOOP(0)
    }
  } else if constexpr (HAS_CS) {
    if (do_cs) GEMM_MAINLOOP(1) else GEMM_MAINLOOP(0)
  } else {
    GEMM_MAINLOOP(0)
  }

#undef GEMM_DTL_LOOP
#undef GEMM_DTL_TILE
#undef GEMM_DFRAGS
#undef GEMM_MAINLOOP
  if constexpr (NBUF > 0) {
    if (do_cs) {
#pragma unroll
      for (int ti = 0; ti < TI; ti++) {
        if (ti % WJ != wj) continue;
        const float t = cs[ti] + __shfl_xor(cs[ti], 32, 64);  // the two halves of each row's reduction values
        const int i = i0 + wi * WTI + ti * 32 + (lane & 31);
        if (lane < 32 && i < g.M) g.colsum[(int64_t)split * g.colsum_stride + i] = t;
      }
    }
  } else if constexpr (HAS_CS) {
    if (do_cs) {
      // thread (m, c) summed rows c*VE .. c*VE+VE-1 over the reduction rows m,
      // m + NT/CPR, ... of every step; the groups m are added in order
      constexpr int CPRA = OA::CPR, GROUPS = NT / CPRA;
      static_assert(GROUPS * BM * 4 <= (int)sizeof(smem), "row-sum staging fits the LDS block");
      float* red = reinterpret_cast<float*>(smem);
      __syncthreads();  // every wave has read its last fragments
#pragma unroll
      for (int e = 0; e < OA::VE; e++) red[(tid / CPRA) * BM + (tid % CPRA) * OA::VE + e] = rs[e];
      __syncthreads();
      for (int r = tid; r < BM; r += NT) {
        float t = 0.f;
#pragma unroll
        for (int m = 0; m < GROUPS; m++) t += red[m * BM + r];
        if (i0 + r < g.M) g.colsum[(int64_t)split * g.colsum_stride + i0 + r] = t;
      }
    }
  }
  gemm_epilogue<T, BM, BN, WI, WJ, EPI, FP8, false>(g, acc, smem, i0, j0, split, tid, lane, wi, wj);
}

template <typename T, int BM, int BN, int BK, int WI, int WJ, int AT, int BT, int EPI, int NBUF, typename TIn>
__global__ void __launch_bounds__(WI * WJ * 64) gemm_kernel(GemmArgs g) {
  const int nt = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  // With a split reduction each XCD takes a contiguous range of (split, tile)
  // pairs in split-major order, so the token rows one split reads are fetched
  // by one or two XCDs' L2 instead of all eight.
  if (gridDim.y > 1) {
    const int logical = xcd_remap_any(blockIdx.x + blockIdx.y * nt, nt * gridDim.y);
    gemm_body<T, BM, BN, BK, WI, WJ, AT, BT, EPI, NBUF, TIn>(g, logical % nt, logical / nt);
  } else {
    gemm_body<T, BM, BN, BK, WI, WJ, AT, BT, EPI, NBUF, TIn>(g, xcd_remap(blockIdx.x, nt), 0);
  }
}

// Several independent products of one shape class in one launch (the weight
// gradients of a layer): problem p owns the logical blocks [block0[p],
// block0[p+1]), split-major inside it as in gemm_kernel; the blocks are
// renumbered so each XCD takes one contiguous range of logical blocks.  Tiles
// go in groups of three row tiles: a 768-wide product's split is then whole
// groups of 3 x 3 tiles, so where an XCD's range ends inside a split it cuts
// between row tiles and the two XCDs share only the column operand's panels
// (the caller orders the problems so those cuts are few).
template <typename T, int BM, int BN, int BK, int WI, int WJ, int AT, int BT, int EPI>
__global__ void __launch_bounds__(WI * WJ * 64) gemm_group_kernel(GemmGroup gg) {
  const int logical = xcd_remap_any(blockIdx.x, gg.block0[gg.count]);
  int p = 0;
#pragma unroll
  for (int q = 1; q < kMaxGemmGroup; q++)
    if (q < gg.count && logical >= gg.block0[q]) p = q;
  const GemmArgs& g = gg.p[p];
  const int nt = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  const int local = logical - gg.block0[p];
  gemm_body<T, BM, BN, BK, WI, WJ, AT, BT, EPI, 0, T, 3>(g, local % nt, local / nt);
}

// Persistent variant for forward and input-gradient products with several
// rounds of output tiles (A reduction-contiguous, operands staged through
// registers, an even number of reduction steps).  Each block walks a
// sequence of output tiles.  While it computes the last two reduction steps
// of a tile it loads the first two of its next tile, before the epilogue, so
// the next tile starts without waiting for memory, the epilogue's stores
// drain while it runs, and no block is launched per tile.  The tiles of one
// XCD form one contiguous range in the grouped order of gemm_kernel, walked
// by that XCD's blocks in turn.
template <typename T, int BM, int BN, int BK, int WI, int WJ, int BT, int EPI>
__global__ void __launch_bounds__(WI * WJ * 64) gemm_persist_kernel(GemmArgs g) {
  constexpr int AT = 0;
  constexpr int NT = WI * WJ * 64;
  constexpr int WTI = BM / WI, WTJ = BN / WJ;
  constexpr int TI = WTI / 32, TJ = WTJ / 32;
  constexpr int NSUB = BK / 16;
  typedef Operand<T, BM, BK, NT, AT> OA;
  typedef Operand<T, BN, BK, NT, BT> OB;
  typedef typename Frag<T>::type FI;
  constexpr int OPER_BYTES = 2 * (OA::ELEMS + OB::ELEMS) * (int)sizeof(T);
  constexpr int STAGE_BYTES = (BM / WI) * (BN + 4) * 4;
  __shared__ __attribute__((aligned(16))) char smem[OPER_BYTES > STAGE_BYTES ? OPER_BYTES : STAGE_BYTES];
  T (*sA)[OA::ELEMS] = reinterpret_cast<T (*)[OA::ELEMS]>(smem);
  T (*sB)[OB::ELEMS] = reinterpret_cast<T (*)[OB::ELEMS]>(smem + 2 * OA::ELEMS * sizeof(T));
  constexpr bool PIPE = true, ILV = NSUB >= 4;
  constexpr bool SCH_ON = false;  // (the ordering made this kernel spill)
  constexpr int SCH_READS = TI + TJ * (BT ? 2 : 1);
  constexpr int SCH_WRITES = ILV ? (OA::PER + NSUB - 1) / NSUB + (OB::PER + NSUB - 1) / NSUB : 0;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wi = wave / WJ, wj = wave % WJ;
  const int nbi = (g.M + BM - 1) / BM, nbj = (g.N + BN - 1) / BN, ntiles = nbi * nbj;
  const int nk = g.K / BK;  // even, >= 2 (checked by the launcher)
  // this XCD's range of logical tiles and this block's slot in it
  const int x = blockIdx.x % 8, slot = blockIdx.x / 8, per = gridDim.x / 8;
  const int q8 = ntiles / 8, r8 = ntiles % 8;
  const int start = x < r8 ? x * (q8 + 1) : r8 * (q8 + 1) + (x - r8) * q8;
  const int cnt = q8 + (x < r8 ? 1 : 0);
  int li = slot;
  if (li >= cnt) return;
  constexpr int GM = 4;
  auto coords = [&](int l, int& i0, int& j0) {
    const int tile = start + l;
    const int group = tile / (GM * nbj);
    const int first_i = group * GM;
    const int gsize = min(nbi - first_i, GM);
    const int tig = tile - group * GM * nbj;
    i0 = (first_i + tig % gsize) * BM;
    j0 = (tig / gsize) * BN;
  };
  const T* A = static_cast<const T*>(g.A);
  const T* Bm = static_cast<const T*>(g.B);
  int i0, j0;
  coords(li, i0, j0);
  OA a0, a1;
  OB b0, b1;
  a0.init(A, g.lda, i0, g.M, tid);
  b0.init(Bm, g.ldb, j0, g.N, tid);
  a1.init(A, g.lda, i0, g.M, tid);
  b1.init(Bm, g.ldb, j0, g.N, tid);
  a0.load(0);
  b0.load(0);
  a1.load(BK);
  b1.load(BK);
  a0.store(sA[0], tid);
  b0.store(sB[0], tid);
  __syncthreads();
  while (true) {
    f32x16 acc[TI][TJ];
#pragma unroll
    for (int ti = 0; ti < TI; ti++)
#pragma unroll
      for (int tj = 0; tj < TJ; tj++) acc[ti][tj] = f32x16{};
    const int lnext = li + per;
    const bool has_next = lnext < cnt;
    int i0n = i0, j0n = j0;  // (without a next tile: harmless re-reads of this one)
    if (has_next) coords(lnext, i0n, j0n);
    for (int kt = 0; kt + 4 <= nk; kt += 2) {
      /* buffer 0 holds step kt, registers 1 hold step kt+1 */
      a0.load((kt + 2) * BK);
      b0.load((kt + 2) * BK);
      if constexpr (ILV) {
        GEMM_COMPUTE_ST(sA[0], sB[0], PIPE,
                        (a1.template store_part<NSUB>(sA[1], tid, ks), b1.template store_part<NSUB>(sB[1], tid, ks)))
      } else {
        GEMM_COMPUTE(sA[0], sB[0], PIPE)
        a1.store(sA[1], tid);
        b1.store(sB[1], tid);
      }
      __syncthreads();
      a1.load((kt + 3) * BK);
      b1.load((kt + 3) * BK);
      if constexpr (ILV) {
        GEMM_COMPUTE_ST(sA[1], sB[1], PIPE,
                        (a0.template store_part<NSUB>(sA[0], tid, ks), b0.template store_part<NSUB>(sB[0], tid, ks)))
      } else {
        GEMM_COMPUTE(sA[1], sB[1], PIPE)
        a0.store(sA[0], tid);
        b0.store(sB[0], tid);
      }
      __syncthreads();
    }
    // the last two steps (nk-2 in buffer 0, nk-1 in registers 1); the
    // registers 0 and then 1 take the next tile's first two steps.  The
    // next tile's load offsets are derived from an opaque copy of the thread
    // index, so the compiler recomputes their per-thread parts here instead
    // of keeping them live through the whole loop (where they spilled).
    int tid_o = tid;
    asm volatile("" : "+v"(tid_o));
    a0.init(A, g.lda, i0n, g.M, tid_o);
    b0.init(Bm, g.ldb, j0n, g.N, tid_o);
    a0.load(0);
    b0.load(0);
    if constexpr (ILV) {
      GEMM_COMPUTE_ST(sA[0], sB[0], PIPE,
                      (a1.template store_part<NSUB>(sA[1], tid, ks), b1.template store_part<NSUB>(sB[1], tid, ks)))
    } else {
      GEMM_COMPUTE(sA[0], sB[0], PIPE)
      a1.store(sA[1], tid);
      b1.store(sB[1], tid);
    }
    __syncthreads();
    a1.init(A, g.lda, i0n, g.M, tid_o);
    b1.init(Bm, g.ldb, j0n, g.N, tid_o);
    a1.load(BK);
    b1.load(BK);
    GEMM_COMPUTE(sA[1], sB[1], PIPE)
    gemm_epilogue<T, BM, BN, WI, WJ, EPI, false, true>(g, acc, smem, i0, j0, 0, tid, lane, wi, wj);
    if (!has_next) break;
    __syncthreads();  // every wave has read its last staged chunk
    a0.store(sA[0], tid);
    b0.store(sB[0], tid);
    __syncthreads();
    li = lnext;
    i0 = i0n;
    j0 = j0n;
  }
}

#undef GEMM_COMPUTE
#undef GEMM_COMPUTE_ST
#undef GEMM_FRAGS

// Blocks of a persistent launch: one per CU with a one-block-per-CU tile
// (256 CUs), rounded down to a multiple of the 8 XCDs; never more than the
// tiles.
constexpr int kPersistBlocks = 256;

template <typename T, int BM, int BN, int WI, int WJ, int BT, int EPI, int BK>
hipError_t launch_persist(hipStream_t st, const GemmArgs& g) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.K <= 0 || g.K % (2 * BK) != 0 || g.M % 8 != 0 || g.N % 8 != 0 || g.lda % 8 != 0 || g.ldb % 8 != 0 ||
      g.splits != 1 || g.colsum != nullptr || EPI == EPI_F32)
    return hipErrorInvalidValue;
  const int ntiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  int blocks = std::min(kPersistBlocks, ntiles);
  blocks = std::max(8, blocks / 8 * 8);
  hipLaunchKernelGGL((gemm_persist_kernel<T, BM, BN, BK, WI, WJ, BT, EPI>), dim3(blocks), dim3(WI * WJ * 64), 0, st, g);
  return hipGetLastError();
}

template <typename T, int BM, int BN, int WI, int WJ, int AT, int BT, int EPI, int BK, int NBUF = 0, typename TIn = T>
hipError_t launch(hipStream_t st, const GemmArgs& g) {
  constexpr int VE = Vec16<TIn>::n;
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.K <= 0 || g.splits < 1 || g.K % BK != 0 || g.K / BK < g.splits || g.M % VE != 0 || g.N % 8 != 0 ||
      g.lda % VE != 0 ||
      g.ldb % VE != 0 || (EPI != EPI_F32 && g.splits != 1) ||
      (g.colsum != nullptr && !gemm_has_colsum(AT, EPI, WI * WJ)))
    return hipErrorInvalidValue;
  const int nbi = (g.M + BM - 1) / BM, nbj = (g.N + BN - 1) / BN;
  dim3 grid(nbi * nbj, g.splits);
  if (sizeof(TIn) == 1 && (g.scale_a == nullptr || g.scale_b == nullptr)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WI, WJ, AT, BT, EPI, NBUF, TIn>), grid, dim3(WI * WJ * 64), 0, st, g);
  return hipGetLastError();
}

// Tile shape and reduction step per operand layout and product shape (bf16),
// from sweeps of the step's matmuls on MI355X.
//  * 128x128, 4 waves of 64x64: two or three blocks per CU hide one block's
//    prologue and epilogue behind the others' main loops; best for small
//    products and short reductions (and the fp32 path).
//  * 8 waves, 256x256 (waves of 128x64, two per SIMD, twice the operand
//    reuse): forward and input-gradient products with large outputs or long
//    reductions (MLP up- and down-projection, tied head, input gradients of
//    fc, qkv and the tied head); with BK = 32 every weight gradient (both
//    operands reduction-strided), split over the reduction into as many
//    uneven parts as make one round of one block per CU.
//  * 8 waves, 256x192 (waves of 64x96), BK = 64: forward and input-gradient
//    products whose output width is a multiple of 192 up to 2304 (the
//    model-width outputs: 16384 x 768 makes 64 x 4 = 256 tiles, one per CU,
//    where 256x256 leaves a quarter of the CUs idle; and the qkv projection).
//  * The 8-wave 256x256 tile with direct-to-LDS operand loads (two LDS
//    buffers, BK = 64): other forward products up to 4096 wide (both operands
//    reduction-contiguous), where it saves the staging registers.  Its single
//    tile of look-ahead is too short for the tied head's long sweep.
//  * TILE_P256_W8 / TILE_P192_W8: the persistent versions of the two 8-wave
//    tiles (gemm_persist_kernel) for forward products with more than one
//    round of tiles (more tiles than CUs) and an even number of reduction
//    steps: at 124M the qkv and tied-head forward products (66 vs 70 us and
//    1347 vs 1487 us, interleaved runs on one box).  Input-gradient products
//    stay per-tile: they run beside the second stream's weight gradients,
//    and a persistent block that lands on a busy CU holds up its whole tile
//    sequence (MLP input gradient persistent: 92 us alone but 220 us in the
//    step; the step 18.53 -> 18.32 ms without it).  The 256x192 tile also
//    serves the MLP input gradient, whose GELU' epilogue spills registers on
//    the 256x256 one.
enum TileKind {
  TILE_128 = 0, TILE_128_K32, TILE_256x192_K32, TILE_256_W8, TILE_256_W8_K32, TILE_D256_W8, TILE_192_W8,
  TILE_P256_W8, TILE_P192_W8
};

TileKind choose_tile(Prec p, int a_t, int b_t, int M, int N, int K) {
  if (p != BF16 || M < 256) return TILE_128;
  const int64_t mn = (int64_t)M * N;
  if (a_t && b_t) return TILE_256_W8_K32;
  auto rounds = [&](int bn) { return (int64_t)((M + 255) / 256) * ((N + bn - 1) / bn) > kPersistBlocks; };
  const bool even = K % 128 == 0;  // an even number of 64-deep reduction steps
  // an input gradient with a very long reduction (the tied head's, over the
  // vocabulary): the 256x256 tile's main loop is faster per CU than the
  // 256x192 one's, and the CUs a 768-wide output leaves idle go to the head's
  // weight gradient, which runs beside it
  if (b_t && K >= 16384 && N % 256 == 0 && mn >= 4000000) return TILE_256_W8;
  // 192-wide outputs: the model-width products and the qkv projection (and
  // any product with a strided second operand whose width is a multiple of
  // 192: on the 256-wide register-path tile the GELU' epilogue spills)
  if (N % 192 == 0 && (N <= 2304 || b_t) && mn >= 4000000)
    return !a_t && !b_t && even && rounds(192) ? TILE_P192_W8 : TILE_192_W8;
  if (K >= 2048 || mn >= 40000000) {
    if (!a_t && !b_t && N <= 4096) return TILE_D256_W8;
    return !a_t && !b_t && even && rounds(256) ? TILE_P256_W8 : TILE_256_W8;
  }
  return TILE_128;
}

int tile_bk(Prec p, TileKind k) {
  if (p != BF16) return 32;
  return (k == TILE_128 || k == TILE_256_W8 || k == TILE_D256_W8 || k == TILE_192_W8 || k == TILE_P256_W8 ||
          k == TILE_P192_W8) ? 64 : 32;
}

template <typename T, int AT, int BT, int EPI>
hipError_t launch_tiled(hipStream_t st, const GemmArgs& g, TileKind k) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (AT == 0 && BT == 0) {
      if (k == TILE_D256_W8) return launch<T, 256, 256, 2, 4, AT, BT, EPI, 64, 2>(st, g);
    }
    // the GELU' epilogue on two reduction-contiguous operands: the direct-to-LDS
    // 256x256 tile, the 256x192 tile and the 128x128 tile only (the register
    // path 256x256 tile spills with it; gemm() maps those choices away)
    constexpr bool no256 = EPI == EPI_GELU_BWD && AT == 0 && BT == 0;
    if constexpr (AT == 0) {
      if (k == TILE_192_W8) return launch<T, 256, 192, 4, 2, AT, BT, EPI, 64>(st, g);
      if constexpr (EPI != EPI_F32 && !no256) {
        if (k == TILE_P192_W8) return launch_persist<T, 256, 192, 4, 2, BT, EPI, 64>(st, g);
        if (k == TILE_P256_W8) return launch_persist<T, 256, 256, 2, 4, BT, EPI, 64>(st, g);
      }
    }
    if constexpr (!no256) {
      if (k == TILE_256_W8) return launch<T, 256, 256, 2, 4, AT, BT, EPI, 64>(st, g);
    }
    if constexpr (AT == 1) {
      if (k == TILE_256x192_K32) return launch<T, 256, 192, 2, 2, AT, BT, EPI, 32>(st, g);
      if (k == TILE_256_W8_K32) return launch<T, 256, 256, 2, 4, AT, BT, EPI, 32>(st, g);
      if (k == TILE_128_K32) return launch<T, 128, 128, 2, 2, AT, BT, EPI, 32>(st, g);
    }
    return launch<T, 128, 128, 2, 2, AT, BT, EPI, 64>(st, g);
  } else {
    return launch<T, 128, 128, 2, 2, AT, BT, EPI, 32>(st, g);
  }
}

template <typename T>
hipError_t dispatch(hipStream_t st, int a_t, int b_t, int epi, const GemmArgs& g, TileKind k) {
  if (!a_t && !b_t) {
    if (epi == EPI_STORE) return launch_tiled<T, 0, 0, EPI_STORE>(st, g, k);
    if (epi == EPI_GELU) return launch_tiled<T, 0, 0, EPI_GELU>(st, g, k);
    if (epi == EPI_RESID) return launch_tiled<T, 0, 0, EPI_RESID>(st, g, k);
    if (epi == EPI_GELU_BWD) return launch_tiled<T, 0, 0, EPI_GELU_BWD>(st, g, k);
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
  TileKind k = choose_tile(p, a_t, b_t, g.M, g.N, g.K);
  if (epi == EPI_GELU_BWD && !a_t && !b_t)
    k = (k == TILE_P256_W8 || k == TILE_256_W8) ? TILE_D256_W8 : k == TILE_P192_W8 ? TILE_192_W8 : k;
  return p == BF16 ? dispatch<bf16>(st, a_t, b_t, epi, g, k) : dispatch<float>(st, a_t, b_t, epi, g, k);
}

int gemm_group_tiles(int M, int N) { return ((M + 255) / 256) * ((N + 255) / 256); }

int gemm_group_split_hint(int M, int N, int K, int group_tiles) {
  // the weight-gradient tile (256x256, BK = 32): as many splits as keep the
  // group's blocks within one round over the CUs, each at least two steps long
  (void)M;
  (void)N;
  if (group_tiles <= 0 || group_tiles >= 256) return 1;
  return std::max(1, std::min(256 / group_tiles, K / 32 / 2));
}

hipError_t gemm_group(hipStream_t st, const GemmArgs* probs, int count) {
  constexpr int BM = 256, BN = 256, BK = 32, WI = 2, WJ = 4;
  if (count < 1 || count > kMaxGemmGroup) return hipErrorInvalidValue;
  GemmGroup gg;
  gg.count = count;
  int blocks = 0;
  for (int i = 0; i < count; i++) {
    const GemmArgs& g = probs[i];
    if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.splits < 1 || g.K % BK != 0 || g.K / BK < g.splits || g.M % 8 != 0 ||
        g.N % 8 != 0 || g.lda % 8 != 0 || g.ldb % 8 != 0)
      return hipErrorInvalidValue;
    gg.p[i] = g;
    gg.block0[i] = blocks;
    blocks += ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.splits;
  }
  for (int i = count; i <= kMaxGemmGroup; i++) gg.block0[i] = blocks;
  hipLaunchKernelGGL((gemm_group_kernel<bf16, BM, BN, BK, WI, WJ, 1, 1, EPI_F32>), dim3(blocks), dim3(WI * WJ * 64), 0,
                     st, gg);
  return hipGetLastError();
}

hipError_t gemm_fp8(hipStream_t st, int epi, const GemmArgs& g) {
  // forward products with FP8 E4M3 operands: the 8-wave tiles of the bf16
  // path, BK = 128 (the same 128-byte LDS rows)
  const bool w192 = g.N % 192 == 0 && g.N <= 2304;
#define FP8_LAUNCH(E)                                                                                  \
  return w192 ? launch<bf16, 256, 192, 4, 2, 0, 0, E, 128, 0, fp8e4>(st, g)                          \
              : launch<bf16, 256, 256, 2, 4, 0, 0, E, 128, 0, fp8e4>(st, g);
  if (epi == EPI_STORE) FP8_LAUNCH(EPI_STORE)
  if (epi == EPI_GELU) FP8_LAUNCH(EPI_GELU)
  if (epi == EPI_RESID) FP8_LAUNCH(EPI_RESID)
#undef FP8_LAUNCH
  return hipErrorInvalidValue;
}

int gemm_split_hint(Prec p, int a_t, int b_t, int M, int N, int K) {
  const TileKind k = choose_tile(p, a_t, b_t, M, N, K);
  const int bm = (k == TILE_128 || k == TILE_128_K32) ? 128 : 256;
  const int bn = (k == TILE_256x192_K32 || k == TILE_192_W8 || k == TILE_P192_W8) ? 192
                 : (k == TILE_256_W8 || k == TILE_256_W8_K32 || k == TILE_D256_W8 || k == TILE_P256_W8) ? 256 : 128;
  const int bk = tile_bk(p, k);
  const int tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  if (a_t && b_t && k == TILE_256_W8_K32) {
    // one round of one block per CU: as many splits as fit beside the tiles
    // (uneven splits are allowed), each at least two reduction steps long
    if (tiles >= 256) return 1;
    return std::max(1, std::min(256 / tiles, K / bk / 2));
  }
  // one block per CU for the large tiles, two for 128x128; powers of two
  const int target = (k == TILE_128 || k == TILE_128_K32) ? 512 : 256;
  int s = 1;
  while (s < 16 && tiles * s < target && K % (2 * s * bk) == 0) s *= 2;
  return s;
}

}  // namespace gpt2k
