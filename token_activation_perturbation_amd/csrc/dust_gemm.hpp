// dust_gemm.hpp -- LDS-tiled bf16 MFMA GEMMs for the two dense contractions
// of the estimator on gfx950:
//   base   delta[t][c] = sum_k X[t][k] W[c][k] - target[t][c]  ("NT": both
//          operands contiguous along the contraction axis k)
//   outer  G[c][i] = sum_t g[t][c] X[t][i]  ("TN": both operands contiguous
//          along the output axes, the token axis t strided), g as its bf16
//          split hi = rn(g), lo = rn(g - hi) (written by the noise kernels),
//          each half an MFMA A operand, fp32 accumulation.
//
// A workgroup of 256 threads (4 waves in a 2x2 grid) computes a 64 x 64
// tile; each wave a 32 x 32 block of 16x16 MFMA tiles
// (v_mfma_f32_16x16x32_bf16: lane l supplies row l % 16 of A and column
// l % 16 of B with the 8 contraction values of group l / 16, and holds D rows
// 4 (l / 16) + 0..3 of column l % 16).  Two designs per contraction:
//  - for aligned operands (the usual case), tiles go straight from HBM to LDS
//    with gfx950's direct-to-LDS loads into XOR-slot-permuted rows
//    (nt_gemm_dma_kernel, tn_outer_dma_kernel);
//  - for any other shape or alignment, element-wise guarded loads staged
//    through registers (nt_gemm_kernel, tn_outer_kernel).
// Both give the same results bit for bit (same tiles, same contraction
// order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dust {
namespace gemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));


__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// A (rows x BK) tile of a row-major bf16 matrix whose rows are contiguous
// along k: element (r, k) at src[r * ld + k].  Each thread moves
// rows * BK / 8 / 256 chunks of 8 values with element-wise guarded loads
// (any ld, any alignment); values outside the matrix are zero.
// LDS row padding in bf16 elements (-DDUST_LDS_PAD=n at build time).
#ifndef DUST_LDS_PAD
#define DUST_LDS_PAD 16
#endif

template <int ROWS, int BK>
struct KMajorTile {
  static constexpr int LDK = BK + DUST_LDS_PAD;  // padded LDS row, in bf16 elements
  static constexpr int kChunks = ROWS * BK / 8 / 256;
  u16x8_t reg[kChunks];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld,
                                       int64_t rows, int64_t kmax, int tid, int64_t r0,
                                       int64_t k0) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
      const int64_t r = r0 + row, k = k0 + kc;
      u16x8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (r < rows) {
        const uint16_t* p = src + r * ld + k;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (k + j < kmax) v[j] = p[j];
      }
      reg[i] = v;
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
      *(u16x8_t*)(lds + row * LDK + kc) = reg[i];
    }
  }
};

__device__ __forceinline__ f32x4_t mfma16(u16x8_t a, u16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Work mapping.  The dispatcher deals workgroups to the 8 XCDs round-robin
// (workgroup b runs on XCD b % 8), and each XCD has its own L2.  So the work
// items (split, m-tile, n-tile) are linearised split-major and XCD x takes
// the contiguous range [x * per_xcd, (x+1) * per_xcd).  Within a split the
// items run in groups of GM m-tiles: m fastest inside a group, then n, then
// the next group.  The base GEMM takes GM = 8, so the workgroups resident on
// one XCD at a time cover a compact block of about 8 A row-blocks and a
// dozen B blocks, which stays in that L2 even when all of B (a 3072 x 768
// weight, 4.7 MB) would not; the outer product, whose B (the layer input's
// columns) has few tiles, takes GM = 1 (n fastest: consecutive workgroups
// share their A row-block), which measured half the L2 misses of GM = 8 at
// the same speed.  grid = 8 * per_xcd; items past the end exit at once.
constexpr int kNtGroupM = 8, kTnGroupM = 1;
struct TileWork {
  int split, m_tile, n_tile;
  bool valid;
};
template <int GM>
__device__ __forceinline__ TileWork map_tile(int tiles_m, int tiles_n, int splits, int per_xcd) {
  const int b = blockIdx.x;
  const int wid = (b % 8) * per_xcd + b / 8;
  const int per_split = tiles_m * tiles_n;
  TileWork w;
  w.valid = wid < per_split * splits;
  w.split = wid / per_split;
  const int r = wid % per_split;
  const int first_m = (r / (GM * tiles_n)) * GM;
  const int size_m = min(tiles_m - first_m, GM);
  const int in_group = r % (GM * tiles_n);
  w.m_tile = first_m + in_group % size_m;
  w.n_tile = in_group / size_m;
  return w;
}

// The MFMAs of one k-tile held in LDS: wave (wm, wn) multiplies rows
// wm * 32 + [0, 32) of A with rows wn * 32 + [0, 32) of B.
template <int BK, int LDK>
__device__ __forceinline__ void mma_tile(const uint16_t* la, const uint16_t* lb, int wm, int wn,
                                         int lane, f32x4_t (&acc)[2][2]) {
  const int fr = lane & 15, fk = (lane >> 4) * 8;
#pragma unroll
  for (int ks = 0; ks < BK; ks += 32) {
    u16x8_t af[2], bfr[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      af[i] = *(const u16x8_t*)(&la[(wm * 32 + i * 16 + fr) * LDK + ks + fk]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      bfr[j] = *(const u16x8_t*)(&lb[(wn * 32 + j * 16 + fr) * LDK + ks + fk]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
  }
}

// gfx950's transposing LDS read, ds_read_b64_tr_b16: within each group of 16
// lanes, output lane i element e is element i % 4 of the 8 bytes that lane
// 4 e + i / 4 addressed (measured on MI355X).  So when the 16 lanes of a
// group address a block of 4 tokens x 16 channels of a token-major tile (lane
// j: token j / 4, channels 4 (j % 4) .. + 3), lane i receives channel i of
// the 4 tokens: half of an MFMA operand fragment, contraction-contiguous.
typedef short v4i16_t __attribute__((ext_vector_type(4)));

// MFMA operand fragment (16 rows = channels ch0 .. ch0 + 15, 8 contraction
// values = tokens k0 + 8 (lane / 16) .. + 7) from a token-major bf16 tile with
// row pitch LDT elements.
template <int LDT>
__device__ __forceinline__ u16x8_t frag_tr(const uint16_t* tile, int ch0, int k0, int lane) {
  const int tok = k0 + 8 * (lane >> 4) + ((lane & 15) >> 2);
  const uint16_t* p = tile + tok * LDT + ch0 + 4 * (lane & 3);
  typedef __attribute__((address_space(3))) v4i16_t* lds_v4_ptr;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)p);
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)(p + 4 * LDT));
  return __builtin_bit_cast(u16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------------------
// Base GEMM: delta[m][n] = sum_k A[m][k] B[n][k] - target[m][n] (target bf16,
// delta fp32), A = X [M = T][K = d_in], B = W [N = d_out][K]; without TARGET
// the plain product (the logits of a head).  64 x 64 tiles, BK = 64.
//
// Software pipeline: S register stages hold the next S k-tiles in flight
// from HBM.  Step kt multiplies tile kt from LDS buffer kt & 1, writes tile
// kt+1 from its register stage into the other LDS buffer, refills that stage
// with tile kt+1+S, and ends with one barrier.  The k loop is unrolled by S so
// every stage index is a compile-time constant.
template <int S, bool TARGET>
__global__ __launch_bounds__(256) void nt_gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int64_t lda, int64_t ldb,
    int32_t M, int32_t N, int64_t K, int32_t tiles_m, int32_t tiles_n, int32_t per_xcd,
    const uint16_t* __restrict__ target, float* __restrict__ out) {
  constexpr int BM = 64, BN = 64, BK = 64, WM = 32, WN = 32;
  constexpr int LDK = BK + DUST_LDS_PAD;
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[2][BN * LDK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const TileWork work = map_tile<kNtGroupM>(tiles_m, tiles_n, 1, per_xcd);
  if (!work.valid) return;
  const int64_t m0 = (int64_t)work.m_tile * BM;
  const int64_t n0 = (int64_t)work.n_tile * BN;
  const int nk = (int)((K + BK - 1) / BK);
  static_assert(S % 2 == 0, "the LDS double buffer is indexed by the stage parity");

  KMajorTile<BM, BK> ta[S];
  KMajorTile<BN, BK> tb[S];
  auto load_stage = [&](int st, int kt) {
    const int64_t k0 = (int64_t)kt * BK;
    ta[st].load(A, lda, M, K, tid, m0, k0);
    tb[st].load(B, ldb, N, K, tid, n0, k0);
  };
  auto store_stage = [&](int st, int buf) {
    ta[st].store(lds_a[buf], tid);
    tb[st].store(lds_b[buf], tid);
  };

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // fetch the epilogue's target values now, so their latency hides behind
  // the k loop: unconditional loads from a clamped address (no branch, no
  // wait); entries outside the matrix are never stored
  uint16_t tgt[2][2][4] = {};
  if constexpr (TARGET) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t row = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + e;
          const int64_t col = n0 + wn * WN + j * 16 + (lane & 15);
          const int64_t rr = row < M ? row : M - 1, cc = col < N ? col : N - 1;
          tgt[i][j][e] = target[rr * N + cc];
        }
  }

  // Branch-free pipeline: the tile count is padded to a multiple of S (the
  // padding tiles lie past K, so they load from a clamped address and store
  // zeros), so the compiler sees one straight-line body per S steps and keeps
  // S tiles of loads in flight instead of waiting at branches.
  const int nk_pad = ((nk + S - 1) / S) * S;
#pragma unroll
  for (int st = 0; st < S; ++st) load_stage(st, st);
  store_stage(0, 0);
  load_stage(0, S);
  __syncthreads();
  for (int kt0 = 0; kt0 < nk_pad; kt0 += S) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int kt = kt0 + s;
      const int cur = s & 1;  // S is even, so kt & 1 == s & 1
      mma_tile<BK, LDK>(lds_a[cur], lds_b[cur], wm, wn, lane, acc);
      const int nxt = (s + 1) % S;
      store_stage(nxt, cur ^ 1);
      load_stage(nxt, kt + 1 + S);
      __syncthreads();
      // keep each step's register work in its step: the scheduler would
      // otherwise hoist later stages' masking above their loads' arrival
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + e;
        const int64_t col = n0 + wn * WN + j * 16 + (lane & 15);
        if (row < M && col < N)
          out[row * N + col] = TARGET ? acc[i][j][e] - bf16_bits_to_f32(tgt[i][j][e])
                                      : acc[i][j][e];
      }
}

// ---------------------------------------------------------------------------
// Outer product over token ranges: out[m][n] = sum_t g[t][m] X[t][n] for t in
// split s's range [t_first + s * t_per_split, min(T, t_first + (s + 1) *
// t_per_split)), s < splits; g as its bf16 split g = g_hi + g_lo (written so by
// the kernels that produce g), both [T][M] (M = d_out), X bf16 [T][N]
// (N = d_in).  partial == 0: one split, out is G itself; else split s writes
// its own [M][N] partial at out + s M N (summed afterwards by a fixed-order
// kernel).  64 x 64 tiles, BK = 64 tokens; two MFMAs (hi, lo) per product.
//
// Both operands are contiguous along the output axes (token-major), so the
// tiles are staged as they lie in HBM, 64 tokens x 64 channels with a row
// pitch of 72 bf16 (144 bytes; nearly free of bank conflicts for the reads
// below), and the transposition happens in the LDS read (frag_tr).  Loads:
// thread t moves chunks t and t + 256 of each tile (token c / 8, channels
// 8 (c % 8) .. + 7) element by element, so any M, N and alignment work.  Rows
// past T re-read row T - 1 and channels past the edge re-read the last one;
// g rows of tokens outside the split are zeroed at the LDS store (X rows need
// not be: their products with zero g vanish).  Pipeline as in
// nt_gemm_kernel.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 split of two floats, hi = rn(v) and lo = rn(v - hi) (v_cvt_pk_bf16_f32,
// round to nearest even), each pair packed in a dword with a in the low half.
// hi + lo carries 16 significant bits of v.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  const f32x2_t v = {a, b};
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  const f32x2_t h = {__uint_as_float(hi << 16), __uint_as_float(hi & 0xFFFF0000u)};
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(v - h, bf16x2_t));
}

template <int S>
__global__ __launch_bounds__(256) void tn_outer_kernel(
    const uint16_t* __restrict__ g_hi, const uint16_t* __restrict__ g_lo,
    const uint16_t* __restrict__ X, int32_t T, int32_t M, int32_t N, int32_t tiles_m,
    int32_t tiles_n, int32_t splits, int32_t per_xcd, int64_t t_first, int64_t t_per_split,
    int32_t partial, float* __restrict__ out) {
  constexpr int BM = 64, BN = 64, BK = 64, LDT = 72;
  __shared__ __attribute__((aligned(16))) uint16_t lds_ah[2][BK * LDT];
  __shared__ __attribute__((aligned(16))) uint16_t lds_al[2][BK * LDT];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[2][BK * LDT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const TileWork work = map_tile<kTnGroupM>(tiles_m, tiles_n, splits, per_xcd);
  if (!work.valid) return;
  const int64_t m0 = (int64_t)work.m_tile * BM;
  const int64_t n0 = (int64_t)work.n_tile * BN;
  const int64_t t_begin = t_first + (int64_t)work.split * t_per_split;
  const int64_t t_end = min((int64_t)T, t_begin + t_per_split);
  const int nk = (int)((t_end - t_begin + BK - 1) / BK);
  static_assert(S % 2 == 0, "the LDS double buffer is indexed by the stage parity");

  // this thread's two chunks: token rows tr[h], channel offsets cc (x8)
  int trow[2], cc[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = tid + 256 * h;
    trow[h] = c >> 3;
    cc[h] = (c & 7) * 8;
  }
  u16x8_t rh[S][2], rl[S][2], rb[S][2];
  auto load_stage = [&](int st, int kt) {
    const int64_t tb = t_begin + (int64_t)kt * BK;
    const int64_t tbc = tb < T ? tb : (int64_t)T - 1;   // uniform
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int64_t t = tbc + trow[h];
      t = t < T ? t : (int64_t)T - 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t ca = m0 + cc[h] + e < M ? m0 + cc[h] + e : (int64_t)M - 1;
        const int64_t cb = n0 + cc[h] + e < N ? n0 + cc[h] + e : (int64_t)N - 1;
        rh[st][h][e] = g_hi[t * M + ca];
        rl[st][h][e] = g_lo[t * M + ca];
        rb[st][h][e] = X[t * N + cb];
      }
    }
  };
  auto store_stage = [&](int st, int buf, int kt) {
    const int64_t tb = t_begin + (int64_t)kt * BK;
    const int64_t left = t_end - tb;                     // uniform
    const int n_ok = (int)(left < 0 ? 0 : (left > 64 ? 64 : left));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // all-ones or zero, applied with ANDs (a select here becomes a branch)
      const uint32_t mk = 0u - (uint32_t)(trow[h] < n_ok);
      const int off = trow[h] * LDT + cc[h];
      *(u32x4_t*)(&lds_ah[buf][off]) = __builtin_bit_cast(u32x4_t, rh[st][h]) & mk;
      *(u32x4_t*)(&lds_al[buf][off]) = __builtin_bit_cast(u32x4_t, rl[st][h]) & mk;
      *(u16x8_t*)(&lds_b[buf][off]) = rb[st][h];
    }
  };
  auto mma = [&](int buf, f32x4_t (&acc)[2][2]) {
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      u16x8_t ah[2], al[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ah[i] = frag_tr<LDT>(lds_ah[buf], wm * 32 + i * 16, ks, lane);
        al[i] = frag_tr<LDT>(lds_al[buf], wm * 32 + i * 16, ks, lane);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = frag_tr<LDT>(lds_b[buf], wn * 32 + j * 16, ks, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = mfma16(ah[i], bf[j], acc[i][j]);
          acc[i][j] = mfma16(al[i], bf[j], acc[i][j]);
        }
    }
  };

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk_pad = ((nk + S - 1) / S) * S;
#pragma unroll
  for (int st = 0; st < S; ++st) load_stage(st, st);
  store_stage(0, 0, 0);
  load_stage(0, S);
  __syncthreads();
  for (int kt0 = 0; kt0 < nk_pad; kt0 += S) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int kt = kt0 + s;
      const int cur = s & 1;
      mma(cur, acc);
      const int nxt = (s + 1) % S;
      store_stage(nxt, cur ^ 1, kt + 1);
      load_stage(nxt, kt + 1 + S);
      __syncthreads();
      // keep each step's register work in its step: the scheduler would
      // otherwise hoist later stages' masking above their loads' arrival
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float* dst = partial ? out + (int64_t)work.split * M * N : out;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + e;
        const int64_t col = n0 + wn * 32 + j * 16 + (lane & 15);
        if (row < M && col < N) dst[row * N + col] = acc[i][j][e];
      }
}

// ---------------------------------------------------------------------------
// The outer product fed by gfx950's direct-to-LDS loads
// (global_load_lds_dwordx4: lane l's 16 bytes land at the instruction's LDS
// base + 16 l, measured on MI355X), for the aligned case (M and N multiples of
// 8, g_hi, g_lo and X 16-byte aligned).  Same work split, contraction order
// and results (bitwise) as tn_outer_kernel; no registers stage the tiles and
// no LDS store instructions run, so three workgroups fit a CU (48 KiB of LDS
// each) and the loads overlap the MFMAs of the other workgroups.
//
// A tile is 64 tokens x 64 channels bf16, a token per 128-byte LDS row whose
// eight 16-byte slots hold the channel chunks permuted: chunk c of row r sits
// in slot c ^ tr_swz(r).  Each DMA instruction fills 8 rows (1 KiB): lane l
// fetches row 8 i + l / 8, chunk (l % 8) ^ tr_swz(row), so its 16 bytes land
// in the right slot.  tr_swz was chosen by an exhaustive search over XOR maps
// of the row bits so that the transposing fragment reads (frag_sw) are free
// of bank conflicts per half-wave on 64 banks.  NS LDS stages of 24 KiB: the
// loads of k-block kt + NS - 1 are issued right after the barrier that opens
// step kt.
// Token rows past T re-read row T - 1, channel chunks past the edge re-read
// the last full chunk (their outputs are never stored); g rows past the
// split's end are zeroed in LDS before the MFMAs read them.

__device__ __forceinline__ int tr_swz(int r) { return (r & 2) | ((r >> 1) & 4); }

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8],
// vmcnt[15:14]; the other counters left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// LDS stages of the direct-to-LDS kernels (-DDUST_NT_DMA_STAGES=n,
// -DDUST_TN_DMA_STAGES=n at build time): block kt + NS - 1 is in flight while
// block kt is multiplied.
#ifndef DUST_NT_DMA_STAGES
#define DUST_NT_DMA_STAGES 3
#endif
#ifndef DUST_TN_DMA_STAGES
#define DUST_TN_DMA_STAGES 2
#endif
// tokens per k-block of the direct-to-LDS outer product (32 or 64)
#ifndef DUST_TN_BK
#define DUST_TN_BK 64
#endif

// Wait until this wave's loads of the oldest block in flight have landed,
// with `ahead` (0 .. NS - 2, uniform) later blocks allowed to stay in
// flight; each block is LOADS load instructions per lane, and vector-memory
// loads complete in issue order for vmcnt.
//
// The barrier that follows is stage_barrier, not __syncthreads: the latter's
// workgroup fence makes the compiler wait for every load in flight (vmcnt 0,
// since a direct-to-LDS load counts as an LDS write), which would drain the
// later stages too.  stage_barrier waits only for this wave's LDS reads
// (lgkmcnt 0: the buffer about to be refilled is no longer read) and keeps
// every memory access on its side of the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int NS, int LOADS>
__device__ __forceinline__ void wait_blocks(int ahead) {
  static_assert(NS >= 2 && NS <= 4, "stages");
  if constexpr (NS == 2) {
    wait_vmcnt<0>();
  } else if constexpr (NS == 3) {
    if (ahead >= 1) wait_vmcnt<LOADS>(); else wait_vmcnt<0>();
  } else {
    if (ahead >= 2) wait_vmcnt<2 * LOADS>();
    else if (ahead == 1) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
  }
}

// frag_tr's fragment from a slot-permuted tile (rows of 128 bytes)
__device__ __forceinline__ u16x8_t frag_sw(const uint8_t* tile, int ch0, int k0, int lane) {
  const int tok = k0 + 8 * (lane >> 4) + ((lane & 15) >> 2);
  const int ch = ch0 + 4 * (lane & 3);
  const int c = ch >> 3, eb = (ch & 7) * 2;
  typedef __attribute__((address_space(3))) v4i16_t* lds_v4_ptr;
  const uint8_t* p0 = tile + tok * 128 + 16 * (c ^ tr_swz(tok)) + eb;
  const uint8_t* p1 = tile + (tok + 4) * 128 + 16 * (c ^ tr_swz(tok + 4)) + eb;
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)p0);
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)p1);
  return __builtin_bit_cast(u16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// frag_sw's fragment read through inline assembly.  The compiler treats the
// transposing-read builtin as touching any LDS address, so before each one
// it waits for every direct-to-LDS load in flight (vmcnt 0), draining the
// next block's loads before the current block is multiplied.  Issued as
// assembly the reads carry no such wait; the caller orders them with the
// block waits and barriers of its pipeline and waits for their results with
// frag_wait before the MFMAs read them.
__device__ __forceinline__ v4i16_t ds_read_tr_asm(const uint8_t* p) {
  v4i16_t r;
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(a));
  return r;
}

__device__ __forceinline__ u16x8_t frag_sw_asm(const uint8_t* tile, int ch0, int k0, int lane) {
  const int tok = k0 + 8 * (lane >> 4) + ((lane & 15) >> 2);
  const int ch = ch0 + 4 * (lane & 3);
  const int c = ch >> 3, eb = (ch & 7) * 2;
  const v4i16_t lo = ds_read_tr_asm(tile + tok * 128 + 16 * (c ^ tr_swz(tok)) + eb);
  const v4i16_t hi = ds_read_tr_asm(tile + (tok + 4) * 128 + 16 * (c ^ tr_swz(tok + 4)) + eb);
  return __builtin_bit_cast(u16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Wait for this wave's LDS reads; the fragments pass through the statement,
// so no use of them can be scheduled before it.
__device__ __forceinline__ void frag_wait(u16x8_t& a0, u16x8_t& a1, u16x8_t& a2, u16x8_t& a3,
                                          u16x8_t& b0, u16x8_t& b1) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(b0), "+v"(b1));
}

__global__ __launch_bounds__(256) void tn_outer_dma_kernel(
    const uint16_t* __restrict__ g_hi, const uint16_t* __restrict__ g_lo,
    const uint16_t* __restrict__ X, int32_t T, int32_t M, int32_t N, int32_t tiles_m,
    int32_t tiles_n, int32_t splits, int32_t per_xcd, int64_t t_first, int64_t t_per_split,
    int32_t partial, float* __restrict__ out) {
  constexpr int BK = DUST_TN_BK, TB = BK * 128, NS = DUST_TN_DMA_STAGES, QN = BK / 32;
  static_assert(BK == 32 || BK == 64, "k-block");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * 3 * TB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const TileWork work = map_tile<kTnGroupM>(tiles_m, tiles_n, splits, per_xcd);
  if (!work.valid) return;
  const int64_t m0 = (int64_t)work.m_tile * 64;
  const int64_t n0 = (int64_t)work.n_tile * 64;
  const int64_t t_begin = t_first + (int64_t)work.split * t_per_split;
  const int64_t t_end = min((int64_t)T, t_begin + t_per_split);
  const int nk = (int)((t_end - t_begin + BK - 1) / BK);

  // this lane's QN DMA rows (instructions QN wave + q of a tile) and the
  // chunks it fetches for them
  int rq[QN];
  int64_t a_ch[QN], b_ch[QN];
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    const int r = 8 * (QN * wave + q) + (lane >> 3);
    const int c = (lane & 7) ^ tr_swz(r);
    rq[q] = r;
    const int64_t am = m0 + 8 * c, bn = n0 + 8 * c;
    a_ch[q] = am < M ? am : M - 8;
    b_ch[q] = bn < N ? bn : N - 8;
  }
  auto issue = [&](int buf, int kt) {
    const int64_t tb = t_begin + (int64_t)kt * BK;
    uint8_t* base = lds + buf * 3 * TB;
#pragma unroll
    for (int q = 0; q < QN; ++q) {
      int64_t t = tb + rq[q];
      t = t < T ? t : (int64_t)T - 1;
      const int dst = (QN * wave + q) * 1024;
      __builtin_amdgcn_global_load_lds(g_hi + t * M + a_ch[q], (lds_void_ptr)(base + dst), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(g_lo + t * M + a_ch[q], (lds_void_ptr)(base + TB + dst), 16,
                                       0, 0);
      __builtin_amdgcn_global_load_lds(X + t * N + b_ch[q], (lds_void_ptr)(base + 2 * TB + dst),
                                       16, 0, 0);
    }
  };

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int b = 0; b < NS - 1 && b < nk; ++b) issue(b, b);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of block kt have landed ...
    wait_blocks<NS, 3 * QN>(min(nk - 1 - kt, NS - 2));
    stage_barrier();  // ... and every wave's; block kt - 1 is no longer read
    const int buf = kt % NS;
    uint8_t* base = lds + buf * 3 * TB;
    const int64_t left = t_end - (t_begin + (int64_t)kt * BK);
    if (left < BK) {
      // g rows past the split's end (rows keep their place; slots permute
      // within a row)
      const int from = (int)(left < 0 ? 0 : left) * 128;
      for (int o = from + 16 * tid; o < TB; o += 16 * 256) {
        *(u32x4_t*)(base + o) = u32x4_t{0u, 0u, 0u, 0u};
        *(u32x4_t*)(base + TB + o) = u32x4_t{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, kt + NS - 1);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      u16x8_t ah[2], al[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ah[i] = frag_sw_asm(base, wm * 32 + i * 16, ks, lane);
        al[i] = frag_sw_asm(base + TB, wm * 32 + i * 16, ks, lane);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = frag_sw_asm(base + 2 * TB, wn * 32 + j * 16, ks, lane);
      frag_wait(ah[0], ah[1], al[0], al[1], bf[0], bf[1]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = mfma16(ah[i], bf[j], acc[i][j]);
          acc[i][j] = mfma16(al[i], bf[j], acc[i][j]);
        }
    }
  }
  float* dst = partial ? out + (int64_t)work.split * M * N : out;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + e;
        const int64_t col = n0 + wn * 32 + j * 16 + (lane & 15);
        if (row < M && col < N) dst[row * N + col] = acc[i][j][e];
      }
}

// ---------------------------------------------------------------------------
// The base GEMM fed by direct-to-LDS loads, for the aligned case (K a
// multiple of 8; A, B 16-byte aligned; lda, ldb multiples of 8).  Same tiles,
// contraction order and results (bitwise) as nt_gemm_kernel; NS LDS stages
// of 16 KiB, blocks up to kt + NS - 1 in flight while block kt is
// multiplied (3 stages: 48 KiB, three workgroups per CU).  An operand tile is
// 64 rows x 64 contraction values bf16, a row per 128 bytes, chunk c of row
// r in slot c ^ nt_swz(r): the 16-byte fragment
// reads (16 rows of one chunk per quarter-wave) then hit every bank once
// (nt_swz found by the same exhaustive search as tr_swz).  Rows past M or N
// re-read the last row (their outputs are never stored); chunks past K
// re-read the last chunk, and A's are zeroed in LDS so they add nothing.
// With a target, the epilogue goes through LDS so that target is read and
// delta written in 16-byte pieces along rows; the plain product (a head's
// logits) is stored straight from the MFMA layout, which measured faster.

__device__ __forceinline__ int nt_swz(int r) { return (r >> 1) & 7; }

template <bool TARGET>
__global__ __launch_bounds__(256) void nt_gemm_dma_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int64_t lda, int64_t ldb,
    int32_t M, int32_t N, int64_t K, int32_t tiles_m, int32_t tiles_n, int32_t per_xcd,
    const uint16_t* __restrict__ target, float* __restrict__ out) {
  constexpr int BK = 64, TB = 64 * 128, NS = DUST_NT_DMA_STAGES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS * 2 * TB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const TileWork work = map_tile<kNtGroupM>(tiles_m, tiles_n, 1, per_xcd);
  if (!work.valid) return;
  const int64_t m0 = (int64_t)work.m_tile * 64;
  const int64_t n0 = (int64_t)work.n_tile * 64;
  const int nk = (int)((K + BK - 1) / BK);

  // this lane's two DMA rows and the chunk it fetches for them
  int ck[2];
  int64_t a_row[2], b_row[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 8 * (2 * wave + q) + (lane >> 3);
    ck[q] = (lane & 7) ^ nt_swz(r);
    a_row[q] = m0 + r < M ? m0 + r : M - 1;
    b_row[q] = n0 + r < N ? n0 + r : N - 1;
  }
  auto issue = [&](int buf, int kt) {
    uint8_t* base = lds + buf * 2 * TB;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      int64_t k = (int64_t)kt * BK + 8 * ck[q];
      k = k < K ? k : K - 8;
      const int dst = (2 * wave + q) * 1024;
      __builtin_amdgcn_global_load_lds(A + a_row[q] * lda + k, (lds_void_ptr)(base + dst), 16, 0,
                                       0);
      __builtin_amdgcn_global_load_lds(B + b_row[q] * ldb + k, (lds_void_ptr)(base + TB + dst), 16,
                                       0, 0);
    }
  };

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // with a target: this thread's 16-column piece of it (the epilogue's row
  // segment) is fetched before the k loop, so its latency hides behind the
  // loop; the loads are older than every block's, so the block waits below
  // cover them too
  const int er = tid >> 2, ec0 = (tid & 3) * 16;
  const bool e_vec = TARGET && m0 + er < M && N - (n0 + ec0) >= 16 && (N & 7) == 0 &&
                     (((uintptr_t)target | (uintptr_t)out) & 15) == 0;
  u32x4_t tv0 = u32x4_t{0u, 0u, 0u, 0u}, tv1 = tv0;
  if (e_vec) {
    const uint16_t* tp = target + (m0 + er) * N + n0 + ec0;
    tv0 = *(const u32x4_t*)tp;
    tv1 = *(const u32x4_t*)(tp + 8);
  }

  for (int b = 0; b < NS - 1 && b < nk; ++b) issue(b, b);
  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of block kt have landed ...
    wait_blocks<NS, 4>(min(nk - 1 - kt, NS - 2));
    stage_barrier();  // ... and every wave's; block kt - 1 is no longer read
    const int buf = kt % NS;
    uint8_t* base = lds + buf * 2 * TB;
    const int64_t left = K - (int64_t)kt * BK;
    if (left < BK) {
      const int row = tid >> 2;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int slot = 2 * (tid & 3) + h;
        if (8 * (slot ^ nt_swz(row)) >= left)
          *(u32x4_t*)(base + row * 128 + 16 * slot) = u32x4_t{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, kt + NS - 1);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      u16x8_t af[2], bfr[2];
      const int ch = ks / 8 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 32 + i * 16 + (lane & 15);
        af[i] = *(const u16x8_t*)(base + r * 128 + 16 * (ch ^ nt_swz(r)));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 32 + j * 16 + (lane & 15);
        bfr[j] = *(const u16x8_t*)(base + TB + r * 128 + 16 * (ch ^ nt_swz(r)));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
    }
  }
  if constexpr (!TARGET) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t row = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + e;
          const int64_t col = n0 + wn * 32 + j * 16 + (lane & 15);
          if (row < M && col < N) out[row * N + col] = acc[i][j][e];
        }
  } else {
    // the 64 x 64 fp32 tile through LDS (row pitch 68 floats), then a row
    // segment of 16 per thread
    constexpr int CP = 68;
    float* ct = (float*)lds;
    __syncthreads();  // every wave is done with the operand tiles
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ct[(wm * 32 + i * 16 + 4 * (lane >> 4) + e) * CP + wn * 32 + j * 16 + (lane & 15)] =
              acc[i][j][e];
    __syncthreads();
    const int r = er, c0 = ec0;
    const int64_t row = m0 + r;
    if (row < M) {
      const float* src = ct + r * CP + c0;
      float* dst = out + row * N + n0 + c0;
      const uint16_t* tp = target + row * N + n0 + c0;
      const int64_t ncols = N - (n0 + c0);  // columns left in this row
      // 16-byte pieces need whole rows of 8-element multiples and aligned bases
      if (e_vec) {
        float4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = *(const float4*)(src + 4 * q);
        const uint32_t tw[8] = {tv0[0], tv0[1], tv0[2], tv0[3], tv1[0], tv1[1], tv1[2], tv1[3]};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q].x -= __uint_as_float(tw[2 * q] << 16);
          v[q].y -= __uint_as_float(tw[2 * q] & 0xFFFF0000u);
          v[q].z -= __uint_as_float(tw[2 * q + 1] << 16);
          v[q].w -= __uint_as_float(tw[2 * q + 1] & 0xFFFF0000u);
          *(float4*)(dst + 4 * q) = v[q];
        }
      } else {
        for (int q = 0; q < 16 && q < ncols; ++q) dst[q] = src[q] - bf16_bits_to_f32(tp[q]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The outer product on 128 x 128 tiles (the aligned case of
// tn_outer_dma_kernel, for problems with enough tiles per token split).
// Each wave multiplies a 64 x 64 block: per 32-token k-block it reads 4 hi,
// 4 lo and 4 X fragments and issues 32 MFMAs, twice the MFMAs per fragment
// of the 64 x 64 kernel.  A 128-channel tile is held as two 64-channel
// sub-tiles in the layout of tn_outer_dma_kernel (a token per 128-byte row,
// chunk c of row r in slot c ^ tr_swz(r)), so wave (wm, wn) reads hi / lo
// sub-tile wm and X sub-tile wn.  k-blocks of 32 tokens, two LDS stages of
// 24 KiB (48 KiB: three workgroups per CU).  Per output element the
// contraction runs over the same 32-token steps in the same order (hi, then
// lo) as in tn_outer_dma_kernel, so for the same token split the results are
// bitwise equal.  Edges as there: token rows past T re-read row T - 1, chunks
// past M or N re-read the last full chunk (never stored), g rows past the
// split's end are zeroed in LDS.

// Wait for this wave's LDS reads: 12 fragments pass through the statement.
__device__ __forceinline__ void frag_wait12(u16x8_t (&a)[4], u16x8_t (&b)[4], u16x8_t (&c)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]),
                 "+v"(b[2]), "+v"(b[3]), "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]));
}

constexpr int kTnBigStage = 6 * 32 * 128;  // bytes of one LDS stage of tn_outer_big_kernel

template <int NS>
__global__ __launch_bounds__(256) void tn_outer_big_kernel(
    const uint16_t* __restrict__ g_hi, const uint16_t* __restrict__ g_lo,
    const uint16_t* __restrict__ X, int32_t T, int32_t M, int32_t N, int32_t tiles_m,
    int32_t tiles_n, int32_t splits, int32_t per_xcd, int64_t t_first, int64_t t_per_split,
    int32_t partial, float* __restrict__ out) {
  constexpr int BK = 32, SUB = BK * 128;  // a 32-token x 64-channel sub-tile
  constexpr int STAGE = 6 * SUB;          // hi (2), lo (2), X (2) sub-tiles
  static_assert(STAGE == kTnBigStage, "stage size");
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];  // NS * STAGE bytes
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const TileWork work = map_tile<kTnGroupM>(tiles_m, tiles_n, splits, per_xcd);
  if (!work.valid) return;
  const int64_t m0 = (int64_t)work.m_tile * 128;
  const int64_t n0 = (int64_t)work.n_tile * 128;
  const int64_t t_begin = t_first + (int64_t)work.split * t_per_split;
  const int64_t t_end = min((int64_t)T, t_begin + t_per_split);
  const int nk = (int)((t_end - t_begin + BK - 1) / BK);

  // this lane's DMA row of every sub-tile (rows 8 wave .. + 7) and the
  // channel offsets it fetches for each half
  const int rq = 8 * wave + (lane >> 3);
  const int cq = (lane & 7) ^ tr_swz(rq);
  int64_t a_ch[2], b_ch[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t am = m0 + 64 * h + 8 * cq, bn = n0 + 64 * h + 8 * cq;
    a_ch[h] = am < M ? am : M - 8;
    b_ch[h] = bn < N ? bn : N - 8;
  }
  auto issue = [&](int buf, int kt) {
    int64_t t = t_begin + (int64_t)kt * BK + rq;
    t = t < T ? t : (int64_t)T - 1;
    uint8_t* base = lds + buf * STAGE + wave * 1024;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __builtin_amdgcn_global_load_lds(g_hi + t * M + a_ch[h], (lds_void_ptr)(base + h * SUB),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(g_lo + t * M + a_ch[h],
                                       (lds_void_ptr)(base + (2 + h) * SUB), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(X + t * N + b_ch[h], (lds_void_ptr)(base + (4 + h) * SUB),
                                       16, 0, 0);
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int b = 0; b < NS - 1 && b < nk; ++b) issue(b, b);
  for (int kt = 0; kt < nk; ++kt) {
    wait_blocks<NS, 6>(min(nk - 1 - kt, NS - 2));
    stage_barrier();
    const int buf = kt % NS;
    uint8_t* base = lds + buf * STAGE;
    const int64_t left = t_end - (t_begin + (int64_t)kt * BK);
    if (left < BK) {
      // g rows past the split's end, in the four hi / lo sub-tiles
      const int from = (int)(left < 0 ? 0 : left) * 128;
      for (int o = from + 16 * tid; o < SUB; o += 16 * 256) {
#pragma unroll
        for (int st = 0; st < 4; ++st) *(u32x4_t*)(base + st * SUB + o) = u32x4_t{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, kt + NS - 1);
    u16x8_t ah[4], al[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ah[i] = frag_sw_asm(base + wm * SUB, i * 16, 0, lane);
      al[i] = frag_sw_asm(base + (2 + wm) * SUB, i * 16, 0, lane);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = frag_sw_asm(base + (4 + wn) * SUB, j * 16, 0, lane);
    frag_wait12(ah, al, bf);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = mfma16(ah[i], bf[j], acc[i][j]);
        acc[i][j] = mfma16(al[i], bf[j], acc[i][j]);
      }
  }
  float* dst = partial ? out + (int64_t)work.split * M * N : out;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + e;
        const int64_t col = n0 + wn * 64 + j * 16 + (lane & 15);
        if (row < M && col < N) dst[row * N + col] = acc[i][j][e];
      }
}

// ---------------------------------------------------------------------------
// The outer product on 128 x 256 tiles (128 channels of g, 256 of the layer
// input): each wave multiplies a 64 x 128 block, reading per 32-token
// k-block 4 hi, 4 lo and 8 X fragments for 64 MFMAs, a third fewer LDS
// bytes per MFMA than tn_outer_big_kernel's 64 x 64 blocks.  The tile is held
// as 64-channel sub-tiles in the layout of tn_outer_dma_kernel (a token per
// 128-byte row, chunk c of row r in slot c ^ tr_swz(r)): hi 0-1, lo 2-3 and
// X 4-7; wave (wm, wn) reads hi / lo sub-tile wm and X sub-tiles 2 wn, 2 wn +
// 1.  Two LDS stages of 32 KiB (two workgroups per CU).  Per output element
// the contraction runs over the same 32-token steps in the same order (hi,
// then lo) as tn_outer_big_kernel, so for the same token split the results
// are bitwise equal; edges as there.

// Wait for this wave's LDS reads: 16 fragments pass through the statement.
__device__ __forceinline__ void frag_wait16(u16x8_t (&a)[4], u16x8_t (&b)[4], u16x8_t (&c)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]),
                 "+v"(b[2]), "+v"(b[3]), "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]),
                 "+v"(c[4]), "+v"(c[5]), "+v"(c[6]), "+v"(c[7]));
}

constexpr int kTnWideStage = 8 * 32 * 128;  // bytes of one LDS stage of tn_outer_wide_kernel

template <int NS>
__global__ __launch_bounds__(256) void tn_outer_wide_kernel(
    const uint16_t* __restrict__ g_hi, const uint16_t* __restrict__ g_lo,
    const uint16_t* __restrict__ X, int32_t T, int32_t M, int32_t N, int32_t tiles_m,
    int32_t tiles_n, int32_t splits, int32_t per_xcd, int64_t t_first, int64_t t_per_split,
    int32_t partial, float* __restrict__ out) {
  constexpr int BK = 32, SUB = BK * 128;  // a 32-token x 64-channel sub-tile
  constexpr int STAGE = 8 * SUB;          // hi (2), lo (2), X (4) sub-tiles
  static_assert(STAGE == kTnWideStage, "stage size");
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];  // NS * STAGE bytes
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const TileWork work = map_tile<kTnGroupM>(tiles_m, tiles_n, splits, per_xcd);
  if (!work.valid) return;
  const int64_t m0 = (int64_t)work.m_tile * 128;
  const int64_t n0 = (int64_t)work.n_tile * 256;
  const int64_t t_begin = t_first + (int64_t)work.split * t_per_split;
  const int64_t t_end = min((int64_t)T, t_begin + t_per_split);
  const int nk = (int)((t_end - t_begin + BK - 1) / BK);

  // this lane's DMA row of every sub-tile (rows 8 wave .. + 7) and the
  // channel offsets it fetches for each 64-channel piece
  const int rq = 8 * wave + (lane >> 3);
  const int cq = (lane & 7) ^ tr_swz(rq);
  int64_t a_ch[2], b_ch[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t am = m0 + 64 * h + 8 * cq;
    a_ch[h] = am < M ? am : M - 8;
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int64_t bn = n0 + 64 * h + 8 * cq;
    b_ch[h] = bn < N ? bn : N - 8;
  }
  auto issue = [&](int buf, int kt) {
    int64_t t = t_begin + (int64_t)kt * BK + rq;
    t = t < T ? t : (int64_t)T - 1;
    uint8_t* base = lds + buf * STAGE + wave * 1024;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __builtin_amdgcn_global_load_lds(g_hi + t * M + a_ch[h], (lds_void_ptr)(base + h * SUB),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds(g_lo + t * M + a_ch[h],
                                       (lds_void_ptr)(base + (2 + h) * SUB), 16, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 4; ++h)
      __builtin_amdgcn_global_load_lds(X + t * N + b_ch[h], (lds_void_ptr)(base + (4 + h) * SUB),
                                       16, 0, 0);
  };

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int b = 0; b < NS - 1 && b < nk; ++b) issue(b, b);
  for (int kt = 0; kt < nk; ++kt) {
    wait_blocks<NS, 8>(min(nk - 1 - kt, NS - 2));
    stage_barrier();
    const int buf = kt % NS;
    uint8_t* base = lds + buf * STAGE;
    const int64_t left = t_end - (t_begin + (int64_t)kt * BK);
    if (left < BK) {
      // g rows past the split's end, in the four hi / lo sub-tiles
      const int from = (int)(left < 0 ? 0 : left) * 128;
      for (int o = from + 16 * tid; o < SUB; o += 16 * 256) {
#pragma unroll
        for (int st = 0; st < 4; ++st) *(u32x4_t*)(base + st * SUB + o) = u32x4_t{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if (kt + NS - 1 < nk) issue((kt + NS - 1) % NS, kt + NS - 1);
    u16x8_t ah[4], al[4], bf[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ah[i] = frag_sw_asm(base + wm * SUB, i * 16, 0, lane);
      al[i] = frag_sw_asm(base + (2 + wm) * SUB, i * 16, 0, lane);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      bf[j] = frag_sw_asm(base + (4 + 2 * wn + (j >> 2)) * SUB, (j & 3) * 16, 0, lane);
    frag_wait16(ah, al, bf);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[i][j] = mfma16(ah[i], bf[j], acc[i][j]);
        acc[i][j] = mfma16(al[i], bf[j], acc[i][j]);
      }
  }
  float* dst = partial ? out + (int64_t)work.split * M * N : out;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + e;
        const int64_t col = n0 + wn * 128 + j * 16 + (lane & 15);
        if (row < M && col < N) dst[row * N + col] = acc[i][j][e];
      }
}

// ---------------------------------------------------------------------------
// The base GEMM on 128 x 128 tiles (the aligned case of nt_gemm_dma_kernel,
// for problems with enough tiles to fill the chip twice over).  Each wave
// multiplies a 64 x 64 block (4 x 4 MFMA tiles), so every operand fragment
// read from LDS feeds four MFMAs instead of two: half the LDS and L2 bytes
// per flop of the 64 x 64 kernel.  Two LDS stages of 32 KiB (64 KiB): two
// workgroups share a CU, so one's epilogue overlaps the other's k loop
// (NS stages: the LDS is dynamic, NS x 32 KiB).
// Same per-element contraction order as nt_gemm_dma_kernel (k-blocks of 64
// in order, two MFMA k-steps each), so the results are bitwise equal.  With a
// target, the epilogue stages the tile through LDS one 64-row half at a
// time (row pitch 132 floats), then each thread subtracts the target from
// 32 consecutive columns of one row and stores them in 16-byte pieces.
constexpr int kNtBigStage = 2 * 128 * 128;  // bytes of one LDS stage of nt_gemm_big_kernel

template <bool TARGET, int NS>
__global__ __launch_bounds__(256) void nt_gemm_big_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int64_t lda, int64_t ldb,
    int32_t M, int32_t N, int64_t K, int32_t tiles_m, int32_t tiles_n, int32_t per_xcd,
    const uint16_t* __restrict__ target, float* __restrict__ out) {
  constexpr int BM = 128, BN = 128, BK = 64;
  constexpr int TBA = BM * 128, TBB = BN * 128, STAGE = TBA + TBB;
  static_assert(STAGE == kNtBigStage, "stage size");
  constexpr int QA = BM / 32, QB = BN / 32;  // DMA instructions per wave and block
  constexpr int FI = BM / 32, FJ = BN / 32;  // MFMA tiles per wave (64 x 64 block)
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];  // NS * STAGE bytes
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const TileWork work = map_tile<kNtGroupM>(tiles_m, tiles_n, 1, per_xcd);
  if (!work.valid) return;
  const int64_t m0 = (int64_t)work.m_tile * BM;
  const int64_t n0 = (int64_t)work.n_tile * BN;
  const int nk = (int)((K + BK - 1) / BK);

  // this lane's DMA rows and the chunk it fetches for them
  int cka[QA], ckb[QB];
  int64_t a_row[QA], b_row[QB];
#pragma unroll
  for (int q = 0; q < QA; ++q) {
    const int r = 8 * (QA * wave + q) + (lane >> 3);
    cka[q] = (lane & 7) ^ nt_swz(r);
    a_row[q] = m0 + r < M ? m0 + r : M - 1;
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int r = 8 * (QB * wave + q) + (lane >> 3);
    ckb[q] = (lane & 7) ^ nt_swz(r);
    b_row[q] = n0 + r < N ? n0 + r : N - 1;
  }
  auto issue = [&](int buf, int kt) {
    uint8_t* base = lds + buf * STAGE;
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      int64_t k = (int64_t)kt * BK + 8 * cka[q];
      k = k < K ? k : K - 8;
      __builtin_amdgcn_global_load_lds(A + a_row[q] * lda + k,
                                       (lds_void_ptr)(base + (QA * wave + q) * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      int64_t k = (int64_t)kt * BK + 8 * ckb[q];
      k = k < K ? k : K - 8;
      __builtin_amdgcn_global_load_lds(B + b_row[q] * ldb + k,
                                       (lds_void_ptr)(base + TBA + (QB * wave + q) * 1024), 16,
                                       0, 0);
    }
  };

  f32x4_t acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // A's chunks past K re-read the last chunk: zero them in the block at
  // `base` (the last one, when K is not a multiple of 64)
  auto zero_tail = [&](uint8_t* base, int64_t left) {
#pragma unroll
    for (int h = 0; h < BM / 64; ++h) {
      const int row = (tid >> 2) + 64 * h;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int slot = 2 * (tid & 3) + e;
        if (8 * (slot ^ nt_swz(row)) >= left)
          *(u32x4_t*)(base + row * 128 + 16 * slot) = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    __syncthreads();
  };
  // the operand fragments of k-step ks (0 or 32) of the block at `base`
  auto read_frags = [&](const uint8_t* base, int ks, u16x8_t (&af)[FI], u16x8_t (&bf)[FJ]) {
    const int ch = ks / 8 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      const int r = wm * 64 + i * 16 + (lane & 15);
      af[i] = *(const u16x8_t*)(base + r * 128 + 16 * (ch ^ nt_swz(r)));
    }
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int r = wn * 64 + j * 16 + (lane & 15);
      bf[j] = *(const u16x8_t*)(base + TBA + r * 128 + 16 * (ch ^ nt_swz(r)));
    }
  };
  auto mma = [&](const u16x8_t (&af)[FI], const u16x8_t (&bf)[FJ]) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
  };
  // the scheduler is asked to alternate two MFMAs with one LDS read, so the
  // next k-step's fragments arrive while this one's MFMAs run
  auto interleave = [&]() {
#pragma unroll
    for (int u = 0; u < FI + FJ; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
  };

  // Software pipeline over k-steps of 32: the fragments of the next k-step
  // are read while the MFMAs of the current one run.  Per block kt: read
  // (kt, 32) while multiplying (kt, 0); then wait for block kt + 1, meet at
  // the barrier (block kt is no longer read: its buffer takes block kt + NS),
  // and read (kt + 1, 0) while multiplying (kt, 32).  Blocks kt + 1 ..
  // kt + NS - 1 are in flight while block kt is multiplied.
  for (int b = 0; b < NS - 1 && b < nk; ++b) issue(b, b);
  wait_blocks<NS, QA + QB>(min(nk - 1, NS - 2));
  stage_barrier();
  if (K < BK) zero_tail(lds, K);
  if (NS - 1 < nk) issue(NS - 1, NS - 1);
  u16x8_t f0a[FI], f0b[FJ], f1a[FI], f1b[FJ];
  read_frags(lds, 0, f0a, f0b);
  // one block; NEXT: block kt + 1 exists (TAIL: it is the last, possibly
  // partial one); the steady-state body (NEXT, not TAIL) has no branch
  // between its LDS reads and their MFMAs, so each wait covers only the
  // fragments it needs
  auto step = [&](int kt, auto next_c, auto tail_c) {
    constexpr bool NEXT = decltype(next_c)::value, TAIL = decltype(tail_c)::value;
    uint8_t* base = lds + (kt % NS) * STAGE;
    read_frags(base, 32, f1a, f1b);
    mma(f0a, f0b);
    interleave();
    if constexpr (NEXT) {
      wait_blocks<NS, QA + QB>(min(nk - 2 - kt, NS - 2));
      stage_barrier();
      uint8_t* next = lds + ((kt + 1) % NS) * STAGE;
      if constexpr (TAIL) {
        const int64_t left = K - (int64_t)(kt + 1) * BK;
        if (left < BK) zero_tail(next, left);
      }
      if (kt + NS < nk) issue(kt % NS, kt + NS);
      read_frags(next, 0, f0a, f0b);
    }
    mma(f1a, f1b);
    interleave();
  };
  using yes = std::true_type;
  using no = std::false_type;
  int kt = 0;
  for (; kt + 2 < nk; ++kt) step(kt, yes{}, no{});
  if (kt + 1 < nk) step(kt++, yes{}, yes{});
  step(kt, no{}, no{});
  if constexpr (!TARGET) {
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t row = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + e;
          const int64_t col = n0 + wn * 64 + j * 16 + (lane & 15);
          if (row < M && col < N) out[row * N + col] = acc[i][j][e];
        }
  } else {
    constexpr int CP = BN + 4;  // 64 rows x 132 floats = 33 KiB of the NS x 32 KiB
    float* ct = (float*)lds;
    const int er = tid >> 2, ec0 = (tid & 3) * 32;
    const bool vec_ok =
        (N & 7) == 0 && (((uintptr_t)target | (uintptr_t)out) & 15) == 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();  // the operand tiles (h = 0) or the last half are no longer read
      if (wm == h) {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
          for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              ct[(i * 16 + 4 * (lane >> 4) + e) * CP + wn * 64 + j * 16 + (lane & 15)] =
                  acc[i][j][e];
      }
      __syncthreads();
      const int64_t row = m0 + 64 * h + er;
      if (row < M) {
        const float* src = ct + er * CP + ec0;
        float* dst = out + row * N + n0 + ec0;
        const uint16_t* tp = target + row * N + n0 + ec0;
        const int64_t ncols = N - (n0 + ec0);
        if (vec_ok && ncols >= 32) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x4_t tw = *(const u32x4_t*)(tp + 8 * q);
            float4 v0 = *(const float4*)(src + 8 * q);
            float4 v1 = *(const float4*)(src + 8 * q + 4);
            v0.x -= __uint_as_float(tw[0] << 16);
            v0.y -= __uint_as_float(tw[0] & 0xFFFF0000u);
            v0.z -= __uint_as_float(tw[1] << 16);
            v0.w -= __uint_as_float(tw[1] & 0xFFFF0000u);
            v1.x -= __uint_as_float(tw[2] << 16);
            v1.y -= __uint_as_float(tw[2] & 0xFFFF0000u);
            v1.z -= __uint_as_float(tw[3] << 16);
            v1.w -= __uint_as_float(tw[3] & 0xFFFF0000u);
            *(float4*)(dst + 8 * q) = v0;
            *(float4*)(dst + 8 * q + 4) = v1;
          }
        } else {
          for (int q = 0; q < 32 && q < ncols; ++q) dst[q] = src[q] - bf16_bits_to_f32(tp[q]);
        }
      }
    }
  }
}

}  // namespace gemm
}  // namespace dust
