// dust_gemm.hpp -- LDS-tiled bf16 MFMA GEMM for the two dense contractions
// of the estimator on gfx950, both in "NT" form C[m][n] = sum_k A[m][k] B[n][k]
// with the contraction axis k contiguous in HBM:
//   base   delta[t][c] = sum_k X[t][k] W[c][k] - target[t][c]
//   outer  G[c][i] = sum_t gT[c][t] XT[i][t], gT = gT_hi + gT_lo (bf16 split
//          of fp32 g, written by transpose_kernel), XT = X transposed.
//
// A workgroup of 256 threads (4 waves in a 2x2 grid) computes a BM x BN tile;
// each wave a (BM/2) x (BN/2) block of 16x16 MFMA tiles
// (v_mfma_f32_16x16x32_bf16: lane l supplies row l % 16 of A and column
// l % 16 of B with the 8 contraction values of group l / 16, and holds D rows
// 4 (l / 16) + 0..3 of column l % 16).  Operand tiles are staged in LDS with a
// padded row of BK + 8 bf16, so every fragment is one ds_read_b128.  LDS is
// double buffered and several k-tiles are in flight from HBM in registers
// (see nt_gemm_kernel), so each step needs a single barrier and the load
// latency is hidden behind the MFMAs of the tiles before it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dust {
namespace gemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));


__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// A (rows x BK) tile of a row-major bf16 matrix whose rows are contiguous
// along k: element (r, k) at src[r * ld + k].  Each thread moves
// rows * BK / 8 / 256 chunks of 8 values.  VEC (ld and kmax multiples of 8,
// 16-byte aligned rows): every chunk is wholly inside or outside the matrix,
// so it is one unconditional 16-byte load from a clamped address, with no
// branch; the out-of-range chunks are zeroed when written to LDS, so nothing
// waits for a load before the store that needs it.  Otherwise element-wise
// guarded loads.
// LDS row padding in bf16 elements (-DDUST_LDS_PAD=n at build time).
#ifndef DUST_LDS_PAD
#define DUST_LDS_PAD 16
#endif

template <int ROWS, int BK, bool VEC>
struct KMajorTile {
  static constexpr int LDK = BK + DUST_LDS_PAD;  // padded LDS row, in bf16 elements
  static constexpr int kChunks = ROWS * BK / 8 / 256;
  u16x8_t reg[kChunks];
  bool in_range[kChunks];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int64_t ld,
                                       int64_t rows, int64_t kmax, int tid, int64_t r0,
                                       int64_t k0) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
      const int64_t r = r0 + row, k = k0 + kc;
      if (VEC) {
        const bool ok = (r < rows) && (k < kmax);
        reg[i] = *(const u16x8_t*)(src + (ok ? r * ld + k : 0));
        in_range[i] = ok;
      } else {
        u16x8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < rows) {
          const uint16_t* p = src + r * ld + k;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (k + j < kmax) v[j] = p[j];
        }
        reg[i] = v;
        in_range[i] = true;
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
    const u16x8_t zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int c = tid + 256 * i;
      const int row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
      *(u16x8_t*)(lds + row * LDK + kc) = in_range[i] ? reg[i] : zero;
    }
  }
};

__device__ __forceinline__ f32x4_t mfma16(u16x8_t a, u16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Work mapping.  The dispatcher deals workgroups to the 8 XCDs round-robin
// (workgroup b runs on XCD b % 8), and each XCD has its own L2.  So the work
// items (split, m-tile, n-tile) are linearised with n fastest, then m, then
// split, and XCD x takes the contiguous range [x * per_xcd, (x+1) * per_xcd):
// the workgroups resident on one XCD at a time share their A row-blocks
// (reused across n) and the B blocks of their split (few enough to stay in
// that L2).  grid = 8 * per_xcd; items past the end exit at once.
struct TileWork {
  int split, m_tile, n_tile;
  bool valid;
};
__device__ __forceinline__ TileWork map_tile(int tiles_m, int tiles_n, int splits, int per_xcd) {
  const int b = blockIdx.x;
  const int wid = (b % 8) * per_xcd + b / 8;
  TileWork w;
  w.valid = wid < tiles_m * tiles_n * splits;
  w.n_tile = wid % tiles_n;
  w.m_tile = (wid / tiles_n) % tiles_m;
  w.split = wid / (tiles_n * tiles_m);
  return w;
}

// C = A B^T over k in [k_begin, k_end).  DUAL: A is the sum of two bf16
// matrices (hi + lo), multiplied separately into the same accumulator.
// EPI_DELTA: out[m][n] = C - target[m][n] (bf16 target), else
// out[split][m][n] = C.  When at != nullptr, the workgroups of n-tile 0 also
// write A transposed, at[k][m] for m < ld_at (ld_at a multiple of 8; rows of
// A past M are zeros), from the A tiles they already hold in LDS.
// The split partials are summed by a separate fixed-order kernel.
//
// Software pipeline: S register stages hold the next S k-tiles in flight
// from HBM.  Step kt multiplies tile kt from LDS buffer kt & 1, writes tile
// kt+1 from its register stage into the other LDS buffer, refills that stage
// with tile kt+1+S, and ends with one barrier.  The k loop is unrolled by S so
// every stage index is a compile-time constant.
template <int BM, int BN, int BK, bool DUAL, bool EPI_DELTA, int S, bool VEC>
__global__ __launch_bounds__(256) void nt_gemm_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ A2,
    const uint16_t* __restrict__ B, int64_t lda, int64_t ldb, int32_t M, int32_t N,
    int64_t K, int32_t tiles_m, int32_t tiles_n, int32_t splits, int32_t per_xcd,
    int64_t k_per_split, const uint16_t* __restrict__ target, float* __restrict__ out,
    uint16_t* __restrict__ at, int64_t ld_at) {
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 16, TN = WN / 16;
  constexpr int LDK = BK + DUST_LDS_PAD;
  constexpr int A_SZ = BM * LDK, B_SZ = BN * LDK;
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][A_SZ];
  __shared__ __attribute__((aligned(16))) uint16_t lds_a2[DUAL ? 2 : 1][DUAL ? A_SZ : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lds_b[2][B_SZ];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const TileWork work = map_tile(tiles_m, tiles_n, splits, per_xcd);
  if (!work.valid) return;
  const int split = work.split;
  const int64_t m0 = (int64_t)work.m_tile * BM;
  const int64_t n0 = (int64_t)work.n_tile * BN;
  const int64_t k_begin = (int64_t)split * k_per_split;
  const int64_t k_end = min(K, k_begin + k_per_split);
  const int nk = (int)((k_end - k_begin + BK - 1) / BK);
  static_assert(S % 2 == 0, "the LDS double buffer is indexed by the stage parity");

  KMajorTile<BM, BK, VEC> ta[S], ta2[DUAL ? S : 1];
  KMajorTile<BN, BK, VEC> tb[S];
  auto load_stage = [&](int st, int kt) {
    const int64_t k0 = k_begin + (int64_t)kt * BK;
    ta[st].load(A, lda, M, k_end, tid, m0, k0);
    if (DUAL) ta2[DUAL ? st : 0].load(A2, lda, M, k_end, tid, m0, k0);
    tb[st].load(B, ldb, N, k_end, tid, n0, k0);
  };
  auto store_stage = [&](int st, int buf) {
    ta[st].store(lds_a[buf], tid);
    if (DUAL) ta2[DUAL ? st : 0].store(lds_a2[DUAL ? buf : 0], tid);
    tb[st].store(lds_b[buf], tid);
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Small tiles: fetch the epilogue's target values now, so their latency
  // hides behind the k loop (a few registers per lane).
  constexpr bool kPrefetchTarget = EPI_DELTA && TM * TN <= 4;
  uint16_t tgt[kPrefetchTarget ? TM : 1][kPrefetchTarget ? TN : 1][4];
  if constexpr (kPrefetchTarget) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t row = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + e;
          const int64_t col = n0 + wn * WN + j * 16 + (lane & 15);
          // unconditional load from a clamped address (no branch, no wait);
          // entries outside the matrix are never stored
          const int64_t rr = row < M ? row : M - 1, cc = col < N ? col : N - 1;
          tgt[i][j][e] = target[rr * N + cc];
        }
  }

  // Branch-free pipeline: the tile count is padded to a multiple of S (the
  // padding tiles lie past k_end, so they load from a clamped address and
  // store zeros), so the compiler sees one straight-line body per S steps
  // and keeps S tiles of loads in flight instead of waiting at branches.
  const int nk_pad = ((nk + S - 1) / S) * S;
#pragma unroll
  for (int st = 0; st < S; ++st) load_stage(st, st);
  store_stage(0, 0);
  load_stage(0, S);
  __syncthreads();

  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int kt0 = 0; kt0 < nk_pad; kt0 += S) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int kt = kt0 + s;
      const int cur = s & 1;  // S is even, so kt & 1 == s & 1
#pragma unroll
      for (int ks = 0; ks < BK; ks += 32) {
        u16x8_t af[TM], af2[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          af[i] = *(const u16x8_t*)(&lds_a[cur][(wm * WM + i * 16 + fr) * LDK + ks + fk]);
          if (DUAL)
            af2[i] = *(const u16x8_t*)(
                &lds_a2[DUAL ? cur : 0][(wm * WM + i * 16 + fr) * LDK + ks + fk]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[j] = *(const u16x8_t*)(&lds_b[cur][(wn * WN + j * 16 + fr) * LDK + ks + fk]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
            if (DUAL) acc[i][j] = mfma16(af2[i], bfr[j], acc[i][j]);
          }
      }
      if (at != nullptr && work.n_tile == 0 && kt < nk) {
        // A tile [BM][BK] of buffer cur -> at rows k0..k0+BK-1, 8 m per chunk
        const int64_t k0 = k_begin + (int64_t)kt * BK;
#pragma unroll
        for (int rep = 0; rep < BM * BK / 8 / 256; ++rep) {
          const int c = tid + 256 * rep;
          const int kk = c % BK, mseg = (c / BK) * 8;
          const int64_t m = m0 + mseg, k = k0 + kk;
          if (k < k_end && m < ld_at) {
            u16x8_t v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = lds_a[cur][(mseg + e) * LDK + kk];
            *(u16x8_t*)(at + k * ld_at + m) = v;
          }
        }
      }
      const int nxt = (s + 1) % S;
      store_stage(nxt, cur ^ 1);
      load_stage(nxt, kt + 1 + S);
      __syncthreads();
    }
  }
  float* dst = EPI_DELTA ? out : out + (int64_t)split * M * N;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + e;
        const int64_t col = n0 + wn * WN + j * 16 + (lane & 15);
        if (row < M && col < N) {
          const int64_t o = row * N + col;
          if constexpr (kPrefetchTarget)
            dst[o] = acc[i][j][e] - bf16_bits_to_f32(tgt[kPrefetchTarget ? i : 0][kPrefetchTarget ? j : 0][e]);
          else if (EPI_DELTA)
            dst[o] = acc[i][j][e] - bf16_bits_to_f32(target[o]);
          else
            dst[o] = acc[i][j][e];
        }
      }
}

// ---------------------------------------------------------------------------
// Transposes for the outer product, 64x64 tiles through LDS, 16-byte
// accesses on both sides.  src [rows][cols] -> dst [cols][ld_dst] with
// ld_dst >= rows (a multiple of 8); padding entries rows..ld_dst-1 are
// written as zeros.
//   SPLIT: src fp32, dst_hi = bf16(src), dst_lo = bf16(src - hi)
//   else : src bf16, dst_hi = src
// VEC: cols a multiple of 8 and src 16-byte aligned (vector loads).
// grid = ceil(ld_dst / 64) * ceil(cols / 64).

template <bool SPLIT, bool VEC>
__global__ __launch_bounds__(256) void transpose_kernel(const void* __restrict__ src,
                                                        int32_t rows, int32_t cols,
                                                        int64_t ld_dst, int32_t tiles_c,
                                                        uint16_t* __restrict__ dst_hi,
                                                        uint16_t* __restrict__ dst_lo) {
  __shared__ float tile[64][65];
  const int tid = threadIdx.x;
  const int tr = blockIdx.x / tiles_c, tc = blockIdx.x % tiles_c;
  const int64_t r0 = (int64_t)tr * 64, c0 = (int64_t)tc * 64;
  // load: thread -> 8 consecutive columns of rows (tid / 8) + 32 j
  {
    const int cc = (tid % 8) * 8;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int rr = tid / 8 + 32 * j;
      const int64_t r = r0 + rr, c = c0 + cc;
      float v[8];
      if (VEC && r < rows && c + 8 <= cols) {
        if (SPLIT) {
          const float4 a = *(const float4*)((const float*)src + r * cols + c);
          const float4 b = *(const float4*)((const float*)src + r * cols + c + 4);
          v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
          v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
          const u16x8_t a = *(const u16x8_t*)((const uint16_t*)src + r * cols + c);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = bf16_bits_to_f32(a[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[e] = 0.f;
          if (r < rows && c + e < cols)
            v[e] = SPLIT ? ((const float*)src)[r * cols + c + e]
                         : bf16_bits_to_f32(((const uint16_t*)src)[r * cols + c + e]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[rr][cc + e] = v[e];
    }
  }
  __syncthreads();
  // store: thread -> output row c = tid / 4 (a source column), 16 source
  // rows starting at (tid % 4) * 16, as two 8-value chunks
  {
    const int cc = tid / 4, rseg = (tid % 4) * 16;
    const int64_t c = c0 + cc;
    if (c < cols) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t r = r0 + rseg + 8 * h;  // multiple of 8
        if (r < ld_dst) {
          u16x8_t hv, lv;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = tile[rseg + 8 * h + e][cc];  // zero where r >= rows
            const uint16_t hb = f32_to_bf16_rne(v);
            hv[e] = hb;
            lv[e] = f32_to_bf16_rne(v - bf16_bits_to_f32(hb));
          }
          *(u16x8_t*)(dst_hi + c * ld_dst + r) = hv;
          if (SPLIT) *(u16x8_t*)(dst_lo + c * ld_dst + r) = lv;
        }
      }
    }
  }
}

}  // namespace gemm
}  // namespace dust
