// dust_attention.hpp -- kernels of local scoring through a recomputed
// attention ("Dust: every token is a member of the population", section
// "What the released code actually does", step 4: the queries, keys or
// values of one block are jittered, only that block's causal attention is
// recomputed from its cached activations, and the change of its output is
// scored against the estimated error of that output, c_s = -<e_s, Delta o_s>).
//
// Included by dust_kernels.hip inside namespace dust, after the noise and
// wave-reduction helpers; it includes nothing itself.
//
// The recomputation is never done literally.  With the clean probabilities
// p_st of one head (causal softmax of <q_s, k_t> / sqrt(d)), its output o_s,
// and m0_s = <e_s, o_s>, each site's output change has a closed form that
// keeps the score at its own scale (no difference of two nearly equal
// attention outputs):
//   values:  Delta o_s = s_i sigma sum_t p_st a_t exactly, so
//            c_s = -s_i sigma sum_t p_st <e_s, a_t>;
//   keys:    the logits move by x_st = s_i sigma <q_s, a_t> / sqrt(d), the
//            new probabilities are p_st e^x_st / Z_s with Z_s = 1 + S1_s,
//            S1_s = sum_t p_st E_st, E = e^x - 1, and
//            c_s = -S2_s / (1 + S1_s), S2_s = sum_t B_st E_st,
//            B_st = p_st <e_s, v_t - o_s> (clean, shared by every draw);
//   queries: the same with x_st = s_i sigma <a_s, k_t> / sqrt(d).
// The score of token s sums c_s over the heads.  Per draw and head that is
// one T x T x d contraction with the noise as an operand (bf16 MFMA, the
// noise split hi + lo so that it keeps 16 significant bits), an element-wise
// pass over the T x T block and two row sums.
//
// Kernels, in launch order:
//   attn_probs_kernel   clean P and m0 (fp32 VALU, once per call)
//   attn_bmat_kernel    clean B (keys and queries)
//   attn_score_t_kernel keys and values: one workgroup per (sequence, head,
//                       block of 64 jittered tokens t, pair of noise
//                       vectors); the noise of its tokens is generated once,
//                       into registers as MFMA operands, and reused over
//                       every block of 64 scored tokens s >= t, whose
//                       partial row sums over its t go to `part`
//   attn_score_s_kernel queries: one workgroup per (sequence, head, block of
//                       64 jittered tokens s, pair of noise vectors); the
//                       noise of its s is generated once and every block of
//                       keys t <= s streams past it, the row sums staying in
//                       registers
//   attn_reduce_kernel  the partial sums added per (token, draw), the closed
//                       forms, the sum over heads, rho [T][K] and its mean
//                       over the draws
#pragma once

// ---------------------------------------------------------------------------
// Clean pass.  One workgroup per (sequence, head, block b of 64 rows s);
// thread (ty, tx) = (tid / 16, tid % 16) owns rows 4 ty + r (r < 4) and, of
// each 64-token key block, columns 4 tx + c (c < 4).  The contraction runs in
// chunks of 32 channels staged through LDS, in fp32.

constexpr int kAttnChunk = 32;

// Loads a [64][32] chunk of a bf16 [rows][D] array (rows r0 .., channels
// c0 ..) transposed into dst[k][row] as fp32; rows at or past `valid` are 0.
__device__ __forceinline__ void attn_load_chunk_t(const uint16_t* __restrict__ src, int64_t r0,
                                                  int valid, int D, int c0,
                                                  float (*dst)[64]) {
  const int row = threadIdx.x >> 2, k8 = (threadIdx.x & 3) * 8;
  u16x8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
  if (row < valid) v = *(const u16x8_t*)(src + (r0 + row) * D + c0 + k8);
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[k8 + e][row] = bf16_to_f32(v[e]);
}

// The same for a fp32 source.
__device__ __forceinline__ void attn_load_chunk_t(const float* __restrict__ src, int64_t r0,
                                                  int valid, int D, int c0,
                                                  float (*dst)[64]) {
  const int row = threadIdx.x >> 2, k8 = (threadIdx.x & 3) * 8;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
  if (row < valid) {
    a = *(const float4*)(src + (r0 + row) * D + c0 + k8);
    b = *(const float4*)(src + (r0 + row) * D + c0 + k8 + 4);
  }
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[k8 + e][row] = v[e];
}

// acc[r][c] += sum_k A[k][4 ty + r] B[k][4 tx + c] over one staged chunk.
__device__ __forceinline__ void attn_chunk_fma(const float (*A)[64], const float (*B)[64],
                                               int ty, int tx, float (&acc)[4][4]) {
#pragma unroll 8
  for (int k = 0; k < kAttnChunk; ++k) {
    const float4 a = *(const float4*)&A[k][4 * ty];
    const float4 b = *(const float4*)&B[k][4 * tx];
    const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(av[r], bv[c], acc[r][c]);
  }
}

// The same with A held as bf16 (the block's queries, exact in bf16).
__device__ __forceinline__ void attn_chunk_fma(const uint16_t (*A)[64], const float (*B)[64],
                                               int ty, int tx, float (&acc)[4][4]) {
#pragma unroll 8
  for (int k = 0; k < kAttnChunk; ++k) {
    const uint2 a = *(const uint2*)&A[k][4 * ty];
    const float4 b = *(const float4*)&B[k][4 * tx];
    const float av[4] = {__uint_as_float(a.x << 16), __uint_as_float(a.x & 0xFFFF0000u),
                         __uint_as_float(a.y << 16), __uint_as_float(a.y & 0xFFFF0000u)};
    const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(av[r], bv[c], acc[r][c]);
  }
}

// The logits <q_s, k_t> of the thread's 4 x 4 entries of the (b, j) block,
// q held transposed in qT (bf16), keys staged chunk by chunk through kT.
// Ends with a barrier (kT is free again).
template <int DH>
__device__ __forceinline__ void attn_logits(const uint16_t (*qT)[64], float (*kT)[64],
                                            const uint16_t* __restrict__ Ka, int64_t krow0,
                                            int kvalid, int D, int hc, int ty, int tx,
                                            float (&acc)[4][4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  for (int kc = 0; kc < DH; kc += kAttnChunk) {
    attn_load_chunk_t(Ka, krow0, kvalid, D, hc + kc, kT);
    __syncthreads();
    attn_chunk_fma(qT + kc, kT, ty, tx, acc);
    __syncthreads();
  }
}

// Clean probabilities, written to Pm, and m0_s = <e_s, o_s>.  LDS: the
// block's queries transposed (bf16), a staged key chunk (fp32), p of one
// key block transposed (fp32) and that block's values (bf16): 56 KB for
// d_head = 128.
template <int DH>
__global__ __launch_bounds__(256) void attn_probs_kernel(
    const uint16_t* __restrict__ Qa, const uint16_t* __restrict__ Ka,
    const uint16_t* __restrict__ Va, const float* __restrict__ E, int32_t L, int32_t Lp,
    int32_t nb, int32_t H, int32_t D, float scale, float* __restrict__ Pm,
    float* __restrict__ m0) {
  __shared__ __attribute__((aligned(16))) uint16_t qT[DH][64];
  __shared__ __attribute__((aligned(16))) float kT[kAttnChunk][64];
  __shared__ __attribute__((aligned(16))) float pT[64][64];  // p of one block, [t][s]
  __shared__ __attribute__((aligned(16))) uint16_t vt[64][DH];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int b = blockIdx.x % nb, sh = blockIdx.x / nb, h = sh % H, seq = sh / H;
  const int s0 = 64 * b, hc = h * DH;
  const int64_t row0 = (int64_t)seq * L;  // the sequence's first token
  const int svalid = min(64, L - s0);
  {
    // queries of the block, transposed: thread moves 8 channels of a row
    for (int c = tid; c < 64 * (DH / 8); c += 256) {
      const int row = c / (DH / 8), k8 = (c % (DH / 8)) * 8;
      u16x8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (row < svalid) v = *(const u16x8_t*)(Qa + (row0 + s0 + row) * D + hc + k8);
#pragma unroll
      for (int e = 0; e < 8; ++e) qT[k8 + e][row] = v[e];
    }
  }
  __syncthreads();

  // 1. row maxima and sums of exp, online over the key blocks
  float mx[4], z[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    mx[r] = -INFINITY;
    z[r] = 0.f;
  }
  float acc[4][4];
  for (int j = 0; j <= b; ++j) {
    const int t0 = 64 * j;
    attn_logits<DH>(qT, kT, Ka, row0 + t0, min(64, L - t0), D, hc, ty, tx, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = s0 + 4 * ty + r;
      float m_new = mx[r];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t = t0 + 4 * tx + c;
        if (t <= s && t < L && s < L) m_new = fmaxf(m_new, acc[r][c] * scale);
      }
      if (m_new == -INFINITY) continue;
      float zr = mx[r] == -INFINITY ? 0.f : z[r] * expf(mx[r] - m_new);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t = t0 + 4 * tx + c;
        if (t <= s && t < L && s < L) zr += expf(acc[r][c] * scale - m_new);
      }
      mx[r] = m_new;
      z[r] = zr;
    }
  }
  // combine over the 16 threads of a row group (lanes tx of one wave); the
  // butterfly leaves every lane with the same value
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float mo = __shfl_xor(mx[r], d), zo = __shfl_xor(z[r], d);
      const float mn = fmaxf(mx[r], mo);
      const float a = mx[r] == -INFINITY ? 0.f : z[r] * expf(mx[r] - mn);
      const float c = mo == -INFINITY ? 0.f : zo * expf(mo - mn);
      mx[r] = mn;
      z[r] = a + c;
    }
  }
  float rz[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rz[r] = z[r] > 0.f ? 1.f / z[r] : 0.f;

  // 2. p written out, and o_s = sum_t p_st v_t (thread: rows 4 ty + r,
  //    channels tx + 16 q)
  constexpr int NO = DH / 16;
  float o[4][NO];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < NO; ++q) o[r][q] = 0.f;
  const int64_t pbase = (int64_t)sh * Lp * Lp;
  for (int j = 0; j <= b; ++j) {
    const int t0 = 64 * j, tvalid = min(64, L - t0);
    attn_logits<DH>(qT, kT, Ka, row0 + t0, tvalid, D, hc, ty, tx, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = s0 + 4 * ty + r;
      float p[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int t = t0 + 4 * tx + c;
        p[c] = (t <= s && t < L && s < L) ? expf(acc[r][c] * scale - mx[r]) * rz[r] : 0.f;
        pT[4 * tx + c][4 * ty + r] = p[c];
      }
      *(float4*)(Pm + pbase + (int64_t)s * Lp + t0 + 4 * tx) = make_float4(p[0], p[1], p[2], p[3]);
    }
    for (int c = tid; c < 64 * (DH / 8); c += 256) {
      const int row = c / (DH / 8), k8 = (c % (DH / 8)) * 8;
      u16x8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (row < tvalid) v = *(const u16x8_t*)(Va + (row0 + t0 + row) * D + hc + k8);
      *(u16x8_t*)&vt[row][k8] = v;
    }
    __syncthreads();
    for (int t = 0; t < 64; ++t) {
      const float4 pr = *(const float4*)&pT[t][4 * ty];
      const float pv[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
      for (int q = 0; q < NO; ++q) {
        const float vv = bf16_to_f32(vt[t][tx + 16 * q]);
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r][q] = __builtin_fmaf(pv[r], vv, o[r][q]);
      }
    }
    __syncthreads();
  }

  // 3. m0_s = <e_s, o_s>, summed over the 16 threads of the row group
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int s = s0 + 4 * ty + r;
    float d = 0.f;
    if (s < L) {
      const float* er = E + (row0 + s) * D + hc;
#pragma unroll
      for (int q = 0; q < NO; ++q) d = __builtin_fmaf(er[tx + 16 * q], o[r][q], d);
    }
#pragma unroll
    for (int dd = 1; dd < 16; dd <<= 1) d += __shfl_xor(d, dd);
    if (tx == 0) m0[(int64_t)sh * Lp + s] = d;
  }
}

// B_st = p_st (<e_s, v_t> - m0_s) of one (s block b, t block j <= b); one
// workgroup per (sequence, head, b, j), the blocks above the diagonal exit.
template <int DH>
__global__ __launch_bounds__(256) void attn_bmat_kernel(
    const float* __restrict__ E, const uint16_t* __restrict__ Va, const float* __restrict__ Pm,
    const float* __restrict__ m0, int32_t L, int32_t Lp, int32_t nb, int32_t H, int32_t D,
    float* __restrict__ Bm) {
  __shared__ __attribute__((aligned(16))) float eT[kAttnChunk][64];
  __shared__ __attribute__((aligned(16))) float vT[kAttnChunk][64];
  const int j = blockIdx.x % nb, b = (blockIdx.x / nb) % nb, sh = blockIdx.x / (nb * nb);
  if (j > b) return;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int h = sh % H, seq = sh / H, hc = h * DH;
  const int s0 = 64 * b, t0 = 64 * j;
  const int64_t row0 = (int64_t)seq * L;
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  for (int kc = 0; kc < DH; kc += kAttnChunk) {
    attn_load_chunk_t(E, row0 + s0, min(64, L - s0), D, hc + kc, eT);
    attn_load_chunk_t(Va, row0 + t0, min(64, L - t0), D, hc + kc, vT);
    __syncthreads();
    attn_chunk_fma(eT, vT, ty, tx, acc);
    __syncthreads();
  }
  const int64_t pbase = (int64_t)sh * Lp * Lp;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int s = s0 + 4 * ty + r;
    const int64_t at = pbase + (int64_t)s * Lp + t0 + 4 * tx;
    const float4 p = *(const float4*)(Pm + at);
    const float mm = m0[(int64_t)sh * Lp + s];
    *(float4*)(Bm + at) = make_float4(p.x * (acc[r][0] - mm), p.y * (acc[r][1] - mm),
                                      p.z * (acc[r][2] - mm), p.w * (acc[r][3] - mm));
  }
}

// ---------------------------------------------------------------------------
// Scores.  Both score kernels hold the noise of 16 tokens per wave as MFMA
// operands (v_mfma_f32_16x16x32_bf16: lane l supplies row / column l % 16
// with the 8 contraction values of group l / 16, and holds D rows
// 4 (l / 16) + i, i < 4, of column l % 16): lane l generates, for its token,
// channels 32 ks + 8 (l / 16) + 0..7 of the head (two noise quads per ks),
// split hi + lo.  A workgroup takes kAttnNV noise vectors.

constexpr int kAttnNV = 2;

// e^x - 1 and e^-x - 1.  Below |x| = 1/4 from the Taylor series of e^x - 1
// split into its even part ev and odd part od (e^x - 1 = ev + od,
// e^-x - 1 = ev - od); the first terms left out, x^8 / 8! and x^9 / 9!, are
// below 2e-9 |x| there.  Elsewhere from the exponential, where e^x - 1 is
// at least 0.22 in size and loses no more than a few ulp.
__device__ __forceinline__ void attn_expm1_pair(float x, float& ep, float& em) {
  const float u = x * x;
  const float od =
      x * __builtin_fmaf(u, __builtin_fmaf(u, __builtin_fmaf(u, 1.f / 5040.f, 1.f / 120.f),
                                           1.f / 6.f),
                         1.f);
  const float ev = u * __builtin_fmaf(u, __builtin_fmaf(u, 1.f / 720.f, 1.f / 24.f), 0.5f);
  ep = ev + od;
  em = ev - od;
  if (fabsf(x) >= 0.25f) {
    ep = expf(x) - 1.f;
    em = expf(-x) - 1.f;
  }
}

// Eight bf16 values from four dwords (each holding two, the first in the low
// half), in order.
__device__ __forceinline__ u16x8_t attn_pack(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const gemm::u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(u16x8_t, v);
}

// The noise of token tg, channels hc + 32 ks + 8 g + 0..7 under noise index
// n, as hi and lo MFMA operands (zero when !valid).
template <int KS>
__device__ __forceinline__ void attn_noise_frags(bool valid, uint32_t n, uint32_t tg, int hc,
                                                 int g, NoiseKey key, u16x8_t (&hi)[KS],
                                                 u16x8_t (&lo)[KS]) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    uint32_t h0 = 0u, h1 = 0u, h2 = 0u, h3 = 0u, l0 = 0u, l1 = 0u, l2 = 0u, l3 = 0u;
    if (valid) {
      const uint32_t q = (uint32_t)(hc + 32 * ks + 8 * g) >> 2;
      float4 a, b;
      noise_quad_x2(q, n, q + 1, n, tg, key, a, b);
      gemm::split_pair(a.x, a.y, h0, l0);
      gemm::split_pair(a.z, a.w, h1, l1);
      gemm::split_pair(b.x, b.y, h2, l2);
      gemm::split_pair(b.z, b.w, h3, l3);
    }
    hi[ks] = attn_pack(h0, h1, h2, h3);
    lo[ks] = attn_pack(l0, l1, l2, l3);
  }
}

// Keys and values: the jittered tokens t are the MFMA rows.  Workgroup
// (unit, noise group): units are (t block j, sequence, head), j slowest so
// the longest rows of blocks start first, dealt to the 8 XCDs round-robin;
// the noise groups of one unit are consecutive on one XCD, so the P and B
// blocks they all read stay in that XCD's L2.  Wave w owns tokens
// 64 j + 16 w + [0, 16).  For every s block b >= j, lane l's D entries are
// (t = 64 j + 16 w + 4 (l / 16) + i, s = 64 b + 16 st + l % 16) for the four
// s tiles st; their partial row sums over the lane's t are summed over the
// lane groups by two halving steps (lane l then holds token s = 64 b + l)
// and over the waves through LDS, and written to
// part[sequence, head][j][sum][draw][s].
template <int SITE, int DH, int NV, bool ANTI>
__global__ __launch_bounds__(256) void attn_score_t_kernel(
    const uint16_t* __restrict__ Qa, const float* __restrict__ E, const float* __restrict__ Pm,
    const float* __restrict__ Bm, int32_t L, int32_t Lp, int32_t nb, int32_t n_seq, int32_t H,
    int32_t D, int32_t K, int32_t K_n, int32_t n_groups, float xscale, NoiseKey key,
    float* __restrict__ part) {
  constexpr int KS = DH / 32;
  constexpr bool KEY = SITE == kAttnKey;
  constexpr int M = KEY ? (ANTI ? 4 : 2) : 1;  // sums per (token, noise vector)
  constexpr int MM = NV * M;
  constexpr int NS = KEY ? 2 : 1;
  __shared__ float red[4][MM][64];
  const int lane = threadIdx.x & 63, w = wave_id(), g = lane >> 4, r16 = lane & 15;
  const int pos = (int)(blockIdx.x >> 3), xcd = (int)(blockIdx.x & 7);
  const int unit = xcd + 8 * (pos / n_groups), grp = pos % n_groups;
  const int shn = n_seq * H;
  if (unit >= nb * shn) return;
  const int j = unit / shn, sh = unit % shn, seq = sh / H, h = sh % H, hc = h * DH;
  const int64_t row0 = (int64_t)seq * L;

  const int tl = 64 * j + 16 * w + r16;
  u16x8_t ahi[NV][KS], alo[NV][KS];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int n = grp * NV + v;
    attn_noise_frags<KS>(tl < L && n < K_n, (uint32_t)n, (uint32_t)(row0 + tl), hc, g, key,
                         ahi[v], alo[v]);
  }

  const int64_t pbase = (int64_t)sh * Lp * Lp;
  const int tcol = 64 * j + 16 * w + 4 * g;
  for (int b = j; b < nb; ++b) {
    const int s0 = 64 * b;
    float4 pv[4], bv[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int64_t at = pbase + (int64_t)(s0 + 16 * st + r16) * Lp + tcol;
      pv[st] = *(const float4*)(Pm + at);
      if constexpr (KEY) bv[st] = *(const float4*)(Bm + at);
    }
    f32x4_t acc[NV][4];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int st = 0; st < 4; ++st) acc[v][st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int sl = s0 + 16 * st + r16;
        const int64_t ro = (row0 + sl) * D + hc + 32 * ks + 8 * g;
        if constexpr (KEY) {
          u16x8_t o = {0, 0, 0, 0, 0, 0, 0, 0};
          if (sl < L) o = *(const u16x8_t*)(Qa + ro);
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            acc[v][st] = gemm::mfma16(ahi[v][ks], o, acc[v][st]);
            acc[v][st] = gemm::mfma16(alo[v][ks], o, acc[v][st]);
          }
        } else {
          float4 e0 = make_float4(0.f, 0.f, 0.f, 0.f), e1 = e0;
          if (sl < L) {
            e0 = *(const float4*)(E + ro);
            e1 = *(const float4*)(E + ro + 4);
          }
          uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
          gemm::split_pair(e0.x, e0.y, h0, l0);
          gemm::split_pair(e0.z, e0.w, h1, l1);
          gemm::split_pair(e1.x, e1.y, h2, l2);
          gemm::split_pair(e1.z, e1.w, h3, l3);
          const u16x8_t oh = attn_pack(h0, h1, h2, h3);
          const u16x8_t ol = attn_pack(l0, l1, l2, l3);
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            acc[v][st] = gemm::mfma16(ahi[v][ks], oh, acc[v][st]);
            acc[v][st] = gemm::mfma16(alo[v][ks], oh, acc[v][st]);
            acc[v][st] = gemm::mfma16(ahi[v][ks], ol, acc[v][st]);
          }
        }
      }
    }
    float vals[4 * MM];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const float pp[4] = {pv[st].x, pv[st].y, pv[st].z, pv[st].w};
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        if constexpr (KEY) {
          const float bb[4] = {bv[st].x, bv[st].y, bv[st].z, bv[st].w};
          float s1p = 0.f, s2p = 0.f, s1m = 0.f, s2m = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float ep, em;
            attn_expm1_pair(xscale * acc[v][st][i], ep, em);
            s1p = __builtin_fmaf(pp[i], ep, s1p);
            s2p = __builtin_fmaf(bb[i], ep, s2p);
            if constexpr (ANTI) {
              s1m = __builtin_fmaf(pp[i], em, s1m);
              s2m = __builtin_fmaf(bb[i], em, s2m);
            }
          }
          vals[st * MM + v * M + 0] = s1p;
          vals[st * MM + v * M + 1] = s2p;
          if constexpr (ANTI) {
            vals[st * MM + v * M + 2] = s1m;
            vals[st * MM + v * M + 3] = s2m;
          }
        } else {
          float sp = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) sp = __builtin_fmaf(pp[i], acc[v][st][i], sp);
          vals[st * MM + v] = sp;
        }
      }
    }
    halve<2 * MM, 32, true>(vals, lane);
    halve<MM, 16, true>(vals, lane);
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) red[w][mm][lane] = vals[mm];
    __syncthreads();
    for (int o = threadIdx.x; o < MM * 64; o += 256) {
      const int mm = o >> 6, sl = o & 63, v = mm / M, m = mm % M;
      const int n = grp * NV + v;
      if (n >= K_n) continue;
      const float tot = red[0][mm][sl] + red[1][mm][sl] + red[2][mm][sl] + red[3][mm][sl];
      // (sum, draw): keys S1, S2 of draw n, or of draws 2n (+) and 2n+1 (-);
      // values the signed sum of draw n, or +S for 2n and -S for 2n+1
      const int type = KEY ? (m & 1) : 0;
      const int draw = ANTI ? 2 * n + (m >> 1) : n;
      const int64_t at = ((((int64_t)sh * nb + j) * NS + type) * K + draw) * Lp + s0 + sl;
      part[at] = tot;
      if constexpr (!KEY && ANTI) part[at + Lp] = -tot;
    }
    __syncthreads();
  }
}

// Queries: the jittered tokens s are the MFMA columns.  Workgroup (unit,
// noise group): units are (s block b, sequence, head), the last blocks (the
// longest rows) first; wave w owns tokens 64 b + 16 w + [0, 16).  For every
// key block j <= b, lane l's D entries are (t = 64 j + 16 tt + 4 (l / 16) + i,
// s = 64 b + 16 w + l % 16) for the four t tiles tt; the lane's row sums
// accumulate over every block and are summed over the lane groups at the
// end, into part[sequence, head][0][sum][draw][s].
template <int DH, int NV, bool ANTI>
__global__ __launch_bounds__(256) void attn_score_s_kernel(
    const uint16_t* __restrict__ Ka, const float* __restrict__ Pm, const float* __restrict__ Bm,
    int32_t L, int32_t Lp, int32_t nb, int32_t n_seq, int32_t H, int32_t D, int32_t K,
    int32_t K_n, int32_t n_groups, float xscale, NoiseKey key, float* __restrict__ part) {
  constexpr int KS = DH / 32;
  constexpr int M = ANTI ? 4 : 2;
  constexpr int MM = NV * M;
  const int lane = threadIdx.x & 63, w = wave_id(), g = lane >> 4, r16 = lane & 15;
  const int pos = (int)(blockIdx.x >> 3), xcd = (int)(blockIdx.x & 7);
  const int unit = xcd + 8 * (pos / n_groups), grp = pos % n_groups;
  const int shn = n_seq * H;
  if (unit >= nb * shn) return;
  const int b = nb - 1 - unit / shn, sh = unit % shn, seq = sh / H, h = sh % H, hc = h * DH;
  const int64_t row0 = (int64_t)seq * L;

  const int sl = 64 * b + 16 * w + r16;
  u16x8_t ahi[NV][KS], alo[NV][KS];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int n = grp * NV + v;
    attn_noise_frags<KS>(sl < L && n < K_n, (uint32_t)n, (uint32_t)(row0 + sl), hc, g, key,
                         ahi[v], alo[v]);
  }
  float S[MM];
#pragma unroll
  for (int mm = 0; mm < MM; ++mm) S[mm] = 0.f;
  const int64_t prow = (int64_t)sh * Lp * Lp + (int64_t)sl * Lp;
  for (int j = 0; j <= b; ++j) {
    const int t0 = 64 * j;
    float4 pv[4], bv[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int64_t at = prow + t0 + 16 * tt + 4 * g;
      pv[tt] = *(const float4*)(Pm + at);
      bv[tt] = *(const float4*)(Bm + at);
    }
    f32x4_t acc[NV][4];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[v][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int t = t0 + 16 * tt + r16;
        u16x8_t kf = {0, 0, 0, 0, 0, 0, 0, 0};
        if (t < L) kf = *(const u16x8_t*)(Ka + (row0 + t) * D + hc + 32 * ks + 8 * g);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          acc[v][tt] = gemm::mfma16(kf, ahi[v][ks], acc[v][tt]);
          acc[v][tt] = gemm::mfma16(kf, alo[v][ks], acc[v][tt]);
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const float pp[4] = {pv[tt].x, pv[tt].y, pv[tt].z, pv[tt].w};
      const float bb[4] = {bv[tt].x, bv[tt].y, bv[tt].z, bv[tt].w};
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float ep, em;
          attn_expm1_pair(xscale * acc[v][tt][i], ep, em);
          S[v * M + 0] = __builtin_fmaf(pp[i], ep, S[v * M + 0]);
          S[v * M + 1] = __builtin_fmaf(bb[i], ep, S[v * M + 1]);
          if constexpr (ANTI) {
            S[v * M + 2] = __builtin_fmaf(pp[i], em, S[v * M + 2]);
            S[v * M + 3] = __builtin_fmaf(bb[i], em, S[v * M + 3]);
          }
        }
    }
  }
#pragma unroll
  for (int mm = 0; mm < MM; ++mm) {
    S[mm] += __shfl_xor(S[mm], 16);
    S[mm] += __shfl_xor(S[mm], 32);
  }
  if (g == 0) {
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) {
      const int v = mm / M, m = mm % M, n = grp * NV + v;
      if (n >= K_n) continue;
      const int type = m & 1;
      const int draw = ANTI ? 2 * n + (m >> 1) : n;
      part[(((int64_t)sh * 2 + type) * K + draw) * Lp + sl] = S[mm];
    }
  }
}

// rho[t][i] = sum over heads of the closed form from the partial sums
// (keys, queries: -S2 / (1 + S1); values: -sigma S) and mean[t] its mean
// over the draws.  One workgroup per (sequence, block of 64 tokens); thread
// (s, ig) = (tid % 64, tid / 64) forms draws ig + 4 r of each chunk of 64,
// which go through LDS to rows of rho; the mean adds the draws in order.
template <int SITE>
__global__ __launch_bounds__(256) void attn_reduce_kernel(
    const float* __restrict__ part, int32_t L, int32_t Lp, int32_t nb, int32_t H, int32_t K,
    int32_t n_slots, float sigma, float* __restrict__ rho, float* __restrict__ mean) {
  constexpr int NS = SITE == kAttnValue ? 1 : 2;
  __shared__ float cb[64][65];
  const int seq = blockIdx.x / nb, b = blockIdx.x % nb;
  const int sl = threadIdx.x & 63, ig = threadIdx.x >> 6;
  const int s = 64 * b + sl;
  const bool sval = s < L;
  const int slots = SITE == kAttnQuery ? 1 : b + 1;
  const int64_t slot_stride = (int64_t)NS * K * Lp, type_stride = (int64_t)K * Lp;
  float macc = 0.f;
  for (int i0 = 0; i0 < K; i0 += 64) {
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
      const int ic = ig + 4 * r, i = i0 + ic;
      float c = 0.f;
      if (sval && i < K) {
        for (int h = 0; h < H; ++h) {
          const int64_t base =
              (((int64_t)(seq * H + h) * n_slots) * NS * K + i) * Lp + s;
          float s1 = 0.f, s2 = 0.f;
          for (int jj = 0; jj < slots; ++jj) {
            s1 += part[base + jj * slot_stride];
            if constexpr (NS == 2) s2 += part[base + jj * slot_stride + type_stride];
          }
          c += SITE == kAttnValue ? -sigma * s1 : -s2 / (1.f + s1);
        }
      }
      cb[sl][ic] = c;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int row = e >> 6, col = e & 63;
      if (64 * b + row < L && i0 + col < K)
        rho[((int64_t)seq * L + 64 * b + row) * K + i0 + col] = cb[row][col];
    }
    if (ig == 0)
      for (int col = 0; col < 64 && i0 + col < K; ++col) macc += cb[sl][col];
    __syncthreads();
  }
  if (ig == 0 && sval) mean[(int64_t)seq * L + s] = macc / (float)K;
}
