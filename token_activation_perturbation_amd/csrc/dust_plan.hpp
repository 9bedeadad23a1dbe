// dust_plan.hpp -- host-only launch plan and workspace layout of dust_estimate.
//
// Pure C++ (no HIP types, no HIP calls): dust_workspace_bytes and
// dust_validate use it on machines without a GPU, and dust_estimate uses the
// very same plan to carve the workspace and size its launches.
#pragma once

#include <cstddef>
#include <cstdint>

namespace dust {

// Noise vectors handled per unrolled batch inside the noise kernels.
constexpr int kNoiseBatch = 16;
// Waves the noise kernels are split into (256 CUs x 4 SIMDs x 16); a build
// may override it with -DDUST_TARGET_WAVES=n.
#ifndef DUST_TARGET_WAVES
#define DUST_TARGET_WAVES 16384
#endif
constexpr int64_t kTargetWaves = DUST_TARGET_WAVES;
// Workgroups the outer product's token split aims for (-DDUST_OUTER_WORKGROUPS).
#ifndef DUST_OUTER_WORKGROUPS
#define DUST_OUTER_WORKGROUPS 2048
#endif
// ... keeping at least this many tokens per split (-DDUST_OUTER_MIN_TOKENS).
#ifndef DUST_OUTER_MIN_TOKENS
#define DUST_OUTER_MIN_TOKENS 512
#endif

// 128 x 128 GEMM tiles: the base GEMM takes them from this many tiles on
// (-DDUST_BIG_TILES_MIN); the outer product when its token splits of at
// least kBigOuterMinTokens give kBigOuterWorkgroups workgroups (three share
// a CU).
#ifndef DUST_BIG_TILES_MIN
#define DUST_BIG_TILES_MIN 512
#endif
#ifndef DUST_BIG_OUTER_WORKGROUPS
#define DUST_BIG_OUTER_WORKGROUPS 768
#endif
#ifndef DUST_BIG_OUTER_MIN_TOKENS
#define DUST_BIG_OUTER_MIN_TOKENS 1024
#endif
constexpr int64_t kBigTilesMin = DUST_BIG_TILES_MIN;
// The outer product on 128 x 256 tiles (outer_wide) where it takes 128 x 128
// tiles and the layer input has at least kWideOuterMinN channels; its token
// split aims for kWideOuterWorkgroups workgroups (two share a CU).
// -DDUST_WIDE_OUTER_MIN_N=n at build time (0 switches it off).
#ifndef DUST_WIDE_OUTER_MIN_N
#define DUST_WIDE_OUTER_MIN_N 512
#endif
#ifndef DUST_WIDE_OUTER_WORKGROUPS
#define DUST_WIDE_OUTER_WORKGROUPS 512
#endif
constexpr int64_t kWideOuterMinN = DUST_WIDE_OUTER_MIN_N;
constexpr int64_t kWideOuterWorkgroups = DUST_WIDE_OUTER_WORKGROUPS;
constexpr int64_t kBigOuterWorkgroups = DUST_BIG_OUTER_WORKGROUPS;
constexpr int64_t kBigOuterMinTokens = DUST_BIG_OUTER_MIN_TOKENS;

struct Plan {
  int64_t T = 0, d_in = 0, d_out = 0;
  int32_t K = 0, K_n = 0, antithetic = 0, dtype = 0;
  int32_t nq = 0;  // channel quads per token, ceil(d_out / 4)

  // jitter-loss kernel: one wave per (token, chunk of noise indices)
  int32_t jl_chunks = 1, jl_per_chunk = 0;
  // reweight kernel: one workgroup of rw_waves waves per token, the noise
  // indices split into rw_waves contiguous ranges of rw_per_wave
  int32_t rw_waves = 1, rw_per_wave = 0;
  // fused single-generation kernel (gamma = 0): one workgroup of fz_waves
  // waves per token, the noise indices split into ranges of fz_per_wave
  int32_t fz_waves = 1, fz_per_wave = 0;
  // base GEMM: 128 x 128 tiles (base_big) when the problem has enough of
  // them to fill the chip twice over, else 64 x 64
  int32_t base_big = 0;
  // outer product: 128 x 128 output tiles (outer_big) or 64 x 64; split of
  // the token (contraction) axis into outer_split ranges of outer_tokens
  int32_t outer_big = 0;
  int32_t outer_wide = 0;  // 128 x 256 tiles (implies outer_big)
  int32_t outer_split = 1;
  int64_t outer_tokens = 0;  // tokens per split (multiple of 64)

  // workspace byte offsets (each 256-byte aligned) and total
  size_t off_delta = 0, off_P = 0, off_Q = 0, off_rho = 0, off_mean = 0,
         off_wgt = 0, off_g = 0, off_gpart = 0,
         off_rloc = 0, off_carry = 0, total = 0;
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Returns false when the sizes cannot be planned (non-positive sizes, K < 2,
// odd K with antithetic pairs, or sizes past the kernels' 32-bit indices).
inline bool make_plan(int64_t T, int64_t d_in, int64_t d_out, int32_t K,
                      int32_t antithetic, int32_t dtype, Plan* p) {
  if (T <= 0 || d_in <= 0 || d_out <= 0 || K < 2) return false;
  if (antithetic && (K % 2) != 0) return false;
  // T below 2^24 keeps every grid (up to 256 threads per token) under 2^32
  // threads; the noise counter words themselves would allow 2^32.
  if (T >= (int64_t(1) << 24) || d_out >= (int64_t(1) << 31) ||
      d_in >= (int64_t(1) << 31))
    return false;
  Plan q;
  q.T = T;
  q.d_in = d_in;
  q.d_out = d_out;
  q.K = K;
  q.antithetic = antithetic ? 1 : 0;
  q.K_n = antithetic ? K / 2 : K;
  q.dtype = dtype;
  q.nq = (int32_t)ceil_div(d_out, 4);
  if ((int64_t)T * q.K_n >= (int64_t(1) << 40)) return false;

  const int64_t batches = ceil_div(q.K_n, kNoiseBatch);
  // jitter-loss: enough (token, chunk) waves to fill the chip
  int64_t chunks = ceil_div(kTargetWaves, T);
  if (chunks > batches) chunks = batches;
  if (chunks < 1) chunks = 1;
  q.jl_per_chunk = (int32_t)(ceil_div(batches, chunks) * kNoiseBatch);
  q.jl_chunks = (int32_t)ceil_div(q.K_n, q.jl_per_chunk);
  // reweight: 1, 2 or 4 waves per token
  int64_t waves = ceil_div(kTargetWaves, T);
  if (waves > 4) waves = 4;
  if (waves > batches) waves = batches;
  if (waves == 3) waves = 2;
  if (waves < 1) waves = 1;
  q.rw_per_wave = (int32_t)(ceil_div(batches, waves) * kNoiseBatch);
  q.rw_waves = (int32_t)ceil_div(q.K_n, q.rw_per_wave);
  // fused: same wave budget; ranges are whole multiples of 4 noise indices
  int64_t fw = ceil_div(kTargetWaves, T);
  if (fw > 4) fw = 4;
  if (fw > ceil_div(q.K_n, 4)) fw = ceil_div(q.K_n, 4);
  if (fw == 3) fw = 2;
  if (fw < 1) fw = 1;
  q.fz_per_wave = (int32_t)(ceil_div(ceil_div(q.K_n, fw), 4) * 4);
  q.fz_waves = (int32_t)ceil_div(q.K_n, q.fz_per_wave);
  // base GEMM: 128 x 128 tiles once there are at least kBigTilesMin of them
  // (two workgroups per CU share it; fewer would leave CUs idle)
  const bool aligned8 = (d_in % 8) == 0 && (d_out % 8) == 0;
  q.base_big = (aligned8 && ceil_div(T, 128) * ceil_div(d_out, 128) >= kBigTilesMin) ? 1 : 0;
  // outer product: 128 x 128 tiles when, with splits of at least
  // kBigOuterMinTokens tokens, there are kBigOuterWorkgroups of them;
  // else 64 x 64 tiles, split until ~DUST_OUTER_WORKGROUPS workgroups with
  // >= DUST_OUTER_MIN_TOKENS tokens per split (measured best on MI355X for
  // 512-wide layers)
  const int64_t tiles128 = ceil_div(d_out, 128) * ceil_div(d_in, 128);
  q.outer_big =
      (aligned8 && tiles128 * ceil_div(T, kBigOuterMinTokens) >= kBigOuterWorkgroups) ? 1 : 0;
  q.outer_wide = (q.outer_big && kWideOuterMinN > 0 && d_in >= kWideOuterMinN) ? 1 : 0;
  const int64_t tiles = q.outer_wide  ? ceil_div(d_out, 128) * ceil_div(d_in, 256)
                        : q.outer_big ? tiles128
                                      : ceil_div(d_out, 64) * ceil_div(d_in, 64);
  // the large tiles' grid is sized to fit one round of resident workgroups
  // (a second round that holds only a few would take nearly as long as the
  // first); the small tiles run many rounds
  int64_t split = q.outer_wide  ? kWideOuterWorkgroups / tiles
                  : q.outer_big ? kBigOuterWorkgroups / tiles
                                : ceil_div(DUST_OUTER_WORKGROUPS, tiles);
  const int64_t max_split =
      ceil_div(T, q.outer_big ? kBigOuterMinTokens : DUST_OUTER_MIN_TOKENS);
  if (split > max_split) split = max_split;
  if (split > 64) split = 64;
  if (split < 1) split = 1;
  q.outer_tokens = ceil_div(ceil_div(T, split), 64) * 64;
  q.outer_split = (int32_t)ceil_div(T, q.outer_tokens);

  size_t off = 0;
  auto take = [&off](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  q.off_delta = take(sizeof(float) * size_t(T) * size_t(d_out));
  q.off_P = take(sizeof(float) * size_t(T) * size_t(q.K_n));
  q.off_Q = take(sizeof(float) * size_t(T) * size_t(q.K_n));
  q.off_rho = take(sizeof(float) * size_t(T) * size_t(K));
  q.off_mean = take(sizeof(float) * size_t(T));
  q.off_wgt = take(sizeof(float) * size_t(T) * size_t(q.K_n));
  q.off_g = take(sizeof(float) * size_t(T) * size_t(d_out));
  q.off_gpart = take(q.outer_split > 1 ? sizeof(float) * size_t(q.outer_split) *
                                             size_t(d_out) * size_t(d_in)
                                       : 0);

  // chunked credit scan (gamma > 0, sequences of >= 2 tokens): the chunks'
  // own scans [T][K], and one head/carry per (sequence, 32-token chunk,
  // draw); (T / seq_len) * ceil(seq_len / 32) <= T / 2 chunks for any
  // seq_len >= 2
  q.off_rloc = take(sizeof(float) * size_t(T) * size_t(K));
  q.off_carry = take(sizeof(float) * size_t(ceil_div(T, 2)) * size_t(K));
  q.total = off;
  *p = q;
  return true;
}

// ---------------------------------------------------------------------------
// Single generation for gamma > 0 (the "chain" path): each sequence is walked
// in reverse token order once per chain (an antithetic pair, or one plain
// draw); one workgroup of kChainWaves waves per (sequence, group of
// kChainGroup chains), kChainPerWave chains per wave.  Every group writes,
// per token, its partial sum of R a ([groups][T][d_out] fp32) and for plain
// draws also its partial sums of a ([groups][T][d_out]) and of rho
// ([T][groups]), with the per-token credit mean M ([T]) after them; all of
// it is placed after the two-pass layout, so the chain path needs a larger
// workspace (dust_workspace_bytes_seq) and a call given only
// dust_workspace_bytes takes the two-pass path.  It is planned only where
// the chains fill the chip (sequences x chains >= kChainMinChains), the
// waves' rows fit the workgroup's LDS (d_out <= kChainMaxDout) and, for plain
// draws, a sequence's mean scan fits LDS (seq_len <= kChainMaxSeqLen).
#ifndef DUST_CHAIN_WAVES
#define DUST_CHAIN_WAVES 8
#endif
#ifndef DUST_CHAIN_PER_WAVE
#define DUST_CHAIN_PER_WAVE 2
#endif
constexpr int32_t kChainWaves = DUST_CHAIN_WAVES;      // -DDUST_CHAIN_WAVES=n
constexpr int32_t kChainPerWave = DUST_CHAIN_PER_WAVE;  // -DDUST_CHAIN_PER_WAVE=n (2 or 4)
constexpr int32_t kChainGroup = kChainWaves * kChainPerWave;
constexpr int64_t kChainMinChains = 2048;
constexpr int64_t kChainMaxDout = 1024;
constexpr int64_t kChainMaxSeqLen = 8192;

struct ChainPlan {
  bool ok = false;
  bool plain = false;     // plain draws (else antithetic pairs)
  int32_t groups = 0;     // chain groups per sequence, ceil(K_n / kChainGroup)
  int64_t n_seq = 0;      // sequences, T / seq_len
  size_t off_part = 0;    // partial sum of R a [groups][T][d_out] fp32
  size_t off_part_s = 0;  // plain: partial sum of a [groups][T][d_out] fp32
  size_t off_rsum = 0;    // plain: partial sum of rho [T][groups] fp32
  size_t off_mean = 0;    // plain: M_t [T] fp32
  size_t total = 0;       // workspace bytes of the chain path
};

inline ChainPlan make_chain_plan(const Plan& p, int64_t seq_len, float gamma) {
  ChainPlan c;
  if (!(gamma > 0.0f) || seq_len < 2 || p.T % seq_len != 0) return c;
  if (p.d_out > kChainMaxDout) return c;
  c.plain = !p.antithetic;
  if (c.plain && seq_len > kChainMaxSeqLen) return c;
  c.n_seq = p.T / seq_len;
  if (c.n_seq * p.K_n < kChainMinChains) return c;
  c.groups = (int32_t)ceil_div(p.K_n, kChainGroup);
  if (c.n_seq * c.groups >= (int64_t(1) << 31)) return c;
  const size_t rows = sizeof(float) * size_t(c.groups) * size_t(p.T) * size_t(p.d_out);
  c.off_part = align256(p.total);
  size_t end = align256(c.off_part + rows);
  if (c.plain) {
    c.off_part_s = end;
    c.off_rsum = align256(c.off_part_s + rows);
    c.off_mean = align256(c.off_rsum + sizeof(float) * size_t(c.groups) * size_t(p.T));
    end = align256(c.off_mean + sizeof(float) * size_t(p.T));
  }
  c.total = end;
  c.ok = true;
  return c;
}

// ---------------------------------------------------------------------------
// Embedding reassembly: G_E[v] = scale sum_{t: ids[t] = v} g[t], by a stable
// counting sort of the token positions by id (per-chunk histograms, their
// prefix sums over chunks, a scan of the totals, a placement pass), then a
// reduce-by-key over fixed tiles of the sorted order and a fix-up that sums
// the partials of the ids whose rows cross tiles.

// Sorted rows per reduce tile, histogram entries (chunks x V) allowed, and
// the largest V whose per-chunk histogram and run starts are kept in LDS
// (V + 1 ints and the kernels' static LDS within 64 KiB).
constexpr int32_t kReassembleTile = 32;
constexpr int64_t kHistCap = int64_t(1) << 22;
constexpr int64_t kLdsHistMaxV = 15360;

struct ReassemblyPlan {
  int64_t T = 0, V = 0, d = 0;
  int32_t n_chunks = 1;      // token chunks, one workgroup each (hist, place)
  int64_t chunk_tokens = 0;  // tokens per chunk (multiple of 256)
  int64_t n_tiles = 0;       // reduce tiles of kReassembleTile sorted rows
  int32_t col_chunks = 0;    // 256-column chunks of a row (64 lanes x 4)
  // byte offsets (each 256-byte aligned), relative to the plan's base, and
  // total: hist [V][n_chunks], count [V], start [V + 1], perm and sid [T],
  // the partial rows [n_tiles][2][d]
  size_t off_hist = 0, off_count = 0, off_start = 0, off_perm = 0, off_sid = 0, off_part = 0,
         total = 0;
};

// Returns false when the sizes cannot be planned (T <= 0, V <= 0, d <= 0, or
// past the kernels' index range).
inline bool make_reassembly_plan(int64_t T, int64_t V, int64_t d, ReassemblyPlan* r) {
  if (T <= 0 || V <= 0 || d <= 0) return false;
  if (T >= (int64_t(1) << 24) || V >= (int64_t(1) << 31) || d >= (int64_t(1) << 31)) return false;
  ReassemblyPlan q;
  q.T = T;
  q.V = V;
  q.d = d;
  int64_t chunks = ceil_div(T, 256);
  if (chunks > 1024) chunks = 1024;
  const int64_t cap = kHistCap / V;
  if (chunks > cap) chunks = cap;
  if (chunks < 1) chunks = 1;
  q.chunk_tokens = ceil_div(ceil_div(T, chunks), 256) * 256;
  q.n_chunks = (int32_t)ceil_div(T, q.chunk_tokens);
  q.n_tiles = ceil_div(T, kReassembleTile);
  const int64_t col_chunks = ceil_div(d, 256);
  if (col_chunks * q.n_tiles >= (int64_t(1) << 31) || col_chunks * V >= (int64_t(1) << 31))
    return false;
  q.col_chunks = (int32_t)col_chunks;
  size_t off = 0;
  auto take = [&off](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  q.off_hist = take(sizeof(int32_t) * size_t(q.n_chunks) * size_t(V));
  q.off_count = take(sizeof(int32_t) * size_t(V));
  q.off_start = take(sizeof(int32_t) * size_t(V + 1));
  q.off_perm = take(sizeof(int32_t) * size_t(T));
  q.off_sid = take(sizeof(int32_t) * size_t(T));
  q.off_part = take(sizeof(float) * size_t(q.n_tiles) * 2 * size_t(d));
  q.total = off;
  *r = q;
  return true;
}

// The embedding estimator's workspace: the estimator's own regions (as for a
// layer with d_out = d; no outer product, so d_in = 1), then the reassembly's.
inline bool make_embedding_plan(int64_t T, int64_t V, int64_t d, int32_t K, int32_t antithetic,
                                int32_t dtype, Plan* p, ReassemblyPlan* r, size_t* r_base,
                                size_t* total) {
  if (!make_plan(T, 1, d, K, antithetic, dtype, p)) return false;
  if (!make_reassembly_plan(T, V, d, r)) return false;
  *r_base = align256(p->total);
  *total = *r_base + r->total;
  return true;
}


// ---------------------------------------------------------------------------
// Local scoring through a recomputed attention (dust_estimate_attention): the
// clean probabilities P and, for keys and queries, the clean weights
// B_st = p_st <e_s, v_t - o_s> of every (sequence, head) as [Lp][Lp] fp32
// (Lp = seq_len rounded up to kAttnBlock; entries past the causal edge or
// the sequence are zero, blocks above the diagonal are never written or
// read), and the score kernels' partial row sums
// [slots][sums][K][Lp] per (sequence, head): keys and values write one slot
// per block of kAttnBlock jittered tokens, queries one; keys and queries two
// sums per (token, draw), values one.  These follow the estimator's own
// regions (make_plan with d_out = heads * d_head).
constexpr int32_t kAttnBlock = 64;
constexpr int64_t kAttnMaxSeqLen = 4096;
// Noise vectors per score workgroup (-DDUST_ATTN_NV=n at build time: 1, 2
// or 4), held in registers as MFMA operands.
#ifndef DUST_ATTN_NV
#define DUST_ATTN_NV 2
#endif
constexpr int kAttnNV = DUST_ATTN_NV;
enum { kAttnQuery = 0, kAttnKey = 1, kAttnValue = 2 };

struct AttnPlan {
  int64_t n_seq = 0, L = 0, Lp = 0, H = 0, dh = 0;
  int32_t nb = 0;       // blocks of kAttnBlock tokens per sequence
  int32_t site = 0;     // kAttnQuery, kAttnKey or kAttnValue
  int32_t n_sums = 0;   // partial sums per (token, draw): 2, or 1 for values
  int32_t n_slots = 0;  // partial slots per token: nb, or 1 for queries
  int32_t nv = 0;       // noise vectors per score workgroup
  int32_t n_groups = 0; // score workgroups per (sequence, head, block): ceil(K_n / nv)
  size_t off_P = 0, off_B = 0, off_part = 0, total = 0;
};

// Returns false when the sizes cannot be planned (d_head not 64 or 128, a
// sequence longer than kAttnMaxSeqLen, an unknown site, or grids past the
// kernels' 32-bit indices).
inline bool make_attn_plan(const Plan& p, int64_t seq_len, int64_t heads, int64_t d_head,
                           int32_t site, AttnPlan* a) {
  if (heads <= 0 || (d_head != 64 && d_head != 128)) return false;
  if (site != kAttnQuery && site != kAttnKey && site != kAttnValue) return false;
  if (seq_len <= 0 || seq_len > kAttnMaxSeqLen || p.T % seq_len != 0) return false;
  if (p.d_out != heads * d_head) return false;
  AttnPlan q;
  q.n_seq = p.T / seq_len;
  q.L = seq_len;
  q.Lp = ceil_div(seq_len, kAttnBlock) * kAttnBlock;
  q.H = heads;
  q.dh = d_head;
  q.nb = (int32_t)(q.Lp / kAttnBlock);
  q.site = site;
  q.n_sums = site == kAttnValue ? 1 : 2;
  q.n_slots = site == kAttnQuery ? 1 : q.nb;
  q.nv = kAttnNV;
  q.n_groups = (int32_t)ceil_div(p.K_n, q.nv);
  const int64_t units = q.n_seq * heads * q.nb;
  if (ceil_div(units, 8) * 8 * q.n_groups >= (int64_t(1) << 31)) return false;
  const size_t sq = size_t(q.n_seq) * size_t(heads);
  const size_t mat = sizeof(float) * sq * size_t(q.Lp) * size_t(q.Lp);
  size_t off = align256(p.total);
  auto take = [&off](size_t bytes) {
    size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  q.off_P = take(mat);
  q.off_B = take(site == kAttnValue ? 0 : mat);
  q.off_part = take(sizeof(float) * sq * size_t(q.n_slots) * size_t(q.n_sums) * size_t(p.K) *
                    size_t(q.Lp));
  q.total = off;
  *a = q;
  return true;
}

}  // namespace dust
