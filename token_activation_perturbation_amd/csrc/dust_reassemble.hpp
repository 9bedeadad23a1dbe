// dust_reassemble.hpp -- gfx950 kernels of the embedding reassembly.
//
// An embedding's weight gradient is the scatter-add of its per-token errors
// into the rows their token ids select ("Dust: every token is a member of
// the population", section "What the released code actually does", step 7):
//   G_E[v] = scale sum_{t: ids[t] = v} g[t].
// Atomics on floats would make the sums depend on timing, so the rows are
// summed in a fixed order instead:
//   hist      per-chunk histograms of the ids, hist[v][chunk] (integer
//             atomics in LDS, or in global memory for a large V: exact)
//   colscan   one wave per id: each chunk's offset inside the id's run
//             (prefix over chunks), the run's length; rows of absent ids
//             are zeroed
//   scan      the runs' starts (prefix over ids), start[V] = T: inside every
//             placement workgroup (in LDS) when V <= kLdsHistMaxV, else a
//             kernel of its own
//   place     a stable counting sort: perm[pos] = t, sid[pos] = ids[t], the
//             tokens of one id in increasing t
//   tile      reduce-by-key over tiles of kReassembleTile sorted rows: runs
//             that lie inside the tile are summed and written; a run that
//             crosses a tile edge leaves a partial (slot 0: the tile's first
//             run, slot 1: its last)
//   fixup     the tile in which a crossing run ends sums the run's partials
//             in tile order and writes the row
// Ids outside [0, V) are clamped into it (memory-safe; the result is then
// unspecified).  All kernels index with 64-bit row offsets.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dust_plan.hpp"

namespace dust {
namespace reassemble {

__device__ __forceinline__ int32_t clamp_id(int32_t id, int32_t V) {
  return id < 0 ? 0 : (id >= V ? V - 1 : id);
}

__device__ __forceinline__ int uniform_wave() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ int32_t wave_incl_scan(int32_t x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

__global__ __launch_bounds__(256) void zero_kernel(int32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}

// hist[v][c] = number of tokens of chunk c with id v.  One workgroup per
// chunk.  LDS: counted in V ints of dynamic LDS, then every entry of the
// chunk's column written; otherwise counted straight into the (zeroed)
// global histogram.
template <bool LDS>
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int32_t T,
                                                   int32_t V, int64_t chunk_tokens,
                                                   int32_t n_chunks, int32_t* __restrict__ hist) {
  extern __shared__ int32_t cnt[];
  const int32_t c = blockIdx.x;
  const int64_t t0 = (int64_t)c * chunk_tokens;
  const int64_t t1 = t0 + chunk_tokens < T ? t0 + chunk_tokens : T;
  if (LDS) {
    for (int32_t v = threadIdx.x; v < V; v += 256) cnt[v] = 0;
    __syncthreads();
    for (int64_t t = t0 + threadIdx.x; t < t1; t += 256) atomicAdd(cnt + clamp_id(ids[t], V), 1);
    __syncthreads();
    for (int32_t v = threadIdx.x; v < V; v += 256) hist[(int64_t)v * n_chunks + c] = cnt[v];
  } else {
    for (int64_t t = t0 + threadIdx.x; t < t1; t += 256)
      atomicAdd(hist + (int64_t)clamp_id(ids[t], V) * n_chunks + c, 1);
  }
}

// One wave per id v: hist[v][c] <- sum_{c' < c} hist[v][c'] (chunk c's
// offset inside v's run; wave scans of 64 chunks at a time), count[v] = the
// run's length; G_E row v zeroed when v has no tokens.
template <bool VEC>
__global__ __launch_bounds__(256) void colscan_kernel(int32_t* __restrict__ hist,
                                                      int32_t n_chunks, int32_t V, int32_t d,
                                                      int32_t* __restrict__ count,
                                                      float* __restrict__ G_E) {
  const int64_t v = (int64_t)blockIdx.x * 4 + uniform_wave();
  if (v >= V) return;
  const int lane = threadIdx.x & 63;
  int32_t* row = hist + v * n_chunks;
  int32_t carry = 0;
  for (int32_t c0 = 0; c0 < n_chunks; c0 += 64) {
    const int32_t c = c0 + lane;
    const int32_t x = c < n_chunks ? row[c] : 0;
    const int32_t incl = wave_incl_scan(x, lane);
    if (c < n_chunks) row[c] = carry + incl - x;
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) count[v] = carry;
  if (carry == 0) {
    float* out = G_E + v * d;
    if (VEC) {
      for (int32_t c = 4 * lane; c < d; c += 256) *(float4*)(out + c) = make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      for (int32_t c = lane; c < d; c += 64) out[c] = 0.f;
    }
  }
}

// a[v] <- sum_{v' < v} a[v'] in place for v < V, and a[V] = the total, by
// the NT threads of one workgroup: contiguous ranges per thread, wave scans
// of the range sums, then a scan of the wave sums.  Every thread of the
// workgroup must call it; a[] is read after a barrier, so the caller's
// writes to it are visible.
template <int NT>
__device__ __forceinline__ void block_exclusive_scan(int32_t* a, int32_t V,
                                                     int32_t* __restrict__ wsum) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t per = ((int64_t)V + NT - 1) / NT;
  const int64_t b = (int64_t)tid * per;
  const int64_t e = b + per < V ? b + per : V;
  __syncthreads();
  int32_t s = 0;
  for (int64_t v = b; v < e; ++v) s += a[v];
  const int32_t incl = wave_incl_scan(s, lane);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int32_t x = lane < NT / 64 ? wsum[lane] : 0;
    const int32_t xi = wave_incl_scan(x, lane);
    if (lane < NT / 64) wsum[lane] = xi - x;
  }
  __syncthreads();
  int32_t run = wsum[w] + incl - s;
  for (int64_t v = b; v < e; ++v) {
    const int32_t x = a[v];
    a[v] = run;
    run += x;
  }
  if (tid == NT - 1) a[V] = run;
}

// count[0..V) copied to a[] with coalesced loads, several in flight.
template <int NT>
__device__ __forceinline__ void copy_counts(const int32_t* __restrict__ count, int32_t V,
                                            int32_t* a) {
#pragma unroll 8
  for (int32_t v = threadIdx.x; v < V; v += NT) a[v] = count[v];
}

// The runs' starts in global memory, for a V too large for the placement
// workgroups' LDS.  One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void start_scan_kernel(const int32_t* __restrict__ count,
                                                          int32_t V, int32_t* __restrict__ start) {
  __shared__ int32_t wsum[16];
  copy_counts<1024>(count, V, start);
  block_exclusive_scan<1024>(start, V, wsum);
}

// The stable placement: chunk c's tokens in sub-blocks of 256, in order;
// a token's position is its id's run start + the chunk's offset in the run
// + the tokens of the same id before it in the sub-block.  The last token of
// each id in a sub-block moves the chunk's offset on (one writer per id).
// SCAN: the run starts are scanned from count[] into this workgroup's LDS
// (dynamic, V + 1 ints), and workgroup 0 also writes them to start[];
// otherwise they are read from start[].
template <bool SCAN>
__global__ __launch_bounds__(256) void place_kernel(const int32_t* __restrict__ ids, int32_t T,
                                                    int32_t V, int64_t chunk_tokens,
                                                    int32_t n_chunks, int32_t* __restrict__ hist,
                                                    const int32_t* __restrict__ count,
                                                    int32_t* __restrict__ start,
                                                    int32_t* __restrict__ perm,
                                                    int32_t* __restrict__ sid) {
  __shared__ __attribute__((aligned(16))) int32_t sh[256];
  __shared__ int32_t wsum[4];
  extern __shared__ int32_t start_l[];
  const int32_t c = blockIdx.x;
  const int i = threadIdx.x;
  if (SCAN) {
    copy_counts<256>(count, V, start_l);
    block_exclusive_scan<256>(start_l, V, wsum);
    __syncthreads();
    if (c == 0)
      for (int32_t v = i; v <= V; v += 256) start[v] = start_l[v];
  }
  const int32_t* st = SCAN ? start_l : start;
  const int64_t t0 = (int64_t)c * chunk_tokens;
  const int64_t t1 = t0 + chunk_tokens < T ? t0 + chunk_tokens : T;
  for (int64_t tb = t0; tb < t1; tb += 256) {
    const int64_t t = tb + i;
    const int32_t id = t < t1 ? clamp_id(ids[t], V) : -1;
    int32_t* off = hist + (int64_t)(id < 0 ? 0 : id) * n_chunks + c;
    // the run start and the chunk's offset, fetched while the ranks are counted
    const int32_t base = id >= 0 ? st[id] + *off : 0;
    sh[i] = id;
    __syncthreads();
    // equal ids before and after this token, four LDS words per read and
    // several reads in flight
    int32_t before = 0, after = 0;
#pragma unroll 8
    for (int j = 0; j < 256; j += 4) {
      const int4 o = *(const int4*)(sh + j);
      before += (j < i && o.x == id) + (j + 1 < i && o.y == id) + (j + 2 < i && o.z == id) +
                (j + 3 < i && o.w == id);
      after += (j > i && o.x == id) + (j + 1 > i && o.y == id) + (j + 2 > i && o.z == id) +
               (j + 3 > i && o.w == id);
    }
    if (id >= 0) {
      const int32_t pos = base + before;
      perm[pos] = (int32_t)t;
      sid[pos] = id;
    }
    __syncthreads();  // every token has read its id's offset for this sub-block
    if (id >= 0 && after == 0) *off += before + 1;
    __syncthreads();  // offsets moved on before the next sub-block reads them
  }
}

template <bool VEC>
__device__ __forceinline__ float4 load_cols(const float* rowp, int32_t c, int32_t d) {
  if (VEC) {
    if (c < d) return *(const float4*)(rowp + c);
    return make_float4(0.f, 0.f, 0.f, 0.f);
  }
  return make_float4(c < d ? rowp[c] : 0.f, c + 1 < d ? rowp[c + 1] : 0.f,
                     c + 2 < d ? rowp[c + 2] : 0.f, c + 3 < d ? rowp[c + 3] : 0.f);
}

template <bool VEC>
__device__ __forceinline__ void store_cols(float* rowp, int32_t c, int32_t d, float4 x) {
  if (VEC) {
    if (c < d) *(float4*)(rowp + c) = x;
    return;
  }
  if (c < d) rowp[c] = x.x;
  if (c + 1 < d) rowp[c + 1] = x.y;
  if (c + 2 < d) rowp[c + 2] = x.z;
  if (c + 3 < d) rowp[c + 3] = x.w;
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 mul4(float s, float4 a) {
  return make_float4(s * a.x, s * a.y, s * a.z, s * a.w);
}

// Reduce-by-key over sorted rows.  One wave per (tile k, 256-column chunk
// j); lane l owns columns 256 j + 4 l .. + 3.  The tile's rows are loaded
// all at once, then summed in sorted order (increasing token within an id).
// A run crosses a tile edge only if it is the tile's first run and the row
// before the tile has its id, or the tile's last run and the row after the
// tile has its id; such a run is stored as a partial (slot 0: first run,
// slot 1: last run), every other run is written (times scale).
template <bool VEC>
__global__ __launch_bounds__(256) void tile_kernel(
    const float* __restrict__ g, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ sid, int32_t T, int32_t d, int32_t col_chunks, int64_t n_units,
    float scale, float* __restrict__ part, float* __restrict__ G_E) {
  constexpr int P = kReassembleTile;
  const int64_t u = (int64_t)blockIdx.x * 4 + uniform_wave();
  if (u >= n_units) return;
  const int64_t k = u / col_chunks;
  const int32_t j = (int32_t)(u - k * col_chunks);
  const int32_t c = j * 256 + 4 * (int32_t)(threadIdx.x & 63);
  const int32_t k0 = (int32_t)(k * P);
  const int32_t n = T - k0 < P ? T - k0 : P;
  float4 r[P];
#pragma unroll
  for (int q = 0; q < P; ++q)
    r[q] = q < n ? load_cols<VEC>(g + (int64_t)perm[k0 + q] * d, c, d)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
  const int32_t first = sid[k0], last = sid[k0 + n - 1];
  const bool first_crosses = k0 > 0 && sid[k0 - 1] == first;
  const bool last_crosses = k0 + n < T && sid[k0 + n] == last;
  auto flush = [&](int32_t v, float4 acc, bool is_first, bool is_last) {
    if ((is_first && first_crosses) || (is_last && last_crosses))
      store_cols<VEC>(part + (k * 2 + (is_first ? 0 : 1)) * d, c, d, acc);
    else
      store_cols<VEC>(G_E + (int64_t)v * d, c, d, mul4(scale, acc));
  };
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int32_t run = first;
  bool at_first = true;
#pragma unroll
  for (int q = 0; q < P; ++q) {
    if (q < n) {
      const int32_t v = sid[k0 + q];
      if (v != run) {
        flush(run, acc, at_first, false);
        acc = make_float4(0.f, 0.f, 0.f, 0.f);
        run = v;
        at_first = false;
      }
      acc = add4(acc, r[q]);
    }
  }
  flush(run, acc, at_first, true);
}

// The runs that cross tiles: a crossing run ends in the tile where it is
// the first run, began before the tile and does not go on past it; that
// tile's wave (one per tile and 256-column chunk) sums the run's partials in
// tile order and writes the row (times scale).
constexpr int32_t kFixupBlock = 64;  // tile sums added per block in the fix-up

template <bool VEC>
__global__ __launch_bounds__(256) void fixup_kernel(const int32_t* __restrict__ sid,
                                                    const int32_t* __restrict__ start, int32_t T,
                                                    const float* __restrict__ part, int32_t d,
                                                    int32_t col_chunks, int64_t n_units,
                                                    float scale, float* __restrict__ G_E) {
  constexpr int P = kReassembleTile;
  const int64_t u = (int64_t)blockIdx.x * 4 + uniform_wave();
  if (u >= n_units) return;
  const int64_t k = u / col_chunks;
  const int32_t j = (int32_t)(u - k * col_chunks);
  const int32_t c = j * 256 + 4 * (int32_t)(threadIdx.x & 63);
  const int32_t k0 = (int32_t)(k * P);
  const int32_t n = T - k0 < P ? T - k0 : P;
  const int32_t v = sid[k0];
  if (k0 == 0 || sid[k0 - 1] != v) return;        // began in this tile
  if (k0 + n < T && sid[k0 + n] == v) return;     // goes on past this tile
  const int32_t s = start[v];
  const int32_t kb = s / P;
  float4 sum = load_cols<VEC>(part + ((int64_t)kb * 2 + (s == kb * P ? 0 : 1)) * d, c, d);
  // the later tiles' sums in blocks of kFixupBlock, each block added first:
  // a run over n tiles then rounds like kFixupBlock + n / kFixupBlock terms
  // instead of n (the heaviest id of a long Zipfian batch spans ~20,000)
  for (int32_t kk = kb + 1; kk <= (int32_t)k;) {
    const int32_t kend = min(kk + kFixupBlock - 1, (int32_t)k);
    float4 blk = load_cols<VEC>(part + (int64_t)kk * 2 * d, c, d);
    for (++kk; kk <= kend; ++kk) blk = add4(blk, load_cols<VEC>(part + (int64_t)kk * 2 * d, c, d));
    sum = add4(sum, blk);
  }
  store_cols<VEC>(G_E + (int64_t)v * d, c, d, mul4(scale, sum));
}

}  // namespace reassemble
}  // namespace dust
