// valu_rates -- issue rates of the vector instructions the noise kernels are
// made of, measured on the GPU it runs on, and the rate of the noise
// generation itself.  The ALU cost model of the noise kernels weights each
// instruction by the rate class measured here.
//
// Each row launches 8192 workgroups of 256 lanes (4 rounds of 8 waves per
// SIMD on a 256-CU part); every lane runs 8 independent dependency chains of
// one instruction (inline assembly, so the instruction is exactly the one
// named) for `iters` steps.  Rate = lanes x steps x 8 / kernel time, reported
// per compute unit per clock, both at the nominal 2.4 GHz and at the shader
// clock measured during the run (s_memtime cycles of the first wave over
// the 100 MHz s_memrealtime).  The generation row runs noise_quad, the
// kernels' own Philox4x32-10 + Box-Muller, and reports quads per second.
//
// Memory: every lane writes exactly one word, out[workgroup * 256 + lane],
// and out holds kBlocks * 256 words; lane 0 of workgroup 0 also writes
// clk[0..1].  Prints one line per row; exits 1 on any HIP error.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "dust_noise.hpp"

namespace {

constexpr int kBlocks = 256 * 32;
constexpr int kIters = 2048;

#define VR_CHECK(x)                                                          \
  do {                                                                       \
    const hipError_t e_ = (x);                                               \
    if (e_ != hipSuccess) {                                                  \
      std::printf("%s: %s\n", #x, hipGetErrorString(e_));                   \
      std::exit(1);                                                          \
    }                                                                        \
  } while (0)

enum Op {
  kXor, kShift, kMul, kFma, kBitop3, kMad64, kMulHi, kCvt, kLog, kSqrt, kSin, kCos,
  kXorS, kBitop3S, kMad64S, kMulLit, kNumOps
};

__device__ __forceinline__ void clock_start(uint64_t& t0, uint64_t& r0) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
}

__device__ __forceinline__ void clock_stop(uint64_t t0, uint64_t r0, uint64_t* clk) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

template <int OP>
__global__ __launch_bounds__(256) void op_kernel(uint32_t* out, uint64_t* clk, int iters,
                                                 uint32_t s) {
  uint32_t x[8];
  uint64_t p[8];
  float f[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = threadIdx.x * 8 + j + blockIdx.x;
    p[j] = x[j];
    f[j] = 1.0f + 0.001f * (float)x[j];
  }
  const uint32_t y = threadIdx.x ^ 0x55u;
  const uint32_t m = (threadIdx.x | 1u) * 0x9E3779B9u;
  const float c1 = 0.999f, c2 = 0.001f;
  uint64_t t0 = 0, r0 = 0;
  clock_start(t0, r0);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint64_t carry;
      switch (OP) {
        case kXor: asm volatile("v_xor_b32 %0, %0, %1" : "+v"(x[j]) : "v"(y)); break;
        case kShift: asm volatile("v_lshrrev_b32 %0, 1, %0" : "+v"(x[j])); break;
        case kMul: asm volatile("v_mul_f32 %0, %0, %1" : "+v"(f[j]) : "v"(c1)); break;
        case kFma: asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(f[j]) : "v"(c1), "v"(c2)); break;
        case kBitop3:
          asm volatile("v_bitop3_b32 %0, %0, %1, %2 bitop3:0x96" : "+v"(x[j]) : "v"(y), "v"(m));
          break;
        case kMad64:
          asm volatile("v_mad_u64_u32 %0, %1, %2, %3, %0" : "+v"(p[j]), "=s"(carry) : "v"(y), "v"(m));
          break;
        case kMulHi: asm volatile("v_mul_hi_u32 %0, %0, %1" : "+v"(x[j]) : "v"(m)); break;
        case kCvt: asm volatile("v_cvt_f32_u32 %0, %0" : "+v"(x[j])); break;
        case kLog: asm volatile("v_log_f32 %0, %0" : "+v"(f[j])); break;
        case kSqrt: asm volatile("v_sqrt_f32 %0, %0" : "+v"(f[j])); break;
        case kSin: asm volatile("v_sin_f32 %0, %0" : "+v"(f[j])); break;
        case kCos: asm volatile("v_cos_f32 %0, %0" : "+v"(f[j])); break;
        case kXorS: asm volatile("v_xor_b32 %0, %1, %0" : "+v"(x[j]) : "s"(s)); break;
        case kBitop3S:
          asm volatile("v_bitop3_b32 %0, %0, %1, %2 bitop3:0x96" : "+v"(x[j]) : "v"(y), "s"(s));
          break;
        case kMad64S:
          asm volatile("v_mad_u64_u32 %0, %1, %2, %3, %0" : "+v"(p[j]), "=s"(carry) : "v"(y), "s"(s));
          break;
        case kMulLit: asm volatile("v_mul_f32 %0, 0x33800000, %0" : "+v"(f[j])); break;
        default: break;
      }
    }
  }
  clock_stop(t0, r0, clk);
  uint32_t r = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) r ^= x[j] ^ (uint32_t)p[j] ^ __float_as_uint(f[j]);
  out[blockIdx.x * 256 + threadIdx.x] = r;
}

// The kernels' generation: quads (quad = this lane, token 7, noise index i).
__global__ __launch_bounds__(256) void generation_kernel(uint32_t* out, uint64_t* clk, int iters,
                                                         uint32_t s) {
  const uint32_t q = blockIdx.x * 256 + threadIdx.x;
  const dust::NoiseKey key{s, s * 3u + 1u};
  float r = 0.f;
  uint64_t t0 = 0, r0 = 0;
  clock_start(t0, r0);
  for (int i = 0; i < iters; i += 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 a = dust::noise_quad(q, 7u, (uint32_t)(i + j), key);
      r += a.x * a.y + a.z * a.w;
    }
  }
  clock_stop(t0, r0, clk);
  out[q] = __float_as_uint(r);
}

struct Row {
  const char* name;
  void (*kernel)(uint32_t*, uint64_t*, int, uint32_t);
};

template <int OP>
Row op_row(const char* name) {
  return Row{name, op_kernel<OP>};
}

}  // namespace

int main() {
  uint32_t* out = nullptr;
  uint64_t* clk = nullptr;
  VR_CHECK(hipMalloc(&out, sizeof(uint32_t) * kBlocks * 256));
  VR_CHECK(hipMalloc(&clk, sizeof(uint64_t) * 2));
  hipEvent_t a, b;
  VR_CHECK(hipEventCreate(&a));
  VR_CHECK(hipEventCreate(&b));
  const double lanes = (double)kBlocks * 256;

  // best of three launches after one warm-up; returns ms and the clock (GHz)
  auto time_row = [&](const Row& row, double& ghz) {
    hipLaunchKernelGGL(row.kernel, dim3(kBlocks), dim3(256), 0, 0, out, clk, kIters, 0x9E3779B9u);
    VR_CHECK(hipGetLastError());
    VR_CHECK(hipDeviceSynchronize());
    float best = 1e30f;
    for (int rep = 0; rep < 3; ++rep) {
      VR_CHECK(hipEventRecord(a, 0));
      hipLaunchKernelGGL(row.kernel, dim3(kBlocks), dim3(256), 0, 0, out, clk, kIters, 0x9E3779B9u);
      VR_CHECK(hipGetLastError());
      VR_CHECK(hipEventRecord(b, 0));
      VR_CHECK(hipEventSynchronize(b));
      float ms = 0.f;
      VR_CHECK(hipEventElapsedTime(&ms, a, b));
      if (ms < best) {
        best = ms;
        uint64_t h[2];
        VR_CHECK(hipMemcpy(h, clk, sizeof h, hipMemcpyDeviceToHost));
        ghz = (double)h[0] / ((double)h[1] / 100e6) / 1e9;
      }
    }
    return (double)best;
  };

  const Row rows[] = {
      op_row<kXor>("v_xor_b32 v,v"),         op_row<kShift>("v_lshrrev_b32 const,v"),
      op_row<kMul>("v_mul_f32 v,v"),         op_row<kFma>("v_fma_f32 v,v,v"),
      op_row<kBitop3>("v_bitop3_b32 v,v,v"), op_row<kMad64>("v_mad_u64_u32 v,v,v64"),
      op_row<kMulHi>("v_mul_hi_u32 v,v"),    op_row<kCvt>("v_cvt_f32_u32 v"),
      op_row<kLog>("v_log_f32 v"),           op_row<kSqrt>("v_sqrt_f32 v"),
      op_row<kSin>("v_sin_f32 v"),           op_row<kCos>("v_cos_f32 v"),
      op_row<kXorS>("v_xor_b32 s,v"),        op_row<kBitop3S>("v_bitop3_b32 v,v,s"),
      op_row<kMad64S>("v_mad_u64_u32 v,s,v64"), op_row<kMulLit>("v_mul_f32 literal,v"),
  };
  std::printf("%-26s %9s %9s %13s %13s\n", "instruction", "ms", "clock GHz", "lanes/CU/clk",
              "at measured");
  for (const Row& row : rows) {
    double ghz = 0.0;
    const double ms = time_row(row, ghz);
    const double per_s = lanes * kIters * 8.0 / (ms * 1e-3);
    std::printf("%-26s %9.3f %9.3f %13.1f %13.1f\n", row.name, ms, ghz, per_s / 256 / 2.4e9,
                per_s / 256 / (ghz * 1e9));
  }
  double ghz = 0.0;
  const double ms = time_row(Row{"generation", generation_kernel}, ghz);
  const double quads_per_s = lanes * kIters / (ms * 1e-3);
  std::printf("%-26s %9.3f %9.3f %13s %13s  %.4e quads/s\n", "generation (noise_quad)", ms, ghz,
              "-", "-", quads_per_s);
  VR_CHECK(hipFree(out));
  VR_CHECK(hipFree(clk));
  return 0;
}
