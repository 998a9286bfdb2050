// Calibration microbenchmarks for the roofline ceilings on gfx950: matrix-core
// rates of the MFMA shapes the kernels use (with fixed and with changing
// operands), the transcendental (v_exp_f32) and
// plain FMA VALU rates, and a streaming HBM copy. Every kernel runs a fixed,
// bounded loop on registers (no memory traffic) except the copy.
//
//   hipcc -O3 --offload-arch=gfx950 calib.hip -o calib && ./calib
//
// Prints one JSON object with per-chip rates.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
      exit(1);                                                                \
    }                                                                         \
  } while (0)

constexpr int ITERS = 4096;
constexpr int CHAINS = 8;  // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_bf16_32(float *out, float seed) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) a[e] = (__bf16)(seed * (threadIdx.x + e)), b[e] = (__bf16)(seed - e);
  f32x4 c[CHAINS];
  for (int i = 0; i < CHAINS; ++i) c[i] = f32x4{0, 0, 0, 0};
  for (int it = 0; it < ITERS; ++it)
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[i], 0, 0, 0);
  float s = 0;
  for (int i = 0; i < CHAINS; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The same products with operands that change from one instruction to the
// next (random mantissas, eight register sets cycled), as in a real GEMM: the
// matrix cores' sustained rate depends on the data they switch.
__device__ __forceinline__ uint32_t xorshift(uint32_t &x) {
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}
__device__ __forceinline__ float rand_unit(uint32_t &x) {  // uniform in [-0.5, 0.5) with a full mantissa
  return __uint_as_float((xorshift(x) & 0x007fffffu) | 0x3f800000u) - 1.5f;
}

__global__ __launch_bounds__(256) void mfma_bf16_32_rand(float *out, float seed) {
  uint32_t x = (threadIdx.x + 1) * 0x9e3779b9u ^ __float_as_uint(seed);
  bf16x8 a[4], b[4];
  for (int k = 0; k < 4; ++k)
    for (int e = 0; e < 8; ++e) a[k][e] = (__bf16)rand_unit(x), b[k][e] = (__bf16)rand_unit(x);
  f32x4 c[CHAINS];
  for (int i = 0; i < CHAINS; ++i) c[i] = f32x4{0, 0, 0, 0};
  for (int it = 0; it < ITERS; it += 4)
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < CHAINS; ++i)
        c[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(u + i) & 3], b[(u + 3 * i + 1) & 3], c[i], 0, 0, 0);
  float s = 0;
  for (int i = 0; i < CHAINS; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_f32_4_rand(float *out, float seed) {
  uint32_t x = (threadIdx.x + 1) * 0x9e3779b9u ^ __float_as_uint(seed);
  float a[8], b[8];
  for (int k = 0; k < 8; ++k) a[k] = rand_unit(x), b[k] = rand_unit(x);
  f32x4 c[CHAINS];
  for (int i = 0; i < CHAINS; ++i) c[i] = f32x4{0, 0, 0, 0};
  for (int it = 0; it < ITERS; it += 8)
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < CHAINS; ++i)
        c[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[(u + i) & 7], b[(u + 3 * i + 1) & 7], c[i], 0, 0, 0);
  float s = 0;
  for (int i = 0; i < CHAINS; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_bf16_16(float *out, float seed) {
  s16x4 a, b;
  for (int e = 0; e < 4; ++e) a[e] = (short)(threadIdx.x + e), b[e] = (short)(seed + e);
  f32x4 c[CHAINS];
  for (int i = 0; i < CHAINS; ++i) c[i] = f32x4{0, 0, 0, 0};
  for (int it = 0; it < ITERS; ++it)
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c[i], 0, 0, 0);
  float s = 0;
  for (int i = 0; i < CHAINS; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_f32_4(float *out, float seed) {
  const float a = seed * threadIdx.x, b = seed + 1.f;
  f32x4 c[CHAINS];
  for (int i = 0; i < CHAINS; ++i) c[i] = f32x4{0, 0, 0, 0};
  for (int it = 0; it < ITERS; ++it)
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) c[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c[i], 0, 0, 0);
  float s = 0;
  for (int i = 0; i < CHAINS; ++i) s += c[i][0] + c[i][1] + c[i][2] + c[i][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// v_exp_f32 on 8 independent values per lane
__global__ __launch_bounds__(256) void valu_exp(float *out, float seed) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = -seed * (threadIdx.x + i) * 1e-6f;
  for (int it = 0; it < ITERS; ++it)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) - 1.0f;
  float s = 0;
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// plain (non-packed) fp32 FMA on 8 independent values per lane
__global__ __launch_bounds__(256) void valu_fma(float *out, float seed) {
  float x[8];
  for (int i = 0; i < 8; ++i) x[i] = seed * (threadIdx.x + i);
  for (int it = 0; it < ITERS; ++it)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 1e-3f);
  float s = 0;
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// exp and FMA interleaved: do transcendentals overlap other VALU work?
__global__ __launch_bounds__(256) void valu_exp_fma(float *out, float seed) {
  float x[8], y[8];
  for (int i = 0; i < 8; ++i) x[i] = -seed * (threadIdx.x + i) * 1e-6f, y[i] = seed * i;
  for (int it = 0; it < ITERS; ++it)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = __builtin_amdgcn_exp2f(x[i]) - 1.0f;
      y[i] = __builtin_fmaf(y[i], 0.999f, 1e-3f);
      y[i] = __builtin_fmaf(y[i], 0.999f, 1e-3f);
      y[i] = __builtin_fmaf(y[i], 0.999f, 1e-3f);
    }
  float s = 0;
  for (int i = 0; i < 8; ++i) s += x[i] + y[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void copy16(const uint4 *__restrict__ src, uint4 *__restrict__ dst, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) dst[i] = src[i];
}

static float time_kernel(void (*k)(float *, float), int grid, float *out) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, 0, out, 0.5f);  // warm-up
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0, 0));
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, 0, out, 0.5f);
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return ms;
}

int main() {
  int dev = 0, cus = 0, clk_khz = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  CHECK(hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeClockRate, dev));
  const int grid = cus * 8;  // 8 workgroups of 4 waves per CU: 8 waves per SIMD
  float *out;
  CHECK(hipMalloc(&out, (size_t)grid * 256 * sizeof(float)));
  const double waves = (double)grid * 4;
  const double per_wave = (double)ITERS * CHAINS;

  const double t_bf32 = time_kernel(mfma_bf16_32, grid, out) * 1e-3;
  const double t_bf16 = time_kernel(mfma_bf16_16, grid, out) * 1e-3;
  const double t_f32 = time_kernel(mfma_f32_4, grid, out) * 1e-3;
  const double t_bf32r = time_kernel(mfma_bf16_32_rand, grid, out) * 1e-3;
  const double t_f32r = time_kernel(mfma_f32_4_rand, grid, out) * 1e-3;
  const double t_exp = time_kernel(valu_exp, grid, out) * 1e-3;
  const double t_fma = time_kernel(valu_fma, grid, out) * 1e-3;
  const double t_mix = time_kernel(valu_exp_fma, grid, out) * 1e-3;
  const double lanes = waves * 256 / 4 * per_wave / CHAINS * 8;  // lane-ops of one 8-wide loop body

  // HBM copy, 1 GiB each way
  const size_t bytes = (size_t)1 << 30;
  uint4 *a, *b;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMemset(a, 1, bytes));
  const size_t n = bytes / sizeof(uint4);
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  hipLaunchKernelGGL(copy16, dim3(cus * 16), dim3(256), 0, 0, a, b, n);
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0, 0));
  for (int r = 0; r < 5; ++r) hipLaunchKernelGGL(copy16, dim3(cus * 16), dim3(256), 0, 0, a, b, n);
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  const double copy_GBps = 2.0 * bytes * 5 / (ms * 1e-3) / 1e9;

  printf("{\"cus\": %d, \"clock_mhz\": %.0f, "
         "\"mfma_bf16_16x16x32_TFLOPs\": %.1f, \"mfma_bf16_16x16x16_TFLOPs\": %.1f, "
         "\"mfma_f32_16x16x4_TFLOPs\": %.1f, \"mfma_bf16_16x16x32_random_TFLOPs\": %.1f, "
         "\"mfma_f32_16x16x4_random_TFLOPs\": %.1f, \"v_exp_f32_Gops\": %.1f, \"v_fma_f32_Gops\": %.1f, "
         "\"exp_plus_3fma_Gexp\": %.1f, \"copy_GBps\": %.1f}\n",
         cus, clk_khz / 1000.0, waves * per_wave * 16384 / t_bf32 / 1e12, waves * per_wave * 8192 / t_bf16 / 1e12,
         waves * per_wave * 2048 / t_f32 / 1e12, waves * per_wave * 16384 / t_bf32r / 1e12,
         waves * per_wave * 2048 / t_f32r / 1e12, lanes / t_exp / 1e9, lanes / t_fma / 1e9, lanes / t_mix / 1e9,
         copy_GBps);
  CHECK(hipFree(out));
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  return 0;
}
