// Microbenchmarks of the MI355X roofs that the attention kernels are measured
// against: bf16 MFMA rate and the shader clock it runs at, v_exp_f32 and
// fp32 FMA issue rates, LDS read bandwidth, and an HBM copy. Each entry point
// runs one timed launch (after one warm-up launch) on the current device and
// returns its results through pointers; every loop has a fixed trip count and
// every access stays inside the buffers the entry point allocates.
//
// Roofline framing: inferensys glossary entry, "Roofline Model" (a kernel is
// bound by arithmetic or by memory bandwidth, whichever it saturates first).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Shader-clock (s_memtime) and real-time (s_memrealtime) counters, read by
// wave 0 of workgroup 0 around its loop: their ratio times the real-time
// counter's rate is the clock the kernel ran at.
struct Stamp {
  unsigned long long t, r;
};
__device__ __forceinline__ Stamp stamp_now() {
  return Stamp{__builtin_amdgcn_s_memtime(), __builtin_amdgcn_s_memrealtime()};
}
__device__ __forceinline__ void stamp_store(unsigned long long* out, Stamp a, Stamp b) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    out[0] = b.t - a.t;
    out[1] = b.r - a.r;
  }
}

// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave.
// Wave 0 of workgroup 0 stamps the shader clock (s_memtime) and the constant
// real-time counter (s_memrealtime) around its loop.
__global__ void __launch_bounds__(256) mfma_kernel(float* out, int iters, unsigned long long* stamps) {
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (float)(i - 3));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const Stamp s0 = stamp_now();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  const Stamp s1 = stamp_now();
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  stamp_store(stamps, s0, s1);
}

// Eight independent chains x = exp2(-x) (stays in (0, 1]) per lane.
__global__ void __launch_bounds__(256) exp_kernel(float* out, int iters, unsigned long long* stamps) {
  float x[8];
  for (int k = 0; k < 8; ++k) x[k] = 0.01f * (float)(threadIdx.x + k);
  const Stamp s0 = stamp_now();
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
  stamp_store(stamps, s0, stamp_now());
  float s = 0.f;
  for (int k = 0; k < 8; ++k) s += x[k];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// Eight independent chains x = x * a + b (a < 1 keeps them bounded) per lane.
__global__ void __launch_bounds__(256) fma_kernel(float* out, int iters, float a, float b,
                                                  unsigned long long* stamps) {
  float x[8];
  for (int k = 0; k < 8; ++k) x[k] = 0.01f * (float)(threadIdx.x + k);
  const Stamp s0 = stamp_now();
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __builtin_fmaf(x[k], a, b);
  stamp_store(stamps, s0, stamp_now());
  float s = 0.f;
  for (int k = 0; k < 8; ++k) s += x[k];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// 16-byte LDS reads (ds_read_b128): lane L of a wave reads chunk L + 64*i of
// a 16 KB buffer (four workgroups fit a CU), so a wave's 64 reads cover 1 KB
// of consecutive banks.
__global__ void __launch_bounds__(256) lds_kernel(float* out, int iters, unsigned long long* stamps) {
  __shared__ f32x4 buf[1024];
  for (int i = threadIdx.x; i < 1024; i += 256) buf[i] = f32x4{(float)i, 1.f, 2.f, 3.f};
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const Stamp s0 = stamp_now();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const f32x4 v = buf[(lane + 64 * ((w * 8 + k + i * 4) & 15)) & 1023];
      acc += v;
    }
  }
  stamp_store(stamps, s0, stamp_now());
  out[blockIdx.x * 256 + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

// An empty kernel: the floor of a launch that depends on the previous one.
__global__ void __launch_bounds__(256) empty_kernel(int* out) {
  if (out != nullptr && threadIdx.x == 0 && blockIdx.x == 0x7fffffff) out[0] = 0;
}

// Copy of n 16-byte elements, UNR per lane per step: workgroup g copies the
// elements g*256*UNR + u*256 + lane over rounds of gridDim.x workgroups.
template <int UNR>
__global__ void __launch_bounds__(256) copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst, int64_t n,
                                                   unsigned long long* stamps) {
  const Stamp s0 = stamp_now();
  const int64_t chunk = 256 * UNR;
  for (int64_t base = (int64_t)blockIdx.x * chunk; base < n; base += (int64_t)gridDim.x * chunk) {
    f32x4 v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      if (i < n) v[u] = __builtin_nontemporal_load(&src[i]);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t i = base + u * 256 + threadIdx.x;
      if (i < n) __builtin_nontemporal_store(v[u], &dst[i]);
    }
  }
  stamp_store(stamps, s0, stamp_now());
}

// Clock (GHz) from a pair of stamps and the real-time counter's rate.
double stamp_ghz(const unsigned long long* dev_stamps) {
  unsigned long long h[2] = {0, 0};
  if (hipMemcpy(h, dev_stamps, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return -1.0;
  int dev = 0, rate_khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1.0;
  if (hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -1.0;
  if (h[1] == 0 || rate_khz <= 0) return -1.0;
  return (double)h[0] / ((double)h[1] / (rate_khz * 1e3)) / 1e9;
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus;
}

// Times launch() once after a warm-up launch; milliseconds, or < 0 on error.
template <typename F>
double timed(F launch) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.0;
  launch();
  if (hipDeviceSynchronize() != hipSuccess) return -1.0;
  (void)hipEventRecord(e0, nullptr);
  launch();
  (void)hipEventRecord(e1, nullptr);
  if (hipEventSynchronize(e1) != hipSuccess) return -1.0;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (hipGetLastError() != hipSuccess) return -1.0;
  return (double)ms;
}

}  // namespace

extern "C" {

// bf16 MFMA: flops per second over `waves_per_simd` x 4 x CUs waves (four
// independent accumulator chains each), and the clock it ran at.
int roofs_mfma(int iters, int waves_per_simd, double* tflops, double* clock_ghz, double* ms_out) {
  const int cus = device_cus();
  if (cus <= 0 || iters <= 0 || waves_per_simd <= 0 || waves_per_simd > 8) return 1;
  const int blocks = cus * waves_per_simd;  // 4 waves per workgroup: one per SIMD
  float* out = nullptr;
  unsigned long long* st = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) return 2;
  if (hipMalloc(&st, 2 * sizeof(unsigned long long)) != hipSuccess) return 2;
  const double ms = timed([&] { mfma_kernel<<<blocks, 256>>>(out, iters, st); });
  *clock_ghz = stamp_ghz(st);
  (void)hipFree(out);
  (void)hipFree(st);
  if (ms <= 0.0) return 3;
  *tflops = (double)blocks * 4 * iters * 4 * (2.0 * 32 * 32 * 16) / (ms * 1e-3) / 1e12;
  *ms_out = ms;
  return 0;
}

// v_exp_f32 (kind 0) or fp32 FMA (kind 1): wave-level instructions per second
// with 4 waves per SIMD, and the clock they ran at.
int roofs_valu(int kind, int iters, double* winst_per_s, double* clock_ghz, double* ms_out) {
  const int cus = device_cus();
  if (cus <= 0 || iters <= 0) return 1;
  const int blocks = cus * 4;
  float* out = nullptr;
  unsigned long long* st = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) return 2;
  if (hipMalloc(&st, 2 * sizeof(unsigned long long)) != hipSuccess) return 2;
  const double ms = kind == 0 ? timed([&] { exp_kernel<<<blocks, 256>>>(out, iters, st); })
                              : timed([&] { fma_kernel<<<blocks, 256>>>(out, iters, 0.999f, 0.001f, st); });
  *clock_ghz = stamp_ghz(st);
  (void)hipFree(out);
  (void)hipFree(st);
  if (ms <= 0.0) return 3;
  *winst_per_s = (double)blocks * 4 * iters * 8 / (ms * 1e-3);
  *ms_out = ms;
  return 0;
}

// ds_read_b128 bytes per second over the whole device (4 waves per SIMD),
// and the clock.
int roofs_lds(int iters, double* bytes_per_s, double* clock_ghz, double* ms_out) {
  const int cus = device_cus();
  if (cus <= 0 || iters <= 0) return 1;
  const int blocks = cus * 4;
  float* out = nullptr;
  unsigned long long* st = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) return 2;
  if (hipMalloc(&st, 2 * sizeof(unsigned long long)) != hipSuccess) return 2;
  const double ms = timed([&] { lds_kernel<<<blocks, 256>>>(out, iters, st); });
  *clock_ghz = stamp_ghz(st);
  (void)hipFree(out);
  (void)hipFree(st);
  if (ms <= 0.0) return 3;
  *bytes_per_s = (double)blocks * 256 * iters * 8 * 16 / (ms * 1e-3);
  *ms_out = ms;
  return 0;
}

// Device-to-device copy of `bytes` (a multiple of 16) with `blocks_per_cu`
// workgroups per CU and `unroll` (1, 4 or 8) 16-byte elements per lane per
// step: read + write bytes per second.
int roofs_copy(int64_t bytes, int blocks_per_cu, int unroll, double* bytes_per_s, double* ms_out) {
  const int cus = device_cus();
  if (cus <= 0 || bytes <= 0 || bytes % 16 != 0 || blocks_per_cu <= 0 || blocks_per_cu > 64) return 1;
  if (unroll != 1 && unroll != 4 && unroll != 8) return 1;
  void *src = nullptr, *dst = nullptr;
  unsigned long long* st = nullptr;
  if (hipMalloc(&src, (size_t)bytes) != hipSuccess) return 2;
  if (hipMalloc(&dst, (size_t)bytes) != hipSuccess || hipMalloc(&st, 16) != hipSuccess) {
    (void)hipFree(src);
    return 2;
  }
  (void)hipMemset(src, 1, (size_t)bytes);
  const int64_t n = bytes / 16;
  const int g = cus * blocks_per_cu;
  const f32x4* s4 = (const f32x4*)src;
  f32x4* d4 = (f32x4*)dst;
  const double ms = timed([&] {
    if (unroll == 1)
      copy_kernel<1><<<g, 256>>>(s4, d4, n, st);
    else if (unroll == 4)
      copy_kernel<4><<<g, 256>>>(s4, d4, n, st);
    else
      copy_kernel<8><<<g, 256>>>(s4, d4, n, st);
  });
  (void)hipFree(src);
  (void)hipFree(dst);
  (void)hipFree(st);
  if (ms <= 0.0) return 3;
  *bytes_per_s = 2.0 * (double)bytes / (ms * 1e-3);
  *ms_out = ms;
  return 0;
}

// Back-to-back launches of an empty kernel of `blocks` workgroups on one
// stream, `count` of them between one pair of events: microseconds per launch.
int roofs_launch(int blocks, int count, double* us_per_launch) {
  if (blocks <= 0 || count <= 0) return 1;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 2;
  for (int i = 0; i < 10; ++i) empty_kernel<<<blocks, 256>>>(nullptr);
  if (hipDeviceSynchronize() != hipSuccess) return 3;
  (void)hipEventRecord(e0, nullptr);
  for (int i = 0; i < count; ++i) empty_kernel<<<blocks, 256>>>(nullptr);
  (void)hipEventRecord(e1, nullptr);
  if (hipEventSynchronize(e1) != hipSuccess) return 3;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (hipGetLastError() != hipSuccess) return 3;
  *us_per_launch = (double)ms * 1e3 / count;
  return 0;
}

}  // extern "C"
