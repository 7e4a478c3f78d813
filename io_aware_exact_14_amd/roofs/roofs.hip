// Microbenchmarks of the MI355X roofs that the attention kernels are measured
// against: bf16 MFMA rate and the shader clock it runs at, issue rates of the
// VALU instructions the kernels use, MFMA / VALU overlap, LDS read bandwidth
// (plain and transpose reads), the compute skeleton of a forward tile step,
// an HBM copy and the empty-launch floor. Each entry point
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

// Issue rate of one VALU instruction kind: eight independent chains per lane
// of that instruction (kinds below), 4 waves per SIMD. The chains keep their
// values bounded and every result is consumed, so nothing is folded away.
//   0 v_exp_f32            x = exp2(-x)
//   1 v_fma_f32            x = x * a + b (a < 1)
//   2 v_dot2c_f32_bf16     x += dot((bf16 pair), (1, 1))
//   3 v_mul_lo_u32         u = u * c
//   4 v_perm_b32           u = perm(u, c, selector)
//   5 v_cvt_pk_bf16_f32    u = bits of the bf16 pair (u as float, a)
//   6 v_pk_mul_lo_u16      u = u * c, two 16-bit halves
//   7 v_cmp + v_cndmask    x = x > a ? x : a + 0.5 (two instructions per step)
//   8 v_mov_b32_dpp + add  u = quad_perm[1,0,3,2](u) + c (two instructions per step)
//   9 exp and fma mixed    chains 0-3 as kind 0, chains 4-7 as kind 1
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
template <int KIND>
__global__ void __launch_bounds__(256) rate_kernel(float* out, int iters, float a, uint32_t c, unsigned long long* stamps) {
  float x[8];
  uint32_t u[8];
  for (int k = 0; k < 8; ++k) {
    x[k] = 0.01f * (float)(threadIdx.x + k);
    u[k] = threadIdx.x * 2654435761u + (uint32_t)k;
  }
  const Stamp s0 = stamp_now();
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (KIND == 0) x[k] = __builtin_amdgcn_exp2f(-x[k]);
      if constexpr (KIND == 1) x[k] = __builtin_fmaf(x[k], a, 0.001f);
      if constexpr (KIND == 2)
        x[k] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u[k]), __builtin_bit_cast(bf16x2, c), x[k], false);
      if constexpr (KIND == 3) u[k] = u[k] * c;
      if constexpr (KIND == 4) u[k] = __builtin_amdgcn_perm(u[k], c, 0x05040100u + (uint32_t)k);
      if constexpr (KIND == 5)
        u[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{__builtin_bit_cast(float, u[k]), a}, bf16x2));
      if constexpr (KIND == 6) u[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, u[k]) * __builtin_bit_cast(u16x2, c));
      if constexpr (KIND == 7) x[k] = x[k] > a ? x[k] : a + 0.5f;
      if constexpr (KIND == 8) u[k] = (uint32_t)__builtin_amdgcn_mov_dpp((int)u[k], 0xB1, 0xF, 0xF, true) + c;
      if constexpr (KIND == 9) {
        if (k < 4)
          x[k] = __builtin_amdgcn_exp2f(-x[k]);
        else
          x[k] = __builtin_fmaf(x[k], a, 0.001f);
      }
    }
  stamp_store(stamps, s0, stamp_now());
  float s = 0.f;
  for (int k = 0; k < 8; ++k) s += x[k] + (float)(u[k] & 7u);
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// MFMA / VALU overlap: per iteration two independent v_mfma_f32_32x32x16_bf16
// (64 cycles of the matrix pipe) and NV fp32 FMAs on other registers.
template <int NV>
__global__ void __launch_bounds__(256) overlap_kernel(float* out, int iters, float a, unsigned long long* stamps) {
  bf16x8 p, q;
  for (int i = 0; i < 8; ++i) {
    p[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
    q[i] = (__bf16)(0.002f * (float)(i - 3));
  }
  f32x16 c0 = {}, c1 = {};
  float x[8];
  for (int k = 0; k < 8; ++k) x[k] = 0.01f * (float)(threadIdx.x + k);
  const Stamp s0 = stamp_now();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p, q, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q, p, c1, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < NV; ++r) x[r & 7] = __builtin_fmaf(x[r & 7], a, 0.001f);
  }
  stamp_store(stamps, s0, stamp_now());
  float s = 0.f;
  for (int k = 0; k < 8; ++k) s += x[k];
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i];
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

// Transpose reads in the pattern of the attention kernels' V^T / K^T
// operands: a 64-row bf16 tile with rows padded to 72 elements; per step each
// lane issues two ds_read_b64_tr_b16 (rows 4*(j/4) + l/32 and 2 further,
// 16-element column group (l/16)&1, 4-element piece j&3 for j = l&15), i.e.
// 16 bytes per lane like the ds_read_b128 kernel.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__global__ void __launch_bounds__(256) lds_tr_kernel(float* out, int iters, unsigned long long* stamps) {
  constexpr int KS = 72;
  __shared__ __attribute__((aligned(16))) __bf16 tile[64 * KS];
  for (int i = threadIdx.x; i < 64 * KS; i += 256) tile[i] = (__bf16)(float)(i & 255);
  __syncthreads();
  const int lane = threadIdx.x & 63, j = lane & 15;
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  uint32_t a0 = 0, a1 = 0;
  const Stamp s0 = stamp_now();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int base = 16 * (k & 3), col0 = 32 * (k >> 2);  // rows base..base+15, columns col0..col0+31
      const __bf16* pp = tile + (base + 4 * (j >> 2) + (lane >> 5)) * KS + col0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
      const u32x2_t x = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pp));
      const u32x2_t y = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pp + 2 * KS)));
      a0 ^= x[0] ^ y[0];  // two-input XORs fold into v_xor3_b32
      a1 ^= x[1] ^ y[1];
    }
  }
  stamp_store(stamps, s0, stamp_now());
  out[blockIdx.x * 256 + threadIdx.x] = (float)(a0 + a1);
}

// Compute skeleton of one forward tile step of the attention kernels, with
// no HBM traffic: per iteration a wave forms S^T (2 key blocks of 32 x its
// 32 queries, D/16 steps each), the softmax arithmetic of its 32 scores per
// lane (FMA, exp2, pairwise bf16 pack, row sum) and O^T += V^T P^T
// (D/32 x 4 products). USE_LDS reads the K fragments (ds_read_b128) and the
// V^T fragments (ds_read_b64_tr_b16 pairs) from one of two 64-key LDS tiles
// written once before the loop, alternating per step as in the kernels'
// double buffer (so the reads stay inside the loop), with the kernels'
// padded row strides; otherwise the operands come from registers. WPE waves
// per SIMD. This bounds what the tile loop can reach when tile loads, stores,
// masking and barriers cost nothing. PIPE software-pipelines the step: the
// next step's S products are issued between this step's exponentials.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <int D, int WPE, bool USE_LDS, bool PIPE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE)))
skeleton_kernel(float* out, int iters, float sl2, unsigned long long* stamps) {
  constexpr int KS = D + (D == 128 ? 24 : 8), NC = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 kt[USE_LDS ? 2 * 64 * KS : 8];
  __shared__ __attribute__((aligned(16))) __bf16 vt[USE_LDS ? 2 * 64 * KS : 8];
  const int tid = threadIdx.x, lane = tid & 63, lo = lane & 31, hi = lane >> 5, j = lane & 15;
  if (USE_LDS) {
    for (int i = tid; i < 2 * 64 * KS; i += 256) {
      kt[i] = (__bf16)(0.001f * (float)(i % 97));
      vt[i] = (__bf16)(0.002f * (float)(i % 89));
    }
  }
  __syncthreads();
  bf16x8 q[NC], k1[USE_LDS ? 1 : NC];  // k1: the second key block's operands in the register variant
  for (int c = 0; c < NC; ++c)
    for (int i = 0; i < 8; ++i) q[c][i] = (__bf16)(0.001f * (float)(tid + i + c));
  if (!USE_LDS)
    for (int c = 0; c < NC; ++c)
      for (int i = 0; i < 8; ++i) k1[c][i] = (__bf16)(0.003f * (float)(tid - i + 2 * c));
  // K fragment of key block kb, d step c, from the tile at element offset t0
  // (row kb*32 + lo, columns 16c + 8hi .. + 7: inside the 64 x KS tile).
  auto kfrag = [&](int t0, int kb, int c) {
    if constexpr (USE_LDS)
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4_t*>(&kt[t0 + (kb * 32 + lo) * KS + c * 16 + hi * 8]));
    else
      return kb ? k1[USE_LDS ? 0 : c] : q[c];  // distinct per key block (no common subexpression)
  };
  f32x16 o[NDB] = {};
  f32x16 sn[2] = {};  // PIPE: the next step's scores
  float l = 0.f;
  if constexpr (PIPE) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(0, kb, c), q[c], sn[kb], 0, 0, 0);
  }
  const Stamp s0 = stamp_now();
  for (int it = 0; it < iters; ++it) {
    const int t0 = (it & 1) * 64 * KS;  // this step's tile
    uint32_t pk[16];
    float rs = 0.f;
    if constexpr (!PIPE) {
      f32x16 s[2] = {};
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(t0, kb, c), q[c], s[kb], 0, 0, 0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * e], sl2, -1.f));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * e + 1], sl2, -1.f));
          pk[kb * 8 + e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, bf16x2));
          rs += p0 + p1;
        }
    } else {
      // The next step's S products (from the other tile), one per chunk,
      // between this step's exponentials; K fragments read three products
      // ahead; sched_barrier fences keep the order.
      const f32x16 s[2] = {sn[0], sn[1]};
      sn[0] = f32x16{};
      sn[1] = f32x16{};
      const int t1 = ((it + 1) & 1) * 64 * KS;
      constexpr int NP = 2 * NC, E = 16 / NP, LA = 3;  // products, score pairs per product, lookahead
      bf16x8 kq[NP];
#pragma unroll
      for (int i = 0; i < LA; ++i) kq[i] = kfrag(t1, i & 1, i >> 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        if (i + LA < NP) kq[i + LA] = kfrag(t1, (i + LA) & 1, (i + LA) >> 1);
        sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[i], q[i >> 1], sn[i & 1], 0, 0, 0);
#pragma unroll
        for (int e2 = 0; e2 < E; ++e2) {
          const int pe = i * E + e2, kb = pe >> 3, e = pe & 7;  // score pair pe of 16
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * e], sl2, -1.f));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][2 * e + 1], sl2, -1.f));
          pk[pe] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, bf16x2));
          rs += p0 + p1;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    l += rs;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4_t{pk[kb * 8 + 4 * hf], pk[kb * 8 + 4 * hf + 1],
                                                            pk[kb * 8 + 4 * hf + 2], pk[kb * 8 + 4 * hf + 3]});
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          bf16x8 vf;
          if constexpr (USE_LDS) {  // rows kb*32 + 16hf + 4hi + j/4 (and + 8) <= 63, columns < 32db + 32
            const __bf16* pp = &vt[t0 + (kb * 32 + 16 * hf + 4 * hi + (j >> 2)) * KS + db * 32 + 16 * ((lane >> 4) & 1) + 4 * (j & 3)];
            const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pp);
            const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pp + 8 * KS));
            vf = __builtin_bit_cast(bf16x8, i16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]});
          } else {
            vf = q[db];
          }
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, b, o[db], 0, 0, 0);
        }
      }
  }
  stamp_store(stamps, s0, stamp_now());
  float sm = l + sn[0][0] + sn[1][1];
  for (int db = 0; db < NDB; ++db)
    for (int i = 0; i < 16; ++i) sm += o[db][i];
  out[blockIdx.x * 256 + threadIdx.x] = sm;
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

// Instruction kind `kind` of rate_kernel (0-9): wave-level loop steps per
// second (kinds 7 and 8 issue two instructions per step) with 4 waves per
// SIMD, and the clock they ran at.
int roofs_valu(int kind, int iters, double* winst_per_s, double* clock_ghz, double* ms_out) {
  const int cus = device_cus();
  if (cus <= 0 || iters <= 0 || kind < 0 || kind > 9) return 1;
  const int blocks = cus * 4;
  float* out = nullptr;
  unsigned long long* st = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) return 2;
  if (hipMalloc(&st, 2 * sizeof(unsigned long long)) != hipSuccess) return 2;
  const float a = 0.999f;
  const uint32_t c = 0x3F803F80u;  // (1, 1) in bf16; an odd multiplier for the integer kinds
  const double ms = timed([&] {
    switch (kind) {
      case 0: rate_kernel<0><<<blocks, 256>>>(out, iters, a, c, st); break;
      case 1: rate_kernel<1><<<blocks, 256>>>(out, iters, a, c, st); break;
      case 2: rate_kernel<2><<<blocks, 256>>>(out, iters, a, c, st); break;
      case 3: rate_kernel<3><<<blocks, 256>>>(out, iters, a, c, st); break;
      case 4: rate_kernel<4><<<blocks, 256>>>(out, iters, a, c, st); break;
      case 5: rate_kernel<5><<<blocks, 256>>>(out, iters, a, c, st); break;
      case 6: rate_kernel<6><<<blocks, 256>>>(out, iters, a, c, st); break;
      case 7: rate_kernel<7><<<blocks, 256>>>(out, iters, a, c, st); break;
      case 8: rate_kernel<8><<<blocks, 256>>>(out, iters, a, c, st); break;
      default: rate_kernel<9><<<blocks, 256>>>(out, iters, a, c, st); break;
    }
  });
  *clock_ghz = stamp_ghz(st);
  (void)hipFree(out);
  (void)hipFree(st);
  if (ms <= 0.0) return 3;
  *winst_per_s = (double)blocks * 4 * iters * 8 / (ms * 1e-3);
  *ms_out = ms;
  return 0;
}

// overlap_kernel with nv (0, 4, 8, 12, 16 or 24) FMAs per two MFMAs:
// shader cycles per SIMD per iteration of one wave (4 waves per SIMD), and
// the clock.
int roofs_overlap(int nv, int iters, double* cycles, double* clock_ghz) {
  const int cus = device_cus();
  if (cus <= 0 || iters <= 0) return 1;
  const int blocks = cus * 4;
  float* out = nullptr;
  unsigned long long* st = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) return 2;
  if (hipMalloc(&st, 2 * sizeof(unsigned long long)) != hipSuccess) return 2;
  const double ms = timed([&] {
    switch (nv) {
      case 0: overlap_kernel<0><<<blocks, 256>>>(out, iters, 0.999f, st); break;
      case 4: overlap_kernel<4><<<blocks, 256>>>(out, iters, 0.999f, st); break;
      case 8: overlap_kernel<8><<<blocks, 256>>>(out, iters, 0.999f, st); break;
      case 12: overlap_kernel<12><<<blocks, 256>>>(out, iters, 0.999f, st); break;
      case 16: overlap_kernel<16><<<blocks, 256>>>(out, iters, 0.999f, st); break;
      case 24: overlap_kernel<24><<<blocks, 256>>>(out, iters, 0.999f, st); break;
      default: break;
    }
  });
  *clock_ghz = stamp_ghz(st);
  (void)hipFree(out);
  (void)hipFree(st);
  if (ms <= 0.0) return 3;
  *cycles = *clock_ghz * 1e9 * ms * 1e-3 / (4.0 * iters);
  return 0;
}

// skeleton_kernel at head dimension d (64 at 4 waves per SIMD, 128 at 2),
// operands from LDS or registers, plain or software-pipelined: SIMD cycles
// per wave tile step, and the clock.
int roofs_skeleton(int d, int use_lds, int pipe, int iters, double* cycles, double* clock_ghz) {
  const int cus = device_cus();
  // The pipelined step needs a second score tile, beyond the 128 registers
  // of four waves per SIMD at d = 64, so it is measured at d = 128 only.
  if (cus <= 0 || iters <= 0 || (d != 64 && d != 128) || (pipe && d == 64)) return 1;
  const int wpe = d == 64 ? 4 : 2;
  const int blocks = cus * wpe;
  float* out = nullptr;
  unsigned long long* st = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) return 2;
  if (hipMalloc(&st, 2 * sizeof(unsigned long long)) != hipSuccess) return 2;
  const float sl2 = 0.18f;
  const int sel = (d == 128 ? 4 : 0) + (use_lds ? 2 : 0) + (pipe ? 1 : 0);
  const double ms = timed([&] {
    switch (sel) {
      case 0: skeleton_kernel<64, 4, false, false><<<blocks, 256>>>(out, iters, sl2, st); break;
      case 2: skeleton_kernel<64, 4, true, false><<<blocks, 256>>>(out, iters, sl2, st); break;
      case 4: skeleton_kernel<128, 2, false, false><<<blocks, 256>>>(out, iters, sl2, st); break;
      case 5: skeleton_kernel<128, 2, false, true><<<blocks, 256>>>(out, iters, sl2, st); break;
      case 6: skeleton_kernel<128, 2, true, false><<<blocks, 256>>>(out, iters, sl2, st); break;
      default: skeleton_kernel<128, 2, true, true><<<blocks, 256>>>(out, iters, sl2, st); break;
    }
  });
  *clock_ghz = stamp_ghz(st);
  (void)hipFree(out);
  (void)hipFree(st);
  if (ms <= 0.0) return 3;
  *cycles = *clock_ghz * 1e9 * ms * 1e-3 / ((double)wpe * iters);
  return 0;
}

// LDS read bytes per second over the whole device (4 waves per SIMD), and
// the clock: kind 0 ds_read_b128 of consecutive chunks, kind 1 the
// transpose-read pattern of lds_tr_kernel.
int roofs_lds(int kind, int iters, double* bytes_per_s, double* clock_ghz, double* ms_out) {
  const int cus = device_cus();
  if (cus <= 0 || iters <= 0 || kind < 0 || kind > 1) return 1;
  const int blocks = cus * 4;
  float* out = nullptr;
  unsigned long long* st = nullptr;
  if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) return 2;
  if (hipMalloc(&st, 2 * sizeof(unsigned long long)) != hipSuccess) return 2;
  const double ms = kind == 0 ? timed([&] { lds_kernel<<<blocks, 256>>>(out, iters, st); })
                              : timed([&] { lds_tr_kernel<<<blocks, 256>>>(out, iters, st); });
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
