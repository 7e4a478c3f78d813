// Materializes the dropout keep bits of one (b, h) window with the same
// device hash the fused kernels use (fa_device.h). Used to check the bits
// bit-exactly; the attention kernels themselves never store the mask.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

__global__ void __launch_bounds__(256) dropout_mask_kernel(uint32_t hk, uint32_t thresh, int64_t i0, int64_t rows,
                                                           int64_t j0, int64_t cols, uint8_t* __restrict__ keep) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * cols) return;
  const int64_t r = idx / cols, c = idx - r * cols;
  const uint32_t rh = fmix32(hk ^ (uint32_t)(i0 + r));
  const uint32_t j = (uint32_t)(j0 + c);
  const uint32_t u = keep_finish((rh + (j >> 1)) * kMixMul);
  keep[idx] = ((j & 1u) ? keep_hi(u, thresh) : keep_lo(u, thresh)) ? 1 : 0;
}

// Host-side copy of the per-(b, h) key derivation (same steps as head_key).
static uint32_t host_fmix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return x;
}

hipError_t launch_dropout_mask(const AttnArgs& a, int b, int h, int64_t i0, int64_t rows, int64_t j0, int64_t cols,
                               uint8_t* keep, hipStream_t s) {
  uint32_t k = host_fmix32(a.seed_lo + 0x9E3779B9u);
  k = host_fmix32(k ^ a.seed_hi);
  k = host_fmix32(k ^ (uint32_t)b);
  k = host_fmix32(k ^ (uint32_t)h);
  const int64_t n = rows * cols;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  dropout_mask_kernel<<<dim3(blocks), dim3(256), 0, s>>>(k, a.thresh, i0, rows, j0, cols, keep);
  return hipGetLastError();
}

}  // namespace fa
