// Internal interface between the C-ABI host layer (fa_api.hip) and the
// kernel launchers. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum class Elt { F32 = 0, F16 = 1, BF16 = 2 };

// Arguments shared by the forward and backward kernels. Tensors are
// [B][H][N][d] contiguous; `bh` indexes B*H slices.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;     // backward: forward output
  const void* dout;  // backward: dO
  void* out;         // forward: O
  float* lse;        // forward: written; backward: read
  void* dq;
  void* dk;
  void* dv;
  float* delta;      // backward workspace: D_i = dO_i . O_i, [B*H][N]
  const uint8_t* bmask;  // block mask [nb][nb] or nullptr
  int N;
  int H;
  int BH;
  int mask_block;
  int nb;
  int causal;
  float scale;       // softmax scale
  float sl2;         // scale * log2(e)
  float rp;          // 1 / (1 - dropout_p)
  float kq;          // 1 - dropout_p
  uint32_t thresh;   // dropout threshold floor(p * 2^16) << 16: a key is kept when its
                     // 16-bit half of the keep word, moved to the top bits, is >= thresh
  uint32_t seed_lo;
  uint32_t seed_hi;
  uint32_t ones16;   // 0x00010001: packed 16-bit ones (a runtime value, so that the packed
                     // keep-factor arithmetic stays packed instead of becoming compares)
  int ncu;           // compute units of the device the call runs on
  int nxcd;          // accelerator complex dies (XCDs) among which workgroup ids are dealt
};

hipError_t launch_fwd(Elt t, int d, bool dropout, const AttnArgs& a, hipStream_t s);
// stage: 1 = dQ (and D), 2 = dK/dV, 3 = both in order
hipError_t launch_bwd(Elt t, Elt gt, int d, bool dropout, int stage, const AttnArgs& a, hipStream_t s);
hipError_t launch_dropout_mask(const AttnArgs& a, int b, int h, int64_t i0, int64_t rows, int64_t j0,
                               int64_t cols, uint8_t* keep, hipStream_t s);

}  // namespace fa
