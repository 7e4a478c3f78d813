// Forward pass of tiled exact attention for gfx950.
//
// One workgroup (4 waves, 256 lanes) owns 128 query rows of one (b, h)
// slice; each wave owns 32 of them and keeps their Q fragments in
// registers for the whole kernel. K and V tiles of BC keys stream through
// LDS (double buffered, register-staged prefetch of the next tile while the
// current one is consumed), so the N x N score matrix exists only as
// 32 x 32 register tiles (FlashAttention milestone page, "The idea": tiling
// with blocks sized for on-chip memory; pixelation article, "1. The Tiling
// Magic").
//
// Per tile and wave:
//   S^T = K Q^T on MFMA (keys are rows, the wave's 32 queries columns, so a
//         lane holds 16 keys of a single query per 32x32 block);
//   mask (causal diagonal tiles, sequence tail), then the online softmax
//   update of the running row maximum m and sum l (FlashAttention milestone
//   page, "The idea": two running numbers per row, earlier partial results
//   rescaled when a larger maximum arrives; pixelation article, "2. The
//   Online Softmax Trick"). The row maximum is an in-lane reduction plus one
//   exchange between the two wave halves; l stays a per-lane partial sum
//   until the epilogue;
//   dropout keep bits from the counter hash (fused step after softmax);
//   O^T += V^T P^T on MFMA: the softmaxed S^T accumulators, rounded to the
//   input type, are directly the B operand, so P never touches LDS; V is
//   stored transposed in LDS so that A-operand reads are contiguous.
// Epilogue: O = O / l / (1 - p), LSE = m + log l (natural log).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <typename T, int D, int BC>
struct FwdCfg {
  static constexpr int BR = 128;                            // queries per workgroup
  static constexpr int EPC = 16 / sizeof(T);                // elements per 16-byte chunk
  static constexpr int KS = D + (sizeof(T) == 2 ? 8 : 4);   // K tile row stride (elements)
  static constexpr int VS = BC + (sizeof(T) == 2 ? 4 : 1);  // V^T tile row stride (elements)
  static constexpr int KCH = D / EPC;                       // 16-byte chunks per K/V row
  static constexpr int NLD = BC * KCH / 256;                // 16-byte loads per lane per tile
  static constexpr int BUF = BC * KS + D * VS;              // elements per LDS buffer
  static_assert(BC % 32 == 0 && (BC * KCH) % 256 == 0, "tile shape");
  static_assert((BC * KS * sizeof(T)) % 16 == 0, "V^T base alignment");
};

template <typename T, int D, int BC, bool DROP>
__global__ void __launch_bounds__(256) fwd_kernel(AttnArgs a) {
  using C = FwdCfg<T, D, BC>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KI = M::KI, KH = M::KH;
  constexpr int NKB = BC / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;   // 32-column blocks of O^T
  constexpr int NC = D / KI;    // MFMA steps over d for S
  constexpr float NEG_INF = -__builtin_inff();

  __shared__ __attribute__((aligned(16))) T smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lo = lane & 31, hi = lane >> 5;

  // Workgroups are numbered tile-major: consecutive ids are different heads
  // of the same query tile, so with B*H a multiple of 8 all tiles of a head
  // land on the same XCD (ids are dealt round-robin over the 8 XCDs) and
  // share its L2. Causal: longest rows first.
  const int nq = (a.N + C::BR - 1) / C::BR;
  const int rank = blockIdx.x / a.BH;
  const int bh = blockIdx.x - rank * a.BH;
  const int qt = a.causal ? (nq - 1 - rank) : rank;
  const int N = a.N;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const T* __restrict__ Qg = static_cast<const T*>(a.q) + hoff;
  const T* __restrict__ Kg = static_cast<const T*>(a.k) + hoff;
  const T* __restrict__ Vg = static_cast<const T*>(a.v) + hoff;
  T* __restrict__ Og = static_cast<T*>(a.out) + hoff;

  const int qtile0 = qt * C::BR;
  const int q0w = qtile0 + w * 32;
  const int q = q0w + lo;
  const bool qvalid = q < N;

  frag qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    qf[c] = qvalid ? load_frag<T>(Qg + q * D + c * KI + hi * KH) : zero_frag<T>();

  uint32_t rowhash = 0;
  if constexpr (DROP) {
    const uint32_t hk = head_key(a.seed_lo, a.seed_hi, (uint32_t)(bh / a.H), (uint32_t)(bh % a.H));
    rowhash = fmix32(hk ^ (uint32_t)q);
  }

  // KV tiles this workgroup visits: causal stops at its diagonal; a block
  // mask skips the tiles of empty blocks (block-sparse variant).
  const int kend = a.causal ? min(N, qtile0 + C::BR) : N;
  const int ntiles = (kend + BC - 1) / BC;
  const uint8_t* bmrow = a.bmask ? a.bmask + (size_t)(qtile0 / a.mask_block) * a.nb : nullptr;
  auto kept = [&](int j) { return bmrow == nullptr || bmrow[(j * BC) / a.mask_block] != 0; };
  auto next_kept = [&](int j) {
    ++j;
    while (j < ntiles && !kept(j)) ++j;
    return j;
  };

  u32x4 kreg[C::NLD], vreg[C::NLD];
  auto gload = [&](int jt) {
    const int k0 = jt * BC;
#pragma unroll
    for (int i = 0; i < C::NLD; ++i) {
      const int c = i * 256 + tid;
      const int row = c / C::KCH, ch = c % C::KCH;  // K: chunk index fastest
      const int key = k0 + row;
      kreg[i] = key < N ? *reinterpret_cast<const u32x4*>(Kg + key * D + ch * C::EPC) : u32x4{0, 0, 0, 0};
      const int vrow = c % BC, vch = c / BC;       // V: key index fastest
      const int vkey = k0 + vrow;
      vreg[i] = vkey < N ? *reinterpret_cast<const u32x4*>(Vg + vkey * D + vch * C::EPC) : u32x4{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
    T* Ks = smem + buf * C::BUF;
    T* Vt = Ks + BC * C::KS;
#pragma unroll
    for (int i = 0; i < C::NLD; ++i) {
      const int c = i * 256 + tid;
      const int row = c / C::KCH, ch = c % C::KCH;
      *reinterpret_cast<u32x4*>(Ks + row * C::KS + ch * C::EPC) = kreg[i];
      const int vrow = c % BC, vch = c / BC;
      if constexpr (sizeof(T) == 2) {
        typedef T t8 __attribute__((ext_vector_type(8)));
        const t8 e = __builtin_bit_cast(t8, vreg[i]);
#pragma unroll
        for (int t = 0; t < 8; ++t) Vt[(vch * 8 + t) * C::VS + vrow] = e[t];
      } else {
        const f32x4 e = __builtin_bit_cast(f32x4, vreg[i]);
#pragma unroll
        for (int t = 0; t < 4; ++t) Vt[(vch * 4 + t) * C::VS + vrow] = e[t];
      }
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = zero16();
  float m_run = NEG_INF, l_run = 0.f;

  int j = kept(0) ? 0 : next_kept(0);
  int cur = 0;
  if (j < ntiles) {
    gload(j);
    sstore(0);
  }
  __syncthreads();

  while (j < ntiles) {
    const int jn = next_kept(j);
    if (jn < ntiles) gload(jn);

    const T* Ks = smem + cur * C::BUF;
    const T* Vt = Ks + BC * C::KS;
    const int k0 = j * BC;
    // The wave has work unless every key of the tile is above its diagonal.
    const bool active = (q0w < N) && (!a.causal || k0 <= q0w + 31);
    if (active) {
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          s[kb] = M::run(load_frag<T>(Ks + (kb * 32 + lo) * C::KS + c * KI + hi * KH), qf[c], s[kb]);
      }

      const bool need_mask = (a.causal && k0 + BC - 1 > q0w) || (k0 + BC > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = k0 + kb * 32 + crow(v, hi);
            if (key >= N || (a.causal && key > q)) s[kb][v] = NEG_INF;
          }
      }

      float mx = NEG_INF;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
      mx = fmaxf(mx, swap_halves(mx));
      const float mnew = fmaxf(m_run, mx * a.sl2);
      const float base = (mnew == NEG_INF) ? 0.f : mnew;
      const float alpha = exp2_fast(m_run - base);
      m_run = mnew;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = exp2_fast(fmaf(s[kb][v], a.sl2, -base));
          rs += p;
          s[kb][v] = p;
        }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;

      if constexpr (DROP) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t key = (uint32_t)(k0 + kb * 32 + crow(v, hi));
            if (fmix32(rowhash ^ key) < a.thresh) s[kb][v] = 0.f;
          }
      }

      if constexpr (KH == 8) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const frag pb = pack8<T>(s[kb][8 * hf + 0], s[kb][8 * hf + 1], s[kb][8 * hf + 2], s[kb][8 * hf + 3],
                                     s[kb][8 * hf + 4], s[kb][8 * hf + 5], s[kb][8 * hf + 6], s[kb][8 * hf + 7]);
            const int kk = kb * 32 + 16 * hf + 4 * hi;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const T* vp = Vt + (db * 32 + lo) * C::VS + kk;
              o[db] = M::run(load_frag_2x4<T>(vp, vp + 8), pb, o[db]);
            }
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kk = kb * 32 + crow(v, hi);
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] = M::run(Vt[(db * 32 + lo) * C::VS + kk], s[kb][v], o[db]);
          }
      }
    }

    if (jn < ntiles) sstore(cur ^ 1);
    __syncthreads();
    cur ^= 1;
    j = jn;
  }

  const float lt = l_run + swap_halves(l_run);
  const float inv = lt > 0.f ? a.rp / lt : 0.f;
  if (qvalid) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T* op = Og + q * D + db * 32 + 8 * g + 4 * hi;
        if constexpr (sizeof(T) == 2) {
          typedef T t4 __attribute__((ext_vector_type(4)));
          t4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = static_cast<T>(o[db][4 * g + e] * inv);
          *reinterpret_cast<t4*>(op) = r;
        } else {
          f32x4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = o[db][4 * g + e] * inv;
          *reinterpret_cast<f32x4*>(op) = r;
        }
      }
    if (hi == 0) a.lse[(size_t)bh * N + q] = lt > 0.f ? (m_run + log2_fast(lt)) * kLn2 : NEG_INF;
  }
}

template <typename T, int D, int BC, bool DROP>
static hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t s) {
  const int nq = (a.N + 127) / 128;
  const dim3 grid((unsigned)(nq * a.BH));
  fwd_kernel<T, D, BC, DROP><<<grid, dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

template <typename T, int D, int BC>
static hipError_t launch_fwd_d(bool dropout, const AttnArgs& a, hipStream_t s) {
  return dropout ? launch_fwd_t<T, D, BC, true>(a, s) : launch_fwd_t<T, D, BC, false>(a, s);
}

hipError_t launch_fwd(Elt t, int d, bool dropout, const AttnArgs& a, hipStream_t s) {
  switch (t) {
    case Elt::BF16:
      return d == 64 ? launch_fwd_d<__bf16, 64, 64>(dropout, a, s) : launch_fwd_d<__bf16, 128, 64>(dropout, a, s);
    case Elt::F16:
      return d == 64 ? launch_fwd_d<_Float16, 64, 64>(dropout, a, s) : launch_fwd_d<_Float16, 128, 64>(dropout, a, s);
    case Elt::F32:
      return d == 64 ? launch_fwd_d<float, 64, 64>(dropout, a, s) : launch_fwd_d<float, 128, 32>(dropout, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
