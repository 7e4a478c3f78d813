// Backward pass of tiled exact attention for gfx950.
//
// Only O and the per-row log-sum-exp were kept from the forward; S and P
// are recomputed tile by tile on chip from Q, K and LSE (FlashAttention
// milestone page, "The idea", recomputation; pixelation article, "The
// Recomputation Trade-off"). The gradients follow from the chain rule on the
// forward definition, with Pd = P * Z / (1 - p):
//   dV = Pd^T dO,  dP = (dO V^T) * Z / (1 - p),  D_i = dO_i . O_i,
//   dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
// With dropout the kernels form dS' = dS (1 - p) = P * (Z * (dO V^T) - D (1 - p))
// and fold 1 / (1 - p) into the final scales of dQ and dK (dV's factor is
// applied at the end too), which saves a multiply per score.
//
// Two kernels, both deterministic (no atomics):
//   bwd_dq_kernel   one workgroup per 128 query rows: D_i (written to the
//                   workspace), then a loop over K/V tiles accumulating dQ.
//                   Mirrors the forward's orientation (S^T = K Q^T, lanes
//                   own a query), so dS^T is directly the B operand of
//                   dQ^T += K^T dS^T; K^T is read from the row-major K tile
//                   with LDS transpose reads. At d = 128 (16-bit) the K/V
//                   tiles are loaded straight into LDS (buffer loads to LDS).
//   bwd_dkdv_kernel one workgroup per 128 (or 256) key rows: a loop over Q tiles in
//                   the orientation S = Q K^T (lanes own a key), so P and dS
//                   are directly the B operands of dV^T += dO^T P and
//                   dK^T += Q^T dS; dO^T and Q^T come from the row-major
//                   tiles through LDS transpose reads.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <typename T, int D, bool USE_DMA = false>
struct TileShape {
  static constexpr int EPC = 16 / sizeof(T);                // elements per 16-byte chunk
  // LDS row stride (elements). 16-bit rows are padded so that both fragment
  // patterns avoid bank conflicts: 16-byte row reads need a stride of 4 mod 8
  // dwords (the 16 rows a 16-lane group reads then land on distinct bank
  // quads), and transpose reads (ds_read_b64_tr_b16) measured 124 B/clk per CU
  // at 272 B against 193 at 144, 288 or 304 B. So 144 B at d = 64 and 304 B at
  // d = 128 (288 B left the row reads 2-way conflicted: +4-8% time).
  static constexpr int KS = D + (sizeof(T) == 2 ? (D == 128 ? 24 : 8) : 4);
  static constexpr int KCH = D / EPC;                       // 16-byte chunks per row
  // With USE_DMA, 16-bit d = 128 tiles are loaded straight into LDS by buffer
  // loads, whose lanes write 16-byte chunks contiguously: rows are then
  // unpadded and their chunks XOR-swizzled (lds_swizzle) instead. The dQ
  // kernel takes it (C4 dQ -8%); in the dK/dV kernel it measured 6% slower
  // than the register-staged loads.
  static constexpr bool DMA = USE_DMA && sizeof(T) == 2 && D == 128;
  static constexpr int RS = DMA ? D : KS;                   // tile row stride (elements)
  // Element (row, col) of a streamed tile; col is a multiple of 4. Padded
  // tiles store tile row r at LDS row lds_row(r) (conflict-free transpose
  // reads); swizzled tiles keep rows in place and move 16-byte chunks.
  static __device__ __forceinline__ int at(int row, int col) {
    if constexpr (DMA)
      return row * D + (((col / EPC) ^ lds_swizzle<D>(row)) * EPC) + (col % EPC);
    else
      return lds_row(row) * KS + col;
  }
  // Transposed fragment (load_frag_tr) of a streamed tile.
  static __device__ __forceinline__ typename Mfma<T>::frag tr(const T* tile, int base, int col0, int lane) {
    if constexpr (DMA)
      return load_frag_tr_swz<T, D>(tile, base, col0, lane);
    else
      return load_frag_tr_rp<T>(tile, KS, base, col0, lane);
  }
};

// ---------------------------------------------------------------------------
// dQ (and D_i)
// ---------------------------------------------------------------------------
template <typename T, typename G, int D, int BC, bool DROP, int WPE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE))) bwd_dq_kernel(AttnArgs a) {
  using S = TileShape<T, D, true>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KI = M::KI, KH = M::KH;
  constexpr int BR = 128;
  constexpr int NKB = BC / 32, NDB = D / 32, NC = D / KI;
  constexpr int NLD = BC * S::KCH / 256;
  constexpr int TILE = BC * S::RS;
  static_assert((BC * S::KCH) % 256 == 0, "tile shape");
  constexpr float NEG_INF = -__builtin_inff(), POS_INF = __builtin_inff();

  // Two tile buffers [K tile | V tile] as separate arrays, with the tile
  // loop unrolled by two, as in the forward kernel: the compiler then tells
  // the direct-to-LDS loads into one buffer from the reads of the other.
  __shared__ __attribute__((aligned(16))) T smem0[2 * TILE];
  __shared__ __attribute__((aligned(16))) T smem1[2 * TILE];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lo = lane & 31, hi = lane >> 5;
  const int N = a.N;
  const int nq = (N + BR - 1) / BR;
  const int rank = blockIdx.x / a.BH;
  const int bh = blockIdx.x - rank * a.BH;
  const int qt = a.causal ? (nq - 1 - rank) : rank;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const T* __restrict__ Qg = static_cast<const T*>(a.q) + hoff;
  const T* __restrict__ Kg = static_cast<const T*>(a.k) + hoff;
  const T* __restrict__ Vg = static_cast<const T*>(a.v) + hoff;
  const T* __restrict__ Og = static_cast<const T*>(a.o) + hoff;
  const T* __restrict__ dOg = static_cast<const T*>(a.dout) + hoff;
  G* __restrict__ dQg = static_cast<G*>(a.dq) + hoff;

  const int qtile0 = qt * BR;
  const int q0w = qtile0 + w * 32;
  const int q = q0w + lo;
  const bool qvalid = q < N;

  // Rows past the end are clamped to row N-1 (never stored; their P is 0),
  // so every load is unconditional.
  const int qc = min(q, N - 1);
  frag qf[NC], dof[NC];
  float dpart = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int off = qc * D + c * KI + hi * KH;
    qf[c] = load_frag<T>(Qg + off);
    dof[c] = load_frag<T>(dOg + off);
    const frag of = load_frag<T>(Og + off);
    if constexpr (KH == 8) {
#pragma unroll
      for (int t = 0; t < 8; ++t) dpart += to_f32<T>(dof[c][t]) * to_f32<T>(of[t]);
    } else {
      dpart += dof[c] * of;
    }
  }
  const float Dq = half_sum(dpart);
  // Rows without a valid key (LSE = -inf) and padding rows get P = 0.
  const float lraw = a.lse[(size_t)bh * N + qc];
  const float lse2 = (!qvalid || lraw == NEG_INF) ? POS_INF : lraw * kLog2e;
  if (qvalid && hi == 0) a.delta[(size_t)bh * N + q] = Dq;
  // The dP products start from -D' of this lane's query, so they yield
  // dP - D' directly. Without dropout D' = D; the 16 registers are spent
  // only on the 64-key tiles at d = 64 (the 32-key kernel fits 128 VGPRs
  // without them, which lets four waves share a SIMD). With dropout the
  // kernel computes dS' = dS (1 - p) = P * (Z * dP - D (1 - p)), D' =
  // D (1 - p), and the factor 1 / (1 - p) moves to dQ's final scale.
  constexpr bool kNegD = (DROP && D == 64) || (D == 64 && BC == 64);
  const float ndq = DROP ? -Dq * a.kq : -Dq;  // -D'
  f32x16 negd;
#pragma unroll
  for (int v = 0; v < 16; ++v) negd[v] = ndq;
  uint32_t rowhash = 0;
  if constexpr (DROP) {
    const uint32_t hk = head_key(a.seed_lo, a.seed_hi, (uint32_t)(bh / a.H), (uint32_t)(bh % a.H));
    rowhash = fmix32(hk ^ (uint32_t)q) + (uint32_t)(2 * hi);  // crow's 4*hi keys = 2*hi pairs
  }

  const int kend = a.causal ? min(N, qtile0 + BR) : N;
  const int ntiles = (kend + BC - 1) / BC;
  const uint8_t* bmrow = a.bmask ? a.bmask + (size_t)(qtile0 / a.mask_block) * a.nb : nullptr;
  const bool mfew = bmrow != nullptr && a.nb <= 64;  // the row's mask fits one 64-bit word
  const uint64_t mrow = mfew ? mask_bits(bmrow, 1, a.nb, lane) : ~0ull;
  auto kept = [&](int j) {
    if (bmrow == nullptr) return true;
    const int blk = (j * BC) / a.mask_block;
    return mfew ? ((mrow >> blk) & 1ull) != 0 : mask_kept(bmrow, blk);
  };
  auto next_kept = [&](int j) {
    ++j;
    while (j < ntiles && !kept(j)) ++j;
    return j;
  };

  u32x4 kreg[S::DMA ? 1 : NLD], vreg[S::DMA ? 1 : NLD];
  auto gload = [&](int jt) {  // rows past the end read as zeros (their scores are masked)
    const int k0 = jt * BC;
    const int rem = (N - k0) * D * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(Kg + (size_t)k0 * D, rem);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(Vg + (size_t)k0 * D, rem);
#pragma unroll
    for (int i = 0; i < (S::DMA ? 1 : NLD); ++i) {
      kreg[i] = buffer_load16(kr, (i * 256 + tid) * 16);
      vreg[i] = buffer_load16(vr, (i * 256 + tid) * 16);
    }
  };
  auto sstore = [&](T* dst) {
#pragma unroll
    for (int i = 0; i < (S::DMA ? 1 : NLD); ++i) {
      const int c = i * 256 + tid;
      const int row = lds_row(c / S::KCH), ch = c % S::KCH;
      *reinterpret_cast<u32x4*>(dst + row * S::KS + ch * S::EPC) = kreg[i];
      *reinterpret_cast<u32x4*>(dst + TILE + row * S::KS + ch * S::EPC) = vreg[i];
    }
  };
  // Direct-to-LDS variant: lane L of wave w fills LDS chunk i*256 + 64*w + L
  // (row c / KCH, physical chunk c % KCH) with the logical chunk the swizzle
  // puts there; rows past the end read as zeros (their scores are masked).
  // The wave index in a scalar register: each load's LDS address (M0) is
  // then scalar arithmetic rather than a vector value moved per load.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto dma = [&](int jt, T* dst) {
    const int k0 = jt * BC;
    const int rem = (N - k0) * D * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(Kg + (size_t)k0 * D, rem);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(Vg + (size_t)k0 * D, rem);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = i * 256 + tid, c0 = i * 256 + wu * 64;
      const int row = c / S::KCH;
      const int voff = (row * S::KCH + ((c % S::KCH) ^ lds_swizzle<D>(row))) * 16;
      buffer_load16_lds(kr, dst + c0 * S::EPC, voff);
      buffer_load16_lds(vr, dst + TILE + c0 * S::EPC, voff);
    }
  };

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = zero16();

  // Lane parts of the K^T transpose-read addresses (swizzled tiles).
  int2 trl[S::DMA ? NDB : 1];
  if constexpr (S::DMA) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) trl[db] = tr_swz_lane<T, D>(db * 32, lane);
  }

  int j = kept(0) ? 0 : next_kept(0);
  if (j < ntiles) {
    if constexpr (S::DMA) {
      dma(j, smem0);
      wait_vmem();
    } else {
      gload(j);
      sstore(smem0);
    }
  }
  __syncthreads();

  auto step = [&](auto rb_tag) {
    constexpr int RB_ = decltype(rb_tag)::value;
    T* const rd = RB_ == 0 ? smem0 : smem1;
    T* const nx = RB_ == 0 ? smem1 : smem0;
    const int jn = next_kept(j);
    if constexpr (S::DMA)
      dma(jn < ntiles ? jn : j, nx);  // nx was last read before the previous barrier
    else
      gload(jn < ntiles ? jn : j);  // unconditional prefetch (see the forward kernel)
    const T* Ks = rd;
    const T* Vs = rd + TILE;
    const int k0 = j * BC;
    const bool active = (q0w < N) && (!a.causal || k0 <= q0w + 31);
    if (active) {
      f32x16 s[NKB], dp[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = zero16();
        dp[kb] = kNegD ? negd : zero16();  // from -D the product yields dP - D directly
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int off = S::at(kb * 32 + lo, c * KI + hi * KH);
          s[kb] = M::run(load_frag<T>(Ks + off), qf[c], s[kb]);
          dp[kb] = M::run(load_frag<T>(Vs + off), dof[c], dp[kb]);
        }
      const bool need_mask = (a.causal && k0 + BC - 1 > q0w) || (k0 + BC > N);
      if (need_mask) {
        // Same single-compare masking as the forward kernel.
        const int t = (a.causal ? min(q, N - 1) : N - 1) - k0 - 4 * hi;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (kb * 32 + 8 * (v >> 2) + (v & 3) > t) s[kb][v] = NEG_INF;
      }
      const uint32_t y = (rowhash + (uint32_t)(k0 >> 1)) * kMixMul;  // pairs k0/2 + offset: one product per tile
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = exp2_fast(fmaf(s[kb][v], a.sl2, -lse2));
          float ds = kNegD ? dp[kb][v] : dp[kb][v] + ndq;  // dP - D'
          if constexpr (DROP) {  // Z * dP - D'; elements v, v + 1 (v even) share a keep word
            const uint32_t off = (uint32_t)(kb * 16 + 4 * (v >> 2) + ((v & 3) >> 1));
            const uint32_t x = keep_mix(y + off * kMixMul);
            const bool keep = (v & 1) ? keep_hi_mixed(x, a.thresh) : keep_lo_mixed(x, a.thresh);
            ds = keep ? ds : ndq;
          }
          s[kb][v] = p * ds;  // dS^T (times 1 - p with dropout)
        }
      if constexpr (KH == 8) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const frag b = frag4<T>(pack2<T>(s[kb][8 * hf + 0], s[kb][8 * hf + 1]), pack2<T>(s[kb][8 * hf + 2], s[kb][8 * hf + 3]),
                                    pack2<T>(s[kb][8 * hf + 4], s[kb][8 * hf + 5]), pack2<T>(s[kb][8 * hf + 6], s[kb][8 * hf + 7]));
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              if constexpr (S::DMA)
                dq[db] = M::run(load_frag_tr_lane<T, D>(Ks, kb * 32 + 16 * hf, trl[db]), b, dq[db]);
              else
                dq[db] = M::run(S::tr(Ks, kb * 32 + 16 * hf, db * 32, lane), b, dq[db]);
            }
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kl = S::at(kb * 32 + crow(v, hi), 0);
#pragma unroll
            for (int db = 0; db < NDB; ++db) dq[db] = M::run(Ks[kl + db * 32 + lo], s[kb][v], dq[db]);
          }
      }
    }
    if constexpr (S::DMA)
      wait_vmem();  // this wave's loads into nx have landed
    else
      sstore(nx);
    __syncthreads();
    j = jn;
  };
  while (j < ntiles) {
    step(std::integral_constant<int, 0>{});
    if (j >= ntiles) break;
    step(std::integral_constant<int, 1>{});
  }

  const float sc = DROP ? a.scale * a.rp : a.scale;
  if constexpr (D == 64 && sizeof(T) == 2) {
    // Staged through LDS as in the dK/dV kernel, one 32-column half at a
    // time (four waves' halves fit the tile buffers): each store then writes
    // 128 contiguous bytes of 8 rows. Row stride 36 floats: 16 consecutive
    // rows start on distinct bank quads.
    constexpr int RS = 32 + 4;
    constexpr int WAVE_FLOATS = 32 * RS;
    static_assert(sizeof(smem0) >= 2 * WAVE_FLOATS * sizeof(float), "staging space in each tile buffer");
    float* st = reinterpret_cast<float*>(w < 2 ? smem0 : smem1) + (w & 1) * WAVE_FLOATS;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = {dq[db][4 * g] * sc, dq[db][4 * g + 1] * sc, dq[db][4 * g + 2] * sc, dq[db][4 * g + 3] * sc};
        *reinterpret_cast<f32x4*>(&st[lo * RS + 8 * g + 4 * hi]) = x;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // 32 rows x 8 pieces of 4 values, 64 lanes
        const int c = i * 64 + lane;
        const int row = c >> 3, ch = c & 7;
        const f32x4 x = *reinterpret_cast<const f32x4*>(&st[row * RS + ch * 4]);
        if (q0w + row < N) store4<G>(dQg + (q0w + row) * D + db * 32 + ch * 4, x[0], x[1], x[2], x[3]);
      }
      __syncthreads();  // the area is reused for the next half
    }
  } else if (qvalid) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4<G>(dQg + q * D + db * 32 + 8 * g + 4 * hi, dq[db][4 * g] * sc, dq[db][4 * g + 1] * sc,
                  dq[db][4 * g + 2] * sc, dq[db][4 * g + 3] * sc);
  }
}

// ---------------------------------------------------------------------------
// dK and dV
// ---------------------------------------------------------------------------
// VLDS: keep the workgroup's V rows in LDS (read as B fragments every tile)
// instead of in registers, which frees 32 VGPRs per lane at d = 128.
// NW: waves per workgroup, each owning 32 keys (BK = 32 NW keys per
// workgroup). Eight waves (256 keys, one workgroup per CU at d = 128) share
// each Q/dO tile between twice the keys, halving the tile loads, LDS stores
// and barriers per key; a workgroup then spans two 128-key column blocks of
// a block mask, so the host takes four waves when there is one.
template <typename T, typename G, int D, int BR, bool DROP, int WPE, bool VLDS, int NW = 4>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE))) bwd_dkdv_kernel(AttnArgs a) {
  constexpr int NT = 64 * NW;
  using S = TileShape<T, D>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KI = M::KI, KH = M::KH;
  constexpr int BK = 32 * NW;  // keys per workgroup
  constexpr int NQB = BR / 32, NDB = D / 32, NC = D / KI;
  constexpr int NLD = BR * S::KCH / NT;
  constexpr int TILE = BR * S::RS;
  static_assert((BR * S::KCH) % NT == 0 && BR <= NT && BK % BR == 0, "tile shape");
  constexpr float NEG_INF = -__builtin_inff(), POS_INF = __builtin_inff();

  __shared__ __attribute__((aligned(16))) T smem[2][2 * TILE];  // [buffer][Q tile | dO tile]
  __shared__ __attribute__((aligned(16))) float side_l[2][BR];  // LSE in log2 units (+inf: no valid key)
  __shared__ __attribute__((aligned(16))) float side_d[2][BR];  // -D_i (times 1 - p with dropout)
  __shared__ __attribute__((aligned(16))) uint32_t side_h[2][BR];  // dropout row words, in the order r0 r2 r1 r3 per four rows
  __shared__ __attribute__((aligned(16))) T vsm[VLDS ? BK * S::KS : 8];  // V rows of this workgroup

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lo = lane & 31, hi = lane >> 5;
  const int N = a.N;
  const int rank = blockIdx.x / a.BH;
  const int bh = blockIdx.x - rank * a.BH;
  const int kt = rank;  // causal: low key tiles see the most query rows, so they go first
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const T* __restrict__ Qg = static_cast<const T*>(a.q) + hoff;
  const T* __restrict__ Kg = static_cast<const T*>(a.k) + hoff;
  const T* __restrict__ Vg = static_cast<const T*>(a.v) + hoff;
  const T* __restrict__ dOg = static_cast<const T*>(a.dout) + hoff;
  const float* __restrict__ Lg = a.lse + (size_t)bh * N;
  const float* __restrict__ Dg = a.delta + (size_t)bh * N;
  G* __restrict__ dKg = static_cast<G*>(a.dk) + hoff;
  G* __restrict__ dVg = static_cast<G*>(a.dv) + hoff;

  const int k0wg = kt * BK;
  const int k0w = k0wg + w * 32;
  const int key = k0w + lo;
  const bool kvalid = key < N;
  // Dropout: keys 2m and 2m + 1 (lanes lo and lo ^ 1 of a quad) share the
  // keep word of pair m; the even key reads its low 16 bits, the odd key its
  // high 16. For each two adjacent query rows r, r + 1 of a lane, the even
  // lane computes row r's word and the odd lane row r + 1's; a DPP swap
  // hands each lane the other word, and one byte permute gathers the lane's
  // two halves into one dword (row r low, row r + 1 high).
  const uint32_t keyh = (uint32_t)(key >> 1) * kMixMul;  // the row words in LDS are row * kMixMul
  const bool odd = (lo & 1) != 0;
  // v_perm_b32(nb, own, sel): bytes 0-3 select own, 4-7 nb.
  const uint32_t psel = odd ? 0x03020706u : 0x05040100u;
  const uint32_t t16 = a.thresh >> 16;

  // Keys past the end are clamped to row N-1: their scores are masked and
  // their gradients never stored.
  frag kf[NC], vf[VLDS ? 1 : NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int off = min(key, N - 1) * D + c * KI + hi * KH;
    kf[c] = load_frag<T>(Kg + off);
    if constexpr (!VLDS) vf[c] = load_frag<T>(Vg + off);
  }
  if constexpr (VLDS) {
    constexpr int NLV = BK * S::KCH / NT;
#pragma unroll
    for (int i = 0; i < NLV; ++i) {
      const int c = i * NT + tid;
      const int row = c / S::KCH, ch = c % S::KCH;
      *reinterpret_cast<u32x4*>(&vsm[row * S::KS + ch * S::EPC]) =
          *reinterpret_cast<const u32x4*>(Vg + (size_t)min(k0wg + row, N - 1) * D + ch * S::EPC);
    }
  }
  uint32_t hk = 0;
  if constexpr (DROP) hk = head_key(a.seed_lo, a.seed_hi, (uint32_t)(bh / a.H), (uint32_t)(bh % a.H));

  // Query tiles this workgroup visits: causal starts at its diagonal; a
  // block mask skips query tiles whose (row block, this column block) is empty.
  const int nqt = (N + BR - 1) / BR;
  const int istart = a.causal ? (k0wg / BR) : 0;
  const int cblk = k0wg / a.mask_block;
  const bool mfew = a.bmask != nullptr && a.nb <= 64;  // the column's mask fits one 64-bit word
  const uint64_t mcol = mfew ? mask_bits(a.bmask + cblk, a.nb, a.nb, lane) : ~0ull;
  auto kept = [&](int i) {
    if (a.bmask == nullptr) return true;
    const int blk = (i * BR) / a.mask_block;
    return mfew ? ((mcol >> blk) & 1ull) != 0 : mask_kept(a.bmask, blk * a.nb + cblk);
  };
  // Query tiles run from the end of the sequence down to the diagonal: every
  // key block of a head then reads the same Q/dO tile at the same iteration,
  // so the workgroups of a head running together share it through L2.
  auto prev_kept = [&](int i) {
    --i;
    while (i >= istart && !kept(i)) --i;
    return i;
  };

  u32x4 qreg[NLD], oreg[NLD];
  float l_reg = POS_INF, d_reg = 0.f;
  uint32_t h_reg = 0;
  auto gload = [&](int it) {
    // Buffer loads over the tile (the resource starts at its first row):
    // rows past the end read as zeros, and the lane offsets are 32-bit
    // constants (the 64-bit address arithmetic of flat loads measured 2-3%
    // of the kernel).
    const int i0 = it * BR;
    const int rem = (N - i0) * D * (int)sizeof(T);
    const __amdgpu_buffer_rsrc_t qr = buffer_rsrc(Qg + (size_t)i0 * D, rem);
    const __amdgpu_buffer_rsrc_t orr = buffer_rsrc(dOg + (size_t)i0 * D, rem);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {  // chunk c = row c / KCH, 16-byte piece c % KCH
      qreg[i] = buffer_load16(qr, (i * NT + tid) * 16);
      oreg[i] = buffer_load16(orr, (i * NT + tid) * 16);
    }
    // Row statistics of the tile: every lane loads, lanes < BR keep. Padding
    // rows (and rows with no valid key) get log2-LSE = +inf, so P = 0.
    const int qi = i0 + (tid % BR);
    const int rem4 = (N - i0) * 4;
    const float l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(Lg + i0, rem4), (tid % BR) * 4, 0, 0));
    const float dd = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(Dg + i0, rem4), (tid % BR) * 4, 0, 0));
    l_reg = (qi >= N || l == NEG_INF) ? POS_INF : l * kLog2e;
    d_reg = DROP ? -dd * a.kq : -dd;  // -D', D' = D (1 - p) with dropout
    if constexpr (DROP) h_reg = fmix32(hk ^ (uint32_t)qi) * kMixMul;  // row word times the first multiplier
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int c = i * NT + tid;
      const int row = lds_row(c / S::KCH), ch = c % S::KCH;
      *reinterpret_cast<u32x4*>(&smem[buf][row * S::KS + ch * S::EPC]) = qreg[i];
      *reinterpret_cast<u32x4*>(&smem[buf][TILE + row * S::KS + ch * S::EPC]) = oreg[i];
    }
    if (tid < BR) {
      side_l[buf][tid] = l_reg;
      side_d[buf][tid] = d_reg;
      // Rows r0..r3 of each group of four are kept in the order r0 r2 r1 r3:
      // an even lane reads its words (r0, r2) and an odd lane (r1, r3) as
      // one 8-byte load.
      side_h[buf][(tid & ~3) | ((tid & 1) << 1) | ((tid >> 1) & 1)] = h_reg;
    }
  };

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  int it = nqt - 1 >= istart && kept(nqt - 1) ? nqt - 1 : prev_kept(nqt - 1);
  if (it >= istart) {
    gload(it);
    sstore(0);
  }
  __syncthreads();

  // The loop body is in fa_bwd_dkdv_tile.inc. At d = 64 with one query
  // block per tile the loop is unrolled by two, so every access names its
  // buffer at compile time (C2 dK/dV -2%); with two query blocks that spills
  // registers, and the d = 128 kernels keep the plain loop.
  if constexpr (D == 64 && NQB == 1) {
    while (it >= istart) {
      {
        constexpr int cur = 0;
#include "fa_bwd_dkdv_tile.inc"
      }
      if (it < istart) break;
      {
        constexpr int cur = 1;
#include "fa_bwd_dkdv_tile.inc"
      }
    }
  } else {
    int cur = 0;
    while (it >= istart) {
#include "fa_bwd_dkdv_tile.inc"
      cur ^= 1;
    }
  }

  const float sc = DROP ? a.scale * a.rp : a.scale;  // dK = scale * sum_i dS'_ij Q_i / (1 - p)
  const float sv = DROP ? a.rp : 1.f;                // dV = sum_i (P * Z)_ij dO_i / (1 - p)
  if constexpr (D == 64 && sizeof(T) == 2) {
    // A lane holds 4-value pieces of 32 rows, so a direct store writes 32
    // bytes to each of 32 rows. Each wave instead stages its 32 rows in LDS
    // (the tile buffers are free now) and stores four whole rows per
    // instruction. Row stride 68 floats: the pieces of 16 rows land on
    // distinct bank quads.
    constexpr int RS = D + 4;
    constexpr int WAVE_FLOATS = 32 * RS;
    static_assert(NW == 4, "the staging areas below hold four waves' rows");
    static_assert(sizeof(smem) >= (VLDS ? 2 : 4) * WAVE_FLOATS * sizeof(float), "staging space in the tile buffers");
    static_assert(!VLDS || sizeof(vsm) >= 2 * WAVE_FLOATS * sizeof(float), "staging space in the V rows");
    float* st;
    if constexpr (VLDS)
      st = (w < 2 ? reinterpret_cast<float*>(&smem[0][0]) : reinterpret_cast<float*>(&vsm[0])) + (w & 1) * WAVE_FLOATS;
    else
      st = reinterpret_cast<float*>(&smem[0][0]) + w * WAVE_FLOATS;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const f32x16* acc = t == 0 ? dk : dv;
      const float f = t == 0 ? sc : sv;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 x = {acc[db][4 * g] * f, acc[db][4 * g + 1] * f, acc[db][4 * g + 2] * f, acc[db][4 * g + 3] * f};
          *reinterpret_cast<f32x4*>(&st[lo * RS + db * 32 + 8 * g + 4 * hi]) = x;
        }
      __syncthreads();
      G* __restrict__ dst = t == 0 ? dKg : dVg;
#pragma unroll
      for (int i = 0; i < 8; ++i) {  // 32 rows x 16 pieces of 4 values, 64 lanes
        const int c = i * 64 + lane;
        const int row = c >> 4, ch = c & 15;
        const f32x4 x = *reinterpret_cast<const f32x4*>(&st[row * RS + ch * 4]);
        if (k0w + row < N) store4<G>(dst + (k0w + row) * D + ch * 4, x[0], x[1], x[2], x[3]);
      }
      __syncthreads();  // the area is reused for dV
    }
  } else if (kvalid) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int off = key * D + db * 32 + 8 * g + 4 * hi;
        store4<G>(dKg + off, dk[db][4 * g] * sc, dk[db][4 * g + 1] * sc, dk[db][4 * g + 2] * sc,
                  dk[db][4 * g + 3] * sc);
        store4<G>(dVg + off, dv[db][4 * g] * sv, dv[db][4 * g + 1] * sv, dv[db][4 * g + 2] * sv,
                  dv[db][4 * g + 3] * sv);
      }
  }
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
// Launch configurations. A dQ workgroup streams BC-key tiles; a dK/dV
// workgroup streams BR-query tiles; WPE is the resident waves per SIMD the
// kernel is compiled for (more waves overlap one wave's softmax and LDS
// work with another's MFMAs, at the price of registers). Short sequences
// (causal rows of at most a few thousand keys) run few tiles per workgroup,
// so they take small tiles and high occupancy; long ones take larger tiles,
// which amortize the per-tile barrier and loads. With VLDS the dK/dV kernel
// keeps the workgroup's V rows in LDS instead of registers. At d = 128 the
// dK/dV kernel runs eight waves (256 keys) per workgroup unless a block mask
// is given (C4 dK/dV -2.7%); at d = 64 eight waves measured slower (+6% at
// 4096 keys with 64-row tiles) and the d = 64 epilogue stages four waves.
template <typename T, typename G, int D, bool DROP, int BC, int WPE>
static hipError_t launch_dq(const AttnArgs& a, hipStream_t s) {
  const int nt = (a.N + 127) / 128;
  bwd_dq_kernel<T, G, D, BC, DROP, WPE><<<dim3((unsigned)(nt * a.BH)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

template <typename T, typename G, int D, bool DROP, int BR, int WPE, bool VLDS, int NW = 4>
static hipError_t launch_dkdv(const AttnArgs& a, hipStream_t s) {
  const int nt = (a.N + 32 * NW - 1) / (32 * NW);
  bwd_dkdv_kernel<T, G, D, BR, DROP, WPE, VLDS, NW><<<dim3((unsigned)(nt * a.BH)), dim3(64 * NW), 0, s>>>(a);
  return hipGetLastError();
}

template <typename T, typename G, int D, bool DROP>
static hipError_t launch_bwd_cfg(int stage, const AttnArgs& a, hipStream_t s) {
  constexpr bool h = sizeof(T) == 2;
  hipError_t e = hipSuccess;
  if (stage & 1) {
    if constexpr (!h)
      e = launch_dq<T, G, D, DROP, D == 64 ? 64 : 32, 1>(a, s);
    else if constexpr (D == 128)
      e = launch_dq<T, G, D, DROP, 64, 2>(a, s);
    else
      e = a.N <= 4096 ? launch_dq<T, G, D, DROP, 32, DROP ? 2 : 3>(a, s) : launch_dq<T, G, D, DROP, 64, 2>(a, s);
    if (e != hipSuccess) return e;
  }
  if (stage & 2) {
    if constexpr (!h)
      e = launch_dkdv<T, G, D, DROP, D == 64 ? 64 : 32, 1, false>(a, s);
    else if constexpr (D == 128)
      e = a.bmask ? launch_dkdv<T, G, D, DROP, 32, 2, true>(a, s) : launch_dkdv<T, G, D, DROP, 32, 2, true, 8>(a, s);
    else
      e = a.N <= 2048 ? launch_dkdv<T, G, D, DROP, 32, DROP ? 2 : 3, true>(a, s)
                      : launch_dkdv<T, G, D, DROP, 64, 2, false>(a, s);
  }
  return e;
}

template <typename T, typename G>
static hipError_t launch_bwd_g(int d, bool dropout, int stage, const AttnArgs& a, hipStream_t s) {
  if (d == 64)
    return dropout ? launch_bwd_cfg<T, G, 64, true>(stage, a, s) : launch_bwd_cfg<T, G, 64, false>(stage, a, s);
  return dropout ? launch_bwd_cfg<T, G, 128, true>(stage, a, s) : launch_bwd_cfg<T, G, 128, false>(stage, a, s);
}

hipError_t launch_bwd(Elt t, Elt gt, int d, bool dropout, int stage, const AttnArgs& a, hipStream_t s) {
  const bool f32grad = gt == Elt::F32;
  switch (t) {
    case Elt::BF16:
      return f32grad ? launch_bwd_g<__bf16, float>(d, dropout, stage, a, s)
                     : launch_bwd_g<__bf16, __bf16>(d, dropout, stage, a, s);
    case Elt::F16:
      return f32grad ? launch_bwd_g<_Float16, float>(d, dropout, stage, a, s)
                     : launch_bwd_g<_Float16, _Float16>(d, dropout, stage, a, s);
    case Elt::F32:
      return launch_bwd_g<float, float>(d, dropout, stage, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
