// Forward pass of tiled exact attention for gfx950.
//
// One workgroup (4 waves, 256 lanes) owns 128 query rows of one (b, h)
// slice; each wave owns 32 of them and keeps their Q fragments in
// registers for the whole kernel. K and V tiles of BC keys stream through
// LDS (double buffered: the next tile is fetched while the current one is
// consumed, staged through registers, or at d = 128 loaded straight into
// LDS by buffer loads), so the N x N score matrix exists only as
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
//   input type, are directly the B operand, so P never touches LDS; the V^T
//   A operand is read from the row-major V tile with LDS transpose reads.
// Epilogue: O = O / l / (1 - p), LSE = m + log l (natural log).
#include "fa_device.h"
#include "fa_kernels.h"



namespace fa {

template <typename T, int D, int BC, int QB>
struct FwdCfg {
  static constexpr int BR = 128 * QB;                       // queries per workgroup (4 waves x 32 x QB)
  static constexpr int EPC = 16 / sizeof(T);                // elements per 16-byte chunk
  // K/V tile row stride (elements). 16-bit rows are padded so that both fragment
  // patterns avoid bank conflicts: 16-byte row reads need a stride of 4 mod 8
  // dwords (the 16 rows a 16-lane group reads then land on distinct bank
  // quads), and transpose reads (ds_read_b64_tr_b16) measured 124 B/clk per CU
  // at 272 B against 193 at 144, 288 or 304 B. So 144 B at d = 64 and 304 B at
  // d = 128 (288 B left the row reads 2-way conflicted: +4-8% time).
  static constexpr int KS = D + (sizeof(T) == 2 ? (D == 128 ? 24 : 8) : 4);
  static constexpr int KCH = D / EPC;                       // 16-byte chunks per K/V row
  static constexpr int NLD = BC * KCH / 256;                // 16-byte loads per lane per tensor per tile
  // 16-bit d = 128 tiles arrive by direct-to-LDS buffer loads: each load
  // instruction writes its 64 lanes' 16-byte chunks contiguously, so rows are
  // unpadded and the chunks of a row are XOR-swizzled instead (lds_swizzle).
  // This frees the 32 staging registers and the LDS stores of the
  // register-staged prefetch: C4 forward -4%. At d = 64 the staged prefetch
  // measured the same at 1024 keys and 1% faster at 4096 and 8192.
  static constexpr bool DMA = sizeof(T) == 2 && D == 128;
  static constexpr int TILE = DMA ? BC * D : BC * KS;       // elements per K (or V) tile
  static_assert(BC % 32 == 0 && (BC * KCH) % 256 == 0, "tile shape");
  static_assert((TILE * sizeof(T)) % 16 == 0, "V tile base alignment");
};

// Rows whose running maximum grew by at most this much (log2 units) keep the
// stale maximum: exponents stay below 2^8, which fp32 sums and the 8-bit
// exponent of bf16/fp16-rounded P absorb, and the O rescale is skipped.
constexpr float kLazyRescale = 8.0f;

// QB: 32-query blocks per wave. Every K fragment and every V^T transpose read
// taken from LDS feeds QB MFMAs, which divides the LDS read traffic per
// flop by QB. Wave w owns the query blocks w, w + 4, ... of the workgroup
// tile, so causal work is spread evenly over the waves. The launches use
// QB = 1 (QB = 2 measured slower at every workload: the register file then
// holds two waves per SIMD); a workgroup of QB > 1 spans 128 * QB rows but
// reads the block-mask row of its first 128, so the host refuses QB > 1 with
// a block mask.
template <typename T, int D, int BC, int QB, bool DROP, int WPE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE))) fwd_kernel(AttnArgs a) {
  using C = FwdCfg<T, D, BC, QB>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KI = M::KI, KH = M::KH;
  constexpr int NKB = BC / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;   // 32-column blocks of O^T
  constexpr int NC = D / KI;    // MFMA steps over d for S
  constexpr int RB = D * (int)sizeof(T);  // bytes per row
  constexpr float NEG_INF = -__builtin_inff();

  // The two tile buffers, each [K tile | V tile] row-major, are separate
  // arrays and the tile loop below is unrolled by two, so every access names
  // its buffer at compile time. The compiler can then tell the direct-to-LDS
  // loads into one buffer from the reads of the other; with one indexed array
  // it waits for those loads before the first transpose read of each tile.
  __shared__ __attribute__((aligned(16))) T smem0[2 * C::TILE];
  __shared__ __attribute__((aligned(16))) T smem1[2 * C::TILE];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lo = lane & 31, hi = lane >> 5;

  // Causal: longest rows first; a grid that fits the device's CUs at WPE
  // workgroups each balances their loads (tile_order).
  const int N = a.N;
  const int nq = (N + C::BR - 1) / C::BR;
  int rank, bh;
  tile_order((int)blockIdx.x, nq, a.BH, a.causal && nq * a.BH <= a.ncu * WPE, a.ncu, a.nxcd, rank, bh);
  const int qt = a.causal ? (nq - 1 - rank) : rank;
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const T* __restrict__ Kg = static_cast<const T*>(a.k) + hoff;
  const T* __restrict__ Vg = static_cast<const T*>(a.v) + hoff;

  const int qtile0 = qt * C::BR;
  int q0b[QB], qb_[QB];  // first query of each of this wave's blocks; this lane's query
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    q0b[b] = qtile0 + (w + 4 * b) * 32;
    qb_[b] = q0b[b] + lo;
  }
  const int qlast = q0b[QB - 1] + 31;  // the wave's highest query

  // Buffer accesses: rows past the end read as zeros (their scores are
  // masked) and their stores are dropped.
  const __amdgpu_buffer_rsrc_t qrs = buffer_rsrc(static_cast<const T*>(a.q) + hoff, N * RB);
  frag qf[QB][NC];
#pragma unroll
  for (int b = 0; b < QB; ++b)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if constexpr (KH == 8)
        qf[b][c] = __builtin_bit_cast(frag, buffer_load16(qrs, qb_[b] * RB + (c * KI + hi * KH) * (int)sizeof(T)));
      else
        qf[b][c] =
            __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qrs, qb_[b] * RB + (c * KI + hi) * 4, 0, 0));
    }

  uint32_t rowhash[QB];
  if constexpr (DROP) {
    const uint32_t hk = head_key(a.seed_lo, a.seed_hi, (uint32_t)(bh / a.H), (uint32_t)(bh % a.H));
#pragma unroll
    for (int b = 0; b < QB; ++b) rowhash[b] = fmix32(hk ^ (uint32_t)qb_[b]) + (uint32_t)(2 * hi);  // crow's 4*hi keys = 2*hi pairs
  }

  // KV tiles this workgroup visits: causal stops at its diagonal; a block
  // mask skips the tiles of empty blocks (block-sparse variant).
  const int kend = a.causal ? min(N, qtile0 + C::BR) : N;
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

  // Lane-constant byte offsets of this lane's 16-byte chunks within a tile.
  int voff[C::NLD];
#pragma unroll
  for (int i = 0; i < C::NLD; ++i) {
    const int c = i * 256 + tid;
    const int row = c / C::KCH;
    voff[i] = row * RB + ((c % C::KCH) ^ (C::DMA ? lds_swizzle<D>(row) : 0)) * 16;
  }
  u32x4 kreg[C::DMA ? 1 : C::NLD], vreg[C::DMA ? 1 : C::NLD];
  // 16-bit: K and V tiles go straight from HBM into LDS buffer `buf`; lane L
  // of wave w fills LDS chunk i*256 + 64*w + L, i.e. row c / KCH and physical
  // chunk c % KCH, with the logical chunk that the swizzle places there.
  // The wave index is read into a scalar register, so each load's LDS
  // address (M0) is scalar arithmetic rather than a vector value moved to a
  // scalar register per load.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  auto dma = [&](int jt, T* dst) {
    const int k0 = jt * BC;
    const int rem = (N - k0) * RB;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(Kg + (size_t)k0 * D, rem);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(Vg + (size_t)k0 * D, rem);
#pragma unroll
    for (int i = 0; i < C::NLD; ++i) {
      const int c0 = i * 256 + wu * 64;  // first chunk this wave writes
      buffer_load16_lds(kr, dst + c0 * C::EPC, voff[i]);
      buffer_load16_lds(vr, dst + C::TILE + c0 * C::EPC, voff[i]);
    }
  };
  auto gload = [&](int jt) {
    const int k0 = jt * BC;
    const int rem = (N - k0) * RB;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(Kg + (size_t)k0 * D, rem);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(Vg + (size_t)k0 * D, rem);
#pragma unroll
    for (int i = 0; i < (C::DMA ? 1 : C::NLD); ++i) {
      kreg[i] = buffer_load16(kr, voff[i]);
      vreg[i] = buffer_load16(vr, voff[i]);
    }
  };
  auto sstore = [&](T* dst) {
#pragma unroll
    for (int i = 0; i < (C::DMA ? 1 : C::NLD); ++i) {
      const int c = i * 256 + tid;
      const int row = lds_row(c / C::KCH), ch = c % C::KCH;
      *reinterpret_cast<u32x4*>(dst + row * C::KS + ch * C::EPC) = kreg[i];
      *reinterpret_cast<u32x4*>(dst + C::TILE + row * C::KS + ch * C::EPC) = vreg[i];
    }
  };

  f32x16 o[QB][NDB];
  float m_run[QB], l_run[QB];  // l_run: per-lane partial row sums
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    m_run[b] = NEG_INF;
    l_run[b] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[b][db] = zero16();
  }

  // Lane parts of the V^T transpose-read addresses (swizzled tiles).
  int2 trl[C::DMA ? NDB : 1];
  if constexpr (C::DMA) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) trl[db] = tr_swz_lane<T, D>(db * 32, lane);
  }

  int j = kept(0) ? 0 : next_kept(0);
  if (j < ntiles) {
    if constexpr (C::DMA) {
      dma(j, smem0);
      wait_vmem();
    } else {
      gload(j);
      sstore(smem0);
    }
  }
  __syncthreads();

  // One tile step: compute on buffer RB while the next tile loads into the
  // other one.
  auto step = [&](auto rb_tag) {
    constexpr int RB_ = decltype(rb_tag)::value;
    T* const rd = RB_ == 0 ? smem0 : smem1;
    T* const nx = RB_ == 0 ? smem1 : smem0;
    const int jn = next_kept(j);
    // Always prefetch (the last iteration reloads its own tile into the idle
    // buffer), so the loads are unconditional and the compiler's wait
    // counting keeps them in flight across the compute below. nx was last
    // read before the previous barrier. Direct-to-LDS loads go out after the
    // S products, so the K fragment reads that open the step do not share
    // the LDS with their writes (C4 forward -2.3 to -3.2%).
    const int jl = jn < ntiles ? jn : j;
    if constexpr (!C::DMA) gload(jl);

    const T* Ks = rd;
    const T* Vs = rd + C::TILE;
    const int k0 = j * BC;
    // The wave has work unless every key of the tile is above all its rows.
    const bool active = (q0b[0] < N) && (!a.causal || k0 <= qlast);
    if (active) {
      f32x16 s[QB][NKB];
      uint32_t pk[QB][NKB][8];  // 16-bit operand types: P as packed pairs
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[b][kb] = zero16();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          frag kf;
          if constexpr (C::DMA) {
            const int row = kb * 32 + lo;
            kf = load_frag<T>(Ks + row * D + (((c * KI + hi * KH) / C::EPC) ^ lds_swizzle<D>(row)) * C::EPC);
          } else {
            kf = load_frag<T>(Ks + lds_row(kb * 32 + lo) * C::KS + c * KI + hi * KH);
          }
#pragma unroll
          for (int b = 0; b < QB; ++b) s[b][kb] = M::run(kf, qf[b][c], s[b][kb]);
        }
      }
      if constexpr (C::DMA) dma(jl, nx);

#pragma unroll
      for (int b = 0; b < QB; ++b) {
        const bool need_mask = (a.causal && k0 + BC - 1 > q0b[b]) || (k0 + BC > N);
        if (need_mask) {
          // Hide keys past min(q, N-1) (causal) or past N-1; key - k0 is a
          // compile-time offset plus 4*hi, so each element costs one compare.
          // The lane terms are recomputed here (q0b is wave-uniform), which
          // keeps them out of the registers live across the tile loop.
          const int ln = lane_id();
          const int t = (a.causal ? min(q0b[b] + (ln & 31), N - 1) : N - 1) - k0 - 4 * (ln >> 5);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (kb * 32 + 8 * (v >> 2) + (v & 3) > t) s[b][kb][v] = NEG_INF;
        }

        float mx = NEG_INF;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[b][kb][v]);
        // A query's keys sit in two lanes. The rescale is needed iff one of
        // them holds a score above the threshold, so the lane's own maximum
        // decides it and the exchange of the halves runs only then.
        if (wave_any(mx * a.sl2 > m_run[b] + kLazyRescale)) {
          const float mnew = fmaxf(m_run[b], half_max(mx) * a.sl2);
          const float alpha = exp2_fast(m_run[b] - (mnew == NEG_INF ? 0.f : mnew));
          m_run[b] = mnew;
          l_run[b] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[b][db][v] *= alpha;
        }
        const float base = (m_run[b] == NEG_INF) ? 0.f : m_run[b];
        if constexpr (KH == 8) {
          // P goes straight to packed 16-bit pairs (the MFMA operand); the
          // row sum adds the fp32 values, so LSE keeps fp32 accuracy.
          float rs = 0.f;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float p0 = exp2_fast(fmaf(s[b][kb][2 * e], a.sl2, -base));
              const float p1 = exp2_fast(fmaf(s[b][kb][2 * e + 1], a.sl2, -base));
              pk[b][kb][e] = pack2<T>(p0, p1);
              rs += p0 + p1;
            }
          l_run[b] += rs;
        } else {
          float rs = 0.f;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const float p = exp2_fast(fmaf(s[b][kb][v], a.sl2, -base));
              rs += p;
              s[b][kb][v] = p;
            }
          l_run[b] += rs;
        }

        if constexpr (DROP && KH != 8) {
          // Keys k0 + kb*32 + crow(v, hi); elements v and v + 1 (v even) are
          // the two keys of pair k0/2 + kb*16 + 4*(v/4) + 2*hi + (v%4)/2: one
          // product per tile, then a constant per pair (keep_finish) whose
          // low half decides the even key and high half the odd one. (The
          // 16-bit path applies the same bits to packed P below.)
          const uint32_t y = (rowhash[b] + (uint32_t)(k0 >> 1)) * kMixMul;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
              const uint32_t off = (uint32_t)(kb * 16 + 4 * (v >> 2) + ((v & 3) >> 1));
              const uint32_t u = keep_finish(y + off * kMixMul);
              s[b][kb][v] = keep_lo(u, a.thresh) ? s[b][kb][v] : 0.f;
              s[b][kb][v + 1] = keep_hi(u, a.thresh) ? s[b][kb][v + 1] : 0.f;
            }
        }
      }

      // O^T += V^T P^T: P^T is the B operand straight from registers; V^T
      // comes from the row-major V tile through LDS transpose reads.
      if constexpr (KH == 8) {
        // Dropout on the packed P: the 16-bit values of a dword are the two
        // keys of one pair (elements 8*hf + 2e, + 1: pair k0/2 + kb*16 +
        // 8*hf + {0, 1, 4, 5}[e] + 2*hi), so the pair's keep word zeroes them
        // with packed integer ops (keep01). The host never launches the
        // dropout kernels with T16 = 0 (every key kept: the plain kernel,
        // whose epilogue applies 1 / (1 - p) too).
        const u16x2 tm1 = {(unsigned short)((a.thresh >> 16) - 1u), (unsigned short)((a.thresh >> 16) - 1u)};
        const u16x2 ones = __builtin_bit_cast(u16x2, a.ones16);
        uint32_t ytile[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) ytile[b] = DROP ? (rowhash[b] + (uint32_t)(k0 >> 1)) * kMixMul : 0u;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            frag pb[QB];
#pragma unroll
            for (int b = 0; b < QB; ++b) {
              uint32_t d4[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                d4[e] = pk[b][kb][4 * hf + e];
                if constexpr (DROP) {
                  const uint32_t off = (uint32_t)(kb * 16 + 8 * hf + 4 * (e >> 1) + (e & 1));
                  d4[e] = keep_pair(d4[e], keep_finish(ytile[b] + off * kMixMul), tm1, ones);
                }
              }
              pb[b] = frag4<T>(d4[0], d4[1], d4[2], d4[3]);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              frag vt;
              if constexpr (C::DMA)
                vt = load_frag_tr_lane<T, D>(Vs, kb * 32 + 16 * hf, trl[db]);
              else
                vt = load_frag_tr_rp<T>(Vs, C::KS, kb * 32 + 16 * hf, db * 32, lane);
#pragma unroll
              for (int b = 0; b < QB; ++b) o[b][db] = M::run(vt, pb[b], o[b][db]);
            }
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kk = lds_row(kb * 32 + crow(v, hi));
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              const float vt = Vs[kk * C::KS + db * 32 + lo];
#pragma unroll
              for (int b = 0; b < QB; ++b) o[b][db] = M::run(vt, s[b][kb][v], o[b][db]);
            }
          }
      }
    }

    if constexpr (C::DMA) {
      if (!active) dma(jl, nx);
      wait_vmem();  // this wave's loads into nx have landed
    } else {
      sstore(nx);
    }
    __syncthreads();
    j = jn;
  };
  while (j < ntiles) {
    step(std::integral_constant<int, 0>{});
    if (j >= ntiles) break;
    step(std::integral_constant<int, 1>{});
  }

  const __amdgpu_buffer_rsrc_t ors = buffer_rsrc(static_cast<T*>(a.out) + hoff, N * RB);
  const __amdgpu_buffer_rsrc_t lrs = buffer_rsrc(a.lse + (size_t)bh * N, N * 4);
  if constexpr (D == 64 && QB == 1 && sizeof(T) == 2) {
    // A lane holds 4-value pieces of its row, so a direct store writes 8
    // bytes to each of 32 rows. Each wave instead stages its 32 rows in the
    // tile buffers (free after the loop's last barrier) and stores 8 whole
    // rows per instruction; rows past the end fall outside the buffer
    // resource and are dropped. Row stride 72 elements (144 bytes): 16
    // consecutive rows start on distinct bank quads.
    typedef T t4 __attribute__((ext_vector_type(4)));
    constexpr int RSE = D + 8;
    constexpr int WAVE_ELTS = 32 * RSE;
    static_assert(sizeof(smem0) >= 4 * WAVE_ELTS * sizeof(T), "staging space in the first tile buffer");
    T* st = smem0 + w * WAVE_ELTS;
    const float lt = half_sum(l_run[0]);
    const float inv = lt > 0.f ? a.rp / lt : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        t4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = static_cast<T>(o[0][db][4 * g + e] * inv);
        *reinterpret_cast<t4*>(&st[lo * RSE + db * 32 + 8 * g + 4 * hi]) = r;
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // 32 rows x 8 pieces of 16 bytes, 64 lanes
      const int c = i * 64 + lane;
      const int row = c >> 3, ch = c & 7;
      buffer_store16(ors, (q0b[0] + row) * RB + ch * 16, *reinterpret_cast<const u32x4*>(&st[row * RSE + ch * 8]));
    }
    buffer_store4(lrs, hi ? 0x7FFFFFF0 : qb_[0] * 4, lt > 0.f ? (m_run[0] + log2_fast(lt)) * kLn2 : NEG_INF);
    return;
  }
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float lt = half_sum(l_run[b]);
    const float inv = lt > 0.f ? a.rp / lt : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int off = qb_[b] * RB + (db * 32 + 8 * g + 4 * hi) * (int)sizeof(T);
        if constexpr (sizeof(T) == 2) {
          typedef T t4 __attribute__((ext_vector_type(4)));
          t4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = static_cast<T>(o[b][db][4 * g + e] * inv);
          buffer_store8(ors, off, __builtin_bit_cast(u32x2, r));
        } else {
          f32x4 r;
#pragma unroll
          for (int e = 0; e < 4; ++e) r[e] = o[b][db][4 * g + e] * inv;
          buffer_store16(ors, off, __builtin_bit_cast(u32x4, r));
        }
      }
    // One writer per row (lanes of the upper half aim past the end and are dropped).
    buffer_store4(lrs, hi ? 0x7FFFFFF0 : qb_[b] * 4, lt > 0.f ? (m_run[b] + log2_fast(lt)) * kLn2 : NEG_INF);
  }
}

// Split-key forward for grids too small to fill the device (few heads and
// short sequences: one 128-row tile per head would leave most CUs idle and
// give each wave a long serial chain of MFMAs). A workgroup owns 32 query
// rows; its four waves take the key tiles j = w, w + 4, ... (32 keys each,
// so causal work spreads evenly), each with its own LDS tile and its own
// running maximum and sum, and the four partial results are merged in LDS
// at the end with the same rescaling the online softmax uses between tiles
// (FlashAttention milestone page, "The idea": two running numbers per row,
// partial results rescaled to a common maximum).
template <typename T, int D>
struct SplitCfg {
  static constexpr int BC = 32;                             // keys per wave tile
  static constexpr int EPC = 16 / sizeof(T);                // elements per 16-byte chunk
  static constexpr int KS = D + (D == 128 ? 24 : 8);         // padded LDS row (elements)
  static constexpr int KCH = D / EPC;                       // 16-byte chunks per row
  static constexpr int NLD = BC * KCH / 64;                 // 16-byte loads per lane per tensor per tile
  static constexpr int TILE = BC * KS;                      // elements per K (or V) tile
  static constexpr int OS = D + 4;                          // fp32 row stride of the partial O
  static constexpr int TILE_BYTES = 4 * 2 * TILE * (int)sizeof(T);
  static constexpr int COMB_BYTES = 4 * 32 * OS * 4;
  static constexpr int BYTES = TILE_BYTES > COMB_BYTES ? TILE_BYTES : COMB_BYTES;
};

template <typename T, int D, bool DROP>
__global__ void __launch_bounds__(256) fwd_split_kernel(AttnArgs a) {
  static_assert(sizeof(T) == 2, "16-bit inputs only: fp32 small grids take fwd_small_kernel");
  using C = SplitCfg<T, D>;
  using M = Mfma<T>;
  using frag = typename M::frag;
  constexpr int KI = M::KI, KH = M::KH;
  constexpr int BC = C::BC, NDB = D / 32, NC = D / KI;
  constexpr int RB = D * (int)sizeof(T);
  constexpr float NEG_INF = -__builtin_inff();

  __shared__ __attribute__((aligned(16))) unsigned char smem[C::BYTES];
  __shared__ float ms[4][32], ls[4][32], mrow[32], lrow[32];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lo = lane & 31, hi = lane >> 5;
  const int N = a.N;
  const int nq = (N + 31) / 32;
  const int rank = blockIdx.x / a.BH;
  const int bh = blockIdx.x - rank * a.BH;
  const int qt = a.causal ? (nq - 1 - rank) : rank;  // causal: longest rows first
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const T* __restrict__ Kg = static_cast<const T*>(a.k) + hoff;
  const T* __restrict__ Vg = static_cast<const T*>(a.v) + hoff;
  const int q0 = qt * 32;
  const int q = q0 + lo;

  const __amdgpu_buffer_rsrc_t qrs = buffer_rsrc(static_cast<const T*>(a.q) + hoff, N * RB);
  frag qf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) qf[c] = __builtin_bit_cast(frag, buffer_load16(qrs, q * RB + (c * KI + hi * KH) * (int)sizeof(T)));
  uint32_t rowhash = 0;
  if constexpr (DROP) {
    const uint32_t hk = head_key(a.seed_lo, a.seed_hi, (uint32_t)(bh / a.H), (uint32_t)(bh % a.H));
    rowhash = fmix32(hk ^ (uint32_t)q) + (uint32_t)(2 * hi);  // crow's 4*hi keys = 2*hi pairs
  }

  const int kend = a.causal ? min(N, q0 + 32) : N;
  const int ntiles = (kend + BC - 1) / BC;
  const uint8_t* bmrow = a.bmask ? a.bmask + (size_t)(q0 / a.mask_block) * a.nb : nullptr;
  const bool mfew = bmrow != nullptr && a.nb <= 64;
  const uint64_t mbits = mfew ? mask_bits(bmrow, 1, a.nb, lane) : ~0ull;

  T* Ks = reinterpret_cast<T*>(smem) + w * 2 * C::TILE;  // this wave's K tile, then its V tile
  T* Vs = Ks + C::TILE;

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = zero16();
  float m_run = NEG_INF, l_run = 0.f;

  for (int j = w; j < ntiles; j += 4) {
    if (bmrow != nullptr) {
      const int blk = (j * BC) / a.mask_block;
      if (mfew ? ((mbits >> blk) & 1ull) == 0 : !mask_kept(bmrow, blk)) continue;
    }
    const int k0 = j * BC;
    // The wave loads its own tile (rows past the end read as zeros). LDS
    // operations of one wave run in order, so these stores follow the reads
    // of the previous tile and precede this tile's reads.
    {
      const int rem = (N - k0) * RB;
      const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(Kg + (size_t)k0 * D, rem);
      const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(Vg + (size_t)k0 * D, rem);
      u32x4 kreg[C::NLD], vreg[C::NLD];
#pragma unroll
      for (int i = 0; i < C::NLD; ++i) {
        const int c = i * 64 + lane;
        const int off = (c / C::KCH) * RB + (c % C::KCH) * 16;
        kreg[i] = buffer_load16(kr, off);
        vreg[i] = buffer_load16(vr, off);
      }
#pragma unroll
      for (int i = 0; i < C::NLD; ++i) {
        const int c = i * 64 + lane;
        const int e = lds_row(c / C::KCH) * C::KS + (c % C::KCH) * C::EPC;
        *reinterpret_cast<u32x4*>(&Ks[e]) = kreg[i];
        *reinterpret_cast<u32x4*>(&Vs[e]) = vreg[i];
      }
    }
    f32x16 sc = zero16();
#pragma unroll
    for (int c = 0; c < NC; ++c) sc = M::run(load_frag<T>(Ks + lds_row(lo) * C::KS + c * KI + hi * KH), qf[c], sc);
    if ((a.causal && k0 + BC - 1 > q0) || (k0 + BC > N)) {
      const int t = (a.causal ? min(q, N - 1) : N - 1) - k0 - 4 * hi;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (8 * (v >> 2) + (v & 3) > t) sc[v] = NEG_INF;
    }
    float mx = NEG_INF;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[v]);
    if (wave_any(mx * a.sl2 > m_run + kLazyRescale)) {  // the exchange only when it rescales
      const float mnew = fmaxf(m_run, half_max(mx) * a.sl2);
      const float alpha = exp2_fast(m_run - (mnew == NEG_INF ? 0.f : mnew));
      m_run = mnew;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[db][v] *= alpha;
    }
    const float base = (m_run == NEG_INF) ? 0.f : m_run;
    uint32_t pk[8];  // P as packed pairs
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p0 = exp2_fast(fmaf(sc[2 * e], a.sl2, -base));
      const float p1 = exp2_fast(fmaf(sc[2 * e + 1], a.sl2, -base));
      pk[e] = pack2<T>(p0, p1);
      l_run += p0 + p1;
    }
    const uint32_t y = DROP ? (rowhash + (uint32_t)(k0 >> 1)) * kMixMul : 0u;
    {
      const u16x2 tm1 = {(unsigned short)((a.thresh >> 16) - 1u), (unsigned short)((a.thresh >> 16) - 1u)};
      const u16x2 ones = __builtin_bit_cast(u16x2, a.ones16);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint32_t d4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          d4[e] = pk[4 * hf + e];
          if constexpr (DROP)  // packed keep factors, as in the 128-row kernel (T16 >= 1)
            d4[e] = keep_pair(d4[e], keep_finish(y + (uint32_t)(8 * hf + 4 * (e >> 1) + (e & 1)) * kMixMul), tm1, ones);
        }
        const frag pb = frag4<T>(d4[0], d4[1], d4[2], d4[3]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = M::run(load_frag_tr_rp<T>(Vs, C::KS, 16 * hf, db * 32, lane), pb, o[db]);
      }
    }
  }

  // Merge the four waves' partial results: M = max_w m_w, a_w = 2^(m_w - M),
  // L = sum_w a_w l_w, O = sum_w a_w O_w / L.
  const float lt = half_sum(l_run);
  if (hi == 0) {
    ms[w][lo] = m_run;
    ls[w][lo] = lt;
  }
  __syncthreads();  // every wave is done with its tile and has posted its row statistics
  float mall = NEG_INF;
#pragma unroll
  for (int x = 0; x < 4; ++x) mall = fmaxf(mall, ms[x][lo]);
  const float aw = (m_run == NEG_INF) ? 0.f : exp2_fast(m_run - mall);
  float* Os = reinterpret_cast<float*>(smem) + w * 32 * C::OS;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = {o[db][4 * g] * aw, o[db][4 * g + 1] * aw, o[db][4 * g + 2] * aw, o[db][4 * g + 3] * aw};
      *reinterpret_cast<f32x4*>(&Os[lo * C::OS + db * 32 + 8 * g + 4 * hi]) = x;
    }
  if (w == 0 && hi == 0) {
    float L = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) L += ms[x][lo] == NEG_INF ? 0.f : ls[x][lo] * exp2_fast(ms[x][lo] - mall);
    mrow[lo] = mall;
    lrow[lo] = L;
  }
  __syncthreads();
  const float* O0 = reinterpret_cast<const float*>(smem);
  T* __restrict__ Og = static_cast<T*>(a.out) + hoff;
  constexpr int C4 = D / 4;  // groups of 4 columns per row
  for (int idx = tid; idx < 32 * C4; idx += 256) {
    const int r = idx / C4, c = (idx % C4) * 4;
    if (q0 + r >= N) continue;
    const float L = lrow[r];
    const float inv = L > 0.f ? a.rp / L : 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < 4; ++x) acc += *reinterpret_cast<const f32x4*>(&O0[(x * 32 + r) * C::OS + c]);
    store4<T>(Og + (size_t)(q0 + r) * D + c, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  }
  if (tid < 32 && q0 + tid < N) {
    const float L = lrow[tid];
    a.lse[(size_t)bh * N + q0 + tid] = L > 0.f ? (mrow[tid] + log2_fast(L)) * kLn2 : NEG_INF;
  }
}

// fp32 forward for grids too small to fill the device. fp32 products run on
// the slow fp32 MFMA (64 clocks for 32x32x2), so the serial MFMA chain of a
// wave is most of such a launch. This kernel takes 16 query rows per
// workgroup, twice as many workgroups as the 32-row split-key kernel, with
// v_mfma_f32_16x16x4_f32, which halves each wave's chain. As in the split-key
// kernel the NW waves take the tiles j = w, w + NW, ... of 128 / NW keys
// with their own LDS tiles and running (m, l), merged in LDS at the end.
//
// v_mfma_f32_16x16x4_f32 operands (wave64; layout checked on the device):
// A (16 x 4): lane l holds row l % 16, k = l / 16; B (4 x 16): lane l holds
// k = l / 16, column l % 16; C (16 x 16): lane l holds rows 4 (l / 16) + v,
// column l % 16, for v = 0..3. Step s of a product over d takes d = 4 s +
// l / 16 in lane l: in that order the scores come out bit-identical to the
// 32x32x2 products (step c: d = 2 c + k) that the backward uses to recompute
// P, so P in the backward matches the forward's to the last bit, as with
// the other forward kernels. (Other orders round differently; against a
// recomputed P off by rounding, fp32 gradients lose about a factor of two.)
// S^T = K Q^T per 16-key block: A = K (row: key), B = Q^T (column: query),
// so lane l holds keys 4 (l / 16) + v of query l % 16, and those elements are
// directly the B operand (k = l / 16 <-> key 4 (l / 16) + v) of the
// product O^T += V^T P^T taken one v at a time.
template <int D, int NW>
struct SmallCfg {
  static constexpr int BC = 128 / NW;               // keys per wave tile (a whole number of 16-key blocks)
  static constexpr int KB = BC / 16;
  static constexpr int KS = D + 4;                  // LDS row stride (floats) of the K/V tiles
  static constexpr int TILE = BC * KS;              // floats per K (or V) tile
  static constexpr int CH = D / 4;                  // 16-byte chunks per row
  static constexpr int NLD = BC * CH / 64;          // 16-byte loads per lane per tensor per tile
  static constexpr int OS = D + 4;                  // fp32 row stride of the partial O
  static constexpr int TILE_BYTES = NW * 2 * TILE * 4;
  static constexpr int COMB_BYTES = NW * 16 * OS * 4;
  static constexpr int BYTES = TILE_BYTES > COMB_BYTES ? TILE_BYTES : COMB_BYTES;
};

template <int D, int NW, bool DROP>
__global__ void __launch_bounds__(64 * NW) fwd_small_kernel(AttnArgs a) {
  using C = SmallCfg<D, NW>;
  constexpr int BC = C::BC, KB = C::KB, NDB = D / 16, NS = D / 4;
  constexpr int RB = D * 4;  // bytes per row
  constexpr float NEG_INF = -__builtin_inff();
  typedef float f32x4_t __attribute__((ext_vector_type(4)));

  __shared__ __attribute__((aligned(16))) unsigned char smem[C::BYTES];
  __shared__ float ms[NW][16], ls[NW][16], mrow[16], lrow[16];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, c16 = lane & 15, g = lane >> 4;
  const int N = a.N;
  const int nq = (N + 15) / 16;
  const int rank = blockIdx.x / a.BH;
  const int bh = blockIdx.x - rank * a.BH;
  const int qt = a.causal ? (nq - 1 - rank) : rank;  // causal: longest rows first
  const size_t hoff = (size_t)bh * (size_t)N * D;
  const float* __restrict__ Kg = static_cast<const float*>(a.k) + hoff;
  const float* __restrict__ Vg = static_cast<const float*>(a.v) + hoff;
  const int q0 = qt * 16;
  const int q = q0 + c16;  // this lane's query (rows past the end read zeros; never stored)

  // Q^T as the B operand: step s takes d = 4 s + g of query q.
  const __amdgpu_buffer_rsrc_t qrs = buffer_rsrc(static_cast<const float*>(a.q) + hoff, N * RB);
  float qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qf[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qrs, q * RB + (4 * s + g) * 4, 0, 0));
  uint32_t rowhash = 0;
  if constexpr (DROP) {
    const uint32_t hk = head_key(a.seed_lo, a.seed_hi, (uint32_t)(bh / a.H), (uint32_t)(bh % a.H));
    rowhash = fmix32(hk ^ (uint32_t)q) + (uint32_t)(2 * g);  // keys 4g + v of a block: pairs 2g + v/2
  }

  const int kend = a.causal ? min(N, q0 + 16) : N;
  const int ntiles = (kend + BC - 1) / BC;
  const uint8_t* bmrow = a.bmask ? a.bmask + (size_t)(q0 / a.mask_block) * a.nb : nullptr;
  const bool mfew = bmrow != nullptr && a.nb <= 64;
  const uint64_t mbits = mfew ? mask_bits(bmrow, 1, a.nb, lane) : ~0ull;

  float* Ks = reinterpret_cast<float*>(smem) + w * 2 * C::TILE;  // this wave's K tile, then its V tile
  float* Vs = Ks + C::TILE;

  f32x4_t o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF, l_run = 0.f;

  for (int j = w; j < ntiles; j += NW) {
    if (bmrow != nullptr) {
      const int blk = (j * BC) / a.mask_block;
      if (mfew ? ((mbits >> blk) & 1ull) == 0 : !mask_kept(bmrow, blk)) continue;
    }
    const int k0 = j * BC;
    {
      // The wave loads its own tile (rows past the end read as zeros); LDS
      // operations of one wave run in order, so these stores follow the
      // reads of its previous tile and precede this tile's reads.
      const int rem = (N - k0) * RB;
      const __amdgpu_buffer_rsrc_t kr = buffer_rsrc(Kg + (size_t)k0 * D, rem);
      const __amdgpu_buffer_rsrc_t vr = buffer_rsrc(Vg + (size_t)k0 * D, rem);
      u32x4 kreg[C::NLD], vreg[C::NLD];
#pragma unroll
      for (int i = 0; i < C::NLD; ++i) {
        const int c = i * 64 + lane;
        const int off = (c / C::CH) * RB + (c % C::CH) * 16;
        kreg[i] = buffer_load16(kr, off);
        vreg[i] = buffer_load16(vr, off);
      }
#pragma unroll
      for (int i = 0; i < C::NLD; ++i) {
        const int c = i * 64 + lane;
        const int e = (c / C::CH) * C::KS + (c % C::CH) * 4;
        *reinterpret_cast<u32x4*>(&Ks[e]) = kreg[i];
        *reinterpret_cast<u32x4*>(&Vs[e]) = vreg[i];
      }
    }
    // S^T of the tile's 16-key blocks: element v of block kb is key k0 + 16 kb + 4 g + v.
    f32x4_t sc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const float* kr = &Ks[(16 * kb + c16) * C::KS + g];  // banks 4 c16 + g: no conflicts
#pragma unroll
      for (int s = 0; s < NS; ++s) sc[kb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[4 * s], qf[s], sc[kb], 0, 0, 0);
    }
    if ((a.causal && k0 + BC - 1 > q0) || (k0 + BC > N)) {
      const int lim = (a.causal ? min(q, N - 1) : N - 1) - k0 - 4 * g;  // key offset 16 kb + v must not exceed it
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (16 * kb + v > lim) sc[kb][v] = NEG_INF;
    }
    float mx = NEG_INF;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) mx = fmaxf(mx, sc[kb][v]);
    if (wave_any(mx * a.sl2 > m_run + kLazyRescale)) {  // the exchanges only when it rescales
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));  // the query's maximum over the tile's keys
      const float mnew = fmaxf(m_run, mx * a.sl2);
      const float alpha = exp2_fast(m_run - (mnew == NEG_INF ? 0.f : mnew));
      m_run = mnew;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
    }
    const float base = (m_run == NEG_INF) ? 0.f : m_run;
    const uint32_t y = DROP ? (rowhash + (uint32_t)(k0 >> 1)) * kMixMul : 0u;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float pv = exp2_fast(fmaf(sc[kb][v], a.sl2, -base));
        l_run += pv;
        sc[kb][v] = pv;
      }
    if constexpr (DROP) {  // elements v, v + 1 (v even) are the two keys of pair (k0 + 16 kb + 4 g + v) / 2
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int v = 0; v < 4; v += 2) {
          const uint32_t u = keep_finish(y + (uint32_t)(8 * kb + (v >> 1)) * kMixMul);
          sc[kb][v] = keep_lo(u, a.thresh) ? sc[kb][v] : 0.f;
          sc[kb][v + 1] = keep_hi(u, a.thresh) ? sc[kb][v + 1] : 0.f;
        }
    }
    // O^T += V^T P^T, one v at a time: B = this lane's element v (k = g <-> key
    // 16 kb + 4 g + v), A = V[that key][16 db + c16].
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float* vr = &Vs[(16 * kb + 4 * g + v) * C::KS + c16];
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[16 * db], sc[kb][v], o[db], 0, 0, 0);
      }
  }

  // Merge the waves' partials (M = max_w m_w, a_w = 2^(m_w - M),
  // L = sum_w a_w l_w, O = sum_w a_w O_w / L). A query's row sum is spread
  // over the four lanes that share its column.
  float lt = l_run + __shfl_xor(l_run, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (g == 0) {
    ms[w][c16] = m_run;
    ls[w][c16] = lt;
  }
  __syncthreads();  // every wave is done with its tiles and has posted its row statistics
  float mall = NEG_INF;
#pragma unroll
  for (int x = 0; x < NW; ++x) mall = fmaxf(mall, ms[x][c16]);
  const float aw = (m_run == NEG_INF) ? 0.f : exp2_fast(m_run - mall);
  float* Os = reinterpret_cast<float*>(smem) + w * 16 * C::OS;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    *reinterpret_cast<f32x4_t*>(&Os[c16 * C::OS + 16 * db + 4 * g]) = o[db] * aw;  // d = 16 db + 4 g + v'
  if (w == 0 && g == 0) {
    float L = 0.f;
#pragma unroll
    for (int x = 0; x < NW; ++x) L += ms[x][c16] == NEG_INF ? 0.f : ls[x][c16] * exp2_fast(ms[x][c16] - mall);
    mrow[c16] = mall;
    lrow[c16] = L;
  }
  __syncthreads();
  const float* O0 = reinterpret_cast<const float*>(smem);
  float* __restrict__ Og = static_cast<float*>(a.out) + hoff;
  constexpr int C4 = D / 4;  // groups of 4 columns per row
  for (int idx = tid; idx < 16 * C4; idx += 64 * NW) {
    const int r = idx / C4, c = (idx % C4) * 4;
    if (q0 + r >= N) continue;
    const float L = lrow[r];
    const float inv = L > 0.f ? a.rp / L : 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < NW; ++x) acc += *reinterpret_cast<const f32x4_t*>(&O0[(x * 16 + r) * C::OS + c]);
    store4<float>(Og + (size_t)(q0 + r) * D + c, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  }
  if (tid < 16 && q0 + tid < N) {
    const float L = lrow[tid];
    a.lse[(size_t)bh * N + q0 + tid] = L > 0.f ? (mrow[tid] + log2_fast(L)) * kLn2 : NEG_INF;
  }
}

// Resident waves per SIMD: with one wave, softmax VALU work, LDS reads and
// MFMAs of a tile run back to back; more waves let them overlap. d = 128
// fits two waves (256 VGPRs, two workgroups' LDS in the 160 KB of a CU);
// the 16-bit d = 64 kernel, with or without dropout, fits 128 VGPRs for
// four (with P packed pairwise the dropout variant needs no spill).
template <typename T, int D, int BC, int QB, bool DROP>
static hipError_t launch_fwd_t(const AttnArgs& a, hipStream_t s) {
  const int nq = (a.N + 128 * QB - 1) / (128 * QB);
  const dim3 grid((unsigned)(nq * a.BH));
  constexpr int WPE = D * QB > 128 ? 1 : (D == 64 && sizeof(T) == 2 ? 4 : 2);  // two query blocks at d = 128 need the whole register file
  fwd_kernel<T, D, BC, QB, DROP, WPE><<<grid, dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

// A grid of 128-row tiles that would occupy at most a quarter of the CUs
// takes a split-key kernel instead, each wave a quarter of the keys: 32-row
// workgroups (four times the workgroups) for 16-bit inputs, 16-row ones
// (eight times) for fp32.
template <typename T, int D>
static hipError_t launch_fwd_split(bool dropout, const AttnArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 4) {  // fp32: 16-row workgroups on 16x16x4 MFMAs
    constexpr int NW = 4;  // 8 waves on 16-key tiles measured slower: the per-tile latency, not the MFMA chain, dominates there
    const dim3 grid((unsigned)(((a.N + 15) / 16) * a.BH));
    if (dropout)
      fwd_small_kernel<D, NW, true><<<grid, dim3(64 * NW), 0, s>>>(a);
    else
      fwd_small_kernel<D, NW, false><<<grid, dim3(64 * NW), 0, s>>>(a);
  } else {
    const dim3 grid((unsigned)(((a.N + 31) / 32) * a.BH));
    if (dropout)
      fwd_split_kernel<T, D, true><<<grid, dim3(256), 0, s>>>(a);
    else
      fwd_split_kernel<T, D, false><<<grid, dim3(256), 0, s>>>(a);
  }
  return hipGetLastError();
}

template <typename T, int D, int BC, int QB>
static hipError_t launch_fwd_d(bool dropout, const AttnArgs& a, hipStream_t s) {
  if (QB > 1 && a.bmask != nullptr) return hipErrorInvalidValue;
  const long tiles = (long)((a.N + 127) / 128) * a.BH;
  if (4 * tiles <= a.ncu) return launch_fwd_split<T, D>(dropout, a, s);
  return dropout ? launch_fwd_t<T, D, BC, QB, true>(a, s) : launch_fwd_t<T, D, BC, QB, false>(a, s);
}

hipError_t launch_fwd(Elt t, int d, bool dropout, const AttnArgs& a, hipStream_t s) {
  switch (t) {
    case Elt::BF16:
      return d == 64 ? launch_fwd_d<__bf16, 64, 64, 1>(dropout, a, s) : launch_fwd_d<__bf16, 128, 64, 1>(dropout, a, s);
    case Elt::F16:
      return d == 64 ? launch_fwd_d<_Float16, 64, 64, 1>(dropout, a, s) : launch_fwd_d<_Float16, 128, 64, 1>(dropout, a, s);
    case Elt::F32:
      return d == 64 ? launch_fwd_d<float, 64, 64, 1>(dropout, a, s) : launch_fwd_d<float, 128, 32, 1>(dropout, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
