// Device-side building blocks for the gfx950 attention kernels: MFMA
// wrappers, operand fragments, type conversion and the dropout hash.
//
// MFMA operand layout used throughout (32x32 output tiles, wave64):
//   A (32 x KI): lane l holds row (l % 32), k elements [KH*(l/32), KH*(l/32)+KH)
//   B (KI x 32): lane l holds column (l % 32), the same k elements
//   C (32 x 32): lane l holds column (l % 32), rows 8*(v/4) + 4*(l/32) + (v%4)
//                for accumulator element v = 0..15
// KI = 16, KH = 8 for bf16/fp16 (v_mfma_f32_32x32x16_{bf16,f16});
// KI = 2,  KH = 1 for fp32      (v_mfma_f32_32x32x2_f32).
// Only the A/B row/column mapping and the C layout matter for results:
// A and B are always filled with the same k order, so the sum over k is the
// same whatever the hardware's internal k order is.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
  using frag = bf16x8;
  using half = bf16x4;
  static constexpr int KI = 16, KH = 8;
  static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<_Float16> {
  using frag = f16x8;
  using half = f16x4;
  static constexpr int KI = 16, KH = 8;
  static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  using frag = float;
  using half = float;
  static constexpr int KI = 2, KH = 1;
  static __device__ __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// KH contiguous elements starting at p (16-byte aligned for 16-bit types).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag load_frag(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(typename Mfma<T>::frag, *reinterpret_cast<const u32x4*>(p));
  } else {
    return *p;
  }
}

template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag zero_frag() {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(typename Mfma<T>::frag, u32x4{0u, 0u, 0u, 0u});
  } else {
    return 0.f;
  }
}

// Two groups of 4 contiguous 16-bit elements (8-byte aligned) joined into
// one 8-element fragment.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag load_frag_2x4(const T* p0, const T* p1) {
  static_assert(sizeof(T) == 2, "16-bit only");
  u32x2 a = *reinterpret_cast<const u32x2*>(p0);
  u32x2 b = *reinterpret_cast<const u32x2*>(p1);
  return __builtin_bit_cast(typename Mfma<T>::frag, u32x4{a[0], a[1], b[0], b[1]});
}

template <typename T> __device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }

template <typename T> __device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }

// Two fp32 values -> one dword holding them as 16-bit values (round to
// nearest even), x0 in the low half. Converting the pair as a two-element
// vector gives one packed conversion instruction.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <typename T> __device__ __forceinline__ uint32_t pack2(float x0, float x1);
template <> __device__ __forceinline__ uint32_t pack2<__bf16>(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, bf16x2));
}
template <> __device__ __forceinline__ uint32_t pack2<_Float16>(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, f16x2));
}

// Four packed dwords (elements 2e, 2e + 1 in dword e) -> one fragment.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag4(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3) {
  return __builtin_bit_cast(typename Mfma<T>::frag, u32x4{d0, d1, d2, d3});
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Combine a value with the one held by the lane 32 positions away (the other
// half of the wave); the result is the same in both lanes of the pair.
__device__ __forceinline__ float half_max(float x) { return fmaxf(x, __shfl_xor(x, 32, 64)); }
__device__ __forceinline__ float half_sum(float x) { return x + __shfl_xor(x, 32, 64); }

// MurmurHash3 32-bit finalizer (Appleby, public domain).
constexpr uint32_t kMixMul = 0x85EBCA6Bu;  // its first multiplier
__device__ __forceinline__ uint32_t keep_mix(uint32_t x) {  // the two steps after that multiply
  x ^= x >> 13;
  return x * 0xC2B2AE35u;
}
__device__ __forceinline__ uint32_t keep_finish(uint32_t x) {  // ... and the last one
  x = keep_mix(x);
  return x ^ (x >> 16);
}
__device__ __forceinline__ uint32_t fmix32(uint32_t x) { return keep_finish((x ^ (x >> 16)) * kMixMul); }

// Keep word of row word r and key pair m = j / 2: mix32(r + m) =
// keep_finish((r + m) * kMixMul); key 2m reads its low 16 bits, key 2m + 1
// its high 16 bits. The multiply distributes over the sum (mod 2^32), so a
// kernel forms (r + tile's first pair) * kMixMul once per tile and adds the
// pair offset times kMixMul, a compile-time constant, per pair; or keeps
// r * kMixMul per row and adds its own pair's m * kMixMul.
//
// With thresh = T16 << 16 (T16 = floor(p * 2^16)): the high half is kept iff
// u >= thresh, the low half iff (u << 16) >= thresh.
__device__ __forceinline__ bool keep_hi(uint32_t u, uint32_t thresh) { return u >= thresh; }
// The same two decisions from x = keep_mix(...), before the last step (u =
// x ^ (x >> 16)): u's high half is x's, and u's low half, lo(x) ^ hi(x), is
// the high half of x ^ (x << 16); thresh has a zero low half, so comparing
// the whole words decides on the high halves. One operation fewer per word
// where the two keys are tested separately.
__device__ __forceinline__ bool keep_hi_mixed(uint32_t x, uint32_t thresh) { return x >= thresh; }
__device__ __forceinline__ bool keep_lo_mixed(uint32_t x, uint32_t thresh) { return (x ^ (x << 16)) >= thresh; }

// The same decisions for both keys of a pair at once, on the word's two
// 16-bit halves as packed integers: half >= T16 <=> sat(half - (T16 - 1)) >= 1,
// so min(sat(half - tm1), 1) is 1 for a kept key and 0 for a dropped one
// (tm1 = T16 - 1 in both halves; T16 >= 1). Multiplying the bits of a
// packed 16-bit pair of P by it keeps or zeroes each value exactly.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// `ones` is {1, 1} passed at run time (AttnArgs::ones16): with a literal 1
// the compiler rewrites the min into two compares and selects.
__device__ __forceinline__ u16x2 keep01(uint32_t u, u16x2 tm1, u16x2 ones) {
  return __builtin_elementwise_min(__builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, u), tm1), ones);
}
__device__ __forceinline__ bool keep_lo(uint32_t u, uint32_t thresh) { return (u << 16) >= thresh; }
// A packed pair of 16-bit P values (low half: the even key) with the pair's
// keep word u applied.
__device__ __forceinline__ uint32_t keep_pair(uint32_t pk, uint32_t u, u16x2 tm1, u16x2 ones) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, pk) * keep01(u, tm1, ones));
}

// Per-(b, h) dropout key from the 64-bit seed.
__device__ __forceinline__ uint32_t head_key(uint32_t seed_lo, uint32_t seed_hi, uint32_t b, uint32_t h) {
  uint32_t k = fmix32(seed_lo + 0x9E3779B9u);
  k = fmix32(k ^ seed_hi);
  k = fmix32(k ^ b);
  return fmix32(k ^ h);
}

// Key index of accumulator element v in a 32x32 C tile whose rows are keys.
__device__ __forceinline__ int crow(int v, int hi) { return 8 * (v >> 2) + 4 * hi + (v & 3); }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// A-operand fragment built from the COLUMNS of a row-major 16-bit LDS tile
// (element (r, c) at tile[r * stride + c]): lane l receives column
// col0 + (l % 32) and the tile rows base + 4*(l/32) + {0,1,2,3} followed by
// base + 8 + 4*(l/32) + {0,1,2,3}, i.e. the same k order as elements
// 8*hf .. 8*hf+7 of a 32x32 accumulator tile (crow) when base = 32*kb + 16*hf.
// Uses the gfx950 LDS transpose read (ds_read_b64_tr_b16): within each group
// of 16 lanes, lane j's element e is element (j % 4) of the 8 bytes addressed
// by lane 4*e + j/4 of the group. `stride` and col0 must be multiples of 4.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag load_frag_tr(const T* tile, int stride, int base, int col0,
                                                                int lane) {
  static_assert(sizeof(T) == 2, "16-bit only");
  const int j = lane & 15;
  const T* p = tile + (base + 4 * (lane >> 5) + (j >> 2)) * stride + col0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * stride));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 xy = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(typename Mfma<T>::frag, xy);
}

// Row permutation of the padded (register-staged) LDS tiles: tile row r is
// stored at LDS row lds_row(r), which swaps bits 0-1 and 2-3 of r. A
// transpose read gathers 4 tile rows 4*x + {0,1,2,3} (the k order of the
// accumulator tile, crow) and each half-wave reads 64 bytes of each; at the
// padded strides (36 dwords at d = 64, 76 at d = 128, both 4 x odd) those
// rows sit 12 or 36 dwords apart mod 64 banks, so their 16-dword windows
// overlap (2-way conflicts). Permuted, the 4 rows are LDS rows y + 4e, 4*9 or
// 4*19 dwords apart per step, i.e. 16-dword windows at 0, 16, 32, 48 mod 64:
// disjoint. 16-byte row reads of 16 consecutive tile rows still hit 16
// distinct bank quads (lds_row permutes each group of 16 rows).
__device__ __forceinline__ constexpr int lds_row(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

// load_frag_tr over a tile whose rows are stored at lds_row(r): the rows
// base + 4*(l/32) + {0..3} (and + 8) of the fragment sit at LDS rows
// base + 4*{0..3} + l/32 (and + 2). base must be a multiple of 16.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag load_frag_tr_rp(const T* tile, int stride, int base, int col0,
                                                                   int lane) {
  static_assert(sizeof(T) == 2, "16-bit only");
  const int j = lane & 15;
  const T* p = tile + (base + 4 * (j >> 2) + (lane >> 5)) * stride + col0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 2 * stride));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 xy = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(typename Mfma<T>::frag, xy);
}

// XOR swizzle (in 16-byte chunks) of an unpadded 16-bit LDS tile row of D
// elements: the logical chunk lc of row r sits at physical chunk
// lc ^ lds_swizzle<D>(r). With 64 banks of 4 bytes, it keeps both read
// patterns free of bank conflicts: 16 consecutive rows read at one logical
// chunk (row fragments) land on 16 distinct 16-byte bank groups, and the
// 4 rows x 4 aligned chunks that half a wave reads with a transpose read
// do too.
template <int D>
__device__ __forceinline__ int lds_swizzle(int r) {
  static_assert(D == 64 || D == 128, "head dimension");
  if constexpr (D == 64)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);  // 128-byte rows: two rows per bank sweep
  else
    return ((r & 3) << 2) | ((r >> 2) & 3);  // 256-byte rows
}

// load_frag_tr over a swizzled, unpadded tile (rows of D elements). Each
// lane's 8 bytes stay inside one 16-byte chunk, so only the chunk index moves.
template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::frag load_frag_tr_swz(const T* tile, int base, int col0, int lane) {
  static_assert(sizeof(T) == 2, "16-bit only");
  const int j = lane & 15;
  const int row = base + 4 * (lane >> 5) + (j >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const T* p0 = tile + row * D + (((col >> 3) ^ lds_swizzle<D>(row)) << 3) + (col & 7);
  const T* p1 = tile + (row + 8) * D + (((col >> 3) ^ lds_swizzle<D>(row + 8)) << 3) + (col & 7);
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 xy = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(typename Mfma<T>::frag, xy);
}

// load_frag_tr_swz split into a lane part and a row part. The lane part
// (element offsets of the fragment's two reads for base row 0 and columns
// col0...) depends only on the lane, because the swizzle depends on the row
// modulo 16 and base is a multiple of 16; the row part is base * D, a
// compile-time constant. tr_swz_lane returns the lane part through an
// identity DPP move, which the optimizer cannot look through: every read's
// address is then "tile + lane part + constant", a short chain from the LDS
// array, and the compiler keeps the array's alias scope on the read. With
// the scope it can tell the reads apart from direct-to-LDS loads into
// another array instead of waiting for those loads to land.
template <typename T, int D>
__device__ __forceinline__ int2 tr_swz_lane(int col0, int lane) {
  static_assert(sizeof(T) == 2, "16-bit only");
  const int j = lane & 15;
  const int row = 4 * (lane >> 5) + (j >> 2);
  const int col = col0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
  const int o0 = row * D + (((col >> 3) ^ lds_swizzle<D>(row)) << 3) + (col & 7);
  const int o1 = (row + 8) * D + (((col >> 3) ^ lds_swizzle<D>(row + 8)) << 3) + (col & 7);
  return make_int2(__builtin_amdgcn_mov_dpp(o0, 0xE4, 0xF, 0xF, false),
                   __builtin_amdgcn_mov_dpp(o1, 0xE4, 0xF, 0xF, false));
}
template <typename T, int D>
__device__ __forceinline__ typename Mfma<T>::frag load_frag_tr_lane(const T* tile, int base, int2 lo) {
  const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + lo.x + base * D));
  const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + lo.y + base * D));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 xy = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(typename Mfma<T>::frag, xy);
}

// Whether byte `idx` of a block mask is nonzero. `idx` must be uniform across
// the wave: the aligned dword holding the byte is read with a scalar load
// (constant address space), which keeps the vector-memory counter free for
// the tile prefetches. The dword never leaves the 4-byte-aligned word that
// holds the byte, so it stays inside the mask's page.
__device__ __forceinline__ bool mask_kept(const uint8_t* bm, int idx) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(bm) + (uintptr_t)idx;
  const __attribute__((address_space(4))) uint32_t* w =
      (const __attribute__((address_space(4))) uint32_t*)(a & ~(uintptr_t)3);
  return ((*w >> (8u * (uint32_t)(a & 3))) & 0xFFu) != 0;
}

// Kept bits of up to 64 block-mask bytes at once: lane l (< n) reads the byte
// at base + l * stride with a vector load; bit l of the wave-uniform result
// is set when that byte is nonzero. Must be reached by all 64 lanes. With
// n <= 64 the kernels test these bits instead of walking the mask byte by
// byte with dependent scalar loads.
__device__ __forceinline__ uint64_t mask_bits(const uint8_t* base, int stride, int n, int lane) {
  const uint8_t v = lane < n ? base[(size_t)lane * (size_t)stride] : (uint8_t)0;
  return __builtin_amdgcn_ballot_w64(v != 0);
}

// Buffer resource over `bytes` bytes starting at `base` (raw, unstrided).
// Buffer loads whose per-lane offset falls outside return zeros and such
// stores are dropped, so tails need no clamping or branches; the
// per-lane (VGPR) offset carries the row offset because the scalar offset is
// not part of the range check. `bytes` must fit in 31 bits (checked by the
// host layer for every per-head tensor).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes < 0 ? 0 : bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
// Direct-to-LDS buffer load: lane L reads 16 bytes at `voff` (zeros past the
// resource's range) and writes them to LDS at lds + 16 * L; `lds` must be
// uniform across the wave (it goes into M0). Completion is counted by the
// vector-memory counter (wait_vmem).
typedef __attribute__((address_space(3))) void lds_void;
template <typename T>
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, T* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}
// s_waitcnt vmcnt(0): every vector-memory load of this wave has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, int voff, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), r, voff, 0, 0);
}
__device__ __forceinline__ void buffer_store8(__amdgpu_buffer_rsrc_t r, int voff, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v), r, voff, 0, 0);
}
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, int voff, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, voff, 0, 0);
}

// This lane's index in its wave (0..63), recomputed from the execution mask
// counters rather than kept in a register across a loop.
__device__ __forceinline__ int lane_id() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Workgroup id -> (rank, bh). A head's tiles are ranked by decreasing work
// (causal: the tile of longest rows first). Ids are dealt round-robin over
// the device's nxcd XCDs, and each XCD hands its ids to its CUs in turn. In
// the plain order (id = rank * BH + bh) consecutive ids are different heads
// of one rank, so with BH a multiple of nxcd all tiles of a head land on one
// XCD (bh % nxcd equals id % nxcd) and share its L2. `balance` is for a grid
// that is resident all at once, with work falling linearly in the rank: an
// XCD's ids then run over its (rank, head) pairs in rounds of one per CU,
// forward in even rounds and backward in odd ones, so a CU that drew a long
// tile in one round draws a short one in the next and the CUs' totals even
// out (MI355X, 8 XCDs of 32 CUs, 8 tiles a head and 16 heads an XCD: 18
// tile-units on every CU, where the plain order gives half the CUs 20 and
// half 16). Heads stay on their XCD either way. A grid that is not all
// resident keeps the plain longest-first order, which a CU freeing a slot
// follows.
__device__ __forceinline__ void tile_order(int id, int nq, int BH, bool balance, int ncu, int nxcd, int& rank,
                                           int& bh) {
  const int cpx = ncu / nxcd;  // CUs per XCD
  if (balance && nxcd > 0 && cpx > 0 && BH % nxcd == 0 && (nq * (BH / nxcd)) % cpx == 0) {
    const int hpx = BH / nxcd;  // heads per XCD
    const int x = id % nxcd, n = id / nxcd;
    const int r = n / cpx, c = n - r * cpx;
    const int k = r * cpx + ((r & 1) ? cpx - 1 - c : c);
    rank = k / hpx;
    bh = (k - rank * hpx) * nxcd + x;
  } else {
    rank = id / BH;
    bh = id - rank * BH;
  }
}

// True if `pred` holds in any lane of the wave.
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// Stores 4 consecutive fp32 values as type G (one vector store).
template <typename G>
__device__ __forceinline__ void store4(G* p, float x0, float x1, float x2, float x3) {
  typedef G g4 __attribute__((ext_vector_type(4)));
  g4 r;
  r[0] = static_cast<G>(x0);
  r[1] = static_cast<G>(x1);
  r[2] = static_cast<G>(x2);
  r[3] = static_cast<G>(x3);
  *reinterpret_cast<g4*>(p) = r;
}

}  // namespace fa
