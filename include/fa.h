/*
 * fa.h -- C ABI of libfa, tiled exact softmax attention for AMD MI355X (gfx950).
 *
 * What is computed (FlashAttention milestone page, nlp-lineage, section "The
 * idea": S = Q K^T, P = softmax(S), O = P V, with matrix product, mask,
 * softmax, dropout and matrix product fused; block-sparse variant in the same
 * section). For every (b, h) slice, with i a query row and j a key row:
 *
 *   S_ij   = scale * (Q_i . K_j)
 *   valid  = (!causal || j <= i) && (!block_mask || block_mask[i/mb][j/mb] != 0)
 *   LSE_i  = log(sum over valid j of exp(S_ij))      (natural log, fp32)
 *   P_ij   = exp(S_ij - LSE_i) if valid, else 0
 *   O_i    = sum_j P_ij * Z_ij / (1 - dropout_p) * V_j
 *
 * The N x N matrices S and P are never written to memory: the kernels tile
 * Q, K and V through on-chip memory and keep the per-row running maximum and
 * sum (online softmax; same section), and the backward recomputes S and P
 * tile by tile from Q, K and LSE (recomputation; same section).
 *
 * Layout: Q, K, V, O, dO, dQ, dK, dV are [B][H][N][d] contiguous row-major;
 * LSE is [B][H][N] fp32. All data pointers are DEVICE pointers, 16-byte
 * aligned, owned by the caller, and must stay valid until the work enqueued
 * on `stream` has run. The library allocates nothing, keeps no pointer after
 * a call returns and holds no mutable global state (calls are thread-safe).
 *
 * Errors: every entry point validates its arguments on the host first; on a
 * failed check it returns a nonzero fa_status and enqueues nothing. Before
 * launching it clears the calling thread's pending HIP error (left by
 * earlier work, not by this call), so FA_ERR_HIP reports a failure of this
 * call's own launches. Faults inside kernels surface at the caller's next
 * synchronization. No C++ exception crosses this ABI. Launches go to the
 * current HIP device, which must be the device of `stream`.
 *
 * Conventions: a query row with no valid key yields O_i = 0, LSE_i = -inf
 * and zero gradient contributions. NaN/Inf inputs propagate without any
 * guarantee.
 *
 * Dropout keep bits Z_ij (the pages name dropout as a fused step but give no
 * generator; this library defines one). With fmix32 the MurmurHash3 32-bit
 * finalizer (x ^= x>>16; x *= 0x85EBCA6B; x ^= x>>13; x *= 0xC2B2AE35;
 * x ^= x>>16, all mod 2^32) and mix32 the same steps without the first
 * shift (x *= 0x85EBCA6B; x ^= x>>13; x *= 0xC2B2AE35; x ^= x>>16), one
 * 32-bit word serves the two keys 2m and 2m+1 of a query row:
 *   key(b,h)  = fmix32(fmix32(fmix32(fmix32(lo32(seed) + 0x9E3779B9) ^ hi32(seed)) ^ b) ^ h)
 *   w(i,m)    = mix32(fmix32(key(b,h) ^ i) + m)      (sum mod 2^32)
 *   half(i,j) = bits [16*(j%2), 16*(j%2)+16) of w(i, j/2)  (even j: low half)
 *   Z_ij      = half(i,j) >= T16,  T16 = floor(dropout_p * 2^16) computed in double
 * With dropout_p == 0 no bit is drawn and Z == 1. A key is kept with
 * probability 1 - T16/2^16 (within 2^-16 of 1 - dropout_p); kept values are
 * scaled by 1 / (1 - dropout_p). w depends on i only through
 * fmix32(key ^ i) + m, so two rows of a head whose row words differ by
 * delta (|delta| < N/2) get keep masks that are copies shifted by 2*delta
 * keys: about N^3 / 2^33 such row pairs per head.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 2

/* Element types of Q, K, V, O, dO (in_dtype) and of dQ, dK, dV (grad_dtype). */
typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,       /* B, H or N negative, N*d*4 bytes >= 2^31, or too many tiles */
  FA_ERR_DTYPE = 3,       /* unknown dtype, or grad_dtype not FA_F32 / in_dtype */
  FA_ERR_HEADDIM = 4,     /* d not in {64, 128} */
  FA_ERR_DROPOUT = 5,     /* dropout_p not in [0, 1) */
  FA_ERR_MASK = 6,        /* mask_block not a positive multiple of 128 */
  FA_ERR_ALIGN = 7,       /* a data pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE = 8,   /* workspace NULL or smaller than fa_bwd_workspace_bytes */
  FA_ERR_HIP = 9,         /* the HIP runtime reported an error at launch */
  FA_ERR_SCALE = 10,      /* scale not finite and > 0 */
  FA_ERR_RANGE = 11,      /* fa_dropout_mask window, (b, h) or size out of range */
  FA_ERR_SCRATCH = 12     /* fa_bwd_noalloc: B*H*N above FA_BWD_NOALLOC_MAX_ROWS */
} fa_status;

/* Rows (B*H*N) that the fixed device scratch of fa_bwd_noalloc holds: 2^22
 * fp32 values, 16 MiB per GPU. */
#define FA_BWD_NOALLOC_MAX_ROWS (1 << 22)

typedef struct {
  int64_t B, H, N, d;       /* batch, heads, sequence length, head dimension */
  int32_t in_dtype;         /* fa_dtype of Q, K, V, O, dO */
  int32_t grad_dtype;       /* fa_dtype of dQ, dK, dV: FA_F32 or in_dtype */
  float scale;              /* S = scale * Q K^T; finite and > 0 (usually 1/sqrt(d)) */
  int32_t causal;           /* nonzero: key j is hidden from query i when j > i */
  double dropout_p;         /* in [0, 1) */
  uint64_t seed;            /* dropout key; ignored when dropout_p == 0 */
  const uint8_t* block_mask;/* NULL = dense; else DEVICE uint8 [nb][nb], row-major,
                               nb = ceil(N / mask_block), nonzero = block kept;
                               shared by every (b, h) */
  int32_t mask_block;       /* block edge of block_mask; a multiple of 128 */
} fa_params;

/* Version of this header's ABI (FA_ABI_VERSION). */
int fa_abi_version(void);

/* Static text for a status code. */
const char* fa_status_string(int status);

/* Host-only validation of the parameter block (no HIP call). */
int fa_check_params(const fa_params* p);

/*
 * Forward pass (FlashAttention milestone page, "The idea": score product,
 * mask, softmax, dropout and value product fused, the softmax computed
 * tile by tile from a running row maximum and sum). Reads Q, K, V; writes O
 * (in_dtype) and LSE (fp32, natural log; the pages keep two numbers per row,
 * LSE_i = m_i + log l_i carries both). Enqueued asynchronously on `stream`
 * (a hipStream_t; NULL = default).
 */
int fa_fwd(const fa_params* p, const void* Q, const void* K, const void* V,
           void* O, float* LSE, void* stream);

/* Device workspace that fa_bwd needs for these parameters, in bytes. */
size_t fa_bwd_workspace_bytes(const fa_params* p);

/*
 * Backward pass (FlashAttention milestone page, "The idea": the backward
 * recomputes S and P tile by tile from Q, K and the stored row statistics
 * instead of reading an N x N matrix; pixelation article, "The Recomputation
 * Trade-off"). Reads Q, K, V, O, LSE, dO; writes dQ, dK, dV (grad_dtype).
 * `workspace` is caller-owned device memory of at least
 * fa_bwd_workspace_bytes(p) bytes; its contents on entry do not matter and
 * on return are unspecified.
 */
int fa_bwd(const fa_params* p, const void* Q, const void* K, const void* V,
           const void* O, const float* LSE, const void* dO,
           void* dQ, void* dK, void* dV,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two stages of fa_bwd, for callers that time or schedule them apart.
 * fa_bwd_dq computes D_i = dO_i . O_i into `workspace` and writes dQ;
 * fa_bwd_dkdv reads D from the same workspace and writes dK and dV, so it
 * must be enqueued after fa_bwd_dq (same stream, or an event between them)
 * with the same parameters, inputs and workspace. fa_bwd == fa_bwd_dq
 * followed by fa_bwd_dkdv on one stream.
 */
/*
 * fa_bwd without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). D_i goes to a fixed
 * device array of FA_BWD_NOALLOC_MAX_ROWS fp32 values inside the library
 * (one per GPU, held until the process ends; its address is looked up on
 * the first call on each device). B*H*N above that maximum returns
 * FA_ERR_SCRATCH and enqueues nothing. All calls on one GPU share the array
 * and nothing needs clearing between them (each call writes every D_i it
 * reads); two calls that overlap on one GPU (other streams, other threads)
 * race on it. Results are bit-identical to fa_bwd.
 */
int fa_bwd_noalloc(const fa_params* p, const void* Q, const void* K, const void* V,
                   const void* O, const float* LSE, const void* dO,
                   void* dQ, void* dK, void* dV, void* stream);

int fa_bwd_dq(const fa_params* p, const void* Q, const void* K, const void* V,
              const void* O, const float* LSE, const void* dO, void* dQ,
              void* workspace, size_t workspace_bytes, void* stream);
int fa_bwd_dkdv(const fa_params* p, const void* Q, const void* K, const void* V,
                const float* LSE, const void* dO, void* dK, void* dV,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dropout keep bits (FlashAttention milestone page, "The idea": dropout is
 * one of the fused steps, regenerated in the backward rather than stored).
 * Writes the keep bits Z_ij (1 = kept) of head (b, h) for query rows
 * [i0, i0+rows) and key columns [j0, j0+cols) into the DEVICE buffer
 * keep[rows][cols], with the same device function the fused kernels use.
 * Masking (causal, block mask) is not applied. With dropout_p == 0 every bit
 * is 1. The window must lie inside [0, N) x [0, N), (b, h) inside
 * [0, B) x [0, H), and rows * cols must stay below 2^39; otherwise the call
 * returns FA_ERR_RANGE.
 */
int fa_dropout_mask(const fa_params* p, int64_t b, int64_t h, int64_t i0, int64_t rows,
                    int64_t j0, int64_t cols, uint8_t* keep, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
