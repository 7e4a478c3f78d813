// C-ABI host layer of libfa: argument validation, kernel selection and
// launch on the caller's stream. Declarations and the contract of every
// entry point are in include/fa.h.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "fa.h"
#include "fa_kernels.h"

// Fixed device scratch of fa_bwd_noalloc: the D_i = dO_i . O_i rows of one
// backward call (fp32 [B][H][N]). Each GPU the library runs on holds its own
// copy from module load until the process ends. Host code never passes this
// name to a kernel: in host code it is a stand-in, not a device address; the
// device address comes from hipGetSymbolAddress (scratch_ptr below).
__device__ __attribute__((aligned(256))) float scratch[FA_BWD_NOALLOC_MAX_ROWS];

namespace {

constexpr int64_t kMaxI32 = 2147483647;
constexpr int kMaxDevices = 64;

// Compute units and XCDs of each device, read once (the tile orders and the
// resident-grid test of the kernels follow the device's topology).
std::atomic<int> g_ncu[kMaxDevices];
std::atomic<int> g_nxcd[kMaxDevices];

hipError_t device_topology(int& ncu, int& nxcd) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached && g_ncu[dev].load(std::memory_order_acquire) > 0) {
    ncu = g_ncu[dev].load(std::memory_order_acquire);
    nxcd = g_nxcd[dev].load(std::memory_order_acquire);
    return hipSuccess;
  }
  int c = 0, x = 0;
  e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (hipDeviceGetAttribute(&x, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || x <= 0) {
    (void)hipGetLastError();  // attribute not reported: treat the device as one die
    x = 1;
  }
  ncu = c > 0 ? c : 1;
  nxcd = x;
  if (cached) {
    g_nxcd[dev].store(nxcd, std::memory_order_release);
    g_ncu[dev].store(ncu, std::memory_order_release);
  }
  return hipSuccess;
}

// Device address of `scratch` on the current device, looked up once per
// device (each device holds its own copy at its own address).
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return hipSuccess;
}

// Clears a pending error that earlier work of the calling thread left behind
// (it is not this call's), then fills in the device topology.
hipError_t prepare_launch(fa::AttnArgs& a) {
  (void)hipGetLastError();
  return device_topology(a.ncu, a.nxcd);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check(const fa_params* p) {
  if (p == nullptr) return FA_ERR_NULL;
  if (p->B < 0 || p->H < 0 || p->N < 0 || p->d < 0) return FA_ERR_SHAPE;
  if (p->d != 64 && p->d != 128) return FA_ERR_HEADDIM;
  if (p->in_dtype < FA_F32 || p->in_dtype > FA_BF16) return FA_ERR_DTYPE;
  if (p->grad_dtype != FA_F32 && p->grad_dtype != p->in_dtype) return FA_ERR_DTYPE;
  // Per-head byte offsets (rows x d x element size) are 32-bit; the grid is one dimension.
  const int64_t elt = p->in_dtype == FA_F32 ? 4 : 2;
  if (p->N > kMaxI32 / (p->d * 4) || p->N > kMaxI32 / (p->d * elt)) return FA_ERR_SHAPE;
  if (p->B > 0 && p->H > kMaxI32 / p->B) return FA_ERR_SHAPE;
  const int64_t bh = p->B * p->H;
  const int64_t tiles = (p->N + 127) / 128;
  if (bh > 0 && tiles > kMaxI32 / bh) return FA_ERR_SHAPE;
  if (!std::isfinite(p->scale) || !(p->scale > 0.f)) return FA_ERR_SCALE;
  if (!(p->dropout_p >= 0.0 && p->dropout_p < 1.0)) return FA_ERR_DROPOUT;
  if (p->block_mask != nullptr && (p->mask_block <= 0 || p->mask_block % 128 != 0)) return FA_ERR_MASK;
  return FA_OK;
}

fa::AttnArgs make_args(const fa_params* p) {
  fa::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.N = (int)p->N;
  a.H = (int)p->H;
  a.BH = (int)(p->B * p->H);
  a.causal = p->causal ? 1 : 0;
  a.bmask = p->block_mask;
  a.mask_block = p->block_mask ? p->mask_block : 128;
  a.nb = (int)((p->N + a.mask_block - 1) / a.mask_block);
  a.scale = p->scale;
  a.sl2 = (float)((double)p->scale * 1.4426950408889634);
  a.rp = (float)(1.0 / (1.0 - p->dropout_p));
  a.kq = (float)(1.0 - p->dropout_p);
  a.thresh = (uint32_t)std::floor(p->dropout_p * 65536.0) << 16;
  a.seed_lo = (uint32_t)(p->seed & 0xFFFFFFFFu);
  a.seed_hi = (uint32_t)(p->seed >> 32);
  a.ones16 = 0x00010001u;
  return a;
}

fa::Elt elt(int32_t t) { return static_cast<fa::Elt>(t); }

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid or too large shape (B, H, N)";
    case FA_ERR_DTYPE: return "unsupported dtype combination";
    case FA_ERR_HEADDIM: return "head dimension d must be 64 or 128";
    case FA_ERR_DROPOUT: return "dropout_p must lie in [0, 1)";
    case FA_ERR_MASK: return "mask_block must be a positive multiple of 128";
    case FA_ERR_ALIGN: return "data pointers must be 16-byte aligned";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP runtime error at launch";
    case FA_ERR_SCALE: return "scale must be finite and > 0";
    case FA_ERR_RANGE: return "window outside [0, N) or (b, h) outside [0, B) x [0, H)";
    case FA_ERR_SCRATCH: return "B*H*N exceeds the fixed scratch of fa_bwd_noalloc (FA_BWD_NOALLOC_MAX_ROWS)";
    default: return "unknown status";
  }
}

int fa_check_params(const fa_params* p) { return check(p); }

int fa_fwd(const fa_params* p, const void* Q, const void* K, const void* V, void* O, float* LSE, void* stream) {
  const int st = check(p);
  if (st != FA_OK) return st;
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULL;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE)) return FA_ERR_ALIGN;
  if (p->B * p->H * p->N == 0) return FA_OK;
  fa::AttnArgs a = make_args(p);
  a.q = Q;
  a.k = K;
  a.v = V;
  a.out = O;
  a.lse = LSE;
  // The dropout kernels draw keep bits only when some key can be dropped
  // (T16 = floor(p * 2^16) >= 1). Below that every key is kept and the plain
  // kernel computes the same output: its epilogue scales by 1 / (1 - p) too.
  const bool dropout = a.thresh != 0;
  hipError_t e = prepare_launch(a);
  if (e == hipSuccess) e = fa::launch_fwd(elt(p->in_dtype), (int)p->d, dropout, a, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(const fa_params* p) {
  if (check(p) != FA_OK) return 0;
  const size_t rows = (size_t)(p->B * p->H * p->N);
  return (rows * sizeof(float) + 255) / 256 * 256;
}

namespace {

// Shared validation and launch of the backward stages (stage bit 1: dQ and D,
// bit 2: dK and dV). Pointers a stage does not touch may be NULL.
int bwd_stage(int stage, const fa_params* p, const void* Q, const void* K, const void* V, const void* O,
              const float* LSE, const void* dO, void* dQ, void* dK, void* dV, void* workspace,
              size_t workspace_bytes, void* stream) {
  const int st = check(p);
  if (st != FA_OK) return st;
  if (!Q || !K || !V || !LSE || !dO) return FA_ERR_NULL;
  if ((stage & 1) && (!O || !dQ)) return FA_ERR_NULL;
  if ((stage & 2) && (!dK || !dV)) return FA_ERR_NULL;
  const void* ptrs[] = {Q, K, V, O, LSE, dO, dQ, dK, dV};
  for (const void* x : ptrs)
    if (x != nullptr && !aligned16(x)) return FA_ERR_ALIGN;
  const size_t need = fa_bwd_workspace_bytes(p);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  if (workspace != nullptr && !aligned16(workspace)) return FA_ERR_ALIGN;
  if (p->B * p->H * p->N == 0) return FA_OK;
  fa::AttnArgs a = make_args(p);
  a.q = Q;
  a.k = K;
  a.v = V;
  a.o = O;
  a.lse = const_cast<float*>(LSE);
  a.dout = dO;
  a.dq = dQ;
  a.dk = dK;
  a.dv = dV;
  a.delta = static_cast<float*>(workspace);
  hipError_t e = prepare_launch(a);
  if (e == hipSuccess)
    e = fa::launch_bwd(elt(p->in_dtype), elt(p->grad_dtype), (int)p->d, p->dropout_p > 0.0, stage, a,
                       (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

int fa_bwd(const fa_params* p, const void* Q, const void* K, const void* V, const void* O, const float* LSE,
           const void* dO, void* dQ, void* dK, void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dK || !dV) return FA_ERR_NULL;  // all three gradients are required here
  return bwd_stage(3, p, Q, K, V, O, LSE, dO, dQ, dK, dV, workspace, workspace_bytes, stream);
}

int fa_bwd_noalloc(const fa_params* p, const void* Q, const void* K, const void* V, const void* O,
                   const float* LSE, const void* dO, void* dQ, void* dK, void* dV, void* stream) {
  const int st = check(p);
  if (st != FA_OK) return st;
  if (!Q || !K || !V || !O || !LSE || !dO || !dQ || !dK || !dV) return FA_ERR_NULL;
  if (p->B * p->H * p->N > (int64_t)FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH;
  if (p->B * p->H * p->N == 0) return FA_OK;
  void* ws = nullptr;
  if (scratch_ptr(&ws) != hipSuccess) return FA_ERR_HIP;
  return bwd_stage(3, p, Q, K, V, O, LSE, dO, dQ, dK, dV, ws, sizeof(float) * (size_t)FA_BWD_NOALLOC_MAX_ROWS,
                   stream);
}

int fa_bwd_dq(const fa_params* p, const void* Q, const void* K, const void* V, const void* O, const float* LSE,
              const void* dO, void* dQ, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_stage(1, p, Q, K, V, O, LSE, dO, dQ, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int fa_bwd_dkdv(const fa_params* p, const void* Q, const void* K, const void* V, const float* LSE, const void* dO,
                void* dK, void* dV, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_stage(2, p, Q, K, V, nullptr, LSE, dO, nullptr, dK, dV, workspace, workspace_bytes, stream);
}

int fa_dropout_mask(const fa_params* p, int64_t b, int64_t h, int64_t i0, int64_t rows, int64_t j0, int64_t cols,
                    uint8_t* keep, void* stream) {
  const int st = check(p);
  if (st != FA_OK) return st;
  if (keep == nullptr) return FA_ERR_NULL;
  if (b < 0 || b >= p->B || h < 0 || h >= p->H) return FA_ERR_RANGE;
  if (i0 < 0 || rows < 0 || j0 < 0 || cols < 0 || i0 + rows > p->N || j0 + cols > p->N) return FA_ERR_RANGE;
  if (rows > 0 && cols > kMaxI32 * 256 / rows) return FA_ERR_RANGE;
  if (rows * cols == 0) return FA_OK;
  fa::AttnArgs a = make_args(p);
  hipError_t e = prepare_launch(a);
  if (e == hipSuccess) e = fa::launch_dropout_mask(a, (int)b, (int)h, i0, rows, j0, cols, keep, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
