// C ABI of libfa.so: argument validation, then kernel launches on the
// caller's stream. Declarations and the contract are in include/fa.h.
#include "fa.h"

#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa_launch.h"

// Static scratch of fa_backward_noalloc: the row terms of the backward pass
// (D, then lse * log2(e), 2 x [B,H,N] fp32) for callers that cannot
// allocate. At most kScratchRows rows (B * H * N): 16 MiB on every GPU the
// library runs on, held until the process ends. Host code never passes this
// name to a kernel (on the host it is only a stand-in): it uses the device
// address that scratch_address() looks up per device.
namespace {
constexpr long long kScratchRows = 2LL << 20;
constexpr size_t kScratchBytes = 2 * (size_t)kScratchRows * sizeof(float);
}  // namespace
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr long long kMaxGrid = 0x7fffffffLL;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by the forward and backward entry points, in the order
// documented in fa.h. Returns FA_OK and sets *empty when there is nothing to
// compute.
int check_common(int B, int H, int Hkv, int N, int d, float scale, int wl, int wr, bool* empty) {
  if (wl < -1 || wr < -1) return FA_ERR_ARG;
  if (!isfinite(scale)) return FA_ERR_ARG;
  if (d != 64 && d != 128 && d != 256) return FA_ERR_HEADDIM;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  // K/V heads: at least one, dividing H (unless there are no heads at all)
  if (Hkv < 0 || (H > 0 && (Hkv == 0 || H % Hkv != 0))) return FA_ERR_SHAPE;
  *empty = (B == 0 || H == 0 || N == 0);
  if (*empty) return FA_OK;
  // one head of one tensor must be addressable with 32-bit byte offsets
  if ((long long)N * d * (long long)sizeof(float) > kMaxGrid) return FA_ERR_SHAPE;
  // every head takes at least one workgroup; this also keeps the grid sizes
  // below from overflowing
  if ((long long)B * H > kMaxGrid) return FA_ERR_SHAPE;
  if (fa::forward_grid_size(B, H, N) > kMaxGrid) return FA_ERR_SHAPE;
  if (fa::backward_grid_size(B, H, Hkv, N) > kMaxGrid) return FA_ERR_SHAPE;
  return FA_OK;
}

int check_ptrs(const void* const* ptrs, int n) {
  for (int i = 0; i < n; ++i)
    if (ptrs[i] == nullptr) return FA_ERR_NULL;
  for (int i = 0; i < n; ++i)
    if (!aligned16(ptrs[i])) return FA_ERR_ALIGN;
  return FA_OK;
}

// The block mask of the block-sparse calls: any address (bytes), a
// nonnegative head stride. nullptr stands for "no mask" inside the library,
// so the block-sparse calls check it here.
int check_mask(const uint8_t* mask, long long stride, int B, int H, int N) {
  if (mask == nullptr) return FA_ERR_NULL;
  if (stride < 0) return FA_ERR_ARG;
  // the last head's mask must be addressable: (B*H - 1) * stride + nb*nb bytes
  // past the pointer in 64 bits (the kernels index it with size_t)
  const long long nb = (N + fa::kMaskBlock - 1) / fa::kMaskBlock;
  const long long heads = (long long)B * H;
  if (stride > 0 && heads > 1 && heads - 1 > (LLONG_MAX - nb * nb) / stride) return FA_ERR_ARG;
  return FA_OK;
}

// A window bound of N - 1 or more cuts no key of an N-key head, so it is the
// same mask as no bound on that side (-1). Mapping it to -1 here keeps every
// bound the kernels see below N, so that a row or key index plus a bound
// stays within int whatever the caller passes (INT_MAX included).
int norm_bound(int w, int N) { return w >= N - 1 ? -1 : w; }

bool workspace_ok(const void* ws, size_t bytes, int B, int H, int N, int d) {
  return ws != nullptr && aligned16(ws) && bytes >= fa_backward_workspace_size(B, H, N, d);
}

int forward_common(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int Hkv, int N, int d, float scale, int wl, int wr, hipStream_t stream,
                   bool f32, bool sparse = false, const uint8_t* mask = nullptr,
                   long long mask_stride = 0) {
  bool empty = false;
  int st = check_common(B, H, Hkv, N, d, scale, wl, wr, &empty);
  if (st != FA_OK || empty) return st;
  wl = norm_bound(wl, N);
  wr = norm_bound(wr, N);
  const void* ptrs[5] = {q, k, v, o, lse};
  st = check_ptrs(ptrs, 5);
  if (st != FA_OK) return st;
  if (sparse && (st = check_mask(mask, mask_stride, B, H, N)) != FA_OK) return st;
  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, wl, wr, stream, Hkv, mask, mask_stride};
  hipError_t e = f32 ? fa::launch_forward_f32(a) : fa::launch_forward_bf16(a);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int grads_common(const void* q, const void* k, const void* v, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N,
                 int d, float scale, int wl, int wr, const void* workspace,
                 size_t workspace_bytes, hipStream_t stream, bool sparse = false,
                 const uint8_t* mask = nullptr, long long mask_stride = 0) {
  bool empty = false;
  int st = check_common(B, H, Hkv, N, d, scale, wl, wr, &empty);
  if (st != FA_OK || empty) return st;
  wl = norm_bound(wl, N);
  wr = norm_bound(wr, N);
  const void* ptrs[8] = {q, k, v, dout, lse, dq, dk, dv};
  st = check_ptrs(ptrs, 8);
  if (st != FA_OK) return st;
  if (sparse && (st = check_mask(mask, mask_stride, B, H, N)) != FA_OK) return st;
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d)) return FA_ERR_WORKSPACE;
  fa::BwdArgs a{q, k, v, nullptr, dout, lse, dq, dk, dv,
                static_cast<float*>(const_cast<void*>(workspace)), B, H, N, d, scale, wl, wr,
                stream, Hkv, mask, mask_stride};
  return fa::launch_backward_grads(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int backward_common(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                    int H, int Hkv, int N, int d, float scale, int wl, int wr, void* workspace,
                    size_t workspace_bytes, hipStream_t stream, bool sparse = false,
                    const uint8_t* mask = nullptr, long long mask_stride = 0) {
  bool empty = false;
  int st = check_common(B, H, Hkv, N, d, scale, wl, wr, &empty);
  if (st != FA_OK || empty) return st;
  wl = norm_bound(wl, N);
  wr = norm_bound(wr, N);
  const void* ptrs[9] = {q, k, v, o, dout, lse, dq, dk, dv};
  st = check_ptrs(ptrs, 9);
  if (st != FA_OK) return st;
  if (sparse && (st = check_mask(mask, mask_stride, B, H, N)) != FA_OK) return st;
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d)) return FA_ERR_WORKSPACE;
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, static_cast<float*>(workspace),
                B, H, N, d, scale, wl, wr, stream, Hkv, mask, mask_stride};
  if (fa::launch_backward_prep(a) != hipSuccess) return FA_ERR_HIP;
  return fa::launch_backward_grads(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// FP8 calls: the sign vector (host memory, d entries of +1 or -1, or NULL
// for no rotation) as a bit mask; false if an entry is neither.
bool sign_mask(const signed char* signs, int d, uint32_t mask[4], int* rotate) {
  mask[0] = mask[1] = mask[2] = mask[3] = 0;
  *rotate = signs != nullptr;
  if (signs == nullptr) return true;
  for (int j = 0; j < d; ++j) {
    if (signs[j] == -1) mask[j >> 5] |= 1u << (j & 31);
    else if (signs[j] != 1) return false;
  }
  return true;
}

int fp8_check(int B, int H, int Hkv, int N, int d, float scale, int wl, int wr, bool* empty) {
  if (d == 256) return FA_ERR_HEADDIM;  // the FP8 path supports d = 64 and 128
  int st = check_common(B, H, Hkv, N, d, scale, wl, wr, empty);
  if (st != FA_OK || *empty) return st;
  if (fa::fp8_prepare_grid_size(B, H, Hkv, N) > kMaxGrid) return FA_ERR_SHAPE;
  return FA_OK;
}

bool fp8_workspace_ok(const void* ws, size_t bytes, int B, int H, int Hkv, int N, int d) {
  return ws != nullptr && aligned16(ws) && bytes >= fa::fp8_layout(B, H, Hkv, N, d).bytes;
}

int fp8_prepare(const void* q, const void* k, const void* v, const signed char* signs, int B,
                int H, int Hkv, int N, int d, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  const void* ptrs[3] = {q, k, v};
  int st = check_ptrs(ptrs, 3);
  if (st != FA_OK) return st;
  fa::Fp8PrepArgs a{q, k, v, {0, 0, 0, 0}, 0, workspace, B, H, Hkv, N, d, stream};
  if (!sign_mask(signs, d, a.sign_mask, &a.rotate)) return FA_ERR_ARG;
  if (!fp8_workspace_ok(workspace, workspace_bytes, B, H, Hkv, N, d)) return FA_ERR_WORKSPACE;
  return fa::launch_fp8_prepare(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fp8_forward(const void* workspace, size_t workspace_bytes, void* o, float* lse, int B, int H,
                int Hkv, int N, int d, float scale, int wl, int wr, hipStream_t stream) {
  const void* ptrs[2] = {o, lse};
  int st = check_ptrs(ptrs, 2);
  if (st != FA_OK) return st;
  if (!fp8_workspace_ok(workspace, workspace_bytes, B, H, Hkv, N, d)) return FA_ERR_WORKSPACE;
  fa::Fp8FwdArgs a{workspace, o, lse, B, H, Hkv, N, d, scale, wl, wr, stream};
  return fa::launch_forward_fp8(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Device address of `scratch` on the current device. Each GPU holds its own
// copy of the array at its own address; it is looked up once per device,
// with that device current, and kept.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
        return FA_ERR_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FA_OK;
}

// The causal flag of the entry points without a window: 1 is the window
// (-1, 0), 0 no mask; anything else is FA_ERR_ARG, reported as an invalid
// bound.
int causal_left(int causal) { return (causal == 0 || causal == 1) ? -1 : -2; }
int causal_right(int causal) { return causal == 1 ? 0 : (causal == 0 ? -1 : -2); }

}  // namespace

extern "C" {

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, hipStream_t stream) {
  return forward_common(q, k, v, o, lse, B, H, H, N, d, scale, causal_left(causal),
                        causal_right(causal), stream, false);
}

int fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int H_kv, int N, int d, float scale, int causal, hipStream_t stream) {
  return forward_common(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal_left(causal),
                        causal_right(causal), stream, false);
}

int fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                   int H, int N, int d, float scale, int causal, hipStream_t stream) {
  return forward_common(q, k, v, o, lse, B, H, H, N, d, scale, causal_left(causal),
                        causal_right(causal), stream, true);
}

size_t fa_backward_workspace_size(int B, int H, int N, int d) {
  bool empty = false;
  if (check_common(B, H, H, N, d, 1.0f, -1, -1, &empty) != FA_OK || empty) return 0;
  return 2 * (size_t)B * (size_t)H * (size_t)N * sizeof(float);  // D and lse * log2(e)
}

int fa_backward_prep(const void* o, const void* dout, const float* lse, int B, int H, int N,
                     int d, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  bool empty = false;
  int st = check_common(B, H, H, N, d, 1.0f, -1, -1, &empty);
  if (st != FA_OK || empty) return st;
  const void* ptrs[3] = {o, dout, lse};
  st = check_ptrs(ptrs, 3);
  if (st != FA_OK) return st;
  if (!workspace_ok(workspace, workspace_bytes, B, H, N, d)) return FA_ERR_WORKSPACE;
  fa::BwdArgs a{nullptr, nullptr, nullptr, o, dout, lse, nullptr, nullptr, nullptr,
                static_cast<float*>(workspace), B, H, N, d, 1.0f, -1, -1, stream, H};
  return fa::launch_backward_prep(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_backward_grads(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int B, int H, int N,
                      int d, float scale, int causal, const void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return grads_common(q, k, v, dout, lse, dq, dk, dv, B, H, H, N, d, scale, causal_left(causal),
                      causal_right(causal), workspace, workspace_bytes, stream);
}

int fa_backward_grads_gqa(const void* q, const void* k, const void* v, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv, int B, int H, int H_kv,
                          int N, int d, float scale, int causal, const void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return grads_common(q, k, v, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale,
                      causal_left(causal), causal_right(causal), workspace, workspace_bytes,
                      stream);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                float scale, int causal, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  return backward_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, scale,
                         causal_left(causal), causal_right(causal), workspace, workspace_bytes,
                         stream);
}

int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                    int H, int H_kv, int N, int d, float scale, int causal, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return backward_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale,
                         causal_left(causal), causal_right(causal), workspace, workspace_bytes,
                         stream);
}

int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                        int H, int N, int d, float scale, int causal, hipStream_t stream) {
  bool empty = false;
  const int wl = causal_left(causal), wr = causal_right(causal);
  int st = check_common(B, H, H, N, d, scale, wl, wr, &empty);
  if (st != FA_OK || empty) return st;
  const void* ptrs[9] = {q, k, v, o, dout, lse, dq, dk, dv};
  st = check_ptrs(ptrs, 9);
  if (st != FA_OK) return st;
  if ((long long)B * H * N > kScratchRows) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != FA_OK) return st;
  // the row-term launch writes every row the grads launch reads: nothing in
  // the scratch needs clearing, whatever an earlier call left there
  return backward_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, H, N, d, scale, wl, wr, ws,
                         kScratchBytes, stream);
}

int fa_forward_window(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int H_kv, int N, int d, float scale, int window_left,
                      int window_right, hipStream_t stream) {
  return forward_common(q, k, v, o, lse, B, H, H_kv, N, d, scale, window_left, window_right,
                        stream, false);
}

int fa_backward_window(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                       int H, int H_kv, int N, int d, float scale, int window_left,
                       int window_right, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return backward_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale,
                         window_left, window_right, workspace, workspace_bytes, stream);
}

int fa_backward_grads_window(const void* q, const void* k, const void* v, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv, int B, int H,
                             int H_kv, int N, int d, float scale, int window_left,
                             int window_right, const void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  return grads_common(q, k, v, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale, window_left,
                      window_right, workspace, workspace_bytes, stream);
}

int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int H_kv, int N, int d, float scale, int window_left,
                            int window_right, const uint8_t* block_mask,
                            long long block_mask_head_stride, hipStream_t stream) {
  return forward_common(q, k, v, o, lse, B, H, H_kv, N, d, scale, window_left, window_right,
                        stream, false, true, block_mask, block_mask_head_stride);
}

int fa_backward_block_sparse(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             int B, int H, int H_kv, int N, int d, float scale, int window_left,
                             int window_right, const uint8_t* block_mask,
                             long long block_mask_head_stride, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return backward_common(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale,
                         window_left, window_right, workspace, workspace_bytes, stream, true,
                         block_mask, block_mask_head_stride);
}

int fa_backward_grads_block_sparse(const void* q, const void* k, const void* v,
                                   const void* dout, const float* lse, void* dq, void* dk,
                                   void* dv, int B, int H, int H_kv, int N, int d, float scale,
                                   int window_left, int window_right, const uint8_t* block_mask,
                                   long long block_mask_head_stride, const void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
  return grads_common(q, k, v, dout, lse, dq, dk, dv, B, H, H_kv, N, d, scale, window_left,
                      window_right, workspace, workspace_bytes, stream, true, block_mask,
                      block_mask_head_stride);
}

size_t fa_forward_fp8_workspace_size(int B, int H, int H_kv, int N, int d) {
  bool empty = false;
  if (fp8_check(B, H, H_kv, N, d, 1.0f, -1, -1, &empty) != FA_OK || empty) return 0;
  return fa::fp8_layout(B, H, H_kv, N, d).bytes;
}

int fa_fp8_prepare(const void* q, const void* k, const void* v, const signed char* signs, int B,
                   int H, int H_kv, int N, int d, void* workspace, size_t workspace_bytes,
                   hipStream_t stream) {
  bool empty = false;
  int st = fp8_check(B, H, H_kv, N, d, 1.0f, -1, -1, &empty);
  if (st != FA_OK || empty) return st;
  return fp8_prepare(q, k, v, signs, B, H, H_kv, N, d, workspace, workspace_bytes, stream);
}

int fa_forward_fp8_prepared(const void* workspace, size_t workspace_bytes, void* o, float* lse,
                            int B, int H, int H_kv, int N, int d, float scale, int causal,
                            hipStream_t stream) {
  bool empty = false;
  const int wl = causal_left(causal), wr = causal_right(causal);
  int st = fp8_check(B, H, H_kv, N, d, scale, wl, wr, &empty);
  if (st != FA_OK || empty) return st;
  return fp8_forward(workspace, workspace_bytes, o, lse, B, H, H_kv, N, d, scale, wl, wr, stream);
}

int fa_forward_fp8(const void* q, const void* k, const void* v, const signed char* signs,
                   void* o, float* lse, int B, int H, int H_kv, int N, int d, float scale,
                   int causal, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  bool empty = false;
  const int wl = causal_left(causal), wr = causal_right(causal);
  int st = fp8_check(B, H, H_kv, N, d, scale, wl, wr, &empty);
  if (st != FA_OK || empty) return st;
  const void* ptrs[2] = {o, lse};
  st = check_ptrs(ptrs, 2);
  if (st != FA_OK) return st;
  st = fp8_prepare(q, k, v, signs, B, H, H_kv, N, d, workspace, workspace_bytes, stream);
  if (st != FA_OK) return st;
  return fp8_forward(workspace, workspace_bytes, o, lse, B, H, H_kv, N, d, scale, wl, wr, stream);
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE:
      return "invalid shape: B, H or N negative, K/V heads not dividing H, or the problem too large";
    case FA_ERR_HEADDIM:
      return "unsupported head dimension (supported: 64, 128, 256; the FP8 calls 64, 128)";
    case FA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case FA_ERR_ARG:
      return "invalid argument: causal must be 0 or 1, window bounds >= -1, scale finite, "
             "signs +1 or -1, block-mask head stride >= 0";
    case FA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case FA_ERR_HIP: return "the HIP runtime reported an error at launch";
    case FA_ERR_SCRATCH:
      return "problem too large for the static scratch of fa_backward_noalloc "
             "(B*H*N at most 2097152)";
    default: return "unknown status";
  }
}

}  // extern "C"
