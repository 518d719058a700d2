// Host-side launch interface between the C ABI (fa_api.hip) and the kernel
// translation units. Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;
  int wl, wr;  // key j visible to query i iff i-wl <= j <= i+wr; -1: no bound on that side
  hipStream_t stream;
  int Hkv;  // K/V heads; divides H (H: multi-head attention)
  // block-sparse mask (nullptr: none): per query head (b, h), at
  // bmask + (b*H + h) * bmask_stride, ceil(N/kMaskBlock)^2 bytes, row-major
  // (query block, key block); a zero byte skips that block
  const uint8_t* bmask = nullptr;
  long long bmask_stride = 0;
  bool masked() const { return wl >= 0 || wr >= 0; }
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* drow;  // workspace: D_i = sum_k dO_ik O_ik, then lse_i * log2(e); 2 x [B,H,N] fp32
  int B, H, N, d;
  float scale;
  int wl, wr;  // key j visible to query i iff i-wl <= j <= i+wr; -1: no bound on that side
  hipStream_t stream;
  int Hkv;  // K/V heads of k, v, dk, dv; divides H (H: multi-head attention)
  // block-sparse mask, as in FwdArgs
  const uint8_t* bmask = nullptr;
  long long bmask_stride = 0;
  bool masked() const { return wl >= 0 || wr >= 0; }
};

// A window bound that never cuts: larger than any distance between a query
// and a key, small enough that i + kUnbounded and i - kUnbounded stay in int.
constexpr int kUnbounded = 1 << 30;

// Query rows and keys per block of a block-sparse mask.
constexpr int kMaskBlock = 128;

// FP8 forward: byte offsets of the workspace regions (each 256-byte
// aligned) and its total size.
struct Fp8Layout {
  size_t q8, qs, k8, ks, v8, vs, bytes;
};
Fp8Layout fp8_layout(int B, int H, int Hkv, int N, int d);

struct Fp8PrepArgs {
  const void* q;
  const void* k;
  const void* v;
  uint32_t sign_mask[4];  // bit j set: sign s_j = -1 (used when rotate != 0)
  int rotate;             // apply diag(s) H to Q and K
  void* workspace;
  int B, H, Hkv, N, d;
  hipStream_t stream;
};

struct Fp8FwdArgs {
  const void* workspace;  // filled by the prepare launch with the same shapes
  void* o;
  float* lse;
  int B, H, Hkv, N, d;
  float scale;
  int wl, wr;
  hipStream_t stream;
};

hipError_t launch_fp8_prepare(const Fp8PrepArgs& a);
hipError_t launch_forward_fp8(const Fp8FwdArgs& a);
long long fp8_prepare_grid_size(int B, int H, int Hkv, int N);

hipError_t launch_forward_bf16(const FwdArgs& a);
hipError_t launch_forward_f32(const FwdArgs& a);
hipError_t launch_backward_prep(const BwdArgs& a);   // uses o, dout, lse, drow
hipError_t launch_backward_grads(const BwdArgs& a);  // uses q, k, v, dout, drow, outputs

// Workgroups the forward launch uses (for grid-size validation).
long long forward_grid_size(int B, int H, int N);
long long backward_grid_size(int B, int H, int Hkv, int N);

}  // namespace fa
