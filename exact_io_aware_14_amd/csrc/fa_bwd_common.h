// Pieces shared by the two sources of the backward pass: fa_bwd.hip (the
// row-term launch and the grads launch at d = 64 and 128) and fa_bwd_w.hip
// (the grads launch at d = 256): the job sizes and kernel parameters, the
// order in which a grads launch hands out its jobs, and the helpers both
// job kinds use.
#pragma once

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_schedule.h"

namespace fa {
namespace {

// d = 64 and 128 job sizes
constexpr int kKeyBlock = 128;  // keys per dK/dV job
constexpr int kQBlock = 256;    // query rows per dQ job

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* drow;  // D_i
  const float* lse2;  // lse_i * log2(e)
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int BH;           // batch * query heads
  int group;        // query heads per K/V head (1: multi-head attention)
  int N;
  int nkb;          // dK/dV jobs (key blocks) per K/V head
  int nqb;          // dQ jobs (query-row blocks) per query head
  float c;          // scale * log2(e)
  float scale;
  int wl, wr;       // masked kernels: key j visible to query i iff i-wl <= j <= i+wr
  int xcd_remap;
  // block-sparse kernels: the mask of query head h (batch * query heads) at
  // bmask + h * bm_stride, nbm x nbm bytes (query block, key block), a zero
  // byte skipping the block
  const uint8_t* bmask;
  long long bm_stride;
  int nbm;
};

// d = 256 job sizes
constexpr int kKeyBlockW = 128;  // keys per dK/dV job
constexpr int kQBlockW = 128;    // query rows per dQ job

// ---------------------------------------------------------------- layout

// Job of this workgroup in the grads launch (sched::grads_job in
// fa_schedule.h: dK/dV and dQ jobs interleaved evenly over each K/V head's
// slots, XCD-aware, the most expensive blocks first).
using Job = sched::Job;

template <bool CAUSAL>
__device__ __forceinline__ Job job_of(const BwdParams& p) {
  return sched::grads_job(blockIdx.x, p.BH, p.group, p.nkb, p.nqb, p.xcd_remap != 0, CAUSAL);
}

// Start loading 64 floats v[row0 .. row0+63] (zeros past N) into `dst`.
__device__ __forceinline__ void fill_vec(unsigned char* dst, const float* g, int row0, int N,
                                         int lane) {
  const auto r = make_rsrc(g + row0, (uint32_t)(N - row0) * 4u);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)dst, 4, (uint32_t)lane * 4u, 0, 0, 0);
}

// 32x32 outputs of this lane (column c, 4 groups of 4 rows) as bf16 rows:
// element r of block db is d = 32*db + 8*(r/4) + 4*half + (r%4).
template <int D>
__device__ __forceinline__ void store_rows(uint16_t* dst, const f32x16* acc, float sc, int half) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + 8 * g4 + 4 * half;
      const uint2 w = {pack_bf16x2(acc[db][4 * g4] * sc, acc[db][4 * g4 + 1] * sc),
                       pack_bf16x2(acc[db][4 * g4 + 2] * sc, acc[db][4 * g4 + 3] * sc)};
      *reinterpret_cast<uint2*>(dst + d0) = w;
    }
}

template <int D>
BwdParams make_params(const BwdArgs& a) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.drow = a.drow;
  p.lse2 = a.drow + (size_t)a.B * a.H * a.N;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.BH = a.B * a.H;
  p.group = a.H / a.Hkv;
  p.N = a.N;
  const int key_block = D == 256 ? kKeyBlockW : kKeyBlock;
  const int q_block = D == 256 ? kQBlockW : kQBlock;
  p.nkb = (a.N + key_block - 1) / key_block;
  p.nqb = (a.N + q_block - 1) / q_block;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  p.wl = a.wl < 0 ? kUnbounded : a.wl;
  p.wr = a.wr < 0 ? kUnbounded : a.wr;
  p.xcd_remap = (p.BH / p.group) % 8 == 0;
  p.bmask = a.bmask;
  p.bm_stride = a.bmask_stride;
  p.nbm = (a.N + kMaskBlock - 1) / kMaskBlock;
  return p;
}

}  // namespace

// the grads launch at d = 256 (fa_bwd_w.hip)
hipError_t launch_grads_wide(const BwdArgs& a);
hipError_t launch_grads_wide_sparse(const BwdArgs& a);  // with a block-sparse mask

}  // namespace fa
