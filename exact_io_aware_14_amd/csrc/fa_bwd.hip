// Backward exact attention for gfx950, in two launches on one stream:
//
//   prep:  D_i = sum_k dO_ik O_ik                               (HBM-bound)
//   grads: one launch holding two kinds of workgroup, interleaved so the
//          most expensive ones of both kinds start first:
//          dK/dV jobs, one per (batch, head, block of 128 keys), walk the
//          query tiles and accumulate dV_j = sum_i P_ij dO_i and
//          dK_j = scale * sum_i dS_ij Q_i for their own keys;
//          dQ jobs, one per (batch, head, block of 128 query rows), walk the
//          key tiles and accumulate dQ_i = scale * sum_j dS_ij K_j
//
// with P_ij = exp(scale q_i.k_j - lse_i) recomputed from the forward pass's
// logsumexp instead of being stored ("Flash Attention: بهینه‌سازی مکانیزم
// توجه در ترنسفورمرها" (deepfa.ir), recomputation technique; "Flash
// Attention: Rivoluzionando l'Efficienza dei Modelli Transformer" (unite.ai),
// key idea 2), dP = dO V^T and dS = P * (dP - D). The pages give no backward
// equations; these are the derivative of softmax(scale Q K^T) V. The
// parallelisation over column blocks of the attention matrix for the
// backward pass is the one of the nearauto.com FlashAttention-2 article,
// section "より優れた並列処理". Every output element is written by exactly one
// workgroup, so no atomics are needed and results are deterministic.
//
// MFMA formulations (32x32x16 bf16; layouts in fa_common.h):
//   dK/dV kernel, lane = key:   S = Q K^T and dP = dO V^T with K^T, V^T held
//     in registers as B operands; dV^T += dO^T P and dK^T += Q^T dS with the
//     probabilities repacked in-lane as B operands and dO^T, Q^T transposed
//     in LDS as A operands.
//   dQ kernel, lane = query:    S^T = K Q^T and dP^T = V dO^T with Q^T, dO^T
//     in registers; dQ^T += K^T dS^T with K^T transposed in LDS.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBlock = 128;  // keys (dK/dV) or query rows (dQ) per workgroup
constexpr int kTile = 64;    // rows of the streamed tile

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;
  const float* drow;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int BH;
  int N;
  int nblk;         // 128-row blocks per head
  float c;          // scale * log2(e)
  float scale;
  int xcd_remap;
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- rows

template <int D>
__global__ __launch_bounds__(kThreads) void bwd_rows_kernel(const uint16_t* o,
                                                            const uint16_t* dout, float* drow,
                                                            long long rows) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = kThreads / kLanesPerRow;
  const long long row = (long long)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int ch = threadIdx.x % kLanesPerRow;
  float acc = 0.0f;
  if (row < rows) {
    uint4 a = *reinterpret_cast<const uint4*>(o + row * D + ch * 8);
    uint4 b = *reinterpret_cast<const uint4*>(dout + row * D + ch * 8);
    const uint32_t* wa = reinterpret_cast<const uint32_t*>(&a);
    const uint32_t* wb = reinterpret_cast<const uint32_t*>(&b);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = __builtin_fmaf(bf_lo(wa[j]), bf_lo(wb[j]), acc);
      acc = __builtin_fmaf(bf_hi(wa[j]), bf_hi(wb[j]), acc);
    }
  }
#pragma unroll
  for (int off = kLanesPerRow / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (ch == 0 && row < rows) drow[row] = acc;
}

// Job of this workgroup in the grads launch. Every head owns 2*nblk jobs,
// alternately dK/dV and dQ, each sequence ordered from the most expensive
// block down (causal: dK/dV of the first key blocks, dQ of the last query
// blocks). Consecutive workgroups go to the 8 XCDs in turn; when the head
// count allows, each XCD gets whole heads so their K/V and Q/dO stay in its L2.
struct Job {
  int bh;
  int blk;
  bool is_dq;
};

template <bool CAUSAL>
__device__ __forceinline__ Job job_of(const BwdParams& p) {
  const int L = blockIdx.x;
  const int per_head = 2 * p.nblk;
  int bh, j;
  if (p.xcd_remap) {
    const int xcd = L & 7, idx = L >> 3;
    bh = (idx / per_head) * 8 + xcd;
    j = idx % per_head;
  } else {
    bh = L % p.BH;
    j = L / p.BH;
  }
  Job job;
  job.bh = bh;
  job.is_dq = (j & 1) != 0;
  const int rank = j >> 1;
  job.blk = (CAUSAL && job.is_dq) ? (p.nblk - 1 - rank) : rank;
  return job;
}

// Four consecutive rows (r0 .. r0+3 of the tile starting at `row0`) of chunk
// `ch`; rows past the end of the buffer read as zeros.
template <int D>
__device__ __forceinline__ void load_rows4(__amdgpu_buffer_rsrc_t r, int row0, int r0, int ch,
                                           uint4 w[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = load8<uint16_t>(r, (uint32_t)((row0 + r0 + i) * D + ch * 8));
}

// ---------------------------------------------------------------- dK / dV

template <int D>
struct KVSmem {
  uint16_t q[kTile * D];    // Q tile, row-major
  uint16_t qt[D * kTile];   // Q tile, transposed
  uint16_t g[kTile * D];    // dO tile, row-major
  uint16_t gt[D * kTile];   // dO tile, transposed
  float lse2[kTile];        // lse * log2(e); +inf past N
  float dr[kTile];          // D_i; 0 past N
};

template <int D>
struct QSmem {
  uint16_t k[kTile * D];   // K tile, row-major
  uint16_t kt[D * kTile];  // K tile, transposed
  uint16_t v[kTile * D];   // V tile, row-major
};

template <int D>
constexpr size_t kGradsSmem = sizeof(KVSmem<D>) > sizeof(QSmem<D>) ? sizeof(KVSmem<D>)
                                                                     : sizeof(QSmem<D>);

template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_job(const BwdParams& p, int bh, int kblk, KVSmem<D>& sm) {
  constexpr int kDK = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kChunks = D / 8;
  constexpr int kGroups = (kTile / 4) * kChunks;  // (4-row group, chunk) pairs per tile
  static_assert(kGroups <= kThreads, "one staging group per thread at most");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int N = p.N;
  const size_t head = (size_t)bh * N;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto qr = make_rsrc(p.q + head * D, head_bytes);
  const auto gr = make_rsrc(p.dout + head * D, head_bytes);

  const int k0 = kblk * kBlock;
  const int kw0 = k0 + wave * 32;  // this wave's first key
  const int mykey = kw0 + col;

  // K^T and V^T columns of this lane's key, as B operands
  bf16x8 kreg[kDK], vreg[kDK];
  {
    const auto kr = make_rsrc(p.k + head * D, head_bytes);
    const auto vr = make_rsrc(p.v + head * D, head_bytes);
#pragma unroll
    for (int kk = 0; kk < kDK; ++kk) {
      const uint32_t e = (uint32_t)(mykey * D + kk * 16 + half * 8);
      kreg[kk] = as_bf16x8(load8<uint16_t>(kr, e));
      vreg[kk] = as_bf16x8(load8<uint16_t>(vr, e));
    }
  }
  f32x16 dvacc[kDB], dkacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) {
    dvacc[i] = zero16();
    dkacc[i] = zero16();
  }

  const int ntiles = (N + kTile - 1) / kTile;
  const int t0 = CAUSAL ? k0 / kTile : 0;  // earlier query rows see none of these keys
  const float c = p.c;
  const int sg = tid / kChunks, sch = tid % kChunks;  // staging group of this thread

  // registers holding the next tile while the current one is computed
  uint4 wq[4], wg[4];
  float l2 = 0.0f, dr = 0.0f;
  auto fetch = [&](int t) {
    const int qs = t * kTile;
    if (tid < kGroups) {  // wave-uniform
      load_rows4<D>(qr, qs, 4 * sg, sch, wq);
      load_rows4<D>(gr, qs, 4 * sg, sch, wg);
    }
    if (tid < kTile) {
      const int row = qs + tid;
      l2 = row < N ? p.lse[head + row] * kLog2e : INFINITY;
      dr = row < N ? p.drow[head + row] : 0.0f;
    }
  };
  if (t0 < ntiles) fetch(t0);

  for (int t = t0; t < ntiles; ++t) {
    const int qs = t * kTile;
    __syncthreads();  // the previous tile is no longer read
    if (tid < kGroups) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st_row<D>(sm.q, 4 * sg + r, sch, wq[r]);
        st_row<D>(sm.g, 4 * sg + r, sch, wg[r]);
      }
      st_tr4<kTile>(sm.qt, 4 * sg, sch, wq);
      st_tr4<kTile>(sm.gt, 4 * sg, sch, wg);
    }
    if (tid < kTile) {
      sm.lse2[tid] = l2;
      sm.dr[tid] = dr;
    }
    __syncthreads();
    if (t + 1 < ntiles) fetch(t + 1);

    if (CAUSAL && qs + kTile - 1 < kw0) continue;  // every row of the tile precedes our keys
    const bool need_mask = CAUSAL && qs < kw0 + 31;

    uint32_t pk[2][8], dsk[2][8];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      f32x16 s = zero16(), dp = zero16();
      const int row = qb * 32 + col;
#pragma unroll
      for (int kk = 0; kk < kDK; ++kk) {
        s = mfma32(ld_row<D>(sm.q, row, 2 * kk + half), kreg[kk], s);
        dp = mfma32(ld_row<D>(sm.g, row, 2 * kk + half), vreg[kk], dp);
      }
      float pv[16], dsv[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int r0 = qb * 32 + 8 * g4 + 4 * half;  // tile rows of elements 4g4..4g4+3
        const f32x4 l2v = *reinterpret_cast<const f32x4*>(&sm.lse2[r0]);
        const f32x4 drv = *reinterpret_cast<const f32x4*>(&sm.dr[r0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g4 + i;
          float pr = fast_exp2(__builtin_fmaf(s[r], c, -l2v[i]));
          if (need_mask) pr = (qs + r0 + i < mykey) ? 0.0f : pr;
          pv[r] = pr;
          dsv[r] = pr * (dp[r] - drv[i]);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        pk[qb][j] = pack_bf16x2(pv[2 * j], pv[2 * j + 1]);
        dsk[qb][j] = pack_bf16x2(dsv[2 * j], dsv[2 * j + 1]);
      }
    }

#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint4 pu = {pk[qb][4 * m], pk[qb][4 * m + 1], pk[qb][4 * m + 2], pk[qb][4 * m + 3]};
        const uint4 du = {dsk[qb][4 * m], dsk[qb][4 * m + 1], dsk[qb][4 * m + 2],
                          dsk[qb][4 * m + 3]};
        const bf16x8 pb = as_bf16x8(pu), db8 = as_bf16x8(du);
        const int chunk = 4 * qb + 2 * m + half;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          dvacc[db] = mfma32(ld_tr<kTile>(sm.gt, db * 32 + col, chunk), pb, dvacc[db]);
          dkacc[db] = mfma32(ld_tr<kTile>(sm.qt, db * 32 + col, chunk), db8, dkacc[db]);
        }
      }
  }

  if (mykey < N) {
    uint16_t* dkg = p.dk + (head + mykey) * D;
    uint16_t* dvg = p.dv + (head + mykey) * D;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * half;
        const uint2 wk = {pack_bf16x2(dkacc[db][4 * g4] * sc, dkacc[db][4 * g4 + 1] * sc),
                          pack_bf16x2(dkacc[db][4 * g4 + 2] * sc, dkacc[db][4 * g4 + 3] * sc)};
        const uint2 wv = {pack_bf16x2(dvacc[db][4 * g4], dvacc[db][4 * g4 + 1]),
                          pack_bf16x2(dvacc[db][4 * g4 + 2], dvacc[db][4 * g4 + 3])};
        *reinterpret_cast<uint2*>(dkg + d0) = wk;
        *reinterpret_cast<uint2*>(dvg + d0) = wv;
      }
  }
}

// ---------------------------------------------------------------- dQ

template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_job(const BwdParams& p, int bh, int qblk, QSmem<D>& sm) {
  constexpr int kDK = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kChunks = D / 8;
  constexpr int kGroups = (kTile / 4) * kChunks;
  static_assert(kGroups <= kThreads, "one staging group per thread at most");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int N = p.N;
  const size_t head = (size_t)bh * N;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto kr = make_rsrc(p.k + head * D, head_bytes);
  const auto vr = make_rsrc(p.v + head * D, head_bytes);

  const int q0 = qblk * kBlock;
  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + col;
  const int wave_last = min(qw0 + 32, N) - 1;

  bf16x8 qreg[kDK], greg[kDK];  // Q^T and dO^T columns of this lane's row
  float l2 = INFINITY, dr = 0.0f;
  {
    const auto qr = make_rsrc(p.q + head * D, head_bytes);
    const auto gr = make_rsrc(p.dout + head * D, head_bytes);
#pragma unroll
    for (int kk = 0; kk < kDK; ++kk) {
      const uint32_t e = (uint32_t)(myq * D + kk * 16 + half * 8);
      qreg[kk] = as_bf16x8(load8<uint16_t>(qr, e));
      greg[kk] = as_bf16x8(load8<uint16_t>(gr, e));
    }
    if (myq < N) {
      l2 = p.lse[head + myq] * kLog2e;
      dr = p.drow[head + myq];
    }
  }
  f32x16 dqacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) dqacc[i] = zero16();

  const int ntiles_all = (N + kTile - 1) / kTile;
  const int ntiles = CAUSAL ? min(ntiles_all, (min(q0 + kBlock, N) - 1) / kTile + 1) : ntiles_all;
  const float c = p.c;
  const int sg = tid / kChunks, sch = tid % kChunks;

  uint4 wk[4], wv[4];
  auto fetch = [&](int t) {
    if (tid < kGroups) {  // wave-uniform
      load_rows4<D>(kr, t * kTile, 4 * sg, sch, wk);
      load_rows4<D>(vr, t * kTile, 4 * sg, sch, wv);
    }
  };
  fetch(0);

  for (int t = 0; t < ntiles; ++t) {
    const int key0 = t * kTile;
    __syncthreads();
    if (tid < kGroups) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        st_row<D>(sm.k, 4 * sg + r, sch, wk[r]);
        st_row<D>(sm.v, 4 * sg + r, sch, wv[r]);
      }
      st_tr4<kTile>(sm.kt, 4 * sg, sch, wk);
    }
    __syncthreads();
    if (t + 1 < ntiles) fetch(t + 1);

    if (CAUSAL && key0 > wave_last) continue;
    const bool need_mask = (key0 + kTile > N) || (CAUSAL && key0 + kTile - 1 > qw0);

    uint32_t dsk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = zero16(), dp = zero16();
      const int row = kb * 32 + col;
#pragma unroll
      for (int kk = 0; kk < kDK; ++kk) {
        s = mfma32(ld_row<D>(sm.k, row, 2 * kk + half), qreg[kk], s);
        dp = mfma32(ld_row<D>(sm.v, row, 2 * kk + half), greg[kk], dp);
      }
      float dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = fast_exp2(__builtin_fmaf(s[r], c, -l2));
        if (need_mask) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          pr = (key < N && (!CAUSAL || key <= myq)) ? pr : 0.0f;
        }
        dsv[r] = pr * (dp[r] - dr);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) dsk[kb][j] = pack_bf16x2(dsv[2 * j], dsv[2 * j + 1]);
    }

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint4 du = {dsk[kb][4 * m], dsk[kb][4 * m + 1], dsk[kb][4 * m + 2],
                          dsk[kb][4 * m + 3]};
        const bf16x8 b = as_bf16x8(du);
        const int chunk = 4 * kb + 2 * m + half;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
          dqacc[db] = mfma32(ld_tr<kTile>(sm.kt, db * 32 + col, chunk), b, dqacc[db]);
      }
  }

  if (myq < N) {
    uint16_t* dqg = p.dq + (head + myq) * D;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + 8 * g4 + 4 * half;
        const uint2 w = {pack_bf16x2(dqacc[db][4 * g4] * sc, dqacc[db][4 * g4 + 1] * sc),
                         pack_bf16x2(dqacc[db][4 * g4 + 2] * sc, dqacc[db][4 * g4 + 3] * sc)};
        *reinterpret_cast<uint2*>(dqg + d0) = w;
      }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void bwd_grads_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kGradsSmem<D>];
  const Job job = job_of<CAUSAL>(p);
  if (job.is_dq)
    dq_job<D, CAUSAL>(p, job.bh, job.blk, *reinterpret_cast<QSmem<D>*>(smem));
  else
    dkdv_job<D, CAUSAL>(p, job.bh, job.blk, *reinterpret_cast<KVSmem<D>*>(smem));
}

template <int D>
BwdParams make_params(const BwdArgs& a) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.drow = a.drow;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.BH = a.B * a.H;
  p.N = a.N;
  p.nblk = (a.N + kBlock - 1) / kBlock;
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  p.xcd_remap = (p.BH % 8) == 0;
  return p;
}

template <int D>
hipError_t launch_prep_typed(const BwdArgs& a) {
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int kRowsPerBlock = kThreads / (D / 8);
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((bwd_rows_kernel<D>), grid, dim3(kThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.dout),
                     a.drow, rows);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_grads_typed(const BwdArgs& a) {
  const BwdParams p = make_params<D>(a);
  const dim3 grid((unsigned)(2LL * p.BH * p.nblk));
  hipLaunchKernelGGL((bwd_grads_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_prep(const BwdArgs& a) {
  return a.d == 64 ? launch_prep_typed<64>(a) : launch_prep_typed<128>(a);
}

hipError_t launch_backward_grads(const BwdArgs& a) {
  if (a.d == 64)
    return a.causal ? launch_grads_typed<64, true>(a) : launch_grads_typed<64, false>(a);
  return a.causal ? launch_grads_typed<128, true>(a) : launch_grads_typed<128, false>(a);
}

long long backward_grid_size(int B, int H, int N) {
  const long long rows = (long long)B * H * N;
  const long long row_blocks = (rows + 15) / 16;
  const long long blocks = 2LL * B * H * ((N + kBlock - 1) / kBlock);
  return row_blocks > blocks ? row_blocks : blocks;
}

}  // namespace fa
