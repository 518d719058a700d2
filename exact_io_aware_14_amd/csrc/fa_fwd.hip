// Forward exact attention for gfx950: one workgroup per (batch, head, block
// of 128 query rows), four waves of 32 query rows each.
//
// Method: the tiled forward with a running row maximum m and row sum l, in
// which the partial output of earlier key tiles is rescaled whenever m grows
// ("Flash Attention: Rivoluzionando l'Efficienza dei Modelli Transformer"
// (unite.ai), sections "L'Algoritmo di Flash Attention" and "La Matematica
// dietro Flash Attention", formulas 1-2; "Attenzione flash"
// (aiunderstanding.org), "Approfondimento tecnico"). The work decomposition
// is the FlashAttention-2 one described on the nearauto.com article
// (section "より優れた並列処理": one worker per row block of the attention
// matrix; section "より良い作業分割": the query rows are split across the
// waves and every wave sees the whole K/V tile, so waves never exchange
// partial results). The normalisation by l happens once at the end, and the
// output is rescaled only when a row maximum has grown by more than 2^8
// (section "非matmul FLOPの減少": fewer non-matmul operations).
//
// Per wave and key tile (BC keys) the kernel computes the transposed score
// tile S^T = K Q^T on MFMA, so that each lane owns one query row (column c of
// the accumulator) and holds 16 of the tile's scores per 32 keys; the two
// halves of the wave hold the other keys of the same rows. The probabilities
// are packed to bf16 in the lane and feed the product O^T += V^T P^T
// directly as its B operand; V is kept transposed in LDS to serve as the A
// operand.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBR = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kBC = 64;                     // keys per tile
constexpr int kThreads = kWaves * 64;
// A row maximum may exceed the reference used for the exponentials by up to
// this many powers of two before the accumulators are rescaled; the
// probabilities then stay below 2^8, far inside fp32 and bf16 range.
constexpr float kRescaleSlack = 8.0f;

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;        // batch * heads
  int N;         // sequence length
  int nqb;       // query blocks per head
  float c;       // |scale| * log2(e), at least 1e-30
  int negate_q;  // scale < 0: Q is negated on load and |scale| is used
  int xcd_remap; // heads grouped per XCD (requires BH % 8 == 0)
};

template <int D>
struct Smem {
  uint16_t k[kBC * D];   // K tile, row-major
  uint16_t vt[D * kBC];  // V tile, transposed
};

template <int D, typename TIn>
struct TileLoader {
  static constexpr int kChunks = D / 8;                       // 16-byte chunks per row
  static constexpr int kKLoads = kBC * kChunks / kThreads;    // K chunks per thread
  static constexpr int kVGroups = (kBC / 4) * kChunks;        // (4-key group, chunk) pairs
  static constexpr int kVLoads = (kVGroups + kThreads - 1) / kThreads;
  static_assert(kBC * kChunks % kThreads == 0, "K tile must split evenly");

  uint4 kreg[kKLoads];
  uint4 vreg[kVLoads][4];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                       int key0, int tid) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      const int id = tid + i * kThreads;
      kreg[i] = load8<TIn>(kr, (uint32_t)((key0 + id / kChunks) * D + (id % kChunks) * 8));
    }
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      const int id = tid + i * kThreads;
      if (id < kVGroups) {  // wave-uniform
        const int ch = id % kChunks, g = id / kChunks;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vreg[i][r] = load8<TIn>(vr, (uint32_t)((key0 + 4 * g + r) * D + ch * 8));
      }
    }
  }

  __device__ __forceinline__ void store(Smem<D>& sm, int tid) {
#pragma unroll
    for (int i = 0; i < kKLoads; ++i) {
      int id = tid + i * kThreads;
      st_row<D>(sm.k, id / kChunks, id % kChunks, kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      int id = tid + i * kThreads;
      if (id < kVGroups) st_tr4<kBC>(sm.vt, 4 * (id / kChunks), id % kChunks, vreg[i]);
    }
  }
};

template <int D, bool CAUSAL, typename TIn, typename TOut>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdParams p) {
  __shared__ Smem<D> sm;
  constexpr int kDK = D / 16;  // MFMA steps along d for S^T
  constexpr int kDB = D / 32;  // 32-row blocks of O^T
  constexpr int kKB = kBC / 32;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- which (head, query block) this workgroup owns
  int bh, qbr;
  const int L = blockIdx.x;
  if (p.xcd_remap) {
    // consecutive workgroups go to the 8 XCDs in turn; give each XCD whole
    // heads so the K/V of a head is re-read from that XCD's L2
    int xcd = L & 7, idx = L >> 3;
    bh = (idx / p.nqb) * 8 + xcd;
    qbr = idx % p.nqb;
  } else {
    bh = L % p.BH;
    qbr = L / p.BH;
  }
  // causal: the longest rows (most key tiles) are dispatched first
  const int qb = CAUSAL ? (p.nqb - 1 - qbr) : qbr;
  const int N = p.N;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  // buffer views of this head; reads past row N return zeros
  const uint32_t head_bytes = (uint32_t)N * D * sizeof(TIn);
  const auto qr = make_rsrc(reinterpret_cast<const TIn*>(p.q) + head_off, head_bytes);
  const auto kr = make_rsrc(reinterpret_cast<const TIn*>(p.k) + head_off, head_bytes);
  const auto vr = make_rsrc(reinterpret_cast<const TIn*>(p.v) + head_off, head_bytes);

  const int q0 = qb * kBR;                        // first row of the block
  const int qw0 = q0 + wave * kRowsPerWave;       // first row of this wave
  const int myq = qw0 + col;                      // this lane's row
  const int wave_last = min(qw0 + kRowsPerWave, N) - 1;

  // ---- Q^T as the B operand of S^T = K Q^T: column = row myq, k-slots = d
  bf16x8 qreg[kDK];
#pragma unroll
  for (int kk = 0; kk < kDK; ++kk) {
    uint4 u = load8<TIn>(qr, (uint32_t)(myq * D + kk * 16 + half * 8));
    if (p.negate_q) u = negate8(u);
    qreg[kk] = as_bf16x8(u);
  }

  f32x16 oacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;  // reference maximum, in units of log2 (scale*log2e*score)
  float l_run = 0.0f;       // this lane's part of the row sum

  const int ktiles_all = (N + kBC - 1) / kBC;
  const int ktiles = CAUSAL ? min(ktiles_all, (min(q0 + kBR, N) - 1) / kBC + 1) : ktiles_all;
  const float c = p.c;

  TileLoader<D, TIn> ld;
  ld.load(kr, vr, 0, tid);

  for (int t = 0; t < ktiles; ++t) {
    __syncthreads();  // every wave is done reading the previous tile
    ld.store(sm, tid);
    __syncthreads();
    if (t + 1 < ktiles) ld.load(kr, vr, (t + 1) * kBC, tid);

    const int key0 = t * kBC;
    if (CAUSAL && key0 > wave_last) continue;  // no visible key for this wave

    // ---- S^T = K Q^T for the BC keys of the tile
    f32x16 s[kKB];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      s[kb] = zero16();
      const int row = kb * 32 + col;
#pragma unroll
      for (int kk = 0; kk < kDK; ++kk)
        s[kb] = mfma32(ld_row<D>(sm.k, row, 2 * kk + half), qreg[kk], s[kb]);
    }

    // ---- masks: keys past N, and keys after the row for causal
    const bool need_mask = (key0 + kBC > N) || (CAUSAL && key0 + kBC - 1 > qw0);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          bool vis = key < N && (!CAUSAL || key <= myq);
          s[kb][r] = vis ? s[kb][r] : -INFINITY;
        }
    }

    // ---- row maximum over the tile (own 16*KB keys, then the other half)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, swap_halves(mx));
    // c > 0, so a fully masked row gives cand = -inf and never grows m_run
    const float cand = mx * c;

    // ---- move the reference maximum only when it is exceeded by the slack.
    // Every row sees key 0 in the first tile, so m_run is finite from then on
    // (on the first tile alpha = 2^-inf = 0 clears the empty accumulators).
    const bool grow = cand > m_run + kRescaleSlack;
    if (__any(grow)) {
      const float m_new = fmaxf(m_run, cand);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < kDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      m_run = m_new;
    }

    // ---- probabilities p = 2^(c*s - m) (masked scores: 2^-inf = 0), summed
    // in fp32 (lse keeps fp32 accuracy) and packed to bf16 for P.V
    uint32_t pk[kKB][8];
    float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float e0 = fast_exp2(__builtin_fmaf(s[kb][2 * r], c, -m_run));
        const float e1 = fast_exp2(__builtin_fmaf(s[kb][2 * r + 1], c, -m_run));
        ls0 += e0;
        ls1 += e1;
        pk[kb][r] = pack_bf16x2(e0, e1);
      }
    }
    l_run += ls0 + ls1;

    // ---- O^T += V^T P^T; P^T slots (kb, m) are accumulator rows 8m..8m+7
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        uint4 bu = {pk[kb][4 * m], pk[kb][4 * m + 1], pk[kb][4 * m + 2], pk[kb][4 * m + 3]};
        const bf16x8 b = as_bf16x8(bu);
        const int chunk = 4 * kb + 2 * m + half;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
          oacc[db] = mfma32(ld_tr<kBC>(sm.vt, db * 32 + col, chunk), b, oacc[db]);
      }
  }

  // ---- epilogue: O = O_acc / l, lse = (m + log2 l) * ln 2
  const float l_tot = l_run + swap_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (myq < N) {
    TOut* og = reinterpret_cast<TOut*>(p.o) + head_off + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * half;
        float x0 = oacc[db][4 * g] * inv, x1 = oacc[db][4 * g + 1] * inv;
        float x2 = oacc[db][4 * g + 2] * inv, x3 = oacc[db][4 * g + 3] * inv;
        if constexpr (sizeof(TOut) == 2) {
          uint2 w = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
          *reinterpret_cast<uint2*>(og + d0) = w;
        } else {
          *reinterpret_cast<float4*>(og + d0) = make_float4(x0, x1, x2, x3);
        }
      }
    if (half == 0) {
      p.lse[(size_t)bh * N + myq] =
          l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, typename TIn, typename TOut>
hipError_t launch_typed(const FwdArgs& a) {
  FwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.BH = a.B * a.H;
  p.N = a.N;
  p.nqb = (a.N + kBR - 1) / kBR;
  // c is kept positive: a zero or denormal scale is raised to 1e-30, which
  // changes no score by more than 1e-27 and keeps c * (-inf) = -inf
  p.c = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  p.negate_q = a.scale < 0.0f;
  p.xcd_remap = (p.BH % 8) == 0;
  dim3 grid((unsigned)((long long)p.BH * p.nqb));
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, TIn, TOut>), grid, dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_dtype(const FwdArgs& a) {
  if (a.d == 64) {
    return a.causal ? launch_typed<64, true, TIn, TOut>(a) : launch_typed<64, false, TIn, TOut>(a);
  }
  return a.causal ? launch_typed<128, true, TIn, TOut>(a) : launch_typed<128, false, TIn, TOut>(a);
}

}  // namespace

hipError_t launch_forward_bf16(const FwdArgs& a) { return launch_dtype<uint16_t, uint16_t>(a); }
hipError_t launch_forward_f32(const FwdArgs& a) { return launch_dtype<float, float>(a); }

long long forward_grid_size(int B, int H, int N) {
  return (long long)B * H * ((N + kBR - 1) / kBR);
}

}  // namespace fa
