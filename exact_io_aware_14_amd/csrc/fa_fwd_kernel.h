// Forward exact attention for gfx950, the kernel (fa_fwd.hip launches it at
// d = 64 and 128, fa_fwd_w.hip at d = 256): one workgroup per (batch, head,
// block of 128 query rows), four waves of 32 query rows each, two
// workgroups per CU at d = 128.
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
// directly as its B operand; the A operand V^T comes from the row-major V
// tile through the transposing LDS read.
//
// K and V tiles move from global memory into LDS with buffer loads that
// write LDS directly (no registers, no VALU), double-buffered: tile t+1
// loads while tile t is computed, with one workgroup barrier per tile. The
// two stages of K and of V are four separate LDS arrays and the tile loop
// is unrolled by two, so every LDS read names the array it reads: the
// compiler then sees that the loads in flight (into the other stage) cannot
// alias it, and does not make the transposing reads wait for them. fp32
// inputs take the same path through registers, rounded to bf16.
#pragma once

#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_schedule.h"

namespace fa {
namespace {

constexpr int kRowsPerWave = 32;
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
  int BH;        // batch * query heads
  int H;         // query heads
  int group;     // query heads per K/V head (1: multi-head attention)
  int N;         // sequence length
  int nqb;       // query blocks per head
  float c;       // |scale| * log2(e), at least 1e-30
  int negate_q;  // scale < 0: Q is negated on load and |scale| is used
  int xcd_remap; // K/V heads grouped per XCD (requires BH / group % 8 == 0)
  int wl, wr;    // masked kernels: key j visible to query i iff i-wl <= j <= i+wr
  // block-sparse kernels: the mask of query head bh at bmask + bh * bm_stride,
  // nbm x nbm bytes (query block, key block), a zero byte skipping the block
  const uint8_t* bmask;
  long long bm_stride;
  int nbm;
};

// Workgroup shape: four waves (128 query rows), two workgroups per CU at
// d = 128 (four at d = 64 with bf16 inputs, at most 128 VGPRs); the waves a SIMD holds belong
// to different workgroups and overlap freely. At d = 256 a wave's Q (64
// registers) and O accumulators (128) leave room for the scores of 32 keys
// only: bf16 inputs take 32-key tiles (two LDS stages of K and V, 64 KB) at
// two workgroups per CU, 256 registers per wave; fp32 inputs take 64-key
// tiles at one workgroup per CU (128 KB of stages, the SIMD's whole register
// file of 512).
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBR = kWaves * kRowsPerWave;  // query rows per workgroup

template <int D, int BC>
struct Layout {
  static constexpr int kTileBytes = BC * D * 2;               // one stage of K or V (rsw)
  static constexpr int kFill = kTileBytes / 1024 / kWaves;  // 1 KB blocks per wave and tile
  static_assert(kFill >= 1 && kTileBytes % (1024 * kWaves) == 0, "tile must split over waves");
};

// SPARSE: a block-sparse mask on top of the window (CAUSAL kernels only).
// PAIR: two query blocks per workgroup under the causal mask (see below).
template <int D, int BC, bool CAUSAL, typename TIn, typename TOut, bool SPARSE = false,
          bool PAIR = false>
__global__ __launch_bounds__(kThreads, D == 256 ? (BC == 32 ? 2 : 1) : (D == 64 && sizeof(TIn) == 2 ? 4 : 2))
void fwd_kernel(FwdParams p) {
  static_assert(!SPARSE || (CAUSAL && kBR == kMaskBlock && kMaskBlock % BC == 0),
                "a workgroup is one query block of the mask, whole tiles one key block");
  using LY = Layout<D, BC>;
  // stages 0 and 1 of the K and V tiles (row-major, swizzle rsw)
  __shared__ __attribute__((aligned(1024))) unsigned char k0[LY::kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[LY::kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[LY::kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[LY::kTileBytes];
  constexpr int kDK = D / 16;   // MFMA steps along d for S^T
  constexpr int kDB = D / 32;   // 32-row blocks of O^T
  constexpr int kKB = BC / 32;  // 32-key blocks of a tile
  // d = 256: operands are read in chunks (4 steps of S^T; 4 blocks of O^T,
  // 2 with 32-key tiles, whose two waves per SIMD have 256 registers each)
  // so that the staging registers stay within bounds; per-lane offsets are
  // kept for the first 128 columns only (kOffDK steps, kOffDB blocks): the
  // swizzle repeats every 256 bytes of a row (rsw)
  constexpr int kChK = D == 256 ? 4 : kDK;
  constexpr int kChB = D == 256 ? (BC == 32 ? 2 : 4) : kDB;
  constexpr int kOffDK = kDK < 8 ? kDK : 8;
  constexpr int kOffDB = kDB < 4 ? kDB : 4;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- which (head, query block) this workgroup owns (fa_schedule.h):
  // masked launches dispatch the longest rows first; PAIR launches (causal
  // mask) take query blocks nqb-1-i and i of one head in turn, so every
  // workgroup walks about nqb+1 key tiles (the middle block of an odd nqb
  // alone), and the second block's first key tile loads while the first
  // block's last one is computed.
  static_assert(!PAIR || (CAUSAL && !SPARSE), "pairs are for the causal mask");
  constexpr bool pair = PAIR;
  const sched::FwdBlock blk =
      sched::fwd_block(blockIdx.x, p.BH, p.group, p.nqb, p.xcd_remap != 0, CAUSAL, PAIR);
  const int bh = blk.bh;
  const int npass = blk.npass;
  const int N = p.N;
  bool prefetched = false;  // this pass's first key tile is already loading into stage 0
  for (int pass = 0; pass < npass; ++pass) {
  const int qb = pass == 1 ? blk.qb_second : blk.qb_first;
  const size_t head_off = (size_t)bh * (size_t)N * D;
  const size_t kv_off = (size_t)(bh / p.group) * (size_t)N * D;
  const TIn* qg = reinterpret_cast<const TIn*>(p.q) + head_off;
  const TIn* kg = reinterpret_cast<const TIn*>(p.k) + kv_off;
  const TIn* vg = reinterpret_cast<const TIn*>(p.v) + kv_off;

  // rows of the block and of this wave, and the key tiles they walk
  const sched::FwdRange rng =
      sched::fwd_range<kBR, kRowsPerWave, BC>(qb, wave, N, p.wl, p.wr, CAUSAL);
  const int qw0 = rng.qw0;              // first row of this wave
  const int myq = qw0 + col;            // this lane's row
  // keys this lane's row sees: lo_key .. lo_key + n_vis - 1 (masked kernels:
  // i - wl .. i + wr within 0 .. N-1; otherwise 0 .. N-1)
  const int lo_key = CAUSAL ? myq - p.wl : 0;
  const int hi_key = CAUSAL ? min(N - 1, myq + p.wr) : N - 1;
  const uint32_t n_vis = hi_key >= lo_key ? (uint32_t)(hi_key - lo_key + 1) : 0u;

  // ---- Q^T as the B operand of S^T = K Q^T: column = row myq, k-slots = d
  bf16x8 qreg[kDK];
  {
    const auto qr = make_rsrc(qg, (uint32_t)N * D * sizeof(TIn));  // rows past N read 0
#pragma unroll
    for (int kk = 0; kk < kDK; ++kk) {
      uint4 u = load8<TIn>(qr, (uint32_t)(myq * D + kk * 16 + half * 8));
      if (p.negate_q) u = negate8(u);
      qreg[kk] = as_bf16x8(u);
    }
  }

  // ---- per-lane LDS offsets, fixed for the whole loop
  uint32_t koff[kOffDK];  // K operand of S^T: row col (+32 kb), chunk 2kk + half
#pragma unroll
  for (int kk = 0; kk < kOffDK; ++kk) koff[kk] = row_offset<D>(col, 2 * kk + half);
  uint32_t voff[kOffDB][2];  // V^T operand: d-block db, read 0/1 (+ rows kb*32 + m*16)
#pragma unroll
  for (int db = 0; db < kOffDB; ++db)
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) voff[db][rd] = rows_t_offset<D>(db, rd, lane);
  // offsets of step kk / block db (compile-time constants past the first 128 columns)
  auto koff_at = [&](int kk) { return koff[kk % kOffDK] + (uint32_t)(kk / kOffDK) * 256u; };
  auto voff_at = [&](int db, int rd) {
    return voff[db % kOffDB][rd] + (uint32_t)(db / kOffDB) * 256u;
  };
  uint32_t fk[LY::kFill];  // direct-fill offsets of this lane (K and V alike)
#pragma unroll
  for (int i = 0; i < LY::kFill; ++i) fk[i] = fill_lane_offset<D, BC, kWaves>(i, wave, lane);

  f32x16 oacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;  // reference maximum, in units of log2 (scale*log2e*score)
  float l_run = 0.0f;       // this lane's part of the row sum
  f32x16 s[kKB];            // S^T of the tile between its MFMA and VALU phases
  uint32_t pk[kKB][8];      // P^T packed to bf16, between its VALU and MFMA phases

  // Masked kernels (CAUSAL: a causal or local window, bounds wl, wr; an
  // unbounded side is 2^30): the workgroup walks key tiles t_first ..
  // t_end-1, those holding a key that one of its rows sees, and each wave
  // computes on the tiles [wt_first, wt_end) that hold one of its keys.
  const int t_first = rng.t_first;
  const int t_end = rng.t_end;
  const int wt_first = rng.wt_first;
  const int wt_end = rng.wt_end;
  const float c = p.c;

  // start loading key tile t of g (K or V) into the stage array dst
  auto fill_tile = [&](const TIn* g, int t, unsigned char* dst, const uint32_t* lane_off) {
    const int key0 = t * BC;
    const auto r = make_rsrc(g + (size_t)key0 * D, (uint32_t)(N - key0) * D * sizeof(TIn));
    if constexpr (sizeof(TIn) == 2) {
      fill_direct<D, BC, kWaves>(dst, r, lane_off, wave);
    } else {
      fill_f32<D, BC, kThreads>(reinterpret_cast<uint16_t*>(dst), r, 0, tid);
    }
  };

  // MFMA phase, first half: O^T += V^T P^T for tile t (slots (kb, m) of P^T
  // are accumulator rows 8m..8m+7). All operand reads are issued before the
  // first product, so the LDS latency is paid once per half phase.
  auto pv = [&](const unsigned char* vs) {
#pragma unroll
    for (int c0 = 0; c0 < kDB; c0 += kChB) {
      bf16x8 a[kKB][2][kChB];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int db = 0; db < kChB; ++db)
            a[kb][m][db] = lds_tr_pair(vs + (kb * 32 + m * 16) * D * 2 + voff_at(c0 + db, 0),
                                       vs + (kb * 32 + m * 16) * D * 2 + voff_at(c0 + db, 1));
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          uint4 bu = {pk[kb][4 * m], pk[kb][4 * m + 1], pk[kb][4 * m + 2], pk[kb][4 * m + 3]};
          const bf16x8 b = as_bf16x8(bu);
#pragma unroll
          for (int db = 0; db < kChB; ++db)
            oacc[c0 + db] = mfma32(a[kb][m][db], b, oacc[c0 + db]);
        }
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * kKB * kChB, 0);  // the LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * kKB * kChB, 0);  // then the MFMAs
    }
  };

  // MFMA phase, second half: S^T = K Q^T for the K tile ks. At d = 64 and
  // 128 the K reads run four ahead of the MFMAs that use them (1-2% faster
  // at d = 128 than issuing every read first; the same at d = 64); at
  // d = 256 each chunk's reads come first.
  auto qk = [&](const unsigned char* ks) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) s[kb] = zero16();
#pragma unroll
    for (int c0 = 0; c0 < kDK; c0 += kChK) {
      bf16x8 a[kChK][kKB];
#pragma unroll
      for (int kk = 0; kk < kChK; ++kk)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
          a[kk][kb] = lds_ld16(ks + kb * 32 * D * 2 + koff_at(c0 + kk));
#pragma unroll
      for (int kk = 0; kk < kChK; ++kk)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) s[kb] = mfma32(a[kk][kb], qreg[c0 + kk], s[kb]);
      constexpr int kN = kChK * kKB;  // reads and MFMAs of the chunk
      constexpr int kAhead = 4;
      if constexpr (D != 256 && kN > kAhead) {
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);  // the first reads
#pragma unroll
        for (int i = 0; i < kN - kAhead; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // an MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the next read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);  // the last MFMAs
      } else {
        __builtin_amdgcn_sched_group_barrier(0x100, kN, 0);  // the LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, kN, 0);  // then the MFMAs
      }
    }
  };

  // VALU phase: masks, online softmax and P for tile t
  auto softmax = [&](int t) {
    const int key0 = t * BC;
    // a tile needs masks where it passes N, the first row's upper bound or
    // the last row's lower bound
    const bool need_mask = sched::fwd_need_mask<BC>(t, rng, N, p.wl, p.wr, CAUSAL);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          s[kb][r] = in_window(key, lo_key, n_vis) ? s[kb][r] : -INFINITY;
        }
    }

    // row maximum over the tile (own 16*KB keys, then the other half)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = halves_max(mx);
    // c > 0, so a fully masked row gives cand = -inf and never grows m_run
    const float cand = mx * c;

    // move the reference maximum only when it is exceeded by the slack. A
    // row's m_run stays -inf until a tile shows it a key (the first tile
    // always does without a lower window bound); alpha = 2^-inf = 0 then
    // clears its still empty accumulators.
    const bool grow = cand > m_run + kRescaleSlack;
    if (__any(grow)) {
      const float m_new = fmaxf(m_run, cand);
      // a row whose maximum does not move keeps its scale (this also covers
      // a row that has seen no key yet: -inf - -inf would give NaN)
      const float alpha = m_new > m_run ? fast_exp2(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < kDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      m_run = m_new;
    }

    // probabilities p = 2^(c*s - m) (masked scores: 2^-inf = 0), summed in
    // fp32 (lse keeps fp32 accuracy) and packed to bf16 for P.V. A row that
    // has seen no key yet has only masked scores here: subtract 0, not -inf.
    const float m_sub = m_run == -INFINITY ? 0.0f : m_run;
    float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float e0 = fast_exp2(__builtin_fmaf(s[kb][2 * r], c, -m_sub));
        const float e1 = fast_exp2(__builtin_fmaf(s[kb][2 * r + 1], c, -m_sub));
        ls0 += e0;
        ls1 += e1;
        pk[kb][r] = pack_bf16x2(e0, e1);
      }
    }
    l_run += ls0 + ls1;
  };

  // ---- tiles. K and V of tile t+1 load while tile t is computed: one
  // barrier per tile, after which tile t is in LDS for every wave and every
  // wave is done with tile t-1, whose stage the loads of tile t+1 overwrite.
  // Tiles t_first, t_first+2, ... use stage 0 (k0, v0), the others stage 1.
  auto step = [&](int t, const unsigned char* kc, const unsigned char* vc, unsigned char* kn,
                  unsigned char* vn) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < t_end) {
      fill_tile(kg, t + 1, kn, fk);
      fill_tile(vg, t + 1, vn, fk);
    } else if (pair && pass + 1 < npass && ((t_end - t_first) & 1) == 0) {
      // an even tile count ends in stage 1: the next pass's first tile (key
      // tile 0, causal) goes into stage 0, which every wave is done with
      fill_tile(kg, 0, kn, fk);
      fill_tile(vg, 0, vn, fk);
      prefetched = true;
    }
    if (t >= wt_first && t < wt_end) {
      qk(kc);
      softmax(t);
      pv(vc);
    }
  };
  if constexpr (!SPARSE) {
    if (!prefetched) {
      if (pass > 0) __syncthreads();  // every wave is done with the last pass's stages
      fill_tile(kg, t_first, k0, fk);
      fill_tile(vg, t_first, v0, fk);
    }
    prefetched = false;
    for (int t = t_first; t < t_end; t += 2) {
      step(t, k0, v0, k1, v1);
      if (t + 1 < t_end) step(t + 1, k1, v1, k0, v0);
    }
  } else {
    // Block-sparse kernels: tile t lies in key block t / kTilesPerBlock of
    // the mask row of this query block; the workgroup walks only the tiles
    // of nonzero blocks, in order, with the same double buffering (tn: the
    // tile after t, loaded while t is computed).
    constexpr int kTilesPerBlock = kMaskBlock / BC;
    MaskScan scan;
    scan.stride = 1;
    scan.n = p.nbm;
    scan.reset(p.bmask + (size_t)bh * (size_t)p.bm_stride + (size_t)qb * p.nbm, nullptr);
    auto next_tile = [&](int t) {  // the first tile >= t of a nonzero block, else t_end
      uint32_t fl;
      const int blk = scan.next(t / kTilesPerBlock, lane, &fl);
      return blk == t / kTilesPerBlock ? t : min(kTilesPerBlock * blk, t_end);
    };
    auto step_to = [&](int t, int tn, const unsigned char* kc, const unsigned char* vc,
                       unsigned char* kn, unsigned char* vn) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tn < t_end) {
        fill_tile(kg, tn, kn, fk);
        fill_tile(vg, tn, vn, fk);
      }
      if (t >= wt_first && t < wt_end) {
        qk(kc);
        softmax(t);
        pv(vc);
      }
    };
    int t = next_tile(t_first);
    if (t < t_end) {
      fill_tile(kg, t, k0, fk);
      fill_tile(vg, t, v0, fk);
    }
    while (t < t_end) {
      int tn = next_tile(t + 1);
      step_to(t, tn, k0, v0, k1, v1);
      t = tn;
      if (t >= t_end) break;
      tn = next_tile(t + 1);
      step_to(t, tn, k1, v1, k0, v0);
      t = tn;
    }
  }

  // ---- epilogue: O = O_acc / l, lse = (m + log2 l) * ln 2
  const float l_tot = halves_sum(l_run);
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
  }  // pass
}

constexpr int kBC = 64;  // keys per tile
// d = 256 with bf16 inputs and no block mask: 32 keys per tile, two
// workgroups per CU (16-18% faster than 64-key tiles at one per CU)
template <int D, typename TIn>
constexpr int tile_keys() { return D == 256 && sizeof(TIn) == 2 ? 32 : kBC; }
// Causal forward launches at d = 128 pair query blocks up to this many blocks
// per head (N <= 8192): measured 2% faster at N = 4096, 2% slower at N = 32768,
// where the paired workgroups stream the head's K/V out of step and share
// less of the L2.
constexpr int kPairMaxBlocks = 64;

template <int D, bool CAUSAL, typename TIn, typename TOut, bool SPARSE = false>
hipError_t launch_typed(const FwdArgs& a) {
  FwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.BH = a.B * a.H;
  p.H = a.H;
  p.group = a.H / a.Hkv;
  p.N = a.N;
  p.nqb = (a.N + kBR - 1) / kBR;
  // c is kept positive: a zero or denormal scale is raised to 1e-30, which
  // changes no score by more than 1e-27 and keeps c * (-inf) = -inf
  p.c = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  p.wl = a.wl < 0 ? kUnbounded : a.wl;
  p.wr = a.wr < 0 ? kUnbounded : a.wr;
  p.negate_q = a.scale < 0.0f;
  p.xcd_remap = (p.BH / p.group) % 8 == 0;
  p.bmask = a.bmask;
  p.bm_stride = a.bmask_stride;
  p.nbm = (a.N + kMaskBlock - 1) / kMaskBlock;
  if constexpr (D == 128 && CAUSAL && !SPARSE) {
    if (p.wl == kUnbounded && p.wr == 0 && p.nqb <= kPairMaxBlocks) {
      dim3 grid((unsigned)((long long)p.BH * ((p.nqb + 1) / 2)));
      hipLaunchKernelGGL((fwd_kernel<D, kBC, true, TIn, TOut, false, true>), grid,
                         dim3(kThreads), 0, a.stream, p);
      return hipGetLastError();
    }
  }
  dim3 grid((unsigned)((long long)p.BH * p.nqb));
  hipLaunchKernelGGL((fwd_kernel<D, tile_keys<D, TIn>(), CAUSAL, TIn, TOut, SPARSE>), grid,
                     dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

// the d = 256 launches (fa_fwd_w.hip)
hipError_t launch_forward_wide_bf16(const FwdArgs& a);
hipError_t launch_forward_wide_f32(const FwdArgs& a);
hipError_t launch_forward_wide_sparse(const FwdArgs& a);  // block-sparse, bf16

}  // namespace fa
