// Backward exact attention for gfx950, in two launches on one stream:
//
//   prep:  D_i = sum_k dO_ik O_ik and lse2_i = lse_i * log2(e) for every row
//          (HBM-bound), into the workspace
//   grads: one launch holding two kinds of workgroup, interleaved so the
//          most expensive ones of both kinds start first:
//          dK/dV jobs, one per (batch, head, block of 128 keys), walk the
//          query tiles and accumulate dV_j = sum_i P_ij dO_i and
//          dK_j = scale * sum_i dS_ij Q_i for their own keys;
//          dQ jobs, one per (batch, head, block of 256 query rows), walk the
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
// Workgroups are 8 waves, two per SIMD, each under 256 registers.
// MFMA formulations (32x32x16 bf16; layouts in fa_common.h):
//   dK/dV job, lane = key: the workgroup's 128 keys of K and V stay in LDS;
//     wave w owns keys 32*(w%4).. and rows 32*(w/4).. of every 64-row query
//     tile. S = Q K^T and dP = dO V^T read both operands as LDS rows;
//     dV^T += dO^T P and dK^T += Q^T dS take P, dS repacked in-lane as B
//     operands and dO^T, Q^T from the row-major tiles through the
//     transposing read. Waves w and w+4 add their partial dK, dV once, at
//     the end, through LDS.
//   dQ job, lane = query: 8 x 32 rows; S^T = K Q^T and dP^T = V dO^T with
//     Q^T, dO^T in registers; dQ^T += K^T dS^T with K^T read through the
//     transposing read.
//
// Tiles of 64 rows move global -> LDS with direct buffer loads (no
// registers), double-buffered: tile t+1 loads while tile t is computed, one
// barrier per tile. Rows past the end of a sequence load as zeros, so they
// add nothing to any gradient (their Q, dO, K and V are zero); only the
// causal mask needs explicit handling, on diagonal tiles.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kKeyBlock = 128;  // keys per dK/dV job
constexpr int kQBlock = 256;    // query rows per dQ job
constexpr int kTile = 64;       // rows of a streamed tile

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
  int nkb;          // dK/dV jobs (128-key blocks) per K/V head
  int nqb;          // dQ jobs (256-row blocks) per query head
  float c;          // scale * log2(e)
  float scale;
  int wl, wr;       // masked kernels: key j visible to query i iff i-wl <= j <= i+wr
  int xcd_remap;
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- prep

constexpr int kPrepThreads = 256;

template <int D>
__global__ __launch_bounds__(kPrepThreads) void bwd_prep_kernel(const uint16_t* o,
                                                            const uint16_t* dout,
                                                            const float* lse, float* drow,
                                                            float* lse2, long long rows) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = kPrepThreads / kLanesPerRow;
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
  if (ch == 0 && row < rows) {
    drow[row] = acc;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------- layout

// Job of this workgroup in the grads launch. Every K/V head owns nkb dK/dV
// jobs and group * nqb dQ jobs (those of its query heads). The two kinds
// are interleaved evenly, each sequence ordered from the most expensive
// block down (causal: dK/dV of the first key blocks, dQ of the last query
// blocks). Consecutive workgroups go to the 8 XCDs in turn;
// when the head count allows, each XCD gets whole K/V heads (with their
// query heads) so that their K/V and Q/dO stay in its L2.
struct Job {
  int bh;    // dK/dV: the K/V head (batch * K/V heads); dQ: the query head
  int blk;
  bool is_dq;
};

template <bool CAUSAL>
__device__ __forceinline__ Job job_of(const BwdParams& p) {
  const int L = blockIdx.x;
  const int ndq = p.group * p.nqb;
  const int per_head = p.nkb + ndq;
  const int bhkv = p.BH / p.group;
  int kvh, j;
  if (p.xcd_remap) {
    const int xcd = L & 7, idx = L >> 3;
    kvh = (idx / per_head) * 8 + xcd;
    j = idx % per_head;
  } else {
    kvh = L % bhkv;
    j = L / bhkv;
  }
  // The head's dQ jobs are spread evenly over its slots (slot j is a dQ job
  // iff floor((j+1) ndq / per_head) > floor(j ndq / per_head)). Within an
  // XCD, consecutive workgroups go to its four shader engines in turn, so
  // each engine must see the same mix of the two kinds: where one engine
  // gets only dK/dV jobs, workgroups wait for it while the other engines
  // have free CUs. The even spread alone alternates the kinds when there
  // are as many of each (at d = 256), which again splits them by engine;
  // rotating the slots of each full group of four by the group index gives
  // every engine both kinds in any case.
  if ((j | 3) < per_head) j = (j & ~3) | (((j & 3) + (j >> 2)) & 3);
  Job job;
  const int before = (int)(((long long)j * ndq) / per_head);
  const int after = (int)(((long long)(j + 1) * ndq) / per_head);
  job.is_dq = after > before;
  const int rank = job.is_dq ? before : j - before;
  if (job.is_dq) {
    // rank r: query block r / group (from the last one under the causal
    // mask) of query head r % group of this K/V head
    const int qbr = rank / p.group;
    job.bh = kvh * p.group + rank % p.group;
    job.blk = CAUSAL ? (p.nqb - 1 - qbr) : qbr;
  } else {
    job.bh = kvh;
    job.blk = rank;
  }
  return job;
}

// LDS of the grads launch (bytes).
template <int D>
struct GLayout {
  static constexpr int kTileBytes = kTile * D * 2;
  static constexpr int kBlockBytes = kKeyBlock * D * 2;
  // dK/dV job: the key block's K and V, then Q and dO tiles, lse2 and D of
  // the tile, the tiles in two stages
  static constexpr int kKb = 0;
  static constexpr int kVb = kBlockBytes;
  static constexpr int kQt = 2 * kBlockBytes;
  static constexpr int kGt = kQt + 2 * kTileBytes;
  static constexpr int kLv = kGt + 2 * kTileBytes;
  static constexpr int kRv = kLv + 2 * kTile * 4;
  static constexpr int kDkdvBytes = kRv + 2 * kTile * 4;
  // dQ job: K and V tiles in two stages
  static constexpr int kKt = 0;
  static constexpr int kVt = 2 * kTileBytes;
  static constexpr int kDqBytes = 4 * kTileBytes;
  static constexpr int kBytes = kDkdvBytes > kDqBytes ? kDkdvBytes : kDqBytes;
  // 1 KB blocks per wave to fill a tile / a key block
  static constexpr int kFillTile = kTileBytes / 1024 / kWaves;
  static constexpr int kFillBlock = kBlockBytes / 1024 / kWaves;
  // partial dK, dV of the four waves w+4 (fp32), laid out [wave][dk|dv][db][r][lane]
  static constexpr int kPartialBytes = 4 * 2 * (D / 32) * 16 * 64 * 4;
  static_assert(kPartialBytes <= kDkdvBytes, "the partials reuse the job's LDS");
};

// Per-lane LDS offsets shared by both jobs.
template <int D>
struct Offsets {
  uint32_t row[D / 16];       // MFMA operand rows: row col (+32 per block), chunk 2kk + half
  uint32_t tr[D / 32][2];     // transposing reads: d-block db, read 0/1 (+ 16-row bases)
  uint32_t ftile[GLayout<D>::kFillTile];
  __device__ __forceinline__ void init(int wave, int lane) {
    const int half = lane >> 5, col = lane & 31;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) row[kk] = row_offset<D>(col, 2 * kk + half);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) tr[db][rd] = rows_t_offset<D>(db, rd, lane);
#pragma unroll
    for (int i = 0; i < GLayout<D>::kFillTile; ++i)
      ftile[i] = fill_lane_offset<D, kTile, kWaves>(i, wave, lane);
  }
};

// Start loading rows row0 .. row0+63 of a head-sized bf16 tensor into `dst`.
template <int D>
__device__ __forceinline__ void fill_tile(unsigned char* dst, const uint16_t* g, int row0, int N,
                                          const Offsets<D>& off, int wave) {
  const auto r = make_rsrc(g + (size_t)row0 * D, (uint32_t)(N - row0) * D * 2u);
  fill_direct<D, kTile, kWaves>(dst, r, off.ftile, wave);
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

// ---------------------------------------------------------------- dK / dV

template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_job(const BwdParams& p, int bh, int kblk,
                                         unsigned char* smem) {
  using LY = GLayout<D>;
  constexpr int kDK = D / 16;
  constexpr int kDB = D / 32;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave & 3;   // key sub-block of this wave
  const int qh = wave >> 2;  // which 32 rows of each query tile
  const int half = lane >> 5, col = lane & 31;
  const int N = p.N;
  const size_t head = (size_t)bh * N;  // bh: the K/V head
  // its query heads are bh*group .. bh*group+group-1
  const size_t qhead0 = (size_t)bh * p.group * N;

  const int k0 = kblk * kKeyBlock;
  const int kw0 = k0 + 32 * kw;  // this wave's first key
  const int mykey = kw0 + col;

  Offsets<D> off;
  off.init(wave, lane);

  // the workgroup's keys of K and V (zeros past N), for the whole job
  {
    const uint32_t bytes = (uint32_t)(N - k0) * D * 2u;
    const auto kr = make_rsrc(p.k + (head + k0) * D, bytes);
    const auto vr = make_rsrc(p.v + (head + k0) * D, bytes);
    uint32_t fb[LY::kFillBlock];
#pragma unroll
    for (int i = 0; i < LY::kFillBlock; ++i)
      fb[i] = fill_lane_offset<D, kKeyBlock, kWaves>(i, wave, lane);
    fill_direct<D, kKeyBlock, kWaves>(smem + LY::kKb, kr, fb, wave);
    fill_direct<D, kKeyBlock, kWaves>(smem + LY::kVb, vr, fb, wave);
  }
  f32x16 dvacc[kDB], dkacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) {
    dvacc[i] = zero16();
    dkacc[i] = zero16();
  }

  // Masked kernels (CAUSAL: a causal or local window): query row i sees key
  // j iff j - wr <= i <= j + wl, so the block's keys k0 .. kend are seen by
  // the rows of query tiles t0 .. ntiles-1 only.
  const int kend = min(k0 + kKeyBlock, N) - 1;
  const int t0 = CAUSAL ? max(0, k0 - p.wr) / kTile : 0;
  const int ntiles = CAUSAL ? min(N - 1, kend + p.wl) / kTile + 1 : (N + kTile - 1) / kTile;
  const int lo_row = mykey - p.wr, hi_row = mykey + p.wl;  // rows that see this lane's key
  const float c = p.c;
  const unsigned char* kb = smem + LY::kKb + kw * 32 * D * 2;  // this wave's key rows

  // load tile t of query head jq of the group into LDS stage st
  auto fill = [&](int jq, int t, int st) {
    const size_t qh = qhead0 + (size_t)jq * N;
    const int r0 = t * kTile;
    fill_tile<D>(smem + LY::kQt + st * LY::kTileBytes, p.q + qh * D, r0, N, off, wave);
    fill_tile<D>(smem + LY::kGt + st * LY::kTileBytes, p.dout + qh * D, r0, N, off, wave);
    if (wave == 0) fill_vec(smem + LY::kLv + st * kTile * 4, p.lse2 + qh, r0, N, lane);
    if (wave == 1) fill_vec(smem + LY::kRv + st * kTile * 4, p.drow + qh, r0, N, lane);
  };

  // one query tile t, in LDS stage ST; MASK: the tile crosses the causal
  // diagonal of this wave's keys
  auto tile = [&](int t, int ST, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int r0 = t * kTile + 32 * qh;  // this wave's first query row
    // the dO tile lies a fixed distance after the Q tile: one address per
    // pair of reads, the distance an immediate offset
    constexpr int kG = LY::kGt - LY::kQt;
    constexpr int kV = LY::kVb - LY::kKb;
    const unsigned char* qt = smem + LY::kQt + ST * LY::kTileBytes + qh * 32 * D * 2;
    const float* l2t = reinterpret_cast<const float*>(smem + LY::kLv + ST * kTile * 4) + 32 * qh;
    const float* drt = reinterpret_cast<const float*>(smem + LY::kRv + ST * kTile * 4) + 32 * qh;

    // ---- S = Q K^T and dP = dO V^T: rows = the wave's 32 queries, column = key
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int k2 = 0; k2 < kDK; k2 += 2) {
      bf16x8 qa[2], ga[2], ka[2], va[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const unsigned char* qp = qt + off.row[k2 + u];
        const unsigned char* kp = kb + off.row[k2 + u];
        qa[u] = lds_ld16(qp);
        ga[u] = lds_ld16(qp + kG);
        ka[u] = lds_ld16(kp);
        va[u] = lds_ld16(kp + kV);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s = mfma32(qa[u], ka[u], s);
        dp = mfma32(ga[u], va[u], dp);
      }
    }

    // ---- P = 2^(c*S - lse2) and dS = P * (dP - D), packed to bf16
    uint32_t pk[8], dsk[8];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int rr = 8 * g4 + 4 * half;  // rows of elements 4g4..4g4+3 (within the 32)
      const f32x4 l2v = *reinterpret_cast<const f32x4*>(&l2t[rr]);
      const f32x4 drv = *reinterpret_cast<const f32x4*>(&drt[rr]);
      float pv[4], dsv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        float pr = fast_exp2(__builtin_fmaf(s[r], c, -l2v[i]));
        if constexpr (MASK) {
          const int row = r0 + rr + i;
          pr = (row < lo_row || row > hi_row) ? 0.0f : pr;
        }
        pv[i] = pr;
        dsv[i] = pr * (dp[r] - drv[i]);
      }
      pk[2 * g4] = pack_bf16x2(pv[0], pv[1]);
      pk[2 * g4 + 1] = pack_bf16x2(pv[2], pv[3]);
      dsk[2 * g4] = pack_bf16x2(dsv[0], dsv[1]);
      dsk[2 * g4 + 1] = pack_bf16x2(dsv[2], dsv[3]);
    }

    // ---- dV^T += dO^T P and dK^T += Q^T dS; slots m are accumulator rows
    // 8m..8m+7 of S, i.e. the wave's rows 16m + ...
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int rb = m * 16 * D * 2;
      bf16x8 gta[kDB], qta[kDB];
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const unsigned char* p0 = qt + off.tr[db][0] + rb;
        const unsigned char* p1 = qt + off.tr[db][1] + rb;
        gta[db] = lds_tr_pair(p0 + kG, p1 + kG);
        qta[db] = lds_tr_pair(p0, p1);
      }
      const uint4 pu = {pk[4 * m], pk[4 * m + 1], pk[4 * m + 2], pk[4 * m + 3]};
      const uint4 du = {dsk[4 * m], dsk[4 * m + 1], dsk[4 * m + 2], dsk[4 * m + 3]};
      const bf16x8 pb = as_bf16x8(pu), db8 = as_bf16x8(du);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        dvacc[db] = mfma32(gta[db], pb, dvacc[db]);
        dkacc[db] = mfma32(qta[db], db8, dkacc[db]);
      }
    }
  };

  // The group's query heads one after another, each over tiles t0 ..
  // ntiles-1; `step` counts the tiles walked and picks the LDS stage. At
  // each step, the tile (and, the first time, the key block) is in LDS for
  // every wave, and every wave is done with the previous step, whose stage
  // the loads of the next step overwrite.
  int step = 0;
  auto sync_fill = [&](int jq, int t) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles)
      fill(jq, t + 1, (step + 1) & 1);
    else if (jq + 1 < p.group)
      fill(jq + 1, t0, (step + 1) & 1);
  };
  // Masked kernels: this wave's rows r0 .. r0+31 of tile t and its keys
  // kw0 .. kw0+31 all see each other for tiles tm1 .. tm2-1 (r0 >= kw0+31-wr
  // and r0+31 <= kw0+wl); the tiles before and after cross a window edge
  // (masked), or show the wave none of its keys (skipped). Each wave walks
  // them in three loops (every iteration passes one barrier), so no loop
  // holds both versions of the tile body. Causal: no tiles after tm2.
  int tm1 = t0, tm2 = ntiles;
  if (CAUSAL) {
    tm1 = min(ntiles, max(t0, ceil_div(kw0 + 31 - p.wr - 32 * qh, kTile)));
    tm2 = min(ntiles, max(tm1, floor_div(kw0 + p.wl - 32 * qh - 31, kTile) + 1));
  }
  auto visible = [&](int t) {
    const int r0 = t * kTile + 32 * qh;
    return r0 + 31 >= kw0 - p.wr && r0 <= kw0 + 31 + p.wl;
  };
  if (t0 < ntiles) fill(0, t0, 0);
  for (int jq = 0; jq < p.group; ++jq) {
    for (int t = t0; t < tm1; ++t, ++step) {
      sync_fill(jq, t);
      if (visible(t)) tile(t, step & 1, std::true_type());
    }
    for (int t = tm1; t < tm2; ++t, ++step) {
      sync_fill(jq, t);
      tile(t, step & 1, std::false_type());
    }
    for (int t = tm2; t < ntiles; ++t, ++step) {
      sync_fill(jq, t);
      if (visible(t)) tile(t, step & 1, std::true_type());
    }
  }

  // ---- waves w+4 hand their partial sums to waves w through LDS
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every wave is done with the tiles
  float* part = reinterpret_cast<float*>(smem) + kw * 2 * kDB * 16 * 64;
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        part[((0 * kDB + db) * 16 + r) * 64 + lane] = dkacc[db][r];
        part[((1 * kDB + db) * 16 + r) * 64 + lane] = dvacc[db][r];
      }
  }
  __syncthreads();
  if (qh == 0 && mykey < N) {
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dkacc[db][r] += part[((0 * kDB + db) * 16 + r) * 64 + lane];
        dvacc[db][r] += part[((1 * kDB + db) * 16 + r) * 64 + lane];
      }
    store_rows<D>(p.dk + (head + mykey) * D, dkacc, p.scale, half);
    store_rows<D>(p.dv + (head + mykey) * D, dvacc, 1.0f, half);
  }
}

// ---------------------------------------------------------------- dQ

template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_job(const BwdParams& p, int bh, int qblk,
                                       unsigned char* smem) {
  using LY = GLayout<D>;
  constexpr int kDK = D / 16;
  constexpr int kDB = D / 32;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int N = p.N;
  const size_t head = (size_t)bh * N;  // bh: the query head
  const size_t kvhead = (size_t)(bh / p.group) * N;
  const uint16_t* kg = p.k + kvhead * D;
  const uint16_t* vg = p.v + kvhead * D;

  const int q0 = qblk * kQBlock;
  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + col;
  const int wave_last = min(qw0 + 32, N) - 1;

  Offsets<D> off;
  off.init(wave, lane);

  bf16x8 qreg[kDK], greg[kDK];  // Q^T and dO^T columns of this lane's row (zeros past N)
  float l2 = 0.0f, dr = 0.0f;
  {
    const uint32_t bytes = (uint32_t)N * D * 2u;
    const auto qr = make_rsrc(p.q + head * D, bytes);
    const auto gr = make_rsrc(p.dout + head * D, bytes);
#pragma unroll
    for (int kk = 0; kk < kDK; ++kk) {
      const uint32_t e = (uint32_t)(myq * D + kk * 16 + half * 8);
      qreg[kk] = as_bf16x8(load8<uint16_t>(qr, e));
      greg[kk] = as_bf16x8(load8<uint16_t>(gr, e));
    }
    if (myq < N) {
      l2 = p.lse2[head + myq];
      dr = p.drow[head + myq];
    }
  }
  f32x16 dqacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) dqacc[i] = zero16();

  // Masked kernels (CAUSAL: a causal or local window): row i sees keys
  // i-wl .. i+wr. The workgroup walks key tiles kt0 .. ntiles-1, those that
  // one of its rows sees; this wave computes on tiles wt0 .. wt1-1.
  const int ntiles_all = (N + kTile - 1) / kTile;
  const int qend = min(q0 + kQBlock, N) - 1;
  const int kt0 = CAUSAL ? max(0, q0 - p.wl) / kTile : 0;
  const int ntiles = CAUSAL ? min(N - 1, qend + p.wr) / kTile + 1 : ntiles_all;
  const int wt0 = CAUSAL ? max(0, qw0 - p.wl) / kTile : 0;
  const int wt1 = qw0 >= N ? wt0 : (CAUSAL ? min(N - 1, wave_last + p.wr) / kTile + 1 : ntiles_all);
  const int lo_key = myq - p.wl, hi_key = myq + p.wr;  // keys this lane's row sees
  const float c = p.c;

  auto fill = [&](int t) {
    const int st = t & 1, r0 = t * kTile;
    fill_tile<D>(smem + LY::kKt + st * LY::kTileBytes, kg, r0, N, off, wave);
    fill_tile<D>(smem + LY::kVt + st * LY::kTileBytes, vg, r0, N, off, wave);
  };

  // one key tile; MASK: it crosses a window edge of this wave's rows
  auto tile = [&](int t, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int ST = t & 1;
    const int key0 = t * kTile;
    const unsigned char* kt = smem + LY::kKt + ST * LY::kTileBytes;
    const unsigned char* vt = smem + LY::kVt + ST * LY::kTileBytes;

    uint32_t dsk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int k4 = 0; k4 < kDK; k4 += 4) {
        bf16x8 ka[4], va[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ka[u] = lds_ld16(kt + kb * 32 * D * 2 + off.row[k4 + u]);
          va[u] = lds_ld16(vt + kb * 32 * D * 2 + off.row[k4 + u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s = mfma32(ka[u], qreg[k4 + u], s);
          dp = mfma32(va[u], greg[k4 + u], dp);
        }
      }
      float dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = fast_exp2(__builtin_fmaf(s[r], c, -l2));
        if constexpr (MASK) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          pr = (key < lo_key || key > hi_key) ? 0.0f : pr;
        }
        dsv[r] = pr * (dp[r] - dr);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) dsk[kb][j] = pack_bf16x2(dsv[2 * j], dsv[2 * j + 1]);
    }

    // ---- dQ^T += K^T dS^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int rb = (kb * 32 + m * 16) * D * 2;
        bf16x8 ka[kDB];
#pragma unroll
        for (int db = 0; db < kDB; ++db)
          ka[db] = lds_tr_pair(kt + rb + off.tr[db][0], kt + rb + off.tr[db][1]);
        const uint4 du = {dsk[kb][4 * m], dsk[kb][4 * m + 1], dsk[kb][4 * m + 2],
                          dsk[kb][4 * m + 3]};
        const bf16x8 b = as_bf16x8(du);
#pragma unroll
        for (int db = 0; db < kDB; ++db) dqacc[db] = mfma32(ka[db], b, dqacc[db]);
      }
  };

  auto sync_fill = [&](int t) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles) fill(t + 1);
  };
  // Key tile t shows all of its keys to all of this wave's rows for tiles
  // tm1 .. tm2-1 (t*64 >= wave_last-wl and t*64+63 <= qw0+wr); the visible
  // tiles before and after cross a window edge (masked). Three loops (every
  // iteration passes one barrier), so no loop holds both tile bodies.
  // Causal: no masked tiles before tm1 = kt0 = 0.
  int tm1 = kt0, tm2 = wt1;
  if (CAUSAL) {
    tm1 = min(ntiles, max(kt0, ceil_div(wave_last - p.wl, kTile)));
    tm2 = min(wt1, max(tm1, floor_div(qw0 + p.wr - (kTile - 1), kTile) + 1));
  }
  if (qw0 >= N) tm2 = tm1;  // no rows: every tile is skipped
  auto visible = [&](int t) { return t >= wt0 && t < wt1; };
  fill(kt0);
  for (int t = kt0; t < tm1; ++t) {
    sync_fill(t);
    if (visible(t)) tile(t, std::true_type());
  }
  for (int t = tm1; t < tm2; ++t) {
    sync_fill(t);
    tile(t, std::false_type());
  }
  for (int t = tm2; t < ntiles; ++t) {
    sync_fill(t);
    if (visible(t)) tile(t, std::true_type());
  }

  if (myq < N) store_rows<D>(p.dq + (head + myq) * D, dqacc, p.scale, half);
}

// ---------------------------------------------------------------- d = 256
//
// At d = 256 a wave's accumulators alone (dK and dV of 32 keys, or dQ) take
// 128-256 registers and a 128-key block of K and V 128 KB, so the grads
// launch uses four-wave workgroups, one wave per SIMD with the whole
// register file (512, accumulators in AGPRs):
//   dK/dV job, 128 keys: wave w owns keys 32w .. 32w+31 over all query
//     rows, with its keys' K in registers (the B operand of S = Q K^T) and
//     the block's V in LDS (64 KB); query tiles of 32 rows (Q and dO, 16 KB
//     each) are double-buffered. Every wave writes its own keys: no
//     exchange between waves.
//   dQ job, 128 rows: as at d = 128 with four waves of 32 rows; K and V
//     tiles of 64 keys (32 KB each) double-buffered.
// Per-lane offsets are kept for the first 128 columns: the row swizzle
// repeats every 256 bytes (rsw), so the rest are constant offsets.

constexpr int kWavesW = 4;
constexpr int kThreadsW = kWavesW * 64;
constexpr int kKeyBlockW = 128;  // keys per dK/dV job
constexpr int kQBlockW = 128;    // query rows per dQ job
constexpr int kQTileW = 32;      // query rows per tile of a dK/dV job
constexpr int kKTileW = 64;      // keys per tile of a dQ job

template <int D>
struct WLayout {
  static constexpr int kQTileBytes = kQTileW * D * 2;
  static constexpr int kVBlockBytes = kKeyBlockW * D * 2;
  static constexpr int kKTileBytes = kKTileW * D * 2;
  // dK/dV job: V of the key block; Q and dO tiles, lse2 and D (64 floats
  // per stage: the vector fill moves 64), each in two stages
  static constexpr int kVb = 0;
  static constexpr int kQt = kVBlockBytes;
  static constexpr int kGt = kQt + 2 * kQTileBytes;
  static constexpr int kLv = kGt + 2 * kQTileBytes;
  static constexpr int kRv = kLv + 2 * 64 * 4;
  static constexpr int kDkdvBytes = kRv + 2 * 64 * 4;
  // dQ job: K and V tiles in two stages
  static constexpr int kKt = 0;
  static constexpr int kVt = 2 * kKTileBytes;
  static constexpr int kDqBytes = 4 * kKTileBytes;
  static constexpr int kBytes = kDkdvBytes > kDqBytes ? kDkdvBytes : kDqBytes;
  static constexpr int kFillQ = kQTileBytes / 1024 / kWavesW;   // 1 KB blocks per wave
  static constexpr int kFillV = kVBlockBytes / 1024 / kWavesW;
  static constexpr int kFillK = kKTileBytes / 1024 / kWavesW;
  static_assert(kBytes <= 160 * 1024, "LDS");
};

template <int D>
struct OffsetsW {
  static constexpr int kRows = D / 16 < 8 ? D / 16 : 8;
  static constexpr int kTr = D / 32 < 4 ? D / 32 : 4;
  uint32_t row[kRows];
  uint32_t tr[kTr][2];
  __device__ __forceinline__ void init(int lane) {
    const int half = lane >> 5, col = lane & 31;
#pragma unroll
    for (int kk = 0; kk < kRows; ++kk) row[kk] = row_offset<D>(col, 2 * kk + half);
#pragma unroll
    for (int db = 0; db < kTr; ++db)
#pragma unroll
      for (int rd = 0; rd < 2; ++rd) tr[db][rd] = rows_t_offset<D>(db, rd, lane);
  }
  __device__ __forceinline__ uint32_t row_at(int kk) const {
    return row[kk % kRows] + (uint32_t)(kk / kRows) * 256u;
  }
  __device__ __forceinline__ uint32_t tr_at(int db, int rd) const {
    return tr[db % kTr][rd] + (uint32_t)(db / kTr) * 256u;
  }
};

template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_job_w(const BwdParams& p, int bh, int kblk,
                                           unsigned char* smem) {
  using LY = WLayout<D>;
  constexpr int kDK = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kChB = 4;  // d-blocks per chunk of the dV/dK products

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int N = p.N;
  const size_t head = (size_t)bh * N;  // bh: the K/V head
  const size_t qhead0 = (size_t)bh * p.group * N;

  const int k0 = kblk * kKeyBlockW;
  const int kw0 = k0 + 32 * wave;  // this wave's first key
  const int mykey = kw0 + col;

  OffsetsW<D> off;
  off.init(lane);

  // the block's V into LDS; this lane's key of K into registers (zeros past N)
  {
    const auto vr = make_rsrc(p.v + (head + k0) * D, (uint32_t)(N - k0) * D * 2u);
    uint32_t fb[LY::kFillV];
#pragma unroll
    for (int i = 0; i < LY::kFillV; ++i) fb[i] = fill_lane_offset<D, kKeyBlockW, kWavesW>(i, wave, lane);
    fill_direct<D, kKeyBlockW, kWavesW>(smem + LY::kVb, vr, fb, wave);
  }
  bf16x8 kreg[kDK];
  {
    const auto kr = make_rsrc(p.k + head * D, (uint32_t)N * D * 2u);
#pragma unroll
    for (int kk = 0; kk < kDK; ++kk)
      kreg[kk] = as_bf16x8(load8<uint16_t>(kr, (uint32_t)(mykey * D + kk * 16 + half * 8)));
  }
  uint32_t fq[LY::kFillQ];
#pragma unroll
  for (int i = 0; i < LY::kFillQ; ++i) fq[i] = fill_lane_offset<D, kQTileW, kWavesW>(i, wave, lane);

  f32x16 dvacc[kDB], dkacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) {
    dvacc[i] = zero16();
    dkacc[i] = zero16();
  }

  // masked kernels: the block's keys are seen by rows k0 - wr .. kend + wl
  const int kend = min(k0 + kKeyBlockW, N) - 1;
  const int t0 = CAUSAL ? max(0, k0 - p.wr) / kQTileW : 0;
  const int ntiles = CAUSAL ? min(N - 1, kend + p.wl) / kQTileW + 1 : (N + kQTileW - 1) / kQTileW;
  const int lo_row = mykey - p.wr, hi_row = mykey + p.wl;  // rows that see this lane's key
  const float c = p.c;
  const unsigned char* vb = smem + LY::kVb + wave * 32 * D * 2;  // this wave's key rows of V

  auto fill = [&](int jq, int t, int st) {
    const size_t qh = qhead0 + (size_t)jq * N;
    const int r0 = t * kQTileW;
    const auto qr = make_rsrc(p.q + (qh + r0) * D, (uint32_t)(N - r0) * D * 2u);
    const auto gr = make_rsrc(p.dout + (qh + r0) * D, (uint32_t)(N - r0) * D * 2u);
    fill_direct<D, kQTileW, kWavesW>(smem + LY::kQt + st * LY::kQTileBytes, qr, fq, wave);
    fill_direct<D, kQTileW, kWavesW>(smem + LY::kGt + st * LY::kQTileBytes, gr, fq, wave);
    if (wave == 0) fill_vec(smem + LY::kLv + st * 64 * 4, p.lse2 + qh, r0, N, lane);
    if (wave == 1) fill_vec(smem + LY::kRv + st * 64 * 4, p.drow + qh, r0, N, lane);
  };

  auto tile = [&](int t, int ST, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int r0 = t * kQTileW;
    const unsigned char* qt = smem + LY::kQt + ST * LY::kQTileBytes;
    const unsigned char* gt = smem + LY::kGt + ST * LY::kQTileBytes;
    const float* l2t = reinterpret_cast<const float*>(smem + LY::kLv + ST * 64 * 4);
    const float* drt = reinterpret_cast<const float*>(smem + LY::kRv + ST * 64 * 4);

    // S = Q K^T and dP = dO V^T: rows = the tile's 32 queries, column = key
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int k2 = 0; k2 < kDK; k2 += 2) {
      bf16x8 qa[2], ga[2], va[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        qa[u] = lds_ld16(qt + off.row_at(k2 + u));
        ga[u] = lds_ld16(gt + off.row_at(k2 + u));
        va[u] = lds_ld16(vb + off.row_at(k2 + u));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s = mfma32(qa[u], kreg[k2 + u], s);
        dp = mfma32(ga[u], va[u], dp);
      }
    }

    uint32_t pk[8], dsk[8];
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int rr = 8 * g4 + 4 * half;
      const f32x4 l2v = *reinterpret_cast<const f32x4*>(&l2t[rr]);
      const f32x4 drv = *reinterpret_cast<const f32x4*>(&drt[rr]);
      float pv[4], dsv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * g4 + i;
        float pr = fast_exp2(__builtin_fmaf(s[r], c, -l2v[i]));
        if constexpr (MASK) {
          const int row = r0 + rr + i;
          pr = (row < lo_row || row > hi_row) ? 0.0f : pr;
        }
        pv[i] = pr;
        dsv[i] = pr * (dp[r] - drv[i]);
      }
      pk[2 * g4] = pack_bf16x2(pv[0], pv[1]);
      pk[2 * g4 + 1] = pack_bf16x2(pv[2], pv[3]);
      dsk[2 * g4] = pack_bf16x2(dsv[0], dsv[1]);
      dsk[2 * g4 + 1] = pack_bf16x2(dsv[2], dsv[3]);
    }

    // dV^T += dO^T P and dK^T += Q^T dS, in chunks of d-blocks
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int rb = m * 16 * D * 2;
      const uint4 pu = {pk[4 * m], pk[4 * m + 1], pk[4 * m + 2], pk[4 * m + 3]};
      const uint4 du = {dsk[4 * m], dsk[4 * m + 1], dsk[4 * m + 2], dsk[4 * m + 3]};
      const bf16x8 pb = as_bf16x8(pu), db8 = as_bf16x8(du);
#pragma unroll
      for (int c0 = 0; c0 < kDB; c0 += kChB) {
        bf16x8 gta[kChB], qta[kChB];
#pragma unroll
        for (int db = 0; db < kChB; ++db) {
          gta[db] = lds_tr_pair(gt + rb + off.tr_at(c0 + db, 0), gt + rb + off.tr_at(c0 + db, 1));
          qta[db] = lds_tr_pair(qt + rb + off.tr_at(c0 + db, 0), qt + rb + off.tr_at(c0 + db, 1));
        }
#pragma unroll
        for (int db = 0; db < kChB; ++db) {
          dvacc[c0 + db] = mfma32(gta[db], pb, dvacc[c0 + db]);
          dkacc[c0 + db] = mfma32(qta[db], db8, dkacc[c0 + db]);
        }
      }
    }
  };

  int step = 0;
  auto sync_fill = [&](int jq, int t) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles)
      fill(jq, t + 1, (step + 1) & 1);
    else if (jq + 1 < p.group)
      fill(jq + 1, t0, (step + 1) & 1);
  };
  // this wave's keys kw0 .. kw0+31 and the rows r0 .. r0+31 of tile t all
  // see each other for tiles tm1 .. tm2-1; the visible tiles before and
  // after are masked (three loops, every iteration passes one barrier)
  int tm1 = t0, tm2 = ntiles;
  if (CAUSAL) {
    tm1 = min(ntiles, max(t0, ceil_div(kw0 + 31 - p.wr, kQTileW)));
    tm2 = min(ntiles, max(tm1, floor_div(kw0 + p.wl - 31, kQTileW) + 1));
  }
  auto visible = [&](int t) {
    const int r0 = t * kQTileW;
    return r0 + 31 >= kw0 - p.wr && r0 <= kw0 + 31 + p.wl;
  };
  if (t0 < ntiles) fill(0, t0, 0);
  for (int jq = 0; jq < p.group; ++jq) {
    for (int t = t0; t < tm1; ++t, ++step) {
      sync_fill(jq, t);
      if (visible(t)) tile(t, step & 1, std::true_type());
    }
    for (int t = tm1; t < tm2; ++t, ++step) {
      sync_fill(jq, t);
      tile(t, step & 1, std::false_type());
    }
    for (int t = tm2; t < ntiles; ++t, ++step) {
      sync_fill(jq, t);
      if (visible(t)) tile(t, step & 1, std::true_type());
    }
  }
  if (mykey < N) {
    store_rows<D>(p.dk + (head + mykey) * D, dkacc, p.scale, half);
    store_rows<D>(p.dv + (head + mykey) * D, dvacc, 1.0f, half);
  }
}

template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_job_w(const BwdParams& p, int bh, int qblk,
                                         unsigned char* smem) {
  using LY = WLayout<D>;
  constexpr int kDK = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kChB = 4;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int N = p.N;
  const size_t head = (size_t)bh * N;  // bh: the query head
  const size_t kvhead = (size_t)(bh / p.group) * N;
  const uint16_t* kg = p.k + kvhead * D;
  const uint16_t* vg = p.v + kvhead * D;

  const int q0 = qblk * kQBlockW;
  const int qw0 = q0 + wave * 32;
  const int myq = qw0 + col;
  const int wave_last = min(qw0 + 32, N) - 1;

  OffsetsW<D> off;
  off.init(lane);
  uint32_t fk[LY::kFillK];
#pragma unroll
  for (int i = 0; i < LY::kFillK; ++i) fk[i] = fill_lane_offset<D, kKTileW, kWavesW>(i, wave, lane);

  bf16x8 qreg[kDK], greg[kDK];
  float l2 = 0.0f, dr = 0.0f;
  {
    const uint32_t bytes = (uint32_t)N * D * 2u;
    const auto qr = make_rsrc(p.q + head * D, bytes);
    const auto gr = make_rsrc(p.dout + head * D, bytes);
#pragma unroll
    for (int kk = 0; kk < kDK; ++kk) {
      const uint32_t e = (uint32_t)(myq * D + kk * 16 + half * 8);
      qreg[kk] = as_bf16x8(load8<uint16_t>(qr, e));
      greg[kk] = as_bf16x8(load8<uint16_t>(gr, e));
    }
    if (myq < N) {
      l2 = p.lse2[head + myq];
      dr = p.drow[head + myq];
    }
  }
  f32x16 dqacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) dqacc[i] = zero16();

  const int ntiles_all = (N + kKTileW - 1) / kKTileW;
  const int qend = min(q0 + kQBlockW, N) - 1;
  const int kt0 = CAUSAL ? max(0, q0 - p.wl) / kKTileW : 0;
  const int ntiles = CAUSAL ? min(N - 1, qend + p.wr) / kKTileW + 1 : ntiles_all;
  const int wt0 = CAUSAL ? max(0, qw0 - p.wl) / kKTileW : 0;
  const int wt1 = qw0 >= N ? wt0 : (CAUSAL ? min(N - 1, wave_last + p.wr) / kKTileW + 1 : ntiles_all);
  const int lo_key = myq - p.wl, hi_key = myq + p.wr;
  const float c = p.c;

  auto fill = [&](int t) {
    const int st = t & 1, r0 = t * kKTileW;
    const auto kr = make_rsrc(kg + (size_t)r0 * D, (uint32_t)(N - r0) * D * 2u);
    const auto vr = make_rsrc(vg + (size_t)r0 * D, (uint32_t)(N - r0) * D * 2u);
    fill_direct<D, kKTileW, kWavesW>(smem + LY::kKt + st * LY::kKTileBytes, kr, fk, wave);
    fill_direct<D, kKTileW, kWavesW>(smem + LY::kVt + st * LY::kKTileBytes, vr, fk, wave);
  };

  auto tile = [&](int t, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int ST = t & 1;
    const int key0 = t * kKTileW;
    const unsigned char* kt = smem + LY::kKt + ST * LY::kKTileBytes;
    const unsigned char* vt = smem + LY::kVt + ST * LY::kKTileBytes;

    uint32_t dsk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int k4 = 0; k4 < kDK; k4 += 4) {
        bf16x8 ka[4], va[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ka[u] = lds_ld16(kt + kb * 32 * D * 2 + off.row_at(k4 + u));
          va[u] = lds_ld16(vt + kb * 32 * D * 2 + off.row_at(k4 + u));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s = mfma32(ka[u], qreg[k4 + u], s);
          dp = mfma32(va[u], greg[k4 + u], dp);
        }
      }
      float dsv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = fast_exp2(__builtin_fmaf(s[r], c, -l2));
        if constexpr (MASK) {
          const int key = key0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          pr = (key < lo_key || key > hi_key) ? 0.0f : pr;
        }
        dsv[r] = pr * (dp[r] - dr);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) dsk[kb][j] = pack_bf16x2(dsv[2 * j], dsv[2 * j + 1]);
    }

    // dQ^T += K^T dS^T, in chunks of d-blocks
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int rb = (kb * 32 + m * 16) * D * 2;
        const uint4 du = {dsk[kb][4 * m], dsk[kb][4 * m + 1], dsk[kb][4 * m + 2],
                          dsk[kb][4 * m + 3]};
        const bf16x8 b = as_bf16x8(du);
#pragma unroll
        for (int c0 = 0; c0 < kDB; c0 += kChB) {
          bf16x8 ka[kChB];
#pragma unroll
          for (int db = 0; db < kChB; ++db)
            ka[db] = lds_tr_pair(kt + rb + off.tr_at(c0 + db, 0), kt + rb + off.tr_at(c0 + db, 1));
#pragma unroll
          for (int db = 0; db < kChB; ++db) dqacc[c0 + db] = mfma32(ka[db], b, dqacc[c0 + db]);
        }
      }
  };

  auto sync_fill = [&](int t) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < ntiles) fill(t + 1);
  };
  int tm1 = kt0, tm2 = wt1;
  if (CAUSAL) {
    tm1 = min(ntiles, max(kt0, ceil_div(wave_last - p.wl, kKTileW)));
    tm2 = min(wt1, max(tm1, floor_div(qw0 + p.wr - (kKTileW - 1), kKTileW) + 1));
  }
  if (qw0 >= N) tm2 = tm1;
  auto visible = [&](int t) { return t >= wt0 && t < wt1; };
  fill(kt0);
  for (int t = kt0; t < tm1; ++t) {
    sync_fill(t);
    if (visible(t)) tile(t, std::true_type());
  }
  for (int t = tm1; t < tm2; ++t) {
    sync_fill(t);
    tile(t, std::false_type());
  }
  for (int t = tm2; t < ntiles; ++t) {
    sync_fill(t);
    if (visible(t)) tile(t, std::true_type());
  }

  if (myq < N) store_rows<D>(p.dq + (head + myq) * D, dqacc, p.scale, half);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreadsW, 1) void bwd_grads_kernel_w(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[WLayout<D>::kBytes];
  const Job job = job_of<CAUSAL>(p);
  if (job.is_dq)
    dq_job_w<D, CAUSAL>(p, job.bh, job.blk, smem);
  else
    dkdv_job_w<D, CAUSAL>(p, job.bh, job.blk, smem);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_grads_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[GLayout<D>::kBytes];
  const Job job = job_of<CAUSAL>(p);
  if (job.is_dq)
    dq_job<D, CAUSAL>(p, job.bh, job.blk, smem);
  else
    dkdv_job<D, CAUSAL>(p, job.bh, job.blk, smem);
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
  return p;
}

template <int D>
hipError_t launch_prep_typed(const BwdArgs& a) {
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int kRowsPerBlock = kPrepThreads / (D / 8);
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((bwd_prep_kernel<D>), grid, dim3(kPrepThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.dout),
                     a.lse, a.drow, a.drow + rows, rows);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_grads_typed(const BwdArgs& a) {
  const BwdParams p = make_params<D>(a);
  const dim3 grid((unsigned)((long long)(p.BH / p.group) * (p.nkb + p.group * p.nqb)));
  if constexpr (D == 256)
    hipLaunchKernelGGL((bwd_grads_kernel_w<D, CAUSAL>), grid, dim3(kThreadsW), 0, a.stream, p);
  else
    hipLaunchKernelGGL((bwd_grads_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_prep(const BwdArgs& a) {
  if (a.d == 64) return launch_prep_typed<64>(a);
  return a.d == 256 ? launch_prep_typed<256>(a) : launch_prep_typed<128>(a);
}

hipError_t launch_backward_grads(const BwdArgs& a) {
  if (a.d == 64)
    return a.masked() ? launch_grads_typed<64, true>(a) : launch_grads_typed<64, false>(a);
  if (a.d == 256)
    return a.masked() ? launch_grads_typed<256, true>(a) : launch_grads_typed<256, false>(a);
  return a.masked() ? launch_grads_typed<128, true>(a) : launch_grads_typed<128, false>(a);
}

long long backward_grid_size(int B, int H, int Hkv, int N) {
  const long long rows = (long long)B * H * N;
  const long long row_blocks = (rows + 15) / 16;
  const long long blocks = (long long)B * Hkv * ((N + kKeyBlock - 1) / kKeyBlock) +
                           (long long)B * H * ((N + kQBlock - 1) / kQBlock);
  return row_blocks > blocks ? row_blocks : blocks;
}

}  // namespace fa
