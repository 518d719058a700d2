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

#include "fa_bwd_common.h"

namespace fa {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kTile = 64;       // rows of a streamed tile

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

// ---------------------------------------------------------------- dK / dV

template <int D, bool CAUSAL, bool SPARSE>
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

  // the job's keys, this wave's keys and the query tiles they walk
  const sched::DkdvRange rng =
      sched::dkdv_range<kKeyBlock, kTile>(kblk, kw, qh, N, p.wl, p.wr, CAUSAL);
  const int k0 = rng.k0;
  const int kw0 = rng.kw0;  // this wave's first key
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
  // d = 128: this wave's 32 keys of K stay in registers for the whole job as
  // the B operand of S = Q K^T (key = column c, k-slots along d; keys past N
  // read as zeros), which takes a quarter of the LDS reads out of the S/dP
  // phase (1-2% faster, bitwise the same results; d = 64 runs four waves
  // per SIMD and has no registers to spare)
  constexpr bool kKReg = D == 128;
  bf16x8 kreg[kKReg ? kDK : 1];
  if constexpr (kKReg) {
    const auto kr = make_rsrc(p.k + (head + k0) * D, (uint32_t)(N - k0) * D * 2u);
#pragma unroll
    for (int kk = 0; kk < kDK; ++kk)
      kreg[kk] = as_bf16x8(load8<uint16_t>(kr, (uint32_t)((32 * kw + col) * D + kk * 16 + half * 8)));
  }

  // Masked kernels (CAUSAL: a causal or local window): query row i sees key
  // j iff j - wr <= i <= j + wl, so the block's keys k0 .. kend are seen by
  // the rows of query tiles t0 .. ntiles-1 only.
  const int t0 = rng.t0;
  const int ntiles = rng.ntiles;
  // rows that see this lane's key: lo_row .. lo_row + n_rows - 1, i.e.
  // j - wr .. j + wl (the count in unsigned: both bounds may be 2^30)
  const int lo_row = mykey - p.wr;
  const uint32_t n_rows = (uint32_t)p.wl + (uint32_t)p.wr + 1u;
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
        if constexpr (kKReg)
          ka[u] = kreg[k2 + u];
        else
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
          pr = in_window(row, lo_row, n_rows) ? pr : 0.0f;
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
  const int tm1 = rng.tm1, tm2 = rng.tm2;
  auto visible = [&](int t) { return sched::dkdv_visible<kTile>(t, rng, qh, p.wl, p.wr); };
  if constexpr (!SPARSE) {
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
  } else {
    // Block-sparse kernels: query tile t of query head jq lies in query
    // block t/2 of that head's mask, in column kblk. The workgroup walks
    // only the tiles of nonzero blocks, in the order above; each wave
    // splits the walk at its own tm1, tm2 as above, so every wave passes
    // the same barriers.
    static_assert(kKeyBlock == kMaskBlock && 2 * kTile == kMaskBlock,
                  "a dK/dV job is one key block of the mask, two tiles one query block");
    const uint8_t* col0 = p.bmask + (size_t)bh * p.group * (size_t)p.bm_stride + kblk;
    MaskScan scan;
    scan.stride = (uint32_t)p.nbm;
    scan.n = p.nbm;
    int scan_head = 0;
    scan.reset(col0, nullptr);
    // the first tile at or after (jq, t) of a nonzero block; jq = group at the end
    auto next_tile = [&](int& jq, int& t) {
      while (jq < p.group) {
        if (scan_head != jq) {
          scan_head = jq;
          scan.reset(col0 + (size_t)jq * (size_t)p.bm_stride, nullptr);
        }
        if (t < ntiles) {
          uint32_t fl;
          const int blk = scan.next(t >> 1, lane, &fl);
          const int tn = blk == (t >> 1) ? t : 2 * blk;
          if (tn < ntiles) {
            t = tn;
            return;
          }
        }
        ++jq;
        t = t0;
      }
    };
    int cj = 0, ct = t0;
    next_tile(cj, ct);
    if (cj < p.group) fill(cj, ct, 0);
    // one tile: load the next one of the walk, then compute (jq, t)
    auto walk_step = [&](auto mask_c) {
      int nj = cj, nt = ct + 1;
      next_tile(nj, nt);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (nj < p.group) fill(nj, nt, (step + 1) & 1);
      if (!decltype(mask_c)::value || visible(ct)) tile(ct, step & 1, mask_c);
      cj = nj;
      ct = nt;
      ++step;
    };
    for (int jq = 0; jq < p.group; ++jq) {
      while (cj == jq && ct < tm1) walk_step(std::true_type());
      while (cj == jq && ct < tm2) walk_step(std::false_type());
      while (cj == jq) walk_step(std::true_type());
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

template <int D, bool CAUSAL, bool SPARSE>
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

  // the job's rows, this wave's rows and the key tiles they walk
  const sched::DqRange rng = sched::dq_range<kQBlock, kTile>(qblk, wave, N, p.wl, p.wr, CAUSAL);
  const int qw0 = rng.qw0;
  const int myq = qw0 + col;

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
  const int kt0 = rng.kt0;
  const int ntiles = rng.ntiles;
  const int wt0 = rng.wt0;
  const int wt1 = rng.wt1;
  // keys this lane's row sees: lo_key .. lo_key + n_keys - 1, i.e. i - wl .. i + wr
  const int lo_key = myq - p.wl;
  const uint32_t n_keys = (uint32_t)p.wl + (uint32_t)p.wr + 1u;
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

    // dQ^T += K^T dS^T for the 32 keys of half kb
    auto accumulate = [&](int kb, const uint32_t* dsk_kb) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int rb = (kb * 32 + m * 16) * D * 2;
        bf16x8 ka[kDB];
#pragma unroll
        for (int db = 0; db < kDB; ++db)
          ka[db] = lds_tr_pair(kt + rb + off.tr[db][0], kt + rb + off.tr[db][1]);
        const uint4 du = {dsk_kb[4 * m], dsk_kb[4 * m + 1], dsk_kb[4 * m + 2], dsk_kb[4 * m + 3]};
        const bf16x8 b = as_bf16x8(du);
#pragma unroll
        for (int db = 0; db < kDB; ++db) dqacc[db] = mfma32(ka[db], b, dqacc[db]);
      }
    };

    // both halves' S, dP and dS, then both halves' dQ products (the MFMAs of
    // the second half's S and dP run under the first half's arithmetic); at
    // d = 64, which runs four waves per SIMD in 128 registers, each half's
    // dS goes into dQ at once instead, which keeps 8 registers fewer live
    // (the products are added in the same order either way)
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
          pr = in_window(key, lo_key, n_keys) ? pr : 0.0f;
        }
        dsv[r] = pr * (dp[r] - dr);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) dsk[kb][j] = pack_bf16x2(dsv[2 * j], dsv[2 * j + 1]);
      if constexpr (D == 64) accumulate(kb, dsk[kb]);
    }
    if constexpr (D != 64) {
      accumulate(0, dsk[0]);
      accumulate(1, dsk[1]);
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
  // Causal: no masked tiles before tm1 = kt0 = 0. No rows: tm2 = tm1.
  const int tm1 = rng.tm1, tm2 = rng.tm2;
  auto visible = [&](int t) { return t >= wt0 && t < wt1; };
  if constexpr (!SPARSE) {
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
  } else {
    // Block-sparse kernels: key tile t lies in key block t/2; waves 0-3
    // hold query block 2*qblk of the head's mask, waves 4-7 block 2*qblk+1.
    // The workgroup walks the tiles where either block is nonzero (their
    // stage is t & 1 as above, so tiles of one block keep alternating
    // stages and a skipped block skips two); a wave computes those where
    // its own block is nonzero.
    static_assert(kQBlock == 2 * kMaskBlock && 2 * kTile == kMaskBlock,
                  "a dQ job is two query blocks of the mask, two tiles one key block");
    const int qbm = 2 * qblk;
    const uint8_t* row0 = p.bmask + (size_t)bh * (size_t)p.bm_stride + (size_t)qbm * p.nbm;
    MaskScan scan;
    scan.stride = 1;
    scan.n = p.nbm;
    scan.reset(row0, qbm + 1 < p.nbm ? row0 + p.nbm : nullptr);
    const uint32_t my_bit = 1u << (wave >> 2);
    // the first tile >= t where either block is nonzero (else ntiles), and its flags
    auto next_tile = [&](int t, uint32_t* fl) {
      const int blk = scan.next(t >> 1, lane, fl);
      return blk == (t >> 1) ? t : min(2 * blk, ntiles);
    };
    uint32_t cf;
    int t = next_tile(kt0, &cf);
    if (t < ntiles) fill(t);
    auto walk_step = [&](auto mask_c) {
      uint32_t nf;
      const int tn = next_tile(t + 1, &nf);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tn < ntiles) fill(tn);
      if ((cf & my_bit) != 0 && (!decltype(mask_c)::value || visible(t))) tile(t, mask_c);
      t = tn;
      cf = nf;
    };
    while (t < tm1) walk_step(std::true_type());
    while (t < tm2) walk_step(std::false_type());
    while (t < ntiles) walk_step(std::true_type());
  }

  if (myq < N) store_rows<D>(p.dq + (head + myq) * D, dqacc, p.scale, half);
}

// At d = 64 the kernels run four waves per SIMD (128 registers, two
// workgroups per CU): 10-15% faster than two, the unmasked kernel without
// spills, the masked one with 11 registers' worth in scratch.
// SPARSE: a block-sparse mask on top of the window (CAUSAL kernels only).
template <int D, bool CAUSAL, bool SPARSE = false>
__global__ __launch_bounds__(kThreads, D == 64 ? 4 : 1)
void bwd_grads_kernel(BwdParams p) {
  static_assert(!SPARSE || CAUSAL, "block-sparse masks use the masked kernels");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[GLayout<D>::kBytes];
  const Job job = job_of<CAUSAL>(p);
  if (job.is_dq)
    dq_job<D, CAUSAL, SPARSE>(p, job.bh, job.blk, smem);
  else
    dkdv_job<D, CAUSAL, SPARSE>(p, job.bh, job.blk, smem);
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

template <int D, bool CAUSAL, bool SPARSE = false>
hipError_t launch_grads_typed(const BwdArgs& a) {
  const BwdParams p = make_params<D>(a);
  const dim3 grid((unsigned)((long long)(p.BH / p.group) * (p.nkb + p.group * p.nqb)));
  hipLaunchKernelGGL((bwd_grads_kernel<D, CAUSAL, SPARSE>), grid, dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_prep(const BwdArgs& a) {
  if (a.d == 64) return launch_prep_typed<64>(a);
  return a.d == 256 ? launch_prep_typed<256>(a) : launch_prep_typed<128>(a);
}

hipError_t launch_backward_grads(const BwdArgs& a) {
  if (a.bmask != nullptr) {  // block-sparse: always the masked kernels
    if (a.d == 64) return launch_grads_typed<64, true, true>(a);
    if (a.d == 128) return launch_grads_typed<128, true, true>(a);
    return launch_grads_wide_sparse(a);
  }
  if (a.d == 64)
    return a.masked() ? launch_grads_typed<64, true>(a) : launch_grads_typed<64, false>(a);
  if (a.d == 256) return launch_grads_wide(a);
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
