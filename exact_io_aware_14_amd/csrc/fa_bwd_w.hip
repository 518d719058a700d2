// Backward exact attention at head dimension 256: the grads launch (the
// row-term launch is shared with the other head dimensions, in
// fa_bwd.hip). The method, the job kinds and their order are those of
// fa_bwd.hip; this file holds the d = 256 shapes of the two jobs.
//
// It is compiled with LLVM's "max-memory-clause" machine scheduler: with
// the default one the dK/dV tile loop rotated accumulator blocks through
// other registers every tile (112-224 AGPR-to-AGPR moves and about 100 AGPR
// reads and writes per 64 MFMAs, the register file being full); with this
// one the loop has none, and the launch takes about a fifth less time (1.42
// to 1.15 ms at B=4, H=8, N=4096, causal) with bitwise the same results.
// The d = 64 and 128 grads kernels run 1-3% slower under that scheduler,
// hence the separate file.
#include "fa_bwd_common.h"

namespace fa {
namespace {

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

template <int D, bool CAUSAL, bool SPARSE>
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

  // the job's keys, this wave's keys (all rows of each 32-row query tile)
  // and the query tiles they walk
  const sched::DkdvRange rng =
      sched::dkdv_range<kKeyBlockW, kQTileW>(kblk, wave, 0, N, p.wl, p.wr, CAUSAL);
  const int k0 = rng.k0;
  const int kw0 = rng.kw0;  // this wave's first key
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
  const int t0 = rng.t0;
  const int ntiles = rng.ntiles;
  // rows that see this lane's key: lo_row .. lo_row + n_rows - 1, i.e.
  // j - wr .. j + wl (the count in unsigned: both bounds may be 2^30)
  const int lo_row = mykey - p.wr;
  const uint32_t n_rows = (uint32_t)p.wl + (uint32_t)p.wr + 1u;
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
  const int tm1 = rng.tm1, tm2 = rng.tm2;
  auto visible = [&](int t) { return sched::dkdv_visible<kQTileW>(t, rng, 0, p.wl, p.wr); };
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
    // block t/4 of that head's mask, in column kblk; the walk over the
    // tiles of nonzero blocks is that of the d = 128 job.
    static_assert(kKeyBlockW == kMaskBlock && 4 * kQTileW == kMaskBlock,
                  "a dK/dV job is one key block of the mask, four tiles one query block");
    const uint8_t* col0 = p.bmask + (size_t)bh * p.group * (size_t)p.bm_stride + kblk;
    MaskScan scan;
    scan.stride = (uint32_t)p.nbm;
    scan.n = p.nbm;
    int scan_head = 0;
    scan.reset(col0, nullptr);
    auto next_tile = [&](int& jq, int& t) {  // first tile at or after (jq, t); jq = group: none
      while (jq < p.group) {
        if (scan_head != jq) {
          scan_head = jq;
          scan.reset(col0 + (size_t)jq * (size_t)p.bm_stride, nullptr);
        }
        if (t < ntiles) {
          uint32_t fl;
          const int blk = scan.next(t >> 2, lane, &fl);
          const int tn = blk == (t >> 2) ? t : 4 * blk;
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
  if (mykey < N) {
    store_rows<D>(p.dk + (head + mykey) * D, dkacc, p.scale, half);
    store_rows<D>(p.dv + (head + mykey) * D, dvacc, 1.0f, half);
  }
}

template <int D, bool CAUSAL, bool SPARSE>
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

  // the job's rows, this wave's rows and the key tiles they walk
  const sched::DqRange rng =
      sched::dq_range<kQBlockW, kKTileW>(qblk, wave, N, p.wl, p.wr, CAUSAL);
  const int qw0 = rng.qw0;
  const int myq = qw0 + col;

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

  const int kt0 = rng.kt0;
  const int ntiles = rng.ntiles;
  const int wt0 = rng.wt0;
  const int wt1 = rng.wt1;
  // keys this lane's row sees: lo_key .. lo_key + n_keys - 1, i.e. i - wl .. i + wr
  const int lo_key = myq - p.wl;
  const uint32_t n_keys = (uint32_t)p.wl + (uint32_t)p.wr + 1u;
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
          pr = in_window(key, lo_key, n_keys) ? pr : 0.0f;
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
    // Block-sparse kernels: the job is query block qblk of the head's mask;
    // key tile t lies in key block t/2. The workgroup walks the tiles of
    // nonzero blocks (stage t & 1 still alternates along the walk: each
    // block is two tiles).
    static_assert(kQBlockW == kMaskBlock && 2 * kKTileW == kMaskBlock,
                  "a dQ job is one query block of the mask, two tiles one key block");
    MaskScan scan;
    scan.stride = 1;
    scan.n = p.nbm;
    scan.reset(p.bmask + (size_t)bh * (size_t)p.bm_stride + (size_t)qblk * p.nbm, nullptr);
    auto next_tile = [&](int t) {  // the first tile >= t of a nonzero block, else ntiles
      uint32_t fl;
      const int blk = scan.next(t >> 1, lane, &fl);
      return blk == (t >> 1) ? t : min(2 * blk, ntiles);
    };
    int t = next_tile(kt0);
    if (t < ntiles) fill(t);
    auto walk_step = [&](auto mask_c) {
      const int tn = next_tile(t + 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tn < ntiles) fill(tn);
      if (!decltype(mask_c)::value || visible(t)) tile(t, mask_c);
      t = tn;
    };
    while (t < tm1) walk_step(std::true_type());
    while (t < tm2) walk_step(std::false_type());
    while (t < ntiles) walk_step(std::true_type());
  }

  if (myq < N) store_rows<D>(p.dq + (head + myq) * D, dqacc, p.scale, half);
}

// SPARSE: a block-sparse mask on top of the window (CAUSAL kernels only).
template <int D, bool CAUSAL, bool SPARSE = false>
__global__ __launch_bounds__(kThreadsW, 1) void bwd_grads_kernel_w(BwdParams p) {
  static_assert(!SPARSE || CAUSAL, "block-sparse masks use the masked kernels");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[WLayout<D>::kBytes];
  const Job job = job_of<CAUSAL>(p);
  if (job.is_dq)
    dq_job_w<D, CAUSAL, SPARSE>(p, job.bh, job.blk, smem);
  else
    dkdv_job_w<D, CAUSAL, SPARSE>(p, job.bh, job.blk, smem);
}

template <bool CAUSAL, bool SPARSE = false>
hipError_t launch_grads_w(const BwdArgs& a) {
  const BwdParams p = make_params<256>(a);
  const dim3 grid((unsigned)((long long)(p.BH / p.group) * (p.nkb + p.group * p.nqb)));
  hipLaunchKernelGGL((bwd_grads_kernel_w<256, CAUSAL, SPARSE>), grid, dim3(kThreadsW), 0,
                     a.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grads_wide(const BwdArgs& a) {
  return a.masked() ? launch_grads_w<true>(a) : launch_grads_w<false>(a);
}

hipError_t launch_grads_wide_sparse(const BwdArgs& a) { return launch_grads_w<true, true>(a); }

}  // namespace fa
