// Scheduling and tile-range arithmetic of the bf16 attention kernels, as
// __host__ __device__ functions: the kernels call them, and the test suite
// compiles the same functions for the host and checks them over many shapes
// and masks (every workgroup slot maps to one block or job, every visible
// (query, key) pair lies in a tile the owning wave walks, tiles walked
// without a mask hold only visible pairs or zero-filled rows, and nothing
// overflows 32 bits).
//
// Masks: key j is visible to query i iff i - wl <= j <= i + wr, with wl, wr
// at most N - 2 (the host maps larger bounds, and "no bound", to kUnbounded
// = 2^30 in the masked kernels; the unmasked kernels ignore wl, wr).
#pragma once

#include <hip/hip_runtime.h>

namespace fa {
namespace sched {

__host__ __device__ inline int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ inline int imax(int a, int b) { return a > b ? a : b; }
// Integer division rounding toward -infinity / +infinity (b > 0).
__host__ __device__ inline int floor_div(int a, int b) {
  return a >= 0 ? a / b : -((b - 1 - a) / b);
}
__host__ __device__ inline int ceil_div(int a, int b) { return -floor_div(-a, b); }

// ---------------------------------------------------------------- forward

// The query blocks of forward workgroup L: block qb_first, then (npass == 2)
// block qb_second, of query head bh.
struct FwdBlock {
  int bh, qb_first, qb_second, npass;
};

// Consecutive workgroups go to the 8 XCDs in turn; with xcd_remap each XCD
// gets whole K/V heads (with all query heads that read them, query head bh
// reading K/V head bh / group) so the K/V of a head is re-read from that
// XCD's L2. Masked launches dispatch the longest rows (most key tiles) first;
// within an XCD their heads go out in pairs when the head count allows, the
// blocks of a pair rank by rank (both heads' longest block, then the next),
// which balances the uneven block lengths while only about two heads' K/V
// are in flight; unmasked launches go head by head. Paired launches (causal
// mask): blocks nqb-1-i and i of one head in one workgroup, head by head.
__host__ __device__ inline FwdBlock fwd_block(int L, int BH, int group, int nqb, bool xcd_remap,
                                              bool masked, bool pair) {
  FwdBlock b;
  int qbr;
  if (pair) {
    const int npair = (nqb + 1) / 2;
    int pi;
    if (xcd_remap) {
      const int xcd = L & 7, idx = L >> 3, slot = idx / npair;
      b.bh = ((slot / group) * 8 + xcd) * group + slot % group;
      pi = idx % npair;
    } else {
      b.bh = L % BH;
      pi = L / BH;
    }
    b.qb_first = nqb - 1 - pi;
    b.qb_second = pi;
    b.npass = b.qb_first != pi ? 2 : 1;
    return b;
  }
  if (xcd_remap) {
    const int xcd = L & 7, idx = L >> 3, hx = BH >> 3;
    const int g2 = (masked && hx % 2 == 0) ? 2 : 1;  // heads per group
    const int grp = idx / (g2 * nqb), within = idx % (g2 * nqb);
    const int slot = grp * g2 + within % g2;
    b.bh = ((slot / group) * 8 + xcd) * group + slot % group;
    qbr = within / g2;
  } else {
    b.bh = L % BH;
    qbr = L / BH;
  }
  b.qb_first = masked ? (nqb - 1 - qbr) : qbr;
  b.qb_second = 0;
  b.npass = 1;
  return b;
}

// Rows and key tiles of wave `wave` (RW rows) of query block qb (BR rows),
// with BC keys per tile: the workgroup walks tiles t_first .. t_end-1, those
// holding a key one of its rows sees, and the wave computes on tiles
// wt_first .. wt_end-1, those holding one of its rows' keys.
struct FwdRange {
  int q0, qw0, wave_last, qlast, t_first, t_end, wt_first, wt_end;
};

template <int BR, int RW, int BC>
__host__ __device__ inline FwdRange fwd_range(int qb, int wave, int N, int wl, int wr,
                                              bool masked) {
  FwdRange r;
  r.q0 = qb * BR;
  r.qw0 = r.q0 + wave * RW;
  r.wave_last = imin(r.qw0 + RW, N) - 1;
  r.qlast = imin(r.q0 + BR, N) - 1;
  const int ktiles_all = (N + BC - 1) / BC;
  r.t_first = masked ? imax(0, r.q0 - wl) / BC : 0;
  r.t_end = masked ? imin(N - 1, r.qlast + wr) / BC + 1 : ktiles_all;
  r.wt_first = masked ? imax(0, r.qw0 - wl) / BC : 0;
  r.wt_end = r.qw0 >= N ? r.wt_first
                        : (masked ? imin(N - 1, r.wave_last + wr) / BC + 1 : ktiles_all);
  return r;
}

// A forward tile needs the per-score masks where it passes N, the wave's
// first row's upper bound or its last row's lower bound.
template <int BC>
__host__ __device__ inline bool fwd_need_mask(int t, const FwdRange& r, int N, int wl, int wr,
                                              bool masked) {
  const int key0 = t * BC;
  return (key0 + BC > N) || (masked && (key0 + BC - 1 > r.qw0 + wr || key0 < r.wave_last - wl));
}

// ---------------------------------------------------------------- backward

// Job of grads workgroup L. Every K/V head owns nkb dK/dV jobs and
// group * nqb dQ jobs (those of its query heads). The two kinds are
// interleaved evenly, each sequence ordered from the most expensive block
// down (masked: dK/dV of the first key blocks, dQ of the last query blocks).
// Consecutive workgroups go to the 8 XCDs in turn; with xcd_remap each XCD
// gets whole K/V heads (with their query heads) so that their K/V and Q/dO
// stay in its L2.
struct Job {
  int bh;    // dK/dV: the K/V head (batch * K/V heads); dQ: the query head
  int blk;   // key block (dK/dV) or query block (dQ)
  bool is_dq;
};

__host__ __device__ inline Job grads_job(int L, int BH, int group, int nkb, int nqb,
                                         bool xcd_remap, bool masked) {
  const int ndq = group * nqb;
  const int per_head = nkb + ndq;
  const int bhkv = BH / group;
  int kvh, j;
  if (xcd_remap) {
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
    // rank r: query block r / group (from the last one under a mask) of
    // query head r % group of this K/V head
    const int qbr = rank / group;
    job.bh = kvh * group + rank % group;
    job.blk = masked ? (nqb - 1 - qbr) : qbr;
  } else {
    job.bh = kvh;
    job.blk = rank;
  }
  return job;
}

// dK/dV job of key block kblk (KB keys), wave (kw, qh): keys kw0 .. kw0+31
// and rows RW qh .. RW qh + RW-1 of every query tile of T rows. The job
// walks query tiles t0 .. ntiles-1 (those holding a row that sees one of its
// keys); the wave's rows see all of its keys in tiles tm1 .. tm2-1 (no
// mask), and the tiles before and after cross a window edge or show the
// wave none of its keys (dkdv_visible).
struct DkdvRange {
  int k0, kw0, kend, t0, ntiles, tm1, tm2;
};

template <int KB, int T, int RW = 32>
__host__ __device__ inline DkdvRange dkdv_range(int kblk, int kw, int qh, int N, int wl, int wr,
                                                bool masked) {
  DkdvRange r;
  r.k0 = kblk * KB;
  r.kw0 = r.k0 + 32 * kw;
  r.kend = imin(r.k0 + KB, N) - 1;
  r.t0 = masked ? imax(0, r.k0 - wr) / T : 0;
  r.ntiles = masked ? imin(N - 1, r.kend + wl) / T + 1 : (N + T - 1) / T;
  r.tm1 = r.t0;
  r.tm2 = r.ntiles;
  if (masked) {
    r.tm1 = imin(r.ntiles, imax(r.t0, ceil_div(r.kw0 + 31 - wr - RW * qh, T)));
    r.tm2 = imin(r.ntiles, imax(r.tm1, floor_div(r.kw0 + wl - RW * qh - (RW - 1), T) + 1));
  }
  return r;
}

template <int T, int RW = 32>
__host__ __device__ inline bool dkdv_visible(int t, const DkdvRange& r, int qh, int wl, int wr) {
  const int r0 = t * T + RW * qh;
  return r0 + (RW - 1) >= r.kw0 - wr && r0 <= r.kw0 + 31 + wl;
}

// dQ job of query block qblk (QB rows), wave `wave` (32 rows): the job walks
// key tiles kt0 .. ntiles-1 (those holding a key one of its rows sees), the
// wave computes on tiles wt0 .. wt1-1, of which tm1 .. tm2-1 show all their
// keys to all of its rows (no mask).
struct DqRange {
  int q0, qw0, wave_last, kt0, ntiles, wt0, wt1, tm1, tm2;
};

template <int QB, int T>
__host__ __device__ inline DqRange dq_range(int qblk, int wave, int N, int wl, int wr,
                                            bool masked) {
  DqRange r;
  r.q0 = qblk * QB;
  r.qw0 = r.q0 + wave * 32;
  r.wave_last = imin(r.qw0 + 32, N) - 1;
  const int ntiles_all = (N + T - 1) / T;
  const int qend = imin(r.q0 + QB, N) - 1;
  r.kt0 = masked ? imax(0, r.q0 - wl) / T : 0;
  r.ntiles = masked ? imin(N - 1, qend + wr) / T + 1 : ntiles_all;
  r.wt0 = masked ? imax(0, r.qw0 - wl) / T : 0;
  r.wt1 = r.qw0 >= N ? r.wt0 : (masked ? imin(N - 1, r.wave_last + wr) / T + 1 : ntiles_all);
  r.tm1 = r.kt0;
  r.tm2 = r.wt1;
  if (masked) {
    r.tm1 = imin(r.ntiles, imax(r.kt0, ceil_div(r.wave_last - wl, T)));
    r.tm2 = imin(r.wt1, imax(r.tm1, floor_div(r.qw0 + wr - (T - 1), T) + 1));
  }
  if (r.qw0 >= N) r.tm2 = r.tm1;  // no rows: every tile is skipped
  return r;
}

}  // namespace sched
}  // namespace fa
