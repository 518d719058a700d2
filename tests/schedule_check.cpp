// Host-side check of the attention kernels' scheduling and tile-range
// arithmetic (exact_io_aware_14_amd/csrc/fa_schedule.h, the functions the
// kernels call), against the definition of the mask: key j is visible to
// query i iff i - wl <= j <= i + wr (within 0 .. N-1), with "no bound"
// passed to the masked kernels as 2^30 and bounds of N-1 or more mapped to
// no bound first, as the library's host code does.
//
// For many shapes, masks and head groupings it checks that
//   * every workgroup slot of a forward launch maps to one (head, query
//     block) and every such pair to exactly one slot (paired launches: two
//     blocks per slot); every grads slot to one dK/dV or dQ job and every
//     job to exactly one slot;
//   * every (query, key) pair a wave's rows see lies in a tile the wave
//     computes, within the tiles the workgroup walks;
//   * every tile a wave computes without per-score masks holds only visible
//     pairs, or rows / keys past N (zero-filled on load, so they add
//     nothing);
//   * every tile a dK/dV wave skips holds no visible pair of its keys;
//   * the ranges stay inside 0 .. number of tiles, and a 64-bit evaluation
//     of the forward's and the dQ job's ranges gives the same values (no
//     32-bit overflow).
// Prints one line per failure (at most 20) and a summary; exit status 1 on
// any failure.

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <set>
#include <tuple>
#include <utility>
#include <vector>

#include "fa_schedule.h"

namespace s = fa::sched;

static long long g_checks = 0, g_fail = 0;

#define CHECK(cond, ...)                                   \
  do {                                                     \
    ++g_checks;                                            \
    if (!(cond)) {                                         \
      if (++g_fail <= 20) {                                \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__);   \
        std::printf(__VA_ARGS__);                          \
        std::printf("\n");                                 \
      }                                                    \
    }                                                      \
  } while (0)

constexpr int kUnbounded = 1 << 30;

// A mask as the kernels see it: masked kernels get (wl, wr) with no bound as
// 2^30; unmasked kernels see every key.
struct Mask {
  bool masked;
  int wl, wr;
};

static Mask make_mask(bool masked, int left, int right, int N) {
  // the library maps bounds of N-1 or more to -1 (no bound)
  if (left >= N - 1) left = -1;
  if (right >= N - 1) right = -1;
  Mask m;
  m.masked = masked;
  m.wl = left < 0 ? kUnbounded : left;
  m.wr = right < 0 ? kUnbounded : right;
  return m;
}

static bool visible(const Mask& m, long long i, long long j, int N) {
  if (i < 0 || i >= N || j < 0 || j >= N) return false;
  if (!m.masked) return true;
  return j >= i - m.wl && j <= i + m.wr;
}

// all pairs of rows a..b and keys c..d visible (empty ranges: true)
static bool all_visible(const Mask& m, int a, int b, int c, int d, int N, bool brute) {
  if (a > b || c > d) return true;
  if (brute) {
    for (int i = a; i <= b; ++i)
      for (int j = c; j <= d; ++j)
        if (!visible(m, i, j, N)) return false;
    return true;
  }
  if (!m.masked) return true;
  return (long long)c >= (long long)b - m.wl && (long long)d <= (long long)a + m.wr;
}

// no pair of rows a..b and keys c..d visible
static bool none_visible(const Mask& m, int a, int b, int c, int d, int N, bool brute) {
  if (a > b || c > d) return true;
  if (brute) {
    for (int i = a; i <= b; ++i)
      for (int j = c; j <= d; ++j)
        if (visible(m, i, j, N)) return false;
    return true;
  }
  if (!m.masked) return false;
  return (long long)d < (long long)a - m.wl || (long long)c > (long long)b + m.wr;
}

// visible keys of row i: [lo, hi] (lo > hi: none)
static std::pair<long long, long long> keys_of(const Mask& m, int i, int N) {
  if (!m.masked) return {0, N - 1};
  long long lo = (long long)i - m.wl, hi = (long long)i + m.wr;
  if (lo < 0) lo = 0;
  if (hi > N - 1) hi = N - 1;
  return {lo, hi};
}

// ---------------------------------------------------------------- forward

constexpr int kBR = 128, kRW = 32;

static void check_forward_map(int BH, int group, int N, bool masked, bool pair) {
  const int nqb = (N + kBR - 1) / kBR;
  const bool xcd = (BH / group) % 8 == 0;
  const long long grid = (long long)BH * (pair ? (nqb + 1) / 2 : nqb);
  std::vector<int> seen((size_t)BH * nqb, 0);
  for (long long L = 0; L < grid; ++L) {
    const s::FwdBlock b = s::fwd_block((int)L, BH, group, nqb, xcd, masked, pair);
    CHECK(b.bh >= 0 && b.bh < BH, "fwd map: bh %d out of range (BH %d L %lld)", b.bh, BH, L);
    CHECK(b.npass == 1 || b.npass == 2, "fwd map: npass %d", b.npass);
    if (b.bh < 0 || b.bh >= BH) continue;
    for (int pass = 0; pass < b.npass; ++pass) {
      const int qb = pass ? b.qb_second : b.qb_first;
      CHECK(qb >= 0 && qb < nqb, "fwd map: qb %d of %d", qb, nqb);
      if (qb >= 0 && qb < nqb) ++seen[(size_t)b.bh * nqb + qb];
    }
    if (pair && b.npass == 2) CHECK(b.qb_first > b.qb_second, "fwd map: pair order");
  }
  for (size_t i = 0; i < seen.size(); ++i)
    CHECK(seen[i] == 1, "fwd map: block %zu seen %d times (BH %d group %d N %d masked %d pair %d)",
          i, seen[i], BH, group, N, masked, pair);
}

template <int kBC>
static void check_forward_ranges(int N, const Mask& m) {
  const int nqb = (N + kBR - 1) / kBR;
  const int ntiles = (N + kBC - 1) / kBC;
  const bool brute = N <= 1100;
  for (int qb = 0; qb < nqb; ++qb) {
    for (int wave = 0; wave < kBR / kRW; ++wave) {
      const s::FwdRange r = s::fwd_range<kBR, kRW, kBC>(qb, wave, N, m.wl, m.wr, m.masked);
      CHECK(r.t_first >= 0 && r.t_end <= ntiles && r.t_first <= r.t_end,
            "fwd range: tiles %d..%d of %d", r.t_first, r.t_end, ntiles);
      // 64-bit evaluation of the same ranges
      {
        const long long q0 = (long long)qb * kBR, qw0 = q0 + wave * kRW;
        const long long wl = m.wl, wr = m.wr;
        const long long wlast = std::min<long long>(qw0 + kRW, N) - 1;
        const long long qlast = std::min<long long>(q0 + kBR, N) - 1;
        const long long tf = m.masked ? std::max<long long>(0, q0 - wl) / kBC : 0;
        const long long te = m.masked ? std::min<long long>(N - 1, qlast + wr) / kBC + 1 : ntiles;
        CHECK(tf == r.t_first && te == r.t_end, "fwd range: 32-bit %d..%d vs 64-bit %lld..%lld",
              r.t_first, r.t_end, tf, te);
        (void)wlast;
      }
      if (r.qw0 >= N) {
        CHECK(r.wt_end == r.wt_first, "fwd range: a wave past N computes tiles");
        continue;
      }
      CHECK(r.t_first <= r.wt_first && r.wt_end <= r.t_end,
            "fwd range: wave tiles %d..%d outside %d..%d", r.wt_first, r.wt_end, r.t_first, r.t_end);
      // every visible key of every row of the wave lies in the wave's tiles
      for (int i = r.qw0; i <= r.wave_last; ++i) {
        const auto k = keys_of(m, i, N);
        if (k.first > k.second) continue;
        CHECK(k.first / kBC >= r.wt_first && k.second / kBC < r.wt_end,
              "fwd range: row %d keys %lld..%lld outside tiles %d..%d (N %d wl %d wr %d)", i,
              k.first, k.second, r.wt_first, r.wt_end, N, m.wl, m.wr);
      }
      for (int t = r.wt_first; t < r.wt_end; ++t) {
        const bool mask = s::fwd_need_mask<kBC>(t, r, N, m.wl, m.wr, m.masked);
        const int key0 = t * kBC, key1 = std::min(N, key0 + kBC) - 1;
        if (key0 + kBC > N) CHECK(mask, "fwd range: tail tile %d without mask (N %d)", t, N);
        if (!mask)
          CHECK(all_visible(m, r.qw0, r.wave_last, key0, key1, N, brute),
                "fwd range: tile %d unmasked with an invisible pair (qb %d wave %d N %d wl %d wr %d)",
                t, qb, wave, N, m.wl, m.wr);
      }
    }
  }
}

// ---------------------------------------------------------------- backward

static void check_grads_map(int BH, int group, int N, bool masked, int KB, int QB) {
  // KB or QB 0: a launch of the other job kind only
  const int nkb = KB ? (N + KB - 1) / KB : 0, nqb = QB ? (N + QB - 1) / QB : 0;
  const int bhkv = BH / group;
  const bool xcd = bhkv % 8 == 0;
  const long long grid = (long long)bhkv * (nkb + group * nqb);
  std::vector<int> seen_kv((size_t)bhkv * nkb, 0), seen_q((size_t)BH * nqb, 0);
  for (long long L = 0; L < grid; ++L) {
    const s::Job j = s::grads_job((int)L, BH, group, nkb, nqb, xcd, masked);
    if (j.is_dq) {
      CHECK(j.bh >= 0 && j.bh < BH && j.blk >= 0 && j.blk < nqb, "grads map: dQ job %d %d", j.bh,
            j.blk);
      if (j.bh >= 0 && j.bh < BH && j.blk >= 0 && j.blk < nqb) ++seen_q[(size_t)j.bh * nqb + j.blk];
    } else {
      CHECK(j.bh >= 0 && j.bh < bhkv && j.blk >= 0 && j.blk < nkb, "grads map: dK/dV job %d %d",
            j.bh, j.blk);
      if (j.bh >= 0 && j.bh < bhkv && j.blk >= 0 && j.blk < nkb) ++seen_kv[(size_t)j.bh * nkb + j.blk];
    }
  }
  for (size_t i = 0; i < seen_kv.size(); ++i)
    CHECK(seen_kv[i] == 1, "grads map: dK/dV job %zu seen %d times (BH %d group %d N %d)", i,
          seen_kv[i], BH, group, N);
  for (size_t i = 0; i < seen_q.size(); ++i)
    CHECK(seen_q[i] == 1, "grads map: dQ job %zu seen %d times (BH %d group %d N %d)", i, seen_q[i],
          BH, group, N);
}

// dK/dV job: key blocks of KB keys, query tiles of T rows; a wave owns 32
// keys (kw) and the 32 rows 32 qh .. of every tile.
template <int KB, int T, int RW = 32>
static void check_dkdv(int N, const Mask& m, int n_kw, int n_qh) {
  const int nkb = (N + KB - 1) / KB;
  const int ntiles_all = (N + T - 1) / T;
  const bool brute = N <= 1100;
  for (int kblk = 0; kblk < nkb; ++kblk)
    for (int kw = 0; kw < n_kw; ++kw)
      for (int qh = 0; qh < n_qh; ++qh) {
        const s::DkdvRange r = s::dkdv_range<KB, T, RW>(kblk, kw, qh, N, m.wl, m.wr, m.masked);
        CHECK(r.t0 >= 0 && r.ntiles <= ntiles_all && r.t0 <= r.tm1 && r.tm1 <= r.tm2 &&
                  r.tm2 <= r.ntiles,
              "dkdv range: %d %d %d %d of %d", r.t0, r.tm1, r.tm2, r.ntiles, ntiles_all);
        const int ka = r.kw0, kb = std::min(N, r.kw0 + 32) - 1;  // the wave's keys
        if (ka > kb) continue;
        for (int t = 0; t < ntiles_all; ++t) {
          const int ra = t * T + RW * qh, rb = std::min(N, ra + RW) - 1;  // the wave's rows of t
          const bool walked = t >= r.t0 && t < r.ntiles;
          const bool unmasked = t >= r.tm1 && t < r.tm2;
          const bool computed =
              unmasked || (walked && s::dkdv_visible<T, RW>(t, r, qh, m.wl, m.wr));
          if (!computed)
            CHECK(none_visible(m, ra, rb, ka, kb, N, brute),
                  "dkdv: tile %d skipped with a visible pair (kblk %d kw %d qh %d N %d wl %d wr %d)",
                  t, kblk, kw, qh, N, m.wl, m.wr);
          if (unmasked)
            CHECK(all_visible(m, ra, rb, ka, kb, N, brute),
                  "dkdv: tile %d unmasked with an invisible pair (kblk %d kw %d qh %d N %d wl %d wr %d)",
                  t, kblk, kw, qh, N, m.wl, m.wr);
        }
      }
}

// dQ job: query blocks of QB rows (32 per wave), key tiles of T keys.
template <int QB, int T>
static void check_dq(int N, const Mask& m) {
  const int nqb = (N + QB - 1) / QB;
  const int ntiles_all = (N + T - 1) / T;
  const bool brute = N <= 1100;
  for (int qblk = 0; qblk < nqb; ++qblk)
    for (int wave = 0; wave < QB / 32; ++wave) {
      const s::DqRange r = s::dq_range<QB, T>(qblk, wave, N, m.wl, m.wr, m.masked);
      CHECK(r.kt0 >= 0 && r.ntiles <= ntiles_all && r.kt0 <= r.tm1 && r.tm1 <= r.tm2,
            "dq range: %d %d %d %d", r.kt0, r.tm1, r.tm2, r.ntiles);
      {
        const long long q0 = (long long)qblk * QB, qend = std::min<long long>(q0 + QB, N) - 1;
        const long long kt0 = m.masked ? std::max<long long>(0, q0 - m.wl) / T : 0;
        const long long nt = m.masked ? std::min<long long>(N - 1, qend + m.wr) / T + 1 : ntiles_all;
        CHECK(kt0 == r.kt0 && nt == r.ntiles, "dq range: 32-bit vs 64-bit");
      }
      if (r.qw0 >= N) {
        CHECK(r.tm1 == r.tm2, "dq: a wave past N computes tiles");
        continue;
      }
      CHECK(r.kt0 <= r.wt0 && r.wt1 <= r.ntiles && r.tm2 <= r.wt1, "dq range: wave tiles");
      for (int i = r.qw0; i <= r.wave_last; ++i) {
        const auto k = keys_of(m, i, N);
        if (k.first > k.second) continue;
        CHECK(k.first / T >= r.wt0 && k.second / T < r.wt1,
              "dq: row %d keys %lld..%lld outside tiles %d..%d", i, k.first, k.second, r.wt0, r.wt1);
      }
      for (int t = 0; t < ntiles_all; ++t) {
        const int key0 = t * T, key1 = std::min(N, key0 + T) - 1;
        const bool unmasked = t >= r.tm1 && t < r.tm2;
        const bool computed =
            unmasked || (t >= r.kt0 && t < r.ntiles && t >= r.wt0 && t < r.wt1);
        if (!computed)
          CHECK(none_visible(m, r.qw0, r.wave_last, key0, key1, N, brute),
                "dq: tile %d skipped with a visible pair (qblk %d wave %d N %d wl %d wr %d)", t,
                qblk, wave, N, m.wl, m.wr);
        if (unmasked)
          CHECK(all_visible(m, r.qw0, r.wave_last, key0, key1, N, brute),
                "dq: tile %d unmasked with an invisible pair (qblk %d wave %d N %d wl %d wr %d)", t,
                qblk, wave, N, m.wl, m.wr);
      }
    }
}

int main() {
  const int lengths[] = {1, 2, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257,
                         300, 333, 511, 512, 513, 700, 1000, 1025, 4096, 4097, 8192, 8320};
  // (left, right) windows, -1 no bound; bounds past N are mapped by make_mask
  const int windows[][2] = {{-1, 0},  {0, 0},    {1, 0},     {16, 0},  {63, 0},    {64, 0},
                            {100, 0}, {5, 7},    {-1, 40},   {200, -1}, {31, 31},  {1000, 1000},
                            {0, 65},  {0, -1},   {-1, 1},    {127, 0}, {128, 128}, {3000, 100},
                            {1023, 0}, {2147483647, 0}, {-1, 2147483647}};
  srand(12345);
  for (int N : lengths) {
    std::vector<Mask> masks;
    masks.push_back(make_mask(false, -1, -1, N));
    for (const auto& w : windows) masks.push_back(make_mask(true, w[0], w[1], N));
    for (int r = 0; r < 6; ++r)  // random bounds up to N + 64, either side possibly unbounded
      masks.push_back(make_mask(true, rand() % 4 == 0 ? -1 : rand() % (N + 64),
                                rand() % 4 == 0 ? -1 : rand() % (N + 64), N));
    for (const Mask& m : masks) {
      check_forward_ranges<64>(N, m);  // 64-key tiles
      check_forward_ranges<32>(N, m);  // 32-key tiles (d = 256, bf16)
      check_dkdv<128, 64>(N, m, 4, 2);  // d <= 128: 128-key jobs, 64-row tiles, 8 waves
      check_dkdv<128, 32>(N, m, 4, 1);  // d = 256: 128-key jobs, 32-row tiles, 4 waves
      check_dkdv<128, 128, 128>(N, m, 4, 1);  // d = 128: 128-key jobs, 128-row tiles, 4 waves
      check_dq<256, 64>(N, m);          // d <= 128: 256-row jobs, 64-key tiles
      check_dq<128, 64>(N, m);          // d = 256: 128-row jobs, 64-key tiles
    }
    const int groupings[][2] = {{1, 1}, {2, 1}, {3, 1}, {8, 1},  {16, 1}, {16, 2},
                                {24, 3}, {32, 4}, {64, 1}, {64, 8}, {48, 6}, {128, 32}};
    for (const auto& g : groupings)
      for (int masked = 0; masked < 2; ++masked) {
        check_forward_map(g[0], g[1], N, masked, false);
        if (masked) check_forward_map(g[0], g[1], N, true, true);
        check_grads_map(g[0], g[1], N, masked, 128, 256);
        check_grads_map(g[0], g[1], N, masked, 128, 128);
        check_grads_map(g[0], g[1], N, masked, 128, 0);  // launches of one job kind
        check_grads_map(g[0], g[1], N, masked, 0, 256);
      }
  }
  std::printf("%lld checks, %lld failures\n", g_checks, g_fail);
  return g_fail ? 1 : 0;
}
