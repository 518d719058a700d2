// FP8 forward with incoherent processing for gfx950.
//
// Method: both products of the forward take FP8 operands, and Q and K are
// first multiplied by a Hadamard transform with random signs, which spreads
// outlier channels over all channels before quantisation ("Flash Attention:
// بهینه‌سازی مکانیزم توجه در ترنسفورمرها" (deepfa.ir), FlashAttention 3,
// section "پردازش ناهمدوس برای FP8"; "Flash Attention: Rivoluzionando
// l'Efficienza dei Modelli Transformer" (unite.ai), section on
// FlashAttention-3, items 2 and 3). With M = diag(s) H (s the signs, H the
// Sylvester Hadamard matrix, H H^T = d I), (Q M)(K M)^T = d Q K^T, so the
// scores are unchanged up to the factor 1/d and only the quantisation error
// moves.
//
// Two kernels:
//
// * fp8_prep_kernel, one workgroup per 64-row tile of Q, K or V. Q and K
//   rows get the sign flips and the fast Walsh-Hadamard transform along d
//   in fp32 (log2 d butterfly stages: all but two inside a lane, those two
//   across the four lanes that share a row), then a power-of-two scale (per
//   query row for Q, per 64-key tile for K) and rounding to OCP e4m3. V is
//   not rotated; it gets a power-of-two scale per column and block of 32
//   keys. K and V^T land in the workspace as the exact byte images the
//   forward's LDS stages hold (swizzled, tile after tile), so the forward
//   fills its stages with plain contiguous copies.
// * fwd_fp8_kernel: the bf16 forward's schedule (a workgroup per 128 query
//   rows, four waves of 32 rows, double-buffered 64-key tiles filled by
//   direct global->LDS loads) on the fp8 MFMA 32x32x64. Each wave computes
//   S^T = K Q^T in two instructions per 32 keys at d = 128 (four times the
//   depth of the bf16 instruction), folds the Q row scale and the K tile
//   scale into the softmax's exponent factor, rounds the probabilities to
//   e4m3 in its own lanes, and computes O^T += V^T P^T with the per-block V
//   scales applied by the instruction's own block-scale operand.
//
// Register layout of v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 x fp8, wave64,
// lane l, half h = l / 32, column c = l % 32), measured on gfx950: lane
// (h, c) holds 32 bytes of row c of A (column c of B); the instruction's
// k = 64 values split into two scale blocks, block 0 made of bytes 0-15 of
// lanes c and c + 32 and block 1 of bytes 16-31 of both, and block g of row
// c is multiplied by 2^(x - 127), x the byte the opsel operand picks from
// lane (g, c)'s scale register. Which byte stands for which k is otherwise
// free, as long as A and B agree. The accumulator layout is that of the
// bf16 32x32 instructions.
//
// Key order chosen here: in a 64-key tile, byte j of lane half h of the P^T
// and V^T operands is key 32 (j / 16) + 16 h + j % 16, so scale block g is
// keys 32g .. 32g+31. For P^T to come out of the S^T accumulator in that
// order inside each lane, row rho of the 32-row K operand block kb reads key
// 32 kb + 16 ((rho >> 2) & 1) + 4 (rho >> 3) + (rho & 3): accumulator
// element r of lane half h then holds key 32 kb + 16 h + r.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_schedule.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kTileKeys = 64;
constexpr float kE4m3Max = 448.0f;
// The probabilities are formed as p = 2^(c s - m + kShift) with m the
// integer reference maximum, which a row maximum may exceed by up to kSlack
// before the reference moves: p <= 2^(kSlack + kShift) = 2^8, inside the
// e4m3 range (448). Relative to the final reference of a row (its maximum
// rounded up to an integer) every p is then 2^8 P times 2^-j, j = 0 .. kSlack
// a whole power of two, so its e4m3 code is that of 2^8 P (the rounding the
// method defines, scale 2^-8) rescaled exactly, except where 2^(kShift) P
// falls below the e4m3 normal range, P < 2^-12, at most 2^-16 off each.
constexpr float kSlack = 2.0f;
constexpr float kShift = 6.0f;
constexpr int kWavesF = 4;
constexpr int kThreadsF = kWavesF * 64;
constexpr int kRowsF = kWavesF * 32;  // query rows per workgroup

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Exponent e of the smallest power of two with m <= 448 * 2^e (m >= 0 finite);
// 0 for m == 0. With m = f 2^k, f in [0.5, 1), and 448 = 0.875 * 2^9:
// e = k - 9, plus one when f > 0.875. No division, so the choice is exact.
__device__ __forceinline__ int scale_exponent(float m) {
  if (!(m > 0.0f)) return 0;
  int k;
  const float f = frexpf(m, &k);
  return k - 9 + (f > 0.875f ? 1 : 0);
}

// e4m3 codes of a and b (round to nearest even; clamped to +-448 first, the
// conversion itself does not saturate) into bytes 0-1 (HI false) or 2-3 of old.
template <bool HI>
__device__ __forceinline__ int cvt_e4m3x2(float a, float b, int old) {
  a = fminf(fmaxf(a, -kE4m3Max), kE4m3Max);
  b = fminf(fmaxf(b, -kE4m3Max), kE4m3Max);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  return (uint32_t)cvt_e4m3x2<true>(c, d, cvt_e4m3x2<false>(a, b, 0));
}

// The same for values known to lie in [0, 448] (the probabilities): no clamp.
__device__ __forceinline__ uint32_t pack_e4m3x4_unclamped(float a, float b, float c, float d) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false),
                                                   true);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Chunk swizzles of the LDS images (16-byte chunks). K tile: row r (a key)
// of D bytes; a K operand read has 16 lanes reading the same chunk of rows
// {0-3, 16-19, 4-7, 20-23} (or {8-11, 24-27, 12-15, 28-31}) + 32 kb; the
// swizzle puts those 16 reads on 16 distinct 16-byte bank groups. V^T tile:
// row c (a column of V) of 64 bytes, read by 16 consecutive rows per chunk.
template <int D>
__device__ __forceinline__ int k_swizzle(int r) {
  return D == 128 ? (((r >> 1) & 3) | ((r >> 2) & 4)) : (((r >> 2) & 1) | ((r >> 3) & 2));
}
__device__ __forceinline__ int vt_swizzle(int c) { return (c >> 2) & 3; }

// ---------------------------------------------------------------- prep

struct PrepParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  unsigned char* q8;   // [B,H,N,D] codes
  float* qs;           // [B,H,N] row factors a_i (/ D when rotated)
  unsigned char* k8;   // [B,Hkv,T] tile images, 64*D bytes each
  float* ks;           // [B,Hkv,T] tile scales
  unsigned char* v8;   // [B,Hkv,T] V^T tile images, 64*D bytes each
  unsigned char* vs;   // [B,Hkv,T,256] E8M0 block scales
  uint32_t sign_mask[4];  // bit j set: s_j = -1
  int rotate;
  int log2d;
  int BH, BHkv, N, T;
};

template <int D>
__global__ __launch_bounds__(256) void fp8_prep_kernel(PrepParams p) {
  constexpr int E = D / 4;  // Q/K elements per lane: four lanes per row
  __shared__ __attribute__((aligned(16))) uint16_t vt[kTileKeys * D];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const long long job = blockIdx.x;
  const long long nq = (long long)p.BH * p.T, nk = (long long)p.BHkv * p.T;

  if (job < nq + nk) {
    // ---- a tile of 64 rows of Q or K
    const bool isq = job < nq;
    const long long j2 = isq ? job : job - nq;
    const int head = (int)(j2 / p.T), t = (int)(j2 % p.T);
    const int r = tid >> 2, part = tid & 3;
    const int row = t * kTileKeys + r;
    const uint16_t* src = (isq ? p.q : p.k) + (size_t)head * p.N * D;
    const auto rs = make_rsrc(src, (uint32_t)p.N * D * 2u);  // rows past N read 0
    float x[E];
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
      const uint4 u = buf_load16(rs, (uint32_t)(row * D + part * E + 8 * i) * 2u);
      x[8 * i + 0] = bf16_lo(u.x);
      x[8 * i + 1] = bf16_hi(u.x);
      x[8 * i + 2] = bf16_lo(u.y);
      x[8 * i + 3] = bf16_hi(u.y);
      x[8 * i + 4] = bf16_lo(u.z);
      x[8 * i + 5] = bf16_hi(u.z);
      x[8 * i + 6] = bf16_lo(u.w);
      x[8 * i + 7] = bf16_hi(u.w);
    }
    if (p.rotate) {
      // y = (x o s) H: sign flips, then the butterflies (u, v) -> (u + v, u - v)
      // over every bit of the index; elements part*E + i live in this lane
      const int bit0 = part * E;
      const int wi = bit0 >> 5;
      const uint32_t word = wi == 0 ? p.sign_mask[0]
                          : wi == 1 ? p.sign_mask[1]
                          : wi == 2 ? p.sign_mask[2] : p.sign_mask[3];
      const uint32_t bits = word >> (bit0 & 31);
#pragma unroll
      for (int i = 0; i < E; ++i)
        x[i] = __uint_as_float(__float_as_uint(x[i]) ^ (((bits >> i) & 1u) << 31));
#pragma unroll
      for (int s = 1; s < E; s <<= 1)
#pragma unroll
        for (int i = 0; i < E; ++i)
          if ((i & s) == 0) {
            const float a = x[i], b = x[i + s];
            x[i] = a + b;
            x[i + s] = a - b;
          }
      // index bits log2(E) and log2(E)+1 select the lane (part bits 0, 1)
#pragma unroll
      for (int lx = 1; lx <= 2; lx <<= 1) {
        const bool upper = (part & lx) != 0;
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const float o = __shfl_xor(x[i], lx, 64);
          x[i] = upper ? (o - x[i]) : (x[i] + o);
        }
      }
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) m = fmaxf(m, fabsf(x[i]));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    if (!isq) {
      // one scale for the whole tile: the other 15 rows of the wave, then the waves
#pragma unroll
      for (int lx = 4; lx < 64; lx <<= 1) m = fmaxf(m, __shfl_xor(m, lx, 64));
      if ((tid & 63) == 0) red[tid >> 6] = m;
      __syncthreads();
      m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    }
    const int e = scale_exponent(m);
    uint32_t w[E / 4];
#pragma unroll
    for (int i = 0; i < E / 4; ++i)
      w[i] = pack_e4m3x4(ldexpf(x[4 * i], -e), ldexpf(x[4 * i + 1], -e), ldexpf(x[4 * i + 2], -e),
                         ldexpf(x[4 * i + 3], -e));
    if (isq) {
      if (row < p.N) {
        unsigned char* dst = p.q8 + ((size_t)head * p.N + row) * D + part * E;
#pragma unroll
        for (int i = 0; i < E / 16; ++i)
          *reinterpret_cast<uint4*>(dst + 16 * i) =
              uint4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
        if (part == 0) p.qs[(size_t)head * p.N + row] = ldexpf(1.0f, e - (p.rotate ? p.log2d : 0));
      }
    } else {
      unsigned char* img = p.k8 + ((size_t)head * p.T + t) * (kTileKeys * D);
#pragma unroll
      for (int i = 0; i < E / 16; ++i) {
        const int ch = part * (E / 16) + i;
        *reinterpret_cast<uint4*>(img + r * D + 16 * (ch ^ k_swizzle<D>(r))) =
            uint4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
      }
      if (tid == 0) p.ks[(size_t)head * p.T + t] = ldexpf(1.0f, e);
    }
    return;
  }

  // ---- a tile of 64 keys of V: per column c and block g of 32 keys, a
  // power-of-two scale and the codes, stored transposed (V^T)
  const long long j3 = job - nq - nk;
  const int head = (int)(j3 / p.T), t = (int)(j3 % p.T);
  const uint16_t* src = p.v + (size_t)head * p.N * D;
  const auto rs = make_rsrc(src, (uint32_t)p.N * D * 2u);
  constexpr int kChunks = kTileKeys * D / 8;
#pragma unroll
  for (int i = 0; i < kChunks / 256; ++i) {
    const int id = tid + 256 * i;
    const int rr = id / (D / 8), ch = id % (D / 8);
    *reinterpret_cast<uint4*>(&vt[rr * D + ch * 8]) =
        buf_load16(rs, (uint32_t)((t * kTileKeys + rr) * D + ch * 8) * 2u);
  }
  __syncthreads();
  if (tid < 2 * D) {
    const int c = tid % D, g = tid / D;
    float y[32];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      y[j] = __uint_as_float((uint32_t)vt[(32 * g + j) * D + c] << 16);
      m = fmaxf(m, fabsf(y[j]));
    }
    // E8M0 holds 2^-127 .. 2^127
    const int e = min(max(scale_exponent(m), -127), 127);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      w[i] = pack_e4m3x4(ldexpf(y[4 * i], -e), ldexpf(y[4 * i + 1], -e), ldexpf(y[4 * i + 2], -e),
                         ldexpf(y[4 * i + 3], -e));
    unsigned char* img = p.v8 + ((size_t)head * p.T + t) * (kTileKeys * D);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4*>(img + c * 64 + 16 * ((2 * g + i) ^ vt_swizzle(c))) =
          uint4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
    p.vs[((size_t)head * p.T + t) * 256 + 4 * (32 * g + (c & 31)) + (c >> 5)] =
        (unsigned char)(127 + e);
  }
}

// ---------------------------------------------------------------- forward

struct Fp8Params {
  const unsigned char* q8;
  const float* qs;
  const unsigned char* k8;
  const float* ks;
  const unsigned char* v8;
  const unsigned char* vs;
  void* o;
  float* lse;
  int BH, H, group, N, nqb, T;
  float c;        // |scale| * log2(e)
  int negate_q;   // scale < 0
  int xcd_remap;  // K/V heads grouped per XCD (BH / group % 8 == 0)
  int wl, wr;     // masked kernels: key j visible to query i iff i-wl <= j <= i+wr
};

__device__ __forceinline__ i32x8 lds_ld32(const unsigned char* p0, const unsigned char* p1) {
  const uint4 a = *reinterpret_cast<const uint4*>(p0);
  const uint4 b = *reinterpret_cast<const uint4*>(p1);
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int SEL>
__device__ __forceinline__ f32x16 mfma_fp8_scale_a(i32x8 a, i32x8 b, f32x16 c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SEL, scale_a, 0, 127);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreadsF, 2) void fwd_fp8_kernel(Fp8Params p) {
  constexpr int kTile = kTileKeys * D;               // bytes of one K or V^T tile image
  constexpr int kBlocks = kTile / 1024 / kWavesF;    // 1 KB fill blocks per wave and tensor
  static_assert(kBlocks >= 1 && kTile % (1024 * kWavesF) == 0, "tile must split over the waves");
  __shared__ __attribute__((aligned(1024))) unsigned char k0[kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[kTile];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[kTile];
  constexpr int kKK = D / 64;  // fp8 MFMA steps along d
  constexpr int kDB = D / 32;  // 32-row blocks of O^T

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- (head, query block) of this workgroup: as in the bf16 forward
  // the workgroup's (head, query block) and the key tiles its rows and this
  // wave's rows walk: the bf16 forward's order and ranges (fa_schedule.h),
  // without pairs
  const sched::FwdBlock blk =
      sched::fwd_block(blockIdx.x, p.BH, p.group, p.nqb, p.xcd_remap != 0, CAUSAL, false);
  const int bh = blk.bh;
  const int qb = blk.qb_first;
  const int N = p.N;
  const int kvh = bh / p.group;
  const sched::FwdRange rng =
      sched::fwd_range<kRowsF, 32, kTileKeys>(qb, wave, N, p.wl, p.wr, CAUSAL);
  const int qw0 = rng.qw0;
  const int myq = qw0 + col;
  // keys this lane's row sees: lo_key .. lo_key + n_vis - 1 (masked kernels:
  // i - wl .. i + wr within 0 .. N-1; otherwise 0 .. N-1)
  const int lo_key = CAUSAL ? myq - p.wl : 0;
  const int hi_key = CAUSAL ? min(N - 1, myq + p.wr) : N - 1;
  const uint32_t n_vis = hi_key >= lo_key ? (uint32_t)(hi_key - lo_key + 1) : 0u;

  // ---- Q^T (B operand): lane (h, c) holds row myq, d = 64 kk + 32 h .. +31
  i32x8 qreg[kKK];
  float c_lane;
  {
    const auto qr = make_rsrc(p.q8 + (size_t)bh * N * D, (uint32_t)N * D);
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      const uint32_t off = (uint32_t)(myq * D + 64 * kk + 32 * half);
      uint4 a = buf_load16(qr, off), b = buf_load16(qr, off + 16);
      if (p.negate_q) {
        a.x ^= 0x80808080u; a.y ^= 0x80808080u; a.z ^= 0x80808080u; a.w ^= 0x80808080u;
        b.x ^= 0x80808080u; b.y ^= 0x80808080u; b.z ^= 0x80808080u; b.w ^= 0x80808080u;
      }
      qreg[kk] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    }
    const auto sr = make_rsrc(p.qs + (size_t)bh * N, (uint32_t)N * 4u);
    const float a_i = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sr, (uint32_t)myq * 4u, 0, 0));
    c_lane = p.c * a_i;
  }

  // ---- LDS offsets of this lane's operand reads
  uint32_t koff[2][kKK][2];  // K block kb, step kk, first/second 16 bytes
  {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int r = 32 * kb + 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int ch = 4 * kk + 2 * half + i;
          koff[kb][kk][i] = (uint32_t)(r * D + 16 * (ch ^ k_swizzle<D>(r)));
        }
    }
  }
  uint32_t voff[kDB][2];  // V^T row 32 db + c: keys 16h.. (chunk h), 32+16h.. (chunk 2+h)
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
    const int r = 32 * db + col;
#pragma unroll
    for (int i = 0; i < 2; ++i) voff[db][i] = (uint32_t)(r * 64 + 16 * ((half + 2 * i) ^ vt_swizzle(r)));
  }

  const unsigned char* kimg = p.k8 + (size_t)kvh * p.T * kTile;
  const unsigned char* vimg = p.v8 + (size_t)kvh * p.T * kTile;
  const float* ksc = p.ks + (size_t)kvh * p.T;
  const unsigned char* vsc = p.vs + (size_t)kvh * p.T * 256;

  f32x16 oacc[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) oacc[i] = zero16();
  float m_run = -INFINITY;  // integer-valued reference maximum (log2 units)
  float l_run = 0.0f;
  f32x16 s[2];
  i32x8 pk;

  const int t_first = rng.t_first;
  const int t_end = rng.t_end;
  const int wt_first = rng.wt_first;
  const int wt_end = rng.wt_end;

  auto fill = [&](int t, unsigned char* kd, unsigned char* vd) {
    const auto kr = make_rsrc(kimg + (size_t)t * kTile, kTile);
    const auto vr = make_rsrc(vimg + (size_t)t * kTile, kTile);
#pragma unroll
    for (int i = 0; i < kBlocks; ++i) {
      const int blk = wave * kBlocks + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (FA_LDS void*)(kd + blk * 1024), 16,
                                               (uint32_t)(blk * 1024 + 16 * lane), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (FA_LDS void*)(vd + blk * 1024), 16,
                                               (uint32_t)(blk * 1024 + 16 * lane), 0, 0, 0);
    }
  };
  // scales of tile t: the K tile's (same for every lane) and this lane's V
  // block-scale dword (byte db: column 32 db + c, keys 32 h .. 32 h + 31)
  auto load_scales = [&](int t, float& kscale, int& vscale) {
    kscale = ksc[t];
    vscale = *reinterpret_cast<const int*>(vsc + (size_t)t * 256 + 4 * lane);
  };

  auto qk = [&](const unsigned char* ks) {
    i32x8 a[2][kKK];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) a[kb][kk] = lds_ld32(ks + koff[kb][kk][0], ks + koff[kb][kk][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) s[kb] = mfma_fp8(a[kb][kk], qreg[kk], s[kb]);
    }
  };

  auto pv = [&](const unsigned char* vs_lds, int vscale) {
    i32x8 a[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db) a[db] = lds_ld32(vs_lds + voff[db][0], vs_lds + voff[db][1]);
    static_for<0, kDB>([&](auto db) { oacc[db] = mfma_fp8_scale_a<db>(a[db], pk, oacc[db], vscale); });
  };

  auto softmax = [&](int t, float ct) {
    const int key0 = t * kTileKeys;
    const bool need_mask = sched::fwd_need_mask<kTileKeys>(t, rng, N, p.wl, p.wr, CAUSAL);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kb + 16 * half + r;
          s[kb][r] = in_window(key, lo_key, n_vis) ? s[kb][r] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = halves_max(mx);
    const float cand = mx * ct;
    const bool grow = cand > m_run + kSlack;
    if (__any(grow)) {
      // the reference moves in whole powers of two, so the rescale is exact
      // and keeps the probabilities on the e4m3 grid of 2^8 P
      const float m_new = fmaxf(m_run, ceilf(cand));
      const float alpha = m_new > m_run ? fast_exp2(m_run - m_new) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < kDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      m_run = m_new;
    }
    const float m_sub = (m_run == -INFINITY ? 0.0f : m_run) - kShift;
    float ls0 = 0.0f, ls1 = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e0 = fast_exp2(__builtin_fmaf(s[kb][4 * i], ct, -m_sub));
        const float e1 = fast_exp2(__builtin_fmaf(s[kb][4 * i + 1], ct, -m_sub));
        const float e2 = fast_exp2(__builtin_fmaf(s[kb][4 * i + 2], ct, -m_sub));
        const float e3 = fast_exp2(__builtin_fmaf(s[kb][4 * i + 3], ct, -m_sub));
        ls0 += e0 + e2;
        ls1 += e1 + e3;
        pk[4 * kb + i] = (int)pack_e4m3x4_unclamped(e0, e1, e2, e3);  // p <= 2^8
      }
    l_run += ls0 + ls1;
  };

  float ks_cur = 0.0f, ks_next = 0.0f;
  int vs_cur = 0, vs_next = 0;
  auto step = [&](int t, const unsigned char* kc, const unsigned char* vc, unsigned char* kn,
                  unsigned char* vn) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    ks_cur = ks_next;
    vs_cur = vs_next;
    if (t + 1 < t_end) {
      fill(t + 1, kn, vn);
      load_scales(t + 1, ks_next, vs_next);
    }
    if (t >= wt_first && t < wt_end) {
      const float ct = fmaxf(c_lane * ks_cur, 1e-30f);
      qk(kc);
      softmax(t, ct);
      pv(vc, vs_cur);
    }
  };
  fill(t_first, k0, v0);
  load_scales(t_first, ks_next, vs_next);
  for (int t = t_first; t < t_end; t += 2) {
    step(t, k0, v0, k1, v1);
    if (t + 1 < t_end) step(t + 1, k1, v1, k0, v0);
  }

  // ---- epilogue: O = O_acc / l, lse = (m - kShift + log2 l) ln 2
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (myq < N) {
    uint16_t* og = reinterpret_cast<uint16_t*>(p.o) + (size_t)bh * N * D + (size_t)myq * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * half;
        uint2 w = {pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv),
                   pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        *reinterpret_cast<uint2*>(og + d0) = w;
      }
    if (half == 0)
      p.lse[(size_t)bh * N + myq] =
          l_tot > 0.0f ? (m_run - kShift + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a, const Fp8Layout& ly) {
  Fp8Params p;
  const unsigned char* ws = static_cast<const unsigned char*>(a.workspace);
  p.q8 = ws + ly.q8;
  p.qs = reinterpret_cast<const float*>(ws + ly.qs);
  p.k8 = ws + ly.k8;
  p.ks = reinterpret_cast<const float*>(ws + ly.ks);
  p.v8 = ws + ly.v8;
  p.vs = ws + ly.vs;
  p.o = a.o;
  p.lse = a.lse;
  p.BH = a.B * a.H;
  p.H = a.H;
  p.group = a.H / a.Hkv;
  p.N = a.N;
  p.nqb = (a.N + kRowsF - 1) / kRowsF;
  p.T = (a.N + kTileKeys - 1) / kTileKeys;
  p.c = fmaxf(fabsf(a.scale) * kLog2e, 1e-30f);
  p.negate_q = a.scale < 0.0f;
  p.xcd_remap = (p.BH / p.group) % 8 == 0;
  p.wl = a.wl < 0 ? kUnbounded : a.wl;
  p.wr = a.wr < 0 ? kUnbounded : a.wr;
  dim3 grid((unsigned)((long long)p.BH * p.nqb));
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), grid, dim3(kThreadsF), 0, a.stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prep(const Fp8PrepArgs& a, const Fp8Layout& ly) {
  PrepParams p;
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.q8 = ws + ly.q8;
  p.qs = reinterpret_cast<float*>(ws + ly.qs);
  p.k8 = ws + ly.k8;
  p.ks = reinterpret_cast<float*>(ws + ly.ks);
  p.v8 = ws + ly.v8;
  p.vs = ws + ly.vs;
  for (int i = 0; i < 4; ++i) p.sign_mask[i] = a.sign_mask[i];
  p.rotate = a.rotate;
  p.log2d = D == 128 ? 7 : 6;
  p.BH = a.B * a.H;
  p.BHkv = a.B * a.Hkv;
  p.N = a.N;
  p.T = (a.N + kTileKeys - 1) / kTileKeys;
  dim3 grid((unsigned)fp8_prepare_grid_size(a.B, a.H, a.Hkv, a.N));
  hipLaunchKernelGGL((fp8_prep_kernel<D>), grid, dim3(256), 0, a.stream, p);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

Fp8Layout fp8_layout(int B, int H, int Hkv, int N, int d) {
  const size_t T = (size_t)((N + kTileKeys - 1) / kTileKeys);
  const size_t rows = (size_t)B * H * N, kvt = (size_t)B * Hkv * T;
  Fp8Layout ly;
  size_t off = 0;
  ly.q8 = off; off = align256(off + rows * d);
  ly.qs = off; off = align256(off + rows * sizeof(float));
  ly.k8 = off; off = align256(off + kvt * kTileKeys * d);
  ly.ks = off; off = align256(off + kvt * sizeof(float));
  ly.v8 = off; off = align256(off + kvt * kTileKeys * d);
  ly.vs = off; off = align256(off + kvt * 256);
  ly.bytes = off;
  return ly;
}

long long fp8_prepare_grid_size(int B, int H, int Hkv, int N) {
  const long long T = (N + kTileKeys - 1) / kTileKeys;
  return (long long)B * (H + 2LL * Hkv) * T;
}

hipError_t launch_fp8_prepare(const Fp8PrepArgs& a) {
  const Fp8Layout ly = fp8_layout(a.B, a.H, a.Hkv, a.N, a.d);
  return a.d == 64 ? launch_prep<64>(a, ly) : launch_prep<128>(a, ly);
}

hipError_t launch_forward_fp8(const Fp8FwdArgs& a) {
  const Fp8Layout ly = fp8_layout(a.B, a.H, a.Hkv, a.N, a.d);
  const bool masked = a.wl >= 0 || a.wr >= 0;
  if (a.d == 64) return masked ? launch_fwd_fp8<64, true>(a, ly) : launch_fwd_fp8<64, false>(a, ly);
  return masked ? launch_fwd_fp8<128, true>(a, ly) : launch_fwd_fp8<128, false>(a, ly);
}

}  // namespace fa
