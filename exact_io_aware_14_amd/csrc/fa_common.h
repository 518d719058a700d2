// Device-side helpers shared by the gfx950 attention kernels.
//
// Register layouts of the bf16 MFMA 32x32x16 instruction used throughout
// (wave64; lane l, half h = l / 32, column c = l % 32):
//   A operand (32 x 16, 8 bf16 per lane): row c, k-slots 8h .. 8h+7
//   B operand (16 x 32, 8 bf16 per lane): column c, k-slots 8h .. 8h+7
//   C/D accumulator (32 x 32, 16 fp32 per lane): column c, element r holds
//     row 8*(r/4) + 4h + (r%4).
// Which k a slot stands for never matters as long as the A and B operands of
// one instruction use the same slot-to-k assignment; the kernels choose that
// assignment so that an accumulator can be repacked as the next operand
// inside its own lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Round two fp32 values to bf16 (nearest even) and pack them in one dword,
// the first value in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 as_u4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes from `base` (raw, unstrided). Loads at
// byte offsets at or past `bytes` return zeros, which is how rows past the
// end of a sequence are zero-filled without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return uint4{v[0], v[1], v[2], v[3]};
}

// Eight consecutive elements starting at element `elem` of a buffer, as
// eight bf16 in a uint4. Storage type bf16 (uint16_t) is loaded as is; fp32
// is rounded to nearest even. Past the end of the buffer: zeros.
template <typename T>
__device__ __forceinline__ uint4 load8(__amdgpu_buffer_rsrc_t r, uint32_t elem);

template <>
__device__ __forceinline__ uint4 load8<uint16_t>(__amdgpu_buffer_rsrc_t r, uint32_t elem) {
  return buf_load16(r, elem * 2u);
}

template <>
__device__ __forceinline__ uint4 load8<float>(__amdgpu_buffer_rsrc_t r, uint32_t elem) {
  const uint4 a = buf_load16(r, elem * 4u);
  const uint4 b = buf_load16(r, elem * 4u + 16u);
  uint4 out;
  out.x = pack_bf16x2(__uint_as_float(a.x), __uint_as_float(a.y));
  out.y = pack_bf16x2(__uint_as_float(a.z), __uint_as_float(a.w));
  out.z = pack_bf16x2(__uint_as_float(b.x), __uint_as_float(b.y));
  out.w = pack_bf16x2(__uint_as_float(b.z), __uint_as_float(b.w));
  return out;
}

// Flip the sign of eight packed bf16 values (exact).
__device__ __forceinline__ uint4 negate8(uint4 u) {
  u.x ^= 0x80008000u;
  u.y ^= 0x80008000u;
  u.z ^= 0x80008000u;
  u.w ^= 0x80008000u;
  return u;
}

// Maximum and sum of x over lanes l and l ^ 32 (the two halves of the
// wave), in every lane. v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second; with x in both, lane l of
// the results holds (x[l], x[l+32]) in the lower half and (x[l-32], x[l]) in
// the upper half: the low-half value first in both, so the two halves add in
// the same order and agree bitwise.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// LDS tiles. A tile of R rows x D columns of bf16 is kept in one of two forms:
//
// * row-major [row][d]: the 16-byte chunk c of row r sits at chunk position
//   c ^ rsw(r). The LDS serves 16 lanes of a 16-byte read per clock from 64
//   banks (256 bytes), and an MFMA operand read has 16 consecutive rows per
//   clock reading the same chunk c: rsw spreads those 16 reads over all 256
//   bytes (d = 128: a row is 256 bytes, rsw = r & 15; d = 64: a row is 128
//   bytes, r & 1 picks the half, rsw = (r >> 1) & 7 the chunk);
// * transposed [d][pos(row)]: each LDS row holds one column d of the tile.
//   Rows are stored at position pos(r), r with bits 2 and 3 swapped, which
//   makes the eight rows one lane needs for one MFMA operand (see below)
//   contiguous. Chunks are XOR-swizzled by (d ^ d/8) & 7: the 32 lanes of a
//   read cover 32 consecutive columns d (distinct d & 7 within every 8
//   lanes), while the 16 lanes of a transposing store cover columns 8 apart
//   (distinct d/8), so neither direction piles onto one bank.
//
// Why the swap: an accumulator element r of the 32x32 MFMA covers row
// 8*(r/4) + 4h + (r%4) of its 32-row block. Repacking accumulator elements
// 8m .. 8m+7 of a lane as the operand slots of one 16-deep MFMA makes slot s
// stand for row 16m + 8*(s/4) + 4h + (s%4); with bits 2 and 3 swapped that
// is position 16m + 8h + s, one 16-byte chunk per lane.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int tpos(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Chunk swizzle of column d of a transposed tile.
__device__ __forceinline__ int tsw(int d) { return (d ^ (d >> 3)) & 7; }

// Chunk swizzle of row r of a row-major tile of width D. It serves both
// read patterns used on these tiles:
//   (a) an MFMA operand read: 16 consecutive rows (a multiple of 16 first),
//       the same 16-byte chunk -> 16 distinct positions of the 256 bytes;
//   (b) a transposing read (below): 4 consecutive rows (a multiple of 4
//       first) x 4 consecutive chunks (a multiple of 4 first) -> 16
//       distinct positions.
// d = 128 (256-byte rows): bits 2-3 of the swizzle come from r & 3 (they
// separate the rows of (b) while the chunk varies bits 0-1) and bits 0-1
// from (r >> 2) & 3, completing (a). d = 64 (128-byte rows, r & 1 picks the
// half of the bank space): bit 2 from (r >> 1) & 1, bits 0-1 from (r >> 2) & 3.
// d = 256 (512-byte rows, two 256-byte bank spans): the d = 128 swizzle; it
// changes only the low four bits of a chunk index, so chunk 16 + c of a row
// sits exactly 256 bytes after chunk c.
template <int D>
__device__ __forceinline__ int rsw(int r) {
  static_assert(D == 64 || D == 128 || D == 256, "tile width");
  return D >= 128 ? (4 * (r & 3) + ((r >> 2) & 3)) : (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
}

// Store chunk `ch` (8 elements) of row `row` into a row-major tile of width D.
template <int D>
__device__ __forceinline__ void st_row(uint16_t* tile, int row, int ch, uint4 val) {
  *reinterpret_cast<uint4*>(&tile[row * D + ((ch ^ rsw<D>(row)) * 8)]) = val;
}

// MFMA operand read: chunk `ch` of row `row` of a row-major tile.
template <int D>
__device__ __forceinline__ bf16x8 ld_row(const uint16_t* tile, int row, int ch) {
  return *reinterpret_cast<const bf16x8*>(&tile[row * D + ((ch ^ rsw<D>(row)) * 8)]);
}

// Store four consecutive rows r0..r0+3 (r0 % 4 == 0) of chunk `ch` (columns
// 8ch..8ch+7) into a transposed tile of R rows: eight 8-byte writes.
template <int R>
__device__ __forceinline__ void st_tr4(uint16_t* tile, int r0, int ch, const uint4 w[4]) {
  const int pos = tpos(r0);  // the four rows stay adjacent: bits 0-1 unchanged
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&w[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&w[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&w[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&w[3]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint2 lo, hi;  // column 8ch+2j from the low halves, 8ch+2j+1 from the high halves
    lo.x = (w0[j] & 0xffffu) | (w1[j] << 16);
    lo.y = (w2[j] & 0xffffu) | (w3[j] << 16);
    hi.x = (w0[j] >> 16) | (w1[j] & 0xffff0000u);
    hi.y = (w2[j] >> 16) | (w3[j] & 0xffff0000u);
    const int d0 = ch * 8 + 2 * j, d1 = d0 + 1;
    *reinterpret_cast<uint2*>(&tile[d0 * R + (((pos >> 3) ^ tsw(d0)) * 8) + (pos & 7)]) = lo;
    *reinterpret_cast<uint2*>(&tile[d1 * R + (((pos >> 3) ^ tsw(d1)) * 8) + (pos & 7)]) = hi;
  }
}

// ---------------------------------------------------------------------------
// Row-major tiles read through the transposing LDS read. ds_read_b64_tr_b16
// works on groups of 16 lanes: lane j of a group points at 4 consecutive
// bf16 (a "row" of 4), and lane i of the group receives element i % 4 of the
// rows pointed at by lanes i/4, i/4+4, i/4+8 and i/4+12. With lane j pointing
// at tile row k0 + j/4, columns d0 + 4*(j%4) .. +3, lane i receives column
// d0 + i of rows k0 .. k0+3: four consecutive tile rows of one column, which
// is an MFMA operand whose k-slots run along the tile rows.
//
// These tiles use the same swizzle rsw as MFMA row reads. Shifting the row by
// a multiple of 16 keeps rsw; within ld_rows_t the second read's rows are 8
// further on, which rows_t_offset accounts for.
// ---------------------------------------------------------------------------

#define FA_LDS __attribute__((address_space(3)))

// Masks with one unsigned compare: x lies in lo .. lo+count-1 iff
// (unsigned)(x - lo) < count, since values below lo wrap to numbers at least
// 2^31 (|x - lo| stays below 2^31 for the bounds used here).
__device__ __forceinline__ bool in_window(int x, int lo, uint32_t count) {
  return (uint32_t)(x - lo) < count;
}

// Scan of the nonzero entries of a block-sparse mask along one row (stride
// 1) or one column (stride nb): entries a[i * stride], i < n, and optionally
// a second sequence b alike (nullptr: none). It reads 64 entries at a time,
// one byte per lane, and keeps them as two 64-bit ballots, so the search is
// scalar; every wave of a workgroup scans the same bytes and finds the same
// entries.
struct MaskScan {
  const uint8_t* a;
  const uint8_t* b;
  uint32_t stride;
  int n;
  int chunk;  // entries 64*chunk .. 64*chunk+63 are in bits_a, bits_b
  uint64_t bits_a, bits_b;

  __device__ __forceinline__ void reset(const uint8_t* a_, const uint8_t* b_) {
    a = a_;
    b = b_;
    chunk = -1;
  }
  // The first i' >= i where a or b is nonzero, else n; *flags gets bit 0 for
  // a[i'] != 0 and bit 1 for b[i'] != 0.
  __device__ __forceinline__ int next(int i, int lane, uint32_t* flags) {
    while (i < n) {
      const int c = i >> 6;
      if (c != chunk) {
        chunk = c;
        const int j = (c << 6) + lane;
        const size_t off = (size_t)j * stride;
        bits_a = __ballot(j < n && a[off] != 0);
        bits_b = b == nullptr ? 0ull : __ballot(j < n && b[off] != 0);
      }
      const uint64_t ra = bits_a >> (i & 63), rb = bits_b >> (i & 63);
      if ((ra | rb) != 0) {
        const int k = __builtin_ctzll(ra | rb);
        *flags = (uint32_t)((ra >> k) & 1) | (uint32_t)(((rb >> k) & 1) << 1);
        return i + k;
      }
      i = (c + 1) << 6;
    }
    *flags = 0;
    return n;
  }
};

// Integer division rounding toward -infinity / +infinity (b > 0).
__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((b - 1 - a) / b); }
__device__ __forceinline__ int ceil_div(int a, int b) { return -floor_div(-a, b); }

__device__ __forceinline__ bf16x4 tr_read(const uint16_t* p) {
  typedef __bf16 v4bf __attribute__((__vector_size__(4 * sizeof(__bf16))));
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                        (FA_LDS v4bf*)(const_cast<uint16_t*>(p))));
}

// Byte offset, within a row-major tile of width D read through tr_read, of
// this lane's pointer for read `rd` (0: k-slots 0-3, 1: k-slots 4-7) of the
// MFMA operand of ld_rows_t with kbase = 0 and d-block db. A kbase that is a
// multiple of 16 adds kbase rows (rsw repeats every 16 rows).
template <int D>
__device__ __forceinline__ uint32_t rows_t_offset(int db, int rd, int lane) {
  const int g = lane >> 4, j = lane & 15, h = lane >> 5;
  const int d0 = db * 32 + 16 * (g & 1) + 4 * (j & 3);
  const int r = 4 * h + (j >> 2) + 8 * rd;
  return (uint32_t)(r * D + (((d0 >> 3) ^ rsw<D>(r)) << 3) + (d0 & 7)) * 2u;
}

// Byte offset, within a row-major tile of width D (swizzle rsw), of chunk ch
// of row `row`.
template <int D>
__device__ __forceinline__ uint32_t row_offset(int row, int ch) {
  return (uint32_t)(row * D + ((ch ^ rsw<D>(row)) << 3)) * 2u;
}

__device__ __forceinline__ bf16x8 lds_ld16(const unsigned char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Two transposing reads form one operand (slots 0-3 from p0, 4-7 from p1).
__device__ __forceinline__ bf16x8 lds_tr_pair(const unsigned char* p0, const unsigned char* p1) {
  const bf16x4 a = tr_read(reinterpret_cast<const uint16_t*>(p0));
  const bf16x4 b = tr_read(reinterpret_cast<const uint16_t*>(p1));
  bf16x8 v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}

// MFMA operand from a row-major tile (swizzle rsw) whose k-slots run along
// the tile rows: lane (h, c) gets column 32*db + c, and slot s stands for tile
// row kbase + 8*(s/4) + 4h + (s%4) -- the row order of the repacked
// accumulator (see above), so P^T or dS^T built from an accumulator pairs
// with it slot for slot.
template <int D>
__device__ __forceinline__ bf16x8 ld_rows_t(const uint16_t* tile, int kbase, int db, int lane) {
  const int g = lane >> 4, j = lane & 15, h = lane >> 5;
  const int d0 = db * 32 + 16 * (g & 1) + 4 * (j & 3);
  const int r0 = kbase + 4 * h + (j >> 2);
  const int r1 = r0 + 8;
  const bf16x4 a = tr_read(tile + r0 * D + (((d0 >> 3) ^ rsw<D>(r0)) << 3) + (d0 & 7));
  const bf16x4 b = tr_read(tile + r1 * D + (((d0 >> 3) ^ rsw<D>(r1)) << 3) + (d0 & 7));
  bf16x8 v;
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
  v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
  return v;
}

// Fill ROWS rows of a row-major bf16 tile (width D) straight from global
// memory into LDS, 16 bytes per lane, with no registers in between: each of
// the WAVES waves moves whole 1 KB blocks (one buffer_load ... lds each); the
// swizzle is applied on the global side (lane l of a block takes the chunk
// that belongs at LDS position 16*l). `r` views the rows from the tile's
// first row on; rows past its end are written as zeros. `wave` must be
// wave-uniform.
template <int D, int ROWS, int WAVES>
__device__ __forceinline__ uint32_t fill_lane_offset(int i, int wave, int lane) {
  constexpr int kRowBytes = D * 2;
  constexpr int kPerWave = ROWS * kRowBytes / 1024 / WAVES;
  constexpr int kRowsPerBlock = 1024 / kRowBytes;
  const int b = wave * kPerWave + i;
  const int row = b * kRowsPerBlock + (lane * 16) / kRowBytes;
  const int pos = ((lane * 16) % kRowBytes) / 16;
  const int ch = pos ^ rsw<D>(row);
  return (uint32_t)(row * kRowBytes + ch * 16);
}

template <int D, int ROWS, int WAVES>
__device__ __forceinline__ void fill_direct(unsigned char* tile, __amdgpu_buffer_rsrc_t r,
                                            const uint32_t* lane_off, int wave) {
  constexpr int kPerWave = ROWS * D * 2 / 1024 / WAVES;
  static_assert(ROWS * D * 2 % (1024 * WAVES) == 0, "blocks must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < kPerWave; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (FA_LDS void*)(tile + (wave * kPerWave + i) * 1024), 16, lane_off[i], 0, 0, 0);
}

// The same tile filled through registers from fp32 rows (rounded to bf16).
template <int D, int ROWS, int THREADS>
__device__ __forceinline__ void fill_f32(uint16_t* tile, __amdgpu_buffer_rsrc_t r, int row0,
                                         int tid) {
  constexpr int kChunks = D / 8;
  static_assert(ROWS * kChunks % THREADS == 0, "chunks must split evenly");
#pragma unroll
  for (int i = 0; i < ROWS * kChunks / THREADS; ++i) {
    const int id = tid + i * THREADS;
    const int row = id / kChunks, ch = id % kChunks;
    const uint4 val = load8<float>(r, (uint32_t)((row0 + row) * D + ch * 8));
    const int pos = ch ^ rsw<D>(row);
    *reinterpret_cast<uint4*>(&tile[row * D + pos * 8]) = val;
  }
}

// MFMA operand read from a transposed tile of R rows: column `d`, positions
// 8*chunk .. 8*chunk+7.
template <int R>
__device__ __forceinline__ bf16x8 ld_tr(const uint16_t* tile, int d, int chunk) {
  return *reinterpret_cast<const bf16x8*>(&tile[d * R + ((chunk ^ tsw(d)) * 8)]);
}

}  // namespace fa
