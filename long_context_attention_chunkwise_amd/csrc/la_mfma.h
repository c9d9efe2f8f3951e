// Device helpers shared by the bf16 matrix-core kernels (forward and
// backward): operand types, the 16x16x32 bf16 MFMA, global and LDS loads in
// operand layout, and the LDS transpose load.  Internal to liblightning.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {
namespace mfma16 {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef __bf16 bf16x4 __attribute__((__vector_size__(8)));
typedef short short4v __attribute__((__vector_size__(8)));
typedef float floatx4 __attribute__((__vector_size__(16)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

constexpr int C = 64;          // tokens per block
constexpr int D = 128;         // q/k head size
constexpr int DV = 128;        // v head size
// LDS row pitches (bf16 elements).  K and V tiles are read mostly through the
// transpose load (a half-wave touches 8 consecutive rows x 16 bytes): a
// 288-byte pitch puts those rows on disjoint banks.  The bf16 state is read
// with 16-byte loads of 16 consecutive rows: a 272-byte pitch does the same
// for that pattern.
constexpr int ROWKV = D + 16;
constexpr int ROWST = D + 8;

__device__ __forceinline__ floatx4 mfma(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld_global16(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Streaming (non-temporal) 16-byte load for data read exactly once in whole
// rows (K and V tiles): measured faster on gfx950 than cached loads.  Q is not
// loaded this way: each Q load covers half of a 128-byte line and relies on
// the cache for the other half.
__device__ __forceinline__ uint4 ld_stream16(const uint16_t* p) {
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

__device__ __forceinline__ bf16x8 ld_lds16(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// LDS transpose load: each lane of a 16-lane group passes the address of 4
// consecutive bf16 values; lane i receives column i of the 4 rows the group
// addressed (see tr_operand).
__device__ __forceinline__ bf16x4 ld_lds_tr(const uint16_t* p) {
  lds_short4v* lp = (lds_short4v*)(uint16_t*)p;  // generic -> LDS address space
  short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp);
  return __builtin_bit_cast(bf16x4, r);
}

// Operand of a token-contracting product, from a row-major [token][col] LDS
// tile: lane (l16, grp) gets column col0 + l16 at the eight token slots
//   32p + 4grp + {0..3}  and  32p + 16 + 4grp + {0..3}.
// The same slot order is used for both operands of every such product, and it
// matches the accumulator layout of two vertically adjacent 16x16 P^T tiles.
//
// With cstride = 8 the 16 columns are col0 + 8j + {0..3} for j = 0..3: lane
// l16 gets column col0 + 8(l16/4) + l16%4.  Two such tiles (col0 and col0+4)
// cover 32 consecutive columns so that the accumulator of a product whose rows
// are those columns holds 8 consecutive columns per lane.
//
// `pitch` is the tile's LDS row pitch in elements.
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* tile, int p, int col0, int l16, int grp,
                                             int cstride = 4, int pitch = ROWKV) {
  const int r = 32 * p + 4 * grp + (l16 >> 2);
  const int c = col0 + cstride * (l16 & 3);
  bf16x4 lo = ld_lds_tr(tile + r * pitch + c);
  bf16x4 hi = ld_lds_tr(tile + (r + 16) * pitch + c);
  bf16x8 out;
  for (int i = 0; i < 4; ++i) {
    out[i] = lo[i];
    out[i + 4] = hi[i];
  }
  return out;
}

// DPP control: rotate each 16-lane row right by 8 (row_ror:8).
constexpr int kDppRowRor8 = 0x128;

// Lane l receives x of lane l ^ 8 (the other half of its 16-lane row): a DPP
// row rotation by 8, four 32-bit moves, every row and bank enabled (so no lane
// keeps the `old` operand).
__device__ __forceinline__ bf16x8 swap_row_halves(bf16x8 x) {
  const u32x4 u = __builtin_bit_cast(u32x4, x);
  u32x4 r;
  for (int i = 0; i < 4; ++i)
    r[i] = unsigned(__builtin_amdgcn_update_dpp(0, int(u[i]), kDppRowRor8, 0xF, 0xF, false));
  return __builtin_bit_cast(bf16x8, r);
}

// Operand layout -> whole 128-byte lines.  In operand layout lane (l16, grp)
// holds row l16 of a 16-row tile at two 16-byte pieces of a line: e, piece
// grp, and o, piece grp + 4 of the line's eight.  In line layout it holds
// piece grp + 4 (l16 / 8) of row l16 % 8 (a) and of row 8 + l16 % 8 (b), so
// one 16-byte access per lane covers eight whole lines.
__device__ __forceinline__ void operand_to_lines(bf16x8 e, bf16x8 o, int l16, bf16x8& a, bf16x8& b) {
  const bool lo = l16 < 8;
  const bf16x8 recv = swap_row_halves(lo ? o : e);
  a = lo ? e : recv;
  b = lo ? recv : o;
}

// Stores two packed bf16 output quarters of a 16-row tile, given in operand
// layout (e: row row0 + l16, 8 columns at piece grp of a 128-byte line; od:
// piece grp + 4), as whole lines: rows row0 + l16 % 8 and row0 + 8 + l16 % 8.
// `line` points at the line's first element in row 0, `ld` is the row pitch
// in elements; rows at or past `nrows` are not written.
__device__ __forceinline__ void store_lines(uint16_t* line, int64_t ld, int64_t row0, int64_t nrows, bf16x8 e,
                                            bf16x8 od, int l16, int grp) {
  bf16x8 a, b;
  operand_to_lines(e, od, l16, a, b);
  const int64_t ra = row0 + (l16 & 7), rb = ra + 8;
  uint16_t* p = line + 8 * grp + 32 * (l16 >> 3);
  if (ra < nrows) *reinterpret_cast<bf16x8*>(p + ra * ld) = a;
  if (rb < nrows) *reinterpret_cast<bf16x8*>(p + rb * ld) = b;
}

__device__ __forceinline__ bf16x4 to_bf16x4(floatx4 x) {
  bf16x4 r;
  for (int i = 0; i < 4; ++i) r[i] = (__bf16)x[i];
  return r;
}

__device__ __forceinline__ bf16x8 pack_tiles(floatx4 lo, floatx4 hi) {
  bf16x8 r;
  for (int i = 0; i < 4; ++i) {
    r[i] = (__bf16)lo[i];
    r[i + 4] = (__bf16)hi[i];
  }
  return r;
}

// Feature-map variants (flags of the forward kernels).
constexpr int kRelu = 1;  // phi = ReLU on q and k
constexpr int kNorm = 2;  // outputs divided by phi(q) . z + eps

typedef short short8v __attribute__((ext_vector_type(8)));

// ReLU of eight bf16 values.  A bf16 bit pattern read as int16 is negative
// exactly when its sign bit is set, so max(x, 0) over int16 lanes keeps
// non-negative values and turns negative ones (and -0) into +0: one packed
// 16-bit integer max per register.
__device__ __forceinline__ bf16x8 relu_bf16x8(bf16x8 x) {
  const short8v zero = {0, 0, 0, 0, 0, 0, 0, 0};
  return __builtin_bit_cast(bf16x8, __builtin_elementwise_max(__builtin_bit_cast(short8v, x), zero));
}

__device__ __forceinline__ uint4 relu_bf16x8(uint4 x) {
  const short8v zero = {0, 0, 0, 0, 0, 0, 0, 0};
  return __builtin_bit_cast(uint4, __builtin_elementwise_max(__builtin_bit_cast(short8v, x), zero));
}

__device__ __forceinline__ bf16x8 ones_bf16x8() {
  bf16x8 r;
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)1.0f;
  return r;
}

// Zero the entries of a diagonal P^T tile above the causal boundary: entry
// (s = 4grp + i, t = l16) within the tile is kept when s <= t.
__device__ __forceinline__ floatx4 causal_mask(floatx4 x, int l16, int grp) {
  for (int i = 0; i < 4; ++i)
    if (4 * grp + i > l16) x[i] = 0.0f;
  return x;
}


}  // namespace mfma16
}  // namespace la
