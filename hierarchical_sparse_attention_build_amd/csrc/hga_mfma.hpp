// Matrix-core (MFMA) fragment types and the 16-key block layout shared by the
// prefill attention on the matrix cores and its backward.
//
// v_mfma_f32_32x32x16 (bf16 or fp16 inputs, fp32 accumulate), D = A B with A
// 32 x 16 and B 16 x 32: lane l supplies row l % 32 of A and column l % 32 of
// B, each as the 8 k-values 8 (l / 32) .. 8 (l / 32) + 7; it receives column
// l % 32 of D at rows 8 (i / 4) + 4 (l / 32) + i % 4, i = 0..15.
#pragma once

#include "hga_device.hpp"

namespace hga {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBlk = 16;  // keys per transposed block

// A transposed block holds 16 keys (or query rows) of D dimensions as D runs
// of 16 values, the 16 of a dimension in the order a 32x32x16 fragment reads
// them when the other operand is a D-fragment of the previous product: lane
// half h takes positions 8h..8h+7.  Position p holds key vblock_key(p).
__device__ __forceinline__ int vblock_key(int p) {
  const int h = p >> 3, j = p & 7;
  return 8 * (j >> 2) + 4 * h + (j & 3);
}

// Byte offset of (dimension d, half h) inside a block of 2-byte values; the
// two 16-byte halves of a dimension swap on every other 8 dimensions, so the
// fragment reads of a wave are free of LDS bank conflicts.
__device__ __forceinline__ int vblock_off(int d, int h) {
  return d * 32 + ((h ^ ((d >> 3) & 1)) << 4);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// A 32x32x16 fragment (A or B operand) whose k index runs down 16 rows of a
// row-major bf16 matrix in LDS (row stride rs bytes, a multiple of 8): lane l
// gets column col0 + l % 32 at rows row0 + 8 (s / 4) + 4 (l / 32) + s % 4,
// s = 0..7 -- the row order of a D-fragment (above), so such a fragment
// contracts with one taken from a previous product's result.
//
// ds_read_b64_tr_b16 works on groups of 16 lanes: slot r (0..3) of lane i
// receives 16-bit element i % 4 of the 8 bytes that lane 4 r + i / 4 of the
// group addressed.  Lane s of a group therefore addresses 4 columns
// (4 (s % 4) onwards) of row s / 4 of a 4-row block; two reads, 8 rows apart,
// give the 8 k-values.
__device__ __forceinline__ bf16x8_t lds_frag_tr(const unsigned char* m, int rs, int row0, int col0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = row0 + 4 * (g >> 1) + (s >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
  const unsigned char* p = m + row * rs + col * 2;
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * rs));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8_t, ab);
}

// The same for v_mfma_f32_16x16x32 (16 x 32 A, 32 x 16 B; lane l supplies row
// or column l % 16 with k-values 8 (l / 16) .. + 7; D: lane l holds column
// l % 16 at rows 4 (l / 16) + i, i = 0..3): lane l gets column col0 + l % 16
// at rows row0 + 16 (s / 4) + 4 (l / 16) + s % 4, s = 0..7 -- the rows two
// 16-row D-fragments give one lane.  Lane s of group g addresses row
// row0 + 4 g + s / 4 (and 16 further down), columns col0 + 4 (s % 4) onwards.
__device__ __forceinline__ bf16x8_t lds_frag_tr16(const unsigned char* m, int rs, int row0, int col0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const unsigned char* p = m + (row0 + 4 * g + (s >> 2)) * rs + (col0 + 4 * (s & 3)) * 2;
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 16 * rs));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8_t, ab);
}

}  // namespace hga
