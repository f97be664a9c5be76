// Device-side building blocks for the gfx950 (CDNA4) attention kernels.
//
// Matrix-core conventions used throughout (wave64, v_mfma_f32_32x32x16_{f16,bf16}):
//   A operand (32 x 16): lane l holds A[m = l % 32][k = 8 * (l / 32) + i], i = 0..7
//   B operand (16 x 32): lane l holds B[k = 8 * (l / 32) + i][n = l % 32]
//   C/D       (32 x 32): lane l, register r holds C[m = mrow(l, r)][n = l % 32]
//                        with mrow(l, r) = 8 * (r / 4) + 4 * (l / 32) + r % 4.
// Because the contraction index k is summed, any relabelling of k that the A and
// B operands share gives the same product; the kernels use this freedom so that
// an accumulator can feed the next product as a B operand without leaving
// registers (its row index m becomes the contraction index).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((__vector_size__(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct F16 {
  using T = _Float16;
  using V8 = f16x8;
  static __device__ __forceinline__ f32x16 mma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
struct BF16 {
  using T = __bf16;
  using V8 = bf16x8;
  static __device__ __forceinline__ f32x16 mma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ int mrow(int g, int r) { return 8 * (r >> 2) + 4 * g + (r & 3); }

template <class DT>
__device__ __forceinline__ typename DT::V8 as_v8(u32x4 x) {
  return __builtin_bit_cast(typename DT::V8, x);
}
template <class DT>
__device__ __forceinline__ typename DT::V8 as_v8(u32x2 lo, u32x2 hi) {
  u32x4 x = {lo.x, lo.y, hi.x, hi.y};
  return __builtin_bit_cast(typename DT::V8, x);
}

// Round-to-nearest-even conversion of 8 fp32 values into one operand register set.
template <class DT>
__device__ __forceinline__ typename DT::V8 pack8(float a0, float a1, float a2, float a3,
                                                 float a4, float a5, float a6, float a7) {
  typename DT::V8 v;
  v[0] = (typename DT::T)a0; v[1] = (typename DT::T)a1; v[2] = (typename DT::T)a2; v[3] = (typename DT::T)a3;
  v[4] = (typename DT::T)a4; v[5] = (typename DT::T)a5; v[6] = (typename DT::T)a6; v[7] = (typename DT::T)a7;
  return v;
}

// Four fp32 values -> four 16-bit values packed in 8 bytes (RNE).
template <class DT>
__device__ __forceinline__ u32x2 pack4(float a0, float a1, float a2, float a3) {
  typedef typename DT::T T;
  typedef T T4 __attribute__((ext_vector_type(4)));
  T4 v;
  v[0] = (T)a0; v[1] = (T)a1; v[2] = (T)a2; v[3] = (T)a3;
  return __builtin_bit_cast(u32x2, v);
}

// ---------------------------------------------------------------------------
// LDS tiles: rows of ROW_BYTES bytes, stored with a per-row XOR swizzle of the
// 16-byte chunks so that 16 consecutive rows read at one column hit 16
// distinct 16-byte bank groups (64 banks x 4 bytes).
// ---------------------------------------------------------------------------
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int row) {
  constexpr int CPR = ROW_BYTES / 16;
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "row length");
  if constexpr (CPR == 16) return row & 15;
  else if constexpr (CPR == 8) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
// Byte offset of element column `col` (16-bit elements) of row `row`.
template <int ROW_BYTES>
__device__ __forceinline__ int tile_off(int row, int col) {
  int chunk = col >> 3;
  return row * ROW_BYTES + ((chunk ^ swz<ROW_BYTES>(row)) << 4) + ((col & 7) << 1);
}

__device__ __forceinline__ u32x4 lds_read16(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(char* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}
__device__ __forceinline__ void lds_write8(char* base, int off, u32x2 v) {
  *reinterpret_cast<u32x2*>(base + off) = v;
}

// gfx950 LDS transpose read. Within each group of 16 lanes, lane t supplies the
// address of four consecutive 16-bit elements of row t/4 (columns 4*(t%4)..+3)
// of a 4 x 16 block; lane t receives column t of that block (rows 0..3).
__device__ __forceinline__ u32x2 lds_read_tr(const char* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Operand with 8 contraction slots taken from rows {rb+0..3, rb+8..11} (or
// {rb+0..3, rb+4..7} when STEP == 4) of a row-major LDS tile, at column
// `colbase + (lane % 32)`. Rows are the contraction index, columns the free index.
template <class DT, int ROW_BYTES, int STEP>
__device__ __forceinline__ typename DT::V8 tr_operand(const char* tile, int rb, int colbase, int lane) {
  const int t = lane & 15;
  const int col = colbase + (lane & 16) + 4 * (t & 3);
  const int row = rb + (t >> 2);
  u32x2 lo = lds_read_tr(tile + tile_off<ROW_BYTES>(row, col));
  u32x2 hi = lds_read_tr(tile + tile_off<ROW_BYTES>(row + STEP, col));
  return as_v8<DT>(lo, hi);
}

// ---------------------------------------------------------------------------
// Work-group ordering: workgroups are handed to the 8 XCDs round-robin, so the
// hardware id is remapped to give each XCD a contiguous run of logical blocks
// (neighbouring tiles of one head then share that XCD's L2).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int hw, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = hw & 7, idx = hw >> 3;
  return x * per + (x < rem ? x : rem) + idx;
}

__device__ __forceinline__ float wave_max_pair(float x) {
  // lanes l and l ^ 32 hold the two halves of one row
  return fmaxf(x, __shfl_xor(x, 32));
}

}  // namespace fa
