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

#include <type_traits>

#include "fa_launch.h"

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
// Largest N d of a dense head whose causal grid runs ranked (xcd_remap_ranked).
constexpr long long kRankedMaxNd = 1ll << 19;
// The 8-wave (256-row) forward and dQ workgroups are used when there are at least
// this many of them, one per compute unit; smaller grids run twice as many 4-wave
// workgroups instead.
constexpr long long kWideMinBlocks = 256;

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
// LDS tiles: rows of ROW_BYTES (128 or 256) bytes whose 16-byte chunks are
// permuted per row: chunk c of row r sits in slot c ^ h(r). gfx950 LDS serves
// 256 bytes per clock from 64 four-byte banks, i.e. 16 slots of 16 bytes; the
// permutation makes the two access shapes the kernels use conflict-free:
//   * operand reads (ds_read_b128): 16 lanes read one chunk column of 16
//     consecutive rows -> 16 distinct slots;
//   * transpose reads (ds_read_b64_tr_b16): 32 lanes read 4 consecutive rows
//     (aligned to 4) x 4 adjacent chunks (aligned to 4) -> 16 distinct slots.
//   256-byte rows: h(r) = 4 (r mod 4) + (r / 4 mod 4)
//   128-byte rows: h(r) = 4 (r / 2 mod 2) + (r / 4 mod 4)   (odd rows start at slot 8)
// h repeats every 16 rows, so offsets of rows 16 apart differ by a constant.
// ---------------------------------------------------------------------------
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int row) {
  static_assert(ROW_BYTES == 128 || ROW_BYTES == 256, "row length");
  if constexpr (ROW_BYTES == 256) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Byte offset of 16-bit element column `col` of row `row`.
template <int ROW_BYTES>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * ROW_BYTES + (((col >> 3) ^ swz<ROW_BYTES>(row)) << 4) + ((col & 7) << 1);
}

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
__device__ __forceinline__ u32x4 lds_read16(const char* base, int off) {
  return *(const lds_u32x4*)((const __attribute__((address_space(3))) char*)(base) + off);
}
__device__ __forceinline__ void lds_write16(char* base, int off, u32x4 v) {
  *(lds_u32x4*)((__attribute__((address_space(3))) char*)(base) + off) = v;
}
__device__ __forceinline__ void lds_write8(char* base, int off, u32x2 v) {
  *(lds_u32x2*)((__attribute__((address_space(3))) char*)(base) + off) = v;
}

// gfx950 LDS transpose read. Within each group of 16 lanes, lane t supplies the
// address of four consecutive 16-bit elements of row t/4 (columns 4*(t%4)..+3)
// of a 4 x 16 block; lane t receives column t of that block (rows 0..3).
// The address is formed in the LDS address space so that constant parts of
// the offset fold into the instruction's immediate field.
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ const lds_char* to_lds(const char* p) { return (const lds_char*)(p); }
__device__ __forceinline__ u32x2 lds_read_tr(const char* base, int off) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(to_lds(base) + off));
  return __builtin_bit_cast(u32x2, v);
}

// Lane-dependent part of a transpose-read operand address. The lane reads
// row row0 + (lane % 16) / 4 at columns colbase + (lane & 16) + 4 (lane % 4).
template <int ROW_BYTES>
__device__ __forceinline__ int tr_off(int row0, int colbase, int lane) {
  const int t = lane & 15;
  return tile_off<ROW_BYTES>(row0 + (t >> 2), colbase + (lane & 16) + 4 * (t & 3));
}

// Operand with 8 contraction slots from two transpose reads (two blocks of 4
// rows) at byte offsets off_lo and off_hi.
template <class DT>
__device__ __forceinline__ typename DT::V8 tr_pair(const char* tile, int off_lo, int off_hi) {
  u32x2 lo = lds_read_tr(tile, off_lo);
  u32x2 hi = lds_read_tr(tile, off_hi);
  return as_v8<DT>(lo, hi);
}

// The same transpose read issued as inline assembly with a compile-time byte
// offset. The compiler makes every LDS access that it cannot prove disjoint
// from an outstanding HBM -> LDS tile copy wait for all copies (the builtin
// above is one); these reads are outside its view, so a copy into the other
// buffer stays in flight. Their results are valid only after lds_wait_tie2().
__device__ __forceinline__ uint32_t lds_addr(const char* p) { return (uint32_t)(size_t)to_lds(p); }
template <int OFF>
__device__ __forceinline__ u32x2 tr_read_imm(uint32_t vaddr) {
  static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS offset field");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(vaddr), "n"(OFF));
  return r;
}
template <class DT, int OFF>
__device__ __forceinline__ typename DT::V8 tr_pair_imm(uint32_t a_lo, uint32_t a_hi) {
  const u32x2 lo = tr_read_imm<OFF>(a_lo);
  const u32x2 hi = tr_read_imm<OFF>(a_hi);
  return as_v8<DT>(lo, hi);
}
// A 16-byte LDS read issued as inline assembly with a compile-time byte offset
// (outside the compiler's view, like tr_read_imm); valid after lds_wait_n().
template <int OFF>
__device__ __forceinline__ u32x4 rd128_imm(uint32_t vaddr) {
  static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS offset field");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(vaddr), "n"(OFF));
  return r;
}
// Wait until at most N LDS operations of this wave are outstanding. LDS
// operations complete in issue order, so every read issued more than N LDS
// operations ago has its result; the operands are tied through the wait so
// that no use of them is scheduled before it.
template <int N, class V>
__device__ __forceinline__ void lds_wait_n(V& a) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}
template <int N, class V>
__device__ __forceinline__ void lds_wait_n4(V& a, V& b, V& c, V& d) {
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "n"(N));
}
// Wait for every outstanding LDS read of this wave; the operands are tied
// through the wait so that no use of them is scheduled before it.
template <class V>
__device__ __forceinline__ void lds_wait_tie2(V& a, V& b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b));
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [I0, N).
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// ---------------------------------------------------------------------------
// Buffer resources: 128-bit descriptors (base, byte range) held in SGPRs.
// Loads past the range return zero, which takes care of ragged tails without
// per-element branches.
// ---------------------------------------------------------------------------
constexpr int kBufferRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferRsrcWord3);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// ---------------------------------------------------------------------------
// Asynchronous tile copy HBM -> LDS (buffer_load_dwordx4 ... lds). Each wave
// instruction fills 1 KB of LDS: lane i's 16 bytes land at the wave's LDS
// address + 16 i. A lane therefore fetches the global chunk that belongs at
// its LDS slot under the row permutation; rows past the buffer range arrive as
// zeros. Global rows are row_stride bytes apart (the row length for a dense
// head, heads x row length for a token-major packed tensor). A wave's
// successive kilobytes are NW KB of LDS apart, a whole number of swizzle
// periods, so one lane offset plus a fixed step serves every chunk.
// Completion is tracked by vmcnt: wait_tile_copies() before the barrier that
// publishes the tile.
// ---------------------------------------------------------------------------
template <int ROW_BYTES, int TILE_BYTES, int NW>
struct TileCopy {
  static constexpr int PER_WAVE = TILE_BYTES / (1024 * NW);
  static_assert(PER_WAVE * 1024 * NW == TILE_BYTES, "tile is a whole number of wave kilobytes");
  static_assert(((1024 * NW) / ROW_BYTES) % 16 == 0, "successive kilobytes are whole swizzle periods apart");
  int goff;    // lane's global byte offset from the tile's first row, for its first kilobyte
  int ustep;   // global byte step between this wave's successive kilobytes
  int wave;    // wave index (uniform)
  __device__ __forceinline__ TileCopy(int wave_, int lane, int row_stride) {
    wave = __builtin_amdgcn_readfirstlane(wave_);
    const int p = 1024 * wave + 16 * lane;
    const int row = p / ROW_BYTES, slot = (p % ROW_BYTES) / 16;
    goff = row * row_stride + ((slot ^ swz<ROW_BYTES>(row)) << 4);
    ustep = (NW * 1024 / ROW_BYTES) * row_stride;
  }
  // kilobyte u (0 <= u < PER_WAVE) of this wave's share only; gbase = byte
  // offset of the tile's first row
  __device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t rs, char* tile, int gbase, int u) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(tile + 1024 * (wave + NW * u)), 16,
        goff + gbase + u * ustep, 0, 0, 0);
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* tile, int gbase) const {
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) issue_one(rs, tile, gbase, u);
  }
};

// ---------------------------------------------------------------------------
// Rows of one (sequence, head): element offsets of row 0 in q/o, k/v and lse/D,
// row counts and row strides, for the dense and the packed layouts.
// ---------------------------------------------------------------------------
struct HeadView {
  size_t q_off, kv_off, stat_off;
  int lq, lk;                                  // query / key rows (lq <= N, lk <= Nk)
  int q_stride, kv_stride, stat_stride;        // elements between consecutive rows
  size_t q_hstep, stat_hstep;                  // offset step to the next query head (same sequence)
};
__device__ __forceinline__ HeadView head_view(const SeqLayout& L, int b, int h, int H, int N, int D) {
  HeadView v;
  const int hk = h / (H / L.Hk);              // key/value head read by query head h
  if (L.cu_q == nullptr) {
    v.lq = N;
    v.lk = L.Nk;
    v.q_off = ((size_t)b * H + h) * (size_t)N * D;
    v.kv_off = ((size_t)b * L.Hk + hk) * (size_t)L.Nk * D;
    v.stat_off = ((size_t)b * H + h) * (size_t)N;
    v.q_stride = D;
    v.kv_stride = D;
    v.stat_stride = 1;
    v.q_hstep = (size_t)N * D;
    v.stat_hstep = (size_t)N;
  } else {
    const int sq = min(max(L.cu_q[b], 0), L.total_q);
    const int eq = min(max(L.cu_q[b + 1], sq), L.total_q);
    const int sk = min(max(L.cu_k[b], 0), L.total_k);
    const int ek = min(max(L.cu_k[b + 1], sk), L.total_k);
    v.lq = min(eq - sq, N);                    // rows past the stated maximum are not computed
    v.lk = min(ek - sk, L.Nk);
    v.q_off = ((size_t)sq * H + h) * D;
    v.kv_off = ((size_t)sk * L.Hk + hk) * D;
    v.stat_off = (size_t)sq * H + h;
    v.q_stride = H * D;
    v.kv_stride = L.Hk * D;
    v.stat_stride = H;
    v.q_hstep = (size_t)D;
    v.stat_hstep = 1;
  }
  return v;
}
// Byte range of `rows` rows of `width` elements, `stride` elements apart.
__device__ __forceinline__ uint32_t span_bytes(int rows, int stride, int width, int elem_bytes) {
  return rows > 0 ? (uint32_t)(((size_t)(rows - 1) * stride + width) * elem_bytes) : 0u;
}

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): ten rounds of two 32 x 32 -> 64-bit products and a
// word permutation with xors of the key, the key advanced by a Weyl sequence
// between rounds. Counter-based: the dropout mask is a pure function of
// (counter, key), so the backward regenerates the forward's mask.
// ---------------------------------------------------------------------------
// a ^ b ^ k in one instruction (gfx950 three-input bitwise op, truth table 0x96);
// k is uniform (a key word)
__device__ __forceinline__ uint32_t xor3_key(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // the key schedule is uniform: advance it in scalar registers each round
    // (hoisted out of the tile loop, its 20 words were kept in vector lanes)
    asm volatile("" : "+s"(k0), "+s"(k1));
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = xor3_key((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3_key((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return u32x4{c0, c1, c2, c3};
}
// One generator call decides a block of 2 queries x 4 keys: element (query
// 2 r + h, key 4 c + u) of head bh is kept iff the 16-bit half h (0 = low) of
// word u is >= threshold (= floor(p 2^16)). Returns the eight keep bits, bit
// 4 h + u.
__device__ __forceinline__ uint32_t keep8(const Dropout& dr, uint32_t c, uint32_t r, uint32_t bh) {
  const u32x4 w = philox4x32_10(c, r, bh, dr.offset, dr.seed_lo, dr.seed_hi);
  uint32_t b = 0u;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    b |= (uint32_t)((w[u] & 0xFFFFu) >= dr.threshold) << u;
    b |= (uint32_t)((w[u] >> 16) >= dr.threshold) << (4 + u);
  }
  return b;
}

// Keep bits of the 16 elements a lane holds in a query-per-lane accumulator
// (forward, dQ): query i (i mod 2 = lane mod 2), keys 4 (c0 + 2 j + g) + u for
// j, u in 0..3 (g = lane / 32), as bit 4 j + u. Lanes 2a and 2a + 1 hold the two
// queries of one generator row pair: each draws two of the four blocks (j = its
// parity and j + 2) and the pair swaps the nibbles that belong to the other query.
__device__ __forceinline__ uint32_t keep16_pair(const Dropout& dr, uint32_t c0, uint32_t i, uint32_t bh, int lane) {
  const uint32_t odd = (uint32_t)lane & 1u, g = ((uint32_t)lane >> 5) & 1u;
  const uint32_t b0 = keep8(dr, c0 + 2u * odd + g, i >> 1, bh);        // block j = odd
  const uint32_t b1 = keep8(dr, c0 + 2u * (odd + 2u) + g, i >> 1, bh); // block j = odd + 2
  const uint32_t sh = 4u * odd;
  const uint32_t own = ((b0 >> sh) & 0xFu) | (((b1 >> sh) & 0xFu) << 4);
  const uint32_t give = ((b0 >> (4u - sh)) & 0xFu) | (((b1 >> (4u - sh)) & 0xFu) << 4);
  // quad_perm [1, 0, 3, 2]: the partner's nibbles of this lane's query, blocks j = 1 - odd, 3 - odd
  const uint32_t got = (uint32_t)__builtin_amdgcn_mov_dpp((int)give, 0xB1, 0xF, 0xF, false);
  const uint32_t even_j = odd ? got : own;    // blocks j = 0, 2
  const uint32_t odd_j = odd ? own : got;     // blocks j = 1, 3
  return (even_j & 0xFu) | ((odd_j & 0xFu) << 4) | ((even_j & 0xF0u) << 4) | ((odd_j & 0xF0u) << 8);
}

// Keep bits of the 16 elements a lane holds in a key-per-lane accumulator
// (dK/dV): key 4 c + (lane & 3), queries i0 + 8 j + v for j, v in 0..3 (i0
// even), as bit 4 j + v. The quad's four keys share one call per row pair
// (i0 + 8 j + 2 s, + 1), P = 2 j + s; quad lane P mod 4 draws pair P (its
// calls P = lane & 3 and P + 4) and the quad broadcasts the eight bits.
template <int V>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, V * 0x55, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t keep16_quad(const Dropout& dr, uint32_t c, uint32_t i0, uint32_t bh, int lane) {
  const uint32_t v = (uint32_t)lane & 3u;
  const uint32_t r0 = (i0 + 8u * (v >> 1) + 2u * (v & 1u)) >> 1;    // pair P = v
  const uint32_t x = keep8(dr, c, r0, bh) | (keep8(dr, c, r0 + 8u, bh) << 8);  // and P + 4 (rows + 16)
  const uint32_t xs[4] = {quad_bcast<0>(x), quad_bcast<1>(x), quad_bcast<2>(x), quad_bcast<3>(x)};
  uint32_t kmask = 0u;
#pragma unroll
  for (int P = 0; P < 8; ++P) {
    const uint32_t byte = (xs[P & 3] >> (8 * (P >> 2))) & 0xFFu;
    const int r = 4 * (P >> 1) + 2 * (P & 1);  // register of row i0 + 8 j + 2 s
    kmask |= ((byte >> v) & 1u) << r;
    kmask |= ((byte >> (4u + v)) & 1u) << (r + 1);
  }
  return kmask;
}

// Wait until this wave's outstanding vector-memory operations (including the
// tile copies above) have completed: s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_tile_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The 8 16-bit values of an operand register set, widened to fp32 (exact).
template <class DT>
__device__ __forceinline__ void unpack8(typename DT::V8 v, float* f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)v[i];
}

// Zero the 16-bit values of an operand register set whose bit in `bits` (bit i
// for value i) is clear, on the packed words: a kept value keeps its bits, a
// dropped one becomes +0, as if it were zeroed before rounding.
template <class DT>
__device__ __forceinline__ typename DT::V8 keep_mask8(typename DT::V8 v, uint32_t bits) {
  u32x4 w = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = (uint32_t)((int32_t)(bits << (31 - 2 * i)) >> 31);   // all ones iff bit 2i
    const uint32_t hi = (uint32_t)((int32_t)(bits << (30 - 2 * i)) >> 31);   // all ones iff bit 2i + 1
    w[i] &= (lo & 0xFFFFu) | (hi & 0xFFFF0000u);
  }
  return __builtin_bit_cast(typename DT::V8, w);
}

// Sum of the 8 16-bit values of an operand register set, accumulated in fp32.
template <class DT>
__device__ __forceinline__ float sum8(typename DT::V8 v, float acc);
template <>
__device__ __forceinline__ float sum8<F16>(f16x8 v, float acc) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 one = {(_Float16)1.f, (_Float16)1.f};
  acc = __builtin_amdgcn_fdot2(h2{v[0], v[1]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2(h2{v[2], v[3]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2(h2{v[4], v[5]}, one, acc, false);
  return __builtin_amdgcn_fdot2(h2{v[6], v[7]}, one, acc, false);
}
template <>
__device__ __forceinline__ float sum8<BF16>(bf16x8 v, float acc) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 one = {(__bf16)1.f, (__bf16)1.f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(b2{v[0], v[1]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(b2{v[2], v[3]}, one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(b2{v[4], v[5]}, one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(b2{v[6], v[7]}, one, acc, false);
}

// Maximum / sum across the lane pair (l, l ^ 32) that shares one row.
__device__ __forceinline__ float pair_max(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// ---------------------------------------------------------------------------
// Kept flags of one row (or one column) of the 128 x 128 block mask, read once
// per workgroup: bit k of lane l's register is the flag of tile 64 k + l
// (tiles 0 .. 2047). next(r) finds the first kept tile >= r with one ballot per
// 64 tiles instead of one memory round trip per tile; tiles past 2047 are read
// from memory.
// ---------------------------------------------------------------------------
struct TileMask {
  const uint8_t* base;   // nullptr: every tile kept
  size_t stride;         // bytes between consecutive tiles' flags
  int n;                 // tiles in the row / column
  uint32_t bits;
  __device__ __forceinline__ TileMask(const uint8_t* base_, size_t stride_, int n_, int lane)
      : base(base_), stride(stride_), n(n_), bits(0u) {
    if (base != nullptr) {
      const int words = min((n + 63) >> 6, 32);
      for (int k = 0; k < words; ++k) {
        const int t = 64 * k + lane;
        if (t < n && base[(size_t)t * stride] != 0) bits |= 1u << k;
      }
    }
  }
  // first kept tile >= r, n if none (call with all lanes of the wave active)
  __device__ __forceinline__ int next(int r) const {
    if (base == nullptr) return r;
    while (r < n) {
      const int k = r >> 6;
      if (k >= 32) {
        while (r < n && base[(size_t)r * stride] == 0) ++r;
        return r;
      }
      const uint64_t w = __builtin_amdgcn_ballot_w64(((bits >> k) & 1u) != 0u) & (~0ull << (r & 63));
      if (w != 0ull) return 64 * k + (int)__builtin_ctzll(w);
      r = 64 * (k + 1);
    }
    return n;
  }
};

// ---------------------------------------------------------------------------
// Work-group ordering: workgroups are handed to the 8 XCDs round-robin
// (hardware id hw goes to XCD hw % 8). Logical blocks come in chunks of
// `chunk` consecutive ids (the blocks of one (sequence, head)); the remap deals
// whole chunks to the XCDs in turn, so a chunk's blocks share one XCD's L2 and
// run back to back there, while consecutive chunks (the heads of one sequence)
// spread over all XCDs and sequences of different lengths load them evenly.
// Ids past the last whole round of 8 chunks map to themselves.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int hw, int total, int chunk) {
  const int round = 8 * chunk;
  if (hw >= (total / round) * round) return hw;
  const int x = hw & 7, idx = hw >> 3;
  return ((idx / chunk) * 8 + x) * chunk + idx % chunk;
}

// Causal grids of the dense layout, where a chunk's blocks differ in length:
// XCD x takes the same chunks x, x + 8, x + 16, ... but runs their blocks rank
// by rank across those chunks (rank 0 = the longest block of every chunk
// first), so each XCD works through its blocks longest first and its last
// rounds hold only short blocks. Interleaving the chunks spreads an XCD's L2
// over all of them, so the callers use it for short heads only (N d <= 2^19:
// causal N=4096 d=128 forward 0.35 -> 0.28 ms, backward -4%; N=1024 d=64
// forward -18%, backward -12%; at N=8192 d=128 the backward lost up to 5%, and
// packed batches of sequences up to 4096 lost 12%), with at most 32 blocks per
// chunk. Applies when the chunks are a whole number of rounds of 8 and at least
// two per XCD; returns false otherwise (the caller keeps xcd_remap).
__device__ __forceinline__ bool xcd_remap_ranked(int hw, int total, int nblk, int& chunk, int& rank) {
  const int nchunks = total / nblk;
  if (nblk > 32 || nchunks < 16 || nchunks % 8 != 0 || nchunks * nblk != total) return false;
  const int G = nchunks / 8;                  // chunks per XCD
  const int x = hw & 7, idx = hw >> 3;
  rank = idx / G;
  chunk = x + 8 * (idx - rank * G);
  return true;
}



// ---------------------------------------------------------------------------
// Store of a wave's 32-row output tile with whole rows per instruction. In the
// MFMA accumulator layout lane l holds row l % 32 and, for each 32-column
// block t, the columns 32 t + mrow(l / 32, r); storing that directly writes
// 8-byte pieces of 32 different rows per instruction (32 L2 requests of 16
// bytes each). The tile goes through a per-wave LDS area instead (rows padded
// by 16 bytes) and is read back with 16 consecutive bytes of one row per lane,
// so that each store instruction writes whole rows. `scale` multiplies this
// lane's row before rounding; rows >= `rows` are not written.
// stage: this wave's own LDS area of stage_bytes<W>() bytes, with no copy in
// flight into it and no other wave using it.
// ---------------------------------------------------------------------------
template <int W>
constexpr int stage_bytes() { return 32 * (2 * W + 16); }

template <class DT, int W>
__device__ __forceinline__ void store_tile_rows(const f32x16 (&acc)[W / 32], float scale, char* stage,
                                                typename DT::T* __restrict__ g0, size_t row_stride, int rows,
                                                int lane) {
  constexpr int RS = 2 * W + 16;              // padded row: 16-byte aligned, rows 4 banks apart
  const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int t = 0; t < W / 32; ++t)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      lds_write8(stage, l32 * RS + (32 * t + 8 * jj + 4 * g) * 2,
                 pack4<DT>(acc[t][4 * jj] * scale, acc[t][4 * jj + 1] * scale, acc[t][4 * jj + 2] * scale,
                           acc[t][4 * jj + 3] * scale));
  constexpr int LPR = W / 8;                  // lanes per row, 16 bytes each
  constexpr int RPI = 64 / LPR;               // rows per instruction
  const int rr = lane / LPR, ch = lane % LPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = i * RPI + rr;
    const u32x4 v = lds_read16(stage, row * RS + ch * 16);
    if (row < rows) *reinterpret_cast<u32x4*>(g0 + (size_t)row * row_stride + ch * 8) = v;
  }
}

}  // namespace fa
