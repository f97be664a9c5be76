// Attention backward for gfx950: recompute P tile by tile from Q, K and the
// saved log-sum-exp and form dQ, dK, dV without atomics.
//
// Method: page 1 ("FlashAttention：不减少一次注意力计算，为什么反而更快"), key design 3:
// P_ij is rebuilt from the saved row statistic, D_i = dO_i . O_i replaces the
// row-wide reduction, dS = P o (dP - D), dV = P^T dO, dQ = dS K, dK = dS^T Q.
// The softmax scale s enters S = s Q K^T, so dQ and dK carry a factor s.
// Page 2 ("FlashAttention 入门", backward section) notes that the default
// backward adds dQ across blocks with atomics and that a deterministic option
// exists at some extra cost; on this chip device-scope fp32 atomics cost more
// than recomputing S and dP once more, so this backward is the deterministic
// form: two kernels, each owning its outputs.
//
//   * dkdv_kernel: one workgroup = NW waves = NW*32 keys of one head. Each wave
//     keeps its 32 rows of K and V in VGPRs (B operands of S = Q K^T and
//     dP = dO V^T) and its fp32 dK^T / dV^T accumulators; Q / dO tiles of 128
//     rows are copied HBM -> LDS directly (double buffered). S and dP keep queries on the accumulator's
//     register index, so P and dS feed dV^T = dO^T P and dK^T = Q^T dS directly
//     as B operands, with dO^T / Q^T from LDS by the transpose read.
//   * dkdv_split_kernel (d = 128): the same products split between wave pairs
//     so that two waves per SIMD fit the register file (see below).
//   * dq_kernel: one workgroup = NW waves = NW*32 queries, laid out like the
//     forward: Q and dO fragments stay in VGPRs, K / V tiles stream through
//     LDS, S^T and dP^T put one query per lane, and dS^T feeds
//     dQ^T = K^T dS^T as a B operand with K^T from the transpose read.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// ---------------------------------------------------------------------------
// D_i = sum_k dO_ik O_ik (fp32 accumulation of the stored 16-bit values)
// ---------------------------------------------------------------------------
template <class DT, int D>
__global__ __launch_bounds__(256) void preprocess_kernel(const void* __restrict__ o_, const void* __restrict__ do_,
                                                         float* __restrict__ Dvec, long long rows) {
  using T = typename DT::T;
  constexpr int TPR = D / 8;                   // threads per row, 8 elements each
  constexpr int RPB = 256 / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float sum = 0.f;
  if (row < rows) {
    const T* o = reinterpret_cast<const T*>(o_) + row * D + c * 8;
    const T* g = reinterpret_cast<const T*>(do_) + row * D + c * 8;
    typename DT::V8 a = as_v8<DT>(*reinterpret_cast<const u32x4*>(o));
    typename DT::V8 b = as_v8<DT>(*reinterpret_cast<const u32x4*>(g));
#pragma unroll
    for (int i = 0; i < 8; ++i) sum = fmaf((float)a[i], (float)b[i], sum);
  }
#pragma unroll
  for (int w = TPR / 2; w > 0; w >>= 1) sum += __shfl_xor(sum, w);
  if (row < rows && c == 0) Dvec[row] = sum;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per block of NW*32 keys, looping over query tiles
// ---------------------------------------------------------------------------
template <int D>
struct DkdvOccupancy { static constexpr int value = D <= 64 ? 2 : 1; };

template <class DT, int D, int BQ, int NW, bool DROP>
__global__ __launch_bounds__(NW * 64, DkdvOccupancy<D>::value) void dkdv_kernel(BwdParams p) {
  using T = typename DT::T;
  using V8 = typename DT::V8;
  constexpr int BK = NW * 32;                 // keys per workgroup
  constexpr int ROWB = D * 2;
  constexpr int QTILE = BQ * ROWB;
  constexpr int KC = D / 16;
  constexpr int MQ = BQ / 32;                 // 32-query halves per tile
  constexpr int DT32 = D / 32;
  static_assert(128 % BK == 0 && 128 % BQ == 0, "block-mask granularity");

  // [Q buf0 | dO buf0 | Q buf1 | dO buf1 | lse2 x2 | D x2]
  __shared__ __attribute__((aligned(16))) char smem[4 * QTILE + 4 * BQ * 4];
  float* const lse_s = reinterpret_cast<float*>(smem + 4 * QTILE);  // [2][BQ]
  float* const dd_s = lse_s + 2 * BQ;                                // [2][BQ]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int N = p.N;

  const int logical = xcd_remap(blockIdx.x, p.total_blocks, p.k_blocks);
  int bh = logical / p.k_blocks;              // (sequence, key/value head)
  int kb = logical - bh * p.k_blocks;         // causal: low key blocks carry the most rows, run first
  if (p.causal && p.L.cu_q == nullptr && (long long)N * D <= kRankedMaxNd)
    xcd_remap_ranked(blockIdx.x, p.total_blocks, p.k_blocks, bh, kb);
  const int k0 = kb * BK;
  const int kw0 = k0 + wave * 32;
  const int kw = kw0 + l32;                   // this lane's key (column of S and dP)
  const int b = bh / p.L.Hk, hk = bh - b * p.L.Hk;
  const int grp = p.H / p.L.Hk;               // query heads reading this key/value head
  const HeadView hv = head_view(p.L, b, hk * grp, p.H, N, D);
  const int lq = hv.lq, lk = hv.lk;
  if (k0 >= lk) return;                       // uniform: this block has no keys of its sequence
  const int off = lk - lq;                    // causal: key j is seen by queries i >= j - off

  const uint32_t q_bytes = span_bytes(lq, hv.q_stride, D, 2), kv_bytes = span_bytes(lk, hv.kv_stride, D, 2);
  const auto k_rs = make_rsrc(reinterpret_cast<const T*>(p.k) + hv.kv_off, kv_bytes);
  const auto v_rs = make_rsrc(reinterpret_cast<const T*>(p.v) + hv.kv_off, kv_bytes);
  const int q_rstride = hv.q_stride * 2;

  // ---- K, V fragments (B operands of S = Q K^T and dP = dO V^T); keys past the sequence read as zero
  V8 kf[KC], vf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    kf[c] = as_v8<DT>(buf_load16(k_rs, (kw * hv.kv_stride + 16 * c + 8 * g) * 2));
    vf[c] = as_v8<DT>(buf_load16(v_rs, (kw * hv.kv_stride + 16 * c + 8 * g) * 2));
  }

  // ---- lane-constant LDS offsets
  int qoff[KC];                               // Q / dO operand rows l32, chunk 2c + g
#pragma unroll
  for (int c = 0; c < KC; ++c) qoff[c] = tile_off<ROWB>(l32, 16 * c + 8 * g);
  int troff[DT32][2];                         // dO^T / Q^T operands: rows 4g (+8) + (lane%16)/4 (+ block base)
#pragma unroll
  for (int d0 = 0; d0 < DT32; ++d0) {
    troff[d0][0] = tr_off<ROWB>(4 * g, 32 * d0, lane);
    troff[d0][1] = tr_off<ROWB>(4 * g + 8, 32 * d0, lane);
  }

  // ---- query tiles: every query head of the group x the tiles that see this key block.
  // Flat index t -> head (t / nspan) of the group, tile i_begin + t % nspan.
  const int n_qt = (lq + BQ - 1) / BQ;
  const int i_begin = p.causal ? max(k0 - off, 0) / BQ : 0;
  const int nspan = max(n_qt - i_begin, 0);
  const int n_t = grp * nspan;
  auto tile_i = [&](int t) { return i_begin + t % nspan; };
  // first kept flat tile >= t (n_t if none): the block-mask column of this key block
  // (the mask comes with the dense layout only)
  const TileMask mcol(p.mask ? p.mask + (k0 / 128) : nullptr, (size_t)p.mask_tiles, p.mask_tiles, lane);
  auto next_kept = [&](int t) {
    while (t < n_t) {
      const int hh = t / nspan, i = tile_i(t);
      const int r = (i * BQ) / 128, r2 = mcol.next(r);
      if (r2 == r) return t;
      const int i2 = (r2 * 128) / BQ;       // first query tile of the next kept row tile
      if (i2 < n_qt) return hh * nspan + (i2 - i_begin);
      t = (hh + 1) * nspan;                 // nothing left for this head
    }
    return n_t;
  };

  const TileCopy<ROWB, QTILE, NW> copy(wave, lane, q_rstride);
  float lse_r = 0.f, dd_r = 0.f;
  // asynchronous copy of flat tile t into LDS buffer buf (rows past the sequence
  // arrive as zeros); its LSE / D go through registers and are stored by sstore()
  auto gload = [&](int t, int buf) {
    char* qt = smem + buf * 2 * QTILE;
    const int hh = t / nspan, i = tile_i(t);
    const size_t qo = hv.q_off + (size_t)hh * hv.q_hstep;
    copy.issue(make_rsrc(reinterpret_cast<const T*>(p.q) + qo, q_bytes), qt, i * BQ * q_rstride);
    copy.issue(make_rsrc(reinterpret_cast<const T*>(p.dO) + qo, q_bytes), qt + QTILE, i * BQ * q_rstride);
    if (tid < BQ) {
      const int q = i * BQ + tid;
      const size_t si = hv.stat_off + (size_t)hh * hv.stat_hstep + (size_t)q * hv.stat_stride;
      const float l = q < lq ? p.lse[si] : -INFINITY;
      // rows past the sequence or with no visible key get P = exp2(s - inf) = 0
      lse_r = (l == -INFINITY) ? INFINITY : l * kLog2e;
      // stored as -D (1 - p): the dP accumulator starts from it (p = 0 without dropout)
      dd_r = q < lq ? -p.Dvec[si] / (DROP ? p.drop.rescale : 1.f) : 0.f;
    }
  };
  auto sstore = [&](int buf) {
    if (tid < BQ) {
      lse_s[buf * BQ + tid] = lse_r;
      dd_s[buf * BQ + tid] = dd_r;
    }
  };

  f32x16 dv[DT32], dk[DT32];
#pragma unroll
  for (int t = 0; t < DT32; ++t) { dv[t] = f32x16{}; dk[t] = f32x16{}; }

  const float c2 = p.scale_log2;
  int t = next_kept(0);
  if (t < n_t) {
    gload(t, 0);
    sstore(0);
  }
  wait_tile_copies();
  __syncthreads();
  int buf = 0;

  while (t < n_t) {
    const int tn = next_kept(t + 1);
    if (tn < n_t) gload(tn, buf ^ 1);       // that buffer was last read before the previous barrier
    const int q0 = tile_i(t) * BQ;
    const char* qt = smem + buf * 2 * QTILE;
    const char* ot = qt + QTILE;
    const float* lt = lse_s + buf * BQ;
    const float* dl = dd_s + buf * BQ;
    const bool edge = (kw0 + 32 > lk) || (p.causal && kw0 + 31 > q0 + off);

#pragma unroll
    for (int mq = 0; mq < MQ; ++mq) {
      // Q and dO rows of this 32-query half, read as one batch, then
      // S and dP for queries q0 + 32 mq + mrow (registers) x this lane's key
      V8 qa[KC], oa[KC];
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        qa[c] = as_v8<DT>(lds_read16(qt, qoff[c] + 32 * mq * ROWB));
        oa[c] = as_v8<DT>(lds_read16(ot, qoff[c] + 32 * mq * ROWB));
      }
      // dP starts from -D (1 - p) (rows 8 jj + 4 g + u in register 4 jj + u), so
      // that the chain ends at dP - D (1 - p) without a subtraction per element
      f32x16 s = f32x16{}, dp;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dl + 32 * mq + 8 * jj + 4 * g);
#pragma unroll
        for (int u = 0; u < 4; ++u) dp[4 * jj + u] = d4[u];
      }
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        s = DT::mma(qa[c], kf[c], s);
        dp = DT::mma(oa[c], vf[c], dp);
      }
      // dO^T / Q^T operands of the dV / dK products, in flight while S and dP run
      V8 ta[DT32][2], tb[DT32][2];
#pragma unroll
      for (int d0 = 0; d0 < DT32; ++d0)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int rb = (32 * mq + 16 * h) * ROWB;
          ta[d0][h] = tr_pair<DT>(ot, troff[d0][0] + rb, troff[d0][1] + rb);
          tb[d0][h] = tr_pair<DT>(qt, troff[d0][0] + rb, troff[d0][1] + rb);
        }
      // dropout keep bits of (query q0 + 32 mq + mrow(g, r), key kw)
      uint32_t kmask = 0xFFFFu;
      if constexpr (DROP) {
        const uint32_t bhq = (uint32_t)(b * p.H + hk * grp + t / nspan);
        // rows mrow(g, r) = 8 (r / 4) + 4 g + r % 4 of this sub-tile
        kmask = keep16_quad(p.drop, (uint32_t)kw >> 2, (uint32_t)(q0 + 32 * mq + 4 * g), bhq, lane);
      }
      float pe[16], de[16];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + 32 * mq + 8 * jj + 4 * g);
        f32x4 d4 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (DROP) d4 = *reinterpret_cast<const f32x4*>(dl + 32 * mq + 8 * jj + 4 * g);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * jj + u;
          pe[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -l4[u]));
          // dP - D with dP = Z o (dO V^T), Z = M / (1 - p): kept (dO V^T - D (1 - p)) / (1 - p),
          // dropped -D
          de[r] = DROP ? (((kmask >> r) & 1) ? dp[r] : d4[u]) * p.drop.rescale : dp[r];
        }
      }
      if (edge) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + 32 * mq + mrow(g, r);
          if (kw >= lk || (p.causal && kw > q + off)) pe[r] = 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) de[r] *= pe[r];
      // B operands: slot i of half h <-> query 32 mq + 16 h + 8 (i / 4) + 4 g + i % 4
      V8 pb[2], sb[2];
      if constexpr (DROP) {                   // dV uses the dropped P (rescaled in the epilogue)
#pragma unroll
        for (int r = 0; r < 16; ++r) pe[r] = ((kmask >> r) & 1) ? pe[r] : 0.f;
      }
      pb[0] = pack8<DT>(pe[0], pe[1], pe[2], pe[3], pe[4], pe[5], pe[6], pe[7]);
      pb[1] = pack8<DT>(pe[8], pe[9], pe[10], pe[11], pe[12], pe[13], pe[14], pe[15]);
      sb[0] = pack8<DT>(de[0], de[1], de[2], de[3], de[4], de[5], de[6], de[7]);
      sb[1] = pack8<DT>(de[8], de[9], de[10], de[11], de[12], de[13], de[14], de[15]);
      // dV^T += dO^T P and dK^T += Q^T dS (contraction over these 32 queries)
#pragma unroll
      for (int d0 = 0; d0 < DT32; ++d0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          dv[d0] = DT::mma(ta[d0][h], pb[h], dv[d0]);
          dk[d0] = DT::mma(tb[d0][h], sb[h], dk[d0]);
        }
      }
    }

    if (tn < n_t) sstore(buf ^ 1);
    wait_tile_copies();
    __syncthreads();
    buf ^= 1;
    t = tn;
  }

  // ---- epilogue: lane holds key kw, dims 32 d0 + mrow(g, r); rows kw0.. go out
  // through this wave's part of the (now idle) tile buffers
  static_assert(2 * NW * stage_bytes<D>() <= 4 * QTILE, "staging fits the tile buffers");
  {
    char* const st = smem + wave * 2 * stage_bytes<D>();
    const int rows = min(32, lk - kw0);
    const size_t row0 = hv.kv_off + (size_t)kw0 * hv.kv_stride;
    store_tile_rows<DT, D>(dk, p.scale, st, reinterpret_cast<T*>(p.dk) + row0, hv.kv_stride, rows, lane);
    store_tile_rows<DT, D>(dv, DROP ? p.drop.rescale : 1.f, st + stage_bytes<D>(), reinterpret_cast<T*>(p.dv) + row0,
                           hv.kv_stride, rows, lane);
  }
}

// ---------------------------------------------------------------------------
// dK, dV for d = 128: role-split wave pairs, 8 waves (two per SIMD) and 128 keys
// per workgroup. Waves w and w + 4 share the 32 keys of group w:
//   role A (waves 0-3) keeps K and dV^T: S = Q K^T, P = exp2(S c - LSE) (rounded
//     to the operand type, written to LDS), dV^T += dO^T P;
//   role B (waves 4-7) keeps V and dK^T: dP = dO V^T, dS = P o (dP - D) with P
//     read back from LDS, dK^T += Q^T dS.
// B runs one query tile behind A: in step n, A forms dV of tile n and S, P of
// tile n + 1 while B forms dS, dK of tile n and dP of tile n + 1, so one barrier
// per tile suffices and each SIMD always has two waves with independent work.
// Three Q/dO tile slots (tiles n and n + 1 in use, n + 2 arriving) and two P
// buffers. dS uses the same rounded P that enters dV (an fp16/bf16 rounding of
// P, inside the gradient tolerance).
// ---------------------------------------------------------------------------
// DROP: role A draws the dropout mask; the P it hands to role B carries the
// mask in the sign bit (negative = dropped), its own dV operand is the dropped P.
template <class DT, int D, int BQ, bool DROP>
__global__ __launch_bounds__(512, 1) void dkdv_split_kernel(BwdParams p) {
  using T = typename DT::T;
  using V8 = typename DT::V8;
  constexpr int NW = 8;
  constexpr int BK = 128;                     // keys per workgroup
  constexpr int ROWB = D * 2;
  constexpr int QTILE = BQ * ROWB;
  constexpr int KC = D / 16;
  constexpr int MQ = BQ / 32;
  constexpr int DT32 = D / 32;
  constexpr int PBUF = 4 * MQ * 2 * 1024;     // P of one tile: [group][half][k][lane] x 16 bytes
  static_assert(MQ == 2 && 128 % BQ == 0, "two 32-query halves per tile; block-mask granularity");

  // [3 x (Q | dO)] [2 x P] [3 x lse2] [3 x D]
  __shared__ __attribute__((aligned(16))) char smem[6 * QTILE + 2 * PBUF + 6 * BQ * 4];
  char* const pbase = smem + 6 * QTILE;
  float* const lse_s = reinterpret_cast<float*>(smem + 6 * QTILE + 2 * PBUF);
  float* const dd_s = lse_s + 3 * BQ;

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave & 3;
  const int N = p.N;

  const int logical = xcd_remap(blockIdx.x, p.total_blocks, p.k_blocks);
  int bh = logical / p.k_blocks;              // (sequence, key/value head)
  int kb = logical - bh * p.k_blocks;         // causal: low key blocks carry the most rows, run first
  if (p.causal && p.L.cu_q == nullptr && (long long)N * D <= kRankedMaxNd)
    xcd_remap_ranked(blockIdx.x, p.total_blocks, p.k_blocks, bh, kb);
  const int k0 = kb * BK;
  const int kw0 = k0 + grp * 32;
  const int kw = kw0 + l32;                   // this lane's key
  const int b = bh / p.L.Hk, hk = bh - b * p.L.Hk;
  const int qgrp = p.H / p.L.Hk;              // query heads reading this key/value head
  const HeadView hv = head_view(p.L, b, hk * qgrp, p.H, N, D);
  const int lq = hv.lq, lk = hv.lk;
  if (k0 >= lk) return;                       // uniform: this block has no keys of its sequence
  const int off = lk - lq;                    // causal: key j is seen by queries i >= j - off

  const uint32_t q_bytes = span_bytes(lq, hv.q_stride, D, 2), kv_bytes = span_bytes(lk, hv.kv_stride, D, 2);
  const uint32_t stat_bytes = span_bytes(lq, hv.stat_stride, 1, 4);
  const auto k_rs = make_rsrc(reinterpret_cast<const T*>(p.k) + hv.kv_off, kv_bytes);
  const auto v_rs = make_rsrc(reinterpret_cast<const T*>(p.v) + hv.kv_off, kv_bytes);
  const int q_rstride = hv.q_stride * 2;

  int qoff[KC];                               // operand rows l32, chunk 2c + g
#pragma unroll
  for (int c = 0; c < KC; ++c) qoff[c] = tile_off<ROWB>(l32, 16 * c + 8 * g);
  int troff[DT32][2];                         // transposed operands: rows 4g (+8) + (lane%16)/4
#pragma unroll
  for (int d0 = 0; d0 < DT32; ++d0) {
    troff[d0][0] = tr_off<ROWB>(4 * g, 32 * d0, lane);
    troff[d0][1] = tr_off<ROWB>(4 * g + 8, 32 * d0, lane);
  }

  // query tiles: every query head of the group x the tiles that see this key
  // block; flat index t -> head t / nspan of the group, tile i_begin + t % nspan
  const int n_qt = (lq + BQ - 1) / BQ;
  const int i_begin = p.causal ? max(k0 - off, 0) / BQ : 0;
  const int nspan = max(n_qt - i_begin, 0);
  const int n_t = qgrp * nspan;
  auto tile_i = [&](int t) { return i_begin + t % nspan; };
  // first kept flat tile >= t (n_t if none): the block-mask column of this key block
  // (the mask comes with the dense layout only)
  const TileMask mcol(p.mask ? p.mask + (k0 / 128) : nullptr, (size_t)p.mask_tiles, p.mask_tiles, lane);
  auto next_kept = [&](int t) {
    while (t < n_t) {
      const int hh = t / nspan, i = tile_i(t);
      const int r = (i * BQ) / 128, r2 = mcol.next(r);
      if (r2 == r) return t;
      const int i2 = (r2 * 128) / BQ;       // first query tile of the next kept row tile
      if (i2 < n_qt) return hh * nspan + (i2 - i_begin);
      t = (hh + 1) * nspan;                 // nothing left for this head
    }
    return n_t;
  };
  auto q_of = [&](int t) { return hv.q_off + (size_t)(t / nspan) * hv.q_hstep; };
  auto stat_of = [&](int t) { return hv.stat_off + (size_t)(t / nspan) * hv.stat_hstep; };

  const TileCopy<ROWB, QTILE, NW> copy(wave, lane, q_rstride);
  constexpr int PW = TileCopy<ROWB, QTILE, NW>::PER_WAVE;
  // LSE / D of a tile go through registers: loaded before its tile copies are
  // issued (so waiting for them never waits for the copies) and converted when
  // stored into their slot
  float lse_r = 0.f, dd_r = 0.f;
  int i_ld = 0;
  auto stat_load = [&](int t) {
    const int i = tile_i(t);
    i_ld = i;
    if (tid < BQ) {
      const auto lse_rs = make_rsrc(p.lse + stat_of(t), stat_bytes);
      const auto dvec_rs = make_rsrc(p.Dvec + stat_of(t), stat_bytes);
      lse_r = buf_load_f32(lse_rs, (i * BQ + tid) * hv.stat_stride * 4);
      dd_r = buf_load_f32(dvec_rs, (i * BQ + tid) * hv.stat_stride * 4);
    }
  };
  auto copy_tile = [&](int t, int slot) {
    char* qt = smem + slot * 2 * QTILE;
    const size_t qo = q_of(t);
    copy.issue(make_rsrc(reinterpret_cast<const T*>(p.q) + qo, q_bytes), qt, tile_i(t) * BQ * q_rstride);
    copy.issue(make_rsrc(reinterpret_cast<const T*>(p.dO) + qo, q_bytes), qt + QTILE, tile_i(t) * BQ * q_rstride);
  };
  auto stat_store = [&](int slot) {
    if (tid < BQ) {
      const int q = i_ld * BQ + tid;
      // rows past N or with no visible key get P = exp2(s - inf) = 0
      lse_s[slot * BQ + tid] = (q >= lq || lse_r == -INFINITY) ? INFINITY : lse_r * kLog2e;
      // stored as -D (1 - p): role B's dP accumulator starts from it (p = 0 without dropout)
      dd_s[slot * BQ + tid] = q < lq ? -dd_r / (DROP ? p.drop.rescale : 1.f) : 0.f;
    }
  };

  f32x16 acc[DT32];                           // A: dV^T, B: dK^T (lane: key kw, rows: dims)
#pragma unroll
  for (int t = 0; t < DT32; ++t) acc[t] = f32x16{};
  const float c2 = p.scale_log2;

  auto run = [&](auto role_tag) {
    constexpr bool A = decltype(role_tag)::value;
    V8 kvf[KC];                               // A: K rows, B: V rows (B operands, keys >= N read as zero)
#pragma unroll
    for (int c = 0; c < KC; ++c)
      kvf[c] = as_v8<DT>(buf_load16(A ? k_rs : v_rs, (kw * hv.kv_stride + 16 * c + 8 * g) * 2));

    V8 pb[MQ][2];                             // A: rounded P of the tile in flight
    f32x16 dp[MQ];                            // B: dP of the tile in flight

    // A: S and P of flat tile t (slot), P also to LDS buffer pslot; B: dP of tile t
    auto front = [&](int t, int slot, int pslot) {
      const char* qt = smem + slot * 2 * QTILE;
      const char* ot = qt + QTILE;
      const float* lt = lse_s + slot * BQ;
      const int q0 = tile_i(t) * BQ;
      const bool edge = (kw0 + 32 > lk) || (p.causal && kw0 + 31 > q0 + off);
      char* pbuf = pbase + pslot * PBUF;
#pragma unroll
      for (int mq = 0; mq < MQ; ++mq) {
        V8 xa[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) xa[c] = as_v8<DT>(lds_read16(A ? qt : ot, qoff[c] + 32 * mq * ROWB));
        // A: S from zero; B: dP from -D (1 - p) (rows 8 jj + 4 g + u in register 4 jj + u)
        f32x16 s = f32x16{};
        if constexpr (!A) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(dd_s + slot * BQ + 32 * mq + 8 * jj + 4 * g);
#pragma unroll
            for (int u = 0; u < 4; ++u) s[4 * jj + u] = d4[u];
          }
        }
#pragma unroll
        for (int c = 0; c < KC; ++c) s = DT::mma(xa[c], kvf[c], s);
        if constexpr (A) {
          float pe[16];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + 32 * mq + 8 * jj + 4 * g);
#pragma unroll
            for (int u = 0; u < 4; ++u) pe[4 * jj + u] = __builtin_amdgcn_exp2f(fmaf(s[4 * jj + u], c2, -l4[u]));
          }
          if (edge) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int q = q0 + 32 * mq + mrow(g, r);
              if (kw >= lk || (p.causal && kw > q + off)) pe[r] = 0.f;
            }
          }
          if constexpr (DROP) {
            const uint32_t bhq = (uint32_t)(b * p.H + hk * qgrp + t / nspan);
            // rows mrow(g, r) = 8 (r / 4) + 4 g + r % 4 of this sub-tile
            const uint32_t kmask = keep16_quad(p.drop, (uint32_t)kw >> 2, (uint32_t)(q0 + 32 * mq + 4 * g), bhq, lane);
            float pd[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const bool keep = (kmask >> r) & 1;
              pd[r] = keep ? pe[r] : 0.f;
              pe[r] = keep ? pe[r] : -pe[r];
            }
            const V8 e0 = pack8<DT>(pe[0], pe[1], pe[2], pe[3], pe[4], pe[5], pe[6], pe[7]);
            const V8 e1 = pack8<DT>(pe[8], pe[9], pe[10], pe[11], pe[12], pe[13], pe[14], pe[15]);
            lds_write16(pbuf, (((grp * MQ + mq) * 2 + 0) * 64 + lane) * 16, __builtin_bit_cast(u32x4, e0));
            lds_write16(pbuf, (((grp * MQ + mq) * 2 + 1) * 64 + lane) * 16, __builtin_bit_cast(u32x4, e1));
            pb[mq][0] = pack8<DT>(pd[0], pd[1], pd[2], pd[3], pd[4], pd[5], pd[6], pd[7]);
            pb[mq][1] = pack8<DT>(pd[8], pd[9], pd[10], pd[11], pd[12], pd[13], pd[14], pd[15]);
          } else {
            pb[mq][0] = pack8<DT>(pe[0], pe[1], pe[2], pe[3], pe[4], pe[5], pe[6], pe[7]);
            pb[mq][1] = pack8<DT>(pe[8], pe[9], pe[10], pe[11], pe[12], pe[13], pe[14], pe[15]);
#pragma unroll
            for (int h = 0; h < 2; ++h)
              lds_write16(pbuf, (((grp * MQ + mq) * 2 + h) * 64 + lane) * 16, __builtin_bit_cast(u32x4, pb[mq][h]));
          }
        } else {
          dp[mq] = s;
        }
      }
    };

    // A: dV^T += dO^T P; B: dS = P o (dP - D), dK^T += Q^T dS (tile in slot, P in pslot).
    // Also issues this wave's share of the copy of flat tile tl into slot lslot,
    // one kilobyte every few products.
    auto back = [&](int slot, int pslot, int tl, int lslot) {
      const char* qt = smem + slot * 2 * QTILE;
      const char* ot = qt + QTILE;
      const float* dl = dd_s + slot * BQ;
      const char* pbuf = pbase + pslot * PBUF;
      char* const nq = smem + lslot * 2 * QTILE;
      const size_t nqo = q_of(tl);
      const auto nq_rs = make_rsrc(reinterpret_cast<const T*>(p.q) + nqo, q_bytes);
      const auto ndo_rs = make_rsrc(reinterpret_cast<const T*>(p.dO) + nqo, q_bytes);
      const int ngb = tile_i(tl) * BQ * q_rstride;
      constexpr int NMF = MQ * DT32 * 2;      // products in back()
      static_assert(NMF % (2 * PW) == 0, "copy spread");
      uint32_t ta[DT32][2];
#pragma unroll
      for (int d0 = 0; d0 < DT32; ++d0)
#pragma unroll
        for (int k = 0; k < 2; ++k) ta[d0][k] = lds_addr(A ? ot : qt) + troff[d0][k];
      static_for<0, MQ>([&](auto mqc) {
        constexpr int mq = decltype(mqc)::value;
        V8 tx[DT32][2];                       // A: dO^T, B: Q^T (rows 32 mq + 16 h ..)
        static_for<0, 2>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
#pragma unroll
          for (int d0 = 0; d0 < DT32; ++d0) tx[d0][h] = tr_pair_imm<DT, (32 * mq + 16 * h) * ROWB>(ta[d0][0], ta[d0][1]);
        });
        V8 bop[2];
        if constexpr (A) {
          bop[0] = pb[mq][0];
          bop[1] = pb[mq][1];
        } else {
          float pe[16], de[16];
#pragma unroll
          for (int h = 0; h < 2; ++h)
            unpack8<DT>(as_v8<DT>(lds_read16(pbuf, (((grp * MQ + mq) * 2 + h) * 64 + lane) * 16)), pe + 8 * h);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            f32x4 d4 = {0.f, 0.f, 0.f, 0.f};
            if constexpr (DROP) d4 = *reinterpret_cast<const f32x4*>(dl + 32 * mq + 8 * jj + 4 * g);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int r = 4 * jj + u;
              if constexpr (DROP) {               // sign bit = dropped; dP = Z o (dO V^T)
                // kept: (dO V^T - D (1 - p)) / (1 - p) = dP - D; dropped: -D
                const bool keep = !__builtin_signbit(pe[r]);
                const float pr = __builtin_fabsf(pe[r]);
                de[r] = ((keep ? dp[mq][r] : d4[u]) * p.drop.rescale) * pr;
              } else {
                de[r] = dp[mq][r] * pe[r];
              }
            }
          }
          bop[0] = pack8<DT>(de[0], de[1], de[2], de[3], de[4], de[5], de[6], de[7]);
          bop[1] = pack8<DT>(de[8], de[9], de[10], de[11], de[12], de[13], de[14], de[15]);
        }
#pragma unroll
        for (int d0 = 0; d0 < DT32; ++d0) lds_wait_tie2(tx[d0][0], tx[d0][1]);
#pragma unroll
        for (int d0 = 0; d0 < DT32; ++d0)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int m = (mq * DT32 + d0) * 2 + h;
            if (m % (NMF / (2 * PW)) == 0) {
              const int u = m / (NMF / (2 * PW));
              if (u < PW) copy.issue_one(nq_rs, nq, ngb, u);
              else copy.issue_one(ndo_rs, nq + QTILE, ngb, u - PW);
            }
            acc[d0] = DT::mma(tx[d0][h], bop[h], acc[d0]);
          }
      });
    };

    // prologue: the first two kept tiles resident, front() of the first
    int t0 = next_kept(0);
    int t1 = t0 < n_t ? next_kept(t0 + 1) : n_t;
    if (t0 < n_t) {
      stat_load(t0);
      copy_tile(t0, 0);
      stat_store(0);
    }
    if (t1 < n_t) {
      stat_load(t1);
      copy_tile(t1, 1);
      stat_store(1);
    }
    wait_tile_copies();
    __syncthreads();
    if (t0 < n_t) front(t0, 0, 0);
    __syncthreads();
    int n = 0;
    while (t0 < n_t) {
      const int t2 = t1 < n_t ? next_kept(t1 + 1) : n_t;
      const int s0 = n % 3, s1 = (n + 1) % 3, s2 = (n + 2) % 3;
      // tile n + 2 into the idle slot s2 (past the last tile: this tile again, never read)
      const int tl = t2 < n_t ? t2 : t0;
      stat_load(tl);
      back(s0, n & 1, tl, s2);
      if (t1 < n_t) front(t1, s1, (n + 1) & 1);
      if (t2 < n_t) stat_store(s2);
      wait_tile_copies();
      __syncthreads();
      ++n;
      t0 = t1;
      t1 = t2;
    }
  };
  if (wave < 4) run(std::integral_constant<bool, true>{});
  else run(std::integral_constant<bool, false>{});

  // ---- epilogue: A writes dV, B writes dK = s dS^T Q (lane: key kw, dims 32 d0 + mrow);
  // rows kw0.. go out through this wave's part of the (now idle) tile slots
  static_assert(8 * stage_bytes<D>() <= 6 * QTILE, "staging fits the tile slots");
  {
    const bool isA = wave < 4;
    const int rows = min(32, lk - kw0);
    T* const dst = reinterpret_cast<T*>(isA ? p.dv : p.dk) + hv.kv_off + (size_t)kw0 * hv.kv_stride;
    store_tile_rows<DT, D>(acc, isA ? (DROP ? p.drop.rescale : 1.f) : p.scale, smem + wave * stage_bytes<D>(), dst,
                           hv.kv_stride, rows, lane);
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per block of NW*32 queries, looping over key tiles
// ---------------------------------------------------------------------------
// Register target: three waves per SIMD (<= 168 VGPRs) at d = 64 (with or
// without dropout), two at d = 128.
template <int D, bool DROP>
struct DqOccupancy { static constexpr int value = D <= 64 ? 3 : 2; };

template <class DT, int D, int BN, int NW, bool DROP>
__global__ __launch_bounds__(NW * 64, (DqOccupancy<D, DROP>::value)) void dq_kernel(BwdParams p) {
  using T = typename DT::T;
  using V8 = typename DT::V8;
  constexpr int BM = NW * 32;
  constexpr int ROWB = D * 2;
  constexpr int TILE = BN * ROWB;
  constexpr int KC = D / 16;
  constexpr int NS = BN / 32;
  constexpr int DT32 = D / 32;
  // a 256-row block (NW = 8) spans two block-mask rows: launched only without a mask
  static_assert((128 % BM == 0 || BM == 256) && 128 % BN == 0, "block-mask granularity");
  // two K/V tile buffers; the epilogue's output staging reuses them
  constexpr int SMEM = 4 * TILE > NW * stage_bytes<D>() ? 4 * TILE : NW * stage_bytes<D>();
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int N = p.N;

  const int logical = xcd_remap(blockIdx.x, p.total_blocks, p.q_blocks);
  int bh = logical / p.q_blocks;
  int qb = logical - bh * p.q_blocks;
  if (p.causal) {                             // longest rows first
    int rank;
    if (p.L.cu_q == nullptr && (long long)N * D <= kRankedMaxNd &&
        xcd_remap_ranked(blockIdx.x, p.total_blocks, p.q_blocks, bh, rank))
      qb = rank;
    qb = p.q_blocks - 1 - qb;
  }
  const int q0 = qb * BM;
  const int qw = q0 + wave * 32 + l32;        // this lane's query
  const int w0 = q0 + __builtin_amdgcn_readfirstlane(wave) * 32;   // this wave's first query
  const int b = bh / p.H, h = bh - b * p.H;
  const HeadView hv = head_view(p.L, b, h, p.H, N, D);
  const int lq = hv.lq, lk = hv.lk;
  if (q0 >= lq) return;                       // uniform: this block has no rows of its sequence
  const int off = lk - lq;                    // causal: query i sees keys j <= i + off

  const uint32_t q_bytes = span_bytes(lq, hv.q_stride, D, 2), kv_bytes = span_bytes(lk, hv.kv_stride, D, 2);
  const auto q_rs = make_rsrc(reinterpret_cast<const T*>(p.q) + hv.q_off, q_bytes);
  const auto k_rs = make_rsrc(reinterpret_cast<const T*>(p.k) + hv.kv_off, kv_bytes);
  const auto v_rs = make_rsrc(reinterpret_cast<const T*>(p.v) + hv.kv_off, kv_bytes);
  const auto do_rs = make_rsrc(reinterpret_cast<const T*>(p.dO) + hv.q_off, q_bytes);
  const int kv_rstride = hv.kv_stride * 2;

  const int n_tiles = (lk + BN - 1) / BN;
  int j_end = n_tiles;
  if (p.causal) {
    const int last_vis = min(q0 + BM, lq) - 1 + off;
    j_end = last_vis < 0 ? 0 : min(n_tiles, last_vis / BN + 1);
  }
  // first kept key tile >= j (j_end if none): the block-mask row of this query block
  const TileMask mask_row(p.mask ? p.mask + (size_t)(q0 / 128) * p.mask_tiles : nullptr, 1, p.mask_tiles, lane);
  auto next_kept = [&](int j) {
    if (j >= j_end) return j_end;
    const int r = (j * BN) / 128, r2 = mask_row.next(r);
    return r2 == r ? j : min((r2 * 128) / BN, j_end);
  };

  // ---- per-query state: Q and dO fragments (B operands of S^T and dP^T), LSE, D
  V8 qf[KC], of[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    qf[c] = as_v8<DT>(buf_load16(q_rs, (qw * hv.q_stride + 16 * c + 8 * g) * 2));
    of[c] = as_v8<DT>(buf_load16(do_rs, (qw * hv.q_stride + 16 * c + 8 * g) * 2));
  }
  float lse2 = INFINITY, dq_d = 0.f;          // rows past the sequence or without a visible key: P = 0
  if (qw < lq) {
    const size_t si = hv.stat_off + (size_t)qw * hv.stat_stride;
    const float l = p.lse[si];
    if (l != -INFINITY) lse2 = l * kLog2e;
    dq_d = p.Dvec[si];
  }

  int koff[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) koff[c] = tile_off<ROWB>(l32, 16 * c + 8 * g);
  int ktoff[DT32][2];                         // K^T operand: rows 4g (+8) + (lane%16)/4 (+ block base)
#pragma unroll
  for (int dt = 0; dt < DT32; ++dt) {
    ktoff[dt][0] = tr_off<ROWB>(4 * g, 32 * dt, lane);
    ktoff[dt][1] = tr_off<ROWB>(4 * g + 8, 32 * dt, lane);
  }
  const TileCopy<ROWB, TILE, NW> copy(wave, lane, kv_rstride);

  f32x16 acc[DT32];
#pragma unroll
  for (int t = 0; t < DT32; ++t) acc[t] = f32x16{};
  const float c2 = p.scale_log2;

  // asynchronous copy of key tile j into LDS buffer buf (keys past the sequence arrive as zeros)
  auto gload = [&](int j, int buf) {
    char* kt = smem + buf * 2 * TILE;
    copy.issue(k_rs, kt, j * BN * kv_rstride);
    copy.issue(v_rs, kt + TILE, j * BN * kv_rstride);
  };

  int j = next_kept(0);
  if (j < j_end) gload(j, 0);
  wait_tile_copies();
  __syncthreads();
  int buf = 0;

  while (j < j_end) {
    const int jn = next_kept(j + 1);
    if (jn < j_end) gload(jn, buf ^ 1);       // that buffer was last read before the previous barrier
    const char* kt = smem + buf * 2 * TILE;
    const char* vt = kt + TILE;
    const int k0 = j * BN;
    // a wave none of whose rows sees the tile only takes its part in the copies and barriers
    if (w0 < lq && (!p.causal || k0 <= w0 + 31 + off)) {
      const bool edge = (k0 + BN > lk) || (p.causal && k0 + BN - 1 > q0 + off);

#pragma unroll
      for (int t = 0; t < NS; ++t) {
        // S^T and dP^T: rows = keys k0 + 32 t + mrow, column = this lane's query
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          s = DT::mma(as_v8<DT>(lds_read16(kt, koff[c] + 32 * t * ROWB)), qf[c], s);
          dp = DT::mma(as_v8<DT>(lds_read16(vt, koff[c] + 32 * t * ROWB)), of[c], dp);
        }
        float de[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) de[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -lse2));
        if (edge) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * t + mrow(g, r);
            if (key >= lk || (p.causal && key > qw + off)) de[r] = 0.f;
          }
        }
        if constexpr (DROP) {                 // dP = Z o (dO V^T), Z = M / (1 - p)
          // keys k0 + 32 t + 8 jj + 4 g + u sit in register 4 jj + u (as in the forward)
          const uint32_t kb16 = keep16_pair(p.drop, (uint32_t)((k0 + 32 * t) >> 2), (uint32_t)qw, (uint32_t)bh, lane);
#pragma unroll
          for (int r = 0; r < 16; ++r) dp[r] = ((kb16 >> r) & 1) ? dp[r] * p.drop.rescale : 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) de[r] *= dp[r] - dq_d;
        V8 sb[2];
        sb[0] = pack8<DT>(de[0], de[1], de[2], de[3], de[4], de[5], de[6], de[7]);
        sb[1] = pack8<DT>(de[8], de[9], de[10], de[11], de[12], de[13], de[14], de[15]);
        // dQ^T += K^T dS^T over these 32 keys
#pragma unroll
        for (int dt = 0; dt < DT32; ++dt) {
#pragma unroll
          for (int h = 0; h < 2; ++h)
            acc[dt] = DT::mma(tr_pair<DT>(kt, ktoff[dt][0] + (32 * t + 16 * h) * ROWB,
                                          ktoff[dt][1] + (32 * t + 16 * h) * ROWB), sb[h], acc[dt]);
        }
      }
    }

    wait_tile_copies();
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  // ---- epilogue: lane holds query qw, dims 32 dt + mrow(g, r); rows q0 + 32 wave..
  // go out through this wave's part of the (now idle) tile buffers
  static_assert(NW * stage_bytes<D>() <= SMEM, "staging fits the shared buffer");
  store_tile_rows<DT, D>(acc, p.scale, smem + wave * stage_bytes<D>(),
                         reinterpret_cast<T*>(p.dq) + hv.q_off + (size_t)(q0 + wave * 32) * hv.q_stride, hv.q_stride,
                         min(32, lq - (q0 + wave * 32)), lane);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_bwd_preprocess(const void* o, const void* dO, float* Dvec, long long rows, int D,
                                 int is_bf16, hipStream_t st) {
  const int rpb = 256 / (D / 8);
  const unsigned blocks = (unsigned)((rows + rpb - 1) / rpb);
  if (D == 64) {
    if (is_bf16) hipLaunchKernelGGL((preprocess_kernel<BF16, 64>), dim3(blocks), dim3(256), 0, st, o, dO, Dvec, rows);
    else hipLaunchKernelGGL((preprocess_kernel<F16, 64>), dim3(blocks), dim3(256), 0, st, o, dO, Dvec, rows);
  } else {
    if (is_bf16) hipLaunchKernelGGL((preprocess_kernel<BF16, 128>), dim3(blocks), dim3(256), 0, st, o, dO, Dvec, rows);
    else hipLaunchKernelGGL((preprocess_kernel<F16, 128>), dim3(blocks), dim3(256), 0, st, o, dO, Dvec, rows);
  }
  return hipGetLastError();
}

// dq_kernel over 128-query blocks (256 at d = 128 on the dense layout without
// block mask or dropout), then the dK/dV kernel over 128-key blocks:
// dkdv_kernel (4 waves, 128-query tiles) at d = 64, dkdv_split_kernel (8 waves,
// 64-query tiles) at d = 128.
template <class DT, int D, int BN_DQ>
static hipError_t launch_bwd_t(const BwdParams& p0, hipStream_t st) {
  BwdParams p = p0;
  constexpr int NW = 4;
  constexpr int BM = NW * 32;
  p.q_blocks = (p.N + BM - 1) / BM;
  p.k_blocks = (p.L.Nk + 127) / 128;
  p.total_blocks = p.B * p.H * p.q_blocks;
  bool wide = false;
  if constexpr (D == 128) {
    // dense layout without block mask or dropout: 8-wave workgroups (256 query rows)
    // share each K/V tile (causal N=65536: HBM reads 2.67 -> 1.77 GB, 11.21 -> 10.97
    // ms; N=8192 unchanged), when there are at least kWideMinBlocks of them (causal
    // B1 H8 N4096 backward with 4-wave dQ workgroups instead: 0.26 -> 0.24 ms)
    wide = !p.drop.on && p.mask == nullptr && p.L.cu_q == nullptr &&
           (long long)p.B * p.H * ((p.N + 255) / 256) >= kWideMinBlocks;
    if (wide) {
      BwdParams p8 = p;
      p8.q_blocks = (p.N + 255) / 256;
      p8.total_blocks = p.B * p.H * p8.q_blocks;
      hipLaunchKernelGGL((dq_kernel<DT, D, BN_DQ, 8, false>), dim3(p8.total_blocks), dim3(512), 0, st, p8);
    }
  }
  if (p.drop.on) hipLaunchKernelGGL((dq_kernel<DT, D, BN_DQ, NW, true>), dim3(p.total_blocks), dim3(NW * 64), 0, st, p);
  else if (!wide) hipLaunchKernelGGL((dq_kernel<DT, D, BN_DQ, NW, false>), dim3(p.total_blocks), dim3(NW * 64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  p.total_blocks = p.B * p.L.Hk * p.k_blocks;
  if constexpr (D == 64) {
    if (p.drop.on) hipLaunchKernelGGL((dkdv_kernel<DT, D, 128, NW, true>), dim3(p.total_blocks), dim3(NW * 64), 0, st, p);
    else hipLaunchKernelGGL((dkdv_kernel<DT, D, 128, NW, false>), dim3(p.total_blocks), dim3(NW * 64), 0, st, p);
  } else {
    if (p.drop.on) hipLaunchKernelGGL((dkdv_split_kernel<DT, D, 64, true>), dim3(p.total_blocks), dim3(512), 0, st, p);
    else hipLaunchKernelGGL((dkdv_split_kernel<DT, D, 64, false>), dim3(p.total_blocks), dim3(512), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int is_bf16, hipStream_t st) {
  if (p.D == 64) {
    return is_bf16 ? launch_bwd_t<BF16, 64, 64>(p, st) : launch_bwd_t<F16, 64, 64>(p, st);
  }
  return is_bf16 ? launch_bwd_t<BF16, 128, 64>(p, st) : launch_bwd_t<F16, 128, 64>(p, st);
}

}  // namespace fa
