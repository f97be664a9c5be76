// Fused attention forward for gfx950: O = softmax(scale * Q K^T) V and the row
// log-sum-exp, without writing the N x N score or probability matrices.
//
// Method: page 1 ("FlashAttention：不减少一次注意力计算，为什么反而更快"), key design 1
// (tiling + fusion) and key design 2 (mergeable online-softmax state); page 3
// ("FlashAttention"), forward-process section (unnormalised accumulator O~,
// one division by l at the end); page 2 ("FlashAttention 入门"), FA2 section
// (grid over batch x heads x query blocks, no atomics in the forward) and FA4
// section (rescale the running state only when the maximum moved enough).
//
// Work decomposition (one workgroup = NW waves = NW*32 query rows of one head):
//   * each wave owns 32 query rows; their Q fragments stay in VGPRs for the
//     whole key loop (B operand of S^T = K Q^T, contraction over d);
//   * K/V tiles of BN keys are copied HBM -> LDS directly (buffer loads with
//     the LDS destination), double buffered: the next tile's copy is in
//     flight while the current one is used;
//   * S^T is computed so that each lane owns ONE query and 16 keys per 32-key
//     sub-tile: the row max needs one cross-half exchange, and the
//     probabilities P^T are already laid out as the B operand of
//     O^T = V^T P^T (contraction over keys); V^T comes from LDS with the
//     gfx950 transpose read;
//   * causal tiles strictly above the diagonal and block-mask zero tiles are
//     never loaded; only diagonal / ragged tiles are masked element-wise.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// Rescale the running state only when the running maximum grows by more than
// this (log2 units); between rescales probabilities stay below 2^8.
constexpr float kRescaleThreshold = 8.0f;
// Probabilities below 2^kRescaleThreshold: a lane's share of a tile's row sum at
// or below this bounds every one of its probabilities by the same amount.
constexpr float kPartialSumLimit = 256.0f;
static_assert(kPartialSumLimit == (float)(1 << (int)kRescaleThreshold), "bound of the rescale rule");

// SPLIT = false: one workgroup = NW*32 query rows of one (sequence, head), all
// kept key tiles; writes O and LSE.
// SPLIT = true (split-KV, packed layout): the rows of a workgroup are the
// group-packed rows r = hh * n_q + i of one (sequence, key/value head) (query
// head hk * G + hh, query row i), so a key/value tile is read once for the G
// query heads that share it (decode: n_q small); the kept key tiles of the
// block are cut into n_splits contiguous ranges, one per workgroup, and each
// writes its normalised partial O and LSE in fp32 for splitkv_merge_kernel.
// DROP: dropout on P after the softmax (dense layout, not with SPLIT): the row
// sum uses the undropped probabilities, the product P V the dropped ones, and
// the epilogue applies 1 / (1 - p) with the normalisation.
// Register target (minimum waves per SIMD): four at d = 64 without dropout
// (<= 128 VGPRs), two at d = 64 with the dropout generator inlined (170 VGPRs,
// so three run) and at d = 128.
template <int D, bool DROP>
struct FwdOccupancy { static constexpr int value = (D <= 64 && !DROP) ? 4 : 2; };

template <class DT, int D, int BN, int NW, bool SPLIT, bool DROP>
__global__ __launch_bounds__(NW * 64, (FwdOccupancy<D, DROP>::value)) void fwd_kernel(FwdParams p) {
  using T = typename DT::T;
  using V8 = typename DT::V8;
  constexpr int BM = NW * 32;
  constexpr int ROWB = D * 2;                 // bytes per K/V row
  constexpr int TILE = BN * ROWB;
  constexpr int KC = D / 16;                  // contraction chunks over d
  constexpr int NS = BN / 32;                 // 32-key sub-tiles per tile
  constexpr int DT32 = D / 32;
  // a 256-row block (NW = 8) spans two block-mask rows: launched only without a mask
  static_assert((128 % BM == 0 || BM == 256) && 128 % BN == 0, "block-mask granularity");
  // two K/V tile buffers; the epilogue's output staging reuses them
  constexpr int SMEM = 4 * TILE > NW * stage_bytes<D>() ? 4 * TILE : NW * stage_bytes<D>();
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int N = p.N;

  int logical = xcd_remap(blockIdx.x, p.total_blocks, SPLIT ? p.q_blocks * p.n_splits : p.q_blocks);
  int split = 0;
  if constexpr (SPLIT) {
    split = logical % p.n_splits;
    logical /= p.n_splits;
  }
  int bh = logical / p.q_blocks;
  int qb = logical - bh * p.q_blocks;
  if (p.causal) {                             // longest rows first
    int rank;
    if (!SPLIT && p.L.cu_q == nullptr && (long long)N * D <= kRankedMaxNd &&
        xcd_remap_ranked(blockIdx.x, p.total_blocks, p.q_blocks, bh, rank))
      qb = rank;
    qb = p.q_blocks - 1 - qb;
  }
  const int q0 = qb * BM;
  const int qw = q0 + wave * 32 + l32;        // this lane's row (split-KV: group-packed row)
  const int HB = SPLIT ? p.L.Hk : p.H;        // heads the grid enumerates
  const int b = bh / HB, hb = bh - b * HB;
  const int G = SPLIT ? p.H / p.L.Hk : 1;     // query heads packed into the rows
  const HeadView hv = head_view(p.L, b, SPLIT ? hb * G : hb, p.H, N, D);
  const int lq = hv.lq, lk = hv.lk;
  const int nrows = G * lq;
  if (q0 >= nrows) return;                    // uniform: this block has no rows of its sequence
  const int off = lk - lq;                    // causal: query i sees keys j <= i + off
  // this lane's query head (within the group) and row
  const int hh = SPLIT ? (qw < nrows ? qw / lq : 0) : 0;
  const int qi = SPLIT ? (qw < nrows ? qw - hh * lq : lq) : qw;
  // first / last row index i of the block (a block that straddles two heads spans all of [0, lq))
  int i_min = q0, i_max = min(q0 + BM, lq) - 1;
  if constexpr (SPLIT) {
    const int r_last = min(q0 + BM, nrows) - 1;
    const int h_first = q0 / lq, h_last = r_last / lq;
    i_min = h_first == h_last ? q0 - h_first * lq : 0;
    i_max = h_first == h_last ? r_last - h_last * lq : lq - 1;
  }

  const uint32_t q_span = SPLIT ? (uint32_t)(((size_t)(lq - 1) * hv.q_stride + (size_t)(G - 1) * hv.q_hstep + D) * 2)
                                : span_bytes(lq, hv.q_stride, D, 2);
  const auto q_rs = make_rsrc(reinterpret_cast<const T*>(p.q) + hv.q_off, q_span);
  const auto k_rs = make_rsrc(reinterpret_cast<const T*>(p.k) + hv.kv_off, span_bytes(lk, hv.kv_stride, D, 2));
  const auto v_rs = make_rsrc(reinterpret_cast<const T*>(p.v) + hv.kv_off, span_bytes(lk, hv.kv_stride, D, 2));
  const int kv_rstride = hv.kv_stride * 2;    // bytes between key rows

  // ---- key-tile range and skipping
  const int n_tiles = (lk + BN - 1) / BN;
  int j_end = n_tiles;
  if (p.causal) {
    const int last_vis = i_max + off;         // last key any row of this block sees
    j_end = last_vis < 0 ? 0 : min(n_tiles, last_vis / BN + 1);
  }
  int j_begin = 0;
  if constexpr (SPLIT) {                      // this workgroup's share of the block's key tiles
    const int chunk = (j_end + p.n_splits - 1) / p.n_splits;
    j_begin = min(split * chunk, j_end);
    j_end = min(j_begin + chunk, j_end);
  }
  // first kept key tile >= j (j_end if none): the block-mask row of this query block
  const TileMask mask_row(p.mask ? p.mask + (size_t)(q0 / 128) * p.mask_tiles : nullptr, 1, p.mask_tiles, lane);
  auto next_kept = [&](int j) {
    if (j >= j_end) return j_end;
    const int r = (j * BN) / 128, r2 = mask_row.next(r);
    return r2 == r ? j : min((r2 * 128) / BN, j_end);
  };

  // ---- Q fragments (B operand of S^T): lane holds row qi of its head, d = 16c + 8g .. +7;
  // rows past the sequence read as zero (split-KV: an offset past the buffer range)
  const int qrow_off = SPLIT ? (qw < nrows ? (qi * hv.q_stride + hh * (int)hv.q_hstep) * 2 : 0x7ff00000)
                             : qw * hv.q_stride * 2;
  V8 qf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) qf[c] = as_v8<DT>(buf_load16(q_rs, qrow_off + (16 * c + 8 * g) * 2));

  // ---- lane-constant LDS offsets
  int koff[KC];                               // K operand: row l32, chunk 2c + g
#pragma unroll
  for (int c = 0; c < KC; ++c) koff[c] = tile_off<ROWB>(l32, 16 * c + 8 * g);
  int voff[DT32][2];                          // V^T operand: rows 4g (+8) + (lane%16)/4 (+ 16-row block base)
#pragma unroll
  for (int dt = 0; dt < DT32; ++dt) {
    voff[dt][0] = tr_off<ROWB>(4 * g, 32 * dt, lane);
    voff[dt][1] = tr_off<ROWB>(4 * g + 8, 32 * dt, lane);
  }
  const TileCopy<ROWB, TILE, NW> copy(wave, lane, kv_rstride);

  f32x16 acc[DT32];
#pragma unroll
  for (int t = 0; t < DT32; ++t) acc[t] = f32x16{};
  float m_run = -INFINITY;   // running reference point, in units of scale*log2(e)*s
  float l_run = 0.f;         // this lane's share of the row sum relative to m_run
  const float c2 = p.scale_log2;

  // asynchronous copy of key tile j into LDS buffer buf (keys >= N arrive as zeros)
  auto gload = [&](int j, int buf) {
    char* kt = smem + buf * 2 * TILE;
    copy.issue(k_rs, kt, j * BN * kv_rstride);
    copy.issue(v_rs, kt + TILE, j * BN * kv_rstride);
  };

  int j = next_kept(j_begin);
  if (j < j_end) gload(j, 0);
  wait_tile_copies();
  __syncthreads();

  // a wave with no row of its sequence (split-KV decode: G * n_q rows of 128) only
  // takes its part in the copies and barriers
  const bool wave_live = q0 + __builtin_amdgcn_readfirstlane(wave) * 32 < nrows;

  // One key tile. The loop runs two of these per turn, one per LDS buffer, so
  // that every operand address is a per-lane offset plus an immediate.
  auto step = [&](auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    const int jn = next_kept(j + 1);
    if (jn < j_end) gload(jn, BUF ^ 1);       // that buffer was last read before the previous barrier
    if (!wave_live) {
      wait_tile_copies();
      __syncthreads();
      j = jn;
      return;
    }

    const char* kt = smem + BUF * 2 * TILE;
    const char* vt = kt + TILE;
    const int k0 = j * BN;

    // S^T sub-tiles: rows = keys k0 + 32 t + mrow, column = this lane's query
    f32x16 s[NS];
    if constexpr (D == 128) {
      // K operand rows read as inline assembly, four reads in flight ahead of the
      // products (the compiler's schedule waits for each read just before its
      // product: 7.8 -> 7.6 ms causal N=65536, 1.07 -> 1.03 ms N=8192)
      constexpr int NR = NS * KC, DEP = 4;
      const uint32_t kbase = lds_addr(kt);
      u32x4 ka[NR];
      auto rd = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        ka[i] = rd128_imm<(i / KC) * 32 * ROWB>(kbase + koff[i % KC]);
      };
      static_for<0, DEP>(rd);
#pragma unroll
      for (int t = 0; t < NS; ++t) s[t] = f32x16{};
      static_for<0, NR>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i + DEP < NR) {
          rd(std::integral_constant<int, i + DEP>{});
          lds_wait_n<DEP>(ka[i]);
        } else {
          lds_wait_n<NR - 1 - i>(ka[i]);
        }
        s[i / KC] = DT::mma(as_v8<DT>(ka[i]), qf[i % KC], s[i / KC]);
      });
    } else {
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        s[t] = f32x16{};
#pragma unroll
        for (int c = 0; c < KC; ++c) s[t] = DT::mma(as_v8<DT>(lds_read16(kt, koff[c] + 32 * t * ROWB)), qf[c], s[t]);
      }
    }

    if ((k0 + BN > lk) || (p.causal && k0 + BN - 1 > i_min + off)) {
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * t + mrow(g, r);
          if (key >= lk || (p.causal && key > qi + off)) s[t][r] = -INFINITY;
        }
    }

    // probabilities relative to the reference m_use, packed as B operands of
    // O^T += V^T P^T; returns this lane's share of their sum, which adds
    // exactly the rounded values the product uses
    V8 pb[NS][2];
    auto probs = [&](float m_use) {
      float lt = 0.f;
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(s[t][r], c2, -m_use));
        pb[t][0] = pack8<DT>(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
        pb[t][1] = pack8<DT>(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
        lt = sum8<DT>(pb[t][0], lt);
        lt = sum8<DT>(pb[t][1], lt);
      }
      return lt;
    };
    // Common case: the probabilities against the current reference stay at or
    // below 2^threshold, which this lane's share of their sum bounds; the tile
    // maximum is then not needed. Otherwise (first tile of the row, or a share
    // above the bound): the tile maximum, a rescale if it grew by more than
    // the threshold (the reference point is arbitrary: exact), and the
    // probabilities again.
    float lt = m_run == -INFINITY ? INFINITY : probs(m_run);
    if (__builtin_amdgcn_ballot_w64(!(lt <= kPartialSumLimit))) {
      float mx = -INFINITY;               // row maximum of this tile (raw scores; the scale is positive)
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
      const float m_tile = pair_max(mx) * c2;
      const bool need = m_tile > m_run + kRescaleThreshold;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.f;
        if (need) m_run = m_tile;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT32; ++t) acc[t] *= alpha;
      }
      lt = probs((m_run == -INFINITY) ? 0.f : m_run);
    }
    l_run += lt;
    if constexpr (DROP) {
#pragma unroll
      for (int t = 0; t < NS; ++t) {
        // keys k0 + 32 t + 8 jj + 4 g + u sit in register 4 jj + u: two generator calls
        // per lane, shared with the lane that holds the other query of the row pair
        const uint32_t kb16 = keep16_pair(p.drop, (uint32_t)((k0 + 32 * t) >> 2), (uint32_t)qw, (uint32_t)bh, lane);
        pb[t][0] = keep_mask8<DT>(pb[t][0], kb16);
        pb[t][1] = keep_mask8<DT>(pb[t][1], kb16 >> 8);
      }
    }

    if constexpr (D == 128) {
      // O^T += V^T P^T with the V^T operands from transpose reads in assembly (no
      // wait for the next tile's copy is inserted before them), one 32-dim group
      // of four operands ahead of its products
      static_assert(BN == 64, "four 16-key operand slots per group");
      const uint32_t vbase = lds_addr(vt);
      V8 va[2][4];
      auto issue = [&](auto dtc) {
        constexpr int dt = decltype(dtc)::value, sl = dt & 1;
        va[sl][0] = tr_pair_imm<DT, 0 * ROWB>(vbase + voff[dt][0], vbase + voff[dt][1]);
        va[sl][1] = tr_pair_imm<DT, 16 * ROWB>(vbase + voff[dt][0], vbase + voff[dt][1]);
        va[sl][2] = tr_pair_imm<DT, 32 * ROWB>(vbase + voff[dt][0], vbase + voff[dt][1]);
        va[sl][3] = tr_pair_imm<DT, 48 * ROWB>(vbase + voff[dt][0], vbase + voff[dt][1]);
      };
      issue(std::integral_constant<int, 0>{});
      static_for<0, DT32>([&](auto dtc) {
        constexpr int dt = decltype(dtc)::value, sl = dt & 1;
        if constexpr (dt + 1 < DT32) {
          issue(std::integral_constant<int, dt + 1>{});
          lds_wait_n4<8>(va[sl][0], va[sl][1], va[sl][2], va[sl][3]);
        } else {
          lds_wait_n4<0>(va[sl][0], va[sl][1], va[sl][2], va[sl][3]);
        }
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) acc[dt] = DT::mma(va[sl][kc], pb[kc >> 1][kc & 1], acc[dt]);
      });
    } else {
#pragma unroll
      for (int dt = 0; dt < DT32; ++dt) {
#pragma unroll
        for (int kc = 0; kc < BN / 16; ++kc) {
          const int t = kc >> 1, h = kc & 1;
          const int rb = (32 * t + 16 * h) * ROWB;
          V8 a = tr_pair<DT>(vt, voff[dt][0] + rb, voff[dt][1] + rb);
          acc[dt] = DT::mma(a, pb[t][h], acc[dt]);
        }
      }
    }

    wait_tile_copies();
    __syncthreads();
    j = jn;
  };
  while (j < j_end) {
    step(std::integral_constant<int, 0>{});
    if (j >= j_end) break;
    step(std::integral_constant<int, 1>{});
  }

  // ---- epilogue: O = O~ / l, LSE = m ln2 + ln l
  if constexpr (SPLIT) {
    const float l_tot = pair_sum(l_run);
    if (qw < nrows) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const size_t prow = (size_t)split * p.part_rows + hv.stat_off + (size_t)hh * hv.stat_hstep +
                          (size_t)qi * hv.stat_stride;
      float* __restrict__ Op = p.o_part + prow * D;
#pragma unroll
      for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          f32x4 w = {acc[dt][4 * jj] * inv, acc[dt][4 * jj + 1] * inv, acc[dt][4 * jj + 2] * inv, acc[dt][4 * jj + 3] * inv};
          *reinterpret_cast<f32x4*>(Op + 32 * dt + 8 * jj + 4 * g) = w;
        }
      if (g == 0) p.lse_part[prow] = l_tot > 0.f ? fmaf(m_run, kLn2, __logf(l_tot)) : -INFINITY;
    }
  } else {
    // O rows q0 + 32 wave.. go out through this wave's part of the (now idle) tile buffers
    static_assert(NW * stage_bytes<D>() <= SMEM, "staging fits the shared buffer");
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? (DROP ? p.drop.rescale : 1.f) / l_tot : 0.f;
    store_tile_rows<DT, D>(acc, inv, smem + wave * stage_bytes<D>(),
                           reinterpret_cast<T*>(p.o) + hv.q_off + (size_t)(q0 + wave * 32) * hv.q_stride, hv.q_stride,
                           min(32, lq - (q0 + wave * 32)), lane);
    if (qw < lq && g == 0)
      p.lse[hv.stat_off + (size_t)qw * hv.stat_stride] = l_tot > 0.f ? fmaf(m_run, kLn2, __logf(l_tot)) : -INFINITY;
  }
}

template <class DT, int D, int BN, int NW>
static hipError_t launch_fwd_t(const FwdParams& p0, hipStream_t st) {
  FwdParams p = p0;
  constexpr int BM = NW * 32;
  p.q_blocks = (p.N + BM - 1) / BM;
  p.total_blocks = p.B * p.H * p.q_blocks;
  if constexpr (NW == 4) {
    if (p.drop.on) {
      hipLaunchKernelGGL((fwd_kernel<DT, D, BN, NW, false, true>), dim3(p.total_blocks), dim3(NW * 64), 0, st, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_kernel<DT, D, BN, NW, false, false>), dim3(p.total_blocks), dim3(NW * 64), 0, st, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-KV merge: per packed row r, LSE = log sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s, the (O, LSE) form of the mergeable softmax
// state (page 1, key design 2; page 2, FA2 section: the saved statistic is
// L = m + log l). Splits with no visible key carry LSE_s = -inf and weight 0.
// D / 4 threads per row, one float4 of every partial per thread.
// ---------------------------------------------------------------------------
template <class DT, int D>
__global__ __launch_bounds__(256) void splitkv_merge_kernel(const float* __restrict__ o_part,
                                                            const float* __restrict__ lse_part, void* o_,
                                                            float* __restrict__ lse, long long rows, int n_splits) {
  using T = typename DT::T;
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const long long r = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c4 = threadIdx.x % TPR;
  if (r >= rows) return;
  float m = -INFINITY;
  for (int s = 0; s < n_splits; ++s) m = fmaxf(m, lse_part[(size_t)s * rows + r]);
  T* __restrict__ o = reinterpret_cast<T*>(o_) + (size_t)r * D + 4 * c4;
  if (m == -INFINITY) {                       // no split saw a key
    *reinterpret_cast<u32x2*>(o) = pack4<DT>(0.f, 0.f, 0.f, 0.f);
    if (c4 == 0) lse[r] = -INFINITY;
    return;
  }
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < n_splits; ++s) {
    const float l = lse_part[(size_t)s * rows + r];
    const float w = __expf(l - m);            // exp(-inf) = 0 for empty splits
    if (w == 0.f) continue;
    const f32x4 x = *reinterpret_cast<const f32x4*>(o_part + ((size_t)s * rows + r) * D + 4 * c4);
    wsum += w;
    acc += w * x;
  }
  const float inv = 1.f / wsum;
  *reinterpret_cast<u32x2*>(o) = pack4<DT>(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  if (c4 == 0) lse[r] = m + __logf(wsum);
}

template <class DT, int D, int BN, int NW>
static hipError_t launch_fwd_splitkv_t(const FwdParams& p0, hipStream_t st) {
  FwdParams p = p0;
  constexpr int BM = NW * 32;
  const int G = p.H / p.L.Hk;
  p.q_blocks = (int)(((long long)G * p.N + BM - 1) / BM);
  p.total_blocks = p.B * p.L.Hk * p.q_blocks * p.n_splits;
  hipLaunchKernelGGL((fwd_kernel<DT, D, BN, NW, true, false>), dim3(p.total_blocks), dim3(NW * 64), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.part_rows == 0) return e;
  constexpr int RPB = 256 / (D / 4);
  const unsigned blocks = (unsigned)((p.part_rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((splitkv_merge_kernel<DT, D>), dim3(blocks), dim3(256), 0, st, p.o_part, p.lse_part, p.o, p.lse,
                     p.part_rows, p.n_splits);
  return hipGetLastError();
}

hipError_t launch_fwd_splitkv(const FwdParams& p, int is_bf16, hipStream_t st) {
  if (p.D == 64) {
    return is_bf16 ? launch_fwd_splitkv_t<BF16, 64, 64, 4>(p, st) : launch_fwd_splitkv_t<F16, 64, 64, 4>(p, st);
  }
  return is_bf16 ? launch_fwd_splitkv_t<BF16, 128, 64, 4>(p, st) : launch_fwd_splitkv_t<F16, 128, 64, 4>(p, st);
}

hipError_t launch_fwd(const FwdParams& p, int is_bf16, hipStream_t st) {
  if (p.D == 64) {
    // d = 64, dense layout, without causal masking, block mask or dropout: 8-wave workgroups (256 query
    // rows) share each K/V tile, halving the tile copies per product (with causal masking
    // the coarser diagonal costs more than that saves); grids of fewer than kWideMinBlocks
    // such workgroups run twice as many 4-wave ones
    if (!p.causal && p.mask == nullptr && !p.drop.on && p.L.cu_q == nullptr &&
        (long long)p.B * p.H * ((p.N + 255) / 256) >= kWideMinBlocks)
      return is_bf16 ? launch_fwd_t<BF16, 64, 64, 8>(p, st) : launch_fwd_t<F16, 64, 64, 8>(p, st);
    return is_bf16 ? launch_fwd_t<BF16, 64, 64, 4>(p, st) : launch_fwd_t<F16, 64, 64, 4>(p, st);
  }
  // d = 128, dense layout, without block mask or dropout: 8-wave workgroups (256 query
  // rows) share each K/V tile (causal N=65536: 7.75 -> 7.50 ms, N=8192: 1.10 -> 1.08 ms;
  // a packed batch of sequences up to 4096 long loses more in ragged ends:
  // 0.96 -> 1.16 ms). Grids of fewer than kWideMinBlocks such workgroups leave compute
  // units idle and run twice as many 4-wave ones instead (causal B1 H8 N4096:
  // 0.100 -> 0.075 ms; B3 H5 N1000: 0.032 -> 0.024 ms).
  if (p.mask == nullptr && !p.drop.on && p.L.cu_q == nullptr &&
      (long long)p.B * p.H * ((p.N + 255) / 256) >= kWideMinBlocks)
    return is_bf16 ? launch_fwd_t<BF16, 128, 64, 8>(p, st) : launch_fwd_t<F16, 128, 64, 8>(p, st);
  return is_bf16 ? launch_fwd_t<BF16, 128, 64, 4>(p, st) : launch_fwd_t<F16, 128, 64, 4>(p, st);
}

}  // namespace fa
