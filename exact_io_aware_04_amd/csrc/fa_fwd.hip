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

template <class DT, int D, int BN, int NW>
__global__ __launch_bounds__(NW * 64, 2) void fwd_kernel(FwdParams p) {
  using T = typename DT::T;
  using V8 = typename DT::V8;
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int ROWB = D * 2;                 // bytes per K/V row
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int TILE = BN * ROWB;
  constexpr int KC = D / 16;                  // contraction chunks over d
  constexpr int NS = BN / 32;                 // 32-key sub-tiles per tile
  constexpr int DT32 = D / 32;
  static_assert(128 % BM == 0 && 128 % BN == 0, "block-mask granularity");

  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int N = p.N;

  const int logical = xcd_remap(blockIdx.x, p.total_blocks);
  const int bh = logical / p.q_blocks;
  int qb = logical - bh * p.q_blocks;
  if (p.causal) qb = p.q_blocks - 1 - qb;     // longest rows first
  const int q0 = qb * BM;
  const int qw = q0 + wave * 32 + l32;        // this lane's query row
  const int b = bh / p.H, h = bh - b * p.H;
  const HeadView hv = head_view(p.L, b, h, p.H, N, D);
  const int lq = hv.lq, lk = hv.lk;
  if (q0 >= lq) return;                       // uniform: this block has no rows of its sequence
  const int off = lk - lq;                    // causal: query i sees keys j <= i + off

  const auto q_rs = make_rsrc(reinterpret_cast<const T*>(p.q) + hv.q_off, span_bytes(lq, hv.q_stride, D, 2));
  const auto k_rs = make_rsrc(reinterpret_cast<const T*>(p.k) + hv.kv_off, span_bytes(lk, hv.kv_stride, D, 2));
  const auto v_rs = make_rsrc(reinterpret_cast<const T*>(p.v) + hv.kv_off, span_bytes(lk, hv.kv_stride, D, 2));
  const int kv_rstride = hv.kv_stride * 2;    // bytes between key rows

  // ---- key-tile range and skipping
  const int n_tiles = (lk + BN - 1) / BN;
  int j_end = n_tiles;
  if (p.causal) {
    const int last_vis = min(q0 + BM, lq) - 1 + off;   // last key any row of this block sees
    j_end = last_vis < 0 ? 0 : min(n_tiles, last_vis / BN + 1);
  }
  const uint8_t* __restrict__ mrow_ptr = p.mask ? p.mask + (size_t)(q0 / 128) * p.mask_tiles : nullptr;
  auto kept = [&](int j) { return mrow_ptr == nullptr || mrow_ptr[(j * BN) / 128] != 0; };
  auto next_kept = [&](int j) { while (j < j_end && !kept(j)) ++j; return j; };

  // ---- Q fragments (B operand of S^T): lane holds Q[qw][16c + 8g .. +7]; rows >= N read as zero
  V8 qf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) qf[c] = as_v8<DT>(buf_load16(q_rs, (qw * hv.q_stride + 16 * c + 8 * g) * 2));

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

  int j = next_kept(0);
  if (j < j_end) gload(j, 0);
  wait_tile_copies();
  __syncthreads();
  int buf = 0;

  while (j < j_end) {
    const int jn = next_kept(j + 1);
    if (jn < j_end) gload(jn, buf ^ 1);     // that buffer was last read before the previous barrier

    const char* kt = smem + buf * 2 * TILE;
    const char* vt = kt + TILE;
    const int k0 = j * BN;

    // S^T sub-tiles: rows = keys k0 + 32 t + mrow, column = this lane's query
    f32x16 s[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      s[t] = f32x16{};
#pragma unroll
      for (int c = 0; c < KC; ++c) s[t] = DT::mma(as_v8<DT>(lds_read16(kt, koff[c] + 32 * t * ROWB)), qf[c], s[t]);
    }

    if ((k0 + BN > lk) || (p.causal && k0 + BN - 1 > q0 + off)) {
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * t + mrow(g, r);
          if (key >= lk || (p.causal && key > qw + off)) s[t][r] = -INFINITY;
        }
    }

    // row maximum of this tile (raw scores; the scale is positive)
    float mx = -INFINITY;
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
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

    // probabilities relative to m_use, packed as B operands of O^T += V^T P^T;
    // the row-sum share adds exactly the rounded values the product uses
    V8 pb[NS][2];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(s[t][r], c2, -m_use));
      pb[t][0] = pack8<DT>(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      pb[t][1] = pack8<DT>(e[8], e[9], e[10], e[11], e[12], e[13], e[14], e[15]);
      l_run = sum8<DT>(pb[t][0], l_run);
      l_run = sum8<DT>(pb[t][1], l_run);
    }

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

    wait_tile_copies();
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  // ---- epilogue: O = O~ / l, LSE = m ln2 + ln l
  {
    const float l_tot = pair_sum(l_run);
    if (qw < lq) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      T* __restrict__ Og = reinterpret_cast<T*>(p.o) + hv.q_off + (size_t)qw * hv.q_stride;
#pragma unroll
      for (int dt = 0; dt < DT32; ++dt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          u32x2 w = pack4<DT>(acc[dt][4 * jj] * inv, acc[dt][4 * jj + 1] * inv,
                              acc[dt][4 * jj + 2] * inv, acc[dt][4 * jj + 3] * inv);
          *reinterpret_cast<u32x2*>(Og + 32 * dt + 8 * jj + 4 * g) = w;
        }
      if (g == 0) {
        p.lse[hv.stat_off + (size_t)qw * hv.stat_stride] = l_tot > 0.f ? fmaf(m_run, kLn2, __logf(l_tot)) : -INFINITY;
      }
    }
  }
}

template <class DT, int D, int BN, int NW>
static hipError_t launch_fwd_t(const FwdParams& p0, hipStream_t st) {
  FwdParams p = p0;
  constexpr int BM = NW * 32;
  p.q_blocks = (p.N + BM - 1) / BM;
  p.total_blocks = p.B * p.H * p.q_blocks;
  hipLaunchKernelGGL((fwd_kernel<DT, D, BN, NW>), dim3(p.total_blocks), dim3(NW * 64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, int is_bf16, hipStream_t st) {
  if (p.D == 64) {
    return is_bf16 ? launch_fwd_t<BF16, 64, 128, 4>(p, st) : launch_fwd_t<F16, 64, 128, 4>(p, st);
  }
  return is_bf16 ? launch_fwd_t<BF16, 128, 64, 4>(p, st) : launch_fwd_t<F16, 128, 64, 4>(p, st);
}

}  // namespace fa
