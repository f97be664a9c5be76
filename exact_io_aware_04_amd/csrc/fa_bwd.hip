// Attention backward for gfx950: recompute P tile by tile from Q, K and the
// saved log-sum-exp, and form dV, dK (on chip, per key block) and dQ (fp32
// atomics into a workspace).
//
// Method: page 1 ("FlashAttention：不减少一次注意力计算，为什么反而更快"), key design 3:
// P_ij is rebuilt from the saved row statistic, D_i = dO_i . O_i replaces the
// row-wide reduction, dS = P o (dP - D), dV = P^T dO, dQ = dS K, dK = dS^T Q;
// page 2 ("FlashAttention 入门"), backward section: dQ is accumulated across
// blocks with atomic adds (so the backward is not bitwise deterministic).
// The softmax scale s enters S = s Q K^T, so dQ and dK carry a factor s.
//
// Work decomposition (one workgroup = NW waves = NW*32 keys of one head):
//   * each wave keeps its 32 rows of K and V in VGPRs (B operands of
//     S = Q K^T and dP = dO V^T) and its 32 x D fp32 dK^T / dV^T accumulators;
//   * Q / dO tiles of BQ rows stream through LDS (double buffered);
//   * S and dP are computed with queries on the accumulator's register index
//     and keys on its lane index, so P and dS feed dV^T = dO^T P and
//     dK^T = Q^T dS directly as B operands (contraction over queries), with
//     dO^T / Q^T read from LDS by the transpose read;
//   * dS^T of all NW waves goes to LDS; the waves then share the BQ x D dQ
//     tile (contraction over the workgroup's keys) and add it to the fp32
//     workspace with atomics.
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

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ x, long long n) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    *reinterpret_cast<f32x4*>(x + i) = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    for (long long t = i; t < n; ++t) x[t] = 0.f;
  }
}

template <class DT>
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc, void* __restrict__ dq_,
                                                         long long n, float scale) {
  const long long i = ((long long)blockIdx.x * 256 + threadIdx.x) * 4;
  typename DT::T* dq = reinterpret_cast<typename DT::T*>(dq_);
  if (i + 3 < n) {
    f32x4 v = *reinterpret_cast<const f32x4*>(acc + i);
    *reinterpret_cast<u32x2*>(dq + i) = pack4<DT>(v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale);
  } else {
    for (long long t = i; t < n; ++t) dq[t] = (typename DT::T)(acc[t] * scale);
  }
}

// ---------------------------------------------------------------------------
// Main backward kernel
// ---------------------------------------------------------------------------
template <int D>
struct BwdOccupancy { static constexpr int value = D <= 64 ? 2 : 1; };

template <class DT, int D, int BQ, int NW>
__global__ __launch_bounds__(NW * 64, BwdOccupancy<D>::value) void bwd_kernel(BwdParams p) {
  using T = typename DT::T;
  using V8 = typename DT::V8;
  constexpr int NT = NW * 64;
  constexpr int BK = NW * 32;                 // keys per workgroup
  constexpr int ROWB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int QTILE = BQ * ROWB;
  constexpr int SROWB = BQ * 2;               // dS^T rows: keys, columns: queries
  constexpr int STILE = BK * SROWB;
  constexpr int KC = D / 16;
  constexpr int MQ = BQ / 32;                 // 32-query halves per tile
  constexpr int DT32 = D / 32;
  constexpr int PER_T = BQ * CPR / NT;        // Q/dO chunks per thread
  constexpr int KPER_T = BK * CPR / NT;
  constexpr int DQ_TILES = MQ * DT32;
  constexpr int DQ_PER_WAVE = DQ_TILES / NW;
  static_assert(PER_T * NT == BQ * CPR && KPER_T * NT == BK * CPR, "copy split");
  static_assert(DQ_PER_WAVE * NW == DQ_TILES && DQ_PER_WAVE >= 1, "dQ split");
  static_assert(NW % DT32 == 0 || DT32 % NW == 0, "dQ tiles per wave share one head-dim block");
  static_assert(BK == 128 && 128 % BQ == 0, "block-mask granularity");
  static_assert(2 * QTILE >= BK * ROWB, "K staging fits the second Q/dO buffer pair");

  // [Q buf0 | dO buf0 | Q buf1 | dO buf1 | dS^T | lse2 x2 | D x2]; the K tile is
  // staged once in the buf1 pair before the first Q/dO tile lands there.
  __shared__ __attribute__((aligned(16))) char smem[4 * QTILE + STILE + 4 * BQ * 4];
  char* const ds_s = smem + 4 * QTILE;
  float* const lse_s = reinterpret_cast<float*>(ds_s + STILE);   // [2][BQ]
  float* const dd_s = lse_s + 2 * BQ;                              // [2][BQ]
  char* const k_s = smem + 2 * QTILE;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int N = p.N;

  const int logical = xcd_remap(blockIdx.x, p.total_blocks);
  const int bh = logical / p.k_blocks;
  const int kb = logical - bh * p.k_blocks;   // causal: low key blocks carry the most rows, run first
  const int k0 = kb * BK;
  const int kw0 = k0 + wave * 32;
  const int kw = kw0 + l32;                   // this lane's key (column of S and dP)

  const size_t hoff = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const auto q_rs = make_rsrc(reinterpret_cast<const T*>(p.q) + hoff, head_bytes);
  const auto k_rs = make_rsrc(reinterpret_cast<const T*>(p.k) + hoff, head_bytes);
  const auto v_rs = make_rsrc(reinterpret_cast<const T*>(p.v) + hoff, head_bytes);
  const auto do_rs = make_rsrc(reinterpret_cast<const T*>(p.dO) + hoff, head_bytes);
  const auto dq_rs = make_rsrc(p.dq_acc + hoff, (uint32_t)N * D * 4);
  const float* __restrict__ lse_g = p.lse + (size_t)bh * N;
  const float* __restrict__ D_g = p.Dvec + (size_t)bh * N;

  // ---- K, V fragments (B operands of S = Q K^T and dP = dO V^T); keys >= N read as zero
  V8 kf[KC], vf[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    kf[c] = as_v8<DT>(buf_load16(k_rs, (kw * D + 16 * c + 8 * g) * 2));
    vf[c] = as_v8<DT>(buf_load16(v_rs, (kw * D + 16 * c + 8 * g) * 2));
  }
  // ---- K tile to LDS, read back transposed as the B operand of dQ = dS K
#pragma unroll
  for (int u = 0; u < KPER_T; ++u) {
    const int idx = tid + u * NT;
    const int r = idx / CPR, c = idx % CPR;
    lds_write16(k_s, tile_off<ROWB>(r, 8 * c), buf_load16(k_rs, ((k0 + r) * D + 8 * c) * 2));
  }

  // ---- lane-constant LDS offsets
  int qoff[KC];                               // Q / dO operand rows l32, chunk 2c + g
#pragma unroll
  for (int c = 0; c < KC; ++c) qoff[c] = tile_off<ROWB>(l32, 16 * c + 8 * g);
  int troff[DT32];                            // dO^T / Q^T operands: rows 4g + (lane%16)/4 (+ block base)
#pragma unroll
  for (int d0 = 0; d0 < DT32; ++d0) troff[d0] = tr_off<ROWB>(4 * g, 32 * d0, lane);
  // dQ work of this wave: head-dim block dq_d0, query halves dq_mq0 .. dq_mq0 + DQ_PER_WAVE - 1
  const int dq_d0 = wave % DT32;
  const int dq_mq0 = (wave / DT32) * DQ_PER_WAVE;
  // (a column shift is not additive under the row swizzle, so one offset per tile)
  int dsoff[DQ_PER_WAVE];
#pragma unroll
  for (int w = 0; w < DQ_PER_WAVE; ++w) dsoff[w] = tr_off<SROWB>(4 * g, 32 * (dq_mq0 + w), lane);

  // ---- query-tile range and skipping
  const int n_qt = (N + BQ - 1) / BQ;
  const int i_begin = p.causal ? k0 / BQ : 0;
  const uint8_t* __restrict__ mcol = p.mask ? p.mask + (k0 / 128) : nullptr;
  auto kept = [&](int i) { return mcol == nullptr || mcol[(size_t)((i * BQ) / 128) * p.mask_tiles] != 0; };
  auto next_kept = [&](int i) { while (i < n_qt && !kept(i)) ++i; return i; };

  int goff[PER_T], soff[PER_T];
#pragma unroll
  for (int u = 0; u < PER_T; ++u) {
    const int idx = tid + u * NT;
    const int r = idx / CPR, c = idx % CPR;
    goff[u] = (r * D + 8 * c) * 2;
    soff[u] = tile_off<ROWB>(r, 8 * c);
  }
  u32x4 qr[PER_T], dr[PER_T];
  float lse_r = 0.f, dd_r = 0.f;
  auto gload = [&](int i) {
    const int base = i * BQ * D * 2;          // rows >= N read as zero
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      qr[u] = buf_load16(q_rs, goff[u] + base);
      dr[u] = buf_load16(do_rs, goff[u] + base);
    }
    if (tid < BQ) {
      const int q = i * BQ + tid;
      const float l = q < N ? lse_g[q] : -INFINITY;
      // rows past N or with no visible key get P = exp2(s - inf) = 0
      lse_r = (l == -INFINITY) ? INFINITY : l * kLog2e;
      dd_r = q < N ? D_g[q] : 0.f;
    }
  };
  auto sstore = [&](int buf) {
    char* qt = smem + buf * 2 * QTILE;
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      lds_write16(qt, soff[u], qr[u]);
      lds_write16(qt + QTILE, soff[u], dr[u]);
    }
    if (tid < BQ) {
      lse_s[buf * BQ + tid] = lse_r;
      dd_s[buf * BQ + tid] = dd_r;
    }
  };

  f32x16 dv[DT32], dk[DT32];
#pragma unroll
  for (int t = 0; t < DT32; ++t) { dv[t] = f32x16{}; dk[t] = f32x16{}; }

  const float c2 = p.scale_log2;
  int i = next_kept(i_begin);
  if (i < n_qt) {
    gload(i);
    sstore(0);
  }
  __syncthreads();
  V8 ktf[BK / 16];                            // K[keys of chunk kc][dim 32 dq_d0 + l32]
  {
    const int koff = tr_off<ROWB>(4 * g, 32 * dq_d0, lane);
#pragma unroll
    for (int kc = 0; kc < BK / 16; ++kc) ktf[kc] = tr_pair<DT>(k_s, koff + 16 * kc * ROWB, 8 * ROWB);
  }
  int buf = 0;

  while (i < n_qt) {
    const int in = next_kept(i + 1);
    if (in < n_qt) gload(in);
    const int q0 = i * BQ;
    const char* qt = smem + buf * 2 * QTILE;
    const char* ot = qt + QTILE;
    const float* lt = lse_s + buf * BQ;
    const float* dl = dd_s + buf * BQ;
    const bool edge = (kw0 + 32 > N) || (p.causal && kw0 + 31 > q0);

#pragma unroll
    for (int mq = 0; mq < MQ; ++mq) {
      // S and dP for queries q0 + 32 mq + mrow (registers) x this lane's key
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        s = DT::mma(as_v8<DT>(lds_read16(qt, qoff[c] + 32 * mq * ROWB)), kf[c], s);
        dp = DT::mma(as_v8<DT>(lds_read16(ot, qoff[c] + 32 * mq * ROWB)), vf[c], dp);
      }
      float pe[16], de[16];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + 32 * mq + 8 * jj + 4 * g);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dl + 32 * mq + 8 * jj + 4 * g);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * jj + u;
          pe[r] = __builtin_amdgcn_exp2f(fmaf(s[r], c2, -l4[u]));
          de[r] = dp[r] - d4[u];
        }
      }
      if (edge) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + 32 * mq + mrow(g, r);
          if (kw >= N || (p.causal && kw > q)) pe[r] = 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) de[r] *= pe[r];
      // B operands: slot i of half h <-> query 32 mq + 16 h + 8 (i / 4) + 4 g + i % 4
      V8 pb[2], sb[2];
      pb[0] = pack8<DT>(pe[0], pe[1], pe[2], pe[3], pe[4], pe[5], pe[6], pe[7]);
      pb[1] = pack8<DT>(pe[8], pe[9], pe[10], pe[11], pe[12], pe[13], pe[14], pe[15]);
      sb[0] = pack8<DT>(de[0], de[1], de[2], de[3], de[4], de[5], de[6], de[7]);
      sb[1] = pack8<DT>(de[8], de[9], de[10], de[11], de[12], de[13], de[14], de[15]);
      // dS^T row (this lane's key) for dQ: each half of sb holds 4 consecutive queries
      {
        const int row = wave * 32 + l32;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w = __builtin_bit_cast(u32x4, sb[h]);
          const int qb0 = 32 * mq + 16 * h + 4 * g;
          lds_write8(ds_s, tile_off<SROWB>(row, qb0), u32x2{w.x, w.y});
          lds_write8(ds_s, tile_off<SROWB>(row, qb0 + 8), u32x2{w.z, w.w});
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS (contraction over these 32 queries)
#pragma unroll
      for (int d0 = 0; d0 < DT32; ++d0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int off = troff[d0] + (32 * mq + 16 * h) * ROWB;
          dv[d0] = DT::mma(tr_pair<DT>(ot, off, 8 * ROWB), pb[h], dv[d0]);
          dk[d0] = DT::mma(tr_pair<DT>(qt, off, 8 * ROWB), sb[h], dk[d0]);
        }
      }
    }

    __syncthreads();   // dS^T of every wave is in LDS

    // dQ tile(s): rows = queries, columns = head dims; contraction over the BK keys
#pragma unroll
    for (int w = 0; w < DQ_PER_WAVE; ++w) {
      const int mq = dq_mq0 + w;
      f32x16 a = f32x16{};
#pragma unroll
      for (int kc = 0; kc < BK / 16; ++kc)
        a = DT::mma(tr_pair<DT>(ds_s, dsoff[w] + 16 * kc * SROWB, 8 * SROWB), ktf[kc], a);
      const int vbase = ((q0 + 32 * mq + 4 * g) * D + 32 * dq_d0 + l32) * 4;   // rows >= N dropped
#pragma unroll
      for (int r = 0; r < 16; ++r) buf_atomic_add(dq_rs, vbase + (8 * (r >> 2) + (r & 3)) * D * 4, a[r]);
    }

    if (in < n_qt) sstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    i = in;
  }

  // ---- epilogue: lane holds key kw, dims 32 d0 + mrow(g, r)
  if (kw < N) {
    T* __restrict__ dkg = reinterpret_cast<T*>(p.dk) + hoff + (size_t)kw * D;
    T* __restrict__ dvg = reinterpret_cast<T*>(p.dv) + hoff + (size_t)kw * D;
    const float sc = p.scale;
#pragma unroll
    for (int d0 = 0; d0 < DT32; ++d0)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int col = 32 * d0 + 8 * jj + 4 * g;
        *reinterpret_cast<u32x2*>(dkg + col) =
            pack4<DT>(dk[d0][4 * jj] * sc, dk[d0][4 * jj + 1] * sc, dk[d0][4 * jj + 2] * sc, dk[d0][4 * jj + 3] * sc);
        *reinterpret_cast<u32x2*>(dvg + col) =
            pack4<DT>(dv[d0][4 * jj], dv[d0][4 * jj + 1], dv[d0][4 * jj + 2], dv[d0][4 * jj + 3]);
      }
  }
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

hipError_t launch_fill_zero(float* x, long long n, hipStream_t st) {
  const unsigned blocks = (unsigned)((n + 1023) / 1024);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, x, n);
  return hipGetLastError();
}

hipError_t launch_dq_convert(const float* acc, void* dq, long long n, float scale, int is_bf16,
                             hipStream_t st) {
  const unsigned blocks = (unsigned)((n + 1023) / 1024);
  if (is_bf16) hipLaunchKernelGGL((dq_convert_kernel<BF16>), dim3(blocks), dim3(256), 0, st, acc, dq, n, scale);
  else hipLaunchKernelGGL((dq_convert_kernel<F16>), dim3(blocks), dim3(256), 0, st, acc, dq, n, scale);
  return hipGetLastError();
}

template <class DT, int D, int BQ, int NW>
static hipError_t launch_bwd_t(const BwdParams& p0, hipStream_t st) {
  BwdParams p = p0;
  constexpr int BK = NW * 32;
  p.k_blocks = (p.N + BK - 1) / BK;
  p.total_blocks = p.B * p.H * p.k_blocks;
  hipLaunchKernelGGL((bwd_kernel<DT, D, BQ, NW>), dim3(p.total_blocks), dim3(NW * 64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, int is_bf16, hipStream_t st) {
  if (p.D == 64) {
    return is_bf16 ? launch_bwd_t<BF16, 64, 64, 4>(p, st) : launch_bwd_t<F16, 64, 64, 4>(p, st);
  }
  return is_bf16 ? launch_bwd_t<BF16, 128, 64, 4>(p, st) : launch_bwd_t<F16, 128, 64, 4>(p, st);
}

}  // namespace fa
