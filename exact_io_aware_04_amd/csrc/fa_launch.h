// Kernel parameter blocks and launchers shared by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Where the rows of one (sequence, head) live. Dense: [B, H, N, d] tensors,
// cu_q == nullptr, Hk == H, Nk == N. Packed variable length: token-major
// q/o [total_q, H, d], k/v [total_k, Hk, d], lse/D [total_q, H]; sequence b
// owns rows cu_q[b] .. cu_q[b+1]-1 (clamped to [0, total_q]) and likewise for
// keys; N and Nk are then the longest query / key sequence (grid extent).
struct SeqLayout {
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
  int Hk;
  int Nk;
};

// Dropout on the probabilities (dense layout): element (head bh = b H + h,
// query i, key j) is dropped iff word j % 4 of Philox4x32-10(counter =
// (j / 4, i, bh, offset), key = (seed_lo, seed_hi)) is below threshold; kept
// elements are scaled by rescale = 1 / (1 - p).
struct Dropout {
  int on;
  uint32_t threshold;
  float rescale;
  uint32_t seed_lo, seed_hi, offset;
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const uint8_t* mask;   // nullptr or [mask_tiles][mask_tiles]
  int B, H, N, D;
  int mask_tiles;
  int causal;
  float scale_log2;      // softmax scale * log2(e)
  SeqLayout L;
  Dropout drop;
  // split-KV form (packed layout only): partial results of split s for packed
  // row r = token * H + head at o_part[(s * part_rows + r) * D], lse_part[s * part_rows + r]
  float* o_part;
  float* lse_part;
  int n_splits;
  long long part_rows;
  int q_blocks;          // set by the launcher
  int total_blocks;      // set by the launcher
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dO;
  const float* lse;
  const float* Dvec;
  void* dq;
  void* dk;
  void* dv;
  const uint8_t* mask;
  int B, H, N, D;
  int mask_tiles;
  int causal;
  float scale;
  float scale_log2;
  SeqLayout L;
  Dropout drop;
  int q_blocks;          // set by the launcher
  int k_blocks;          // set by the launcher
  int total_blocks;      // set by the launcher
};

hipError_t launch_fwd(const FwdParams& p, int is_bf16, hipStream_t st);
hipError_t launch_fwd_splitkv(const FwdParams& p, int is_bf16, hipStream_t st);
hipError_t launch_bwd_preprocess(const void* o, const void* dO, float* Dvec, long long rows, int D,
                                 int is_bf16, hipStream_t st);
hipError_t launch_bwd(const BwdParams& p, int is_bf16, hipStream_t st);

}  // namespace fa
