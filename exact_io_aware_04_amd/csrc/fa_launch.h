// Kernel parameter blocks and launchers shared by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

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
  int q_blocks;          // set by the launcher
  int k_blocks;          // set by the launcher
  int total_blocks;      // set by the launcher
};

hipError_t launch_fwd(const FwdParams& p, int is_bf16, hipStream_t st);
hipError_t launch_bwd_preprocess(const void* o, const void* dO, float* Dvec, long long rows, int D,
                                 int is_bf16, hipStream_t st);
hipError_t launch_bwd(const BwdParams& p, int is_bf16, hipStream_t st);

}  // namespace fa
