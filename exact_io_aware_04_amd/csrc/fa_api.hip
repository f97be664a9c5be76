// C ABI layer: argument validation (before any HIP call) and kernel dispatch.
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

// A failed launch is reported once on stderr with HIP's own description, then
// surfaces to the caller as FA_ERR_HIP.
fa_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return FA_OK;
  fprintf(stderr, "libfa: %s: %s (%d)\n", where, hipGetErrorString(e), (int)e);
  return FA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

fa_status check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  // element count must fit comfortably in signed 64-bit
  const long double elems = (long double)B * H * (long double)N * d;
  if (elems > 9.0e18L) return FA_ERR_SHAPE;
  // the kernels form byte offsets inside one head in 32-bit signed integers,
  // also for the rows of a last tile that reach past N; N d < 2^29 keeps the
  // head's 16-bit data below 1 GiB, with room for those rows (the largest
  // accepted head is tested)
  if ((long long)N * d >= (1LL << 29)) return FA_ERR_SHAPE;
  // the dispatch grid counts work-items in 32 bits: blocks * 256 threads < 2^32
  const long double blocks = (long double)B * H * ((N + 31) / 32 + 1);
  if (blocks * 256.0L > 4.0e9L) return FA_ERR_SHAPE;
  return FA_OK;
}

// The D preprocess treats its input as rows x d with 64-bit row indices (dense
// [B, H, N] rows, or the total_q x Hq rows of a packed batch): only the
// dispatch grid (rows / (2048 / d) blocks of 256 work-items) limits it.
fa_status check_preprocess_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  const long double rows = (long double)B * H * (long double)N;
  const long double blocks = ceill(rows / (2048.0L / d));
  if (blocks * 256.0L > 4.0e9L) return FA_ERR_SHAPE;
  return FA_OK;
}

fa_status check_dtype(fa_dtype dt) { return (dt == FA_F16 || dt == FA_BF16) ? FA_OK : FA_ERR_DTYPE; }

fa_status check_scale(float s) { return (isfinite(s) && s > 0.f) ? FA_OK : FA_ERR_SCALE; }

fa_status check_mask(const uint8_t* m, int mb) { return (m != nullptr && mb != 128) ? FA_ERR_MASK : FA_OK; }

// Packed variable-length batches: byte offsets inside one (sequence, head) are
// 32-bit (rows up to max_seqlen, heads x d elements apart), and the dispatch
// grids (query blocks of 128 x 256 threads or, for the d = 64 forward without
// causal masking, 256 x 512 threads; key blocks of 128 x 512 threads) count
// work-items in 32 bits.
fa_status check_varlen(int batch, int total_q, int total_k, int max_q, int max_k, int Hq, int Hk, int d) {
  if (batch < 1 || total_q < 0 || total_k < 0 || max_q < 1 || max_k < 1 || Hq < 1 || Hk < 1) return FA_ERR_SHAPE;
  if (Hq % Hk != 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEADDIM;
  if ((long long)max_q * Hq * d * 2 >= (1LL << 31) || (long long)max_k * Hk * d * 2 >= (1LL << 31)) return FA_ERR_SHAPE;
  if ((long long)max_q * Hq * 4 >= (1LL << 31)) return FA_ERR_SHAPE;
  const long double qg = (long double)batch * Hq *
                         fmaxl(((max_q + 127) / 128) * 256.0L, ((max_q + 255) / 256) * 512.0L);
  const long double kg = (long double)batch * Hk * ((max_k + 127) / 128) * 512.0L;
  if (qg > 4.0e9L || kg > 4.0e9L) return FA_ERR_SHAPE;
  return FA_OK;
}

// Dropout parameters: p in [0, 1) (finite); the drop decision compares a 16-bit
// generator draw with floor(p 2^16) and kept values are scaled by 1 / (1 - p).
fa_status make_dropout(float p_drop, uint64_t seed, uint32_t offset, fa::Dropout* d) {
  if (!(p_drop >= 0.f && p_drop < 1.f)) return FA_ERR_DROPOUT;
  d->on = 1;
  const double t = floor((double)p_drop * 65536.0);
  d->threshold = t >= 65535.0 ? 0xFFFFu : (uint32_t)t;
  d->rescale = (float)(1.0 / (1.0 - (double)p_drop));
  d->seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  d->seed_hi = (uint32_t)(seed >> 32);
  d->offset = offset;
  return FA_OK;
}

fa::SeqLayout dense_layout(int H, int N) {
  fa::SeqLayout L{};
  L.cu_q = nullptr;
  L.cu_k = nullptr;
  L.Hk = H;
  L.Nk = N;
  return L;
}

#define FA_TRY(x)                     \
  do {                                \
    fa_status s_ = (x);               \
    if (s_ != FA_OK) return s_;       \
  } while (0)

}  // namespace

extern "C" {

static fa_status fwd_dense(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                           int d, fa_dtype dt, float scale, int causal, const uint8_t* block_mask, int mask_block,
                           const fa::Dropout& drop, void* stream, const char* where) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  FA_TRY(check_shape(B, H, N, d));
  FA_TRY(check_dtype(dt));
  FA_TRY(check_mask(block_mask, mask_block));
  FA_TRY(check_scale(scale));
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;

  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.mask = block_mask;
  p.B = B; p.H = H; p.N = N; p.D = d;
  p.mask_tiles = (N + 127) / 128;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.L = dense_layout(H, N);
  p.drop = drop;
  return hip_status(fa::launch_fwd(p, dt == FA_BF16, reinterpret_cast<hipStream_t>(stream)), where);
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                 int d, fa_dtype dt, float scale, int causal, const uint8_t* block_mask, int mask_block,
                 void* stream) {
  return fwd_dense(q, k, v, o, lse, B, H, N, d, dt, scale, causal, block_mask, mask_block, fa::Dropout{}, stream,
                   "fa_fwd");
}

fa_status fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                         int d, fa_dtype dt, float scale, int causal, const uint8_t* block_mask, int mask_block,
                         float p_drop, uint64_t seed, uint32_t offset, void* stream) {
  fa::Dropout drop{};
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  FA_TRY(make_dropout(p_drop, seed, offset, &drop));
  return fwd_dense(q, k, v, o, lse, B, H, N, d, dt, scale, causal, block_mask, mask_block, drop, stream,
                   "fa_fwd_dropout");
}

static fa_status fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q, int total_k,
                            int max_seqlen_q, int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt, float scale,
                            int causal, const fa::Dropout& drop, void* stream, const char* where) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  FA_TRY(check_varlen(batch, total_q, total_k, max_seqlen_q, max_seqlen_k, Hq, Hk, d));
  FA_TRY(check_dtype(dt));
  FA_TRY(check_scale(scale));
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;

  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.mask = nullptr;
  p.B = batch; p.H = Hq; p.N = max_seqlen_q; p.D = d;
  p.mask_tiles = 0;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.L.cu_q = cu_seqlens_q;
  p.L.cu_k = cu_seqlens_k;
  p.L.total_q = total_q;
  p.L.total_k = total_k;
  p.L.Hk = Hk;
  p.L.Nk = max_seqlen_k;
  p.drop = drop;
  return hip_status(fa::launch_fwd(p, dt == FA_BF16, reinterpret_cast<hipStream_t>(stream)), where);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q, int total_k,
                        int max_seqlen_q, int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt, float scale,
                        int causal, void* stream) {
  return fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k, max_seqlen_q,
                    max_seqlen_k, Hq, Hk, d, dt, scale, causal, fa::Dropout{}, stream, "fa_fwd_varlen");
}

fa_status fa_fwd_varlen_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q,
                                int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hk, int d,
                                fa_dtype dt, float scale, int causal, float p_drop, uint64_t seed, uint32_t offset,
                                void* stream) {
  fa::Dropout drop{};
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  FA_TRY(make_dropout(p_drop, seed, offset, &drop));
  return fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k, max_seqlen_q,
                    max_seqlen_k, Hq, Hk, d, dt, scale, causal, drop, stream, "fa_fwd_varlen_dropout");
}

// Split-KV arguments other than the partial-result buffers.
static fa_status splitkv_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q,
                               int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hk, int d,
                               fa_dtype dt, float scale, int n_splits) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  FA_TRY(check_varlen(batch, total_q, total_k, max_seqlen_q, max_seqlen_k, Hq, Hk, d));
  if (n_splits < 1 || n_splits > FA_MAX_SPLITS) return FA_ERR_SHAPE;
  // group-packed rows (Hq / Hk heads x max_seqlen_q) index the grid in 32 bits
  const long double blocks = (long double)batch * Hk * (((long double)(Hq / Hk) * max_seqlen_q + 127) / 128) * n_splits;
  if (blocks * 256.0L > 4.0e9L) return FA_ERR_SHAPE;
  FA_TRY(check_dtype(dt));
  FA_TRY(check_scale(scale));
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  return FA_OK;
}

static fa_status splitkv_launch(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q,
                                int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt,
                                float scale, int causal, int n_splits, float* o_partial, float* lse_partial,
                                void* stream, const char* where) {
  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.mask = nullptr;
  p.B = batch; p.H = Hq; p.N = max_seqlen_q; p.D = d;
  p.mask_tiles = 0;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.L.cu_q = cu_seqlens_q;
  p.L.cu_k = cu_seqlens_k;
  p.L.total_q = total_q;
  p.L.total_k = total_k;
  p.L.Hk = Hk;
  p.L.Nk = max_seqlen_k;
  p.o_part = o_partial;
  p.lse_part = lse_partial;
  p.n_splits = n_splits;
  p.part_rows = (long long)total_q * Hq;
  return hip_status(fa::launch_fwd_splitkv(p, dt == FA_BF16, reinterpret_cast<hipStream_t>(stream)), where);
}

fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q, int total_k,
                         int max_seqlen_q, int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt, float scale,
                         int causal, int n_splits, float* o_partial, float* lse_partial, void* stream) {
  FA_TRY(splitkv_check(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k, max_seqlen_q,
                       max_seqlen_k, Hq, Hk, d, dt, scale, n_splits));
  if (!o_partial || !lse_partial) return FA_ERR_NULL;
  if (!aligned16(o_partial) || !aligned16(lse_partial)) return FA_ERR_ALIGN;
  return splitkv_launch(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k, max_seqlen_q,
                        max_seqlen_k, Hq, Hk, d, dt, scale, causal, n_splits, o_partial, lse_partial, stream,
                        "fa_fwd_splitkv");
}

// ---------------------------------------------------------------------------
// Split-KV without allocation: the partial results live in this file-scope
// device array instead of caller-provided workspace. Each GPU the library runs
// on holds its own copy (FA_NOALLOC_SCRATCH_BYTES) until the process ends. In
// host code `scratch` only names the symbol; its device address is looked up
// with hipGetSymbolAddress once per device (that device current) and kept.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's `scratch` (looked up on the first call per device).
fa_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "fa_fwd_splitkv_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    fprintf(stderr, "libfa: fa_fwd_splitkv_noalloc: device %d beyond the %d the library tracks\n", dev, kMaxDevices);
    return FA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "fa_fwd_splitkv_noalloc: hipGetSymbolAddress");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}
}  // namespace

fa_status fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q,
                                 int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt,
                                 float scale, int causal, int n_splits, void* stream) {
  FA_TRY(splitkv_check(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k, max_seqlen_q,
                       max_seqlen_k, Hq, Hk, d, dt, scale, n_splits));
  // partials: o [n_splits, total_q, Hq, d] at offset 0, lse [n_splits, total_q, Hq] after it (256-byte aligned)
  const size_t rows = (size_t)n_splits * (size_t)total_q * (size_t)Hq;
  const size_t o_bytes = (rows * (size_t)d * 4 + 255) & ~(size_t)255;
  if (o_bytes + rows * 4 > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void* base = nullptr;
  FA_TRY(scratch_address(&base));
  // every partial the merge reads is written by its split first: nothing to clear
  float* o_part = reinterpret_cast<float*>(base);
  float* lse_part = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(base) + o_bytes);
  return splitkv_launch(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k, max_seqlen_q,
                        max_seqlen_k, Hq, Hk, d, dt, scale, causal, n_splits, o_part, lse_part, stream,
                        "fa_fwd_splitkv_noalloc");
}

fa_status fa_bwd_preprocess(const void* o, const void* dO, float* D, int B, int H, int N, int d, fa_dtype dt,
                            void* stream) {
  if (!o || !dO || !D) return FA_ERR_NULL;
  FA_TRY(check_preprocess_shape(B, H, N, d));
  FA_TRY(check_dtype(dt));
  if (!aligned16(o) || !aligned16(dO) || !aligned16(D)) return FA_ERR_ALIGN;
  const long long rows = (long long)B * H * N;
  return hip_status(fa::launch_bwd_preprocess(o, dO, D, rows, d, dt == FA_BF16, reinterpret_cast<hipStream_t>(stream)),
                    "fa_bwd_preprocess");
}

static fa_status bwd_dense(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                           const float* D, void* dq, void* dk, void* dv, int B, int H, int N, int d, fa_dtype dt,
                           float scale, int causal, const uint8_t* block_mask, int mask_block,
                           const fa::Dropout& drop, void* stream, const char* where) {
  if (!q || !k || !v || !dO || !lse || !D || !dq || !dk || !dv) return FA_ERR_NULL;
  FA_TRY(check_shape(B, H, N, d));
  FA_TRY(check_dtype(dt));
  FA_TRY(check_mask(block_mask, mask_block));
  FA_TRY(check_scale(scale));
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(lse) || !aligned16(D) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGN;

  fa::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.dO = dO; p.lse = lse; p.Dvec = D;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.mask = block_mask;
  p.B = B; p.H = H; p.N = N; p.D = d;
  p.mask_tiles = (N + 127) / 128;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.L = dense_layout(H, N);
  p.drop = drop;
  return hip_status(fa::launch_bwd(p, dt == FA_BF16, reinterpret_cast<hipStream_t>(stream)), where);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* D,
                 void* dq, void* dk, void* dv, int B, int H, int N, int d, fa_dtype dt, float scale, int causal,
                 const uint8_t* block_mask, int mask_block, void* stream) {
  return bwd_dense(q, k, v, dO, lse, D, dq, dk, dv, B, H, N, d, dt, scale, causal, block_mask, mask_block,
                   fa::Dropout{}, stream, "fa_bwd");
}

fa_status fa_bwd_dropout(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                         const float* D, void* dq, void* dk, void* dv, int B, int H, int N, int d, fa_dtype dt,
                         float scale, int causal, const uint8_t* block_mask, int mask_block, float p_drop,
                         uint64_t seed, uint32_t offset, void* stream) {
  fa::Dropout drop{};
  if (!q || !k || !v || !dO || !lse || !D || !dq || !dk || !dv) return FA_ERR_NULL;
  FA_TRY(make_dropout(p_drop, seed, offset, &drop));
  return bwd_dense(q, k, v, dO, lse, D, dq, dk, dv, B, H, N, d, dt, scale, causal, block_mask, mask_block, drop,
                   stream, "fa_bwd_dropout");
}

static fa_status bwd_varlen(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                            const float* D, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                            const int* cu_seqlens_k, int batch, int total_q, int total_k, int max_seqlen_q,
                            int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt, float scale, int causal,
                            const fa::Dropout& drop, void* stream, const char* where) {
  if (!q || !k || !v || !dO || !lse || !D || !dq || !dk || !dv || !cu_seqlens_q || !cu_seqlens_k)
    return FA_ERR_NULL;
  FA_TRY(check_varlen(batch, total_q, total_k, max_seqlen_q, max_seqlen_k, Hq, Hk, d));
  FA_TRY(check_dtype(dt));
  FA_TRY(check_scale(scale));
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(lse) || !aligned16(D) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGN;

  fa::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.dO = dO; p.lse = lse; p.Dvec = D;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.mask = nullptr;
  p.B = batch; p.H = Hq; p.N = max_seqlen_q; p.D = d;
  p.mask_tiles = 0;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.L.cu_q = cu_seqlens_q;
  p.L.cu_k = cu_seqlens_k;
  p.L.total_q = total_q;
  p.L.total_k = total_k;
  p.L.Hk = Hk;
  p.L.Nk = max_seqlen_k;
  p.drop = drop;
  return hip_status(fa::launch_bwd(p, dt == FA_BF16, reinterpret_cast<hipStream_t>(stream)), where);
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                        const float* D, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                        const int* cu_seqlens_k, int batch, int total_q, int total_k, int max_seqlen_q,
                        int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt, float scale, int causal,
                        void* stream) {
  return bwd_varlen(q, k, v, dO, lse, D, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                    max_seqlen_q, max_seqlen_k, Hq, Hk, d, dt, scale, causal, fa::Dropout{}, stream,
                    "fa_bwd_varlen");
}

fa_status fa_bwd_varlen_dropout(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                                const float* D, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                                const int* cu_seqlens_k, int batch, int total_q, int total_k, int max_seqlen_q,
                                int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt, float scale, int causal,
                                float p_drop, uint64_t seed, uint32_t offset, void* stream) {
  fa::Dropout drop{};
  if (!q || !k || !v || !dO || !lse || !D || !dq || !dk || !dv || !cu_seqlens_q || !cu_seqlens_k)
    return FA_ERR_NULL;
  FA_TRY(make_dropout(p_drop, seed, offset, &drop));
  return bwd_varlen(q, k, v, dO, lse, D, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                    max_seqlen_q, max_seqlen_k, Hq, Hk, d, dt, scale, causal, drop, stream,
                    "fa_bwd_varlen_dropout");
}

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: sizes must be >= 1 (heads: Hq a multiple of Hk) and fit the index range";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: dtype must be FA_F16 or FA_BF16";
    case FA_ERR_HEADDIM: return "FA_ERR_HEADDIM: head dimension must be 64 or 128";
    case FA_ERR_MASK: return "FA_ERR_MASK: block_mask requires mask_block == 128";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensor pointers must be 16-byte aligned";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP kernel launch failed";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0";
    case FA_ERR_DROPOUT: return "FA_ERR_DROPOUT: dropout probability must satisfy 0 <= p < 1";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: split-KV partial results exceed the library's static scratch (FA_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown fa_status";
}

}  // extern "C"
