/* fa.h — C ABI of the gfx950 fused attention library (libfa.so).
 *
 * The operation is exact scaled-dot-product attention, O = softmax(s Q K^T) V
 * with s the softmax scale, computed per (batch, head) over rows of length d.
 * Sources (web pages on FlashAttention, cited by title and section):
 *   [P1] "FlashAttention：不减少一次注意力计算，为什么反而更快" (awesome.papernotes.org),
 *        key design 1 (operator and tiling), key design 2 (mergeable softmax
 *        state; the saved log-sum-exp L = m + log l), key design 3 (backward by
 *        recomputation, D_i = dO_i . O_i, dS = P o (dP - D)), IO section
 *        (block-sparse variant: zero blocks skipped, exact inside kept blocks).
 *   [P2] "FlashAttention 入门：从 FA1 到 FA4 的 IO 感知注意力" (oripoin.cn),
 *        FA1 section (causal: keys j > i skipped or masked), backward section
 *        (the default backward adds dQ with atomics and is not bitwise
 *        deterministic; a deterministic option exists).
 *   [P3] "FlashAttention" (lyirs.cc), forward-process section (unnormalised
 *        accumulator, one final division by l).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *     allocates nothing, keeps no state, and returns without synchronising.
 *     Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *   - Tensors q, k, v, o, dO, dq, dk, dv are contiguous [B, H, N, d] with d
 *     fastest, 16-bit elements of type `dt`. lse and D are contiguous
 *     [B, H, N] float32. Pointers must be 16-byte aligned.
 *   - Attention is square self-attention (N queries, N keys per head).
 *   - causal != 0 keeps key j for query i only when j <= i [P2, FA1 section].
 *   - block_mask, when not NULL, is a row-major uint8 [T, T] tile mask with
 *     T = ceil(N / mask_block), shared by every (batch, head); tile (a, b)
 *     nonzero keeps queries a*mask_block.. with keys b*mask_block..; zero
 *     tiles are skipped [P1, IO section]. mask_block must be 128. causal and
 *     block_mask combine with a logical AND. A masked pair is -inf before the
 *     softmax: each row normalises over its kept keys only. A row with no
 *     kept key yields O = 0 and LSE = -inf and receives no gradient.
 *   - scale is the softmax scale s (callers normally pass 1/sqrt(d)); it must
 *     be finite and > 0.
 *   - Outputs must not alias inputs. Arguments are validated before any HIP
 *     call; on a validation error nothing is enqueued. Asynchronous device
 *     faults surface at the caller's next synchronisation, as with any HIP
 *     library.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,     /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,    /* B, H or N < 1, N*d >= 2^29 (per-head byte offsets are 32-bit), or the grid is too large */
  FA_ERR_DTYPE = -3,    /* dt is not FA_F16 or FA_BF16 */
  FA_ERR_HEADDIM = -4,  /* d is not 64 or 128 */
  FA_ERR_MASK = -5,     /* block_mask given with mask_block != 128 */
  FA_ERR_ALIGN = -6,    /* a tensor pointer is not 16-byte aligned */
  FA_ERR_HIP = -7,      /* a HIP launch reported an error */
  FA_ERR_SCALE = -8,    /* scale is not finite and > 0 */
  FA_ERR_DROPOUT = -9,  /* dropout probability outside [0, 1) */
  FA_ERR_SCRATCH = -10  /* fa_fwd_splitkv_noalloc: partial results beyond FA_NOALLOC_SCRATCH_BYTES */
} fa_status;

/* Forward [P1 key designs 1-2; P3 forward process].
 * Writes o = softmax(scale * q k^T) v, rounded to dt (round to nearest even),
 * and lse[b,h,i] = ln sum_j exp(scale * q_i . k_j) over kept keys (float32,
 * natural log of the scaled scores). Deterministic: identical inputs give
 * identical bits. No N x N buffer is used. */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, fa_dtype dt, float scale, int causal,
                 const uint8_t* block_mask, int mask_block, void* stream);

/* Backward preprocess [P1 key design 3]: D[b,h,i] = sum_c dO[b,h,i,c] * o[b,h,i,c],
 * products and sum in float32, using the stored 16-bit o from fa_fwd. The
 * B*H*N rows are indexed in 64 bits (no per-head limit: a packed batch passes
 * B = 1, H = Hq, N = total_q); FA_ERR_SHAPE only if the row count exceeds
 * the dispatch grid (2^28 rows at d = 128, 2^29 at d = 64). */
fa_status fa_bwd_preprocess(const void* o, const void* dO, float* D,
                            int B, int H, int N, int d, fa_dtype dt, void* stream);

/* Backward by recomputation [P1 key design 3; P2 backward section].
 * Inputs: q, k, v, dO (the gradient of o), lse from fa_fwd and D from
 * fa_bwd_preprocess, with the same shape, scale, causal flag and mask as the
 * forward. Writes dq, dk, dv (dt, rounded to nearest even). P is rebuilt tile
 * by tile from q, k and lse; no N x N buffer and no workspace is used. This is
 * the deterministic form of the backward (no atomics): one kernel owns each
 * key block's dk, dv rows, another each query block's dq rows, so identical
 * inputs give identical bits. */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* dO,
                 const float* lse, const float* D, void* dq, void* dk, void* dv,
                 int B, int H, int N, int d, fa_dtype dt, float scale,
                 int causal, const uint8_t* block_mask, int mask_block, void* stream);

/* ------------------------------------------------------------------------
 * Dropout on the attention probabilities [P1, key design 2 table and key
 * design 3: the forward keeps the generator state, not the mask, and the
 * backward regenerates the mask].
 *   O = (P o Z) V with Z = M / (1 - p_drop), M the keep mask, P the softmax
 *   probabilities; lse is that of the scores (dropout acts after the softmax),
 *   so fa_bwd_preprocess applies unchanged (D_i = dO_i . O_i still holds).
 *   Mask: one Philox4x32-10 call (Salmon, Moraes, Dror, Shaw, SC 2011) with
 *   counter (j / 4, i / 2, bh, offset) and key (seed mod 2^32, seed / 2^32)
 *   decides the 2 x 4 block of queries i, keys j it covers: element (head
 *   bh = b*H + h, query i, key j) is dropped iff the 16-bit half i % 2 (0 =
 *   low) of word j % 4 is below floor(p_drop * 2^16), so the dropped fraction
 *   is within 2^-16 of p_drop. The same (p_drop, seed, offset) must be passed to
 *   the forward and the backward; `offset` separates independent masks drawn
 *   with one seed. Otherwise identical to fa_fwd / fa_bwd (dense layout,
 *   causal, block mask). FA_ERR_DROPOUT unless 0 <= p_drop < 1; p_drop = 0
 *   reproduces fa_fwd / fa_bwd bit for bit.
 * ------------------------------------------------------------------------ */
fa_status fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int N, int d, fa_dtype dt, float scale, int causal,
                         const uint8_t* block_mask, int mask_block, float p_drop, uint64_t seed,
                         uint32_t offset, void* stream);

fa_status fa_bwd_dropout(const void* q, const void* k, const void* v, const void* dO,
                         const float* lse, const float* D, void* dq, void* dk, void* dv,
                         int B, int H, int N, int d, fa_dtype dt, float scale, int causal,
                         const uint8_t* block_mask, int mask_block, float p_drop, uint64_t seed,
                         uint32_t offset, void* stream);

/* ------------------------------------------------------------------------
 * Packed variable-length batches with grouped key/value heads
 * [P2, usage section: "padding and shapes" (variable-length sequences packed
 * through cumulative offsets, no padding) and the library-interface list
 * (multi-query / grouped-query attention); P1 key designs 1-3 for the
 * operator itself].
 *
 *   q, o, dO, dq: token-major [total_q, Hq, d]; k, v, dk, dv: [total_k, Hk, d];
 *   lse, D: float32 [total_q, Hq]. Hq must be a multiple of Hk; query head h
 *   reads key/value head h / (Hq / Hk) (Hk == 1: multi-query attention).
 *   cu_seqlens_q, cu_seqlens_k: DEVICE int32 arrays of batch + 1 cumulative
 *   offsets; sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   and key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1. The kernels clamp
 *   every offset to [0, total] (so malformed offsets cannot address outside
 *   the tensors), and rows of a sequence beyond max_seqlen_q / max_seqlen_k
 *   are not computed: the caller passes the true maxima.
 *   causal != 0 with n_q queries and n_k keys in a sequence: query i sees key
 *   j iff j <= i + (n_k - n_q), i.e. the queries are the last n_q positions
 *   of the key sequence (a reading: the pages only note that one backend
 *   refuses causal attention with unequal lengths). Queries that see no key
 *   get O = 0, LSE = -inf and no gradient; sequences with no query rows leave
 *   their keys' dk, dv at zero.
 *   Limits (FA_ERR_SHAPE otherwise): batch, max_seqlen_*, Hq, Hk >= 1,
 *   total_* >= 0, max_seqlen_q * Hq * d * 2 and max_seqlen_k * Hk * d * 2
 *   below 2^31. No block mask on this path. Otherwise the conventions of the
 *   dense entry points apply (device pointers, 16-byte alignment, no
 *   allocation, stream-ordered, validation before any HIP call).
 *   D for fa_bwd_varlen comes from fa_bwd_preprocess(o, dO, D, 1, Hq,
 *   total_q, d, dt, stream): the packed rows are contiguous in the same order.
 * ------------------------------------------------------------------------ */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q, int total_k,
                        int max_seqlen_q, int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt, float scale,
                        int causal, void* stream);

/* Split-KV forward [P1, key design 2 (mergeable softmax state) and its
 * history/outlook section (the state as an associative reduction for long
 * key/value caches in decode); P2, FA2 section (saved L = m + log l)].
 * Same inputs, outputs and conventions as fa_fwd_varlen. Each (sequence,
 * key/value head) processes the Hq / Hk query heads of its group together
 * (their rows packed: a key/value tile is read once for the whole group), and
 * the key tiles each row block sees are cut into n_splits contiguous ranges
 * computed by separate workgroups. Split s writes its normalised partial
 * output O_s (fp32) and LSE_s into caller-provided workspace; a second kernel
 * merges them: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
 *   o_partial:   float32 [n_splits, total_q, Hq, d]   (16-byte aligned)
 *   lse_partial: float32 [n_splits, total_q, Hq]
 *   1 <= n_splits <= FA_MAX_SPLITS, else FA_ERR_SHAPE.
 * The result equals fa_fwd_varlen's up to floating-point rounding order. */
#define FA_MAX_SPLITS 256
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                         const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q, int total_k,
                         int max_seqlen_q, int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt, float scale,
                         int causal, int n_splits, float* o_partial, float* lse_partial, void* stream);

/* Split-KV forward that allocates nothing and takes no workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. Same arguments, result and
 * conventions as fa_fwd_splitkv, without o_partial / lse_partial: the partial
 * results live in a static device array of FA_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends. The call makes no
 * allocation of any kind (its first call on a device looks the array's
 * address up once).
 *   Limit: the partial results, R * d * 4 bytes rounded up to a multiple of
 *   256 plus R * 4 bytes with R = n_splits * total_q * Hq, must fit in
 *   FA_NOALLOC_SCRATCH_BYTES, else FA_ERR_SCRATCH (checked before any HIP
 *   call; nothing enqueued). E.g. 8 splits of 32 decode rows x 32 query heads
 *   at d = 128 use 4.2 MB of the 32 MiB.
 *   Every call on a GPU shares that GPU's array: calls that may overlap on one
 *   GPU (other streams, other host threads) race and must be serialised by the
 *   caller. The array keeps the last call's contents; no part of it needs to
 *   start at any particular value. */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
fa_status fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q,
                                 int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt,
                                 float scale, int causal, int n_splits, void* stream);

/* Gradients for fa_fwd_varlen. dk, dv of a key/value head sum the
 * contributions of every query head that reads it (computed inside one
 * workgroup per key block, no atomics: deterministic). */
fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                        const float* D, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                        const int* cu_seqlens_k, int batch, int total_q, int total_k, int max_seqlen_q,
                        int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt, float scale, int causal,
                        void* stream);

/* Dropout on packed batches [P1, key design 2 table and key design 3, as for
 * fa_fwd_dropout; P2 usage section for the packed layout]: fa_fwd_varlen /
 * fa_bwd_varlen with the mask of fa_fwd_dropout, where query head h of
 * sequence b is mask head bh = b * Hq + h and i, j are the query and key
 * positions inside the sequence (0 = its first row). dk, dv of a shared
 * key/value head sum the contributions of the query heads that read it, each
 * with its own mask. The same (p_drop, seed, offset) must be passed to the
 * forward and the backward. FA_ERR_DROPOUT unless 0 <= p_drop < 1; p_drop = 0
 * reproduces fa_fwd_varlen / fa_bwd_varlen bit for bit. */
fa_status fa_fwd_varlen_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                                const int* cu_seqlens_q, const int* cu_seqlens_k, int batch, int total_q,
                                int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hk, int d,
                                fa_dtype dt, float scale, int causal, float p_drop, uint64_t seed, uint32_t offset,
                                void* stream);

fa_status fa_bwd_varlen_dropout(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                                const float* D, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                                const int* cu_seqlens_k, int batch, int total_q, int total_k, int max_seqlen_q,
                                int max_seqlen_k, int Hq, int Hk, int d, fa_dtype dt, float scale, int causal,
                                float p_drop, uint64_t seed, uint32_t offset, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* fa_status_string(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
