/*
 * msa.h -- C ABI of libmsa.so, the MI355X (gfx950) forward path of MiniMax
 * Sparse Attention (MSA).
 *
 * What the calls compute (sources cited by page title and section):
 *  - Index Branch [hyper.ai paper page 2606.13392, 方法 (Method); Telegram
 *    review quant_prune_distill post 751, "Метод"]: one index-query head per
 *    GQA group and one index-key head per layer give raw dot-product scores
 *    s[t,g,j] = idx_q[t,g] . idx_k[j] for every visible key j <= t; the scores
 *    are max-pooled over aligned blocks of block_size tokens; per (query
 *    token, group) the topk blocks with the largest maxima are kept, the block
 *    holding the query (L(t) = t / block_size) always being one of them.
 *    Equal maxima go to the lower block index.  block_idx rows list the kept
 *    blocks in ascending order and are padded with -1 to length topk
 *    (exactly min(topk, L(t)+1) entries are valid).
 *  - Main Branch [same page, 方法; hamidun.com news "MiniMax выпустила MSA",
 *    "Как устроен MSA"]: exact softmax attention of every query head h over
 *    the keys of the kept blocks of its group g = h / (Hq/G), restricted to
 *    keys j <= t, with scale softmax_scale (1/sqrt(head_dim) by default).
 *  - Prefill and decode [hyper.ai page, 一句话总结 (summary): prefill and
 *    decode speed-ups at 1M context].
 *
 * Conventions shared by every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller, row-major and
 *    contiguous (innermost dimension last).  bf16 tensors are IEEE bfloat16
 *    bit patterns (uint16) and must be 16-byte aligned; int32 and fp32
 *    tensors must be 4-byte aligned.  The library never allocates or frees
 *    device memory and keeps no state between calls.
 *  - The caller supplies a device workspace of at least
 *    msa_workspace_bytes(op, dims) bytes (256-byte aligned); its contents on
 *    entry do not matter and are clobbered.
 *  - Every call validates all arguments on the host before enqueueing any
 *    work and returns a status; on a non-zero status nothing was enqueued
 *    (except MSA_ERR_HIP, where earlier launches of the same call may have
 *    been enqueued).  On MSA_OK the work is enqueued on hip_stream (a
 *    hipStream_t; NULL = the default stream) and the call returns without
 *    waiting.  Outputs are bitwise reproducible run to run.
 *  - Calls on different streams with disjoint workspaces may run
 *    concurrently; calls sharing a workspace must be ordered by the caller.
 *  - A call only launches kernels on hip_stream (no allocation, no memset,
 *    no host synchronisation), so it can be captured into a HIP graph and
 *    replayed; replays read the tensors' current contents, cache_lens
 *    included.  Exceptions: msa_decode with MSA_CHECK_LENS (it waits for the
 *    stream) and calls made while msa_profile_begin is active.
 *  - Inputs must be finite; NaN or Inf inputs give unspecified outputs.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define MSA_OK 0
#define MSA_ERR_INVALID_ARG 1  /* null pointer, non-positive size, Hq % G != 0, bad flag mix */
#define MSA_ERR_UNSUPPORTED 2  /* head_dim != 128, index_dim not in {64,128}, block_size not in
                                  {32,64,128}, or Hq/G above 128 (prefill) / 16 (decode) */
#define MSA_ERR_ALIGNMENT 3    /* a tensor pointer misaligned (see above), or workspace not 256-byte aligned */
#define MSA_ERR_WORKSPACE 4    /* workspace_bytes < msa_workspace_bytes(op, dims) */
#define MSA_ERR_HIP 5          /* a HIP launch failed; see msa_status_string / msa_last_hip_error */

/* ---- dims.flags ---- */
/* Main branch over ALL visible blocks (full causal attention, the dense
   baseline); the index branch is skipped.  block_idx must be NULL. */
#define MSA_DENSE 0x1u
/* block_idx is an INPUT: the main branch attends to the given blocks and the
   index branch is skipped.  Entries outside [0, L(t)] (e.g. -1) are ignored;
   valid entries of a row must be distinct. */
#define MSA_GIVEN_INDICES 0x2u
/* Forced sink block: block 0, the start of the sequence, is selected beside
   the local block whenever a row keeps at least two blocks (m = min(k, L+1)
   >= 2); k counts both, and the other m-2 places go to the best of blocks
   1..L-1.  The variant the pages ablate [hyper.ai paper page 2606.13392,
   实验 (Experiments): hard-coded selection of the sequence start and of the
   local window].  A rule of the index branch: invalid with MSA_DENSE or
   MSA_GIVEN_INDICES. */
#define MSA_FORCE_SINK 0x4u
/* Decode only: validate cache_lens before any launch.  The call copies the
   batch lengths to the host on hip_stream and waits for that stream, then
   returns MSA_ERR_INVALID_ARG if any length lies outside [1, Lmax].  Without
   this flag msa_decode stays fully asynchronous and clamps out-of-range
   lengths to [1, Lmax] on the device.  Invalid with every other operation and
   with msa_decode_noalloc (which must not synchronize). */
#define MSA_CHECK_LENS 0x8u
/* Index Branch in one pass, for msa_index_topk and msa_prefill: every key
   block's maximum score is offered at once to a running list of the row's
   best candidates held in registers, so no block-score table is written and
   no separate top-k launch runs [hyper.ai paper page 2606.13392, 方法
   (Method): the index scores, Block-Max and Top-k with the forced local
   block].  The selection is bit-identical to the default two-pass path,
   which writes a table of one fp32 per row and candidate block (about 2.2 GB
   for 128K tokens, 8 groups, B = 128) and is the faster of the two; this path
   trades that speed for a smaller workspace (msa_index_topk needs none).
   topk must be <= 17, else MSA_ERR_UNSUPPORTED.  Invalid with MSA_DENSE,
   MSA_GIVEN_INDICES, decode, msa_index_scores, msa_indexer_kl and
   msa_prefill_backward. */
#define MSA_ONE_PASS_INDEX 0x10u

/* ---- operations for msa_workspace_bytes ---- */
#define MSA_OP_INDEX_TOPK 0
#define MSA_OP_PREFILL 1
#define MSA_OP_DECODE 2
#define MSA_OP_INDEXER_KL 3
#define MSA_OP_BACKWARD 4

typedef struct msa_dims {
  int32_t batch;         /* sequences, >= 1 */
  int32_t seqlen;        /* prefill: T (queries == keys); decode: cache capacity Lmax */
  int32_t num_q_heads;   /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;  /* G: GQA groups = KV heads = index-query heads */
  int32_t head_dim;      /* d: 128 */
  int32_t index_dim;     /* d_idx: 64 or 128 */
  int32_t block_size;    /* B: 32, 64 or 128 */
  int32_t topk;          /* k >= 1, counts the forced local block; k > number of
                            visible blocks selects all of them */
  float softmax_scale;   /* <= 0 selects 1/sqrt(head_dim) */
  uint32_t flags;        /* MSA_DENSE, MSA_GIVEN_INDICES, MSA_FORCE_SINK, MSA_CHECK_LENS,
                            MSA_ONE_PASS_INDEX */
  int32_t query_chunk;   /* prefill: query tokens per internal pass, a multiple of
                            block_size; 0 = the library's default (bounds the
                            workspace).  Ignored by decode. */
  int32_t reserved;      /* must be 0 */
} msa_dims;

/*
 * Index Branch only (prefill shapes).
 *   idx_q     [batch, T, G, index_dim] bf16
 *   idx_k     [batch, T, index_dim]    bf16
 *   block_idx [batch, T, G, topk]      int32, OUTPUT
 * Flags: MSA_FORCE_SINK and MSA_ONE_PASS_INDEX, or 0.  Integer-valued idx inputs whose dot
 * products stay below 2^24 in magnitude give exact scores, hence a unique,
 * exact selection.
 */
int msa_index_topk(const msa_dims* dims, const void* idx_q, const void* idx_k,
                   int32_t* block_idx, void* workspace, size_t workspace_bytes,
                   void* hip_stream);

/*
 * Index scores + Block-Max pooling only (the first half of the Index Branch),
 * for query tokens [t0, t1) of prefill-shaped inputs:
 *   scores[s][t - t0][g][b] = max over keys j of block b of idx_q[s,t,g] . idx_k[s,j]
 * for every candidate block b < L(t) = t / block_size, in fp32 (products of
 * bf16 values accumulated in fp32).  scores is [batch, t1 - t0, G, row_stride]
 * fp32 with row_stride a multiple of 4 and >= L(t1 - 1); entries b >= L(t) of
 * a row are unspecified.
 * superblock_max (nullable): [batch, t1 - t0, G, sb_stride] fp32 OUTPUT with
 * sb_stride >= ceil(L(t1 - 1) / 16); entry i of a row is the largest score of
 * the row's candidate blocks b in [16 i, 16 i + 16), b < L(t), for
 * i < ceil(L(t) / 16) (later entries unspecified).  The selection reads these
 * run maxima to skip runs of rows with more than 1024 candidates that cannot
 * hold a selected block; with superblock_max non-NULL the kernel variant that
 * writes them runs, so both variants can be checked.  4-byte aligned.
 * No workspace.  Flags must be 0 or MSA_FORCE_SINK (scores do not depend on it).
 */
int msa_index_scores(const msa_dims* dims, const void* idx_q, const void* idx_k, float* scores,
                     int32_t t0, int32_t t1, int32_t row_stride, float* superblock_max,
                     int32_t sb_stride, void* hip_stream);

/*
 * Prefill: Index Branch + Main Branch over a whole causal sequence.
 *   q         [batch, T, Hq, d] bf16
 *   k, v      [batch, T, G, d]  bf16
 *   idx_q     [batch, T, G, index_dim] bf16   (unused with MSA_DENSE or
 *   idx_k     [batch, T, index_dim]    bf16    MSA_GIVEN_INDICES; may be NULL)
 *   out       [batch, T, Hq, d] bf16 OUTPUT (round to nearest even)
 *   lse       [batch, T, Hq] fp32 OUTPUT, natural-log sum of exp of the scaled
 *             logits over the attended keys; may be NULL
 *   block_idx [batch, T, G, topk] int32: OUTPUT (may be NULL), INPUT with
 *             MSA_GIVEN_INDICES, must be NULL with MSA_DENSE
 */
int msa_prefill(const msa_dims* dims, const void* q, const void* k, const void* v,
                const void* idx_q, const void* idx_k, void* out, float* lse,
                int32_t* block_idx, void* workspace, size_t workspace_bytes,
                void* hip_stream);

/*
 * Decode: one new query token per sequence against its caches.
 *   q           [batch, Hq, d] bf16
 *   k_cache,
 *   v_cache     [batch, Lmax, G, d] bf16 (Lmax = dims->seqlen)
 *   idx_q       [batch, G, index_dim] bf16      (unused with MSA_DENSE or
 *   idx_k_cache [batch, Lmax, index_dim] bf16    MSA_GIVEN_INDICES; may be NULL)
 *   cache_lens  [batch] int32, DEVICE: tokens in each cache INCLUDING the new
 *               one (the query sits at position cache_lens[s]-1); each value
 *               must lie in [1, Lmax].  Out-of-range values are clamped to
 *               that range on the device, unless dims->flags holds
 *               MSA_CHECK_LENS: then the call returns MSA_ERR_INVALID_ARG
 *               before any launch (and synchronizes hip_stream to read them)
 *   out         [batch, Hq, d] bf16 OUTPUT;  lse [batch, Hq] fp32 OUTPUT or NULL
 *   block_idx   [batch, G, topk] int32: OUTPUT (may be NULL), INPUT with
 *               MSA_GIVEN_INDICES, must be NULL with MSA_DENSE
 */
int msa_decode(const msa_dims* dims, const void* q, const void* k_cache,
               const void* v_cache, const void* idx_q, const void* idx_k_cache,
               const int32_t* cache_lens, void* out, float* lse, int32_t* block_idx,
               void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * msa_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, kernels and results as msa_decode;
 * the workspace is a library-owned device array of msa_decode_noalloc_limit()
 * bytes (32 MiB), one per GPU, held until the process ends.  Shapes whose
 * msa_workspace_bytes(MSA_OP_DECODE, dims) exceeds that limit return
 * MSA_ERR_WORKSPACE before any launch (8 sequences at 1M context, block 128,
 * top-k 16 need about 10 MiB; all-blocks mode at that context does not fit).
 * The call allocates nothing; it looks up the array's device address once per
 * GPU (hipGetSymbolAddress, on the first call with that GPU current).  Every
 * call on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (on different streams, or from different threads) race; calls ordered
 * on one stream do not.
 */
int msa_decode_noalloc(const msa_dims* dims, const void* q, const void* k_cache,
                       const void* v_cache, const void* idx_q, const void* idx_k_cache,
                       const int32_t* cache_lens, void* out, float* lse, int32_t* block_idx,
                       void* hip_stream);
size_t msa_decode_noalloc_limit(void);

/*
 * Indexer KL loss and its gradient into the index-branch inputs: the signal
 * that trains the Index Branch [Telegram review quant_prune_distill post 751,
 * "Метод": KL between the index branch and the head-averaged main branch,
 * stop-gradient through the main branch's probabilities and on the index
 * inputs; hyper.ai paper page 2606.13392, 方法 (Method): KL on the selected
 * tokens, gradient detach on the Index Branch inputs].
 * Per (token t, group g) row, over the tokens J = {j <= t in the row's
 * selected blocks}:
 *   p_I(j) = softmax over J of idx_q[t,g] . idx_k[j]
 *   p_M(j) = mean over the group's heads h of exp(scale q[t,h].k[j,g] - lse[t,h])
 *   kl[t,g] = sum_j p_M(j) (ln p_M(j) - ln p_I(j))
 * and, for the loss sum_{t,g} kl[t,g] with p_M held constant,
 *   d_idx_q[t,g] = sum_j (p_I(j) - p_M(j)) idx_k[j]
 *   d_idx_k[j]   = sum over rows using j of (p_I(j) - p_M(j)) idx_q[t,g]
 *   q         [batch, T, Hq, d] bf16;  k [batch, T, G, d] bf16
 *   idx_q     [batch, T, G, index_dim] bf16;  idx_k [batch, T, index_dim] bf16
 *   block_idx [batch, T, G, topk] int32: the selection (e.g. msa_prefill's);
 *             entries outside [0, L(t)] are ignored, valid entries must be
 *             distinct
 *   lse       [batch, T, Hq] fp32: the main branch's log-sum-exp over the same
 *             selection (msa_prefill's lse output)
 *   kl        [batch, T, G] fp32 OUTPUT (0 for a row without valid entries)
 *   d_idx_q   [batch, T, G, index_dim] fp32 OUTPUT
 *   d_idx_k   [batch, T, index_dim] fp32 OUTPUT (keys never selected get 0)
 * dims: prefill shapes (any Hq / G up to 128, as for msa_prefill), flags must
 * be 0.  d_idx_q 16-byte aligned, the other fp32 pointers
 * 4-byte aligned.  dS = p_I - p_M
 * enters the gradient products rounded to bf16 (fp32 accumulation).
 * Deterministic: fixed-order sums, no atomics on values.
 */
int msa_indexer_kl(const msa_dims* dims, const void* q, const void* k, const void* idx_q,
                   const void* idx_k, const int32_t* block_idx, const float* lse, float* kl,
                   float* d_idx_q, float* d_idx_k, void* workspace, size_t workspace_bytes,
                   void* hip_stream);

/*
 * Backward of the main branch: dq, dk, dv of the block-sparse attention with
 * the selection held fixed.  The selection is a top-k, piecewise constant in
 * the index inputs, and the index branch learns through msa_indexer_kl only
 * [Telegram review quant_prune_distill post 751, "Метод": stop-gradient on the
 * index branch; hyper.ai paper page 2606.13392, 方法 (Method): gradient detach
 * on the Index Branch inputs, standard scaled dot-product attention over the
 * gathered Key/Value vectors].  Per (token t, head h), g = h / R, over the
 * tokens J = {j <= t in the row's selected blocks}, P_j = exp(scale q[t,h].k[j,g]
 * - lse[t,h]) and dO = dout[t,h]:
 *   dv[j,g] += P_j dO;   dS_j = scale P_j (dO.v[j,g] - dO.out[t,h])
 *   dq[t,h]  = sum_j dS_j k[j,g];   dk[j,g] += dS_j q[t,h]
 *   q, out, dout [batch, T, Hq, d] bf16;  k, v [batch, T, G, d] bf16
 *   lse        [batch, T, Hq] fp32: the forward's log-sum-exp (msa_prefill's lse)
 *   block_idx  [batch, T, G, topk] int32: the forward's selection (entries
 *              outside [0, L(t)] ignored, valid entries distinct)
 *   dq [batch, T, Hq, d], dk and dv [batch, T, G, d] fp32 OUTPUTS (a row with
 *              nothing to attend gets dq = 0; keys no row attends get 0)
 * dims: prefill shapes, flags must be 0, Hq / G <= 128.  bf16 pointers 16-byte
 * aligned, fp32 and int32 pointers 4-byte aligned.  P and dS enter the
 * gradient products rounded to bf16, and dq is summed from one bf16 partial
 * per selected block (fp32 accumulation throughout).  Deterministic:
 * fixed-order sums, no atomics on values.
 */
int msa_prefill_backward(const msa_dims* dims, const void* q, const void* k, const void* v,
                         const void* out, const float* lse, const void* dout,
                         const int32_t* block_idx, float* dq, float* dk, float* dv,
                         void* workspace, size_t workspace_bytes, void* hip_stream);

/* Workspace bytes needed by op for dims (0 when none is needed).  Returns
   (size_t)-1 when dims are invalid for op. */
size_t msa_workspace_bytes(int op, const msa_dims* dims);

/* Static text for a status code (never NULL). */
const char* msa_status_string(int status);

/* Text of the HIP error behind the calling thread's last MSA_ERR_HIP ("" if none). */
const char* msa_last_hip_error(void);

/* ABI version of this header: 1. */
int msa_abi_version(void);

/*
 * Stage timing (a measurement aid; not part of the attention computation).
 * Between msa_profile_begin() and msa_profile_end(), every stage of every
 * msa_prefill / msa_decode / msa_index_topk call records a HIP event on the
 * call's stream at its start, and each call records one at its end; a
 * stage's time is the elapsed time from its event to the next event on the
 * same stream.  While profiling is off nothing is recorded.
 *
 * msa_profile_end() stops recording, waits for the recorded events and writes
 * MSA_STAGE_COUNT entries to out (indexed by stage; launches = number of
 * timed launches of the stage, total_ms = their summed time).  It returns
 * MSA_ERR_INVALID_ARG when out or n_stages is NULL or max_stages <
 * MSA_STAGE_COUNT, MSA_ERR_HIP when an event could not be created, recorded
 * or read.  Profiling is process-wide; calls on several host threads are
 * recorded together.
 */
#define MSA_STAGE_INDEX_PREFILL 0      /* index scores + Block-Max, prefill      */
#define MSA_STAGE_TOPK_PREFILL 1       /* Top-k with the forced local block       */
#define MSA_STAGE_BLOCK_LISTS 2        /* per-block lists of (token, slot) pairs  */
#define MSA_STAGE_KV_OUTER 3           /* block-major attention, partial outputs  */
#define MSA_STAGE_QUERY_MAJOR 4        /* local block + merge of the partials     */
#define MSA_STAGE_QUERY_MAJOR_DENSE 5  /* all-blocks (MSA_DENSE) prefill          */
#define MSA_STAGE_INDEX_DECODE 6       /* index scores + Block-Max, decode        */
#define MSA_STAGE_TOPK_DECODE 7
#define MSA_STAGE_DECODE_ATTN 8        /* per-(sequence, group) attention         */
#define MSA_STAGE_DECODE_COMBINE 9     /* combine of the split partials (dense)   */
#define MSA_STAGE_INDEXER_KL 10        /* msa_indexer_kl, all of its kernels      */
#define MSA_STAGE_BWD_PREP 11          /* backward: dO.out, block lists, list sort */
#define MSA_STAGE_BWD_LISTS 12         /* backward: per-list dq / dk / dv products */
#define MSA_STAGE_BWD_MERGE 13         /* backward: fixed-order dq and dk/dv sums  */
#define MSA_STAGE_INDEX_ONE_PASS 14    /* Index Branch in one pass (MSA_ONE_PASS_INDEX) */
#define MSA_STAGE_COUNT 15

typedef struct msa_stage_time {
  int32_t stage;
  int32_t launches;
  double total_ms;
} msa_stage_time;

int msa_profile_begin(void);
int msa_profile_end(msa_stage_time* out, int32_t max_stages, int32_t* n_stages);
/* Static name of a stage (never NULL). */
const char* msa_stage_name(int32_t stage);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
