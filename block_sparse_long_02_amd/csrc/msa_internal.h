// Host-side launchers of the libmsa kernels (internal; not part of the C ABI).
// Every launcher enqueues on `st` and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

// Tokens (query rows) handled by one workgroup of the attention kernels:
// 4 waves x 32 rows = 128 (token, head) rows; tokens per tile = 128 / R.
constexpr int kAttnRows = 128;

hipError_t launch_fill_i32(int32_t* p, size_t n, int32_t value, hipStream_t st);

// Stage boundary for msa_profile_*: records an event on st while profiling
// is on (stage = MSA_STAGE_*, or -1 at the end of a call); no-op otherwise.
void prof_mark(hipStream_t st, int stage);

// ---- Index Branch, prefill: scores + Block-Max for query tokens [t0, t0+tc) ----
// S is [batch][tc*G][s_stride] fp32; row (t-t0)*G+g holds blocks 0..L(t)-1.
// Superblocks are runs of kSuperBlock consecutive blocks; SM (nullable) is
// [batch][tc*G][sm_stride] fp32 and SM[row][i] is the largest S[row][b] over
// the row's candidate blocks b in [16 i, 16 i + 16) with b < L(t), for
// i < ceil(L(t) / 16): the top-k reads only the superblocks that can hold
// a selected block.
constexpr int kSuperBlock = 16;
// Rows with more candidate blocks than this take the superblock path; SM is
// only needed (and only computed) when a chunk has such rows.
constexpr int kSbMinCandidates = 1024;
hipError_t launch_index_blockmax_prefill(const uint16_t* idx_q, const uint16_t* idx_k, float* S,
                                         int batch, int T, int G, int di, int B, int t0, int tc,
                                         int s_stride, float* SM, int sm_stride, hipStream_t st);

// ---- Index Branch in one pass (scores, Block-Max, Top-k; no score table) ----
// Each row keeps its best want = m - 1 (less the forced sink) candidates in
// 16 register slots, so topk is at most kOnePassMaxTopk.  Output rows as in
// launch_topk_prefill.
constexpr int kOnePassMaxTopk = 17;
hipError_t launch_index_topk_one_pass(const uint16_t* idx_q, const uint16_t* idx_k, int32_t* bidx, long bidx_rows,
                                      int bidx_t_off, int batch, int T, int G, int di, int B, int k, bool sink,
                                      int t0, int tc, hipStream_t st);

// ---- Top-k with the forced local block ----
// prefill rows: (s, t in [t0, t0+tc), g); output row address
//   bidx + ((s*bidx_rows + (t - bidx_t_off))*G + g)*k
// sink: block 0 is forced too when a row keeps at least two blocks.
hipError_t launch_topk_prefill(const float* S, int s_stride, const float* SM, int sm_stride,
                               int32_t* bidx, long bidx_rows,
                               int bidx_t_off, int batch, int G, int B, int k, bool sink, int t0, int tc,
                               hipStream_t st);
// decode rows: (s, g); query position cache_lens[s]-1; output bidx + (s*G+g)*k
hipError_t launch_topk_decode(const float* S, int s_stride, int32_t* bidx, const int32_t* lens,
                              int Lmax, int batch, int G, int B, int k, bool sink, hipStream_t st);

// ---- Main Branch, prefill ----
// Query tokens per window of the block lists: the lists of (token, slot)
// pairs are kept per (sequence, group, window, block), so that consecutive
// block-major workgroups touch the q rows of one window.  The forward uses
// 4096-token windows (at 128K its lists build in 0.97 ms against 1.5 ms with
// 8192, 3.2 ms with 16384); the indexer KL and the backward keep 8192, which
// halves their per-list partial blocks and bounds the list sort's LDS keys.
#ifndef MSA_LIST_WINDOW
#define MSA_LIST_WINDOW 8192
#endif
constexpr int kListWindow = MSA_LIST_WINDOW;
#ifndef MSA_FWD_LIST_WINDOW
#define MSA_FWD_LIST_WINDOW 4096
#endif
constexpr int kFwdListWindow = MSA_FWD_LIST_WINDOW;
// Workgroup size of the multi-workgroup scans over the lists.
constexpr int kScanItems = 4096;
// Tiles of one block list served by one block-major workgroup (the K/V
// block is staged once for all of them).
#ifndef MSA_TILES_PER_ITEM
#define MSA_TILES_PER_ITEM 8
#endif
constexpr int kTilesPerItem = MSA_TILES_PER_ITEM;

struct PrefillMainArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  float* lse;             // may be null
  const int32_t* bidx;    // selection rows (see launch_topk_prefill addressing)
  long bidx_rows;
  int bidx_t_off;
  int batch, T, Hq, G, B, topk;
  int t0, tc;             // query chunk
  int KS;                 // partial slots per (token, group) = min(topk, nb)
  int rank_bits;          // list entry = local token << rank_bits | slot; 2^rank_bits >= KS
  int include_local;      // lists also hold each row's local block (entries b <= L(t))
  int nbl;                // block lists per (batch, group, window) = nb
  int window;             // query tokens per list window
  int nwin;               // windows in this chunk = ceil(tc / window)
  long nlists;            // batch * G * nwin * nbl
  float scale_log2;       // softmax_scale * log2(e)
  // workspace
  int32_t* cnt;           // [nlists]
  int32_t* offs;          // [nlists]
  int32_t* bsum;          // [2 * ceil(nlists / kScanItems)] per-scan-block totals (entries, tiles)
  int32_t* rinfo;         // [batch*tc*G] per (token, group) row: partial slots | has_local << 30
  int32_t* epos;          // [batch*tc*G*KS] slot of an entry within its list; after the
                          // scatter pass, the entry's absolute position in list order
  int32_t* entries;       // [batch*tc*G*KS]
  int2* work;             // [max_work]
  int32_t* n_work;        // [1]
  long max_work;
  uint16_t* pO;           // [entries*R][128] fp16 unnormalised partial outputs in list order, scaled by 2^-e
  float2* pS;             // [entries*R] (max*c + e, sum * 2^-e), base-2 domain
};
hipError_t launch_prefill_main_sparse(const PrefillMainArgs& a, hipStream_t st);
// Block lists of a chunk (cnt, offs, epos -> list positions, entries, rinfo)
// and the work list of tiles of mt entries (a.work, a.n_work).
hipError_t launch_block_lists(const PrefillMainArgs& a, int mt, hipStream_t st);
// Sort every list's entries by (token, slot) and rewrite epos (after
// launch_block_lists): fixed summation order over a list.
hipError_t launch_sort_lists(const PrefillMainArgs& a, hipStream_t st);
// Another work list over the same lists, tiles of mt entries (a.bsum reused).
hipError_t launch_list_work(const PrefillMainArgs& a, int mt, int2* work, int32_t* n_work, hipStream_t st);
hipError_t launch_prefill_main_dense(const PrefillMainArgs& a, hipStream_t st);

// ---- Indexer KL loss (training signal of the index branch) ----
struct IndexerKlArgs {
  PrefillMainArgs l;      // lists of the chunk (include_local = 1); q, k, scale used
  const uint16_t* idx_q;  // [batch][T][G][di]
  const uint16_t* idx_k;  // [batch][T][di]
  const float* lse;       // [batch][T][Hq] main branch log-sum-exp (natural log)
  int di;
  float* kl;              // [batch][T][G]
  float* d_idx_q;         // [batch][T][G][di]
  float* d_idx_k;         // [batch][T][di]
  bool accumulate_dk;     // add onto d_idx_k (query chunks after the first)
  // workspace
  int2* work_a;           // work list over tiles of 128 entries
  int32_t* n_work_a;
  long max_work_a;
  float2* stat;           // [E] per entry (max, sum) of the index scores, base 2
  float* lse_i;           // [batch*tc*G] per row index log2-sum-exp
  uint16_t* ds;           // [E][B] bf16 p_I - p_M per entry and key
  float* kl_e;            // [E] per entry KL term
  uint16_t* dq_e;         // [E][di] per entry d idx_q term, bf16
  float* dk_part;         // [nlists][B][di] per list d idx_k partial
};
hipError_t launch_indexer_kl(const IndexerKlArgs& a, hipStream_t st);

// ---- Main-branch backward (selection held fixed) ----
struct BwdArgs {
  PrefillMainArgs l;      // lists of the chunk (include_local = 1); q, k, v, lse, scale used
  const uint16_t* o;      // [batch][T][Hq][128] forward output
  const uint16_t* dout;   // [batch][T][Hq][128]
  float* dq;              // [batch][T][Hq][128]
  float* dk;              // [batch][T][G][128]
  float* dv;              // [batch][T][G][128]
  bool accumulate;        // add dk, dv onto earlier query chunks
  // workspace
  float* delta;           // [batch*tc*Hq] dO . out
  int32_t* slot_of;       // [nlists] work item (partial slot) of a non-empty list
  uint16_t* dqp;          // [E*R][128] bf16 dq partial rows in list order
  float* part;            // [max_work][2][B][128] dk, dv partial per list
};
hipError_t launch_prefill_backward(const BwdArgs& a, hipStream_t st);

// ---- Decode ----
hipError_t launch_index_blockmax_decode(const uint16_t* idx_q, const uint16_t* idx_k,
                                        const int32_t* lens, float* S, int batch, int Lmax, int G,
                                        int di, int B, int s_stride, hipStream_t st);
struct DecodeMainArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* lens;
  uint16_t* out;
  float* lse;
  const int32_t* bidx;    // [batch][G][topk] (sparse / given)
  int batch, Lmax, Hq, G, B, topk;
  bool dense;
  int nsplit;             // work items per (s, g)
  int sub;                // sparse / given: work items per selected block (each covers B / sub keys)
  int blocks_per_split;   // dense: consecutive blocks per work item
  float scale_log2;
  float* pO;              // [batch*G*nsplit*R*128]
  float* pS;              // [batch*G*nsplit*R]
};
hipError_t launch_decode_main(const DecodeMainArgs& a, hipStream_t st);

}  // namespace msa
