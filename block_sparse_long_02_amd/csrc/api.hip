// C ABI of libmsa (declared in include/msa.h): host-side validation,
// workspace planning, the query-chunk loop and stream-ordered launches.
// Every argument check happens here, before any work is enqueued; no C++
// exception crosses the ABI.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "msa.h"
#include "msa_internal.h"

namespace {

thread_local char g_hip_err[256] = "";

constexpr size_t kAlignWs = 256;
// Default upper bound of the prefill workspace (per call).  Query chunks are
// sized so that the block-score table and the block-major partials of one
// chunk fit in it; MI355X has 288 GB of HBM per GPU.
constexpr size_t kDefaultPrefillBudget = 80ull << 30;
constexpr long kMaxInt32 = 2147483647L;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
  size_t total = 0;
  size_t add(size_t bytes) {
    const size_t off = total;
    total += round_up(bytes, kAlignWs);
    return off;
  }
};

int check_dims(const msa_dims* d, bool decode) {
  if (d == nullptr) return MSA_ERR_INVALID_ARG;
  if (d->batch < 1 || d->seqlen < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->topk < 1)
    return MSA_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return MSA_ERR_INVALID_ARG;
  if (d->reserved != 0 || d->query_chunk < 0) return MSA_ERR_INVALID_ARG;
  if (!isfinite(d->softmax_scale)) return MSA_ERR_INVALID_ARG;
  const uint32_t known = MSA_DENSE | MSA_GIVEN_INDICES | MSA_FORCE_SINK | MSA_CHECK_LENS | MSA_ONE_PASS_INDEX;
  if ((d->flags & ~known) != 0) return MSA_ERR_INVALID_ARG;
  if ((d->flags & MSA_CHECK_LENS) && !decode) return MSA_ERR_INVALID_ARG;  // a decode-only option
  // a prefill form of the index branch
  if ((d->flags & MSA_ONE_PASS_INDEX) && (decode || (d->flags & (MSA_DENSE | MSA_GIVEN_INDICES))))
    return MSA_ERR_INVALID_ARG;
  if ((d->flags & MSA_DENSE) && (d->flags & MSA_GIVEN_INDICES)) return MSA_ERR_INVALID_ARG;
  // the sink is a rule of the index branch's selection
  if ((d->flags & MSA_FORCE_SINK) && (d->flags & (MSA_DENSE | MSA_GIVEN_INDICES))) return MSA_ERR_INVALID_ARG;
  if (d->head_dim != 128) return MSA_ERR_UNSUPPORTED;
  if (d->index_dim != 64 && d->index_dim != 128) return MSA_ERR_UNSUPPORTED;
  if (d->block_size != 32 && d->block_size != 64 && d->block_size != 128) return MSA_ERR_UNSUPPORTED;
  const int R = d->num_q_heads / d->num_kv_heads;
  if (R > (decode ? 16 : msa::kAttnRows)) return MSA_ERR_UNSUPPORTED;
  if (!decode && d->query_chunk > 0 && d->query_chunk % d->block_size != 0) return MSA_ERR_INVALID_ARG;
  if ((d->flags & MSA_ONE_PASS_INDEX) && d->topk > msa::kOnePassMaxTopk) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

float log2_scale(const msa_dims* d) {
  const float sc = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
  return sc * 1.4426950408889634f;
}

// ---------------------------------------------------------------------------
// Prefill / index_topk plan
// ---------------------------------------------------------------------------
struct PrefillPlan {
  int nb = 0, KS = 0, R = 0, mt = 0, rank_bits = 0;
  int Tc = 0, nchunks = 0;
  int s_stride_max = 0, sm_stride_max = 0;
  long max_work = 0;
  bool with_scores = false, with_main = false;
  bool one_pass = false;  // MSA_ONE_PASS_INDEX: the index branch writes no score table
  size_t off_S = 0, off_SM = 0, off_bidx = 0, off_cnt = 0, off_offs = 0, off_bsum = 0, off_rinfo = 0, off_epos = 0,
         off_entries = 0, off_work = 0, off_nwork = 0, off_pO = 0, off_pS = 0;
  size_t total = 0;
};

// superblock maxima per row: ceil(L / 16) floats, padded to a multiple of 4
int sm_stride_for(int L) {
  const int n = (L + msa::kSuperBlock - 1) / msa::kSuperBlock;
  return (int)round_up((size_t)(n > 1 ? n : 1), 4);
}

size_t per_token_bytes(const msa_dims* d, const PrefillPlan& p) {
  const size_t G = (size_t)d->num_kv_heads;
  size_t b = 0;
  if (p.with_scores && !p.one_pass) b += G * ((size_t)p.s_stride_max + (size_t)p.sm_stride_max) * 4;
  if (p.with_scores && !(p.one_pass && !p.with_main)) b += G * (size_t)d->topk * 4;
  if (p.with_main) b += G * 4 + G * (size_t)p.KS * (4 + 4 + (size_t)p.R * (128 * 2 + 8));
  return b;
}

int make_prefill_plan(const msa_dims* d, bool index_only, PrefillPlan* p) {
  int st = check_dims(d, false);
  if (st != MSA_OK) return st;
  if (index_only && (d->flags & ~(MSA_FORCE_SINK | MSA_ONE_PASS_INDEX)) != 0) return MSA_ERR_INVALID_ARG;
  const int T = d->seqlen, B = d->block_size, G = d->num_kv_heads;
  p->nb = (T + B - 1) / B;
  p->KS = d->topk < p->nb ? d->topk : p->nb;
  while ((1 << p->rank_bits) < p->KS) ++p->rank_bits;
  p->R = d->num_q_heads / G;
  p->mt = msa::kAttnRows / p->R;
  p->with_scores = index_only || !(d->flags & (MSA_DENSE | MSA_GIVEN_INDICES));
  p->with_main = !index_only && !(d->flags & MSA_DENSE);
  p->one_pass = (d->flags & MSA_ONE_PASS_INDEX) != 0;
  const int Lmax = (T - 1) / B;
  // rows of the block-score table start 64-byte aligned (the index kernel
  // stores 16 block maxima per row at a time)
  p->s_stride_max = (int)round_up((size_t)(Lmax > 1 ? Lmax : 1), 16);
  p->sm_stride_max = sm_stride_for(Lmax);
  if (!p->with_scores && !p->with_main) {  // dense prefill needs no workspace
    p->Tc = T;
    p->nchunks = 1;
    p->total = 0;
    return MSA_OK;
  }
  const size_t ptb = per_token_bytes(d, *p) * (size_t)d->batch;
  long tc_max;
  if (d->query_chunk > 0) {
    tc_max = d->query_chunk;
  } else {
    tc_max = (long)(kDefaultPrefillBudget / (ptb ? ptb : 1));
    tc_max = tc_max / B * B;
    if (tc_max < B) tc_max = B;
  }
  // keep per-chunk entry counts and indices inside int32
  const long per_tok_entries = (long)d->batch * G * p->KS;
  if (p->with_main) {
    const long lim = (kMaxInt32 / 2) / (per_tok_entries ? per_tok_entries : 1);
    if (tc_max > lim) tc_max = lim / B * B;
    // packed list entries (local token << rank_bits | slot) stay in int32
    const long lim2 = (long)kMaxInt32 >> p->rank_bits;
    if (tc_max > lim2) tc_max = lim2 / B * B;
    // list ids (batch, group, window, block) stay in int32
    const long lists_per_win = (long)d->batch * G * p->nb;
    const long max_win = (kMaxInt32 - 1) / lists_per_win;
    if (max_win < 1) return MSA_ERR_UNSUPPORTED;
    if ((tc_max + msa::kFwdListWindow - 1) / msa::kFwdListWindow > max_win) tc_max = max_win * msa::kFwdListWindow;
    if (tc_max < B) return MSA_ERR_UNSUPPORTED;
  }
  if (tc_max >= T) {
    p->Tc = T;
    p->nchunks = 1;
  } else {
    const long nch = (T + tc_max - 1) / tc_max;
    long tc = (T + nch - 1) / nch;
    tc = (long)round_up((size_t)tc, (size_t)B);
    if (tc > tc_max) tc = tc_max;
    p->Tc = (int)tc;
    p->nchunks = (int)((T + tc - 1) / tc);
  }
  Layout L;
  const size_t nb_ = (size_t)d->batch, Tc = (size_t)p->Tc, G_ = (size_t)G;
  if (p->with_scores) {
    if (!p->one_pass) {
      p->off_S = L.add(nb_ * Tc * G_ * (size_t)p->s_stride_max * 4);
      p->off_SM = L.add(nb_ * Tc * G_ * (size_t)p->sm_stride_max * 4);
    }
    // the one-pass msa_index_topk needs no workspace at all
    if (!(p->one_pass && index_only)) p->off_bidx = L.add(nb_ * Tc * G_ * (size_t)d->topk * 4);
  }
  if (p->with_main) {
    const size_t nwin = ((size_t)p->Tc + msa::kFwdListWindow - 1) / msa::kFwdListWindow;
    const size_t nlists = nb_ * G_ * nwin * (size_t)p->nb;
    const size_t nscan = (nlists + msa::kScanItems - 1) / msa::kScanItems;
    const size_t emax = nb_ * Tc * G_ * (size_t)p->KS;
    p->max_work = (long)((emax + p->mt - 1) / p->mt + nlists);
    p->off_cnt = L.add(nlists * 4);
    p->off_offs = L.add(nlists * 4);
    p->off_bsum = L.add(nscan * 8);
    p->off_rinfo = L.add(nb_ * Tc * G_ * 4);
    p->off_epos = L.add(emax * 4);
    p->off_entries = L.add(emax * 4);
    p->off_work = L.add((size_t)p->max_work * 8);
    p->off_nwork = L.add(4);
    // partial rows are stored in blocks of 32 rows (8 KiB)
    p->off_pO = L.add(round_up(emax * (size_t)p->R, 32) * 128 * 2);
    p->off_pS = L.add(emax * (size_t)p->R * 8);
  }
  p->total = L.total;
  return MSA_OK;
}

// ---------------------------------------------------------------------------
// Indexer KL plan: block lists over every selected block (local included),
// per-entry terms and per-list d idx_k partials of one query chunk.
// ---------------------------------------------------------------------------
constexpr size_t kDefaultKlBudget = 64ull << 30;

struct KlPlan {
  int nb = 0, KS = 0, R = 0, mt = 0, rank_bits = 0;
  int Tc = 0, nchunks = 0;
  size_t off_cnt = 0, off_offs = 0, off_bsum = 0, off_rinfo = 0, off_epos = 0, off_entries = 0, off_work = 0,
         off_nwork = 0, off_work_a = 0, off_nwork_a = 0, off_stat = 0, off_lse_i = 0, off_ds = 0, off_kl_e = 0,
         off_dq_e = 0, off_dk = 0, total = 0;
  long max_work = 0, max_work_a = 0;
};

// workspace bytes of a chunk of tc tokens
size_t kl_chunk_bytes(const msa_dims* d, const KlPlan& p, long tc, KlPlan* out) {
  Layout L;
  const size_t nb_ = (size_t)d->batch, G_ = (size_t)d->num_kv_heads, B_ = (size_t)d->block_size;
  const size_t di = (size_t)d->index_dim;
  const size_t nwin = ((size_t)tc + msa::kListWindow - 1) / msa::kListWindow;
  const size_t nlists = nb_ * G_ * nwin * (size_t)p.nb;
  const size_t nscan = (nlists + msa::kScanItems - 1) / msa::kScanItems;
  const size_t rows = nb_ * (size_t)tc * G_;
  const size_t emax = rows * (size_t)p.KS;
  KlPlan q = p;
  q.max_work = (long)((emax + p.mt - 1) / p.mt + nlists);
  q.max_work_a = (long)((emax + 127) / 128 + nlists);
  q.off_cnt = L.add(nlists * 4);
  q.off_offs = L.add(nlists * 4);
  q.off_bsum = L.add(nscan * 8);
  q.off_rinfo = L.add(rows * 4);
  q.off_epos = L.add(emax * 4);
  q.off_entries = L.add(emax * 4);
  q.off_work = L.add((size_t)q.max_work * 8);
  q.off_nwork = L.add(4);
  q.off_work_a = L.add((size_t)q.max_work_a * 8);
  q.off_nwork_a = L.add(4);
  q.off_stat = L.add(emax * 8);
  q.off_lse_i = L.add(rows * 4);
  q.off_ds = L.add(emax * B_ * 2);
  q.off_kl_e = L.add(emax * 4);
  q.off_dq_e = L.add(emax * di * 2);
  q.off_dk = L.add(nlists * B_ * di * 4);
  q.total = L.total;
  if (out != nullptr) *out = q;
  return q.total;
}

int make_kl_plan(const msa_dims* d, KlPlan* p) {
  int st = check_dims(d, false);
  if (st != MSA_OK) return st;
  if (d->flags != 0) return MSA_ERR_INVALID_ARG;
  const int T = d->seqlen, B = d->block_size, G = d->num_kv_heads;
  p->R = d->num_q_heads / G;
  p->nb = (T + B - 1) / B;
  p->KS = d->topk < p->nb ? d->topk : p->nb;
  p->mt = msa::kAttnRows / p->R;
  while ((1 << p->rank_bits) < p->KS) ++p->rank_bits;
  // largest chunk (a multiple of the list window, else of B) within the budget and the int32 limits
  const long per_tok_entries = (long)d->batch * G * p->KS;
  long lim = (kMaxInt32 / 2) / (per_tok_entries ? per_tok_entries : 1);
  const long lim2 = (long)kMaxInt32 >> p->rank_bits;
  if (lim2 < lim) lim = lim2;
  const long lists_per_win = (long)d->batch * G * p->nb;
  const long max_win = (kMaxInt32 - 1) / lists_per_win;
  if (max_win < 1) return MSA_ERR_UNSUPPORTED;
  if (max_win * msa::kListWindow < lim) lim = max_win * msa::kListWindow;
  long tc;
  if (d->query_chunk > 0) {
    tc = d->query_chunk < T ? d->query_chunk : T;
  } else {
    tc = ((long)T + msa::kListWindow - 1) / msa::kListWindow * msa::kListWindow;
    while (tc > msa::kListWindow && kl_chunk_bytes(d, *p, tc, nullptr) > kDefaultKlBudget) tc -= msa::kListWindow;
    while (tc > B && kl_chunk_bytes(d, *p, tc, nullptr) > kDefaultKlBudget) tc -= B;
    if (tc > T) tc = T;
  }
  if (tc > lim) tc = lim / B * B;
  if (tc < 1) return MSA_ERR_UNSUPPORTED;
  p->Tc = (int)tc;
  p->nchunks = (int)((T + tc - 1) / tc);
  kl_chunk_bytes(d, *p, tc, p);
  return MSA_OK;
}

// ---------------------------------------------------------------------------
// Backward plan: block lists over every selected block (local included), the
// dq partial rows (bf16, one per entry and head) and one dk/dv partial block
// per non-empty list, for one query chunk.
// ---------------------------------------------------------------------------
constexpr size_t kDefaultBwdBudget = 64ull << 30;

struct BwdPlan {
  int nb = 0, KS = 0, R = 0, rank_bits = 0;
  int Tc = 0, nchunks = 0;
  size_t off_delta = 0, off_cnt = 0, off_offs = 0, off_bsum = 0, off_rinfo = 0, off_epos = 0, off_entries = 0,
         off_work = 0, off_nwork = 0, off_slot = 0, off_dqp = 0, off_part = 0, total = 0;
  long max_lists = 0;  // non-empty lists of a chunk, at most
};

// Non-empty lists of any chunk of a tc-token split, at most: block b of window
// w can hold entries only when b <= L of the window's last token.
long bwd_max_lists(const msa_dims* d, const BwdPlan& p, long tc) {
  const long W = msa::kListWindow, B = d->block_size, T = d->seqlen;
  long best = 0;
  for (long t0 = 0; t0 < T; t0 += tc) {
    const long len = T - t0 < tc ? T - t0 : tc;
    long n = 0;
    for (long w = 0; w * W < len; ++w) {
      const long last = t0 + ((w + 1) * W < len ? (w + 1) * W : len) - 1;
      const long nbw = last / B + 1;
      n += nbw < p.nb ? nbw : p.nb;
    }
    if (n > best) best = n;
  }
  best *= (long)d->batch * d->num_kv_heads;
  const long emax = (long)d->batch * tc * d->num_kv_heads * p.KS;
  return best < emax ? best : emax;
}

size_t bwd_chunk_bytes(const msa_dims* d, const BwdPlan& p, long tc, BwdPlan* out) {
  Layout L;
  const size_t nb_ = (size_t)d->batch, G_ = (size_t)d->num_kv_heads, B_ = (size_t)d->block_size;
  const size_t nwin = ((size_t)tc + msa::kListWindow - 1) / msa::kListWindow;
  const size_t nlists = nb_ * G_ * nwin * (size_t)p.nb;
  const size_t nscan = (nlists + msa::kScanItems - 1) / msa::kScanItems;
  const size_t rows = nb_ * (size_t)tc * G_;
  const size_t emax = rows * (size_t)p.KS;
  BwdPlan q = p;
  q.max_lists = bwd_max_lists(d, p, tc);
  q.off_delta = L.add(nb_ * (size_t)tc * (size_t)d->num_q_heads * 4);
  q.off_cnt = L.add(nlists * 4);
  q.off_offs = L.add(nlists * 4);
  q.off_bsum = L.add(nscan * 8);
  q.off_rinfo = L.add(rows * 4);
  q.off_epos = L.add(emax * 4);
  q.off_entries = L.add(emax * 4);
  q.off_work = L.add((size_t)q.max_lists * 8);
  q.off_nwork = L.add(4);
  q.off_slot = L.add(nlists * 4);
  q.off_dqp = L.add(emax * (size_t)p.R * 128 * 2);
  q.off_part = L.add((size_t)q.max_lists * 2 * B_ * 128 * 4);
  q.total = L.total;
  if (out != nullptr) *out = q;
  return q.total;
}

int make_bwd_plan(const msa_dims* d, BwdPlan* p) {
  int st = check_dims(d, false);
  if (st != MSA_OK) return st;
  if (d->flags != 0) return MSA_ERR_INVALID_ARG;
  const int T = d->seqlen, B = d->block_size, G = d->num_kv_heads;
  p->R = d->num_q_heads / G;
  p->nb = (T + B - 1) / B;
  p->KS = d->topk < p->nb ? d->topk : p->nb;
  while ((1 << p->rank_bits) < p->KS) ++p->rank_bits;
  // largest chunk (a multiple of the list window, else of B) within the budget and the int32 limits
  const long per_tok_entries = (long)d->batch * G * p->KS;
  long lim = (kMaxInt32 / 2) / (per_tok_entries ? per_tok_entries : 1);
  const long lim2 = (long)kMaxInt32 >> p->rank_bits;
  if (lim2 < lim) lim = lim2;
  const long lists_per_win = (long)d->batch * G * p->nb;
  const long max_win = (kMaxInt32 - 1) / lists_per_win;
  if (max_win < 1) return MSA_ERR_UNSUPPORTED;
  if (max_win * msa::kListWindow < lim) lim = max_win * msa::kListWindow;
  long tc;
  if (d->query_chunk > 0) {
    tc = d->query_chunk < T ? d->query_chunk : T;
  } else {
    tc = ((long)T + msa::kListWindow - 1) / msa::kListWindow * msa::kListWindow;
    while (tc > msa::kListWindow && bwd_chunk_bytes(d, *p, tc, nullptr) > kDefaultBwdBudget) tc -= msa::kListWindow;
    while (tc > B && bwd_chunk_bytes(d, *p, tc, nullptr) > kDefaultBwdBudget) tc -= B;
    if (tc > T) tc = T;
  }
  if (tc > lim) tc = lim / B * B;
  if (tc < 1) return MSA_ERR_UNSUPPORTED;
  p->Tc = (int)tc;
  p->nchunks = (int)((T + tc - 1) / tc);
  bwd_chunk_bytes(d, *p, tc, p);
  return MSA_OK;
}

// ---------------------------------------------------------------------------
// Decode plan
// ---------------------------------------------------------------------------
#ifndef MSA_DEC_ITEM_KEYS
#define MSA_DEC_ITEM_KEYS 64
#endif

struct DecodePlan {
  int nbmax = 0, R = 0, s_stride = 0, nsplit = 0, bps = 0, sub = 1;
  bool with_scores = false;
  size_t off_S = 0, off_bidx = 0, off_pO = 0, off_pS = 0, total = 0;
};

int make_decode_plan(const msa_dims* d, DecodePlan* p) {
  int st = check_dims(d, true);
  if (st != MSA_OK) return st;
  const int B = d->block_size, G = d->num_kv_heads;
  p->nbmax = (d->seqlen + B - 1) / B;
  p->R = d->num_q_heads / G;
  p->s_stride = (int)round_up((size_t)p->nbmax, 4);
  p->with_scores = !(d->flags & (MSA_DENSE | MSA_GIVEN_INDICES));
  if (d->flags & MSA_DENSE) {
    p->bps = 2048 / B;  // 2048 keys per work item
    p->nsplit = (p->nbmax + p->bps - 1) / p->bps;
  } else {
    // blocks are split into work items of MSA_DEC_ITEM_KEYS keys: one key
    // tile per wave, so no wave waits for two loads in turn
    p->sub = B > MSA_DEC_ITEM_KEYS ? B / MSA_DEC_ITEM_KEYS : 1;
    const int sel = (d->flags & MSA_GIVEN_INDICES) ? d->topk : (d->topk < p->nbmax ? d->topk : p->nbmax);
    p->nsplit = sel * p->sub;
  }
  Layout L;
  const size_t nb_ = (size_t)d->batch, G_ = (size_t)G;
  if (p->with_scores) {
    p->off_S = L.add(nb_ * G_ * (size_t)p->s_stride * 4);
    p->off_bidx = L.add(nb_ * G_ * (size_t)d->topk * 4);
  }
  p->off_pO = L.add(nb_ * G_ * (size_t)p->nsplit * p->R * 128 * 4);
  p->off_pS = L.add(nb_ * G_ * (size_t)p->nsplit * p->R * 4);
  p->total = L.total;
  return MSA_OK;
}

bool misaligned(const void* ptr, size_t a) { return ptr != nullptr && ((uintptr_t)ptr % a) != 0; }

int hip_fail(hipError_t e) {
  snprintf(g_hip_err, sizeof(g_hip_err), "%s (%d)", hipGetErrorString(e), (int)e);
  return MSA_ERR_HIP;
}

int check_workspace(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return MSA_OK;
  if (ws == nullptr) return MSA_ERR_INVALID_ARG;
  if (misaligned(ws, kAlignWs)) return MSA_ERR_ALIGNMENT;
  if (ws_bytes < need) return MSA_ERR_WORKSPACE;
  return MSA_OK;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Index Branch for one chunk: scores + top-k into (bidx, rows, t_off).
hipError_t run_index_chunk(const msa_dims* d, const PrefillPlan& p, const void* idx_q,
                           const void* idx_k, void* ws, int t0, int tc, int32_t* bidx, long bidx_rows,
                           int t_off, hipStream_t st) {
  const int B = d->block_size;
  if (p.one_pass) {
    msa::prof_mark(st, MSA_STAGE_INDEX_ONE_PASS);
    return msa::launch_index_topk_one_pass(static_cast<const uint16_t*>(idx_q), static_cast<const uint16_t*>(idx_k),
                                           bidx, bidx_rows, t_off, d->batch, d->seqlen, d->num_kv_heads,
                                           d->index_dim, B, d->topk, (d->flags & MSA_FORCE_SINK) != 0, t0, tc, st);
  }
  const int Lc = (t0 + tc - 1) / B;
  const int s_stride = (int)round_up((size_t)(Lc > 1 ? Lc : 1), 16);
  const int sm_stride = sm_stride_for(Lc);
  float* S = at<float>(ws, p.off_S);
  float* SM = Lc > msa::kSbMinCandidates ? at<float>(ws, p.off_SM) : nullptr;
  msa::prof_mark(st, MSA_STAGE_INDEX_PREFILL);
  hipError_t e = msa::launch_index_blockmax_prefill(
      static_cast<const uint16_t*>(idx_q), static_cast<const uint16_t*>(idx_k), S, d->batch,
      d->seqlen, d->num_kv_heads, d->index_dim, B, t0, tc, s_stride, SM, sm_stride, st);
  if (e != hipSuccess) return e;
  msa::prof_mark(st, MSA_STAGE_TOPK_PREFILL);
  return msa::launch_topk_prefill(S, s_stride, SM, sm_stride, bidx, bidx_rows, t_off, d->batch, d->num_kv_heads, B,
                                  d->topk, (d->flags & MSA_FORCE_SINK) != 0, t0, tc, st);
}

// ---------------------------------------------------------------------------
// Library-owned decode scratch for msa_decode_noalloc: a fixed device array
// (one copy per GPU, held until the process ends) whose device address is
// looked up once per device.  Host code never passes the array's own name to
// a kernel: that name is a host-side stand-in, not a device address.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = 32ull << 20;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return MSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (ptr == nullptr || misaligned(ptr, kAlignWs)) return MSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

int run_decode(const msa_dims* dims, const DecodePlan& p, const void* q, const void* k_cache, const void* v_cache,
               const void* idx_q, const void* idx_k_cache, const int32_t* cache_lens, void* out, float* lse,
               int32_t* block_idx, void* workspace, size_t workspace_bytes, void* hip_stream);

}  // namespace

extern "C" {

int msa_abi_version(void) { return 1; }

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG: null pointer, non-positive size, Hq % G != 0 or bad flags";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED: head_dim, index_dim, block_size or heads per group not supported";
    case MSA_ERR_ALIGNMENT: return "MSA_ERR_ALIGNMENT: tensor or workspace pointer misaligned";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE: workspace smaller than msa_workspace_bytes()";
    case MSA_ERR_HIP: return "MSA_ERR_HIP: a HIP launch failed (see msa_last_hip_error)";
    default: return "unknown msa status";
  }
}

const char* msa_last_hip_error(void) { return g_hip_err; }

size_t msa_workspace_bytes(int op, const msa_dims* dims) {
  if (op == MSA_OP_INDEX_TOPK || op == MSA_OP_PREFILL) {
    PrefillPlan p;
    if (make_prefill_plan(dims, op == MSA_OP_INDEX_TOPK, &p) != MSA_OK) return (size_t)-1;
    return p.total;
  }
  if (op == MSA_OP_DECODE) {
    DecodePlan p;
    if (make_decode_plan(dims, &p) != MSA_OK) return (size_t)-1;
    return p.total;
  }
  if (op == MSA_OP_INDEXER_KL) {
    KlPlan p;
    if (make_kl_plan(dims, &p) != MSA_OK) return (size_t)-1;
    return p.total;
  }
  if (op == MSA_OP_BACKWARD) {
    BwdPlan p;
    if (make_bwd_plan(dims, &p) != MSA_OK) return (size_t)-1;
    return p.total;
  }
  return (size_t)-1;
}

int msa_index_topk(const msa_dims* dims, const void* idx_q, const void* idx_k, int32_t* block_idx,
                   void* workspace, size_t workspace_bytes, void* hip_stream) {
  PrefillPlan p;
  int st = make_prefill_plan(dims, true, &p);
  if (st != MSA_OK) return st;
  if (idx_q == nullptr || idx_k == nullptr || block_idx == nullptr) return MSA_ERR_INVALID_ARG;
  if (misaligned(idx_q, 16) || misaligned(idx_k, 16) || misaligned(block_idx, 4)) return MSA_ERR_ALIGNMENT;
  if ((st = check_workspace(p.total, workspace, workspace_bytes)) != MSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * p.Tc;
    const int tc = (dims->seqlen - t0) < p.Tc ? dims->seqlen - t0 : p.Tc;
    hipError_t e = run_index_chunk(dims, p, idx_q, idx_k, workspace, t0, tc, block_idx, dims->seqlen, 0, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  msa::prof_mark(s, -1);
  return MSA_OK;
}

int msa_index_scores(const msa_dims* dims, const void* idx_q, const void* idx_k, float* scores,
                     int32_t t0, int32_t t1, int32_t row_stride, float* superblock_max,
                     int32_t sb_stride, void* hip_stream) {
  int st = check_dims(dims, false);
  if (st != MSA_OK) return st;
  if ((dims->flags & ~MSA_FORCE_SINK) != 0) return MSA_ERR_INVALID_ARG;  // scores do not depend on it
  if (idx_q == nullptr || idx_k == nullptr || scores == nullptr) return MSA_ERR_INVALID_ARG;
  if (t0 < 0 || t1 <= t0 || t1 > dims->seqlen) return MSA_ERR_INVALID_ARG;
  const int Lc = (t1 - 1) / dims->block_size;
  if (row_stride < 4 || row_stride % 4 != 0 || row_stride < Lc) return MSA_ERR_INVALID_ARG;
  if (superblock_max != nullptr && (sb_stride < (Lc + msa::kSuperBlock - 1) / msa::kSuperBlock || sb_stride < 1))
    return MSA_ERR_INVALID_ARG;
  if (misaligned(idx_q, 16) || misaligned(idx_k, 16) || misaligned(scores, 16) || misaligned(superblock_max, 4))
    return MSA_ERR_ALIGNMENT;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  msa::prof_mark(s, MSA_STAGE_INDEX_PREFILL);
  hipError_t e = msa::launch_index_blockmax_prefill(
      static_cast<const uint16_t*>(idx_q), static_cast<const uint16_t*>(idx_k), scores, dims->batch,
      dims->seqlen, dims->num_kv_heads, dims->index_dim, dims->block_size, t0, t1 - t0, row_stride,
      superblock_max, superblock_max != nullptr ? sb_stride : 0, s);
  msa::prof_mark(s, -1);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

int msa_prefill(const msa_dims* dims, const void* q, const void* k, const void* v, const void* idx_q,
                const void* idx_k, void* out, float* lse, int32_t* block_idx, void* workspace,
                size_t workspace_bytes, void* hip_stream) {
  PrefillPlan p;
  int st = make_prefill_plan(dims, false, &p);
  if (st != MSA_OK) return st;
  const bool dense = dims->flags & MSA_DENSE, given = dims->flags & MSA_GIVEN_INDICES;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return MSA_ERR_INVALID_ARG;
  if (!dense && !given && (idx_q == nullptr || idx_k == nullptr)) return MSA_ERR_INVALID_ARG;
  if (dense && block_idx != nullptr) return MSA_ERR_INVALID_ARG;
  if (given && block_idx == nullptr) return MSA_ERR_INVALID_ARG;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) ||
      misaligned(idx_q, 16) || misaligned(idx_k, 16) || misaligned(lse, 4) || misaligned(block_idx, 4))
    return MSA_ERR_ALIGNMENT;
  if ((st = check_workspace(p.total, workspace, workspace_bytes)) != MSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);

  msa::PrefillMainArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.batch = dims->batch;
  a.T = dims->seqlen;
  a.Hq = dims->num_q_heads;
  a.G = dims->num_kv_heads;
  a.B = dims->block_size;
  a.topk = dims->topk;
  a.KS = p.KS;
  a.rank_bits = p.rank_bits;
  a.nbl = p.nb;
  a.scale_log2 = log2_scale(dims);

  if (dense) {
    a.t0 = 0;
    a.tc = dims->seqlen;
    msa::prof_mark(s, MSA_STAGE_QUERY_MAJOR_DENSE);
    hipError_t e = msa::launch_prefill_main_dense(a, s);
    msa::prof_mark(s, -1);
    return e == hipSuccess ? MSA_OK : hip_fail(e);
  }
  a.cnt = at<int32_t>(workspace, p.off_cnt);
  a.offs = at<int32_t>(workspace, p.off_offs);
  a.rinfo = at<int32_t>(workspace, p.off_rinfo);
  a.epos = at<int32_t>(workspace, p.off_epos);
  a.entries = at<int32_t>(workspace, p.off_entries);
  a.work = at<int2>(workspace, p.off_work);
  a.n_work = at<int32_t>(workspace, p.off_nwork);
  a.bsum = at<int32_t>(workspace, p.off_bsum);
  a.pO = at<uint16_t>(workspace, p.off_pO);
  a.pS = at<float2>(workspace, p.off_pS);

  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * p.Tc;
    const int tc = (dims->seqlen - t0) < p.Tc ? dims->seqlen - t0 : p.Tc;
    int32_t* bidx;
    long rows;
    int t_off;
    if (block_idx != nullptr) {
      bidx = block_idx;
      rows = dims->seqlen;
      t_off = 0;
    } else {
      bidx = at<int32_t>(workspace, p.off_bidx);
      rows = p.Tc;
      t_off = t0;
    }
    if (!given) {
      hipError_t e = run_index_chunk(dims, p, idx_q, idx_k, workspace, t0, tc, bidx, rows, t_off, s);
      if (e != hipSuccess) return hip_fail(e);
    }
    a.bidx = bidx;
    a.bidx_rows = rows;
    a.bidx_t_off = t_off;
    a.t0 = t0;
    a.tc = tc;
    const long emax = (long)dims->batch * tc * dims->num_kv_heads * p.KS;
    a.window = msa::kFwdListWindow;
    a.nwin = (tc + msa::kFwdListWindow - 1) / msa::kFwdListWindow;
    a.nlists = (long)dims->batch * dims->num_kv_heads * a.nwin * p.nb;
    a.max_work = (emax + p.mt - 1) / p.mt + a.nlists;
    hipError_t e = msa::launch_prefill_main_sparse(a, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  msa::prof_mark(s, -1);
  return MSA_OK;
}

int msa_indexer_kl(const msa_dims* dims, const void* q, const void* k, const void* idx_q, const void* idx_k,
                   const int32_t* block_idx, const float* lse, float* kl, float* d_idx_q, float* d_idx_k,
                   void* workspace, size_t workspace_bytes, void* hip_stream) {
  KlPlan p;
  int st = make_kl_plan(dims, &p);
  if (st != MSA_OK) return st;
  if (q == nullptr || k == nullptr || idx_q == nullptr || idx_k == nullptr || block_idx == nullptr ||
      lse == nullptr || kl == nullptr || d_idx_q == nullptr || d_idx_k == nullptr)
    return MSA_ERR_INVALID_ARG;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(idx_q, 16) || misaligned(idx_k, 16) ||
      misaligned(block_idx, 4) || misaligned(lse, 4) || misaligned(kl, 4) || misaligned(d_idx_q, 16) ||
      misaligned(d_idx_k, 4))
    return MSA_ERR_ALIGNMENT;
  if ((st = check_workspace(p.total, workspace, workspace_bytes)) != MSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  msa::IndexerKlArgs a{};
  msa::PrefillMainArgs& l = a.l;
  l.q = static_cast<const uint16_t*>(q);
  l.k = static_cast<const uint16_t*>(k);
  l.batch = dims->batch;
  l.T = dims->seqlen;
  l.Hq = dims->num_q_heads;
  l.G = dims->num_kv_heads;
  l.B = dims->block_size;
  l.topk = dims->topk;
  l.KS = p.KS;
  l.rank_bits = p.rank_bits;
  l.include_local = 1;
  l.nbl = p.nb;
  l.scale_log2 = log2_scale(dims);
  l.bidx = block_idx;
  l.bidx_rows = dims->seqlen;
  l.bidx_t_off = 0;
  l.cnt = at<int32_t>(workspace, p.off_cnt);
  l.offs = at<int32_t>(workspace, p.off_offs);
  l.bsum = at<int32_t>(workspace, p.off_bsum);
  l.rinfo = at<int32_t>(workspace, p.off_rinfo);
  l.epos = at<int32_t>(workspace, p.off_epos);
  l.entries = at<int32_t>(workspace, p.off_entries);
  l.work = at<int2>(workspace, p.off_work);
  l.n_work = at<int32_t>(workspace, p.off_nwork);
  a.idx_q = static_cast<const uint16_t*>(idx_q);
  a.idx_k = static_cast<const uint16_t*>(idx_k);
  a.lse = lse;
  a.di = dims->index_dim;
  a.kl = kl;
  a.d_idx_q = d_idx_q;
  a.d_idx_k = d_idx_k;
  a.work_a = at<int2>(workspace, p.off_work_a);
  a.n_work_a = at<int32_t>(workspace, p.off_nwork_a);
  a.stat = at<float2>(workspace, p.off_stat);
  a.lse_i = at<float>(workspace, p.off_lse_i);
  a.ds = at<uint16_t>(workspace, p.off_ds);
  a.kl_e = at<float>(workspace, p.off_kl_e);
  a.dq_e = at<uint16_t>(workspace, p.off_dq_e);
  a.dk_part = at<float>(workspace, p.off_dk);
  msa::prof_mark(s, MSA_STAGE_INDEXER_KL);
  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * p.Tc;
    const int tc = (dims->seqlen - t0) < p.Tc ? dims->seqlen - t0 : p.Tc;
    const long emax = (long)dims->batch * tc * dims->num_kv_heads * p.KS;
    l.t0 = t0;
    l.tc = tc;
    l.window = msa::kListWindow;
    l.nwin = (tc + msa::kListWindow - 1) / msa::kListWindow;
    l.nlists = (long)dims->batch * dims->num_kv_heads * l.nwin * p.nb;
    l.max_work = (emax + p.mt - 1) / p.mt + l.nlists;
    a.max_work_a = (emax + 127) / 128 + l.nlists;
    a.accumulate_dk = c > 0;
    hipError_t e = msa::launch_indexer_kl(a, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  msa::prof_mark(s, -1);
  return MSA_OK;
}

int msa_prefill_backward(const msa_dims* dims, const void* q, const void* k, const void* v, const void* out,
                         const float* lse, const void* dout, const int32_t* block_idx, float* dq, float* dk,
                         float* dv, void* workspace, size_t workspace_bytes, void* hip_stream) {
  BwdPlan p;
  int st = make_bwd_plan(dims, &p);
  if (st != MSA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || lse == nullptr || dout == nullptr ||
      block_idx == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return MSA_ERR_INVALID_ARG;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(out, 16) || misaligned(dout, 16) ||
      misaligned(lse, 4) || misaligned(block_idx, 4) || misaligned(dq, 16) || misaligned(dk, 4) ||
      misaligned(dv, 4))
    return MSA_ERR_ALIGNMENT;
  if ((st = check_workspace(p.total, workspace, workspace_bytes)) != MSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  msa::BwdArgs a{};
  msa::PrefillMainArgs& l = a.l;
  l.q = static_cast<const uint16_t*>(q);
  l.k = static_cast<const uint16_t*>(k);
  l.v = static_cast<const uint16_t*>(v);
  l.lse = const_cast<float*>(lse);  // read only
  l.batch = dims->batch;
  l.T = dims->seqlen;
  l.Hq = dims->num_q_heads;
  l.G = dims->num_kv_heads;
  l.B = dims->block_size;
  l.topk = dims->topk;
  l.KS = p.KS;
  l.rank_bits = p.rank_bits;
  l.include_local = 1;
  l.nbl = p.nb;
  l.scale_log2 = log2_scale(dims);
  l.bidx = block_idx;
  l.bidx_rows = dims->seqlen;
  l.bidx_t_off = 0;
  l.cnt = at<int32_t>(workspace, p.off_cnt);
  l.offs = at<int32_t>(workspace, p.off_offs);
  l.bsum = at<int32_t>(workspace, p.off_bsum);
  l.rinfo = at<int32_t>(workspace, p.off_rinfo);
  l.epos = at<int32_t>(workspace, p.off_epos);
  l.entries = at<int32_t>(workspace, p.off_entries);
  l.work = at<int2>(workspace, p.off_work);
  l.n_work = at<int32_t>(workspace, p.off_nwork);
  a.o = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = at<float>(workspace, p.off_delta);
  a.slot_of = at<int32_t>(workspace, p.off_slot);
  a.dqp = at<uint16_t>(workspace, p.off_dqp);
  a.part = at<float>(workspace, p.off_part);
  for (int c = 0; c < p.nchunks; ++c) {
    const int t0 = c * p.Tc;
    const int tc = (dims->seqlen - t0) < p.Tc ? dims->seqlen - t0 : p.Tc;
    l.t0 = t0;
    l.tc = tc;
    l.window = msa::kListWindow;
    l.nwin = (tc + msa::kListWindow - 1) / msa::kListWindow;
    l.nlists = (long)dims->batch * dims->num_kv_heads * l.nwin * p.nb;
    l.max_work = p.max_lists;
    a.accumulate = c > 0;
    hipError_t e = msa::launch_prefill_backward(a, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  msa::prof_mark(s, -1);
  return MSA_OK;
}

int msa_decode(const msa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
               const void* idx_q, const void* idx_k_cache, const int32_t* cache_lens, void* out,
               float* lse, int32_t* block_idx, void* workspace, size_t workspace_bytes,
               void* hip_stream) {
  DecodePlan p;
  int st = make_decode_plan(dims, &p);
  if (st != MSA_OK) return st;
  return run_decode(dims, p, q, k_cache, v_cache, idx_q, idx_k_cache, cache_lens, out, lse, block_idx, workspace,
                    workspace_bytes, hip_stream);
}

int msa_decode_noalloc(const msa_dims* dims, const void* q, const void* k_cache, const void* v_cache,
                       const void* idx_q, const void* idx_k_cache, const int32_t* cache_lens, void* out,
                       float* lse, int32_t* block_idx, void* hip_stream) {
  DecodePlan p;
  int st = make_decode_plan(dims, &p);
  if (st != MSA_OK) return st;
  if (dims->flags & MSA_CHECK_LENS) return MSA_ERR_INVALID_ARG;  // it would synchronize the stream
  if (p.total > kScratchBytes) return MSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != MSA_OK) return st;
  return run_decode(dims, p, q, k_cache, v_cache, idx_q, idx_k_cache, cache_lens, out, lse, block_idx, ws,
                    kScratchBytes, hip_stream);
}

size_t msa_decode_noalloc_limit(void) { return kScratchBytes; }

}  // extern "C"

namespace {

int run_decode(const msa_dims* dims, const DecodePlan& p, const void* q, const void* k_cache, const void* v_cache,
               const void* idx_q, const void* idx_k_cache, const int32_t* cache_lens, void* out, float* lse,
               int32_t* block_idx, void* workspace, size_t workspace_bytes, void* hip_stream) {
  int st = MSA_OK;
  const bool dense = dims->flags & MSA_DENSE, given = dims->flags & MSA_GIVEN_INDICES;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || cache_lens == nullptr || out == nullptr)
    return MSA_ERR_INVALID_ARG;
  if (!dense && !given && (idx_q == nullptr || idx_k_cache == nullptr)) return MSA_ERR_INVALID_ARG;
  if (dense && block_idx != nullptr) return MSA_ERR_INVALID_ARG;
  if (given && block_idx == nullptr) return MSA_ERR_INVALID_ARG;
  if (misaligned(q, 16) || misaligned(k_cache, 16) || misaligned(v_cache, 16) || misaligned(out, 16) ||
      misaligned(idx_q, 16) || misaligned(idx_k_cache, 16) || misaligned(cache_lens, 4) ||
      misaligned(lse, 4) || misaligned(block_idx, 4))
    return MSA_ERR_ALIGNMENT;
  if ((st = check_workspace(p.total, workspace, workspace_bytes)) != MSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (dims->flags & MSA_CHECK_LENS) {
    // opt-in host check of the lengths: one small copy and a wait on the stream
    int32_t lens_h[256];
    for (int s0 = 0; s0 < dims->batch; s0 += 256) {
      const int n = dims->batch - s0 < 256 ? dims->batch - s0 : 256;
      hipError_t e = hipMemcpyAsync(lens_h, cache_lens + s0, (size_t)n * 4, hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      if (e != hipSuccess) return hip_fail(e);
      for (int i = 0; i < n; ++i)
        if (lens_h[i] < 1 || lens_h[i] > dims->seqlen) return MSA_ERR_INVALID_ARG;
    }
  }

  int32_t* bidx = block_idx;
  if (!dense && !given) {
    if (bidx == nullptr) bidx = at<int32_t>(workspace, p.off_bidx);
    float* S = at<float>(workspace, p.off_S);
    msa::prof_mark(s, MSA_STAGE_INDEX_DECODE);
    hipError_t e = msa::launch_index_blockmax_decode(
        static_cast<const uint16_t*>(idx_q), static_cast<const uint16_t*>(idx_k_cache), cache_lens, S,
        dims->batch, dims->seqlen, dims->num_kv_heads, dims->index_dim, dims->block_size, p.s_stride, s);
    if (e != hipSuccess) return hip_fail(e);
    msa::prof_mark(s, MSA_STAGE_TOPK_DECODE);
    e = msa::launch_topk_decode(S, p.s_stride, bidx, cache_lens, dims->seqlen, dims->batch,
                                dims->num_kv_heads, dims->block_size, dims->topk,
                                (dims->flags & MSA_FORCE_SINK) != 0, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  msa::DecodeMainArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.lens = cache_lens;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.bidx = bidx;
  a.batch = dims->batch;
  a.Lmax = dims->seqlen;
  a.Hq = dims->num_q_heads;
  a.G = dims->num_kv_heads;
  a.B = dims->block_size;
  a.topk = dims->topk;
  a.dense = dense;
  a.nsplit = p.nsplit;
  a.sub = p.sub;
  a.blocks_per_split = p.bps;
  a.scale_log2 = log2_scale(dims);
  a.pO = at<float>(workspace, p.off_pO);
  a.pS = at<float>(workspace, p.off_pS);
  hipError_t e = msa::launch_decode_main(a, s);
  msa::prof_mark(s, -1);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

}  // namespace
