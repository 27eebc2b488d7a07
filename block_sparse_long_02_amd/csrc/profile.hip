// Per-stage timing of libmsa's own launches (a measurement aid behind the
// msa_profile_* calls of include/msa.h).  While profiling is on, every stage
// boundary of a prefill or decode call records a HIP event on the caller's
// stream; a stage lasts from its mark to the next mark on the same stream.
// Nothing is recorded while profiling is off (one relaxed atomic load per
// stage boundary).
#include <atomic>
#include <mutex>
#include <vector>

#include "msa.h"
#include "msa_internal.h"

namespace msa {
namespace {

struct Mark {
  hipStream_t stream;
  int stage;  // MSA_STAGE_*, or -1 for the end of a call
  hipEvent_t ev;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Mark> g_marks;
bool g_failed = false;

void drop_marks() {
  for (Mark& m : g_marks) (void)hipEventDestroy(m.ev);
  g_marks.clear();
}

}  // namespace

void prof_mark(hipStream_t st, int stage) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  hipEvent_t ev;
  if (hipEventCreate(&ev) != hipSuccess) {
    std::lock_guard<std::mutex> lk(g_mu);
    g_failed = true;
    return;
  }
  if (hipEventRecord(ev, st) != hipSuccess) {
    (void)hipEventDestroy(ev);
    std::lock_guard<std::mutex> lk(g_mu);
    g_failed = true;
    return;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  g_marks.push_back({st, stage, ev});
}

}  // namespace msa

extern "C" {

int msa_profile_begin(void) {
  std::lock_guard<std::mutex> lk(msa::g_mu);
  msa::drop_marks();
  msa::g_failed = false;
  msa::g_on.store(true);
  return MSA_OK;
}

int msa_profile_end(msa_stage_time* out, int32_t max_stages, int32_t* n_stages) {
  std::lock_guard<std::mutex> lk(msa::g_mu);
  msa::g_on.store(false);
  if (out == nullptr || n_stages == nullptr || max_stages < MSA_STAGE_COUNT) {
    msa::drop_marks();
    return MSA_ERR_INVALID_ARG;
  }
  for (int i = 0; i < MSA_STAGE_COUNT; ++i) out[i] = msa_stage_time{i, 0, 0.0};
  *n_stages = MSA_STAGE_COUNT;
  int status = msa::g_failed ? MSA_ERR_HIP : MSA_OK;
  const size_t n = msa::g_marks.size();
  for (size_t i = 0; i < n && status == MSA_OK; ++i) {
    const msa::Mark& m = msa::g_marks[i];
    if (m.stage < 0) continue;
    size_t j = i + 1;  // next mark on the same stream closes this stage
    while (j < n && msa::g_marks[j].stream != m.stream) ++j;
    if (j == n) continue;
    float ms = 0.f;
    if (hipEventSynchronize(msa::g_marks[j].ev) != hipSuccess ||
        hipEventElapsedTime(&ms, m.ev, msa::g_marks[j].ev) != hipSuccess) {
      status = MSA_ERR_HIP;
      break;
    }
    out[m.stage].launches += 1;
    out[m.stage].total_ms += ms;
  }
  msa::drop_marks();
  return status;
}

const char* msa_stage_name(int32_t stage) {
  switch (stage) {
    case MSA_STAGE_INDEX_PREFILL: return "index_blockmax_prefill_kernel";
    case MSA_STAGE_TOPK_PREFILL: return "topk_prefill_kernel";
    case MSA_STAGE_BLOCK_LISTS: return "block lists (count, scan, scatter kernels)";
    case MSA_STAGE_KV_OUTER: return "kv_outer_kernel";
    case MSA_STAGE_QUERY_MAJOR: return "query_major_kernel<false>";
    case MSA_STAGE_QUERY_MAJOR_DENSE: return "dense_attn_kernel";
    case MSA_STAGE_INDEX_DECODE: return "decode_index_kernel";
    case MSA_STAGE_TOPK_DECODE: return "topk_decode_kernel";
    case MSA_STAGE_DECODE_ATTN: return "decode_attn_kernel";
    case MSA_STAGE_DECODE_COMBINE: return "decode_combine_kernel";
    case MSA_STAGE_INDEXER_KL: return "indexer KL (lists, stats, entry, list, reduction kernels)";
    case MSA_STAGE_BWD_PREP: return "backward prep (delta, block lists, list sort kernels)";
    case MSA_STAGE_BWD_LISTS: return "bwd_list_kernel";
    case MSA_STAGE_BWD_MERGE: return "backward merge (bwd_dq_kernel, bwd_dkv_kernel)";
    case MSA_STAGE_INDEX_ONE_PASS: return "index_topk_one_pass_kernel";
    default: return "unknown stage";
  }
}

}  // extern "C"
