// Top-k block selection with the forced local block, one wavefront per row.
//
// Definition [hyper.ai paper page 2606.13392, 方法 (Method) and 核心贡献
// (Contributions); Telegram review quant_prune_distill post 751, "Метод"]:
// per (query token, group) the blocks with the largest Block-Max scores are
// kept and the block holding the query is always kept.  Reading adopted for
// the unstated details: the local block L counts inside k, so m = min(k, L+1)
// blocks are kept -- L itself plus the m-1 best of the candidate blocks
// 0..L-1 under the order (score descending, block index ascending); the row
// is written in ascending block order and padded with -1.
//
// The selection is exp-free and exact (it compares the same fp32 maxima the
// index kernel produced, mapped to order-preserving uint32 keys):
//  1. each lane takes the max key over its strided share of the candidates;
//     the (m-1)-th largest of the 64 lane maxima is a lower bound lb of the
//     (m-1)-th largest key overall (valid while m-1 <= 64);
//  2. candidates with key >= lb are compacted, in ascending block order, into
//     a per-wave LDS list (ballot + prefix popcount);
//  3. the exact threshold tau = (m-1)-th largest key is found by a 32-step
//     bitwise search whose counts are wave ballots;
//  4. all keys > tau are kept, and of the keys == tau the lowest block
//     indices fill the remaining places; a second ballot/prefix pass writes
//     them out in ascending order, followed by L and the -1 padding.
// When more than kCap candidates survive (many exact ties, e.g. integer
// inputs), steps 3-4 run directly over all candidates in global memory.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kTopkWaves = 4;
constexpr int kCap = 512;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int popc(uint64_t x) { return __popcll(x); }

// kth (>= 1) largest key among at most one key per lane (0 = no key).
__device__ __forceinline__ uint32_t kth_largest_lanes(uint32_t key, int kth) {
  uint32_t tau = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = tau | (1u << bit);
    if (popc(__ballot(key >= c)) >= kth) tau = c;
  }
  return tau;
}

// Keys and block ids of the candidate list, either the compacted LDS list or
// the whole S row.
struct LdsList {
  const uint32_t* key;
  const int32_t* blk;
  __device__ uint32_t k(int i) const { return key[i]; }
  __device__ int32_t b(int i) const { return blk[i]; }
};
struct RowList {
  const float* row;
  __device__ uint32_t k(int i) const { return order_key(row[i]); }
  __device__ int32_t b(int i) const { return i; }
};

template <class List>
__device__ void select_and_write(const List& lst, int n, int mp, int L, int k, int32_t* out,
                                 int lane) {
  const uint64_t lt = lanemask_lt();
  uint32_t tau = 0;
  if (n <= kWave) {
    const uint32_t key = lane < n ? lst.k(lane) : 0u;
    tau = kth_largest_lanes(key, mp);
  } else {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = tau | (1u << bit);
      int cnt = 0;
      for (int i0 = 0; i0 < n; i0 += kWave) {
        const int i = i0 + lane;
        const uint32_t key = i < n ? lst.k(i) : 0u;
        cnt += popc(__ballot(key >= c));
      }
      if (cnt >= mp) tau = c;
    }
  }
  int cgt = 0;
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = i0 + lane;
    const uint32_t key = i < n ? lst.k(i) : 0u;
    cgt += popc(__ballot(key > tau));
  }
  const int need = mp - cgt;  // >= 1 by construction of tau
  int base = 0, eq_seen = 0;
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = i0 + lane;
    const bool in = i < n;
    const uint32_t key = in ? lst.k(i) : 0u;
    const bool eq = in && key == tau;
    const uint64_t beq = __ballot(eq);
    const int eq_rank = eq_seen + popc(beq & lt);
    const bool sel = in && (key > tau || (eq && eq_rank < need));
    const uint64_t bs = __ballot(sel);
    if (sel) out[base + popc(bs & lt)] = lst.b(i);
    base += popc(bs);
    eq_seen += popc(beq);
  }
  if (lane == 0) out[mp] = L;
  for (int j = mp + 1 + lane; j < k; j += kWave) out[j] = -1;
}

__device__ void select_row(const float* __restrict__ srow, int L, int k, int32_t* __restrict__ out,
                           uint32_t* skey, int32_t* sblk, int lane) {
  const int m = (k < L + 1) ? k : L + 1;
  const int mp = m - 1;
  if (mp == L) {  // every visible block is kept (covers L == 0)
    for (int j = lane; j < k; j += kWave) out[j] = (j <= L) ? j : -1;
    return;
  }
  if (mp == 0) {  // k == 1: the local block alone
    for (int j = lane; j < k; j += kWave) out[j] = (j == 0) ? L : -1;
    return;
  }
  // 1. lower bound from the lane maxima
  uint32_t lmax = 0;
  for (int j = lane; j < L; j += kWave) lmax = max(lmax, order_key(srow[j]));
  const uint32_t lb = (mp <= kWave) ? kth_largest_lanes(lmax, mp) : 0u;
  // 2. compact survivors in ascending block order
  const uint64_t lt = lanemask_lt();
  int n = 0;
  for (int j0 = 0; j0 < L; j0 += kWave) {
    const int j = j0 + lane;
    const uint32_t key = j < L ? order_key(srow[j]) : 0u;
    const bool sv = j < L && key >= lb;
    const uint64_t bal = __ballot(sv);
    const int pos = n + popc(bal & lt);
    if (sv && pos < kCap) {
      skey[pos] = key;
      sblk[pos] = j;
    }
    n += popc(bal);
  }
  wave_lds_sync();
  if (n <= kCap) {
    select_and_write(LdsList{skey, sblk}, n, mp, L, k, out, lane);
  } else {
    select_and_write(RowList{srow}, L, mp, L, k, out, lane);
  }
}

__global__ __launch_bounds__(256) void topk_prefill_kernel(const float* __restrict__ S, int s_stride,
                                                           int32_t* __restrict__ bidx, long bidx_rows,
                                                           int bidx_t_off, int G, int B, int k,
                                                           int t0, int tc, long n_rows) {
  __shared__ uint32_t skey[kTopkWaves][kCap];
  __shared__ int32_t sblk[kTopkWaves][kCap];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * kTopkWaves + wave;
  if (row >= n_rows) return;
  const long rows_chunk = (long)tc * G;
  const long s = row / rows_chunk;
  const long r = row % rows_chunk;
  const int t = t0 + (int)(r / G);
  const int g = (int)(r % G);
  const float* srow = S + (size_t)row * s_stride;
  int32_t* out = bidx + ((size_t)(s * bidx_rows + (t - bidx_t_off)) * G + g) * (size_t)k;
  select_row(srow, t / B, k, out, skey[wave], sblk[wave], lane);
}

__global__ __launch_bounds__(256) void topk_decode_kernel(const float* __restrict__ S, int s_stride,
                                                          int32_t* __restrict__ bidx,
                                                          const int32_t* __restrict__ lens, int Lmax,
                                                          int G, int B, int k, long n_rows) {
  __shared__ uint32_t skey[kTopkWaves][kCap];
  __shared__ int32_t sblk[kTopkWaves][kCap];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * kTopkWaves + wave;
  if (row >= n_rows) return;
  const long s = row / G;
  const int len = min(max(lens[s], 1), Lmax);
  const float* srow = S + (size_t)row * s_stride;
  int32_t* out = bidx + (size_t)row * k;
  select_row(srow, (len - 1) / B, k, out, skey[wave], sblk[wave], lane);
}

}  // namespace

hipError_t launch_topk_prefill(const float* S, int s_stride, int32_t* bidx, long bidx_rows,
                               int bidx_t_off, int batch, int G, int B, int k, int t0, int tc,
                               hipStream_t st) {
  const long n_rows = (long)batch * tc * G;
  const long grid = (n_rows + kTopkWaves - 1) / kTopkWaves;
  topk_prefill_kernel<<<dim3((unsigned)grid), 256, 0, st>>>(S, s_stride, bidx, bidx_rows, bidx_t_off,
                                                            G, B, k, t0, tc, n_rows);
  return hipGetLastError();
}

hipError_t launch_topk_decode(const float* S, int s_stride, int32_t* bidx, const int32_t* lens,
                              int Lmax, int batch, int G, int B, int k, hipStream_t st) {
  const long n_rows = (long)batch * G;
  const long grid = (n_rows + kTopkWaves - 1) / kTopkWaves;
  topk_decode_kernel<<<dim3((unsigned)grid), 256, 0, st>>>(S, s_stride, bidx, lens, Lmax, G, B, k,
                                                           n_rows);
  return hipGetLastError();
}

}  // namespace msa
