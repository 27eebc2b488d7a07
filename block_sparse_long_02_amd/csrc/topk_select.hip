// Top-k block selection with the forced local block, one wavefront per row.
//
// Definition [hyper.ai paper page 2606.13392, 方法 (Method) and 核心贡献
// (Contributions); Telegram review quant_prune_distill post 751, "Метод"]:
// per (query token, group) the blocks with the largest Block-Max scores are
// kept and the block holding the query is always kept.  Reading adopted for
// the unstated details: the local block L counts inside k, so m = min(k, L+1)
// blocks are kept -- L itself plus the m-1 best of the candidate blocks
// 0..L-1 under the order (score descending, block index ascending); the row
// is written in ascending block order and padded with -1.  With the sink
// variant (the pages' experiments compare hard-coded selection of the
// sequence start and the local window), block 0 is forced as well whenever
// the row keeps two or more blocks, and the remaining picks come from blocks
// 1..L-1.
//
// The selection is exp-free and exact (it compares the same fp32 maxima the
// index kernel produced, mapped to order-preserving uint32 keys):
//  1. each lane takes the max key over its strided share of the candidates;
//     any lb that m-1 lane maxima reach is a lower bound of the (m-1)-th
//     largest key overall (valid while m-1 <= 64); lb is taken on the keys'
//     top 16 bits only, a 16-step search;
//  2. candidates with key >= lb are compacted, in ascending block order, into
//     a per-wave LDS list (ballot + prefix popcount);
//  3. the exact threshold tau = (m-1)-th largest key is found by a 32-step
//     bitwise search whose counts are wave ballots;
//  4. all keys > tau are kept, and of the keys == tau the lowest block
//     indices fill the remaining places; a second ballot/prefix pass writes
//     them out in ascending order, followed by L and the -1 padding.
// When more than kCap candidates survive (many exact ties, e.g. integer
// inputs), steps 3-4 run directly over all candidates in global memory.
//
// Prefill rows also come with superblock maxima (the largest score of every
// run of 16 candidate blocks).  The want-th largest superblock maximum lb is
// a lower bound of the want-th largest candidate score: want superblocks
// each hold a candidate scoring >= lb.  So every block that can be selected,
// ties at the threshold included, lies in a superblock whose maximum is
// >= lb, and step 2 reads only those superblocks (at 1M tokens a row has up
// to 512 superblocks, of which a few dozen pass).
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

// A lower bound of the kth (>= 1) largest key among at most one key per lane
// (0 = no key): the largest multiple of 2^16 that kth keys reach, found on
// the top 16 bits only (sign, exponent and 7 mantissa bits of the scores).
__device__ __forceinline__ uint32_t kth_largest_lanes_hi16(uint32_t key, int kth) {
  uint32_t tau = 0;
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t c = tau | (1u << bit);
    if (popc(__ballot(key >= c)) >= kth) tau = c;
  }
  return tau;
}

// kth (>= 1) largest key among at most one key per lane (0 = no key).
__device__ __forceinline__ uint32_t kth_largest_lanes(uint32_t key, int kth) {
  uint32_t tau = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = tau | (1u << bit);
    if (popc(__ballot(key >= c)) >= kth) tau = c;
  }
  return tau;
}

// Keys and block ids of a candidate list in ascending block order: a
// compacted LDS list, or a contiguous range [b0, b0 + n) of an S row.
struct LdsList {
  const uint32_t* key;
  const int32_t* blk;
  __device__ uint32_t k(int i) const { return key[i]; }
  __device__ int32_t b(int i) const { return blk[i]; }
};
struct RowList {
  const float* row;  // row + b0
  int b0;
  __device__ uint32_t k(int i) const { return order_key(row[i]); }
  __device__ int32_t b(int i) const { return b0 + i; }
};

// Candidates per lane held in registers by the one-read paths of
// select_best and compact_candidates (lists of up to 64 * kRegKeys).
constexpr int kRegKeys = 16;

// Selects the `want` (1 <= want <= n) best entries of lst[0, n) under
// (key descending, block ascending) and hands them to emit(pos, key, blk) in
// list order, pos = 0 .. want-1.  Wave-uniform control flow.  Lists of up to
// 64 * kRegKeys entries are read once into registers; the 32-step threshold
// search then needs only ballots.
template <int NR = kRegKeys, class List, class Emit>
__device__ __forceinline__ void select_best(const List& lst, int n, int want, int lane, Emit emit) {
  const uint64_t lt = lanemask_lt();
  if (n <= kWave * NR) {
    uint32_t key[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = i * kWave + lane;
      key[i] = j < n ? lst.k(j) : 0u;
    }
    const int nch = (n + kWave - 1) / kWave;
    uint32_t tau = 0;
    if (n <= kWave) {
      tau = kth_largest_lanes(key[0], want);
    } else {
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = tau | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < NR; ++i)
          if (i < nch) cnt += popc(__ballot(key[i] >= c));
        if (cnt >= want) tau = c;
      }
    }
    int cgt = 0;
#pragma unroll
    for (int i = 0; i < NR; ++i)
      if (i < nch) cgt += popc(__ballot(key[i] > tau));
    const int need = want - cgt;  // >= 1 by construction of tau
    int base = 0, eq_seen = 0;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (i < nch) {  // wave-uniform
        const int j = i * kWave + lane;
        const bool in = j < n;
        const bool eq = in && key[i] == tau;
        const uint64_t beq = __ballot(eq);
        const int eq_rank = eq_seen + popc(beq & lt);
        const bool sel = in && (key[i] > tau || (eq && eq_rank < need));
        const uint64_t bs = __ballot(sel);
        if (sel) emit(base + popc(bs & lt), key[i], lst.b(j));
        base += popc(bs);
        eq_seen += popc(beq);
      }
    }
    return;
  }
  uint32_t tau = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = tau | (1u << bit);
    int cnt = 0;
    for (int i0 = 0; i0 < n; i0 += kWave) {
      const int i = i0 + lane;
      const uint32_t key = i < n ? lst.k(i) : 0u;
      cnt += popc(__ballot(key >= c));
    }
    if (cnt >= want) tau = c;
  }
  int cgt = 0;
  for (int i0 = 0; i0 < n; i0 += kWave) {
    const int i = i0 + lane;
    const uint32_t key = i < n ? lst.k(i) : 0u;
    cgt += popc(__ballot(key > tau));
  }
  const int need = want - cgt;  // >= 1 by construction of tau
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
    if (sel) emit(base + popc(bs & lt), key, lst.b(i));
    base += popc(bs);
    eq_seen += popc(beq);
  }
}

// Compacts the candidates of srow[b0, b0 + n) whose key may be among the
// `want` best (key >= the want-th largest lane maximum, when want <= 64) into
// skey/sblk in block order; returns the number of survivors (entries beyond
// kCap are counted but not stored).  Rows of up to 64 * kRegKeys candidates
// are read once, all loads in flight together, and compacted from registers.
template <int NR = kRegKeys>
__device__ __forceinline__ int compact_candidates(const float* __restrict__ srow, int b0, int n, int want, uint32_t* skey,
                                  int32_t* sblk, int lane) {
  const uint64_t lt = lanemask_lt();
  int cnt = 0;
  if (n <= kWave * NR) {
    uint32_t key[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int j = i * kWave + lane;
      key[i] = j < n ? order_key(srow[b0 + j]) : 0u;
    }
    uint32_t lmax = 0;
#pragma unroll
    for (int i = 0; i < NR; ++i) lmax = max(lmax, key[i]);
    const uint32_t lb = (want <= kWave) ? kth_largest_lanes_hi16(lmax, want) : 0u;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (i * kWave < n) {  // wave-uniform
        const int j = i * kWave + lane;
        const bool sv = j < n && key[i] >= lb;
        const uint64_t bal = __ballot(sv);
        const int pos = cnt + popc(bal & lt);
        if (sv && pos < kCap) {
          skey[pos] = key[i];
          sblk[pos] = b0 + j;
        }
        cnt += popc(bal);
      }
    }
  } else {
    uint32_t lmax = 0;
    for (int j = lane; j < n; j += kWave) lmax = max(lmax, order_key(srow[b0 + j]));
    const uint32_t lb = (want <= kWave) ? kth_largest_lanes_hi16(lmax, want) : 0u;
    for (int j0 = 0; j0 < n; j0 += kWave) {
      const int j = j0 + lane;
      const uint32_t key = j < n ? order_key(srow[b0 + j]) : 0u;
      const bool sv = j < n && key >= lb;
      const uint64_t bal = __ballot(sv);
      const int pos = cnt + popc(bal & lt);
      if (sv && pos < kCap) {
        skey[pos] = key;
        sblk[pos] = b0 + j;
      }
      cnt += popc(bal);
    }
  }
  wave_lds_sync();
  return cnt;
}

// Superblock-pruned form of compact_candidates for the candidates c0..L-1:
// sm[i] is the largest candidate score in blocks [16 i, 16 i + 16).  With
// c0 = 1 (block 0 forced), superblock 0 also covers block 0, so it is left
// out of the bound and always read.  Survivors (keys >= lb) are compacted in
// ascending block order; the passing superblock ids go through slist (LDS,
// kCap entries).  Returns the survivor count (entries beyond kCap are counted
// but not stored), or -1 when the row has too few or too many superblocks
// for this path.
static_assert(kSuperBlock == 16, "the superblock gather maps 4 superblocks of 16 blocks onto a wave");
static_assert(kSbMinCandidates == kWave * kRegKeys, "superblock rows start where the register path ends");
template <int kSbRegs>  // superblock maxima per lane held in registers (rows of up to 64 * kSbRegs superblocks)
__device__ __forceinline__ int compact_candidates_sb(const float* __restrict__ srow, const float* __restrict__ sm,
                                                     int c0, int L, int want, uint32_t* skey, int32_t* sblk,
                                                     int32_t* slist, int lane) {
  const int nsb = (L + kSuperBlock - 1) / kSuperBlock;
  const int s_lo = c0 > 0 ? 1 : 0;
  // rows that compact_candidates reads once into registers are cheaper there
  if (L - c0 <= kSbMinCandidates || nsb - s_lo <= want || nsb > kWave * kSbRegs) return -1;  // wave-uniform
  const uint64_t lt = lanemask_lt();
  uint32_t key[kSbRegs];
#pragma unroll
  for (int i = 0; i < kSbRegs; ++i) {
    const int j = i * kWave + lane;
    key[i] = (j >= s_lo && j < nsb) ? order_key(sm[j]) : 0u;
  }
  const int nch = (nsb + kWave - 1) / kWave;
  // lb: the largest multiple of 2^16 that want bound keys reach (a lower
  // bound of the want-th largest, found on the top 16 bits; counts by ballots)
  uint32_t lb = 0;
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t c = lb | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kSbRegs; ++i)
      if (i < nch) cnt += popc(__ballot(key[i] >= c));
    if (cnt >= want) lb = c;
  }
  // passing superblocks, ascending
  int P = 0;
#pragma unroll
  for (int i = 0; i < kSbRegs; ++i) {
    if (i < nch) {  // wave-uniform
      const int j = i * kWave + lane;
      const bool pass = j < nsb && (j < s_lo || key[i] >= lb);
      const uint64_t bal = __ballot(pass);
      if (pass) slist[P + popc(bal & lt)] = j;
      P += popc(bal);
    }
  }
  wave_lds_sync();
  // gather the passing superblocks, 4 per step (16 lanes each), 4 steps of
  // loads in flight before their compaction
  const int sub = lane >> 4, off = lane & (kSuperBlock - 1);
  int cnt = 0;
  for (int i0 = 0; i0 < P; i0 += 16) {
    uint32_t kk[4];
    int bl[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int si = i0 + 4 * u + sub;
      bl[u] = -1;
      kk[u] = 0u;
      if (si < P) {
        const int b = slist[si] * kSuperBlock + off;
        if (b >= c0 && b < L) {
          bl[u] = b;
          kk[u] = order_key(srow[b]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool sv = bl[u] >= 0 && kk[u] >= lb;
      const uint64_t bal = __ballot(sv);
      const int pos = cnt + popc(bal & lt);
      if (sv && pos < kCap) {
        skey[pos] = kk[u];
        sblk[pos] = bl[u];
      }
      cnt += popc(bal);
    }
  }
  wave_lds_sync();
  return cnt;
}

__device__ __forceinline__ void write_trivial(int L, int mp, int k, int32_t* out, int lane) {
  if (mp == L) {  // every visible block is kept (covers L == 0)
    for (int j = lane; j < k; j += kWave) out[j] = (j <= L) ? j : -1;
  } else {        // k == 1: the local block alone
    for (int j = lane; j < k; j += kWave) out[j] = (j == 0) ? L : -1;
  }
}

// Forced blocks of a row: the local block L always; with `sink`, block 0 too
// whenever the row keeps at least two blocks.  The free picks are the `want`
// best of the candidates c0..L-1 (c0 = 1 when block 0 is forced).
struct RowPlan {
  int m;      // blocks kept: min(k, L+1)
  bool fs;    // block 0 forced
  int c0;     // first free candidate
  int want;   // free picks among c0..L-1
};
__device__ __forceinline__ RowPlan row_plan(int L, int k, bool sink) {
  RowPlan r;
  r.m = (k < L + 1) ? k : L + 1;
  r.fs = sink && L >= 1 && r.m >= 2;
  r.c0 = r.fs ? 1 : 0;
  r.want = r.m - 1 - (r.fs ? 1 : 0);
  return r;
}

__device__ __forceinline__ void select_row(const float* __restrict__ srow, int L, int k, bool sink,
                                           int32_t* __restrict__ out, uint32_t* skey, int32_t* sblk, int lane,
                                           const float* __restrict__ smrow = nullptr, int32_t* slist = nullptr) {
  const RowPlan rp = row_plan(L, k, sink);
  const int mp = rp.m - 1;
  if (mp == L || mp == 0) {  // every visible block, or the local block alone
    write_trivial(L, mp, k, out, lane);
    return;
  }
  if (rp.want > 0) {
    const int off = rp.fs ? 1 : 0;
    int n = -1;
    if (smrow != nullptr) {  // register arrays sized to the row's superblocks
      const int nsb = (L + kSuperBlock - 1) / kSuperBlock;
      n = nsb <= kWave * 2 ? compact_candidates_sb<2>(srow, smrow, rp.c0, L, rp.want, skey, sblk, slist, lane)
        : nsb <= kWave * 4 ? compact_candidates_sb<4>(srow, smrow, rp.c0, L, rp.want, skey, sblk, slist, lane)
                           : compact_candidates_sb<kCap / kWave>(srow, smrow, rp.c0, L, rp.want, skey, sblk, slist, lane);
    }
    if (n < 0) {
      const int nc = L - rp.c0;
      n = nc <= kWave * 2   ? compact_candidates<2>(srow, rp.c0, nc, rp.want, skey, sblk, lane)
        : nc <= kWave * 4   ? compact_candidates<4>(srow, rp.c0, nc, rp.want, skey, sblk, lane)
        : nc <= kWave * 8   ? compact_candidates<8>(srow, rp.c0, nc, rp.want, skey, sblk, lane)
        : nc <= kWave * 12  ? compact_candidates<12>(srow, rp.c0, nc, rp.want, skey, sblk, lane)
                            : compact_candidates(srow, rp.c0, nc, rp.want, skey, sblk, lane);
    }
    auto emit = [&](int pos, uint32_t, int32_t blk) { out[off + pos] = blk; };
    if (n <= kWave) select_best<1>(LdsList{skey, sblk}, n, rp.want, lane, emit);
    else if (n <= kCap) select_best(LdsList{skey, sblk}, n, rp.want, lane, emit);
    else select_best(RowList{srow + rp.c0, rp.c0}, L - rp.c0, rp.want, lane, emit);
  }
  if (lane == 0) {
    if (rp.fs) out[0] = 0;
    out[mp] = L;
  }
  for (int j = mp + 1 + lane; j < k; j += kWave) out[j] = -1;
}

// SB: the chunk has rows long enough for the superblock path (SM given);
// without it the kernel carries neither that path nor its LDS list.
template <bool SB>
__global__ __launch_bounds__(256) void topk_prefill_kernel(const float* __restrict__ S, int s_stride,
                                                           const float* __restrict__ SM, int sm_stride,
                                                           int32_t* __restrict__ bidx, long bidx_rows,
                                                           int bidx_t_off, int G, int B, int k, bool sink,
                                                           int t0, int tc, long n_rows) {
  __shared__ uint32_t skey[kTopkWaves][kCap];
  __shared__ int32_t sblk[kTopkWaves][kCap];
  __shared__ int32_t slist[SB ? kTopkWaves : 1][SB ? kCap : 1];
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
  if constexpr (SB) {
    select_row(srow, t / B, k, sink, out, skey[wave], sblk[wave], lane, SM + (size_t)row * sm_stride, slist[wave]);
  } else {
    select_row(srow, t / B, k, sink, out, skey[wave], sblk[wave], lane);
  }
}

// Decode rows are few (batch x G) and long (up to Lmax / B candidates): one
// 16-wave workgroup per row.  Each wave keeps the best min(m-1, n_w) blocks
// of its contiguous partition; the union of those lists, in block order,
// contains the row's best m-1 (a total order), and wave 0 selects them.
constexpr int kDecWaves = 16;
constexpr int kDecMaxKeep = kWave;  // two-level path for m-1 <= 64

__global__ __launch_bounds__(1024) void topk_decode_kernel(const float* __restrict__ S, int s_stride,
                                                           int32_t* __restrict__ bidx,
                                                           const int32_t* __restrict__ lens, int Lmax,
                                                           int G, int B, int k, bool sink) {
  __shared__ uint32_t skey[kDecWaves][kCap];
  __shared__ int32_t sblk[kDecWaves][kCap];
  __shared__ uint32_t mkey[kDecWaves * kDecMaxKeep];
  __shared__ int32_t mblk[kDecWaves * kDecMaxKeep];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long row = blockIdx.x;
  const long s = row / G;
  const int len = min(max(lens[s], 1), Lmax);
  const int L = (len - 1) / B;
  const float* srow = S + (size_t)row * s_stride;
  int32_t* out = bidx + (size_t)row * k;
  const RowPlan rp = row_plan(L, k, sink);
  const int mp = rp.m - 1;
  const int ncand = L - rp.c0;
  if (mp == L || mp == 0 || rp.want == 0 || rp.want > kDecMaxKeep || ncand <= kWave * kDecWaves) {
    // uniform across the workgroup: one wave does the whole row
    if (wave == 0) select_row(srow, L, k, sink, out, skey[0], sblk[0], lane);
    return;
  }
  // level 1: per-wave partitions of the candidates c0..L-1.  Wave w keeps
  // min(want, its candidates) and writes them, in block order, straight into
  // the combined list at the sum of the earlier waves' counts (known without
  // communication), so the combined list is in block order too.
  const int per = (ncand + kDecWaves - 1) / kDecWaves;
  auto kept_of = [&](int w) { return min(rp.want, max(0, min(per, L - (rp.c0 + w * per)))); };
  int off_w = 0, total = 0;
  for (int w = 0; w < kDecWaves; ++w) {  // uniform scalar arithmetic
    if (w == wave) off_w = total;
    total += kept_of(w);
  }
  const int b0 = rp.c0 + wave * per;
  const int nw = max(0, min(per, L - b0));
  if (nw > 0) {
    const int want = min(rp.want, nw);
    const int n = nw <= kWave * 8 ? compact_candidates<8>(srow, b0, nw, want, skey[wave], sblk[wave], lane)
                                  : compact_candidates(srow, b0, nw, want, skey[wave], sblk[wave], lane);
    auto emit = [&](int pos, uint32_t key, int32_t blk) {
      mkey[off_w + pos] = key;
      mblk[off_w + pos] = blk;
    };
    if (n <= kWave) select_best<1>(LdsList{skey[wave], sblk[wave]}, n, want, lane, emit);
    else if (n <= kCap) select_best(LdsList{skey[wave], sblk[wave]}, n, want, lane, emit);
    else select_best(RowList{srow + b0, b0}, nw, want, lane, emit);
  }
  __syncthreads();
  // level 2: wave 0 selects among the combined list
  if (wave == 0) {
    const int off = rp.fs ? 1 : 0;
    auto emit = [&](int pos, uint32_t, int32_t blk) { out[off + pos] = blk; };
    if (total <= kWave * 4) select_best<4>(LdsList{mkey, mblk}, total, rp.want, lane, emit);
    else select_best(LdsList{mkey, mblk}, total, rp.want, lane, emit);
    if (lane == 0) {
      if (rp.fs) out[0] = 0;
      out[mp] = L;
    }
    for (int j = mp + 1 + lane; j < k; j += kWave) out[j] = -1;
  }
}

}  // namespace

hipError_t launch_topk_prefill(const float* S, int s_stride, const float* SM, int sm_stride,
                               int32_t* bidx, long bidx_rows,
                               int bidx_t_off, int batch, int G, int B, int k, bool sink, int t0, int tc,
                               hipStream_t st) {
  const long n_rows = (long)batch * tc * G;
  const long grid = (n_rows + kTopkWaves - 1) / kTopkWaves;
  if (SM != nullptr)
    topk_prefill_kernel<true><<<dim3((unsigned)grid), 256, 0, st>>>(S, s_stride, SM, sm_stride, bidx, bidx_rows,
                                                                    bidx_t_off, G, B, k, sink, t0, tc, n_rows);
  else
    topk_prefill_kernel<false><<<dim3((unsigned)grid), 256, 0, st>>>(S, s_stride, SM, sm_stride, bidx, bidx_rows,
                                                                     bidx_t_off, G, B, k, sink, t0, tc, n_rows);
  return hipGetLastError();
}

hipError_t launch_topk_decode(const float* S, int s_stride, int32_t* bidx, const int32_t* lens,
                              int Lmax, int batch, int G, int B, int k, bool sink, hipStream_t st) {
  const long n_rows = (long)batch * G;
  topk_decode_kernel<<<dim3((unsigned)n_rows), 1024, 0, st>>>(S, s_stride, bidx, lens, Lmax, G, B, k, sink);
  return hipGetLastError();
}

}  // namespace msa
