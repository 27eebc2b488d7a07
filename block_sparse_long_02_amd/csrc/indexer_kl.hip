// Indexer KL loss of MSA on gfx950: the loss that trains the Index Branch and
// its gradient into the index-branch inputs.
//
// Definition [Telegram review quant_prune_distill post 751, "Метод": a KL
// divergence between the index branch's outputs and the main branch's
// head-averaged outputs, stop-gradient through the main branch's
// probabilities and on the index inputs; hyper.ai paper page 2606.13392,
// 方法 (Method): the KL loss aligns the Index Branch's distribution with the
// Main Branch's on the selected tokens, with the index inputs detached].
// Per (token t, group g) row over the tokens J of its selected blocks (j <= t):
//   p_I(j) = softmax_j(idx_q[t,g] . idx_k[j])
//   p_M(j) = mean over the R heads h of g of exp(scale q[t,h].k[j,g] - lse[t,h])
//   KL     = sum_j p_M(j) (ln p_M(j) - ln p_I(j))
//   dS(j)  = p_I(j) - p_M(j)          (gradient of the summed KL w.r.t. the score)
//   d idx_q[t,g] = sum_j dS(j) idx_k[j],   d idx_k[j] += dS(j) idx_q[t,g]
// lse is the main branch's log-sum-exp over the same selection (the prefill's
// lse output), so exp(x - lse) is exactly the main branch's attention weight.
//
// Work split (block-major, the same (s, g, window, block) lists as the
// prefill's main branch, here including each row's local block):
//  1. kl_index_stats_kernel: per list entry, the max and sum of 2^(s log2 e)
//     over the block's keys <= t (MFMA, tiles of 128 entries);
//  2. kl_row_lse_kernel: per row, the index log-sum-exp (fixed slot order);
//  3. kl_entry_kernel: per entry, the R heads' logits (summed in the lane)
//     and the index logits on MFMA, p_M, p_I, the entry's KL term and dS
//     (bf16, row-major per entry);
//  4. kl_list_kernel: per list, d idx_q of each entry (dS . idx_k, stored in
//     bf16: 2^-8 relative, well inside what the row sums need) and the list's
//     d idx_k partial (dS^T . idx_q, fp32) on MFMA, over the entries in
//     (token, slot) order (the lists are sorted right after they are built);
//  5. kl_row_out_kernel / kl_dk_reduce_kernel: fixed-order sums per row and
//     per key block.  No atomic touches a value: results are reproducible.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int D = 128;  // head_dim

__device__ __forceinline__ size_t kl_list_of(const PrefillMainArgs& l, long lid, int* b, int* g, int* s) {
  *b = (int)(lid % l.nbl);
  const long sgw = lid / l.nbl;
  const long sg = sgw / l.nwin;
  *g = (int)(sg % l.G);
  *s = (int)(sg / l.G);
  return (size_t)lid;
}

// Rows [0, NR) of an NR x C bf16 block (row stride `stride` elements) into
// LDS with row stride ldsr; rows >= nvalid are zero-filled.  16 lanes per
// 256-byte row; every load is issued before the first store, so the staging
// costs one memory latency.
template <int C, int NR>
__device__ __forceinline__ void stage_rows(bf16_t* dst, int ldsr, const bf16_t* __restrict__ src, size_t stride,
                                           int nvalid, int tid) {
  constexpr int CPR = C / 8;
  constexpr int N = NR * CPR / 256;  // chunks per thread
  static_assert(N >= 1 && N * 256 == NR * CPR, "whole chunks per thread");
  u32x4 v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int c = tid + 256 * i, r = c / CPR, part = c % CPR;
    v[i] = *reinterpret_cast<const u32x4*>(src + (size_t)min(r, nvalid - 1) * stride + part * 8);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int c = tid + 256 * i, r = c / CPR, part = c % CPR;
    if (r >= nvalid) v[i] = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(dst + r * ldsr + part * 8) = v[i];
  }
}

// 4x4 transpose of 16-bit values: r[i] holds 4 values of row i; o[j] gets
// column j (rows 0..3).
__device__ __forceinline__ void transpose4x4(const u32x2 (&r)[4], u32x2 (&o)[4]) {
  o[0] = u32x2{(r[0][0] & 0xffffu) | (r[1][0] << 16), (r[2][0] & 0xffffu) | (r[3][0] << 16)};
  o[1] = u32x2{(r[0][0] >> 16) | (r[1][0] & 0xffff0000u), (r[2][0] >> 16) | (r[3][0] & 0xffff0000u)};
  o[2] = u32x2{(r[0][1] & 0xffffu) | (r[1][1] << 16), (r[2][1] & 0xffffu) | (r[3][1] << 16)};
  o[3] = u32x2{(r[0][1] >> 16) | (r[1][1] & 0xffff0000u), (r[2][1] >> 16) | (r[3][1] & 0xffff0000u)};
}

// S^T tile (32 keys x 32 rows) = A[32 keys x C] . Qop^T, A rows from LDS.
template <int C>
__device__ __forceinline__ f32x16 logit_tile(const bf16_t* As, int ldsr, int key0, const bf16x8* qop, int col,
                                             int half) {
  f32x16 acc = {};
  const bf16_t* arow = As + (key0 + col) * ldsr + 8 * half;
#pragma unroll
  for (int ks = 0; ks < C / 16; ++ks)
    acc = mfma32x32x16(*reinterpret_cast<const bf16x8*>(arow + 16 * ks), qop[ks], acc);
  return acc;
}

// ---------------------------------------------------------------------------
// 1. Index statistics per entry: (m, l) with m = max of s log2 e over the
//    block's keys <= t and l = sum of 2^(s log2 e - m).  Tiles of 128 entries
//    (4 waves x 32), one entry per MFMA column.
// ---------------------------------------------------------------------------
template <int DI, int BS>
__global__ __launch_bounds__(256, 2) void kl_index_stats_kernel(IndexerKlArgs a) {
  constexpr int KP = DI + 8;
  constexpr int KT = BS / 32;
  constexpr int MT = 128;
  __shared__ __attribute__((aligned(16))) bf16_t Is[BS * KP];
  const PrefillMainArgs& l = a.l;
  const int w = blockIdx.x;
  if (w >= a.n_work_a[0]) return;
  const int2 wk = a.work_a[w];
  int b, g, s;
  const size_t lid = kl_list_of(l, wk.x, &b, &g, &s);
  const int count = l.cnt[lid];
  const int off = l.offs[lid];
  const int tile0 = wk.y * kTilesPerItem;
  const int ntile = min(kTilesPerItem, (count + MT - 1) / MT - tile0);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int kb = b * l.B;
  stage_rows<DI, BS>(Is, KP, a.idx_k + ((size_t)s * l.T + kb) * DI, DI, min(BS, l.T - kb), tid);
  __syncthreads();
  for (int it = 0; it < ntile; ++it) {
    const int pos = (tile0 + it) * MT + wave * 32 + col;
    const bool valid = pos < count;
    const int ent = l.entries[off + min(pos, count - 1)];
    const int t = l.t0 + (ent >> l.rank_bits);
    bf16x8 qop[DI / 16];
    const bf16_t* qp = a.idx_q + (((size_t)s * l.T + t) * l.G + g) * DI;
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks) qop[ks] = load_bf16x8(qp + 16 * ks + 8 * half);
    // online max and sum over the key tiles; key kb <= t, so the first tile
    // of the row's lane pair always has a finite entry
    float m = -INFINITY, sum = 0.f;
#pragma unroll 1
    for (int kt = 0; kt < KT; ++kt) {
      const f32x16 acc = logit_tile<DI>(Is, KP, kt * 32, qop, col, half);
      float sv[16];
      float tm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = kb + kt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        sv[i] = (j <= t) ? acc[i] * kLog2e : -INFINITY;
        tm = fmaxf(tm, sv[i]);
      }
      tm = fmaxf(tm, __shfl_xor(tm, 32, kWave));
      const float mn = fmaxf(m, tm);
      float ts = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) ts += __builtin_amdgcn_exp2f(sv[i] - mn);
      ts += __shfl_xor(ts, 32, kWave);
      sum = (m == -INFINITY ? 0.f : sum * __builtin_amdgcn_exp2f(m - mn)) + ts;
      m = mn;
    }
    if (valid && half == 0) a.stat[off + pos] = make_float2(m, sum);
  }
}

// ---------------------------------------------------------------------------
// 2. Per row (s, t, g): log2-sum-exp of the index scores over its entries.
// ---------------------------------------------------------------------------
__global__ void kl_row_lse_kernel(IndexerKlArgs a) {
  const PrefillMainArgs& l = a.l;
  const long n_rows = (long)l.batch * l.tc * l.G;
  const long row = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= n_rows) return;
  const int nv = l.rinfo[row] & 0x3fffffff;
  const int32_t* pos = l.epos + (size_t)row * l.KS;
  // slots in groups of 8 whose position and statistics loads are issued together
  float M = -INFINITY;
  for (int q0 = 0; q0 < nv; q0 += 8) {
    float2 st[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) st[u] = a.stat[pos[min(q0 + u, nv - 1)]];
#pragma unroll
    for (int u = 0; u < 8; ++u) M = fmaxf(M, st[u].x);
  }
  float sum = 0.f;
  for (int q0 = 0; q0 < nv; q0 += 8) {
    float2 st[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) st[u] = a.stat[pos[min(q0 + u, nv - 1)]];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q0 + u < nv) sum += st[u].y * __builtin_amdgcn_exp2f(st[u].x - M);
  }
  a.lse_i[row] = nv > 0 ? M + __log2f(sum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// 3. Per entry: the main branch's and the index branch's distributions over
//    the block's keys, the entry's KL term and dS = p_I - p_M (bf16).  Tiles
//    of 128 entries (4 waves x 32, one entry per MFMA column); the R heads of
//    the group are visited in turn and their exp(x - lse) summed in the lane,
//    so p_M needs no cross-lane work and the index logits are computed once.
// ---------------------------------------------------------------------------
// Key tiles per pass over the R heads' q rows (each pass re-reads them) and
// workgroups per CU the entry kernel is compiled for.
#ifndef MSA_KL_ENTRY_KC
#define MSA_KL_ENTRY_KC 4
#endif
#ifndef MSA_KL_ENTRY_MINB
#define MSA_KL_ENTRY_MINB 2
#endif

template <int DI, int BS>
__global__ __launch_bounds__(256, MSA_KL_ENTRY_MINB) void kl_entry_kernel(IndexerKlArgs a) {
  constexpr int KROW = D + 8, KP = DI + 8;
  constexpr int KT = BS / 32;
  constexpr int KC = KT < MSA_KL_ENTRY_KC ? KT : MSA_KL_ENTRY_KC;
  constexpr int MT = 128;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[BS * KROW];
  __shared__ __attribute__((aligned(16))) bf16_t Is[BS * KP];
  const PrefillMainArgs& l = a.l;
  const int w = blockIdx.x;
  if (w >= a.n_work_a[0]) return;
  const int2 wk = a.work_a[w];
  int b, g, s;
  const size_t lid = kl_list_of(l, wk.x, &b, &g, &s);
  const int R = l.Hq / l.G;
  const int count = l.cnt[lid];
  const int off = l.offs[lid];
  const int tile0 = wk.y * kTilesPerItem;
  const int ntile = min(kTilesPerItem, (count + MT - 1) / MT - tile0);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int kb = b * l.B;
  const size_t kvstride = (size_t)l.G * D;
  const int nkey = min(BS, l.T - kb);
  stage_rows<D, BS>(Ks, KROW, l.k + ((size_t)s * l.T + kb) * kvstride + (size_t)g * D, kvstride, nkey, tid);
  stage_rows<DI, BS>(Is, KP, a.idx_k + ((size_t)s * l.T + kb) * DI, DI, nkey, tid);
  __syncthreads();
  const float c = l.scale_log2;
  const float invR = 1.0f / (float)R;

  for (int it = 0; it < ntile; ++it) {
    const int pos = (tile0 + it) * MT + wave * 32 + col;
    const bool valid = pos < count;
    const int ent = l.entries[off + min(pos, count - 1)];
    const int tl = ent >> l.rank_bits;
    const int t = l.t0 + tl;
    const size_t qrow = ((size_t)s * l.T + t) * l.Hq + (size_t)g * R;  // first head of the group
    const bf16_t* ip = a.idx_q + (((size_t)s * l.T + t) * l.G + g) * DI;
    const float lse2_i = a.lse_i[((size_t)s * l.tc + tl) * l.G + g];
    bf16_t* dsrow = a.ds + (size_t)(off + min(pos, count - 1)) * BS;
    float kl = 0.f;
    // chunks of KC key tiles: the q rows are read once per chunk (all of the
    // block's tiles by default)
#pragma unroll 1
    for (int k0 = 0; k0 < KT; k0 += KC) {
      float pm[KC][16];  // sum over the heads of exp(x - lse): R * p_M
#pragma unroll
      for (int kt = 0; kt < KC; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) pm[kt][i] = 0.f;
      // The heads' logit tiles in sequence (head, key tile): the products of
      // the next step (this head's next key tile, or the next head's first)
      // are issued before the exps of the current one, so the matrix unit has
      // work while the vector unit sums exp(x - lse).  Head r's q rows sit in
      // one register set while head r + 1's are fetched into the other; the
      // loop is unrolled by two so that no set is copied.  After the last head
      // the next step is computed and unused.
      bf16x8 qa[D / 16], qb[D / 16];
      auto load_q = [&](bf16x8* dst, int r) {
        const size_t row = qrow + (size_t)min(r, R - 1);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) dst[ks] = load_bf16x8(l.q + row * D + 16 * ks + 8 * half);
      };
      load_q(qa, 0);
      float lse_a = a.lse[qrow], lse_b = 0.f;
      f32x16 xcur = logit_tile<D>(Ks, KROW, k0 * 32, qa, col, half);
      auto head = [&](const bf16x8* qo, bf16x8* qn, int rn, float lse, float& lse_n) {
        load_q(qn, rn);
        lse_n = a.lse[qrow + min(rn, R - 1)];
        // The key operands are read from LDS in every head through an offset
        // the compiler cannot see through: held in registers across the heads
        // (its choice otherwise) they would take 128 registers per lane and
        // leave room for only one wave per SIMD.
        int koff = 0;
        asm volatile("" : "+v"(koff));
        const bf16_t* Kh = Ks + koff;
        const float lse2 = lse * kLog2e;
#pragma unroll
        for (int kt = 0; kt < KC; ++kt) {
          const f32x16 xnxt = kt + 1 < KC ? logit_tile<D>(Kh, KROW, (k0 + kt + 1) * 32, qo, col, half)
                                          : logit_tile<D>(Kh, KROW, k0 * 32, qn, col, half);
#pragma unroll
          for (int i = 0; i < 16; ++i) pm[kt][i] += __builtin_amdgcn_exp2f(xcur[i] * c - lse2);
          xcur = xnxt;
        }
      };
#pragma unroll 1
      for (int r = 0; r < R; r += 2) {
        head(qa, qb, r + 1, lse_a, lse_b);
        if (r + 1 >= R) break;
        head(qb, qa, r + 2, lse_b, lse_a);
      }
      // the index query, read only now so that it holds no registers in the
      // head loop
      bf16x8 iop[DI / 16];
#pragma unroll
      for (int ks = 0; ks < DI / 16; ++ks) iop[ks] = load_bf16x8(ip + 16 * ks + 8 * half);
#pragma unroll
      for (int kt = 0; kt < KC; ++kt) {
        const f32x16 si = logit_tile<DI>(Is, KP, (k0 + kt) * 32, iop, col, half);
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = kb + (k0 + kt) * 32 + 8 * (i / 4) + 4 * half + (i % 4);
          const bool ok = j <= t;
          const float p_m = ok ? pm[kt][i] * invR : 0.f;
          const float l2pi = si[i] * kLog2e - lse2_i;
          const float p_i = ok ? __builtin_amdgcn_exp2f(l2pi) : 0.f;
          // branch-free: p_m = 0 adds nothing (the log is taken of at least
          // the smallest normal, so it stays finite)
          kl += p_m * (__log2f(fmaxf(p_m, 1.17549435e-38f)) - l2pi);
          ds[i] = p_i - p_m;
        }
        if (valid) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            bf16x4 v;
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = (__bf16)ds[4 * i4 + u];
            *reinterpret_cast<bf16x4*>(dsrow + (k0 + kt) * 32 + 8 * i4 + 4 * half) = v;
          }
        }
      }
    }
    kl += __shfl_xor(kl, 32, kWave);
    if (valid && half == 0) a.kl_e[off + pos] = kl * kLn2;
  }
}

// ---------------------------------------------------------------------------
// 4. Per list: d idx_q of every entry (dS . idx_k of the block) and the
//    list's d idx_k partial (dS^T . idx_q over its entries), both on MFMA,
//    over chunks of 32 entries.
// ---------------------------------------------------------------------------
// Element offset of 16-byte chunk c of row r in an unpadded tile of rows of
// NC chunks: the chunk sits at c ^ s(r), with s chosen so that 16 consecutive
// rows read one chunk each (row-per-lane operand reads) and 4 consecutive
// rows read 64 bytes each (transposing reads, 32 lanes) both fall on 16
// distinct 16-byte positions of a 256-byte bank window.
template <int NC>
__device__ __forceinline__ int kl_swz(int r, int c) {
  int sw;
  if constexpr (NC >= 16) sw = 4 * (r & 3) + ((r >> 2) & 3);
  else if constexpr (NC == 8) sw = 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  else sw = (r >> 2) & 3;
  return r * (NC * 8) + ((c ^ sw) * 8);
}

template <int DI, int BS>
__global__ __launch_bounds__(256) void kl_list_kernel(IndexerKlArgs a) {
  constexpr int EC = 32;                  // entries per chunk
  constexpr int KC = BS / 8, QC = DI / 8;  // 16-byte chunks per key row / per index row
  constexpr int NT = (BS / 32) * (DI / 32);  // d idx_k output tiles of the list
  constexpr int TPW = (NT + 3) / 4;          // tiles per wave
  __shared__ __attribute__((aligned(16))) bf16_t IkT[DI * BS];  // [c][key]
  __shared__ __attribute__((aligned(16))) bf16_t Dr[EC * BS];   // [entry][key]
  __shared__ __attribute__((aligned(16))) bf16_t Qr[EC * DI];   // [entry][c]
  const PrefillMainArgs& l = a.l;
  const long lid = blockIdx.x;
  const int count = l.cnt[lid];
  if (count == 0) return;
  int b, g, s;
  kl_list_of(l, lid, &b, &g, &s);
  const int off = l.offs[lid];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int kb = b * l.B;
  const int nkey = min(BS, l.T - kb);

  // idx_k block, transposed through registers in 4 keys x 4 c units:
  // IkT[c][key], read row-per-lane by the d idx_q product.
  for (int u = tid; u < (BS / 4) * (DI / 4); u += 256) {
    const int k4 = u / (DI / 4), c4 = u % (DI / 4);
    u32x2 r[4], o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 4 * k4 + i;
      r[i] = key < nkey ? *reinterpret_cast<const u32x2*>(a.idx_k + ((size_t)s * l.T + kb + key) * DI + 4 * c4)
                        : u32x2{0u, 0u};
    }
    transpose4x4(r, o);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x2*>(IkT + kl_swz<KC>(4 * c4 + j, k4 >> 1) + 4 * (k4 & 1)) = o[j];
  }
  f32x16 dk[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) dk[i] = f32x16{};

  // Each thread stages one 4 entries x 4 keys unit of the chunk's dS rows and
  // one 4 entries x 4 dims unit of its idx_q rows, both row-major: the d idx_q
  // product reads dS rows per lane, the d idx_k product reads dS and idx_q
  // with entries as the contraction index through the transposing LDS read.
  // The next chunk's units are fetched into registers while the current chunk
  // computes, and the entries that address its idx_q rows one chunk earlier.
  constexpr int NUD = (EC / 4) * (BS / 4), NUQ = (EC / 4) * (DI / 4);
  static_assert(NUD <= 256 && NUQ <= 256, "one unit per thread");
  const bool has_d = tid < NUD, has_q = tid < NUQ;
  const int de4 = tid / (BS / 4), dk4 = tid % (BS / 4);
  const int qe4 = tid / (DI / 4), qc4 = tid % (DI / 4);
  u32x2 dsr[4], qsr[4];
  int ent4[4];
  auto load_ent = [&](int c0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int en = c0 + 4 * qe4 + i;
      ent4[i] = has_q && en < count ? l.entries[off + en] : -1;
    }
  };
  auto load_data = [&](int c0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int en = c0 + 4 * de4 + i;
      dsr[i] = has_d && en < count ? *reinterpret_cast<const u32x2*>(a.ds + (size_t)(off + en) * BS + 4 * dk4)
                                   : u32x2{0u, 0u};
      const int e = ent4[i];
      qsr[i] = e >= 0 ? *reinterpret_cast<const u32x2*>(
                            a.idx_q + (((size_t)s * l.T + l.t0 + (e >> l.rank_bits)) * l.G + g) * DI + 4 * qc4)
                      : u32x2{0u, 0u};
    }
  };
  auto store = [&]() {
    if (has_d) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x2*>(Dr + kl_swz<KC>(4 * de4 + i, dk4 >> 1) + 4 * (dk4 & 1)) = dsr[i];
    }
    if (has_q) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x2*>(Qr + kl_swz<QC>(4 * qe4 + i, qc4 >> 1) + 4 * (qc4 & 1)) = qsr[i];
    }
  };
  // Transposing read (ds_read_b64_tr_b16) of a row-major swizzled tile: in
  // each 16-lane group, lane 4a + c addresses the 8-byte word of row
  // r0 + c of the group's 4 rows at column 4a, so that lane l receives rows
  // r0 .. r0 + 3 at column c0 + l % 32, with r0 = rb + 4 (l / 32).
  const int tr_row = 4 * half + ((lane >> 2) & 3);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto tr_d = [&](int rb, int c0) { return kl_swz<KC>(rb + tr_row, (c0 + tr_col) >> 3) + (tr_col & 7); };
  auto tr_q = [&](int rb, int c0) { return kl_swz<QC>(rb + tr_row, (c0 + tr_col) >> 3) + (tr_col & 7); };

  load_ent(0);
  load_data(0);
  load_ent(EC);
  for (int c0 = 0; c0 < count; c0 += EC) {
    const int n = min(EC, count - c0);
    __syncthreads();  // the previous chunk's LDS reads are done (and IkT is written)
    store();
    __syncthreads();
    if (c0 + EC < count) {
      load_data(c0 + EC);
      load_ent(c0 + 2 * EC);
    }
    // d idx_q of the chunk's entries: [entry][c] = sum_key dS[entry][key] idx_k[key][c]
    if (wave < DI / 32) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < BS / 16; ++ks) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(Dr + kl_swz<KC>(col, 2 * ks + half));
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(IkT + kl_swz<KC>(32 * wave + col, 2 * ks + half));
        acc = mfma32x32x16(av, bv, acc);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int en = 8 * (i / 4) + 4 * half + (i % 4);
        if (en < n) a.dq_e[(size_t)(off + c0 + en) * DI + 32 * wave + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[i]);
      }
    }
    // d idx_k partial: [key][c] += sum_entry dS[entry][key] idx_q[entry][c].
    // Both operands come from the transposing read, rows (entries) 16 ks + 4 h
    // .. + 3 and 8 further for lane half h, the same k-slot order on both sides.
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tix = wave + 4 * i;
      if (tix < NT) {
        const int kt = tix / (DI / 32), dt = tix % (DI / 32);
#pragma unroll
        for (int ks = 0; ks < EC / 16; ++ks) {
          const bf16x8 av = join_bf16x4(lds_read_tr16(Dr + tr_d(16 * ks, 32 * kt)),
                                        lds_read_tr16(Dr + tr_d(16 * ks + 8, 32 * kt)));
          const bf16x8 bv = join_bf16x4(lds_read_tr16(Qr + tr_q(16 * ks, 32 * dt)),
                                        lds_read_tr16(Qr + tr_q(16 * ks + 8, 32 * dt)));
          dk[i] = mfma32x32x16(av, bv, dk[i]);
        }
      }
    }
  }
  float* part = a.dk_part + (size_t)lid * BS * DI;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tix = wave + 4 * i;
    if (tix < NT) {
      const int kt = tix / (DI / 32), dt = tix % (DI / 32);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = 32 * kt + 8 * (v / 4) + 4 * half + (v % 4);
        part[(size_t)key * DI + 32 * dt + col] = dk[i][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 5a. Per row and 4 index dimensions: KL and d idx_q, summed in slot order.
// ---------------------------------------------------------------------------
__global__ void kl_row_out_kernel(IndexerKlArgs a) {
  const PrefillMainArgs& l = a.l;
  const int dq4 = a.di / 4;
  const long n = (long)l.batch * l.tc * l.G * dq4;
  const long x = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= n) return;
  const long row = x / dq4;
  const int c4 = (int)(x % dq4);
  const long per_b = (long)l.tc * l.G;
  const int s = (int)(row / per_b);
  const int tl = (int)((row % per_b) / l.G);
  const int g = (int)(row % l.G);
  const size_t orow = ((size_t)s * l.T + l.t0 + tl) * l.G + g;
  const int nv = l.rinfo[row] & 0x3fffffff;
  const int32_t* pos = l.epos + (size_t)row * l.KS;
  f32x4 dq = {0.f, 0.f, 0.f, 0.f};
  float kl = 0.f;
  // slots in groups of 8 whose position and term loads are issued together
  for (int q0 = 0; q0 < nv; q0 += 8) {
    int pq[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) pq[u] = pos[min(q0 + u, nv - 1)];
    bf16x4 v[8];
    float ke[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v[u] = *reinterpret_cast<const bf16x4*>(a.dq_e + (size_t)pq[u] * a.di + 4 * c4);
      ke[u] = a.kl_e[pq[u]];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q0 + u < nv) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dq[e] += (float)v[u][e];
        kl += ke[u];
      }
  }
  *reinterpret_cast<f32x4*>(a.d_idx_q + orow * a.di + 4 * c4) = dq;
  if (c4 == 0) a.kl[orow] = kl;
}

// ---------------------------------------------------------------------------
// 5b. Per key block: d idx_k = sum over the block's lists (group, window) of
//     their partials, in that order; added onto earlier query chunks.  The
//     block's elements are split over kDkSplit workgroups; the lists' counts
//     are read 256 at a time in parallel and walked in order by every thread.
// ---------------------------------------------------------------------------
constexpr int kDkSplit = 4;

template <int DI, int BS>
__global__ __launch_bounds__(256) void kl_dk_reduce_kernel(IndexerKlArgs a) {
  constexpr int PER = BS * DI / 256 / kDkSplit;  // elements per thread
  __shared__ int live[256];
  const PrefillMainArgs& l = a.l;
  const int b = blockIdx.x, s = blockIdx.y, z = blockIdx.z;
  const int kb = b * l.B;
  const int nkey = min(BS, l.T - kb);
  const int nall = l.G * l.nwin;  // lists of this key block, in (group, window) order
  const int u0 = z * (BS * DI / kDkSplit);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int base = 0; base < nall; base += 256) {
    __syncthreads();
    {
      const int x = base + (int)threadIdx.x;
      const size_t lid = (((size_t)s * l.G + x / l.nwin) * l.nwin + x % l.nwin) * l.nbl + b;
      live[threadIdx.x] = x < nall && l.cnt[lid] > 0;
    }
    __syncthreads();
    const int n = min(256, nall - base);
    for (int i = 0; i < n; ++i) {
      if (!live[i]) continue;
      const int x = base + i;
      const size_t lid = (((size_t)s * l.G + x / l.nwin) * l.nwin + x % l.nwin) * l.nbl + b;
      const float* part = a.dk_part + lid * BS * DI + u0;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += part[threadIdx.x + 256 * e];
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int u = u0 + threadIdx.x + 256 * e;
    if (u < nkey * DI) {
      float* dst = a.d_idx_k + ((size_t)s * l.T + kb) * DI + u;
      *dst = a.accumulate_dk ? *dst + acc[e] : acc[e];
    }
  }
}

}  // namespace

hipError_t launch_indexer_kl(const IndexerKlArgs& a, hipStream_t st) {
  const PrefillMainArgs& l = a.l;
  const int R = l.Hq / l.G;
  const int mt = kAttnRows / R;
  hipError_t err = launch_block_lists(l, mt, st);
  if (err != hipSuccess) return err;
  // entries in (token, slot) order within each list before any per-entry
  // value is written: the d idx_k sums then run in a fixed order
  if ((err = launch_sort_lists(l, st)) != hipSuccess) return err;
  if ((err = launch_list_work(l, 128, a.work_a, a.n_work_a, st)) != hipSuccess) return err;
  const long n_rows = (long)l.batch * l.tc * l.G;
#define MSA_KL_DISPATCH(KERNEL, GRID, ...)                                                        \
  do {                                                                                            \
    if (a.di == 128) {                                                                            \
      if (l.B == 128) KERNEL<128, 128><<<GRID, 256, 0, st>>>(__VA_ARGS__);                        \
      else if (l.B == 64) KERNEL<128, 64><<<GRID, 256, 0, st>>>(__VA_ARGS__);                     \
      else KERNEL<128, 32><<<GRID, 256, 0, st>>>(__VA_ARGS__);                                    \
    } else {                                                                                      \
      if (l.B == 128) KERNEL<64, 128><<<GRID, 256, 0, st>>>(__VA_ARGS__);                         \
      else if (l.B == 64) KERNEL<64, 64><<<GRID, 256, 0, st>>>(__VA_ARGS__);                      \
      else KERNEL<64, 32><<<GRID, 256, 0, st>>>(__VA_ARGS__);                                     \
    }                                                                                             \
  } while (0)
  if (a.max_work_a > 0) MSA_KL_DISPATCH(kl_index_stats_kernel, dim3((unsigned)a.max_work_a), a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  kl_row_lse_kernel<<<(unsigned)((n_rows + 255) / 256), 256, 0, st>>>(a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.max_work_a > 0) MSA_KL_DISPATCH(kl_entry_kernel, dim3((unsigned)a.max_work_a), a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  MSA_KL_DISPATCH(kl_list_kernel, dim3((unsigned)l.nlists), a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const long nout = n_rows * (a.di / 4);
  kl_row_out_kernel<<<(unsigned)((nout + 255) / 256), 256, 0, st>>>(a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int nb = (l.T + l.B - 1) / l.B;
  MSA_KL_DISPATCH(kl_dk_reduce_kernel, dim3((unsigned)nb, (unsigned)l.batch, (unsigned)kDkSplit), a);
#undef MSA_KL_DISPATCH
  return hipGetLastError();
}

}  // namespace msa
