// Main Branch of MSA on gfx950: exact softmax GQA attention restricted to the
// selected blocks [hyper.ai paper page 2606.13392, 方法 (Method): attention is
// limited to the tokens of the selected blocks, computed as standard scaled
// dot-product attention over their gathered keys and values; hamidun.com news
// "MiniMax выпустила MSA", "Как устроен MSA": the main branch is exact].
//
// Work split (an MI355X design choice, in the spirit of the pages' KV-outer
// kernel, 核心贡献 / Contributions):
//  * non-local selected blocks (b < L(t)) are processed block-major: for every
//    (sequence, group, block) a list of the (token, slot) pairs that chose it
//    is built by a counting sort; a workgroup loads one K/V block into LDS
//    once and serves up to 128 (token, head) query rows of that list with
//    MFMA, writing a normalised partial output and its log-sum-exp per row.
//    K/V bytes are thereby shared across query tokens as well as across the R
//    heads of a group; no causal mask is needed since b < L(t) lies wholly
//    before t.
//  * the local block L(t) is processed query-major (flash attention over the
//    keys [L(t)*B, t] with the causal mask), and the same kernel then merges
//    the row's partials in fixed slot order -- no atomics touch any value, so
//    outputs are bitwise reproducible.
//  * dense mode (every visible block) runs the query-major kernel over keys
//    [0, t] with online softmax.
//
// Numerics: bf16 x bf16 products, fp32 accumulation, softmax in fp32 in the
// base-2 domain (logit * scale * log2 e), probabilities rounded to bf16 for
// the P.V product, output rounded to bf16 (nearest even).
#include <type_traits>

#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int D = 128;          // head_dim
constexpr int KROW = D + 8;     // LDS row stride of K tiles (bf16)

// ---------------------------------------------------------------------------
// LDS staging helpers (256 threads) for tiles of NK keys.
// K tile: rows [key][D] -> Ks[key*KROW + d]
// V tile: transposed -> Vt[d*VROW + key], so that a lane can fetch 4
// consecutive keys of one d with one 8-byte read (PV operand layout).
// Keys >= nvalid (>= 1) are zero-filled.  Every load of a tile is issued
// before its first LDS write, so a tile costs one memory latency.
// ---------------------------------------------------------------------------
template <int NK>
__device__ __forceinline__ void stage_k(bf16_t* Ks, const bf16_t* __restrict__ kbase, size_t kstride, int nvalid,
                                        int tid) {
  constexpr int N = NK * (D / 8) / 256;  // 16-byte chunks per thread
  static_assert(N * 256 == NK * (D / 8), "whole chunks per thread");
  u32x4 v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int c = tid + 256 * i;
    v[i] = *reinterpret_cast<const u32x4*>(kbase + (size_t)min(c >> 4, nvalid - 1) * kstride + (c & 15) * 8);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int c = tid + 256 * i;
    if ((c >> 4) >= nvalid) v[i] = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(Ks + (c >> 4) * KROW + (c & 15) * 8) = v[i];
  }
}

// A 4-key x 4-d unit u of the V^T staging: the low 5 bits pick 8 d-quads x 4
// key-quads, so the 32 lanes of a half-wave write 32 distinct bank pairs of
// V^T rows whose stride is 2 (mod 64) dwords (conflict-free ds_write_b64),
// while each 8-lane group still reads 64 contiguous bytes of a V row.
__device__ __forceinline__ void vt_unit(int u, int& k4, int& dq) {
  dq = ((u >> 5) & 3) * 8 + (u & 7);
  k4 = (u >> 7) * 4 + ((u >> 3) & 3);
}

// The all-blocks kernel's V^T tiles: each 16-key group of a row holds its
// 4-key quads in the order 0, 2, 1, 3, so the 8 keys a lane feeds to a 16-key
// PV slice ({4h..4h+3} and {8+4h..8+4h+3} for half h) sit in 16 contiguous
// bytes (one 16-byte read); rows are 8 keys longer than the tile (272-byte
// rows at 128 keys: 16 lanes reading 16 bytes at one column touch 64
// distinct banks).
constexpr int kVtPadQ = 8;
__device__ __forceinline__ int vt_quad_pos(int k4) { return (k4 & ~3) | ((k4 & 1) << 1) | ((k4 >> 1) & 1); }

// Its staging units (4 keys x 4 d each, 8-byte V^T row writes): the LDS
// takes 8-byte writes 16 lanes at a time over 32 banks (128 bytes), so each
// 16-lane group holds two adjacent d-quads (V^T rows 4 apart: 64 bytes apart
// mod 128 at the 272-byte row stride) x 8 key-quads (8 bytes apart): 16
// distinct bank pairs.  The 64 lanes of a load instruction cover 8 d-quads x
// 8 key-quads: 8 V rows, 64 contiguous bytes each.
__device__ __forceinline__ void vt_unit_q(int u, int& k4, int& dq) {
  dq = (u & 1) + 2 * ((u >> 4) & 3) + 8 * ((u >> 6) & 3);
  k4 = ((u >> 1) & 7) + 8 * (u >> 8);
}

// 4x4 transpose of 16-bit lanes: o[j] = (r0[j], r1[j], r2[j], r3[j])
__device__ __forceinline__ void transpose_4x4(const u32x2 (&r)[4], u32x2 (&o)[4]) {
  o[0] = u32x2{(r[0][0] & 0xffffu) | (r[1][0] << 16), (r[2][0] & 0xffffu) | (r[3][0] << 16)};
  o[1] = u32x2{(r[0][0] >> 16) | (r[1][0] & 0xffff0000u), (r[2][0] >> 16) | (r[3][0] & 0xffff0000u)};
  o[2] = u32x2{(r[0][1] & 0xffffu) | (r[1][1] << 16), (r[2][1] & 0xffffu) | (r[3][1] << 16)};
  o[3] = u32x2{(r[0][1] >> 16) | (r[1][1] & 0xffff0000u), (r[2][1] >> 16) | (r[3][1] & 0xffff0000u)};
}

template <int NK>
__device__ __forceinline__ void stage_vt(bf16_t* Vt, int vrow, const bf16_t* __restrict__ vbase, size_t vstride,
                                         int nvalid, int tid) {
  constexpr int N = (NK / 4) * (D / 4) / 256;  // units of 4 keys x 4 d per thread
  static_assert(N * 256 == (NK / 4) * (D / 4), "whole units per thread");
  u32x2 r[N][4];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    int k4, dq;
    vt_unit(tid + 256 * n, k4, dq);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[n][i] = *reinterpret_cast<const u32x2*>(vbase + (size_t)min(k4 * 4 + i, nvalid - 1) * vstride + dq * 4);
  }
#pragma unroll
  for (int n = 0; n < N; ++n) {
    int k4, dq;
    vt_unit(tid + 256 * n, k4, dq);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (k4 * 4 + i >= nvalid) r[n][i] = u32x2{0u, 0u};
    u32x2 o[4];
    transpose_4x4(r[n], o);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(Vt + (dq * 4 + j) * vrow + k4 * 4) = o[j];
  }
}

// Whole-block K/V staging through registers with compile-time trip counts:
// every global load of the block is issued before the first LDS write.
template <int BS, int NTH = 256>
struct BlockRegs {
  u32x4 k[BS * 16 / NTH];     // 16-byte chunks of K rows: chunk c = tid + NTH i
  u32x2 v[BS * 8 / NTH][4];   // 4 keys x 4 d units of V: unit u = tid + NTH i
};

template <int BS, int NTH = 256>
__device__ __forceinline__ void block_load(BlockRegs<BS, NTH>& r, const bf16_t* __restrict__ kbase,
                                           const bf16_t* __restrict__ vbase, size_t stride, int tid) {
#pragma unroll
  for (int i = 0; i < BS * 16 / NTH; ++i) {
    const int c = tid + NTH * i;
    r.k[i] = *reinterpret_cast<const u32x4*>(kbase + (size_t)(c >> 4) * stride + (c & 15) * 8);
  }
#pragma unroll
  for (int i = 0; i < BS * 8 / NTH; ++i) {
    const int u = tid + NTH * i;
    int k4, dq;
    vt_unit(u, k4, dq);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r.v[i][j] = *reinterpret_cast<const u32x2*>(vbase + (size_t)(k4 * 4 + j) * stride + dq * 4);
  }
}

// QUADS: the all-blocks kernel's V^T layout (vt_unit_q, vt_quad_pos).
template <int BS, int NTH = 256, bool QUADS = false>
__device__ __forceinline__ void block_store(const BlockRegs<BS, NTH>& r, bf16_t* Ks, bf16_t* Vt, int vrow, int tid) {
#pragma unroll
  for (int i = 0; i < BS * 16 / NTH; ++i) {
    const int c = tid + NTH * i;
    *reinterpret_cast<u32x4*>(Ks + (c >> 4) * KROW + (c & 15) * 8) = r.k[i];
  }
#pragma unroll
  for (int i = 0; i < BS * 8 / NTH; ++i) {
    const int u = tid + NTH * i;
    int k4, dq;
    if (QUADS) vt_unit_q(u, k4, dq);
    else vt_unit(u, k4, dq);
    u32x2 o[4];
    transpose_4x4(r.v[i], o);
    const int kpos = QUADS ? vt_quad_pos(k4) : k4;
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(Vt + (dq * 4 + j) * vrow + kpos * 4) = o[j];
  }
}

// S^T tiles of KT consecutive 32-key tiles at once: acc[kt] = K[32 kt ..][D] . Q^T.
// The KT A operands of a k-step are read from LDS together and the next
// k-step's are read before the current k-step's products, so one LDS
// latency is paid per tile set instead of one per product.  Every
// accumulator still sums its k-steps in order 0..D/16-1 (the same products
// in the same order as one tile at a time).
template <int KT>
__device__ __forceinline__ void qk_tiles(const bf16_t* Ks, const bf16x8* qop, f32x16 (&acc)[KT], int col, int half) {
  constexpr int KS = D / 16;
  const bf16_t* arow = Ks + col * KROW + 8 * half;
  bf16x8 a[2][KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) a[0][kt] = *reinterpret_cast<const bf16x8*>(arow + kt * 32 * KROW);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < KS) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        a[cur ^ 1][kt] = *reinterpret_cast<const bf16x8*>(arow + kt * 32 * KROW + 16 * (ks + 1));
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) acc[kt] = mfma32x32x16(a[cur][kt], qop[ks], ks == 0 ? f32x16{} : acc[kt]);
  }
}

// O^T[4 d-tiles] += V^T . P^T over the 2 KT 16-key slices of KT key tiles;
// the four d-tiles' A operands of a slice are read together and the next
// slice's before the current slice's products.  Each d-tile accumulates its
// slices in key order (as one pv_step after another would).
template <int KT, bool QUADS = false>
__device__ __forceinline__ void pv_tiles(const bf16_t* Vt, int vrow, const bf16x8 (*p)[2], f32x16 (&o)[4], int col,
                                         int half) {
  constexpr int NS = 2 * KT;
  const bf16_t* vr = Vt + col * vrow + (QUADS ? 8 : 4) * half;
  bf16x8 a[2][4];
  auto load = [&](int sl, bf16x8 (&dst)[4]) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const bf16_t* r = vr + dt * 32 * vrow + 16 * sl;
      dst[dt] = QUADS ? *reinterpret_cast<const bf16x8*>(r)
                      : join_bf16x4(*reinterpret_cast<const u32x2*>(r), *reinterpret_cast<const u32x2*>(r + 8));
    }
  };
  load(0, a[0]);
#pragma unroll
  for (int sl = 0; sl < NS; ++sl) {
    const int cur = sl & 1;
    if (sl + 1 < NS) load(sl + 1, a[cur ^ 1]);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32x32x16(a[cur][dt], p[sl >> 1][sl & 1], o[dt]);
  }
}

__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& a, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)a[base + e];
  return r;
}

__device__ __forceinline__ void load_q(bf16x8* qop, const bf16_t* qp, bool ok, int half) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qop[ks] = ok ? load_bf16x8(qp + 16 * ks + 8 * half) : zero_bf16x8();
}

// ---------------------------------------------------------------------------
// Block lists: counting sort of the (token, slot) pairs by
// (s, g, window, block).  Entry of a row = tl << rank_bits | rank, rank = position
// among the row's valid non-local entries (so partial storage needs only
// KS = min(k, nb) slots per row).
// ---------------------------------------------------------------------------
__global__ void fill_i32_kernel(int32_t* p, size_t n, int32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__device__ __forceinline__ size_t list_id(const PrefillMainArgs& a, int s, int g, int tl, int b) {
  const int w = tl / a.window;
  return (((size_t)s * a.G + g) * a.nwin + w) * a.nbl + b;
}

// Selection entries are read kSelChunk at a time so that their loads are all
// in flight together.
constexpr int kSelChunk = 8;

__device__ __forceinline__ void load_sel_chunk(int (&ev)[kSelChunk], const int32_t* __restrict__ br, int j0,
                                               int topk) {
#pragma unroll
  for (int u = 0; u < kSelChunk; ++u) ev[u] = (j0 + u < topk) ? br[j0 + u] : -1;
}

// Counts the entries of every block list and records per row the number of
// partial slots (valid non-local entries, at most KS) and whether the row
// attends its local block (a given selection may omit it).
//
// Popular blocks gather thousands of entries per list, so one global atomic
// per entry would serialise on a few addresses.  A workgroup of up to
// kCountRows rows therefore aggregates in LDS first: each entry's list id is
// hashed into an LDS table whose counter hands out the entry's local rank;
// then one global atomicAdd per distinct list reserves the workgroup's range,
// and each entry's slot is that base plus its local rank.  Entries whose id
// finds no free LDS slot take a global atomic directly.  epos holds, between
// the phases, (table slot << 16 | local rank), or the direct slot | bit 31.
constexpr int kCountRows = 128;
constexpr int kHashBits = 12;
constexpr int kHashSlots = 1 << kHashBits;
constexpr uint32_t kHashEmpty = 0xffffffffu;
constexpr uint32_t kDirect = 0x80000000u;

// At most kCountRows rows per workgroup, fewer when rows carry many slots, so
// that the hash table stays at most half full (rows_wg * KS <= kHashSlots / 2);
// a probe gives up after kMaxProbe slots and takes the direct path.
constexpr int kMaxProbe = 64;

__host__ __device__ inline int count_rows_per_wg(int KS) {
  const int r = kHashSlots / (2 * (KS > 0 ? KS : 1));
  return r < 1 ? 1 : (r > kCountRows ? kCountRows : r);
}

__global__ __launch_bounds__(kCountRows) void lists_count_kernel(PrefillMainArgs a, int rows_wg) {
  __shared__ uint32_t hkey[kHashSlots];
  __shared__ int32_t hval[kHashSlots];  // local counts, then the reserved global bases
  const int tid = threadIdx.x;
  for (int i = tid; i < kHashSlots; i += kCountRows) {
    hkey[i] = kHashEmpty;
    hval[i] = 0;
  }
  __syncthreads();

  const long n_rows = (long)a.batch * a.tc * a.G;
  const long row = (long)blockIdx.x * rows_wg + tid;
  // local ranks fit 16 bits while a workgroup holds fewer than 2^16 entries
  const bool use_lds = (long)rows_wg * a.KS < 65536;
  int rank = 0;
  if (tid < rows_wg && row < n_rows) {
    const long per_b = (long)a.tc * a.G;
    const int s = (int)(row / per_b);
    const int tl = (int)((row % per_b) / a.G);
    const int g = (int)(row % a.G);
    const int t = a.t0 + tl;
    const int L = t / a.B;
    const int32_t* br = a.bidx + ((size_t)((long)s * a.bidx_rows + (t - a.bidx_t_off)) * a.G + g) * a.topk;
    bool has_local = false;
    for (int j0 = 0; j0 < a.topk; j0 += kSelChunk) {
      int ev[kSelChunk];
      load_sel_chunk(ev, br, j0, a.topk);
#pragma unroll
      for (int u = 0; u < kSelChunk; ++u) {
        const int e = ev[u];
        has_local |= (e == L);
        if (e >= 0 && (e < L || (a.include_local && e == L)) && rank < a.KS) {
          const size_t lid = list_id(a, s, g, tl, e);
          uint32_t code = kDirect;
          if (use_lds) {
            const uint32_t key = (uint32_t)lid;
            uint32_t slot = (key * 2654435761u) >> (32 - kHashBits);
            for (int p = 0; p < kMaxProbe; ++p) {
              const uint32_t prev = atomicCAS(&hkey[slot], kHashEmpty, key);
              if (prev == kHashEmpty || prev == key) {
                code = (slot << 16) | (uint32_t)atomicAdd(&hval[slot], 1);
                break;
              }
              slot = (slot + 1) & (kHashSlots - 1);
            }
          }
          if (code == kDirect) code = kDirect | (uint32_t)atomicAdd(&a.cnt[lid], 1);
          a.epos[(size_t)row * a.KS + rank] = (int32_t)code;
          ++rank;
        }
      }
    }
    a.rinfo[row] = rank | (has_local ? (1 << 30) : 0);
  }
  __syncthreads();
  for (int i = tid; i < kHashSlots; i += kCountRows)
    if (hkey[i] != kHashEmpty) hval[i] = atomicAdd(&a.cnt[hkey[i]], hval[i]);
  __syncthreads();
  for (int q = 0; q < rank; ++q) {
    int32_t* ep = a.epos + (size_t)row * a.KS + q;
    const uint32_t code = (uint32_t)*ep;
    *ep = (code & kDirect) ? (int32_t)(code & ~kDirect) : hval[code >> 16] + (int32_t)(code & 0xffffu);
  }
}

// Exclusive scan of (x, y) pairs across a 1024-thread workgroup; returns the
// thread's exclusive prefix and writes the workgroup totals.
__device__ __forceinline__ int2 block_exclusive_scan(int2 v, int2* total) {
  __shared__ int2 wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int2 x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int yx = __shfl_up(x.x, o, kWave), yy = __shfl_up(x.y, o, kWave);
    if (lane >= o) { x.x += yx; x.y += yy; }
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int2 w = lane < 16 ? wsum[lane] : make_int2(0, 0);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int yx = __shfl_up(w.x, o, kWave), yy = __shfl_up(w.y, o, kWave);
      if (lane >= o) { w.x += yx; w.y += yy; }
    }
    if (lane < 16) wsum[lane] = w;
  }
  __syncthreads();
  const int2 base = wave > 0 ? wsum[wave - 1] : make_int2(0, 0);
  *total = wsum[15];
  __syncthreads();
  return make_int2(base.x + x.x - v.x, base.y + x.y - v.y);
}

// Work items of a list of c entries: groups of up to kTilesPerItem tiles of
// mt tokens.
__device__ __forceinline__ int list_items(int c, int mt) {
  const int tiles = (c + mt - 1) / mt;
  return (tiles + kTilesPerItem - 1) / kTilesPerItem;
}

// Phase 1: per scan block (kScanItems lists) totals of entries and work items.
__global__ __launch_bounds__(1024) void lists_scan_reduce_kernel(const int32_t* __restrict__ cnt,
                                                                 int32_t* __restrict__ bsum, long nlists,
                                                                 int mt) {
  const long i0 = (long)blockIdx.x * kScanItems + threadIdx.x * 4;
  int2 v = make_int2(0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long i = i0 + j;
    const int c = i < nlists ? cnt[i] : 0;
    v.x += c;
    v.y += list_items(c, mt);
  }
  int2 tot;
  block_exclusive_scan(v, &tot);
  if (threadIdx.x == 0) {
    bsum[2 * blockIdx.x] = tot.x;
    bsum[2 * blockIdx.x + 1] = tot.y;
  }
}

// Phase 2 (one workgroup): exclusive scan of the block totals, in place;
// n_work = number of work items.
__global__ __launch_bounds__(1024) void lists_scan_top_kernel(int32_t* __restrict__ bsum, int nblk,
                                                              int32_t* __restrict__ n_work) {
  int2 carry = make_int2(0, 0);
  for (int base = 0; base < nblk; base += 1024) {
    const int i = base + threadIdx.x;
    const int2 v = i < nblk ? make_int2(bsum[2 * i], bsum[2 * i + 1]) : make_int2(0, 0);
    int2 tot;
    const int2 ex = block_exclusive_scan(v, &tot);
    if (i < nblk) {
      bsum[2 * i] = carry.x + ex.x;
      bsum[2 * i + 1] = carry.y + ex.y;
    }
    carry.x += tot.x;
    carry.y += tot.y;
  }
  if (threadIdx.x == 0) n_work[0] = carry.y;
}

// Phase 3: list offsets and the flat work list (list id, tile group).
__global__ __launch_bounds__(1024) void lists_scan_final_kernel(const int32_t* __restrict__ cnt,
                                                                const int32_t* __restrict__ bsum,
                                                                int32_t* __restrict__ offs,
                                                                int2* __restrict__ work, long nlists, int mt) {
  const long i0 = (long)blockIdx.x * kScanItems + threadIdx.x * 4;
  int c[4];
  int2 v = make_int2(0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long i = i0 + j;
    c[j] = i < nlists ? cnt[i] : 0;
    v.x += c[j];
    v.y += list_items(c[j], mt);
  }
  int2 tot;
  const int2 ex = block_exclusive_scan(v, &tot);
  int e_off = bsum[2 * blockIdx.x] + ex.x;
  int t_off = bsum[2 * blockIdx.x + 1] + ex.y;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long i = i0 + j;
    if (i < nlists) {
      offs[i] = e_off;
      const int items = list_items(c[j], mt);
      for (int tj = 0; tj < items; ++tj) work[t_off + tj] = make_int2((int)i, tj);
      e_off += c[j];
      t_off += items;
    }
  }
}

__global__ void lists_scatter_kernel(PrefillMainArgs a) {
  const long n_rows = (long)a.batch * a.tc * a.G;
  const long row = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= n_rows) return;
  const long per_b = (long)a.tc * a.G;
  const int s = (int)(row / per_b);
  const int tl = (int)((row % per_b) / a.G);
  const int g = (int)(row % a.G);
  const int t = a.t0 + tl;
  const int L = t / a.B;
  const int32_t* br = a.bidx + ((size_t)((long)s * a.bidx_rows + (t - a.bidx_t_off)) * a.G + g) * a.topk;
  const int nv = a.rinfo[row] & 0x3fffffff;
  int rank = 0;
  for (int j0 = 0; j0 < a.topk && rank < nv; j0 += kSelChunk) {
    int ev[kSelChunk];
    load_sel_chunk(ev, br, j0, a.topk);
#pragma unroll
    for (int u = 0; u < kSelChunk; ++u) {
      const int e = ev[u];
      if (e >= 0 && (e < L || (a.include_local && e == L)) && rank < a.KS) {
        const size_t lid = list_id(a, s, g, tl, e);
        const size_t slot = (size_t)row * a.KS + rank;
        const int pos = a.offs[lid] + a.epos[slot];
        a.entries[pos] = (tl << a.rank_bits) | rank;
        a.epos[slot] = pos;  // from here on: the entry's position in the list order
        ++rank;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp16 partial rows, stored in list order: the R rows of the list entry at
// position p are rows p*R .. p*R+R-1.  Rows are grouped in blocks of 32
// consecutive rows (8 KiB); inside a block, chunk c (0..7, 16 bytes: values
// 8*h8 .. 8*h8+7 of d-tile dt, c = 2 dt + h8) of lane half h of the block's
// row j sits at byte 1024 c + 512 h + 16 j.  Value i (= 8*h8 + j') of d-tile
// dt of half h has d = 32*dt + 8*(i/4) + 4*h + (i%4) (the MFMA output layout).
// So the 64 lanes of a wave holding 32 consecutive rows store (and a merge
// lane group of one entry's R rows reads) whole 512-byte runs per
// instruction, where a row-major layout would touch 32 scattered 32-byte
// pieces.
// The row is the unnormalised sum O = sum_j p_j v_j over one block's keys
// (p_j <= 1 after subtracting the row maximum), scaled by 2^-e with e chosen
// per K/V block from max|V|: |O| <= BS * max|V| * 2^-e < 2^15, so the fp16
// store cannot overflow for any finite input.  e = 0 whenever max|V| lies in
// [2^-6, 2^8), where values too small for fp16 normals are below 2^-8 max|V|
// and their absolute error is negligible.
// ---------------------------------------------------------------------------
constexpr int kPartBlockRows = 32;
constexpr int kPartBlockBytes = kPartBlockRows * D * 2;   // 8 KiB

// Byte offset of chunk 0 of half `half` of global partial row `row`.
__device__ __forceinline__ size_t partial_row_byte(size_t row, int half) {
  return (row / kPartBlockRows) * kPartBlockBytes + (row % kPartBlockRows) * 16 + half * 512;
}
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int block_scale_exp(float vmax) {
  if (!(vmax > 0.f) || (vmax >= 0x1p-6f && vmax < 0x1p8f)) return 0;
  int x;
  frexpf(vmax, &x);  // vmax = m * 2^x, m in [0.5, 1)
  const int e = x - 8;
  return e < -100 ? -100 : (e > 126 ? 126 : e);
}

// Stores a lane's half of a row through a buffer resource; byte offsets at or
// beyond the resource's size (lanes without a list entry) are dropped by the
// hardware range check.
__device__ __forceinline__ void store_partial_row(__amdgpu_buffer_rsrc_t rs, int row_byte, const f32x16* o) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      f16x8 v;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (_Float16)o[dt][8 * h8 + j];
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, row_byte + 1024 * (2 * dt + h8), 0,
                                             0);
    }
}

// p: chunk 0 of the lane's half row (partial_row_byte)
__device__ __forceinline__ void accumulate_partial_row(float (*acc)[16], const uint8_t* p, float w) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      const f16x8 v = *reinterpret_cast<const f16x8*>(p + 1024 * (2 * dt + h8));
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[dt][8 * h8 + j] += w * (float)v[j];
    }
}

// Largest |v| of the block's V values a thread staged (bf16 bit patterns;
// the magnitude order of non-NaN bf16 equals the unsigned order of their
// low 15 bits).
template <int BS>
__device__ __forceinline__ float block_vmax_part(const BlockRegs<BS, 256>& r) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < BS / 32; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t x = r.v[i][j][w] & 0x7fff7fffu;
        m = max(m, max(x & 0xffffu, x >> 16));
      }
  return __uint_as_float(m << 16);
}

// ---------------------------------------------------------------------------
// Block-major kernel: one (s, g, window, block) list and up to
// kTilesPerItem of its tiles of 128/R tokens per workgroup; the K/V block is
// staged in LDS once and the next tile's q rows are fetched while the current
// tile computes.  Writes, per (list entry, head) row, the unnormalised
// partial output O (fp16, scaled by 2^-e) and (max*c + e, sum * 2^-e) in the
// base-2 domain, so that the partial's softmax weight is 2^(max*c) * sum.
//
// The tile loop has no branch around memory operations: the prefetches are
// clamped to rows that exist and lanes without an entry store through a
// buffer resource that drops their writes.  With identical memory-operation
// counts on every path, the wait for the prefetched q rows need not also wait
// for the previous tile's partial stores.
// ---------------------------------------------------------------------------
template <int BS>
__device__ __forceinline__ void kv_outer_item(const PrefillMainArgs& a, int w, bf16_t* Ks, bf16_t* Vt,
                                              float* vmax_w) {
  constexpr int VROW = BS + 4;
  constexpr int KT = BS / 32;
  const int2 wk = a.work[w];
  const long lid = wk.x;
  const int b = (int)(lid % a.nbl);
  const long sgw = lid / a.nbl;
  const long sg = sgw / a.nwin;
  const int g = (int)(sg % a.G);
  const int s = (int)(sg / a.G);
  const int R = a.Hq / a.G;
  const int mt = kAttnRows / R;
  const int count = a.cnt[lid];  // >= 1: work items exist for non-empty lists only
  const int off = a.offs[lid];
  const int tile0 = wk.y * kTilesPerItem;
  const int ntile = min(kTilesPerItem, (count + mt - 1) / mt - tile0);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int row = wave * 32 + col;
  const int e = row / R, r = row % R;
  const int h = g * R + r;
  const float c = a.scale_log2;

  // The lane's list entry (token << rank_bits | rank) in tile `tile`, clamped
  // into the list: a lane without an entry computes on another entry's q row
  // and its stores are dropped (every MFMA column and lane statistic belongs
  // to one row only).
  auto entry_at = [&](int tile) -> int { return a.entries[(size_t)off + min(tile * mt + e, count - 1)]; };
  const size_t q_base = ((size_t)s * a.T + a.t0) * a.Hq + h;
  auto q_row = [&](int ent) -> const bf16_t* { return a.q + (q_base + (size_t)(ent >> a.rank_bits) * a.Hq) * D; };

  // first tile's entries and q rows, then the K/V block; staging the block
  // waits for all of them
  const int ent0 = entry_at(tile0);
  int ent_n = entry_at(tile0 + min(1, ntile - 1));
  bf16x8 qop[D / 16];
  load_q(qop, q_row(ent0), true, half);
  const size_t kvstride = (size_t)a.G * D;
  const size_t kvoff = ((size_t)s * a.T + (size_t)b * a.B) * kvstride + (size_t)g * D;
  BlockRegs<BS> regs;
  block_load<BS>(regs, a.k + kvoff, a.v + kvoff, kvstride, tid);
  block_store<BS>(regs, Ks, Vt, VROW, tid);
  {
    const float vm = wave_max(block_vmax_part<BS>(regs));
    if (lane == 0) vmax_w[wave] = vm;
  }
  __syncthreads();
  // Per-block power-of-two scale of the stored partials, folded into the
  // exponent: p' = 2^(x c - m c - ex) = p 2^-ex, so O' = sum p' v = O 2^-ex and
  // l' = l 2^-ex come out of the products already scaled (a power-of-two
  // factor is exact in fp32 and bf16), and the statistics hold m c + ex.
  const int ex = block_scale_exp(fmaxf(fmaxf(vmax_w[0], vmax_w[1]), fmaxf(vmax_w[2], vmax_w[3])));
  const int stat_byte = half == 0 ? (e * R + r) * 8 : 0x40000000;

  for (int it = 0; it < ntile; ++it) {
    // The K/V tile is loop-invariant; an opaque zero offset keeps its LDS
    // operand reads inside the loop instead of hoisting them into registers
    // (the offset, not the pointer, is opaque, so the reads stay LDS reads).
    int lds_off = 0;
    asm volatile("" : "+s"(lds_off));
    const bf16_t* ks_ = Ks + lds_off;
    const bf16_t* vt_ = Vt + lds_off;

    f32x16 sacc[KT];
    qk_tiles<KT>(ks_, qop, sacc, col, half);

    // q of this tile is dead: fetch the next tile's rows into the same
    // registers (the last tile re-reads its own), and the entries after it
    load_q(qop, q_row(ent_n), true, half);
    ent_n = entry_at(tile0 + min(it + 2, ntile - 1));

    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mce = mx * c + (float)ex;
    bf16x8 pop[KT][2];
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        sacc[kt][i] = __builtin_amdgcn_exp2f(sacc[kt][i] * c - mce);
        sacc[kt][i + 1] = __builtin_amdgcn_exp2f(sacc[kt][i + 1] * c - mce);
        l0 += sacc[kt][i];
        l1 += sacc[kt][i + 1];
      }
      pop[kt][0] = to_bf16x8(sacc[kt], 0);
      pop[kt][1] = to_bf16x8(sacc[kt], 8);
    }
    float l = l0 + l1;
    l += __shfl_xor(l, 32, kWave);

    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
    pv_tiles<KT>(vt_, VROW, pop, oacc, col, half);

    // rows of this tile: list positions off + (tile0+it)*mt ... + nrow - 1
    const int p0 = off + (tile0 + it) * mt;
    const int nrow = min(mt, count - (tile0 + it) * mt);
    // partial rows p0*R .. (p0+nrow)*R - 1 through a resource starting at
    // their first 32-row block; lanes past the tile's rows get an offset
    // beyond the resource and are dropped
    const size_t g0 = (size_t)p0 * R;
    const size_t blk0 = g0 / kPartBlockRows;
    const size_t blk1 = (g0 + (size_t)nrow * R - 1) / kPartBlockRows;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<uint8_t*>(a.pO) + blk0 * kPartBlockBytes, (short)0,
        (int)((blk1 - blk0 + 1) * kPartBlockBytes), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(a.pS + (size_t)p0 * R, (short)0, nrow * R * 8, kBufferWord3);
    const int row_byte = e < nrow ? (int)(partial_row_byte(g0 + row, half) - blk0 * kPartBlockBytes) : 0x7ff00000;
    store_partial_row(ro, row_byte, oacc);
    const float2 st = make_float2(mce, l);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, st), rs, stat_byte, 0, 0);
  }
}

template <int BS>
__global__ __launch_bounds__(256, 2) void kv_outer_kernel(PrefillMainArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t Ks[BS * KROW];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[D * (BS + 4)];
  __shared__ float vmax_w[4];
  const int w = blockIdx.x;
  if (w >= a.n_work[0]) return;
  kv_outer_item<BS>(a, w, Ks, Vt, vmax_w);
}

// ---------------------------------------------------------------------------
// Query-major kernel: a workgroup owns up to 128/R consecutive tokens of one
// (s, g) with all R heads of the group and runs online-softmax attention over
// key tiles of KTILE keys in [k_lo, t_last], masking per row to
// [lo(t), t] with lo(t) = L(t)*B (sparse: the local block) or 0 (dense).
// Sparse mode then merges the partials of the row's non-local blocks.
// ---------------------------------------------------------------------------
template <bool DENSE>
__global__ __launch_bounds__(256, 2) void query_major_kernel(PrefillMainArgs a) {
  constexpr int KTILE = 64;
  constexpr int VROW = KTILE + 4;
  constexpr int KT = KTILE / 32;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[KTILE * KROW];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[D * VROW];

  const int R = a.Hq / a.G;
  const int mt = kAttnRows / R;
  const int g = blockIdx.y, s = blockIdx.z;
  const int tl0 = blockIdx.x * mt;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int row = wave * 32 + col;
  const int e = row / R, r = row % R;
  const int tl = tl0 + e;
  const bool valid = e < mt && tl < a.tc;
  const int tlc = min(tl, a.tc - 1);
  const int t = a.t0 + tlc;
  const int h = g * R + r;
  const int L = t / a.B;

  // the row's own key window; a given selection may omit the local block
  int lo = DENSE ? 0 : L * a.B;
  int info = 0;
  bool has_local = true;
  if (!DENSE) {
    info = a.rinfo[((size_t)s * a.tc + tlc) * a.G + g];
    has_local = (info >> 30) & 1;
  }
  const int hi = (valid && has_local) ? t : lo - 1;  // empty window when not attended

  const int t_first = a.t0 + tl0;
  const int t_last = a.t0 + min(tl0 + mt, a.tc) - 1;
  const int k_lo = DENSE ? 0 : (t_first / a.B) * a.B;
  const int k_hi = t_last;

  bf16x8 qop[D / 16];
  load_q(qop, a.q + (((size_t)s * a.T + t) * a.Hq + h) * D, valid, half);

  const size_t kvstride = (size_t)a.G * D;
  const bf16_t* kseq = a.k + (size_t)s * a.T * kvstride + (size_t)g * D;
  const bf16_t* vseq = a.v + (size_t)s * a.T * kvstride + (size_t)g * D;
  const float c = a.scale_log2;

  float m = -INFINITY, l = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};

  for (int kb = k_lo; kb <= k_hi; kb += KTILE) {
    const int nvalid = min(KTILE, k_hi + 1 - kb);
    __syncthreads();
    stage_k<KTILE>(Ks, kseq + (size_t)kb * kvstride, kvstride, nvalid, tid);
    stage_vt<KTILE>(Vt, VROW, vseq + (size_t)kb * kvstride, kvstride, nvalid, tid);
    __syncthreads();

    f32x16 sacc[KT];
    qk_tiles<KT>(Ks, qop, sacc, col, half);
    float tmx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = kb + kt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        const bool ok = j >= lo && j <= hi;
        sacc[kt][i] = ok ? sacc[kt][i] : -INFINITY;
        tmx = fmaxf(tmx, sacc[kt][i]);
      }
    tmx = fmaxf(tmx, __shfl_xor(tmx, 32, kWave));
    const float m_new = fmaxf(m, tmx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m - m_use) * c);
    const float muc = m_use * c;
    bf16x8 pop[KT][2];
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[kt][i] = __builtin_amdgcn_exp2f(sacc[kt][i] * c - muc);
        ps += sacc[kt][i];
      }
      pop[kt][0] = to_bf16x8(sacc[kt], 0);
      pop[kt][1] = to_bf16x8(sacc[kt], 8);
    }
    ps += __shfl_xor(ps, 32, kWave);
    l = l * alpha + ps;
    m = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    pv_tiles<KT>(Vt, VROW, pop, oacc, col, half);
  }
  if (!valid) return;

  // The row's terms in the base-2 domain: the local window has weight
  // 2^(m*c) * l and unnormalised output oacc; partial q has weight
  // 2^(s1_q) * s2_q and stored output O_q, both relative to 2^(s1_q).
  const float lse2_loc = (l > 0.f) ? m * c + __log2f(l) : -INFINITY;
  float M2 = lse2_loc;
  float o[4][16];
  float sumw;
  if (!DENSE) {
    const int nv = info & 0x3fffffff;  // partial slots 0..nv-1
    // list positions of the row's partials; rows pos*R + r of pO / pS
    const int32_t* pos = a.epos + (((size_t)s * a.tc + tl) * a.G + g) * a.KS;
    // pass 1: the largest log-weight.  Both passes take the slots in groups
    // whose position and statistics loads are issued together (slots past nv
    // read the last one again and get weight 0).
    constexpr int QG = 16;
    for (int q0 = 0; q0 < nv; q0 += QG) {
      int pq[QG];
#pragma unroll
      for (int u = 0; u < QG; ++u) pq[u] = pos[min(q0 + u, nv - 1)];
      float2 st[QG];
#pragma unroll
      for (int u = 0; u < QG; ++u) st[u] = a.pS[(size_t)pq[u] * R + r];
#pragma unroll
      for (int u = 0; u < QG; ++u) M2 = fmaxf(M2, st[u].x + __log2f(st[u].y));
    }
    const float M2u = (M2 == -INFINITY) ? 0.f : M2;
    const float wl = (l > 0.f) ? __builtin_amdgcn_exp2f(m * c - M2u) : 0.f;
    sumw = wl * l;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = oacc[dt][i] * wl;
    // pass 2: weighted partials in slot order, in groups of QG2 (registers)
    constexpr int QG2 = 8;
    for (int q0 = 0; q0 < nv; q0 += QG2) {
      int pq[QG2];
#pragma unroll
      for (int u = 0; u < QG2; ++u) pq[u] = pos[min(q0 + u, nv - 1)];
#pragma unroll
      for (int u = 0; u < QG2; ++u) {
        const size_t prow = (size_t)pq[u] * R + r;
        const float2 st = a.pS[prow];
        const float w = q0 + u < nv ? __builtin_amdgcn_exp2f(st.x - M2u) : 0.f;
        sumw += w * st.y;
        accumulate_partial_row(o, reinterpret_cast<const uint8_t*>(a.pO) + partial_row_byte(prow, half), w);
      }
    }
    M2 = M2u;
  } else {
    const float inv_l = (l > 0.f) ? 1.0f / l : 0.f;
    sumw = (l > 0.f) ? 1.f : 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = oacc[dt][i] * inv_l;
  }

  const float invw = (sumw > 0.f) ? 1.0f / sumw : 0.f;
  bf16_t* dst = a.out + (((size_t)s * a.T + t) * a.Hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      bf16x4 v4;
      v4[0] = (__bf16)(o[dt][4 * i4] * invw);
      v4[1] = (__bf16)(o[dt][4 * i4 + 1] * invw);
      v4[2] = (__bf16)(o[dt][4 * i4 + 2] * invw);
      v4[3] = (__bf16)(o[dt][4 * i4 + 3] * invw);
      *reinterpret_cast<bf16x4*>(dst + dt * 32 + i4 * 8 + 4 * half) = v4;
    }
  if (a.lse != nullptr && half == 0) {
    const float lse2 = (sumw > 0.f) ? M2 + __log2f(sumw) : -INFINITY;
    a.lse[((size_t)s * a.T + t) * a.Hq + h] = lse2 * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Dense (all visible blocks) causal attention: the all-blocks comparison
// mode.  A workgroup owns 256/R consecutive tokens of one (s, g) with the R
// heads of the group (256 query rows, 32 per wave, 8 waves) and runs
// online-softmax attention over 128-key tiles of [0, t_last].  K/V tiles are
// double-buffered in LDS: the next tile's loads are issued before the current
// tile's products and written to the other buffer after them, so one barrier
// per tile separates the two and the load latency hides behind the products.
// Only tiles that reach past the first token of the workgroup are masked
// (keys j > t); the others are wholly visible to every row.  Workgroups are
// issued longest-first.
// ---------------------------------------------------------------------------
// Loads of one K/V tile through buffer resources whose base is the tile's
// first row and whose size ends at the sequence's last row: the lanes' byte
// offsets are computed once (tile-invariant), the row steps between a
// thread's chunks are scalar offsets, and rows past the sequence read as 0.
// Rows past the last query row of the workgroup are read as they are: the
// causal mask gives them probability 0.
template <int NK, int NTH>
__device__ __forceinline__ void block_load_buf(BlockRegs<NK, NTH>& r, __amdgpu_buffer_rsrc_t rk,
                                               __amdgpu_buffer_rsrc_t rv, int koff, const int* voff, int rowbytes) {
#pragma unroll
  for (int i = 0; i < NK * 16 / NTH; ++i)
    r.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, i * (NTH / 16) * rowbytes, 0));
#pragma unroll
  for (int i = 0; i < NK * 8 / NTH; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r.v[i][j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, voff[i], j * rowbytes, 0));
}

// 8 waves (two per SIMD, one workgroup per CU): 256 query rows share every
// staged 128-key tile; tiles are double-buffered in LDS (137 KB).
constexpr int kDenseRows = 256;
constexpr int kDenseThreads = 512;

__global__ __launch_bounds__(kDenseThreads, 1) void dense_attn_kernel(PrefillMainArgs a) {
  constexpr int KTILE = 128;
  constexpr int VROW = KTILE + kVtPadQ;
  constexpr int KT = KTILE / 32;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][KTILE * KROW];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[2][D * VROW];

  const int R = a.Hq / a.G;
  const int mt = kDenseRows / R;
  const int g = blockIdx.y, s = blockIdx.z;
  const int tl0 = ((int)gridDim.x - 1 - (int)blockIdx.x) * mt;   // longest rows first
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int row = wave * 32 + col;
  const int e = row / R, r = row % R;
  const int tl = tl0 + e;
  const bool valid = e < mt && tl < a.tc;
  const int t = a.t0 + min(tl, a.tc - 1);
  const int h = g * R + r;
  const int hi = valid ? t : -1;   // rows without a token see no key

  const int t_first = a.t0 + tl0;
  const int t_last = a.t0 + min(tl0 + mt, a.tc) - 1;
  const int ntiles = t_last / KTILE + 1;

  bf16x8 qop[D / 16];
  load_q(qop, a.q + (((size_t)s * a.T + t) * a.Hq + h) * D, valid, half);

  const size_t kvstride = (size_t)a.G * D;
  const bf16_t* kseq = a.k + (size_t)s * a.T * kvstride + (size_t)g * D;
  const bf16_t* vseq = a.v + (size_t)s * a.T * kvstride + (size_t)g * D;
  const float c = a.scale_log2;

  BlockRegs<KTILE, kDenseThreads> regs;
  const int rowbytes = (int)(kvstride * 2);
  const int koff = (tid >> 4) * rowbytes + (tid & 15) * 16;
  int voff[KTILE * 8 / kDenseThreads];
#pragma unroll
  for (int i = 0; i < KTILE * 8 / kDenseThreads; ++i) {
    int k4, dq;
    vt_unit_q(tid + kDenseThreads * i, k4, dq);
    voff[i] = k4 * 4 * rowbytes + dq * 8;
  }
  auto load_tile = [&](int kn) {
    const int nrows = min(KTILE, a.T - kn);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(kseq + (size_t)kn * kvstride), (short)0, nrows * rowbytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(vseq + (size_t)kn * kvstride), (short)0, nrows * rowbytes, kBufferWord3);
    block_load_buf<KTILE, kDenseThreads>(regs, rk, rv, koff, voff, rowbytes);
  };
  load_tile(0);
  block_store<KTILE, kDenseThreads, true>(regs, Ks[0], Vt[0], VROW, tid);
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};

  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int kb = it * KTILE;
    if (it + 1 < ntiles) load_tile(kb + KTILE);  // uniform
    f32x16 sacc[KT];
    qk_tiles<KT>(Ks[cur], qop, sacc, col, half);
    float tmx = -INFINITY;
    if (kb + KTILE - 1 > t_first) {  // uniform: a tile on the diagonal
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = kb + kt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
          sacc[kt][i] = j <= hi ? sacc[kt][i] : -INFINITY;
          tmx = fmaxf(tmx, sacc[kt][i]);
        }
    } else {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmx = fmaxf(tmx, sacc[kt][i]);
    }
    tmx = fmaxf(tmx, __shfl_xor(tmx, 32, kWave));
    // Lazy rescaling: the reference maximum m moves only when a tile's
    // maximum exceeds it by more than 8 in the base-2 exponent, so most tiles
    // skip rescaling the accumulators; probabilities stay below 2^8 (exact
    // softmax is shift-invariant, and fp32 / bf16 keep their relative
    // precision there).  A row's first keys always set m (m = -inf before).
    const bool grow = (tmx - m) * c > 8.0f;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // uniform
      const float m_new = grow ? tmx : m;
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      m = m_new;
    }
    const float muc = (m == -INFINITY) ? 0.f : m * c;
    bf16x8 pop[KT][2];
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        sacc[kt][i] = __builtin_amdgcn_exp2f(sacc[kt][i] * c - muc);
        sacc[kt][i + 1] = __builtin_amdgcn_exp2f(sacc[kt][i + 1] * c - muc);
        ps0 += sacc[kt][i];
        ps1 += sacc[kt][i + 1];
      }
      pop[kt][0] = to_bf16x8(sacc[kt], 0);
      pop[kt][1] = to_bf16x8(sacc[kt], 8);
    }
    float ps = ps0 + ps1;
    ps += __shfl_xor(ps, 32, kWave);
    l += ps;
    pv_tiles<KT, true>(Vt[cur], VROW, pop, oacc, col, half);
    if (it + 1 < ntiles) block_store<KTILE, kDenseThreads, true>(regs, Ks[cur ^ 1], Vt[cur ^ 1], VROW, tid);
    __syncthreads();
  }
  if (!valid) return;

  const float inv_l = (l > 0.f) ? 1.0f / l : 0.f;
  bf16_t* dst = a.out + (((size_t)s * a.T + t) * a.Hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      bf16x4 v4;
      v4[0] = (__bf16)(oacc[dt][4 * i4] * inv_l);
      v4[1] = (__bf16)(oacc[dt][4 * i4 + 1] * inv_l);
      v4[2] = (__bf16)(oacc[dt][4 * i4 + 2] * inv_l);
      v4[3] = (__bf16)(oacc[dt][4 * i4 + 3] * inv_l);
      *reinterpret_cast<bf16x4*>(dst + dt * 32 + i4 * 8 + 4 * half) = v4;
    }
  if (a.lse != nullptr && half == 0)
    a.lse[((size_t)s * a.T + t) * a.Hq + h] = (l > 0.f) ? (m * c + __log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, size_t n, int32_t value, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  fill_i32_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>(p, n, value);
  return hipGetLastError();
}

// Sorts each block list's entries (tl << rank_bits | slot, all distinct) and
// points every row slot at its entry's new list position, so that sums over a
// list run in an order that does not depend on how the integer atomics filled
// it.  A token enters a list at most once, so the order is the tokens' order:
// each entry sets its token's bit in a window-sized bitmap in LDS and its rank
// is the number of bits below it (a prefix count over the bitmap's words).
// Lists of at most 64 entries count the smaller keys directly.  A list in
// which a token occurs twice (only possible with duplicate selections, which
// are invalid input) is sorted by the bitonic network instead, and a list
// longer than kListWindow (the same case) keeps its order.
__global__ __launch_bounds__(256) void lists_sort_kernel(PrefillMainArgs a) {
  constexpr int kWords = kListWindow / 32;
  constexpr int kPer = kListWindow / 256;  // entries per thread at most
  static_assert(kWords <= 256, "one bitmap word per thread");
  __shared__ uint32_t key[kListWindow];
  __shared__ uint32_t bits[kWords];
  __shared__ int wsum[4];
  __shared__ int dup;
  const long lid = blockIdx.x;
  const int count = a.cnt[lid];
  if (count < 2 || count > kListWindow) return;
  const int g = (int)((lid / a.nbl) / a.nwin % a.G);
  const int s = (int)((lid / a.nbl) / a.nwin / a.G);
  const int w = (int)((lid / a.nbl) % a.nwin);
  const int off = a.offs[lid];
  const int tid = threadIdx.x;
  const uint32_t mask = (1u << a.rank_bits) - 1u;
  auto place = [&](uint32_t e, int pos) {
    a.entries[off + pos] = (int32_t)e;
    const long row = ((long)s * a.tc + (long)(e >> a.rank_bits)) * a.G + g;
    a.epos[(size_t)row * a.KS + (e & mask)] = off + pos;
  };
  if (count <= 64) {
    const uint32_t mine = tid < count ? (uint32_t)a.entries[off + tid] : 0xffffffffu;
    key[tid] = mine;
    __syncthreads();
    if (tid < count) {
      int rank = 0;
      for (int i = 0; i < count; ++i) rank += key[i] < mine ? 1 : 0;
      place(mine, rank);
    }
    return;
  }
  // every entry is read (into registers) before any is written back
  const int wbase = w * a.window;
  const int nwords = (a.window + 31) / 32;
  uint32_t mine[kPer];
  if (tid < kWords) bits[tid] = 0u;
  if (tid == 0) dup = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = tid + 256 * j;
    mine[j] = i < count ? (uint32_t)a.entries[off + i] : 0u;
  }
  __syncthreads();
  int seen = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (tid + 256 * j < count) {
      const int loc = (int)(mine[j] >> a.rank_bits) - wbase;
      const uint32_t bit = 1u << (loc & 31);
      seen |= (atomicOr(&bits[loc >> 5], bit) & bit) != 0u;
    }
  if (seen) dup = 1;
  __syncthreads();
  if (dup == 0) {
    // exclusive prefix of the words' popcounts, one word per thread
    const int lane = tid & 63, wave = tid >> 6;
    const int c = tid < nwords ? __builtin_popcount(bits[tid]) : 0;
    int x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = x - c;
    for (int v = 0; v < wave; ++v) before += wsum[v];
    __syncthreads();  // every thread has read wsum before key[] is reused
    if (tid < kWords) key[tid] = (uint32_t)before;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (tid + 256 * j < count) {
        const int loc = (int)(mine[j] >> a.rank_bits) - wbase;
        const int rank = (int)key[loc >> 5] + __builtin_popcount(bits[loc >> 5] & ((1u << (loc & 31)) - 1u));
        place(mine[j], rank);
      }
    return;
  }
  int n2 = 1;
  while (n2 < count) n2 <<= 1;
  for (int i = tid; i < n2; i += 256) key[i] = i < count ? (uint32_t)a.entries[off + i] : 0xffffffffu;
  __syncthreads();
  for (int kk = 2; kk <= n2; kk <<= 1)
    for (int jj = kk >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < n2; i += 256) {
        const int p = i ^ jj;
        if (p > i) {
          const uint32_t x = key[i], y = key[p];
          const bool up = (i & kk) == 0;
          if ((x > y) == up) {
            key[i] = y;
            key[p] = x;
          }
        }
      }
      __syncthreads();
    }
  for (int i = tid; i < count; i += 256) place(key[i], i);
}

hipError_t launch_sort_lists(const PrefillMainArgs& a, hipStream_t st) {
  if (a.nlists > 0) lists_sort_kernel<<<(unsigned)a.nlists, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_list_work(const PrefillMainArgs& a, int mt, int2* work, int32_t* n_work, hipStream_t st) {
  const int nblk = (int)((a.nlists + kScanItems - 1) / kScanItems);
  lists_scan_reduce_kernel<<<nblk, 1024, 0, st>>>(a.cnt, a.bsum, a.nlists, mt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  lists_scan_top_kernel<<<1, 1024, 0, st>>>(a.bsum, nblk, n_work);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  lists_scan_final_kernel<<<nblk, 1024, 0, st>>>(a.cnt, a.bsum, a.offs, work, a.nlists, mt);
  return hipGetLastError();
}

hipError_t launch_block_lists(const PrefillMainArgs& a, int mt, hipStream_t st) {
  hipError_t err = launch_fill_i32(a.cnt, (size_t)a.nlists, 0, st);
  if (err != hipSuccess) return err;
  const long n_rows = (long)a.batch * a.tc * a.G;
  const int rows_wg = count_rows_per_wg(a.KS);
  lists_count_kernel<<<(unsigned)((n_rows + rows_wg - 1) / rows_wg), kCountRows, 0, st>>>(a, rows_wg);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = launch_list_work(a, mt, a.work, a.n_work, st)) != hipSuccess) return err;
  lists_scatter_kernel<<<(unsigned)((n_rows + 255) / 256), 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill_main_sparse(const PrefillMainArgs& a, hipStream_t st) {
  prof_mark(st, MSA_STAGE_BLOCK_LISTS);
  const int R = a.Hq / a.G;
  const int mt = kAttnRows / R;
  hipError_t err = launch_block_lists(a, mt, st);
  if (err != hipSuccess) return err;
  if (a.max_work > 0) {
    prof_mark(st, MSA_STAGE_KV_OUTER);
    const dim3 grid((unsigned)a.max_work);
    if (a.B == 128) kv_outer_kernel<128><<<grid, 256, 0, st>>>(a);
    else if (a.B == 64) kv_outer_kernel<64><<<grid, 256, 0, st>>>(a);
    else kv_outer_kernel<32><<<grid, 256, 0, st>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const dim3 qgrid((unsigned)((a.tc + mt - 1) / mt), a.G, a.batch);
  prof_mark(st, MSA_STAGE_QUERY_MAJOR);
  query_major_kernel<false><<<qgrid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill_main_dense(const PrefillMainArgs& a, hipStream_t st) {
  const int R = a.Hq / a.G;
  const int mtd = kDenseRows / R;
  const dim3 qgrid((unsigned)((a.tc + mtd - 1) / mtd), a.G, a.batch);
  dense_attn_kernel<<<qgrid, kDenseThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
