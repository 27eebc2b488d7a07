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
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int D = 128;          // head_dim
constexpr int KROW = D + 8;     // LDS row stride of K tiles (bf16)

// ---------------------------------------------------------------------------
// LDS staging helpers (256 threads).
// K tile: rows [key][D] -> Ks[key*KROW + d]
// V tile: transposed -> Vt[d*VROW + key], so that a lane can fetch 4
// consecutive keys of one d with one 8-byte read (PV operand layout).
// Keys >= nvalid are zero-filled.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void stage_k(bf16_t* Ks, const bf16_t* __restrict__ kbase, size_t kstride,
                                        int nkeys, int nvalid, int tid) {
  const int nch = nkeys * (D / 8);
  for (int c = tid; c < nch; c += 256) {
    const int key = c >> 4, part = c & 15;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (key < nvalid) val = *reinterpret_cast<const u32x4*>(kbase + (size_t)key * kstride + part * 8);
    *reinterpret_cast<u32x4*>(Ks + key * KROW + part * 8) = val;
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

__device__ __forceinline__ void stage_vt(bf16_t* Vt, int vrow, const bf16_t* __restrict__ vbase,
                                         size_t vstride, int nkeys, int nvalid, int tid) {
  // unit = 4 keys x 4 d; 32 units per 4-key group
  const int nunits = (nkeys / 4) * (D / 4);
  for (int u = tid; u < nunits; u += 256) {
    int k4, dq;
    vt_unit(u, k4, dq);
    u32x2 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = k4 * 4 + i;
      r[i] = u32x2{0u, 0u};
      if (key < nvalid) r[i] = *reinterpret_cast<const u32x2*>(vbase + (size_t)key * vstride + dq * 4);
    }
    // 4x4 transpose of 16-bit lanes: o[j] = (r0[j], r1[j], r2[j], r3[j])
    u32x2 o[4];
    o[0] = u32x2{(r[0][0] & 0xffffu) | (r[1][0] << 16), (r[2][0] & 0xffffu) | (r[3][0] << 16)};
    o[1] = u32x2{(r[0][0] >> 16) | (r[1][0] & 0xffff0000u), (r[2][0] >> 16) | (r[3][0] & 0xffff0000u)};
    o[2] = u32x2{(r[0][1] & 0xffffu) | (r[1][1] << 16), (r[2][1] & 0xffffu) | (r[3][1] << 16)};
    o[3] = u32x2{(r[0][1] >> 16) | (r[1][1] & 0xffff0000u), (r[2][1] >> 16) | (r[3][1] & 0xffff0000u)};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x2*>(Vt + (dq * 4 + j) * vrow + k4 * 4) = o[j];
  }
}

// Whole-block K/V staging through registers with compile-time trip counts:
// every global load of the block is issued before the first LDS write.
template <int BS>
struct BlockRegs {
  u32x4 k[BS / 16];     // 16-byte chunks of K rows: chunk c = tid + 256 i
  u32x2 v[BS / 32][4];  // 4 keys x 4 d units of V: unit u = tid + 256 i
};

template <int BS>
__device__ __forceinline__ void block_load(BlockRegs<BS>& r, const bf16_t* __restrict__ kbase,
                                           const bf16_t* __restrict__ vbase, size_t stride, int tid) {
#pragma unroll
  for (int i = 0; i < BS / 16; ++i) {
    const int c = tid + 256 * i;
    r.k[i] = *reinterpret_cast<const u32x4*>(kbase + (size_t)(c >> 4) * stride + (c & 15) * 8);
  }
#pragma unroll
  for (int i = 0; i < BS / 32; ++i) {
    const int u = tid + 256 * i;
    int k4, dq;
    vt_unit(u, k4, dq);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r.v[i][j] = *reinterpret_cast<const u32x2*>(vbase + (size_t)(k4 * 4 + j) * stride + dq * 4);
  }
}

template <int BS>
__device__ __forceinline__ void block_store(const BlockRegs<BS>& r, bf16_t* Ks, bf16_t* Vt, int vrow, int tid) {
#pragma unroll
  for (int i = 0; i < BS / 16; ++i) {
    const int c = tid + 256 * i;
    *reinterpret_cast<u32x4*>(Ks + (c >> 4) * KROW + (c & 15) * 8) = r.k[i];
  }
#pragma unroll
  for (int i = 0; i < BS / 32; ++i) {
    const int u = tid + 256 * i;
    int k4, dq;
    vt_unit(u, k4, dq);
    const u32x2* x = r.v[i];
    u32x2 o[4];
    o[0] = u32x2{(x[0][0] & 0xffffu) | (x[1][0] << 16), (x[2][0] & 0xffffu) | (x[3][0] << 16)};
    o[1] = u32x2{(x[0][0] >> 16) | (x[1][0] & 0xffff0000u), (x[2][0] >> 16) | (x[3][0] & 0xffff0000u)};
    o[2] = u32x2{(x[0][1] & 0xffffu) | (x[1][1] << 16), (x[2][1] & 0xffffu) | (x[3][1] << 16)};
    o[3] = u32x2{(x[0][1] >> 16) | (x[1][1] & 0xffff0000u), (x[2][1] >> 16) | (x[3][1] & 0xffff0000u)};
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(Vt + (dq * 4 + j) * vrow + k4 * 4) = o[j];
  }
}

// S^T tile (32 keys x 32 query rows) = K[32 x D] . Q^T, A operand from LDS.
__device__ __forceinline__ f32x16 qk_tile(const bf16_t* Ks, int key0, const bf16x8* qop, int col,
                                          int half) {
  f32x16 acc = {};
  const bf16_t* arow = Ks + (key0 + col) * KROW + 8 * half;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    acc = mfma32x32x16(*reinterpret_cast<const bf16x8*>(arow + 16 * ks), qop[ks], acc);
  return acc;
}

// O^T[d-tile] += V^T[32 d x 16 keys] . P^T, for the 16-key slice starting at key0.
__device__ __forceinline__ f32x16 pv_step(const bf16_t* Vt, int vrow, int dt, int key0, bf16x8 p,
                                          f32x16 acc, int col, int half) {
  const bf16_t* vr = Vt + (dt * 32 + col) * vrow + key0 + 4 * half;
  const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
  return mfma32x32x16(join_bf16x4(lo, hi), p, acc);
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
// (s, g, window, block).  Entry of a row = tl * KS + rank, rank = position
// among the row's valid non-local entries (so partial storage needs only
// KS = min(k, nb) slots per row).
// ---------------------------------------------------------------------------
__global__ void fill_i32_kernel(int32_t* p, size_t n, int32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__device__ __forceinline__ size_t list_id(const PrefillMainArgs& a, int s, int g, int tl, int b) {
  const int w = tl / kListWindow;
  return (((size_t)s * a.G + g) * a.nwin + w) * a.nbl + b;
}

__global__ void lists_count_kernel(PrefillMainArgs a) {
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
  int rank = 0;
  for (int j = 0; j < a.topk && rank < a.KS; ++j) {
    const int e = br[j];
    if (e >= 0 && e < L) {
      a.epos[(size_t)row * a.KS + rank] = atomicAdd(&a.cnt[list_id(a, s, g, tl, e)], 1);
      ++rank;
    }
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
  int rank = 0;
  for (int j = 0; j < a.topk && rank < a.KS; ++j) {
    const int e = br[j];
    if (e >= 0 && e < L) {
      const size_t lid = list_id(a, s, g, tl, e);
      a.entries[(size_t)a.offs[lid] + a.epos[(size_t)row * a.KS + rank]] = tl * a.KS + rank;
      ++rank;
    }
  }
}

// ---------------------------------------------------------------------------
// fp16 partial rows.  A row holds 128 values in a lane-native order: lane half
// h of the MFMA output layout stores its 16 values of d-tile dt at positions
// dt*32 + h*16 + i, where value i has d = 32*dt + 8*(i/4) + 4*h + (i%4).  The
// row is scaled by 2^-e so that its largest magnitude lies in [2^14, 2^15)
// (exact power-of-two scaling; no fp16 overflow for any finite input).
// ---------------------------------------------------------------------------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int row_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int x;
  frexpf(amax, &x);  // amax = m * 2^x, m in [0.5, 1)
  int e = x - 15;
  return e < -100 ? -100 : (e > 100 ? 100 : e);
}

__device__ __forceinline__ void store_partial_row(uint16_t* row, const f32x16* o, float mul, int half) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      f16x8 v;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (_Float16)(o[dt][8 * h8 + j] * mul);
      *reinterpret_cast<f16x8*>(row + dt * 32 + half * 16 + h8 * 8) = v;
    }
}

__device__ __forceinline__ void accumulate_partial_row(float (*acc)[16], const uint16_t* row, float w, int half) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int h8 = 0; h8 < 2; ++h8) {
      const f16x8 v = *reinterpret_cast<const f16x8*>(row + dt * 32 + half * 16 + h8 * 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[dt][8 * h8 + j] += w * (float)v[j];
    }
}

// ---------------------------------------------------------------------------
// Block-major kernel: one (s, g, window, block) list and up to
// kTilesPerItem of its tiles of 128/R tokens per workgroup; the K/V block is
// staged in LDS once and the next tile's q rows are fetched while the current
// tile computes.  Writes, per (token, head) row, the normalised partial
// output (fp16 row-scaled) and (lse2, scale exponent), lse2 = max*c +
// log2(sum) in the base-2 domain.
// ---------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(256, 2) void kv_outer_kernel(PrefillMainArgs a) {
  constexpr int VROW = BS + 4;
  constexpr int KT = BS / 32;
  __shared__ __attribute__((aligned(16))) bf16_t Ks[BS * KROW];
  __shared__ __attribute__((aligned(16))) bf16_t Vt[D * VROW];

  const int w = blockIdx.x;
  if (w >= a.n_work[0]) return;
  const int2 wk = a.work[w];
  const long lid = wk.x;
  const int b = (int)(lid % a.nbl);
  const long sgw = lid / a.nbl;
  const long sg = sgw / a.nwin;
  const int g = (int)(sg % a.G);
  const int s = (int)(sg / a.G);
  const int R = a.Hq / a.G;
  const int mt = kAttnRows / R;
  const int count = a.cnt[lid];
  const int off = a.offs[lid];
  const int tile0 = wk.y * kTilesPerItem;
  const int ntile = min(kTilesPerItem, (count + mt - 1) / mt - tile0);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int row = wave * 32 + col;
  const int e = row / R, r = row % R;
  const int h = g * R + r;
  const float c = a.scale_log2;

  // the lane's (token, rank) in tile `tile` of the list, and its q row
  auto locate = [&](int tile, int& tl, int& rank) -> bool {
    const int e0 = tile * mt;
    const bool valid = e < mt && e0 + e < count;
    tl = 0;
    rank = 0;
    if (valid) {
      const int ent = a.entries[(size_t)off + e0 + e];
      tl = ent / a.KS;
      rank = ent % a.KS;
    }
    return valid;
  };

  // issue every global load first: list entry, the K/V block, the q row
  int tl, rank;
  bool valid = locate(tile0, tl, rank);
  const size_t kvstride = (size_t)a.G * D;
  const size_t kvoff = ((size_t)s * a.T + (size_t)b * a.B) * kvstride + (size_t)g * D;
  BlockRegs<BS> regs;
  block_load<BS>(regs, a.k + kvoff, a.v + kvoff, kvstride, tid);
  bf16x8 qop[D / 16];
  load_q(qop, a.q + (((size_t)s * a.T + a.t0 + tl) * a.Hq + h) * D, valid, half);
  block_store<BS>(regs, Ks, Vt, VROW, tid);
  __syncthreads();

  for (int it = 0; it < ntile; ++it) {
    // prefetch the next tile's q rows while this one computes
    int tl_n = 0, rank_n = 0;
    bool valid_n = false;
    bf16x8 qop_n[D / 16];
    if (it + 1 < ntile) {
      valid_n = locate(tile0 + it + 1, tl_n, rank_n);
      load_q(qop_n, a.q + (((size_t)s * a.T + a.t0 + tl_n) * a.Hq + h) * D, valid_n, half);
    }

    // The K/V tile is loop-invariant; an opaque zero offset keeps its LDS
    // operand reads inside the loop instead of hoisting them into registers
    // (the offset, not the pointer, is opaque, so the reads stay LDS reads).
    int lds_off = 0;
    asm volatile("" : "+s"(lds_off));
    const bf16_t* ks_ = Ks + lds_off;
    const bf16_t* vt_ = Vt + lds_off;

    f32x16 sacc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) sacc[kt] = qk_tile(ks_, kt * 32, qop, col, half);

    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mc = mx * c;
    float l = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(sacc[kt][i] * c - mc);
        sacc[kt][i] = p;
        l += p;
      }
    l += __shfl_xor(l, 32, kWave);

    bf16x8 pop[KT][2];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      pop[kt][0] = to_bf16x8(sacc[kt], 0);
      pop[kt][1] = to_bf16x8(sacc[kt], 8);
    }
    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      oacc[dt] = f32x16{};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        oacc[dt] = pv_step(vt_, VROW, dt, kt * 32, pop[kt][0], oacc[dt], col, half);
        oacc[dt] = pv_step(vt_, VROW, dt, kt * 32 + 16, pop[kt][1], oacc[dt], col, half);
      }
    }

    // normalised row = oacc / l, stored as fp16 scaled by 2^-e
    const float inv = 1.0f / l;
    float amax = 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(oacc[dt][i]));
    amax = fmaxf(amax, __shfl_xor(amax, 32, kWave)) * inv;
    const int ex = row_scale_exp(amax);
    if (valid) {
      const size_t prow = ((((size_t)s * a.tc + tl) * a.G + g) * a.KS + rank) * R + r;
      store_partial_row(a.pO + prow * D, oacc, inv * ldexpf(1.0f, -ex), half);
      if (half == 0) a.pS[prow] = make_float2(mc + __log2f(l), (float)ex);
    }

    if (it + 1 < ntile) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) qop[ks] = qop_n[ks];
      valid = valid_n;
      tl = tl_n;
      rank = rank_n;
    }
  }
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
  const int t = a.t0 + min(tl, a.tc - 1);
  const int h = g * R + r;
  const int L = t / a.B;

  // the row's own key window
  int lo = DENSE ? 0 : L * a.B;
  bool has_local = true;
  const int32_t* br = nullptr;
  if (!DENSE) {
    br = a.bidx + ((size_t)((long)s * a.bidx_rows + (t - a.bidx_t_off)) * a.G + g) * a.topk;
    // given selections may omit the local block
    has_local = false;
    for (int j = 0; j < a.topk; ++j)
      if (br[j] == L) { has_local = true; break; }
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
    stage_k(Ks, kseq + (size_t)kb * kvstride, kvstride, KTILE, nvalid, tid);
    stage_vt(Vt, VROW, vseq + (size_t)kb * kvstride, kvstride, KTILE, nvalid, tid);
    __syncthreads();

    f32x16 sacc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) sacc[kt] = qk_tile(Ks, kt * 32, qop, col, half);
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
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(sacc[kt][i] * c - muc);
        sacc[kt][i] = p;
        ps += p;
      }
    ps += __shfl_xor(ps, 32, kWave);
    l = l * alpha + ps;
    m = m_new;
    bf16x8 pop[KT][2];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      pop[kt][0] = to_bf16x8(sacc[kt], 0);
      pop[kt][1] = to_bf16x8(sacc[kt], 8);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        oacc[dt] = pv_step(Vt, VROW, dt, kt * 32, pop[kt][0], oacc[dt], col, half);
        oacc[dt] = pv_step(Vt, VROW, dt, kt * 32 + 16, pop[kt][1], oacc[dt], col, half);
      }
    }
  }
  if (!valid) return;

  // lse2 of the local window (base-2 domain); -inf when nothing was attended
  const float lse2_loc = (l > 0.f) ? m * c + __log2f(l) : -INFINITY;
  float M2 = lse2_loc;
  float scale_loc = (l > 0.f) ? 1.0f / l : 0.f;  // oacc is unnormalised
  float o[4][16];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = oacc[dt][i];

  float sumw = 0.f;
  if (!DENSE) {
    const size_t prow0 = (((size_t)s * a.tc + tl) * a.G + g) * a.KS;
    const int R_ = R;
    // the row's partial slots are its valid non-local entries, ranks 0..nv-1
    int nv = 0;
    for (int j = 0; j < a.topk && nv < a.KS; ++j) {
      const int eb = br[j];
      nv += (eb >= 0 && eb < L) ? 1 : 0;
    }
    const float2* ps = a.pS + prow0 * R_ + r;     // rank q at ps[q * R_]
    const uint16_t* po = a.pO + (prow0 * R_ + r) * D;
    const size_t po_step = (size_t)R_ * D;
    // pass 1: the merged maximum
    for (int q = 0; q < nv; ++q) M2 = fmaxf(M2, ps[(size_t)q * R_].x);
    const float M2u = (M2 == -INFINITY) ? 0.f : M2;
    const float wl = (l > 0.f) ? __builtin_amdgcn_exp2f(lse2_loc - M2u) : 0.f;
    sumw = wl;
    const float f = wl * scale_loc;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= f;
    // pass 2: weighted partials in rank (= slot) order; the weight folds in
    // the row scale 2^e
#ifndef MSA_COMBINE_UNROLL
#define MSA_COMBINE_UNROLL 2
#endif
#pragma unroll MSA_COMBINE_UNROLL
    for (int q = 0; q < nv; ++q) {
      const float2 st = ps[(size_t)q * R_];
      sumw += __builtin_amdgcn_exp2f(st.x - M2u);
      accumulate_partial_row(o, po + (size_t)q * po_step, __builtin_amdgcn_exp2f(st.x - M2u + st.y), half);
    }
    M2 = M2u;
  } else {
    sumw = (l > 0.f) ? 1.f : 0.f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= scale_loc;
    M2 = lse2_loc;
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

}  // namespace

hipError_t launch_fill_i32(int32_t* p, size_t n, int32_t value, hipStream_t st) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  fill_i32_kernel<<<dim3((unsigned)blocks), 256, 0, st>>>(p, n, value);
  return hipGetLastError();
}

hipError_t launch_prefill_main_sparse(const PrefillMainArgs& a, hipStream_t st) {
  hipError_t err = launch_fill_i32(a.cnt, (size_t)a.nlists, 0, st);
  if (err != hipSuccess) return err;
  const long n_rows = (long)a.batch * a.tc * a.G;
  const unsigned rgrid = (unsigned)((n_rows + 255) / 256);
  lists_count_kernel<<<rgrid, 256, 0, st>>>(a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int R = a.Hq / a.G;
  const int mt = kAttnRows / R;
  const int nblk = (int)((a.nlists + kScanItems - 1) / kScanItems);
  lists_scan_reduce_kernel<<<nblk, 1024, 0, st>>>(a.cnt, a.bsum, a.nlists, mt);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  lists_scan_top_kernel<<<1, 1024, 0, st>>>(a.bsum, nblk, a.n_work);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  lists_scan_final_kernel<<<nblk, 1024, 0, st>>>(a.cnt, a.bsum, a.offs, a.work, a.nlists, mt);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  lists_scatter_kernel<<<rgrid, 256, 0, st>>>(a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.max_work > 0) {
    const dim3 grid((unsigned)a.max_work);
    if (a.B == 128) kv_outer_kernel<128><<<grid, 256, 0, st>>>(a);
    else if (a.B == 64) kv_outer_kernel<64><<<grid, 256, 0, st>>>(a);
    else kv_outer_kernel<32><<<grid, 256, 0, st>>>(a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const dim3 qgrid((unsigned)((a.tc + mt - 1) / mt), a.G, a.batch);
  query_major_kernel<false><<<qgrid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_prefill_main_dense(const PrefillMainArgs& a, hipStream_t st) {
  const int R = a.Hq / a.G;
  const int mt = kAttnRows / R;
  const dim3 qgrid((unsigned)((a.tc + mt - 1) / mt), a.G, a.batch);
  query_major_kernel<true><<<qgrid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
