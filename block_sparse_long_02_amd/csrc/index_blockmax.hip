// Index Branch of MSA on gfx950: fused index scoring + Block-Max pooling.
//
// Definition [hyper.ai paper page 2606.13392, 方法 (Method); Telegram review
// quant_prune_distill post 751, "Метод"]: every (query token t, GQA group g)
// row scores each visible key j with the raw dot product
// idx_q[t,g] . idx_k[j] (one index-key head per layer, shared by all groups),
// and the scores are max-pooled over aligned blocks of B keys.
//
// Only blocks 0..L(t)-1 are produced: the local block L(t) is always kept by
// the selection and its score is never compared, and every earlier block is
// fully visible (all its keys are < L(t)*B <= t), so no causal mask is needed.
// The T x T score matrix is never stored: each 32x32 MFMA tile of scores is
// max-reduced in registers and only one float per (row, block) leaves the CU.
//
// Prefill kernel layout: a workgroup owns 128*NT consecutive (t, g) rows (4
// waves x NT column tiles of 32 rows, idx_q kept in registers as the MFMA B
// operand; NT = 3 for index_dim 128, 4 for 64) and streams idx_k one block at
// a time through double-buffered LDS as the A operand, so each idx_k byte
// fetched feeds 128*NT rows and each A operand read from LDS feeds NT MFMAs.
// Workgroups are issued longest-first (latest tokens have the most blocks).
// Beside S, each row gets the maximum of every run of 16 of its candidate
// blocks (a superblock), so the top-k can skip the runs that cannot hold a
// selected block.
//
// A second kernel takes the Index Branch in one pass (scores, Block-Max and
// the Top-k with the forced blocks) for topk <= 17, keeping each row's best
// candidates in registers instead of writing S.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

// NT 32-row column tiles per wave, 4 waves: 128 * NT (t, g) rows per
// workgroup; NT is as large as the register file allows without spills.
template <int DI>
constexpr int idx_nt() { return DI == 128 ? 3 : 4; }

__device__ __forceinline__ void shift_in(f32x4& lo, f32x4& hi, float v) {
  lo[0] = lo[1]; lo[1] = lo[2]; lo[2] = lo[3]; lo[3] = hi[0];
  hi[0] = hi[1]; hi[1] = hi[2]; hi[2] = hi[3]; hi[3] = v;
}

// WITH_SM: also write the superblock maxima SM (chunks with rows of more
// than kSbMinCandidates candidate blocks).
template <int DI, int B, int NT, bool WITH_SM>
__global__ __launch_bounds__(256, 2) void index_blockmax_prefill_kernel(
    const bf16_t* __restrict__ idx_q, const bf16_t* __restrict__ idx_k, float* __restrict__ S,
    int T, int G, int t0, int tc, int s_stride, float* __restrict__ SM, int sm_stride, int n_tiles) {
  constexpr int ROWS = 128 * NT;
  constexpr int KPAD = DI + 8;            // LDS row stride (bf16): +16 B against bank conflicts
  constexpr int KSTEPS = DI / 16;         // MFMA k-steps per 32x32 tile
  constexpr int CPR = DI / 8;             // 16-byte chunks per idx_k row
  constexpr int NCH = B * CPR;            // 16-byte chunks per block
  constexpr int MAXCH = (NCH + 255) / 256;  // staging chunks per thread
  constexpr int KTILES = B / 32;
  __shared__ __attribute__((aligned(16))) bf16_t kbuf[2][B * KPAD];

  const int s = blockIdx.y;
  const int tile = n_tiles - 1 - (int)blockIdx.x;   // longest rows first
  const int rows_chunk = tc * G;
  const int r0 = tile * ROWS;
  const int r_last = min(r0 + ROWS, rows_chunk) - 1;
  const int nblk = (t0 + r_last / G) / B;  // candidate blocks needed by the last row
  if (nblk <= 0) return;                   // uniform across the workgroup

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;

  // B operands: idx_q rows of this wave's NT 32-row column tiles.
  bf16x8 qop[NT][KSTEPS];
  int row_idx[NT], row_L[NT];
  bool row_ok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = r0 + wave * 32 * NT + nt * 32 + col;
    row_idx[nt] = r;
    row_ok[nt] = r < rows_chunk;
    row_L[nt] = (t0 + r / G) / B;  // the row's candidate blocks are 0 .. row_L - 1
    const bf16_t* qp = idx_q + ((size_t)s * T * G + (size_t)t0 * G + (size_t)(row_ok[nt] ? r : 0)) * DI;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qop[nt][ks] = row_ok[nt] ? load_bf16x8(qp + 16 * ks + 8 * half) : zero_bf16x8();
  }

  const bf16_t* kseq = idx_k + (size_t)s * T * DI;

  // Staging: each thread moves up to MAXCH 16-byte chunks of a B x DI block.
  u32x4 stg[MAXCH];
#define MSA_IDX_GLOAD(BLK)                                                               \
  {                                                                                      \
    const u32x4* src_ = reinterpret_cast<const u32x4*>(kseq + (size_t)(BLK) * B * DI);   \
    _Pragma("unroll") for (int i = 0; i < MAXCH; ++i) {                                  \
      const int c_ = tid + i * 256;                                                      \
      if (NCH % 256 == 0 || c_ < NCH) stg[i] = src_[c_];                                 \
    }                                                                                    \
  }
#define MSA_IDX_LSTORE(BUF)                                                              \
  {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < MAXCH; ++i) {                                  \
      const int c_ = tid + i * 256;                                                      \
      if (NCH % 256 == 0 || c_ < NCH)                                                    \
        *reinterpret_cast<u32x4*>(&kbuf[BUF][(c_ / CPR) * KPAD + (c_ % CPR) * 8]) = stg[i]; \
    }                                                                                    \
  }

  MSA_IDX_GLOAD(0);
  MSA_IDX_LSTORE(0);
  __syncthreads();

  // Block maxima are written in groups of 16 consecutive blocks, 64 bytes
  // per row: both halves of the wave hold every row maximum (after the
  // cross-half shuffle), so half h keeps blocks 8h..8h+7 of the group (two
  // float4, filled as a shift register: each of the half's blocks enters at
  // the end, so after its eighth the oldest sits first) and each row
  // receives 64 contiguous bytes per group.
  f32x4 sb[NT], sb2[NT];
  float smx[NT];   // running superblock maximum over the row's candidate blocks
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    sb[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    sb2[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    smx[nt] = -INFINITY;
  }

  for (int b = 0; b < nblk; ++b) {
    const int cur = b & 1;
    if (b + 1 < nblk) MSA_IDX_GLOAD(b + 1);

    float mx[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) mx[nt] = -INFINITY;
    // One key tile at a time keeps NT accumulators live (no spills).  The A
    // operand of k-step ks + 2 is read right after the products of k-step ks
    // issue (two operand registers in turn; the last two k-steps of a key
    // tile read the first two of the next), and scheduling groups keep that
    // order, so each read has two k-steps of products to land.
    const bf16_t* abase = &kbuf[cur][col * KPAD + 8 * half];
    bf16x8 aop[2];
    aop[0] = *reinterpret_cast<const bf16x8*>(abase);
    aop[1] = *reinterpret_cast<const bf16x8*>(abase + 16);
#pragma unroll 1
    for (int kt = 0; kt < KTILES; ++kt) {
      f32x16 acc[NT];
      const bf16_t* arow = abase + kt * 32 * KPAD;
      const bf16_t* anext = abase + min(kt + 1, KTILES - 1) * 32 * KPAD;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8 a = aop[ks & 1];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma32x32x16(a, qop[nt][ks], ks == 0 ? f32x16{} : acc[nt]);
        aop[ks & 1] = *reinterpret_cast<const bf16x8*>(ks + 2 < KSTEPS ? arow + 16 * (ks + 2)
                                                                        : anext + 16 * (ks + 2 - KSTEPS));
      }
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);   // the k-step's products
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // then the read two k-steps ahead
      }
      // a chain of three-input maxima: one VALU instruction per two scores
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx[nt] = fmaxf(fmaxf(mx[nt], acc[nt][i]), acc[nt][i + 1]);
    }
    const int slot16 = b & 15;
    const bool mine = (slot16 >> 3) == half;  // this half keeps block b
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float v = fmaxf(mx[nt], __shfl_xor(mx[nt], 32, kWave));
      if (mine) shift_in(sb[nt], sb2[nt], v);
      if (WITH_SM && b < row_L[nt]) smx[nt] = fmaxf(smx[nt], v);
    }
    // a superblock is one 16-block store group: its maximum leaves with it
    if (WITH_SM && (b % kSuperBlock == kSuperBlock - 1 || b == nblk - 1)) {  // uniform
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (row_ok[nt] && half == 0)
          SM[((size_t)s * rows_chunk + (size_t)row_idx[nt]) * sm_stride + b / kSuperBlock] = smx[nt];
        smx[nt] = -INFINITY;
      }
    }
    // At the group's end every float4 is stored; at the row range's end only
    // the float4s holding blocks of the last group (those starting at or
    // before block b), so every store stays below round_up(nblk, 4) <= s_stride.
    if (slot16 == 15 || b == nblk - 1) {  // uniform
      // a last, partial group: shift this half's entries into their places
      for (int j = slot16 + 1; j < 16; ++j)
        if ((j >> 3) == half) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) shift_in(sb[nt], sb2[nt], 0.f);
        }
      const int first = 8 * half;         // group offset of this half's first float4
      const bool w1 = slot16 == 15 || first <= slot16;
      const bool w2 = slot16 == 15 || first + 4 <= slot16;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (row_ok[nt]) {
          float* dst = S + ((size_t)s * rows_chunk + (size_t)row_idx[nt]) * s_stride + (b & ~15) + first;
          if (w1) *reinterpret_cast<f32x4*>(dst) = sb[nt];
          if (w2) *reinterpret_cast<f32x4*>(dst + 4) = sb2[nt];
        }
      }
    }

    if (b + 1 < nblk) MSA_IDX_LSTORE(cur ^ 1);
    __syncthreads();
  }
#undef MSA_IDX_GLOAD
#undef MSA_IDX_LSTORE
}

// ---------------------------------------------------------------------------
// Building blocks of the one-pass kernel below: the staging and scoring of
// index_blockmax_prefill_kernel, written as functions.  That kernel keeps its
// own inline copy: its instruction schedule was measured as it stands, and
// the compiler schedules the function form differently.
// ---------------------------------------------------------------------------

// LDS row stride of a staged idx_k block (bf16): +16 B against bank conflicts
template <int DI>
constexpr int kpad() { return DI + 8; }

// Staging of one B x DI idx_k block by 256 threads: MAXCH 16-byte chunks per
// thread, global -> registers (issued a block ahead) -> LDS.
template <int DI, int B>
struct KStage {
  static constexpr int CPR = DI / 8;                  // 16-byte chunks per idx_k row
  static constexpr int NCH = B * CPR;                 // 16-byte chunks per block
  static constexpr int MAXCH = (NCH + 255) / 256;     // chunks per thread
  u32x4 stg[MAXCH];
  __device__ __forceinline__ void load(const bf16_t* kseq, int blk, int tid) {
    const u32x4* src = reinterpret_cast<const u32x4*>(kseq + (size_t)blk * B * DI);
#pragma unroll
    for (int i = 0; i < MAXCH; ++i) {
      const int c = tid + i * 256;
      if (NCH % 256 == 0 || c < NCH) stg[i] = src[c];
    }
  }
  __device__ __forceinline__ void store(bf16_t* kb, int tid) const {
#pragma unroll
    for (int i = 0; i < MAXCH; ++i) {
      const int c = tid + i * 256;
      if (NCH % 256 == 0 || c < NCH) *reinterpret_cast<u32x4*>(&kb[(c / CPR) * kpad<DI>() + (c % CPR) * 8]) = stg[i];
    }
  }
};

// The maxima over one staged key block of this lane's half of each of its NT
// rows' scores (the other half of a row sits in lane ^ 32): the block's 32-key
// tiles against the idx_q operands of the wave's NT column tiles, each 32x32
// tile of scores max-reduced as soon as it is complete.
template <int DI, int B, int NT>
__device__ __forceinline__ void block_half_max(const bf16_t* kb, const bf16x8 (&qop)[NT][DI / 16], int col,
                                               int half, float (&mx)[NT]) {
  constexpr int KPAD = kpad<DI>();
  constexpr int KSTEPS = DI / 16;         // MFMA k-steps per 32x32 tile
  constexpr int KTILES = B / 32;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) mx[nt] = -INFINITY;
  // One key tile at a time keeps NT accumulators live (no spills).  The A
  // operand of k-step ks + 2 is read right after the products of k-step ks
  // issue (two operand registers in turn; the last two k-steps of a key
  // tile read the first two of the next), and scheduling groups keep that
  // order, so each read has two k-steps of products to land.
  const bf16_t* abase = kb + col * KPAD + 8 * half;
  bf16x8 aop[2];
  aop[0] = *reinterpret_cast<const bf16x8*>(abase);
  aop[1] = *reinterpret_cast<const bf16x8*>(abase + 16);
#pragma unroll 1
  for (int kt = 0; kt < KTILES; ++kt) {
    f32x16 acc[NT];
    const bf16_t* arow = abase + kt * 32 * KPAD;
    const bf16_t* anext = abase + min(kt + 1, KTILES - 1) * 32 * KPAD;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const bf16x8 a = aop[ks & 1];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma32x32x16(a, qop[nt][ks], ks == 0 ? f32x16{} : acc[nt]);
      aop[ks & 1] = *reinterpret_cast<const bf16x8*>(ks + 2 < KSTEPS ? arow + 16 * (ks + 2)
                                                                      : anext + 16 * (ks + 2 - KSTEPS));
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);   // the k-step's products
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // then the read two k-steps ahead
    }
    // a chain of three-input maxima: one VALU instruction per two scores
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx[nt] = fmaxf(fmaxf(mx[nt], acc[nt][i]), acc[nt][i + 1]);
  }
}

// The idx_q rows of a wave's NT 32-row column tiles as MFMA B operands (zero
// for rows past the chunk).
template <int DI, int NT>
__device__ __forceinline__ void load_q_operands(const bf16_t* idx_q, int s, int T, int G, int t0, int rows_chunk,
                                                int r_first, int col, int half, bf16x8 (&qop)[NT][DI / 16]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = r_first + nt * 32 + col;
    const bool ok = r < rows_chunk;
    const bf16_t* qp = idx_q + ((size_t)s * T * G + (size_t)t0 * G + (size_t)(ok ? r : 0)) * DI;
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks) qop[nt][ks] = ok ? load_bf16x8(qp + 16 * ks + 8 * half) : zero_bf16x8();
  }
}

// ---------------------------------------------------------------------------
// The Index Branch in one pass: the scoring loop above, and after each key
// block every row offers its block maximum to a running list of its best
// `want` candidates (want = m - 1 with m = min(k, L(t) + 1), one less with
// the forced sink), so neither the score table nor a top-k pass is needed.
//
// A row's list has 16 slots, eight in each of the two lanes that hold the
// row (lane and lane ^ 32); slot 8 * half + p sits in lkey/lblk[nt][p].  Keys
// are order_key() of the block maxima.  While the list fills, block b takes
// slot b - c0 (c0 = 1 with the sink, else 0); once it is full, a block enters
// only with a key strictly above the weakest entry (lowest key, then highest
// block), which it replaces.  Blocks arrive in ascending order, so an equal
// key never displaces an earlier block: the list ends as the row's best
// `want` blocks under (score descending, block ascending), the selection
// rule of the two-pass path.  A row's list always fills, since want never
// exceeds its number of candidate blocks.  The weakest entry is kept in
// wkey/wblk and recomputed (both lanes, one shuffle) only after a list
// changes; a wave ballot skips the update when no row of the wave takes the
// block.  At the end each lane writes its entries at their rank in block
// order, after block 0 with the sink, and the local block L(t) closes the
// row's m entries; -1 fills the rest.
// ---------------------------------------------------------------------------
template <int DI, int B, int NT>
__global__ __launch_bounds__(256, 2) void index_topk_one_pass_kernel(
    const bf16_t* __restrict__ idx_q, const bf16_t* __restrict__ idx_k, int32_t* __restrict__ bidx,
    long bidx_rows, int bidx_t_off, int T, int G, int t0, int tc, int k, int sink, int n_tiles) {
  constexpr int ROWS = 128 * NT;
  __shared__ __attribute__((aligned(16))) bf16_t kbuf[2][B * kpad<DI>()];

  const int s = blockIdx.y;
  const int tile = n_tiles - 1 - (int)blockIdx.x;   // longest rows first
  const int rows_chunk = tc * G;
  const int r0 = tile * ROWS;
  const int r_last = min(r0 + ROWS, rows_chunk) - 1;
  const int nblk = (t0 + r_last / G) / B;  // candidate blocks needed by the last row

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;

  bf16x8 qop[NT][DI / 16];
  load_q_operands<DI, NT>(idx_q, s, T, G, t0, rows_chunk, r0 + wave * 32 * NT, col, half, qop);
  int row_idx[NT], row_L[NT], row_c0[NT], row_want[NT];
  bool row_ok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = r0 + wave * 32 * NT + nt * 32 + col;
    row_idx[nt] = r;
    row_ok[nt] = r < rows_chunk;
    const int L = (t0 + (row_ok[nt] ? r : r_last) / G) / B;
    const int m = k < L + 1 ? k : L + 1;
    const bool fs = sink && L >= 1 && m >= 2;
    row_L[nt] = L;
    row_c0[nt] = fs ? 1 : 0;
    row_want[nt] = m - 1 - (fs ? 1 : 0);
  }

  uint32_t lkey[NT][8];
  int lblk[NT][8];
  uint32_t wkey[NT];
  int wblk[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      lkey[nt][p] = 0xffffffffu;   // an empty slot is never the weakest
      lblk[nt][p] = -1;
    }
    wkey[nt] = 0u;
    wblk[nt] = -1;
  }
  // the weakest entry among the row's first `want` slots, over both lanes
  auto weakest = [&](int nt) {
    uint32_t k0 = 0xffffffffu;
    int b0 = -1;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const bool valid = 8 * half + p < row_want[nt];
      const bool weaker = lkey[nt][p] < k0 || (lkey[nt][p] == k0 && lblk[nt][p] > b0);
      if (valid && weaker) {
        k0 = lkey[nt][p];
        b0 = lblk[nt][p];
      }
    }
    const uint32_t k1 = (uint32_t)__shfl_xor((int)k0, 32, kWave);
    const int b1 = __shfl_xor(b0, 32, kWave);
    const bool other = k1 < k0 || (k1 == k0 && b1 > b0);
    wkey[nt] = other ? k1 : k0;
    wblk[nt] = other ? b1 : b0;
  };

  const bf16_t* kseq = idx_k + (size_t)s * T * DI;
  KStage<DI, B> stage;
  if (nblk > 0) {  // uniform
    stage.load(kseq, 0, tid);
    stage.store(kbuf[0], tid);
  }
  __syncthreads();

  for (int b = 0; b < nblk; ++b) {
    const int cur = b & 1;
    if (b + 1 < nblk) stage.load(kseq, b + 1, tid);

    float mx[NT];
    block_half_max<DI, B, NT>(kbuf[cur], qop, col, half, mx);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float v = fmaxf(mx[nt], __shfl_xor(mx[nt], 32, kWave));
      const int c0 = row_c0[nt], want = row_want[nt];
      const bool cand = b >= c0 && b < row_L[nt] && want > 0;
      const int slot = b - c0;                 // while the list fills: its next free slot
      const bool fill = cand && slot < want;
      const uint32_t key = order_key(v);
      const bool beat = cand && !fill && key > wkey[nt];
      if (__builtin_amdgcn_ballot_w64(fill || beat) != 0) {  // uniform: some row of the wave takes block b
        const bool mine_fill = fill && (slot >> 3) == half;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          // the weakest entry's block is unique within the row's list
          const bool put = (mine_fill && (slot & 7) == p) || (beat && lblk[nt][p] == wblk[nt]);
          lkey[nt][p] = put ? key : lkey[nt][p];
          lblk[nt][p] = put ? b : lblk[nt][p];
        }
        if (__builtin_amdgcn_ballot_w64((fill && slot == want - 1) || beat) != 0) weakest(nt);
      }
    }

    if (b + 1 < nblk) stage.store(kbuf[cur ^ 1], tid);
    __syncthreads();
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    int oblk[8];   // the other lane's slots of the same row
#pragma unroll
    for (int p = 0; p < 8; ++p) oblk[p] = __shfl_xor(lblk[nt][p], 32, kWave);
    if (!row_ok[nt]) continue;
    const int r = row_idx[nt];
    const int t = t0 + r / G, g = r % G;
    const int L = row_L[nt], want = row_want[nt], c0 = row_c0[nt];
    const int m = want + 1 + c0;
    int32_t* out = bidx + ((size_t)((long)s * bidx_rows + (t - bidx_t_off)) * G + g) * (size_t)k;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      if (8 * half + p < want) {
        const int me = lblk[nt][p];
        int rank = c0;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          rank += (8 * half + q < want && lblk[nt][q] < me) ? 1 : 0;
          rank += (8 * (1 - half) + q < want && oblk[q] < me) ? 1 : 0;
        }
        out[rank] = me;
      }
    }
    if (half == 0) {
      if (c0) out[0] = 0;
      out[m - 1] = L;
      for (int j = m; j < k; ++j) out[j] = -1;
    }
  }
}

}  // namespace

hipError_t launch_index_blockmax_prefill(const uint16_t* idx_q, const uint16_t* idx_k, float* S,
                                         int batch, int T, int G, int di, int B, int t0, int tc,
                                         int s_stride, float* SM, int sm_stride, hipStream_t st) {
  const long rows = (long)tc * G;
  const int rows_per_wg = 128 * (di == 128 ? idx_nt<128>() : idx_nt<64>());
  const int n_tiles = (int)((rows + rows_per_wg - 1) / rows_per_wg);
  dim3 grid(n_tiles, batch);
#define MSA_IDX_LAUNCH(DI_, B_)                                                                         \
  do {                                                                                                  \
    if (SM != nullptr)                                                                                  \
      index_blockmax_prefill_kernel<DI_, B_, idx_nt<DI_>(), true><<<grid, 256, 0, st>>>(                \
          idx_q, idx_k, S, T, G, t0, tc, s_stride, SM, sm_stride, n_tiles);                             \
    else                                                                                                \
      index_blockmax_prefill_kernel<DI_, B_, idx_nt<DI_>(), false><<<grid, 256, 0, st>>>(               \
          idx_q, idx_k, S, T, G, t0, tc, s_stride, SM, sm_stride, n_tiles);                             \
  } while (0)
  if (di == 128) {
    if (B == 128) MSA_IDX_LAUNCH(128, 128);
    else if (B == 64) MSA_IDX_LAUNCH(128, 64);
    else MSA_IDX_LAUNCH(128, 32);
  } else {
    if (B == 128) MSA_IDX_LAUNCH(64, 128);
    else if (B == 64) MSA_IDX_LAUNCH(64, 64);
    else MSA_IDX_LAUNCH(64, 32);
  }
#undef MSA_IDX_LAUNCH
  return hipGetLastError();
}

hipError_t launch_index_topk_one_pass(const uint16_t* idx_q, const uint16_t* idx_k, int32_t* bidx, long bidx_rows,
                                      int bidx_t_off, int batch, int T, int G, int di, int B, int k, bool sink,
                                      int t0, int tc, hipStream_t st) {
  if (k < 1 || k > kOnePassMaxTopk) return hipErrorInvalidValue;
  // two row tiles per wave: the running lists take the registers of the third
  constexpr int NT = 2;
  const long rows = (long)tc * G;
  const int n_tiles = (int)((rows + 128 * NT - 1) / (128 * NT));
  dim3 grid(n_tiles, batch);
#define MSA_ONE_PASS_LAUNCH(DI_, B_)                                                                   \
  index_topk_one_pass_kernel<DI_, B_, NT><<<grid, 256, 0, st>>>(idx_q, idx_k, bidx, bidx_rows, bidx_t_off, \
                                                                T, G, t0, tc, k, sink ? 1 : 0, n_tiles)
  if (di == 128) {
    if (B == 128) MSA_ONE_PASS_LAUNCH(128, 128);
    else if (B == 64) MSA_ONE_PASS_LAUNCH(128, 64);
    else MSA_ONE_PASS_LAUNCH(128, 32);
  } else {
    if (B == 128) MSA_ONE_PASS_LAUNCH(64, 128);
    else if (B == 64) MSA_ONE_PASS_LAUNCH(64, 64);
    else MSA_ONE_PASS_LAUNCH(64, 32);
  }
#undef MSA_ONE_PASS_LAUNCH
  return hipGetLastError();
}

}  // namespace msa
