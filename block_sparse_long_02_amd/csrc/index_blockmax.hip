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

}  // namespace msa
