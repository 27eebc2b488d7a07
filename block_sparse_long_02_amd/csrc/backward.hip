// Backward of the MSA Main Branch on gfx950: dq, dk, dv of the block-sparse
// softmax attention with the selection held fixed.
//
// The selection is a top-k of block maxima, piecewise constant in the index
// inputs, and the index branch learns only through its own KL loss with its
// inputs detached [Telegram review quant_prune_distill post 751, "Метод":
// stop-gradient on the index branch; hyper.ai paper page 2606.13392, 方法
// (Method): gradient detach on the Index Branch inputs].  What remains is the
// gradient of plain softmax attention over each row's gathered tokens J
// [same page, 方法: standard scaled dot-product attention over the gathered
// Key/Value vectors].  Per (token t, head h), g = h / R, P = softmax_J(x),
// x_j = scale q[t,h].k[j,g], with dO = d loss / d out[t,h]:
//   dv[j,g] += P_j dO,   dP_j = dO . v[j,g],   Delta = dO . out[t,h]
//   dS_j = scale P_j (dP_j - Delta)
//   dq[t,h] = sum_j dS_j k[j,g],   dk[j,g] += dS_j q[t,h]
// P is rebuilt from the forward's lse: P_j = exp(x_j - lse[t,h]).
//
// Work split (block-major, the prefill's (s, g, window, block) lists, here
// holding every selected block of a row, its local block included):
//  1. bwd_delta_kernel: Delta per (token, head) row;
//  2. the lists, then each list's entries sorted by (token, slot)
//     (launch_sort_lists), so that the dk/dv sums below run in an order that
//     does not depend on how the lists were filled (their positions come
//     from integer atomics);
//  3. bwd_list_kernel: one workgroup per list.  K of the block sits in LDS,
//     each wave owns one 32-key tile (its K and V rows in registers) and
//     steps over the list's (entry, head) rows: S = Q K^T and dP = dO V^T on
//     MFMA, P and dS in the accumulator layout (one key per lane), dv += P^T dO
//     and dk += dS^T Q straight from there, and dq = dS K through LDS.  dq
//     leaves as one bf16 partial row per (entry, head), in list order; dk and
//     dv as one fp32 partial block per list.  dS is kept without the softmax
//     scale, which the two merges apply;
//  4. bwd_dq_kernel: per (token, head), the partials summed in slot order;
//  5. bwd_dkv_kernel: per (sequence, group, key block), the lists' partials
//     summed in (window) order.  No atomic touches a value.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int D = 128;  // head_dim

__device__ __forceinline__ void bwd_list_of(const PrefillMainArgs& l, long lid, int* b, int* g, int* s) {
  *b = (int)(lid % l.nbl);
  const long sg = (lid / l.nbl) / l.nwin;
  *g = (int)(sg % l.G);
  *s = (int)(sg / l.G);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// ---------------------------------------------------------------------------
// 1. Delta[s, tl, h] = dO . out over the head dimension (fp32); 16 lanes per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a) {
  const PrefillMainArgs& l = a.l;
  const long nrows = (long)l.batch * l.tc * l.Hq;
  const long row = (long)blockIdx.x * 16 + threadIdx.x / 16;
  const int part = threadIdx.x % 16;
  float acc = 0.f;
  if (row < nrows) {
    const long per_b = (long)l.tc * l.Hq;
    const size_t grow = ((size_t)(row / per_b) * l.T + l.t0) * l.Hq + (size_t)(row % per_b);
    const bf16x8 o = load_bf16x8(a.o + grow * D + part * 8);
    const bf16x8 d = load_bf16x8(a.dout + grow * D + part * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += (float)o[i] * (float)d[i];
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kWave);
  if (row < nrows && part == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// 3. Per list: dq partial rows, dk / dv partial block.
// ---------------------------------------------------------------------------
// Row tiles of 32 (entry, head) rows per wave per step: two for 128-key
// blocks (each wave owns one key tile), one otherwise (waves also split rows).
#ifndef MSA_BWD_RTW128
#define MSA_BWD_RTW128 2
#endif
// Workgroups per CU the list kernel is compiled for (register budget).
#ifndef MSA_BWD_MIN_BLOCKS
#define MSA_BWD_MIN_BLOCKS 1
#endif
template <int BS>
constexpr int bwd_rtw() { return BS == 128 ? MSA_BWD_RTW128 : 1; }

// K, q and dO rows in LDS are 256 bytes with 16-byte chunk c of row r stored
// at chunk position c ^ bwd_swz(r).  They are read one row per lane (16
// consecutive rows, one chunk: 16 distinct positions, as bwd_swz is a
// bijection of r mod 16) and through the transposing read, whose 32 lanes
// take 64 bytes (chunks 4m .. 4m+3) of 4 rows 4n .. 4n+3: the positions
// 4 (m ^ (r & 3)) + ((c & 3) ^ (r >> 2 & 3)) are 16 distinct, so all 64 banks
// are hit once.  (A padded row stride satisfies only one of the two
// patterns: 304 bytes left the transposing read 2-way conflicted.)
__device__ __forceinline__ int bwd_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// Element offset of the lane's 8-byte word for the transposing read of the
// rows row0 + 0..7 at d tile dt (row0 a multiple of 8): the lane's row is
// row0 + 4 (lane / 32) + (lane / 4) % 4, its 8 bytes the (lane % 4)-th of the
// row's 32 bytes at column 32 dt + 16 ((lane / 16) % 2).
__device__ __forceinline__ int bwd_tr_off(int lane, int row0, int dt) {
  const int r = row0 + 4 * (lane >> 5) + ((lane >> 2) & 3);
  const int c = 4 * dt + 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
  return r * D + ((c ^ bwd_swz(r)) * 8) + 4 * (lane & 1);
}

template <int BS>
struct BwdLds {
  static constexpr int KT = BS / 32;          // key tiles of the block
  static constexpr int NRG = 4 / KT;          // row groups: waves sharing a key tile
  static constexpr int RTW = bwd_rtw<BS>();   // row tiles per wave per step
  static constexpr int RT = NRG * RTW;        // row tiles per step
  static constexpr int SR = 32 * RT;          // (entry, head) rows per step
  // K, q and dO rows: 256 bytes, swizzled by chunk (bwd_swz)
  static constexpr int KR = D;                // K row stride
  static constexpr int QR = D;                // q / dO row stride
  static constexpr int DSR = BS + 8;          // dS row stride (keys)
  static constexpr int o_k = 0;
  static constexpr int o_qr = o_k + BS * KR * 2;
  static constexpr int o_or = o_qr + SR * QR * 2;
  static constexpr int o_ds = o_or + SR * QR * 2;
  static constexpr int o_lse = o_ds + SR * DSR * 2;
  static constexpr int o_del = o_lse + SR * 4;
  static constexpr int o_tok = o_del + SR * 4;
  static constexpr int loop_bytes = o_tok + SR * 4;
  // after the row loop: dk/dv accumulators of the row groups, KT * 32 keys x 128 x 2
  static constexpr int red_bytes = NRG > 1 ? KT * 32 * D * 2 * 4 : 0;
  static constexpr int bytes = loop_bytes > red_bytes ? loop_bytes : red_bytes;
  static_assert(bytes <= 160 * 1024, "LDS of one workgroup");
};

template <int BS>
__global__ __launch_bounds__(256, MSA_BWD_MIN_BLOCKS) void bwd_list_kernel(BwdArgs a) {
  using Lds = BwdLds<BS>;
  constexpr int KT = Lds::KT, NRG = Lds::NRG, RTW = Lds::RTW, RT = Lds::RT, SR = Lds::SR;
  constexpr int KR = Lds::KR, QR = Lds::QR, DSR = Lds::DSR;
  constexpr int CPT = SR * (D / 8) / 256;  // 16-byte chunks of q (and of dO) per thread per step
  __shared__ __attribute__((aligned(16))) unsigned char smem[Lds::bytes];
  bf16_t* Ks = reinterpret_cast<bf16_t*>(smem + Lds::o_k);
  bf16_t* Qr = reinterpret_cast<bf16_t*>(smem + Lds::o_qr);
  bf16_t* Or = reinterpret_cast<bf16_t*>(smem + Lds::o_or);
  bf16_t* DSr = reinterpret_cast<bf16_t*>(smem + Lds::o_ds);
  float* rlse = reinterpret_cast<float*>(smem + Lds::o_lse);
  float* rdel = reinterpret_cast<float*>(smem + Lds::o_del);
  int* rtok = reinterpret_cast<int*>(smem + Lds::o_tok);

  const PrefillMainArgs& l = a.l;
  const int w = blockIdx.x;
  if (w >= l.n_work[0]) return;
  const long lid = l.work[w].x;
  const int count = l.cnt[lid];
  int b, g, s;
  bwd_list_of(l, lid, &b, &g, &s);
  const int off = l.offs[lid];
  const int R = l.Hq / l.G;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane & 31, half = lane >> 5;
  const int kt = wave % KT, rg = wave / KT;
  const int kb = b * l.B;
  const int nkey = min(BS, l.T - kb);
  const size_t kvstride = (size_t)l.G * D;
  const bf16_t* kblk = l.k + ((size_t)s * l.T + kb) * kvstride + (size_t)g * D;
  const bf16_t* vblk = l.v + ((size_t)s * l.T + kb) * kvstride + (size_t)g * D;
  if (tid == 0) a.slot_of[lid] = w;

  // K of the block row-major in LDS (the dq product reads it through the
  // transposing LDS read) and this wave's 32-key tile of K and V in registers
  // (B operands of S = Q K^T and dP = dO V^T, k-slots = head dim).  Every load
  // is issued before the first LDS write.  Keys past the sequence read its
  // last key: every row masks them (key > t), so their P and dS are zero.
  constexpr int NKC = BS * (D / 8) / 256;  // 16-byte chunks of K per thread
  const int klast = nkey - 1;
  u32x4 kc[NKC];
#pragma unroll
  for (int i = 0; i < NKC; ++i) {
    const int c = tid + 256 * i;
    kc[i] = *reinterpret_cast<const u32x4*>(kblk + (size_t)min(c >> 4, klast) * kvstride + (c & 15) * 8);
  }
  bf16x8 kreg[D / 16], vreg[D / 16];
  {
    const int kr = min(32 * kt + col, klast);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      kreg[ks] = load_bf16x8(kblk + (size_t)kr * kvstride + 16 * ks + 8 * half);
      vreg[ks] = load_bf16x8(vblk + (size_t)kr * kvstride + 16 * ks + 8 * half);
    }
  }
#pragma unroll
  for (int i = 0; i < NKC; ++i) {
    const int c = tid + 256 * i;
    *reinterpret_cast<u32x4*>(Ks + (c >> 4) * KR + (((c & 15) ^ bwd_swz(c >> 4)) * 8)) = kc[i];
  }

  const int nr = count * R;  // (entry, head) rows of the list, row = entry position * R + head
  const __amdgpu_buffer_rsrc_t dq_rs =
      __builtin_amdgcn_make_buffer_rsrc(a.dqp + (size_t)off * R * D, (short)0, nr * D * 2, kBufferWord3);
  const int nsteps = (nr + SR - 1) / SR;
  const float c2 = l.scale_log2;

  // Staging of a step's rows, 8 lanes per row: thread tid owns rows
  // tid / 8 + 32 j (j < NRW) of every step and the 16-byte chunks tid % 8 and
  // 8 + tid % 8 of each, so that one load instruction covers 8 rows x 128
  // contiguous bytes (whole cache lines) and the 16-byte LDS writes of 8
  // lanes fill the 8 bank groups of one row (the 16-byte row padding shifts
  // each row by one group).  Rows are stored row-major; the products that run
  // over rows read them back through the transposing LDS read.  Each row's
  // (list position, head) advances by a constant each step.  With 64-row
  // steps the next step's rows are fetched while the current one computes;
  // 128-row steps are fetched in two parts in place, as an early fetch would
  // not fit next to the accumulators.  The entries that address a step's
  // rows are loaded one step earlier still.
  // No branch guards a load: rows past the list read a row that exists and
  // carry t = -1, which zeroes their P and dS; with the same memory
  // operations on every path, the wait for a step's rows need not also wait
  // for the previous step's dq stores.
  constexpr int NRW = SR / 32;                   // rows per thread per step
  static_assert(CPT == 2 * NRW, "two 16-byte chunks of each row per thread");
  constexpr int CPR = CPT <= 4 ? CPT : 4;        // chunks per part
  constexpr int NPART = CPT / CPR;
  constexpr int RPP = CPR / 2;                   // rows per part
  constexpr bool kAhead = NPART == 1;
  const int r8 = tid >> 3, c8 = tid & 7;
  // a thread's rows r8 + 32 j share r8 mod 16: its first instruction takes
  // the chunk half that puts rows r8 and r8 + 1 (one 16-lane group) on
  // different position halves
  const int hsel = ((bwd_swz(r8) >> 3) ^ r8) & 1;
  const int pos8 = c8 ^ (bwd_swz(r8) & 7);  // position of chunk c8 (+8) within its half
  const int step_q = SR / R, step_r = SR % R;  // list-position and head advance per step
  int cur_p[NRW], cur_r[NRW];                   // row of the next entry load, per row slot
  int ent[NRW], ent_r[NRW];                     // that load's result and its head
  bool ent_ok[NRW];                             // whether that row is in the list
  int row_e[NRW], row_r[NRW];                   // entry (-1: none) and head of the rows being fetched
#pragma unroll
  for (int j = 0; j < NRW; ++j) {
    cur_p[j] = (r8 + 32 * j) / R;
    cur_r[j] = (r8 + 32 * j) % R;
    ent[j] = 0;
    ent_r[j] = 0;
    ent_ok[j] = false;
    row_e[j] = -1;
    row_r[j] = 0;
  }
  u32x4 qs[CPR], os[CPR];
  // t, lse and Delta of row r8 + 32 c8 (lanes with c8 < NRW)
  float lse_v = 0.f, del_v = 0.f;
  int tok_v = -1;
  auto load_ent = [&]() {
#pragma unroll
    for (int j = 0; j < NRW; ++j) {
      ent_r[j] = cur_r[j];
      ent_ok[j] = cur_p[j] * R + cur_r[j] < nr;
      ent[j] = l.entries[off + min(cur_p[j], count - 1)];
      cur_p[j] += step_q;
      cur_r[j] += step_r;
      if (cur_r[j] >= R) {
        cur_r[j] -= R;
        ++cur_p[j];
      }
    }
  };
  auto take_ent = [&]() {
#pragma unroll
    for (int j = 0; j < NRW; ++j) {
      row_e[j] = ent_ok[j] ? ent[j] : -1;
      row_r[j] = ent_r[j];
    }
  };
  auto row_of = [&](int e, int r) {  // (sequence row of the token, head) -> row of q / dO / lse
    const int tl = e >= 0 ? e >> l.rank_bits : 0;
    return ((size_t)s * l.T + l.t0 + tl) * l.Hq + (size_t)g * R + r;
  };
  auto fetch = [&](int part0) {
#pragma unroll
    for (int jj = 0; jj < RPP; ++jj) {
      const int j = part0 * RPP + jj;
      const size_t grow = row_of(row_e[j], row_r[j]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        qs[2 * jj + h] = *reinterpret_cast<const u32x4*>(l.q + grow * D + (c8 + 8 * (h ^ hsel)) * 8);
        os[2 * jj + h] = *reinterpret_cast<const u32x4*>(a.dout + grow * D + (c8 + 8 * (h ^ hsel)) * 8);
      }
    }
    if (part0 == 0) {
      int e = row_e[0], r = row_r[0];
#pragma unroll
      for (int j = 1; j < NRW; ++j)
        if (c8 == j) {
          e = row_e[j];
          r = row_r[j];
        }
      const int tl = e >= 0 ? e >> l.rank_bits : 0;
      lse_v = l.lse[row_of(e, r)];  // scaled when stored: arithmetic on it here would wait for the step's loads
      del_v = a.delta[((size_t)s * l.tc + tl) * l.Hq + (size_t)g * R + r];
      tok_v = e >= 0 ? l.t0 + tl : -1;
    }
  };
  auto store = [&](int part0) {
#pragma unroll
    for (int jj = 0; jj < RPP; ++jj) {
      const int row = r8 + 32 * (part0 * RPP + jj);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // chunk c8 + 8 (h ^ hsel) sits at position (c8 + 8 (h ^ hsel)) ^ bwd_swz(row)
        const int pos = pos8 + 8 * ((h ^ hsel) ^ (bwd_swz(r8) >> 3));
        *reinterpret_cast<u32x4*>(Qr + row * QR + pos * 8) = qs[2 * jj + h];
        *reinterpret_cast<u32x4*>(Or + row * QR + pos * 8) = os[2 * jj + h];
      }
    }
    if (part0 == 0 && c8 < NRW) {
      const int row = r8 + 32 * c8;
      rlse[row] = lse_v * kLog2e;
      rdel[row] = del_v;
      rtok[row] = tok_v;
    }
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  load_ent();
  if (kAhead) {
    take_ent();
    fetch(0);
    load_ent();
    // Each later step's rows are waited for with the previous step's RT * 4
    // dq stores issued after them.  The same number of stores here, at an
    // offset past the resource (dropped by the range check), gives the path
    // into the loop the same count, so the wait need not cover the stores.
#pragma unroll
    for (int i = 0; i < RT * 4; ++i)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, dq_rs, nr * D * 2 + 16 * i, 0, 0);
  }
  for (int step = 0; step < nsteps; ++step) {
    __syncthreads();  // the previous step's LDS reads are done (and Ks is written)
    if (kAhead) {
      store(0);
    } else {
      take_ent();
#pragma unroll
      for (int part0 = 0; part0 < NPART; ++part0) {
        fetch(part0);
        store(part0);
      }
      load_ent();
    }
    __syncthreads();
    if (kAhead && step + 1 < nsteps) {
      take_ent();
      fetch(0);
      load_ent();
    }

    const int j = kb + 32 * kt + col;
    const int fcol = bwd_swz(col);  // rows r0 + col, r0 a multiple of 32
    // dS rows keep each 16-key group in the order 0-3, 8-11, 4-7, 12-15 (bits
    // 2 and 3 of the key swapped), the k-slot order of K read through the
    // transposing LDS read: lane half h then reads its 8 keys contiguously
    const int dscol = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
    // S = Q K^T and dP = dO V^T of all the wave's row tiles first: the next
    // tile's products run on the matrix unit while the vector unit takes the
    // current tile's exps and dS
    f32x16 S[RTW], dP[RTW];
#pragma unroll
    for (int u = 0; u < RTW; ++u) {
      const int r0 = (rg * RTW + u) * 32;
      S[u] = f32x16{};
      dP[u] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int qo = (r0 + col) * QR + (((2 * ks + half) ^ fcol) * 8);
        S[u] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(Qr + qo), kreg[ks], S[u]);
        dP[u] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(Or + qo), vreg[ks], dP[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < RTW; ++u) {
      const int r0 = (rg * RTW + u) * 32;
      // the lane's 16 rows are 4 runs of 4: their t, lse and Delta in 16-byte reads
      i32x4 tk[4];
      f32x4 lv[4], dl[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int rr = r0 + 8 * q4 + 4 * half;
        tk[q4] = *reinterpret_cast<const i32x4*>(rtok + rr);
        lv[q4] = *reinterpret_cast<const f32x4*>(rlse + rr);
        dl[q4] = *reinterpret_cast<const f32x4*>(rdel + rr);
      }
      // lane: key j of its tile, rows r0 + 8*(i/4) + 4*half + (i%4)
      bf16x8 p8[2], d8[2];
      uint32_t dsbits[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // rows past the list carry t = -1, so one compare masks them and the
        // keys after t in the local block (exp of a masked entry is finite and dropped)
        const float e = __builtin_amdgcn_exp2f(S[u][i] * c2 - lv[i / 4][i % 4]);
        const float p = j <= tk[i / 4][i % 4] ? e : 0.f;
        const float ds = p * (dP[u][i] - dl[i / 4][i % 4]);  // the softmax scale is applied in the merges
        p8[i / 8][i % 8] = (__bf16)p;
        d8[i / 8][i % 8] = (__bf16)ds;
        dsbits[i] = bf16_bits(ds);
      }
      // dS rows in 4-byte words: lanes 2m and 2m+1 hold adjacent keys (the
      // column swap keeps bit 0), so for rows i, i+1 the even lane writes
      // row i's pair and the odd lane row i+1's, each taking the other half
      // from its neighbour (a DPP swap of adjacent lanes)
      const bool odd = col & 1;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const uint32_t lo = dsbits[i], hi = dsbits[i + 1];
        const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? lo : hi), 0xB1, 0xF, 0xF, false);
        const int row = r0 + 8 * (i / 4) + 4 * half + (i % 4) + (odd ? 1 : 0);
        const uint32_t word = odd ? ((hi << 16) | recv) : ((recv << 16) | lo);
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(DSr) + row * DSR + 32 * kt + (dscol & ~1)) = word;
      }
      // dv[key][d] += P^T dO, dk[key][d] += dS^T Q over this row tile (k-slots =
      // rows: {0-3, 8-11} + 4 half of each 16-row slice, as in p8 / d8)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int o0 = bwd_tr_off(lane, r0 + 16 * ks, dt), o1 = bwd_tr_off(lane, r0 + 16 * ks + 8, dt);
          const bf16x8 ob = join_bf16x4(lds_read_tr16(Or + o0), lds_read_tr16(Or + o1));
          const bf16x8 qb = join_bf16x4(lds_read_tr16(Qr + o0), lds_read_tr16(Qr + o1));
          dv[dt] = mfma32x32x16(p8[ks], ob, dv[dt]);
          dk[dt] = mfma32x32x16(d8[ks], qb, dk[dt]);
        }
      }
    }
    __syncthreads();  // dS rows of the step complete
    // dq^T[d][row] = sum over the block's keys of K^T[d][key] dS^T[key][row]:
    // the wave's RT (row tile, d tile) pairs share one row tile, whose dS
    // operands are read once; each d tile's K^T operands are read before its
    // products.  Each lane ends with one row and 4 runs of 4 consecutive d,
    // stored as 8-byte bf16 groups.  Unrolled (where registers allow) so that
    // the compiler can count the stores when the next step waits for its rows.
    static_assert(4 % RT == 0, "a wave's pairs share one row tile");
    const int rt2 = (wave * RT) >> 2;
    bf16x8 dsb[BS / 16];
#pragma unroll
    for (int ks = 0; ks < BS / 16; ++ks)
      dsb[ks] = *reinterpret_cast<const bf16x8*>(DSr + (rt2 * 32 + col) * DSR + 16 * ks + 8 * half);
    constexpr int kPairUnroll = RT <= 2 ? RT : 1;
#pragma unroll kPairUnroll
    for (int ii = 0; ii < RT; ++ii) {
      const int dt = (wave * RT + ii) & 3;
      bf16x8 ka[BS / 16];
#pragma unroll
      for (int ks = 0; ks < BS / 16; ++ks) {
        ka[ks] = join_bf16x4(lds_read_tr16(Ks + bwd_tr_off(lane, 16 * ks, dt)),
                             lds_read_tr16(Ks + bwd_tr_off(lane, 16 * ks + 8, dt)));
      }
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < BS / 16; ++ks) acc = mfma32x32x16(ka[ks], dsb[ks], acc);
      // rows past the list fall outside the resource and their stores are dropped
      const int rho = step * SR + rt2 * 32 + col;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 v;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = (__bf16)acc[4 * i4 + u];
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), dq_rs,
                                              (rho * D + 32 * dt + 4 * half + 8 * i4) * 2, 0, 0);
      }
    }
  }

  // row groups of one key tile add up in a fixed order (group 0 + 1 + ...)
  if constexpr (NRG > 1) {
    float* red = reinterpret_cast<float*>(smem);
    for (int rr = 1; rr < NRG; ++rr) {
      __syncthreads();
      if (rg == rr) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            red[(((kt * 2 + 0) * 4 + dt) * 16 + i) * 64 + lane] = dk[dt][i];
            red[(((kt * 2 + 1) * 4 + dt) * 16 + i) * 64 + lane] = dv[dt][i];
          }
      }
      __syncthreads();
      if (rg == 0) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            dk[dt][i] += red[(((kt * 2 + 0) * 4 + dt) * 16 + i) * 64 + lane];
            dv[dt][i] += red[(((kt * 2 + 1) * 4 + dt) * 16 + i) * 64 + lane];
          }
      }
    }
  }
  if (rg == 0) {
    float* pk = a.part + (size_t)w * 2 * BS * D;
    float* pv = pk + (size_t)BS * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kr = 32 * kt + 8 * (i / 4) + 4 * half + (i % 4);
        pk[(size_t)kr * D + 32 * dt + col] = dk[dt][i];
        pv[(size_t)kr * D + 32 * dt + col] = dv[dt][i];
      }
  }
}

// ---------------------------------------------------------------------------
// 4. dq[s, t, h] = sum over the row's entries, in slot order, of its partials.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  const PrefillMainArgs& l = a.l;
  const long nrows = (long)l.batch * l.tc * l.Hq;
  const long x = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = x >> 4;
  const int part = (int)(x & 15);
  if (row >= nrows) return;
  const int R = l.Hq / l.G;
  const long per_b = (long)l.tc * l.Hq;
  const int s = (int)(row / per_b);
  const int tl = (int)((row % per_b) / l.Hq);
  const int h = (int)(row % l.Hq);
  const int g = h / R, r = h - g * R;
  const long rowg = ((long)s * l.tc + tl) * l.G + g;
  const int nv = l.rinfo[rowg] & 0x3fffffff;
  const int32_t* pos = l.epos + (size_t)rowg * l.KS;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // slots in groups of 8 whose position and partial loads are issued together
  for (int q0 = 0; q0 < nv; q0 += 8) {
    int pq[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) pq[u] = pos[min(q0 + u, nv - 1)];
    bf16x8 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = load_bf16x8(a.dqp + ((size_t)pq[u] * R + r) * D + part * 8);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q0 + u < nv)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += (float)v[u][i];
  }
  const float sc = l.scale_log2 * kLn2;
  float* dst = a.dq + (((size_t)s * l.T + l.t0 + tl) * l.Hq + h) * D + part * 8;
  *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0] * sc, acc[1] * sc, acc[2] * sc, acc[3] * sc};
  *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4] * sc, acc[5] * sc, acc[6] * sc, acc[7] * sc};
}

// ---------------------------------------------------------------------------
// 5. dk, dv of a key block of one (sequence, group): its lists' partials in
//    window order; added onto earlier query chunks.  The block's dk and dv
//    elements are split over kDkvSplit workgroups; the lists' counts are read
//    in parallel and walked in order by every thread.
// ---------------------------------------------------------------------------
constexpr int kDkvSplit = 4;

template <int BS>
__global__ __launch_bounds__(256) void bwd_dkv_kernel(BwdArgs a) {
  constexpr int PER = 2 * BS * D / 256 / kDkvSplit;  // elements per thread (dk block, then dv block)
  __shared__ int slot[256];
  const PrefillMainArgs& l = a.l;
  const int b = blockIdx.x, g = blockIdx.y % l.G, s = blockIdx.y / l.G, z = blockIdx.z;
  const int kb = b * l.B;
  const int nkey = min(BS, l.T - kb);
  const int u0 = z * (2 * BS * D / kDkvSplit);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int base = 0; base < l.nwin; base += 256) {
    __syncthreads();
    {
      const int x = base + (int)threadIdx.x;
      const size_t lid = (((size_t)s * l.G + g) * l.nwin + x) * l.nbl + b;
      slot[threadIdx.x] = x < l.nwin && l.cnt[lid] > 0 ? a.slot_of[lid] : -1;
    }
    __syncthreads();
    const int n = min(256, l.nwin - base);
    for (int i = 0; i < n; ++i) {
      const int sl = slot[i];
      if (sl < 0) continue;
      const float* part = a.part + (size_t)sl * 2 * BS * D + u0;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += part[threadIdx.x + 256 * e];
    }
  }
  const float sc = l.scale_log2 * kLn2;  // dk carries the softmax scale, dv does not
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int u = u0 + threadIdx.x + 256 * e;
    const bool is_k = u < BS * D;
    const int uu = is_k ? u : u - BS * D;
    const int kr = uu / D, dd = uu % D;
    if (kr < nkey) {
      float* dst = (is_k ? a.dk : a.dv) + (((size_t)s * l.T + kb + kr) * l.G + g) * D + dd;
      const float v = is_k ? acc[e] * sc : acc[e];
      *dst = a.accumulate ? *dst + v : v;
    }
  }
}

}  // namespace

// mt for the lists' work list: large enough that every non-empty list is one item
constexpr int kBwdListTile = 1 << 28;

hipError_t launch_prefill_backward(const BwdArgs& a, hipStream_t st) {
  const PrefillMainArgs& l = a.l;
  const long nrows = (long)l.batch * l.tc * l.Hq;
  prof_mark(st, MSA_STAGE_BWD_PREP);
  bwd_delta_kernel<<<(unsigned)((nrows + 15) / 16), 256, 0, st>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if ((err = launch_block_lists(l, kBwdListTile, st)) != hipSuccess) return err;
  if ((err = launch_sort_lists(l, st)) != hipSuccess) return err;
  prof_mark(st, MSA_STAGE_BWD_LISTS);
  if (l.max_work > 0) {
    if (l.B == 128) bwd_list_kernel<128><<<(unsigned)l.max_work, 256, 0, st>>>(a);
    else if (l.B == 64) bwd_list_kernel<64><<<(unsigned)l.max_work, 256, 0, st>>>(a);
    else bwd_list_kernel<32><<<(unsigned)l.max_work, 256, 0, st>>>(a);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  prof_mark(st, MSA_STAGE_BWD_MERGE);
  bwd_dq_kernel<<<(unsigned)((nrows * 16 + 255) / 256), 256, 0, st>>>(a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const dim3 grid((unsigned)((l.T + l.B - 1) / l.B), (unsigned)(l.G * l.batch), (unsigned)kDkvSplit);
  if (l.B == 128) bwd_dkv_kernel<128><<<grid, 256, 0, st>>>(a);
  else if (l.B == 64) bwd_dkv_kernel<64><<<grid, 256, 0, st>>>(a);
  else bwd_dkv_kernel<32><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
