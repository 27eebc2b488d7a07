// MSA decode step on gfx950: one new query token per sequence against its
// caches [hyper.ai paper page 2606.13392, 一句话总结 (summary) and 方法
// (Method): the same Index Branch and Main Branch, reported for decode at 1M
// context].  The query sits at position len-1 of a cache of len tokens.
//
// 1. decode_index_kernel streams the index-key cache once (the dominant
//    bytes of the step) and produces the Block-Max score of every candidate
//    block 0..L-1 for all G groups at once: each 16-key x 32-dim slice is the
//    MFMA A operand and the G index queries form the B operand (columns), so
//    every idx_k byte read feeds all groups.  Grid: sequences x block ranges;
//    each wave owns one block (at 8 x 1M, two blocks per wave streamed the
//    cache 6 % slower: fewer, longer waves leave more of it idle between
//    their load bursts).
// 2. the shared top-k kernel selects the blocks (local block forced).
// 3. decode_attn_kernel: 8 waves per (sequence, group) share its selected
//    blocks (or, in dense mode, runs of consecutive blocks), attend them on
//    MFMA with online softmax and merge in LDS in fixed order (no atomics).
// 4. only when one workgroup cannot hold all work items of a (sequence,
//    group) (dense mode, large top-k), decode_combine_kernel merges the
//    workgroups' normalised partials in fixed order.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int D = 128;
constexpr int kDecBlocksPerWave = 1;

template <int DI, int BS>
__global__ __launch_bounds__(256) void decode_index_kernel(const bf16_t* __restrict__ idx_q,
                                                           const bf16_t* __restrict__ idx_k,
                                                           const int32_t* __restrict__ lens,
                                                           float* __restrict__ S, int Lmax, int G,
                                                           int s_stride) {
  constexpr int KSTEPS = DI / 32;
  constexpr int KT = BS / 16;
  const int s = blockIdx.y;
  const int len = min(max(lens[s], 1), Lmax);
  const int L = (len - 1) / BS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b0 = (blockIdx.x * 4 + wave) * kDecBlocksPerWave;
  if (b0 >= L) return;
  const int b1 = min(b0 + kDecBlocksPerWave, L);
  const int c16 = lane & 15, q4 = lane >> 4;
  const int ntiles = (G + 15) / 16;

  const bf16_t* kseq = idx_k + (size_t)s * Lmax * DI;
  for (int nt = 0; nt < ntiles; ++nt) {
    const int g = nt * 16 + c16;
    bf16x8 qop[KSTEPS];
    const bf16_t* qp = idx_q + ((size_t)s * G + g) * DI;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qop[ks] = (g < G) ? load_bf16x8(qp + 32 * ks + 8 * q4) : zero_bf16x8();

    for (int b = b0; b < b1; ++b) {
      bf16x8 av[KT][KSTEPS];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const bf16_t* kr = kseq + ((size_t)b * BS + kt * 16 + c16) * DI + 8 * q4;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) av[kt][ks] = load_bf16x8(kr + 32 * ks);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        f32x4 acc = {};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) acc = mfma16x16x32(av[kt][ks], qop[ks], acc);
        mx = fmaxf(mx, fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      if (q4 == 0 && g < G) S[((size_t)s * G + g) * s_stride + b] = mx;
    }
  }
}

// ---------------------------------------------------------------------------
// Decode attention.  A workgroup of kDecAttnWaves waves owns (s, g, part x)
// and work items part*W*ipw .. ; wave w takes items x*W*ipw + w + W*i,
// i < ipw.  A work item is a part of a selected block (sparse / given; 64
// keys) or a run of blocks_per_split consecutive blocks (dense).  Each wave
// attends its keys in sub-tiles of up to 64 with online softmax: S^T =
// K.Q^T on MFMA with the K rows loaded straight into the A operand; the V
// rows go unchanged into the wave's own LDS area and come back as the P.V
// operand through the transposing LDS read.  The waves then merge in LDS in
// fixed order; with one part per (s, g) the merge writes the output, else a
// normalised partial that decode_combine_kernel merges.
// ---------------------------------------------------------------------------
constexpr int kDecAttnWaves = 8;
// (s, g) rows below which a decode step splits each row over several
// workgroups: one per CU of the 256 on MI355X.
#ifndef MSA_DEC_FILL_ROWS
#define MSA_DEC_FILL_ROWS 256
#endif
constexpr long kDecFillRows = MSA_DEC_FILL_ROWS;

template <int BS>
struct DecTile {
  static constexpr int NK = BS < 64 ? BS : 64;   // keys per sub-tile
  static constexpr int VR = D + 8;               // row stride (bf16) of the staged key-major V tile
  static constexpr int VT_BYTES = NK * VR * 2;   // per wave
  static constexpr int CMB_BYTES = (64 * 64 + 2 * 64) * 4;
  static constexpr int AREA = VT_BYTES > CMB_BYTES ? VT_BYTES : CMB_BYTES;
};

__device__ __forceinline__ void dec_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int BS>
__global__ __launch_bounds__(kDecAttnWaves * 64) void decode_attn_kernel(DecodeMainArgs a, int ipw, int nparts) {
  using Tl = DecTile<BS>;
  constexpr int NK = Tl::NK, KTL = NK / 32;
  __shared__ __attribute__((aligned(16))) unsigned char dec_smem[kDecAttnWaves * Tl::AREA];

  const int x = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int R = a.Hq / a.G;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, col = lane & 31, half = lane >> 5;
  unsigned char* area = dec_smem + (size_t)wave * Tl::AREA;
  bf16_t* Vt = reinterpret_cast<bf16_t*>(area);  // key-major V sub-tile, row stride Tl::VR
  const int len = min(max(a.lens[s], 1), a.Lmax);
  const int t = len - 1;
  const int L = t / a.B;
  const float c = a.scale_log2;
  const int tro = tr_lane_off(lane, Tl::VR);  // transposing-read offset of this lane (row-major V)

  // B operand: Q^T, column = head (col < R)
  const bool hv = col < R;
  bf16x8 qop[D / 16];
  {
    const bf16_t* qp = a.q + ((size_t)s * a.Hq + g * R + (hv ? col : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qop[ks] = hv ? load_bf16x8(qp + 16 * ks + 8 * half) : zero_bf16x8();
  }
  const size_t kvstride = (size_t)a.G * D;
  const bf16_t* kseq = a.k + (size_t)s * a.Lmax * kvstride + (size_t)g * D;
  const bf16_t* vseq = a.v + (size_t)s * a.Lmax * kvstride + (size_t)g * D;

  float m = -INFINITY, l = 0.f;
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};

  for (int i = 0; i < ipw; ++i) {
    const int item = x * kDecAttnWaves * ipw + wave + kDecAttnWaves * i;
    if (item >= a.nsplit) break;
    int k_lo, k_end;  // keys [k_lo, k_end) of this item
    if (a.dense) {
      const int blk_lo = item * a.blocks_per_split;
      const int blk_hi = min(blk_lo + a.blocks_per_split - 1, L);
      k_lo = blk_lo * a.B;
      k_end = min((blk_hi + 1) * a.B, len);
    } else {
      // item = selected entry * sub + part: part `part` of the block's keys
      const int e = a.bidx[((size_t)s * a.G + g) * a.topk + item / a.sub];
      if (e < 0 || e > L) continue;  // -1 padding
      const int span = a.B / a.sub;
      k_lo = e * a.B + (item % a.sub) * span;
      k_end = min(k_lo + span, len);
    }
    if (k_lo >= k_end) continue;
    for (int kb = k_lo; kb < k_end; kb += NK) {
      // K rows as MFMA A operands, V units for the transposed LDS tile
      bf16x8 kop[KTL][D / 16];
#pragma unroll
      for (int kt = 0; kt < KTL; ++kt) {
        const int key = kb + kt * 32 + col;
        const bool kv = key < k_end;
        const bf16_t* kr = kseq + (size_t)(kv ? key : kb) * kvstride + 8 * half;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) kop[kt][ks] = kv ? load_bf16x8(kr + 16 * ks) : zero_bf16x8();
      }
      // V rows as they are in memory, 16 bytes per lane per load; the P.V
      // operands are read back transposed by the gfx950 transposing LDS read
      constexpr int VP = NK * (D / 8) / 64;  // 16-byte pieces per lane
      u32x4 vv[VP];
#pragma unroll
      for (int u = 0; u < VP; ++u) {
        const int p = lane + 64 * u;
        const int key = kb + (p >> 4);
        vv[u] = key < k_end ? *reinterpret_cast<const u32x4*>(vseq + (size_t)key * kvstride + (p & 15) * 8)
                            : u32x4{0u, 0u, 0u, 0u};
      }
      dec_wave_sync();  // previous sub-tile's V reads are done
#pragma unroll
      for (int u = 0; u < VP; ++u) {
        const int p = lane + 64 * u;
        *reinterpret_cast<u32x4*>(Vt + (p >> 4) * Tl::VR + (p & 15) * 8) = vv[u];
      }
      dec_wave_sync();

      f32x16 sacc[KTL];
#pragma unroll
      for (int kt = 0; kt < KTL; ++kt) {
        sacc[kt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) sacc[kt] = mfma32x32x16(kop[kt][ks], qop[ks], sacc[kt]);
      }
      float tmx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KTL; ++kt)
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
          const int key = kb + kt * 32 + 8 * (ii / 4) + 4 * half + (ii % 4);
          sacc[kt][ii] = key < k_end ? sacc[kt][ii] : -INFINITY;
          tmx = fmaxf(tmx, sacc[kt][ii]);
        }
      tmx = fmaxf(tmx, __shfl_xor(tmx, 32, kWave));
      const float m_new = fmaxf(m, tmx);  // finite: the sub-tile has >= 1 key
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
      const float muc = m_new * c;
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < KTL; ++kt)
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
          const float p = __builtin_amdgcn_exp2f(sacc[kt][ii] * c - muc);
          sacc[kt][ii] = p;
          ps += p;
        }
      ps += __shfl_xor(ps, 32, kWave);
      l = l * alpha + ps;
      m = m_new;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) oacc[dt][ii] *= alpha;
#pragma unroll
        for (int kt = 0; kt < KTL; ++kt) {
          bf16x8 p0, p1;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p0[e] = (__bf16)sacc[kt][e];
            p1[e] = (__bf16)sacc[kt][8 + e];
          }
          // keys kt*32 + {0-3, 8-11} + 4 half (p0) and + 16 (p1), at column d
          const bf16_t* vb = Vt + kt * 32 * Tl::VR + dt * 32 + tro;
          oacc[dt] = mfma32x32x16(join_bf16x4(lds_read_tr16(vb), lds_read_tr16(vb + 8 * Tl::VR)), p0, oacc[dt]);
          oacc[dt] = mfma32x32x16(join_bf16x4(lds_read_tr16(vb + 16 * Tl::VR), lds_read_tr16(vb + 24 * Tl::VR)), p1,
                                  oacc[dt]);
        }
      }
    }
  }

  // merge the waves (fixed order) through LDS
  __syncthreads();
  float* cm = reinterpret_cast<float*>(area);  // [64 values][64 lanes], then m[64], l[64]
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) cm[(dt * 16 + ii) * 64 + lane] = oacc[dt][ii];
  cm[64 * 64 + lane] = m;
  cm[64 * 64 + 64 + lane] = l;
  __syncthreads();
  // wave w merges value slots [8w, 8w+8) of every lane
  float M = -INFINITY;
  for (int w = 0; w < kDecAttnWaves; ++w) {
    const float* cw = reinterpret_cast<const float*>(dec_smem + (size_t)w * Tl::AREA);
    M = fmaxf(M, cw[64 * 64 + lane]);
  }
  const float Mu = (M == -INFINITY) ? 0.f : M;
  float sw = 0.f, acc[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) acc[v] = 0.f;
  for (int w = 0; w < kDecAttnWaves; ++w) {
    const float* cw = reinterpret_cast<const float*>(dec_smem + (size_t)w * Tl::AREA);
    const float mw = cw[64 * 64 + lane];
    const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mw - Mu) * c);
    sw += f * cw[64 * 64 + 64 + lane];
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] += f * cw[(wave * 8 + v) * 64 + lane];
  }
  if (!hv) return;
  const int h = g * R + col;
  const float inv = sw > 0.f ? 1.0f / sw : 0.f;
  const float lse2 = sw > 0.f ? Mu * c + __log2f(sw) : -INFINITY;
  // value slot (dt, ii) = wave*8 + v  ->  d = 32 dt + 8 (ii/4) + 4 half + ii%4
  if (nparts == 1) {
    bf16_t* dst = a.out + ((size_t)s * a.Hq + h) * D;
#pragma unroll
    for (int v = 0; v < 8; v += 4) {
      const int slot = wave * 8 + v, dt = slot / 16, ii = slot % 16;
      bf16x4 o4;
#pragma unroll
      for (int j = 0; j < 4; ++j) o4[j] = (__bf16)(acc[v + j] * inv);
      *reinterpret_cast<bf16x4*>(dst + 32 * dt + 8 * (ii / 4) + 4 * half) = o4;
    }
    if (a.lse != nullptr && wave == 0 && half == 0) a.lse[(size_t)s * a.Hq + h] = lse2 * kLn2;
  } else {
    const size_t prow = (((size_t)s * a.G + g) * nparts + x) * R + col;
    float* dst = a.pO + prow * D;
#pragma unroll
    for (int v = 0; v < 8; v += 4) {
      const int slot = wave * 8 + v, dt = slot / 16, ii = slot % 16;
      *reinterpret_cast<f32x4*>(dst + 32 * dt + 8 * (ii / 4) + 4 * half) =
          f32x4{acc[v] * inv, acc[v + 1] * inv, acc[v + 2] * inv, acc[v + 3] * inv};
    }
    if (wave == 0 && half == 0) a.pS[prow] = lse2;
  }
}

// Merges the nparts partials of one (s, g, head r) in fixed order; one
// workgroup per (r, g, s), one thread per output dimension.  The loads of a
// pass do not depend on each other, so four are kept in flight.
__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeMainArgs a, int nparts) {
  const int r = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int R = a.Hq / a.G;
  const int d = threadIdx.x;
  const size_t base = ((size_t)s * a.G + g) * nparts;
  float M2 = -INFINITY;
#pragma unroll 4
  for (int j = 0; j < nparts; ++j) M2 = fmaxf(M2, a.pS[(base + j) * R + r]);
  const float Mu = (M2 == -INFINITY) ? 0.f : M2;
  float sw = 0.f, acc = 0.f;
#pragma unroll 4
  for (int j = 0; j < nparts; ++j) {
    const size_t prow = (base + j) * R + r;
    const float w = __builtin_amdgcn_exp2f(a.pS[prow] - Mu);
    sw += w;
    acc += w * a.pO[prow * D + d];
  }
  const int h = g * R + r;
  const float ov = (sw > 0.f) ? acc / sw : 0.f;
  a.out[((size_t)s * a.Hq + h) * D + d] = __builtin_bit_cast(bf16_t, (__bf16)ov);
  if (a.lse != nullptr && d == 0)
    a.lse[(size_t)s * a.Hq + h] = (sw > 0.f) ? (Mu + __log2f(sw)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_index_blockmax_decode(const uint16_t* idx_q, const uint16_t* idx_k,
                                        const int32_t* lens, float* S, int batch, int Lmax, int G,
                                        int di, int B, int s_stride, hipStream_t st) {
  const int nbmax = (Lmax + B - 1) / B;
  const int per_wg = 4 * kDecBlocksPerWave;
  const dim3 grid((unsigned)((nbmax + per_wg - 1) / per_wg), batch);
#define MSA_DEC_IDX(DI_, BS_)                                                                     \
  decode_index_kernel<DI_, BS_><<<grid, 256, 0, st>>>(idx_q, idx_k, lens, S, Lmax, G, s_stride)
  if (di == 128) {
    if (B == 128) MSA_DEC_IDX(128, 128);
    else if (B == 64) MSA_DEC_IDX(128, 64);
    else MSA_DEC_IDX(128, 32);
  } else {
    if (B == 128) MSA_DEC_IDX(64, 128);
    else if (B == 64) MSA_DEC_IDX(64, 64);
    else MSA_DEC_IDX(64, 32);
  }
#undef MSA_DEC_IDX
  return hipGetLastError();
}

// Work items per wave and workgroups per (s, g) for nsplit items over
// `rows` = batch * G (s, g) rows.
void decode_partition(int nsplit, long rows, int* ipw, int* nparts) {
  // Up to 4 items per wave keep one workgroup per (s, g) when there are
  // enough rows to fill the chip; with fewer than one row per CU, or long
  // dense runs, each wave takes one item and the combine kernel merges the
  // workgroups of a row.
  if (nsplit <= kDecAttnWaves * 4 && rows >= kDecFillRows) {
    *ipw = (nsplit + kDecAttnWaves - 1) / kDecAttnWaves;
    *nparts = 1;
  } else {
    *ipw = 1;
    *nparts = (nsplit + kDecAttnWaves - 1) / kDecAttnWaves;
  }
}

hipError_t launch_decode_main(const DecodeMainArgs& a, hipStream_t st) {
  int ipw, nparts;
  decode_partition(a.nsplit, (long)a.batch * a.G, &ipw, &nparts);
  const dim3 grid(nparts, a.G, a.batch);
  prof_mark(st, MSA_STAGE_DECODE_ATTN);
#define MSA_DEC_ATTN(BS_)                                                                          \
  decode_attn_kernel<BS_><<<grid, kDecAttnWaves * 64, 0, st>>>(a, ipw, nparts)
  // the kernel's tile shape follows the keys of one work item
  const int span = a.dense ? a.B : a.B / a.sub;
  if (span == 128) MSA_DEC_ATTN(128);
  else if (span == 64) MSA_DEC_ATTN(64);
  else MSA_DEC_ATTN(32);
#undef MSA_DEC_ATTN
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nparts == 1) return err;
  prof_mark(st, MSA_STAGE_DECODE_COMBINE);
  decode_combine_kernel<<<dim3(a.Hq / a.G, a.G, a.batch), 128, 0, st>>>(a, nparts);
  return hipGetLastError();
}

}  // namespace msa
