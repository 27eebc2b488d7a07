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
//    each wave owns a few consecutive blocks.
// 2. the shared top-k kernel selects the blocks (local block forced).
// 3. decode_attn_kernel: one workgroup per (sequence, group, work item); a
//    work item is one selected block (sparse) or a run of consecutive blocks
//    (dense), attended with online softmax; it writes a normalised partial
//    output and its base-2 log-sum-exp per head.
// 4. decode_combine_kernel merges the work items of each (sequence, group) in
//    fixed order (no atomics) and rounds to bf16.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int D = 128;
constexpr int kDecMaxR = 16;     // query heads per group handled by the decode kernels
constexpr int kDecBlocksPerWave = 2;
constexpr int kDecKeyTile = 64;

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

// One (s, g, work item) per workgroup of 256 threads.
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeMainArgs a) {
  __shared__ float qs[kDecMaxR][D];
  __shared__ __attribute__((aligned(16))) bf16_t Kt[kDecKeyTile][D + 8];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[kDecKeyTile][D];
  __shared__ float P[kDecMaxR][kDecKeyTile];
  __shared__ float m_run[kDecMaxR], l_run[kDecMaxR], alpha_s[kDecMaxR];

  const int j = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int R = a.Hq / a.G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int len = min(max(a.lens[s], 1), a.Lmax);
  const int t = len - 1;
  const int L = t / a.B;

  int blk_lo, blk_hi;  // inclusive block range of this work item
  if (a.dense) {
    blk_lo = j * a.blocks_per_split;
    blk_hi = min(blk_lo + a.blocks_per_split - 1, L);
  } else {
    const int e = a.bidx[((size_t)s * a.G + g) * a.topk + j];
    blk_lo = e;
    blk_hi = (e >= 0 && e <= L) ? e : e - 1;  // empty when not a visible block
  }
  const size_t prow0 = (((size_t)s * a.G + g) * a.nsplit + j) * R;
  if (blk_lo > blk_hi || blk_lo < 0) {
    for (int i = tid; i < R; i += 256) a.pS[prow0 + i] = -INFINITY;
    for (int i = tid; i < R * D; i += 256) a.pO[prow0 * D + i] = 0.f;
    return;
  }
  const int k_lo = blk_lo * a.B;
  const int k_hi = min((blk_hi + 1) * a.B, len) - 1;

  for (int i = tid; i < R * D; i += 256) {
    const int r = i / D, d = i % D;
    qs[r][d] = (float)__builtin_bit_cast(__bf16, a.q[((size_t)s * a.Hq + g * R + r) * D + d]);
  }
  if (tid < kDecMaxR) {
    m_run[tid] = -INFINITY;
    l_run[tid] = 0.f;
  }
  float o[kDecMaxR / 2];
#pragma unroll
  for (int i = 0; i < kDecMaxR / 2; ++i) o[i] = 0.f;
  const int od = tid & (D - 1), oh = tid >> 7;  // PV ownership: d, heads oh + 2i

  const size_t kvstride = (size_t)a.G * D;
  const bf16_t* kseq = a.k + (size_t)s * a.Lmax * kvstride + (size_t)g * D;
  const bf16_t* vseq = a.v + (size_t)s * a.Lmax * kvstride + (size_t)g * D;
  const float c = a.scale_log2;

  for (int kb = k_lo; kb <= k_hi; kb += kDecKeyTile) {
    const int nvalid = min(kDecKeyTile, k_hi + 1 - kb);
    __syncthreads();
    for (int ci = tid; ci < kDecKeyTile * (D / 8); ci += 256) {
      const int key = ci >> 4, part = ci & 15;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (key < nvalid) {
        kv = *reinterpret_cast<const uint4*>(kseq + (size_t)(kb + key) * kvstride + part * 8);
        vv = *reinterpret_cast<const uint4*>(vseq + (size_t)(kb + key) * kvstride + part * 8);
      }
      *reinterpret_cast<uint4*>(&Kt[key][part * 8]) = kv;
      *reinterpret_cast<uint4*>(&Vs[key][part * 8]) = vv;
    }
    __syncthreads();
    // scores: key = lane, heads wave + 4i
    for (int r = wave; r < R; r += 4) {
      float acc = 0.f;
      const bf16_t* kr = &Kt[lane][0];
#pragma unroll 8
      for (int d8 = 0; d8 < D / 8; ++d8) {
        const uint4 kk = *reinterpret_cast<const uint4*>(kr + d8 * 8);
        const uint32_t w[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc += qs[r][d8 * 8 + 2 * e] * __uint_as_float(w[e] << 16);
          acc += qs[r][d8 * 8 + 2 * e + 1] * __uint_as_float(w[e] & 0xffff0000u);
        }
      }
      const float x = (lane < nvalid) ? acc * c : -INFINITY;
      const float tmx = wave_max(x);
      const float m_old = m_run[r];
      const float m_new = fmaxf(m_old, tmx);
      const float p = __builtin_amdgcn_exp2f(x - m_new);
      const float ps = wave_sum(p);
      P[r][lane] = p;
      if (lane == 0) {
        const float al = __builtin_amdgcn_exp2f(m_old - m_new);
        alpha_s[r] = al;
        l_run[r] = l_run[r] * al + ps;
        m_run[r] = m_new;
      }
    }
    __syncthreads();
    // P.V: thread owns d = od for heads oh + 2i
#pragma unroll
    for (int i = 0; i < kDecMaxR / 2; ++i) {
      const int r = oh + 2 * i;
      if (r < R) {
        float acc = o[i] * alpha_s[r];
        for (int key = 0; key < nvalid; ++key)
          acc += P[r][key] * (float)__builtin_bit_cast(__bf16, Vs[key][od]);
        o[i] = acc;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kDecMaxR / 2; ++i) {
    const int r = oh + 2 * i;
    if (r < R) a.pO[(prow0 + r) * D + od] = o[i] / l_run[r];
  }
  if (tid < R) a.pS[prow0 + tid] = m_run[tid] + __log2f(l_run[tid]);
}

__global__ __launch_bounds__(128) void decode_combine_kernel(DecodeMainArgs a) {
  const int g = blockIdx.x, s = blockIdx.y;
  const int R = a.Hq / a.G;
  const int d = threadIdx.x;
  for (int r = 0; r < R; ++r) {
    const size_t base = ((size_t)s * a.G + g) * a.nsplit;
    float M2 = -INFINITY;
    for (int j = 0; j < a.nsplit; ++j) M2 = fmaxf(M2, a.pS[(base + j) * R + r]);
    const float Mu = (M2 == -INFINITY) ? 0.f : M2;
    float sw = 0.f, acc = 0.f;
    for (int j = 0; j < a.nsplit; ++j) {
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

hipError_t launch_decode_main(const DecodeMainArgs& a, hipStream_t st) {
  decode_attn_kernel<<<dim3(a.nsplit, a.G, a.batch), 256, 0, st>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  decode_combine_kernel<<<dim3(a.G, a.batch), 128, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace msa
