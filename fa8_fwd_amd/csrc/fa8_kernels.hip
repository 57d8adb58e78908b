// gfx950 (MI355X) kernels of the FP8 attention forward.
//
// One kernel template serves the full forward pass (one query head per workgroup, 128 query
// rows) and the split-KV decode pass (the q heads of one KV head packed into 32 rows). Per KV
// tile of 64 keys, each wave of 32 query rows does:
//   S^T = K Q^T          FP8 MFMA 32x32x64 (E4M3 x E4M3 -> fp32); rows = keys, cols = queries,
//                        so one lane owns one query row (the page's "QK^T" step)
//   scale, mask          x = S * c, c = softmax_scale * dq * dk * log2(e)  (q/k descales folded
//                        into the softmax scale: "Native FP8 ... for Hopper", Design, Descales)
//   row max, lazy rescale: the stored max m moves to the tile max only when it grows by more
//                        than TAU = 0.75 <= log2(448) - 8 ("fp8 on the sheared forward",
//                        Correctness fix), so the biased P never exceeds the E4M3 range
//   P = exp2(x - m + 8)  one FMA feeds v_exp_f32 (the fused exp2 bias; 2^8 pre-scale of P:
//                        Design, "P in FP8"); P cast to E4M3 (RNE); row sum l in fp32 over
//                        the rounded P, the values the PV product actually uses
//   O_t = V^T P^T        FP8 MFMA from zero for this tile only, then O = alpha*O + O_t in fp32
//                        (Design, "Two-level PV accumulation")
// and at the end O *= dv / l, LSE = ln2 * (m + log2 l - 8) (bias removed from the LSE).
//
// Layout choices for gfx950 (measured MFMA lane layouts; see the design notes):
//  * MFMA operands: lane L holds row L%32 of A (col L%32 of B) and 32 bytes of the contraction
//    dimension, lanes 0-31 one half and 32-63 the other; A and B use the same byte<->k order, so
//    any k permutation applied to both operands leaves the product unchanged.
//  * The S^T accumulator of a 32-key block puts key 8*(r/4) + 4*(L/32) + r%4 in register r of
//    lane L. Cast to E4M3 in register order, those bytes are already the B operand (P^T) of the
//    PV MFMA; the A operand (V^T) is read with the same key permutation by ds_read_b64_tr_b8
//    from the row-major V tile (no separate transpose pass over V).
//  * K and V tiles are row-major in LDS with a per-row XOR swizzle of their 16-byte chunks so
//    the 32 row reads of an operand hit distinct banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa8_internal.h"

namespace fa8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

#define FA8_LDS __attribute__((address_space(3)))

constexpr float kTau = 0.75f;    // lazy-rescale slack in log2 units, <= log2(448) - 8
constexpr float kBias = 8.0f;    // P is computed as 2^(x - m + 8)
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ v16f mfma_32x32x64_fp8(v8i a, v8i b, v16f c) {
  // format codes 0/0 = E4M3 for both operands; zero scale operands select the unscaled MFMA
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Position of 16-byte chunk `ch` of a row holding NCH chunks, XOR-swizzled by `sv` inside the
// largest aligned power-of-two group of chunks that fits in the row.
template <int NCH>
__device__ __forceinline__ int swz(int ch, int sv) {
  if ((ch | 7) < NCH) return ch ^ (sv & 7);
  if ((ch | 3) < NCH) return ch ^ (sv & 3);
  if ((ch | 1) < NCH) return ch ^ (sv & 1);
  return ch;
}
__device__ __forceinline__ int k_sv(int row) { return row & 7; }
// V is read 8 rows at a time by ds_read_b64_tr_b8 with row sets {0-3, 8-11} + 4h (+16r):
// bits 0, 1 and 3 of the row make those 8 rows land in 8 different chunks.
__device__ __forceinline__ int v_sv(int row) { return (row & 3) | ((row >> 1) & 4); }

__device__ __forceinline__ v4i ld_global16(const uint8_t* ptr) {
  return *reinterpret_cast<const v4i*>(ptr);
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t f16_bits(float x) {
  _Float16 h = (_Float16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
// Four consecutive outputs as 4 x 16-bit in 8 bytes.
__device__ __forceinline__ void store4_half(void* dst, float a, float b, float c, float d, bool fp16) {
  uint32_t lo, hi;
  if (fp16) {
    lo = f16_bits(a) | (f16_bits(b) << 16);
    hi = f16_bits(c) | (f16_bits(d) << 16);
  } else {
    lo = bf16_rne_bits(a) | (bf16_rne_bits(b) << 16);
    hi = bf16_rne_bits(c) | (bf16_rne_bits(d) << 16);
  }
  v2i v = {(int)lo, (int)hi};
  *reinterpret_cast<v2i*>(dst) = v;
}

__device__ __forceinline__ float load_descale(const float* p, int64_t sb, int64_t sh, int b, int kvh) {
  return p ? p[(int64_t)b * sb + (int64_t)kvh * sh] : 1.0f;
}

template <int D, int DV, int NW, bool PACKED>
__global__ void __launch_bounds__(NW * 64)
fa8_attn_kernel(const KParams p) {
  constexpr int BN = kKvTile;
  constexpr int NT = NW * 64;
  constexpr int BM = NW * 32;
  constexpr int KS = (D + 63) / 64;       // k-steps of the QK MFMA (d padded to 64)
  constexpr int NB = DV / 32;             // 32-wide dv blocks of the PV MFMA
  constexpr int KCH = D / 16, VCH = DV / 16;
  constexpr int KTILE = BN * D, VTILE = BN * DV, STAGE = KTILE + VTILE;
  constexpr int KCHUNKS = BN * KCH, VCHUNKS = BN * VCH;
  constexpr int KPT = (KCHUNKS + NT - 1) / NT, VPT = (VCHUNKS + NT - 1) / NT;
  static_assert(DV % 32 == 0 && D % 32 == 0, "head dims must be multiples of 32");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hgrp = lane >> 5, lrow = lane & 31;
  const int b = blockIdx.z;
  const int g = p.g;

  int kvh, mblock, split = 0, hq_fixed = 0;
  if constexpr (PACKED) {
    kvh = blockIdx.x / p.nmb;
    mblock = blockIdx.x - kvh * p.nmb;
    split = blockIdx.y;
  } else {
    hq_fixed = blockIdx.y;
    kvh = hq_fixed / g;
    // causal: heaviest (last) row blocks first
    mblock = p.causal ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  }

  const int q0 = p.cu_q ? p.cu_q[b] : 0;
  const int sq = p.cu_q ? p.cu_q[b + 1] - q0 : p.max_sq;
  int sk;
  if (p.used_k) sk = p.used_k[b];
  else if (p.cu_k) sk = p.cu_k[b + 1] - p.cu_k[b];
  else sk = p.max_sk;

  const int rows_total = PACKED ? sq * g : sq;
  const int rb0 = mblock * BM;
  if (rb0 >= rows_total) return;               // uniform: no valid row in this block
  const int rb1 = min(rb0 + BM, rows_total) - 1;
  const int i_first = PACKED ? rb0 / g : rb0;
  const int i_last = PACKED ? rb1 / g : rb1;

  const int shift = sk - sq;                   // bottom-right alignment: i' = i + sk - sq
  auto lo_of = [&](int i) { return p.wl >= 0 ? max(0, i + shift - p.wl) : 0; };
  auto hi_of = [&](int i) { return p.wr >= 0 ? min(sk, i + shift + p.wr + 1) : sk; };

  int wg_lo = lo_of(i_first), wg_hi = hi_of(i_last);       // union of the rows' key ranges
  int full_lo = lo_of(i_last), full_hi = hi_of(i_first);   // keys visible to every row
  if (wg_hi <= wg_lo) { wg_lo = 0; wg_hi = 0; }
  if constexpr (PACKED) {
    // split s covers granules [g0 + s*n/S, g0 + (s+1)*n/S) of the block's granule range
    const int g0 = wg_lo / BN, g1 = (wg_hi + BN - 1) / BN, n = g1 - g0;
    const int s0 = g0 + (int)(((int64_t)split * n) / p.nsplit);
    const int s1 = g0 + (int)(((int64_t)(split + 1) * n) / p.nsplit);
    wg_lo = max(wg_lo, s0 * BN);
    wg_hi = min(wg_hi, s1 * BN);
    full_lo = max(full_lo, s0 * BN);
    full_hi = min(full_hi, s1 * BN);
  }
  const int t_begin = wg_lo / BN;
  const int t_end = wg_hi > wg_lo ? (wg_hi + BN - 1) / BN : t_begin;

  // this lane's query row
  const int ridx = rb0 + wave * 32 + lrow;
  const bool valid = ridx <= rb1;
  const int qi = PACKED ? ridx / g : ridx;
  const int qh = PACKED ? kvh * g + (ridx - qi * g) : hq_fixed;
  int my_lo = 0, my_hi = 0;
  if (valid) {
    my_lo = max(lo_of(qi), wg_lo);
    my_hi = min(hi_of(qi), wg_hi);
  }

  const float dq = load_descale(p.dq, p.dq_sb, p.dq_sh, b, kvh);
  const float dk = load_descale(p.dk, p.dk_sb, p.dk_sh, b, kvh);
  const float dvs = load_descale(p.dv, p.dv_sb, p.dv_sh, b, kvh);
  const float c = p.scale_log2 * dq * dk;

  // Q rows as the B operand of S^T = K Q^T: lane holds d-bytes [64ks + 32*hgrp, +32)
  v8i qop[KS];
  {
    const uint8_t* qrow = p.q + (p.cu_q ? (int64_t)(q0 + qi) * p.q_rs : (int64_t)b * p.q_bs + (int64_t)qi * p.q_rs) +
                          (int64_t)qh * p.q_hs;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const int off = ks * 64 + hgrp * 32;
      v4i a = {0, 0, 0, 0}, a2 = {0, 0, 0, 0};
      if (valid && off < D) {
        a = ld_global16(qrow + off);
        a2 = ld_global16(qrow + off + 16);
      }
      qop[ks] = (v8i){a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
    }
  }

  // K/V row addressing
  const bool paged = p.page_shift >= 0;
  const int32_t* trow = paged ? p.table + (int64_t)b * p.table_stride : nullptr;
  const int64_t kbase = paged ? (int64_t)kvh * p.k_hs
                              : (p.cu_k ? (int64_t)p.cu_k[b] * p.k_rs : (int64_t)b * p.k_bs) + (int64_t)kvh * p.k_hs;
  const int64_t vbase = paged ? (int64_t)kvh * p.v_hs
                              : (p.cu_k ? (int64_t)p.cu_k[b] * p.v_rs : (int64_t)b * p.v_bs) + (int64_t)kvh * p.v_hs;
  const int pmask = paged ? (1 << p.page_shift) - 1 : 0;
  auto koff = [&](int j) -> int64_t {
    if (paged) {
      const int64_t page = trow[j >> p.page_shift];
      return page * p.k_bs + (int64_t)(j & pmask) * p.k_rs + kbase;
    }
    return kbase + (int64_t)j * p.k_rs;
  };
  auto voff = [&](int j) -> int64_t {
    if (paged) {
      const int64_t page = trow[j >> p.page_shift];
      return page * p.v_bs + (int64_t)(j & pmask) * p.v_rs + vbase;
    }
    return vbase + (int64_t)j * p.v_rs;
  };

  v4i kreg[KPT], vreg[VPT];
  auto gload = [&](int t) {
    const int j0 = t * BN;
#pragma unroll
    for (int u = 0; u < KPT; u++) {
      const int cidx = tid + u * NT;
      v4i x = {0, 0, 0, 0};
      if (KCHUNKS % NT == 0 || cidx < KCHUNKS) {
        const int row = cidx / KCH, ch = cidx - row * KCH;
        const int j = j0 + row;
        if (j < sk) x = ld_global16(p.k + koff(j) + ch * 16);
      }
      kreg[u] = x;
    }
#pragma unroll
    for (int u = 0; u < VPT; u++) {
      const int cidx = tid + u * NT;
      v4i x = {0, 0, 0, 0};
      if (VCHUNKS % NT == 0 || cidx < VCHUNKS) {
        const int row = cidx / VCH, ch = cidx - row * VCH;
        const int j = j0 + row;
        if (j < sk) x = ld_global16(p.v + voff(j) + ch * 16);
      }
      vreg[u] = x;
    }
  };
  auto swrite = [&](int stage) {
    uint8_t* kt = smem + stage * STAGE;
    uint8_t* vt = kt + KTILE;
#pragma unroll
    for (int u = 0; u < KPT; u++) {
      const int cidx = tid + u * NT;
      if (KCHUNKS % NT == 0 || cidx < KCHUNKS) {
        const int row = cidx / KCH, ch = cidx - row * KCH;
        *reinterpret_cast<v4i*>(kt + row * D + swz<KCH>(ch, k_sv(row)) * 16) = kreg[u];
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; u++) {
      const int cidx = tid + u * NT;
      if (VCHUNKS % NT == 0 || cidx < VCHUNKS) {
        const int row = cidx / VCH, ch = cidx - row * VCH;
        *reinterpret_cast<v4i*>(vt + row * DV + swz<VCH>(ch, v_sv(row)) * 16) = vreg[u];
      }
    }
  };

  // running softmax state of this lane's row (shared by lanes L and L^32)
  float m_run = kNegInf, l_run = 0.0f;
  v16f oacc[NB];
#pragma unroll
  for (int n = 0; n < NB; n++)
#pragma unroll
    for (int r = 0; r < 16; r++) oacc[n][r] = 0.0f;

  // per-lane constant of the transposed V read: key offset within a 16-key group
  const int trj = (lane & 15) >> 1;
  const int tr_key = 8 * (trj >> 2) + 4 * hgrp + (trj & 3);
  const int tr_chunk_hi = (lane >> 4) & 1;
  const int tr_byte = 8 * (lane & 1);

  if (t_begin < t_end) {
    gload(t_begin);
    swrite(0);
    __syncthreads();
  }
  for (int t = t_begin; t < t_end; t++) {
    const int st = (t - t_begin) & 1;
    if (t + 1 < t_end) gload(t + 1);
    const uint8_t* kt = smem + st * STAGE;
    const uint8_t* vt = kt + KTILE;
    const int j0 = t * BN;

    // ---- S^T = K Q^T ----
    v16f sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
#pragma unroll
      for (int r = 0; r < 16; r++) sacc[kb][r] = 0.0f;
      const int row = kb * 32 + lrow;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const int off = ks * 64 + hgrp * 32;
        v8i kop = {0, 0, 0, 0, 0, 0, 0, 0};
        if (off < D) {
          const int ch = off >> 4;
          const v4i a = *reinterpret_cast<const v4i*>(kt + row * D + swz<KCH>(ch, k_sv(row)) * 16);
          const v4i a2 = *reinterpret_cast<const v4i*>(kt + row * D + swz<KCH>(ch + 1, k_sv(row)) * 16);
          kop = (v8i){a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
        }
        sacc[kb] = mfma_32x32x64_fp8(kop, qop[ks], sacc[kb]);
      }
    }

    // ---- mask (only tiles that cross some row's key bounds) ----
    const bool need_mask = (j0 < full_lo) || (j0 + BN > full_hi);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * hgrp + (r & 3);
          if (j < my_lo || j >= my_hi) sacc[kb][r] = kNegInf;
        }
    }

    // ---- row max (lanes L and L^32 share a row), lazy rescale ----
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int r = 0; r < 16; r++) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * c;
    float alpha = 1.0f;
    if (mt - m_run > kTau) {          // also true when m_run = -inf and mt is finite
      alpha = fast_exp2(m_run - mt);  // 0 when m_run = -inf
      m_run = mt;
    }
    const float nb = (m_run == kNegInf) ? 0.0f : kBias - m_run;

    // ---- P = 2^(S*c - m + 8), row sum, E4M3 pack in PV-operand order ----
    v8i pop;
    float lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; w++) {
      const int kb = w >> 2, r0 = 4 * (w & 3);
      const float p0 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 0], c, nb));
      const float p1 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 1], c, nb));
      const float p2 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 2], c, nb));
      const float p3 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 3], c, nb));
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
      pop[w] = word;
      // the row sum is taken over the rounded P that enters the PV product, so O is an exact
      // convex combination of V rows (weights sum to 1 whatever the E4M3 rounding)
      const auto r01 = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
      const auto r23 = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
      lsum += (r01[0] + r01[1]) + (r23[0] + r23[1]);
    }
    l_run = alpha * l_run + lsum;

    // ---- O_tile = V^T P^T from zero, then O = alpha * O + O_tile ----
#pragma unroll
    for (int n = 0; n < NB; n++) {
      v8i vop;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int row = 16 * r + tr_key;
        const int ch = 2 * n + tr_chunk_hi;
        const int off = row * DV + swz<VCH>(ch, v_sv(row)) * 16 + tr_byte;
        const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA8_LDS v2i*)((FA8_LDS uint8_t*)smem + (st * STAGE + KTILE + off)));
        vop[2 * r] = x[0];
        vop[2 * r + 1] = x[1];
      }
      v16f zero;
#pragma unroll
      for (int r = 0; r < 16; r++) zero[r] = 0.0f;
      const v16f ot = mfma_32x32x64_fp8(vop, pop, zero);
#pragma unroll
      for (int r = 0; r < 16; r++) oacc[n][r] = __builtin_fmaf(alpha, oacc[n][r], ot[r]);
    }

    if (t + 1 < t_end) swrite(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!valid) return;
  const bool nonempty = l_tot > 0.0f;
  const float inv = nonempty ? dvs / l_tot : 0.0f;
  const float lse = nonempty ? (m_run + __log2f(l_tot) - kBias) * kLn2 : kNegInf;

  if constexpr (PACKED) {
    const int64_t prow = (((int64_t)split * p.batch + b) * p.max_sq + qi) * p.hq + qh;
    float* orow = p.o_part + prow * DV;
#pragma unroll
    for (int n = 0; n < NB; n++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        const int dvi = 32 * n + 8 * q4 + 4 * hgrp;
        v4f v = {oacc[n][4 * q4] * inv, oacc[n][4 * q4 + 1] * inv, oacc[n][4 * q4 + 2] * inv, oacc[n][4 * q4 + 3] * inv};
        *reinterpret_cast<v4f*>(orow + dvi) = v;
      }
    if (hgrp == 0) p.lse_part[prow] = lse;
  } else {
    const int64_t orow_off = (p.cu_q ? (int64_t)(q0 + qi) * p.o_rs : (int64_t)b * p.o_bs + (int64_t)qi * p.o_rs) +
                             (int64_t)qh * p.o_hs;
    uint16_t* orow = reinterpret_cast<uint16_t*>(p.out) + orow_off;
    const bool fp16 = p.out_fp16 != 0;
#pragma unroll
    for (int n = 0; n < NB; n++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        const int dvi = 32 * n + 8 * q4 + 4 * hgrp;
        store4_half(orow + dvi, oacc[n][4 * q4] * inv, oacc[n][4 * q4 + 1] * inv, oacc[n][4 * q4 + 2] * inv,
                    oacc[n][4 * q4 + 3] * inv, fp16);
      }
    if (p.lse && hgrp == 0) {
      const int64_t loff = p.cu_q ? (int64_t)qh * p.l_hs + (int64_t)(q0 + qi) * p.l_rs
                                  : (int64_t)b * p.l_bs + (int64_t)qh * p.l_hs + (int64_t)qi * p.l_rs;
      p.lse[loff] = lse;
    }
  }
}

// Log-sum-exp merge of split partials: one thread per 4 output elements of one row.
__global__ void __launch_bounds__(256) fa8_combine_kernel(const CParams c) {
  const int tpr = c.dv / 4;
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rows = (int64_t)c.batch * c.max_sq * c.hq;
  const int64_t row = gt / tpr;
  const int q = (int)(gt - row * tpr);
  if (row >= rows) return;
  const int h = (int)(row % c.hq);
  const int i = (int)((row / c.hq) % c.max_sq);
  const int b = (int)(row / ((int64_t)c.hq * c.max_sq));
  const int q0 = c.cu_q ? c.cu_q[b] : 0;
  const int sq = c.cu_q ? c.cu_q[b + 1] - q0 : c.max_sq;
  if (i >= sq) return;
  float mx = kNegInf;
  for (int s = 0; s < c.nsplit; s++) mx = fmaxf(mx, c.lse_part[(int64_t)s * rows + row]);
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float den = 0.0f;
  if (mx != kNegInf) {
    for (int s = 0; s < c.nsplit; s++) {
      const float ls = c.lse_part[(int64_t)s * rows + row];
      if (ls == kNegInf) continue;
      const float w = __expf(ls - mx);
      den += w;
      const v4f o = *reinterpret_cast<const v4f*>(c.o_part + ((int64_t)s * rows + row) * c.dv + 4 * q);
      acc += w * o;
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  const int64_t ooff = (c.cu_q ? (int64_t)(q0 + i) * c.o_rs : (int64_t)b * c.o_bs + (int64_t)i * c.o_rs) +
                       (int64_t)h * c.o_hs + 4 * q;
  store4_half(reinterpret_cast<uint16_t*>(c.out) + ooff, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv,
              c.out_fp16 != 0);
  if (c.lse && q == 0) {
    const int64_t loff = c.cu_q ? (int64_t)h * c.l_hs + (int64_t)(q0 + i) * c.l_rs
                                : (int64_t)b * c.l_bs + (int64_t)h * c.l_hs + (int64_t)i * c.l_rs;
    c.lse[loff] = den > 0.0f ? mx + __logf(den) : kNegInf;
  }
}

template <int D, int DV>
static hipError_t launch_prefill_t(const KParams& kp, hipStream_t stream) {
  constexpr int NW = kPrefillRows / 32;
  dim3 grid((unsigned)kp.nmb, (unsigned)kp.hq, (unsigned)kp.batch);
  hipLaunchKernelGGL((fa8_attn_kernel<D, DV, NW, false>), grid, dim3(NW * 64), 0, stream, kp);
  return hipGetLastError();
}
template <int D, int DV>
static hipError_t launch_decode_t(const KParams& kp, hipStream_t stream) {
  constexpr int NW = kDecodeRows / 32;
  dim3 grid((unsigned)(kp.hkv * kp.nmb), (unsigned)kp.nsplit, (unsigned)kp.batch);
  hipLaunchKernelGGL((fa8_attn_kernel<D, DV, NW, true>), grid, dim3(NW * 64), 0, stream, kp);
  return hipGetLastError();
}

#define FA8_DISPATCH(FN, d, dv, kp, stream)                                   \
  do {                                                                        \
    if (d == 64 && dv == 64) return FN<64, 64>(kp, stream);                   \
    if (d == 96 && dv == 96) return FN<96, 96>(kp, stream);                   \
    if (d == 128 && dv == 128) return FN<128, 128>(kp, stream);               \
    if (d == 192 && dv == 192) return FN<192, 192>(kp, stream);               \
    if (d == 256 && dv == 256) return FN<256, 256>(kp, stream);               \
    if (d == 192 && dv == 128) return FN<192, 128>(kp, stream);               \
    return hipErrorInvalidValue;                                              \
  } while (0)

hipError_t launch_prefill(const KParams& kp, int d, int dv, hipStream_t stream) {
  FA8_DISPATCH(launch_prefill_t, d, dv, kp, stream);
}
hipError_t launch_decode(const KParams& kp, int d, int dv, hipStream_t stream) {
  FA8_DISPATCH(launch_decode_t, d, dv, kp, stream);
}
hipError_t launch_combine(const CParams& cp, hipStream_t stream) {
  const int64_t threads = (int64_t)cp.batch * cp.max_sq * cp.hq * (cp.dv / 4);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(fa8_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, cp);
  return hipGetLastError();
}

}  // namespace fa8
