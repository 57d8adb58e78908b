// Per-(batch, kv head) FP8 quantization of a bf16/fp16 Q: the step before the attention path.
// The block quantization formula of the FlashAttention-3 page ("Low-Precision FP8 Attention
// with Block Scaling"): scale = max|X_block| / 448, X_fp8 = clip(round(X / scale), -448, 448),
// with the block = every query row of one sequence and the q heads of one kv head, which is the
// granularity of the attention path's q descale. Each code is decided in fp32: s = amax / 448
// (1 for a block of zeros), y = x / s (IEEE division), clip to [-448, 448], round to nearest
// even E4M3.
//
// Two launches over chunks of kQuantRows rows of one (batch, kv head): the first writes the max
// |x| of each group of kAmaxChunks chunks into the workspace entries of those chunks, the second
// reduces the entries of its block, writes the descale (chunk 0) and quantizes its chunk.
// HBM-bound: Q is read twice, the codes written once.
//
// The quotient x / s: for 2^-96 <= s < inf the second launch takes q0 = x * r with r = 1 / s
// (IEEE, once per block), the residual x - q0 * s by FMA, and q0 + residual * r by FMA, with the
// sign of x. That is 4 instructions where the IEEE division takes about 10, and for every bf16
// and fp16 input it gives the E4M3 code of the IEEE quotient (exhaustive check over every input
// value and block maximum, with fp32 subnormals kept as these kernels run them). Smaller s (the
// residual would fall among the fp32 subnormals and lose bits) and non-finite s divide.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa8_internal.h"

namespace fa8 {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;

// 8 consecutive input elements (16 bytes) as fp32
__device__ __forceinline__ void load8(const void* base, int64_t off, bool fp16, float (&x)[8]) {
  const v4i w = *reinterpret_cast<const v4i*>(reinterpret_cast<const uint16_t*>(base) + off);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t u = (uint32_t)w[i];
    if (fp16) {
      x[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFF));
      x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
    } else {
      x[2 * i] = __builtin_bit_cast(float, u << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, u & 0xFFFF0000u);
    }
  }
}

struct Chunk {
  int64_t in_row0;    // element offset of the chunk's first row, head kvh * g
  int64_t out_row0;   // byte offset of the same
  int rows;           // rows of the chunk inside the sequence (0 .. kQuantRows)
};

// Rows [c * kQuantRows, (c + nc) * kQuantRows) of sequence b (cut to the sequence), heads of kv head kvh
__device__ __forceinline__ Chunk chunk_of(const QParams& p, int b, int kvh, int c, int nc = 1) {
  const int q0 = p.cu_q ? p.cu_q[b] : 0;
  const int sq = p.cu_q ? p.cu_q[b + 1] - q0 : p.max_sq;
  const int r0 = c * kQuantRows;
  Chunk ch;
  ch.rows = max(0, min(sq - r0, nc * kQuantRows));
  const int64_t row = p.cu_q ? (int64_t)q0 + r0 : (int64_t)r0;
  ch.in_row0 = (p.cu_q ? 0 : (int64_t)b * p.q_bs) + row * p.q_rs + (int64_t)kvh * p.g * p.q_hs;
  ch.out_row0 = (p.cu_q ? 0 : (int64_t)b * p.o_bs) + row * p.o_rs + (int64_t)kvh * p.g * p.o_hs;
  return ch;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); w++) v = fmaxf(v, red[w]);
  return v;
}

}  // namespace

// grid (ceil(chunks / kAmaxChunks), heads_kv, batch), 256 threads: the max |x| over chunks
// [c0, c0 + kAmaxChunks) -> ws[(b hkv + kvh) chunks + c] for each of those chunks c (the block
// reduction takes the max over all entries, so an entry may hold the max of more than its chunk)
// Chunks per workgroup of the first launch. On a [2, 8192, 32, 128] bf16 Q the pair of launches
// measured 57 us with 4 (1024 workgroups), 58.5 us with 1 and 69 us with 8.
constexpr int kAmaxChunks = 4;
__global__ void __launch_bounds__(256) fa8_quant_amax_kernel(const QParams p) {
  __shared__ float red[4];
  const int c0 = blockIdx.x * kAmaxChunks, kvh = blockIdx.y, b = blockIdx.z;
  const Chunk ch = chunk_of(p, b, kvh, c0, kAmaxChunks);
  const int vpr = p.g * (p.d / 8);                 // 8-element vectors per row of the block
  const int nv = ch.rows * vpr;
  const bool fp16 = p.in_fp16 != 0;
  const int nt = (int)blockDim.x;
  float m = 0.0f;
  // four vectors per thread and pass, their loads issued together
  constexpr int U = 4;
  if (nt % vpr == 0) {
    // whole rows per pass: a thread keeps its head and column (no divisions in the loop)
    const int row0 = (int)threadIdx.x / vpr, rem = (int)threadIdx.x - row0 * vpr;
    const int h = rem / (p.d / 8), col = (rem - h * (p.d / 8)) * 8;
    const int step = nt / vpr;
    const int64_t base = ch.in_row0 + (int64_t)h * p.q_hs + col;
    for (int r0 = row0; r0 < ch.rows; r0 += U * step) {
      float x[U][8];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int r = r0 + u * step;
        if (r < ch.rows) {
          load8(p.q, base + (int64_t)r * p.q_rs, fp16, x[u]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; i++) x[u][i] = 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(x[u][i]));
    }
  } else {
    for (int v0 = threadIdx.x; v0 < nv; v0 += U * nt) {
      float x[U][8];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int v = v0 + u * nt;
        if (v < nv) {
          const int r = v / vpr, rem = v - r * vpr;
          const int h = rem / (p.d / 8), col = (rem - h * (p.d / 8)) * 8;
          load8(p.q, ch.in_row0 + (int64_t)r * p.q_rs + (int64_t)h * p.q_hs + col, fp16, x[u]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; i++) x[u][i] = 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; u++)
#pragma unroll
        for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(x[u][i]));
    }
  }
  m = block_max(m, red);
  if (threadIdx.x < kAmaxChunks && c0 + (int)threadIdx.x < p.nchunk)
    p.ws[((int64_t)b * p.hkv + kvh) * p.nchunk + c0 + threadIdx.x] = m;
}

// x / s, both paths as the header comment describes (FAST only for 2^-96 <= s < inf)
template <bool FAST>
__device__ __forceinline__ float quotient(float x, float s, float r) {
  if constexpr (FAST) {
    const float q0 = x * r;
    const float e = __builtin_fmaf(-q0, s, x);
    return __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
  } else {
    return x / s;
  }
}

// Codes of the 8 elements at (row, h, col) of the chunk
template <bool FAST>
__device__ __forceinline__ void apply_vec(const QParams& p, const Chunk& ch, float s, float r, bool fp16, int row,
                                          int h, int col) {
  float x[8];
  load8(p.q, ch.in_row0 + (int64_t)row * p.q_rs + (int64_t)h * p.q_hs + col, fp16, x);
  int w[2];
#pragma unroll
  for (int k = 0; k < 2; k++) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; i++) y[i] = fminf(fmaxf(quotient<FAST>(x[4 * k + i], s, r), -kE4M3Max), kE4M3Max);
    int word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w[k] = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
  }
  uint8_t* dst = reinterpret_cast<uint8_t*>(p.q_out) + ch.out_row0 + (int64_t)row * p.o_rs + (int64_t)h * p.o_hs + col;
  *reinterpret_cast<v2i*>(dst) = (v2i){w[0], w[1]};
}

// E4M3 codes of one chunk, every element divided by the block's s
template <bool FAST>
__device__ __forceinline__ void apply_chunk(const QParams& p, const Chunk& ch, float s) {
  const float r = 1.0f / s;
  const int vpr = p.g * (p.d / 8);
  const int nv = ch.rows * vpr;
  const bool fp16 = p.in_fp16 != 0;
  const int nt = (int)blockDim.x;
  if (nt % vpr == 0) {
    // the workgroup covers whole rows per pass: a thread keeps its head and column, and steps
    // nt / vpr rows at a time (no divisions in the loop)
    const int row0 = (int)threadIdx.x / vpr, rem = (int)threadIdx.x - row0 * vpr;
    const int h = rem / (p.d / 8), col = (rem - h * (p.d / 8)) * 8;
    const int step = nt / vpr;
#pragma unroll 4
    for (int row = row0; row < ch.rows; row += step) apply_vec<FAST>(p, ch, s, r, fp16, row, h, col);
  } else {
#pragma unroll 4
    for (int v = threadIdx.x; v < nv; v += nt) {
      const int row = v / vpr, rem = v - row * vpr;
      const int h = rem / (p.d / 8), col = (rem - h * (p.d / 8)) * 8;
      apply_vec<FAST>(p, ch, s, r, fp16, row, h, col);
    }
  }
}

// grid (chunks, heads_kv, batch), 256 threads: block descale and E4M3 codes of the chunk
__global__ void __launch_bounds__(256) fa8_quant_apply_kernel(const QParams p) {
  __shared__ float red[4];
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const float* part = p.ws + ((int64_t)b * p.hkv + kvh) * p.nchunk;
  float m = 0.0f;
  for (int i = threadIdx.x; i < p.nchunk; i += blockDim.x) m = fmaxf(m, part[i]);
  const float amax = block_max(m, red);
  const float s = amax > 0.0f ? amax / kE4M3Max : 1.0f;
  if (c == 0 && threadIdx.x == 0) p.descale[(int64_t)b * p.hkv + kvh] = s;
  const Chunk ch = chunk_of(p, b, kvh, c);
  // s is the same for the whole workgroup
  if (s >= 0x1p-96f && s <= 3.40282347e38f) apply_chunk<true>(p, ch, s);
  else apply_chunk<false>(p, ch, s);
}

hipError_t launch_quantize_q(const QParams& qp, hipStream_t stream) {
  const dim3 grid((unsigned)qp.nchunk, (unsigned)qp.hkv, (unsigned)qp.batch);
  const dim3 grid_amax((unsigned)((qp.nchunk + kAmaxChunks - 1) / kAmaxChunks), (unsigned)qp.hkv, (unsigned)qp.batch);
  hipLaunchKernelGGL(fa8_quant_amax_kernel, grid_amax, dim3(256), 0, stream, qp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fa8_quant_apply_kernel, grid, dim3(256), 0, stream, qp);
  return hipGetLastError();
}

}  // namespace fa8
