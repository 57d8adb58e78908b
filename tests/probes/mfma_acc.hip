// Test probe (not part of the library): how gfx950's FP8 matrix cores add the accumulator
// input C to a dot product, v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and unit scales
// (the PV product of the attention kernels). One wave per 32 x 32 output block; `steps` products
// of 64-element contractions are added to an initial C0 in one of two ways:
//   mode 0: chained through the accumulator, D = mfma(A_s, B_s, D) from D = C0
//   mode 1: each product from a zero accumulator, added to D in fp32
// A and B are raw operand registers: [steps][blocks][64 lanes][32 bytes]; both operands put
// element k of a row (A) or column (B) in the same lane half and byte, so the contraction pairs
// A's byte y of lane i + 32h with B's byte y of lane j + 32h. C0 and D: [blocks][64][16] fp32 in
// the accumulator's own order (lane L, register r: row 8(r/4) + 4(L/32) + r%4, column L%32).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(64) mfma_acc_probe(const uint8_t* A, const uint8_t* B, const float* C0, int steps,
                                                     int nblk, int mode, float* D) {
  const int L = threadIdx.x, blk = blockIdx.x;
  v16f acc;
  for (int r = 0; r < 16; r++) acc[r] = C0[((size_t)blk * 64 + L) * 16 + r];
  for (int s = 0; s < steps; s++) {
    const size_t off = (((size_t)s * nblk + blk) * 64 + L) * 32;
    const v8i a = *(const v8i*)(A + off);
    const v8i b = *(const v8i*)(B + off);
    if (mode == 0) {
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
    } else {
      const v16f t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, (v16f){}, 0, 0, 0, 0, 0, 0);
      for (int r = 0; r < 16; r++) acc[r] += t[r];
    }
  }
  for (int r = 0; r < 16; r++) D[((size_t)blk * 64 + L) * 16 + r] = acc[r];
}
}  // namespace

// Returns 0 on success, 1 for bad sizes or mode, 2 on a HIP error.
extern "C" int mfma_acc_probe_run(const void* A, const void* B, const void* C0, int steps, int nblk, int mode,
                                  void* D) {
  if (steps < 0 || nblk <= 0 || nblk > 65535 || (mode != 0 && mode != 1)) return 1;
  hipLaunchKernelGGL(mfma_acc_probe, dim3(nblk), dim3(64), 0, 0, (const uint8_t*)A, (const uint8_t*)B,
                     (const float*)C0, steps, nblk, mode, (float*)D);
  return hipDeviceSynchronize() == hipSuccess ? 0 : 2;
}
