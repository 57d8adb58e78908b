// Test probe (not part of the library): the precision of gfx950's FP8 matrix-core dot products,
// v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and E8M0 block scales, as the attention
// kernels use it for S = K Q^T. One wave per 32 x 32 block of (key, query) pairs, d = 128 bytes
// per row in two 64-element k-steps; a row's 16-byte chunks c = 4s + h and 4s + 2 + h go to lane
// half h of k-step s, so hardware k-block t of step s is d-block 2s + t (32 elements), scaled by
// the lane's scale byte. Two results per pair:
//   out[0]: both k-steps chained through the accumulator (as the kernels do)
//   out[1]: each 32-element block alone from a zero accumulator, the four summed in fp32
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v16f mm(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// K [nk][128] E4M3, ks [nk][4] E8M0, Q [nq][128], qs [nq][4]; nk, nq multiples of 32;
// out [2][nk][nq] fp32
__global__ void __launch_bounds__(64) mfma_dot_probe(const uint8_t* K, const uint8_t* ks, const uint8_t* Q,
                                                     const uint8_t* qs, int nk, int nq, float* out) {
  const int L = threadIdx.x, h = L >> 5, lr = L & 31;
  const int krow = blockIdx.x * 32 + lr, qrow = blockIdx.y * 32 + lr;
  v8i kop[2], qop[2];
  int ksc[2], qsc[2];
  for (int s = 0; s < 2; s++) {
    const v4i a = *(const v4i*)(K + (size_t)krow * 128 + 64 * s + 16 * h);
    const v4i a2 = *(const v4i*)(K + (size_t)krow * 128 + 64 * s + 32 + 16 * h);
    kop[s] = (v8i){a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
    const v4i b = *(const v4i*)(Q + (size_t)qrow * 128 + 64 * s + 16 * h);
    const v4i b2 = *(const v4i*)(Q + (size_t)qrow * 128 + 64 * s + 32 + 16 * h);
    qop[s] = (v8i){b[0], b[1], b[2], b[3], b2[0], b2[1], b2[2], b2[3]};
    ksc[s] = ks[krow * 4 + 2 * s + h];
    qsc[s] = qs[qrow * 4 + 2 * s + h];
  }
  v16f chained = mm(kop[0], qop[0], (v16f){}, ksc[0], qsc[0]);
  chained = mm(kop[1], qop[1], chained, ksc[1], qsc[1]);
  v16f blocks = {};
  for (int s = 0; s < 2; s++)
    for (int t = 0; t < 2; t++) {
      v8i ka = kop[s];
      for (int w = 0; w < 4; w++) ka[4 * (1 - t) + w] = 0;   // keep hardware k-block t only
      const v16f r = mm(ka, qop[s], (v16f){}, ksc[s], qsc[s]);
      for (int i = 0; i < 16; i++) blocks[i] += r[i];
    }
  const size_t plane = (size_t)nk * nq;
  for (int r = 0; r < 16; r++) {
    const int key = blockIdx.x * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
    const size_t o = (size_t)key * nq + blockIdx.y * 32 + lr;
    out[o] = chained[r];
    out[plane + o] = blocks[r];
  }
}
}  // namespace

// Returns 0 on success, 1 for sizes that are not positive multiples of 32, 2 on a HIP error.
extern "C" int mfma_dot_probe_run(const void* K, const void* ks, const void* Q, const void* qs, int nk, int nq,
                                  void* out) {
  if (nk <= 0 || nq <= 0 || nk % 32 || nq % 32) return 1;
  hipLaunchKernelGGL(mfma_dot_probe, dim3(nk / 32, nq / 32), dim3(64), 0, 0, (const uint8_t*)K, (const uint8_t*)ks,
                     (const uint8_t*)Q, (const uint8_t*)qs, nk, nq, (float*)out);
  return hipDeviceSynchronize() == hipSuccess ? 0 : 2;
}
