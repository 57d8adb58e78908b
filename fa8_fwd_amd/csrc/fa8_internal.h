// Internal interface between the host-side ABI (fa8_host.cpp) and the gfx950 kernels
// (fa8_kernels.hip). Everything here is resolved on the host from fa8_fwd_params.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa8 {

struct KParams {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  int64_t q_bs, q_rs, q_hs;
  int64_t k_bs, k_rs, k_hs;   // k_bs: page stride when paged
  int64_t v_bs, v_rs, v_hs;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* used_k;
  const int32_t* table;
  int64_t table_stride;
  int32_t page_shift;         // log2(page_size); -1 when not paged
  const float* dq; int64_t dq_sb, dq_sh;
  const float* dk; int64_t dk_sb, dk_sh;
  const float* dv; int64_t dv_sb, dv_sh;
  float scale_log2;           // softmax_scale * log2(e)
  int32_t batch, hq, hkv, g, max_sq, max_sk;
  int32_t wl, wr;             // -1 = unbounded; wr = 0 when causal
  int32_t causal;
  void* out; int64_t o_bs, o_rs, o_hs; int32_t out_fp16;
  int32_t o_vec16;            // out 16-byte aligned, its strides multiples of 8 elements
  float* lse; int64_t l_bs, l_hs, l_rs;
  float* o_part; float* lse_part; int32_t nsplit;
  int32_t nmb;                // row blocks per (batch, head) (decode) or per (batch, q head) (prefill)
  int32_t bk8;                // prefill with per-sequence lengths: ceil(batch * hkv / 8), else 0
  const float* sink;          // [hq] sink logits or null (prefill finalize only)
  int32_t decode_kernel;      // -1: the library's choice; 0: per-head kernel; 1: several heads per wave
  const int32_t* sched;       // balanced decode schedule (fa8_decode_schedule), or null for static splits
  int32_t* sched_out;         // the schedule buffer the decode waves write when they compute it
  int32_t sched_inline;       // 1: every wave computes the schedule itself (batch <= 64)
  int32_t sched_workers;      // W of the balanced schedule
  // MXFP8 block scales (E8M0 bytes; strides in bytes), MX prefill only
  const uint8_t* q_mx; int64_t qmx_bs, qmx_rs, qmx_hs;
  const uint8_t* k_mx; int64_t kmx_bs, kmx_rs, kmx_hs;
  const uint8_t* v_mx; int64_t vmx_bs, vmx_ts, vmx_hs;   // vmx_ts: per 32-key block
};

struct CParams {
  const float* o_part;
  const float* lse_part;
  int32_t nsplit, batch, max_sq, hq, dv;
  const int32_t* cu_q;
  void* out; int64_t o_bs, o_rs, o_hs; int32_t out_fp16;
  int32_t o_vec16;            // out 16-byte aligned, its strides multiples of 8 elements
  float* lse; int64_t l_bs, l_hs, l_rs;
  const float* sink;          // [hq] sink logits or null
  const int32_t* sched;       // balanced decode schedule (partial slots per sequence), or null
};

// Q quantizer: one chunk = kQuantRows rows of one (batch, kv head) block.
struct QParams {
  const void* q; int64_t q_bs, q_rs, q_hs; int32_t in_fp16;   // strides in elements
  const int32_t* cu_q;
  void* q_out; int64_t o_bs, o_rs, o_hs;                      // strides in bytes
  float* descale;                                             // [batch, hkv]
  float* ws;                                                  // [batch, hkv, nchunk]
  int32_t batch, max_sq, hkv, g, d, nchunk;
};
constexpr int kQuantRows = 32;
hipError_t launch_quantize_q(const QParams& qp, hipStream_t stream);

// Rows per workgroup of the prefill kernels (4 waves of 32 rows, 256 threads) and of the decode
// kernel.
constexpr int kPrefillRows = 128;
constexpr int kPrefillThreads = 256;

// Workgroups of a prefill launch: one per (row block, q head, batch), or, with per-sequence
// lengths, 8 * bk8 * nmb * g (the round-robin deal of (batch, kv head) groups over the 8 XCDs
// rounds the group count up to a multiple of 8).
inline int64_t prefill_grid(const KParams& k) {
  return k.bk8 > 0 ? (int64_t)8 * k.bk8 * k.nmb * k.g : (int64_t)k.nmb * k.hq * k.batch;
}
constexpr int kDecodeRows = 32;
constexpr int kKvTile = 64;

// kv heads per wave the several-heads decode kernel would use for this problem, or 0 when it
// cannot take it; and the same subject to kp.decode_kernel (0 when the per-head kernel is used).
int decode_heads_applicable(const KParams& kp, int d, int dv);
int decode_heads_choice(const KParams& kp, int d, int dv);
// Workgroups per split of the decode kernel launch_decode picks; per worker of a balanced schedule.
int decode_units_per_split(const KParams& kp, int d, int dv);
int decode_units_per_worker(const KParams& kp, int d, int dv);

hipError_t launch_prefill(const KParams& kp, int d, int dv, hipStream_t stream);
hipError_t launch_prefill_mx(const KParams& kp, int d, int dv, hipStream_t stream);
hipError_t launch_decode(const KParams& kp, int d, int dv, hipStream_t stream);
// Balanced schedule: fa8_decode_schedule_kernel, then the decode kernels with one wave per
// (kv head unit, worker); kp.sched set, one row block per kv head.
hipError_t launch_decode_schedule(const KParams& kp, int32_t workers, int32_t* sched, hipStream_t stream);
hipError_t launch_decode_sched(const KParams& kp, int d, int dv, int32_t workers, hipStream_t stream);
hipError_t launch_combine(const CParams& cp, hipStream_t stream);
// Device address (on the current device) of the library's static scratch array of
// FA8_NOALLOC_SCRATCH_BYTES bytes.
hipError_t noalloc_scratch(void** ptr);

}  // namespace fa8
