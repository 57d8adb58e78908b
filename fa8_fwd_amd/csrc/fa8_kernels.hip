// gfx950 (MI355X) kernels of the FP8 attention forward.
//
// Two kernels share one per-tile routine (attn_tile): the full forward pass (fa8_prefill_kernel,
// four waves and 128 query rows of one query head per workgroup) and the split-KV decode pass
// (fa8_decode_kernel, one wave per workgroup, the q heads of one KV head packed as 32 rows).
// Per KV tile, each wave of 32 query rows does:
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
//   O_t = V^T P^T        FP8 MFMA from zero over this tile only, then O = alpha*O + O_t in fp32
//                        (Design, "Two-level PV accumulation")
// and at the end O *= dv / l, LSE = ln2 * (m + log2 l - 8) (bias removed from the LSE).
//
// Layout choices for gfx950 (from measured MFMA lane layouts):
//  * MFMA operands: lane L holds row L%32 of A (col L%32 of B) and 32 bytes of the contraction
//    dimension, lanes 0-31 one half and 32-63 the other; A and B use the same byte<->k order, so
//    any k permutation applied to both operands leaves the product unchanged.
//  * The S^T accumulator of a 32-key block puts key 8*(r/4) + 4*(L/32) + r%4 in register r of
//    lane L. Cast to E4M3 in register order, those bytes are already the B operand (P^T) of the
//    PV MFMA; the A operand (V^T) is read with the same key permutation by ds_read_b64_tr_b8
//    from the row-major V tile (no separate transpose pass over V).
//  * K and V tiles are row-major in LDS with a per-row XOR swizzle of their 16-byte chunks so
//    the rows that one LDS read instruction touches fall in distinct banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "fa8.h"
#include "fa8_internal.h"

// Split partials of fa8_fwd_decode_noalloc: one static array per GPU the library runs on, held
// until the process ends. Host code never passes this name to a kernel (on the host it is only a
// stand-in for the symbol): fa8::noalloc_scratch resolves the device address once per device.
static __device__ __align__(256) uint8_t scratch[FA8_NOALLOC_SCRATCH_BYTES];

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
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLog2E4M3Max = 8.80735492205760410f;   // log2(448), E4M3's largest finite value
constexpr float kNegInf = -__builtin_huge_valf();

// 1 KB read by the decode kernel's pipeline-filler loads (one 16-byte chunk per lane): a small
// block that stays cached, so those loads cost no HBM traffic. Never written.
__device__ __attribute__((aligned(1024))) uint8_t g_filler[1024];

__device__ __forceinline__ v16f mfma_32x32x64_fp8(v8i a, v8i b, v16f c) {
  // format codes 0/0 = E4M3 for both operands; zero scale operands select the unscaled MFMA
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_16x16x128_fp8(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Orders this wave's LDS accesses in the compiler's view without a hardware barrier: a wave's
// LDS instructions execute in issue order, so a one-wave workgroup exchanging data between its
// lanes through LDS only needs the compiler to keep program order. (__syncthreads would also
// wait for every outstanding global load, draining the prefetched tiles.)
__device__ __forceinline__ void wave_lds_order() { __asm__ __volatile__("" ::: "memory"); }

// Position of 16-byte chunk `ch` of a row holding NCH chunks, XOR-swizzled by `sv` inside the
// largest aligned power-of-two group of chunks that fits in the row (an involution).
template <int NCH>
__device__ __forceinline__ int swz(int ch, int sv) {
  if ((ch | 7) < NCH) return ch ^ (sv & 7);
  if ((ch | 3) < NCH) return ch ^ (sv & 3);
  if ((ch | 1) < NCH) return ch ^ (sv & 1);
  return ch;
}
// K rows are read 16 consecutive rows at a time (one 16-byte chunk each) by ds_read_b128; the LDS
// serves 256 bytes per cycle from 64 banks, so rows that share a 256-byte window (2 rows of
// 128 bytes, 4 of 64) need different chunk positions: the swizzle key is the window index of
// the row, which gives 16 distinct (window offset, chunk) pairs for 16 rows.
template <int D>
__device__ __forceinline__ int k_sv(int row) {
  return D == 64 ? (row >> 2) : (D == 128 ? (row >> 1) : row);
}
// V is read 8 rows at a time by ds_read_b64_tr_b8 with row sets {0-3, 8-11} + 4h (+16r):
// bits 0, 1 and 3 of the row make those 8 rows land in 8 different chunks.
__device__ __forceinline__ int v_sv(int row) { return (row & 3) | ((row >> 1) & 4); }
// Same for the 16x16 decode tile, whose transposed V reads touch rows {0-3, 16-19} + 4h (+32r).
__device__ __forceinline__ int v_sv16(int row) { return (row & 3) | ((row >> 2) & 4); }

__device__ __forceinline__ v4i ld_global16(const uint8_t* ptr) {
  return *reinterpret_cast<const v4i*>(ptr);
}
// 16-byte buffer load of lane offset voff from a wave-uniform base whose valid range is nrec
// bytes: offsets at or past nrec return zeros without a memory access. The base and range are
// made explicitly uniform so they live in scalar registers. Non-temporal cache policy.
__device__ __forceinline__ v4i ld_buffer16_nt(const uint8_t* base, int nrec, uint32_t voff) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint8_t* ub = reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)ub, (short)0, __builtin_amdgcn_readfirstlane(nrec), 0x00020000);
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 2));
}
// 16 bytes per lane global -> LDS (M0 = wave-uniform LDS destination, lane L writes LDS bytes
// [dst + 16 L, +16)), from a uniform base plus this lane's 32-bit offset (saddr form) or from a
// per-lane address (vaddr form). Issued as inline assembly on purpose: the compiler's wait-count
// pass cannot tell which LDS bytes such a copy writes, so with the builtin every later LDS read
// would wait for all outstanding copies, serializing the next tile's copy with this tile's math.
// Callers order the copies with explicit wait_vmcnt + barriers. The s_nop covers the
// SGPR-write-to-VMEM and M0 hazards of operands produced just before the statement.
__device__ __forceinline__ void copy16_to_lds(const uint8_t* base, uint32_t voff, uint32_t lds_dst) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint64_t ua = ((uint64_t)hi << 32) | lo;
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
  __asm__ __volatile__(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(ua), "s"(m0)
      : "memory", "m0");
}
__device__ __forceinline__ void copy16_to_lds_vaddr(const uint8_t* src, uint32_t lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
  __asm__ __volatile__(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(m0)
      : "memory", "m0");
}
// 16 bytes per lane buffer -> LDS: lane L's bytes at offset voff of the buffer described by the
// wave-uniform descriptor rsrc land at LDS [lds_dst + 16 L, +16); offsets at or past the
// descriptor's range read as zeros without a memory access. Inline assembly for the same reason
// as copy16_to_lds.
__device__ __forceinline__ void buffer_copy16_to_lds(v4i rsrc, uint32_t voff, uint32_t lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_dst);
  __asm__ __volatile__(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(m0)
      : "memory", "m0");
}
// Descriptor of nrec bytes from a wave-uniform base (no stride, raw buffer).
__device__ __forceinline__ v4i buffer_rsrc(const uint8_t* base, uint32_t nrec) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return (v4i){(int)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (int)(__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffff),
               (int)__builtin_amdgcn_readfirstlane(nrec), 0x00020000};
}
// E4M3 (RNE) of a and b into bytes 0 and 1 of the result; bytes 2 and 3 are left unspecified
// (the caller fills them with the high-half conversion). As inline assembly so that the
// destination is not first cleared for the half the instruction keeps.
__device__ __forceinline__ int cvt_pk_fp8_lo(float a, float b) {
  int r;
  __asm__("v_cvt_pk_fp8_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// max of three floats as one v_maximum3_f32 (IEEE 754-2019 maximum, which needs no quieting of
// its inputs: fmaxf would first quiet each MFMA result with an extra v_max_f32 x, x). A builtin
// rather than inline assembly, so the compiler knows the instruction and schedules it freely.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
// Cross-lane moves within a wave through the gfx950 permlane swaps (VALU, no LDS round trip).
// permlane16_swap(x, x) leaves {x of row 2k, x of row 2k+1} in both rows of each pair of
// 16-lane rows, permlane32_swap(x, x) leaves {x of rows 0-1, x of rows 2-3} in both halves.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// the value x of lane ^ 16 / lane ^ 32
__device__ __forceinline__ uint32_t from_xor16(uint32_t x, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return ((lane >> 4) & 1) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t from_xor32(uint32_t x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (lane >> 5) ? r[0] : r[1];
}
// Streaming load (non-temporal hint): for data read exactly once, like decode's K/V.
__device__ __forceinline__ v4i ld_global16_nt(const uint8_t* ptr) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(ptr));
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
__device__ __forceinline__ v2i pack4_half(float a, float b, float c, float d, bool fp16) {
  uint32_t lo, hi;
  if (fp16) {
    lo = f16_bits(a) | (f16_bits(b) << 16);
    hi = f16_bits(c) | (f16_bits(d) << 16);
  } else {
    lo = bf16_rne_bits(a) | (bf16_rne_bits(b) << 16);
    hi = bf16_rne_bits(c) | (bf16_rne_bits(d) << 16);
  }
  return (v2i){(int)lo, (int)hi};
}

__device__ __forceinline__ void store4_half(void* dst, float a, float b, float c, float d, bool fp16) {
  *reinterpret_cast<v2i*>(dst) = pack4_half(a, b, c, d, fp16);
}

__device__ __forceinline__ float load_descale(const float* p, int64_t sb, int64_t sh, int b, int kvh) {
  return p ? p[(int64_t)b * sb + (int64_t)kvh * sh] : 1.0f;
}

// Key-position ranges of one query row, bottom-right aligned.
struct RowRange {
  int sk, shift, wl, wr;
  __device__ int lo(int i) const { return wl >= 0 ? max(0, i + shift - wl) : 0; }
  __device__ int hi(int i) const { return wr >= 0 ? min(sk, i + shift + wr + 1) : sk; }
};

// Sequence lengths of batch b.
struct SeqInfo {
  int q0, sq, sk;
};
__device__ __forceinline__ SeqInfo seq_info(const KParams& p, int b) {
  SeqInfo s;
  s.q0 = p.cu_q ? p.cu_q[b] : 0;
  s.sq = p.cu_q ? p.cu_q[b + 1] - s.q0 : p.max_sq;
  if (p.used_k) s.sk = p.used_k[b];
  else if (p.cu_k) s.sk = p.cu_k[b + 1] - p.cu_k[b];
  else s.sk = p.max_sk;
  // b is uniform: keep the lengths in scalar registers (the loads above may be vector loads)
  s.q0 = __builtin_amdgcn_readfirstlane(s.q0);
  s.sq = __builtin_amdgcn_readfirstlane(s.sq);
  s.sk = __builtin_amdgcn_readfirstlane(s.sk);
  return s;
}

// The same lengths for a lane's own b (b may differ between lanes).
__device__ __forceinline__ SeqInfo seq_info_lane(const KParams& p, int b) {
  SeqInfo s;
  s.q0 = p.cu_q ? p.cu_q[b] : 0;
  s.sq = p.cu_q ? p.cu_q[b + 1] - s.q0 : p.max_sq;
  if (p.used_k) s.sk = p.used_k[b];
  else if (p.cu_k) s.sk = p.cu_k[b + 1] - p.cu_k[b];
  else s.sk = p.max_sk;
  return s;
}

// Keys seen by the query rows i_first .. i_last of one sequence: their union [lo, hi) and the
// range [full_lo, full_hi) every one of them sees (tiles inside it need no mask); an empty union
// is [0, 0).
struct DecodeKeys {
  int lo, hi, full_lo, full_hi;
};
__device__ __forceinline__ DecodeKeys decode_keys(const RowRange& rr, int i_first, int i_last) {
  DecodeKeys k{0, 0, 0, 0};
  if (i_last >= i_first) {
    k.lo = rr.lo(i_first);
    k.hi = rr.hi(i_last);
    k.full_lo = rr.lo(i_last);
    k.full_hi = rr.hi(i_first);
  }
  if (k.hi <= k.lo) { k.lo = 0; k.hi = 0; }
  return k;
}
// Granules (of kKvTile keys, counted from key 0) [g0, g1) that hold the union of a decode
// block's keys: g0 = lo / kKvTile, g1 = ceil(hi / kKvTile); none for an empty union.
__device__ __forceinline__ int union_granule0(const DecodeKeys& k) { return k.lo / kKvTile; }
__device__ __forceinline__ int union_granules(const DecodeKeys& k) {
  return k.hi > k.lo ? (k.hi + kKvTile - 1) / kKvTile - k.lo / kKvTile : 0;
}
// Static split s of S over a decode block's n granules: [g0 + floor(s n / S), g0 + floor((s+1) n / S)).
__device__ __forceinline__ void split_range(const DecodeKeys& k, int split, int nsplit, int& s0, int& s1) {
  const int g0 = union_granule0(k), n = union_granules(k);
  s0 = g0 + (int)(((int64_t)split * n) / nsplit);
  s1 = g0 + (int)(((int64_t)(split + 1) * n) / nsplit);
}

// Balanced decode schedule (written by fa8_decode_schedule_kernel): sched[0] = G, the granules
// of all sequences; sched[1] = W, the workers; gst = sched + 2 holds the exclusive prefix of the
// sequences' granule counts ([batch + 1] entries), pst = gst + batch + 1 the exclusive prefix of
// their segment counts. Worker w of W takes global granules [floor(w G / W), floor((w+1) G / W));
// global granule x belongs to worker owner(x) = floor(((x + 1) W - 1) / G). A segment is one
// (sequence, worker) pair whose granules meet; segment j of sequence b (pst[b] <= j < pst[b+1])
// is that of worker owner(gst[b]) + j - pst[b], and j is also its partial slot.
__device__ __forceinline__ int sched_owner(int x, int W, int G) { return (int)(((int64_t)(x + 1) * W - 1) / G); }
// Segment j from the schedule computed by the wave itself (at most 64 sequences: lane b holds
// sequence b), the same integers fa8_decode_schedule_kernel writes; the first wave of the grid
// also writes them to the schedule buffer for the combine.
__device__ __forceinline__ bool sched_segment_inline(const KParams& p, int j, int& b, int& gs0, int& gs1) {
  const int lane = threadIdx.x & 63;
  const int W = p.sched_workers;
  int v = 0, g0 = 0;
  if (lane < p.batch) {
    const SeqInfo si = seq_info_lane(p, lane);
    const RowRange rr{si.sk, si.sk - si.sq, p.wl, p.wr};
    const DecodeKeys k = decode_keys(rr, 0, si.sq - 1);
    v = union_granules(k);
    g0 = union_granule0(k);
  }
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  const int G = __builtin_amdgcn_readlane(incl, 63);
  const int gst = incl - v;
  const int n = (v > 0) ? sched_owner(gst + v - 1, W, G) - sched_owner(gst, W, G) + 1 : 0;
  int nincl = n;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(nincl, o);
    if (lane >= o) nincl += u;
  }
  const int pst = nincl - n;
  const int nseg = __builtin_amdgcn_readlane(nincl, 63);
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    int32_t* out = p.sched_out;
    if (lane == 0) {
      out[0] = G;
      out[1] = W;
      out[2 + p.batch] = G;
      out[3 + 2 * p.batch] = nseg;
    }
    if (lane < p.batch) {
      out[2 + lane] = gst;
      out[3 + p.batch + lane] = pst;
    }
  }
  if (j >= nseg) return false;
  // the last b with pst[b] <= j (pst nondecreasing over lanes 0 .. batch-1, pst[0] = 0)
  const int cnt = __popcll(__builtin_amdgcn_ballot_w64(lane < p.batch && pst <= j));
  b = cnt - 1;
  const int gb0 = __builtin_amdgcn_readlane(gst, b), gv = __builtin_amdgcn_readlane(v, b);
  const int w = sched_owner(gb0, W, G) + (j - __builtin_amdgcn_readlane(pst, b));
  const int A = (int)(((int64_t)w * G) / W), Z = (int)(((int64_t)(w + 1) * G) / W);
  const int sg0 = __builtin_amdgcn_readlane(g0, b);
  gs0 = sg0 + max(A, gb0) - gb0;
  gs1 = sg0 + min(Z, gb0 + gv) - gb0;
  return true;
}

// Segment j: its sequence b and granules [gs0, gs1) of that sequence (absolute, counted from its
// key 0); false when j is past the last segment. Wave-uniform.
__device__ __forceinline__ bool sched_segment(const KParams& p, int j, int& b, int& gs0, int& gs1) {
  if (p.sched_inline) return sched_segment_inline(p, j, b, gs0, gs1);
  const int32_t* gst = p.sched + 2;
  const int32_t* pst = gst + p.batch + 1;
  if (j >= __builtin_amdgcn_readfirstlane(pst[p.batch])) return false;
  const int G = __builtin_amdgcn_readfirstlane(p.sched[0]);
  const int W = __builtin_amdgcn_readfirstlane(p.sched[1]);
  // the last b with pst[b] <= j (pst[0] = 0, nondecreasing, pst[batch] > j), by a 64-way search
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = p.batch;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const bool le = idx < hi && pst[idx] <= j;
    const int cnt = __popcll(__builtin_amdgcn_ballot_w64(le));   // lanes 0 .. cnt-1 (monotone), cnt >= 1
    lo = lo + (cnt - 1) * step;
    hi = min(hi, lo + step);
  }
  b = lo;
  const int gb0 = __builtin_amdgcn_readfirstlane(gst[b]), gb1 = __builtin_amdgcn_readfirstlane(gst[b + 1]);
  const int w = sched_owner(gb0, W, G) + (j - __builtin_amdgcn_readfirstlane(pst[b]));
  const int A = (int)(((int64_t)w * G) / W), Z = (int)(((int64_t)(w + 1) * G) / W);
  const SeqInfo si = seq_info(p, b);
  const RowRange rr{si.sk, si.sk - si.sq, p.wl, p.wr};
  const int g0 = union_granule0(decode_keys(rr, 0, si.sq - 1));
  gs0 = g0 + max(A, gb0) - gb0;
  gs1 = g0 + min(Z, gb1) - gb0;
  return true;
}

// Element offsets of K/V row j of (batch b, kv head kvh).
struct KvAddr {
  const int32_t* trow;   // block-table row, or null
  int64_t kbase, vbase;  // offset of key 0 (non-paged) or of the kv head within a page (paged)
  int64_t k_ps, v_ps, k_rs, v_rs;
  int shift, pmask;
  __device__ int64_t k(int j) const {
    if (trow) return (int64_t)trow[j >> shift] * k_ps + (int64_t)(j & pmask) * k_rs + kbase;
    return kbase + (int64_t)j * k_rs;
  }
  __device__ int64_t v(int j) const {
    if (trow) return (int64_t)trow[j >> shift] * v_ps + (int64_t)(j & pmask) * v_rs + vbase;
    return vbase + (int64_t)j * v_rs;
  }
};
__device__ __forceinline__ KvAddr kv_addr(const KParams& p, int b, int kvh) {
  KvAddr a;
  const bool paged = p.page_shift >= 0;
  a.trow = paged ? p.table + (int64_t)b * p.table_stride : nullptr;
  a.kbase = paged ? (int64_t)kvh * p.k_hs
                  : (p.cu_k ? (int64_t)p.cu_k[b] * p.k_rs : (int64_t)b * p.k_bs) + (int64_t)kvh * p.k_hs;
  a.vbase = paged ? (int64_t)kvh * p.v_hs
                  : (p.cu_k ? (int64_t)p.cu_k[b] * p.v_rs : (int64_t)b * p.v_bs) + (int64_t)kvh * p.v_hs;
  a.k_ps = p.k_bs;
  a.v_ps = p.v_bs;
  a.k_rs = p.k_rs;
  a.v_rs = p.v_rs;
  a.shift = paged ? p.page_shift : 0;
  a.pmask = paged ? (1 << p.page_shift) - 1 : 0;
  return a;
}

// Q row of this lane as the B operand of S^T = K Q^T: d-bytes [64ks + 32*hgrp, +32).
template <int D>
__device__ __forceinline__ void load_q(const uint8_t* qrow, bool valid, int hgrp, v8i (&qop)[(D + 63) / 64]) {
#pragma unroll
  for (int ks = 0; ks < (D + 63) / 64; ks++) {
    const int off = ks * 64 + hgrp * 32;
    v4i a = {0, 0, 0, 0}, a2 = {0, 0, 0, 0};
    if (valid && off < D) {
      a = ld_global16(qrow + off);
      a2 = ld_global16(qrow + off + 16);
    }
    qop[ks] = (v8i){a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
  }
}

// A operand (V^T) of the PV MFMA for k-step pk (keys 64 pk ..) and output column block n, in
// the key order of the S^T accumulator (the order attn_tile uses).
template <int DV>
__device__ __forceinline__ v8i pv_operand_mx(const FA8_LDS uint8_t* vt, int pk, int n, int lane) {
  constexpr int VCH = DV / 16;
  const int hgrp = lane >> 5;
  const int trj = (lane & 15) >> 1;
  const int tr_key = 8 * (trj >> 2) + 4 * hgrp + (trj & 3);
  const int tr_chunk_hi = (lane >> 4) & 1;
  const int tr_byte = 8 * (lane & 1);
  v8i vop;
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int row = 64 * pk + 16 * r + tr_key;
    const int ch = 2 * n + tr_chunk_hi;
    const int off = row * DV + swz<VCH>(ch, v_sv(row)) * 16 + tr_byte;
    const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA8_LDS v2i*)(vt + off));
    vop[2 * r] = x[0];
    vop[2 * r + 1] = x[1];
  }
  return vop;
}

// S^T = K Q^T of one tile of BN keys (the first part of attn_tile).
template <int D, int BN>
__device__ __forceinline__ void qk_tile(const FA8_LDS uint8_t* kt, const v8i (&qop)[(D + 63) / 64], int lane,
                                        v16f (&sacc)[BN / 32]) {
  constexpr int KB = BN / 32;        // 32-key blocks of S^T
  constexpr int KS = (D + 63) / 64;  // k-steps of QK
  constexpr int KCH = D / 16;
  const int hgrp = lane >> 5, lrow = lane & 31;
#pragma unroll
  for (int kb = 0; kb < KB; kb++) {
#pragma unroll
    for (int r = 0; r < 16; r++) sacc[kb][r] = 0.0f;
    const int row = kb * 32 + lrow;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const int off = ks * 64 + hgrp * 32;
      v8i kop = {0, 0, 0, 0, 0, 0, 0, 0};
      if (off < D) {
        const int ch = off >> 4;
        const v4i a = *(const FA8_LDS v4i*)(kt + row * D + swz<KCH>(ch, k_sv<D>(row)) * 16);
        const v4i a2 = *(const FA8_LDS v4i*)(kt + row * D + swz<KCH>(ch + 1, k_sv<D>(row)) * 16);
        kop = (v8i){a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
      }
      sacc[kb] = mfma_32x32x64_fp8(kop, qop[ks], sacc[kb]);
    }
  }
}

// The rest of a tile given its S^T: mask, row max, lazy rescale of l and O, P, PV onto O and
// the row sum (the second part of attn_tile).
// Per-lane part of the LDS offset of the V^T operand for output column block n (the key order
// of the S^T accumulator, read by ds_read_b64_tr_b8 from the row-major swizzled V tile): the
// swizzle key of a row depends only on its bits 0, 1 and 3, which the 16-row and 64-row steps
// of the read leave alone, so row block r of k-step pk adds the constant (64 pk + 16 r) * DV.
template <int DV>
__device__ __forceinline__ uint32_t v_lane_offset(int n, int lane) {
  constexpr int VCH = DV / 16;
  const int hgrp = lane >> 5;
  const int trj = (lane & 15) >> 1;
  const int tr_key = 8 * (trj >> 2) + 4 * hgrp + (trj & 3);
  const int tr_chunk_hi = (lane >> 4) & 1;
  const int tr_byte = 8 * (lane & 1);
  return (uint32_t)(tr_key * DV + swz<VCH>(2 * n + tr_chunk_hi, v_sv(tr_key)) * 16 + tr_byte);
}

template <int D, int DV, int BN>
__device__ __forceinline__ void softmax_pv_tile(const FA8_LDS uint8_t* vt, const uint32_t (&voff)[DV / 32],
                                                v16f (&sacc)[BN / 32], float c, bool need_mask, int j0, int my_lo,
                                                int my_hi, int lane, float& m_run, float& nb, float& l_run,
                                                v16f (&oacc)[DV / 32]) {
  constexpr int KB = BN / 32;        // 32-key blocks of S^T
  constexpr int PK = BN / 64;        // 64-key k-steps of PV
  constexpr int NB = DV / 32;
  const int hgrp = lane >> 5;

  // ---- mask (only tiles that cross some row's key bounds): key j is visible iff
  //      my_lo <= j < my_hi, one unsigned compare (an empty row has span 0) ----
  if (need_mask) {
    const uint32_t span = (uint32_t)max(my_hi - my_lo, 0);
    const int base = j0 + 4 * hgrp - my_lo;
#pragma unroll
    for (int kb = 0; kb < KB; kb++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const uint32_t rel = (uint32_t)(base + kb * 32 + 8 * (r >> 2) + (r & 3));
        if (rel >= span) sacc[kb][r] = kNegInf;
      }
  }

  // ---- row max (lanes L and L^32 share a row), lazy rescale ----
  // four independent chains, so consecutive max instructions do not wait on each other
  float mxc[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
  for (int kb = 0; kb < KB; kb++)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mxc[(r >> 1) & 3] = max3f(mxc[(r >> 1) & 3], sacc[kb][r], sacc[kb][r + 1]);
  float mx = max3f(mxc[0], mxc[1], __builtin_elementwise_maximum(mxc[2], mxc[3]));
  mx = max_xor32(mx);
  const float mt = mx * c;
  // ---- rescale, only when some row of the wave moved its max (rare once the maxima settle): the
  //      new max, alpha = 2^(m_old - m_new) (0 when m_old = -inf), the exponent offset
  //      nb = 8 - m (kept across tiles) and O = alpha * O. The PV products below accumulate onto
  //      O on the matrix cores, whose accumulator input is added at fp32 precision on gfx950
  //      (measured: chained accumulation over 128k keys matches a separate fp32 fold of per-tile
  //      products to within 4e-6 of sum |p v|, with no drift), so no separate O_tile and fold are
  //      needed ----
  const bool up = mt - m_run > kTau;   // also true when m_run = -inf and mt is finite
  if (__builtin_amdgcn_ballot_w64(up)) {
    // O is still all zeros while every row of the wave had m = -inf (its first visible tile):
    // scaling it would change nothing
    const bool o_live = __builtin_amdgcn_ballot_w64(m_run != kNegInf) != 0;
    float alpha = 1.0f;
    if (up) {
      alpha = fast_exp2(m_run - mt);
      m_run = mt;
      nb = kBias - m_run;
    }
    l_run *= alpha;
    if (o_live) {
#pragma unroll
      for (int n = 0; n < NB; n++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[n][r] *= alpha;
    }
  }

  // ---- P = 2^(S*c - m + 8) as E4M3 in PV-operand order, its row sum on the matrix cores and
  //      O += V^T P^T. Each 64-key half's PV MFMAs follow its own exponentials, so they overlap
  //      those of the next half. Row sum: P as the B operand of the 16x16x128 MFMA, whose column
  //      j collects lanes j, j+16, j+32 and j+48 (both key halves of query rows j and j+16); a
  //      selector A operand (E4M3 1.0 = 0x38 in lane i+16q when q%2 == (i/4)%2, else 0) makes
  //      output rows 4(L/16) .. +3 of lane L the sum over the keys of query row L%32, the lane's
  //      own row, at half the MFMA work of a 32x32 product ----
  const int sel = (((lane >> 4) & 1) == (((lane & 15) >> 2) & 1)) ? 0x38383838 : 0;
  const v8i rsel = {sel, sel, sel, sel, sel, sel, sel, sel};
  auto v_operand = [&](int pk, int n) {
    v8i vop;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA8_LDS v2i*)(vt + voff[n] + (64 * pk + 16 * r) * DV));
      vop[2 * r] = x[0];
      vop[2 * r + 1] = x[1];
    }
    return vop;
  };
  v4f rs;
#pragma unroll
  for (int pk = 0; pk < PK; pk++) {
    v8i pop;
#pragma unroll
    for (int w = 0; w < 8; w++) {
      const int kb = 2 * pk + (w >> 2), r0 = 4 * (w & 3);
      const float p0 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 0], c, nb));
      const float p1 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 1], c, nb));
      const float p2 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 2], c, nb));
      const float p3 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 3], c, nb));
      int word = cvt_pk_fp8_lo(p0, p1);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
      pop[w] = word;
    }
#pragma unroll
    for (int n = 0; n < NB; n++) oacc[n] = mfma_32x32x64_fp8(v_operand(pk, n), pop, oacc[n]);
    // the row sum after the PV MFMAs of the half: its result is read last
    rs = (pk == 0) ? mfma_16x16x128_fp8(rsel, pop, (v4f){0.0f, 0.0f, 0.0f, 0.0f}) : mfma_16x16x128_fp8(rsel, pop, rs);
  }
  l_run += rs[0];
}

// One KV tile of BN keys (LDS K tile at kt, V tile at vt, both row-major and swizzled) for the
// 32 query rows of this wave. Updates the running max m, row sum l and O accumulators.
template <int D, int DV, int BN>
__device__ __forceinline__ void attn_tile(const FA8_LDS uint8_t* kt, const FA8_LDS uint8_t* vt,
                                          const v8i (&qop)[(D + 63) / 64], float c, bool need_mask, int j0,
                                          int my_lo, int my_hi, int lane, const uint32_t (&voff)[DV / 32],
                                          float& m_run, float& nb, float& l_run, v16f (&oacc)[DV / 32]) {
  v16f sacc[BN / 32];
  qk_tile<D, BN>(kt, qop, lane, sacc);
  softmax_pv_tile<D, DV, BN>(vt, voff, sacc, c, need_mask, j0, my_lo, my_hi, lane, m_run, nb, l_run, oacc);
}

// One 64-key tile for decode, on the 16x16x128 FP8 MFMA: NQB blocks of 16 query rows (decode
// rows are few, so 16-wide blocks waste less than 32-wide ones). Lane L owns query row L%16 of
// each block and the keys 16kb + 4*(L/16) + r of the S^T accumulators; the PV product runs over
// a 128-key contraction whose upper 64 keys are zero (the tile has 64). Row max and row sum
// combine the four lanes L, L^16, L^32, L^48 of a row.
template <int D, int DV, int NQB>
__device__ __forceinline__ void attn_tile16(const FA8_LDS uint8_t* kt, const FA8_LDS uint8_t* vt,
                                            const v8i (&qop)[NQB][(D + 127) / 128], float c, bool need_mask,
                                            int j0, const int (&my_lo)[NQB], const int (&my_hi)[NQB], int lane,
                                            float (&m_run)[NQB], float (&l_run)[NQB],
                                            v4f (&oacc)[NQB][DV / 16]) {
  constexpr int KS = (D + 127) / 128;
  constexpr int NB = DV / 16;
  constexpr int KCH = D / 16, VCH = DV / 16;
  const int h = lane >> 4, l16 = lane & 15;

  // ---- S^T = K Q^T: 4 blocks of 16 keys ----
  v4f sacc[NQB][4];
#pragma unroll
  for (int kb = 0; kb < 4; kb++) {
#pragma unroll
    for (int qb = 0; qb < NQB; qb++) sacc[qb][kb] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    const int row = kb * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const int off = ks * 128 + h * 32;
      v8i kop = {0, 0, 0, 0, 0, 0, 0, 0};
      if (off < D) {
        const int ch = off >> 4;
        const v4i a = *(const FA8_LDS v4i*)(kt + row * D + swz<KCH>(ch, k_sv<D>(row)) * 16);
        const v4i a2 = *(const FA8_LDS v4i*)(kt + row * D + swz<KCH>(ch + 1, k_sv<D>(row)) * 16);
        kop = (v8i){a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
      }
#pragma unroll
      for (int qb = 0; qb < NQB; qb++) sacc[qb][kb] = mfma_16x16x128_fp8(kop, qop[qb][ks], sacc[qb][kb]);
    }
  }

  v8i pop[NQB];
  float alpha[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; qb++) {
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 4; kb++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int j = j0 + kb * 16 + 4 * h + r;
          if (j < my_lo[qb] || j >= my_hi[qb]) sacc[qb][kb][r] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; kb++) mx = fmaxf(mx, fmaxf(fmaxf(sacc[qb][kb][0], sacc[qb][kb][1]),
                                                     fmaxf(sacc[qb][kb][2], sacc[qb][kb][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt = mx * c;
    alpha[qb] = 1.0f;
    if (mt - m_run[qb] > kTau) {
      alpha[qb] = fast_exp2(m_run[qb] - mt);
      m_run[qb] = mt;
    }
    const float nb = (m_run[qb] == kNegInf) ? 0.0f : kBias - m_run[qb];
    float lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const float p0 = fast_exp2(__builtin_fmaf(sacc[qb][w][0], c, nb));
      const float p1 = fast_exp2(__builtin_fmaf(sacc[qb][w][1], c, nb));
      const float p2 = fast_exp2(__builtin_fmaf(sacc[qb][w][2], c, nb));
      const float p3 = fast_exp2(__builtin_fmaf(sacc[qb][w][3], c, nb));
      int word = cvt_pk_fp8_lo(p0, p1);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
      pop[qb][w] = word;
      pop[qb][w + 4] = 0;
      const auto r01 = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
      const auto r23 = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
      lsum += (r01[0] + r01[1]) + (r23[0] + r23[1]);
    }
    l_run[qb] = alpha[qb] * l_run[qb] + lsum;
  }

  // ---- O_tile = V^T P^T from zero, then O = alpha * O + O_tile ----
  const int trj = l16 >> 1;
  const int tr_key = 16 * (trj >> 2) + 4 * h + (trj & 3);
  const int tr_byte = 8 * (lane & 1);
#pragma unroll
  for (int n = 0; n < NB; n++) {
    v8i vop = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 2; r++) {
      const int row = 32 * r + tr_key;
      const int off = row * DV + swz<VCH>(n, v_sv16(row)) * 16 + tr_byte;
      const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA8_LDS v2i*)(vt + off));
      vop[2 * r] = x[0];
      vop[2 * r + 1] = x[1];
    }
#pragma unroll
    for (int qb = 0; qb < NQB; qb++) {
      const v4f ot = mfma_16x16x128_fp8(vop, pop[qb], (v4f){0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
      for (int r = 0; r < 4; r++) oacc[qb][n][r] = __builtin_fmaf(alpha[qb], oacc[qb][n][r], ot[r]);
    }
  }
}

// Final normalization and store of one lane's row (or its partial for split-KV decode). bias
// is P's exponent offset (8 for E4M3 P, 0 for MXFP8 P, whose block scales carry the range).
// Without SPLIT, a learnable sink logit z (p.sink) joins the row sum here with the same
// offset as P: the stored max m rises to z2 = z log2 e when z2 is larger (alpha = 2^(m - m')
// rescales l and O; every term stays below 2^8), then l += 2^(z2 - m' + 8). Split partials
// leave the sink to the combine.
// Output scale and LSE of one row at the end of its key range: O = O_acc * dvs / l,
// LSE = ln 2 * (m + log2 l - bias). With a sink logit z (when with_sink), the stored max is
// first raised to z log2 e if that is larger, and the sink's term 2^(z log2 e - m + bias)
// joins l; a row with no visible key and no sink gets O = 0 and LSE = -inf.
struct RowScale {
  float inv, lse;
};
__device__ __forceinline__ RowScale row_scale(const KParams& p, bool with_sink, int qh, float m_run, float l_tot,
                                              float dvs, float bias) {
  const float z2 = (with_sink && p.sink) ? p.sink[qh] * kLog2e : kNegInf;
  if (z2 != kNegInf) {
    const float mf = fmaxf(m_run, z2);
    const float a = (m_run == kNegInf) ? 0.0f : fast_exp2(m_run - mf);
    l_tot = a * l_tot + fast_exp2(z2 - mf + bias);
    dvs *= a;
    m_run = mf;
  }
  const bool nonempty = l_tot > 0.0f;
  return {nonempty ? dvs / l_tot : 0.0f, nonempty ? (m_run + __log2f(l_tot) - bias) * kLn2 : kNegInf};
}

// Final output of one wave's 32 rows for DV in {64, 128, 256} when the output allows 16-byte
// stores: the MFMA layout leaves each lane 4-column pieces of its row, so a direct store writes
// 8 bytes into each of 32 rows per instruction. Instead the wave stages its rows in LDS
// (`stage`: 32 rows x DV halves, its own region; every 16-byte chunk c of row r at chunk
// c ^ (r mod DV/8), which spreads both the writes and the row reads over the banks) and writes
// whole rows with 16-byte lanes. Rows past row_last are staged but not stored.
template <int DV, bool FP16>
__device__ __forceinline__ void store_rows_staged_t(const KParams& p, const v16f (&oacc)[DV / 32], float inv, int lane,
                                                    int b, int q0, int row0, int row_last, int qh,
                                                    FA8_LDS uint8_t* stage) {
  constexpr int NB = DV / 32;
  constexpr int CPR = DV / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;   // rows per store instruction
  constexpr int NI = 32 / RPI;    // store instructions per wave
  static_assert(CPR * RPI == 64 && (CPR & (CPR - 1)) == 0, "rows must split into 16-byte lanes");
  const int hgrp = lane >> 5, lrow = lane & 31;
  // lane (row lrow, half hgrp) holds columns 32n + 8q4 + 4hgrp .. +3: half hgrp of chunk 4n + q4
#pragma unroll
  for (int n = 0; n < NB; n++)
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
      const int c = 4 * n + q4;
      const int pos = lrow * (2 * DV) + ((c ^ (lrow & (CPR - 1))) << 4) + 8 * hgrp;
      *(FA8_LDS v2i*)(stage + pos) = pack4_half(oacc[n][4 * q4] * inv, oacc[n][4 * q4 + 1] * inv,
                                                oacc[n][4 * q4 + 2] * inv, oacc[n][4 * q4 + 3] * inv, FP16);
    }
  // the reads below take chunks other lanes of this wave wrote: the wave's LDS operations are
  // performed in order, and the fence keeps the compiler from moving a read above a write
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const int rr = lane / CPR, c = lane % CPR;
  // every read first (all 32 staged rows are in bounds), then the stores of the rows that exist
  v4i x[NI];
#pragma unroll
  for (int i = 0; i < NI; i++) {
    const int r = RPI * i + rr;
    x[i] = *(const FA8_LDS v4i*)(stage + r * (2 * DV) + ((c ^ (r & (CPR - 1))) << 4));
  }
#pragma unroll
  for (int i = 0; i < NI; i++) {
    const int qi = row0 + RPI * i + rr;
    if (qi <= row_last) {
      const int64_t off = (p.cu_q ? (int64_t)(q0 + qi) * p.o_rs : (int64_t)b * p.o_bs + (int64_t)qi * p.o_rs) +
                          (int64_t)qh * p.o_hs + 8 * c;
      *reinterpret_cast<v4i*>(reinterpret_cast<uint16_t*>(p.out) + off) = x[i];
    }
  }
}
template <int DV>
__device__ __forceinline__ void store_rows_staged(const KParams& p, const v16f (&oacc)[DV / 32], float inv, int lane,
                                                  int b, int q0, int row0, int row_last, int qh,
                                                  FA8_LDS uint8_t* stage) {
  // the output type is chosen once, outside the conversion and store loops
  if (p.out_fp16) store_rows_staged_t<DV, true>(p, oacc, inv, lane, b, q0, row0, row_last, qh, stage);
  else store_rows_staged_t<DV, false>(p, oacc, inv, lane, b, q0, row0, row_last, qh, stage);
}

template <int DV, bool SPLIT>
__device__ __forceinline__ void store_row(const KParams& p, const v16f (&oacc)[DV / 32], float m_run, float l_tot,
                                          float dvs, int hgrp, int b, int q0, int qi, int qh, int split,
                                          float bias = kBias) {
  constexpr int NB = DV / 32;
  const RowScale rsc = row_scale(p, !SPLIT, qh, m_run, l_tot, dvs, bias);
  const float inv = rsc.inv, lse = rsc.lse;
  if constexpr (SPLIT) {
    const int64_t prow = (((int64_t)split * p.batch + b) * p.max_sq + qi) * p.hq + qh;
    float* orow = p.o_part + prow * DV;
#pragma unroll
    for (int n = 0; n < NB; n++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        const int dvi = 32 * n + 8 * q4 + 4 * hgrp;
        v4f v = {oacc[n][4 * q4] * inv, oacc[n][4 * q4 + 1] * inv, oacc[n][4 * q4 + 2] * inv,
                 oacc[n][4 * q4 + 3] * inv};
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

// ------------------------------------------------------------------------------------------
// Full forward pass: 4 waves x 32 query rows of one query head; KV tiles of BN keys staged in
// LDS by direct global->LDS loads (two stages, so the next tile lands while this one is used).
// Workgroups are numbered so that each XCD (workgroup id mod 8) receives a contiguous run of
// the work list, ordered by (batch, kv head), so the workgroups that share K/V share an L2.
// With per-sequence lengths (varlen or seqused_k) a contiguous run would hand whole sequences
// of very different lengths to single XCDs, so there (p.bk8 > 0) the (batch, kv head) groups
// are dealt to the XCDs round-robin instead, row block by row block, the deal rotating by
// one XCD every kRankChunk row blocks: every XCD sees every sequence, and the row blocks of
// one group that lie close together (and share K/V) still meet in one L2. Rank r there is each
// sequence's own r-th row block counted from its last one (causal) or first one, so the ranks
// that only some sequences have come last. Within one rank the groups' order rotates by one
// group per rank: an XCD hands its workgroups to its shader engines in a fixed rotation by
// dispatch position and dispatches in order, so a sequence that kept its position from rank to
// rank would keep its shader engines, fill them while the others idle, and stall the dispatch.
// ------------------------------------------------------------------------------------------
constexpr int kRankChunk = 8;

struct PrefillWork {
  int bk, mbi, hg;   // (batch * hkv + kv head), row-block rank, q head within the kv group
};

__device__ __forceinline__ PrefillWork prefill_work(const KParams& p) {
  const int L = (int)blockIdx.x;
  const int xcd = L & 7, slot = L >> 3;
  const int g = p.g;
  PrefillWork wk;
  if (p.bk8 == 0) {
    const int nwork = (int)gridDim.x;
    const int per = nwork >> 3, rem = nwork & 7;
    const int w = xcd * per + min(xcd, rem) + slot;
    wk.hg = w % g;
    const int t1 = w / g;
    wk.mbi = t1 % p.nmb;
    wk.bk = t1 / p.nmb;
  } else {
    // grid = 8 * bk8 * nmb * g; XCD x takes at rank r the groups bk = ((x - r/kRankChunk) mod 8) + 8 i,
    // i = (j + r) mod bk8 at the rank's j-th position
    wk.hg = slot % g;
    const int t1 = slot / g;
    wk.mbi = t1 / p.bk8;
    const int i = (t1 % p.bk8 + wk.mbi % p.bk8) % p.bk8;
    wk.bk = ((xcd - wk.mbi / kRankChunk) & 7) + 8 * i;   // >= batch * hkv: no work
  }
  return wk;
}
template <int D, int DV, int BN, bool PAGED>
__global__ void __launch_bounds__(256, 2) fa8_prefill_kernel(const KParams p) {
  constexpr int NW = 4, BM = NW * 32;
  constexpr int KTILE = BN * D, VTILE = BN * DV, STAGE = KTILE + VTILE;
  constexpr int KINST = KTILE / 1024 / NW, VINST = VTILE / 1024 / NW;   // 1 KB DMA loads per wave
  static_assert(KTILE % (1024 * NW) == 0 && VTILE % (1024 * NW) == 0, "tile must split into 1 KB loads");
  constexpr int KCH = D / 16, VCH = DV / 16;
  constexpr int NB = DV / 32;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps LDS tile addresses scalar
  const int hgrp = lane >> 5, lrow = lane & 31;

  // ---- XCD-aware work index ----
  const int g = p.g;
  const PrefillWork wk = prefill_work(p);
  if (wk.bk >= p.batch * p.hkv) return;   // uniform: a slot of the round-robin deal with no group
  const int hg = wk.hg, mbi = wk.mbi;
  const int kvh = wk.bk % p.hkv, b = wk.bk / p.hkv;
  const int qh = kvh * g + hg;

  const SeqInfo si = seq_info(p, b);
  // causal: heaviest row blocks first; with per-sequence lengths the ranks count from each
  // sequence's own last row block
  const int nmb_b = p.bk8 ? (si.sq + BM - 1) / BM : p.nmb;
  const int mblock = p.causal ? nmb_b - 1 - mbi : mbi;
  const int rb0 = mblock * BM;
  if (mblock < 0 || rb0 >= si.sq) return;  // uniform: no valid row in this block
  const int rb1 = min(rb0 + BM, si.sq) - 1;
  const RowRange rr{si.sk, si.sk - si.sq, p.wl, p.wr};
  int wg_lo = rr.lo(rb0), wg_hi = rr.hi(rb1);
  const int full_lo = rr.lo(rb1), full_hi = rr.hi(rb0);
  if (wg_hi <= wg_lo) { wg_lo = 0; wg_hi = 0; }
  const int t_begin = wg_lo / BN;
  const int t_end = wg_hi > wg_lo ? (wg_hi + BN - 1) / BN : t_begin;

  const int qi = rb0 + wave * 32 + lrow;
  const bool valid = qi <= rb1;
  int my_lo = 0, my_hi = 0;
  if (valid) {
    my_lo = rr.lo(qi);
    my_hi = rr.hi(qi);
  }
  // keys any row of this wave sees: a tile outside them would add exact zeros (P = 0, no
  // rescale), so the wave skips its math (it still copies its share and meets the barriers)
  const int w_first = rb0 + wave * 32, w_last = min(w_first + 31, rb1);
  int wv_lo = 0, wv_hi = 0;
  if (w_first <= rb1) {
    wv_lo = rr.lo(w_first);
    wv_hi = rr.hi(w_last);
  }

  const float dq = load_descale(p.dq, p.dq_sb, p.dq_sh, b, kvh);
  const float dk = load_descale(p.dk, p.dk_sb, p.dk_sh, b, kvh);
  const float dvs = load_descale(p.dv, p.dv_sb, p.dv_sh, b, kvh);
  const float c = p.scale_log2 * dq * dk;

  v8i qop[(D + 63) / 64];
  load_q<D>(p.q + (p.cu_q ? (int64_t)(si.q0 + qi) * p.q_rs : (int64_t)b * p.q_bs + (int64_t)qi * p.q_rs) +
                (int64_t)qh * p.q_hs,
            valid, hgrp, qop);

  const KvAddr ka = kv_addr(p, b, kvh);
  // Direct global->LDS loads of tile t into stage st. Load instruction i of this wave fills
  // LDS bytes [1024*(wave*KINST + i), +1024) of the K tile, lane L its 16 bytes at 16*L: that
  // position is physical chunk pc of row r, which holds logical chunk swz(pc) (an involution).
  // Contiguous K/V: a buffer descriptor per tile whose range ends at the sequence's last row, and
  // per-lane offsets fixed for the whole loop; rows past the sequence read as zeros (masked to
  // P = 0, and 0 * V = 0). Paged K/V: per-lane addresses through the block table; rows past the
  // sequence read its last valid row.
  uint32_t k_off[KINST], v_off[VINST];
#pragma unroll
  for (int i = 0; i < KINST; i++) {
    const int pos = (wave * KINST + i) * 1024 + lane * 16;
    const int row = pos / D, pc = (pos - row * D) >> 4;
    k_off[i] = (uint32_t)(row * (int)ka.k_rs + swz<KCH>(pc, k_sv<D>(row)) * 16);
  }
#pragma unroll
  for (int i = 0; i < VINST; i++) {
    const int pos = (wave * VINST + i) * 1024 + lane * 16;
    const int row = pos / DV, pc = (pos - row * DV) >> 4;
    v_off[i] = (uint32_t)(row * (int)ka.v_rs + swz<VCH>(pc, v_sv(row)) * 16);
  }
  // LDS destination of this wave's first copy instruction into stage 0 (K, then V), uniform
  const uint32_t kdst0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((FA8_LDS uint8_t*)smem + wave * KINST * 1024));
  const uint32_t vdst0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)reinterpret_cast<uintptr_t>((FA8_LDS uint8_t*)smem + KTILE + wave * VINST * 1024));
  auto dma_tile = [&](int t, int st) {
    FA8_LDS uint8_t* kt = (FA8_LDS uint8_t*)smem + st * STAGE;
    FA8_LDS uint8_t* vt = kt + KTILE;
    const int j0 = t * BN;
    if constexpr (!PAGED) {
      // valid rows of the tile: at most BN rows x row stride < 2^31 bytes (checked on the host)
      const int rows = min(si.sk - j0, BN);
      const v4i kr = buffer_rsrc(p.k + ka.kbase + (int64_t)j0 * ka.k_rs, (uint32_t)((rows - 1) * (int)ka.k_rs + D));
      const v4i vr = buffer_rsrc(p.v + ka.vbase + (int64_t)j0 * ka.v_rs, (uint32_t)((rows - 1) * (int)ka.v_rs + DV));
#pragma unroll
      for (int i = 0; i < KINST; i++) buffer_copy16_to_lds(kr, k_off[i], kdst0 + st * STAGE + i * 1024);
#pragma unroll
      for (int i = 0; i < VINST; i++) buffer_copy16_to_lds(vr, v_off[i], vdst0 + st * STAGE + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < KINST; i++) {
        const int blk = wave * KINST + i;
        const int pos = blk * 1024 + lane * 16;
        const int row = pos / D, pc = (pos - row * D) >> 4;
        const int j = min(j0 + row, si.sk - 1);
        copy16_to_lds_vaddr(p.k + ka.k(j) + swz<KCH>(pc, k_sv<D>(row)) * 16,
                            (uint32_t)reinterpret_cast<uintptr_t>(kt + blk * 1024));
      }
#pragma unroll
      for (int i = 0; i < VINST; i++) {
        const int blk = wave * VINST + i;
        const int pos = blk * 1024 + lane * 16;
        const int row = pos / DV, pc = (pos - row * DV) >> 4;
        const int j = min(j0 + row, si.sk - 1);
        copy16_to_lds_vaddr(p.v + ka.v(j) + swz<VCH>(pc, v_sv(row)) * 16,
                            (uint32_t)reinterpret_cast<uintptr_t>(vt + blk * 1024));
      }
    }
  };

  // per-lane V operand offsets, computed once and held in registers for the whole loop (the
  // empty asm keeps the compiler from recomputing them in every tile)
  uint32_t voff[NB];
#pragma unroll
  for (int n = 0; n < NB; n++) {
    voff[n] = v_lane_offset<DV>(n, lane);
    __asm__ __volatile__("" : "+v"(voff[n]));
  }
  float m_run = kNegInf, nb = 0.0f, l_run = 0.0f;   // nb = 8 - m_run (0 while m_run = -inf)
  v16f oacc[NB];
#pragma unroll
  for (int n = 0; n < NB; n++)
#pragma unroll
    for (int r = 0; r < 16; r++) oacc[n][r] = 0.0f;

  if (t_begin < t_end) {
    dma_tile(t_begin, 0);
    wait_vmcnt<0>();
    __syncthreads();
  }
  // Tile t uses stage (t - t_begin) & 1. For d + dv <= 256 the loop runs two tiles per iteration
  // so that each tile's stage is a constant: the LDS operand addresses are then one per-lane
  // register plus an immediate offset, with no per-tile address arithmetic (larger head dims keep
  // one tile per iteration: the second copy of the loop body would not fit their registers).
  auto tile = [&](int t, auto stage) __attribute__((always_inline)) {
    const int st = stage;
    if (t + 1 < t_end) dma_tile(t + 1, st ^ 1);
    const FA8_LDS uint8_t* kt = (const FA8_LDS uint8_t*)smem + st * STAGE;
    const int j0 = t * BN;
    const bool need_mask = (j0 < full_lo) || (j0 + BN > full_hi);
    if (j0 < wv_hi && j0 + BN > wv_lo)
      attn_tile<D, DV, BN>(kt, kt + KTILE, qop, c, need_mask, j0, my_lo, my_hi, lane, voff, m_run, nb, l_run, oacc);
    wait_vmcnt<0>();   // this wave's loads of tile t+1 have landed in LDS
    __syncthreads();   // ... and every other wave's; all reads of stage st are done
  };
  if constexpr (D + DV <= 256) {
    int t = t_begin;
    for (; t + 1 < t_end; t += 2) {
      tile(t, std::integral_constant<int, 0>{});
      tile(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < t_end) tile(t, std::integral_constant<int, 0>{});
  } else {
    for (int t = t_begin; t < t_end; t++) tile(t, (t - t_begin) & 1);
  }

  const float l_tot = l_run;   // the MFMA row sums already cover both lanes of a row
  if constexpr (DV == 64 || DV == 128 || DV == 256) {
    static_assert(NW * 32 * 2 * DV <= 2 * STAGE, "the staged output must fit in the two tile stages");
    if (p.o_vec16) {
      // the loop ended on a barrier with no copy in flight: the tile stages are free
      const RowScale rsc = row_scale(p, true, qh, m_run, l_tot, dvs, kBias);
      if (valid && hgrp == 0 && p.lse) {
        const int64_t loff = p.cu_q ? (int64_t)qh * p.l_hs + (int64_t)(si.q0 + qi) * p.l_rs
                                    : (int64_t)b * p.l_bs + (int64_t)qh * p.l_hs + (int64_t)qi * p.l_rs;
        p.lse[loff] = rsc.lse;
      }
      store_rows_staged<DV>(p, oacc, rsc.inv, lane, b, si.q0, rb0 + wave * 32, rb1, qh,
                            (FA8_LDS uint8_t*)smem + wave * (32 * 2 * DV));
      return;
    }
  }
  if (!valid) return;
  store_row<DV, false>(p, oacc, m_run, l_tot, dvs, hgrp, b, si.q0, qi, qh, 0);
}

// ------------------------------------------------------------------------------------------
// MXFP8 forward pass (the MXFP8 forward of the FlashAttention-4 MXFP8 page, sections 2.1 and
// 2.1.3). The structure of fa8_prefill_kernel; both products run on the block-scaled MFMA,
// which applies one E8M0 scale per lane to the 32 contraction elements that scale covers.
// Measured lane layout of v_mfma_scale_f32_32x32x64_f8f6f4: the scale byte of lane L scales
// hardware k-block L/32 of row (A) or column (B) L%32, and k-block t is dwords 4t..4t+3 of BOTH
// lanes of that row (L%32 and L%32+32). So:
//  * Q and K (blocks of 32 along d): lane half h loads d-chunks 4ks+h and 4ks+2+h (16 bytes
//    each) of k-step ks, which puts d [64ks, 64ks+32) in k-block 0 and [64ks+32, 64ks+64) in
//    k-block 1, and supplies the scale of d-block 2ks+h;
//  * P and V (blocks of 32 keys): the S^T accumulator order already puts keys [64pk, 64pk+32)
//    of a 64-key step in dwords 0-3 of both lane halves and keys [64pk+32, 64pk+64) in dwords
//    4-7 (and the transposed V reads follow the same key order), so lane half h supplies the
//    scales of key block 2pk+h.
// Per query row and 32-key block, the block's max x_b (log2 units) gives the shared exponent
// X = ceil(x_b - m - log2 448) (m the running max), the smallest power of two that brings the
// block's largest P = 2^(x_b - m) to at most 448 (computed with a margin of a few ulps, so that
// fp32 rounding cannot push it past 448), clamped to [-127, 127]; P = 2^(x - m - X) is rounded
// to E4M3 with scale byte X + 127. Each block's max comes from the row max's own reduction (two
// lanes hold a block's 32 keys), so no extra pass over P is needed.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ v16f mfma_32x32x64_mx(v8i a, v8i b, v16f c, int sa, int sb) {
  // E4M3 operands; opsel 0 takes each lane's scale from byte 0 of sa / sb
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Q row of this lane as the B operand in the block-scaled order: k-step ks takes d-chunks
// 4ks+h and 4ks+2+h (h = lane half).
template <int D>
__device__ __forceinline__ void load_q_mx(const uint8_t* qrow, bool valid, int hgrp, v8i (&qop)[D / 64]) {
#pragma unroll
  for (int ks = 0; ks < D / 64; ks++) {
    v4i a = {0, 0, 0, 0}, a2 = {0, 0, 0, 0};
    if (valid) {
      a = ld_global16(qrow + (4 * ks + hgrp) * 16);
      a2 = ld_global16(qrow + (4 * ks + 2 + hgrp) * 16);
    }
    qop[ks] = (v8i){a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
  }
}

// One BN-key tile with MXFP8 operands. kt/vt: K and V tiles (row-major, swizzled); ksc: the
// tile's K scales [BN][D/32]; vsc: its V scales [BN/32][DV]; qsc: this lane's Q scale bytes
// (d-block 2ks + h for k-step ks).
template <int D, int DV, int BN>
__device__ __forceinline__ void attn_tile_mx(const FA8_LDS uint8_t* kt, const FA8_LDS uint8_t* vt,
                                             const FA8_LDS uint8_t* ksc, const FA8_LDS uint8_t* vsc,
                                             const v8i (&qop)[D / 64], const int (&qsc)[D / 64], float c,
                                             bool need_mask, int j0, int my_lo, int my_hi, int lane, float& m_run,
                                             float& l_run, v16f (&oacc)[DV / 32]) {
  constexpr int KB = BN / 32, PK = BN / 64, KS = D / 64, NB = DV / 32, KCH = D / 16, NBD = D / 32;
  const int hgrp = lane >> 5, lrow = lane & 31;

  // ---- S^T = K Q^T, each k-step scaled by the K and Q block scales ----
  v16f sacc[KB];
  const FA8_LDS uint8_t* ksc_lane = ksc + lrow * NBD;             // key row lrow of block 0
#pragma unroll
  for (int kb = 0; kb < KB; kb++) {
    const int row = kb * 32 + lrow;
    // this key row's D/32 scale bytes
    const uint32_t kw = (NBD == 4) ? *(const FA8_LDS uint32_t*)(ksc_lane + kb * 32 * NBD)
                                   : (uint32_t)*(const FA8_LDS uint16_t*)(ksc_lane + kb * 32 * NBD);
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const v4i a = *(const FA8_LDS v4i*)(kt + row * D + swz<KCH>(4 * ks + hgrp, k_sv<D>(row)) * 16);
      const v4i a2 = *(const FA8_LDS v4i*)(kt + row * D + swz<KCH>(4 * ks + 2 + hgrp, k_sv<D>(row)) * 16);
      const v8i kop = {a[0], a[1], a[2], a[3], a2[0], a2[1], a2[2], a2[3]};
      const int sa = (int)((kw >> (8 * (2 * ks + hgrp))) & 0xffu);
      sacc[kb] = (ks == 0) ? mfma_32x32x64_mx(kop, qop[0], (v16f){}, sa, qsc[0])
                           : mfma_32x32x64_mx(kop, qop[ks], sacc[kb], sa, qsc[ks]);
    }
    __builtin_amdgcn_sched_barrier(0);   // bounds how far the K operand reads run ahead
  }

  // ---- mask ----
  if (need_mask) {
    const uint32_t span = (uint32_t)max(my_hi - my_lo, 0);
    const int base = j0 + 4 * hgrp - my_lo;
#pragma unroll
    for (int kb = 0; kb < KB; kb++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const uint32_t rel = (uint32_t)(base + kb * 32 + 8 * (r >> 2) + (r & 3));
        if (rel >= span) sacc[kb][r] = kNegInf;
      }
  }

  // ---- per 32-key block max (two lanes hold a block's keys), row max, lazy rescale ----
  float bmax[KB];
#pragma unroll
  for (int kb = 0; kb < KB; kb++) {
    float m0 = max3f(sacc[kb][0], sacc[kb][1], sacc[kb][2]);
    float m1 = max3f(sacc[kb][3], sacc[kb][4], sacc[kb][5]);
    m0 = max3f(m0, sacc[kb][6], sacc[kb][7]);
    m1 = max3f(m1, sacc[kb][8], sacc[kb][9]);
    m0 = max3f(m0, sacc[kb][10], sacc[kb][11]);
    m1 = max3f(m1, sacc[kb][12], sacc[kb][13]);
    m0 = max3f(m0, sacc[kb][14], sacc[kb][15]);
    bmax[kb] = max_xor32(__builtin_elementwise_maximum(m0, m1));
  }
  float mx = bmax[0];
#pragma unroll
  for (int kb = 1; kb < KB; kb++) mx = __builtin_elementwise_maximum(mx, bmax[kb]);
  const float mt = mx * c;
  float alpha = 1.0f;
  if (mt - m_run > kTau) {
    alpha = fast_exp2(m_run - mt);
    m_run = mt;
  }

  // ---- P per 32-key block: shared exponent X, E4M3(2^(x - m - X)), scale X + 127 ----
  int pscale[KB];
  float nbk[KB];
  // X is raised by a margin of a few fp32 ulps of m (and exp2's own), so that the largest P of a
  // block cannot round past 448 and no clamp per element is needed
  const float margin = __builtin_fmaf(fabsf(m_run), 0x1p-21f, 0x1p-12f);
#pragma unroll
  for (int kb = 0; kb < KB; kb++) {
    const float y = bmax[kb] * c - m_run;                   // -inf for an all-masked block
    const float xe = (m_run == kNegInf) ? -127.0f : fmaxf(ceilf(y - kLog2E4M3Max + margin), -127.0f);
    pscale[kb] = (int)xe + 127;
    nbk[kb] = (m_run == kNegInf) ? 0.0f : -(m_run + xe);
  }
  // O = alpha O only when some row of the wave moved its max; the PV products then accumulate
  // onto O on the matrix cores (their accumulator input is added at fp32 precision, as in
  // attn_tile). P of each 64-key half, its PV MFMAs (V block scale x P block scale) right after
  // its exponentials, so they overlap those of the next half, and its row-sum MFMA.
  if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
    for (int n = 0; n < NB; n++)
#pragma unroll
      for (int r = 0; r < 16; r++) oacc[n][r] *= alpha;
  }
  const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838};
  const FA8_LDS uint8_t* vsc_lane = vsc + hgrp * DV + lrow;        // block hgrp, column lrow
  v16f rs;
#pragma unroll
  for (int pk = 0; pk < PK; pk++) {
    v8i pop;
#pragma unroll
    for (int w = 0; w < 8; w++) {
      const int kb = 2 * pk + (w >> 2), r0 = 4 * (w & 3);
      const float p0 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 0], c, nbk[kb]));
      const float p1 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 1], c, nbk[kb]));
      const float p2 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 2], c, nbk[kb]));
      const float p3 = fast_exp2(__builtin_fmaf(sacc[kb][r0 + 3], c, nbk[kb]));
      int word = cvt_pk_fp8_lo(p0, p1);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
      pop[w] = word;
    }
    const int psc = hgrp ? pscale[2 * pk + 1] : pscale[2 * pk];   // this lane half's key block
#pragma unroll
    for (int n = 0; n < NB; n++) {
      __builtin_amdgcn_sched_barrier(0);   // one V operand read ahead at a time
      const int sa = (int)vsc_lane[2 * pk * DV + 32 * n];
      oacc[n] = mfma_32x32x64_mx(pv_operand_mx<DV>(vt, pk, n, lane), pop, oacc[n], sa, psc);
    }
    // row sum of the stored P times its scales
    rs = (pk == 0) ? mfma_32x32x64_mx(ones, pop, (v16f){}, 127, psc) : mfma_32x32x64_mx(ones, pop, rs, 127, psc);
  }
  l_run = alpha * l_run + rs[0];
}

// 4 waves x 32 query rows of one query head; K/V tiles by direct global->LDS copies (two
// stages), their scale blocks by ordinary loads stored to LDS before the end-of-tile barrier.
template <int D, int DV>
__global__ void __launch_bounds__(256, 2) fa8_prefill_mx_kernel(const KParams p) {
  constexpr int BN = 128, NW = 4, BM = NW * 32;
  constexpr int KTILE = BN * D, VTILE = BN * DV;
  constexpr int KSC = BN * (D / 32), VSC = (BN / 32) * DV;     // scale bytes per tile
  constexpr int STAGE = KTILE + VTILE + KSC + VSC;
  constexpr int KINST = KTILE / 1024 / NW, VINST = VTILE / 1024 / NW;
  static_assert(KTILE % (1024 * NW) == 0 && VTILE % (1024 * NW) == 0, "tile must split into 1 KB loads");
  static_assert(D == 64 || D == 128, "MX prefill head dims");
  constexpr int KCH = D / 16, VCH = DV / 16, NB = DV / 32, NBD = D / 32;
  constexpr int VLANES = VSC / 16;                            // lanes loading the V scales
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hgrp = lane >> 5, lrow = lane & 31;

  const int nwork = (int)gridDim.x;
  const int L = (int)blockIdx.x;
  const int xcd = L & 7, slot = L >> 3;
  const int per = nwork >> 3, rem = nwork & 7;
  const int w = xcd * per + min(xcd, rem) + slot;
  const int g = p.g;
  const int hg = w % g;
  const int t1 = w / g;
  const int mbi = t1 % p.nmb;
  const int bk = t1 / p.nmb;
  const int kvh = bk % p.hkv, b = bk / p.hkv;
  const int mblock = p.causal ? p.nmb - 1 - mbi : mbi;
  const int qh = kvh * g + hg;

  const SeqInfo si = seq_info(p, b);
  const int rb0 = mblock * BM;
  if (rb0 >= si.sq) return;
  const int rb1 = min(rb0 + BM, si.sq) - 1;
  const RowRange rr{si.sk, si.sk - si.sq, p.wl, p.wr};
  int wg_lo = rr.lo(rb0), wg_hi = rr.hi(rb1);
  const int full_lo = rr.lo(rb1), full_hi = rr.hi(rb0);
  if (wg_hi <= wg_lo) { wg_lo = 0; wg_hi = 0; }
  const int t_begin = wg_lo / BN;
  const int t_end = wg_hi > wg_lo ? (wg_hi + BN - 1) / BN : t_begin;

  const int qi = rb0 + wave * 32 + lrow;
  const bool valid = qi <= rb1;
  int my_lo = 0, my_hi = 0;
  if (valid) {
    my_lo = rr.lo(qi);
    my_hi = rr.hi(qi);
  }
  const float c = p.scale_log2;

  v8i qop[D / 64];
  load_q_mx<D>(p.q + (int64_t)b * p.q_bs + (int64_t)qi * p.q_rs + (int64_t)qh * p.q_hs, valid, hgrp, qop);
  int qsc[D / 64];
  {
    uint32_t qw = 0x7f7f7f7fu;
    if (valid) {
      const uint8_t* qs = p.q_mx + (int64_t)b * p.qmx_bs + (int64_t)qi * p.qmx_rs + (int64_t)qh * p.qmx_hs;
      qw = (NBD == 4) ? *(const uint32_t*)qs : (uint32_t)*(const uint16_t*)qs;
    }
#pragma unroll
    for (int ks = 0; ks < D / 64; ks++) qsc[ks] = (int)((qw >> (8 * (2 * ks + hgrp))) & 0xffu);
  }

  const KvAddr ka = kv_addr(p, b, kvh);
  uint32_t k_off[KINST], v_off[VINST];
#pragma unroll
  for (int i = 0; i < KINST; i++) {
    const int pos = (wave * KINST + i) * 1024 + lane * 16;
    const int row = pos / D, pc = (pos - row * D) >> 4;
    k_off[i] = (uint32_t)(row * (int)ka.k_rs + swz<KCH>(pc, k_sv<D>(row)) * 16);
  }
#pragma unroll
  for (int i = 0; i < VINST; i++) {
    const int pos = (wave * VINST + i) * 1024 + lane * 16;
    const int row = pos / DV, pc = (pos - row * DV) >> 4;
    v_off[i] = (uint32_t)(row * (int)ka.v_rs + swz<VCH>(pc, v_sv(row)) * 16);
  }
  auto dma_tile = [&](int t, int st) __attribute__((always_inline)) {
    FA8_LDS uint8_t* kt = (FA8_LDS uint8_t*)smem + st * STAGE;
    FA8_LDS uint8_t* vt = kt + KTILE;
    const int j0 = t * BN;
    const int rows = min(si.sk - j0, BN);
    const v4i kr = buffer_rsrc(p.k + ka.kbase + (int64_t)j0 * ka.k_rs, (uint32_t)((rows - 1) * (int)ka.k_rs + D));
    const v4i vr = buffer_rsrc(p.v + ka.vbase + (int64_t)j0 * ka.v_rs, (uint32_t)((rows - 1) * (int)ka.v_rs + DV));
#pragma unroll
    for (int i = 0; i < KINST; i++)
      buffer_copy16_to_lds(kr, k_off[i], (uint32_t)reinterpret_cast<uintptr_t>(kt + (wave * KINST + i) * 1024));
#pragma unroll
    for (int i = 0; i < VINST; i++)
      buffer_copy16_to_lds(vr, v_off[i], (uint32_t)reinterpret_cast<uintptr_t>(vt + (wave * VINST + i) * 1024));
  };
  // Scale blocks of tile t: threads 0..BN-1 read the D/32 K scale bytes of key j0 + tid (keys
  // past the sequence: any value, their scores are masked); threads BN..BN+VLANES-1 read 16
  // bytes of the tile's BN/32 V scale rows (blocks past the sequence: any value, their P is 0).
  const int64_t kmx_base = (int64_t)b * p.kmx_bs + (int64_t)kvh * p.kmx_hs;
  const int64_t vmx_base = (int64_t)b * p.vmx_bs + (int64_t)kvh * p.vmx_hs;
  const int nvblk = (si.sk + 31) / 32;
  auto load_scales = [&](int t) __attribute__((always_inline)) -> v4i {
    v4i x = {0x7f7f7f7f, 0x7f7f7f7f, 0x7f7f7f7f, 0x7f7f7f7f};
    if (tid < BN) {
      const int j = t * BN + tid;
      if (j < si.sk) {
        const uint8_t* src = p.k_mx + kmx_base + (int64_t)j * p.kmx_rs;
        x[0] = (NBD == 4) ? *(const int*)src : (int)*(const uint16_t*)src;
      }
    } else if (tid < BN + VLANES) {
      const int u = tid - BN;
      const int blk = t * (BN / 32) + u / (DV / 16), col = (u % (DV / 16)) * 16;
      if (blk < nvblk) x = ld_global16(p.v_mx + vmx_base + (int64_t)blk * p.vmx_ts + col);
    }
    return x;
  };
  auto store_scales = [&](v4i x, int st) __attribute__((always_inline)) {
    FA8_LDS uint8_t* ks = (FA8_LDS uint8_t*)smem + st * STAGE + KTILE + VTILE;
    if (tid < BN) {
      if constexpr (NBD == 4) *(FA8_LDS int*)(ks + tid * 4) = x[0];
      else *(FA8_LDS uint16_t*)(ks + tid * 2) = (uint16_t)x[0];
    } else if (tid < BN + VLANES) {
      *(FA8_LDS v4i*)(ks + KSC + (tid - BN) * 16) = x;
    }
  };

  float m_run = kNegInf, l_run = 0.0f;
  v16f oacc[NB];
#pragma unroll
  for (int n = 0; n < NB; n++)
#pragma unroll
    for (int r = 0; r < 16; r++) oacc[n][r] = 0.0f;

  // The scales of tile t+1 are read from global memory one iteration early and stored to LDS
  // at the start of tile t, next to that tile's K/V copies: nothing conditional follows the
  // tile's arithmetic in the loop body (the compiler would sink that arithmetic past it).
  v4i sc_next = {0, 0, 0, 0};
  if (t_begin < t_end) {
    dma_tile(t_begin, 0);
    store_scales(load_scales(t_begin), 0);
    sc_next = load_scales(t_begin + 1);
    wait_vmcnt<0>();
    __syncthreads();
  }
  for (int t = t_begin; t < t_end; t++) {
    const int st = (t - t_begin) & 1;
    if (t + 1 < t_end) {
      dma_tile(t + 1, st ^ 1);
      store_scales(sc_next, st ^ 1);   // stage st^1 is not read during tile t
      sc_next = load_scales(t + 2);    // lands before the end-of-tile wait
    }
    const FA8_LDS uint8_t* kt = (const FA8_LDS uint8_t*)smem + st * STAGE;
    const int j0 = t * BN;
    const bool need_mask = (j0 < full_lo) || (j0 + BN > full_hi);
    attn_tile_mx<D, DV, BN>(kt, kt + KTILE, kt + KTILE + VTILE, kt + KTILE + VTILE + KSC, qop, qsc, c, need_mask,
                            j0, my_lo, my_hi, lane, m_run, l_run, oacc);
    wait_vmcnt<0>();
    __syncthreads();
  }

  static_assert(NW * 32 * 2 * DV <= 2 * STAGE, "the staged output must fit in the two tile stages");
  if (p.o_vec16) {
    // the loop ended on a barrier with no copy or scale store in flight: the stages are free
    const RowScale rsc = row_scale(p, true, qh, m_run, l_run, 1.0f, 0.0f);
    if (valid && hgrp == 0 && p.lse)
      p.lse[(int64_t)b * p.l_bs + (int64_t)qh * p.l_hs + (int64_t)qi * p.l_rs] = rsc.lse;
    store_rows_staged<DV>(p, oacc, rsc.inv, lane, b, 0, rb0 + wave * 32, rb1, qh,
                          (FA8_LDS uint8_t*)smem + wave * (32 * 2 * DV));
    return;
  }
  if (!valid) return;
  store_row<DV, false>(p, oacc, m_run, l_run, 1.0f, hgrp, b, 0, qi, qh, 0, 0.0f);
}

// ------------------------------------------------------------------------------------------
// Split-KV decode: one wave per (kv head, split, batch, row block). The q heads that share the
// kv head are packed as rows r = i*g + (h mod g) of one block of up to 32 rows, handled as NQB
// blocks of 16 by the 16x16x128 MFMA. KV tiles of 64 keys (one split granule) go global ->
// registers -> one LDS stage; the next tile's loads are issued as soon as the current tile is
// in LDS, so they are in flight while it is computed (about 16 KB per wave, with two waves per
// SIMD).
//
// Paged K/V (PAGEMODE 1 and 2) walks the split in windows of 64 block-table entries: one vector
// load puts page win_base + i in lane i, then every tile inside the window takes its page
// numbers from that register, by v_readlane when each load instruction's rows lie in one page
// (PAGEMODE 1: page_size >= 64 / (d/16)) or by a lane shuffle (PAGEMODE 2). The tile loop has
// no branches around its loads, so the compiler's in-order vector-memory wait counts stay
// exact. Contiguous K/V is PAGEMODE 0.
// ------------------------------------------------------------------------------------------
// Waves per SIMD of the per-head decode kernel, and the tiles each keeps in flight in registers
// (DEPTH x (d + dv) / 4 registers of staging). d + dv <= 256 with one 16-row block per wave: two
// waves per SIMD with one stage each (about 200 registers); on the long-KV decode workload
// (131072 keys, 8 q heads per kv head) that measured 6-7% faster than one wave with two stages.
// Otherwise one wave per SIMD with the whole 512-entry register file: two stages (faster than
// three or four when this kernel carried the paged GQA decode workload; the extra requests in
// flight only lengthen the memory queues), one where two would spill.
template <int D, int DV, int NQB>
constexpr int decode_waves() {
  return (D + DV <= 256 && NQB == 1) ? 2 : 1;
}
template <int D, int DV, int NQB>
constexpr int decode_depth() {
  if (decode_waves<D, DV, NQB>() == 2) return 1;
  if (D + DV <= 256) return 2;
  if (D + DV >= 512 || NQB == 2) return 1;   // two stages would spill
  return 2;
}

// One (batch b, kv head kvh, row block mblock) of the per-head decode over the keys of granules
// [gs0, gs1) of sequence b (intersected with the block's visible keys), or, when !SCHED, over
// those of static split `ga` (gb unused); the partial goes to partial slot `slot`.
template <int D, int DV, int NQB, int PAGEMODE, bool SCHED>
__device__ __forceinline__ void perhead_segment(const KParams& p, int b, int kvh, int mblock, int ga, int gb,
                                                int64_t slot, uint8_t* smem) {
  constexpr int DEPTH = decode_depth<D, DV, NQB>();
  constexpr int BN = kKvTile;
  constexpr int KCH = D / 16, VCH = DV / 16;
  constexpr int KTILE = BN * D, VTILE = BN * DV;
  constexpr int KPT = KCH, VPT = VCH;        // 16-byte chunks per lane per tile (64 rows x NCH / 64)
  constexpr int KS = (D + 127) / 128;
  constexpr int NB = DV / 16;
  constexpr int BM = kDecodeRows;            // rows of a decode block (NQB * 16 of them are computed)
  static_assert(BN == kKvTile, "granules are KV tiles");

  const int lane = threadIdx.x;
  const int h4 = lane >> 4, l16 = lane & 15;
  const int g = p.g;

  const SeqInfo si = seq_info(p, b);
  const int rows_total = si.sq * g;
  const int rb0 = mblock * BM;
  if (rb0 >= rows_total) return;
  const int rb1 = min(rb0 + BM, rows_total) - 1;
  const int i_first = rb0 / g, i_last = rb1 / g;
  const RowRange rr{si.sk, si.sk - si.sq, p.wl, p.wr};
  const DecodeKeys dk0 = decode_keys(rr, i_first, i_last);
  int gs0 = ga, gs1 = gb;
  if constexpr (!SCHED) split_range(dk0, ga, p.nsplit, gs0, gs1);
  const int wg_lo = max(dk0.lo, gs0 * BN), wg_hi = min(dk0.hi, gs1 * BN);
  const int full_lo = max(dk0.full_lo, gs0 * BN), full_hi = min(dk0.full_hi, gs1 * BN);
  const int t_begin = wg_lo / BN;
  const int t_end = wg_hi > wg_lo ? (wg_hi + BN - 1) / BN : t_begin;

  const float dq = load_descale(p.dq, p.dq_sb, p.dq_sh, b, kvh);
  const float dk = load_descale(p.dk, p.dk_sb, p.dk_sh, b, kvh);
  const float dvs = load_descale(p.dv, p.dv_sb, p.dv_sh, b, kvh);
  const float c = p.scale_log2 * dq * dk;

  // this lane's row in each 16-row block: Q as the B operand, d-bytes [128ks + 32*h4, +32)
  bool valid[NQB];
  int qi[NQB], qh[NQB], my_lo[NQB], my_hi[NQB];
  v8i qop[NQB][KS];
#pragma unroll
  for (int qb = 0; qb < NQB; qb++) {
    const int ridx = rb0 + qb * 16 + l16;
    valid[qb] = ridx <= rb1;
    qi[qb] = ridx / g;
    qh[qb] = kvh * g + (ridx - qi[qb] * g);
    my_lo[qb] = 0;
    my_hi[qb] = 0;
    if (valid[qb]) {
      my_lo[qb] = max(rr.lo(qi[qb]), wg_lo);
      my_hi[qb] = min(rr.hi(qi[qb]), wg_hi);
    }
    const uint8_t* qrow = p.q + (p.cu_q ? (int64_t)(si.q0 + qi[qb]) * p.q_rs
                                        : (int64_t)b * p.q_bs + (int64_t)qi[qb] * p.q_rs) +
                          (int64_t)qh[qb] * p.q_hs;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const int off = ks * 128 + h4 * 32;
      v4i x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
      if (valid[qb] && off < D) {
        x0 = ld_global16(qrow + off);
        x1 = ld_global16(qrow + off + 16);
      }
      qop[qb][ks] = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
  }

  const KvAddr ka = kv_addr(p, b, kvh);
  const int jlast = si.sk - 1;
  // Rows of one 64-lane load instruction: 64 / NCH (they lie in one page under PAGEMODE 1).
  constexpr int KRPI = (64 % KCH == 0) ? 64 / KCH : 1, VRPI = (64 % VCH == 0) ? 64 / VCH : 1;
  static_assert(PAGEMODE != 1 || (64 % KCH == 0 && 64 % VCH == 0), "PAGEMODE 1 needs whole rows per load");
  // Block-table window (paged): lane i describes page win_base + i (clamped to the sequence's
  // last page). PAGEMODE 1 keeps the address of that page's K and V rows of this kv head as
  // 32-bit halves; PAGEMODE 2 keeps the page number.
  int win_base = 0, win_pg = 0;
  uint32_t wk_lo = 0, wk_hi = 0, wv_lo = 0, wv_hi = 0;
  auto load_window = [&](int base) {
    win_base = base;
    win_pg = ka.trow[min(win_base + lane, jlast >> ka.shift)];
    if constexpr (PAGEMODE == 1) {
      const uint64_t ko = reinterpret_cast<uint64_t>(p.k + (int64_t)win_pg * ka.k_ps + ka.kbase);
      const uint64_t vo = reinterpret_cast<uint64_t>(p.v + (int64_t)win_pg * ka.v_ps + ka.vbase);
      wk_lo = (uint32_t)ko; wk_hi = (uint32_t)(ko >> 32);
      wv_lo = (uint32_t)vo; wv_hi = (uint32_t)(vo >> 32);
    }
  };
  // Per-lane byte offset inside a load instruction's rows when 64 / NCH whole rows make one
  // instruction: row lane / NCH of the instruction, chunk lane % NCH (the same for every
  // instruction and tile).
  const uint32_t lane_off_k = (uint32_t)((lane / KCH) * (int)ka.k_rs + (lane % KCH) * 16);
  const uint32_t lane_off_v = (uint32_t)((lane / VCH) * (int)ka.v_rs + (lane % VCH) * 16);

  // This lane's 16-byte chunk of load instruction u of the tile starting at key j0.
  // PAGEMODE 0 and 1 use buffer loads whose range (num_records) ends at the sequence's last key:
  // chunks of rows past it return zeros without a memory access, and a step past the window
  // end (real == false) gets an empty range, so all of its loads return zeros and cost no
  // memory traffic. (Contiguous rows and page rows at most 64 rows x row stride < 2^31 bytes
  // from the base, checked on the host.)
  // PAGEMODE 1: an instruction's rows lie in one page (page_size >= rows per instruction, both
  // powers of two), so its base is uniform: the window's page offset + the in-page row offset.
  // PAGEMODE 2 (pages smaller than one instruction's rows): per-lane page lookup by a lane
  // shuffle, rows clamped to the last valid key, and a filler step reads a small cached block.
  auto chunk_load = [&](bool is_v, int j0, int u, bool real) -> v4i {
    const int NCH = is_v ? VCH : KCH;
    const int rpi = is_v ? VRPI : KRPI;
    const int rs = (int)(is_v ? ka.v_rs : ka.k_rs);
    const uint8_t* base_ptr = is_v ? p.v : p.k;
    if constexpr (PAGEMODE == 1) {
      const int jr = j0 + u * rpi;                                               // uniform
      const int idx = min((jr >> ka.shift) - win_base, 63);
      const uint32_t lo = __builtin_amdgcn_readlane(is_v ? wv_lo : wk_lo, idx);
      const uint32_t hi = __builtin_amdgcn_readlane(is_v ? wv_hi : wk_hi, idx);
      const uint8_t* base = reinterpret_cast<const uint8_t*>((((uint64_t)hi) << 32) | lo) +
                            (uint32_t)((jr & ka.pmask) * rs);   // uniform
      const int rem = si.sk - jr;   // rows of this instruction that are keys of the sequence
      const int nrec = (real && rem > 0) ? min(rem, rpi) * rs : 0;
      return ld_buffer16_nt(base, nrec, is_v ? lane_off_v : lane_off_k);
    } else if constexpr (PAGEMODE == 0) {
      const int64_t kvbase = is_v ? ka.vbase : ka.kbase;
      if ((is_v ? VRPI : KRPI) * NCH == 64) {
        // whole rows per instruction: uniform base at the instruction's first row
        const int jr = j0 + u * rpi;
        const uint8_t* base = base_ptr + kvbase + (int64_t)jr * rs;
        const int rem = si.sk - jr;
        const int nrec = (real && rem > 0) ? min(rem, rpi) * rs : 0;
        return ld_buffer16_nt(base, nrec, is_v ? lane_off_v : lane_off_k);
      } else {
        const int cid = u * 64 + lane;
        const int row = cid / NCH, ch = cid - row * NCH;
        const uint8_t* base = base_ptr + kvbase + (int64_t)j0 * rs;
        const int rem = si.sk - j0;
        const int nrec = (real && rem > 0) ? min(rem, BN) * rs : 0;
        return ld_buffer16_nt(base, nrec, (uint32_t)(row * rs + ch * 16));
      }
    } else {
      const int cid = u * 64 + lane;
      const int row = cid / NCH, ch = cid - row * NCH;
      const int j = min(j0 + row, jlast);
      const int page = __shfl(win_pg, (j >> ka.shift) - win_base);
      const uint8_t* ptr = base_ptr + (is_v ? ka.vbase : ka.kbase) + (int64_t)page * (is_v ? ka.v_ps : ka.k_ps) +
                           (int64_t)(j & ka.pmask) * rs + ch * 16;
      return ld_global16_nt(real ? ptr : g_filler + lane * 16);
    }
  };
  v4i kr[DEPTH][KPT], vr[DEPTH][VPT];
  // Loads of tile t into one register stage. A step past the window end (real == false)
  // issues the same loads, which then return zeros (or read the filler block): every step
  // issues the same loads, so the compiler's in-order wait counts are exact and each tile's
  // wait leaves the DEPTH-1 younger tiles in flight. (Forced inline: at d = 256 with the
  // per-lane page lookup the compiler would otherwise make it a call with a stack frame.)
  auto gload = [&](int t, bool real, v4i (&ks)[KPT], v4i (&vs)[VPT]) __attribute__((always_inline)) {
    const int j0 = t * BN;
#pragma unroll
    for (int u = 0; u < KPT; u++) ks[u] = chunk_load(false, j0, u, real);
#pragma unroll
    for (int u = 0; u < VPT; u++) vs[u] = chunk_load(true, j0, u, real);
  };
  // Registers -> LDS (swizzled rows).
  auto swrite = [&](v4i (&ks)[KPT], v4i (&vs)[VPT]) {
#pragma unroll
    for (int u = 0; u < KPT; u++) {
      const int cid = u * 64 + lane;
      const int row = cid / KCH, ch = cid - row * KCH;
      *reinterpret_cast<v4i*>(smem + row * D + swz<KCH>(ch, k_sv<D>(row)) * 16) = ks[u];
    }
#pragma unroll
    for (int u = 0; u < VPT; u++) {
      const int cid = u * 64 + lane;
      const int row = cid / VCH, ch = cid - row * VCH;
      *reinterpret_cast<v4i*>(smem + KTILE + row * DV + swz<VCH>(ch, v_sv16(row)) * 16) = vs[u];
    }
  };

  float m_run[NQB], l_run[NQB];
  v4f oacc[NQB][NB];
#pragma unroll
  for (int qb = 0; qb < NQB; qb++) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.0f;
#pragma unroll
    for (int n = 0; n < NB; n++) oacc[qb][n] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  }

  const FA8_LDS uint8_t* kt = (const FA8_LDS uint8_t*)smem;
  // Tiles [w0, w1) with DEPTH register stages: tile t (stage t mod DEPTH) goes registers -> LDS,
  // then tile t+DEPTH's loads reuse that stage (a scheduling barrier keeps them ahead of the
  // compute), then tile t is computed from LDS; DEPTH tiles are always in flight. Steps past w1
  // run with dummy loads and no compute, so loads and waits never sit under a branch.
  auto step = [&](auto stage, int t, int w1) {
    constexpr int st = decltype(stage)::value;
    wave_lds_order();   // the previous tile's LDS reads are issued before these writes
    swrite(kr[st], vr[st]);
    wave_lds_order();
    gload(t + DEPTH, t + DEPTH < w1, kr[st], vr[st]);
    __builtin_amdgcn_sched_barrier(0);
    if (t < w1) {
      const int j0 = t * BN;
      const bool need_mask = (j0 < full_lo) || (j0 + BN > full_hi);
      attn_tile16<D, DV, NQB>(kt, kt + KTILE, qop, c, need_mask, j0, my_lo, my_hi, lane, m_run, l_run, oacc);
    }
  };
  auto run_tiles = [&](int w0, int w1) {
    // issue order = consumption order, so each tile's wait leaves the later tiles in flight
    gload(w0, true, kr[0], vr[0]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DEPTH > 1) gload(w0 + 1, w0 + 1 < w1, kr[1 % DEPTH], vr[1 % DEPTH]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DEPTH > 2) gload(w0 + 2, w0 + 2 < w1, kr[2 % DEPTH], vr[2 % DEPTH]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (DEPTH > 3) gload(w0 + 3, w0 + 3 < w1, kr[3 % DEPTH], vr[3 % DEPTH]);
    __builtin_amdgcn_sched_barrier(0);
    for (int t = w0; t < w1; t += DEPTH) {
      step(std::integral_constant<int, 0>{}, t, w1);
      if constexpr (DEPTH > 1) step(std::integral_constant<int, 1 % DEPTH>{}, t + 1, w1);
      if constexpr (DEPTH > 2) step(std::integral_constant<int, 2 % DEPTH>{}, t + 2, w1);
      if constexpr (DEPTH > 3) step(std::integral_constant<int, 3 % DEPTH>{}, t + 3, w1);
    }
  };

  if constexpr (PAGEMODE == 0) {
    if (t_begin < t_end) run_tiles(t_begin, t_end);
  } else {
    int t = t_begin;
    while (t < t_end) {
      // window of 64 entries from this tile's first page; then the tiles whose rows all fall in it
      load_window((t * BN) >> ka.shift);
      wait_vmcnt<0>();
      int w1 = t + 1;
      while (w1 < t_end && ((min(w1 * BN + BN - 1, jlast) >> ka.shift) - win_base) < 64) w1++;
      run_tiles(t, w1);
      t = w1;
    }
  }

#pragma unroll
  for (int qb = 0; qb < NQB; qb++) {
    float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!valid[qb]) continue;
    const bool nonempty = l_tot > 0.0f;
    const float inv = nonempty ? dvs / l_tot : 0.0f;
    const float lse = nonempty ? (m_run[qb] + __log2f(l_tot) - kBias) * kLn2 : kNegInf;
    const int64_t prow = (slot * p.max_sq + qi[qb]) * p.hq + qh[qb];
    float* orow = p.o_part + prow * DV;
#pragma unroll
    for (int n = 0; n < NB; n++) {
      v4f v = {oacc[qb][n][0] * inv, oacc[qb][n][1] * inv, oacc[qb][n][2] * inv, oacc[qb][n][3] * inv};
      *reinterpret_cast<v4f*>(orow + 16 * n + 4 * h4) = v;
    }
    if (h4 == 0) p.lse_part[prow] = lse;
  }
}

// One wave per (kv head, row block, split, batch) with static splits, or per (kv head, segment) of
// a balanced schedule (SCHED; one row block per kv head).
template <int D, int DV, int NQB, int PAGEMODE, bool SCHED>
__global__ void __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(decode_waves<D, DV, NQB>(), decode_waves<D, DV, NQB>())))
fa8_decode_kernel(const KParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kKvTile * (D + DV)];
  if constexpr (SCHED) {
    int b, s0, s1;
    if (!sched_segment(p, blockIdx.y, b, s0, s1)) return;
    perhead_segment<D, DV, NQB, PAGEMODE, true>(p, b, blockIdx.x, 0, s0, s1, blockIdx.y, smem);
  } else {
    const int b = blockIdx.z, split = blockIdx.y;
    const int kvh = blockIdx.x / p.nmb, mblock = blockIdx.x - kvh * p.nmb;
    perhead_segment<D, DV, NQB, PAGEMODE, false>(p, b, kvh, mblock, split, 0, (int64_t)split * p.batch + b, smem);
  }
}

// ------------------------------------------------------------------------------------------
// Split-KV decode with several kv heads per wave, for GQA shapes with few query rows per kv
// head: one wave per (group of HPW kv heads, split, batch). The Sq*g rows of each of the HPW
// heads together fill the 16 rows of one 16x16 MFMA block (HPW * Sq * g <= 16), so no MFMA row
// is padding. A step covers BN = 64 / HPW keys of all HPW heads (16 KB at d = dv = 128), loaded
// into registers as whole token rows of the group (the HPW heads of a token are HPW * d
// contiguous bytes) and staged through one LDS stage, with the pipeline of the per-head kernel.
//   S^T (16 keys x 16 rows) of key block kb: sum over heads a of K_a . Q_a'^T, where Q_a' is Q
//     with the rows of the other heads zeroed, so every row only sees its own head's keys.
//   O^T (16 dv x 16 rows) of a step: one 16x16x128 MFMA per 16 dv columns. Its 128 K slots are
//     four groups of 32; group kg belongs to (head a = kg / KB, key block kb = kg % KB) and holds
//     that block's 16 keys (16 slots, the rest zero). Row r's P enters only the groups of r's
//     own head, so the sum over all slots is exactly sum_j P[r][j] V_head(r)[j].
// ------------------------------------------------------------------------------------------
// PAGED: K/V through the block table; STEP_PAGE: page_size >= BN, so each step's rows lie in
// one page (or K/V are contiguous) and one descriptor per step serves all of its loads.
template <int D, int DV, int HPW>
struct HeadsGeom {
  static constexpr int KB = 4 / HPW, BN = 16 * KB;
  static constexpr int KR = HPW * D, VR = HPW * DV;
  static constexpr int SMEM = BN * KR + BN * VR;
};

// One (batch b, kv heads kvh0 .. kvh0 + HPW - 1) of the several-heads decode over the keys of
// granules [ra, rb) of sequence b (intersected with the rows' visible keys), or, when !SCHED,
// over those of static split `ra`; the partial goes to partial slot `slot` (rows
// slot * max_seqlen_q * heads_q + i * heads_q + h).
template <int D, int DV, int HPW, bool PAGED, bool STEP_PAGE, bool SCHED>
__device__ __forceinline__ void heads_segment(const KParams& p, int b, int kvh0, int ra, int rb, int64_t slot,
                                              uint8_t* smem) {
  static_assert(HPW == 2 || HPW == 4, "two or four kv heads per wave");
  constexpr int KB = 4 / HPW;                        // 16-key blocks per step
  constexpr int BN = 16 * KB;                        // keys per step
  constexpr int KR = HPW * D, VR = HPW * DV;         // bytes of one token's K / V row for the heads
  static_assert(KR <= 1024 && VR <= 1024, "a load instruction holds whole rows");
  constexpr int KLPR = KR / 16, VLPR = VR / 16;      // lanes per row in a load instruction
  constexpr int KRPI = 64 / KLPR, VRPI = 64 / VLPR;  // rows per load instruction
  constexpr int KPT = BN / KRPI, VPT = BN / VRPI;    // load instructions per step
  constexpr int KTILE = BN * KR, VTILE = BN * VR;
  constexpr int KSW = (KLPR < 16 ? KLPR : 16) - 1, VSW = (VLPR < 16 ? VLPR : 16) - 1;   // swizzle masks
  constexpr int KS = (D + 127) / 128;
  constexpr int NB = DV / 16;
  constexpr int DEPTH = 1;   // one register stage + the LDS stage; two waves per SIMD overlap
  static_assert(HeadsGeom<D, DV, HPW>::SMEM == KTILE + VTILE, "LDS size");

  const int lane = threadIdx.x;
  const int kg = lane >> 4, l16 = lane & 15;
  const int g = p.g;
  const SeqInfo si = seq_info(p, b);
  const RowRange rr{si.sk, si.sk - si.sq, p.wl, p.wr};

  // ---- key range of the wave (all query tokens of the batch), cut to the given granules ----
  const DecodeKeys dk0 = decode_keys(rr, 0, si.sq - 1);
  int gs0 = ra, gs1 = rb;
  if constexpr (!SCHED) split_range(dk0, ra, p.nsplit, gs0, gs1);
  const int wg_lo = max(dk0.lo, gs0 * kKvTile), wg_hi = min(dk0.hi, gs1 * kKvTile);
  const int full_lo = max(dk0.full_lo, gs0 * kKvTile), full_hi = min(dk0.full_hi, gs1 * kKvTile);
  const int t_begin = wg_lo / BN;
  const int t_end = wg_hi > wg_lo ? (wg_hi + BN - 1) / BN : t_begin;

  // ---- this lane's row: head slot a, query token qi, q head qg of the group ----
  const int rp = p.max_sq * g;                       // rows per kv head (host: HPW * rp <= 16)
  const int my_a = l16 / rp, rq = l16 - my_a * rp;
  const int qi = rq / g, qg = rq - qi * g;
  const bool valid = my_a < HPW && qi < si.sq;
  const int kvh = kvh0 + min(my_a, HPW - 1);
  const int qh = kvh * g + qg;
  const float dq = load_descale(p.dq, p.dq_sb, p.dq_sh, b, kvh);
  const float dk = load_descale(p.dk, p.dk_sb, p.dk_sh, b, kvh);
  // the v descale of each head slot, wave-uniform (scalar registers): the lane's own one is
  // picked after the key loop, so it holds no vector register through the loop
  float dvs_slot[HPW];
#pragma unroll
  for (int a = 0; a < HPW; a++) dvs_slot[a] = load_descale(p.dv, p.dv_sb, p.dv_sh, b, kvh0 + a);
  const float c = p.scale_log2 * dq * dk;
  int my_lo = 0, my_hi = 0;
  if (valid) {
    my_lo = max(rr.lo(qi), wg_lo);
    my_hi = min(rr.hi(qi), wg_hi);
  }

  // Q of this row as the B operand (d-bytes [128ks + 32kg, +32)), once per head slot with the
  // other slots' rows zeroed
  v8i qm[HPW][KS];
  {
    const uint8_t* qrow = p.q + (p.cu_q ? (int64_t)(si.q0 + qi) * p.q_rs : (int64_t)b * p.q_bs + (int64_t)qi * p.q_rs) +
                          (int64_t)qh * p.q_hs;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const int off = ks * 128 + kg * 32;
      v4i x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
      if (valid && off < D) {
        x0 = ld_global16(qrow + off);
        x1 = ld_global16(qrow + off + 16);
      }
      const v8i q8 = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
      for (int a = 0; a < HPW; a++) qm[a][ks] = (a == my_a) ? q8 : (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  // ---- K/V rows ----
  const int shift = PAGED ? p.page_shift : 0, pmask = PAGED ? (1 << p.page_shift) - 1 : 0;
  const int jlast = si.sk - 1;
  const int k_rs = (int)p.k_rs, v_rs = (int)p.v_rs;   // row strides: page_size (or 64) rows < 2^31 bytes
  const uint8_t* kbase = p.k + (int64_t)kvh0 * p.k_hs +
                         (PAGED ? 0 : (p.cu_k ? (int64_t)p.cu_k[b] * p.k_rs : (int64_t)b * p.k_bs));
  const uint8_t* vbase = p.v + (int64_t)kvh0 * p.v_hs +
                         (PAGED ? 0 : (p.cu_k ? (int64_t)p.cu_k[b] * p.v_rs : (int64_t)b * p.v_bs));
  // block-table window: lane i holds the K and V addresses of page win_base + i (clamped to the
  // sequence's last page) for this group's first head, as 32-bit halves
  int win_base = 0;
  uint32_t wk_lo = 0, wk_hi = 0, wv_lo = 0, wv_hi = 0;
  auto load_window = [&](int base) {
    win_base = base;
    const int pg = p.table[(int64_t)b * p.table_stride + min(win_base + lane, jlast >> shift)];
    const uint64_t ka = reinterpret_cast<uint64_t>(kbase + (int64_t)pg * p.k_bs);
    const uint64_t va = reinterpret_cast<uint64_t>(vbase + (int64_t)pg * p.v_bs);
    wk_lo = (uint32_t)ka; wk_hi = (uint32_t)(ka >> 32);
    wv_lo = (uint32_t)va; wv_hi = (uint32_t)(va >> 32);
  };
  // per-lane offset inside a load instruction: row lane / LPR of the instruction, chunk lane % LPR
  const uint32_t lane_off_k = (uint32_t)((lane / KLPR) * k_rs + (lane % KLPR) * 16);
  const uint32_t lane_off_v = (uint32_t)((lane / VLPR) * v_rs + (lane % VLPR) * 16);
  // Load instruction u of the step at key j0: rows [j0 + u*RPI, +RPI), uniform base; a buffer
  // range ending at the sequence's last key makes rows past it (and every load of a filler step,
  // real == false) return zeros without a memory access. Paged: the rows of one instruction lie
  // in one page (page_size >= rows per instruction, both powers of two).
  auto chunk_load = [&](bool is_v, int j0, int u, bool real) -> v4i {
    const int rpi = is_v ? VRPI : KRPI;
    const int rs = is_v ? v_rs : k_rs;
    const int jr = j0 + u * rpi;                                             // uniform
    const uint8_t* base;
    if constexpr (PAGED) {
      const int idx = min((jr >> shift) - win_base, 63);
      const uint32_t lo = __builtin_amdgcn_readlane(is_v ? wv_lo : wk_lo, idx);
      const uint32_t hi = __builtin_amdgcn_readlane(is_v ? wv_hi : wk_hi, idx);
      base = reinterpret_cast<const uint8_t*>((((uint64_t)hi) << 32) | lo) + (uint32_t)((jr & pmask) * rs);
    } else {
      base = (is_v ? vbase : kbase) + (int64_t)jr * rs;
    }
    const int rem = si.sk - jr;
    const int nrec = (real && rem > 0) ? min(rem, rpi) * rs : 0;
    return ld_buffer16_nt(base, nrec, is_v ? lane_off_v : lane_off_k);
  };
  // STEP_PAGE: the uniform base of the step's first row and the bytes of its rows that are keys
  auto step_base = [&](bool is_v, int j0) -> const uint8_t* {
    const int rs = is_v ? v_rs : k_rs;
    if constexpr (PAGED) {
      const int idx = min((j0 >> shift) - win_base, 63);
      const uint32_t lo = __builtin_amdgcn_readlane(is_v ? wv_lo : wk_lo, idx);
      const uint32_t hi = __builtin_amdgcn_readlane(is_v ? wv_hi : wk_hi, idx);
      return reinterpret_cast<const uint8_t*>((((uint64_t)hi) << 32) | lo) + (uint32_t)((j0 & pmask) * rs);
    } else {
      return (is_v ? vbase : kbase) + (int64_t)j0 * rs;
    }
  };
  v4i kr[DEPTH][KPT], vr[DEPTH][VPT];
  auto gload = [&](int t, bool real, v4i (&ks)[KPT], v4i (&vs)[VPT]) {
    const int j0 = t * BN;
    if constexpr (STEP_PAGE) {
      // one descriptor per step whose range is the step's key rows; instruction u adds its
      // first row to the per-lane offset (the range check applies to the whole offset)
      const int rem = si.sk - j0;
      const int rows = (real && rem > 0) ? min(rem, BN) : 0;
      const uint8_t* kb0 = step_base(false, j0);
      const uint8_t* vb0 = step_base(true, j0);
#pragma unroll
      for (int u = 0; u < KPT; u++) ks[u] = ld_buffer16_nt(kb0, rows * k_rs, lane_off_k + (uint32_t)(u * KRPI * k_rs));
#pragma unroll
      for (int u = 0; u < VPT; u++) vs[u] = ld_buffer16_nt(vb0, rows * v_rs, lane_off_v + (uint32_t)(u * VRPI * v_rs));
    } else {
#pragma unroll
      for (int u = 0; u < KPT; u++) ks[u] = chunk_load(false, j0, u, real);
#pragma unroll
      for (int u = 0; u < VPT; u++) vs[u] = chunk_load(true, j0, u, real);
    }
  };
  // registers -> LDS: row r of the step at r*R, its 16-byte chunk c at position c ^ (r & SW)
  auto swrite = [&](v4i (&ks)[KPT], v4i (&vs)[VPT]) {
#pragma unroll
    for (int u = 0; u < KPT; u++) {
      const int r = u * KRPI + lane / KLPR, ch = lane % KLPR;
      *reinterpret_cast<v4i*>(smem + r * KR + ((ch ^ (r & KSW)) << 4)) = ks[u];
    }
#pragma unroll
    for (int u = 0; u < VPT; u++) {
      const int r = u * VRPI + lane / VLPR, ch = lane % VLPR;
      *reinterpret_cast<v4i*>(smem + KTILE + r * VR + ((ch ^ (r & VSW)) << 4)) = vs[u];
    }
  };

  // Two-level PV accumulation: oblk accumulates the PV products of up to four steps (64 keys)
  // on the MFMA; it is folded into the fp32 oacc every fourth step, and before a step whose
  // lazy rescale moves the running max of any row (then O = alpha (oacc + oblk) first).
  float m_run = kNegInf, l_run = 0.0f;
  v4f oacc[NB], oblk[NB];
#pragma unroll
  for (int n = 0; n < NB; n++) {
    oacc[n] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    oblk[n] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  }

  // PV operand geometry of this lane: K-slot group kg = (head ga, key block gb); dword j of the
  // group holds keys 16 gb + 4 (kg ^ j) + [0, 4). The two transposed reads (e = 0, 1) give
  // dwords 2e, 2e + 1; source lane s of a 16-lane group points at key byte s >> 1, column half
  // s & 1 of the 16 dv columns.
  const int ga = kg / KB, gb = kg % KB;
  const bool my_group = (my_a == ga);
  int tr_off[2];
#pragma unroll
  for (int e = 0; e < 2; e++) {
    const int byte = l16 >> 1;
    const int row = 16 * gb + 4 * ((2 * e + (byte >> 2)) ^ kg) + (byte & 3);
    tr_off[e] = row * VR + 8 * (l16 & 1);
  }
  const int tr_sw0 = (16 * gb + 4 * ((0 + ((l16 >> 1) >> 2)) ^ kg) + ((l16 >> 1) & 3)) & VSW;
  const int tr_sw1 = (16 * gb + 4 * ((2 + ((l16 >> 1) >> 2)) ^ kg) + ((l16 >> 1) & 3)) & VSW;

  const FA8_LDS uint8_t* kt = (const FA8_LDS uint8_t*)smem;
  const FA8_LDS uint8_t* vt = kt + KTILE;
  auto compute = [&](int t) {
    const int j0 = t * BN;
    const bool need_mask = (j0 < full_lo) || (j0 + BN > full_hi);
    // ---- S^T per key block ----
    v4f sacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; kb++) {
      sacc[kb] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
      const int krow = 16 * kb + l16;
#pragma unroll
      for (int a = 0; a < HPW; a++)
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
          const int off = ks * 128 + kg * 32;
          v8i kop = {0, 0, 0, 0, 0, 0, 0, 0};
          if (off < D) {
            const int ch = (a * D + off) >> 4;
            const v4i x0 = *(const FA8_LDS v4i*)(kt + krow * KR + ((ch ^ (krow & KSW)) << 4));
            const v4i x1 = *(const FA8_LDS v4i*)(kt + krow * KR + (((ch + 1) ^ (krow & KSW)) << 4));
            kop = (v8i){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
          }
          sacc[kb] = mfma_16x16x128_fp8(kop, qm[a][ks], sacc[kb]);
        }
    }
    // ---- mask, row max (over the row's 4 lanes), lazy rescale, P ----
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int j = j0 + 16 * kb + 4 * kg + r;
          if (j < my_lo || j >= my_hi) sacc[kb][r] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KB; kb++)
      mx = fmaxf(mx, fmaxf(fmaxf(sacc[kb][0], sacc[kb][1]), fmaxf(sacc[kb][2], sacc[kb][3])));
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    const float mt = mx * c;
    float alpha = 1.0f;
    const bool moved = mt - m_run > kTau;
    if (moved) {
      alpha = fast_exp2(m_run - mt);
      m_run = mt;
    }
    if (__builtin_amdgcn_ballot_w64(moved)) {   // uniform: fold before the scale changes
#pragma unroll
      for (int n = 0; n < NB; n++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          oacc[n][r] = alpha * (oacc[n][r] + oblk[n][r]);
          oblk[n][r] = 0.0f;
        }
    }
    const float nb = (m_run == kNegInf) ? 0.0f : kBias - m_run;
    int pw[KB];
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; kb++) {
      const float p0 = fast_exp2(__builtin_fmaf(sacc[kb][0], c, nb));
      const float p1 = fast_exp2(__builtin_fmaf(sacc[kb][1], c, nb));
      const float p2 = fast_exp2(__builtin_fmaf(sacc[kb][2], c, nb));
      const float p3 = fast_exp2(__builtin_fmaf(sacc[kb][3], c, nb));
      int word = cvt_pk_fp8_lo(p0, p1);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
      pw[kb] = word;
      const auto r01 = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
      const auto r23 = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
      lsum += (r01[0] + r01[1]) + (r23[0] + r23[1]);
    }
    l_run = alpha * l_run + lsum;
    // ---- P' (B operand): dword j of group kg = block gb's P of lane (row, kg ^ j) ----
    // (lane ^ 16x sends the block the receiving lane's group needs: pw[(kg ^ x) % KB])
    int pd[4];
    pd[0] = pw[gb];
    const uint32_t s1 = (uint32_t)pw[(kg ^ 1) % KB];
    const uint32_t r1 = from_xor16(s1, lane);
    pd[1] = (int)r1;
    pd[2] = (int)from_xor32((uint32_t)pw[(kg ^ 2) % KB], lane);
    pd[3] = (int)from_xor32(r1, lane);            // s1 of lane ^ 48 (pw[(kg ^ 3) % KB] == s1 there)
    const v8i pop = my_group ? (v8i){pd[0], pd[1], pd[2], pd[3], 0, 0, 0, 0} : (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    // ---- O^T of the step accumulated on the MFMA; fold every fourth step ----
#pragma unroll
    for (int n = 0; n < NB; n++) {
      const int ch = ga * NB + n;
      const v2i x0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA8_LDS v2i*)(vt + tr_off[0] + ((ch ^ tr_sw0) << 4)));
      const v2i x1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA8_LDS v2i*)(vt + tr_off[1] + ((ch ^ tr_sw1) << 4)));
      const v8i vop = {x0[0], x0[1], x1[0], x1[1], 0, 0, 0, 0};
      oblk[n] = mfma_16x16x128_fp8(vop, pop, oblk[n]);
    }
    if ((t & 3) == 3) {
#pragma unroll
      for (int n = 0; n < NB; n++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          oacc[n][r] += oblk[n][r];
          oblk[n][r] = 0.0f;
        }
    }
  };

  // Steps [w0, w1) with DEPTH register stages (as in the per-head kernel): step t goes registers
  // -> LDS, step t+DEPTH's loads reuse that stage, then step t is computed from LDS.
  auto step = [&](auto stage, int t, int w1) {
    constexpr int st = decltype(stage)::value;
    wave_lds_order();   // the previous step's LDS reads are issued before these writes
    swrite(kr[st], vr[st]);
    wave_lds_order();
    gload(t + DEPTH, t + DEPTH < w1, kr[st], vr[st]);
    __builtin_amdgcn_sched_barrier(0);
    if (t < w1) compute(t);
  };
  auto run_steps = [&](int w0, int w1) {
    gload(w0, true, kr[0], vr[0]);
    __builtin_amdgcn_sched_barrier(0);
    for (int t = w0; t < w1; t += DEPTH) step(std::integral_constant<int, 0>{}, t, w1);
  };
  if constexpr (!PAGED) {
    if (t_begin < t_end) run_steps(t_begin, t_end);
  } else {
    int t = t_begin;
    while (t < t_end) {
      // window of 64 entries from this step's first page; then the steps whose rows all fall in it
      load_window((t * BN) >> shift);
      wait_vmcnt<0>();
      int w1 = t + 1;
      while (w1 < t_end && ((min(w1 * BN + BN - 1, jlast) >> shift) - win_base) < 64) w1++;
      run_steps(t, w1);
      t = w1;
    }
  }

#pragma unroll
  for (int n = 0; n < NB; n++)
#pragma unroll
    for (int r = 0; r < 4; r++) oacc[n][r] += oblk[n][r];
  float l_tot = sum_xor16(l_run);
  l_tot = sum_xor32(l_tot);
  if (!valid) return;
  float dvs = dvs_slot[0];
#pragma unroll
  for (int a = 1; a < HPW; a++)
    if (my_a == a) dvs = dvs_slot[a];
  const bool nonempty = l_tot > 0.0f;
  const float inv = nonempty ? dvs / l_tot : 0.0f;
  const float lse = nonempty ? (m_run + __log2f(l_tot) - kBias) * kLn2 : kNegInf;
  const int64_t prow = (slot * p.max_sq + qi) * p.hq + qh;
  float* orow = p.o_part + prow * DV;
#pragma unroll
  for (int n = 0; n < NB; n++) {
    const v4f v = {oacc[n][0] * inv, oacc[n][1] * inv, oacc[n][2] * inv, oacc[n][3] * inv};
    *reinterpret_cast<v4f*>(orow + 16 * n + 4 * kg) = v;
  }
  if (kg == 0) p.lse_part[prow] = lse;
}

// One wave per (group of HPW kv heads, split, batch) with static splits (split s of a sequence
// covers granules [g0 + floor(s n / S), g0 + floor((s + 1) n / S)) of its n visible granules), or
// per (group, segment) of a balanced schedule (SCHED; sched_segment).
template <int D, int DV, int HPW, bool PAGED, bool STEP_PAGE, bool SCHED>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
fa8_decode_heads_kernel(const KParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[HeadsGeom<D, DV, HPW>::SMEM];
  if constexpr (SCHED) {
    int b, s0, s1;
    if (!sched_segment(p, blockIdx.y, b, s0, s1)) return;
    heads_segment<D, DV, HPW, PAGED, STEP_PAGE, true>(p, b, blockIdx.x * HPW, s0, s1, blockIdx.y, smem);
  } else {
    const int b = blockIdx.z, split = blockIdx.y;
    heads_segment<D, DV, HPW, PAGED, STEP_PAGE, false>(p, b, blockIdx.x * HPW, split, 0,
                                                       (int64_t)split * p.batch + b, smem);
  }
}

// Inclusive prefix sum of v over the 1024 threads of a workgroup; *total receives the sum of all.
__device__ __forceinline__ int block_scan1024(int v, int* total, int* s_w) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  __syncthreads();   // s_w is free (a previous call's readers are done)
  if (lane == 63) s_w[wv] = v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int k = 0; k < 16; k++) {
    const int t = s_w[k];
    before += (k < wv) ? t : 0;
    all += t;
  }
  *total = all;
  return v + before;
}

// Writes the balanced decode schedule (layout at sched_segment) for W workers: one workgroup of
// 1024 threads, sequences in chunks of 1024. Sequence b's granules are those of the union of its
// rows' visible keys (the granules a static split would share out); its partial slots are the
// workers its granules meet.
__global__ void __launch_bounds__(1024) fa8_decode_schedule_kernel(const KParams p, int32_t W, int32_t* sched) {
  __shared__ int s_w[16];
  int32_t* gst = sched + 2;
  int32_t* pst = gst + p.batch + 1;
  auto granules = [&](int b) -> int {
    if (b >= p.batch) return 0;
    const SeqInfo si = seq_info_lane(p, b);
    const RowRange rr{si.sk, si.sk - si.sq, p.wl, p.wr};
    return union_granules(decode_keys(rr, 0, si.sq - 1));
  };
  // pass 1: granule prefix and G; with at most 1024 sequences the lengths are read once and the
  // segment prefix follows in the same pass
  const int b0 = (int)threadIdx.x;
  const int v0 = granules(b0);
  int tot0;
  const int excl0 = block_scan1024(v0, &tot0, s_w) - v0;
  if (b0 < p.batch) gst[b0] = excl0;
  int G = tot0;
  for (int base = 1024; base < p.batch; base += 1024) {
    const int b = base + (int)threadIdx.x;
    const int v = granules(b);
    int tot;
    const int incl = block_scan1024(v, &tot, s_w);
    if (b < p.batch) gst[b] = G + incl - v;
    G += tot;
  }
  // pass 2: segments per sequence and their prefix
  auto segments = [&](int gb0, int v) { return v > 0 ? sched_owner(gb0 + v - 1, W, G) - sched_owner(gb0, W, G) + 1 : 0; };
  const int n0 = segments(excl0, v0);
  int ntot0;
  const int nexcl0 = block_scan1024(n0, &ntot0, s_w) - n0;
  if (b0 < p.batch) pst[b0] = nexcl0;
  int gcarry = tot0, pcarry = ntot0;
  for (int base = 1024; base < p.batch; base += 1024) {
    const int b = base + (int)threadIdx.x;
    const int v = granules(b);
    int tot, ntot;
    const int gb0 = gcarry + block_scan1024(v, &tot, s_w) - v;
    const int n = segments(gb0, v);
    const int nincl = block_scan1024(n, &ntot, s_w);
    if (b < p.batch) pst[b] = pcarry + nincl - n;
    gcarry += tot;
    pcarry += ntot;
  }
  if (threadIdx.x == 0) {
    sched[0] = G;
    sched[1] = W;
    gst[p.batch] = G;
    pst[p.batch] = pcarry;
  }
}

// The partial rows one output row (b, i, h) merges: static splits s = 0 .. nsplit-1 at row
// (s * batch + b) * max_sq * hq + i * hq + h; with a balanced schedule the slots pst[b] ..
// pst[b+1]-1 at row slot * max_sq * hq + i * hq + h.
struct PartialRows {
  int n;
  int64_t first, stride;
  __device__ int64_t at(int s) const { return first + (int64_t)s * stride; }
};
__device__ __forceinline__ PartialRows partial_rows(const CParams& c, int b, int i, int h, int64_t row, int64_t rows) {
  PartialRows r;
  if (c.sched) {
    const int32_t* pst = c.sched + 2 + c.batch + 1;
    const int p0 = pst[b];
    r.n = pst[b + 1] - p0;
    r.stride = (int64_t)c.max_sq * c.hq;
    r.first = (int64_t)p0 * r.stride + (int64_t)i * c.hq + h;
  } else {
    r.n = c.nsplit;
    r.first = row;
    r.stride = rows;
  }
  return r;
}

// Log-sum-exp merge of split partials: one thread per 4 output elements of one row. IDX32: the
// launch has fewer than 2^31 threads, so the row and its (b, i, h) come from 32-bit divisions
// (a 64-bit division by a run-time value is a long instruction sequence ahead of every load).
template <bool IDX32>
__global__ void __launch_bounds__(256) fa8_combine_kernel(const CParams c) {
  typedef typename std::conditional<IDX32, uint32_t, int64_t>::type idx_t;
  const idx_t tpr = (idx_t)(c.dv / 4);
  const idx_t gt = (idx_t)blockIdx.x * blockDim.x + threadIdx.x;
  const idx_t rows = (idx_t)c.batch * c.max_sq * c.hq;
  const idx_t row = gt / tpr;
  const int q = (int)(gt - row * tpr);
  if (row >= rows) return;
  const idx_t rq = row / (idx_t)c.hq;
  const int h = (int)(row - rq * (idx_t)c.hq);
  const int b = (int)(rq / (idx_t)c.max_sq);
  const int i = (int)(rq - (idx_t)b * (idx_t)c.max_sq);
  // the sequence's query rows and its partial slots are independent loads, issued together
  const PartialRows pr = partial_rows(c, b, i, h, row, rows);
  const int q0 = c.cu_q ? c.cu_q[b] : 0;
  const int sq = c.cu_q ? c.cu_q[b + 1] - q0 : c.max_sq;
  if (i >= sq) return;
  // One pass over the splits in batches of 16 whose LSE and partial loads are all issued before
  // any is used (the kernel is bound by memory latency, not bandwidth): a running max, with the
  // sums rescaled when a batch raises it, so a problem of up to 16 splits costs one round trip.
  constexpr int SB = 16;
  // a sink logit is one more denominator term without a value
  const float z = c.sink ? c.sink[h] : kNegInf;
  float mx = z;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  float den = (z == kNegInf) ? 0.0f : 1.0f;          // e^(z - mx) with mx = z
  for (int s0 = 0; s0 < pr.n; s0 += SB) {
    float ls[SB];
    v4f o[SB];
#pragma unroll
    for (int k = 0; k < SB; k++) {
      const bool in = s0 + k < pr.n;
      const int64_t pi = pr.at(s0 + k);
      ls[k] = in ? c.lse_part[pi] : kNegInf;
      o[k] = in ? *reinterpret_cast<const v4f*>(c.o_part + pi * c.dv + 4 * q) : (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    }
    float bm = mx;
#pragma unroll
    for (int k = 0; k < SB; k++) bm = fmaxf(bm, ls[k]);
    if (bm == kNegInf) continue;                     // every split so far empty
    if (bm != mx) {                                  // rescale what the earlier batches added
      const float r = (mx == kNegInf) ? 0.0f : __expf(mx - bm);
      den *= r;
      acc *= r;
      mx = bm;
    }
#pragma unroll
    for (int k = 0; k < SB; k++) {
      // an empty split (LSE = -inf) has weight 0 and O = 0
      const float w = (ls[k] == kNegInf) ? 0.0f : __expf(ls[k] - mx);
      den += w;
      acc += w * o[k];
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

// Combine for many splits: one workgroup per (output row, block of CGP column groups of 4
// columns), SP = kWideThreads / CGP split lanes x CGP column groups. Split lane sp takes splits
// sp, sp + SP, ...; the lanes' maxima, weight sums and weighted partial rows meet in LDS. With
// S = 256 and dv = 128 each thread loads 8 splits, all issued together, instead of one row's
// thread walking 256, and each row is spread over four workgroups (a single workgroup reading a
// row's 256 partials ran at one compute unit's share of the memory bandwidth).
constexpr int kWideThreads = 256;
template <int CGP>
__global__ void __launch_bounds__(kWideThreads) fa8_combine_wide_kernel(const CParams c) {
  constexpr int SP = kWideThreads / CGP;
  constexpr int SB = 8;
  __shared__ float s_mx[SP], s_den[SP];
  __shared__ v4f s_acc[SP][CGP];
  const int tid = threadIdx.x;
  const int tpr = c.dv / 4;
  const int ncb = (tpr + CGP - 1) / CGP;                 // column blocks per row
  const int64_t rows = (int64_t)c.batch * c.max_sq * c.hq;
  const int64_t row = blockIdx.x / ncb;
  const int cb = (int)(blockIdx.x - row * ncb);
  const int q = cb * CGP + tid % CGP, sp = tid / CGP;
  const int h = (int)(row % c.hq);
  const int i = (int)((row / c.hq) % c.max_sq);
  const int b = (int)(row / ((int64_t)c.hq * c.max_sq));
  const int q0 = c.cu_q ? c.cu_q[b] : 0;
  const int sq = c.cu_q ? c.cu_q[b + 1] - q0 : c.max_sq;
  if (i >= sq) return;   // uniform over the workgroup
  const PartialRows pr = partial_rows(c, b, i, h, row, rows);
  // one pass per split lane: a running maximum rescales the lane's weight sum and accumulator
  // whenever a batch of LSEs raises it, so every partial is read once
  float mx = kNegInf, den = 0.0f;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const bool has_cols = q < tpr;
  for (int s0 = sp; s0 < pr.n; s0 += SB * SP) {
    float ls[SB];
    v4f o[SB];
#pragma unroll
    for (int k = 0; k < SB; k++) {
      const int sidx = s0 + k * SP;
      const bool in = sidx < pr.n;
      const int64_t pi = pr.at(sidx);
      ls[k] = in ? c.lse_part[pi] : kNegInf;
      o[k] = (in && has_cols) ? *reinterpret_cast<const v4f*>(c.o_part + pi * c.dv + 4 * q)
                              : (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    }
    float bm = mx;
#pragma unroll
    for (int k = 0; k < SB; k++) bm = fmaxf(bm, ls[k]);
    if (bm == kNegInf) continue;    // every split so far empty
    if (bm != mx) {
      const float r = (mx == kNegInf) ? 0.0f : __expf(mx - bm);
      den *= r;
      acc *= r;
      mx = bm;
    }
#pragma unroll
    for (int k = 0; k < SB; k++) {
      const float w = (ls[k] == kNegInf) ? 0.0f : __expf(ls[k] - mx);   // empty split: weight 0
      den += w;
      acc += w * o[k];
    }
  }
  s_acc[sp][tid % CGP] = acc;
  if (tid % CGP == 0) {
    s_mx[sp] = mx;
    s_den[sp] = den;
  }
  __syncthreads();
  if (sp != 0 || q >= tpr) return;
  // a sink logit is one more denominator term without a value (added once, here)
  const float z = c.sink ? c.sink[h] : kNegInf;
  mx = z;
#pragma unroll 8
  for (int k = 0; k < SP; k++) mx = fmaxf(mx, s_mx[k]);
  den = (z == kNegInf) ? 0.0f : __expf(z - mx);
  acc = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  if (mx != kNegInf) {
#pragma unroll 8
    for (int k = 0; k < SP; k++) {
      const float r = (s_mx[k] == kNegInf) ? 0.0f : __expf(s_mx[k] - mx);   // lane with no split: 0
      den += r * s_den[k];
      acc += r * s_acc[k][tid];
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

// KV tile of the prefill kernel: 64 keys when d + dv > 256 (a two-stage pair of 128-key tiles
// would not fit twice in LDS) and at (128, 128), where it leaves 152 VGPRs and so three waves per
// SIMD instead of two (measured 4.5% faster on the causal prefill; slower at d = 64, where 128-key
// tiles already run three); else 128.
template <int D, int DV>
constexpr int prefill_tile() { return (D == 128 && DV == 128) || (D + DV) > 256 ? 64 : 128; }

template <int D, int DV>
static hipError_t launch_prefill_t(const KParams& kp, hipStream_t stream) {
  const int64_t nwork = prefill_grid(kp);
  if (kp.page_shift >= 0)
    hipLaunchKernelGGL((fa8_prefill_kernel<D, DV, prefill_tile<D, DV>(), true>), dim3((unsigned)nwork), dim3(256), 0,
                       stream, kp);
  else
    hipLaunchKernelGGL((fa8_prefill_kernel<D, DV, prefill_tile<D, DV>(), false>), dim3((unsigned)nwork), dim3(256), 0,
                       stream, kp);
  return hipGetLastError();
}
template <int D, int DV, int NQB, int PAGEMODE, bool SCHED>
static void launch_decode_k(const KParams& kp, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa8_decode_kernel<D, DV, NQB, PAGEMODE, SCHED>), grid, dim3(64), 0, stream, kp);
}
template <int D, int DV, int NQB, bool SCHED>
static void launch_decode_q(const KParams& kp, dim3 grid, hipStream_t stream) {
  // the rows of one 64-lane load instruction (64 / (d/16) rows) lie in one page
  constexpr int rows_k = (64 % (D / 16) == 0) ? 64 / (D / 16) : 1 << 30;
  constexpr int rows_v = (64 % (DV / 16) == 0) ? 64 / (DV / 16) : 1 << 30;
  if (kp.page_shift < 0) {
    launch_decode_k<D, DV, NQB, 0, SCHED>(kp, grid, stream);
    return;
  }
  if constexpr (rows_k < (1 << 30) && rows_v < (1 << 30)) {
    if ((1 << kp.page_shift) >= rows_k && (1 << kp.page_shift) >= rows_v) {
      launch_decode_k<D, DV, NQB, 1, SCHED>(kp, grid, stream);
      return;
    }
  }
  launch_decode_k<D, DV, NQB, 2, SCHED>(kp, grid, stream);
}
// static splits: (kv head x row block, split, batch); balanced schedule: (kv head, worker, 1)
template <int D, int DV, bool SCHED>
static hipError_t launch_decode_tt(const KParams& kp, hipStream_t stream) {
  const dim3 grid = SCHED ? dim3((unsigned)kp.hkv, (unsigned)kp.nsplit, 1u)
                          : dim3((unsigned)(kp.hkv * kp.nmb), (unsigned)kp.nsplit, (unsigned)kp.batch);
  // blocks hold min(32, Sq * g) rows: one 16-row MFMA block suffices up to 16
  if ((int64_t)kp.max_sq * kp.g <= 16)
    launch_decode_q<D, DV, 1, SCHED>(kp, grid, stream);
  else
    launch_decode_q<D, DV, 2, SCHED>(kp, grid, stream);
  return hipGetLastError();
}
template <int D, int DV>
static hipError_t launch_decode_t(const KParams& kp, hipStream_t stream) {
  return launch_decode_tt<D, DV, false>(kp, stream);
}
template <int D, int DV>
static hipError_t launch_decode_sched_t(const KParams& kp, hipStream_t stream) {
  return launch_decode_tt<D, DV, true>(kp, stream);
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
hipError_t launch_prefill_mx(const KParams& kp, int d, int dv, hipStream_t stream) {
  const int64_t nwork = prefill_grid(kp);   // fixed-length inputs only: bk8 = 0
  if (d == 64 && dv == 64)
    hipLaunchKernelGGL((fa8_prefill_mx_kernel<64, 64>), dim3((unsigned)nwork), dim3(256), 0, stream, kp);
  else if (d == 128 && dv == 128)
    hipLaunchKernelGGL((fa8_prefill_mx_kernel<128, 128>), dim3((unsigned)nwork), dim3(256), 0, stream, kp);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
// ---- several kv heads per wave: applicability and launch ----
// Returns the kv heads per wave of fa8_decode_heads_kernel for this problem, or 0 when the
// per-head kernel is used: (d, dv) in {(64, 64), (128, 128)}, the heads of a token row adjacent
// in memory (head stride == head dim), 2 or 4 kv heads whose Sq * g rows fit one 16-row block,
// and (paged) pages holding at least the rows of one 64-lane load. (Eight heads per wave, two
// row blocks, measured slower: fewer waves and register spills.)
int decode_heads_applicable(const KParams& kp, int d, int dv) {
  if (!((d == 64 && dv == 64) || (d == 128 && dv == 128))) return 0;
  if (kp.k_hs != d || kp.v_hs != dv) return 0;
  const int64_t rp = (int64_t)kp.max_sq * kp.g;
  if (rp < 1 || rp > 8) return 0;
  for (int hpw = (rp <= 4 ? 4 : 2); hpw >= 2; hpw /= 2) {
    if (kp.hkv % hpw) continue;
    const int rows_per_load = 1024 / (hpw * d);
    if (kp.page_shift >= 0 && (1 << kp.page_shift) < rows_per_load) continue;
    return hpw;
  }
  return 0;
}
int decode_heads_choice(const KParams& kp, int d, int dv) {
  return kp.decode_kernel == 0 ? 0 : decode_heads_applicable(kp, d, dv);
}

template <int D, int DV, int HPW, bool PAGED, bool STEP_PAGE>
static hipError_t launch_heads_t(const KParams& kp, hipStream_t stream) {
  if (kp.sched) {
    const dim3 grid((unsigned)(kp.hkv / HPW), (unsigned)kp.nsplit, 1u);
    hipLaunchKernelGGL((fa8_decode_heads_kernel<D, DV, HPW, PAGED, STEP_PAGE, true>), grid, dim3(64), 0, stream, kp);
  } else {
    const dim3 grid((unsigned)(kp.hkv / HPW), (unsigned)kp.nsplit, (unsigned)kp.batch);
    hipLaunchKernelGGL((fa8_decode_heads_kernel<D, DV, HPW, PAGED, STEP_PAGE, false>), grid, dim3(64), 0, stream, kp);
  }
  return hipGetLastError();
}

// steps of 64 / H keys; a step lies in one page when the page holds at least that many rows
#define FA8_HEADS_CASE(DD, H)                                                         \
  if (d == DD && hpw == H) {                                                          \
    if (kp.page_shift < 0) return launch_heads_t<DD, DD, H, false, true>(kp, stream); \
    if ((1 << kp.page_shift) >= 64 / H) return launch_heads_t<DD, DD, H, true, true>(kp, stream); \
    return launch_heads_t<DD, DD, H, true, false>(kp, stream);                      \
  }

hipError_t launch_decode(const KParams& kp, int d, int dv, hipStream_t stream) {
  const int hpw = decode_heads_choice(kp, d, dv);
  if (hpw) {
    FA8_HEADS_CASE(64, 2)
    FA8_HEADS_CASE(64, 4)
    FA8_HEADS_CASE(128, 2)
    FA8_HEADS_CASE(128, 4)
    return hipErrorInvalidValue;
  }
  if (kp.sched) FA8_DISPATCH(launch_decode_sched_t, d, dv, kp, stream);
  FA8_DISPATCH(launch_decode_t, d, dv, kp, stream);
}
hipError_t launch_decode_sched(const KParams& kp, int d, int dv, int32_t workers, hipStream_t stream) {
  KParams k = kp;
  k.nsplit = workers + kp.batch;   // grid.y: one wave per possible segment (at most W + batch)
  return launch_decode(k, d, dv, stream);
}
hipError_t launch_decode_schedule(const KParams& kp, int32_t workers, int32_t* sched, hipStream_t stream) {
  hipLaunchKernelGGL(fa8_decode_schedule_kernel, dim3(1), dim3(1024), 0, stream, kp, workers, sched);
  return hipGetLastError();
}

int decode_units_per_split(const KParams& kp, int d, int dv) {
  const int hpw = decode_heads_choice(kp, d, dv);
  if (hpw) return kp.batch * (kp.hkv / hpw);
  return kp.batch * kp.hkv * kp.nmb;
}
int decode_units_per_worker(const KParams& kp, int d, int dv) {
  const int hpw = decode_heads_choice(kp, d, dv);
  return hpw ? kp.hkv / hpw : kp.hkv;
}
// Many splits over few rows: the row-per-workgroup kernel, whose split lanes load in parallel;
// otherwise one thread per 4 output elements walking the splits.
hipError_t launch_combine(const CParams& cp, hipStream_t stream) {
  const int64_t rows = (int64_t)cp.batch * cp.max_sq * cp.hq;
  // many partials per row: static splits above 16, or a schedule averaging more than 16
  // workers per sequence (cp.nsplit holds the worker count then)
  const bool wide = cp.sched ? cp.nsplit > 16 * (int64_t)cp.batch : cp.nsplit > 16;
  if (wide && rows < (1 << 20)) {
    constexpr int CGP = 8;
    const int ncb = (cp.dv / 4 + CGP - 1) / CGP;
    const dim3 grid((unsigned)(rows * ncb));
    hipLaunchKernelGGL(fa8_combine_wide_kernel<CGP>, grid, dim3(kWideThreads), 0, stream, cp);
    return hipGetLastError();
  }
  const int64_t threads = rows * (cp.dv / 4);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks * 256 < ((int64_t)1 << 31))
    hipLaunchKernelGGL(fa8_combine_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, cp);
  else
    hipLaunchKernelGGL(fa8_combine_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, cp);
  return hipGetLastError();
}

// Device address of `scratch` on the current device, looked up with hipGetSymbolAddress the first
// time a device asks (with that device current) and kept per device.
hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace fa8
