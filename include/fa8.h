/*
 * fa8.h: C ABI of an FP8 (E4M3) attention forward for AMD Instinct MI355X (gfx950).
 *
 * Computes O = softmax(Q K^T * scale) V with E4M3FN Q/K/V, an online softmax in exp2 with lazy
 * rescaling, P pre-scaled by 2^8 and rounded to E4M3, and two-level PV accumulation into fp32 O
 * ("[Cute,Fwd,Sm90] Native FP8 (E4M3 Q/K/V) forward for Hopper", Summary and Design; the
 * lazy-rescale bound log2(448) - 8 from "fp8 on the sheared forward", Correctness fix).
 *
 * General rules for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library never allocates,
 *    frees, synchronizes, or copies device memory to the host (except the optional validator
 *    enabled by the environment variable FA8_VALIDATE=1, which copies index arrays to the host
 *    and therefore must not be used during stream capture).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and is
 *    asynchronous. Every launch decision depends only on the host-side values in the arguments,
 *    never on device data, so a call may be captured in a HIP graph and replayed.
 *  - Q/K/V are E4M3FN bytes (OCP 8-bit float: bias 7, 3 mantissa bits, max 448, no infinities).
 *    E5M2 or mixed formats cannot be expressed through this ABI.
 *  - Strides are in ELEMENTS of the tensor (bytes for E4M3, 2-byte units for fp16/bf16 output,
 *    4-byte units for fp32). The last dimension (d or dv) is always contiguous. Q/K/V base
 *    pointers must be 16-byte aligned and their strides multiples of 16; output and LSE strides
 *    must keep 8-byte alignment of every 4-element group (output strides multiples of 4).
 *  - A status other than FA8_OK means nothing was launched; fa8_last_error() then returns a
 *    thread-local message describing the problem.
 *  - Contract violations that only device data can reveal are the caller's responsibility and
 *    are undefined behaviour (out-of-bounds device reads or writes): a block table narrower than
 *    ceil(seqused_k[b] / page_size) entries for some b, a page index >= the pool size, a
 *    sequence length above max_seqlen_q / max_seqlen_k, or cu_seqlens that are not
 *    nondecreasing. FA8_VALIDATE=1 checks what the ABI can see (lengths against the maxima,
 *    monotone cu_seqlens, non-negative page indices; the pool size is not an argument) on host
 *    copies and returns FA8_ERR_INVALID on a violation; it first synchronizes `stream` (so that it
 *    sees index arrays written there), which is why it cannot run under stream capture.
 */
#ifndef FA8_H
#define FA8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA8_OK = 0,
  FA8_ERR_INVALID = 1,      /* a bad argument: shape, stride, pointer, alignment, limit */
  FA8_ERR_UNSUPPORTED = 2,  /* a valid request this library does not implement (e.g. (d, dv)) */
  FA8_ERR_HIP = 3           /* the HIP runtime reported an error when launching */
} fa8_status;

typedef enum { FA8_OUT_BF16 = 0, FA8_OUT_FP16 = 1 } fa8_out_dtype;

/* Keys per split granule of the split-KV decode (see fa8_fwd_decode_splitkv). */
#define FA8_SPLIT_GRANULE 64
/* Packed (query token, query head) rows per block of the split-KV decode. */
#define FA8_DECODE_BLOCK_ROWS 32
/* Largest number of splits fa8_fwd_decode_splitkv and fa8_combine accept. */
#define FA8_MAX_SPLITS 256

/*
 * A dequantization scale ("descale") for Q, K or V: the real value of an element is its
 * E4M3 value times the descale. The page's descales are 0-d or (batch, kv_heads), contiguous
 * or broadcast, read in place ("Native FP8 ... for Hopper", Design, Descales):
 *   ptr == NULL                  -> 1.0
 *   stride_b == stride_h == 0    -> one scalar *ptr
 *   otherwise                    -> ptr[b * stride_b + kv_head * stride_h] (fp32, device)
 * Q's descale is indexed by the KV head of the query head (kv_head = h / (heads_q / heads_kv)).
 * Q and K descales multiply the softmax scale; the V descale multiplies the output after the
 * softmax normalization.
 */
typedef struct {
  const float* ptr;
  int64_t stride_b;
  int64_t stride_h;
} fa8_descale;

/*
 * Problem description shared by fa8_fwd_prefill, fa8_fwd_decode_splitkv and fa8_check_params.
 *
 * Q and O: fixed length [batch, max_seqlen_q, heads_q, d] (O: dv) addressed with
 *   (q_batch_stride, q_row_stride, q_head_stride); or varlen [total_q, heads_q, d] when
 *   cu_seqlens_q ([batch + 1] int32, device) is set: sequence b owns token rows
 *   cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and q_batch_stride is ignored.
 * K and V: fixed length [batch, max_seqlen_k, heads_kv, d|dv]; varlen [total_k, heads_kv, d|dv]
 *   with cu_seqlens_k; or paged [num_pages, page_size, heads_kv, d|dv] when block_table is set,
 *   where *_batch_stride is the PAGE stride, and key j of sequence b lives in page
 *   block_table[b * block_table_stride + j / page_size] at row j % page_size.
 *   page_size must be a power of two.
 * Key lengths: seqused_k[b] if set, else from cu_seqlens_k, else max_seqlen_k. Paged K/V
 *   requires seqused_k.
 * Masks (rows aligned bottom-right: query i of a sequence sits at key position
 *   i' = i + Sk_b - Sq_b, so the newest query sees the whole sequence): key j is visible to
 *   query i iff j < Sk_b, j <= i' + wr and j >= i' - wl, where wr = 0 if causal else
 *   window_right (no bound if < 0) and wl = window_left (no bound if < 0). A row with no
 *   visible key gets O = 0 and LSE = -inf.
 * GQA: heads_q must be a multiple of heads_kv; query head h reads kv head h / (heads_q/heads_kv).
 * softmax_scale: <= 0 selects 1/sqrt(d).
 * lse (optional, fp32): natural-log log-sum-exp of the scaled scores per row, at
 *   lse[b * lse_batch_stride + h * lse_head_stride + i * lse_row_stride] (fixed length) or
 *   lse[h * lse_head_stride + (cu_seqlens_q[b] + i) * lse_row_stride] (varlen).
 * sink (optional, device, [heads_q] fp32): a learnable sink logit z_h per query head, in
 *   natural-log units (not multiplied by softmax_scale or the descales). It joins the softmax
 *   denominator and carries no value: O = dv * sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{z_h}),
 *   LSE = ln(sum_j e^{s_j} + e^{z_h}); a row with no visible key gets O = 0 and LSE = z_h
 *   ("Native FP8 ... for Hopper", Summary, lists the learnable sink among the supported
 *   features; the sheared fp8 page, Summary, carries the 2^8 P offset through the sink term).
 *   fa8_fwd_prefill adds it at the end of each row; fa8_fwd_decode_splitkv leaves it out of the
 *   partials and fa8_combine adds it once. NULL: no sink.
 * (d, dv) must be one of (64,64), (96,96), (128,128), (192,192), (256,256), (192,128)
 *   ("Native FP8 ... for Hopper", Supported); anything else is FA8_ERR_UNSUPPORTED.
 * Sizes: every dimension >= 0 (an empty problem launches nothing and returns FA8_OK); batch < 2^16;
 *   max_seqlen_q, max_seqlen_k < 2^30; heads < 2^16.
 * Score precision: the scores S = Q K^T are computed by the FP8 matrix cores, whose dot products
 *   carry an error up to about 2^-14 of sum_i |q_i k_i| (measured on gfx950, unscaled and
 *   block-scaled operands alike); each scaled score, and so the LSE, carries that error times
 *   softmax_scale * q_descale * k_descale. For inputs of ordinary magnitude (scores of a few
 *   units) it is far below the E4M3 rounding of P; it grows with the magnitude of the products.
 */
typedef struct {
  int32_t batch, heads_q, heads_kv, d, dv;
  int32_t max_seqlen_q, max_seqlen_k;
  const void* q;
  const void* k;
  const void* v;
  int64_t q_batch_stride, q_row_stride, q_head_stride;
  int64_t k_batch_stride, k_row_stride, k_head_stride;
  int64_t v_batch_stride, v_row_stride, v_head_stride;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const int32_t* seqused_k;
  const int32_t* block_table;
  int64_t block_table_stride;
  int32_t page_size;
  fa8_descale q_descale, k_descale, v_descale;
  float softmax_scale;
  int32_t causal, window_left, window_right;
  void* out;                       /* fp16 or bf16 per out_dtype */
  int64_t o_batch_stride, o_row_stride, o_head_stride;
  int32_t out_dtype;               /* fa8_out_dtype */
  float* lse;                      /* optional */
  int64_t lse_batch_stride, lse_head_stride, lse_row_stride;
  const float* sink;               /* optional, [heads_q] */
} fa8_fwd_params;

/*
 * Full forward pass into p->out (and p->lse when set): one workgroup per block of query rows
 * of one query head, looping over the visible KV tiles ("Native FP8 ... for Hopper", Design;
 * the method's steps: FP8 Q K^T, scale and mask, lazy-rescaled exp2 softmax with the 2^8 P
 * bias, E4M3 P, FP8 PV accumulated into fp32 O, v descale and 1/l at the end). Works for
 * fixed, varlen and paged K/V. KV tile: 64 keys at (d, dv) = (128, 128) and when d + dv > 256,
 * else 128, counted from key 0 of the sequence; each tile is one step of the online softmax (row max, lazy rescale of l
 * and O, P, PV onto O; the matrix cores add their accumulator input at fp32 precision, so O
 * needs no separate per-tile fold). FA8_ERR_INVALID also when the launch would need 2^32 or
 * more threads: ceil(max_seqlen_q / 128) x query heads x batch workgroups of 256 threads (for
 * varlen or seqused_k inputs the batch x kv-head count is rounded up to a multiple of 8 first).
 * The grid is sized from host-side values only, so with varlen inputs every sequence gets the row
 * blocks of max_seqlen_q; those past a sequence's own length return at once, and a batch of one
 * long and many short sequences launches mostly such idle workgroups (each costs a dispatch).
 */
fa8_status fa8_fwd_prefill(const fa8_fwd_params* p, void* stream);

/*
 * Split-KV partial pass for decode-shaped problems ("Native FP8 ... for Hopper", Decode
 * launches: a direct (head, split, batch) grid; the q heads sharing a KV head are packed into
 * the rows of one tile). Writes, for every split s, the attention restricted to that split's
 * keys, already normalized, plus its LSE:
 *   o_partial  [num_splits, batch, max_seqlen_q, heads_q, dv] fp32, contiguous
 *   lse_partial[num_splits, batch, max_seqlen_q, heads_q]     fp32, contiguous
 * (fa8_decode_workspace_bytes gives the combined size). Rows past a sequence's own Sq_b are
 * not written. Split partition: the query rows of one (batch, kv head) block see the keys of
 * granules [g0, g1) of FA8_SPLIT_GRANULE keys (the union of their visible ranges, rounded out
 * to granules); split s covers granules [g0 + floor(s*n/S), g0 + floor((s+1)*n/S)), n = g1-g0,
 * intersected with each row's own visible keys. An empty split writes O = 0, LSE = -inf.
 * Row blocks: the (query token i, query head h) pairs of one (batch, kv head) are packed as
 * rows r = i * g + (h - kv_head * g), g = heads_q / heads_kv, and cut into blocks of
 * FA8_DECODE_BLOCK_ROWS consecutive rows; each block is partitioned into splits on its own.
 * p->out and p->lse are not touched; fa8_combine produces them.
 * num_splits: 1 .. FA8_MAX_SPLITS.
 */
fa8_status fa8_fwd_decode_splitkv(const fa8_fwd_params* p, int32_t num_splits, float* o_partial,
                                  float* lse_partial, void* stream);

/*
 * For callers that cannot allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the split-KV decode and its combine in one call, writing
 * p->out (and p->lse when set) exactly as fa8_fwd_decode_splitkv into caller buffers followed by
 * fa8_combine would, with the split partials held in a scratch area the library owns: one static
 * device array of FA8_NOALLOC_SCRATCH_BYTES per GPU, kept until the process ends. Nothing is
 * allocated or freed. num_splits: 1 .. FA8_MAX_SPLITS, or 0 for fa8_decode_num_splits_for(p, 0).
 * FA8_ERR_INVALID when the partials (fa8_decode_workspace_bytes) do not fit the scratch area,
 * or for the argument errors of fa8_fwd_decode_splitkv and fa8_combine. Every call on one GPU
 * uses the same scratch: calls that may overlap on one GPU (several streams, several threads)
 * race and must be serialized by the caller. No part of the scratch needs clearing: every
 * partial the combine reads is written by the decode first.
 */
#define FA8_NOALLOC_SCRATCH_BYTES (32u << 20)
fa8_status fa8_fwd_decode_noalloc(const fa8_fwd_params* p, int32_t num_splits, void* stream);

/*
 * Balanced split-KV decode for skewed sequence lengths: the split counts follow each request's
 * length, computed on the device into a caller-owned buffer of fixed size, so every launch
 * decision stays host-side and a graph that replays these calls sees fresh lengths each time
 * (the static splits of fa8_fwd_decode_splitkv give a long and a short sequence the same number
 * of splits, which leaves the waves of short sequences idle at the end; the Hopper FP8 page lists
 * dynamic per-request splits among the features it does not include, and the FlashInfer
 * fp8_paged_mqa_logits page describes a device-side schedule with the hazard of replaying a stale
 * one under CUDA graphs). Two calls, in stream order:
 *   fa8_fwd_decode_scheduled derives the schedule for num_workers workers from the device-side
 *                            lengths, writes it into `schedule` and writes the partials, one wave
 *                            per (kv head unit, segment) (up to 64 sequences every wave derives
 *                            the schedule itself; beyond, one small kernel writes it first);
 *   fa8_combine_scheduled    reads the schedule and merges each row's partials into out / lse.
 * fa8_decode_schedule writes the same schedule on its own (to inspect it, or to size work).
 * Partition: each sequence's visible keys (the union over its query rows, rounded out to
 * FA8_SPLIT_GRANULE-key granules as for the static splits) are laid end to end, G granules in
 * all; worker w of W takes granules [floor(w G / W), floor((w + 1) G / W)) of that list, so every
 * worker has the same number of granules within one. The segments of a sequence are its workers
 * owner(first granule) .. owner(last granule), owner(x) = floor(((x + 1) W - 1) / G) (when W > G
 * some workers hold no granule, and such a worker between two of a sequence's workers gives it an
 * empty segment); each is one online softmax over its keys (as one static split) and writes one
 * partial (an empty one O = 0, LSE = -inf), at partial slot j for the j-th segment in (sequence,
 * worker) order.
 * Schedule layout (int32, fa8_decode_schedule_bytes(batch)): [0] G, [1] W, then the exclusive
 * prefix of the sequences' granule counts ([batch + 1] entries), then the exclusive prefix of
 * their segment counts ([batch + 1] entries; sequence b owns slots pst[b] .. pst[b+1]-1).
 * Partials: o_partial [num_workers + batch, max_seqlen_q, heads_q, dv] and lse_partial
 * [num_workers + batch, max_seqlen_q, heads_q] fp32 (fa8_decode_scheduled_workspace_bytes; at
 * most W + batch - 1 slots are used). Limits: num_workers + batch <= FA8_MAX_WORKERS; at most 32
 * packed rows (max_seqlen_q x heads_q / heads_kv) per kv head, else FA8_ERR_UNSUPPORTED.
 * kernel: as for fa8_fwd_decode_splitkv_ex. The combine must read the schedule the decode wrote
 * for the same lengths (same stream, in order); a schedule left from other lengths gives wrong
 * merges.
 */
#define FA8_MAX_WORKERS 65535
size_t fa8_decode_schedule_bytes(int32_t batch);
size_t fa8_decode_scheduled_workspace_bytes(int32_t num_workers, int32_t batch, int32_t max_seqlen_q,
                                            int32_t heads_q, int32_t dv);
/* Workers for the balanced decode from host-side values only: about one wave per SIMD (4 per
 * compute unit over the kv head units of a worker), at least four granules per worker on average
 * when every sequence is max_seqlen_k long. cu_count <= 0 means 256. */
int32_t fa8_decode_num_workers(const fa8_fwd_params* p, int32_t cu_count);
fa8_status fa8_decode_schedule(const fa8_fwd_params* p, int32_t num_workers, int32_t* schedule, void* stream);
fa8_status fa8_fwd_decode_scheduled(const fa8_fwd_params* p, int32_t num_workers, int32_t* schedule,
                                    int32_t kernel, float* o_partial, float* lse_partial, void* stream);
fa8_status fa8_combine_scheduled(const float* o_partial, const float* lse_partial, const int32_t* schedule,
                                 int32_t num_workers, int32_t batch, int32_t max_seqlen_q,
                                 const int32_t* cu_seqlens_q, int32_t heads_q, int32_t dv, void* out,
                                 int64_t o_batch_stride, int64_t o_row_stride, int64_t o_head_stride,
                                 int32_t out_dtype, float* lse, int64_t lse_batch_stride,
                                 int64_t lse_head_stride, int64_t lse_row_stride, const float* sink,
                                 void* stream);

/* Decode kernels fa8_fwd_decode_splitkv_ex can be asked for (fa8_decode_plan_info.kernel).
 * AUTO is the library's choice (what fa8_fwd_decode_splitkv uses). PER_HEAD takes every problem.
 * HEAD_GROUP (several kv heads per wave, whole token rows) takes (d, dv) = (64, 64) or
 * (128, 128) with the heads of a token row adjacent in memory (head stride = head dim), at most
 * 8 packed rows (max_seqlen_q x heads_q / heads_kv) per kv head, heads_kv a multiple of 2 and,
 * when paged, pages of at least 1024 / (heads per wave x d) rows; other problems return
 * FA8_ERR_UNSUPPORTED. Both compute the same partition and the same method; their blocking
 * differs (fa8_decode_plan_ex), so results may differ in rounding. */
typedef enum {
  FA8_DECODE_AUTO = -1,
  FA8_DECODE_PER_HEAD = 0,
  FA8_DECODE_HEAD_GROUP = 1
} fa8_decode_kernel;

/* fa8_fwd_decode_splitkv with an explicit kernel choice (a fa8_decode_kernel value). */
fa8_status fa8_fwd_decode_splitkv_ex(const fa8_fwd_params* p, int32_t num_splits, int32_t kernel,
                                     float* o_partial, float* lse_partial, void* stream);

/*
 * Merges split partials into the final output: LSE = log sum_s exp(LSE_s),
 * O = sum_s exp(LSE_s - LSE) * O_s, written as fp16/bf16 (round to nearest even). Rows whose
 * splits are all empty get O = 0 and LSE = -inf. The split-KV combine is part of each decode
 * step ("Native FP8 ... for Hopper", Performance). Layouts of o_partial / lse_partial as for
 * fa8_fwd_decode_splitkv; out/lse addressing as in fa8_fwd_params (cu_seqlens_q may be NULL
 * for fixed-length rows; lse may be NULL). sink (optional, [heads_q] fp32, as in
 * fa8_fwd_params): one more term e^{z_h} of the denominator with no value, i.e.
 * LSE = log(sum_s exp(LSE_s) + exp(z_h)); rows with every split empty then get O = 0, LSE = z_h.
 */
fa8_status fa8_combine(const float* o_partial, const float* lse_partial, int32_t num_splits,
                       int32_t batch, int32_t max_seqlen_q, const int32_t* cu_seqlens_q,
                       int32_t heads_q, int32_t dv, void* out, int64_t o_batch_stride,
                       int64_t o_row_stride, int64_t o_head_stride, int32_t out_dtype, float* lse,
                       int64_t lse_batch_stride, int64_t lse_head_stride, int64_t lse_row_stride,
                       const float* sink, void* stream);

/*
 * Per-(batch, kv head) FP8 quantization of a bf16 or fp16 Q, the step before the attention path
 * (the block quantization formula of the FlashAttention-3 page, "Low-Precision FP8 Attention
 * with Block Scaling": scale = max|X_block| / 448, X_fp8 = clip(round(X / scale), -448, 448)).
 * The block is every query row of sequence b and the q heads h with h / (heads_q / heads_kv)
 * == kvh, the granularity of fa8_fwd_params.q_descale. Each code is decided in fp32:
 * s = amax / 448 (s = 1 for a block of zeros or an empty sequence), y = x / s (IEEE division),
 * clip to [-448, 448], round to nearest even E4M3FN. Outputs: q_out (E4M3 bytes, its own
 * strides) and q_descale[b * heads_kv + kvh] = s, ready to pass as a (batch, kv_heads) descale.
 * q: [batch, max_seqlen_q, heads_q, d] (strides in elements) or varlen [total_q, heads_q, d] with
 * cu_seqlens_q; in_dtype: FA8_OUT_BF16 or FA8_OUT_FP16 (the element type of q). d must be one of
 * the supported head dims; q, q_out and their row and head strides 16-byte / 8-byte aligned.
 * workspace: fa8_quantize_q_workspace_bytes(p) bytes of device memory (4-byte aligned), caller
 * owned, contents irrelevant on entry. Two launches on stream; nothing is allocated.
 */
typedef struct {
  int32_t batch, heads_q, heads_kv, d, max_seqlen_q;
  const void* q;
  int32_t in_dtype;
  int64_t q_batch_stride, q_row_stride, q_head_stride;    /* elements */
  const int32_t* cu_seqlens_q;
  void* q_out;
  int64_t o_batch_stride, o_row_stride, o_head_stride;    /* bytes */
  float* q_descale;                                       /* [batch, heads_kv] */
} fa8_quant_params;

int64_t fa8_quantize_q_workspace_bytes(const fa8_quant_params* p);
fa8_status fa8_quantize_q(const fa8_quant_params* p, void* workspace, void* stream);

/*
 * MXFP8 forward pass (the MXFP8 forward of the FlashAttention-4 MXFP8 page, sections 1, 2.1
 * and 2.1.3): Q, K and V are E4M3FN elements with E8M0 block scales, one scale per 32
 * elements along each product's contraction dimension: along d for Q and K, along the keys
 * for V. An E8M0 scale is one unsigned byte e with value 2^(e - 127); 0xFF is NaN (OCP
 * Microscaling Formats specification). The real value of an element is its E4M3 value times
 * its block's scale. Both products run on the block-scaled MFMA: S = Q K^T with the Q and K
 * scales, then O = P V with P converted online to MXFP8: for each query row and each block of
 * 32 keys, the block's largest score x (log2 units, s * softmax_scale * log2 e) against the
 * row's running max m gives the shared exponent X = ceil(x - m - log2 448): the smallest power
 * of two that brings the block's largest P = 2^(x - m) to at most 448, so no element is clipped
 * (evaluated with a margin of a few fp32 ulps of m, which can raise X by one next to an integer)
 * (the page derives its scale from the block amax's exponent and mantissa bits; the amax
 * itself comes from the softmax's block maxima), clamped to [-127, 127]. The block stores
 * E4M3(2^(s' - m - X)) (s' the scaled score, round to nearest even) with scale 2^X. The online
 * softmax keeps the
 * lazy rescale of fa8_fwd_prefill (the running max moves only when a tile's max exceeds it by
 * more than 0.75); there is no 2^8 offset (the block scales cover the range). The row sum is
 * taken over the stored P times its scales, and each tile's PV is accumulated onto fp32 O on
 * the matrix cores as in fa8_fwd_prefill.
 *
 * p: as for fa8_fwd_prefill with these limits: (d, dv) = (64, 64) or (128, 128); fixed-length
 *   Q and K/V (cu_seqlens_q, cu_seqlens_k, seqused_k and block_table NULL); the descales of p
 *   must be absent (ptr NULL: the block scales replace them). Masks, GQA, softmax_scale, lse,
 *   sink and out_dtype as for fa8_fwd_prefill.
 * s: the three scale tensors (uint8 E8M0, device, caller owned; strides in bytes, last
 *   dimension contiguous):
 *   q: [batch, max_seqlen_q, heads_q, d/32]  element (b, i, h, c) at
 *      q + b*q_batch_stride + i*q_row_stride + h*q_head_stride + c
 *   k: [batch, max_seqlen_k, heads_kv, d/32] (same addressing with k_*)
 *   v: [batch, ceil(max_seqlen_k/32), heads_kv, dv]: the scale of keys 32t .. 32t+31 of
 *      column c at v + b*v_batch_stride + t*v_block_stride + kvh*v_head_stride + c
 *   q and k pointers and strides must be multiples of d/32; v's pointer and strides multiples
 *   of 16. Otherwise FA8_ERR_INVALID; other shapes or layouts FA8_ERR_UNSUPPORTED.
 */
typedef struct {
  const uint8_t* q;
  int64_t q_batch_stride, q_row_stride, q_head_stride;
  const uint8_t* k;
  int64_t k_batch_stride, k_row_stride, k_head_stride;
  const uint8_t* v;
  int64_t v_batch_stride, v_block_stride, v_head_stride;
} fa8_mx_scales;

fa8_status fa8_fwd_prefill_mx(const fa8_fwd_params* p, const fa8_mx_scales* s, void* stream);

/* Runs the host-side validation of fa8_fwd_prefill (num_splits == 0) or of
 * fa8_fwd_decode_splitkv (num_splits >= 1) without launching anything, so that a caller can
 * check a problem before graph capture. Needs no GPU. The checks are the interface limits the
 * Hopper FP8 page states (Design and Supported: the (d, dv) set, E4M3 inputs, 0-d or
 * (batch, kv_heads) descales, the 32-bit offsets inside a tile) plus this ABI's own layout rules
 * above. */
fa8_status fa8_check_params(const fa8_fwd_params* p, int32_t num_splits);

/* Split count from host-side values only, so that it holds under graph capture ("Native FP8 ...
 * for Hopper", Design, Decode launches: static splits chosen from host-known sizes): the count
 * fa8_decode_num_splits_for gives for the per-head decode kernel with one row block per
 * (batch, kv head) (max_seqlen_q x heads_q / heads_kv <= 32): about 16 workgroups per compute
 * unit over batch x heads_kv x splits, without splits shorter than four granules. cu_count <= 0
 * means 256 (MI355X). Always returns 1 .. FA8_MAX_SPLITS. */
int32_t fa8_decode_num_splits(int32_t batch, int32_t heads_kv, int32_t max_seqlen_k, int32_t cu_count);

/* Split count for fa8_fwd_decode_splitkv on the problem p (host-side values only, graph-safe),
 * for the decode kernel the library will pick for it: enough workgroups to keep cu_count compute
 * units busy over a few rounds, without splits shorter than four granules. cu_count <= 0 means
 * 256 (MI355X). Returns 1 .. FA8_MAX_SPLITS; 1 when p is NULL or fails validation. */
int32_t fa8_decode_num_splits_for(const fa8_fwd_params* p, int32_t cu_count);

/* How fa8_fwd_decode_splitkv computes a problem; the result is identical for every call with
 * the same host-side values. Within one split, the keys are processed in blocks of block_keys
 * keys (counted from key 0): one online-softmax step (row max, lazy rescale, P, PV) per block.
 * key_groups independent online-softmax states may share a split: state k takes the blocks b
 * with b mod key_groups == k, and the states of a row are merged by the same log-sum-exp rule
 * as fa8_combine before the split's partial is written (the split-KV construction of "Native
 * FP8 ... for Hopper", Design, Decode launches); the kernels here use key_groups = 1.
 * kernel: 0 = one wave per (kv head, split, batch, 32-row block); 1 = one wave per (group of
 * heads_per_workgroup kv heads, split, batch), whose rows fill one 16-row MFMA block. Needs no
 * GPU. */
typedef struct {
  int32_t kernel;
  int32_t block_keys;
  int32_t key_groups;
  int32_t heads_per_workgroup;
  int64_t workgroups;
} fa8_decode_plan_info;
fa8_status fa8_decode_plan(const fa8_fwd_params* p, int32_t num_splits, fa8_decode_plan_info* info);
/* The same for an explicit kernel choice (a fa8_decode_kernel value; FA8_ERR_UNSUPPORTED when that
 * kernel cannot take the problem). */
fa8_status fa8_decode_plan_ex(const fa8_fwd_params* p, int32_t num_splits, int32_t kernel,
                              fa8_decode_plan_info* info);

/* Bytes of o_partial + lse_partial for the given problem (o_partial first, then lse_partial,
 * each 256-byte aligned), or 0 on overflow: the caller-owned split-KV workspace, fp32 partial O
 * and LSE per split ("Native FP8 ... for Hopper", Design, Decode launches: the split partials
 * merged by the combine that the Performance section times inside each decode step). */
size_t fa8_decode_workspace_bytes(int32_t num_splits, int32_t batch, int32_t max_seqlen_q,
                                  int32_t heads_q, int32_t dv);

/* Thread-local description of the last non-OK status returned on this thread ("" if none): the
 * message behind FA8_ERR_INVALID / FA8_ERR_UNSUPPORTED, which the Hopper FP8 page's Design has
 * raised for unsupported inputs (E5M2, mixed dtypes, MLA, block sparsity, other head dims). */
const char* fa8_last_error(void);

/* Library version string. */
const char* fa8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA8_H */
