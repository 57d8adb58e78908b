// Host side of the C ABI declared in include/fa8.h: argument validation, launch configuration
// from host-known values only, the optional FA8_VALIDATE checks, and error reporting.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "fa8.h"
#include "fa8_internal.h"

namespace {

thread_local std::string g_last_error;

fa8_status fail(fa8_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fa8_status ok() {
  g_last_error.clear();
  return FA8_OK;
}

bool supported_dims(int d, int dv) {
  return (d == dv && (d == 64 || d == 96 || d == 128 || d == 192 || d == 256)) || (d == 192 && dv == 128);
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; }

int ilog2_exact(int x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < x) s++;
  return s;
}

constexpr int64_t kMaxLen = (int64_t)1 << 30;
// A launch's grid may hold at most 2^32 - 1 threads along x: 2^24 workgroups of 256 threads
// (prefill), 2^26 of 64 (decode).
constexpr int64_t kMaxGridThreads = (int64_t)1 << 32;
constexpr int64_t kMaxDecodeGridX = (int64_t)1 << 26;

fa8_status check_descale(const fa8_descale& ds, const char* name) {
  if (!ds.ptr) return FA8_OK;
  if (!aligned(ds.ptr, 4)) return fail(FA8_ERR_INVALID, "%s_descale pointer is not 4-byte aligned", name);
  if (ds.stride_b < 0 || ds.stride_h < 0) return fail(FA8_ERR_INVALID, "%s_descale strides must be >= 0", name);
  return FA8_OK;
}

// Workgroups of a prefill launch with `rows` query rows per workgroup (fa8::prefill_grid of the
// kernel parameters the launch builds).
int64_t prefill_workgroups(const fa8_fwd_params* p, int rows) {
  const int64_t nmb = ((int64_t)p->max_seqlen_q + rows - 1) / rows;
  const int64_t g = p->heads_kv > 0 ? p->heads_q / p->heads_kv : 0;
  if (p->cu_seqlens_q || p->cu_seqlens_k || p->seqused_k)
    return (int64_t)8 * (((int64_t)p->batch * p->heads_kv + 7) / 8) * nmb * g;
  return nmb * p->heads_q * p->batch;
}

// Validation shared by prefill (num_splits == 0) and decode (num_splits >= 1).
fa8_status validate(const fa8_fwd_params* p, int32_t num_splits) {
  if (!p) return fail(FA8_ERR_INVALID, "params is NULL");
  if (p->batch < 0 || p->heads_q < 0 || p->heads_kv < 0 || p->max_seqlen_q < 0 || p->max_seqlen_k < 0)
    return fail(FA8_ERR_INVALID, "negative size (batch %d, heads %d/%d, seqlens %d/%d)", p->batch, p->heads_q,
                p->heads_kv, p->max_seqlen_q, p->max_seqlen_k);
  if (!supported_dims(p->d, p->dv))
    return fail(FA8_ERR_UNSUPPORTED, "(d, dv) = (%d, %d) is not supported; use (64,64), (96,96), (128,128), "
                "(192,192), (256,256) or (192,128)", p->d, p->dv);
  if (num_splits < 0 || num_splits > FA8_MAX_SPLITS)
    return fail(FA8_ERR_INVALID, "num_splits %d outside 1..%d", num_splits, FA8_MAX_SPLITS);
  if (p->heads_kv == 0 || p->heads_q == 0) {
    if (p->heads_q != 0 || p->heads_kv != 0) return fail(FA8_ERR_INVALID, "heads_q and heads_kv must both be > 0");
  } else if (p->heads_q % p->heads_kv != 0) {
    return fail(FA8_ERR_INVALID, "heads_q (%d) must be a multiple of heads_kv (%d)", p->heads_q, p->heads_kv);
  }
  if (p->heads_q >= 65536 || p->heads_kv >= 65536) return fail(FA8_ERR_INVALID, "too many heads");
  if (p->batch >= 65536) return fail(FA8_ERR_INVALID, "batch %d >= 65536", p->batch);
  if (p->max_seqlen_q >= kMaxLen || p->max_seqlen_k >= kMaxLen) return fail(FA8_ERR_INVALID, "sequence length >= 2^30");
  if (p->out_dtype != FA8_OUT_BF16 && p->out_dtype != FA8_OUT_FP16)
    return fail(FA8_ERR_INVALID, "out_dtype %d is neither FA8_OUT_BF16 nor FA8_OUT_FP16", p->out_dtype);
  if (p->window_left < -1 || p->window_right < -1)
    return fail(FA8_ERR_INVALID, "window sizes must be >= -1 (got %d, %d)", p->window_left, p->window_right);
  const bool empty = p->batch == 0 || p->heads_q == 0 || p->max_seqlen_q == 0;
  if (empty) return FA8_OK;

  if (!p->q || !p->k || !p->v) return fail(FA8_ERR_INVALID, "q, k and v must be non-NULL");
  if (!aligned(p->q, 16) || !aligned(p->k, 16) || !aligned(p->v, 16))
    return fail(FA8_ERR_INVALID, "q, k and v must be 16-byte aligned");
  const int64_t s16[] = {p->q_row_stride, p->q_head_stride, p->k_row_stride, p->k_head_stride, p->v_row_stride,
                         p->v_head_stride, p->cu_seqlens_q ? 0 : p->q_batch_stride, p->k_batch_stride, p->v_batch_stride};
  for (int64_t s : s16)
    if (s < 0 || s % 16 != 0) return fail(FA8_ERR_INVALID, "q/k/v strides must be non-negative multiples of 16 elements");
  if (p->block_table) {
    if (ilog2_exact(p->page_size) < 0) return fail(FA8_ERR_INVALID, "page_size %d must be a power of two", p->page_size);
    if (!p->seqused_k) return fail(FA8_ERR_INVALID, "paged K/V needs seqused_k");
    if (p->cu_seqlens_k) return fail(FA8_ERR_INVALID, "paged K/V cannot also use cu_seqlens_k");
    if (p->block_table_stride < (p->max_seqlen_k + p->page_size - 1) / p->page_size)
      return fail(FA8_ERR_INVALID, "block_table_stride %lld < ceil(max_seqlen_k / page_size)",
                  (long long)p->block_table_stride);
    if (!aligned(p->block_table, 4)) return fail(FA8_ERR_INVALID, "block_table must be 4-byte aligned");
  }
  {
    // row offsets inside one page (paged) or one KV tile of up to 128 keys (contiguous) are 32-bit
    const int64_t rows = p->block_table ? (int64_t)p->page_size : 128;
    const int64_t rs = p->k_row_stride > p->v_row_stride ? p->k_row_stride : p->v_row_stride;
    if (rows * rs + 256 >= ((int64_t)1 << 31))
      return fail(FA8_ERR_INVALID, "K/V row stride %lld too large for %lld rows", (long long)rs, (long long)rows);
  }
  if (num_splits == 0) {
    if (!p->out) return fail(FA8_ERR_INVALID, "out must be non-NULL");
    if (!aligned(p->out, 8)) return fail(FA8_ERR_INVALID, "out must be 8-byte aligned");
    const int64_t so[] = {p->o_row_stride, p->o_head_stride, p->cu_seqlens_q ? 0 : p->o_batch_stride};
    for (int64_t s : so)
      if (s < 0 || s % 4 != 0) return fail(FA8_ERR_INVALID, "out strides must be non-negative multiples of 4");
    if (p->lse && !aligned(p->lse, 4)) return fail(FA8_ERR_INVALID, "lse must be 4-byte aligned");
    const int64_t wgs = prefill_workgroups(p, fa8::kPrefillRows);
    const int nt = fa8::kPrefillThreads;
    if (wgs * nt >= kMaxGridThreads)
      return fail(FA8_ERR_INVALID, "prefill needs %lld workgroups of %d threads, more than one launch can hold "
                  "(2^32 threads)", (long long)wgs, nt);
  } else {
    const int64_t rows = (int64_t)p->max_seqlen_q * (p->heads_q / p->heads_kv);
    if (rows > kMaxLen) return fail(FA8_ERR_INVALID, "too many packed decode rows");
  }
  fa8_status st;
  if ((st = check_descale(p->q_descale, "q")) != FA8_OK) return st;
  if ((st = check_descale(p->k_descale, "k")) != FA8_OK) return st;
  if ((st = check_descale(p->v_descale, "v")) != FA8_OK) return st;
  return FA8_OK;
}

// FA8_VALIDATE=1: device-data contract checks on host copies (synchronous; not graph-safe).
bool validate_env() {
  const char* e = getenv("FA8_VALIDATE");
  return e && e[0] == '1';
}

// The copies below run after everything already enqueued on the caller's stream (the index
// arrays may have just been written there): the stream is synchronized first.
template <typename T>
bool copy_down(std::vector<T>& dst, const T* src, size_t n) {
  dst.resize(n);
  if (n == 0) return true;
  return hipMemcpy(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

fa8_status validate_device_data(const fa8_fwd_params* p, void* stream) {
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
    return fail(FA8_ERR_HIP, "FA8_VALIDATE: cannot synchronize the stream");
  const int B = p->batch;
  std::vector<int32_t> cuq, cuk, used, table;
  if (p->cu_seqlens_q) {
    if (!copy_down(cuq, p->cu_seqlens_q, (size_t)B + 1)) return fail(FA8_ERR_HIP, "FA8_VALIDATE: cannot read cu_seqlens_q");
    for (int b = 0; b < B; b++) {
      const int32_t n = cuq[b + 1] - cuq[b];
      if (cuq[b] < 0 || n < 0 || n > p->max_seqlen_q)
        return fail(FA8_ERR_INVALID, "FA8_VALIDATE: cu_seqlens_q invalid at batch %d (len %d, max %d)", b, n, p->max_seqlen_q);
    }
  }
  if (p->cu_seqlens_k) {
    if (!copy_down(cuk, p->cu_seqlens_k, (size_t)B + 1)) return fail(FA8_ERR_HIP, "FA8_VALIDATE: cannot read cu_seqlens_k");
    for (int b = 0; b < B; b++) {
      const int32_t n = cuk[b + 1] - cuk[b];
      if (cuk[b] < 0 || n < 0 || (!p->seqused_k && n > p->max_seqlen_k))
        return fail(FA8_ERR_INVALID, "FA8_VALIDATE: cu_seqlens_k invalid at batch %d", b);
    }
  }
  if (p->seqused_k) {
    if (!copy_down(used, p->seqused_k, (size_t)B)) return fail(FA8_ERR_HIP, "FA8_VALIDATE: cannot read seqused_k");
    for (int b = 0; b < B; b++)
      if (used[b] < 0 || used[b] > p->max_seqlen_k || (!cuk.empty() && used[b] > cuk[b + 1] - cuk[b]))
        return fail(FA8_ERR_INVALID, "FA8_VALIDATE: seqused_k[%d] = %d out of range", b, used[b]);
  }
  if (p->block_table) {
    if (!copy_down(table, p->block_table, (size_t)B * (size_t)p->block_table_stride))
      return fail(FA8_ERR_HIP, "FA8_VALIDATE: cannot read block_table");
    for (int b = 0; b < B; b++) {
      const int np = (used[b] + p->page_size - 1) / p->page_size;
      for (int j = 0; j < np; j++)
        if (table[(size_t)b * p->block_table_stride + j] < 0)
          return fail(FA8_ERR_INVALID, "FA8_VALIDATE: negative page index at batch %d entry %d", b, j);
    }
  }
  return FA8_OK;
}

fa8::KParams make_kparams(const fa8_fwd_params* p) {
  fa8::KParams k;
  memset(&k, 0, sizeof k);
  k.q = (const uint8_t*)p->q;
  k.k = (const uint8_t*)p->k;
  k.v = (const uint8_t*)p->v;
  k.q_bs = p->q_batch_stride; k.q_rs = p->q_row_stride; k.q_hs = p->q_head_stride;
  k.k_bs = p->k_batch_stride; k.k_rs = p->k_row_stride; k.k_hs = p->k_head_stride;
  k.v_bs = p->v_batch_stride; k.v_rs = p->v_row_stride; k.v_hs = p->v_head_stride;
  k.cu_q = p->cu_seqlens_q;
  k.cu_k = p->block_table ? nullptr : p->cu_seqlens_k;
  k.used_k = p->seqused_k;
  k.table = p->block_table;
  k.table_stride = p->block_table_stride;
  k.page_shift = p->block_table ? ilog2_exact(p->page_size) : -1;
  k.dq = p->q_descale.ptr; k.dq_sb = p->q_descale.stride_b; k.dq_sh = p->q_descale.stride_h;
  k.dk = p->k_descale.ptr; k.dk_sb = p->k_descale.stride_b; k.dk_sh = p->k_descale.stride_h;
  k.dv = p->v_descale.ptr; k.dv_sb = p->v_descale.stride_b; k.dv_sh = p->v_descale.stride_h;
  const double scale = p->softmax_scale > 0.0f ? (double)p->softmax_scale : 1.0 / std::sqrt((double)p->d);
  k.scale_log2 = (float)(scale * 1.4426950408889634);
  k.batch = p->batch; k.hq = p->heads_q; k.hkv = p->heads_kv; k.g = p->heads_q / p->heads_kv;
  k.max_sq = p->max_seqlen_q; k.max_sk = p->max_seqlen_k;
  // a window at least as long as any sequence is no window
  const int64_t span = (int64_t)p->max_seqlen_q + p->max_seqlen_k;
  k.wl = (p->window_left < 0 || p->window_left >= span) ? -1 : p->window_left;
  k.wr = p->causal ? 0 : ((p->window_right < 0 || p->window_right >= span) ? -1 : p->window_right);
  k.causal = p->causal ? 1 : 0;
  k.out = p->out; k.o_bs = p->o_batch_stride; k.o_rs = p->o_row_stride; k.o_hs = p->o_head_stride;
  k.out_fp16 = p->out_dtype == FA8_OUT_FP16;
  k.o_vec16 = aligned(p->out, 16) && p->o_row_stride % 8 == 0 && p->o_head_stride % 8 == 0 &&
              (p->cu_seqlens_q || p->o_batch_stride % 8 == 0);
  k.lse = p->lse; k.l_bs = p->lse_batch_stride; k.l_hs = p->lse_head_stride; k.l_rs = p->lse_row_stride;
  k.sink = p->sink;
  k.decode_kernel = -1;
  return k;
}

}  // namespace

extern "C" {

const char* fa8_last_error(void) { return g_last_error.c_str(); }

const char* fa8_version(void) { return "fa8 0.1.0 gfx950"; }

fa8_status fa8_check_params(const fa8_fwd_params* p, int32_t num_splits) {
  fa8_status st = validate(p, num_splits);
  return st == FA8_OK ? ok() : st;
}

}  // extern "C"

namespace {
// Split count for `units` one-wave workgroups per split: about `waves_per_cu` waves per compute
// unit, without splits shorter than four granules, within 1 .. FA8_MAX_SPLITS.
int32_t splits_for(int64_t units, int32_t max_seqlen_k, int32_t cu_count, int waves_per_cu) {
  if (cu_count <= 0) cu_count = 256;
  units = std::max<int64_t>(1, units);
  const int64_t target = (int64_t)cu_count * waves_per_cu;
  const int64_t granules = ((int64_t)max_seqlen_k + FA8_SPLIT_GRANULE - 1) / FA8_SPLIT_GRANULE;
  int64_t s = (target + units - 1) / units;
  s = std::min<int64_t>(s, std::max<int64_t>(1, granules / 4));
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(s, FA8_MAX_SPLITS));
}
// Waves per compute unit the split heuristic aims at: several-heads kernel about one per SIMD
// (more concurrent streams measured slower), per-head kernel about four per SIMD (measured best
// at the paged GQA decode shape).
constexpr int kHeadsWavesPerCu = 4, kPerHeadWavesPerCu = 16;

int decode_kernel_for(const fa8::KParams& k, const fa8_fwd_params* p, int32_t requested, fa8_status* st) {
  *st = FA8_OK;
  if (requested < -1 || requested > 1) {
    *st = fail(FA8_ERR_INVALID, "decode kernel %d is not one of -1, 0, 1", requested);
    return 0;
  }
  if (requested == 1 && !fa8::decode_heads_applicable(k, p->d, p->dv)) {
    *st = fail(FA8_ERR_UNSUPPORTED, "the several-heads decode kernel cannot take this problem");
    return 0;
  }
  return requested;
}
}  // namespace

extern "C" {

int32_t fa8_decode_num_splits(int32_t batch, int32_t heads_kv, int32_t max_seqlen_k, int32_t cu_count) {
  if (batch <= 0 || heads_kv <= 0 || max_seqlen_k <= 0) return 1;
  return splits_for((int64_t)batch * heads_kv, max_seqlen_k, cu_count, kPerHeadWavesPerCu);
}

int32_t fa8_decode_num_splits_for(const fa8_fwd_params* p, int32_t cu_count) {
  if (!p || validate(p, 1) != FA8_OK) return 1;
  if (p->batch <= 0 || p->heads_kv <= 0 || p->max_seqlen_k <= 0 || p->max_seqlen_q <= 0) return 1;
  fa8::KParams k = make_kparams(p);
  const int64_t rows = (int64_t)p->max_seqlen_q * k.g;
  k.nmb = (int32_t)((rows + fa8::kDecodeRows - 1) / fa8::kDecodeRows);
  const bool heads = fa8::decode_heads_choice(k, p->d, p->dv) != 0;
  return splits_for(fa8::decode_units_per_split(k, p->d, p->dv), p->max_seqlen_k, cu_count,
                    heads ? kHeadsWavesPerCu : kPerHeadWavesPerCu);
}

fa8_status fa8_decode_plan_ex(const fa8_fwd_params* p, int32_t num_splits, int32_t kernel,
                              fa8_decode_plan_info* info) {
  if (!info) return fail(FA8_ERR_INVALID, "info must be non-NULL");
  if (num_splits < 1) return fail(FA8_ERR_INVALID, "num_splits must be >= 1 (got %d)", num_splits);
  fa8_status st = validate(p, num_splits);
  if (st != FA8_OK) return st;
  fa8::KParams k = make_kparams(p);
  k.nsplit = num_splits;
  const int64_t rows = (int64_t)p->max_seqlen_q * k.g;
  k.nmb = (int32_t)((rows + fa8::kDecodeRows - 1) / fa8::kDecodeRows);
  k.decode_kernel = decode_kernel_for(k, p, kernel, &st);
  if (st != FA8_OK) return st;
  const int hpw = fa8::decode_heads_choice(k, p->d, p->dv);
  if (hpw) {
    info->kernel = 1;
    info->block_keys = 64 / hpw;
    info->key_groups = 1;
    info->heads_per_workgroup = hpw;
  } else {
    info->kernel = 0;
    info->block_keys = fa8::kKvTile;
    info->key_groups = 1;
    info->heads_per_workgroup = 1;
  }
  info->workgroups = (int64_t)fa8::decode_units_per_split(k, p->d, p->dv) * num_splits;
  return ok();
}

fa8_status fa8_decode_plan(const fa8_fwd_params* p, int32_t num_splits, fa8_decode_plan_info* info) {
  return fa8_decode_plan_ex(p, num_splits, -1, info);
}

size_t fa8_decode_workspace_bytes(int32_t num_splits, int32_t batch, int32_t max_seqlen_q, int32_t heads_q,
                                  int32_t dv) {
  if (num_splits < 0 || batch < 0 || max_seqlen_q < 0 || heads_q < 0 || dv < 0) return 0;
  const unsigned __int128 rows = (unsigned __int128)num_splits * batch * max_seqlen_q * heads_q;
  const unsigned __int128 ob = rows * dv * 4, lb = rows * 4;
  const unsigned __int128 tot = ((ob + 255) / 256) * 256 + ((lb + 255) / 256) * 256;
  if (tot > (unsigned __int128)SIZE_MAX) return 0;
  return (size_t)tot;
}

fa8_status fa8_fwd_prefill(const fa8_fwd_params* p, void* stream) {
  fa8_status st = validate(p, 0);
  if (st != FA8_OK) return st;
  if (p->batch == 0 || p->heads_q == 0 || p->max_seqlen_q == 0) return ok();
  if (validate_env() && (st = validate_device_data(p, stream)) != FA8_OK) return st;
  fa8::KParams k = make_kparams(p);
  const int rows = fa8::kPrefillRows;
  k.nmb = (p->max_seqlen_q + rows - 1) / rows;
  // lengths read on the device: deal the (batch, kv head) groups to the XCDs round-robin
  if (p->cu_seqlens_q || p->cu_seqlens_k || p->seqused_k)
    k.bk8 = (int32_t)(((int64_t)p->batch * p->heads_kv + 7) / 8);
  if (fa8::prefill_grid(k) != prefill_workgroups(p, rows)) return fail(FA8_ERR_INVALID, "internal: prefill grid mismatch");
  hipError_t e = fa8::launch_prefill(k, p->d, p->dv, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA8_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa8_status fa8_fwd_prefill_mx(const fa8_fwd_params* p, const fa8_mx_scales* s, void* stream) {
  if (!s) return fail(FA8_ERR_INVALID, "MX scales must be non-NULL");
  fa8_status st = validate(p, 0);
  if (st != FA8_OK) return st;
  if (!((p->d == 64 && p->dv == 64) || (p->d == 128 && p->dv == 128)))
    return fail(FA8_ERR_UNSUPPORTED, "MX prefill supports (d, dv) = (64, 64) or (128, 128), not (%d, %d)", p->d, p->dv);
  if (p->cu_seqlens_q || p->cu_seqlens_k || p->seqused_k || p->block_table)
    return fail(FA8_ERR_UNSUPPORTED, "MX prefill takes fixed-length Q and K/V only");
  if (p->q_descale.ptr || p->k_descale.ptr || p->v_descale.ptr)
    return fail(FA8_ERR_INVALID, "MX prefill takes no descales (the block scales replace them)");
  if (!s->q || !s->k || !s->v) return fail(FA8_ERR_INVALID, "MX scale pointers must be non-NULL");
  const int64_t nb = p->d / 32;
  auto mult = [](int64_t x, int64_t m) { return x % m == 0; };
  if (!mult((int64_t)(uintptr_t)s->q, nb) || !mult(s->q_batch_stride, nb) || !mult(s->q_row_stride, nb) ||
      !mult(s->q_head_stride, nb) || !mult((int64_t)(uintptr_t)s->k, nb) || !mult(s->k_batch_stride, nb) ||
      !mult(s->k_row_stride, nb) || !mult(s->k_head_stride, nb))
    return fail(FA8_ERR_INVALID, "Q/K scale pointers and strides must be multiples of d/32 = %d", (int)nb);
  if (!mult((int64_t)(uintptr_t)s->v, 16) || !mult(s->v_batch_stride, 16) || !mult(s->v_block_stride, 16) ||
      !mult(s->v_head_stride, 16))
    return fail(FA8_ERR_INVALID, "V scale pointer and strides must be multiples of 16");
  if (s->q_batch_stride < 0 || s->q_row_stride < 0 || s->q_head_stride < 0 || s->k_batch_stride < 0 ||
      s->k_row_stride < 0 || s->k_head_stride < 0 || s->v_batch_stride < 0 || s->v_block_stride < 0 ||
      s->v_head_stride < 0)
    return fail(FA8_ERR_INVALID, "MX scale strides must be non-negative");
  if (p->batch == 0 || p->heads_q == 0 || p->max_seqlen_q == 0) return ok();
  fa8::KParams k = make_kparams(p);
  k.nmb = (p->max_seqlen_q + fa8::kPrefillRows - 1) / fa8::kPrefillRows;
  if (fa8::prefill_grid(k) != prefill_workgroups(p, fa8::kPrefillRows))
    return fail(FA8_ERR_INVALID, "internal: prefill grid mismatch");
  k.q_mx = s->q; k.qmx_bs = s->q_batch_stride; k.qmx_rs = s->q_row_stride; k.qmx_hs = s->q_head_stride;
  k.k_mx = s->k; k.kmx_bs = s->k_batch_stride; k.kmx_rs = s->k_row_stride; k.kmx_hs = s->k_head_stride;
  k.v_mx = s->v; k.vmx_bs = s->v_batch_stride; k.vmx_ts = s->v_block_stride; k.vmx_hs = s->v_head_stride;
  hipError_t e = fa8::launch_prefill_mx(k, p->d, p->dv, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA8_ERR_HIP, "MX prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa8_status fa8_fwd_decode_splitkv_ex(const fa8_fwd_params* p, int32_t num_splits, int32_t kernel, float* o_partial,
                                     float* lse_partial, void* stream) {
  if (num_splits < 1) return fail(FA8_ERR_INVALID, "num_splits must be >= 1 (got %d)", num_splits);
  fa8_status st = validate(p, num_splits);
  if (st != FA8_OK) return st;
  fa8::KParams k = make_kparams(p);
  k.decode_kernel = decode_kernel_for(k, p, kernel, &st);
  if (st != FA8_OK) return st;
  if (p->batch == 0 || p->heads_q == 0 || p->max_seqlen_q == 0) return ok();
  if (!o_partial || !lse_partial) return fail(FA8_ERR_INVALID, "o_partial and lse_partial must be non-NULL");
  if (!aligned(o_partial, 16) || !aligned(lse_partial, 4))
    return fail(FA8_ERR_INVALID, "o_partial must be 16-byte aligned and lse_partial 4-byte aligned");
  if (validate_env() && (st = validate_device_data(p, stream)) != FA8_OK) return st;
  k.o_part = o_partial;
  k.lse_part = lse_partial;
  k.nsplit = num_splits;
  const int64_t rows = (int64_t)p->max_seqlen_q * k.g;
  k.nmb = (int32_t)((rows + fa8::kDecodeRows - 1) / fa8::kDecodeRows);
  if ((int64_t)k.nmb * p->heads_kv >= kMaxDecodeGridX) return fail(FA8_ERR_INVALID, "decode grid too large");
  hipError_t e = fa8::launch_decode(k, p->d, p->dv, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA8_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa8_status fa8_fwd_decode_splitkv(const fa8_fwd_params* p, int32_t num_splits, float* o_partial, float* lse_partial,
                                  void* stream) {
  return fa8_fwd_decode_splitkv_ex(p, num_splits, -1, o_partial, lse_partial, stream);
}

// ---- balanced decode schedule ----
size_t fa8_decode_schedule_bytes(int32_t batch) {
  if (batch < 0) return 0;
  return (size_t)(2 + 2 * ((int64_t)batch + 1)) * sizeof(int32_t);
}

size_t fa8_decode_scheduled_workspace_bytes(int32_t num_workers, int32_t batch, int32_t max_seqlen_q, int32_t heads_q,
                                            int32_t dv) {
  if (num_workers < 1 || batch < 0) return 0;
  return fa8_decode_workspace_bytes((int32_t)std::min<int64_t>((int64_t)num_workers + batch, INT32_MAX), 1,
                                    max_seqlen_q, heads_q, dv);
}

int32_t fa8_decode_num_workers(const fa8_fwd_params* p, int32_t cu_count) {
  if (!p || validate(p, 1) != FA8_OK) return 1;
  if (p->batch <= 0 || p->heads_kv <= 0 || p->max_seqlen_k <= 0 || p->max_seqlen_q <= 0) return 1;
  fa8::KParams k = make_kparams(p);
  k.nmb = 1;
  if (cu_count <= 0) cu_count = 256;
  const int64_t units = std::max(1, fa8::decode_units_per_worker(k, p->d, p->dv));
  // about one wave per SIMD for either kernel (equal shares leave no idle tail to fill, and more
  // concurrent streams measured slower); the segments cut at sequence ends add up to batch more
  const int64_t target = (int64_t)cu_count * kHeadsWavesPerCu;
  // at least four granules per worker on average when every sequence is max_seqlen_k long
  const int64_t granules = (int64_t)p->batch * (((int64_t)p->max_seqlen_k + FA8_SPLIT_GRANULE - 1) / FA8_SPLIT_GRANULE);
  int64_t w = (target + units - 1) / units;
  w = std::min<int64_t>(w, std::max<int64_t>(1, granules / 4));
  w = std::min<int64_t>(w, FA8_MAX_WORKERS - p->batch);
  return (int32_t)std::max<int64_t>(1, w);
}

namespace {
fa8_status validate_scheduled(const fa8_fwd_params* p, int32_t num_workers) {
  fa8_status st = validate(p, 1);
  if (st != FA8_OK) return st;
  if (num_workers < 1 || (int64_t)num_workers + p->batch > FA8_MAX_WORKERS)
    return fail(FA8_ERR_INVALID, "num_workers %d outside 1 .. %d - batch", num_workers, FA8_MAX_WORKERS);
  if ((int64_t)p->max_seqlen_q * (p->heads_kv > 0 ? p->heads_q / p->heads_kv : 0) > fa8::kDecodeRows)
    return fail(FA8_ERR_UNSUPPORTED, "the balanced decode schedule takes at most %d packed rows per kv head "
                "(max_seqlen_q x heads_q / heads_kv)", fa8::kDecodeRows);
  return FA8_OK;
}
}  // namespace

fa8_status fa8_decode_schedule(const fa8_fwd_params* p, int32_t num_workers, int32_t* schedule, void* stream) {
  fa8_status st = validate_scheduled(p, num_workers);
  if (st != FA8_OK) return st;
  if (!schedule || !aligned(schedule, 4)) return fail(FA8_ERR_INVALID, "schedule must be non-NULL and 4-byte aligned");
  if (p->batch == 0) return ok();
  if (validate_env() && (st = validate_device_data(p, stream)) != FA8_OK) return st;
  fa8::KParams k = make_kparams(p);
  hipError_t e = fa8::launch_decode_schedule(k, num_workers, schedule, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA8_ERR_HIP, "schedule launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa8_status fa8_fwd_decode_scheduled(const fa8_fwd_params* p, int32_t num_workers, int32_t* schedule,
                                    int32_t kernel, float* o_partial, float* lse_partial, void* stream) {
  fa8_status st = validate_scheduled(p, num_workers);
  if (st != FA8_OK) return st;
  fa8::KParams k = make_kparams(p);
  k.decode_kernel = decode_kernel_for(k, p, kernel, &st);
  if (st != FA8_OK) return st;
  if (p->batch == 0 || p->heads_q == 0 || p->max_seqlen_q == 0) return ok();
  if (!schedule || !aligned(schedule, 4)) return fail(FA8_ERR_INVALID, "schedule must be non-NULL and 4-byte aligned");
  if (!o_partial || !lse_partial) return fail(FA8_ERR_INVALID, "o_partial and lse_partial must be non-NULL");
  if (!aligned(o_partial, 16) || !aligned(lse_partial, 4))
    return fail(FA8_ERR_INVALID, "o_partial must be 16-byte aligned and lse_partial 4-byte aligned");
  k.o_part = o_partial;
  k.lse_part = lse_partial;
  k.nmb = 1;
  k.sched = schedule;
  k.sched_out = schedule;
  k.sched_workers = num_workers;
  if (p->heads_kv >= kMaxDecodeGridX) return fail(FA8_ERR_INVALID, "decode grid too large");
  // up to 64 sequences every wave derives the schedule from the lengths itself (and the first
  // writes it for the combine); beyond, the schedule kernel writes it first
  k.sched_inline = p->batch <= 64 ? 1 : 0;
  hipError_t e = hipSuccess;
  if (!k.sched_inline) e = fa8::launch_decode_schedule(k, num_workers, schedule, (hipStream_t)stream);
  if (e == hipSuccess) e = fa8::launch_decode_sched(k, p->d, p->dv, num_workers, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA8_ERR_HIP, "scheduled decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

fa8_status fa8_fwd_decode_noalloc(const fa8_fwd_params* p, int32_t num_splits, void* stream) {
  if (!p) return fail(FA8_ERR_INVALID, "params is NULL");
  if (num_splits == 0) num_splits = fa8_decode_num_splits_for(p, 0);
  if (num_splits < 1) return fail(FA8_ERR_INVALID, "num_splits must be >= 1, or 0 (got %d)", num_splits);
  fa8_status st = validate(p, num_splits);
  if (st != FA8_OK) return st;
  if (p->batch == 0 || p->heads_q == 0 || p->max_seqlen_q == 0) return ok();
  // the combine's output checks, before anything is launched
  if (!p->out || !aligned(p->out, 8)) return fail(FA8_ERR_INVALID, "out must be non-NULL and 8-byte aligned");
  const int64_t so[] = {p->o_row_stride, p->o_head_stride, p->cu_seqlens_q ? 0 : p->o_batch_stride};
  for (int64_t s : so)
    if (s < 0 || s % 4 != 0) return fail(FA8_ERR_INVALID, "out strides must be non-negative multiples of 4");
  if (p->lse && !aligned(p->lse, 4)) return fail(FA8_ERR_INVALID, "lse must be 4-byte aligned");
  const size_t need = fa8_decode_workspace_bytes(num_splits, p->batch, p->max_seqlen_q, p->heads_q, p->dv);
  if (need == 0 || need > (size_t)FA8_NOALLOC_SCRATCH_BYTES)
    return fail(FA8_ERR_INVALID, "the split partials need %zu bytes; the library's scratch holds %zu (fewer splits, "
                "or fa8_fwd_decode_splitkv with caller buffers)", need, (size_t)FA8_NOALLOC_SCRATCH_BYTES);
  void* base = nullptr;
  hipError_t e = fa8::noalloc_scratch(&base);
  if (e != hipSuccess) return fail(FA8_ERR_HIP, "cannot resolve the scratch address: %s", hipGetErrorString(e));
  const size_t o_bytes = (size_t)num_splits * p->batch * p->max_seqlen_q * p->heads_q * p->dv * sizeof(float);
  float* op = (float*)base;
  float* lp = (float*)((uint8_t*)base + (o_bytes + 255) / 256 * 256);
  if ((st = fa8_fwd_decode_splitkv(p, num_splits, op, lp, stream)) != FA8_OK) return st;
  return fa8_combine(op, lp, num_splits, p->batch, p->max_seqlen_q, p->cu_seqlens_q, p->heads_q, p->dv, p->out,
                     p->o_batch_stride, p->o_row_stride, p->o_head_stride, p->out_dtype, p->lse, p->lse_batch_stride,
                     p->lse_head_stride, p->lse_row_stride, p->sink, stream);
}

namespace {
fa8_status combine_impl(const float* o_partial, const float* lse_partial, const int32_t* sched, int32_t num_splits,
                        int32_t batch, int32_t max_seqlen_q, const int32_t* cu_seqlens_q, int32_t heads_q, int32_t dv,
                        void* out, int64_t o_batch_stride, int64_t o_row_stride, int64_t o_head_stride,
                        int32_t out_dtype, float* lse, int64_t lse_batch_stride, int64_t lse_head_stride,
                        int64_t lse_row_stride, const float* sink, void* stream);
}  // namespace

fa8_status fa8_combine_scheduled(const float* o_partial, const float* lse_partial, const int32_t* schedule,
                                 int32_t num_workers, int32_t batch, int32_t max_seqlen_q, const int32_t* cu_seqlens_q,
                                 int32_t heads_q, int32_t dv, void* out, int64_t o_batch_stride, int64_t o_row_stride,
                                 int64_t o_head_stride, int32_t out_dtype, float* lse, int64_t lse_batch_stride,
                                 int64_t lse_head_stride, int64_t lse_row_stride, const float* sink, void* stream) {
  if (num_workers < 1 || (int64_t)num_workers + batch > FA8_MAX_WORKERS)
    return fail(FA8_ERR_INVALID, "num_workers %d outside 1 .. %d - batch", num_workers, FA8_MAX_WORKERS);
  if (!schedule || !aligned(schedule, 4)) return fail(FA8_ERR_INVALID, "schedule must be non-NULL and 4-byte aligned");
  return combine_impl(o_partial, lse_partial, schedule, num_workers, batch, max_seqlen_q, cu_seqlens_q, heads_q, dv,
                      out, o_batch_stride, o_row_stride, o_head_stride, out_dtype, lse, lse_batch_stride,
                      lse_head_stride, lse_row_stride, sink, stream);
}

fa8_status fa8_combine(const float* o_partial, const float* lse_partial, int32_t num_splits, int32_t batch,
                       int32_t max_seqlen_q, const int32_t* cu_seqlens_q, int32_t heads_q, int32_t dv, void* out,
                       int64_t o_batch_stride, int64_t o_row_stride, int64_t o_head_stride, int32_t out_dtype,
                       float* lse, int64_t lse_batch_stride, int64_t lse_head_stride, int64_t lse_row_stride,
                       const float* sink, void* stream) {
  if (num_splits < 1 || num_splits > FA8_MAX_SPLITS)
    return fail(FA8_ERR_INVALID, "num_splits %d outside 1..%d", num_splits, FA8_MAX_SPLITS);
  return combine_impl(o_partial, lse_partial, nullptr, num_splits, batch, max_seqlen_q, cu_seqlens_q, heads_q, dv, out,
                      o_batch_stride, o_row_stride, o_head_stride, out_dtype, lse, lse_batch_stride, lse_head_stride,
                      lse_row_stride, sink, stream);
}

}  // extern "C"

namespace {
fa8_status combine_impl(const float* o_partial, const float* lse_partial, const int32_t* sched, int32_t num_splits,
                        int32_t batch, int32_t max_seqlen_q, const int32_t* cu_seqlens_q, int32_t heads_q, int32_t dv,
                        void* out, int64_t o_batch_stride, int64_t o_row_stride, int64_t o_head_stride,
                        int32_t out_dtype, float* lse, int64_t lse_batch_stride, int64_t lse_head_stride,
                        int64_t lse_row_stride, const float* sink, void* stream) {
  if (batch < 0 || max_seqlen_q < 0 || heads_q < 0 || max_seqlen_q >= kMaxLen || heads_q >= 65536 || batch >= 65536)
    return fail(FA8_ERR_INVALID, "bad sizes (batch %d, max_seqlen_q %d, heads_q %d)", batch, max_seqlen_q, heads_q);
  if (dv != 64 && dv != 96 && dv != 128 && dv != 192 && dv != 256)
    return fail(FA8_ERR_UNSUPPORTED, "dv = %d is not supported", dv);
  if (out_dtype != FA8_OUT_BF16 && out_dtype != FA8_OUT_FP16) return fail(FA8_ERR_INVALID, "bad out_dtype %d", out_dtype);
  if (batch == 0 || max_seqlen_q == 0 || heads_q == 0) return ok();
  if (!o_partial || !lse_partial || !out) return fail(FA8_ERR_INVALID, "o_partial, lse_partial and out must be non-NULL");
  if (!aligned(o_partial, 16) || !aligned(lse_partial, 4) || !aligned(out, 8) || (lse && !aligned(lse, 4)))
    return fail(FA8_ERR_INVALID, "misaligned pointer");
  const int64_t so[] = {o_row_stride, o_head_stride, cu_seqlens_q ? 0 : o_batch_stride};
  for (int64_t s : so)
    if (s < 0 || s % 4 != 0) return fail(FA8_ERR_INVALID, "out strides must be non-negative multiples of 4");
  fa8::CParams c;
  memset(&c, 0, sizeof c);
  c.o_part = o_partial; c.lse_part = lse_partial; c.nsplit = num_splits;
  c.batch = batch; c.max_sq = max_seqlen_q; c.hq = heads_q; c.dv = dv; c.cu_q = cu_seqlens_q;
  c.out = out; c.o_bs = o_batch_stride; c.o_rs = o_row_stride; c.o_hs = o_head_stride;
  c.out_fp16 = out_dtype == FA8_OUT_FP16;
  c.lse = lse; c.l_bs = lse_batch_stride; c.l_hs = lse_head_stride; c.l_rs = lse_row_stride;
  c.sink = sink;
  c.sched = sched;
  hipError_t e = fa8::launch_combine(c, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA8_ERR_HIP, "combine launch failed: %s", hipGetErrorString(e));
  return ok();
}
}  // namespace

// ---- Q quantizer ----
namespace {
fa8_status validate_quant(const fa8_quant_params* p) {
  if (!p) return fail(FA8_ERR_INVALID, "params is NULL");
  if (p->batch < 0 || p->heads_q <= 0 || p->heads_kv <= 0 || p->max_seqlen_q < 0)
    return fail(FA8_ERR_INVALID, "batch, heads and max_seqlen_q must be non-negative (heads > 0)");
  if (p->heads_q % p->heads_kv) return fail(FA8_ERR_INVALID, "heads_q must be a multiple of heads_kv");
  if (!(p->d == 64 || p->d == 96 || p->d == 128 || p->d == 192 || p->d == 256))
    return fail(FA8_ERR_UNSUPPORTED, "head dim %d is not supported", p->d);
  if (p->in_dtype != FA8_OUT_BF16 && p->in_dtype != FA8_OUT_FP16)
    return fail(FA8_ERR_INVALID, "in_dtype must be FA8_OUT_BF16 or FA8_OUT_FP16");
  if (p->batch >= (1 << 16) || p->heads_q >= (1 << 16) || (int64_t)p->max_seqlen_q >= kMaxLen)
    return fail(FA8_ERR_INVALID, "sizes out of range");
  if (p->batch == 0 || p->max_seqlen_q == 0) return FA8_OK;
  if (!p->q || !p->q_out || !p->q_descale) return fail(FA8_ERR_INVALID, "q, q_out and q_descale must be non-NULL");
  if (!aligned(p->q, 16) || !aligned(p->q_out, 8) || !aligned(p->q_descale, 4))
    return fail(FA8_ERR_INVALID, "q must be 16-byte, q_out 8-byte and q_descale 4-byte aligned");
  if ((p->q_row_stride | p->q_head_stride | (p->cu_seqlens_q ? 0 : p->q_batch_stride)) % 8)
    return fail(FA8_ERR_INVALID, "q strides must be multiples of 8 elements");
  if ((p->o_row_stride | p->o_head_stride | (p->cu_seqlens_q ? 0 : p->o_batch_stride)) % 8)
    return fail(FA8_ERR_INVALID, "q_out strides must be multiples of 8 bytes");
  if (p->q_row_stride < 0 || p->q_head_stride < 0 || p->q_batch_stride < 0 || p->o_row_stride < 0 ||
      p->o_head_stride < 0 || p->o_batch_stride < 0)
    return fail(FA8_ERR_INVALID, "strides must be non-negative");
  return FA8_OK;
}
int64_t quant_chunks(const fa8_quant_params* p) { return ((int64_t)p->max_seqlen_q + fa8::kQuantRows - 1) / fa8::kQuantRows; }
}  // namespace

extern "C" int64_t fa8_quantize_q_workspace_bytes(const fa8_quant_params* p) {
  if (!p || p->batch <= 0 || p->heads_kv <= 0 || p->max_seqlen_q <= 0) return 0;
  return (int64_t)p->batch * p->heads_kv * quant_chunks(p) * (int64_t)sizeof(float);
}

extern "C" fa8_status fa8_quantize_q(const fa8_quant_params* p, void* workspace, void* stream) {
  fa8_status st = validate_quant(p);
  if (st != FA8_OK) return st;
  if (p->batch == 0 || p->max_seqlen_q == 0) return ok();
  if (!workspace || !aligned(workspace, 4)) return fail(FA8_ERR_INVALID, "workspace must be non-NULL and 4-byte aligned");
  const int64_t nchunk = quant_chunks(p);
  if (nchunk >= ((int64_t)1 << 31)) return fail(FA8_ERR_INVALID, "max_seqlen_q too large");
  fa8::QParams q{};
  q.q = p->q; q.q_bs = p->q_batch_stride; q.q_rs = p->q_row_stride; q.q_hs = p->q_head_stride;
  q.in_fp16 = p->in_dtype == FA8_OUT_FP16;
  q.cu_q = p->cu_seqlens_q;
  q.q_out = p->q_out; q.o_bs = p->o_batch_stride; q.o_rs = p->o_row_stride; q.o_hs = p->o_head_stride;
  q.descale = p->q_descale;
  q.ws = (float*)workspace;
  q.batch = p->batch; q.max_sq = p->max_seqlen_q; q.hkv = p->heads_kv; q.g = p->heads_q / p->heads_kv;
  q.d = p->d; q.nchunk = (int32_t)nchunk;
  hipError_t e = fa8::launch_quantize_q(q, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA8_ERR_HIP, "quantizer launch failed: %s", hipGetErrorString(e));
  return ok();
}
