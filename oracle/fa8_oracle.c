/*
 * fa8 oracle: exact attention in fp64 on E4M3-dequantized inputs.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header or table with the
 * HIP library; it is deliberately plain and slow so that it can be checked by eye.
 *
 * What it computes (the definition of the forward pass that the FP8 kernels approximate;
 * "Native FP8 (E4M3 Q/K/V) forward for Hopper", Summary and Design sections, and the
 * sheared-forward fp8 page, Summary):
 *
 *   for each batch b, query head h, query row i:
 *     kvh   = h / (Hq / Hkv)                       (q heads of a group are consecutive)
 *     q, k_j, v_j = E4M3FN-decoded bytes           (decode table below)
 *     i'    = i + Sk_b - Sq_b                      (bottom-right aligned causal/window)
 *     J     = { j in [0, Sk_b) : j <= i' + wr, j >= i' - wl } ∩ [klo, khi)
 *             wr = 0 when causal, else window_right (unbounded if < 0);
 *             wl = window_left (unbounded if < 0)
 *     r_j   = sum_c q_c k_{j,c}                    (exact in fp64, see note)
 *     s_j   = softmax_scale * dq[b,kvh] * dk[b,kvh] * r_j
 *     m     = max_J s_j,  w_j = exp(s_j - m),  l = sum_J w_j
 *     O     = dv[b,kvh] * sum_J w_j v_j / l,    LSE = m + ln l   (natural log)
 *     J empty  ->  O = 0, LSE = -inf
 *
 *   with a learnable sink (one logit z_h per query head, natural-log units, not scaled by the
 *   softmax scale; listed among the supported features of the Hopper FP8 page, Summary, and
 *   carried through the row sum by the sheared fp8 page, Summary): the sink joins the softmax
 *   denominator and carries no value,
 *     l     = sum_J exp(s_j - m) + exp(z_h - m),  m = max(max_J s_j, z_h)
 *     O     = dv[b,kvh] * sum_J w_j v_j / l,    LSE = m + ln l
 *     J empty  ->  O = 0, LSE = z_h
 *
 *   with MXFP8 block scales (the MXFP8 forward of the FlashAttention-4 MXFP8 page, sections 1
 *   and 2.1: E4M3 elements with one E8M0 scale per 32 elements along each product's
 *   contraction dimension, i.e. along d for Q and K and along the keys for V; E8M0 as defined
 *   by the OCP Microscaling Formats specification: an unsigned 8-bit exponent with bias 127,
 *   value 2^(e - 127), 0xFF = NaN):
 *     q_c   = E4M3(q8_c) * 2^(qs[c / 32] - 127)     per query row
 *     k_j,c = E4M3(k8_j,c) * 2^(ks_j[c / 32] - 127) per key row
 *     v_j,c = E4M3(v8_j,c) * 2^(vs[j / 32][c] - 127)   key blocks counted from the sequence start
 *   and otherwise the same definition (descales, when also given, still multiply).
 *
 * Note: every E4M3 value is an integer multiple of 2^-9 with magnitude <= 448 = 229376*2^-9,
 * so each product q_c*k_c is an integer multiple of 2^-18 below 2^36 * 2^-18 and any sum of up
 * to 256 of them stays below 2^44 * 2^-18: the dot product is exact in fp64 whatever the order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* E4M3FN as defined by the OCP 8-bit floating point specification: 1 sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals (m/8) * 2^-6; the
 * pattern S.1111.111 is NaN; there are no infinities; the largest finite value is 448. */
static double e4m3_value(unsigned code) {
  unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
  double mag;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

static double g_table[256];
static int g_table_ready = 0;
static void build_table(void) {
  if (g_table_ready) return;
  for (unsigned c = 0; c < 256; c++) g_table[c] = e4m3_value(c);
  g_table_ready = 1;
}

void fa8_oracle_e4m3_table(double* out256) {
  build_table();
  for (int c = 0; c < 256; c++) out256[c] = g_table[c];
}

typedef struct {
  int32_t batch, heads_q, heads_kv, d, dv;
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  /* element (byte) strides */
  int64_t q_ss, q_sh;          /* Q: per token, per head */
  const int64_t* q_base;       /* [B] offset of batch b's first query token */
  const int32_t* seqlen_q;     /* [B] */
  int64_t k_ss, k_sh, v_ss, v_sh;   /* K/V: per token (within a page when paged), per head */
  const int64_t* k_base;       /* [B] offset of batch b's first key (non-paged) */
  const int64_t* v_base;       /* [B] */
  const int32_t* seqlen_k;     /* [B] */
  const int32_t* block_table;  /* [B, bt_stride] or NULL */
  int64_t bt_stride;
  int32_t page_size;
  int64_t k_ps, v_ps;          /* page strides (paged only) */
  const double* q_descale;     /* [B*Hkv], row-major (b, kvh) */
  const double* k_descale;
  const double* v_descale;
  double softmax_scale;
  int32_t causal, window_left, window_right;
  const double* sink;          /* [Hq] sink logits, or NULL (no sink) */
  /* MXFP8 block scales (E8M0 bytes), each NULL when absent; non-paged layouts only.
   * Q: [.., d/32] per query row at q_mx + qmx_base[b] + i*qmx_ss + h*qmx_sh;
   * K: [.., d/32] per key row at k_mx + kmx_base[b] + j*kmx_ss + kvh*kmx_sh;
   * V: [.., dv] per 32-key block at v_mx + vmx_base[b] + (j/32)*vmx_sb + kvh*vmx_sh. */
  const uint8_t* q_mx;
  int64_t qmx_ss, qmx_sh;
  const int64_t* qmx_base;
  const uint8_t* k_mx;
  int64_t kmx_ss, kmx_sh;
  const int64_t* kmx_base;
  const uint8_t* v_mx;
  int64_t vmx_sb, vmx_sh;
  const int64_t* vmx_base;
} fa8_oracle_params;

/* E8M0 scale byte (OCP Microscaling Formats): 2^(e - 127); 0xFF encodes NaN. */
static double e8m0_value(unsigned e) {
  if (e == 255u) return NAN;
  return ldexp(1.0, (int)e - 127);
}

static int64_t key_offset(const fa8_oracle_params* p, int b, int64_t j, int kvh, int is_v) {
  int64_t ss = is_v ? p->v_ss : p->k_ss, sh = is_v ? p->v_sh : p->k_sh;
  if (p->block_table) {
    int64_t page = p->block_table[(int64_t)b * p->bt_stride + j / p->page_size];
    int64_t ps = is_v ? p->v_ps : p->k_ps;
    return page * ps + (j % p->page_size) * ss + (int64_t)kvh * sh;
  }
  const int64_t* base = is_v ? p->v_base : p->k_base;
  return base[b] + j * ss + (int64_t)kvh * sh;
}

/* One output row. scores: scratch of at least Sk_b doubles. */
static void one_row(const fa8_oracle_params* p, int b, int h, int i, int64_t klo, int64_t khi,
                    double* scores, double* out, double* lse) {
  int g = p->heads_q / p->heads_kv;
  int kvh = h / g;
  int64_t sq = p->seqlen_q[b], sk = p->seqlen_k[b];
  int64_t ip = (int64_t)i + sk - sq;
  int64_t lo = 0, hi = sk;
  int64_t wr = p->causal ? 0 : p->window_right;
  if (wr >= 0 && ip + wr + 1 < hi) hi = ip + wr + 1;
  if (p->window_left >= 0 && ip - p->window_left > lo) lo = ip - p->window_left;
  if (klo > lo) lo = klo;
  if (khi < hi) hi = khi;
  const double z = p->sink ? p->sink[h] : -INFINITY;
  for (int c = 0; c < p->dv; c++) out[c] = 0.0;
  if (hi <= lo) { *lse = z; return; }

  double dq = p->q_descale ? p->q_descale[b * p->heads_kv + kvh] : 1.0;
  double dk = p->k_descale ? p->k_descale[b * p->heads_kv + kvh] : 1.0;
  double dv = p->v_descale ? p->v_descale[b * p->heads_kv + kvh] : 1.0;
  double sigma = p->softmax_scale * dq * dk;

  const uint8_t* qrow = p->q + p->q_base[b] + (int64_t)i * p->q_ss + (int64_t)h * p->q_sh;
  double qv[512];
  for (int c = 0; c < p->d; c++) qv[c] = g_table[qrow[c]];
  if (p->q_mx) {
    const uint8_t* qs = p->q_mx + p->qmx_base[b] + (int64_t)i * p->qmx_ss + (int64_t)h * p->qmx_sh;
    for (int c = 0; c < p->d; c++) qv[c] *= e8m0_value(qs[c / 32]);
  }

  double m = -INFINITY;
  for (int64_t j = lo; j < hi; j++) {
    const uint8_t* krow = p->k + key_offset(p, b, j, kvh, 0);
    const uint8_t* ks = p->k_mx ? p->k_mx + p->kmx_base[b] + j * p->kmx_ss + (int64_t)kvh * p->kmx_sh : NULL;
    double r = 0.0;
    for (int c = 0; c < p->d; c++) r += qv[c] * (ks ? g_table[krow[c]] * e8m0_value(ks[c / 32]) : g_table[krow[c]]);
    double s = sigma * r;
    scores[j - lo] = s;
    if (s > m) m = s;
  }
  if (z > m) m = z;
  double l = (z == -INFINITY) ? 0.0 : exp(z - m);
  for (int64_t j = lo; j < hi; j++) {
    double w = exp(scores[j - lo] - m);
    l += w;
    const uint8_t* vrow = p->v + key_offset(p, b, j, kvh, 1);
    const uint8_t* vs = p->v_mx ? p->v_mx + p->vmx_base[b] + (j / 32) * p->vmx_sb + (int64_t)kvh * p->vmx_sh : NULL;
    for (int c = 0; c < p->dv; c++) out[c] += w * (vs ? g_table[vrow[c]] * e8m0_value(vs[c]) : g_table[vrow[c]]);
  }
  for (int c = 0; c < p->dv; c++) out[c] = dv * out[c] / l;
  *lse = m + log(l);
}

/* Computes n requested rows (rb[r], rh[r], ri[r]) with optional key ranges [klo, khi)
 * (either pointer may be NULL: no restriction). out: [n, dv] fp64; lse: [n] fp64.
 * Returns 0, or -1 on an argument error. */
int fa8_oracle_attention(const fa8_oracle_params* p, int64_t n, const int32_t* rb, const int32_t* rh,
                         const int32_t* ri, const int64_t* klo, const int64_t* khi, double* out,
                         double* lse, int32_t num_threads) {
  if (!p || p->heads_kv <= 0 || p->heads_q % p->heads_kv != 0 || p->d > 512 || p->d <= 0 || p->dv <= 0)
    return -1;
  if (p->block_table && p->page_size <= 0) return -1;
  if (p->block_table && (p->q_mx || p->k_mx || p->v_mx)) return -1;
  if ((p->q_mx && !p->qmx_base) || (p->k_mx && !p->kmx_base) || (p->v_mx && !p->vmx_base)) return -1;
  build_table();
  int64_t maxk = 1;
  for (int b = 0; b < p->batch; b++)
    if (p->seqlen_k[b] > maxk) maxk = p->seqlen_k[b];
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads > 0 ? num_threads : 1)
  for (int64_t r = 0; r < n; r++) {
    double* scores = (double*)malloc(sizeof(double) * (size_t)maxk);
    if (!scores) {
#pragma omp atomic write
      err = 1;
      continue;
    }
    int64_t lo = klo ? klo[r] : 0;
    int64_t hi = khi ? khi[r] : INT64_MAX;
    one_row(p, rb[r], rh[r], ri[r], lo, hi, scores, out + r * p->dv, lse + r);
    free(scores);
  }
  return err ? -1 : 0;
}
