/*
 * CPU oracle for the gated delta-rule recurrence of Chunkwise-Parallel Recurrent (CPR)
 * Gated DeltaNet, in the fixed binary32 operation order of the execution contract.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may load or call this file:
 * only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py use it.
 * It shares no code, header, constant or helper with the HIP library.
 *
 * What it computes (per sequence n, value head h, state row i; every row is independent):
 *   S_t = a_t * S_{t-1} * (I - b_t k_t k_t^T) + b_t v_t k_t^T,     o_t = S_t q_t
 * The recurrence is the gated delta rule (Yang, Kautz & Hatamizadeh, "Gated Delta Networks:
 * Improving Mamba2 with Delta Rule", ICLR 2025). The IsoExec pages name CPR Gated DeltaNet
 * and state that decode resyncs the hidden state every C tokens (IsoExec, agentlenshq.com,
 * section "Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet"); they pin reductions to a
 * fixed binary tree with fp32 accumulation (same page, section on achieving parallel
 * invariance) and pin accumulation dtype and reduction decomposition per (region, case)
 * (same page, section on contract structure).
 *
 * Readings taken where the pages are silent (each one is part of the hashed contract):
 *  - row i of S, s in R^{d_k}, is updated on its own, left to right in the formula:
 *      x_e = a * s_e                         (binary32 multiply, round to nearest even)
 *      u   = dot(x, k)                       (contract dot product, below)
 *      d   = b * (v_i - u)                   (subtract, then multiply; both rounded)
 *      s_e = fmaf(d, k_e, x_e)               (one fused multiply-add per element)
 *      o_i = dot(s, q)                       (read out from the updated state)
 *  - dot(x, y) over d_k elements: 16 leaves of m = d_k/16 contiguous elements; a leaf
 *    starts with the rounded product x[l*m]*y[l*m] and adds the rest with fmaf in
 *    ascending index; the 16 leaf sums are then added pairwise in natural order:
 *    (0+1),(2+3),... then (01+23),... then (0123+4567),... then (0..7 + 8..15).
 *  - q, k, v stored as bf16 are widened to binary32 exactly; a and b are binary32.
 *  - the query/key head of value head h is h / (Hv/Hk).
 *  - a chunk-boundary state is the state after in-sequence index j with (j+1) % C == 0;
 *    a sequence of length T_n emits floor(T_n / C) of them, in order, packed over n.
 *  - decode takes the state that has absorbed pos[n] tokens and applies token pos[n];
 *    when (pos[n]+1) % C == 0 it also writes the new state as the resync checkpoint.
 *
 * Built with gcc -O2 -ffp-contract=off -fno-fast-math so that no product is fused except
 * through fmaf, and without flush-to-zero, so binary32 denormals are kept.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_LEAVES 16
#define ORACLE_MAX_D 1024

/* Storage dtype of q, k, v: 0 = binary32, 1 = bfloat16 (the high 16 bits of a binary32). */
static float load_widened(const void *base, int64_t index, int dtype) {
  if (dtype == 0) return ((const float *)base)[index];
  uint32_t bits = (uint32_t)((const uint16_t *)base)[index] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

/* The contract's dot product (see header comment). */
static float contract_dot(const float *x, const float *y, int d) {
  float leaf[ORACLE_LEAVES];
  int m = d / ORACLE_LEAVES;
  for (int l = 0; l < ORACLE_LEAVES; ++l) {
    const float *xl = x + l * m, *yl = y + l * m;
    float acc = xl[0] * yl[0];
    for (int e = 1; e < m; ++e) acc = fmaf(xl[e], yl[e], acc);
    leaf[l] = acc;
  }
  for (int width = 1; width < ORACLE_LEAVES; width *= 2)
    for (int l = 0; l < ORACLE_LEAVES; l += 2 * width) leaf[l] = leaf[l] + leaf[l + width];
  return leaf[0];
}

/* One token of the recurrence for one state row s[0..d_k): returns o_i. */
static float row_token(float *s, int dk, float a, float b, float v_i, const float *k,
                       const float *q) {
  float x[ORACLE_MAX_D];
  for (int e = 0; e < dk; ++e) x[e] = a * s[e];
  float u = contract_dot(x, k, dk);
  float diff = v_i - u;
  float delta = b * diff;
  for (int e = 0; e < dk; ++e) s[e] = fmaf(delta, k[e], x[e]);
  return contract_dot(s, q, dk);
}

typedef struct {
  int N, Hk, Hv, dk, dv, C, dtype;
  const int32_t *cu;
  const void *q, *k, *v;
  const float *a, *b, *S0;
  /* Output placement for the rows of head pair p = (n, h):
     o:     row i, in-sequence token j -> o_base[p] + j * o_tok_stride + i
     chunk: row i, boundary c          -> cs_base[p] + c * cs_stride + i * dk
     final: row i                      -> fs_base[p] + i * dk                        */
  int npairs;
  const int32_t *pair_n, *pair_h;
  float **o_base;
  int64_t o_tok_stride;
  float **cs_base;
  int64_t cs_stride;
  float **fs_base;
  /* work distribution */
  int nthreads;
} scan_job;

typedef struct {
  const scan_job *job;
  int64_t unit_begin, unit_end; /* units are (pair, row) = pair * dv + i */
} scan_slice;

static void scan_one_row(const scan_job *J, int p, int i) {
  int n = J->pair_n[p], h = J->pair_h[p];
  int group = J->Hv / J->Hk;
  int hk = h / group;
  int dk = J->dk;
  float s[ORACLE_MAX_D], kq[ORACLE_MAX_D], qq[ORACLE_MAX_D];
  for (int e = 0; e < dk; ++e)
    s[e] = J->S0 ? J->S0[(((int64_t)n * J->Hv + h) * J->dv + i) * dk + e] : 0.0f;
  int64_t bos = J->cu[n], eos = J->cu[n + 1];
  for (int64_t t = bos; t < eos; ++t) {
    int64_t j = t - bos;
    int64_t qk_off = (t * J->Hk + hk) * (int64_t)dk;
    for (int e = 0; e < dk; ++e) {
      kq[e] = load_widened(J->k, qk_off + e, J->dtype);
      qq[e] = load_widened(J->q, qk_off + e, J->dtype);
    }
    float v_i = load_widened(J->v, (t * J->Hv + h) * (int64_t)J->dv + i, J->dtype);
    float a = J->a[t * J->Hv + h], b = J->b[t * J->Hv + h];
    float o_i = row_token(s, dk, a, b, v_i, kq, qq);
    if (J->o_base && J->o_base[p]) J->o_base[p][j * J->o_tok_stride + i] = o_i;
    if (J->cs_base && J->cs_base[p] && (j + 1) % J->C == 0) {
      float *dst = J->cs_base[p] + ((j + 1) / J->C - 1) * J->cs_stride + (int64_t)i * dk;
      memcpy(dst, s, sizeof(float) * dk);
    }
  }
  if (J->fs_base && J->fs_base[p]) memcpy(J->fs_base[p] + (int64_t)i * dk, s, sizeof(float) * dk);
}

static void *scan_worker(void *arg) {
  scan_slice *S = (scan_slice *)arg;
  for (int64_t u = S->unit_begin; u < S->unit_end; ++u)
    scan_one_row(S->job, (int)(u / S->job->dv), (int)(u % S->job->dv));
  return NULL;
}

static int run_scan(const scan_job *J) {
  int64_t units = (int64_t)J->npairs * J->dv;
  int nt = J->nthreads < 1 ? 1 : J->nthreads;
  if (nt > 256) nt = 256;
  if (units < nt) nt = units > 0 ? (int)units : 1;
  pthread_t th[256];
  scan_slice sl[256];
  for (int w = 0; w < nt; ++w) {
    sl[w].job = J;
    sl[w].unit_begin = units * w / nt;
    sl[w].unit_end = units * (w + 1) / nt;
  }
  for (int w = 1; w < nt; ++w)
    if (pthread_create(&th[w], NULL, scan_worker, &sl[w]) != 0) return -2;
  scan_worker(&sl[0]);
  for (int w = 1; w < nt; ++w) pthread_join(th[w], NULL);
  return 0;
}

static int check_dims(int N, int Hk, int Hv, int dk, int dv, int C, int dtype) {
  if (N < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk != 0) return -1;
  if (dk <= 0 || dk % ORACLE_LEAVES != 0 || dk > ORACLE_MAX_D || dv <= 0 || C <= 0) return -1;
  if (dtype != 0 && dtype != 1) return -1;
  return 0;
}

/*
 * Full scan over a packed batch. Layouts (row-major):
 *   cu_seqlens [N+1]; q, k [T, Hk, dk]; v [T, Hv, dv]; a, b [T, Hv]; S0 [N, Hv, dv, dk]
 *   o [T, Hv, dv]; chunk_states [sum_n floor(T_n/C), Hv, dv, dk]; final_state [N, Hv, dv, dk]
 * S0, o, chunk_states and final_state may each be NULL. Returns 0, or < 0 on bad sizes.
 */
int oracle_scan(int N, int Hk, int Hv, int dk, int dv, int C, int dtype, const int32_t *cu_seqlens,
                const void *q, const void *k, const void *v, const float *a, const float *b,
                const float *S0, float *o, float *chunk_states, float *final_state, int nthreads) {
  if (check_dims(N, Hk, Hv, dk, dv, C, dtype)) return -1;
  int npairs = N * Hv;
  int32_t *pn = malloc(sizeof(int32_t) * (npairs + 1)), *ph = malloc(sizeof(int32_t) * (npairs + 1));
  float **ob = calloc(npairs + 1, sizeof(float *)), **cb = calloc(npairs + 1, sizeof(float *));
  float **fb = calloc(npairs + 1, sizeof(float *));
  if (!pn || !ph || !ob || !cb || !fb) return -3;
  int64_t chunk_before = 0;
  for (int n = 0; n < N; ++n) {
    int64_t Tn = (int64_t)cu_seqlens[n + 1] - cu_seqlens[n];
    for (int h = 0; h < Hv; ++h) {
      int p = n * Hv + h;
      pn[p] = n;
      ph[p] = h;
      if (o) ob[p] = o + ((int64_t)cu_seqlens[n] * Hv + h) * dv;
      if (chunk_states) cb[p] = chunk_states + (chunk_before * Hv + h) * (int64_t)dv * dk;
      if (final_state) fb[p] = final_state + ((int64_t)n * Hv + h) * dv * dk;
    }
    chunk_before += Tn / C;
  }
  scan_job J = {N, Hk, Hv, dk, dv, C, dtype, cu_seqlens, q, k, v, a, b, S0,
                npairs, pn, ph, ob, (int64_t)Hv * dv, cb, (int64_t)Hv * dv * dk, fb, nthreads};
  int rc = run_scan(&J);
  free(pn); free(ph); free(ob); free(cb); free(fb);
  return rc;
}

/*
 * Scan restricted to a list of (n, h) pairs, for sampled comparisons at large sizes.
 * Outputs are compact, one block per listed pair, in list order:
 *   o_sel      concatenation of [T_n, dv] blocks
 *   chunk_sel  concatenation of [floor(T_n/C), dv, dk] blocks
 *   final_sel  [npairs, dv, dk]
 * Any of the three may be NULL.
 */
int oracle_scan_pairs(int N, int Hk, int Hv, int dk, int dv, int C, int dtype,
                      const int32_t *cu_seqlens, const void *q, const void *k, const void *v,
                      const float *a, const float *b, const float *S0, int npairs,
                      const int32_t *pair_n, const int32_t *pair_h, float *o_sel,
                      float *chunk_sel, float *final_sel, int nthreads) {
  if (check_dims(N, Hk, Hv, dk, dv, C, dtype) || npairs < 0) return -1;
  for (int p = 0; p < npairs; ++p)
    if (pair_n[p] < 0 || pair_n[p] >= N || pair_h[p] < 0 || pair_h[p] >= Hv) return -1;
  float **ob = calloc(npairs + 1, sizeof(float *)), **cb = calloc(npairs + 1, sizeof(float *));
  float **fb = calloc(npairs + 1, sizeof(float *));
  if (!ob || !cb || !fb) return -3;
  int64_t o_at = 0, c_at = 0;
  for (int p = 0; p < npairs; ++p) {
    int n = pair_n[p];
    int64_t Tn = (int64_t)cu_seqlens[n + 1] - cu_seqlens[n];
    if (o_sel) ob[p] = o_sel + o_at * dv;
    if (chunk_sel) cb[p] = chunk_sel + c_at * (int64_t)dv * dk;
    if (final_sel) fb[p] = final_sel + (int64_t)p * dv * dk;
    o_at += Tn;
    c_at += Tn / C;
  }
  scan_job J = {N, Hk, Hv, dk, dv, C, dtype, cu_seqlens, q, k, v, a, b, S0,
                npairs, pair_n, pair_h, ob, (int64_t)dv, cb, (int64_t)dv * dk, fb, nthreads};
  int rc = run_scan(&J);
  free(ob); free(cb); free(fb);
  return rc;
}

/*
 * One decode step for every sequence n with pos[n] >= 0 (a negative pos marks an idle slot,
 * which is left untouched). Layouts: q, k [N, Hk, dk]; v [N, Hv, dv]; a, b [N, Hv];
 * state [N, Hv, dv, dk] in/out; o [N, Hv, dv]; resync [N, Hv, dv, dk] or NULL.
 */
int oracle_decode_step(int N, int Hk, int Hv, int dk, int dv, int C, int dtype,
                       const int32_t *pos, const void *q, const void *k, const void *v,
                       const float *a, const float *b, float *state, float *o, float *resync) {
  if (check_dims(N, Hk, Hv, dk, dv, C, dtype)) return -1;
  int group = Hv / Hk;
  float kq[ORACLE_MAX_D], qq[ORACLE_MAX_D];
  for (int n = 0; n < N; ++n) {
    if (pos[n] < 0) continue;
    for (int h = 0; h < Hv; ++h) {
      int hk = h / group;
      int64_t qk_off = ((int64_t)n * Hk + hk) * dk;
      for (int e = 0; e < dk; ++e) {
        kq[e] = load_widened(k, qk_off + e, dtype);
        qq[e] = load_widened(q, qk_off + e, dtype);
      }
      float A = a[(int64_t)n * Hv + h], B = b[(int64_t)n * Hv + h];
      for (int i = 0; i < dv; ++i) {
        float *s = state + (((int64_t)n * Hv + h) * dv + i) * dk;
        float v_i = load_widened(v, ((int64_t)n * Hv + h) * dv + i, dtype);
        o[((int64_t)n * Hv + h) * dv + i] = row_token(s, dk, A, B, v_i, kq, qq);
        if (resync && ((int64_t)pos[n] + 1) % C == 0)
          memcpy(resync + (((int64_t)n * Hv + h) * dv + i) * dk, s, sizeof(float) * dk);
      }
    }
  }
  return 0;
}

/* The contract dot product on its own, exposed so that tests can pin the reduction order. */
float oracle_dot(const float *x, const float *y, int d) { return contract_dot(x, y, d); }
