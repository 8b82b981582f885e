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

/* ========================================================================================
 * Backward of the recurrence (gradients of a loss L given dL/do and dL/dS_final).
 *
 * The pages give no backward; this is the exact derivative of the forward above, taken in
 * this reading's fixed binary32 order. Per row i of (n, h), with sh = dL/ds (d_k values,
 * starting from dS_final's row or +0), for t = T_n-1 down to 0, g = do[t,h,i], and the
 * forward quantities of token t (x = a*s_{t-1}, u, diff = v_i - u, delta = b*diff, s_t)
 * recomputed in the forward order:
 *   sh_e  = fmaf(g, q_e, sh_e)                    dL/ds_t including o_t = s_t . q
 *   pq_e  = g * s_t,e                             row's share of dq_t
 *   dh    = dot(sh, k)                            dL/d delta (contract dot)
 *   dv_i  = b * dh                                dL/dv_i
 *   pb    = dh * diff                             row's share of db_t
 *   uh    = -dv_i                                 dL/du
 *   xh_e  = fmaf(uh, k_e, sh_e)                   dL/dx
 *   pk_e  = fmaf(uh, x_e, delta * sh_e)           row's share of dk_t
 *   pa    = dot(xh, s_{t-1})                      row's share of da_t (contract dot)
 *   sh_e  = a * xh_e                              dL/ds_{t-1}
 * dS0 row = sh after t = 0. The shares are summed over the d_v rows of (n, h) by a pairwise
 * tree in natural row order in which a pair whose second half holds no row passes the first
 * half through unchanged; dq and dk then sum the value heads of a q/k group left to right.
 * ======================================================================================== */

static void row_forward(float *s, int dk, float a, float b, float v_i, const float *k,
                        float *x_out, float *u_out, float *diff_out, float *delta_out) {
  for (int e = 0; e < dk; ++e) x_out[e] = a * s[e];
  float u = contract_dot(x_out, k, dk);
  float diff = v_i - u;
  float delta = b * diff;
  for (int e = 0; e < dk; ++e) s[e] = fmaf(delta, k[e], x_out[e]);
  *u_out = u;
  *diff_out = diff;
  *delta_out = delta;
}

/* pairwise tree over `count` present rows, stride `stride` between row values */
static float row_tree(float *vals, int count, int stride) {
  int P = 1;
  while (P < count) P *= 2;
  for (int w = 1; w < P; w *= 2)
    for (int j = 0; j + w < count; j += 2 * w) vals[(int64_t)j * stride] =
        vals[(int64_t)j * stride] + vals[(int64_t)(j + w) * stride];
  return vals[0];
}

typedef struct {
  int N, Hk, Hv, dk, dv, C, dtype;
  const int32_t *cu;
  const void *q, *k, *v;
  const float *a, *b, *S0, *dO, *dSf;
  float *dq, *dkk, *dvv, *da, *db, *dS0;
  int ngroups; /* (n, hk) pairs */
} bwd_job;

typedef struct {
  const bwd_job *job;
  int begin, end;
  int rc;
} bwd_slice;

static void backward_group(const bwd_job *J, int grp) {
  const int n = grp / J->Hk, hk = grp % J->Hk;
  const int G = J->Hv / J->Hk, dk = J->dk, dv = J->dv, C = J->C;
  const int64_t bos = J->cu[n], Tn = (int64_t)J->cu[n + 1] - J->cu[n];
  /* per value head of the group: its dq, dk shares summed over rows, [Tn][dk] each */
  float *DQh = calloc((size_t)G * (Tn ? Tn : 1) * dk, sizeof(float));
  float *DKh = calloc((size_t)G * (Tn ? Tn : 1) * dk, sizeof(float));
  int64_t nck = Tn / C + 1; /* states at in-sequence positions 0, C, 2C, ... (start of each block) */
  float *ck = malloc(sizeof(float) * (size_t)nck * dv * dk);
  float *blk = malloc(sizeof(float) * (size_t)(C + 1) * dv * dk); /* states s_{t0-1} .. s_{t0+C-1} */
  float *sh = malloc(sizeof(float) * (size_t)dv * dk);
  float *pq = malloc(sizeof(float) * (size_t)dv * dk), *pk = malloc(sizeof(float) * (size_t)dv * dk);
  float *pa = malloc(sizeof(float) * dv), *pb = malloc(sizeof(float) * dv);
  float kq[ORACLE_MAX_D], qq[ORACLE_MAX_D], x[ORACLE_MAX_D], xh[ORACLE_MAX_D];
  if (!DQh || !DKh || !ck || !blk || !sh || !pq || !pk || !pa || !pb) goto done;
  for (int g = 0; g < G; ++g) {
    const int h = hk * G + g;
    /* forward, keeping the state at the start of every C-token block */
    float *s = blk;
    for (int i = 0; i < dv; ++i)
      for (int e = 0; e < dk; ++e)
        s[(int64_t)i * dk + e] = J->S0 ? J->S0[(((int64_t)n * J->Hv + h) * dv + i) * dk + e] : 0.0f;
    for (int64_t j = 0; j < Tn; ++j) {
      if (j % C == 0) memcpy(ck + (j / C) * dv * dk, s, sizeof(float) * dv * dk);
      const int64_t t = bos + j;
      for (int e = 0; e < dk; ++e) kq[e] = load_widened(J->k, (t * J->Hk + hk) * (int64_t)dk + e, J->dtype);
      const float A = J->a[t * J->Hv + h], B = J->b[t * J->Hv + h];
      for (int i = 0; i < dv; ++i) {
        float u, diff, delta;
        const float v_i = load_widened(J->v, (t * J->Hv + h) * (int64_t)dv + i, J->dtype);
        row_forward(s + (int64_t)i * dk, dk, A, B, v_i, kq, x, &u, &diff, &delta);
      }
    }
    /* backward, block by block from the end, recomputing each block's states */
    for (int i = 0; i < dv; ++i)
      for (int e = 0; e < dk; ++e)
        sh[(int64_t)i * dk + e] = J->dSf ? J->dSf[(((int64_t)n * J->Hv + h) * dv + i) * dk + e] : 0.0f;
    for (int64_t blk0 = (Tn - 1) / C * C; Tn > 0 && blk0 >= 0; blk0 -= C) {
      const int64_t len = Tn - blk0 < C ? Tn - blk0 : C;
      memcpy(blk, ck + (blk0 / C) * dv * dk, sizeof(float) * dv * dk);
      for (int64_t j = 0; j < len; ++j) {
        const int64_t t = bos + blk0 + j;
        memcpy(blk + (j + 1) * dv * dk, blk + j * dv * dk, sizeof(float) * dv * dk);
        for (int e = 0; e < dk; ++e) kq[e] = load_widened(J->k, (t * J->Hk + hk) * (int64_t)dk + e, J->dtype);
        const float A = J->a[t * J->Hv + h], B = J->b[t * J->Hv + h];
        for (int i = 0; i < dv; ++i) {
          float u, diff, delta;
          const float v_i = load_widened(J->v, (t * J->Hv + h) * (int64_t)dv + i, J->dtype);
          row_forward(blk + (j + 1) * dv * dk + (int64_t)i * dk, dk, A, B, v_i, kq, x, &u, &diff, &delta);
        }
      }
      for (int64_t j = len - 1; j >= 0; --j) {
        const int64_t t = bos + blk0 + j;
        for (int e = 0; e < dk; ++e) {
          kq[e] = load_widened(J->k, (t * J->Hk + hk) * (int64_t)dk + e, J->dtype);
          qq[e] = load_widened(J->q, (t * J->Hk + hk) * (int64_t)dk + e, J->dtype);
        }
        const float A = J->a[t * J->Hv + h], B = J->b[t * J->Hv + h];
        for (int i = 0; i < dv; ++i) {
          const float *s_prev = blk + j * dv * dk + (int64_t)i * dk;
          float s_cur[ORACLE_MAX_D];
          memcpy(s_cur, s_prev, sizeof(float) * dk);
          float u, diff, delta;
          const float v_i = load_widened(J->v, (t * J->Hv + h) * (int64_t)dv + i, J->dtype);
          row_forward(s_cur, dk, A, B, v_i, kq, x, &u, &diff, &delta);
          const float gg = J->dO[(t * J->Hv + h) * (int64_t)dv + i];
          float *shr = sh + (int64_t)i * dk;
          for (int e = 0; e < dk; ++e) shr[e] = fmaf(gg, qq[e], shr[e]);
          for (int e = 0; e < dk; ++e) pq[(int64_t)i * dk + e] = gg * s_cur[e];
          const float dh = contract_dot(shr, kq, dk);
          const float dvi = B * dh;
          J->dvv[(t * J->Hv + h) * (int64_t)dv + i] = dvi;
          pb[i] = dh * diff;
          const float uh = -dvi;
          for (int e = 0; e < dk; ++e) xh[e] = fmaf(uh, kq[e], shr[e]);
          for (int e = 0; e < dk; ++e) {
            const float ds = delta * shr[e];
            pk[(int64_t)i * dk + e] = fmaf(uh, x[e], ds);
          }
          pa[i] = contract_dot(xh, s_prev, dk);
          for (int e = 0; e < dk; ++e) shr[e] = A * xh[e];
        }
        J->da[t * J->Hv + h] = row_tree(pa, dv, 1);
        J->db[t * J->Hv + h] = row_tree(pb, dv, 1);
        for (int e = 0; e < dk; ++e) {
          DQh[((int64_t)g * Tn + (t - bos)) * dk + e] = row_tree(pq + e, dv, dk);
          DKh[((int64_t)g * Tn + (t - bos)) * dk + e] = row_tree(pk + e, dv, dk);
        }
      }
    }
    for (int i = 0; i < dv; ++i)
      memcpy(J->dS0 + (((int64_t)n * J->Hv + h) * dv + i) * dk, sh + (int64_t)i * dk, sizeof(float) * dk);
  }
  /* q/k group: value heads left to right */
  for (int64_t j = 0; j < Tn; ++j)
    for (int e = 0; e < dk; ++e) {
      float accq = DQh[j * dk + e], acck = DKh[j * dk + e];
      for (int g = 1; g < G; ++g) {
        accq = accq + DQh[((int64_t)g * Tn + j) * dk + e];
        acck = acck + DKh[((int64_t)g * Tn + j) * dk + e];
      }
      J->dq[((bos + j) * J->Hk + hk) * (int64_t)dk + e] = accq;
      J->dkk[((bos + j) * J->Hk + hk) * (int64_t)dk + e] = acck;
    }
done:
  free(DQh); free(DKh); free(ck); free(blk); free(sh); free(pq); free(pk); free(pa); free(pb);
}

static void *bwd_worker(void *arg) {
  bwd_slice *S = (bwd_slice *)arg;
  for (int g = S->begin; g < S->end; ++g) backward_group(S->job, g);
  return NULL;
}

/*
 * Gradients of the recurrence over a packed batch. Inputs as for oracle_scan, plus
 * dO [T, Hv, dv] and dS_final [N, Hv, dv, dk] (NULL = 0). Outputs: dq, dk [T, Hk, dk];
 * dv [T, Hv, dv]; da, db [T, Hv]; dS0 [N, Hv, dv, dk]. Threads over (sequence, q/k head).
 */
int oracle_backward(int N, int Hk, int Hv, int dk, int dv, int C, int dtype,
                    const int32_t *cu_seqlens, const void *q, const void *k, const void *v,
                    const float *a, const float *b, const float *S0, const float *dO,
                    const float *dS_final, float *dq, float *dk_out, float *dv_out, float *da,
                    float *db, float *dS0, int nthreads) {
  if (check_dims(N, Hk, Hv, dk, dv, C, dtype)) return -1;
  bwd_job J = {N, Hk, Hv, dk, dv, C, dtype, cu_seqlens, q, k, v, a, b, S0, dO, dS_final,
               dq, dk_out, dv_out, da, db, dS0, N * Hk};
  int nt = nthreads < 1 ? 1 : (nthreads > 256 ? 256 : nthreads);
  if (J.ngroups < nt) nt = J.ngroups > 0 ? J.ngroups : 1;
  pthread_t th[256];
  bwd_slice sl[256];
  for (int w = 0; w < nt; ++w) {
    sl[w].job = &J;
    sl[w].begin = (int)((int64_t)J.ngroups * w / nt);
    sl[w].end = (int)((int64_t)J.ngroups * (w + 1) / nt);
  }
  for (int w = 1; w < nt; ++w)
    if (pthread_create(&th[w], NULL, bwd_worker, &sl[w]) != 0) return -2;
  bwd_worker(&sl[0]);
  for (int w = 1; w < nt; ++w) pthread_join(th[w], NULL);
  return 0;
}

/* ========================================================================================
 * Linear region: Y = X W, every output the contract dot product above.
 *
 * The IsoExec pages make a tensor-parallel matrix product invariant by splitting its K
 * dimension into contiguous leaves, accumulating each leaf in binary32 in a fixed schedule
 * and combining the leaves in a fixed order (agentlenshq.com, section on achieving parallel
 * invariance: tensor parallelism). Reading taken: the leaves and their combination are
 * those of the contract dot, so
 *   Y[m, n] = dot(X[m, 0..K), W[0..K, n])      (16 leaves of K/16; leaf = rounded first
 *                                               product, then fmaf ascending; pairwise tree)
 * with X [M, K] and W [K, N] row-major, binary32 or bf16 (widened exactly), Y [M, N]
 * binary32. Row m of Y depends on row m of X and on W only (batch invariance).
 * ======================================================================================== */

typedef struct {
  int M, N, K;
  const float *xf; /* X widened, [M, K] */
  const void *w;
  int wdtype;
  float *y;
  int n0, n1;
} lin_job;

static void *lin_worker(void *arg) {
  const lin_job *J = (const lin_job *)arg;
  float *col = (float *)malloc((size_t)J->K * sizeof(float));
  if (!col) return (void *)1;
  for (int n = J->n0; n < J->n1; ++n) {
    for (int k = 0; k < J->K; ++k) col[k] = load_widened(J->w, (int64_t)k * J->N + n, J->wdtype);
    for (int m = 0; m < J->M; ++m)
      J->y[(int64_t)m * J->N + n] = contract_dot(J->xf + (int64_t)m * J->K, col, J->K);
  }
  free(col);
  return NULL;
}

int oracle_linear(int M, int N, int K, int xdtype, int wdtype, const void *x, const void *w,
                  float *y, int nthreads) {
  if (M < 0 || N < 0 || K < ORACLE_LEAVES || K % ORACLE_LEAVES != 0) return -1;
  if ((xdtype != 0 && xdtype != 1) || (wdtype != 0 && wdtype != 1)) return -1;
  if (M == 0 || N == 0) return 0;
  float *xf = (float *)malloc((size_t)M * K * sizeof(float));
  if (!xf) return -2;
  for (int64_t e = 0; e < (int64_t)M * K; ++e) xf[e] = load_widened(x, e, xdtype);
  int nt = nthreads < 1 ? 1 : (nthreads > 256 ? 256 : nthreads);
  if (N < nt) nt = N;
  pthread_t th[256];
  lin_job jobs[256];
  for (int t = 0; t < nt; ++t) {
    lin_job j = {M, N, K, xf, w, wdtype, y, (int)((int64_t)N * t / nt),
                 (int)((int64_t)N * (t + 1) / nt)};
    jobs[t] = j;
  }
  int rc = 0, started = 1;
  for (; started < nt; ++started)
    if (pthread_create(&th[started], NULL, lin_worker, &jobs[started]) != 0) break;
  for (int t = started; t < nt; ++t)  /* a thread that could not start: its share runs here */
    if (lin_worker(&jobs[t]) != NULL) rc = -2;
  if (lin_worker(&jobs[0]) != NULL) rc = -2;
  for (int t = 1; t < started; ++t) {
    void *ret = NULL;
    pthread_join(th[t], &ret);
    if (ret != NULL) rc = -2;
  }
  free(xf);
  return rc;
}

/* ========================================================================================
 * Two-level CPR: the IsoExec pages' literal reading of CPR, in which chunk-boundary states
 * come from a chunkwise transition and the outputs inside a chunk from the recurrence run
 * in parallel between chunks, and decode resynchronises its state every C tokens
 * (agentlenshq.com, section "Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet").
 *
 * Readings taken (per sequence n and value head h; chunk c = in-sequence tokens
 * [cC, min((c+1)C, T_n))):
 *  - transition of a full chunk: S_end = S_start A_c + B_c with
 *      A_c [d_k, d_k]: row j starts as the unit row e_j and absorbs the chunk's tokens with
 *                      v_i = +0 through the contract row update (x = a s; u = dot(x, k);
 *                      d = b (0 - u); s = fmaf(d, k, x));
 *      B_c [d_v, d_k]: row i starts at +0 and absorbs the chunk's tokens with v_i;
 *  - boundary states: S_0 = the initial state; after every full chunk
 *      S_{c+1}[i, j] = B_c[i, j] + sum_k S_c[i, k] A_c[k, j]   as fused multiply-adds in
 *      ascending k with B_c[i, j] first (the order of the binary32 matrix instructions);
 *      S_{c+1} is the chunk state;
 *  - outputs: the rows restart from S_c at every chunk start and absorb the chunk's tokens
 *    through the contract row update, o_t = dot(s_t, q_t);
 *  - final state: S after the last chunk when T_n is a multiple of C, else the restarted
 *    rows after the last (partial) chunk's last token;
 *  - decode: the running rows restart from the boundary state at every chunk start; each
 *    step writes its token to a C-slot cache; after a chunk's last token the step rebuilds
 *    A_c and B_c from the cache, sets the boundary state and the running rows to S_{c+1}
 *    and writes it as the resync checkpoint.
 * ======================================================================================== */

/* One token on a row without the readout (the transitions keep no output). */
static void row_absorb(float *s, int dk, float a, float b, float v_i, const float *key) {
  float x[ORACLE_MAX_D];
  for (int e = 0; e < dk; ++e) x[e] = a * s[e];
  float u = contract_dot(x, key, dk);
  float diff = v_i - u;
  float delta = b * diff;
  for (int e = 0; e < dk; ++e) s[e] = fmaf(delta, key[e], x[e]);
}

/* S_next[i, :] = B[i, :] + S[i, :] A, fused multiply-adds in ascending k from B. */
static void boundary_step(const float *S, const float *A, const float *B, float *S_next,
                          int dv, int dk) {
  for (int i = 0; i < dv; ++i)
    for (int j = 0; j < dk; ++j) {
      float acc = B[(int64_t)i * dk + j];
      for (int kk = 0; kk < dk; ++kk) acc = fmaf(S[(int64_t)i * dk + kk], A[(int64_t)kk * dk + j], acc);
      S_next[(int64_t)i * dk + j] = acc;
    }
}

/* A_c and B_c of the tokens given as arrays: k [n_tok][dk], v [n_tok][dv], a, b [n_tok]. */
static void chunk_transition(const float *k, const float *v, const float *a, const float *b,
                             int n_tok, int dk, int dv, float *A, float *B) {
  for (int j = 0; j < dk; ++j)
    for (int e = 0; e < dk; ++e) A[(int64_t)j * dk + e] = j == e ? 1.0f : 0.0f;
  memset(B, 0, sizeof(float) * (size_t)dv * dk);
  for (int t = 0; t < n_tok; ++t) {
    const float *kt = k + (int64_t)t * dk;
    for (int j = 0; j < dk; ++j) row_absorb(A + (int64_t)j * dk, dk, a[t], b[t], 0.0f, kt);
    for (int i = 0; i < dv; ++i)
      row_absorb(B + (int64_t)i * dk, dk, a[t], b[t], v[(int64_t)t * dv + i], kt);
  }
}

typedef struct {
  int N, Hk, Hv, dk, dv, C, dtype;
  const int32_t *cu;
  const void *q, *k, *v;
  const float *a, *b, *S0;
  float *o, *cs, *fs;
  int npairs, nthreads;
} cpr2_job;

typedef struct {
  const cpr2_job *job;
  int begin, end;
  int rc;
} cpr2_slice;

static int cpr2_pair(const cpr2_job *J, int pair) {
  const int n = pair / J->Hv, h = pair % J->Hv, hk = h / (J->Hv / J->Hk);
  const int dk = J->dk, dv = J->dv, C = J->C;
  const int64_t bos = J->cu[n], eos = J->cu[n + 1];
  int64_t cbase = 0; /* chunk states of earlier sequences */
  for (int m = 0; m < n; ++m) cbase += (J->cu[m + 1] - J->cu[m]) / C;
  const size_t st = (size_t)dv * dk;
  float *S = (float *)malloc(sizeof(float) * st), *R = (float *)malloc(sizeof(float) * st);
  float *Sn = (float *)malloc(sizeof(float) * st), *B = (float *)malloc(sizeof(float) * st);
  float *A = (float *)malloc(sizeof(float) * (size_t)dk * dk);
  float *kb = (float *)malloc(sizeof(float) * (size_t)C * dk);
  float *qb = (float *)malloc(sizeof(float) * (size_t)C * dk);
  float *vb = (float *)malloc(sizeof(float) * (size_t)C * dv);
  float ab[256], bb[256];
  if (!S || !R || !Sn || !B || !A || !kb || !qb || !vb || C > 256) {
    free(S); free(R); free(Sn); free(B); free(A); free(kb); free(qb); free(vb);
    return -2;
  }
  for (size_t e = 0; e < st; ++e)
    S[e] = J->S0 ? J->S0[((int64_t)n * J->Hv + h) * (int64_t)st + (int64_t)e] : 0.0f;
  memcpy(R, S, sizeof(float) * st);
  int64_t c = 0;
  for (int64_t t0 = bos; t0 < eos; t0 += C, ++c) {
    const int n_tok = (int)(eos - t0 < C ? eos - t0 : C);
    for (int t = 0; t < n_tok; ++t) {
      const int64_t qk_off = ((t0 + t) * J->Hk + hk) * (int64_t)dk;
      for (int e = 0; e < dk; ++e) {
        kb[(int64_t)t * dk + e] = load_widened(J->k, qk_off + e, J->dtype);
        qb[(int64_t)t * dk + e] = load_widened(J->q, qk_off + e, J->dtype);
      }
      for (int i = 0; i < dv; ++i)
        vb[(int64_t)t * dv + i] = load_widened(J->v, ((t0 + t) * J->Hv + h) * (int64_t)dv + i, J->dtype);
      ab[t] = J->a[(t0 + t) * J->Hv + h];
      bb[t] = J->b[(t0 + t) * J->Hv + h];
    }
    /* outputs: the rows restart from the boundary state S */
    memcpy(R, S, sizeof(float) * st);
    for (int t = 0; t < n_tok; ++t)
      for (int i = 0; i < dv; ++i) {
        float o_i = row_token(R + (int64_t)i * dk, dk, ab[t], bb[t], vb[(int64_t)t * dv + i],
                              kb + (int64_t)t * dk, qb + (int64_t)t * dk);
        if (J->o) J->o[((t0 + t) * J->Hv + h) * (int64_t)dv + i] = o_i;
      }
    if (n_tok == C) { /* a full chunk: the next boundary state through the transition */
      chunk_transition(kb, vb, ab, bb, C, dk, dv, A, B);
      boundary_step(S, A, B, Sn, dv, dk);
      memcpy(S, Sn, sizeof(float) * st);
      if (J->cs)
        memcpy(J->cs + ((cbase + c) * J->Hv + h) * (int64_t)st, S, sizeof(float) * st);
    }
  }
  if (J->fs) {
    const int64_t Tn = eos - bos;
    const float *fin = (Tn % C == 0) ? S : R;
    memcpy(J->fs + ((int64_t)n * J->Hv + h) * (int64_t)st, fin, sizeof(float) * st);
  }
  free(S); free(R); free(Sn); free(B); free(A); free(kb); free(qb); free(vb);
  return 0;
}

static void *cpr2_worker(void *arg) {
  cpr2_slice *sl = (cpr2_slice *)arg;
  for (int p = sl->begin; p < sl->end; ++p)
    if (cpr2_pair(sl->job, p) != 0) sl->rc = -2;
  return NULL;
}

int oracle_cpr2_scan(int N, int Hk, int Hv, int dk, int dv, int C, int dtype,
                     const int32_t *cu_seqlens, const void *q, const void *k, const void *v,
                     const float *a, const float *b, const float *S0, float *o,
                     float *chunk_states, float *final_state, int nthreads) {
  if (check_dims(N, Hk, Hv, dk, dv, C, dtype) || C > 256) return -1;
  cpr2_job J = {N, Hk, Hv, dk, dv, C, dtype, cu_seqlens, q, k, v, a, b, S0,
                o, chunk_states, final_state, N * Hv, nthreads};
  int nt = nthreads < 1 ? 1 : (nthreads > 256 ? 256 : nthreads);
  if (J.npairs < nt) nt = J.npairs > 0 ? J.npairs : 1;
  pthread_t th[256];
  cpr2_slice sl[256];
  for (int w = 0; w < nt; ++w) {
    sl[w].job = &J;
    sl[w].begin = (int)((int64_t)J.npairs * w / nt);
    sl[w].end = (int)((int64_t)J.npairs * (w + 1) / nt);
    sl[w].rc = 0;
  }
  int started = 1;
  for (; started < nt; ++started)
    if (pthread_create(&th[started], NULL, cpr2_worker, &sl[started]) != 0) break;
  for (int w = started; w < nt; ++w) cpr2_worker(&sl[w]);
  cpr2_worker(&sl[0]);
  for (int w = 1; w < started; ++w) pthread_join(th[w], NULL);
  for (int w = 0; w < nt; ++w)
    if (sl[w].rc) return sl[w].rc;
  return 0;
}

/* One decode step of the two-level reading for N sequences (pos[n] < 0: idle slot).
 * state: running rows [N, Hv, dv, dk]; boundary: S_c [N, Hv, dv, dk]; the cache holds the
 * current chunk's tokens, widened: ck [N, C, Hk, dk], cv [N, C, Hv, dv], ca, cb [N, C, Hv]. */
int oracle_cpr2_decode_step(int N, int Hk, int Hv, int dk, int dv, int C, int dtype,
                            const int32_t *pos, const void *q, const void *k, const void *v,
                            const float *a, const float *b, float *state, float *boundary,
                            float *ck, float *cv, float *ca, float *cb, float *o,
                            float *resync) {
  if (check_dims(N, Hk, Hv, dk, dv, C, dtype) || C > 256) return -1;
  const size_t st = (size_t)dv * dk;
  float *A = (float *)malloc(sizeof(float) * (size_t)dk * dk);
  float *B = (float *)malloc(sizeof(float) * st), *Sn = (float *)malloc(sizeof(float) * st);
  float *kb = (float *)malloc(sizeof(float) * (size_t)C * dk);
  float *vb = (float *)malloc(sizeof(float) * (size_t)C * dv);
  float ab[256], bb[256], kq[ORACLE_MAX_D], qq[ORACLE_MAX_D];
  if (!A || !B || !Sn || !kb || !vb) {
    free(A); free(B); free(Sn); free(kb); free(vb);
    return -2;
  }
  const int group = Hv / Hk;
  for (int n = 0; n < N; ++n) {
    if (pos[n] < 0) continue;
    const int slot = pos[n] % C;
    for (int hk = 0; hk < Hk; ++hk)
      for (int e = 0; e < dk; ++e)
        ck[(((int64_t)n * C + slot) * Hk + hk) * dk + e] =
            load_widened(k, ((int64_t)n * Hk + hk) * dk + e, dtype);
    for (int h = 0; h < Hv; ++h) {
      for (int i = 0; i < dv; ++i)
        cv[(((int64_t)n * C + slot) * Hv + h) * dv + i] =
            load_widened(v, ((int64_t)n * Hv + h) * dv + i, dtype);
      ca[((int64_t)n * C + slot) * Hv + h] = a[(int64_t)n * Hv + h];
      cb[((int64_t)n * C + slot) * Hv + h] = b[(int64_t)n * Hv + h];
    }
    for (int h = 0; h < Hv; ++h) {
      const int hk = h / group;
      for (int e = 0; e < dk; ++e) {
        kq[e] = load_widened(k, ((int64_t)n * Hk + hk) * dk + e, dtype);
        qq[e] = load_widened(q, ((int64_t)n * Hk + hk) * dk + e, dtype);
      }
      float *R = state + ((int64_t)n * Hv + h) * (int64_t)st;
      const float an = a[(int64_t)n * Hv + h], bn = b[(int64_t)n * Hv + h];
      for (int i = 0; i < dv; ++i)
        o[((int64_t)n * Hv + h) * dv + i] =
            row_token(R + (int64_t)i * dk, dk, an, bn,
                      load_widened(v, ((int64_t)n * Hv + h) * dv + i, dtype), kq, qq);
      if ((pos[n] + 1) % C == 0) { /* the chunk is complete: resynchronise */
        for (int t = 0; t < C; ++t) {
          for (int e = 0; e < dk; ++e)
            kb[(int64_t)t * dk + e] = ck[(((int64_t)n * C + t) * Hk + hk) * dk + e];
          for (int i = 0; i < dv; ++i)
            vb[(int64_t)t * dv + i] = cv[(((int64_t)n * C + t) * Hv + h) * dv + i];
          ab[t] = ca[((int64_t)n * C + t) * Hv + h];
          bb[t] = cb[((int64_t)n * C + t) * Hv + h];
        }
        chunk_transition(kb, vb, ab, bb, C, dk, dv, A, B);
        float *S = boundary + ((int64_t)n * Hv + h) * (int64_t)st;
        boundary_step(S, A, B, Sn, dv, dk);
        memcpy(S, Sn, sizeof(float) * st);
        memcpy(R, Sn, sizeof(float) * st);
        if (resync) memcpy(resync + ((int64_t)n * Hv + h) * (int64_t)st, Sn, sizeof(float) * st);
      }
    }
  }
  free(A); free(B); free(Sn); free(kb); free(vb);
  return 0;
}
