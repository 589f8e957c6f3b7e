/*
 * oracle.c -- plain fp64 CPU attention, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY. This is the parity oracle for the GPU library. Only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load or call it; the GPU
 * library never includes, links or calls anything here, and nothing here comes from the GPU
 * library.
 *
 * What it computes. The pages describe FlashAttention-2 as exact attention: it returns the
 * same mathematical output as standard self-attention, which materialises the full N x N
 * score matrix ("Flash Attention spiegata: una guida completa", datacamp, section
 * "Attention standard vs Flash attention"; wiki article "FlashAttention-2", section on the
 * attention problem in transformers). So this oracle is that standard definition written
 * out, with no tiling and no online softmax:
 *
 *   s_ij  = scale * <q_i, k_j>              for every visible key j of query row i
 *   m_i   = max_j s_ij,  p_ij = exp(s_ij - m_i),  l_i = sum_j p_ij   (stable softmax)
 *   O_i   = sum_j p_ij v_j / l_i,           LSE_i = m_i + ln l_i     (natural log)
 *
 * Visible keys: all j when not causal; j <= i when causal (square Q/K, top-left aligned).
 * Sliding window W >= 0 (causal only): j is visible to i iff i - W <= j <= i, the local
 * attention of the sliding-window models that "Flash Attention 2: attivarla (llama.cpp,
 * Ollama, vLLM)" names in its section on the cases where the method does not help; the page
 * gives no formula, so the window is read as W keys before the query plus the query itself.
 * Grouped-query heads: query head hq reads key/value head hq / (Hq / Hkv).
 *
 * Backward (textbook chain rule of L = sum O . dO, the "recomputation" section of the
 * datacamp page only says the method recomputes scores instead of storing them; the
 * gradients themselves are the ones of the standard definition):
 *
 *   P_ij  = p_ij / l_i,   dP_ij = <dO_i, v_j>,   D_i = sum_j P_ij dP_ij   (softmax Jacobian)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i
 *   (dK, dV of a key/value head sum over the query heads that share it)
 *
 * All arithmetic is fp64; every sum runs in index order, so results do not depend on the
 * thread count. Rows can be restricted to a sample: the forward, the row statistics and dQ
 * take query rows, dK/dV take key rows; dK/dV and dQ read the statistics m, l, D of the query
 * rows they visit.
 *
 * Layouts: q, dO [B,Hq,N,d]; k, v [B,Hkv,N,d]; all contiguous row-major fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const double *q, *k, *v, *dO;
  int64_t B, Hq, Hkv, N, d;
  int causal;
  int64_t window; /* < 0: no window */
  double scale;
  const int32_t* rows; /* query rows (forward, dq) or key rows (dkdv), per slice */
  int64_t nrows;
  const double *m, *l, *D; /* per-row statistics [B,Hq,N] */
  double *out0, *out1, *out2;
  int64_t nitems;
  int64_t next; /* work counter, atomic */
  int kind;
  int error;
} job_t;

enum { K_FWD = 0, K_STATS = 1, K_DQ = 2, K_DKDV = 3 };

static double dot(const double* a, const double* b, int64_t d) {
  double s = 0.0;
  for (int64_t c = 0; c < d; ++c) s += a[c] * b[c];
  return s;
}

/* Visible keys of query row i are first_key(i) <= j < visible_keys(i). */
static int64_t visible_keys(const job_t* J, int64_t i) { return J->causal ? i + 1 : J->N; }
static int64_t first_key(const job_t* J, int64_t i) {
  return (J->window >= 0 && i > J->window) ? i - J->window : 0;
}
/* Query rows that see key j are first_query(j) <= i < last_query(j). */
static int64_t last_query(const job_t* J, int64_t j) {
  return (J->window >= 0 && j + J->window + 1 < J->N) ? j + J->window + 1 : J->N;
}

/* Scores, stable softmax numerators and row statistics of query row i.
   On return s[j] = p_ij = exp(s_ij - m) for *j0_out <= j < nvis; *m_out, *l_out set. */
static int64_t softmax_row(const job_t* J, const double* qi, const double* Kh, int64_t i,
                           double* s, double* m_out, double* l_out, int64_t* j0_out) {
  int64_t nvis = visible_keys(J, i), j0 = first_key(J, i);
  double m = -INFINITY;
  for (int64_t j = j0; j < nvis; ++j) {
    s[j] = J->scale * dot(qi, Kh + j * J->d, J->d);
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int64_t j = j0; j < nvis; ++j) {
    s[j] = exp(s[j] - m);
    l += s[j];
  }
  *m_out = m;
  *l_out = l;
  *j0_out = j0;
  return nvis;
}

static void do_item(job_t* J, int64_t item, double* s, double* acc) {
  const int64_t N = J->N, d = J->d, group = J->Hq / J->Hkv;
  if (J->kind == K_FWD || J->kind == K_DQ) {
    int64_t slice = item / J->nrows, r = item % J->nrows; /* slice = b*Hq + hq */
    int64_t b = slice / J->Hq, hq = slice % J->Hq, g = hq / group;
    int64_t i = J->rows[slice * J->nrows + r];
    const double* qi = J->q + (slice * N + i) * d;
    const double* Kh = J->k + (b * J->Hkv + g) * N * d;
    const double* Vh = J->v + (b * J->Hkv + g) * N * d;
    double m, l;
    int64_t j0;
    int64_t nvis = softmax_row(J, qi, Kh, i, s, &m, &l, &j0);
    if (J->kind == K_FWD) {
      for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
      for (int64_t j = j0; j < nvis; ++j)
        for (int64_t c = 0; c < d; ++c) acc[c] += s[j] * Vh[j * d + c];
      double* o = J->out0 + (slice * J->nrows + r) * d;
      for (int64_t c = 0; c < d; ++c) o[c] = acc[c] / l;
      J->out1[slice * J->nrows + r] = m + log(l);
    } else {
      const double* dOi = J->dO + (slice * N + i) * d;
      double Di = J->D[slice * N + i];
      for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
      for (int64_t j = j0; j < nvis; ++j) {
        double P = s[j] / l;
        double dP = dot(dOi, Vh + j * d, d);
        double dS = P * (dP - Di);
        for (int64_t c = 0; c < d; ++c) acc[c] += dS * Kh[j * d + c];
      }
      double* dq = J->out0 + (slice * J->nrows + r) * d;
      for (int64_t c = 0; c < d; ++c) dq[c] = J->scale * acc[c];
    }
  } else if (J->kind == K_STATS) {
    int64_t slice = item / J->nrows, r = item % J->nrows;
    int64_t i = J->rows[slice * J->nrows + r];
    int64_t b = slice / J->Hq, hq = slice % J->Hq, g = hq / group;
    const double* qi = J->q + (slice * N + i) * d;
    const double* dOi = J->dO + (slice * N + i) * d;
    const double* Kh = J->k + (b * J->Hkv + g) * N * d;
    const double* Vh = J->v + (b * J->Hkv + g) * N * d;
    double m, l;
    int64_t j0;
    int64_t nvis = softmax_row(J, qi, Kh, i, s, &m, &l, &j0);
    double D = 0.0;
    for (int64_t j = j0; j < nvis; ++j) D += (s[j] / l) * dot(dOi, Vh + j * d, d);
    J->out0[item] = m;
    J->out1[item] = l;
    J->out2[item] = D;
  } else { /* K_DKDV: item = (b*Hkv + g) * nrows + r, key row j */
    int64_t kslice = item / J->nrows, r = item % J->nrows;
    int64_t b = kslice / J->Hkv, g = kslice % J->Hkv;
    int64_t j = J->rows[kslice * J->nrows + r];
    const double* kj = J->k + (kslice * N + j) * d;
    const double* vj = J->v + (kslice * N + j) * d;
    double* dk = acc;
    double* dv = acc + d;
    for (int64_t c = 0; c < 2 * d; ++c) acc[c] = 0.0;
    for (int64_t hq = g * group; hq < (g + 1) * group; ++hq) {
      int64_t slice = b * J->Hq + hq;
      int64_t i0 = J->causal ? j : 0; /* query rows that see key j */
      int64_t i1 = last_query(J, j);
      for (int64_t i = i0; i < i1; ++i) {
        const double* qi = J->q + (slice * N + i) * d;
        const double* dOi = J->dO + (slice * N + i) * d;
        double sij = J->scale * dot(qi, kj, d);
        double P = exp(sij - J->m[slice * N + i]) / J->l[slice * N + i];
        double dP = dot(dOi, vj, d);
        double dS = P * (dP - J->D[slice * N + i]);
        for (int64_t c = 0; c < d; ++c) {
          dv[c] += P * dOi[c];
          dk[c] += dS * qi[c];
        }
      }
    }
    double* odk = J->out0 + item * d;
    double* odv = J->out1 + item * d;
    for (int64_t c = 0; c < d; ++c) {
      odk[c] = J->scale * dk[c];
      odv[c] = dv[c];
    }
  }
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  double* s = (double*)malloc(sizeof(double) * (size_t)(J->N > 0 ? J->N : 1));
  double* acc = (double*)malloc(sizeof(double) * (size_t)(2 * J->d));
  if (!s || !acc) {
    __atomic_store_n(&J->error, 1, __ATOMIC_RELAXED);
    free(s);
    free(acc);
    return NULL;
  }
  for (;;) {
    int64_t it = __atomic_fetch_add(&J->next, 1, __ATOMIC_RELAXED);
    if (it >= J->nitems) break;
    do_item(J, it, s, acc);
  }
  free(s);
  free(acc);
  return NULL;
}

static int run(job_t* J, int nthreads) {
  if (J->nitems <= 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > J->nitems) nthreads = (int)J->nitems;
  J->next = 0;
  J->error = 0;
  pthread_t th[256];
  int created[256];
  for (int t = 1; t < nthreads; ++t) created[t] = pthread_create(&th[t], NULL, worker, J) == 0;
  worker(J);
  for (int t = 1; t < nthreads; ++t)
    if (created[t]) pthread_join(th[t], NULL);
  return J->error ? -2 : 0;
}

static int check_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                       int64_t window) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1) return -1;
  if (window >= 0 && !causal) return -1; /* a window is defined for causal attention only */
  if (Hq % Hkv != 0) return -1;
  return 0;
}

static int check_rows(const int32_t* rows, int64_t nslices, int64_t nrows, int64_t N) {
  if (nrows < 0 || (nrows > 0 && !rows)) return -1;
  for (int64_t t = 0; t < nslices * nrows; ++t)
    if (rows[t] < 0 || rows[t] >= N) return -1;
  return 0;
}

/* O [B,Hq,nrows,d] and LSE [B,Hq,nrows] for query rows rows[(b*Hq+hq)*nrows + r]. */
int oracle_forward(const double* q, const double* k, const double* v, int64_t B, int64_t Hq,
                   int64_t Hkv, int64_t N, int64_t d, int causal, int64_t window,
                   double scale, const int32_t* rows, int64_t nrows, double* o, double* lse, int nthreads) {
  if (check_shape(B, Hq, Hkv, N, d, causal, window) || check_rows(rows, B * Hq, nrows, N)) return -1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.N = N; J.d = d;
  J.causal = causal != 0; J.window = window < 0 ? -1 : window; J.scale = scale; J.rows = rows; J.nrows = nrows;
  J.out0 = o; J.out1 = lse; J.nitems = B * Hq * nrows; J.kind = K_FWD;
  return run(&J, nthreads);
}

/* Per-row statistics of query rows rows[(b*Hq+hq)*nrows + r]: the row max m, the softmax
   denominator l = sum_j exp(s_ij - m) and D = sum_j P_ij dP_ij, each [B,Hq,nrows]. */
int oracle_row_stats(const double* q, const double* k, const double* v, const double* dO,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                     int64_t window, double scale, const int32_t* rows, int64_t nrows, double* m,
                     double* l, double* D, int nthreads) {
  if (check_shape(B, Hq, Hkv, N, d, causal, window) || check_rows(rows, B * Hq, nrows, N)) return -1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.dO = dO; J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.N = N; J.d = d;
  J.causal = causal != 0; J.window = window < 0 ? -1 : window; J.scale = scale;
  J.rows = rows; J.nrows = nrows;
  J.out0 = m; J.out1 = l; J.out2 = D; J.nitems = B * Hq * nrows; J.kind = K_STATS;
  return run(&J, nthreads);
}

/* dQ [B,Hq,nrows,d] for query rows rows[(b*Hq+hq)*nrows + r]; needs D from oracle_row_stats. */
int oracle_backward_dq(const double* q, const double* k, const double* v, const double* dO,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                       int64_t window, double scale, const double* D, const int32_t* rows, int64_t nrows,
                       double* dq, int nthreads) {
  if (check_shape(B, Hq, Hkv, N, d, causal, window) || check_rows(rows, B * Hq, nrows, N)) return -1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.dO = dO; J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.N = N; J.d = d;
  J.causal = causal != 0; J.window = window < 0 ? -1 : window; J.scale = scale; J.D = D; J.rows = rows; J.nrows = nrows;
  J.out0 = dq; J.nitems = B * Hq * nrows; J.kind = K_DQ;
  return run(&J, nthreads);
}

/* dK, dV [B,Hkv,nrows,d] for key rows rows[(b*Hkv+g)*nrows + r]; needs m, l, D of all rows. */
int oracle_backward_dkdv(const double* q, const double* k, const double* v, const double* dO,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int causal,
                         int64_t window, double scale, const double* m, const double* l, const double* D,
                         const int32_t* rows, int64_t nrows, double* dk, double* dv,
                         int nthreads) {
  if (check_shape(B, Hq, Hkv, N, d, causal, window) || check_rows(rows, B * Hkv, nrows, N)) return -1;
  job_t J;
  memset(&J, 0, sizeof J);
  J.q = q; J.k = k; J.v = v; J.dO = dO; J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.N = N; J.d = d;
  J.causal = causal != 0; J.window = window < 0 ? -1 : window; J.scale = scale; J.m = m; J.l = l; J.D = D;
  J.rows = rows; J.nrows = nrows;
  J.out0 = dk; J.out1 = dv; J.nitems = B * Hkv * nrows; J.kind = K_DKDV;
  return run(&J, nthreads);
}

/*
 * Decode-shaped attention: Nq query rows against a cache of Nk key/value rows (Nq <= Nk when
 * causal). The causal mask is aligned to the END of the cache: query row i stands at cache
 * position Nk - Nq + i and sees keys j <= Nk - Nq + i -- the rows being decoded are the newest
 * tokens. This is the long-KV-cache inference shape of the decoding pages (FlashDecoding++ is
 * in the wiki article's literature list; the qualellm.it guide centres on local inference
 * with long contexts); they give no formula, so it is the plain definition with that
 * alignment. q, o [B,Hq,Nq,d]; k, v [B,Hkv,Nk,d]; lse [B,Hq,Nq]; natural log.
 */
int oracle_decode(const double* q, const double* k, const double* v, int64_t B, int64_t Hq,
                  int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int causal, double scale,
                  double* o, double* lse) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1 || Hq % Hkv) return -1;
  if (causal && Nq > Nk) return -1;
  const int64_t group = Hq / Hkv;
  double* s = (double*)malloc(sizeof(double) * (size_t)Nk);
  if (!s) return -2;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t hq = 0; hq < Hq; ++hq) {
      const int64_t g = hq / group;
      const double* Kh = k + (b * Hkv + g) * Nk * d;
      const double* Vh = v + (b * Hkv + g) * Nk * d;
      for (int64_t i = 0; i < Nq; ++i) {
        const double* qi = q + ((b * Hq + hq) * Nq + i) * d;
        const int64_t nvis = causal ? Nk - Nq + i + 1 : Nk;
        double m = -INFINITY;
        for (int64_t j = 0; j < nvis; ++j) {
          s[j] = scale * dot(qi, Kh + j * d, d);
          if (s[j] > m) m = s[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < nvis; ++j) {
          s[j] = exp(s[j] - m);
          l += s[j];
        }
        double* oi = o + ((b * Hq + hq) * Nq + i) * d;
        for (int64_t c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int64_t j = 0; j < nvis; ++j) acc += s[j] * Vh[j * d + c];
          oi[c] = acc / l;
        }
        lse[(b * Hq + hq) * Nq + i] = m + log(l);
      }
    }
  free(s);
  return 0;
}
