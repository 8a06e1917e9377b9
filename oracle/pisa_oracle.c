/*
 * PISA CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 implementation of what the PISA hot path computes.  Only
 * the tests, the smoke check and the benchmark's CPU-baseline leg may load it;
 * the product library never links, calls or falls back to it, and it shares no
 * code, header or constant with the HIP path.
 *
 * Source of the method: "Block Sparse Attention with Log-Linear Complexity"
 * (PISA), the hyper.ai page (a Chinese rendering of the paper; the only page
 * that gives definitions).  Sections cited below by their headings:
 *   [BSA]  块稀疏注意力   block-sparse attention, the o_t equation
 *   [PYR]  金字塔键块层级 pyramid key-block hierarchy: the level-0 equation,
 *                          the level-size ceiling equation, the Concat
 *                          equation and the mean-pooling equation
 *   [SEL]  由粗到细的Top-K选择 coarse-to-fine top-K: the initial-set
 *                          equation {1}, the expansion (union of children)
 *                          equation, the candidate bound gK, the keep-all
 *                          rule for <= K valid candidates, and the LSE block
 *                          score equation (l >= 1)
 *   [KER]  内核实现       kernel implementation: the GQA score-sum equation
 *                          (u = sum over the query heads of a KV head)
 *   [BSA-flat]            the same BSA section's description of flat
 *                          selection that scores every one of ceil(N/C)
 *                          block summaries per query
 *
 * Readings taken where the page is silent:
 *   - 0-based block indices; children of block j are {2j, 2j+1} clipped to
 *     the level size (contiguous blocks, Concat order).  Leaf j holds tokens
 *     [jC, min(jC+C, N)).
 *   - A ragged parent is the mean of its existing children's summaries (the
 *     mean-pooling equation taken literally), not the mean of its raw keys.
 *   - L is the first level with one block; with N <= C, L = 1.
 *   - scale = 1/sqrt(d) unless the caller passes another; natural log / exp.
 *   - Query head h' belongs to KV head h' / G_Q (contiguous GQA groups).
 *   - Causal rule: a block at any level is valid for query t iff its first
 *     token is <= t; raw-key LSE and attention drop keys i > t; an
 *     intermediate LSE runs over the valid children only, using their
 *     full-sequence summaries.  The pyramid is built once over all N tokens.
 *   - Ties in every top-K go to the lower block index.
 *   - Fewer than K valid blocks: all are kept; output is ascending, -1 padded.
 *   - The leaf score u^(1) of every kept leaf is reported, also when the leaf
 *     level had <= K candidates and was kept without scoring.
 *   - Flat selector score: one logit q . (leaf mean) * scale per query head,
 *     summed over the GQA group.
 *
 * Everything is computed in double precision from the exact input values
 * (bf16 inputs are widened bit-exactly).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

typedef struct {
  int32_t B, N, Hq, Hkv, D; /* q [B][Hq][N][D]; k, v [B][Hkv][N][D]         */
  int32_t C, K;             /* leaf size, per-level budget                  */
  int32_t causal;           /* 0 or 1                                       */
  int32_t dtype;            /* ORACLE_F32 or ORACLE_BF16                    */
  int32_t q_sampled;        /* 0: q is [B][Hq][N][D] indexed by position t;
                               1: q is [B][Hq][nt][D] indexed by sample s   */
  double scale;             /* logit scale (the caller passes 1/sqrt(D))    */
} oracle_problem;

/* counters[] layout (int64), filled by oracle_select:                       */
enum {
  CNT_QUERIES = 0,       /* (b, h, t) routed                                 */
  CNT_SCORED_BLOCKS = 1, /* candidates scored at levels >= 2                 */
  CNT_CHILD_DOTS = 2,    /* child summaries dotted (per KV group, x G_Q for head-dots) */
  CNT_LEAF_PAIRS = 3,    /* (query, candidate leaf) pairs scored at level 1  */
  CNT_LEAF_KEY_DOTS = 4, /* raw keys dotted at level 1 (x G_Q for head-dots) */
  CNT_MAX_CAND = 5,      /* largest candidate set seen after filtering       */
  CNT_MAX_KEPT = 6,      /* largest kept set                                 */
  CNT_SCORED_LEVELS = 7, /* levels (>= 2) where scoring happened, summed     */
  CNT_LEVEL_BASE = 16,   /* [16 + l]: candidates after filtering at level l  */
  CNT_LEN = 80
};

static double widen(const void* base, int dtype, int64_t i) {
  if (dtype == ORACLE_BF16) {
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
  }
  return (double)((const float*)base)[i];
}

/* ---- [PYR] level sizes: M_1 = ceil(N/C), M_{l+1} = ceil(M_l / 2) ------- */
int64_t oracle_level_rows(int64_t n, int32_t C, int32_t level) {
  int64_t m = (n + C - 1) / C;
  for (int32_t l = 1; l < level; ++l) m = (m + 1) / 2;
  return m;
}

int32_t oracle_levels(int64_t n, int32_t C) {
  int64_t m = (n + C - 1) / C;
  int32_t L = 1;
  while (m > 1) {
    m = (m + 1) / 2;
    ++L;
  }
  return L;
}

/* Rows of all levels 1..L stacked, level 1 first. */
int64_t oracle_pyramid_rows(int64_t n, int32_t C) {
  int32_t L = oracle_levels(n, C);
  int64_t r = 0;
  for (int32_t l = 1; l <= L; ++l) r += oracle_level_rows(n, C, l);
  return r;
}

/* First token of block j at level l (l >= 1): j * C * 2^(l-1). */
static int64_t block_start(int64_t j, int32_t C, int32_t l) {
  return j * (int64_t)C * ((int64_t)1 << (l - 1));
}

/* ---- [PYR] mean-pooled summaries for one (b, h) head ------------------ *
 * k: [n][D] rows (row stride `row_stride` elements), pyr: levels stacked.
 * Level 1: mean of the raw keys of each leaf.  Level l+1: mean of the
 * existing children's summaries.                                          */
void oracle_pyramid(const void* k, int32_t dtype, int64_t row_stride, int64_t n, int32_t D,
                    int32_t C, double* pyr) {
  int32_t L = oracle_levels(n, C);
  int64_t M1 = oracle_level_rows(n, C, 1);
  for (int64_t j = 0; j < M1; ++j) {
    int64_t lo = j * C, hi = lo + C < n ? lo + C : n;
    for (int32_t d = 0; d < D; ++d) {
      double s = 0.0;
      for (int64_t i = lo; i < hi; ++i) s += widen(k, dtype, i * row_stride + d);
      pyr[j * D + d] = s / (double)(hi - lo);
    }
  }
  double* child = pyr;
  int64_t mc = M1;
  for (int32_t l = 2; l <= L; ++l) {
    double* par = child + mc * D;
    int64_t mp = (mc + 1) / 2;
    for (int64_t j = 0; j < mp; ++j) {
      int64_t nch = (2 * j + 1 < mc) ? 2 : 1;
      for (int32_t d = 0; d < D; ++d) {
        double s = 0.0;
        for (int64_t r = 2 * j; r < 2 * j + nch; ++r) s += child[r * D + d];
        par[j * D + d] = s / (double)nch;
      }
    }
    child = par;
    mc = mp;
  }
}

/* Element offset of query head hq at position t (sample s of nt). */
static int64_t query_offset(const oracle_problem* p, int32_t b, int32_t hq, int64_t t, int64_t s,
                            int64_t nt) {
  if (p->q_sampled) return (((int64_t)b * p->Hq + hq) * nt + s) * p->D;
  return (((int64_t)b * p->Hq + hq) * p->N + t) * p->D;
}

/* log-sum-exp; an empty set (or all -inf) gives -inf. */
static double lse(const double* x, int64_t n) {
  double m = -INFINITY;
  for (int64_t i = 0; i < n; ++i)
    if (x[i] > m) m = x[i];
  if (m == -INFINITY) return -INFINITY;
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += exp(x[i] - m);
  return m + log(s);
}

typedef struct {
  double u;
  int64_t j;
} scored;

/* Order of every top-K: score descending, then block index ascending. */
static int by_score_then_index(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->u > y->u) return -1;
  if (x->u < y->u) return 1;
  return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int by_index(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  return (x->j < y->j) ? -1 : (x->j > y->j);
}

static double dot_q(const void* q, int32_t dtype, int64_t qoff, const double* row, int32_t D) {
  double s = 0.0;
  for (int32_t d = 0; d < D; ++d) s += widen(q, dtype, qoff + d) * row[d];
  return s;
}

static double dot_qk(const void* q, const void* k, int32_t dtype, int64_t qoff, int64_t koff,
                     int32_t D) {
  double s = 0.0;
  for (int32_t d = 0; d < D; ++d) s += widen(q, dtype, qoff + d) * widen(k, dtype, koff + d);
  return s;
}

/* [SEL] LSE block score of block j at level l >= 2 for one query head:
 * log-sum-exp over the valid children r of q . summary_r * scale. */
static double score_intermediate(const oracle_problem* p, const void* q, int64_t qoff,
                                 const double* child_level, int64_t m_child, int32_t l, int64_t j,
                                 int64_t t, double* buf) {
  int64_t n = 0;
  for (int64_t r = 2 * j; r <= 2 * j + 1 && r < m_child; ++r) {
    if (p->causal && block_start(r, p->C, l - 1) > t) continue;
    buf[n++] = dot_q(q, p->dtype, qoff, child_level + r * p->D, p->D) * p->scale;
  }
  return lse(buf, n);
}

/* [SEL] at l = 1 the children are the raw keys: the exact raw-key LSE. */
static double score_leaf(const oracle_problem* p, const void* q, const void* k, int64_t qoff,
                         int64_t kbase, int64_t j, int64_t t, double* buf, int64_t* nkeys) {
  int64_t lo = j * p->C, hi = lo + p->C < p->N ? lo + p->C : p->N;
  int64_t n = 0;
  for (int64_t i = lo; i < hi; ++i) {
    if (p->causal && i > t) break;
    buf[n++] = dot_qk(q, k, p->dtype, qoff, kbase + i * p->D, p->D) * p->scale;
  }
  *nkeys = n;
  return lse(buf, n);
}

/* ---- routing for one (b, h, t) ----------------------------------------- */
static void route_one(const oracle_problem* p, const void* q, const void* k, const double* pyr,
                      const int64_t* level_off, int32_t L, int32_t b, int32_t h, int64_t t,
                      int64_t s, int64_t nt, int32_t* idx_out, double* score_out, double* gap_out, int64_t* cnt) {
  const int32_t G = p->Hq / p->Hkv;
  const int32_t K = p->K;
  const int64_t N = p->N;
  const int32_t D = p->D;
  const int64_t kbase = ((int64_t)b * p->Hkv + h) * N * D;
  int64_t cap = 4 * (int64_t)K + 4;
  scored* A = (scored*)malloc(sizeof(scored) * cap);
  scored* next = (scored*)malloc(sizeof(scored) * cap);
  double* buf = (double*)malloc(sizeof(double) * (p->C > 2 ? p->C : 2));
  int64_t nA = 1;
  double min_gap = INFINITY;
  A[0].j = 0; /* [SEL] the coarsest level starts from its single block */
  A[0].u = 0.0;
  int64_t nI = 0;

  for (int32_t l = L; l >= 1; --l) {
    const int64_t ml = oracle_level_rows(N, p->C, l);
    /* drop invalid candidates (causal rule; every index is < M_l) */
    int64_t nv = 0;
    for (int64_t a = 0; a < nA; ++a) {
      if (A[a].j >= ml) continue;
      if (p->causal && block_start(A[a].j, p->C, l) > t) continue;
      A[nv++] = A[a];
    }
    nA = nv;
    if (nA > cnt[CNT_MAX_CAND]) cnt[CNT_MAX_CAND] = nA;
    if (CNT_LEVEL_BASE + l < CNT_LEN) cnt[CNT_LEVEL_BASE + l] += nA;

    int must_score = (nA > K);
    if (l == 1 || must_score) {
      /* [SEL] LSE score per query head, [KER] summed over the GQA group */
      for (int64_t a = 0; a < nA; ++a) {
        double u = 0.0;
        for (int32_t g = 0; g < G; ++g) {
          int32_t hq = h * G + g;
          int64_t qoff = query_offset(p, b, hq, t, s, nt);
          if (l == 1) {
            int64_t nk = 0;
            u += score_leaf(p, q, k, qoff, kbase, A[a].j, t, buf, &nk);
            if (must_score) cnt[CNT_LEAF_KEY_DOTS] += (g == 0) ? nk : 0;
          } else {
            const double* child_level = pyr + level_off[l - 1] * D;
            u += score_intermediate(p, q, qoff, child_level, oracle_level_rows(N, p->C, l - 1),
                                    l, A[a].j, t, buf);
          }
        }
        A[a].u = u;
        if (must_score) {
          if (l == 1) {
            cnt[CNT_LEAF_PAIRS] += 1;
          } else {
            cnt[CNT_SCORED_BLOCKS] += 1;
            int64_t m_child = oracle_level_rows(N, p->C, l - 1);
            for (int64_t r = 2 * A[a].j; r <= 2 * A[a].j + 1 && r < m_child; ++r)
              if (!(p->causal && block_start(r, p->C, l - 1) > t)) cnt[CNT_CHILD_DOTS] += 1;
          }
        }
      }
    }
    if (must_score) {
      qsort(A, (size_t)nA, sizeof(scored), by_score_then_index);
      double gap = A[K - 1].u - A[K].u;
      if (gap < min_gap) min_gap = gap;
      if (l >= 2) cnt[CNT_SCORED_LEVELS] += 1;
      nI = K;
    } else {
      nI = nA; /* [SEL] <= K valid candidates are all kept */
    }
    if (nI > cnt[CNT_MAX_KEPT]) cnt[CNT_MAX_KEPT] = nI;

    if (l > 1) {
      /* [SEL] expansion: union of the kept blocks' children */
      const int64_t m_child = oracle_level_rows(N, p->C, l - 1);
      int64_t nn = 0;
      for (int64_t a = 0; a < nI; ++a)
        for (int64_t r = 2 * A[a].j; r <= 2 * A[a].j + 1 && r < m_child; ++r) {
          next[nn].j = r;
          next[nn].u = 0.0;
          ++nn;
        }
      scored* tmp = A;
      A = next;
      next = tmp;
      nA = nn;
    }
  }
  /* output the leaf set ascending, -1 padded */
  qsort(A, (size_t)nI, sizeof(scored), by_index);
  for (int32_t s = 0; s < K; ++s) {
    idx_out[s] = (s < nI) ? (int32_t)A[s].j : -1;
    score_out[s] = (s < nI) ? A[s].u : -INFINITY;
  }
  *gap_out = min_gap;
  cnt[CNT_QUERIES] += 1;
  free(A);
  free(next);
  free(buf);
}

static void fill_level_offsets(int64_t n, int32_t C, int32_t L, int64_t* off) {
  off[1] = 0;
  for (int32_t l = 1; l < L; ++l) off[l + 1] = off[l] + oracle_level_rows(n, C, l);
}

/* ---- public: PISA selection for the query positions ts[0..nt) --------- *
 * idx, score: [B][Hkv][nt][K];  min_gap: [B][Hkv][nt] (smallest gap between
 * the K-th and (K+1)-th scores over the levels that were scored; +inf if
 * none);  counters: CNT_LEN int64 (accumulated).  Returns 0 on success.    */
int oracle_select(const oracle_problem* p, const void* q, const void* k, const int32_t* ts,
                  int64_t nt, int32_t* idx, double* score, double* min_gap, int64_t* counters) {
  if (p->Hq % p->Hkv != 0 || p->C < 1 || p->K < 1 || p->N < 1) return 1;
  const int32_t L = oracle_levels(p->N, p->C);
  int64_t level_off[66];
  fill_level_offsets(p->N, p->C, L, level_off);
  const int64_t rows = oracle_pyramid_rows(p->N, p->C);
  double* pyr = (double*)malloc(sizeof(double) * rows * p->D);
  if (!pyr) return 2;
  for (int32_t b = 0; b < p->B; ++b)
    for (int32_t h = 0; h < p->Hkv; ++h) {
      const int64_t kbase = ((int64_t)b * p->Hkv + h) * (int64_t)p->N * p->D;
      oracle_pyramid((const char*)k + kbase * (p->dtype == ORACLE_BF16 ? 2 : 4), p->dtype, p->D,
                     p->N, p->D, p->C, pyr);
      int64_t local[CNT_LEN];
      memset(local, 0, sizeof local);
#pragma omp parallel
      {
        int64_t mine[CNT_LEN];
        memset(mine, 0, sizeof mine);
#pragma omp for schedule(dynamic, 16)
        for (int64_t s = 0; s < nt; ++s) {
          int64_t o = ((int64_t)b * p->Hkv + h) * nt + s;
          route_one(p, q, k, pyr, level_off, L, b, h, ts[s], s, nt, idx + o * p->K,
                    score + o * p->K, min_gap + o, mine);
        }
#pragma omp critical
        for (int c = 0; c < CNT_LEN; ++c) {
          if (c == CNT_MAX_CAND || c == CNT_MAX_KEPT)
            local[c] = mine[c] > local[c] ? mine[c] : local[c];
          else
            local[c] += mine[c];
        }
      }
      for (int c = 0; c < CNT_LEN; ++c) {
        if (c == CNT_MAX_CAND || c == CNT_MAX_KEPT)
          counters[c] = local[c] > counters[c] ? local[c] : counters[c];
        else
          counters[c] += local[c];
      }
    }
  free(pyr);
  return 0;
}

/* ---- public: [BSA] softmax attention over the keys of the given leaves -- *
 * idx: [B][Hkv][nt][K] leaf indices (-1 = none); o: [B][Hq][nt][D];
 * lse: [B][Hq][nt].  Key i of leaf j attends when i < N and (not causal or
 * i <= t).  A query with no attended key gets o = 0, lse = -inf.           */
int oracle_attention(const oracle_problem* p, const void* q, const void* k, const void* v,
                     const int32_t* ts, int64_t nt, const int32_t* idx, double* o, double* lse_out) {
  if (p->Hq % p->Hkv != 0) return 1;
  const int32_t G = p->Hq / p->Hkv;
  const int64_t N = p->N;
  const int32_t D = p->D;
  const int64_t total = (int64_t)p->B * p->Hq * nt;
#pragma omp parallel
  {
    int64_t cap = (int64_t)p->K * p->C;
    double* z = (double*)malloc(sizeof(double) * (cap > 0 ? cap : 1));
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (cap > 0 ? cap : 1));
    double* acc = (double*)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 16)
    for (int64_t w = 0; w < total; ++w) {
      int64_t s = w % nt;
      int32_t hq = (int32_t)((w / nt) % p->Hq);
      int32_t b = (int32_t)(w / nt / p->Hq);
      int32_t h = hq / G;
      int64_t t = ts[s];
      const int32_t* sel = idx + (((int64_t)b * p->Hkv + h) * nt + s) * p->K;
      int64_t qoff = query_offset(p, b, hq, t, s, nt);
      int64_t kvbase = ((int64_t)b * p->Hkv + h) * N * D;
      int64_t n = 0;
      for (int32_t a = 0; a < p->K; ++a) {
        int64_t j = sel[a];
        if (j < 0) continue;
        int64_t lo = j * p->C, hi = lo + p->C < N ? lo + p->C : N;
        for (int64_t i = lo; i < hi; ++i) {
          if (p->causal && i > t) break;
          key[n] = i;
          z[n] = dot_qk(q, k, p->dtype, qoff, kvbase + i * D, D) * p->scale;
          ++n;
        }
      }
      double* out = o + w * D;
      double m = -INFINITY;
      for (int64_t i = 0; i < n; ++i)
        if (z[i] > m) m = z[i];
      for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;
      if (n == 0) {
        for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
        lse_out[w] = -INFINITY;
        continue;
      }
      double den = 0.0;
      for (int64_t i = 0; i < n; ++i) {
        double e = exp(z[i] - m);
        den += e;
        for (int32_t d = 0; d < D; ++d) acc[d] += e * widen(v, p->dtype, kvbase + key[i] * D + d);
      }
      for (int32_t d = 0; d < D; ++d) out[d] = acc[d] / den;
      lse_out[w] = m + log(den);
    }
    free(z);
    free(key);
    free(acc);
  }
  return 0;
}

/* ---- public: gradients of [BSA] attention over a fixed selection ------- *
 * o_t = sum_i p_i v_i with p = softmax(z), z_i = q_t . k_i * scale over the
 * keys i of the kept leaves (i <= t when causal).  For L = sum_t dO_t . o_t:
 *   dv_i += p_i dO_t,   dp_i = dO_t . v_i,   D_t = dO_t . o_t,
 *   ds_i = p_i (dp_i - D_t),   dq_t = scale sum_i ds_i k_i,
 *   dk_i += scale ds_i q_t.
 * The selection is index-valued, so no gradient flows through it.  Every
 * position t in [0, N): idx [B][Hkv][N][K]; q, dout [B][Hq][N][D] (dtype of
 * the problem); k, v [B][Hkv][N][D].  dq [B][Hq][N][D], dk, dv [B][Hkv][N][D]
 * in fp64.                                                                   */
int oracle_attention_backward(const oracle_problem* p, const void* q, const void* k, const void* v,
                              const int32_t* idx, const void* dout, double* dq, double* dk, double* dv) {
  if (p->Hq % p->Hkv != 0 || p->q_sampled) return 1;
  const int32_t G = p->Hq / p->Hkv;
  const int64_t N = p->N;
  const int32_t D = p->D;
  memset(dq, 0, sizeof(double) * (size_t)p->B * p->Hq * N * D);
  memset(dk, 0, sizeof(double) * (size_t)p->B * p->Hkv * N * D);
  memset(dv, 0, sizeof(double) * (size_t)p->B * p->Hkv * N * D);
#pragma omp parallel
  {
    const int64_t cap = (int64_t)p->K * p->C;
    double* z = (double*)malloc(sizeof(double) * (cap > 0 ? cap : 1));
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (cap > 0 ? cap : 1));
    double* o = (double*)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)p->B * p->Hkv; ++bh) {  /* a head's dk, dv belong to one thread */
      const int32_t b = (int32_t)(bh / p->Hkv), h = (int32_t)(bh % p->Hkv);
      const int64_t kvbase = bh * N * D;
      for (int64_t t = 0; t < N; ++t) {
        const int32_t* sel = idx + (bh * N + t) * p->K;
        int64_t n = 0;
        for (int32_t a = 0; a < p->K; ++a) {
          const int64_t j = sel[a];
          if (j < 0) continue;
          const int64_t lo = j * p->C, hi = lo + p->C < N ? lo + p->C : N;
          for (int64_t i = lo; i < hi; ++i) {
            if (p->causal && i > t) break;
            key[n++] = i;
          }
        }
        if (n == 0) continue;
        for (int32_t g = 0; g < G; ++g) {
          const int32_t hq = h * G + g;
          const int64_t qoff = (((int64_t)b * p->Hq + hq) * N + t) * D;
          double m = -INFINITY;
          for (int64_t a = 0; a < n; ++a) {
            z[a] = dot_qk(q, k, p->dtype, qoff, kvbase + key[a] * D, D) * p->scale;
            if (z[a] > m) m = z[a];
          }
          double den = 0.0;
          for (int64_t a = 0; a < n; ++a) {
            z[a] = exp(z[a] - m);
            den += z[a];
          }
          for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
          for (int64_t a = 0; a < n; ++a) {
            z[a] /= den; /* p_i */
            for (int32_t d = 0; d < D; ++d) o[d] += z[a] * widen(v, p->dtype, kvbase + key[a] * D + d);
          }
          double Dt = 0.0;
          for (int32_t d = 0; d < D; ++d) Dt += widen(dout, p->dtype, qoff + d) * o[d];
          for (int64_t a = 0; a < n; ++a) {
            const int64_t ko = kvbase + key[a] * D;
            double dp = 0.0;
            for (int32_t d = 0; d < D; ++d) dp += widen(dout, p->dtype, qoff + d) * widen(v, p->dtype, ko + d);
            const double ds = z[a] * (dp - Dt);
            for (int32_t d = 0; d < D; ++d) {
              dq[qoff + d] += p->scale * ds * widen(k, p->dtype, ko + d);
              dk[ko + d] += p->scale * ds * widen(q, p->dtype, qoff + d);
              dv[ko + d] += z[a] * widen(dout, p->dtype, qoff + d);
            }
          }
        }
      }
    }
    free(z);
    free(key);
    free(o);
  }
  return 0;
}

/* ---- public: [BSA-flat] single-level selector -------------------------- *
 * Every valid leaf j is scored by sum over the GQA group of
 * q_{h',t} . P_1[j] * scale; the top K by (score desc, index asc) are kept.
 * idx, score: [B][Hkv][nt][K], ascending, -1 / -inf padded.                 */
int oracle_flat_select(const oracle_problem* p, const void* q, const void* k, const int32_t* ts,
                       int64_t nt, int32_t* idx, double* score) {
  if (p->Hq % p->Hkv != 0) return 1;
  const int32_t G = p->Hq / p->Hkv;
  const int64_t M1 = oracle_level_rows(p->N, p->C, 1);
  double* leaves = (double*)malloc(sizeof(double) * oracle_pyramid_rows(p->N, p->C) * p->D);
  if (!leaves) return 2;
  for (int32_t b = 0; b < p->B; ++b)
    for (int32_t h = 0; h < p->Hkv; ++h) {
      const int64_t kbase = ((int64_t)b * p->Hkv + h) * (int64_t)p->N * p->D;
      oracle_pyramid((const char*)k + kbase * (p->dtype == ORACLE_BF16 ? 2 : 4), p->dtype, p->D,
                     p->N, p->D, p->C, leaves);
#pragma omp parallel
      {
        scored* all = (scored*)malloc(sizeof(scored) * M1);
#pragma omp for schedule(dynamic, 16)
        for (int64_t s = 0; s < nt; ++s) {
          int64_t t = ts[s];
          int64_t n = 0;
          for (int64_t j = 0; j < M1; ++j) {
            if (p->causal && j * p->C > t) break;
            double u = 0.0;
            for (int32_t g = 0; g < G; ++g) {
              int64_t qoff = query_offset(p, b, h * G + g, t, s, nt);
              u += dot_q(q, p->dtype, qoff, leaves + j * p->D, p->D) * p->scale;
            }
            all[n].u = u;
            all[n].j = j;
            ++n;
          }
          qsort(all, (size_t)n, sizeof(scored), by_score_then_index);
          int64_t keep = n < p->K ? n : p->K;
          qsort(all, (size_t)keep, sizeof(scored), by_index);
          int64_t o = ((int64_t)b * p->Hkv + h) * nt + s;
          for (int32_t a = 0; a < p->K; ++a) {
            idx[o * p->K + a] = (a < keep) ? (int32_t)all[a].j : -1;
            score[o * p->K + a] = (a < keep) ? all[a].u : -INFINITY;
          }
        }
        free(all);
      }
    }
  free(leaves);
  return 0;
}

/* ---- public: exact leaf top-K (quality reference) --------------------- *
 * Every valid leaf j is scored by the level-1 block score of [SEL] (the
 * exact raw-key LSE, causally masked, summed over the GQA group) and the top
 * K by (score desc, index asc) are kept: what the descent would return if
 * every leaf were a candidate.  idx, score: [B][Hkv][nt][K], ascending,
 * -1 / -inf padded.                                                          */
int oracle_exact_topk(const oracle_problem* p, const void* q, const void* k, const int32_t* ts, int64_t nt,
                      int32_t* idx, double* score) {
  if (p->Hq % p->Hkv != 0) return 1;
  const int32_t G = p->Hq / p->Hkv;
  const int64_t M1 = oracle_level_rows(p->N, p->C, 1);
  for (int32_t b = 0; b < p->B; ++b)
    for (int32_t h = 0; h < p->Hkv; ++h) {
      const int64_t kbase = ((int64_t)b * p->Hkv + h) * (int64_t)p->N * p->D;
#pragma omp parallel
      {
        scored* all = (scored*)malloc(sizeof(scored) * M1);
        double* buf = (double*)malloc(sizeof(double) * p->C);
#pragma omp for schedule(dynamic, 1)
        for (int64_t s = 0; s < nt; ++s) {
          const int64_t t = ts[s];
          int64_t n = 0;
          for (int64_t j = 0; j < M1; ++j) {
            if (p->causal && j * p->C > t) break;
            double u = 0.0;
            for (int32_t g = 0; g < G; ++g) {
              int64_t nk = 0;
              u += score_leaf(p, q, k, query_offset(p, b, h * G + g, t, s, nt), kbase, j, t, buf, &nk);
            }
            all[n].u = u;
            all[n].j = j;
            ++n;
          }
          qsort(all, (size_t)n, sizeof(scored), by_score_then_index);
          const int64_t keep = n < p->K ? n : p->K;
          qsort(all, (size_t)keep, sizeof(scored), by_index);
          const int64_t o = ((int64_t)b * p->Hkv + h) * nt + s;
          for (int32_t a = 0; a < p->K; ++a) {
            idx[o * p->K + a] = (a < keep) ? (int32_t)all[a].j : -1;
            score[o * p->K + a] = (a < keep) ? all[a].u : -INFINITY;
          }
        }
        free(buf);
        free(all);
      }
    }
  return 0;
}

/* ---- public: level-1 block score of given leaves ([SEL] score, l = 1) ---- *
 * For every (b, h, sample s) and every listed leaf j = leaves[b][h][s][a]
 * (a < nl): u = sum over the GQA group of the raw-key LSE of
 * q_{h',t} . k_i * scale over the keys i of leaf j (i <= t when causal),
 * [KER] GQA sum.  Entries < 0 or >= ceil(N/C), and leaves with no valid key,
 * give -inf.  out: [B][Hkv][nt][nl].  This scores whatever set a selector
 * returned, so a set can be checked without re-running the descent.        */
int oracle_leaf_scores(const oracle_problem* p, const void* q, const void* k, const int32_t* ts, int64_t nt,
                       const int32_t* leaves, int32_t nl, double* out) {
  if (p->Hq % p->Hkv != 0 || nl < 0) return 1;
  const int32_t G = p->Hq / p->Hkv;
  const int64_t M1 = oracle_level_rows(p->N, p->C, 1);
  for (int32_t b = 0; b < p->B; ++b)
    for (int32_t h = 0; h < p->Hkv; ++h) {
      const int64_t kbase = ((int64_t)b * p->Hkv + h) * (int64_t)p->N * p->D;
#pragma omp parallel
      {
        double* buf = (double*)malloc(sizeof(double) * p->C);
#pragma omp for schedule(dynamic, 4)
        for (int64_t s = 0; s < nt; ++s) {
          const int64_t t = ts[s];
          const int64_t o = (((int64_t)b * p->Hkv + h) * nt + s) * nl;
          for (int32_t a = 0; a < nl; ++a) {
            const int64_t j = leaves[o + a];
            double u = -INFINITY;
            if (j >= 0 && j < M1) {
              u = 0.0;
              for (int32_t g = 0; g < G; ++g) {
                int64_t nk = 0;
                u += score_leaf(p, q, k, query_offset(p, b, h * G + g, t, s, nt), kbase, j, t, buf, &nk);
              }
            }
            out[o + a] = u;
          }
        }
        free(buf);
      }
    }
  return 0;
}

/* ---- public: pyramid of every (b, h) head, stacked [B][Hkv][rows][D] --- */
int oracle_build_pyramid(const oracle_problem* p, const void* k, double* pyr) {
  const int64_t rows = oracle_pyramid_rows(p->N, p->C);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < (int64_t)p->B * p->Hkv; ++bh) {
    const int64_t kbase = bh * (int64_t)p->N * p->D;
    oracle_pyramid((const char*)k + kbase * (p->dtype == ORACLE_BF16 ? 2 : 4), p->dtype, p->D,
                   p->N, p->D, p->C, pyr + bh * rows * p->D);
  }
  return 0;
}

int oracle_counter_len(void) { return CNT_LEN; }

/* Host threads the oracle's parallel loops use. */
int oracle_threads(void) { return omp_get_max_threads(); }
