/*
 * attn_oracle.c -- plain CPU reference for grouped-query attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header, table or helper with the HIP
 * library; both sides only receive the same seeded inputs.
 *
 * What it computes (the definition, not the tiled method):
 *
 *   For query head h the key/value head is hk = h / g with g = Hq / Hkv
 *   (integer division: g consecutive query heads share one K/V head).
 *   Source: BootstrapAI evolution log, entry "Kernel 9 -- GQA Flash Attention
 *   (MHA/GQA/MQA Unified)", the one-line head mapping and the MHA/GQA/MQA
 *   mode table (MHA: Hkv = Hq, GQA: 1 < Hkv < Hq, MQA: Hkv = 1).
 *
 *   s_j  = scale * sum_c q[b,h,i,c] * k[b,hk,j,c]        j in the visible set J
 *   m    = max_j s_j
 *   e_j  = exp(s_j - m),   l = sum_j e_j
 *   o[c] = (sum_j e_j * v[b,hk,j,c]) / l
 *
 *   Visible set J: all keys 0..Nk-1 when not causal.  When causal, query row
 *   i sits at absolute position q_offset + i and sees keys j <= q_offset + i
 *   (diagonal included), the chunked-prefill alignment of the kaispace.site
 *   note on Chunked Prefill (a long prompt split into chunks that attend to
 *   everything before them).
 *
 *   The tiled online-softmax recurrence of the BootstrapAI log ("Kernel 2 --
 *   tiling", running max with the exp(m_old - m_new) rescale) and the
 *   split-sequence decode of the microLLM-rocm optimization log (experiments
 *   283/284 and 291/292) are exact rearrangements of this definition in real
 *   arithmetic, so the oracle evaluates the definition directly: two passes
 *   per row (max, then exp/sum/weighted sum), fp64 throughout, every sum in
 *   ascending index order.
 *
 *   Decode (single new token per sequence, KV cache of capacity Smax):
 *   row b attends cache slots [0, n) with n = clamp(seqlens[b], 0, Smax),
 *   no mask (the query is the newest token, its own K/V already appended).
 *   n == 0 gives an all-zero output row (documented reading; the pages are
 *   silent on empty caches).
 *
 *   Decode with append (oracle_attn_decode_append): the new token's K/V rows
 *   are first written to cache slot pos = positions[b] of each K/V head,
 *   then the row attends slots [0, pos]; rows with pos outside [0, Smax) are
 *   inactive (no write, zero output).  Sources at that function.
 *
 *   Backward (oracle_attn_bwd): dQ, dK, dV of a loss with dL/dO given, the
 *   K/V gradients summed over the query heads of each K/V head.  Formulas
 *   and sources at that function.
 *
 * Inputs are the exact values the GPU consumes, widened to double by the
 * caller (fp32 as is, bf16 by appending 16 zero bits).  Layout is contiguous
 * row-major: q,o [B,Hq,Nq,d]; k,v [B,Hkv,Nk,d]; caches [B,Hkv,Smax,d].
 *
 * Return value: 0 on success, -1 on an invalid argument, -2 when a scratch
 * allocation fails.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int check_shapes(long B, long Hq, long Hkv, long Nq, long Nk, long d) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nk <= 0 || d <= 0) return -1;
  if (Hq % Hkv != 0) return -1;
  return 0;
}

/*
 * One output row: query (b, h, i).  scores is caller scratch of length Nk.
 * Writes d values to out and, when probs != NULL, the Nk softmax weights
 * (zero for keys outside the visible set).
 */
static void attend_row(const double* q, const double* k, const double* v,
                       long B, long Hq, long Hkv, long Nq, long Nk, long d,
                       int causal, long q_offset, double scale,
                       long b, long h, long i, double* scores, double* out,
                       double* probs) {
  (void)B;
  const long g = Hq / Hkv;
  const long hk = h / g;
  const double* qrow = q + ((b * Hq + h) * Nq + i) * d;
  const double* kbase = k + (b * Hkv + hk) * Nk * d;
  const double* vbase = v + (b * Hkv + hk) * Nk * d;

  /* visible keys are 0 .. last (inclusive) */
  long last = Nk - 1;
  if (causal && q_offset + i < last) last = q_offset + i;

  double m = -INFINITY;
  for (long j = 0; j <= last; ++j) {
    double dot = 0.0;
    for (long c = 0; c < d; ++c) dot += qrow[c] * kbase[j * d + c];
    scores[j] = scale * dot;
    if (scores[j] > m) m = scores[j];
  }
  double l = 0.0;
  for (long j = 0; j <= last; ++j) {
    scores[j] = exp(scores[j] - m);
    l += scores[j];
  }
  for (long c = 0; c < d; ++c) out[c] = 0.0;
  for (long j = 0; j <= last; ++j) {
    const double e = scores[j];
    for (long c = 0; c < d; ++c) out[c] += e * vbase[j * d + c];
  }
  for (long c = 0; c < d; ++c) out[c] /= l;
  if (probs) {
    for (long j = 0; j < Nk; ++j) probs[j] = (j <= last) ? scores[j] / l : 0.0;
  }
}

/* Full forward: o[B,Hq,Nq,d]. */
int oracle_attn_fwd(const double* q, const double* k, const double* v, double* o,
                    long B, long Hq, long Hkv, long Nq, long Nk, long d,
                    int causal, long q_offset, double scale) {
  if (!q || !k || !v || !o) return -1;
  if (check_shapes(B, Hq, Hkv, Nq, Nk, d)) return -1;
  if (causal && q_offset < 0) return -1;
  const long rows = B * Hq * Nq;
  int failed = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)Nk);
    if (!scores) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (long r = 0; r < rows; ++r) {
        const long i = r % Nq;
        const long h = (r / Nq) % Hq;
        const long b = r / (Nq * Hq);
        attend_row(q, k, v, B, Hq, Hkv, Nq, Nk, d, causal, q_offset, scale, b, h, i,
                   scores, o + r * d, NULL);
      }
      free(scores);
    }
  }
  return failed ? -2 : 0;
}

/*
 * Selected rows only: row_ids[n] = (b*Hq + h)*Nq + i; o_rows[n_rows, d].
 * Lets the tests check sampled outputs of shapes too large for a full pass.
 */
int oracle_attn_fwd_rows(const double* q, const double* k, const double* v,
                         long B, long Hq, long Hkv, long Nq, long Nk, long d,
                         int causal, long q_offset, double scale,
                         const int64_t* row_ids, long n_rows, double* o_rows) {
  if (!q || !k || !v || !row_ids || !o_rows || n_rows < 0) return -1;
  if (check_shapes(B, Hq, Hkv, Nq, Nk, d)) return -1;
  if (causal && q_offset < 0) return -1;
  const long rows = B * Hq * Nq;
  for (long n = 0; n < n_rows; ++n)
    if (row_ids[n] < 0 || row_ids[n] >= rows) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)Nk);
    if (!scores) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (long n = 0; n < n_rows; ++n) {
        const long r = (long)row_ids[n];
        const long i = r % Nq;
        const long h = (r / Nq) % Hq;
        const long b = r / (Nq * Hq);
        attend_row(q, k, v, B, Hq, Hkv, Nq, Nk, d, causal, q_offset, scale, b, h, i,
                   scores, o_rows + n * d, NULL);
      }
      free(scores);
    }
  }
  return failed ? -2 : 0;
}

/* Softmax weights of one row (b, h, i): probs[Nk], zero where masked. */
int oracle_attn_probs(const double* q, const double* k, const double* v,
                      long B, long Hq, long Hkv, long Nq, long Nk, long d,
                      int causal, long q_offset, double scale,
                      long b, long h, long i, double* probs) {
  if (!q || !k || !v || !probs) return -1;
  if (check_shapes(B, Hq, Hkv, Nq, Nk, d)) return -1;
  if (causal && q_offset < 0) return -1;
  if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Nq) return -1;
  double* scores = (double*)malloc(sizeof(double) * (size_t)Nk);
  double* out = (double*)malloc(sizeof(double) * (size_t)d);
  if (!scores || !out) {
    free(scores);
    free(out);
    return -2;
  }
  attend_row(q, k, v, B, Hq, Hkv, Nq, Nk, d, causal, q_offset, scale, b, h, i, scores,
             out, probs);
  free(scores);
  free(out);
  return 0;
}

/*
 * KV-cache decode: q,o [B,Hq,d]; kc,vc [B,Hkv,Smax,d]; seqlens[B].
 * Row b attends slots [0, n), n = clamp(seqlens[b], 0, Smax); slots at or
 * beyond n are never read.  The GQA-direct cache addressing (no K/V head
 * copies) follows microLLM-rocm experiment 004 and the per-head capacity
 * stride of experiment 062.
 */
int oracle_attn_decode(const double* q, const double* kc, const double* vc,
                       const int32_t* seqlens, double* o,
                       long B, long Hq, long Hkv, long Smax, long d, double scale) {
  if (!q || !kc || !vc || !seqlens || !o) return -1;
  if (check_shapes(B, Hq, Hkv, 1, Smax, d)) return -1;
  const long rows = B * Hq;
  int failed = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)Smax);
    if (!scores) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long r = 0; r < rows; ++r) {
        const long h = r % Hq;
        const long b = r / Hq;
        long n = seqlens[b];
        if (n < 0) n = 0;
        if (n > Smax) n = Smax;
        double* out = o + r * d;
        if (n == 0) {
          for (long c = 0; c < d; ++c) out[c] = 0.0;
          continue;
        }
        /* Same definition as attend_row with Nq = 1 over the first n slots:
           q row (b, h) and the cache of head hk restricted to n keys. */
        const long g = Hq / Hkv;
        const long hk = h / g;
        const double* qrow = q + (b * Hq + h) * d;
        const double* kbase = kc + (b * Hkv + hk) * Smax * d;
        const double* vbase = vc + (b * Hkv + hk) * Smax * d;
        double m = -INFINITY;
        for (long j = 0; j < n; ++j) {
          double dot = 0.0;
          for (long c = 0; c < d; ++c) dot += qrow[c] * kbase[j * d + c];
          scores[j] = scale * dot;
          if (scores[j] > m) m = scores[j];
        }
        double l = 0.0;
        for (long j = 0; j < n; ++j) {
          scores[j] = exp(scores[j] - m);
          l += scores[j];
        }
        for (long c = 0; c < d; ++c) out[c] = 0.0;
        for (long j = 0; j < n; ++j)
          for (long c = 0; c < d; ++c) out[c] += scores[j] * vbase[j * d + c];
        for (long c = 0; c < d; ++c) out[c] /= l;
      }
      free(scores);
    }
  }
  return failed ? -2 : 0;
}

/*
 * Decode step that first appends the new token's K/V at a per-row position.
 *
 * Sources: the microLLM-rocm optimization log, experiment 025 (the K and V
 * cache stores of one position done together, in one launch) and the
 * per-row position table of experiments 083/084 and 098 (rows at different
 * positions decode in one batch, each through its own small metadata entry;
 * an inactive row is skipped explicitly, experiment 097).
 *
 * Steps, in that order:
 *   1. append: for every row b whose position pos = positions[b] lies in
 *      [0, Smax), and every K/V head hk, cache slot pos of head hk takes the
 *      new rows: kc[b,hk,pos,:] = k_new[b,hk,:], vc[b,hk,pos,:] = v_new[b,hk,:];
 *   2. attend: each query head of row b attends slots [0, pos] -- the new
 *      token included, so n = pos + 1 -- by the decode definition above.
 * A row with pos < 0 or pos >= Smax is inactive (documented reading: the
 * pages fix no behaviour at the capacity boundary): nothing is written and
 * its output rows are zero.  kc and vc are updated in place.
 */
int oracle_attn_decode_append(const double* q, const double* knew, const double* vnew,
                              double* kc, double* vc, const int32_t* positions, double* o,
                              long B, long Hq, long Hkv, long Smax, long d, double scale) {
  if (!q || !knew || !vnew || !kc || !vc || !positions || !o) return -1;
  if (check_shapes(B, Hq, Hkv, 1, Smax, d)) return -1;
  int32_t* lens = (int32_t*)malloc(sizeof(int32_t) * (size_t)B);
  if (!lens) return -2;
  for (long b = 0; b < B; ++b) {
    const long pos = positions[b];
    const int active = pos >= 0 && pos < Smax;
    lens[b] = active ? (int32_t)(pos + 1) : 0;
    if (!active) continue;
    for (long hk = 0; hk < Hkv; ++hk) {
      const double* ksrc = knew + (b * Hkv + hk) * d;
      const double* vsrc = vnew + (b * Hkv + hk) * d;
      double* kdst = kc + ((b * Hkv + hk) * Smax + pos) * d;
      double* vdst = vc + ((b * Hkv + hk) * Smax + pos) * d;
      memcpy(kdst, ksrc, sizeof(double) * (size_t)d);
      memcpy(vdst, vsrc, sizeof(double) * (size_t)d);
    }
  }
  const int rc = oracle_attn_decode(q, kc, vc, lens, o, B, Hq, Hkv, Smax, d, scale);
  free(lens);
  return rc;
}

/*
 * Backward of the forward definition, for a scalar loss L whose gradient
 * with respect to O is dout (layout of o).
 *
 * Source: the microLLM-rocm optimization log, experiments 044 and 051-054:
 * one forward/backward boundary for QK, causal softmax, PV and the GQA head
 * mapping, with K/V heads never copied; the backward recomputes each row's
 * probabilities and reduces the K/V gradients over the query heads that
 * share a K/V head (first with atomics, exp. 051; then as an explicit
 * reduction, exps. 052/054).  The formulas are the chain rule through the
 * definition above, for query head h, K/V head hk = h / g and visible keys
 * J of row i:
 *
 *   P_ij  = softmax over J of s_ij            (the forward's weights)
 *   dP_ij = sum_c dout[b,h,i,c] * v[b,hk,j,c]
 *   D_i   = sum_{j in J} P_ij * dP_ij
 *   dS_ij = P_ij * (dP_ij - D_i)              (softmax Jacobian)
 *   dq[b,h,i,:]  = scale * sum_{j in J} dS_ij * k[b,hk,j,:]
 *   dk[b,hk,j,:] = scale * sum over h with h / g = hk, rows i: dS_ij * q[b,h,i,:]
 *   dv[b,hk,j,:] =         sum over h with h / g = hk, rows i: P_ij * dout[b,h,i,:]
 *
 * Masked keys get no gradient.  Each (b, hk) is one task (its g query heads
 * in ascending order, rows ascending), so every sum has a fixed order.
 * dq has the layout of q, dk and dv that of k and v.
 */
int oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dout,
                    double* dq, double* dk, double* dv,
                    long B, long Hq, long Hkv, long Nq, long Nk, long d,
                    int causal, long q_offset, double scale) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
  if (check_shapes(B, Hq, Hkv, Nq, Nk, d)) return -1;
  if (causal && q_offset < 0) return -1;
  const long g = Hq / Hkv;
  const long tasks = B * Hkv;
  int failed = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)Nk);
    double* probs = (double*)malloc(sizeof(double) * (size_t)Nk);
    double* dp = (double*)malloc(sizeof(double) * (size_t)Nk);
    double* orow = (double*)malloc(sizeof(double) * (size_t)d);
    if (!scores || !probs || !dp || !orow) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long t = 0; t < tasks; ++t) {
        const long b = t / Hkv;
        const long hk = t % Hkv;
        const double* kbase = k + (b * Hkv + hk) * Nk * d;
        const double* vbase = v + (b * Hkv + hk) * Nk * d;
        double* dkbase = dk + (b * Hkv + hk) * Nk * d;
        double* dvbase = dv + (b * Hkv + hk) * Nk * d;
        for (long x = 0; x < Nk * d; ++x) {
          dkbase[x] = 0.0;
          dvbase[x] = 0.0;
        }
        for (long r = 0; r < g; ++r) {
          const long h = hk * g + r;
          for (long i = 0; i < Nq; ++i) {
            const long row = (b * Hq + h) * Nq + i;
            const double* qrow = q + row * d;
            const double* dorow = dout + row * d;
            double* dqrow = dq + row * d;
            attend_row(q, k, v, B, Hq, Hkv, Nq, Nk, d, causal, q_offset, scale, b, h, i,
                       scores, orow, probs);
            long last = Nk - 1;
            if (causal && q_offset + i < last) last = q_offset + i;
            double D = 0.0;
            for (long j = 0; j <= last; ++j) {
              double dot = 0.0;
              for (long c = 0; c < d; ++c) dot += dorow[c] * vbase[j * d + c];
              dp[j] = dot;
              D += probs[j] * dot;
            }
            for (long c = 0; c < d; ++c) dqrow[c] = 0.0;
            for (long j = 0; j <= last; ++j) {
              const double ds = probs[j] * (dp[j] - D);
              for (long c = 0; c < d; ++c) {
                dqrow[c] += scale * ds * kbase[j * d + c];
                dkbase[j * d + c] += scale * ds * qrow[c];
                dvbase[j * d + c] += probs[j] * dorow[c];
              }
            }
          }
        }
      }
    }
    free(scores);
    free(probs);
    free(dp);
    free(orow);
  }
  return failed ? -2 : 0;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
