/*
 * Plain fp64 reference for softmax attention — TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. It shares no code with the HIP kernels and is written
 * to be checked by eye, not to be fast: every output row materialises its
 * full row of scores, applies the mask by exclusion, and runs a two-pass
 * softmax (max, then exp / sum / weighted sum of V).
 *
 * What it computes (the plain definition that flash attention reaches up to
 * rounding order), for batch b, query row i, q-head h:
 *
 *   hk      = h / (Hq / Hkv)                  GQA: consecutive groups of Hq/Hkv
 *                                             q-heads share one kv-head
 *           ("Flash-Attention: Context (CTE)", section "GQA and multi-head")
 *   qpos    = i + (Skv - Sq)                  query position, bottom-right aligned
 *   visible = (!causal || j <= qpos) && (window <= 0 || j >= qpos - window + 1)
 *           (causal predicate q_pos >= k_pos: CTE page, "the diagonal
 *            affine_select mask"; window k_pos >= q_pos - window + 1:
 *            optimum-neuron attention guide, "Sliding window")
 *   s_j     = scale * sum_d q[b,i,h,d] * k[b,j,hk,d]         for visible j
 *   m       = max_j s_j
 *   l       = sum_j exp(s_j - m)
 *   o[d]    = sum_j exp(s_j - m) * v[b,j,hk,d] / l
 *   lse     = m + log(l)                      natural-log log-sum-exp
 *           (two-pass softmax of the decode page's torch reference,
 *            "The single-query decode attention"; scale applied to the
 *            scores: CTE page, section "Scale")
 *
 * Attention sink (optional, one logit sink[h] per q-head, in the units of the
 * scaled scores): it joins the softmax as one more logit that has no value
 * row, so it enters the max and the sum but not the weighted sum of V
 * ("Flash-Attention: Context (CTE)": the sink logit appended as an extra
 * column of the section max and its exp appended to the sums; one sink per
 * q-head, broadcast over the batch, on the decode page):
 *   m   = max(max_j s_j, sink[h])
 *   l   = sum_j exp(s_j - m) + exp(sink[h] - m)
 *   o   = sum_j exp(s_j - m) v_j / l,   lse = m + log(l)
 * A sink of -inf is no sink.
 *
 * A row with no visible key gets o = 0 and lse = -inf, or lse = sink[h] with
 * a sink (the convention of the minfer "8n" page, section 3.2, epilogue: an
 * all-masked row is zero). Masked keys are skipped, never multiplied by zero,
 * so NaN in masked K/V cannot leak.
 *
 * Layouts: q is [B, Sq, Hq, D], k and v are [B, Skv, Hkv, D], addressed with
 * element strides (batch, seq, head); the head_dim stride is 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

static int visible_at(int64_t qpos, int64_t j, int causal, int64_t window)
{
    if (causal && j > qpos) return 0;
    if (window > 0 && j < qpos - window + 1) return 0;
    return 1;
}

static int visible(int64_t i, int64_t j, int64_t Sq, int64_t Skv, int causal, int64_t window)
{
    return visible_at(i + (Skv - Sq), j, causal, window);
}

/* mask[i*Skv + j] = 1 if query row i sees key j */
void oracle_visible_mask(int64_t Sq, int64_t Skv, int causal, int64_t window, uint8_t* mask)
{
    for (int64_t i = 0; i < Sq; ++i)
        for (int64_t j = 0; j < Skv; ++j)
            mask[i * Skv + j] = (uint8_t)visible(i, j, Sq, Skv, causal, window);
}

/* One output row. s is scratch of length Skv. Returns the lse. */
static double attention_row(const double* qrow, const double* k, const int64_t* k_st,
                            const double* v, const int64_t* v_st, int64_t b, int64_t hk,
                            int64_t qpos, int64_t Skv, int64_t D, double scale,
                            int causal, int64_t window, int has_sink, double sink, double* s,
                            double* orow)
{
    double m = -INFINITY;
    int64_t nvis = 0;
    for (int64_t j = 0; j < Skv; ++j) {
        if (!visible_at(qpos, j, causal, window)) continue;
        const double* krow = k + b * k_st[0] + j * k_st[1] + hk * k_st[2];
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += qrow[d] * krow[d];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
        ++nvis;
    }
    for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
    if (has_sink && sink == -INFINITY) has_sink = 0;
    if (has_sink && sink > m) m = sink;
    if (nvis == 0 && !has_sink) return -INFINITY;

    double l = has_sink ? exp(sink - m) : 0.0;
    for (int64_t j = 0; j < Skv; ++j) {
        if (!visible_at(qpos, j, causal, window)) continue;
        double p = exp(s[j] - m);
        const double* vrow = v + b * v_st[0] + j * v_st[1] + hk * v_st[2];
        l += p;
        for (int64_t d = 0; d < D; ++d) orow[d] += p * vrow[d];
    }
    for (int64_t d = 0; d < D; ++d) orow[d] /= l;
    return m + log(l);
}

/*
 * Attention for a list of output rows.
 *   rows:  nrows triples (b, i, h)
 *   sinks: [Hq] sink logits, or NULL for none
 *   qpos:  [Sq] position of query row i (the same for every b), or NULL for
 *          i + (Skv - Sq); key j is visible to a row at position P iff j <= P
 *          (causal) and j >= P - window + 1 (the minfer page's positions input:
 *          KV positions are data, section 3.1)
 *   o:     [nrows, D] output; lse: [nrows] output (may be NULL)
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_attention_rows(const double* q, const int64_t* q_st, const double* k, const int64_t* k_st,
                          const double* v, const int64_t* v_st, int64_t Hq, int64_t Hkv,
                          int64_t Sq, int64_t Skv, int64_t D, double scale, int causal,
                          int64_t window, const double* sinks, const int64_t* qpos, const int64_t* rows,
                          int64_t nrows, double* o, double* lse)
{
    if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || Sq < 0 || Skv < 0) return -1;
    const int64_t group = Hq / Hkv;
    int failed = 0;
#pragma omp parallel reduction(| : failed)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
        if (!s) failed = 1;
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!s) continue;
            const int64_t b = rows[3 * r], i = rows[3 * r + 1], h = rows[3 * r + 2];
            const double* qrow = q + b * q_st[0] + i * q_st[1] + h * q_st[2];
            const int64_t pos = qpos ? qpos[i] : i + (Skv - Sq);
            double L = attention_row(qrow, k, k_st, v, v_st, b, h / group, pos, Skv, D, scale,
                                     causal, window, sinks != NULL, sinks ? sinks[h] : 0.0, s,
                                     o + r * D);
            if (lse) lse[r] = L;
        }
        free(s);
    }
    return failed ? -1 : 0;
}
