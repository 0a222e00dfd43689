/*
 * hsw_oracle.c -- plain fp64 CPU oracle for the attention core of a hybrid
 * sliding-window-attention transformer (MiMo-V2.6 Flash/Pro shapes).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no source, header, table or helper with the
 * HIP library.  Every function is the plain definition written out in double
 * precision with straightforward loops; the only parallelism is an OpenMP
 * loop over independent (query, head) pairs, which does not change any
 * result (each pair is computed by one thread in a fixed order).
 *
 * Sources (the pages the method is described on):
 *  - colibri "MiMo-V2.6 (Xiaomi)", section "What the engine implements":
 *    hybrid layer pattern, per-kind KV heads and RoPE theta (1e4 windowed,
 *    1e7 full), a 128-position ring on windowed layers, partial rotate-half
 *    RoPE on the first int(192*0.334)=64 dims of 192-wide q/k heads, 128-wide
 *    values, the value scale applied before attention, and a per-head sink
 *    logit that joins the softmax denominator and nothing else.
 *  - colibri, section "System One mode and prompt reuse": full layers keep
 *    K/V rows by position; a windowed layer keeps position p in slot p mod 128.
 *  - gaudi-cookbook "MiMo-V2.6-Flash on Gaudi 2", section "What was built":
 *    the decode window is exactly the last 128 positions; per-block sink
 *    copies of (sink - log n) sum to one sink term; section "Tiled
 *    global-attention prefill": softmax is per query row.
 *
 * Readings where the pages are silent (each is an explicit argument here,
 * never a hidden constant): the softmax scale tau is passed in (1/sqrt(192)
 * is the caller's choice); positions are 0-based; the window holds the
 * current token and the W-1 before it; query head h reads KV head
 * h / (Hq/Hkv); rotate-half pairs are (i, i + R/2) with inv_freq[i] =
 * theta^(-2i/R) and the rotation z -> z * exp(+i*angle) on z = x[i] + i x[i+R/2].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define HSWO_OK 0
#define HSWO_E_RANGE -1   /* a key the definition needs is not in the inputs */
#define HSWO_E_ARG -2     /* inconsistent sizes */

int hswo_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Rotary frequencies for partial RoPE: inv_freq[i] = theta^(-2i/R), i < R/2.
 * colibri "What the engine implements" (theta per layer kind, R = 64). */
void hswo_inv_freq(double theta, int rope_dim, double *inv_freq) {
    for (int i = 0; i < rope_dim / 2; ++i)
        inv_freq[i] = pow(theta, -2.0 * (double)i / (double)rope_dim);
}

/* Partial rotate-half RoPE at absolute position pos[t] on every head:
 *   y[i]      = x[i] cos(a) - x[i+R/2] sin(a)
 *   y[i+R/2]  = x[i+R/2] cos(a) + x[i] sin(a),   a = pos * inv_freq[i]
 *   y[d]      = x[d]                              for d >= R.
 * x, y: [n_tok][n_heads][d] contiguous; angles and products in fp64.
 * colibri "What the engine implements" (partial RoPE, rotate-half style);
 * gaudi-cookbook "The RoPE fix for large positions" (angles must be exact
 * at large positions: they are formed and reduced in double here). */
void hswo_rope(int64_t n_tok, int n_heads, int d, int rope_dim, double theta,
               const int64_t *pos, const double *x, double *y) {
    int half = rope_dim / 2;
    double *inv_freq = (double *)malloc(sizeof(double) * (half > 0 ? half : 1));
    hswo_inv_freq(theta, rope_dim, inv_freq);
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tok; ++t) {
        for (int h = 0; h < n_heads; ++h) {
            const double *xr = x + (t * n_heads + h) * (int64_t)d;
            double *yr = y + (t * n_heads + h) * (int64_t)d;
            for (int i = 0; i < half; ++i) {
                double a = (double)pos[t] * inv_freq[i];
                double c = cos(a), s = sin(a);
                yr[i] = xr[i] * c - xr[i + half] * s;
                yr[i + half] = xr[i + half] * c + xr[i] * s;
            }
            for (int e = rope_dim; e < d; ++e) yr[e] = xr[e];
        }
    }
    free(inv_freq);
}

/* Where a token's K/V row goes (integer definition, exact):
 *   kind 0 (ring)    : slot = pos mod ring_slots   (colibri "System One mode":
 *                      position p in slot p mod 128)
 *   kind 1 (pool)    : row  = seq_base + pos        (full layers keep rows by
 *                      position)
 *   kind 2 (staging) : row  = t (the token's index in the call). */
int64_t hswo_dst_index(int kind, int64_t t, int64_t pos, int64_t seq_base,
                       int64_t ring_slots) {
    if (kind == 0) {
        int64_t r = pos % ring_slots;
        return r < 0 ? r + ring_slots : r;
    }
    if (kind == 1) return seq_base + pos;
    return t;
}

/* One query row over an explicit list of keys given by row pointers, for
 * the `group` query heads that share one KV head (q and o hold their rows
 * one after the other).  For each head h, logits l_j = tau * <q_h, k_j>; with
 * a sink s_h (when sinks is not NULL):
 *   m = max(s_h, max_j l_j),  Z = exp(s_h-m) + sum_j exp(l_j-m),
 *   o_h = sum_j exp(l_j-m) * (lambda * v_j) / Z,  lse = m + log Z.
 * Without a sink the s terms are dropped.  colibri "What the engine
 * implements" (sink in the denominator only; value scale before attention).
 * Every head runs the same operations in the same order as it would alone:
 * the key loop is outside the head loop only so that each K and V row is
 * read once for the whole group.  logit holds group * nkeys values. */
static void attend_group(int group, int dqk, int dv, double tau, double lambda,
                         const double *sinks, const double *q, int64_t nkeys,
                         const double *const *krows, const double *const *vrows,
                         double *logit, double *m, double *z, double *o,
                         double *lse, double *qt, double *acc) {
    /* qt[e][h] = q_h[e]: the heads' dot products then advance together over
     * e (acc[h] still sums its products in the order e = 0, 1, ...) */
    for (int h = 0; h < group; ++h)
        for (int e = 0; e < dqk; ++e) qt[e * group + h] = q[h * (int64_t)dqk + e];
    for (int h = 0; h < group; ++h) m[h] = sinks ? sinks[h] : -INFINITY;
    for (int64_t j = 0; j < nkeys; ++j) {
        for (int h = 0; h < group; ++h) acc[h] = 0.0;
        for (int e = 0; e < dqk; ++e) {
            const double ke = krows[j][e];
            for (int h = 0; h < group; ++h) acc[h] += qt[e * group + h] * ke;
        }
        for (int h = 0; h < group; ++h) {
            double lj = tau * acc[h];
            logit[h * nkeys + j] = lj;
            if (lj > m[h]) m[h] = lj;
        }
    }
    for (int h = 0; h < group; ++h) {
        z[h] = sinks ? exp(sinks[h] - m[h]) : 0.0;
        for (int e = 0; e < dv; ++e) o[h * (int64_t)dv + e] = 0.0;
    }
    for (int64_t j = 0; j < nkeys; ++j) {
        for (int h = 0; h < group; ++h) {
            double p = exp(logit[h * nkeys + j] - m[h]);
            z[h] += p;
            double *oh = o + h * (int64_t)dv;
            for (int e = 0; e < dv; ++e) oh[e] += p * (lambda * vrows[j][e]);
        }
    }
    for (int h = 0; h < group; ++h) {
        for (int e = 0; e < dv; ++e) o[h * (int64_t)dv + e] /= z[h];
        if (lse) lse[h] = (nkeys > 0 || sinks) ? m[h] + log(z[h]) : -INFINITY;
    }
}

/* First key position of the query at position p: a window of W positions
 * holds p-W+1 .. p (the token and the W-1 before it), clipped at 0; W = 0 is
 * full causal attention, 0 .. p.  colibri "System One mode and prompt
 * reuse" (128 slots, the token written before it attends); gaudi-cookbook
 * "What was built" (exactly the last 128 positions). */
static int64_t first_key(int64_t p, int64_t window) {
    int64_t lo = window > 0 ? p - window + 1 : 0;
    return lo < 0 ? 0 : lo;
}

/* Attention over K/V laid out linearly by absolute position.
 *   q   [nq][Hq][dqk], qpos [nq]
 *   k   [nk][Hkv][dqk], v [nk][Hkv][dv]; key row j holds position kpos0 + j
 *   window W > 0: key set of a query at p is positions max(0, p-W+1) .. p;
 *   W == 0: positions 0 .. p (full causal attention).
 *   sinks [Hq] or NULL; o [nq][Hq][dv]; lse [nq][Hq] or NULL.
 * Returns HSWO_E_RANGE if some query needs a key outside kpos0 .. kpos0+nk-1.
 * colibri "What the engine implements" and "System One mode" (the window of
 * 128 positions; full layers by position); gaudi-cookbook "What was built"
 * (exactly the last 128 positions). */
int hswo_attn_linear(int hq, int hkv, int dqk, int dv, int64_t window,
                     double tau, double lambda, const double *sinks,
                     int64_t nq, const double *q, const int64_t *qpos,
                     int64_t nk, const double *k, const double *v,
                     int64_t kpos0, double *o, double *lse) {
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || window < 0) return HSWO_E_ARG;
    int group = hq / hkv;
    int64_t cap = 1;                           /* most keys any query sees */
    for (int64_t i = 0; i < nq; ++i) {
        int64_t lo = first_key(qpos[i], window);
        if (qpos[i] < 0 || lo < kpos0 || qpos[i] > kpos0 + nk - 1) return HSWO_E_RANGE;
        if (qpos[i] - lo + 1 > cap) cap = qpos[i] - lo + 1;
    }
    int err = HSWO_OK;
    #pragma omp parallel
    {
        double *logit = (double *)malloc(sizeof(double) * cap * group);
        double *mz = (double *)malloc(sizeof(double) * 3 * group);
        double *qt = (double *)malloc(sizeof(double) * group * dqk);
        const double **kr = (const double **)malloc(sizeof(double *) * cap);
        const double **vr = (const double **)malloc(sizeof(double *) * cap);
        if (!logit || !mz || !qt || !kr || !vr) {
            #pragma omp atomic write
            err = HSWO_E_ARG;
        } else {
            /* one (query row, KV head) at a time: its `group` query heads
             * h = g * group .. share the key rows */
            #pragma omp for schedule(dynamic, 1)
            for (int64_t ig = 0; ig < nq * hkv; ++ig) {
                int64_t i = ig / hkv;
                int g = (int)(ig % hkv);
                int64_t p = qpos[i];
                int64_t lo = first_key(p, window);
                int64_t n = p - lo + 1;
                for (int64_t j = 0; j < n; ++j) {
                    int64_t row = lo + j - kpos0;
                    kr[j] = k + (row * hkv + g) * (int64_t)dqk;
                    vr[j] = v + (row * hkv + g) * (int64_t)dv;
                }
                int64_t ih0 = i * hq + (int64_t)g * group;   /* first (row, head) of the group */
                attend_group(group, dqk, dv, tau, lambda, sinks ? sinks + g * group : NULL,
                             q + ih0 * (int64_t)dqk, n, kr, vr, logit, mz, mz + group,
                             o + ih0 * (int64_t)dv, lse ? lse + ih0 : NULL, qt, mz + 2 * group);
            }
        }
        free(logit);
        free(mz);
        free(qt);
        free(kr);
        free(vr);
    }
    return err;
}

/* Decode over a ring of `slots` positions per (sequence, KV head).
 *   q [ns][Hq][dqk], pos [ns] (position of the new token, already written)
 *   kring [ns][Hkv][slots][dqk], vring [ns][Hkv][slots][dv]
 * Slot t holds position P - ((P - t) mod slots); it is used iff that
 * position is >= 0.  colibri "System One mode" (position p in slot p mod 128,
 * the ring records the position each slot holds); gaudi-cookbook "What was
 * built" (exactly the last 128 positions). */
int hswo_ring_decode(int hq, int hkv, int dqk, int dv, int64_t slots,
                     double tau, double lambda, const double *sinks,
                     int64_t ns, const double *q, const int64_t *pos,
                     const double *kring, const double *vring, double *o,
                     double *lse) {
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || slots <= 0) return HSWO_E_ARG;
    int group = hq / hkv;
    int err = HSWO_OK;
    #pragma omp parallel
    {
        double *logit = (double *)malloc(sizeof(double) * slots * group);
        double *mz = (double *)malloc(sizeof(double) * 3 * group);
        double *qt = (double *)malloc(sizeof(double) * group * dqk);
        const double **kr = (const double **)malloc(sizeof(double *) * slots);
        const double **vr = (const double **)malloc(sizeof(double *) * slots);
        if (!logit || !mz || !qt || !kr || !vr) {
            #pragma omp atomic write
            err = HSWO_E_ARG;
        } else {
            /* one (sequence, KV head) at a time, with its `group` query heads */
            #pragma omp for schedule(dynamic, 4)
            for (int64_t sg = 0; sg < ns * hkv; ++sg) {
                int64_t s = sg / hkv;
                int g = (int)(sg % hkv);
                int64_t P = pos[s];
                int64_t n = 0;
                for (int64_t t = 0; t < slots; ++t) {
                    int64_t back = (P - t) % slots;
                    if (back < 0) back += slots;
                    int64_t held = P - back;
                    if (held < 0) continue;
                    kr[n] = kring + ((s * hkv + g) * slots + t) * (int64_t)dqk;
                    vr[n] = vring + ((s * hkv + g) * slots + t) * (int64_t)dv;
                    ++n;
                }
                int64_t sh0 = s * hq + (int64_t)g * group;
                attend_group(group, dqk, dv, tau, lambda, sinks ? sinks + g * group : NULL,
                             q + sh0 * (int64_t)dqk, n, kr, vr, logit, mz, mz + group,
                             o + sh0 * (int64_t)dv, lse ? lse + sh0 : NULL, qt, mz + 2 * group);
            }
        }
        free(logit);
        free(mz);
        free(qt);
        free(kr);
        free(vr);
    }
    return err;
}

/* Split-K partial of one (query, head) over key positions [a, b) intersected
 * with its key set, no sink:  m = max l_j,  l = sum exp(l_j - m),
 * acc = sum exp(l_j - m) * lambda * v_j  (unnormalised).  An empty range
 * gives m = -inf, l = 0, acc = 0.  Keys are linear by position from kpos0.
 * Used to check the log-sum-exp combine (gaudi-cookbook "What was built":
 * per-block decode partials; "What it taught about Gaudi": count the sink
 * once per sequence, not once per block). */
int hswo_attn_partial(int hq, int hkv, int dqk, int dv, int64_t window,
                      double tau, double lambda, int64_t nq, const double *q,
                      const int64_t *qpos, int64_t nk, const double *k,
                      const double *v, int64_t kpos0, int64_t a, int64_t b,
                      double *m_out, double *l_out, double *acc_out) {
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return HSWO_E_ARG;
    int group = hq / hkv;
    for (int64_t ih = 0; ih < nq * hq; ++ih) {
        int64_t i = ih / hq;
        int g = (int)(ih % hq) / group;
        int64_t p = qpos[i];
        int64_t lo = first_key(p, window);
        if (lo < a) lo = a;
        int64_t hi = p < b - 1 ? p : b - 1;
        double m = -INFINITY, l = 0.0;
        double *acc = acc_out + ih * (int64_t)dv;
        for (int e = 0; e < dv; ++e) acc[e] = 0.0;
        const double *qr = q + ih * (int64_t)dqk;
        for (int64_t j = lo; j <= hi; ++j) {
            if (j < kpos0 || j >= kpos0 + nk) return HSWO_E_RANGE;
            const double *kr = k + ((j - kpos0) * hkv + g) * (int64_t)dqk;
            double d = 0.0;
            for (int e = 0; e < dqk; ++e) d += qr[e] * kr[e];
            if (tau * d > m) m = tau * d;
        }
        for (int64_t j = lo; j <= hi; ++j) {
            const double *kr = k + ((j - kpos0) * hkv + g) * (int64_t)dqk;
            const double *vr = v + ((j - kpos0) * hkv + g) * (int64_t)dv;
            double d = 0.0;
            for (int e = 0; e < dqk; ++e) d += qr[e] * kr[e];
            double p_ = exp(tau * d - m);
            l += p_;
            for (int e = 0; e < dv; ++e) acc[e] += p_ * (lambda * vr[e]);
        }
        m_out[ih] = m;
        l_out[ih] = l;
    }
    return HSWO_OK;
}

/* Fold one sink logit s into a partial (m, l, acc): the sink joins the
 * denominator only, so acc is rescaled and l gains exp(s - m'). */
void hswo_join_sink(int64_t n, int dv, const double *sink, double *m,
                    double *l, double *acc) {
    for (int64_t i = 0; i < n; ++i) {
        double mn = m[i] > sink[i] ? m[i] : sink[i];
        double r = (m[i] == -INFINITY) ? 0.0 : exp(m[i] - mn);
        l[i] = l[i] * r + exp(sink[i] - mn);
        for (int e = 0; e < dv; ++e) acc[i * (int64_t)dv + e] *= r;
        m[i] = mn;
    }
}

/* Log-sum-exp merge of n_parts partials for n rows:
 *   M = max_c m_c,  Z = sum_c exp(m_c - M) l_c,
 *   o = sum_c exp(m_c - M) acc_c / Z,  lse = M + log Z.
 * Partials are laid out [n_parts][n] (m, l) and [n_parts][n][dv] (acc). */
void hswo_lse_merge(int64_t n_parts, int64_t n, int dv, const double *m,
                    const double *l, const double *acc, double *o,
                    double *lse) {
    for (int64_t i = 0; i < n; ++i) {
        double M = -INFINITY;
        for (int64_t c = 0; c < n_parts; ++c)
            if (m[c * n + i] > M) M = m[c * n + i];
        double z = 0.0;
        for (int e = 0; e < dv; ++e) o[i * (int64_t)dv + e] = 0.0;
        for (int64_t c = 0; c < n_parts; ++c) {
            double mc = m[c * n + i];
            if (mc == -INFINITY) continue;
            double w = exp(mc - M);
            z += w * l[c * n + i];
            for (int e = 0; e < dv; ++e)
                o[i * (int64_t)dv + e] += w * acc[(c * n + i) * (int64_t)dv + e];
        }
        for (int e = 0; e < dv; ++e) o[i * (int64_t)dv + e] /= z;
        if (lse) lse[i] = M + log(z);
    }
}

/* ------------------------------------------------------------------------
 * Vision encoder (ViT) attention.  colibri "MiMo-V2.6 (Xiaomi)", the model
 * description's "vision" entry: 2D RoPE, grouped-query attention, full
 * attention in 4 of 28 blocks and a 1D window of 64 tokens in the others,
 * row and column order of the 2x2 merge units alternating, a sink on the
 * first key of the window blocks; the same page ("Verifying it") has the
 * gateway's patches equal to the Qwen2-VL processor's.
 *
 * Readings where the page is brief (each an explicit argument or stated
 * here, never a hidden constant):
 *  - a picture's tokens come in merge-unit order: the four patches of a 2x2
 *    unit consecutive (top-left, top-right, bottom-left, bottom-right), units
 *    row by row over the (h/2) x (w/2) unit grid (the Qwen2-VL processor's
 *    order);
 *  - "row order" of a window block is that order; "column order" takes the
 *    units column by column (each unit's four patches still consecutive);
 *  - attention is bidirectional within one picture; a window block cuts the
 *    picture's tokens, in the block's order, into consecutive windows of
 *    `window` tokens (the last may be shorter) and a token attends to its
 *    window;
 *  - the sink is a real key: the picture's first token in the block's order,
 *    seen by every window (once: the first window already holds it); a
 *    learned per-head sink logit (denominator only, as on the text model's
 *    windowed layers) may be given as well;
 *  - 2D RoPE is rotate-half over the whole head: pair (i, i + d/2), i < d/2,
 *    turns by row * f(i) for i < d/4 and col * f(i - d/4) above, with
 *    f(j) = theta^(-j / (d/4)) (the frequencies a 1D rotary of width d/2
 *    uses).
 * ------------------------------------------------------------------------ */

/* Patch coordinates of each token of an h x w patch grid (h, w even) in
 * merge-unit order, and the column-order permutation: col_order[j] is the
 * token at position j of the column order. */
int hswo_vit_layout(int h, int w, int32_t *row, int32_t *col, int32_t *col_order) {
    if (h <= 0 || w <= 0 || h % 2 || w % 2) return HSWO_E_ARG;
    int uh = h / 2, uw = w / 2;
    for (int t = 0; t < h * w; ++t) {
        int u = t / 4, e = t % 4;
        row[t] = 2 * (u / uw) + e / 2;
        col[t] = 2 * (u % uw) + e % 2;
    }
    for (int j = 0; j < h * w; ++j) {
        int uc = j / 4;                      /* unit index in column order */
        int ur = uc % uh, ucl = uc / uh;     /* its unit row and column */
        col_order[j] = 4 * (ur * uw + ucl) + j % 4;
    }
    return HSWO_OK;
}

/* 2D rotate-half RoPE of x [n_tok][n_heads][d] at patch coordinates
 * (row[t], col[t]); angles and products in fp64 (reading above). */
void hswo_rope_2d(int64_t n_tok, int n_heads, int d, double theta,
                  const int32_t *row, const int32_t *col, const double *x,
                  double *y) {
    int half = d / 2, quarter = d / 4;
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n_tok; ++t) {
        for (int h = 0; h < n_heads; ++h) {
            const double *xr = x + (t * n_heads + h) * (int64_t)d;
            double *yr = y + (t * n_heads + h) * (int64_t)d;
            for (int i = 0; i < half; ++i) {
                int f = i < quarter ? i : i - quarter;
                double coord = i < quarter ? (double)row[t] : (double)col[t];
                double a = coord * pow(theta, -(double)f / (double)quarter);
                double c = cos(a), s = sin(a);
                yr[i] = xr[i] * c - xr[i + half] * s;
                yr[i + half] = xr[i + half] * c + xr[i] * s;
            }
            for (int e = 2 * half; e < d; ++e) yr[e] = xr[e];
        }
    }
}

/* ViT attention over n_img pictures packed by cu[0..n_img] (token rows).
 *   q [T][Hq][d], k [T][Hkv][d], v [T][Hkv][dv], o [T][Hq][dv]
 *   order: NULL (row order) or per picture a permutation, order[cu[s] + j] =
 *          the picture-local token at position j of the block's order
 *   window 0: every token of the picture; window W > 0: the W-token window
 *          of the token's position in the order, plus (sink_key != 0) the
 *          token at order position 0 when it is not in that window
 *   sinks [Hq] or NULL: learned sink logits (denominator only)
 * Returns HSWO_E_ARG on inconsistent sizes or an order entry out of range. */
int hswo_vit_attn(int n_img, const int64_t *cu, const int32_t *order, int window,
                  int sink_key, int hq, int hkv, int d, int dv, double tau,
                  const double *sinks, const double *q, const double *k,
                  const double *v, double *o) {
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0 || window < 0 || d <= 0 || d > 256) return HSWO_E_ARG;
    int group = hq / hkv;
    int64_t maxlen = 1;
    for (int s = 0; s < n_img; ++s) {
        int64_t n = cu[s + 1] - cu[s];
        if (n < 0) return HSWO_E_ARG;
        if (n > maxlen) maxlen = n;
        if (order)
            for (int64_t j = 0; j < n; ++j)
                if (order[cu[s] + j] < 0 || order[cu[s] + j] >= n) return HSWO_E_ARG;
    }
    int err = HSWO_OK;
    for (int s = 0; s < n_img; ++s) {
        int64_t base = cu[s], n = cu[s + 1] - cu[s];
        #pragma omp parallel
        {
            double *logit = (double *)malloc(sizeof(double) * (maxlen + 1));
            const double **kr = (const double **)malloc(sizeof(double *) * (maxlen + 1));
            const double **vr = (const double **)malloc(sizeof(double *) * (maxlen + 1));
            if (!logit || !kr || !vr) {
                #pragma omp atomic write
                err = HSWO_E_ARG;
            } else {
                #pragma omp for schedule(dynamic, 4)
                for (int64_t jh = 0; jh < n * hq; ++jh) {
                    int64_t j = jh / hq;                 /* position in the order */
                    int h = (int)(jh % hq), g = h / group;
                    int64_t t = base + (order ? order[base + j] : j);   /* the token's row */
                    int64_t lo = 0, hi = n, nk = 0;
                    if (window > 0) {
                        lo = (j / window) * window;
                        hi = lo + window < n ? lo + window : n;
                        if (sink_key && lo > 0) {
                            int64_t r0 = base + (order ? order[base] : 0);
                            kr[nk] = k + (r0 * hkv + g) * (int64_t)d;
                            vr[nk] = v + (r0 * hkv + g) * (int64_t)dv;
                            ++nk;
                        }
                    }
                    for (int64_t jj = lo; jj < hi; ++jj) {
                        int64_t r = base + (order ? order[base + jj] : jj);
                        kr[nk] = k + (r * hkv + g) * (int64_t)d;
                        vr[nk] = v + (r * hkv + g) * (int64_t)dv;
                        ++nk;
                    }
                    double mz[3], qt[256];
                    attend_group(1, d, dv, tau, 1.0, sinks ? sinks + h : NULL,
                                 q + (t * hq + h) * (int64_t)d, nk, kr, vr, logit,
                                 mz, mz + 1, o + (t * hq + h) * (int64_t)dv, NULL, qt, mz + 2);
                }
            }
            free(logit);
            free(kr);
            free(vr);
        }
    }
    return err;
}
