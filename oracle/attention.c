/*
 * Oracle: plain fp64 attention over explicitly gathered K/V.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library. The product path never
 * calls it, links it or shares code with it.
 *
 * What it computes (TensorSharp "高级功能" page, section "原生分页注意力": a
 * paged-attention call gathers each sequence's K/V out of the paged buffers
 * and runs ordinary attention over them; section "连续批处理与分页 KV 缓存":
 * many sequences are packed into one call). Attention itself is the textbook
 * definition, written out once per (query row, query head):
 *
 *   rows of sequence s are q[qsl[s] .. qsl[s+1]); q_len = qsl[s+1] - qsl[s];
 *   row r of s sits at absolute position p = ctx_s - q_len + r and sees the
 *   keys t = 0 .. p (the appended rows are the last q_len positions);
 *   query head h reads KV head g = h / (Hq / Hkv);
 *   x_t = scale * sum_d q[d] * k_t[d]                 (d ascending)
 *   M   = max(max_t x_t, sigma_h if sinks)
 *   w_t = exp(x_t - M)
 *   Z   = sum_t w_t + (exp(sigma_h - M) if sinks)
 *   out = (sum_t w_t * v_t) / Z
 *
 * The sink (same page, "WithSinks variant"; the "per-head attention-sink bias"
 * of the DSpark drafter) is one logit per query head that enters the softmax
 * denominator only: it carries no value vector and is not multiplied by scale.
 *
 * Two optional restrictions of the visible keys (oracle_attention_masked):
 *   - tree windows (TensorFold page, section on the GPU accept kernel: a
 *     verify round lays its drafts out as a chain or a tree of at most 16
 *     rows): with base = ctx - q_len, row r sees every key below base, its
 *     own key base + r, and the window key base + j (j < r) when bit j of its
 *     mask is set; a chain is the mask with every bit below r set;
 *   - a sliding window of W keys (TensorSharp "高级功能" page: the drafters'
 *     sliding-window KV rings and SWA-1024 in "MTP / NextN 推测解码", the
 *     sliding-window layers and window-bounded prefix reuse in "性能优化"):
 *     row r also needs t > p - W.
 * Both only remove keys; the row's own key always stays visible.
 *
 * Inputs arrive as float (every bf16 and fp32 value is exact in float), or K/V
 * as double (dequantized 8-bit values: code times per-token scale), and are
 * widened to double before any arithmetic; all sums are in double, in index
 * order. Output is double.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

/* One key/value element as double: from float storage, or from double
 * storage (dequantized 8-bit pools, whose values a float may not hold). */
static inline double kv_at(const void *base, int64_t idx, int kv64)
{
    return kv64 ? ((const double *)base)[idx] : (double)((const float *)base)[idx];
}

/* Is key t visible to row r (position p) of a sequence whose last q_len
 * positions are query rows? tree_mask: the row's mask word or NULL (causal);
 * window: 0 for none, else the number of keys ending at p that stay visible. */
static int visible(int64_t t, int64_t p, int64_t r, int64_t base, const uint32_t *tree_mask,
                   int64_t window)
{
    if (t > p)
        return 0;
    if (window > 0 && t <= p - window)
        return 0;
    if (tree_mask && t >= base) {
        const int64_t j = t - base;  /* window index, 0 .. r */
        if (j != r && !((*tree_mask >> j) & 1u))
            return 0;
    }
    return 1;
}

static int attend(const float *q, const void *k, const void *v, int kv64,
                  const int64_t *key_start, const int32_t *qsl, int32_t num_seqs,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  double scale, const float *sinks, const uint32_t *tree_mask, int64_t window,
                  double *out, int32_t num_threads)
{
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0 || window < 0)
        return -1;
    for (int32_t s = 0; s < num_seqs; ++s) {
        int64_t ctx = key_start[s + 1] - key_start[s];
        int32_t q_len = qsl[s + 1] - qsl[s];
        if (q_len < 0 || q_len > ctx)
            return -1;
        if (tree_mask && q_len > 32)
            return -1;               /* a mask word covers 32 window rows */
    }
    const int32_t group = num_q_heads / num_kv_heads;
    const int64_t total_rows = qsl[num_seqs];
    const int64_t items = total_rows * num_q_heads;
    const int64_t D = head_dim;

#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads)
    for (int64_t item = 0; item < items; ++item) {
        const int64_t i = item / num_q_heads;      /* global query row */
        const int32_t h = (int32_t)(item % num_q_heads);
        int32_t s = 0;                               /* sequence owning row i */
        while (qsl[s + 1] <= i)
            ++s;
        const int64_t ctx = key_start[s + 1] - key_start[s];
        const int64_t q_len = qsl[s + 1] - qsl[s];
        const int64_t r = i - qsl[s];
        const int64_t p = ctx - q_len + r;           /* last visible key */
        const int64_t base = ctx - q_len;            /* first window position */
        const uint32_t *mrow = tree_mask ? tree_mask + i : NULL;
        const int32_t g = h / group;
        const float *qi = q + (i * num_q_heads + h) * D;
        double *o = out + (i * num_q_heads + h) * D;

        /* scores and their maximum */
        double M = -INFINITY;
        for (int64_t t = 0; t <= p; ++t) {
            if (!visible(t, p, r, base, mrow, window))
                continue;
            const int64_t kt = ((key_start[s] + t) * num_kv_heads + g) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d)
                dot += (double)qi[d] * kv_at(k, kt + d, kv64);
            double x = scale * dot;
            if (x > M)
                M = x;
        }
        if (sinks && (double)sinks[h] > M)
            M = (double)sinks[h];

        for (int64_t d = 0; d < D; ++d)
            o[d] = 0.0;
        double Z = 0.0;
        for (int64_t t = 0; t <= p; ++t) {
            if (!visible(t, p, r, base, mrow, window))
                continue;
            const int64_t kt = ((key_start[s] + t) * num_kv_heads + g) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d)
                dot += (double)qi[d] * kv_at(k, kt + d, kv64);
            double w = exp(scale * dot - M);
            Z += w;
            for (int64_t d = 0; d < D; ++d)
                o[d] += w * kv_at(v, kt + d, kv64);
        }
        if (sinks)
            Z += exp((double)sinks[h] - M);
        for (int64_t d = 0; d < D; ++d)
            o[d] /= Z;
    }
    return 0;
}

/*
 * q      [total_rows][Hq][D]          query rows, packed per sequence
 * k, v   [key_start[S]][Hkv][D]       gathered keys/values; sequence s owns
 *                                      positions key_start[s] .. key_start[s+1]
 * qsl    [S+1]                         query-row offsets
 * sinks  [Hq] or NULL
 * out    [total_rows][Hq][D]
 * Returns 0, or -1 on inconsistent sizes (q_len > ctx, Hq % Hkv != 0).
 */
int oracle_attention(const float *q, const float *k, const float *v,
                     const int64_t *key_start, const int32_t *qsl, int32_t num_seqs,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     double scale, const float *sinks, double *out, int32_t num_threads)
{
    return attend(q, k, v, 0, key_start, qsl, num_seqs, num_q_heads, num_kv_heads, head_dim, scale,
                  sinks, NULL, 0, out, num_threads);
}

/* The same with double keys and values. */
int oracle_attention_kv64(const float *q, const double *k, const double *v,
                          const int64_t *key_start, const int32_t *qsl, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          double scale, const float *sinks, double *out, int32_t num_threads)
{
    return attend(q, k, v, 1, key_start, qsl, num_seqs, num_q_heads, num_kv_heads, head_dim, scale,
                  sinks, NULL, 0, out, num_threads);
}

/* Either K/V storage (kv64 = 0: float, 1: double) with the optional tree
 * masks (tree_mask [total_rows] or NULL; every q_len <= 32 when given) and
 * sliding window (0 = none). */
int oracle_attention_masked(const float *q, const void *k, const void *v, int32_t kv64,
                            const int64_t *key_start, const int32_t *qsl, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            double scale, const float *sinks, const uint32_t *tree_mask,
                            int64_t window, double *out, int32_t num_threads)
{
    return attend(q, k, v, kv64 != 0, key_start, qsl, num_seqs, num_q_heads, num_kv_heads, head_dim,
                  scale, sinks, tree_mask, window, out, num_threads);
}
