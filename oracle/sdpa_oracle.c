/*
 * Plain fp64 CPU oracle for scaled dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP implementation.
 *
 * What it computes is the definition itself, written out with no tiling,
 * no online softmax and no fused steps:
 *
 *   Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V
 *       "Aufmerksamkeit ist alles, was Sie brauchen", section 3.2.1, eq. (1);
 *       "Attention Is All You Need" (cookipedia), section "Transformer の構造".
 *
 * per (batch b, head h, query row i), each (b, h) slice being one instance of
 * eq. (1) ("all heads in parallel": cookipedia article, "Transformer の構造";
 * German translation, section 3.2.2).  The row steps follow the proof section
 * (証明) of the formula page "トランスフォーマーの注意機構":
 *   1. scores   s_j = (q . k_j) / tau, tau = sqrt(d_k) by default
 *               (the page's first display; the square root is lost in its
 *               extraction and restored from the same page's remark that the
 *               divisor for d_k = 4 is 2, and from eq. (1) of the paper);
 *   2. weights  a_j = e^{s_j} / sum_i e^{s_i} (second display).  The largest
 *               score is subtracted first; this leaves every a_j unchanged
 *               because weights depend only on score differences (fourth
 *               display, a_j / a_i = e^{s_j - s_i});
 *   3. output   o = sum_j a_j v_j (third display);
 *   4. lse      log sum_i e^{s_i}, the smoothed maximum named in the page's
 *               closing "広がる学問 / 数学" paragraph, returned as m + ln Z.
 *
 * Masks (both set a score to -inf before the softmax, so its weight is
 * exactly 0: formula page, section 応用, "先を読まない仕掛け"):
 *   causal   key j is valid for query i only if j <= i: the strict upper
 *            triangle of Q K^T is masked, the diagonal kept (cookipedia
 *            article, section "原論文でのデコーダ").  Applied top-left aligned
 *            for any Lq, Lk.
 *   key_lens key j is valid only if j < clamp(key_lens[b], 0, Lk) (padding of
 *            variable-length batches; D2L-74-Transformer, "Layer Norm").
 * A row with no valid key returns o = 0 and lse = -inf.
 *
 * Inputs may be fp64, fp32 or bf16 (raw 16-bit patterns); every element is
 * widened to fp64 exactly before any arithmetic.  Outputs are fp64.
 *
 * General form (oracle_sdpa_ex): values of their own width d_v (German
 * translation, section 3.2.1: queries and keys of dimension d_k, values of
 * dimension d_v), any divisor tau (the temperature form of section 証明),
 * and an optional additive mask added to the scaled scores before the
 * softmax, -inf entries dropping their key as the causal mask does (formula
 * page, section 応用; the toy model of the cookipedia article, section
 * "トイモデル", builds its decoder mask this way).  A row whose valid keys all
 * carry -inf returns o = 0 and lse = -inf, as a row with no valid key.
 *
 * Backward (oracle_sdpa_bwd): the gradients of a scalar loss L with
 * dL/dO = dout, following the same proof section:
 *   dL/da_j = dout . v_j                    (from the output display)
 *   dL/ds_l = sum_j dL/da_j * da_j/ds_l,  with the page's Jacobian display
 *             da_j/ds_l = a_j (delta_jl - a_l),
 *           = a_l (dL/da_l - sum_j a_j dL/da_j)
 *   dL/dq   = sum_l dL/ds_l k_l / tau,  dL/dk_l += dL/ds_l q / tau  (score)
 *   dL/dv_j += a_j dout                     (output display)
 * summed over the query rows of each (b, h) slice.  Masked keys have a_j = 0
 * and receive nothing; a row with no valid key contributes nothing.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 };

/* Exact widening of one stored element to fp64. */
static double load_elem(const void* base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_F64) return ((const double*)base)[idx];
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    /* bf16: the 16 stored bits are the top half of an IEEE binary32. */
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * One query row of one (b, h) slice.  `work` holds at least Lk doubles.
 * q_off, kv_off: element offsets of the row of Q and of the (b, h) slice of
 * K and V.
 */
/*
 * Steps 1 and 2 for one query row with n_valid >= 1 keys: work[j] = a_j.
 * Returns m + ln Z (step 4).
 */
static double row_weights(const void* q, const void* k, int dtype, int64_t q_off,
                          int64_t kv_off, int64_t d, int64_t n_valid, double tau,
                          double* work)
{
    /* 1. scores */
    for (int64_t j = 0; j < n_valid; ++j) {
        double z = 0.0;
        for (int64_t t = 0; t < d; ++t)
            z += load_elem(q, dtype, q_off + t) * load_elem(k, dtype, kv_off + j * d + t);
        work[j] = z / tau;
    }
    /* 2. weights, after subtracting the largest score */
    double m = work[0];
    for (int64_t j = 1; j < n_valid; ++j)
        if (work[j] > m) m = work[j];
    double Z = 0.0;
    for (int64_t j = 0; j < n_valid; ++j) {
        work[j] = exp(work[j] - m);
        Z += work[j];
    }
    for (int64_t j = 0; j < n_valid; ++j) work[j] /= Z;
    /* 4. log-sum-exp of the valid scores */
    return m + log(Z);
}

static void attention_row(const void* q, const void* k, const void* v,
                          int dtype, int64_t q_off, int64_t kv_off,
                          int64_t d, int64_t n_valid, double tau,
                          double* o, double* lse, double* work)
{
    if (n_valid <= 0) {
        for (int64_t t = 0; t < d; ++t) o[t] = 0.0;
        *lse = -INFINITY;
        return;
    }
    *lse = row_weights(q, k, dtype, q_off, kv_off, d, n_valid, tau, work);
    /* 3. output: weighted sum of the value rows */
    for (int64_t t = 0; t < d; ++t) {
        double acc = 0.0;
        for (int64_t j = 0; j < n_valid; ++j)
            acc += work[j] * load_elem(v, dtype, kv_off + j * d + t);
        o[t] = acc;
    }
}

/* Number of valid keys for query row i of batch b. */
static int64_t valid_keys(int64_t i, int64_t b, int64_t Lk, int causal,
                          const int32_t* key_lens)
{
    int64_t hi = Lk;
    if (key_lens) {
        int64_t len = key_lens[b];
        if (len < 0) len = 0;
        if (len < hi) hi = len;
    }
    if (causal && i + 1 < hi) hi = i + 1;
    return hi;
}

static int check_args(const void* q, const void* k, const void* v, int dtype,
                      int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                      int causal, double* out, double* lse)
{
    if (!q || !k || !v || !out || !lse) return 1;
    if (dtype < ORACLE_F64 || dtype > ORACLE_BF16) return 1;
    if (B < 1 || H < 1 || Lq < 1 || Lk < 1 || d < 1) return 1;
    if (causal != 0 && causal != 1) return 1;
    return 0;
}

/*
 * A chosen set of rows: rows[r] = (b * H + h) * Lq + i.  out is nrows x d,
 * lse has nrows entries.  tau <= 0 selects tau = sqrt(d).  nthreads <= 0
 * uses the OpenMP default.  Returns 0 on success, 1 on bad arguments.
 */
int oracle_sdpa_rows(const void* q, const void* k, const void* v, int dtype,
                     int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                     int causal, const int32_t* key_lens, double tau,
                     const int64_t* rows, int64_t nrows,
                     double* out, double* lse, int nthreads)
{
    if (check_args(q, k, v, dtype, B, H, Lq, Lk, d, causal, out, lse)) return 1;
    if (nrows < 0 || (nrows > 0 && !rows)) return 1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= B * H * Lq) return 1;
    if (!(tau > 0.0)) tau = sqrt((double)d);
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    int bad = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double* work = (double*)malloc(sizeof(double) * (size_t)Lk);
        if (!work) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!work) continue;
            int64_t row = rows[r];
            int64_t i = row % Lq;
            int64_t bh = row / Lq;
            int64_t b = bh / H;
            int64_t n_valid = valid_keys(i, b, Lk, causal, key_lens);
            attention_row(q, k, v, dtype, row * d, bh * Lk * d, d, n_valid, tau,
                          out + r * d, lse + r, work);
        }
        free(work);
    }
    return bad ? 2 : 0;
}

/*
 * Every row.  q and out are [B, H, Lq, d], k and v are [B, H, Lk, d], lse is
 * [B, H, Lq], all contiguous row-major.
 */
int oracle_sdpa(const void* q, const void* k, const void* v, int dtype,
                int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                int causal, const int32_t* key_lens, double tau,
                double* out, double* lse, int nthreads)
{
    if (check_args(q, k, v, dtype, B, H, Lq, Lk, d, causal, out, lse)) return 1;
    if (!(tau > 0.0)) tau = sqrt((double)d);
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    const int64_t nrows = B * H * Lq;
    int bad = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double* work = (double*)malloc(sizeof(double) * (size_t)Lk);
        if (!work) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t row = 0; row < nrows; ++row) {
            if (!work) continue;
            int64_t i = row % Lq;
            int64_t bh = row / Lq;
            int64_t b = bh / H;
            int64_t n_valid = valid_keys(i, b, Lk, causal, key_lens);
            attention_row(q, k, v, dtype, row * d, bh * Lk * d, d, n_valid, tau,
                          out + row * d, lse + row, work);
        }
        free(work);
    }
    return bad ? 2 : 0;
}

/*
 * Gradients.  q, dout, dq are [B, H, Lq, d]; k, v, dk, dv are [B, H, Lk, d];
 * all contiguous row-major; dout has the inputs' dtype, dq/dk/dv are fp64.
 * Slices are independent and run in parallel; inside a slice the query rows
 * are taken in order, so dk and dv are summed in a fixed order.
 */
int oracle_sdpa_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                    int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d,
                    int causal, const int32_t* key_lens, double tau,
                    double* dq, double* dk, double* dv, int nthreads)
{
    if (!dout || !dq || !dk || !dv) return 1;
    if (check_args(q, k, v, dtype, B, H, Lq, Lk, d, causal, dq, dk)) return 1;
    if (!(tau > 0.0)) tau = sqrt((double)d);
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    int bad = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)Lk);
        double* da = (double*)malloc(sizeof(double) * (size_t)Lk);
        if (!a || !da) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            if (!a || !da) continue;
            const int64_t b = bh / H;
            const int64_t kv_off = bh * Lk * d;
            for (int64_t x = 0; x < Lk * d; ++x) dk[kv_off + x] = dv[kv_off + x] = 0.0;
            for (int64_t i = 0; i < Lq; ++i) {
                const int64_t q_off = (bh * Lq + i) * d;
                for (int64_t t = 0; t < d; ++t) dq[q_off + t] = 0.0;
                const int64_t n_valid = valid_keys(i, b, Lk, causal, key_lens);
                if (n_valid <= 0) continue;
                row_weights(q, k, dtype, q_off, kv_off, d, n_valid, tau, a);
                /* dL/da_j = dout . v_j and c = sum_j a_j dL/da_j */
                double c = 0.0;
                for (int64_t j = 0; j < n_valid; ++j) {
                    double z = 0.0;
                    for (int64_t t = 0; t < d; ++t)
                        z += load_elem(dout, dtype, q_off + t) * load_elem(v, dtype, kv_off + j * d + t);
                    da[j] = z;
                    c += a[j] * z;
                }
                for (int64_t j = 0; j < n_valid; ++j) {
                    const double ds = a[j] * (da[j] - c);   /* dL/ds_j */
                    for (int64_t t = 0; t < d; ++t) {
                        dq[q_off + t] += ds * load_elem(k, dtype, kv_off + j * d + t) / tau;
                        dk[kv_off + j * d + t] += ds * load_elem(q, dtype, q_off + t) / tau;
                        dv[kv_off + j * d + t] += a[j] * load_elem(dout, dtype, q_off + t);
                    }
                }
            }
        }
        free(a);
        free(da);
    }
    return bad ? 2 : 0;
}

/*
 * General form.  q is [B, H, Lq, d], k is [B, H, Lk, d], v is [B, H, Lk, dv],
 * out is [B, H, Lq, dv], lse [B, H, Lq], mask NULL or fp64 [B, H, Lq, Lk], all
 * contiguous row-major.  Per row:
 *   1. s_j = (q . k_j) / tau + mask_ij   over the valid keys j
 *   2. m = max_j s_j; if m = -inf the row is empty (o = 0, lse = -inf);
 *      a_j = e^{s_j - m} / Z with Z = sum_j e^{s_j - m}
 *   3. o = sum_j a_j v_j (width dv)
 *   4. lse = m + ln Z
 */
int oracle_sdpa_ex(const void* q, const void* k, const void* v, int dtype,
                   int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t d, int64_t dv,
                   int causal, const int32_t* key_lens, double tau, const double* mask,
                   double* out, double* lse, int nthreads)
{
    if (check_args(q, k, v, dtype, B, H, Lq, Lk, d, causal, out, lse)) return 1;
    if (dv < 1) return 1;
    if (!(tau > 0.0)) tau = sqrt((double)d);
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    const int64_t nrows = B * H * Lq;
    int bad = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double* sc = (double*)malloc(sizeof(double) * (size_t)Lk);
        if (!sc) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t row = 0; row < nrows; ++row) {
            if (!sc) continue;
            const int64_t i = row % Lq, bh = row / Lq, b = bh / H;
            const int64_t n = valid_keys(i, b, Lk, causal, key_lens);
            double* o = out + row * dv;
            /* 1. scores plus the additive mask */
            double m = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                double z = 0.0;
                for (int64_t t = 0; t < d; ++t)
                    z += load_elem(q, dtype, row * d + t) * load_elem(k, dtype, (bh * Lk + j) * d + t);
                sc[j] = z / tau + (mask ? mask[row * Lk + j] : 0.0);
                if (sc[j] > m) m = sc[j];
            }
            if (n <= 0 || m == -INFINITY) {
                for (int64_t t = 0; t < dv; ++t) o[t] = 0.0;
                lse[row] = -INFINITY;
                continue;
            }
            /* 2. weights */
            double Z = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                sc[j] = exp(sc[j] - m);
                Z += sc[j];
            }
            /* 3. output of width dv */
            for (int64_t t = 0; t < dv; ++t) {
                double acc = 0.0;
                for (int64_t j = 0; j < n; ++j)
                    acc += sc[j] / Z * load_elem(v, dtype, (bh * Lk + j) * dv + t);
                o[t] = acc;
            }
            /* 4. log-sum-exp */
            lse[row] = m + log(Z);
        }
        free(sc);
    }
    return bad ? 2 : 0;
}
