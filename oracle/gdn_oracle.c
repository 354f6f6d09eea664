/*
 * gdn_oracle.c -- plain, slow fp64 reference of the gated-delta-rule (GDN) mixer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  It shares no
 * code, header, table or helper with the HIP library, and never calls it.
 *
 * What it computes, and where that is stated:
 *   - The mixer (the Qwen3.5 hybrid model's linear-attention layer) is a
 *     depthwise causal conv1d of width 4 over the packed q/k/v channels with a
 *     3-row tail state, then SiLU, then L2-normalised q and k (q also scaled
 *     by dk^-1/2), then per value head the recurrence
 *         S <- alpha * S * (I - beta k k^T) + beta v k^T,   o = S q,
 *         alpha = exp(-exp(A_log) * softplus(a + dt_bias)),  beta = sigmoid(b).
 *     S is dv x dk; this file stores its transpose M = S^T as [dk][dv]
 *     (dv contiguous), so the same step reads
 *         M <- alpha * (M - beta k (k^T M)) + beta k v^T,   o = M^T q.
 *   - Verify windows hold at most 16 rows, and the engine records each row's
 *     recurrent state and conv tail; the rows of a window must give what the
 *     same rows give as one-row steps, bit for bit: page "perf(qwen3_5 cuda):
 *     deliver the first token before drafting", commit note on the MLX affine
 *     4-bit checkpoint on the native CUDA server.
 *   - A window's rows may form a tree in which each row names its parent; the
 *     conv taps and the delta rule then follow each row's own branch; one-row
 *     steps and prompt passes change the state in place: same page, commit
 *     note on tree-shaped verify windows.
 *   - A verify round packs every stream's window together, at most 16 streams
 *     of 16 rows: page "perf(qwen27 cuda): reduce repeated-prompt TTFT", commit
 *     note on the qwen3_5 checkpoint with the 27B's shapes.
 *   - The prompt oracle is the plain recurrence, row after row.
 *   - Instead of every row's state, a verify pass may log each row's decay,
 *     write and key, and keeping a row then replays the kept path onto the
 *     stream's recurrence (and the kept rows' raw inputs become the conv
 *     tail): same page, commit note on tree-shaped verify windows.  Reading:
 *     the write of row t is the vector delta_t with M_t = alpha_t M_p +
 *     khat_t delta_t^T, i.e. delta_t = beta_t (v_t - alpha_t M_p^T khat_t).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   conv is a cross-correlation, y_t = sum_j w[c][j] x_{t-3+j}[c], no bias;
 *   the tail holds the last three raw (pre-conv) rows, oldest first; SiLU acts
 *   on every channel; channels are [q | k | v], head-major; value head h uses
 *   key head h / (hv / hk); khat = k / sqrt(|k|^2 + 1e-6),
 *   qhat = q / sqrt(|q|^2 + 1e-6) / sqrt(dk); o is read after the update.
 *
 * Arithmetic is fp64 throughout, from the exact bf16 / fp32 input values.
 * Parallelism (OpenMP over (stream, value head)) never changes a result: no
 * sum crosses those units.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CONV_W 4
#define TAIL 3

typedef struct {
    int32_t hk, hv, dk, dv;
} oracle_shape;

static int channels(const oracle_shape *s) { return 2 * s->hk * s->dk + s->hv * s->dv; }

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* softplus(x) = log(1 + e^x), in the form that neither overflows nor cancels. */
static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static double silu(double y) { return y * sigmoid(y); }

/* Decay alpha and write strength beta of one (row, value head). */
void gdn_oracle_gates(double a, double b, double a_log, double dt_bias,
                      double *alpha, double *beta)
{
    double g = -exp(a_log) * softplus(a + dt_bias);
    *alpha = exp(g);
    *beta = sigmoid(b);
}

/* Causal depthwise conv of channels [c0, c0 + count) of one row: taps[j] is
 * the raw row x_{t-3+j} (taps[3] = the current row).  Writes the conv output
 * before (optional) and after SiLU, indexed from c0, and (optional) the
 * magnitude of each output: the magnitude of the conv's terms, sum_j
 * |w_j x_j|, times SiLU's gate sigmoid(y) (silu(y) = y sigmoid(y)). */
static void conv_silu_range(const float *conv_w, const uint16_t *const taps[4], int c0, int count,
                            double *pre, double *post, double *mag)
{
    for (int c = c0; c < c0 + count; ++c) {
        double y = 0.0, ymag = 0.0;
        for (int j = 0; j < CONV_W; ++j) {
            const double term = (double)conv_w[(size_t)c * CONV_W + j] * bf16_value(taps[j][c]);
            y += term;
            ymag += fabs(term);
        }
        if (pre) pre[c - c0] = y;
        if (post) post[c - c0] = silu(y);
        if (mag) mag[c - c0] = sigmoid(y) * ymag;
    }
}

/* The same for all C channels of a row. */
void gdn_oracle_conv_silu(int32_t C, const float *conv_w, const uint16_t *const taps[4],
                          double *pre, double *post)
{
    conv_silu_range(conv_w, taps, 0, C, pre, post, NULL);
}

/* Everything value head h needs from one row: normalised q and k of its key
 * head, its v, and its gates.  Only the conv channels of those heads are
 * computed: q of key head kh, k of key head kh, v of value head h.  With mag
 * (optional: [dk] q, [dk] k, [dv] v) also the magnitude of each (the conv's
 * term magnitude through SiLU's gate, then the same normalisation scale). */
static void head_inputs(const oracle_shape *s, const float *conv_w, const uint16_t *const taps[4],
                        int h, double a, double b, double a_log, double dt_bias,
                        double *qhat, double *khat, double *v, double *alpha, double *beta,
                        double *mag)
{
    const int r = s->hv / s->hk;
    const int kh = h / r;
    double *qm = mag, *km = mag ? mag + s->dk : NULL, *vm = mag ? mag + 2 * s->dk : NULL;
    conv_silu_range(conv_w, taps, kh * s->dk, s->dk, NULL, qhat, qm);
    conv_silu_range(conv_w, taps, s->hk * s->dk + kh * s->dk, s->dk, NULL, khat, km);
    conv_silu_range(conv_w, taps, 2 * s->hk * s->dk + h * s->dv, s->dv, NULL, v, vm);
    double qq = 0.0, kk = 0.0;
    for (int i = 0; i < s->dk; ++i) {
        qq += qhat[i] * qhat[i];
        kk += khat[i] * khat[i];
    }
    const double qs = 1.0 / sqrt(qq + 1e-6) / sqrt((double)s->dk);
    const double ks = 1.0 / sqrt(kk + 1e-6);
    for (int i = 0; i < s->dk; ++i) {
        qhat[i] = qhat[i] * qs;
        khat[i] = khat[i] * ks;
        if (mag) {
            qm[i] *= qs;
            km[i] *= ks;
        }
    }
    gdn_oracle_gates(a, b, a_log, dt_bias, alpha, beta);
}

/* One step of the recurrence on M = S^T ([dk][dv]), in the literal product
 * form M <- alpha (M - beta k (k^T M)) + beta k v^T, then o = M^T q. */
static void delta_step(int dk, int dv, const double *khat, const double *qhat,
                       const double *v, double alpha, double beta, double *M,
                       double *kTM, double *o)
{
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += khat[i] * M[(size_t)i * dv + j];
        kTM[j] = acc;
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) {
            double *m = &M[(size_t)i * dv + j];
            *m = alpha * (*m - beta * khat[i] * kTM[j]) + beta * khat[i] * v[j];
        }
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += M[(size_t)i * dv + j] * qhat[i];
        o[j] = acc;
    }
}

/* The magnitudes of one step, for error bounds that respect cancellation
 * (a readout o_j = sum_i M_ij q_i, a write v_j - alpha (k^T M)_j or a conv
 * output can be far smaller than the terms it adds up, and no finite-
 * precision evaluation keeps a small relative error on such a value).  The
 * step that starts from state M is carried out on magnitudes: |M| for the
 * state, km, qm, vm for khat, qhat and v, every sum as the sum of its terms'
 * magnitudes and every product as the product of magnitudes (alpha, beta >= 0):
 *     U = |M|^T km,   A = alpha (|M| + beta km U^T) + beta km vm^T,   O = A^T qm,
 * and the row's write delta = beta (v - alpha k^T M) has magnitude
 * W = beta (vm + alpha U).  A ([dk][dv]) gets the new state's magnitudes, O
 * (optional) the readout's, W (optional) the write's; U is scratch [dv].
 * The magnitudes start from the state a row is given, not from magnitudes
 * carried across rows: carried, alpha (I + beta km km^T) would grow them by
 * up to alpha (1 + beta) a row, where the step itself, alpha (I - beta k
 * k^T), never grows the state. */
static void magnitude_step(int dk, int dv, const double *km, const double *qm, const double *vm,
                           double alpha, double beta, const double *M, double *A, double *U,
                           double *O, double *W)
{
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += km[i] * fabs(M[(size_t)i * dv + j]);
        U[j] = acc;
        if (W) W[j] = beta * (vm[j] + alpha * acc);
    }
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            A[(size_t)i * dv + j] = alpha * (fabs(M[(size_t)i * dv + j]) + beta * km[i] * U[j]) +
                                    beta * km[i] * vm[j];
    if (O)
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += A[(size_t)i * dv + j] * qm[i];
            O[j] = acc;
        }
}

/* The recurrence alone, on inputs given directly: T rows of alpha, beta,
 * khat [T][dk], qhat [T][dk] and v [T][dv], from M0 [dk][dv].  Writes the
 * final state and o [T][dv]; M_all [T][dk][dv] (optional) gets every row's
 * state, o_mag [T][dv] (optional) each readout's magnitude (magnitude_step
 * with |khat|, |qhat| and |v|). */
void gdn_oracle_raw_recurrence(int32_t dk, int32_t dv, int32_t T, const double *alpha,
                               const double *beta, const double *khat, const double *qhat,
                               const double *v, const double *M0, double *M_out,
                               double *o, double *M_all, double *o_mag)
{
    const size_t msz = (size_t)dk * dv;
    double *M = malloc(sizeof(double) * msz);
    double *tmp = malloc(sizeof(double) * (size_t)dv);
    double *A = o_mag ? malloc(sizeof(double) * msz) : NULL;
    double *am = o_mag ? malloc(sizeof(double) * (size_t)(2 * dk + dv)) : NULL;
    memcpy(M, M0, sizeof(double) * msz);
    for (int t = 0; t < T; ++t) {
        const double *k = khat + (size_t)t * dk, *q = qhat + (size_t)t * dk, *vt = v + (size_t)t * dv;
        if (A) {
            for (int i = 0; i < dk; ++i) {
                am[i] = fabs(k[i]);
                am[dk + i] = fabs(q[i]);
            }
            for (int j = 0; j < dv; ++j) am[2 * dk + j] = fabs(vt[j]);
            magnitude_step(dk, dv, am, am + dk, am + 2 * dk, alpha[t], beta[t], M, A, tmp,
                           o_mag + (size_t)t * dv, NULL);
        }
        delta_step(dk, dv, k, q, vt, alpha[t], beta[t], M, tmp, o + (size_t)t * dv);
        if (M_all) memcpy(M_all + (size_t)t * msz, M, sizeof(double) * msz);
    }
    memcpy(M_out, M, sizeof(double) * msz);
    free(M);
    free(tmp);
    free(A);
    free(am);
}

/*
 * Rows of one stream, as a tree.  Row i (local index) hangs off parent[i]
 * (parent[i] < i; -1 = the stream's committed state and tail).  A chain is the
 * tree with parent[i] = i - 1.  For each row:
 *   tail_i = (tail_p[1], tail_p[2], x_i)  where tail_p is the parent's tail,
 *   taps   = (tail_p[0], tail_p[1], tail_p[2], x_i),
 *   M_i    = delta step of M_p with row i's inputs.
 * Results go to o [rows][hv][dv] (fp64), and optionally to each row's tail
 * (raw bf16 bits, [rows][3][C]) and state ([rows][hv][dk][dv] as fp64 and/or
 * fp32).  final_state / final_tail (optional) get the last row's.
 */
typedef struct {
    const oracle_shape *s;
    const float *conv_w, *a_log, *dt_bias;
    const uint16_t *qkv, *a, *b;   /* rows of this stream: [rows][C], [rows][hv] */
    const int32_t *parent;         /* [rows] local, or NULL = chain              */
    const uint16_t *tail0;         /* [3][C]                                     */
    const double *state0;          /* [hv][dk][dv]                               */
    int32_t rows;
    double *o;                     /* [rows][hv][dv]                             */
    uint16_t *tail_snap;           /* [rows][3][C] or NULL                        */
    double *snap64;                /* [rows][hv][dk][dv] or NULL                  */
    float *snap32;                 /* [rows][hv][dk][dv] or NULL                  */
    double *final_state;           /* [hv][dk][dv] or NULL                        */
    uint16_t *final_tail;          /* [3][C] or NULL                              */
    double *log_alpha;             /* [rows][hv] or NULL: each row's decay        */
    double *log_delta;             /* [rows][hv][dv] or NULL: each row's write    */
    double *log_key;               /* [rows][hk][dk] or NULL: each row's khat     */
    double *o_mag;                 /* [rows][hv][dv] or NULL: magnitude of each o */
    double *log_delta_mag;         /* [rows][hv][dv] or NULL: ... of each write   */
    float *snap_mag;               /* [rows][hv][dk][dv] or NULL: ... of each state */
    double *final_mag;             /* [hv][dk][dv] or NULL: ... of the last state */
} stream_job;

/* Per-row tails of a stream (bf16 bits): node tails follow the parents. */
static uint16_t *stream_tails(const stream_job *jb)
{
    const int C = channels(jb->s);
    uint16_t *tails = malloc(sizeof(uint16_t) * (size_t)jb->rows * TAIL * C);
    for (int i = 0; i < jb->rows; ++i) {
        const int p = jb->parent ? jb->parent[i] : i - 1;
        const uint16_t *tp = p < 0 ? jb->tail0 : tails + (size_t)p * TAIL * C;
        uint16_t *ti = tails + (size_t)i * TAIL * C;
        memcpy(ti, tp + C, sizeof(uint16_t) * 2 * C);               /* (tail_p[1], tail_p[2]) */
        memcpy(ti + 2 * C, jb->qkv + (size_t)i * C, sizeof(uint16_t) * C); /* x_i */
    }
    return tails;
}

/* The recurrence of one value head over one stream's rows. */
static void stream_head(const stream_job *jb, const uint16_t *tails, int h)
{
    const oracle_shape *s = jb->s;
    const int C = channels(s), dk = s->dk, dv = s->dv;
    const size_t msz = (size_t)dk * dv;
    const int is_tree = jb->parent != NULL;
    const int mags = jb->o_mag || jb->log_delta_mag || jb->snap_mag || jb->final_mag;
    /* a chain needs only the running state; a tree keeps every node's */
    double *states = malloc(sizeof(double) * msz * (is_tree ? (size_t)jb->rows : 1));
    double *cur = malloc(sizeof(double) * msz);
    double *amag = mags ? malloc(sizeof(double) * msz) : NULL;   /* the row's state magnitudes */
    double *qhat = malloc(sizeof(double) * dk), *khat = malloc(sizeof(double) * dk);
    double *v = malloc(sizeof(double) * dv), *tmp = malloc(sizeof(double) * dv);
    double *inmag = malloc(sizeof(double) * (size_t)(2 * dk + dv));   /* q, k, v magnitudes */
    const double *M0 = jb->state0 + (size_t)h * msz;
    memcpy(cur, M0, sizeof(double) * msz);
    for (int i = 0; i < jb->rows; ++i) {
        const int p = is_tree ? jb->parent[i] : i - 1;
        if (is_tree) memcpy(cur, p < 0 ? M0 : states + (size_t)p * msz, sizeof(double) * msz);
        const uint16_t *tp = p < 0 ? jb->tail0 : tails + (size_t)p * TAIL * C;
        const uint16_t *taps[4] = {tp, tp + C, tp + 2 * C, jb->qkv + (size_t)i * C};
        double alpha, beta;
        head_inputs(s, jb->conv_w, taps, h, bf16_value(jb->a[(size_t)i * s->hv + h]),
                    bf16_value(jb->b[(size_t)i * s->hv + h]), jb->a_log[h], jb->dt_bias[h],
                    qhat, khat, v, &alpha, &beta, mags ? inmag : NULL);
        const size_t oo = ((size_t)i * s->hv + h) * dv;
        if (mags)   /* from the state the row starts from, before the update */
            magnitude_step(dk, dv, inmag + dk, inmag, inmag + 2 * dk, alpha, beta, cur, amag, tmp,
                           jb->o_mag ? jb->o_mag + oo : NULL,
                           jb->log_delta_mag ? jb->log_delta_mag + oo : NULL);
        delta_step(dk, dv, khat, qhat, v, alpha, beta, cur, tmp, jb->o + oo);
        /* the log: tmp holds k^T M of the row's starting state */
        if (jb->log_alpha) jb->log_alpha[(size_t)i * s->hv + h] = alpha;
        if (jb->log_delta)
            for (int j = 0; j < dv; ++j)
                jb->log_delta[oo + j] = beta * (v[j] - alpha * tmp[j]);
        if (jb->log_key && h % (s->hv / s->hk) == 0)   /* one value head per key head writes it */
            memcpy(jb->log_key + ((size_t)i * s->hk + h / (s->hv / s->hk)) * dk, khat,
                   sizeof(double) * dk);
        if (is_tree) memcpy(states + (size_t)i * msz, cur, sizeof(double) * msz);
        const size_t off = ((size_t)i * s->hv + h) * msz;
        if (jb->snap64) memcpy(jb->snap64 + off, cur, sizeof(double) * msz);
        if (jb->snap32)
            for (size_t e = 0; e < msz; ++e) jb->snap32[off + e] = (float)cur[e];
        if (jb->snap_mag)
            for (size_t e = 0; e < msz; ++e) jb->snap_mag[off + e] = (float)amag[e];
    }
    if (jb->final_state && jb->rows > 0)
        memcpy(jb->final_state + (size_t)h * msz, cur, sizeof(double) * msz);
    if (jb->final_mag)
        for (size_t e = 0; e < msz; ++e)
            jb->final_mag[(size_t)h * msz + e] = jb->rows > 0 ? amag[e] : fabs(M0[e]);
    free(states); free(cur); free(amag); free(qhat); free(khat); free(v); free(tmp); free(inmag);
}

static void finish_tails(const stream_job *jb, const uint16_t *tails)
{
    const int C = channels(jb->s);
    if (jb->tail_snap)
        memcpy(jb->tail_snap, tails, sizeof(uint16_t) * (size_t)jb->rows * TAIL * C);
    if (jb->final_tail && jb->rows > 0)
        memcpy(jb->final_tail, tails + (size_t)(jb->rows - 1) * TAIL * C,
               sizeof(uint16_t) * TAIL * C);
}

/* Runs many streams; OpenMP threads take (stream, value head) units. */
static void run_streams(const stream_job *jobs, int n, int hv)
{
    uint16_t **tails = malloc(sizeof(uint16_t *) * (size_t)(n > 0 ? n : 1));
    for (int s = 0; s < n; ++s) tails[s] = stream_tails(&jobs[s]);
    const long units = (long)n * hv;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u) stream_head(&jobs[u / hv], tails[u / hv], (int)(u % hv));
    for (int s = 0; s < n; ++s) {
        finish_tails(&jobs[s], tails[s]);
        free(tails[s]);
    }
    free(tails);
}

static void fill_job(stream_job *jb, const oracle_shape *s, const float *conv_w,
                     const float *a_log, const float *dt_bias, const int32_t *row_start,
                     int stream, const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                     const uint16_t *tail, const double *state)
{
    const int C = channels(s);
    const int r0 = row_start[stream];
    memset(jb, 0, sizeof *jb);
    jb->s = s;
    jb->conv_w = conv_w; jb->a_log = a_log; jb->dt_bias = dt_bias;
    jb->qkv = qkv + (size_t)r0 * C;
    jb->a = a + (size_t)r0 * s->hv;
    jb->b = b + (size_t)r0 * s->hv;
    jb->tail0 = tail + (size_t)stream * TAIL * C;
    jb->state0 = state + (size_t)stream * s->hv * s->dk * s->dv;
    jb->rows = row_start[stream + 1] - r0;
}

/*
 * Verify windows (parent == NULL: each stream's rows form a chain) or trees
 * (parent[r] = local parent index of packed row r, -1 for a root).  Inputs:
 * row_start [n+1] (host), qkv [R][C] bf16 bits, a, b [R][hv] bf16 bits, tail
 * [n][3][C] bf16 bits, state [n][hv][dk][dv] fp64.  Outputs (any may be NULL
 * but o): o [R][hv][dv] fp64, tail_snap [R][3][C], snap64 / snap32
 * [R][hv][dk][dv], and the log: log_alpha [R][hv], log_delta [R][hv][dv],
 * log_key [R][hk][dk]; and the magnitudes (the step on magnitudes, see
 * magnitude_step) of every o (o_mag [R][hv][dv]), every write (log_delta_mag
 * [R][hv][dv]) and every row's state (snap_mag [R][hv][dk][dv], fp32).
 * Returns 0, or -1 on a malformed layout.
 */
int gdn_oracle_window(const oracle_shape *s, const float *conv_w, const float *a_log,
                      const float *dt_bias, int32_t n, const int32_t *row_start,
                      const int32_t *parent, const uint16_t *qkv, const uint16_t *a,
                      const uint16_t *b, const uint16_t *tail, const double *state,
                      double *o, uint16_t *tail_snap, double *snap64, float *snap32,
                      double *log_alpha, double *log_delta, double *log_key, double *o_mag,
                      double *log_delta_mag, float *snap_mag)
{
    if (s->hk <= 0 || s->hv <= 0 || s->hv % s->hk || s->dk <= 0 || s->dv <= 0 || n < 0)
        return -1;
    const int C = channels(s);
    const size_t msz = (size_t)s->dk * s->dv;
    stream_job *jobs = calloc((size_t)(n > 0 ? n : 1), sizeof *jobs);
    for (int st = 0; st < n; ++st) {
        if (row_start[st + 1] < row_start[st]) { free(jobs); return -1; }
        fill_job(&jobs[st], s, conv_w, a_log, dt_bias, row_start, st, qkv, a, b, tail, state);
        const int r0 = row_start[st];
        if (parent) {
            jobs[st].parent = parent + r0;
            for (int i = 0; i < jobs[st].rows; ++i)
                if (parent[r0 + i] < -1 || parent[r0 + i] >= i) { free(jobs); return -1; }
        }
        jobs[st].o = o + (size_t)r0 * s->hv * s->dv;
        if (tail_snap) jobs[st].tail_snap = tail_snap + (size_t)r0 * TAIL * C;
        if (snap64) jobs[st].snap64 = snap64 + (size_t)r0 * s->hv * msz;
        if (snap32) jobs[st].snap32 = snap32 + (size_t)r0 * s->hv * msz;
        if (log_alpha) jobs[st].log_alpha = log_alpha + (size_t)r0 * s->hv;
        if (log_delta) jobs[st].log_delta = log_delta + (size_t)r0 * s->hv * s->dv;
        if (log_key) jobs[st].log_key = log_key + (size_t)r0 * s->hk * s->dk;
        if (o_mag) jobs[st].o_mag = o_mag + (size_t)r0 * s->hv * s->dv;
        if (log_delta_mag) jobs[st].log_delta_mag = log_delta_mag + (size_t)r0 * s->hv * s->dv;
        if (snap_mag) jobs[st].snap_mag = snap_mag + (size_t)r0 * s->hv * msz;
    }
    run_streams(jobs, n, s->hv);
    free(jobs);
    return 0;
}

/*
 * Prompt passes: each of the n prompts runs its rows as one chain from its
 * stream's state and tail, and its final state and tail replace them (in
 * place).  state is fp64 [n][hv][dk][dv] in/out, tail [n][3][C] bf16 bits
 * in/out, o [T][hv][dv] fp64; optional magnitudes (see magnitude_step) of
 * every o (o_mag [T][hv][dv]) and of each final state (final_mag
 * [n][hv][dk][dv], |state| for an empty prompt).  A prompt of zero rows leaves
 * its stream as it was.
 */
int gdn_oracle_prefill(const oracle_shape *s, const float *conv_w, const float *a_log,
                       const float *dt_bias, int32_t n, const int32_t *seq_start,
                       const uint16_t *qkv, const uint16_t *a, const uint16_t *b,
                       uint16_t *tail, double *state, double *o, double *o_mag,
                       double *final_mag)
{
    if (s->hk <= 0 || s->hv <= 0 || s->hv % s->hk || s->dk <= 0 || s->dv <= 0 || n < 0)
        return -1;
    const int C = channels(s);
    const size_t ssz = (size_t)s->hv * s->dk * s->dv;
    /* inputs are copied so that the in-place results never feed a later read */
    double *state_in = malloc(sizeof(double) * ssz * (size_t)(n > 0 ? n : 1));
    uint16_t *tail_in = malloc(sizeof(uint16_t) * (size_t)TAIL * C * (n > 0 ? n : 1));
    memcpy(state_in, state, sizeof(double) * ssz * (size_t)n);
    memcpy(tail_in, tail, sizeof(uint16_t) * (size_t)TAIL * C * n);
    stream_job *jobs = calloc((size_t)(n > 0 ? n : 1), sizeof *jobs);
    for (int st = 0; st < n; ++st) {
        if (seq_start[st + 1] < seq_start[st]) {
            free(jobs); free(state_in); free(tail_in);
            return -1;
        }
        fill_job(&jobs[st], s, conv_w, a_log, dt_bias, seq_start, st, qkv, a, b, tail_in,
                 state_in);
        jobs[st].o = o + (size_t)seq_start[st] * s->hv * s->dv;
        if (o_mag) jobs[st].o_mag = o_mag + (size_t)seq_start[st] * s->hv * s->dv;
        if (final_mag) jobs[st].final_mag = final_mag + (size_t)st * ssz;
        jobs[st].final_state = state + (size_t)st * ssz;
        jobs[st].final_tail = tail + (size_t)st * TAIL * C;
    }
    run_streams(jobs, n, s->hv);
    free(jobs);
    free(state_in);
    free(tail_in);
    return 0;
}

/* Commit: a stream's state and tail become those recorded for its accepted
 * row (packed index), or stay as they are for -1. */
int gdn_oracle_commit(const oracle_shape *s, int32_t n, int32_t total_rows,
                      const int32_t *accept, const uint16_t *tail_snap, const double *snap64,
                      uint16_t *tail, double *state)
{
    const int C = channels(s);
    const size_t ssz = (size_t)s->hv * s->dk * s->dv;
    for (int st = 0; st < n; ++st) {
        const int r = accept[st];
        if (r < -1 || r >= total_rows) return -1;
        if (r < 0) continue;
        memcpy(state + (size_t)st * ssz, snap64 + (size_t)r * ssz, sizeof(double) * ssz);
        memcpy(tail + (size_t)st * TAIL * C, tail_snap + (size_t)r * TAIL * C,
               sizeof(uint16_t) * TAIL * C);
    }
    return 0;
}

/* Replay of logged rows onto one head's state M [dk][dv], in the given order:
 * M <- alpha_t M + khat_t delta_t^T for each row t (the step of the
 * recurrence, given its logged write). */
void gdn_oracle_replay(int32_t dk, int32_t dv, int32_t n, const double *alpha, const double *delta,
                       const double *key, double *M)
{
    for (int t = 0; t < n; ++t)
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j) {
                double *m = &M[(size_t)i * dv + j];
                *m = alpha[t] * *m + key[(size_t)t * dk + i] * delta[(size_t)t * dv + j];
            }
}

/*
 * Commit by replay.  accept[s] is the packed index of stream s's kept row
 * (within its window [row_start[s], row_start[s+1])) or -1 to keep the stream
 * as it is.  The kept path runs from the stream's state to that row through
 * the parents (parent == NULL: the window's rows in order); every head of
 * the state gets the path's logged rows replayed in path order, and the conv
 * tail becomes the last three raw rows along the path, continuing into the
 * old tail for a path of fewer than three rows.  Logs as gdn_oracle_window
 * writes them; state fp64 [n][hv][dk][dv] and tail [n][3][C] in/out.
 * Returns 0, or -1 on a malformed layout or accepted row.
 */
int gdn_oracle_commit_replay(const oracle_shape *s, int32_t n, const int32_t *row_start,
                             const int32_t *parent, const int32_t *accept, const uint16_t *qkv,
                             const double *log_alpha, const double *log_delta,
                             const double *log_key, uint16_t *tail, double *state)
{
    if (s->hk <= 0 || s->hv <= 0 || s->hv % s->hk || s->dk <= 0 || s->dv <= 0 || n < 0)
        return -1;
    const int C = channels(s), dk = s->dk, dv = s->dv, r = s->hv / s->hk;
    const size_t msz = (size_t)dk * dv;
    for (int st = 0; st < n; ++st) {
        const int r0 = row_start[st], r1 = row_start[st + 1];
        if (r1 < r0) return -1;
        const int acc = accept[st];
        if (acc == -1) continue;
        if (acc < r0 || acc >= r1) return -1;
        /* the path, leaf first, then reversed */
        int path[64], len = 0;
        for (int i = acc - r0; i >= 0; i = parent ? parent[r0 + i] : i - 1) {
            if (len == 64 || (parent && parent[r0 + i] >= i)) return -1;
            path[len++] = i;
        }
        for (int a = 0, b = len - 1; a < b; ++a, --b) {
            const int t = path[a]; path[a] = path[b]; path[b] = t;
        }
        double *al = malloc(sizeof(double) * len), *de = malloc(sizeof(double) * len * dv);
        double *ke = malloc(sizeof(double) * len * dk);
        for (int h = 0; h < s->hv; ++h) {
            for (int q = 0; q < len; ++q) {
                const size_t row = (size_t)r0 + path[q];
                al[q] = log_alpha[row * s->hv + h];
                memcpy(de + (size_t)q * dv, log_delta + (row * s->hv + h) * dv, sizeof(double) * dv);
                memcpy(ke + (size_t)q * dk, log_key + (row * s->hk + h / r) * dk, sizeof(double) * dk);
            }
            gdn_oracle_replay(dk, dv, len, al, de, ke, state + ((size_t)st * s->hv + h) * msz);
        }
        free(al); free(de); free(ke);
        /* new tail (x_{t-2}, x_{t-1}, x_t) along the path: path row q - 2 + j,
         * or old tail row len + j for q - 2 + j < 0 */
        uint16_t *tl = tail + (size_t)st * TAIL * C;
        uint16_t *nt = malloc(sizeof(uint16_t) * TAIL * C);
        for (int j = 0; j < TAIL; ++j) {
            const int q = len - TAIL + j;
            const uint16_t *src = q >= 0 ? qkv + (size_t)(r0 + path[q]) * C : tl + (size_t)(len + j) * C;
            memcpy(nt + (size_t)j * C, src, sizeof(uint16_t) * C);
        }
        memcpy(tl, nt, sizeof(uint16_t) * TAIL * C);
        free(nt);
    }
    return 0;
}

int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
