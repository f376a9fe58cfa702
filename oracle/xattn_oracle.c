/*
 * Reference oracle for one-history-to-many-candidates cross-attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct CPU
 * statement of what the GPU library computes.  Only the test-suite, the
 * package's smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library, and the
 * HIP library never calls it.
 *
 * Everything is IEEE double precision, plain loops, no blocking, no fusion,
 * no -ffast-math.  Every output element is produced by exactly one loop
 * iteration in a fixed order, so results do not depend on the thread count.
 *
 * What is computed (sources are the pages on the subject):
 *   - ReST reading note (paper-archivist), section 3.3.1, Eq. (7):
 *       CrossAttn(Z, H) = softmax((Z W_Q) H^T / sqrt(d_h)) H   (gate and W_o
 *       left to the caller), where the encoder output H is used as both key
 *       and value with no projection (projection-free K/V).
 *   - ReST reading note, section 3.3.2, Eq. (8): token-specific
 *       parameterisation - query token type s has its own W_Q[s].
 *   - ReST reading note, section 3.5 (shared-prefix serving): H is computed
 *       once per request and all N candidates' query tokens are decoded
 *       against that one memory.
 *   - TransX technical report (paper-daily), section 2: the behaviour memory
 *       is turned into separate keys and values that each candidate's query
 *       cross-attends; here K and V are inputs (separate-K/V mode).
 *
 * Readings where the pages leave a step open:
 *   - multi-head split: head h uses feature columns [h*d_h, (h+1)*d_h) of
 *     Z W_Q, of K and of V; d_h = d / heads; the score scale is 1/sqrt(d_h);
 *   - query row numbering: candidate c's slot s is row c*q + s, slot s uses
 *     W_Q[s];
 *   - weight storage: wt[s][o][i] holds W_Q[s] of Eq. (7) at (i, o), i.e.
 *     Q[row][o] = sum_i Z[row][i] * wt[s][o][i]  (output-major storage);
 *   - a request with no memory rows (L_r = 0) yields all-zero output rows;
 *   - no mask: every query row of request r sees all L_r memory rows.
 *
 * Parity pins for every function are in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

/* Request that owns query row `row`: cu_cand[r]*q <= row < cu_cand[r+1]*q. */
static int request_of_row(int R, const int *cu_cand, int q, long row)
{
    for (int r = 0; r < R; ++r)
        if ((long)cu_cand[r] * q <= row && row < (long)cu_cand[r + 1] * q)
            return r;
    return -1;
}

static int check_offsets(int R, const int *cu)
{
    if (cu[0] != 0)
        return 0;
    for (int r = 0; r < R; ++r)
        if (cu[r + 1] < cu[r])
            return 0;
    return 1;
}

/*
 * TSP query projection, Eq. (8) applied to W_Q of Eq. (7):
 *   Q[row][o] = sum_{i<d} Z[row][i] * wt[row % q][o][i]
 * Z: [n_rows][d], wt: [q][d][d], Q: [n_rows][d].
 */
int oracle_project(long n_rows, int q, int d, const double *Z,
                   const double *wt, double *Q)
{
    if (n_rows < 0 || q < 1 || d < 1 || !Z || !wt || !Q)
        return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (long row = 0; row < n_rows; ++row) {
        const double *w = wt + (size_t)(row % q) * d * d;
        for (int o = 0; o < d; ++o) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i)
                acc += Z[(size_t)row * d + i] * w[(size_t)o * d + i];
            Q[(size_t)row * d + o] = acc;
        }
    }
    return ORACLE_OK;
}

/*
 * Output gate and output projection of Eq. (7) (ReST reading note, section
 * 3.3.1), with the gate projection token-specific (section 3.3.2, Eq. (8):
 * W_go is one of the candidate-side transforms that get per-slot weights;
 * W_o is not listed among them and is shared by all slots):
 *   G[row][o] = sigmoid( sum_{i<d} Z[row][i] * wgo[row % q][o][i] )
 *   Y[row][p] = sum_{o<d} ( O[row][o] * G[row][o] ) * wo[p][o]
 * O is the concatenated multi-head attention output of the same rows.
 * Weights are stored output-major like W_Q.  Z, O, Y: [n_rows][d];
 * wgo: [q][d][d]; wo: [d][d].
 */
int oracle_output(long n_rows, int q, int d, const double *Z, const double *wgo,
                  const double *O, const double *wo, double *Y)
{
    if (n_rows < 0 || q < 1 || d < 1 || !Z || !wgo || !O || !wo || !Y)
        return ORACLE_EINVAL;
#pragma omp parallel
    {
        double *x = malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(static)
        for (long row = 0; row < n_rows; ++row) {
            const double *w = wgo + (size_t)(row % q) * d * d;
            for (int o = 0; o < d; ++o) {
                double acc = 0.0;
                for (int i = 0; i < d; ++i)
                    acc += Z[(size_t)row * d + i] * w[(size_t)o * d + i];
                x[o] = O[(size_t)row * d + o] / (1.0 + exp(-acc));
            }
            for (int p = 0; p < d; ++p) {
                double acc = 0.0;
                for (int o = 0; o < d; ++o)
                    acc += x[o] * wo[(size_t)p * d + o];
                Y[(size_t)row * d + p] = acc;
            }
        }
        free(x);
    }
    return ORACLE_OK;
}

/*
 * Softmax weights of one (query row, head) over its request's memory rows:
 *   p[j] = exp(s_j - max_k s_k) / sum_k exp(s_k - max_k s_k),
 *   s_j  = <Q[row, head cols], K[kv0 + j, head cols]> / sqrt(d_h).
 * `qrow` is the projected query row (d values).  Writes L values to p.
 */
static void softmax_weights(const double *qrow, const double *K, int d,
                            int d_h, int head, int kv0, int L, double *p)
{
    const double scale = 1.0 / sqrt((double)d_h);
    double m = -INFINITY;
    for (int j = 0; j < L; ++j) {
        double s = 0.0;
        for (int e = 0; e < d_h; ++e)
            s += qrow[head * d_h + e] * K[(size_t)(kv0 + j) * d + head * d_h + e];
        p[j] = s * scale;
        if (p[j] > m)
            m = p[j];
    }
    double z = 0.0;
    for (int j = 0; j < L; ++j) {
        p[j] = exp(p[j] - m);
        z += p[j];
    }
    for (int j = 0; j < L; ++j)
        p[j] /= z;
}

/*
 * Cross-attention output, Eq. (7) up to (not including) the output gate and
 * W_o, for the query rows listed in `rows` (or every row when rows == NULL).
 *   O[k][h*d_h + e] = sum_j p_{row,h}[j] * V[kv0 + j][h*d_h + e]
 * with V = K when V == NULL (projection-free K/V).
 * Z: [total_cand*q][d]; K, V: [cu_kv[R]][d]; O: [n_out][d] where
 * n_out = n_rows if rows != NULL else total_cand*q.
 */
/*
 * Shared body of oracle_forward and oracle_forward_prefix.  kv_len (one int
 * per candidate, or NULL) restricts candidate c to the first
 * min(max(kv_len[c], 0), L_r) memory rows of its request: the prefix-valid
 * reading of the per-candidate cutoff (ReST reading note, section 3.5, ULT:
 * each sample sees only the part of its user's sequence that precedes it).
 * A candidate with no visible row gets zeros, like a request with L_r = 0.
 */
static int forward_impl(int R, const int *cu_kv, const int *cu_cand, int q, int d,
                        int heads, const double *Z, const double *wt,
                        const double *K, const double *V, const int *kv_len,
                        const long *rows, long n_rows, double *O)
{
    if (R < 0 || q < 1 || d < 1 || heads < 1 || d % heads != 0 || !cu_kv ||
        !cu_cand || !Z || !wt || !K || !O)
        return ORACLE_EINVAL;
    if (!check_offsets(R, cu_kv) || !check_offsets(R, cu_cand))
        return ORACLE_EINVAL;
    const int d_h = d / heads;
    const double *Vm = V ? V : K;
    const long total_rows = (long)cu_cand[R] * q;
    const long n_out = rows ? n_rows : total_rows;
    int max_L = 0;
    for (int r = 0; r < R; ++r)
        if (cu_kv[r + 1] - cu_kv[r] > max_L)
            max_L = cu_kv[r + 1] - cu_kv[r];
    if (rows)
        for (long k = 0; k < n_rows; ++k)
            if (rows[k] < 0 || rows[k] >= total_rows)
                return ORACLE_EINVAL;

    int bad = 0;
#pragma omp parallel
    {
        double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
        double *p = (double *)malloc(sizeof(double) * (size_t)(max_L > 0 ? max_L : 1));
        if (!qrow || !p) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (long k = 0; k < n_out; ++k) {
                const long row = rows ? rows[k] : k;
                const int r = request_of_row(R, cu_cand, q, row);
                const int kv0 = cu_kv[r], L = cu_kv[r + 1] - cu_kv[r];
                /* visible memory rows of this row's candidate */
                int Lc = L;
                if (kv_len) {
                    const int want = kv_len[row / q];
                    Lc = want < 0 ? 0 : (want < L ? want : L);
                }
                /* Q = Z W_Q[slot] for this row (Eq. (7) with Eq. (8)). */
                const double *w = wt + (size_t)(row % q) * d * d;
                for (int o = 0; o < d; ++o) {
                    double acc = 0.0;
                    for (int i = 0; i < d; ++i)
                        acc += Z[(size_t)row * d + i] * w[(size_t)o * d + i];
                    qrow[o] = acc;
                }
                for (int h = 0; h < heads; ++h) {
                    double *out = O + (size_t)k * d + h * d_h;
                    if (Lc == 0) {
                        for (int e = 0; e < d_h; ++e)
                            out[e] = 0.0;
                        continue;
                    }
                    softmax_weights(qrow, K, d, d_h, h, kv0, Lc, p);
                    for (int e = 0; e < d_h; ++e) {
                        double acc = 0.0;
                        for (int j = 0; j < Lc; ++j)
                            acc += p[j] * Vm[(size_t)(kv0 + j) * d + h * d_h + e];
                        out[e] = acc;
                    }
                }
            }
        }
        free(qrow);
        free(p);
    }
    return bad ? ORACLE_EINVAL : ORACLE_OK;
}

int oracle_forward(int R, const int *cu_kv, const int *cu_cand, int q, int d,
                   int heads, const double *Z, const double *wt,
                   const double *K, const double *V, const long *rows,
                   long n_rows, double *O)
{
    return forward_impl(R, cu_kv, cu_cand, q, d, heads, Z, wt, K, V, NULL, rows,
                        n_rows, O);
}

/* Forward with a per-candidate prefix cutoff kv_len[total_cand] (see
 * forward_impl). */
int oracle_forward_prefix(int R, const int *cu_kv, const int *cu_cand, int q, int d,
                          int heads, const double *Z, const double *wt,
                          const double *K, const double *V, const int *kv_len,
                          const long *rows, long n_rows, double *O)
{
    if (!kv_len)
        return ORACLE_EINVAL;
    return forward_impl(R, cu_kv, cu_cand, q, d, heads, Z, wt, K, V, kv_len, rows,
                        n_rows, O);
}

/*
 * Softmax weights of query row `row`, head `head` (debug / pin helper).
 * Writes L_r values into p (caller sizes p to at least L_r).
 */
int oracle_probs(int R, const int *cu_kv, const int *cu_cand, int q, int d,
                 int heads, const double *Z, const double *wt, const double *K,
                 long row, int head, double *p)
{
    if (R < 0 || q < 1 || d < 1 || heads < 1 || d % heads != 0 || !p)
        return ORACLE_EINVAL;
    if (!check_offsets(R, cu_kv) || !check_offsets(R, cu_cand))
        return ORACLE_EINVAL;
    if (row < 0 || row >= (long)cu_cand[R] * q || head < 0 || head >= heads)
        return ORACLE_EINVAL;
    const int d_h = d / heads;
    const int r = request_of_row(R, cu_cand, q, row);
    const int kv0 = cu_kv[r], L = cu_kv[r + 1] - cu_kv[r];
    double *qrow = (double *)malloc(sizeof(double) * (size_t)d);
    if (!qrow)
        return ORACLE_EINVAL;
    const double *w = wt + (size_t)(row % q) * d * d;
    for (int o = 0; o < d; ++o) {
        double acc = 0.0;
        for (int i = 0; i < d; ++i)
            acc += Z[(size_t)row * d + i] * w[(size_t)o * d + i];
        qrow[o] = acc;
    }
    if (L > 0)
        softmax_weights(qrow, K, d, d_h, head, kv0, L, p);
    free(qrow);
    return ORACLE_OK;
}

/*
 * Varlen plan (integer).  Ragged requests are packed with no padding, the
 * property the pages rely on for variable-length batches (ReST reading note
 * section 5.5: padding removal; HELIX card: padding-free variable-length
 * execution; TransX section 2: per-request memory sent to that request's
 * candidates).
 *
 *   cu_q[r]      = q * cu_cand[r]                              (r = 0..R)
 *   row_req[row] = r  for cu_q[r] <= row < cu_q[r+1]
 *   tiles        = work items {r, s, c0, nc}: candidates [c0, c0+nc) of
 *                  request r, query slot s, nc <= tile_m.  Every (row) is
 *                  covered exactly once.
 *   order        = requests by memory length L_r descending, ties by r
 *                  ascending (longest-processing-time first, since a tile's
 *                  cost is proportional to L_r); inside a request, candidate
 *                  blocks in ascending order and, per block, slots 0..q-1.
 *                  Requests with no candidates contribute no tiles.
 * row_req may be NULL.  tiles holds 4 ints per tile; max_tiles bounds it.
 */
int oracle_plan(int R, const int *cu_kv, const int *cu_cand, int q, int tile_m,
                int *cu_q, int *row_req, int *tiles, long max_tiles,
                long *n_tiles)
{
    if (R < 0 || q < 1 || tile_m < 1 || !cu_kv || !cu_cand || !cu_q || !n_tiles)
        return ORACLE_EINVAL;
    if (!check_offsets(R, cu_kv) || !check_offsets(R, cu_cand))
        return ORACLE_EINVAL;
    for (int r = 0; r <= R; ++r)
        cu_q[r] = q * cu_cand[r];
    if (row_req)
        for (int r = 0; r < R; ++r)
            for (long row = cu_q[r]; row < cu_q[r + 1]; ++row)
                row_req[row] = r;

    /* Order requests: selection by (L desc, r asc), written out plainly. */
    int *order = (int *)malloc(sizeof(int) * (size_t)(R > 0 ? R : 1));
    char *taken = (char *)calloc((size_t)(R > 0 ? R : 1), 1);
    if (!order || !taken) {
        free(order);
        free(taken);
        return ORACLE_EINVAL;
    }
    for (int k = 0; k < R; ++k) {
        int best = -1;
        for (int r = 0; r < R; ++r) {
            if (taken[r])
                continue;
            const int L = cu_kv[r + 1] - cu_kv[r];
            if (best < 0 || L > cu_kv[best + 1] - cu_kv[best])
                best = r;
        }
        taken[best] = 1;
        order[k] = best;
    }

    long n = 0;
    for (int k = 0; k < R; ++k) {
        const int r = order[k];
        const int N = cu_cand[r + 1] - cu_cand[r];
        for (int b = 0; b * tile_m < N; ++b)
            for (int s = 0; s < q; ++s) {
                if (tiles) {
                    if (n >= max_tiles) {
                        free(order);
                        free(taken);
                        return ORACLE_EINVAL;
                    }
                    tiles[4 * n + 0] = r;
                    tiles[4 * n + 1] = s;
                    tiles[4 * n + 2] = cu_cand[r] + b * tile_m;
                    tiles[4 * n + 3] = (N - b * tile_m < tile_m) ? N - b * tile_m : tile_m;
                }
                ++n;
            }
    }
    *n_tiles = n;
    free(order);
    free(taken);
    return ORACLE_OK;
}

/*
 * Backward pass of the cross-attention (NEXT-2): the gradients of the scalar
 * <dO, O(Z, W_Q, K, V)> with respect to Z, W_Q, K and V, where O is
 * forward_impl's output (same readings, same optional prefix cutoff kv_len).
 * Under projection-free K/V (V == NULL) the memory H is both key and value,
 * so its gradient is the sum of both roles; summed over every query row of
 * the request, this is the TransX report's "candidate gradients sum back into
 * the one encoding" (section 2, trajectory packing; ReST reading note
 * section 3.5, ULT).
 *
 * Chain rule for one query row i of request r and head h (q_i, k_j, v_j, o_i
 * the head slices, c = 1/sqrt(d_h), j over the row's visible memory rows):
 *   s_ij = c <q_i, k_j>,  p_ij = exp(s_ij) / sum_k exp(s_ik),  o_i = sum_j p_ij v_j
 *   dv_j  += p_ij do_i
 *   dp_ij  = <do_i, v_j>
 *   ds_ij  = sum_k dp_ik * (d p_ik / d s_ij) = p_ij (dp_ij - sum_k p_ik dp_ik)
 *            (softmax Jacobian: d p_ik / d s_ij = p_ik (delta_kj - p_ij))
 *   dq_i   = c sum_j ds_ij k_j
 *   dk_j  += c ds_ij q_i
 * then, through the projection Q[row][o] = sum_i Z[row][i] wt[s][o][i]:
 *   dZ[row][i]   = sum_o dQ[row][o] wt[row % q][o][i]
 *   dwt[s][o][i] = sum over rows of slot s of dQ[row][o] Z[row][i]
 *
 * Z, dZ, dO, dQ: [total_cand*q][d]; wt, dwt: [q][d][d] (output-major, like
 * wt); K, dK: [total_kv][d] (dK is dH when V == NULL); V, dV: [total_kv][d]
 * (dV must be NULL when V is).  dQ may be NULL.  Memory rows no query row
 * sees get zero gradients.  Accumulation order is fixed (rows ascending), so
 * the result does not depend on the thread count.
 */
int oracle_backward(int R, const int *cu_kv, const int *cu_cand, int q, int d,
                    int heads, const double *Z, const double *wt, const double *K,
                    const double *V, const int *kv_len, const double *dO, double *dQ,
                    double *dZ, double *dwt, double *dK, double *dV)
{
    if (R < 0 || q < 1 || d < 1 || heads < 1 || d % heads != 0 || !cu_kv ||
        !cu_cand || !Z || !wt || !K || !dO || !dZ || !dwt || !dK)
        return ORACLE_EINVAL;
    if ((V == NULL) != (dV == NULL))
        return ORACLE_EINVAL;
    if (!check_offsets(R, cu_kv) || !check_offsets(R, cu_cand))
        return ORACLE_EINVAL;
    const int d_h = d / heads;
    const double c = 1.0 / sqrt((double)d_h);
    const double *Vm = V ? V : K;
    const long total_rows = (long)cu_cand[R] * q;
    const long total_kv = cu_kv[R];
    int max_L = 0;
    for (int r = 0; r < R; ++r)
        if (cu_kv[r + 1] - cu_kv[r] > max_L)
            max_L = cu_kv[r + 1] - cu_kv[r];

    double *Q = (double *)malloc(sizeof(double) * (size_t)(total_rows > 0 ? total_rows : 1) * d);
    double *gQ = dQ ? dQ : (double *)malloc(sizeof(double) * (size_t)(total_rows > 0 ? total_rows : 1) * d);
    /* key-role and value-role gradients kept apart until the end */
    double *gK = (double *)calloc((size_t)(total_kv > 0 ? total_kv : 1) * d, sizeof(double));
    double *gV = (double *)calloc((size_t)(total_kv > 0 ? total_kv : 1) * d, sizeof(double));
    if (!Q || !gQ || !gK || !gV) {
        free(Q);
        if (!dQ)
            free(gQ);
        free(gK);
        free(gV);
        return ORACLE_EINVAL;
    }
    if (oracle_project(total_rows, q, d, Z, wt, Q) != ORACLE_OK) {
        free(Q);
        if (!dQ)
            free(gQ);
        free(gK);
        free(gV);
        return ORACLE_EINVAL;
    }

    int bad = 0;
    /* one task per (request, head): it owns that head's columns of the
     * request's query rows and memory rows, so tasks never share an output */
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(max_L > 0 ? max_L : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(max_L > 0 ? max_L : 1));
        if (!p || !dp) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic)
            for (long task = 0; task < (long)R * heads; ++task) {
                const int r = (int)(task / heads), h = (int)(task % heads);
                const int kv0 = cu_kv[r], L = cu_kv[r + 1] - cu_kv[r];
                for (long row = (long)cu_cand[r] * q; row < (long)cu_cand[r + 1] * q; ++row) {
                    const double *qi = Q + (size_t)row * d + h * d_h;
                    const double *doi = dO + (size_t)row * d + h * d_h;
                    double *dqi = gQ + (size_t)row * d + h * d_h;
                    for (int e = 0; e < d_h; ++e)
                        dqi[e] = 0.0;
                    int Lc = L;
                    if (kv_len) {
                        const int want = kv_len[row / q];
                        Lc = want < 0 ? 0 : (want < L ? want : L);
                    }
                    if (Lc == 0)
                        continue;   /* the output row is the constant 0 */
                    softmax_weights(Q + (size_t)row * d, K, d, d_h, h, kv0, Lc, p);
                    double pdp = 0.0;
                    for (int j = 0; j < Lc; ++j) {
                        const double *vj = Vm + (size_t)(kv0 + j) * d + h * d_h;
                        double a = 0.0;
                        for (int e = 0; e < d_h; ++e)
                            a += doi[e] * vj[e];
                        dp[j] = a;
                        pdp += p[j] * a;
                    }
                    for (int j = 0; j < Lc; ++j) {
                        const double ds = p[j] * (dp[j] - pdp);
                        const double *kj = K + (size_t)(kv0 + j) * d + h * d_h;
                        double *gkj = gK + (size_t)(kv0 + j) * d + h * d_h;
                        double *gvj = gV + (size_t)(kv0 + j) * d + h * d_h;
                        for (int e = 0; e < d_h; ++e) {
                            dqi[e] += c * ds * kj[e];
                            gkj[e] += c * ds * qi[e];
                            gvj[e] += p[j] * doi[e];
                        }
                    }
                }
            }
        }
        free(p);
        free(dp);
    }

    /* through the projection */
#pragma omp parallel for schedule(static)
    for (long row = 0; row < total_rows; ++row) {
        const double *w = wt + (size_t)(row % q) * d * d;
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int o = 0; o < d; ++o)
                acc += gQ[(size_t)row * d + o] * w[(size_t)o * d + i];
            dZ[(size_t)row * d + i] = acc;
        }
    }
#pragma omp parallel for schedule(static)
    for (long so = 0; so < (long)q * d; ++so) {
        const int s = (int)(so / d), o = (int)(so % d);
        double *out = dwt + (size_t)s * d * d + (size_t)o * d;
        for (int i = 0; i < d; ++i)
            out[i] = 0.0;
        for (long row = s; row < total_rows; row += q) {
            const double g = gQ[(size_t)row * d + o];
            for (int i = 0; i < d; ++i)
                out[i] += g * Z[(size_t)row * d + i];
        }
    }

    /* memory gradients: separate roles, or both roles of H summed */
    for (long k = 0; k < total_kv * d; ++k) {
        if (V) {
            dK[k] = gK[k];
            dV[k] = gV[k];
        } else {
            dK[k] = gK[k] + gV[k];
        }
    }
    free(Q);
    if (!dQ)
        free(gQ);
    free(gK);
    free(gV);
    return bad ? ORACLE_EINVAL : ORACLE_OK;
}
