/*
 * oracle.c -- plain CPU oracle for speculative-decoding draft verification.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load this file's library. The GPU library neither links
 * nor calls it, and the two share no source, header, table or helper.
 *
 * Source of every rule below: the web page "大模型投机解码：Medusa、MTP、EAGLE、
 * DFlash、DDTree 与 DSpark" (chzhyang.github.io), cited as [SD §n]:
 *   [SD §1]  what speculative decoding guarantees: acceptance probability
 *            alpha = min(1, p/q) (the displayed equation), everything after the
 *            first rejection is dropped (the A B C D example), the correction
 *            token comes from the normalised positive residual [p - q]+, an
 *            extra token comes from p when every draft passes, greedy results
 *            follow the target argmax, and temperature / truncation must be
 *            folded into both p and q.
 *   [SD §2]  cost model: A excludes the correction / extra token.
 *   [SD §5 DDTree]  factorised score Q(u) = prod_i q_i(u_i) (displayed
 *            equation), best-first selection of prefixes under a node budget,
 *            a walk that follows the target's token and stops at the first node
 *            with no matching child, whose target token becomes the extra token.
 *   [SD §5 DSpark]  prefix survival s_j = prod_{i<=j} c_i and expected advance
 *            1 + sum_{j<=k} s_j for verify length k.
 *
 * Plain scalar loops, fp64 arithmetic. Two quantities are computed in fp32
 * because an fp32 rounding decides an ordering and both sides must take the
 * same integer decision: the tree score Q (fp32 product, left to right in depth
 * order) and the prefix survival s_j (fp32 running product). OpenMP is used only
 * across independent sequences; it changes no arithmetic.
 *
 * Readings where the page leaves a step open (each one is listed in the design
 * notes of the repository):
 *   - uniforms: per sequence K+1 of them; u_i drives accept test i, u_k drives
 *     the one final sample (correction or extra token);
 *   - accept iff p(y) > 0 and u*q(y) <= p(y);
 *   - inverse CDF in token-id order: the first j whose running mass exceeds
 *     the scaled uniform;
 *   - top-k keeps exactly k ids, ordered by (logit desc, id asc) on the raw
 *     logits; NaN logits are never kept;
 *   - T == 0 means greedy;
 *   - a row whose kept logits have no finite maximum, or whose exponential sum
 *     is not a finite positive number, is "non-finite": all its probabilities
 *     are 0 and the sequence is flagged;
 *   - tree ties: (Q desc, depth asc, rank tuple lexicographic asc);
 *   - verify length: the smallest k maximising 1 + sum_{j<=k} s_j - cost*k.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BAD_TOKEN 1
#define ORC_NONFINITE 2
#define ORC_MARGIN_ACCEPT 1
#define ORC_MARGIN_SAMPLE 2

int orc_version(void) { return 1; }

/* ------------------------------------------------------------------------ */
/* Top-k ordering: (logit desc, id asc).                                     */
/* ------------------------------------------------------------------------ */
typedef struct { double x; int id; } orc_key;

static int orc_cmp_desc(const void* a, const void* b) {
    const orc_key* p = (const orc_key*)a;
    const orc_key* q = (const orc_key*)b;
    if (p->x > q->x) return -1;
    if (p->x < q->x) return 1;
    return (p->id < q->id) ? -1 : (p->id > q->id);
}

/*
 * Distribution shaping [SD §1: temperature and truncation belong inside p and q].
 * p[t] = exp(z_t - m) / sum_{s in S} exp(z_s - m) for t in S, 0 elsewhere, where
 * z = x / T and S is the kept set (all ids, or the first top_k ids under
 * (x desc, id asc), NaN never kept). Returns 1 for a valid row, 0 for a
 * non-finite one (then p is all zeros).
 */
int orc_transform_row(const float* logits, int V, double T, int top_k, double* p) {
    unsigned char* keep = (unsigned char*)calloc((size_t)V, 1);
    if (top_k >= 1 && top_k < V) {
        orc_key* ks = (orc_key*)malloc(sizeof(orc_key) * (size_t)V);
        int n = 0;
        for (int t = 0; t < V; ++t) {
            double x = (double)logits[t];
            if (isnan(x)) continue;
            ks[n].x = x; ks[n].id = t; ++n;
        }
        qsort(ks, (size_t)n, sizeof(orc_key), orc_cmp_desc);
        int take = n < top_k ? n : top_k;
        for (int r = 0; r < take; ++r) keep[ks[r].id] = 1;
        free(ks);
    } else {
        for (int t = 0; t < V; ++t) keep[t] = 1;
    }
    double m = -INFINITY;
    int any = 0;
    for (int t = 0; t < V; ++t) {
        if (!keep[t]) continue;
        double z = (double)logits[t] / T;
        if (!any || z > m) m = z;           /* NaN never raises m */
        any = 1;
    }
    for (int t = 0; t < V; ++t) p[t] = 0.0;
    int valid = any && isfinite(m);
    if (valid) {
        double S = 0.0;
        for (int t = 0; t < V; ++t) {
            if (!keep[t]) continue;
            double e = exp((double)logits[t] / T - m);
            p[t] = e;
            S += e;
        }
        if (!(isfinite(S) && S > 0.0)) {
            valid = 0;
        } else {
            for (int t = 0; t < V; ++t) p[t] /= S;
        }
        if (!valid) for (int t = 0; t < V; ++t) p[t] = 0.0;
    }
    free(keep);
    return valid;
}

/*
 * Greedy choice [SD §1: greedy results follow the target argmax]: the lowest id
 * among the maxima of the raw logits, NaN ignored; -1 if every entry is NaN.
 */
int orc_argmax_row(const float* logits, int V) {
    int best = -1;
    double bx = 0.0;
    for (int t = 0; t < V; ++t) {
        double x = (double)logits[t];
        if (isnan(x)) continue;
        if (best < 0 || x > bx) { best = t; bx = x; }
    }
    return best;
}

/*
 * Inverse CDF in token-id order: the first j with sum_{t<=j} w_t > target
 * (target >= 0, so that j always carries positive mass). If rounding leaves the
 * total at or below target, the last j with w_j > 0.
 * Returns -1 if w has no positive entry. *margin is set when target lies within
 * tol of the running mass just before or just after the chosen token.
 */
static int orc_inverse_cdf(const double* w, int V, double target, double tol, int* margin) {
    double C = 0.0;
    int last_pos = -1;
    for (int j = 0; j < V; ++j) {
        double prev = C;
        C += w[j];
        if (w[j] > 0.0) last_pos = j;
        if (C > target) {
            if (fabs(target - prev) < tol || fabs(target - C) < tol) *margin = 1;
            return j;
        }
    }
    if (last_pos >= 0) *margin = 1;     /* reached only through rounding */
    return last_pos;
}

/*
 * Stochastic chain verification [SD §1].
 *
 * Layout: sequence b has k_b = cu[b+1]-cu[b] draft positions (k_b = K_max for
 * every b when cu == NULL, with cu[b] = b*K_max). Draft row i of b is draft row
 * cu[b]+i; target row i is target row cu[b]+b+i for i = 0..k_b (row k_b is the
 * extra-token row). uniforms[cu[b]+b+i] drives accept test i; uniforms[cu[b]+b+k_b]
 * drives the final sample.
 *
 * Per sequence:
 *   acc_i = p_i(y_i) > 0 && u_i q_i(y_i) <= p_i(y_i)   (the ratio test alpha = min(1, p/q))
 *   A     = first i with !acc_i, else k                 (nothing after a rejection is kept)
 *   A < k: r = max(p_A - q_A, 0), R = sum r, next = inverse CDF of r at u_k R
 *          (if R == 0 through rounding: inverse CDF of p_A at u_k)
 *   A = k: next = inverse CDF of p_k at u_k             (the extra token)
 * T == 0 selects the greedy rule of orc_verify_greedy.
 *
 * Outputs: A_out[b], next_out[b] (-1 if no token can be drawn), probs_out[2*r]
 * = (p_i(y_i), q_i(y_i)) for every draft row r (NULL to skip), R_out[b] (0 for the
 * extra token), status_out[b] (ORC_BAD_TOKEN / ORC_NONFINITE bits, raised only by
 * positions 0..A and the row the final token is drawn from), margin_out[b]
 * (ORC_MARGIN_* bits: an accept test with |u q - p| < margin_rel * p, or a
 * sampled token whose scaled uniform lies within margin_rel * total of a CDF step).
 */
void orc_verify_chain(const float* target, const float* draft, const int32_t* tokens,
                      const float* uniforms, const int32_t* cu, int B, int K_max, int V,
                      double T, int top_k, double margin_rel,
                      int32_t* A_out, int32_t* next_out, double* probs_out, double* R_out,
                      int32_t* status_out, int32_t* margin_out, int nthreads) {
    (void)nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int b = 0; b < B; ++b) {
        int d0 = cu ? cu[b] : b * K_max;
        int k = cu ? cu[b + 1] - cu[b] : K_max;
        int t0 = d0 + b;
        int status = 0, margin = 0;
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        double* q = (double*)malloc(sizeof(double) * (size_t)V);
        double* r = (double*)malloc(sizeof(double) * (size_t)V);
        int A = k;
        int next = -1;
        double Rm = 0.0;

        if (T == 0.0) {
            /* greedy semantics */
            for (int i = 0; i < k; ++i) {
                int g = orc_argmax_row(target + (size_t)(t0 + i) * V, V);
                int y = tokens[d0 + i];
                if (probs_out) { probs_out[2 * (d0 + i)] = 0.0; probs_out[2 * (d0 + i) + 1] = 0.0; }
                if (A == k) {
                    if (y < 0 || y >= V) status |= ORC_BAD_TOKEN;
                    if (g < 0) status |= ORC_NONFINITE;
                    if (!(g >= 0 && y == g)) A = i;
                }
            }
            next = orc_argmax_row(target + (size_t)(t0 + A) * V, V);
            if (next < 0) status |= ORC_NONFINITE;
        } else {
            double u_fin = (double)uniforms[t0 + k];
            int acc_done = 0;
            for (int i = 0; i < k; ++i) {
                int vp = orc_transform_row(target + (size_t)(t0 + i) * V, V, T, top_k, p);
                int vq = orc_transform_row(draft + (size_t)(d0 + i) * V, V, T, top_k, q);
                int y = tokens[d0 + i];
                int yok = (y >= 0 && y < V);
                double py = yok ? p[y] : 0.0, qy = yok ? q[y] : 0.0;
                if (probs_out) { probs_out[2 * (d0 + i)] = py; probs_out[2 * (d0 + i) + 1] = qy; }
                if (acc_done) continue;
                double u = (double)uniforms[t0 + i];
                int acc = vp && vq && yok && py > 0.0 && u * qy <= py;
                if (!yok) status |= ORC_BAD_TOKEN;
                if (!vp || !vq) status |= ORC_NONFINITE;
                if (vp && vq && yok && py > 0.0 && fabs(u * qy - py) < margin_rel * py)
                    margin |= ORC_MARGIN_ACCEPT;
                if (!acc) {
                    A = i;
                    acc_done = 1;
                    /* residual at the first rejection */
                    double R = 0.0;
                    if (!vp) {
                        next = -1;
                    } else {
                        for (int t = 0; t < V; ++t) {
                            double qt = vq ? q[t] : 0.0;
                            double d = p[t] - qt;
                            r[t] = d > 0.0 ? d : 0.0;
                            R += r[t];
                        }
                        int mg = 0;
                        if (R > 0.0) {
                            next = orc_inverse_cdf(r, V, u_fin * R, margin_rel * R, &mg);
                        } else {
                            next = orc_inverse_cdf(p, V, u_fin, margin_rel, &mg);
                        }
                        if (mg) margin |= ORC_MARGIN_SAMPLE;
                    }
                    Rm = R;
                }
            }
            if (A == k) {
                int vp = orc_transform_row(target + (size_t)(t0 + k) * V, V, T, top_k, p);
                if (!vp) {
                    status |= ORC_NONFINITE;
                    next = -1;
                } else {
                    int mg = 0;
                    next = orc_inverse_cdf(p, V, u_fin, margin_rel, &mg);
                    if (mg) margin |= ORC_MARGIN_SAMPLE;
                }
                Rm = 0.0;
            }
        }
        A_out[b] = A;
        next_out[b] = next;
        if (R_out) R_out[b] = Rm;
        if (status_out) status_out[b] = status;
        if (margin_out) margin_out[b] = margin;
        free(p); free(q); free(r);
    }
}

/*
 * Cap-accept verification [SD §9 DSpark: the full window is verified, the
 * committed length is limited]. Padded layout (sequence b: target rows
 * b*(K+1) .. b*(K+1)+K, draft rows b*K .., uniforms as the target rows). The
 * committed result is the chain verification of the first kc = clamp(cap[b],
 * 0, K) positions (uniforms 0..kc-1 for the tests, uniform kc for the final
 * draw); A_full_out[b] is the first rejection over all K positions. Both are
 * plain calls of orc_verify_chain on one sequence; probs_out ([B*K, 2]) covers
 * the whole window.
 */
void orc_verify_chain_capped(const float* target, const float* draft, const int32_t* tokens,
                             const float* uniforms, const int32_t* cap, int B, int K, int V,
                             double T, int top_k, double margin_rel, int32_t* A_out,
                             int32_t* next_out, int32_t* A_full_out, double* probs_out,
                             double* R_out, int32_t* status_out, int32_t* margin_out,
                             int nthreads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int b = 0; b < B; ++b) {
        const float* tw = target + (size_t)b * (K + 1) * V;
        const float* dw = draft + (size_t)b * K * V;
        const int32_t* yw = tokens + (size_t)b * K;
        const float* uw = uniforms + (size_t)b * (K + 1);
        int kc = cap[b] < 0 ? 0 : (cap[b] > K ? K : cap[b]);
        int32_t cu_c[2] = {0, kc}, cu_f[2] = {0, K};
        int32_t A_f, next_f, st_f, mg_f;
        double R_f;
        /* the whole window: A over all K positions, and every p(y), q(y) */
        orc_verify_chain(tw, dw, yw, uw, cu_f, 1, K, V, T, top_k, margin_rel, &A_f, &next_f,
                         probs_out ? probs_out + (size_t)2 * b * K : NULL, &R_f, &st_f, &mg_f, 1);
        /* the committed part: the first kc positions */
        orc_verify_chain(tw, dw, yw, uw, cu_c, 1, kc, V, T, top_k, margin_rel, A_out + b,
                         next_out + b, NULL, R_out ? R_out + b : NULL,
                         status_out ? status_out + b : NULL, margin_out ? margin_out + b : NULL, 1);
        A_full_out[b] = A_f;
    }
}

/*
 * Greedy chain verification [SD §1: greedy results follow the target argmax]:
 * g_i = lowest-id argmax of target row i, acc_i = (y_i == g_i), A = first
 * mismatch (else k), next = g_A. Same layout as orc_verify_chain. argmax_out
 * (optional, [R_t]) receives g for every target row.
 */
void orc_verify_greedy(const float* target, const int32_t* tokens, const int32_t* cu,
                       int B, int K_max, int V, int32_t* A_out, int32_t* next_out,
                       int32_t* status_out, int32_t* argmax_out, int nthreads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int b = 0; b < B; ++b) {
        int d0 = cu ? cu[b] : b * K_max;
        int k = cu ? cu[b + 1] - cu[b] : K_max;
        int t0 = d0 + b;
        int A = k, status = 0;
        for (int i = 0; i <= k; ++i) {
            int g = orc_argmax_row(target + (size_t)(t0 + i) * V, V);
            if (argmax_out) argmax_out[t0 + i] = g;
            if (i < k && A == k) {
                int y = tokens[d0 + i];
                if (y < 0 || y >= V) status |= ORC_BAD_TOKEN;
                if (g < 0) status |= ORC_NONFINITE;
                if (!(g >= 0 && y == g)) A = i;
            }
        }
        int next = orc_argmax_row(target + (size_t)(t0 + A) * V, V);
        if (next < 0) status |= ORC_NONFINITE;
        A_out[b] = A;
        next_out[b] = next;
        if (status_out) status_out[b] = status;
    }
}

/*
 * DDTree candidate tree [SD §5 DDTree].
 *
 * marg: [B, K, V] per-depth draft marginals (q_1 .. q_K; row d is depth d+1).
 * L_d = ids of row d sorted by (q desc, id asc), cut to N-1 entries. A prefix is
 * a tuple of ranks (r_1..r_m), m <= K, naming tokens L_1[r_1] .. L_m[r_m]; its
 * score is Q = fl32(...fl32(q_1(L_1[r_1]) * q_2(L_2[r_2]))... * q_m(L_m[r_m])).
 * Order of prefixes: Q desc, then m asc, then the rank tuple lexicographically asc.
 *
 * The tree is the root (node 0: token -1, parent -1, depth 0, score 1, mask bit 0)
 * plus the first N-1 prefixes in that order, numbered in that order. The order
 * puts every parent before its children, so the plain way to list it is a
 * frontier scan: repeatedly take the best unselected child of any selected node
 * (no heap). anc_mask[n] has bit n and the bits of all ancestors.
 * Returns nothing; n_nodes[b] is N unless the whole trie has fewer prefixes.
 */
void orc_build_tree(const float* marg, int B, int K, int V, int N,
                    int32_t* node_token, int32_t* node_parent, int32_t* node_depth,
                    float* node_score, uint64_t* node_anc, int32_t* n_nodes, int nthreads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int b = 0; b < B; ++b) {
        int W = (N - 1) < V ? (N - 1) : V;       /* candidates kept per depth */
        int* L = (int*)malloc(sizeof(int) * (size_t)K * (size_t)(W > 0 ? W : 1));
        orc_key* ks = (orc_key*)malloc(sizeof(orc_key) * (size_t)V);
        for (int d = 0; d < K; ++d) {
            const float* row = marg + ((size_t)b * K + d) * V;
            for (int t = 0; t < V; ++t) { ks[t].x = (double)row[t]; ks[t].id = t; }
            qsort(ks, (size_t)V, sizeof(orc_key), orc_cmp_desc);
            for (int r = 0; r < W; ++r) L[d * W + r] = ks[r].id;
        }
        free(ks);
        /* per node: rank tuple, score, child table */
        int* ranks = (int*)calloc((size_t)N * (size_t)(K > 0 ? K : 1), sizeof(int));
        int* child = (int*)malloc(sizeof(int) * (size_t)N * (size_t)(W > 0 ? W : 1));
        for (int i = 0; i < N * (W > 0 ? W : 1); ++i) child[i] = -1;
        int32_t* tok = node_token + (size_t)b * N;
        int32_t* par = node_parent + (size_t)b * N;
        int32_t* dep = node_depth + (size_t)b * N;
        float* sc = node_score + (size_t)b * N;
        uint64_t* an = node_anc + (size_t)b * N;
        for (int n = 0; n < N; ++n) { tok[n] = -1; par[n] = -1; dep[n] = 0; sc[n] = 0.0f; an[n] = 0; }
        tok[0] = -1; par[0] = -1; dep[0] = 0; sc[0] = 1.0f; an[0] = 1ull;
        int n = 1;
        while (n < N) {
            int bs = -1, br = -1;
            float bq = 0.0f;
            for (int s = 0; s < n; ++s) {
                int m = dep[s];
                if (m >= K) continue;
                for (int r = 0; r < W; ++r) {
                    if (child[s * W + r] >= 0) continue;
                    float qv = marg[((size_t)b * K + m) * V + L[m * W + r]];
                    float Qc = sc[s] * qv;                  /* fp32 product */
                    int better = 0;
                    if (bs < 0) better = 1;
                    else if (Qc > bq) better = 1;
                    else if (Qc == bq) {
                        int mc = m + 1, mb = dep[bs] + 1;
                        if (mc < mb) better = 1;
                        else if (mc == mb) {
                            /* lexicographic compare of (ranks[s][0..m-1], r) vs (ranks[bs][..], br) */
                            int cmp = 0;
                            for (int j = 0; j < m && cmp == 0; ++j) {
                                int a = ranks[s * K + j], c = ranks[bs * K + j];
                                cmp = (a < c) ? -1 : (a > c);
                            }
                            if (cmp == 0) cmp = (r < br) ? -1 : (r > br);
                            if (cmp < 0) better = 1;
                        }
                    }
                    if (better) { bs = s; br = r; bq = Qc; }
                }
            }
            if (bs < 0) break;                              /* trie exhausted */
            int m = dep[bs];
            for (int j = 0; j < m; ++j) ranks[n * K + j] = ranks[bs * K + j];
            ranks[n * K + m] = br;
            tok[n] = L[m * W + br];
            par[n] = bs;
            dep[n] = m + 1;
            sc[n] = bq;
            an[n] = an[bs] | (1ull << n);
            child[bs * W + br] = n;
            ++n;
        }
        n_nodes[b] = n;
        free(L); free(ranks); free(child);
    }
}

/*
 * Tree walk [SD §5 DDTree]: from the root, take the target's token g = argmax
 * of the current node's target row (lowest id on ties); if a child carries g,
 * move there and record it; otherwise g is the extra token. target: [B, N, V],
 * row n = node n. path_out: [B, N] accepted node ids, -1 padded.
 */
void orc_verify_tree(const float* target, const int32_t* node_token, const int32_t* node_parent,
                     const int32_t* n_nodes, int B, int N, int V,
                     int32_t* path_out, int32_t* A_out, int32_t* next_out, int nthreads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int b = 0; b < B; ++b) {
        const int32_t* tok = node_token + (size_t)b * N;
        const int32_t* par = node_parent + (size_t)b * N;
        int nn = n_nodes[b];
        int32_t* path = path_out + (size_t)b * N;
        for (int i = 0; i < N; ++i) path[i] = -1;
        int node = 0, len = 0, next = -1;
        for (;;) {
            int g = orc_argmax_row(target + ((size_t)b * N + node) * V, V);
            int found = -1;
            for (int c = 1; c < nn && g >= 0; ++c)
                if (par[c] == node && tok[c] == g) { found = c; break; }
            if (found < 0) { next = g; break; }
            path[len++] = found;
            node = found;
        }
        A_out[b] = len;
        next_out[b] = next;
    }
}

/*
 * Sampled tree walk [SD §5 DDTree: the walk follows the token the target
 * picks at each node, and the first node without a matching child turns that
 * token into the extra token; SD §1: temperature and truncation belong inside
 * p, and the chain's ratio test is not a rule for a tree]. The drafted tree is
 * fixed (its nodes are not samples from q), so no draft probability enters:
 * at node n the target picks its token by sampling p_n itself, the inverse
 * CDF of the transformed row n (orc_transform_row with T, top_k) at
 * uniforms[b*N + n]. Each node is visited at most once, so every pick uses a
 * fresh uniform and each committed token is a draw from the target given the
 * tokens before it. T == 0 is the argmax walk of orc_verify_tree.
 *
 * Outputs as orc_verify_tree, plus status_out[b] (ORC_NONFINITE when a
 * visited row is non-finite; the walk then stops with next = -1) and
 * margin_out[b] (ORC_MARGIN_SAMPLE when a pick's uniform lies within
 * margin_rel of a CDF step).
 */
void orc_verify_tree_sampled(const float* target, const int32_t* node_token,
                             const int32_t* node_parent, const int32_t* n_nodes,
                             const float* uniforms, int B, int N, int V, double T, int top_k,
                             double margin_rel, int32_t* path_out, int32_t* A_out,
                             int32_t* next_out, int32_t* status_out, int32_t* margin_out,
                             int nthreads) {
    if (T == 0.0) {
        orc_verify_tree(target, node_token, node_parent, n_nodes, B, N, V, path_out, A_out,
                        next_out, nthreads);
        for (int b = 0; b < B; ++b) {
            if (status_out) status_out[b] = next_out[b] < 0 ? ORC_NONFINITE : 0;
            if (margin_out) margin_out[b] = 0;
        }
        return;
    }
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int b = 0; b < B; ++b) {
        const int32_t* tok = node_token + (size_t)b * N;
        const int32_t* par = node_parent + (size_t)b * N;
        int nn = n_nodes[b];
        int32_t* path = path_out + (size_t)b * N;
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        for (int i = 0; i < N; ++i) path[i] = -1;
        int node = 0, len = 0, next = -1, status = 0, margin = 0;
        for (;;) {
            int valid = orc_transform_row(target + ((size_t)b * N + node) * V, V, T, top_k, p);
            if (!valid) {
                status |= ORC_NONFINITE;
                next = -1;
                break;
            }
            int mg = 0;
            int g = orc_inverse_cdf(p, V, (double)uniforms[(size_t)b * N + node], margin_rel, &mg);
            if (mg) margin |= ORC_MARGIN_SAMPLE;
            int found = -1;
            for (int c = 1; c < nn; ++c)
                if (par[c] == node && tok[c] == g) { found = c; break; }
            if (found < 0) { next = g; break; }
            path[len++] = found;
            node = found;
        }
        A_out[b] = len;
        next_out[b] = next;
        if (status_out) status_out[b] = status;
        if (margin_out) margin_out[b] = margin;
        free(p);
    }
}

/*
 * Verify-length choice [SD §5 DSpark]: s_0 = 1, s_j = fl32(s_{j-1} * c_j);
 * k* = the smallest k in [0, K] maximising f(k) = 1 + sum_{j<=k} s_j - cost*k
 * (f in fp64 over the fp32 s_j); expected advance 1 + sum_{j<=k*} s_j;
 * cu_sel = exclusive prefix sum of k* ([B+1], optional). margin_out[b] = 1 when
 * some |s_j - cost| < 1e-6.
 */
void orc_select_len(const float* conf, int B, int K, float cost, int32_t* k_sel,
                    double* adv_out, int32_t* cu_sel, int32_t* margin_out) {
    for (int b = 0; b < B; ++b) {
        float s = 1.0f;
        double sum = 0.0, best_f = 1.0, best_sum = 0.0;
        int best_k = 0, margin = 0;
        for (int j = 1; j <= K; ++j) {
            s = s * conf[(size_t)b * K + (j - 1)];
            sum += (double)s;
            double f = 1.0 + sum - (double)cost * (double)j;
            if (f > best_f) { best_f = f; best_k = j; best_sum = sum; }
            if (fabs((double)s - (double)cost) < 1e-6) margin = 1;
        }
        k_sel[b] = best_k;
        if (adv_out) adv_out[b] = 1.0 + best_sum;
        if (margin_out) margin_out[b] = margin;
    }
    if (cu_sel) {
        cu_sel[0] = 0;
        for (int b = 0; b < B; ++b) cu_sel[b + 1] = cu_sel[b] + k_sel[b];
    }
}

/*
 * EAGLE-2-style verification tree [SD §4 EAGLE-2: expanded candidates are
 * re-ranked by cumulative confidence and the final tree is chosen from them].
 * Candidates of sequence b (topological order, candidate 0 the root): parent,
 * token and conditional probability; candidate i is usable if 0 <= parent < i,
 * its parent is usable (the root is) and its probability lies in [0, 1]. Its
 * confidence is the fp32 product of the probabilities from the root down. The
 * tree: the root plus the first N-1 usable candidates by (confidence desc,
 * depth asc, index asc), numbered in that order.
 */
typedef struct {
    float conf;
    int depth;
    int idx;
} OrcCand;

static int orc_cand_cmp(const void* a, const void* b) {
    const OrcCand* x = (const OrcCand*)a;
    const OrcCand* y = (const OrcCand*)b;
    if (x->conf != y->conf) return x->conf > y->conf ? -1 : 1;
    if (x->depth != y->depth) return x->depth < y->depth ? -1 : 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

void orc_rerank_tree(const int32_t* cand_parent, const int32_t* cand_token, const float* cand_prob,
                     const int32_t* n_cand, int B, int M, int N, int32_t* node_token,
                     int32_t* node_parent, int32_t* node_depth, float* node_score,
                     uint64_t* node_anc, int32_t* node_cand, int32_t* n_nodes) {
    for (int b = 0; b < B; ++b) {
        const int32_t* par = cand_parent + (size_t)b * M;
        const int32_t* tok = cand_token + (size_t)b * M;
        const float* prob = cand_prob + (size_t)b * M;
        int nc = n_cand[b] < 0 ? 0 : (n_cand[b] > M ? M : n_cand[b]);
        float* conf = (float*)malloc(sizeof(float) * (size_t)(M + 1));
        int* depth = (int*)malloc(sizeof(int) * (size_t)(M + 1));
        int* usable = (int*)malloc(sizeof(int) * (size_t)(M + 1));
        int* node_of = (int*)malloc(sizeof(int) * (size_t)(M + 1));
        OrcCand* list = (OrcCand*)malloc(sizeof(OrcCand) * (size_t)(M + 1));
        int nl = 0;
        for (int i = 0; i < M; ++i) { usable[i] = 0; node_of[i] = -1; }
        if (nc > 0) { usable[0] = 1; conf[0] = 1.0f; depth[0] = 0; node_of[0] = 0; }
        for (int i = 1; i < nc; ++i) {
            int p = par[i];
            float q = prob[i];
            if (p < 0 || p >= i || !usable[p] || !(q >= 0.0f && q <= 1.0f)) continue;
            usable[i] = 1;
            conf[i] = conf[p] * q;
            depth[i] = depth[p] + 1;
            list[nl].conf = conf[i];
            list[nl].depth = depth[i];
            list[nl].idx = i;
            ++nl;
        }
        qsort(list, (size_t)nl, sizeof(OrcCand), orc_cand_cmp);
        int kept = nl < N - 1 ? nl : N - 1;
        size_t o = (size_t)b * N;
        for (int n = 0; n < N; ++n) {
            node_token[o + n] = -1; node_parent[o + n] = -1; node_depth[o + n] = 0;
            node_score[o + n] = 0.0f; node_anc[o + n] = 0; if (node_cand) node_cand[o + n] = -1;
        }
        node_score[o] = 1.0f; node_anc[o] = 1; if (node_cand) node_cand[o] = 0;
        for (int r = 0; r < kept; ++r) node_of[list[r].idx] = r + 1;
        for (int r = 0; r < kept; ++r) {
            int c = list[r].idx, n = r + 1;
            node_token[o + n] = tok[c];
            node_parent[o + n] = node_of[par[c]];
            node_depth[o + n] = depth[c];
            node_score[o + n] = conf[c];
            node_anc[o + n] = node_anc[o + node_of[par[c]]] | ((uint64_t)1 << n);
            if (node_cand) node_cand[o + n] = c;
        }
        n_nodes[b] = 1 + kept;
        free(conf); free(depth); free(usable); free(node_of); free(list);
    }
}

/*
 * Accepted-path KV compaction [SD §5 DDTree: the KV cache keeps only the
 * accepted path]. kv: n_rows rows of row_bytes bytes; draft node n (1..N-1) of
 * sequence b sits at row row_base[b] + n - 1. Afterwards row row_base[b] + i
 * holds what row row_base[b] + path[b*N + i] - 1 held before the call (i <
 * accepted_len[b]); nothing else changes. Sequences whose draft region is not
 * inside [0, n_rows) are skipped, as are path entries outside [1, N-1]. Every
 * source is read from a copy of the rows taken before any move.
 */
void orc_compact_kv(unsigned char* kv, long long row_bytes, long long n_rows,
                    const long long* row_base, const int32_t* path, const int32_t* accepted_len,
                    int B, int N) {
    unsigned char* before = (unsigned char*)malloc((size_t)(row_bytes * n_rows));
    memcpy(before, kv, (size_t)(row_bytes * n_rows));
    for (int b = 0; b < B; ++b) {
        long long r0 = row_base[b];
        int A = accepted_len[b];
        if (A < 0) A = 0;
        if (A > N - 1) A = N - 1;
        if (r0 < 0 || r0 + (N - 1) > n_rows) continue;
        for (int i = 0; i < A; ++i) {
            int n = path[(size_t)b * N + i];
            if (n < 1 || n > N - 1) continue;
            memcpy(kv + (size_t)((r0 + i) * row_bytes), before + (size_t)((r0 + n - 1) * row_bytes),
                   (size_t)row_bytes);
        }
    }
    free(before);
}

/*
 * Verify length with a per-position cost table [SD §5 DSpark: is one more
 * verified position worth its cost]: cost[j-1] is the cost of verifying
 * position j; k* = the smallest k in [0, K] maximising
 * f(k) = 1 + sum_{j<=k} s_j - sum_{j<=k} cost[j-1], both sums running in fp64
 * over the fp32 s_j and costs; expected advance 1 + sum_{j<=k*} s_j.
 * margin_out[b] = 1 when another k comes within 1e-6 of the best f.
 */
void orc_select_len_table(const float* conf, int B, int K, const float* cost, int32_t* k_sel,
                          double* adv_out, int32_t* cu_sel, int32_t* margin_out) {
    for (int b = 0; b < B; ++b) {
        float s = 1.0f;
        double sum_s = 0.0, sum_c = 0.0, best_f = 1.0, best_sum = 0.0;
        double fk[65];
        int best_k = 0, margin = 0;
        fk[0] = 1.0;
        for (int j = 1; j <= K; ++j) {
            s = s * conf[(size_t)b * K + (j - 1)];
            sum_s += (double)s;
            sum_c += (double)cost[j - 1];
            double f = 1.0 + sum_s - sum_c;
            fk[j] = f;
            if (f > best_f) { best_f = f; best_k = j; best_sum = sum_s; }
        }
        for (int j = 0; j <= K; ++j)
            if (j != best_k && fabs(fk[j] - best_f) < 1e-6) margin = 1;
        k_sel[b] = best_k;
        if (adv_out) adv_out[b] = 1.0 + best_sum;
        if (margin_out) margin_out[b] = margin;
    }
    if (cu_sel) {
        cu_sel[0] = 0;
        for (int b = 0; b < B; ++b) cu_sel[b + 1] = cu_sel[b] + k_sel[b];
    }
}

/* ------------------------------------------------------------------------ */
/* Validity checks of another implementation's results where the oracle's  */
/* own decision sits at a rounding margin. They re-evaluate the definitions */
/* above in fp64 on this oracle's p and q, at the decision the other side   */
/* took, and accept it when it is one of the results that rounding allows.  */
/* ------------------------------------------------------------------------ */

/*
 * 1 when token j is a valid inverse-CDF draw from weights w (token-id order)
 * at the scaled point x, allowing a slack of tol on the point: w_j > 0,
 * C_{j-1} <= x + tol and C_j > x - tol, with C the running sum of w.
 */
static int orc_cdf_draw_ok(const double* w, int V, int j, double x, double tol) {
    if (j < 0 || j >= V || !(w[j] > 0.0)) return 0;
    double C = 0.0;
    for (int t = 0; t < j; ++t) C += w[t];
    return C <= x + tol && C + w[j] > x - tol;
}

/*
 * Chain result check [SD §1: the ratio test alpha = min(1, p/q), nothing kept
 * after the first rejection, the correction from the normalised [p - q]+, the
 * extra token from p]. For sequence b (layout as orc_verify_chain, T > 0) and
 * the pair (A_in[b], next_in[b]) to check:
 *   bit 1 of valid_out[b]: 0 <= A <= k, every position i < A passes the test
 *          with slack, p_i(y_i) > 0 and u_i q_i(y_i) <= p_i(y_i) (1 + tol),
 *          and position A < k fails it with slack: the token or a row is bad,
 *          p_A(y_A) == 0, or u_A q_A(y_A) > p_A(y_A) (1 - tol);
 *   bit 2: next is the draw the chain rule makes at that A, within slack:
 *          the final row's weights w (the residual max(p_A - q_A, 0) with
 *          total R > 0 and point u_k R; p_A at u_k if R == 0; p_k at u_k
 *          when A == k), checked by orc_cdf_draw_ok with tol times the
 *          total; next == -1 exactly when that row is non-finite.
 * status_out[b] receives the status bits the chain rule raises at that A.
 */
void orc_check_chain(const float* target, const float* draft, const int32_t* tokens,
                     const float* uniforms, const int32_t* cu, int B, int K_max, int V, double T,
                     int top_k, double tol, const int32_t* A_in, const int32_t* next_in,
                     int32_t* valid_out, int32_t* status_out, int nthreads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int b = 0; b < B; ++b) {
        int d0 = cu ? cu[b] : b * K_max;
        int k = cu ? cu[b + 1] - cu[b] : K_max;
        int t0 = d0 + b;
        int A = A_in[b], nx = next_in[b];
        int valid = 0, status = 0;
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        double* q = (double*)malloc(sizeof(double) * (size_t)V);
        if (A >= 0 && A <= k) {
            int a_ok = 1;
            for (int i = 0; i <= A && i < k; ++i) {
                int vp = orc_transform_row(target + (size_t)(t0 + i) * V, V, T, top_k, p);
                int vq = orc_transform_row(draft + (size_t)(d0 + i) * V, V, T, top_k, q);
                int y = tokens[d0 + i];
                int yok = (y >= 0 && y < V);
                double py = yok ? p[y] : 0.0, qy = yok ? q[y] : 0.0;
                double u = (double)uniforms[t0 + i];
                int good = vp && vq && yok;
                if (!yok) status |= ORC_BAD_TOKEN;
                if (!vp || !vq) status |= ORC_NONFINITE;
                if (i < A) {
                    if (!(good && py > 0.0 && u * qy <= py * (1.0 + tol))) a_ok = 0;
                } else {
                    if (good && py > 0.0 && u * qy <= py * (1.0 - tol)) a_ok = 0;
                }
            }
            if (a_ok) valid |= 1;
            /* the final draw at this A */
            double u_fin = (double)uniforms[t0 + k];
            int row = t0 + A;
            int vp = orc_transform_row(target + (size_t)row * V, V, T, top_k, p);
            if (A == k && !vp) status |= ORC_NONFINITE;
            if (!vp) {
                if (nx == -1) valid |= 2;
            } else if (A < k) {
                int vq = orc_transform_row(draft + (size_t)(d0 + A) * V, V, T, top_k, q);
                double R = 0.0;
                for (int t = 0; t < V; ++t) {
                    double d = p[t] - (vq ? q[t] : 0.0);
                    q[t] = d > 0.0 ? d : 0.0;
                    R += q[t];
                }
                if (R > 0.0 ? orc_cdf_draw_ok(q, V, nx, u_fin * R, tol * R)
                            : orc_cdf_draw_ok(p, V, nx, u_fin, tol))
                    valid |= 2;
            } else if (orc_cdf_draw_ok(p, V, nx, u_fin, tol)) {
                valid |= 2;
            }
        }
        valid_out[b] = valid;
        if (status_out) status_out[b] = status;
        free(p); free(q);
    }
}

/*
 * Sampled tree walk check [SD §5 DDTree, the walk of orc_verify_tree_sampled].
 * Follows the given path (path_in [B, N], A_in, next_in) from the root: at
 * each visited node the committed token (the next node's token, or next at
 * the end) must be a valid draw of that node's transformed row at its uniform
 * (orc_cdf_draw_ok with slack tol), each path entry must be a child of the
 * node before it carrying that token, the final token must have no child at
 * the last node, and the path entries past A must be -1. A non-finite row
 * ends the walk with next == -1. valid_out[b] = 1 when all hold.
 */
void orc_check_tree_sampled(const float* target, const int32_t* node_token,
                            const int32_t* node_parent, const int32_t* n_nodes,
                            const float* uniforms, int B, int N, int V, double T, int top_k,
                            double tol, const int32_t* path_in, const int32_t* A_in,
                            const int32_t* next_in, int32_t* valid_out, int nthreads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int b = 0; b < B; ++b) {
        const int32_t* tok = node_token + (size_t)b * N;
        const int32_t* par = node_parent + (size_t)b * N;
        const int32_t* path = path_in + (size_t)b * N;
        int nn = n_nodes[b];
        int A = A_in[b];
        int ok = A >= 0 && A < N;
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        for (int i = (ok ? A : N); i < N; ++i)
            if (path[i] != -1) ok = 0;
        int node = 0;
        for (int j = 0; ok && j <= A; ++j) {
            int valid = orc_transform_row(target + ((size_t)b * N + node) * V, V, T, top_k, p);
            double u = (double)uniforms[(size_t)b * N + node];
            if (!valid) {
                ok = (j == A && next_in[b] == -1);
                break;
            }
            if (j < A) {
                int c = path[j];
                if (c < 1 || c >= nn || par[c] != node) { ok = 0; break; }
                if (!orc_cdf_draw_ok(p, V, tok[c], u, tol)) ok = 0;
                node = c;
            } else {
                int g = next_in[b];
                if (!orc_cdf_draw_ok(p, V, g, u, tol)) ok = 0;
                for (int c = 1; c < nn && ok; ++c)
                    if (par[c] == node && tok[c] == g) ok = 0;
            }
        }
        valid_out[b] = ok;
        free(p);
    }
}

/*
 * Length choice check [SD §5 DSpark, the rule of orc_select_len]: k_in[b] is
 * valid when every s_j, j <= k, exceeds cost - tol and s_{k+1} (if any) does
 * not exceed cost + tol, with s the fp32 running product of the confidences.
 */
void orc_check_select_len(const float* conf, int B, int K, float cost, double tol,
                          const int32_t* k_in, int32_t* valid_out) {
    for (int b = 0; b < B; ++b) {
        int k = k_in[b];
        int ok = k >= 0 && k <= K;
        float s = 1.0f;
        for (int j = 1; ok && j <= K; ++j) {
            s = s * conf[(size_t)b * K + (j - 1)];
            if (j <= k && !((double)s > (double)cost - tol)) ok = 0;
            if (j == k + 1 && (double)s > (double)cost + tol) ok = 0;
        }
        valid_out[b] = ok;
    }
}

/*
 * EAGLE-2-style expansion step [SD §4 EAGLE-2: the candidate tree grows by
 * expanding the branches of highest cumulative path confidence; the final
 * tree is re-ranked from the candidates (orc_rerank_tree)].
 *
 * Candidates of sequence b live in [B, M] arrays in topological order, as in
 * orc_rerank_tree, plus cand_conf, the cumulative confidence (-1 marks an
 * unusable candidate). One call grows the tree by one layer:
 *   - n_cand[b] == 0 starts the tree: candidate 0 is the root (parent -1,
 *     token -1, prob 1, conf 1) and the root is the one node expanded.
 *     Otherwise slot w < W names the node expand_in[b, w], which is expanded
 *     when 0 <= id < n_cand[b] and cand_conf[b, id] >= 0.
 *   - The children of the node in slot w are child_token[b, w, c] with
 *     conditional probability child_prob[b, w, c], c < C. The expanded
 *     slots' children are appended in slot order, C per slot, from n0 (the
 *     count before the call, after the root) while the index stays below M.
 *     A child's confidence is fl32(conf[parent] * prob) when prob lies in
 *     [0, 1], else -1.
 *   - n_cand[b] becomes the new count.
 *   - expand_out[b, 0..W) receives the appended candidates with confidence
 *     >= 0 ordered by (confidence desc, index asc), the first W, -1 padded:
 *     the nodes the next call expands.
 */
typedef struct {
    float conf;
    int idx;
} OrcExp;

static int orc_exp_cmp(const void* a, const void* b) {
    const OrcExp* x = (const OrcExp*)a;
    const OrcExp* y = (const OrcExp*)b;
    if (x->conf != y->conf) return x->conf > y->conf ? -1 : 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

void orc_expand_tree(int32_t* cand_parent, int32_t* cand_token, float* cand_prob, float* cand_conf,
                     int32_t* n_cand, const int32_t* expand_in, int32_t* expand_out,
                     const int32_t* child_token, const float* child_prob, int B, int M, int W,
                     int C) {
    for (int b = 0; b < B; ++b) {
        int32_t* par = cand_parent + (size_t)b * M;
        int32_t* tok = cand_token + (size_t)b * M;
        float* prob = cand_prob + (size_t)b * M;
        float* conf = cand_conf + (size_t)b * M;
        int n0 = n_cand[b];
        if (n0 < 0) n0 = 0;
        if (n0 > M) n0 = M;
        /* the nodes expanded by this call, slot by slot (-1: slot not expanded) */
        int* node = (int*)malloc(sizeof(int) * (size_t)(W > 0 ? W : 1));
        for (int w = 0; w < W; ++w) node[w] = -1;
        if (n0 == 0) {
            par[0] = -1; tok[0] = -1; prob[0] = 1.0f; conf[0] = 1.0f;
            n0 = 1;
            if (W > 0) node[0] = 0;
        } else {
            for (int w = 0; w < W; ++w) {
                int id = expand_in[(size_t)b * W + w];
                if (id >= 0 && id < n0 && conf[id] >= 0.0f) node[w] = id;
            }
        }
        int n = n0;
        for (int w = 0; w < W; ++w) {
            if (node[w] < 0) continue;
            for (int c = 0; c < C && n < M; ++c) {
                float q = child_prob[((size_t)b * W + w) * C + c];
                par[n] = node[w];
                tok[n] = child_token[((size_t)b * W + w) * C + c];
                prob[n] = q;
                conf[n] = (q >= 0.0f && q <= 1.0f) ? conf[node[w]] * q : -1.0f;
                ++n;
            }
        }
        n_cand[b] = n;
        OrcExp* list = (OrcExp*)malloc(sizeof(OrcExp) * (size_t)(n - n0 + 1));
        int nl = 0;
        for (int i = n0; i < n; ++i)
            if (conf[i] >= 0.0f) { list[nl].conf = conf[i]; list[nl].idx = i; ++nl; }
        qsort(list, (size_t)nl, sizeof(OrcExp), orc_exp_cmp);
        for (int w = 0; w < W; ++w) expand_out[(size_t)b * W + w] = w < nl ? list[w].idx : -1;
        free(list);
        free(node);
    }
}
