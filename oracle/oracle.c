/*
 * oracle.c -- plain, slow, single-threaded, fp64 CPU oracle of the speculative
 * verification step: token-tree build, tree-masked attention, acceptance /
 * selection / resampling, and the KV commit of the accepted path.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no source, header,
 * table or helper with the HIP library, and neither one includes the other.
 *
 * Sources (web pages; cited by page title and section):
 *   [ReDrafter] "Recurrent Drafter for Fast Speculative Decoding in Large
 *               Language Models": sections "Dynamic Tree Attention" and
 *               "The Full Speculative Decoding Loop" (Steps 3-6).
 *   [Clover]    "Clover: Regressive Lightweight Speculative Decoding with
 *               Sequential Knowledge": section "Inference-Time Verification:
 *               Token Tree Construction and Tree Attention" (mask, Figure 4).
 *   [ResiSpec]  paperpeel 2608.24411 (residual drift in multi-candidate
 *               verification): section 4 (residual distribution, sequential
 *               verification of N candidates), section 5 "Practical
 *               Implementation" (GetProxy residual shaping, read literally in
 *               part 7) and Appendix B.1 (path marginals).
 *
 * Conventions (readings where the pages are silent; each one is listed in the
 * design notes of the repository):
 *   - Tree position 0 is the root: the last token already sampled by the target,
 *     whose K/V are not cached yet.  Draft nodes are 1..T-1; T = n_nodes[b]
 *     counts the root.
 *   - Beams are numbered into the tree in beam-major order of first appearance.
 *   - The attention mask of node i holds i itself, the root and every ancestor.
 *   - Target row t is the target distribution for the children of node t (and
 *     for the bonus token after t); dft_row[t] names the draft row the children
 *     of t were drawn from.
 *   - Padding: parent/token/depth = -1 and an all-zero mask for t >= T.
 *
 * Pins: every function is checked in the test suite against values the pages
 * print, closed forms, brute force or a second formulation.  Per-path
 * rejection (mode 1) is not distribution-exact when a node has two or more
 * children (only sequential checking is), so its tree-level output law is
 * pinned to its own definition instead: the joint law of (stop node, next
 * token) on a fixed tree with siblings, summed exactly over every accept
 * pattern, against 1e6 seeded trials.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR -1

#define ORC_GREEDY 0
#define ORC_REJECT_PATH 1
#define ORC_REJECT_RECURSIVE 2

/* |ratio - u| below this counts as a decision near-tie (both sides count). */
#define ORC_NEAR_TIE 1e-5
/* A running-sum boundary within this distance of the threshold u * total of an
 * inverse-CDF draw from a normalised distribution counts as a sampling near-tie. */
#define ORC_CDF_NEAR_TIE 1e-9

/* ------------------------------------------------------------------------ */
/* small helpers                                                             */
/* ------------------------------------------------------------------------ */

/* bf16 -> double, exact: a bf16 is the top 16 bits of an IEEE binary32. */
static double bf16_to_double(uint16_t h)
{
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double load_elem(int dtype, const void *base, size_t idx)
{
    if (dtype == 0) return (double)((const float *)base)[idx];
    return bf16_to_double(((const uint16_t *)base)[idx]);
}

static int anc_has(const uint64_t *row, int a)
{
    return (int)((row[a >> 6] >> (a & 63)) & 1u);
}

static void anc_set(uint64_t *row, int a)
{
    row[a >> 6] |= (uint64_t)1 << (a & 63);
}

/* ------------------------------------------------------------------------ */
/* 1. Tree construction                                                      */
/* ------------------------------------------------------------------------ */

/* Finish a tree whose parent[] and token[] are filled for nodes 0..T-1:
 * depth by walking to the root, ancestor mask = self + every ancestor + root
 * ([Clover] tree mask: M_ij = 1 iff j is an ancestor of i or i = j). */
static void finish_tree(int T, int T_cap, int n_words, int32_t *parent, int32_t *depth,
                        uint64_t *anc, int32_t *token)
{
    for (int t = 0; t < T_cap; ++t) {
        uint64_t *row = anc + (size_t)t * n_words;
        for (int w = 0; w < n_words; ++w) row[w] = 0;
        if (t >= T) {
            parent[t] = -1;
            token[t] = -1;
            depth[t] = -1;
            continue;
        }
        int d = 0;
        int cur = t;
        anc_set(row, t);
        while (cur != 0) {
            cur = parent[cur];
            anc_set(row, cur);
            ++d;
        }
        depth[t] = d;
    }
}

/*
 * Beams -> token tree ([ReDrafter] "Dynamic Tree Attention": candidates share
 * prefixes; the packed beam keeps each distinct prefix once, and the mask lets a
 * token see only its own prefix).  Written as a textbook trie insertion: walk
 * each beam from the root, reuse the child that carries the same token, else
 * append a new node.  Node ids are given in beam-major order of first
 * appearance.  beam_node[i][k] = node holding beam i's prefix of length k+1.
 *
 * Layout: beams [B][W][L], root_token [B]; outputs n_nodes [B], parent/token/
 * depth [B][T_cap], anc [B][T_cap][ceil(T_cap/64)], beam_node [B][W][L] (or NULL).
 */
int orc_build_tree_beams(int B, int W, int L, int T_cap, const int32_t *beams,
                         const int32_t *root_token, int32_t *n_nodes, int32_t *parent,
                         int32_t *token, int32_t *depth, uint64_t *anc, int32_t *beam_node)
{
    if (B < 0 || W < 1 || L < 1 || T_cap < 1 + W * L) return ORC_ERR;
    int n_words = (T_cap + 63) / 64;
    for (int b = 0; b < B; ++b) {
        int32_t *par = parent + (size_t)b * T_cap;
        int32_t *tok = token + (size_t)b * T_cap;
        int T = 1;
        par[0] = -1;
        tok[0] = root_token[b];
        for (int i = 0; i < W; ++i) {
            int cur = 0;
            for (int k = 0; k < L; ++k) {
                int32_t x = beams[((size_t)b * W + i) * L + k];
                int child = -1;
                for (int c = 1; c < T; ++c) {
                    if (par[c] == cur && tok[c] == x) {
                        child = c;
                        break;
                    }
                }
                if (child < 0) {
                    child = T++;
                    par[child] = cur;
                    tok[child] = x;
                }
                if (beam_node) beam_node[((size_t)b * W + i) * L + k] = child;
                cur = child;
            }
        }
        n_nodes[b] = T;
        finish_tree(T, T_cap, n_words, par, depth + (size_t)b * T_cap,
                    anc + (size_t)b * T_cap * n_words, tok);
    }
    return ORC_OK;
}

/*
 * Explicit candidate tree (static trees of parallel heads, [Clover] "Token tree
 * construction"; caterpillars of i.i.d. candidates, [ResiSpec] section 4).
 * Candidate j (0-based) becomes node j+1; cand_parent[j] is its parent's tree
 * index and must lie in [0, j].  Duplicate siblings are kept as given.
 * A sequence whose parent list is not topological becomes a root-only tree and
 * its bad flag is set.
 */
int orc_build_tree_explicit(int B, int N, int T_cap, const int32_t *cand_parent,
                            const int32_t *cand_token, const int32_t *root_token,
                            int32_t *n_nodes, int32_t *parent, int32_t *token, int32_t *depth,
                            uint64_t *anc, int32_t *bad)
{
    if (B < 0 || N < 0 || T_cap < 1 + N) return ORC_ERR;
    int n_words = (T_cap + 63) / 64;
    for (int b = 0; b < B; ++b) {
        int32_t *par = parent + (size_t)b * T_cap;
        int32_t *tok = token + (size_t)b * T_cap;
        int ok = 1;
        for (int j = 0; j < N; ++j) {
            int32_t p = cand_parent[(size_t)b * N + j];
            if (p < 0 || p > j) ok = 0;
        }
        int T = ok ? N + 1 : 1;
        par[0] = -1;
        tok[0] = root_token[b];
        for (int j = 0; j < T - 1; ++j) {
            par[j + 1] = cand_parent[(size_t)b * N + j];
            tok[j + 1] = cand_token[(size_t)b * N + j];
        }
        n_nodes[b] = T;
        if (bad) bad[b] = !ok;
        finish_tree(T, T_cap, n_words, par, depth + (size_t)b * T_cap,
                    anc + (size_t)b * T_cap * n_words, tok);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 2. Tree-masked attention                                                  */
/* ------------------------------------------------------------------------ */

/*
 * One output row of tree attention ([ReDrafter] Step 4: one forward pass over
 * the packed beam under the tree mask, each token attending only to its own
 * prefix; [Clover] mask M_ij).  Query (b, t, h) attends to every context key
 * 0..ctx-1 and to the tree keys ctx+a for every a in mask(t) (self, ancestors,
 * root).  Scores are q.k * scale; softmax with max subtraction; all in fp64.
 * Query head h reads KV head h / (H / Hkv).  Rows t >= T are zero.
 *
 * Layout: q [B][T_cap][H][D], k/v [B][Hkv][cap][D], out_row [D].
 */
static void attention_row(int dtype, int T_cap, int H, int Hkv, int D, int cap,
                          const void *q, const void *kc, const void *vc, int ctx, int T,
                          const uint64_t *anc_row, double scale, int b, int t, int h,
                          double *out_row, double *score_buf)
{
    for (int d = 0; d < D; ++d) out_row[d] = 0.0;
    if (t >= T) return;
    int g = h / (H / Hkv);
    size_t q_off = (((size_t)b * T_cap + t) * H + h) * D;
    size_t kv_base = ((size_t)b * Hkv + g) * (size_t)cap * D;
    int n_keys = ctx + T;
    double m = -INFINITY;
    for (int j = 0; j < n_keys; ++j) {
        if (j >= ctx && !anc_has(anc_row, j - ctx)) {
            score_buf[j] = -INFINITY;
            continue;
        }
        double s = 0.0;
        for (int d = 0; d < D; ++d)
            s += load_elem(dtype, q, q_off + d) * load_elem(dtype, kc, kv_base + (size_t)j * D + d);
        s *= scale;
        score_buf[j] = s;
        if (s > m) m = s;
    }
    double denom = 0.0;
    for (int j = 0; j < n_keys; ++j) {
        if (score_buf[j] == -INFINITY) continue;
        double w = exp(score_buf[j] - m);
        denom += w;
        for (int d = 0; d < D; ++d)
            out_row[d] += w * load_elem(dtype, vc, kv_base + (size_t)j * D + d);
    }
    for (int d = 0; d < D; ++d) out_row[d] /= denom;
}

/*
 * Tree attention for a list of rows.  sel holds n_sel (b, t, h) triples; with
 * sel == NULL every row of [B][T_cap][H] is computed in that order.  out is
 * [n_rows][D] fp64.  scale <= 0 means 1/sqrt(D).  Returns ORC_ERR on bad
 * shapes, or when ctx_len[b] + n_nodes[b] exceeds the cache capacity.
 */
int orc_tree_attention(int dtype, int B, int T_cap, int H, int Hkv, int D, int cap,
                       const void *q, const void *kc, const void *vc, const int32_t *ctx_len,
                       const int32_t *n_nodes, const uint64_t *anc, double scale, int n_sel,
                       const int32_t *sel, double *out)
{
    if (B < 1 || T_cap < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || D < 1) return ORC_ERR;
    if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
    int n_words = (T_cap + 63) / 64;
    for (int b = 0; b < B; ++b)
        if (ctx_len[b] < 0 || n_nodes[b] < 1 || n_nodes[b] > T_cap || ctx_len[b] + n_nodes[b] > cap)
            return ORC_ERR;
    size_t n_rows = sel ? (size_t)n_sel : (size_t)B * T_cap * H;
    double *score_buf = (double *)malloc(sizeof(double) * ((size_t)cap + 1));
    if (!score_buf) return ORC_ERR;
    for (size_t r = 0; r < n_rows; ++r) {
        int b, t, h;
        if (sel) {
            b = sel[3 * r];
            t = sel[3 * r + 1];
            h = sel[3 * r + 2];
            if (b < 0 || b >= B || t < 0 || t >= T_cap || h < 0 || h >= H) {
                free(score_buf);
                return ORC_ERR;
            }
        } else {
            b = (int)(r / ((size_t)T_cap * H));
            t = (int)((r / H) % T_cap);
            h = (int)(r % H);
        }
        attention_row(dtype, T_cap, H, Hkv, D, cap, q, kc, vc, ctx_len[b], n_nodes[b],
                      anc + ((size_t)b * T_cap + t) * n_words, scale, b, t, h,
                      out + r * D, score_buf);
    }
    free(score_buf);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 3. Verification                                                           */
/* ------------------------------------------------------------------------ */

/* Softmax of one logits row in fp64: p(v) = exp(l_v - max) / sum_v' exp(l_v' - max). */
static void softmax_row(int V, const float *logits, double *p)
{
    double m = -INFINITY;
    for (int v = 0; v < V; ++v)
        if ((double)logits[v] > m) m = (double)logits[v];
    double s = 0.0;
    for (int v = 0; v < V; ++v) {
        p[v] = exp((double)logits[v] - m);
        s += p[v];
    }
    for (int v = 0; v < V; ++v) p[v] /= s;
}

/* Greedy target token: the first index holding the row maximum (ties go to
 * the lowest index), decided on the fp32 logits themselves. */
static int argmax_row(int V, const float *logits)
{
    int best = 0;
    for (int v = 1; v < V; ++v)
        if (logits[v] > logits[best]) best = v;
    return best;
}

/* Unnormalised residual mass in closed form, Z(c) = sum_v max(0, p(v) - c q(v)).
 * Used by the closed-form identity pin only (orc_residual_chain). */
static double residual_mass(int V, const double *p, const double *q, double c)
{
    double z = 0.0;
    for (int v = 0; v < V; ++v) {
        double w = p[v] - c * (q ? q[v] : 0.0);
        if (w > 0.0) z += w;
    }
    return z;
}

/* One rejection ([ResiSpec] section 4): r <- max(0, r - q) / sum_v max(0, r - q).
 * Returns the normaliser; when it is not positive r is left untouched. */
static double residual_step(int V, double *r, const double *q)
{
    double z = 0.0;
    for (int v = 0; v < V; ++v) {
        double w = r[v] - q[v];
        if (w > 0.0) z += w;
    }
    if (!(z > 0.0)) return z;
    for (int v = 0; v < V; ++v) {
        double w = r[v] - q[v];
        r[v] = w > 0.0 ? w / z : 0.0;
    }
    return z;
}

/*
 * Inverse-CDF draw from the distribution r (weights, summing to about one) in
 * ascending vocabulary order: the smallest v whose running sum exceeds u * S,
 * S being the total of r.  If rounding leaves no such v, the last v with
 * positive weight.  *near is set when a running-sum boundary lies within
 * ORC_CDF_NEAR_TIE of u * S.
 */
static int sample_inverse_cdf(int V, const double *r, double u, int *near)
{
    double total = 0.0;
    for (int v = 0; v < V; ++v)
        if (r[v] > 0.0) total += r[v];
    double thr = u * total;
    double run = 0.0;
    int last_pos = -1;
    *near = 0;
    for (int v = 0; v < V; ++v) {
        if (!(r[v] > 0.0)) continue;
        last_pos = v;
        double before = run;
        run += r[v];
        if (run > thr) {
            if (fabs(run - thr) < ORC_CDF_NEAR_TIE || fabs(before - thr) < ORC_CDF_NEAR_TIE)
                *near = 1;
            return v;
        }
    }
    return last_pos < 0 ? 0 : last_pos;
}

/*
 * Verification of one packed tree per sequence.
 *
 * Rows: tgt [B][T_cap][V] fp32 target logits (row t = distribution after node
 * t); dft [B][R][V] fp32 draft logits, dft_row [B][T_cap] (row the children of
 * t were drawn from, -1 if none).  p_t = softmax(tgt[t]), q_t = softmax of the
 * draft row of t.  Uniforms: u_node [B][T_cap] (one per node, index 0 unused),
 * u_final [B].
 *
 * GREEDY ([ReDrafter] Step 5, token matches): node t is accepted iff its token
 *   equals the argmax of its parent's target row.
 * REJECT_PATH ([ReDrafter] Step 5, rejection sampling after Leviathan et al.):
 *   node t is accepted iff u_node[t] < p_par(x) / q_par(x), independently per
 *   node; a candidate stops at its first rejection.
 * In both, a node is kept when it and all its ancestors are accepted; the
 * longest kept prefix over all candidates wins ([ReDrafter] "What longest
 * accepted prefix means"), ties going to the lowest node index (= lowest beam
 * index).  At the stop node s the next token is argmax p_s (GREEDY); for
 * REJECT_PATH it is drawn with u_final from norm(max(0, p_s - q_s)) when s has
 * children (all rejected) and from p_s when s is a leaf.
 * REJECT_RECURSIVE ([ResiSpec] section 4, sequential verification): walk from
 *   the root; the children of s are checked in index order against the current
 *   target p' (p' = p_s at first): accept child x iff u < p'(x)/q_s(x); on a
 *   rejection p' <- norm(max(0, p' - q_s)).  An acceptance moves to that child
 *   and restarts with p' = p_child.  When s has no child left, the next token
 *   is drawn from p'.  p' is kept as an explicit normalised vector, renormalised
 *   after every rejection exactly as the definition reads.  A rejection whose
 *   residual has no positive mass (possible only through rounding) rejects the
 *   remaining children and draws from p_s; it is counted in fallback[b].
 *
 * Outputs: acc_len [B] (depth of the stop node), acc_path [B][T_cap] (root
 * first, -1 after the path), next_token [B], p_tok/q_tok [B][T_cap]
 * (p_par(token), q_par(token); 0 for the root, padding, and q in GREEDY),
 * decision [B][T_cap] (1 accepted, 0 rejected, -1 untested), near_tie [B]
 * (decision near-ties |ratio - u| < 1e-5 plus a CDF near-tie), fallback [B].
 */
int orc_verify(int mode, int B, int T_cap, int V, int R, const float *tgt, const float *dft,
               const int32_t *dft_row, const int32_t *n_nodes, const int32_t *parent,
               const int32_t *token, const int32_t *depth, const float *u_node,
               const float *u_final, int32_t *acc_len, int32_t *acc_path, int32_t *next_token,
               double *p_tok, double *q_tok, int8_t *decision, int32_t *near_tie,
               int32_t *fallback)
{
    if (mode < ORC_GREEDY || mode > ORC_REJECT_RECURSIVE) return ORC_ERR;
    if (B < 0 || T_cap < 1 || V < 1) return ORC_ERR;
    if (mode != ORC_GREEDY && (!dft || !dft_row || R < 1)) return ORC_ERR;

    double *p_rows = (double *)malloc(sizeof(double) * (size_t)T_cap * V);
    double *q_rows = (double *)malloc(sizeof(double) * (size_t)T_cap * V);
    int *has_q = (int *)malloc(sizeof(int) * (size_t)T_cap);
    int *acc = (int *)malloc(sizeof(int) * (size_t)T_cap);
    int *chain = (int *)malloc(sizeof(int) * (size_t)T_cap);
    int *n_child = (int *)malloc(sizeof(int) * (size_t)T_cap);
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    if (!p_rows || !q_rows || !has_q || !acc || !chain || !n_child || !r) {
        free(p_rows); free(q_rows); free(has_q); free(acc); free(chain); free(n_child); free(r);
        return ORC_ERR;
    }
    int rc = ORC_OK;

    for (int b = 0; b < B && rc == ORC_OK; ++b) {
        int T = n_nodes[b];
        const int32_t *par = parent + (size_t)b * T_cap;
        const int32_t *tok = token + (size_t)b * T_cap;
        const int32_t *dep = depth + (size_t)b * T_cap;
        const float *ub = u_node + (size_t)b * T_cap;
        int32_t *path = acc_path + (size_t)b * T_cap;
        int8_t *dec = decision + (size_t)b * T_cap;
        double *pt = p_tok + (size_t)b * T_cap;
        double *qt = q_tok + (size_t)b * T_cap;
        if (T < 1 || T > T_cap) { rc = ORC_ERR; break; }

        for (int t = 0; t < T_cap; ++t) {
            path[t] = -1;
            dec[t] = -1;
            pt[t] = 0.0;
            qt[t] = 0.0;
            n_child[t] = 0;
            has_q[t] = 0;
        }
        for (int t = 1; t < T; ++t) {
            if (par[t] < 0 || par[t] >= t || tok[t] < 0 || tok[t] >= V) { rc = ORC_ERR; break; }
            n_child[par[t]]++;
        }
        if (rc != ORC_OK) break;
        near_tie[b] = 0;
        fallback[b] = 0;

        /* distributions of every node row */
        for (int t = 0; t < T; ++t) {
            softmax_row(V, tgt + ((size_t)b * T_cap + t) * V, p_rows + (size_t)t * V);
            if (mode != ORC_GREEDY) {
                int r = dft_row[(size_t)b * T_cap + t];
                if (r >= 0 && r < R) {
                    softmax_row(V, dft + ((size_t)b * R + r) * V, q_rows + (size_t)t * V);
                    has_q[t] = 1;
                } else if (n_child[t] > 0) {
                    rc = ORC_ERR;
                }
            }
        }
        if (rc != ORC_OK) break;
        for (int t = 1; t < T; ++t) {
            pt[t] = p_rows[(size_t)par[t] * V + tok[t]];
            if (mode != ORC_GREEDY) qt[t] = q_rows[(size_t)par[t] * V + tok[t]];
        }

        int stop = 0;

        if (mode == ORC_GREEDY || mode == ORC_REJECT_PATH) {
            for (int t = 1; t < T; ++t) {
                if (mode == ORC_GREEDY) {
                    acc[t] = tok[t] == argmax_row(V, tgt + ((size_t)b * T_cap + par[t]) * V);
                } else {
                    double ratio = qt[t] > 0.0 ? pt[t] / qt[t] : (pt[t] > 0.0 ? INFINITY : 0.0);
                    double u = (double)ub[t];
                    acc[t] = u < ratio;
                    if (fabs(ratio - u) < ORC_NEAR_TIE) near_tie[b]++;
                }
                dec[t] = (int8_t)acc[t];
            }
            chain[0] = 1;
            for (int t = 1; t < T; ++t) chain[t] = acc[t] && chain[par[t]];
            for (int t = 1; t < T; ++t)
                if (chain[t] && dep[t] > dep[stop]) stop = t;
            if (mode == ORC_REJECT_PATH) {
                /* draw from p_s, or from norm(max(0, p_s - q_s)) when every child of
                 * the stop node was rejected */
                memcpy(r, p_rows + (size_t)stop * V, sizeof(double) * (size_t)V);
                if (n_child[stop] > 0 && !(residual_step(V, r, q_rows + (size_t)stop * V) > 0.0)) {
                    fallback[b] = 1;
                    memcpy(r, p_rows + (size_t)stop * V, sizeof(double) * (size_t)V);
                }
            }
        } else {
            /* sequential multi-candidate verification, residual renormalised after
             * each rejection */
            int s = 0;
            for (;;) {
                const double *q = has_q[s] ? q_rows + (size_t)s * V : NULL;
                memcpy(r, p_rows + (size_t)s * V, sizeof(double) * (size_t)V);
                int moved = 0, dead = 0;
                for (int ch = s + 1; ch < T; ++ch) {
                    if (par[ch] != s) continue;
                    if (dead) {
                        dec[ch] = 0;
                        continue;
                    }
                    int x = tok[ch];
                    double ratio = q[x] > 0.0 ? r[x] / q[x] : (r[x] > 0.0 ? INFINITY : 0.0);
                    double u = (double)ub[ch];
                    if (fabs(ratio - u) < ORC_NEAR_TIE) near_tie[b]++;
                    if (u < ratio) {
                        dec[ch] = 1;
                        s = ch;
                        moved = 1;
                        break;
                    }
                    dec[ch] = 0;
                    if (!(residual_step(V, r, q) > 0.0)) {
                        dead = 1;
                        fallback[b] = 1;
                        memcpy(r, p_rows + (size_t)s * V, sizeof(double) * (size_t)V);
                    }
                }
                if (moved) continue;
                stop = s;
                break;
            }
        }

        acc_len[b] = dep[stop];
        for (int cur = stop; cur >= 0; cur = par[cur]) path[dep[cur]] = cur;

        if (mode == ORC_GREEDY) {
            next_token[b] = argmax_row(V, tgt + ((size_t)b * T_cap + stop) * V);
        } else {
            int near = 0;
            next_token[b] = sample_inverse_cdf(V, r, (double)u_final[b], &near);
            near_tie[b] += near;
        }
    }
    free(r);
    free(p_rows); free(q_rows); free(has_q); free(acc); free(chain); free(n_child);
    return rc;
}

/*
 * Greedy verification by walking the tree from the root ([ReDrafter] section
 * "The Full Speculative Decoding Loop", Step 5, token matches): the same
 * acceptance as orc_verify in ORC_GREEDY, found by visiting only the rows that
 * the decision needs.  The nodes whose whole path is accepted are explored
 * depth by depth: the frontier starts as {root}; every frontier node's target
 * row gives its greedy token (argmax, lowest index on ties); its children are
 * tested against it, and the accepted ones form the next frontier.  The stop
 * node is the lowest-index node of the deepest non-empty frontier (the deepest
 * survivor, lowest index on ties) and the next token is its greedy token.
 *
 * Outputs as orc_verify, except that only tested nodes (children of frontier
 * nodes) get decision (1 / 0) and p_tok; all other entries are -1 and 0.
 * rows_read[b] counts the target rows read: one per frontier node.
 */
int orc_verify_greedy_walk(int B, int T_cap, int V, const float *tgt, const int32_t *n_nodes,
                           const int32_t *parent, const int32_t *token, const int32_t *depth,
                           int32_t *acc_len, int32_t *acc_path, int32_t *next_token,
                           double *p_tok, int8_t *decision, int32_t *rows_read)
{
    if (B < 0 || T_cap < 1 || V < 1) return ORC_ERR;
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    int *front = (int *)malloc(sizeof(int) * (size_t)T_cap);
    int *next = (int *)malloc(sizeof(int) * (size_t)T_cap);
    int *greedy = (int *)malloc(sizeof(int) * (size_t)T_cap);
    if (!p || !front || !next || !greedy) {
        free(p); free(front); free(next); free(greedy);
        return ORC_ERR;
    }
    int rc = ORC_OK;
    for (int b = 0; b < B && rc == ORC_OK; ++b) {
        const int T = n_nodes[b];
        const int32_t *par = parent + (size_t)b * T_cap;
        const int32_t *tok = token + (size_t)b * T_cap;
        const int32_t *dep = depth + (size_t)b * T_cap;
        int32_t *path = acc_path + (size_t)b * T_cap;
        int8_t *dec = decision + (size_t)b * T_cap;
        double *pt = p_tok + (size_t)b * T_cap;
        if (T < 1 || T > T_cap) { rc = ORC_ERR; break; }
        for (int t = 1; t < T; ++t)
            if (par[t] < 0 || par[t] >= t || tok[t] < 0 || tok[t] >= V) { rc = ORC_ERR; break; }
        if (rc != ORC_OK) break;
        for (int t = 0; t < T_cap; ++t) {
            path[t] = -1;
            dec[t] = -1;
            pt[t] = 0.0;
        }
        int n_front = 1, stop = 0, reads = 0;
        front[0] = 0;
        while (n_front > 0) {
            /* the frontier is in increasing node order: its first node is the
             * lowest-index survivor of this depth */
            stop = front[0];
            int n_next = 0;
            for (int i = 0; i < n_front; ++i) {
                const int f = front[i];
                const float *row = tgt + ((size_t)b * T_cap + f) * V;
                greedy[f] = argmax_row(V, row);
                softmax_row(V, row, p);
                ++reads;
                for (int c = f + 1; c < T; ++c) {
                    if (par[c] != f) continue;
                    dec[c] = (int8_t)(tok[c] == greedy[f]);
                    pt[c] = p[tok[c]];
                    if (dec[c]) next[n_next++] = c;
                }
            }
            /* children of different frontier nodes interleave in index order */
            for (int i = 1; i < n_next; ++i)
                for (int j = i; j > 0 && next[j - 1] > next[j]; --j) {
                    const int x = next[j]; next[j] = next[j - 1]; next[j - 1] = x;
                }
            memcpy(front, next, sizeof(int) * (size_t)n_next);
            n_front = n_next;
        }
        acc_len[b] = dep[stop];
        for (int cur = stop; cur >= 0; cur = par[cur]) path[dep[cur]] = cur;
        next_token[b] = greedy[stop];
        rows_read[b] = reads;
    }
    free(p); free(front); free(next); free(greedy);
    return rc;
}

/*
 * Rejection-mode verification by walking the tree from the root, reading only
 * the rows the decisions need ([ReDrafter] "The Full Speculative Decoding
 * Loop", Step 5, rejection sampling; [ResiSpec] section 4, sequential
 * verification).  The acceptance, stop node and next token are those of
 * orc_verify in the same mode; what changes is which rows are read.
 *
 * ORC_REJECT_PATH: the nodes whose whole path is accepted are explored depth by
 *   depth.  The frontier starts as {root}; for every frontier node f with
 *   children, f's target row and draft row give p_f and q_f, and each child c
 *   (token x) is accepted iff u_node[c] < p_f(x) / q_f(x).  The accepted
 *   children form the next frontier.  The stop node s is the lowest-index node
 *   of the deepest non-empty frontier.  The next token is drawn with u_final
 *   from norm(max(0, p_s - q_s)) if s has children (all rejected), else from
 *   p_s, whose target row is read then.
 * ORC_REJECT_RECURSIVE: the walk of orc_verify, reading the target and draft
 *   rows of each node it moves to (when it has children) and, at a stop node
 *   without children, that node's target row.
 *
 * Outputs as orc_verify, except that only tested nodes (children of nodes
 * whose rows were read) get decision, p_tok and q_tok; all other entries are
 * -1, 0 and 0, and near_tie counts the tested nodes' near-ties (plus a CDF
 * near-tie).  rows_tgt[b] and rows_dft[b] count the target and draft rows read
 * (a row read twice is counted twice).
 */
int orc_verify_reject_walk(int mode, int B, int T_cap, int V, int R, const float *tgt,
                           const float *dft, const int32_t *dft_row, const int32_t *n_nodes,
                           const int32_t *parent, const int32_t *token, const int32_t *depth,
                           const float *u_node, const float *u_final, int32_t *acc_len,
                           int32_t *acc_path, int32_t *next_token, double *p_tok, double *q_tok,
                           int8_t *decision, int32_t *near_tie, int32_t *fallback,
                           int32_t *rows_tgt, int32_t *rows_dft)
{
    if (mode != ORC_REJECT_PATH && mode != ORC_REJECT_RECURSIVE) return ORC_ERR;
    if (B < 0 || T_cap < 1 || V < 1 || !dft || !dft_row || R < 1) return ORC_ERR;
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    double *r = (double *)malloc(sizeof(double) * (size_t)V);
    int *front = (int *)malloc(sizeof(int) * (size_t)T_cap);
    int *next = (int *)malloc(sizeof(int) * (size_t)T_cap);
    int *n_child = (int *)malloc(sizeof(int) * (size_t)T_cap);
    if (!p || !q || !r || !front || !next || !n_child) {
        free(p); free(q); free(r); free(front); free(next); free(n_child);
        return ORC_ERR;
    }
    int rc = ORC_OK;
    for (int b = 0; b < B && rc == ORC_OK; ++b) {
        const int T = n_nodes[b];
        const int32_t *par = parent + (size_t)b * T_cap;
        const int32_t *tok = token + (size_t)b * T_cap;
        const int32_t *dep = depth + (size_t)b * T_cap;
        const int32_t *drow = dft_row + (size_t)b * T_cap;
        const float *ub = u_node + (size_t)b * T_cap;
        int32_t *path = acc_path + (size_t)b * T_cap;
        int8_t *dec = decision + (size_t)b * T_cap;
        double *pt = p_tok + (size_t)b * T_cap;
        double *qt = q_tok + (size_t)b * T_cap;
        if (T < 1 || T > T_cap) { rc = ORC_ERR; break; }
        for (int t = 0; t < T_cap; ++t) {
            path[t] = -1;
            dec[t] = -1;
            pt[t] = 0.0;
            qt[t] = 0.0;
            n_child[t] = 0;
        }
        for (int t = 1; t < T; ++t) {
            if (par[t] < 0 || par[t] >= t || tok[t] < 0 || tok[t] >= V) { rc = ORC_ERR; break; }
            n_child[par[t]]++;
        }
        for (int t = 0; t < T && rc == ORC_OK; ++t)
            if (n_child[t] > 0 && (drow[t] < 0 || drow[t] >= R)) rc = ORC_ERR;
        if (rc != ORC_OK) break;
        near_tie[b] = 0;
        fallback[b] = 0;
        int n_tgt = 0, n_dft = 0;
        const float *tgt_b = tgt + (size_t)b * T_cap * V;
        const float *dft_b = dft + (size_t)b * R * V;
        int stop = 0;
        int rows_of = -1;   /* node whose p (and q) are in p / q */
        int draw_resid = 0; /* draw from the residual (1) or from p_stop (0) */

        if (mode == ORC_REJECT_PATH) {
            int n_front = 1;
            front[0] = 0;
            while (n_front > 0) {
                stop = front[0];
                int n_next = 0;
                for (int i = 0; i < n_front; ++i) {
                    const int f = front[i];
                    if (n_child[f] == 0) continue;
                    softmax_row(V, tgt_b + (size_t)f * V, p);
                    softmax_row(V, dft_b + (size_t)drow[f] * V, q);
                    ++n_tgt;
                    ++n_dft;
                    rows_of = f;
                    for (int c = f + 1; c < T; ++c) {
                        if (par[c] != f) continue;
                        const int x = tok[c];
                        pt[c] = p[x];
                        qt[c] = q[x];
                        const double ratio = q[x] > 0.0 ? p[x] / q[x] : (p[x] > 0.0 ? INFINITY : 0.0);
                        const double u = (double)ub[c];
                        if (fabs(ratio - u) < ORC_NEAR_TIE) near_tie[b]++;
                        dec[c] = (int8_t)(u < ratio);
                        if (dec[c]) next[n_next++] = c;
                    }
                }
                for (int i = 1; i < n_next; ++i)
                    for (int j = i; j > 0 && next[j - 1] > next[j]; --j) {
                        const int x = next[j]; next[j] = next[j - 1]; next[j - 1] = x;
                    }
                memcpy(front, next, sizeof(int) * (size_t)n_next);
                n_front = n_next;
            }
            if (n_child[stop] > 0) {
                /* the stop node's rows were read when it was on the frontier */
                if (rows_of != stop) {
                    softmax_row(V, tgt_b + (size_t)stop * V, p);
                    softmax_row(V, dft_b + (size_t)drow[stop] * V, q);
                    ++n_tgt;
                    ++n_dft;
                }
                memcpy(r, p, sizeof(double) * (size_t)V);
                if (residual_step(V, r, q) > 0.0) {
                    draw_resid = 1;
                } else {
                    fallback[b] = 1;
                }
            }
        } else {
            int s = 0;
            for (;;) {
                int moved = 0, dead = 0, rejected = 0;
                if (n_child[s] > 0) {
                    softmax_row(V, tgt_b + (size_t)s * V, p);
                    softmax_row(V, dft_b + (size_t)drow[s] * V, q);
                    ++n_tgt;
                    ++n_dft;
                    rows_of = s;
                    memcpy(r, p, sizeof(double) * (size_t)V);
                    for (int c = s + 1; c < T; ++c) {
                        if (par[c] != s) continue;
                        const int x = tok[c];
                        pt[c] = p[x];
                        qt[c] = q[x];
                        if (dead) {
                            dec[c] = 0;
                            continue;
                        }
                        const double ratio = q[x] > 0.0 ? r[x] / q[x] : (r[x] > 0.0 ? INFINITY : 0.0);
                        const double u = (double)ub[c];
                        if (fabs(ratio - u) < ORC_NEAR_TIE) near_tie[b]++;
                        if (u < ratio) {
                            dec[c] = 1;
                            s = c;
                            moved = 1;
                            break;
                        }
                        dec[c] = 0;
                        rejected = 1;
                        if (!(residual_step(V, r, q) > 0.0)) {
                            dead = 1;
                            fallback[b] = 1;
                        }
                    }
                }
                if (moved) continue;
                stop = s;
                draw_resid = rejected && !dead;
                break;
            }
        }

        acc_len[b] = dep[stop];
        for (int cur = stop; cur >= 0; cur = par[cur]) path[dep[cur]] = cur;
        if (!draw_resid) {
            /* p_stop: a leaf's (or a fallback's) target row */
            if (rows_of != stop) {
                softmax_row(V, tgt_b + (size_t)stop * V, p);
                ++n_tgt;
            }
            memcpy(r, p, sizeof(double) * (size_t)V);
        }
        int near = 0;
        next_token[b] = sample_inverse_cdf(V, r, (double)u_final[b], &near);
        near_tie[b] += near;
        rows_tgt[b] = n_tgt;
        rows_dft[b] = n_dft;
    }
    free(p); free(q); free(r); free(front); free(next); free(n_child);
    return rc;
}

/*
 * Residual chain of one (p, q) pair, for pins of the closed form.
 * literal = 0: closed form, c_0 = 0, Z_0 = 1, c_{k+1} = c_k + Z_k,
 *   Z_{k+1} = sum max(0, p - c_{k+1} q); dist_k = max(0, p - c_k q) / Z_k.
 * literal = 1: the definition iterated ([ResiSpec] section 4):
 *   dist_0 = p, dist_{k+1} = max(0, dist_k - q) / sum max(0, dist_k - q).
 * dist is [K+1][V]; mass (may be NULL) gets Z_k (closed form) or the
 * normaliser of step k (literal, 1 for k = 0).  A zero normaliser stops the
 * chain and leaves the later rows zero; the number of rows filled is returned.
 */
int orc_residual_chain(int V, const double *p, const double *q, int K, int literal,
                       double *dist, double *mass)
{
    int filled = 0;
    if (!literal) {
        double c = 0.0, z = 1.0;
        for (int k = 0; k <= K; ++k) {
            if (k > 0) {
                c += z;
                z = residual_mass(V, p, q, c);
            }
            if (mass) mass[k] = z;
            if (!(z > 0.0)) break;
            for (int v = 0; v < V; ++v) {
                double w = p[v] - c * q[v];
                dist[(size_t)k * V + v] = w > 0.0 ? w / z : 0.0;
            }
            filled = k + 1;
        }
    } else {
        for (int v = 0; v < V; ++v) dist[v] = p[v];
        if (mass) mass[0] = 1.0;
        filled = 1;
        for (int k = 1; k <= K; ++k) {
            double z = 0.0;
            for (int v = 0; v < V; ++v) {
                double w = dist[(size_t)(k - 1) * V + v] - q[v];
                if (w > 0.0) z += w;
            }
            if (mass) mass[k] = z;
            if (!(z > 0.0)) break;
            for (int v = 0; v < V; ++v) {
                double w = dist[(size_t)(k - 1) * V + v] - q[v];
                dist[(size_t)k * V + v] = w > 0.0 ? w / z : 0.0;
            }
            filled = k + 1;
        }
    }
    for (int k = filled; k <= K; ++k)
        for (int v = 0; v < V; ++v) dist[(size_t)k * V + v] = 0.0;
    return filled;
}

/* ------------------------------------------------------------------------ */
/* 4. KV commit                                                              */
/* ------------------------------------------------------------------------ */

/*
 * Move the accepted path's K/V into contiguous cache slots ([ReDrafter] Step 6:
 * accepted tokens are appended to the context and the next step starts from
 * there).  For i = 1..acc_len: slot ctx + acc_path[i] -> slot ctx + i, for K and
 * V of every KV head; the root stays at slot ctx.  All sources are read before
 * any slot is written.  ctx_len[b] becomes ctx + acc_len + 1.
 * elem_bytes is 2 (bf16) or 4 (fp32); caches are [B][Hkv][cap][D].
 */
int orc_kv_compact(int elem_bytes, int B, int Hkv, int D, int cap, int T_cap, uint8_t *kc,
                   uint8_t *vc, int32_t *ctx_len, const int32_t *acc_len, const int32_t *acc_path)
{
    if (elem_bytes != 2 && elem_bytes != 4) return ORC_ERR;
    size_t row = (size_t)D * elem_bytes;
    uint8_t *tmp = (uint8_t *)malloc(row * (size_t)T_cap);
    if (!tmp) return ORC_ERR;
    for (int b = 0; b < B; ++b) {
        int ctx = ctx_len[b];
        int n = acc_len[b];
        const int32_t *path = acc_path + (size_t)b * T_cap;
        if (n < 0 || n >= T_cap || ctx + n + 1 > cap) { free(tmp); return ORC_ERR; }
        for (int i = 1; i <= n; ++i)
            if (path[i] < i || ctx + path[i] >= cap) { free(tmp); return ORC_ERR; }
        for (int g = 0; g < Hkv; ++g) {
            for (int which = 0; which < 2; ++which) {
                uint8_t *base = (which ? vc : kc) + ((size_t)b * Hkv + g) * (size_t)cap * row;
                for (int i = 1; i <= n; ++i)
                    memcpy(tmp + (size_t)i * row, base + (size_t)(ctx + path[i]) * row, row);
                for (int i = 1; i <= n; ++i)
                    memcpy(base + (size_t)(ctx + i) * row, tmp + (size_t)i * row, row);
            }
        }
        ctx_len[b] = ctx + n + 1;
    }
    free(tmp);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 5. Beam search pruning                                                    */
/* ------------------------------------------------------------------------ */

/* One candidate of the pruning step: its score and its index j * V + v in the
 * flattened (beam, token) grid. */
typedef struct {
    float s;
    long idx;
} orc_cand;

/* Descending score; equal scores keep the lower flattened index first. */
static int orc_cand_cmp(const void *a, const void *b)
{
    const orc_cand *x = (const orc_cand *)a, *y = (const orc_cand *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/*
 * Scoring and pruning of one beam-search step ([ReDrafter] section "Beam Search
 * During Inference", steps 1 and 3): every extension of beam j by token v gets
 * the cumulative log-probability score[j] + logp[j][v] (fp32, the precision
 * the selection is taken in), and the K_out best of the K_in * V extensions
 * become the next beams.  Ties go to the lower flattened index j * V + v (the
 * pages name no tie rule).  beam_score NULL means all zero (the first step,
 * with one row).  Outputs per sequence, best first: parent beam, token, score.
 * When hist_in is given ([B][K_in][len] token histories), hist_out
 * [B][K_out][len + 1] gets the parent's history followed by the new token.
 * All candidates are sorted in full; a library sort serves as the step.
 */
int orc_beam_topk(int B, int K_in, int K_out, int V, const float *logp, const float *beam_score,
                  int32_t *out_parent, int32_t *out_token, float *out_score,
                  const int32_t *hist_in, int len, int32_t *hist_out)
{
    if (B < 0 || K_in < 1 || V < 1 || K_out < 1 || (long)K_out > (long)K_in * V) return ORC_ERR;
    const long n = (long)K_in * V;
    orc_cand *c = (orc_cand *)malloc(sizeof(orc_cand) * (size_t)n);
    if (!c) return ORC_ERR;
    for (int b = 0; b < B; ++b) {
        for (int j = 0; j < K_in; ++j) {
            const float base = beam_score ? beam_score[(size_t)b * K_in + j] : 0.0f;
            const float *row = logp + ((size_t)b * K_in + j) * (size_t)V;
            for (int v = 0; v < V; ++v) {
                c[(long)j * V + v].s = base + row[v];
                c[(long)j * V + v].idx = (long)j * V + v;
            }
        }
        qsort(c, (size_t)n, sizeof(orc_cand), orc_cand_cmp);
        for (int k = 0; k < K_out; ++k) {
            const int j = (int)(c[k].idx / V), v = (int)(c[k].idx % V);
            out_parent[(size_t)b * K_out + k] = j;
            out_token[(size_t)b * K_out + k] = v;
            out_score[(size_t)b * K_out + k] = c[k].s;
            if (hist_in && hist_out) {
                const int32_t *src = hist_in + ((size_t)b * K_in + j) * (size_t)len;
                int32_t *dst = hist_out + ((size_t)b * K_out + k) * (size_t)(len + 1);
                for (int i = 0; i < len; ++i) dst[i] = src[i];
                dst[len] = v;
            }
        }
    }
    free(c);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 6. Dynamic tree selection                                                 */
/* ------------------------------------------------------------------------ */

typedef struct {
    float s;
    int i;
} orc_node_score;

static int orc_node_cmp(const void *a, const void *b)
{
    const orc_node_score *x = (const orc_node_score *)a, *y = (const orc_node_score *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

/*
 * Dynamic draft-tree selection under a node budget ([Drafters] page, the
 * EAGLE-2 paragraph: a branch is scored by the product of the drafter's
 * confidences along its path from the root, and the highest-scoring ones are
 * kept; [Clover] sizes its tree by a node budget).  Candidate i is node i + 1
 * with parent node cand_parent[i] in [0, i] (0 = root), token cand_token[i]
 * and log-confidence cand_logp[i] <= 0.  In log form the path score is
 * S(root) = 0, S(node) = S(parent) + logp, an fp32 sum taken from the root
 * down.  The N_keep candidates with the highest S are kept, the lower index on
 * ties; since logp <= 0 a parent scores at least as high as its child and has
 * the lower index, so the kept set holds every kept node's parent.  Output per
 * sequence: the kept candidates in their original order as an explicit
 * candidate list -- kept candidate k is node k + 1, keep_parent[k] the new
 * number of its parent node (0 = root) -- with keep_token, keep_src (original
 * candidate index) and keep_score (S).  Invalid input (a parent out of range,
 * logp > 0 or NaN) returns ORC_ERR.
 */
int orc_select_tree(int B, int N, int N_keep, const int32_t *cand_parent,
                    const int32_t *cand_token, const float *cand_logp, int32_t *keep_parent,
                    int32_t *keep_token, int32_t *keep_src, float *keep_score)
{
    if (B < 0 || N < 1 || N_keep < 1 || N_keep > N) return ORC_ERR;
    float *S = (float *)malloc(sizeof(float) * (size_t)(N + 1));
    orc_node_score *ns = (orc_node_score *)malloc(sizeof(orc_node_score) * (size_t)N);
    int *kept = (int *)malloc(sizeof(int) * (size_t)N);
    int *newnode = (int *)malloc(sizeof(int) * (size_t)(N + 1));
    if (!S || !ns || !kept || !newnode) {
        free(S); free(ns); free(kept); free(newnode);
        return ORC_ERR;
    }
    int rc = ORC_OK;
    for (int b = 0; b < B && rc == ORC_OK; ++b) {
        const int32_t *par = cand_parent + (size_t)b * N;
        const int32_t *tok = cand_token + (size_t)b * N;
        const float *lp = cand_logp + (size_t)b * N;
        S[0] = 0.0f;
        for (int i = 0; i < N; ++i) {
            if (par[i] < 0 || par[i] > i || !(lp[i] <= 0.0f)) { rc = ORC_ERR; break; }
            S[i + 1] = S[par[i]] + lp[i]; /* the parent node precedes node i + 1 */
        }
        if (rc != ORC_OK) break;
        for (int i = 0; i < N; ++i) {
            ns[i].s = S[i + 1];
            ns[i].i = i;
            kept[i] = 0;
        }
        qsort(ns, (size_t)N, sizeof(orc_node_score), orc_node_cmp);
        for (int k = 0; k < N_keep; ++k) kept[ns[k].i] = 1;
        newnode[0] = 0;
        int k = 0;
        for (int i = 0; i < N; ++i) {
            if (!kept[i]) continue;
            if (par[i] > 0 && !kept[par[i] - 1]) { rc = ORC_ERR; break; } /* cannot happen */
            newnode[i + 1] = k + 1;
            keep_parent[(size_t)b * N_keep + k] = newnode[par[i]];
            keep_token[(size_t)b * N_keep + k] = tok[i];
            keep_src[(size_t)b * N_keep + k] = i;
            keep_score[(size_t)b * N_keep + k] = S[i + 1];
            ++k;
        }
    }
    free(S); free(ns); free(kept); free(newnode);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* 7. Residual shaping (ResiSpec), literal reading, and path marginals       */
/* ------------------------------------------------------------------------ */

/*
 * GetProxy of [ResiSpec] section 5, "Practical Implementation: The ResiSpec
 * Algorithm", taken step by step.  p is the current target, q the draft and x0
 * the candidate just rejected (p(x0) < q(x0)).
 *   Step 1 (budget and projection): Z = |q(x0) - p(x0)|; r(x) = min(Z q(x), p(x)).
 *   Step 2 (capacity-aware redistribution): the deficit Z - sum r is moved onto
 *     tokens with p > r, never past p, so that sum r = Z.
 *   Step 3 (proxy): k = p - r, with k(x0) set to q(x0) (local alignment).
 * The page leaves open how the water-filling spreads the deficit and whether x0
 * takes part in Steps 1-2.  Readings:
 *   fill 0: the draft shape is raised until the budget is met,
 *           r(x) = min(lam Z q(x), p(x)) with the smallest lam >= 1 giving
 *           sum r = Z (bisection on lam down to fp64 resolution);
 *   fill 1: the deficit is spread in proportion to the remaining capacity
 *           p(x) - r(x) (one step; no token passes p).
 *   x0_mode 0: x0 is left out of Steps 1-2, r(x0) = 0.  This is the reading
 *           under which k is a distribution: sum k = 1 + r(x0) in general.
 *   x0_mode 1: x0 takes part in Steps 1-2 as written; k then sums to 1 + r(x0).
 * The residual the next candidate is tested against is that of the test with
 * the proxy, max(0, p - k) normalised: r off x0, 0 at x0 (p(x0) - q(x0) < 0).
 * Outputs r [V] and k [V]; *z_out = Z.  Returns ORC_ERR for a bad argument or
 * when q(x0) <= p(x0) (x0 cannot have been rejected).
 */
int orc_resispec_proxy(int V, const double *p, const double *q, int x0, int fill, int x0_mode,
                       double *r, double *k, double *z_out)
{
    if (V < 1 || x0 < 0 || x0 >= V || (fill != 0 && fill != 1) ||
        (x0_mode != 0 && x0_mode != 1))
        return ORC_ERR;
    if (!(q[x0] > p[x0])) return ORC_ERR;
    const double Z = fabs(q[x0] - p[x0]);
    /* Step 1 */
    double sum = 0.0;
    for (int v = 0; v < V; ++v) {
        r[v] = (v == x0 && x0_mode == 0) ? 0.0 : fmin(Z * q[v], p[v]);
        sum += r[v];
    }
    /* Step 2 */
    if (sum < Z) {
        if (fill == 0) {
            double lo = 1.0, hi = 2.0;
            for (;;) {
                double s = 0.0;
                for (int v = 0; v < V; ++v)
                    if (!(v == x0 && x0_mode == 0)) s += fmin(hi * Z * q[v], p[v]);
                if (s >= Z || hi > 1e300) break;
                lo = hi;
                hi *= 2.0;
            }
            for (int it = 0; it < 2000 && lo < hi; ++it) {
                double mid = 0.5 * (lo + hi);
                if (!(mid > lo && mid < hi)) break;
                double s = 0.0;
                for (int v = 0; v < V; ++v)
                    if (!(v == x0 && x0_mode == 0)) s += fmin(mid * Z * q[v], p[v]);
                if (s < Z) lo = mid;
                else hi = mid;
            }
            for (int v = 0; v < V; ++v)
                r[v] = (v == x0 && x0_mode == 0) ? 0.0 : fmin(hi * Z * q[v], p[v]);
        } else {
            double cap = 0.0;
            for (int v = 0; v < V; ++v)
                if (!(v == x0 && x0_mode == 0)) cap += p[v] - r[v];
            const double deficit = Z - sum;
            if (cap > 0.0)
                for (int v = 0; v < V; ++v)
                    if (!(v == x0 && x0_mode == 0)) r[v] += deficit * (p[v] - r[v]) / cap;
        }
    }
    /* Step 3 */
    for (int v = 0; v < V; ++v) k[v] = p[v] - r[v];
    k[x0] = q[x0];
    *z_out = Z;
    return ORC_OK;
}

/* Path-marginal recursion: adds `weight` times the output distribution of the
 * remaining n candidates, starting from target p, to out. */
static int marginal_rec(int V, int n, const double *p, const double *q, int shape, int fill,
                        int x0_mode, double weight, double *out, double *scratch)
{
    if (n == 0) {
        for (int v = 0; v < V; ++v) out[v] += weight * p[v];
        return ORC_OK;
    }
    double *pn = scratch;            /* the residual after rejecting x */
    double *k = scratch + V;         /* the proxy (shape 1) */
    double *deeper = scratch + 2 * V;
    for (int x = 0; x < V; ++x) {
        if (!(q[x] > 0.0)) continue;  /* never proposed */
        const double a = p[x] >= q[x] ? 1.0 : p[x] / q[x];
        out[x] += weight * q[x] * a;   /* x proposed and accepted */
        if (a >= 1.0) continue;
        const double w_rej = weight * q[x] * (1.0 - a);
        double z = 0.0;
        if (shape == 0) {
            /* [ResiSpec] section 4: norm(max(0, p - q)) */
            for (int v = 0; v < V; ++v) {
                const double d = p[v] - q[v];
                pn[v] = d > 0.0 ? d : 0.0;
                z += pn[v];
            }
        } else {
            double Z;
            if (orc_resispec_proxy(V, p, q, x, fill, x0_mode, pn, k, &Z) != ORC_OK) return ORC_ERR;
            for (int v = 0; v < V; ++v) {
                const double d = p[v] - k[v];
                pn[v] = d > 0.0 ? d : 0.0;
                z += pn[v];
            }
        }
        if (!(z > 0.0)) return ORC_ERR;
        for (int v = 0; v < V; ++v) pn[v] /= z;
        if (marginal_rec(V, n - 1, pn, q, shape, fill, x0_mode, w_rej, out, deeper) != ORC_OK)
            return ORC_ERR;
    }
    return ORC_OK;
}

/*
 * Output distribution of sequential verification of n candidates drawn i.i.d.
 * from q, by summing every path ([ResiSpec] Appendix B.1): candidate i is
 * accepted with probability min(1, p_{i-1}(x)/q(x)) against the current target
 * p_{i-1} (p_0 = p); after a rejection the target becomes the next residual;
 * after n rejections the token is drawn from p_n.  shape 0: the residual of
 * section 4, norm(max(0, p - q)).  shape 1: the residual of the proxy test of
 * section 5 (orc_resispec_proxy with `fill` and `x0_mode`); the test itself is
 * unchanged, since k(x) = q(x) at the candidate.  Every path is enumerated:
 * V^n of them (n <= 8).  out [V].
 */
int orc_multicand_marginal(int V, int n, const double *p, const double *q, int shape, int fill,
                           int x0_mode, double *out)
{
    if (V < 1 || n < 0 || n > 8 || (shape != 0 && shape != 1)) return ORC_ERR;
    double *scratch = (double *)malloc(sizeof(double) * (size_t)V * 2 * (size_t)(n + 1) + 8);
    if (!scratch) return ORC_ERR;
    for (int v = 0; v < V; ++v) out[v] = 0.0;
    int rc = marginal_rec(V, n, p, q, shape, fill, x0_mode, 1.0, out, scratch);
    free(scratch);
    return rc;
}
