/*
 * tmv_oracle.c -- plain, slow CPU oracle for the teacher's tree-verification step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file: only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no source, header, table or helper with the HIP library.
 *
 * Arithmetic: fp64 for every floating-point quantity (bf16 inputs are widened exactly),
 * exact integers (64/128-bit) everywhere else.  Loops follow the definitions directly;
 * nothing is blocked, fused or reordered.
 *
 * Sources (pages of the reference set):
 *   [EP-pt]  "EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend NPUs",
 *            Portuguese technical summary, section 2 (methodology and architecture).
 *   [EP-zh]  the independently written Chinese technical summary of the same paper,
 *            section 2.1 (branchable KV cache, commit modes), 2.2 (accelerator-safe tree
 *            tensors: virtual root row 0, ancestor table, invariant checks), 2.3 (fused
 *            tree-masked teacher pass, a node sees its ancestors and itself).
 *   [SDH]    "Speculative Decoding Hierarquico: Medusa, EAGLE-2 e Multi-Token Prediction",
 *            sections on modified rejection sampling (acceptance min(1,p/q), residual
 *            max(0,p-q) normalised, the identity min(q,p)+max(0,p-q)=p), on Medusa trees
 *            (tree attention mask; the longest valid path is kept) and its FAQ (a
 *            correction token is drawn when every guess is refused).
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 *   - ancestor table orientation: anc[i][k] = parent^k(i), saturating at the root 0,
 *     width D_max+1; depth(i) = number of hops from i to 0.
 *   - "validity closure": a valid node's parent is valid (or is the root).
 *   - error precedence: the smallest nonzero code over the nodes of a sequence wins and
 *     the whole sequence becomes inert (all-zero rows).
 *   - argmax ties go to the smallest token; among equally deep matched nodes the
 *     smallest node id wins; the bonus token after a full accept is the teacher's
 *     choice at the last accepted node.
 *   - sampling on a tree: children of a node are tried in ascending id, each by the
 *     chain rule against the current residual, kept in threshold form; exact integer
 *     fixed point (below).
 *   - RNG: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11), key {seed, (step<<32)|b},
 *     block n uses counter {n+1,0,0,0}; draw n is 64-bit word n%4 of block n/4.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

enum {
    REF_OK = 0, REF_ERR_ARG = 1, REF_ERR_RANGE = 2, REF_ERR_CYCLE = 3, REF_ERR_DEPTH = 4,
    REF_ERR_CLOSURE = 5, REF_ERR_INPUT = 6
};
enum { REF_PARENTS_VROOT = 0, REF_PARENTS_NEG1 = 1 };
enum { REF_F32 = 0, REF_BF16 = 1 };

typedef unsigned __int128 u128;

/* smallest nonzero code wins */
static int merge_code(int a, int b)
{
    if (a == REF_OK) return b;
    if (b == REF_OK) return a;
    return a < b ? a : b;
}

/* exact widening of one element of a f32 or bf16 array */
static double load_elem(const void *base, int dtype, int64_t idx)
{
    if (dtype == REF_F32) return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------------------
 * Tree tensors [EP-zh §2.2, EP-pt §2]: parents remapped onto the virtual root row 0,
 * ancestor table whose entries all lie in [0, M_b], range / acyclicity / depth /
 * validity-closure checks, per-sequence status.
 *
 *   parents  VROOT: [B][M_max+1], column 0 ignored, node i's parent in [0, M_b]
 *            NEG1 : [B][M_max], node r (0-based) has parent -1 (the root) or 0..M_b-1;
 *                   remapped here: node r -> r+1, parent -1 -> 0, parent v -> v+1
 *   valid    [B][M_max+1] or NULL (all of 1..M_b valid)
 *   anc      [B][M_max+1][D_max+1]   depth [B][M_max+1]   status [B]
 * ---------------------------------------------------------------------------------- */
int tmvref_build_ancestors(int B, int M_max, int D_max, int parent_format,
                           const int32_t *parents, const uint8_t *valid,
                           const int32_t *n_nodes,
                           int32_t *anc, int32_t *depth, int32_t *status)
{
    if (B < 0 || M_max < 0 || D_max < 0) return REF_ERR_ARG;
    const int W = D_max + 1, R = M_max + 1;
    int32_t *par = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
    uint8_t *ok = (uint8_t *)malloc((size_t)R);
    if (!par || !ok) { free(par); free(ok); return REF_ERR_ARG; }

    for (int b = 0; b < B; ++b) {
        int32_t *A = anc + (int64_t)b * R * W;
        int32_t *Dp = depth + (int64_t)b * R;
        for (int64_t e = 0; e < (int64_t)R * W; ++e) A[e] = 0;
        for (int i = 0; i < R; ++i) Dp[i] = 0;

        const int M = n_nodes[b];
        if (M < 0 || M > M_max) { status[b] = REF_ERR_RANGE; continue; }

        /* parent of every node in virtual-root form; -1 marks a value that cannot be
         * remapped (a NEG1 entry below -1), which the walk reports as RANGE */
        for (int i = 1; i <= M; ++i) {
            if (parent_format == REF_PARENTS_VROOT) {
                par[i] = parents[(int64_t)b * R + i];
            } else {
                int32_t raw = parents[(int64_t)b * M_max + (i - 1)];
                par[i] = raw == -1 ? 0 : (raw < -1 ? -1 : raw + 1);
            }
            ok[i] = valid ? (valid[(int64_t)b * R + i] != 0) : 1;
        }

        int st = REF_OK;
        for (int i = 1; i <= M; ++i) {
            if (!ok[i]) continue;
            int code = REF_OK, d = 0, h = i, k = 0;
            for (;;) {
                if (k <= D_max) A[(int64_t)i * W + k] = h;
                int p = par[h];
                if (p < 0 || p > M) { code = REF_ERR_RANGE; break; }
                if (p == 0) { d = k + 1; break; }
                if (!ok[p]) { code = REF_ERR_CLOSURE; break; }
                h = p;
                ++k;
                /* M hops without reaching the root revisit a node: a cycle */
                if (k >= M) { code = REF_ERR_CYCLE; break; }
            }
            if (code == REF_OK && d > D_max) code = REF_ERR_DEPTH;
            Dp[i] = d;
            st = merge_code(st, code);
        }
        if (st != REF_OK) {
            for (int64_t e = 0; e < (int64_t)R * W; ++e) A[e] = 0;
            for (int i = 0; i < R; ++i) Dp[i] = 0;
        }
        status[b] = st;
    }
    free(par);
    free(ok);
    return REF_OK;
}

/* ------------------------------------------------------------------------------------
 * Tree-masked attention [EP-zh §2.3, EP-pt §2, SDH Medusa section]: node i, query
 * head h attends to the committed prefix [0,P_b) plus the cache slots of its own
 * ancestor path including itself; node j's K/V live at slot P_b + j - 1.
 * GQA: kv head = h / (Hq/Hkv).  Scores, softmax and the weighted sum in fp64.
 *
 *   q        [B][M_max][Hq][d] (element strides q_stride[0..2], d contiguous); row r = node r+1
 *   k, v     [B][Hkv][L_cap][d] (element strides kv_stride[0..2], d contiguous)
 *   out      dense fp64 [B][M_max][Hq][d]; rows of inert nodes are 0
 *   row_select [B][M_max] or NULL: rows with 0 are skipped (left 0) -- a filter only
 *   status   in/out: a prefix that does not fit (P_b<0 or P_b+M_b>L_cap) sets INPUT
 * ---------------------------------------------------------------------------------- */
int tmvref_tree_attention(int B, int M_max, int D_max, int Hq, int Hkv, int d, int dtype,
                          const void *q, const int64_t *q_stride,
                          const void *k, const void *v, const int64_t *kv_stride, int L_cap,
                          const int32_t *prefix_len, const int32_t *n_nodes,
                          const int32_t *anc, const int32_t *depth, int32_t *status,
                          double scale, const uint8_t *row_select, double *out)
{
    if (B < 0 || M_max < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d <= 0) return REF_ERR_ARG;
    const int g = Hq / Hkv, W = D_max + 1, R = M_max + 1;
    const int64_t out_elems = (int64_t)B * M_max * Hq * d;
    for (int64_t e = 0; e < out_elems; ++e) out[e] = 0.0;

    int64_t *cols = (int64_t *)malloc(sizeof(int64_t) * ((size_t)L_cap + 1));
    double *s = (double *)malloc(sizeof(double) * ((size_t)L_cap + 1));
    if (!cols || !s) { free(cols); free(s); return REF_ERR_ARG; }

    for (int b = 0; b < B; ++b) {
        if (status[b] != REF_OK) continue;
        const int P = prefix_len[b], M = n_nodes[b];
        if (P < 0 || (int64_t)P + M > L_cap) { status[b] = REF_ERR_INPUT; continue; }
        for (int j = 1; j <= M; ++j) {
            const int dep = depth[(int64_t)b * R + j];
            if (dep < 1) continue;                      /* inert row */
            if (row_select && !row_select[(int64_t)b * M_max + (j - 1)]) continue;

            /* visible columns: the whole prefix, then the path j -> ... -> depth-1 node */
            int64_t nc = 0;
            for (int t = 0; t < P; ++t) cols[nc++] = t;
            for (int kk = 0; kk < dep; ++kk) {
                int node = anc[((int64_t)b * R + j) * W + kk];
                cols[nc++] = (int64_t)P + node - 1;
            }

            for (int h = 0; h < Hq; ++h) {
                const int kvh = h / g;
                const int64_t qoff = b * q_stride[0] + (int64_t)(j - 1) * q_stride[1] + h * q_stride[2];
                double mx = -INFINITY;
                for (int64_t c = 0; c < nc; ++c) {
                    const int64_t koff = b * kv_stride[0] + kvh * kv_stride[1] + cols[c] * kv_stride[2];
                    double dot = 0.0;
                    for (int e = 0; e < d; ++e)
                        dot += load_elem(q, dtype, qoff + e) * load_elem(k, dtype, koff + e);
                    s[c] = scale * dot;
                    if (s[c] > mx) mx = s[c];
                }
                double den = 0.0;
                for (int64_t c = 0; c < nc; ++c) { s[c] = exp(s[c] - mx); den += s[c]; }
                double *o = out + (((int64_t)b * M_max + (j - 1)) * Hq + h) * d;
                for (int64_t c = 0; c < nc; ++c) {
                    const int64_t voff = b * kv_stride[0] + kvh * kv_stride[1] + cols[c] * kv_stride[2];
                    const double w = s[c] / den;
                    for (int e = 0; e < d; ++e) o[e] += w * load_elem(v, dtype, voff + e);
                }
            }
        }
    }
    free(cols);
    free(s);
    return REF_OK;
}

/* ------------------------------------------------------------------------------------
 * Greedy acceptance [SDH Medusa section: the longest valid path is kept; greedy-only
 * teacher decoding is the baseline of EP-pt §4].
 *   t(u) = argmax_x logits[b][u][x] (smallest x on ties) for u = 0 and every live node;
 *   node i matches iff every edge on its path matches: tokens[c] == t(parent(c));
 *   a* = deepest matching node (smallest id on ties; 0 if none);
 *   accept_len = depth(a*), path = ids root->leaf, next_token = t(a*).
 * NaN in a scanned row, or a live node's token outside [0,V), sets INPUT.
 *   tokens  [B][M_max+1] (column 0 ignored);  logits row (b,u) at b*stride_b + u*stride_row
 * ---------------------------------------------------------------------------------- */
int tmvref_accept_greedy(int B, int M_max, int D_max, int V, const int32_t *tokens,
                         int row_dtype, const void *logits, int64_t stride_b, int64_t stride_row,
                         const int32_t *n_nodes, const int32_t *anc, const int32_t *depth,
                         int32_t *status, int32_t *accept_len, int32_t *path, int32_t *next_token)
{
    if (B < 0 || M_max < 0 || D_max < 0 || V <= 0) return REF_ERR_ARG;
    const int W = D_max + 1, R = M_max + 1;
    int32_t *t = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
    if (!t) return REF_ERR_ARG;

    for (int b = 0; b < B; ++b) {
        accept_len[b] = 0;
        next_token[b] = 0;
        for (int j = 0; j < D_max; ++j) path[(int64_t)b * D_max + j] = 0;
        if (status[b] != REF_OK) continue;
        const int M = n_nodes[b];
        const int32_t *Dp = depth + (int64_t)b * R;
        const int32_t *A = anc + (int64_t)b * R * W;
        const int32_t *tok = tokens + (int64_t)b * R;

        int bad = 0;
        for (int u = 0; u <= M && !bad; ++u) {
            if (u > 0 && Dp[u] < 1) continue;
            if (u > 0 && (tok[u] < 0 || tok[u] >= V)) { bad = 1; break; }
            const int64_t base = b * stride_b + u * stride_row;
            double best = 0.0;
            int arg = -1;
            for (int x = 0; x < V; ++x) {
                double val = load_elem(logits, row_dtype, base + x);
                if (isnan(val)) { bad = 1; break; }
                if (arg < 0 || val > best) { best = val; arg = x; }
            }
            t[u] = arg;
        }
        if (bad) { status[b] = REF_ERR_INPUT; continue; }

        int star = 0, star_depth = 0;
        for (int i = 1; i <= M; ++i) {
            const int dep = Dp[i];
            if (dep < 1) continue;
            int match = 1;
            for (int kk = 0; kk < dep; ++kk) {
                int child = A[(int64_t)i * W + kk], par = A[(int64_t)i * W + kk + 1];
                if (tok[child] != t[par]) { match = 0; break; }
            }
            if (match && dep > star_depth) { star = i; star_depth = dep; }
        }
        accept_len[b] = star_depth;
        for (int j = 0; j < star_depth; ++j)
            path[(int64_t)b * D_max + j] = A[(int64_t)star * W + (star_depth - 1 - j)];
        next_token[b] = t[star];
    }
    free(t);
    return REF_OK;
}

/* ------------------------------------------------------------------------------------
 * LM-head logits in fp64 (the teacher's projection whose argmax the greedy rule takes)
 * [SDH roofline section: decode reads the LM-head weights once per step; the argmax of
 * each verified row's logits is the teacher's greedy choice of the Medusa section].
 *   logits[i][x] = sum_k h[i][k] * w[x][k], h and w bf16 bit patterns widened exactly;
 *   bound[i][x]  = sum_k |h[i][k] * w[x][k]| (the scale of the rounding error any fp32
 *                  accumulation order can make: at most K * 2^-24 * bound), or NULL.
 *   h [n][K] contiguous, w row x at x * w_stride.
 * ---------------------------------------------------------------------------------- */
int tmvref_lm_head_logits(int n, int K, int V, const uint16_t *h, const uint16_t *w, int64_t w_stride,
                          double *logits, double *bound)
{
    if (n < 0 || K < 0 || V < 0 || w_stride < K) return REF_ERR_ARG;
    for (int i = 0; i < n; ++i) {
        for (int x = 0; x < V; ++x) {
            double acc = 0.0, mag = 0.0;
            for (int k = 0; k < K; ++k) {
                const double pr = load_elem(h, REF_BF16, (int64_t)i * K + k) *
                                  load_elem(w, REF_BF16, (int64_t)x * w_stride + k);
                acc += pr;
                mag += fabs(pr);
            }
            logits[(int64_t)i * V + x] = acc;
            if (bound) bound[(int64_t)i * V + x] = mag;
        }
    }
    return REF_OK;
}

/* ------------------------------------------------------------------------------------
 * Philox4x64-10 (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3", SC'11):
 * 10 rounds of two 64x64->128 multiplies with the published multipliers and Weyl key
 * increments.
 * ---------------------------------------------------------------------------------- */
static void philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4])
{
    uint64_t x0 = ctr_in[0], x1 = ctr_in[1], x2 = ctr_in[2], x3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        u128 p0 = (u128)0xD2E7470EE14C6C93ULL * x0;
        u128 p1 = (u128)0xCA5A826395121157ULL * x2;
        uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
        uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
        x0 = hi1 ^ x1 ^ k0;
        x1 = lo1;
        x2 = hi0 ^ x3 ^ k1;
        x3 = lo0;
        k0 += 0x9E3779B97F4A7C15ULL;
        k1 += 0xBB67AE8584CAA73BULL;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* the n-th 64-bit word of the stream with the given key */
static uint64_t philox_word(uint64_t seed, uint64_t stream, uint64_t n)
{
    uint64_t ctr[4] = { n / 4 + 1, 0, 0, 0 }, key[2] = { seed, stream }, out[4];
    philox4x64_10(ctr, key, out);
    return out[n % 4];
}

/* exported for the RNG pin: n words of stream {seed, stream} from word 0 */
void tmvref_philox_words(uint64_t seed, uint64_t stream, int64_t n, uint64_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = philox_word(seed, stream, (uint64_t)i);
}

/* ------------------------------------------------------------------------------------
 * Sampling acceptance [SDH, modified rejection sampling and its FAQ], extended to trees
 * by trying a node's children one after another against the current residual.
 *
 * Threshold form (mathematics; our reading of how the residual is iterated): at node u
 * the teacher row p and the draft row q stay fixed, so the distribution left after j
 * refusals is (p - c_j q)+ normalised, with c_0 = 0 and c_{j+1} = c_j + sum (p - c_j q)+.
 * (One refusal maps r = (p - c q)+ / Z to (r - q)+ normalised, and where it is positive
 * r - q equals (p - (c + Z) q) / Z.)
 *
 * Exact integer fixed point (our reading; the pages give real-valued formulas):
 *   WP(y) = floor(p[u][y] * 2^31), WQ(y) = floor(q[u][y] * 2^31); SP, SQ their exact
 *   sums.  At a node without children q is not read and SQ = 1, WQ = 0.
 *   State (M, T): R(y) = max(0, WP(y) * SQ - WQ(y) * M), T = sum R > 0; M = 0 on arrival
 *   (R = WP * SQ, i.e. p itself; M / SP plays c_j).
 *   Child c with token x, U = word >> 40 (24 bits):
 *     accept  iff  U * WQ(x) * T < R(x) * SQ * 2^24     (i.e. u * q(x) < p_cur(x))
 *     refuse  ->   M' = M + floor(T / SQ); the state becomes (M', sum R_M') unless that
 *                  sum is 0 (empty residual: the state is kept)
 *   Draw with word: t = floor((word >> 32) * T / 2^32), the token is the least x with
 *   sum_{y<=x} R(y) > t.  Stop at the first node whose children are all refused
 *   (correction) or at a node without children (bonus), drawing next_token there.
 *   Bounds: V <= 2^24 and M_max * V < 2^33 give SP, SQ < 2^55, M < 2^64, R < 2^87,
 *   T < 2^111 and both sides of the accept test < 2^166.
 * Rows visited with entries outside [0,1] / non-finite, a zero p row, a zero q row
 * under a node with children, or a live token outside [0,V) set INPUT.
 *   p, q  [B][M_max+1][V] fp32 (row u = distribution after node u; row 0 after the prefix)
 * ---------------------------------------------------------------------------------- */

/* quantise row u of a distribution tensor; returns 0 on a malformed entry */
static int quantise_row(const float *row, int V, uint64_t *w, uint64_t *sum)
{
    uint64_t s = 0;
    for (int x = 0; x < V; ++x) {
        double val = (double)row[x];
        if (!(val >= 0.0 && val <= 1.0)) return 0;      /* also rejects NaN */
        w[x] = (uint64_t)floor(val * 2147483648.0);
        s += w[x];
    }
    *sum = s;
    return 1;
}

static u128 residual_at(uint64_t wp, uint64_t wq, uint64_t SQ, uint64_t M)
{
    u128 a = (u128)wp * SQ, c = (u128)wq * M;
    return a > c ? a - c : 0;
}

/* a * b as three little-endian 64-bit words */
static void mul_u128_u64(u128 a, uint64_t b, uint64_t out[3])
{
    u128 lo = (u128)(uint64_t)a * b, hi = (u128)(uint64_t)(a >> 64) * b;
    u128 mid = (lo >> 64) + (uint64_t)hi;
    out[0] = (uint64_t)lo;
    out[1] = (uint64_t)mid;
    out[2] = (uint64_t)(hi >> 64) + (uint64_t)(mid >> 64);
}

static int accept_test(uint64_t u24, uint64_t wq_x, u128 T, u128 r_x, uint64_t SQ)
{
    uint64_t l[3], r[3];
    mul_u128_u64(T, u24 * wq_x, l);
    mul_u128_u64(r_x << 24, SQ, r);
    for (int i = 2; i >= 0; --i)
        if (l[i] != r[i]) return l[i] < r[i];
    return 0;
}

/* floor(word_hi * T / 2^32) without overflow for T < 2^127 */
static u128 draw_target(uint64_t word, u128 T)
{
    const uint64_t wh = word >> 32;
    return (u128)wh * (T >> 32) + (((u128)wh * (uint64_t)(T & 0xffffffffu)) >> 32);
}

/* exported for pins: the integer accept test and the inverse-CDF draw on one row */
int tmvref_sample_accept_test(uint64_t u24, uint64_t wq_x, uint64_t T_lo, uint64_t T_hi, uint64_t r_lo,
                              uint64_t r_hi, uint64_t SQ)
{
    return accept_test(u24, wq_x, ((u128)T_hi << 64) | T_lo, ((u128)r_hi << 64) | r_lo, SQ);
}

int tmvref_sample_draw(const uint64_t *w_lo, const uint64_t *w_hi, int V, uint64_t word)
{
    u128 T = 0, c = 0;
    for (int x = 0; x < V; ++x) T += ((u128)w_hi[x] << 64) | w_lo[x];
    const u128 t = draw_target(word, T);
    for (int x = 0; x < V; ++x) {
        c += ((u128)w_hi[x] << 64) | w_lo[x];
        if (c > t) return x;
    }
    return V - 1;   /* unreachable: t < T */
}

int tmvref_accept_sample(int B, int M_max, int D_max, int V, const int32_t *tokens,
                         const float *p, const float *q, uint64_t seed, uint64_t step,
                         const int32_t *n_nodes, const int32_t *anc, const int32_t *depth,
                         int32_t *status, int32_t *accept_len, int32_t *path, int32_t *next_token)
{
    if (B < 0 || M_max < 0 || D_max < 0 || V <= 0 || V > (1 << 24)) return REF_ERR_ARG;
    if ((uint64_t)M_max * (uint64_t)V >= (1ull << 33)) return REF_ERR_ARG;
    const int W = D_max + 1, R = M_max + 1;
    uint64_t *wp = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)V);
    uint64_t *wq = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)V);
    int32_t *kids = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
    if (!wp || !wq || !kids) { free(wp); free(wq); free(kids); return REF_ERR_ARG; }

    for (int b = 0; b < B; ++b) {
        accept_len[b] = 0;
        next_token[b] = 0;
        for (int j = 0; j < D_max; ++j) path[(int64_t)b * D_max + j] = 0;
        if (status[b] != REF_OK) continue;
        const int M = n_nodes[b];
        const int32_t *Dp = depth + (int64_t)b * R;
        const int32_t *A = anc + (int64_t)b * R * W;
        const int32_t *tok = tokens + (int64_t)b * R;
        const uint64_t stream = (step << 32) | (uint64_t)(uint32_t)b;
        const float *pb = p + (int64_t)b * R * V, *qb = q + (int64_t)b * R * V;

        int bad = 0;
        for (int i = 1; i <= M; ++i)
            if (Dp[i] >= 1 && (tok[i] < 0 || tok[i] >= V)) bad = 1;

        uint64_t n = 0;
        int u = 0, acc = 0, out_tok = 0;
        while (!bad) {
            int nk = 0;
            for (int c = 1; c <= M; ++c)
                if (Dp[c] >= 1 && A[(int64_t)c * W + 1] == u) kids[nk++] = c;
            uint64_t SP = 0, SQ = 1;
            if (!(quantise_row(pb + (int64_t)u * V, V, wp, &SP) && SP > 0)) { bad = 1; break; }
            if (nk > 0) {
                if (!(quantise_row(qb + (int64_t)u * V, V, wq, &SQ) && SQ > 0)) { bad = 1; break; }
            } else {
                memset(wq, 0, sizeof(uint64_t) * (size_t)V);
            }
            uint64_t Mc = 0;
            u128 T = (u128)SP * SQ;
            int moved = 0;
            for (int ci = 0; ci < nk; ++ci) {
                const int c = kids[ci], x = tok[c];
                const uint64_t U = philox_word(seed, stream, n++) >> 40;
                if (accept_test(U, wq[x], T, residual_at(wp[x], wq[x], SQ, Mc), SQ)) {
                    path[(int64_t)b * D_max + acc] = c;
                    ++acc;
                    u = c;
                    moved = 1;
                    break;
                }
                const uint64_t Mn = Mc + (uint64_t)(T / SQ);
                u128 Tn = 0;
                for (int y = 0; y < V; ++y) Tn += residual_at(wp[y], wq[y], SQ, Mn);
                if (Tn > 0) { Mc = Mn; T = Tn; }
            }
            if (moved) continue;
            const u128 t = draw_target(philox_word(seed, stream, n++), T);
            u128 cum = 0;
            for (int y = 0; y < V; ++y) {
                cum += residual_at(wp[y], wq[y], SQ, Mc);
                if (cum > t) { out_tok = y; break; }
            }
            break;
        }
        if (bad) {
            status[b] = REF_ERR_INPUT;
            for (int j = 0; j < D_max; ++j) path[(int64_t)b * D_max + j] = 0;
            continue;
        }
        accept_len[b] = acc;
        next_token[b] = out_tok;
    }
    free(wp); free(wq); free(kids);
    return REF_OK;
}

/* ------------------------------------------------------------------------------------
 * Path-index commit with prefix sharing [EP-zh §2.1, EP-pt §2]: the committed prefix
 * is left untouched; for j < A_b the row at slot P_b + path[j] - 1 is copied to slot
 * P_b + j (all sources are read before any destination is written), for every layer,
 * KV head, and both K and V.  new_len = P_b + A_b.  A sequence whose status is not OK,
 * or whose lengths / path do not fit, moves nothing and keeps new_len = P_b (a fit
 * problem also sets INPUT).
 *   caches [n_layers][B][Hkv][L_cap][d], element strides stride[0..3], d contiguous
 * ---------------------------------------------------------------------------------- */
int tmvref_commit(int n_layers, int B, int Hkv, int d, int L_cap, int M_max, int D_max,
                  int elem_bytes, void *k_cache, void *v_cache, const int64_t *stride,
                  const int32_t *prefix_len, const int32_t *n_nodes,
                  const int32_t *accept_len, const int32_t *path,
                  int32_t *status, int32_t *new_len)
{
    if (n_layers < 0 || B < 0 || Hkv <= 0 || d <= 0 || D_max < 0 || (elem_bytes != 2 && elem_bytes != 4))
        return REF_ERR_ARG;
    (void)M_max;    /* kept for symmetry with the device entry point */
    const size_t row_bytes = (size_t)d * elem_bytes;
    uint8_t *snap = (uint8_t *)malloc(row_bytes * ((size_t)D_max + 1));
    if (!snap) return REF_ERR_ARG;

    for (int b = 0; b < B; ++b) {
        const int P = prefix_len[b];
        new_len[b] = P;
        if (status[b] != REF_OK) continue;
        const int M = n_nodes[b], A = accept_len[b];
        int fits = P >= 0 && (int64_t)P + M <= L_cap && A >= 0 && A <= D_max && A <= M;
        for (int j = 0; fits && j < A; ++j) {
            int node = path[(int64_t)b * D_max + j];
            if (node < 1 || node > M) fits = 0;
        }
        if (!fits) { status[b] = REF_ERR_INPUT; continue; }
        new_len[b] = P + A;

        for (int layer = 0; layer < n_layers; ++layer)
            for (int h = 0; h < Hkv; ++h)
                for (int which = 0; which < 2; ++which) {
                    uint8_t *base = (uint8_t *)(which == 0 ? k_cache : v_cache);
                    const int64_t head_off = layer * stride[0] + b * stride[1] + h * stride[2];
                    for (int j = 0; j < A; ++j) {
                        int64_t src = (int64_t)P + path[(int64_t)b * D_max + j] - 1;
                        memcpy(snap + (size_t)j * row_bytes,
                               base + (head_off + src * stride[3]) * elem_bytes, row_bytes);
                    }
                    for (int j = 0; j < A; ++j) {
                        int64_t dst = (int64_t)P + j;
                        memcpy(base + (head_off + dst * stride[3]) * elem_bytes,
                               snap + (size_t)j * row_bytes, row_bytes);
                    }
                }
    }
    free(snap);
    return REF_OK;
}

/* ------------------------------------------------------------------------------------
 * Best-first prefix tree from per-position draft marginals [BAS, sections 1-3]
 * (BAS = the BASTION technical summary: block-diffusion marginals, path scores,
 * best-first expansion, budget controller).
 *   q[b][k][x] = q_{k+1}(x), the drafter's marginal for position k+1 (k = 0..D-1).
 *   A node at depth d is a token tuple (x_1..x_d) with path score
 *   rho = q_1(x_1) * ... * q_d(x_d) (section 1).  Best-first expansion adds, again and
 *   again, the node with the largest score among those whose parent is already in the
 *   tree (section 2).  The surrogate of a tree is the sum of its scores (section 2); the
 *   controller keeps growing the tree while S(n) = A(n) * L_AR / C(n) rises (section 3).
 * Readings (ours; the pages give no tie rule, arithmetic or cost model):
 *   - rho in fp64, in depth order: rho(child) = rho(parent) * (double)q.
 *   - ranks per position by (q descending, token ascending); equal scores go to the
 *     shallower node, then to the lexicographically smaller rank tuple.  Only the N_max
 *     best tokens of a position can enter a tree of N_max nodes (any other token is
 *     beaten by N_max siblings), so candidates are drawn from those ranks.
 *   - node ids in the order the nodes are added (1..n); parents in virtual-root form.
 *   - controller: A(n) = sum of the first n scores, S(n) = A(n) * l_ar / cost[n-1]; the
 *     tree keeps n* nodes, the smallest n with S(n+1) < S(n) (all of them if S never
 *     falls).  Without a cost table n* = N_max.
 *   - a q row with an entry outside [0,1] or NaN sets status INPUT.
 * ---------------------------------------------------------------------------------- */
typedef struct { float v; int32_t tok; } ref_rank;

static int ref_rank_cmp(const void *a, const void *b)
{
    const ref_rank *x = (const ref_rank *)a, *y = (const ref_rank *)b;
    if (x->v != y->v) return x->v > y->v ? -1 : 1;
    return (x->tok > y->tok) - (x->tok < y->tok);
}

/* does node (depth da, ranks ra) come before node (db, rb) at equal score? */
static int ref_tuple_before(int da, const int *ra, int db, const int *rb)
{
    if (da != db) return da < db;
    for (int k = 0; k < da; ++k)
        if (ra[k] != rb[k]) return ra[k] < rb[k];
    return 0;
}

int tmvref_tree_best_first(int B, int D, int V, int N_max, const float *q, const double *cost, double l_ar,
                           int32_t *parents, int32_t *tokens, int32_t *n_nodes, double *rho, int32_t *status)
{
    if (B < 0 || D < 1 || D > 8 || V < 1 || N_max < 1 || N_max > 128) return REF_ERR_ARG;
    const int R = N_max + 1;
    const int K = V < N_max ? V : N_max;            /* ranks per position */
    ref_rank *row = (ref_rank *)malloc(sizeof(ref_rank) * (size_t)V);
    int32_t *rtok = (int32_t *)malloc(sizeof(int32_t) * (size_t)D * K);
    float *rq = (float *)malloc(sizeof(float) * (size_t)D * K);
    if (!row || !rtok || !rq) { free(row); free(rtok); free(rq); return REF_ERR_ARG; }
    int depth[129], ranks[129][8];
    double sc[129];
    unsigned char child_in[129][128];

    for (int b = 0; b < B; ++b) {
        for (int j = 0; j < R; ++j) {
            parents[(int64_t)b * R + j] = 0;
            tokens[(int64_t)b * R + j] = 0;
            rho[(int64_t)b * R + j] = j == 0 ? 1.0 : 0.0;
        }
        n_nodes[b] = 0;
        if (status[b] != REF_OK) continue;
        int bad = 0;
        for (int k = 0; k < D && !bad; ++k) {
            const float *qr = q + ((int64_t)b * D + k) * V;
            for (int x = 0; x < V; ++x) {
                if (!(qr[x] >= 0.0f && qr[x] <= 1.0f)) { bad = 1; break; }
                row[x].v = qr[x];
                row[x].tok = x;
            }
            if (bad) break;
            qsort(row, (size_t)V, sizeof(ref_rank), ref_rank_cmp);
            for (int r = 0; r < K; ++r) { rtok[k * K + r] = row[r].tok; rq[k * K + r] = row[r].v; }
        }
        if (bad) { status[b] = REF_ERR_INPUT; continue; }

        /* best-first: node 0 is the root (depth 0, score 1) */
        depth[0] = 0;
        sc[0] = 1.0;
        memset(child_in, 0, sizeof(child_in));
        int n = 0;
        while (n < N_max) {
            int bp = -1, br = -1, bd = 0, bt[8] = {0};
            double bs = 0.0;
            for (int p = 0; p <= n; ++p) {
                if (depth[p] >= D) continue;
                for (int r = 0; r < K; ++r) {
                    if (child_in[p][r]) continue;
                    const double s = sc[p] * (double)rq[depth[p] * K + r];
                    int t[8];
                    for (int k = 0; k < depth[p]; ++k) t[k] = ranks[p][k];
                    t[depth[p]] = r;
                    const int d = depth[p] + 1;
                    if (bp < 0 || s > bs || (s == bs && ref_tuple_before(d, t, bd, bt))) {
                        bp = p; br = r; bs = s; bd = d;
                        for (int k = 0; k < d; ++k) bt[k] = t[k];
                    }
                }
            }
            if (bp < 0) break;                      /* every possible node is in the tree */
            ++n;
            depth[n] = bd;
            for (int k = 0; k < bd; ++k) ranks[n][k] = bt[k];
            sc[n] = bs;
            child_in[bp][br] = 1;
            parents[(int64_t)b * R + n] = bp;
            tokens[(int64_t)b * R + n] = rtok[(bd - 1) * K + br];
            rho[(int64_t)b * R + n] = bs;
        }
        int keep = n;
        if (cost) {
            double A = 0.0, s_prev = 0.0;
            for (int m = 1; m <= n; ++m) {
                A += rho[(int64_t)b * R + m];
                const double s = A * l_ar / cost[m - 1];
                if (m > 1 && s < s_prev) { keep = m - 1; break; }
                s_prev = s;
            }
        }
        for (int j = keep + 1; j < R; ++j) {
            parents[(int64_t)b * R + j] = 0;
            tokens[(int64_t)b * R + j] = 0;
            rho[(int64_t)b * R + j] = 0.0;
        }
        n_nodes[b] = keep;
    }
    free(row); free(rtok); free(rq);
    return REF_OK;
}
