/*
 * specverify.h -- C ABI of the speculative-verification library for AMD MI355X
 * (gfx950): token-tree build, tree-masked GQA attention, acceptance/selection
 * with residual resampling, and the KV commit of the accepted path.
 *
 * Sources (web pages; cited by title and section):
 *   [ReDrafter] "Recurrent Drafter for Fast Speculative Decoding in Large
 *               Language Models", sections "Dynamic Tree Attention" and "The
 *               Full Speculative Decoding Loop" (Steps 3-6).
 *   [Clover]    "Clover: Regressive Lightweight Speculative Decoding with
 *               Sequential Knowledge", section "Inference-Time Verification:
 *               Token Tree Construction and Tree Attention" (Figure 4 mask).
 *   [ResiSpec]  paperpeel 2608.24411 (residual drift in multi-candidate
 *               speculative decoding), section 4 (residual distribution and
 *               sequential verification of N candidates).
 *
 * General contract
 *   - Every pointer argument is caller-owned DEVICE memory unless stated
 *     otherwise.  The library never allocates; scratch memory ("workspace") is
 *     passed in, sized by the matching *_workspace_size query, 256-byte aligned.
 *   - Every call validates its host-side arguments, returns a negative
 *     spec_status without launching anything on a violation, and otherwise
 *     enqueues its kernels on `stream` (a hipStream_t; NULL = default stream)
 *     and returns SPEC_OK without synchronising.
 *   - Problems only visible on the device (a bad parent index, a token outside
 *     the vocabulary, a context that overflows the cache) are OR-ed into the
 *     optional device status word `status` (int32, SPEC_DEV_* bits); the
 *     affected sequence gets a defined, safe result (see each call).  The word
 *     is never cleared by the library.
 *   - Results are bitwise deterministic from run to run.
 *
 * Tree conventions
 *   - Tree position 0 is the root: the last token the target produced, whose
 *     K/V are not in the context yet.  Draft nodes are 1..T_b-1, where
 *     T_b = n_nodes[b] counts the root ([Clover] counts tree size without the
 *     root; T_b = size + 1).  T_cap >= every T_b bounds all per-node arrays;
 *     T_cap <= SPEC_MAX_TREE.
 *   - Every parent index is smaller than its child's.
 *   - anc[b][t] is a bitmask of ceil(T_cap/64) uint64 words: bit a (word a/64,
 *     bit a%64) is set iff node a is t itself, the root or an ancestor of t
 *     ([Clover] Figure 4: M_ij = 1 iff j is an ancestor of i or i = j).
 *   - Padding nodes t >= T_b have parent = token = depth = -1 and anc = 0.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_MAX_TREE 128 /* largest T_cap (root included) */
#define SPEC_MAX_BEAM_TOPK 16 /* largest K_out of spec_beam_topk */
#define SPEC_MAX_SELECT 1024  /* largest candidate count of spec_select_tree */

typedef enum {
    SPEC_OK = 0,
    SPEC_ERR_INVALID = -1,     /* bad argument value or null pointer            */
    SPEC_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head dim)     */
    SPEC_ERR_CAPACITY = -3,    /* a size exceeds a capacity (T_cap, cache cap)  */
    SPEC_ERR_WORKSPACE = -4,   /* workspace missing, too small or misaligned    */
    SPEC_ERR_HIP = -5          /* the HIP runtime refused a launch              */
} spec_status;

/* device status bits (OR-ed into *status) */
#define SPEC_DEV_BAD_PARENT 0x1   /* explicit tree not topological               */
#define SPEC_DEV_BAD_TOKEN 0x2    /* token outside [0, V)                        */
#define SPEC_DEV_BAD_ROW 0x4      /* an inner node has no valid draft row        */
#define SPEC_DEV_CTX_RANGE 0x8    /* ctx_len + n_nodes > cache capacity, etc.    */
#define SPEC_DEV_RESIDUAL_ZERO 0x10 /* a residual had no mass (rounding only)    */
#define SPEC_DEV_SYNC_TIMEOUT 0x20  /* a cross-workgroup wait gave up            */
#define SPEC_DEV_BAD_TREE 0x40    /* n_nodes/parent/depth inconsistent           */

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;
typedef enum { SPEC_TREE_BEAMS = 0, SPEC_TREE_EXPLICIT = 1 } spec_tree_kind;
typedef enum {
    SPEC_GREEDY = 0,
    SPEC_REJECT_PATH = 1,
    SPEC_REJECT_RECURSIVE = 2,
    SPEC_GREEDY_WALK = 3,
    SPEC_REJECT_PATH_WALK = 4,
    SPEC_REJECT_RECURSIVE_WALK = 5
} spec_verify_mode;

/* Library version as 10000*major + 100*minor + patch (host only). */
int spec_version(void);

/* Name of a spec_status value (static string, host only). */
const char *spec_status_string(int status);

/*
 * spec_build_tree -- pack draft candidates into a token tree.
 *
 * [ReDrafter] "Dynamic Tree Attention": beam-search candidates of equal length
 * share prefixes; the packed beam keeps every distinct prefix once and the tree
 * mask lets each token attend only to its own prefix.  Static trees of parallel
 * heads ([Clover] "Token tree construction") and i.i.d. multi-candidate trees
 * ([ResiSpec] section 4) come in explicit form.
 *
 * kind == SPEC_TREE_BEAMS:
 *   cand_token [B][W][L] int32: W candidates of L tokens each (the root is not
 *   part of them); cand_parent must be NULL.  Nodes are numbered in beam-major
 *   order of first appearance of each distinct prefix.  Requires
 *   1 + W*L <= T_cap.  beam_node [B][W][L] (nullable) receives the node holding
 *   each candidate's prefix of length k+1.
 * kind == SPEC_TREE_EXPLICIT:
 *   N = W*L candidates (pass W = 1, L = N); cand_token [B][N] and
 *   cand_parent [B][N] int32 give node j+1's token and its parent's tree index,
 *   which must lie in [0, j].  Duplicate siblings are kept.  A sequence whose
 *   parent list is not topological becomes a root-only tree and raises
 *   SPEC_DEV_BAD_PARENT.  beam_node must be NULL.  Requires 1 + N <= T_cap.
 * root_token [B]: token of node 0.
 * Outputs: n_nodes [B] (T_b, root included), parent/token/depth [B][T_cap],
 * anc [B][T_cap][ceil(T_cap/64)] uint64.
 */
int spec_build_tree(int kind, int B, int W, int L, int T_cap, const int32_t *cand_token,
                    const int32_t *cand_parent, const int32_t *root_token, int32_t *n_nodes,
                    int32_t *parent, int32_t *token, int32_t *depth, uint64_t *anc,
                    int32_t *beam_node, int32_t *status, void *stream);

/*
 * spec_tree_attention -- one attention pass of every tree query over the
 * context plus its own tree prefix.
 *
 * [ReDrafter] Step 4: the target processes the packed beam in one forward pass
 * under the tree mask, and each token's result equals the one it would get had
 * its prefix been decoded token by token.  For sequence b, node t < T_b and
 * query head h (KV head g = h / (H/Hkv); consecutive query heads share a KV
 * head): keys are the context slots 0..ctx-1 and the tree slots ctx+a for every
 * a with anc bit a set; out = softmax(scale * q.k) v over those keys.
 *
 * dt: SPEC_F32 (q, caches and out fp32) or SPEC_BF16 (bf16; fp32 accumulation
 * and softmax).  D must be 64 or 128 for bf16, 1..256 for fp32.  On the bf16
 * path one (b, KV head) cache row block, cache_cap * D * 2 bytes, must stay
 * below 2^31 (SPEC_ERR_UNSUPPORTED otherwise).
 * q [B][T_cap][H][D]; k_cache, v_cache [B][Hkv][cache_cap][D]: the tree's own
 * K/V already sit at slots ctx..ctx+T_b-1 (node t at ctx+t); ctx_len [B]
 * (device) with ctx_len[b] <= max_ctx (host bound used to size the launch);
 * n_nodes [B]; anc as above.  scale <= 0 selects 1/sqrt(D).
 * out [B][T_cap][H][D] (same dtype as q): rows t >= T_b are zero.  A sequence
 * with ctx_len[b] + n_nodes[b] > cache_cap or ctx_len[b] > max_ctx gets zero
 * rows and raises SPEC_DEV_CTX_RANGE.
 * ws: spec_tree_attention_workspace_size() bytes (may be 0 bytes / NULL when
 * the query returns 0).
 */
size_t spec_tree_attention_workspace_size(int dt, int B, int T_cap, int H, int Hkv, int D,
                                          int max_ctx);
int spec_tree_attention(int dt, int B, int T_cap, int H, int Hkv, int D, int cache_cap,
                        int max_ctx, const void *q, const void *k_cache, const void *v_cache,
                        const int32_t *ctx_len, const int32_t *n_nodes, const uint64_t *anc,
                        float scale, void *out, void *ws, size_t ws_bytes, int32_t *status,
                        void *stream);

/*
 * spec_verify -- accept a prefix of the tree per sequence and draw the next token.
 *
 * p_t = softmax(tgt[b][t]) is the target distribution after node t;
 * q_t = softmax(dft[b][dft_row[b][t]]) the draft distribution the children of
 * t were drawn from.  Node t >= 1 with parent s and token x is tested:
 *   SPEC_GREEDY           ([ReDrafter] Step 5, token matches): accepted iff
 *                         x == argmax p_s (lowest index on ties).
 *   SPEC_REJECT_PATH      ([ReDrafter] Step 5, rejection sampling): accepted iff
 *                         u_node[t] < p_s(x) / q_s(x), independently per node.
 *   In both, a node survives when it and all its ancestors are accepted; the
 *   deepest survivor wins, lowest node index on ties (= lowest beam index).  The
 *   next token at the stop node s is argmax p_s (GREEDY), or is drawn with
 *   u_final from norm(max(0, p_s - q_s)) if s has children and from p_s if it
 *   is a leaf (REJECT_PATH).
 *   SPEC_REJECT_RECURSIVE ([ResiSpec] section 4): from the root, the children of
 *                         the current node s are tested in index order against
 *                         a running target p' (p_s at first): accept x iff
 *                         u_node[child] < p'(x) / q_s(x); each rejection sets
 *                         p' <- norm(max(0, p' - q_s)).  An acceptance moves to
 *                         that child.  With no child left, the next token is
 *                         drawn from p' with u_final.
 *   SPEC_GREEDY_WALK      the acceptance, stop node and next token of
 *                         SPEC_GREEDY, found by reading only the target rows
 *                         of nodes whose whole path is accepted: from the root,
 *                         depth by depth, each such node's row is scanned and
 *                         its children are tested.  Only tested nodes (children
 *                         of such nodes) get decision and p_tok; the others get
 *                         -1 and 0.
 * Draws are inverse-CDF in ascending vocabulary order: the smallest v whose
 * running sum exceeds u_final * total.
 *
 * tgt [B][T_cap][V] fp32; dft [B][R][V] fp32 and dft_row [B][T_cap] (entries
 * in [0, R) for every node with children; -1 otherwise) -- both NULL (R = 0)
 * in SPEC_GREEDY; n_nodes/parent/token/depth from spec_build_tree; u_node
 * [B][T_cap] and u_final [B] in [0, 1) (u_node[b][0] unused).
 * Outputs: acc_len [B] (depth of the stop node); acc_path [B][T_cap] (node ids
 * root first, -1 after the path); next_token [B]; p_tok, q_tok [B][T_cap]
 * (nullable: p_s(x) and q_s(x) of each node's own token under its parent; 0
 * for the root, for padding and q in GREEDY); decision [B][T_cap] int8
 * (nullable: 1 accepted, 0 rejected, -1 untested); near_tie [B] (nullable:
 * count of decisions with |ratio - u| < 1e-5 plus one if the draw's threshold
 * fell within 1e-9 of a running-sum boundary).
 * A bad token or missing draft row raises a SPEC_DEV_* bit and the sequence
 * accepts nothing (acc_len 0, next_token = argmax p_0).
 * Workgroups that meet (P > 1 per sequence in the rejection modes, the greedy
 * walk) form a grid sized to be resident on the device at once, and it expects
 * the CUs free to take it; SPEC_COOPERATIVE_LAUNCH=1 in the environment (read
 * at each call) launches such grids cooperatively instead (guaranteed
 * residency, some 17 us slower per call).  A meeting that cannot complete ends at its wait bound and raises
 * SPEC_DEV_SYNC_TIMEOUT.
 * A call that raised SPEC_DEV_SYNC_TIMEOUT has undefined acceptance outputs;
 * its workspace stays usable (every call tags its exchange words with a new
 * epoch, so words left by late workgroups of an earlier call never match).
 * ws: spec_verify_workspace_size() bytes, no initial contents needed.  Calls
 * that overlap in time must not share a workspace.  The workspace size is 0
 * (and the call returns SPEC_ERR_UNSUPPORTED) for a vocabulary beyond what
 * the row merge stages: more than 1024 chunks of 16384 entries (V > 16777216)
 * in the one-pass modes, V * 4 >= 2^31 in SPEC_GREEDY_WALK.
 */
size_t spec_verify_workspace_size(int mode, int B, int T_cap, int V, int R);
int spec_verify(int mode, int B, int T_cap, int V, int R, const float *tgt, const float *dft,
                const int32_t *dft_row, const int32_t *n_nodes, const int32_t *parent,
                const int32_t *token, const int32_t *depth, const float *u_node,
                const float *u_final, int32_t *acc_len, int32_t *acc_path, int32_t *next_token,
                float *p_tok, float *q_tok, int8_t *decision, int32_t *near_tie, void *ws,
                size_t ws_bytes, int32_t *status, void *stream);

/*
 * spec_verify_noalloc -- spec_verify with the library's own workspace, for
 * callers that cannot allocate device memory (code under stream capture, tight
 * serving loops, harnesses that forbid allocation).
 *
 * Arguments, outputs and device status are spec_verify's, without ws and
 * ws_bytes.  The workspace is a 4 MiB device array inside the library, one per
 * device, held until the process ends; the call itself allocates nothing.
 * Returns SPEC_ERR_CAPACITY (nothing launched) when
 * spec_verify_workspace_size() for the arguments exceeds 4 MiB (4194304
 * bytes), and SPEC_ERR_HIP if the array's address cannot be obtained.  Every
 * call on one device shares that device's array: calls that overlap in time
 * on one device (on different streams, or from different host threads) race
 * and must not be issued.
 */
int spec_verify_noalloc(int mode, int B, int T_cap, int V, int R, const float *tgt,
                        const float *dft, const int32_t *dft_row, const int32_t *n_nodes,
                        const int32_t *parent, const int32_t *token, const int32_t *depth,
                        const float *u_node, const float *u_final, int32_t *acc_len,
                        int32_t *acc_path, int32_t *next_token, float *p_tok, float *q_tok,
                        int8_t *decision, int32_t *near_tie, int32_t *status, void *stream);

/*
 * spec_kv_compact -- commit the accepted path's K/V to contiguous cache slots.
 *
 * [ReDrafter] Step 6: the accepted tokens join the context and the next step
 * starts from the last accepted position.  For every b and i = 1..acc_len[b]:
 * slot ctx + acc_path[b][i] moves to slot ctx + i, for K and V of all Hkv heads
 * (all sources are read before any slot is written, so overlapping moves are
 * safe); the root stays at slot ctx.  Then ctx_len[b] += acc_len[b] + 1 (the
 * root and the accepted tokens; next_token is the next step's root).
 * dt selects the element size; k_cache, v_cache [B][Hkv][cache_cap][D] in
 * place; ctx_len [B] in/out, each in [0, cache_cap); acc_len [B], acc_path
 * [B][T_cap] from spec_verify.  One path's rows of one KV head must fit 64 KiB
 * ((T_cap - 1) * D * element size <= 65536; SPEC_ERR_UNSUPPORTED otherwise).
 * ctx_len[b] holds nothing but the length at any time: it is read, then
 * written once after every read of it.
 * ws: spec_kv_compact_workspace_size(B) bytes (per sequence an arrival
 * counter of the call's workgroups), zero-filled before its first use; every
 * call returns it to zero.  Calls that overlap in time must not share it.
 * A path that is not increasing or leaves the cache raises SPEC_DEV_CTX_RANGE
 * and that sequence is left untouched.
 */
size_t spec_kv_compact_workspace_size(int B);
int spec_kv_compact(int dt, int B, int Hkv, int D, int cache_cap, int T_cap, void *k_cache,
                    void *v_cache, int32_t *ctx_len, const int32_t *acc_len,
                    const int32_t *acc_path, void *ws, size_t ws_bytes, int32_t *status,
                    void *stream);

/*
 * spec_beam_topk -- the pruning step of beam search, feeding spec_build_tree.
 *
 * [ReDrafter] section "Beam Search During Inference", steps 1 and 3: every
 * extension of beam j by token v scores score[j] + logp[j][v] (the cumulative
 * log-probability; an fp32 sum), and the K_out best of the K_in * V
 * extensions become the next beams, best first.  Equal scores go to the lower
 * flattened index j * V + v (the pages name no tie rule); -0.0 counts as +0.0,
 * and NaN scores have no defined place.
 * logp [B][K_in][V] fp32 (device); beam_score [B][K_in] fp32, or NULL for all
 * zero (the first step, K_in = 1).  Outputs [B][K_out]: out_parent (beam j),
 * out_token (v), out_score (the sum).  hist_out [B][K_out][hist_len + 1]
 * (NULL: no histories) gets each new beam's history, its parent's from
 * hist_in [B][K_in][hist_len] (NULL allowed when hist_len is 0) followed by
 * its token -- after L steps the [B][W][L] beams input of spec_build_tree.
 * Requires 1 <= K_out <= SPEC_MAX_BEAM_TOPK and K_out <= K_in * V
 * (SPEC_ERR_CAPACITY otherwise) and K_in * V < 2^31 (SPEC_ERR_UNSUPPORTED).
 * ws: spec_beam_topk_workspace_size() bytes (no initial contents needed).
 * Calls that overlap in time must not share a workspace.
 */
size_t spec_beam_topk_workspace_size(int B, int K_in, int K_out, int V);
int spec_beam_topk(int B, int K_in, int K_out, int V, const float *logp, const float *beam_score,
                   int32_t *out_parent, int32_t *out_token, float *out_score,
                   const int32_t *hist_in, int hist_len, int32_t *hist_out, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * spec_select_tree -- keep the best branches of a draft tree under a node budget.
 *
 * [Drafters] "Speculative Decoding, Part 2: A History of Drafters", the EAGLE-2
 * paragraph: a branch scores the product of the drafter's confidences along
 * its path from the root, the highest-scoring branches are kept, and a parent
 * always scores at least as high as its children; [Clover] sizes its tree by
 * a node budget.  In log form: S(root) = 0, S(node) = S(parent) + logp(node),
 * an fp32 sum from the root down.  The N_keep candidates with the highest S
 * are kept, the lower candidate index on ties, so every kept node's parent is
 * kept too.
 * Candidate i of sequence b is node i + 1: cand_parent [B][N] (its parent
 * node, in [0, i]; 0 = root), cand_token [B][N], cand_logp [B][N] (its
 * log-confidence, <= 0).  Outputs [B][N_keep], the kept candidates in their
 * original order as an explicit candidate list for spec_build_tree (kept
 * candidate k is node k + 1): keep_parent (the new number of its parent node),
 * keep_token, keep_src (original candidate index; nullable) and keep_score
 * (S; nullable).  A sequence with a parent out of range, logp > 0 or NaN gets
 * keep_parent = -1 (spec_build_tree then makes it a root-only tree) and
 * raises SPEC_DEV_BAD_PARENT.
 * Requires 1 <= N_keep <= N <= SPEC_MAX_SELECT and N_keep < SPEC_MAX_TREE.
 * No workspace.
 */
int spec_select_tree(int B, int N, int N_keep, const int32_t *cand_parent,
                     const int32_t *cand_token, const float *cand_logp, int32_t *keep_parent,
                     int32_t *keep_token, int32_t *keep_src, float *keep_score, int32_t *status,
                     void *stream);

/*
 * spec_last_device_status -- the SPEC_DEV_* bits a status word holds, read on
 * the host once `stream` has finished.
 *
 * The calls are asynchronous, so problems seen by their kernels cannot be
 * returned by the call (general contract above).  status_dev: a caller's
 * device status word, as passed to the calls, or NULL for the library's own
 * word on the current device, which every call that is passed no status word
 * uses instead.  Synchronises `stream` (hipStream_t; NULL = default stream)
 * and returns the word's bits (>= 0), or SPEC_ERR_HIP if the runtime fails.
 * The library's own word is cleared after it is read; a caller's word is left
 * as it is.  Not for use inside stream capture (it synchronises).
 */
int spec_last_device_status(const int32_t *status_dev, void *stream);

/*
 * spec_copy_probe -- plain streaming copy of n_bytes (multiple of 16) from src
 * to dst, for bandwidth and memory-counter calibration of the platform.
 */
int spec_copy_probe(const void *src, void *dst, size_t n_bytes, void *stream);

/*
 * spec_read_probe -- plain streaming read of n_bytes (multiple of 16) from src
 * for the platform's achievable read bandwidth (the ceiling of read-dominated
 * calls such as the attention): workgroup g of n_blocks (256 threads each)
 * reads the 256 KiB chunks g, g + n_blocks, ... front to back with
 * non-temporal loads; out[n_blocks] (fp32, device) receives one partial sum
 * per workgroup.
 */
int spec_read_probe(const void *src, size_t n_bytes, float *out, int n_blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
