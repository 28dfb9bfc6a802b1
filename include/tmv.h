/*
 * tmv.h -- C ABI of libtmv.so: the teacher's tree-verification step of tree speculative
 * decoding, on AMD Instinct MI355X (gfx950).
 *
 * Four calls, one per stage of a verify step, all enqueued on the caller's HIP stream:
 *
 *   tmv_tree_build_ancestors   parents -> virtual-root ancestor table + invariant checks
 *   tmv_tree_verify_attention  tree-masked attention of every draft node over the
 *                              committed prefix plus its own ancestor path
 *   tmv_tree_accept            greedy longest matching path, or modified rejection
 *                              sampling with a max(0, p - q) residual
 *   tmv_kv_commit_path         prefix-sharing compaction of the accepted path's K/V rows
 *
 * Paged K/V caches (block tables) have their own attention and commit calls, and a
 * best-first tree builder with a budget controller produces trees for the step.
 *
 * Conventions shared by every call
 *   - Every pointer argument is DEVICE memory owned by the caller (for example a torch
 *     tensor's data_ptr), except the small int64 stride arrays, which are HOST arrays read
 *     during the call.  The library keeps no global state and allocates nothing; scratch
 *     memory comes from a caller workspace whose size the *_workspace call returns.  The
 *     attention and accept workspaces hold counters: zero-fill them once before their
 *     first use; every completed call leaves them ready for the next call of any shape
 *     they are large enough for (after a TMV_ERR_DEVICE status, zero-fill again).  Calls
 *     that may run at the same time (different streams) must not share a workspace.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are asynchronous; none
 *     synchronises the host.
 *   - The return value reports problems the host can see (TMV_ERR_ARG: bad sizes, null
 *     pointers, unsupported shapes; nothing was launched) or a failed launch
 *     (TMV_ERR_DEVICE).  Problems in the data (a malformed tree, a NaN logit, a prefix that
 *     does not fit) are reported per sequence in the caller's device array status[B]: a
 *     stage only ever moves a sequence from TMV_OK to an error, and a failed sequence is
 *     inert downstream (zero outputs, accept length 0, nothing committed).
 *   - No stage ever reads or writes outside the buffers described below, and no output
 *     ever holds a negative or out-of-range index.
 *
 * Node numbering (virtual root): row 0 is a virtual root that carries no K/V; draft nodes
 * are 1..M_b.  This and the ancestor table follow section 2.2 of the Chinese technical
 * summary of "EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend NPUs"
 * (parent pointers remapped onto a root row 0 so every gather index lies in [0, M]).
 *
 * Limits (host-checked): 0 <= M_max <= 128, 0 <= D_max <= 128, B >= 0, V >= 1.
 */
#ifndef TMV_H
#define TMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes (return values and per-sequence status words) */
enum {
    TMV_OK = 0,
    TMV_ERR_ARG = 1,      /* host-visible bad argument; nothing launched               */
    TMV_ERR_RANGE = 2,    /* a parent index outside [0, M_b] (incl. a -1 sentinel), or
                             M_b outside [0, M_max]                                     */
    TMV_ERR_CYCLE = 3,    /* a parent chain never reaches the root                      */
    TMV_ERR_DEPTH = 4,    /* a node deeper than D_max                                   */
    TMV_ERR_CLOSURE = 5,  /* a valid node under an invalid one                          */
    TMV_ERR_INPUT = 6,    /* malformed data: NaN / out-of-range probabilities, a token
                             outside [0,V), a prefix or path that does not fit the cache */
    TMV_ERR_DEVICE = 7    /* a kernel launch failed, or per sequence: the device could
                             not complete it (the sampling walk's bounded wait, an
                             attention row block spread over XCDs)                      */
};

enum { TMV_F32 = 0, TMV_BF16 = 1 };                       /* element types           */
enum { TMV_PARENTS_VROOT = 0, TMV_PARENTS_NEG1 = 1 };     /* parent table formats    */
enum { TMV_ACCEPT_GREEDY = 0, TMV_ACCEPT_SAMPLE = 1 };    /* acceptance rules        */

/* Human-readable name of a status code (static string). */
const char *tmv_status_string(int code);

/* ABI version of this library (increments on any signature change). */
int tmv_abi_version(void);

/*
 * tmv_tree_build_ancestors -- accelerator-safe tree tensors.
 * Defined by section 2.2 of the Chinese EAGLE-Pangu technical summary (virtual root 0,
 * precomputed ancestor table, range / acyclicity / validity-closure checks before any
 * fused kernel) and section 2 of the Portuguese one (negative sentinels replaced by a
 * valid root index).
 *
 *   parents   VROOT: int32 [B][M_max+1]; column 0 is ignored; node i in 1..M_b has parent
 *                    parents[b][i] in [0, M_b] (0 = the virtual root).
 *             NEG1 : int32 [B][M_max]; node r in 0..M_b-1 (0-based) has parent -1 (the
 *                    original root) or 0..M_b-1; remapped here to node r+1 with parent
 *                    -1 -> 0 and v -> v+1.  Values below -1 are RANGE errors.
 *   valid     uint8 [B][M_max+1] or NULL (NULL: nodes 1..M_b are all valid).  Invalid
 *             nodes are inert; a valid node whose parent is invalid is a CLOSURE error.
 *   n_nodes   int32 [B]: M_b.
 *   anc       out int32 [B][M_max+1][D_max+1]: anc[b][i][k] = parent^k(i), saturating at
 *             0; anc[b][i][depth(i)] = 0.  Row 0, rows > M_b and invalid rows are all 0.
 *   depth     out int32 [B][M_max+1]: hops from node i to the root (0 for inert rows).
 *   status    out int32 [B]: written (not merged) by this stage: TMV_OK or the smallest
 *             error code found among the sequence's nodes; a failed sequence's anc/depth
 *             rows are all 0.
 */
int tmv_tree_build_ancestors(int B, int M_max, int D_max, int parent_format,
                             const int32_t *parents, const uint8_t *valid,
                             const int32_t *n_nodes,
                             int32_t *anc, int32_t *depth, int32_t *status,
                             void *stream);

/*
 * tmv_tree_verify_attention -- tree-masked attention of the flattened draft tree.
 * Defined by section 2.3 of the Chinese EAGLE-Pangu technical summary (all speculative
 * nodes evaluated in one teacher pass; node k attends only to its ancestor path,
 * itself included) and the Medusa section of "Speculative Decoding Hierarquico: Medusa,
 * EAGLE-2 e Multi-Token Prediction" (parallel nodes see only their direct ancestors).
 * Equivalently: node i's output equals causal attention over the linear sequence
 * prefix + path(i).  The 4D mask of the pages is never materialised: each row's
 * ancestor set is a bitmask built in registers from `anc`.
 *
 *   dtype     TMV_F32 or TMV_BF16 for q, k_cache, v_cache and out (fp32 accumulation).
 *   q         [B][M_max][Hq][d] with element strides q_stride = {batch, node, head}; d is
 *             contiguous; row r holds node r+1.
 *   k_cache,
 *   v_cache   [B][Hkv][L_cap][d] with element strides kv_stride = {batch, head, slot}; d is
 *             contiguous.  Slots [0, P_b) hold the committed prefix; node j's K/V (written
 *             by the caller's teacher layer) live at slot P_b + j - 1.
 *   prefix_len int32 [B]: P_b.  A sequence with P_b < 0 or P_b + M_b > L_cap gets status
 *             TMV_ERR_INPUT and zero outputs.
 *   anc, depth, n_nodes, status: from tmv_tree_build_ancestors (status in/out).
 *   scale     softmax scale (typically 1/sqrt(d)).
 *   out       [B][M_max][Hq][d] with element strides o_stride = {batch, node, head}: one
 *             row per node and query head; rows of inert nodes (beyond M_b, invalid, or
 *             in a failed sequence) are written as 0.
 *   GQA: query head h reads KV head h / (Hq/Hkv).  Requires Hq % Hkv == 0, d in {64,128},
 *        Hq/Hkv <= 16, 1 <= L_cap, q and the caches 16-byte aligned with strides that
 *        are multiples of 16 bytes (bf16: out too; TMV_ERR_ARG otherwise).
 *   workspace: tmv_tree_verify_attention_workspace() bytes, 16-byte aligned.  It opens
 *        with a fixed 32 KiB block of 64-bit arrival words (one per split row block; the
 *        last split of a block to finish merges it) followed by the split-KV partials, which
 *        every call rewrites.  The counter block must be zero before the first call and
 *        every completed call leaves it zero, so zero-fill a new workspace once; it then
 *        stays valid for calls of any shape whose size it covers.
 *   The splits of a row block exchange their partials through the L2 of the XCD they share
 *   (the workgroups of a block have equal ids mod 8, which the hardware deals round-robin
 *   to the 8 XCDs).  A block whose splits are found on several XCDs is not merged: its rows
 *   are written as 0 and the sequence gets TMV_ERR_DEVICE.
 */
size_t tmv_tree_verify_attention_workspace(int dtype, int B, int M_max, int Hq, int Hkv,
                                           int d, int L_cap);
int tmv_tree_verify_attention(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d,
                              const void *q, const int64_t *q_stride,
                              const void *k_cache, const void *v_cache,
                              const int64_t *kv_stride, int L_cap,
                              const int32_t *prefix_len, const int32_t *n_nodes,
                              const int32_t *anc, const int32_t *depth, int32_t *status,
                              float scale, void *out, const int64_t *o_stride,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * tmv_tree_verify_attention_plan -- tmv_tree_verify_attention with its launch plan pinned
 * (for tuning sweeps and tests that must exercise every plan; results agree with the
 * library's own choice within the attention tolerance, and are bit-identical across
 * reruns of one plan).  The plan of the bf16 kernels is (rows sharing each staged K/V
 * chunk, token splits per row block):
 *   rows_per_group  d = 128: 64, 128 or 256; d = 64: 32 or 128; 0 = the library's choice.
 *   splits          1 .. 16; 0 = the library's choice.  (Split-KV is dropped when the
 *                   call has 256 or more row blocks.)  ORed with TMV_PLAN_SCATTER_XCD
 *                   (d = 128, 2 .. 16 splits, B * Hkv a multiple of 8): split s of each row
 *                   block goes to a different XCD, a placement the partial exchange rejects
 *                   (rows 0, TMV_ERR_DEVICE) -- for tests of that path; TMV_ERR_ARG when the
 *                   shape does not allow it.
 * Other values are ignored (the library's choice).  fp32 calls have no plan.  The
 * workspace must hold tmv_tree_verify_attention_plan_workspace() bytes for the same plan.
 */
#define TMV_PLAN_SCATTER_XCD 0x100
size_t tmv_tree_verify_attention_plan_workspace(int dtype, int B, int M_max, int Hq, int Hkv, int d, int L_cap,
                                                int rows_per_group, int splits);
int tmv_tree_verify_attention_plan(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d,
                                   const void *q, const int64_t *q_stride,
                                   const void *k_cache, const void *v_cache,
                                   const int64_t *kv_stride, int L_cap,
                                   const int32_t *prefix_len, const int32_t *n_nodes,
                                   const int32_t *anc, const int32_t *depth, int32_t *status,
                                   float scale, void *out, const int64_t *o_stride,
                                   int rows_per_group, int splits,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * tmv_tree_verify_attention_paged -- the same attention over a paged K/V cache.
 * Defined by the runtime-memory question of "Speculative Decoding Hierarquico: Medusa,
 * EAGLE-2 e Multi-Token Prediction" (vLLM's PagedAttention keeps the cache in pages
 * allocated on demand; during tree verification the ancestors' pages are shared, the
 * pages of rejected branches are freed afterwards and only the accepted path stays).
 * Results are those of tmv_tree_verify_attention over the cache the pages describe.
 *   k_pages,
 *   v_pages      [num_pages][Hkv][page_size][d] pools with element strides
 *                page_stride = {page, head, slot}; d contiguous.
 *   block_table  int32 [B][table_stride]: logical slot t of sequence b (prefix slots
 *                [0, P_b), then node j at P_b + j - 1) lives in page
 *                block_table[b][t / page_size] at row t % page_size.  Entries
 *                [0, max_blocks) are read; every entry that holds a slot below P_b + M_b
 *                must be in [0, num_pages), else the sequence gets TMV_ERR_INPUT and zero
 *                outputs (other entries may hold anything).  Pages may be shared between
 *                sequences (a common prefix).
 *   The capacity is L_cap = max_blocks * page_size.  Requires dtype TMV_BF16, d = 128,
 *   page_size a power of two in [16, 2^20], 1 <= max_blocks <= 4096, table_stride >=
 *   max_blocks, page_size * page_stride[2] * 2 < 2^31 bytes, and the alignment rules of
 *   tmv_tree_verify_attention (TMV_ERR_ARG otherwise).  Every other argument is as there.
 *   workspace: tmv_tree_verify_attention_paged_workspace() bytes, same contract.
 */
size_t tmv_tree_verify_attention_paged_workspace(int B, int M_max, int Hq, int Hkv, int d, int page_size,
                                                 int max_blocks);
int tmv_tree_verify_attention_paged(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d,
                                    const void *q, const int64_t *q_stride,
                                    const void *k_pages, const void *v_pages,
                                    const int64_t *page_stride, int num_pages, int page_size,
                                    const int32_t *block_table, int64_t table_stride, int max_blocks,
                                    const int32_t *prefix_len, const int32_t *n_nodes,
                                    const int32_t *anc, const int32_t *depth, int32_t *status,
                                    float scale, void *out, const int64_t *o_stride,
                                    void *workspace, size_t workspace_bytes, void *stream);
/*
 * tmv_tree_verify_attention_noalloc -- tmv_tree_verify_attention without a workspace, for
 * callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and per-sequence errors;
 * the call allocates nothing.  Its scratch (arrival counters and split partials) is a
 * fixed 32 MiB array on every device the library runs on, held until the process ends
 * and cleared by a small kernel on the device's first call.
 *   - A call whose workspace (tmv_tree_verify_attention_workspace) exceeds 32 MiB returns
 *     TMV_ERR_ARG and launches nothing.
 *   - Every call on one device shares that device's array: calls that may overlap on one
 *     device (different streams, or host threads) race and must be serialised by the
 *     caller.  A completed call leaves the array ready for the next one.
 */
int tmv_tree_verify_attention_noalloc(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d,
                                      const void *q, const int64_t *q_stride,
                                      const void *k_cache, const void *v_cache,
                                      const int64_t *kv_stride, int L_cap,
                                      const int32_t *prefix_len, const int32_t *n_nodes,
                                      const int32_t *anc, const int32_t *depth, int32_t *status,
                                      float scale, void *out, const int64_t *o_stride, void *stream);

/* The paged call with its launch plan pinned, as tmv_tree_verify_attention_plan. */
size_t tmv_tree_verify_attention_paged_plan_workspace(int B, int M_max, int Hq, int Hkv, int d, int page_size,
                                                      int max_blocks, int rows_per_group, int splits);
int tmv_tree_verify_attention_paged_plan(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d,
                                         const void *q, const int64_t *q_stride,
                                         const void *k_pages, const void *v_pages,
                                         const int64_t *page_stride, int num_pages, int page_size,
                                         const int32_t *block_table, int64_t table_stride, int max_blocks,
                                         const int32_t *prefix_len, const int32_t *n_nodes,
                                         const int32_t *anc, const int32_t *depth, int32_t *status,
                                         float scale, void *out, const int64_t *o_stride,
                                         int rows_per_group, int splits,
                                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * tmv_tree_accept -- choose the accepted path and the next token.
 *
 * GREEDY (Medusa section of the hierarchical speculative decoding blog: the longest
 * valid branch is kept; teacher-greedy decoding is the baseline of section 4 of the
 * Portuguese EAGLE-Pangu summary):
 *   t(u) = argmax_x teacher[b][u][x] (smallest x on ties; -0 and +0 are equal) for u = 0
 *   and every live node;
 *   node i matches iff every node c on its path has tokens[c] == t(parent(c));
 *   the deepest matching node a* (smallest id on ties; 0 if none) gives
 *   accept_len = depth(a*), path = its ancestors root->leaf, next_token = t(a*).
 *   teacher: logits, f32 or bf16 (row_dtype).  NaN in a scanned row -> TMV_ERR_INPUT.
 *
 * SAMPLE (modified rejection sampling section of the same blog: a draft token x is kept
 *   with probability min(1, p(x)/q(x)); on refusal the rest is dropped and a correction
 *   is drawn from max(0, p - q) renormalised; its FAQ: a correction is emitted when all
 *   guesses are refused).  On a tree, the children of the current node are tried in
 *   ascending id, each against the residual left by the refused siblings; a walk that
 *   reaches a node without children draws a bonus token from that node's p.
 *   teacher = p, draft_q = q: f32 probabilities; row u is the distribution after node u
 *   (row 0 after the prefix); children of u must have been drawn from q row u.
 *   Arithmetic is exact integer fixed point.  WP(x) = floor(p(x) 2^31) and WQ(x) =
 *   floor(q(x) 2^31) have exact sums SP and SQ; SQ = 1 at a node without children, whose
 *   q row is not read.  Against one draft row, the residual left after j refusals is
 *   (p - c_j q)+ renormalised.  It is held as M and T, with R(y) = max(0, WP(y) SQ -
 *   WQ(y) M) and T = sum R; M = 0 on arrival at a node.
 *     accept:  iff U24 * WQ(x) * T < R(x) * SQ * 2^24 (exact, 192-bit).
 *     refusal: M += floor(T / SQ), unless the new residual sums to 0 (the state is kept).
 *     draw:    the least x with sum_{y<=x} R(y) > floor((word >> 32) * T / 2^32).
 *   Requires V <= 2^24.
 *   Random words: Philox4x64-10, key {seed, (step << 32) | b}, block n at counter
 *   {n+1, 0, 0, 0}, word n = 64-bit lane n % 4 of block n / 4 (numpy's Philox stream);
 *   one word per tried child, one per final draw, in walk order.
 *   Visited rows with entries outside [0,1] or NaN, a zero p row, or a zero q row under a
 *   node with children -> TMV_ERR_INPUT.
 *
 *   tokens     int32 [B][M_max+1] draft tokens (column 0 ignored); a live node's token
 *              outside [0, V) -> TMV_ERR_INPUT.
 *   teacher    [B][M_max+1][V] rows at teacher + b*t_stride_b + u*t_stride_row (elements).
 *   draft_q    SAMPLE only: f32 rows at draft_q + b*q_stride_b + u*q_stride_row; NULL for
 *              GREEDY.
 *   accept_len out int32 [B]; path out int32 [B][D_max] (node ids root->leaf, then 0);
 *   next_token out int32 [B].  All 0 for a failed sequence.
 *   workspace: tmv_tree_accept_workspace() bytes, 16-byte aligned.  Every completed call
 *     leaves it zero; zero-fill it once before first use.
 *     GREEDY: one workgroup per (sequence, row, 4096-entry chunk).  When they are all
 *     resident at once (the kernel's occupancy times the compute units), one launch: per
 *     (sequence, row) a key and an arrival counter, per sequence an arrival counter; a
 *     row's chunks merge their argmax keys with a device-scope atomic maximum, the last
 *     chunk of a row to arrive counts the row in, the last row of a sequence chooses its
 *     path, and each counter and key is reset by whoever completes it.  Otherwise two
 *     launches: the chunk keys are written to the workspace and a second kernel merges
 *     them and chooses the paths.
 *     SAMPLE: one synchronisation block per sequence.  K workgroups walk a sequence
 *     together, one per vocabulary slice, and meet after every row pass; K = (the walk
 *     kernel's resident workgroups per compute unit x compute units) / B, at most 64, so the
 *     whole launch is resident on an otherwise idle device (the results do not depend on K).
 *     - A workgroup that waits more than 2 ms for the other slices (kernels on other streams
 *       can hold compute units) gives up: the sequence ends with status TMV_ERR_DEVICE and
 *       zero outputs, every workgroup still exits, and the workspace is again left zero.
 */
size_t tmv_tree_accept_workspace(int mode, int B, int M_max, int V);
int tmv_tree_accept(int mode, int B, int M_max, int D_max, int V,
                    const int32_t *tokens, int row_dtype, const void *teacher,
                    int64_t t_stride_b, int64_t t_stride_row,
                    const float *draft_q, int64_t q_stride_b, int64_t q_stride_row,
                    uint64_t seed, uint64_t step,
                    const int32_t *n_nodes, const int32_t *anc, const int32_t *depth,
                    int32_t *status, int32_t *accept_len, int32_t *path, int32_t *next_token,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * tmv_tree_accept_wait -- tmv_tree_accept with the sampling walk's wait bound given in
 * microseconds (tmv_tree_accept uses 2000): how long a workgroup waits for the other slices
 * of its sequence before the sequence ends with TMV_ERR_DEVICE.  For callers that share the
 * device with long-running kernels on other streams (a larger bound), or that prefer to
 * fail fast; 0 gives up at the first wait that is not already met.  GREEDY ignores it.
 */
int tmv_tree_accept_wait(int mode, int B, int M_max, int D_max, int V,
                         const int32_t *tokens, int row_dtype, const void *teacher,
                         int64_t t_stride_b, int64_t t_stride_row,
                         const float *draft_q, int64_t q_stride_b, int64_t q_stride_row,
                         uint64_t seed, uint64_t step,
                         const int32_t *n_nodes, const int32_t *anc, const int32_t *depth,
                         int32_t *status, int32_t *accept_len, int32_t *path, int32_t *next_token,
                         void *workspace, size_t workspace_bytes, uint32_t wait_us, void *stream);

/*
 * tmv_tree_accept_lm_head -- greedy acceptance straight from the teacher's LM head: the
 * logits of row u are hidden_u . W^T, and only their argmax t(u) is needed, so the logits
 * are reduced to t(u) as an MFMA GEMM produces them and are never written (roofline
 * section of "Speculative Decoding Hierarquico: Medusa, EAGLE-2 e Multi-Token Prediction":
 * decode is bound by reading weights; the LM head is read once per step).  The path rule
 * is exactly tmv_tree_accept's GREEDY rule on those logits.
 *   K          hidden size: 512, 1024, 2048, 4096 or 8192.
 *   hidden     bf16 [B][M_max+1][K], element strides {h_stride_b, h_stride_row}, K
 *              contiguous: row u holds the teacher's final hidden state after node u (row 0:
 *              after the committed prefix).
 *   lm_head    bf16 [V][K], row x at x * w_stride_row (>= K), K contiguous.
 *   Arithmetic: bf16 products accumulated in fp32 (v_mfma_f32_16x16x32_bf16), so t(u) is
 *              the argmax of fp32 sums; it agrees with the exact argmax wherever the top two
 *              logits differ by more than the fp32 accumulation error (K * 2^-24 *
 *              sum_k |h_k w_k| for each of them).  Ties: smallest token.  A NaN logit in a
 *              live row sets TMV_ERR_INPUT.
 *   row_argmax int32 [B][M_max+1] or NULL: t(u) of every live row, -1 elsewhere.
 *   Rows: up to 64 rows (B * (M_max+1)) stream the weights once; more rows go in blocks of
 *              272, each streaming them once.
 *   Other arguments and outputs as tmv_tree_accept (GREEDY).
 *   Requires hidden, lm_head and the workspace 16-byte aligned, strides multiples of 8
 *   elements, and both tensors spanning less than 2 GiB (TMV_ERR_ARG otherwise).
 *   workspace: tmv_tree_accept_lm_head_workspace() bytes, 16-byte aligned: one 64-bit key
 *   per row, merged with atomics.  Zero-fill it once before its first use; every completed
 *   call leaves it zero.
 */
size_t tmv_tree_accept_lm_head_workspace(int B, int M_max);
int tmv_tree_accept_lm_head(int B, int M_max, int D_max, int K, int V, const int32_t *tokens,
                            const void *hidden, int64_t h_stride_b, int64_t h_stride_row,
                            const void *lm_head, int64_t w_stride_row,
                            const int32_t *n_nodes, const int32_t *anc, const int32_t *depth,
                            int32_t *status, int32_t *accept_len, int32_t *path, int32_t *next_token,
                            int32_t *row_argmax, void *workspace, size_t workspace_bytes, void *stream);

/*
 * tmv_kv_commit_path -- prefix-sharing path-index commit, in place.
 * Defined by section 2.1 of the Chinese EAGLE-Pangu technical summary (commit by
 * accepted length or by path index; a prefix-sharing fast reorder moves only the newly
 * accepted segment) and section 2 of the Portuguese one.
 * For every layer, KV head and both caches: the rows at slots P_b + path[b][j] - 1,
 * j < accept_len[b], are read first and then written to slots P_b + j; rows whose source
 * equals their destination are not touched; the prefix [0, P_b) and every other slot are
 * left unchanged.  new_len[b] = P_b + accept_len[b].
 *   dtype      TMV_F32 or TMV_BF16 (rows are moved as bytes).
 *   k_cache,
 *   v_cache    [n_layers][B][Hkv][L_cap][d] with element strides
 *              kv_stride = {layer, batch, head, slot}; d contiguous.
 *   A sequence whose status is not OK moves nothing (new_len = P_b).  A sequence whose
 *   P_b, M_b, accept_len or path entries do not fit (P_b < 0, P_b + M_b > L_cap,
 *   accept_len outside [0, min(D_max, M_b)], a path entry outside [1, M_b]) moves nothing
 *   and gets TMV_ERR_INPUT.  Requires d * element size <= 512 bytes and a multiple of 16.
 */
int tmv_kv_commit_path(int dtype, int n_layers, int B, int Hkv, int d, int L_cap,
                       int M_max, int D_max,
                       void *k_cache, void *v_cache, const int64_t *kv_stride,
                       const int32_t *prefix_len, const int32_t *n_nodes,
                       const int32_t *accept_len, const int32_t *path,
                       int32_t *status, int32_t *new_len, void *stream);

/*
 * tmv_kv_commit_path_paged -- the same commit over paged K/V pools.
 * Defined by the runtime-memory question of "Speculative Decoding Hierarquico: Medusa,
 * EAGLE-2 e Multi-Token Prediction" (only the accepted path is integrated into the
 * sequence; the pages of rejected branches are freed).  Moves exactly the rows
 * tmv_kv_commit_path moves, with logical slot t of sequence b at page
 * block_table[b][t / page_size], row t % page_size.  The table is not changed; after
 * the call, pages that hold only slots >= new_len[b] carry nothing the sequence needs and
 * the caller may free them.
 *   k_pages,
 *   v_pages      [n_layers][num_pages][Hkv][page_size][d] with element strides
 *                page_stride = {layer, page, head, slot}; d contiguous.  One table serves
 *                every layer.
 *   L_cap = max_blocks * page_size.  A sequence whose moving rows touch a page entry
 *   outside [0, num_pages) moves nothing and gets TMV_ERR_INPUT (new_len = P_b); the
 *   other rules are those of tmv_kv_commit_path.  Requires page_size a power of two in
 *   [1, 2^20], max_blocks >= 1, table_stride >= max_blocks.
 */
int tmv_kv_commit_path_paged(int dtype, int n_layers, int B, int Hkv, int d, int num_pages, int page_size,
                             const int32_t *block_table, int64_t table_stride, int max_blocks,
                             int M_max, int D_max, void *k_pages, void *v_pages,
                             const int64_t *page_stride, const int32_t *prefix_len,
                             const int32_t *n_nodes, const int32_t *accept_len, const int32_t *path,
                             int32_t *status, int32_t *new_len, void *stream);

/*
 * tmv_kv_commit_path_paged_evict -- the paged commit, then block eviction: the block table
 * is rewritten so that only the accepted path stays in the sequence.  Defined by the same
 * runtime-memory question (pages of the tree allocated for the step; after the parallel
 * step the blocks of discarded branches are evicted; only the accepted path is kept).
 *   Rows move exactly as tmv_kv_commit_path_paged moves them; only blocks holding slots of
 *   [P_b, P_b + A_b) are written (partial blocks).  Then, for every sequence whose status
 *   is TMV_OK, each block i of the tree's slots [P_b, P_b + M_b) with i * page_size >=
 *   new_len[b] -- nothing in it is still part of the sequence -- has a valid page entry
 *   (in [0, num_pages)) cleared to -1 in block_table, and that page number is appended to
 *   freed_pages at index atomicAdd(freed_count, 1) (caller-owned device int32 array and
 *   counter, in any order).  An entry whose index would reach freed_capacity is left in
 *   the table instead.  Blocks of a failed sequence and blocks past the tree are never
 *   touched.  The pages of evicted blocks must belong to their sequence alone (pages of
 *   the prefix, which a sequence may share, are never evicted).  At most ceil(M_b /
 *   page_size) + 1 blocks per sequence are evicted.
 */
int tmv_kv_commit_path_paged_evict(int dtype, int n_layers, int B, int Hkv, int d, int num_pages, int page_size,
                                   int32_t *block_table, int64_t table_stride, int max_blocks,
                                   int M_max, int D_max, void *k_pages, void *v_pages,
                                   const int64_t *page_stride, const int32_t *prefix_len,
                                   const int32_t *n_nodes, const int32_t *accept_len, const int32_t *path,
                                   int32_t *status, int32_t *new_len, int32_t *freed_pages, int32_t *freed_count,
                                   int freed_capacity, void *stream);

/*
 * tmv_tree_best_first -- a best-first prefix tree from per-position draft marginals, and
 * the hardware-aware budget controller that chooses its size.
 * Defined by sections 1-3 of the BASTION technical summary:
 *   - a block-diffusion drafter gives one marginal q_k per future position;
 *   - a node at depth d (tokens x_1..x_d) has path score rho = q_1(x_1) * ... * q_d(x_d);
 *   - best-first expansion repeatedly adds the highest-scoring node whose parent is in the
 *     tree, which is optimal for the surrogate A(T) = sum of its scores;
 *   - the controller keeps growing the tree while S(n) = A(n) * L_AR / C(n) rises.
 * Readings:
 *   - rho is an fp64 product in depth order.
 *   - Equal scores go to the shallower node, then to the smaller rank tuple, with ranks per
 *     position by (q descending, token ascending).
 *   - Nodes are numbered in the order they are added.
 *   - The tree keeps the smallest n with S(n+1) < S(n), or every node if S never falls.
 *   q          f32 [B][D][V] rows at q + b*q_stride_b + k*q_stride_k (elements),
 *              vocabulary contiguous; row k is the marginal of position k+1.
 *   N_max      budget, 1..128.  D in 1..8, V in 1..262144.
 *   cost       f64 [N_max] device array, cost[n-1] = C(n), the caller's measured cost of
 *              verifying an n-node tree (for example µs per verify step); NULL keeps N_max
 *              nodes.  l_ar = L_AR (cost units per autoregressive token).
 *   parents    out int32 [B][N_max+1], virtual-root form (parents[b][i] < i, column 0 = 0);
 *   tokens     out int32 [B][N_max+1] (column 0 = 0);
 *   n_nodes    out int32 [B];
 *   rho        out f64 [B][N_max+1] (rho[b][0] = 1).  Entries past n_nodes are 0.
 *   status     in/out int32 [B]: a sequence whose status is not OK is skipped (n_nodes 0);
 *              a q row with an entry outside [0,1] or NaN sets TMV_ERR_INPUT.
 *   workspace: tmv_tree_best_first_workspace() bytes, 16-byte aligned, no initialisation.
 * Together, parents, n_nodes and tokens are the input of tmv_tree_build_ancestors
 * (TMV_PARENTS_VROOT, M_max = N_max) and of the verify step.
 */
size_t tmv_tree_best_first_workspace(int B, int D, int V, int N_max);
int tmv_tree_best_first(int B, int D, int V, int N_max, const float *q, int64_t q_stride_b,
                        int64_t q_stride_k, const double *cost, double l_ar, int32_t *parents,
                        int32_t *tokens, int32_t *n_nodes, double *rho, int32_t *status,
                        void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* TMV_H */
