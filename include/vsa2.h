/* vsa2.h -- C interface of the VSA2 sparse-attention layer for MI355X (gfx950).
 *
 * The method is the attention layer of "Improving Video Sparse Attention with
 * Fine-grained Router and Sparse Rebasing" (arXiv 2609.32882): a fine-grained
 * router (§2.2 Eq.(5)-(7)), a per-sequence TopK (Eq.(8)-(9)), a block-sparse
 * fine branch (Eq.(12)), a cube-pooled coarse branch (Eq.(1)-(4)) and a tanh
 * gate (Eq.(13)-(14)); the router takes no gradient (§2.1).
 *
 * Conventions (all entry points):
 *  - Every tensor argument is DEVICE memory owned by the caller, contiguous,
 *    row-major, 16-byte aligned.  The library never allocates or frees; the
 *    scratch it needs comes from a caller workspace `ws` of at least the size
 *    vsa2_workspace_size() reports (its contents need not be initialised).
 *  - Q, K, V, O_f, O, dO, dQ, dK, dV are [batch, heads, L, head_dim] in the
 *    storage dtype of vsa2_problem.dtype, tokens in cube-tiled order (§2.2
 *    "Permutation"): the 64 tokens of each 4x4x4 cube are contiguous (cubes in
 *    raster order over the (T/4, Y/4, X/4) cube grid); inside a cube the eight
 *    2x2x2 sub-cubes follow in raster order, each holding its 8 tokens in
 *    raster order.  Router pooling windows are therefore the contiguous groups
 *    of 8 tokens and the attention blocks the contiguous groups of 64.
 *  - Attention block B = 64 (one 4x4x4 cube) by default, router pool R = 8
 *    (2x2x2), so G = 8.  With block_tokens = 128 a block is two x-adjacent
 *    cubes (4x4x8), contiguous in the order above (cubes 2m, 2m+1), G = 16;
 *    blocks are numbered like these cube pairs.  B = 128 is the blog's
 *    inference for the paper's own runs (its §07); the paper gives no 3D cut.
 *    "nb" below counts blocks: nb = L / B.
 *  - MMDiT text conditioning (§2.2 after Eq.(12): the fine branch extends to
 *    full video-to-text and text-to-video attention): with text_tokens = Nt
 *    > 0 every per-token tensor of the attention (Q, K, V, O_f, O, dO, dQ,
 *    dK, dV and LSE) holds L video slots followed by Lt = 64 ceil(Nt / 64)
 *    text rows, the last Lt - Nt of them padding: [batch, heads, L + Lt, d].
 *    Video queries attend to their selected video blocks and to every text
 *    token; text queries attend to every video and text token (one softmax
 *    per row).  The router, TopK, coarse branch and gate see the video alone
 *    (X, dX, G stay [.., L, ..]); a text row's O is its O_f.
 *  - Padded grids (§2.2 "Kernel Implementation"): a latent side that is not a
 *    multiple of the block's side (4, and 8 along x for B = 128) is padded up
 *    to one, and every tensor holds the padded grid: L = B nb slots with
 *    nb = ceil(T/4) ceil(Y/4) ceil(X/(B/16)), in the order above.  Pad slots are not tokens.  Their input values are never read into
 *    a result (they must be finite); pad rows of O_f, O, G, dQ, dK, dV and dX
 *    are written as 0 and their LSE as -inf.  Pooling windows average their
 *    real tokens; a 2x2x2 window holding none is no router key and adds no
 *    router row; the coarse gradient of a block goes to its n real tokens as
 *    1/n each (1/B without padding).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns without synchronising.
 *  - Errors: argument and shape errors are reported before anything is
 *    enqueued and leave outputs untouched (VSA2_E_ARG / VSA2_E_SHAPE /
 *    VSA2_E_WORKSPACE / VSA2_E_UNSUPPORTED); a failed kernel launch returns
 *    VSA2_E_HIP.  Numerical outputs are bitwise deterministic for identical
 *    inputs on the same device (no floating-point atomics).
 */
#ifndef VSA2_H
#define VSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum vsa2_status {
  VSA2_OK = 0,
  VSA2_E_ARG = 1,         /* NULL pointer, misaligned pointer, bad scalar argument   */
  VSA2_E_SHAPE = 2,       /* empty or oversized grid (more than 46,340 cubes, more  */
                          /* than 65,535 batch x heads, or batch x heads x (cubes + */
                          /* text cubes + 8) x 256 beyond 2^32), head_dim not 64/128*/
  VSA2_E_WORKSPACE = 3,   /* workspace smaller than vsa2_workspace_size() reports     */
  VSA2_E_HIP = 4,         /* a HIP call or kernel launch failed                       */
  VSA2_E_UNSUPPORTED = 5, /* valid request the library does not implement             */
  VSA2_E_SCRATCH = 6      /* beyond the fixed scratch of vsa2_route_noalloc           */
};

enum vsa2_dtype { VSA2_F32 = 0, VSA2_BF16 = 1 };

/* Operations, for vsa2_workspace_size(). */
enum vsa2_op {
  VSA2_OP_POOL = 0,
  VSA2_OP_ROUTE = 1,
  VSA2_OP_TOPK = 2,
  VSA2_OP_PLAN = 3,
  VSA2_OP_FWD = 4,
  VSA2_OP_BWD = 5,
  VSA2_OP_COARSE = 6,
  VSA2_OP_COARSE_BWD = 7,
  VSA2_OP_ROUTE_COARSE = 8,
  VSA2_OP_TOPK_ROW = 9
};

typedef struct vsa2_problem {
  int32_t batch;          /* >= 1                                                     */
  int32_t heads;          /* >= 1 (multi-head attention: as many K/V heads as Q heads)*/
  int32_t head_dim;       /* d: 64 or 128                                             */
  int32_t lat_t, lat_y, lat_x; /* latent grid, each >= 1; padded up to whole blocks   */
  int32_t dtype;          /* vsa2_dtype of Q, K, V, O_f, O, dO, dQ, dK, dV, X, dX     */
  float softmax_scale;    /* <= 0 selects 1/sqrt(head_dim)                            */
  int32_t block_tokens;   /* attention block B: 64 (0 selects it) or 128, see above   */
  int32_t text_tokens;    /* MMDiT text tokens Nt >= 0 joining the fine branch, above */
  int32_t router_pool;    /* edge of the router's pooling window, below: 2 (0 selects */
                          /* it), 1 or 4; anything else is VSA2_E_SHAPE               */
} vsa2_problem;

/* The router's pooling window (paper §2.2 Eq.(5), R = pool^3 tokens, G = 64 / R
 * pooled tokens per cube).  2: the 2x2x2 windows the method uses (R = 8, G =
 * 8).  The two ends exist for the special cases the paper names: 1 (R = 1, G
 * = 64) makes the router the token-level softmax averaged over each 64 x 64
 * tile, i.e. the oracle block scores P_oracle of Eq.(10)-(11); 4 (R = 64, G =
 * 1) makes it the coarse branch's P_c of Eq.(2).  Pools 1 and 4 need 64-token
 * blocks on an unpadded grid (vsa2_pool and vsa2_route return
 * VSA2_E_UNSUPPORTED otherwise); they cost more (pool 1 runs the router over
 * every token, with an nb*8 x nb*8 intermediate in the workspace) and serve
 * checks, not training. */

/* Human-readable name of a status code (static string). */
const char* vsa2_status_string(int status);

/* Bytes of workspace `op` needs for problem `p` (topk: average KV cubes per
 * query cube; d_model: width of X for the coarse/gate ops, else ignored).
 * Pure host computation; enqueues nothing. */
int vsa2_workspace_size(const vsa2_problem* p, int32_t op, int32_t topk, int32_t d_model, size_t* bytes);

/* Bytes of the work schedule of the fine branch for budget `topk` (0 when the
 * problem needs none).  The schedule answers the question the paper's
 * per-sequence TopK (§2.2 Eq.(8)-(9)) leaves open: every query cube holds its
 * own number of KV cubes (and every KV cube is selected by its own number of
 * query cubes), and the blog's reproduction notes (its §12) leave the
 * scheduler of these unequal lists to the implementer (its §10 counts the
 * imbalance and the block-sparse memory traffic among the gap to the ideal
 * speed-up).  For every (batch, head) it orders the query cubes (forward, dQ)
 * and the KV cubes (dK/dV) by a min-hash of their lists, so cubes that gather
 * the same tiles run next to each other on one XCD's L2; cuts the order into
 * 8 ranges of equal work, one per XCD; and puts each range's long lists
 * first.  The fine kernels then run as many workgroups as fit on the device,
 * each taking cubes from its XCD's queue and then from the others (the
 * forward two consecutive cubes at a time, staging each KV cube of their two
 * lists once), and give the same results, bit for bit, as with no schedule.
 * Written by vsa2_topk_per_seq, vsa2_topk_per_row and vsa2_plan_from_csr from
 * the selection they produce or receive, read by vsa2_sparse_attn_fwd/bwd.
 * Built by attention block (a cube, or with block_tokens = 128 a pair of
 * cubes that one workgroup runs whole).  With text_tokens > 0 and 64-token
 * blocks every text cube is one more item (its list is every cube), and the
 * text items of all heads open the queues (text cubes 2u, 2u + 1 of a head
 * side by side, for the forward's pairs); with text_tokens > 0 and
 * block_tokens = 128 the size is 0 and the kernels run one workgroup per cube.
 * A schedule built for another selection of the same problem is still valid
 * (it lists every block once), only balanced for that selection; a buffer that
 * no build for this problem wrote is recognised by its header, and the fine
 * kernels then take the blocks in plain order, with the same results.
 * Layout (opaque to callers): for query blocks, then KV blocks, a 256-byte
 * header (queue starts and lengths, the item count, a marker) and
 * batch*heads*(nb + ntc) int32 items (ntc text cubes). */
int vsa2_sched_size(const vsa2_problem* p, int32_t topk, size_t* bytes);

/* Bytes of the `pooled` buffer written by vsa2_pool (see there). */
int vsa2_pooled_size(const vsa2_problem* p, size_t* bytes);

/* Bytes of the `saved` buffer written by vsa2_coarse_gate (see there). */
int vsa2_saved_size(const vsa2_problem* p, size_t* bytes);

/* Per-sequence budget k = min(nb * topk, nb^2) selected pairs per (batch, head),
 * nb = L / 64 cubes of the padded grid (paper §2.2 Eq.(9): N*K blocks per
 * sequence). */
int vsa2_budget(const vsa2_problem* p, int32_t topk, int64_t* k);

/* Mean pooling of the router (Eq.(5), windows of R = router_pool^3 tokens) and
 * of the coarse branch (Eq.(1), cubes of 64 tokens), one read of Q, K, V.
 *   pooled (written), in order, each [batch, heads, rows, d] in the storage dtype:
 *     Q_r, K_r    rows = L/R   (router operands; bf16 storage rounds the fp32 mean
 *                               to nearest-even, the router's stated precision;
 *                               pool 1 copies the tokens; pool 4 has no rows here,
 *                               its router operands are Q_c, K_c)
 *     Q_c, K_c, V_c rows = nbp = nb rounded up to a multiple of 64; rows >= nb are 0
 *   Size from vsa2_pooled_size(). */
int vsa2_pool(const vsa2_problem* p, const void* q, const void* k, const void* v,
              void* pooled, void* stream);

/* Fine-grained router, Eq.(6)-(7), fused: two passes over the pooled keys
 * (log-sum-exp, then softmax + G x G mean pooling), P_hat_r never stored.
 *   pooled: from vsa2_pool.
 *   scores (written): fp32 [batch, heads, nb, nb], P_r[i][j] = mean over the
 *     G x G pooled (query, key) pairs of cubes i, j of softmax_b(q_a.k_b*scale).
 *     Every row sums to 1/G (padded grids: to the number of the cube's 2x2x2
 *     windows that hold a real token, over 64).  Pool 1: the passes run over
 *     the tokens with 8 x 8 means per pair of 2x2x2 sub-cubes, written to the
 *     workspace, and a third kernel averages each 8 x 8 block of those into
 *     P_r (the mean of means of equal-sized groups is the 64 x 64 mean).
 *     Pool 4: P_c, as vsa2_route_coarse computes it.
 *   ws: vsa2_workspace_size(VSA2_OP_ROUTE). */
int vsa2_route(const vsa2_problem* p, const void* pooled, float* scores,
               void* ws, size_t ws_bytes, void* stream);

/* Per-sequence TopK, Eq.(8)-(9): for every (batch, head) keep the k largest of
 * the nb*nb block scores (k from vsa2_budget; ties at the cut-off go to the
 * lower flat index i*nb + j).  Exact radix select on the fp32 bit patterns.
 *   scores: fp32 [batch, heads, nb, nb], finite and >= 0.
 *   row_ptr (written) int32 [batch, heads, nb+1]; col_idx (written) int32
 *     [batch, heads, k]: selected KV cubes of query cube i are
 *     col_idx[row_ptr[i] .. row_ptr[i+1]), ascending.  row_ptr[nb] = k.
 *   col_ptr, row_idx (written): the same selection by KV cube (CSC), query
 *     cubes ascending; used by the backward pass.  Both NULL for a selection
 *     only the forward runs on (inference): no CSC is built, and the schedule
 *     gets only its query-cube side.  One NULL without the other is
 *     VSA2_E_ARG.
 *   sched (written): the work schedule of this selection, sched_bytes >=
 *     vsa2_sched_size() and 256-byte aligned; NULL builds none (the fine
 *     kernels then run one workgroup per cube).
 *   ws: vsa2_workspace_size(VSA2_OP_TOPK). */
int vsa2_topk_per_seq(const vsa2_problem* p, const float* scores, int32_t topk,
                      int32_t* row_ptr, int32_t* col_idx, int32_t* col_ptr, int32_t* row_idx,
                      void* sched, size_t sched_bytes, void* ws, size_t ws_bytes, void* stream);

/* CSC form (col_ptr, row_idx) of a caller-chosen selection given as CSR
 * (row_ptr, col_idx, same layout as vsa2_topk_per_seq, exactly k entries per
 * (batch, head), columns ascending and distinct in each row).  Entries
 * outside [0, nb) are ignored.  A column listed twice in one row is a caller
 * error that stays memory-safe: the CSC holds the pair once and the unused
 * CSC slots at the end of the list are never read (col_ptr[nb] is then below
 * k), while the forward and the dQ pass, which read the CSR, take the KV
 * cube's keys twice into that row's softmax.
 *   sched (written, or NULL): the work schedule, as for vsa2_topk_per_seq.
 *   ws: vsa2_workspace_size(VSA2_OP_PLAN). */
int vsa2_plan_from_csr(const vsa2_problem* p, int32_t topk, const int32_t* row_ptr, const int32_t* col_idx,
                       int32_t* col_ptr, int32_t* row_idx, void* sched, size_t sched_bytes,
                       void* ws, size_t ws_bytes, void* stream);

/* vsa2_route for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and result as vsa2_route, with the router's scratch (the
 * log-sum-exp of every pooled query and, on padded grids, one key-existence
 * word per 64 pooled keys: vsa2_workspace_size(VSA2_OP_ROUTE) bytes) taken
 * from a fixed array in device memory that the library holds on every GPU it
 * runs on until the process ends, instead of a caller workspace.
 *   The array holds vsa2_route_noalloc_limit() bytes (8 MiB; at 720p with 20
 *   heads the router needs 2.2 MB): a larger problem returns VSA2_E_SCRATCH
 *   before anything is enqueued.  The call allocates and frees nothing.
 *   Every call on one GPU shares that GPU's array and leaves its scratch
 *   there; calls that overlap on one GPU (two streams, two host threads)
 *   race and must be ordered by the caller. */
int vsa2_route_noalloc(const vsa2_problem* p, const void* pooled, float* scores, void* stream);

/* Size in bytes of vsa2_route_noalloc's fixed device scratch. */
int vsa2_route_noalloc_limit(size_t* bytes);

/* vsa2_route for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and result as vsa2_route, with the router's scratch (the
 * log-sum-exp of every pooled query and, on padded grids, one key-existence
 * word per 64 pooled keys: vsa2_workspace_size(VSA2_OP_ROUTE) bytes) taken
 * from a fixed array in device memory that the library holds on every GPU it
 * runs on until the process ends, instead of a caller workspace.
 *   The array holds vsa2_route_noalloc_limit() bytes (8 MiB; at 720p with 20
 *   heads the router needs 2.2 MB): a larger problem returns VSA2_E_SCRATCH
 *   before anything is enqueued.  The call allocates and frees nothing.
 *   Every call on one GPU shares that GPU's array and leaves its scratch
 *   there; calls that overlap on one GPU (two streams, two host threads)
 *   race and must be ordered by the caller. */
int vsa2_route_noalloc(const vsa2_problem* p, const void* pooled, float* scores, void* stream);

/* Size in bytes of vsa2_route_noalloc's fixed device scratch. */
int vsa2_route_noalloc_limit(size_t* bytes);

/* The VSA router the paper compares against (§1 and Figure 1 left; Eq.(1)-(2)):
 * block scores from the coarse branch's own attention map,
 * P_c = softmax(Q_c K_c^T * scale) over the nb block means, no G x G pooling.
 *   pooled: from vsa2_pool (its Q_c, K_c).
 *   scores (written): fp32 [batch, heads, nb, nb] = P_c; every row sums to 1.
 *   ws: vsa2_workspace_size(VSA2_OP_ROUTE_COARSE). */
int vsa2_route_coarse(const vsa2_problem* p, const void* pooled, float* scores,
                      void* ws, size_t ws_bytes, void* stream);

/* The VSA router's TopK: every query block keeps its own min(topk, nb)
 * largest scores (ties to the lower column), instead of the per-sequence
 * budget of Eq.(8)-(9).  Same outputs, sizes and budget (vsa2_budget) as
 * vsa2_topk_per_seq; row_ptr[i] = i min(topk, nb).
 *   scores: fp32 [batch, heads, nb, nb], finite and >= 0.
 *   col_ptr, row_idx: as for vsa2_topk_per_seq (both NULL: forward only).
 *   sched (written, or NULL): the work schedule, as for vsa2_topk_per_seq.
 *   ws: vsa2_workspace_size(VSA2_OP_TOPK_ROW). */
int vsa2_topk_per_row(const vsa2_problem* p, const float* scores, int32_t topk, int32_t* row_ptr,
                      int32_t* col_idx, int32_t* col_ptr, int32_t* row_idx, void* sched, size_t sched_bytes,
                      void* ws, size_t ws_bytes, void* stream);

/* Fine branch forward, Eq.(12): block-sparse attention of every query cube
 * over its selected KV cubes only (-inf mask elsewhere, §2.1).
 *   row_ptr, col_idx: the selection (CSR as above, k = vsa2_budget(topk)).
 *   sched: the schedule the call that produced this selection wrote, or NULL
 *     (one workgroup per query cube, results equal); vsa2_sched_size() bytes.
 *   o_f (written): storage dtype [batch, heads, L, d].
 *   lse (written): fp32 [batch, heads, L], natural-log log-sum-exp of the scaled
 *     scores of each query over its selected keys (kept for the backward).
 *   A query cube with no selected KV cube gets o_f = 0 and lse = -inf.
 *   ws: vsa2_workspace_size(VSA2_OP_FWD): 256 bytes (the schedule's queue
 *     counters) when the problem has a schedule, else 0 (ws may be NULL). */
int vsa2_sparse_attn_fwd(const vsa2_problem* p, int32_t topk, const void* q, const void* k, const void* v,
                         const int32_t* row_ptr, const int32_t* col_idx, const void* sched, void* o_f, float* lse,
                         void* ws, size_t ws_bytes, void* stream);

/* Fine branch backward with the selection held fixed (the router takes no
 * gradient, §2.1-§2.2), plus the coarse-branch gradients spread back to the
 * tokens.
 *   q, k, v, o_f, lse: as in / out of vsa2_sparse_attn_fwd; d_o = dL/dO (the
 *     gate adds O_f with weight one, Eq.(14), so dL/dO_f = dL/dO).
 *   row_ptr, col_idx, col_ptr, row_idx: the selection in CSR and CSC form.
 *   sched: the selection's schedule or NULL (one workgroup per cube); the
 *     results are the same bit for bit.
 *   dqkv_c: fp32 [3, batch, heads, nb, d] gradients w.r.t. the pooled Q_c, K_c,
 *     V_c (from vsa2_coarse_gate_bwd) or NULL; each token of cube c receives
 *     1/64 of row c (the adjoint of the mean pooling).
 *   dq, dk, dv (written, overwritten): storage dtype [batch, heads, L, d].
 *   dK and dV are accumulated per KV cube over its query list in a fixed order
 *   (no atomics), so results are bitwise reproducible.
 *   ws: vsa2_workspace_size(VSA2_OP_BWD). */
int vsa2_sparse_attn_bwd(const vsa2_problem* p, int32_t topk, const void* q, const void* k, const void* v,
                         const void* o_f, const float* lse, const void* d_o,
                         const int32_t* row_ptr, const int32_t* col_idx,
                         const int32_t* col_ptr, const int32_t* row_idx, const void* sched,
                         const float* dqkv_c, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                         void* stream);

/* Coarse branch, Eq.(1)-(4), and gated merge, Eq.(13)-(14).
 *   pooled: from vsa2_pool.  x: storage dtype [batch, L, d_model] hidden states
 *   in the same token order.  w_g: fp32 [d_model, heads], one gate column per
 *   head (zero at initialisation gives O = O_f).  o_f: fine-branch output.
 *   o (written): storage dtype [batch, heads, L, d], O = tanh(X W_g) * O_c + O_f.
 *   saved (written, fp32, for the backward; size vsa2_saved_size):
 *     O_hat_c [batch, heads, nb, d] | lse_c [batch, heads, nb] | G [batch, heads, L]
 *   ws: vsa2_workspace_size(VSA2_OP_COARSE, d_model). */
int vsa2_coarse_gate(const vsa2_problem* p, const void* pooled, const void* x, int32_t d_model,
                     const float* w_g, const void* o_f, void* o, float* saved,
                     void* ws, size_t ws_bytes, void* stream);

/* Backward of vsa2_coarse_gate.
 *   d_o: dL/dO.  saved: as written by vsa2_coarse_gate for the same inputs.
 *   dqkv_c (written): fp32 [3, batch, heads, nb, d], gradients w.r.t. Q_c, K_c, V_c
 *     (pass it to vsa2_sparse_attn_bwd).
 *   dx (written): storage dtype [batch, L, d_model]; dw_g (written): fp32
 *     [d_model, heads], reduced over tokens in a fixed order.
 *   ws: vsa2_workspace_size(VSA2_OP_COARSE_BWD, d_model). */
int vsa2_coarse_gate_bwd(const vsa2_problem* p, const void* pooled, const void* x, int32_t d_model,
                         const float* w_g, const float* saved, const void* d_o,
                         float* dqkv_c, void* dx, float* dw_g, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostic kernel timer (for benchmarks and tests, not for production use).
 * vsa2_kernel_timer_start(kernel, capacity): from now on every launch of the
 * given kernel records one HIP event on its launch stream right before the
 * launch and one right after, for at most `capacity` launches (capacity in
 * 1..4096; events are created once and reused).  Several kernels may be
 * armed at the same time.
 * vsa2_kernel_timer_stop(kernel, ms, launches): waits for the last recorded
 * event of that kernel, writes the summed launch durations in milliseconds
 * and the number of launches timed, and disarms it.
 * Not thread-safe: arm, run and stop from one host thread.
 * ------------------------------------------------------------------------- */
enum vsa2_kernel {
  VSA2_K_FINE_FWD = 0,        /* block-sparse attention forward (fine branch)         */
  VSA2_K_BWD_DKDV = 1,        /* fine-branch dK/dV (KV-cube major)                    */
  VSA2_K_BWD_DQ = 2,          /* fine-branch dQ (query-cube major)                    */
  VSA2_K_ROUTER_LSE = 3,      /* router pass 1: log-sum-exp of every pooled query     */
  VSA2_K_ROUTER_SCORES = 4,   /* router pass 2: softmax + 8x8 block mean              */
  VSA2_K_COUNT = 5
};
int vsa2_kernel_timer_start(int32_t kernel, int32_t capacity);
int vsa2_kernel_timer_stop(int32_t kernel, float* ms, int32_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* VSA2_H */
