/* ddt.h -- C ABI of libddt.so: the DDTree tree-verification step on MI355X (gfx950).
 *
 * One verify round of tree speculative decoding on a hybrid model (full-attention
 * layers with a KV cache, Gated DeltaNet layers with a fixed-size recurrent state and
 * a short-conv state):
 *   ddt_build_tree     draft tree of B nodes from the drafter's per-depth logits
 *   ddt_tree_attn      tree-masked attention of every node over prefix + ancestors
 *   ddt_tree_attn_rope the same, from pre-rotation q and tree K/V: RoPE at positions
 *                      prefix + depth, tree K/V written to their scratch
 *   ddt_tree_rope      the rotation step alone (for ddt_tree_attn_paged callers)
 *   ddt_tree_attn_paged the same over a paged committed cache (block table + page pool)
 *   ddt_gdn_tree_step  short conv + gated delta rule, every node from its parent
 *   ddt_gdn_tree_step_deferred / ddt_gdn_tree_states  the same with the node states
 *                      written by a second call (e.g. on another stream)
 *   ddt_tree_accept    greedy walk of the tree against the target's argmax tokens
 *   ddt_tree_accept_sampled  the walk over sampled target tokens (Gumbel-max draws)
 *   ddt_commit         copy only the accepted path into the committed buffers
 *   ddt_commit_paged   the same with the KV rows scattered into a paged cache
 *   ddt_gdn_replay     (alternative to storing node states) advance the committed GDN
 *                      and conv state along the accepted path
 *
 * Conventions shared by every call
 *   - Tensor arguments are DEVICE pointers owned by the caller; the library allocates
 *     no device memory and keeps no state between calls.  Scratch space, where a call
 *     needs it, is a caller-provided device buffer `ws` of at least the size the
 *     matching *_workspace() query returns.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  It returns a status synchronously after host-side validation and the
 *     launches; a fault inside a kernel surfaces at the caller's next stream sync.
 *   - No call synchronises the device or reads device memory on the host: lengths
 *     such as prefix_len and acc_len are read on the device, so a round can be
 *     captured in a HIP graph.
 *   - Arrays are row-major, leftmost index slowest.  n = batch, B = budget (non-root
 *     nodes), T = B+1 tree rows (row 0 is the root), L = maximum depth, V = vocab,
 *     P = committed prefix length (per sequence, on the device), Pmax = cache capacity.
 *   - bf16 data is IEEE bfloat16 (upper half of a float32), stored as 16-bit words.
 *   - Limits: 1 <= B <= 64 (one 64-bit mask word per row, root implicit), L <= 63.
 *   - Errors: DDT_ERR_ARG for a null pointer or an out-of-range size;
 *     DDT_ERR_UNSUPPORTED for a dtype or head size outside the built set;
 *     DDT_ERR_WORKSPACE for a workspace smaller than the query; DDT_ERR_HIP when a
 *     launch fails.  ddt_last_error() returns a message for the last failure on the
 *     calling thread.
 *
 * Sources (web pages on DDTree tree speculative decoding):
 *   [notes]  "DDTree on vLLM: candid research notes on tree speculation for Qwen3.6"
 *            (lotusmake.com): sections "Why hybrid attention makes it hard",
 *            "What broke along the way", "Where the next step is".
 *   [arch]   "From DDTree to drafter training" (magik.net): section
 *            "The Architecture of DDTree".
 *   [spec]   "The architecture of speculation" (magik.net): section
 *            "The DDTree Integration Challenge".
 */
#ifndef DDT_H
#define DDT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DDT_OK = 0,
  DDT_ERR_ARG = 1,
  DDT_ERR_UNSUPPORTED = 2,
  DDT_ERR_WORKSPACE = 3,
  DDT_ERR_HIP = 4
} ddt_status;

typedef enum { DDT_F32 = 0, DDT_BF16 = 1 } ddt_dtype;

/* Name of a status code (static string). */
const char* ddt_status_string(int status);
/* Message describing the last failed call on this thread ("" if none). */
const char* ddt_last_error(void);
/* ABI version of this header/library pair. */
int ddt_abi_version(void);

/* ---------------------------------------------------------------- tree build
 * [arch]: a block drafter gives one distribution per future position; take the
 * top-K tokens and log-probs of every depth, seed a max-heap with the best depth-1
 * token, pop the globally best node, push its next-ranked sibling and its best
 * child, stop after B pops; flatten into ids, per-depth positions and an
 * ancestor-only mask.  [notes] "What broke along the way": depth logits are not
 * branch-conditioned, so a node's score is the sum of its path's log-probs.
 *
 *   draft_logits [n][L][V] (dt)  row d = logits of depth d+1 (full-vocab log-softmax
 *                                is taken in fp32)
 *   K            candidates per depth (0 = B; must be <= 64)
 *   root_token   [n] int32       token of row 0 (the previous round's bonus token)
 * outputs, rows in pop order (parents precede children):
 *   tok, parent, depth [n][T] int32   row 0: root_token, -1, 0
 *   score [n][T] f32                  summed log-prob (row 0: 0)
 *   anc   [n][T] u64                  bit j set <=> row j+1 is an ancestor of, or is,
 *                                     the row (row 0 implicit, anc[0] = 0)
 * Heap order: score desc, token id asc, parent row asc.  Rows left unused because the
 * tree has fewer than B prefixes get tok = parent = depth = -1, score = -inf, anc = 0.
 * Position ids are prefix_len + depth.  Requires V <= 2^20 and ceil(V/16384)*K <= 2048.
 */
size_t ddt_build_tree_workspace(int n, int L, int V, int B, int K);
int ddt_build_tree(const void* draft_logits, int dt, int n, int L, int V, int B, int K,
                   const int32_t* root_token, int32_t* tok, int32_t* parent, int32_t* depth,
                   float* score, uint64_t* anc, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- tree build, no allocation
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): ddt_build_tree with the same arguments
 * and results, minus the workspace.  Its scratch is a static device array of
 * ddt_build_tree_noalloc_max_scratch() bytes (8 MiB) per device, held from the first call
 * on a device until the process ends; the call allocates nothing and calls no allocating
 * routine.  A size whose scratch (ddt_build_tree_workspace) exceeds it is rejected with
 * DDT_ERR_WORKSPACE before any HIP call (n = 64 at L = 15, V = 151936, K = 64 fits).
 * Every call on a device shares that device's array: calls that overlap on one device
 * (different streams, or host threads) race and must be serialised by the caller.
 * stream must belong to the current device.  The array needs no clearing: every call
 * writes the scratch it reads.
 */
size_t ddt_build_tree_noalloc_max_scratch(void);
int ddt_build_tree_noalloc(const void* draft_logits, int dt, int n, int L, int V, int B, int K,
                           const int32_t* root_token, int32_t* tok, int32_t* parent, int32_t* depth,
                           float* score, uint64_t* anc, void* stream);

/* ---------------------------------------------------------------- tree attention
 * [notes] "Why hybrid attention makes it hard": each tree row attends to the
 * committed prefix plus its own ancestors and never to its siblings.  [arch]: one
 * verify pass over root + all nodes with an ancestor-only mask.
 *
 *   q       [n][T][Hq][D]     (dt) queries of the tree rows (post-RoPE)
 *   k_cache [n][Hkv][Pmax][D] (dt) committed keys; rows >= prefix_len[s] are ignored
 *   v_cache [n][Hkv][Pmax][D] (dt)
 *   prefix_len [n] int32 (device), each in [0, Pmax]
 *   k_tree, v_tree [n][Hkv][T][D] (dt) keys/values of the tree rows (separate scratch;
 *                  the committed cache is not written)
 *   anc     [n][T] u64        masks from ddt_build_tree
 *   out     [n][T][Hq][D]     (dt)
 * Query head h uses kv head h / (Hq/Hkv).  Scores, softmax and accumulation in fp32;
 * bf16 products on the matrix cores.  scale <= 0 selects D^-1/2.
 * Built: D in {64, 128, 256}; Hq % Hkv == 0; Hq/Hkv <= 16.
 */
size_t ddt_tree_attn_workspace(int n, int B, int Hq, int Hkv, int D, int Pmax, int dt);
int ddt_tree_attn(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* prefix_len, const void* k_tree, const void* v_tree,
                  const uint64_t* anc, int n, int B, int Hq, int Hkv, int D, int Pmax,
                  float scale, int dt, void* out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- paged committed cache
 * [notes] "Why hybrid attention makes it hard", "Where the next step is": the
 * ancestor-mask branch attention is to run over the serving engine's paged KV blocks.
 * Paged layout of a layer's committed keys (values alike):
 *   k_pages [num_pages][Hkv][page_size][D] (dt): a page holds page_size consecutive
 *           positions of every kv head of one sequence;
 *   block_table [n][max_blocks] int32 (device): position p of sequence s is slot
 *           p % page_size of page block_table[s][p / page_size];
 *   capacity max_blocks * page_size plays the role of Pmax.
 * ddt_tree_attn_paged computes exactly ddt_tree_attn over the cache this table
 * describes (same q, k_tree, v_tree, anc, out, scale, workspace rules; workspace size
 * from ddt_tree_attn_paged_workspace).  Table entries for positions < prefix_len[s]
 * must lie in [0, num_pages): an entry outside is clamped into the range (the output
 * is then wrong, but no access leaves the pool).
 * ddt_commit_paged is ddt_commit with the accepted KV rows written to positions
 * P..P+a through the table; a sequence whose destination pages are not all in
 * [0, num_pages), or that would pass the capacity, is not committed (acc_len = -1).
 * Built: page_size a power of two in [1, 65536]; max_blocks * page_size <= 2^30.
 */
size_t ddt_tree_attn_paged_workspace(int n, int B, int Hq, int Hkv, int D, int max_blocks, int page_size,
                                     int dt);
int ddt_tree_attn_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                        int max_blocks, int page_size, int num_pages, const int32_t* prefix_len,
                        const void* k_tree, const void* v_tree, const uint64_t* anc, int n, int B, int Hq,
                        int Hkv, int D, float scale, int dt, void* out, void* ws, size_t ws_bytes,
                        void* stream);

/* ---------------------------------------------------------------- tree attention with RoPE by depth
 * [notes] "What broke along the way", "Where the next step is": positions and RoPE of
 * the tree rows follow the branch depth; the tree's K/V go to scratch, never into the
 * committed cache.  Same attention as ddt_tree_attn, from pre-rotation inputs:
 *   pos[s][t] = prefix_len[s] + depth[s][t]   (depth as written by ddt_build_tree)
 *   RoPE, rotate-half layout: for j < rot_dim/2 the channel pair (j, j + rot_dim/2) turns
 *   by pos * theta^(-2j/rot_dim):  x_j' = x_j cos - x_{j+r/2} sin,
 *   x_{j+r/2}' = x_{j+r/2} cos + x_j sin; channels >= rot_dim are unchanged.
 *   q      [n][T][Hq][D]   queries before rotation (read only)
 *   k_new  [n][T][Hkv][D]  the tree rows' keys before rotation, token-major (read only)
 *   v_new  [n][T][Hkv][D]  the tree rows' values, token-major (read only)
 *   k_tree, v_tree [n][Hkv][T][D]  WRITTEN: rotated keys / copied values, the layout
 *                  ddt_tree_attn reads and ddt_commit copies into the cache
 *   other arguments as ddt_tree_attn (k_cache/v_cache hold already-rotated keys).
 * Angles are formed in fp64 and applied in fp32; rotated values are rounded to dt.
 * ws: ddt_tree_attn_rope_workspace() bytes (the rotated queries, then the attention's
 * own workspace); required.  Built: rot_dim a multiple of 16 in [16, D]; theta > 1.
 */
size_t ddt_tree_attn_rope_workspace(int n, int B, int Hq, int Hkv, int D, int Pmax, int dt);
/* The rotation step alone (the first kernel of ddt_tree_attn_rope): rotated queries
 * to q_out [n][T][Hq][D], rotated keys / copied values to k_tree / v_tree.  For callers
 * that then attend with ddt_tree_attn_paged.  Same arguments and limits as above. */
int ddt_tree_rope(const void* q, const void* k_new, const void* v_new, const int32_t* depth,
                  const int32_t* prefix_len, int rot_dim, float theta, int n, int B, int Hq, int Hkv, int D,
                  int dt, void* q_out, void* k_tree, void* v_tree, void* stream);
int ddt_tree_attn_rope(const void* q, const void* k_new, const void* v_new, const int32_t* depth, int rot_dim,
                       float theta, const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                       void* k_tree, void* v_tree, const uint64_t* anc, int n, int B, int Hq, int Hkv, int D,
                       int Pmax, float scale, int dt, void* out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- GDN tree step
 * [notes] "Why hybrid attention makes it hard": every node reads the Gated DeltaNet
 * state and the short-conv state of its parent and writes its own to scratch, never
 * to the committed state.  [spec]: per-branch state, not one shared state.
 * Per node i with parent p (the committed state when p < 0), per head:
 *   conv:  window = [conv state of p (W-1 rows, oldest first), x_i];
 *          y = SiLU(sum_j conv_w[c][j] * window[j][c]); conv_scratch[i] = window[1..W-1]
 *          channels C = 2*H*dk hold [q | k]; q *= dk^-1/2; k /= sqrt(|k|^2 + 1e-6)
 *   delta: S' = g_i S_p;  S_i = S' + beta_i (v_i - S' k_i) k_i^T;  o_i = S_i q_i
 *   x [n][T][C] (act_dt), conv_w [C][W] (f32), conv_state [n][W-1][C] (act_dt),
 *   conv_scratch [n][T][W-1][C] (act_dt, written; exact copies of inputs)
 *   v [n][T][H][dv] (act_dt), beta, g [n][T][H] (f32)
 *   S [n][H][dv][dk] (f32, committed, read only), S_scratch [n][T][H][dv][dk] (f32, written)
 *   o [n][T][H][dv] (act_dt, written)
 *   parent [n][T] int32: parent[i] < i, or < 0 for a row that reads the committed state
 *   L: the tree's depth bound, 0 <= L <= 63.  Every row is processed whatever its depth
 *      by parent chain; L only selects the method (bf16 activations, states stored and
 *      L <= 16: chunk form, every state formed from S and its path's w k^T terms;
 *      otherwise the node-by-node walk).  Both agree to fp32 rounding.
 *   ws: workspace of ddt_gdn_tree_step_workspace() bytes (per-node q, k and k.q, or k
 *       and w, in fp32, the tree's depth-first order or depths, and the path records)
 * S_scratch and conv_scratch may both be NULL: then no node state is stored (o is still
 * written for every node) and the commit replays the accepted path with ddt_gdn_replay.
 * x, conv_state, conv_scratch, S, S_scratch and ws must be 16-byte aligned.
 * Built: dk = dv in {32, 64, 128}; W in [2, 8]; C == 2*H*dk.
 */
size_t ddt_gdn_tree_step_workspace(int n, int B, int H, int dk);
int ddt_gdn_tree_step(const void* x, const float* conv_w, const void* conv_state,
                      void* conv_scratch, const void* v, const float* beta, const float* g,
                      const float* S, float* S_scratch, void* o, const int32_t* parent,
                      int n, int B, int L, int H, int dk, int dv, int C, int W, int act_dt,
                      void* ws, size_t ws_bytes, void* stream);

/* The same step with the node states written by a call of their own, so that a caller can
 * run that write (the step's 93% of bytes; only the commit reads it) on another stream
 * while the next layers run: [notes] "Why hybrid attention makes it hard" (each node's
 * state goes to scratch; the commit reads the accepted one).
 * ddt_gdn_tree_step_deferred: everything of ddt_gdn_tree_step (chunk form) except S_scratch:
 *   o and conv_scratch are written, and each node's k, w, decay products and ancestor
 *   records are left in ws.  Same arguments and limits as ddt_gdn_tree_step without
 *   S_scratch; conv_scratch is required; bf16 activations only (DDT_ERR_UNSUPPORTED
 *   otherwise); any depth (the state write costs more for deeper nodes).
 * ddt_gdn_tree_states: writes S_scratch [n][T][H][dv][dk] (f32) from the committed S and
 *   the ws a ddt_gdn_tree_step_deferred call with the same n, B, H, dk left.  The caller
 *   keeps that ws and S unchanged and orders this call after that one (same stream, or an
 *   event); with several layers in flight each needs a ws of its own.
 * Results are the same as ddt_gdn_tree_step's with L <= 16, bit for bit.
 */
int ddt_gdn_tree_step_deferred(const void* x, const float* conv_w, const void* conv_state,
                               void* conv_scratch, const void* v, const float* beta, const float* g,
                               const float* S, void* o, const int32_t* parent, int n, int B, int L,
                               int H, int dk, int dv, int C, int W, int act_dt, void* ws,
                               size_t ws_bytes, void* stream);
int ddt_gdn_tree_states(const float* S, float* S_scratch, int n, int B, int H, int dk, int dv,
                        const void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- tree walk
 * [arch]: after the verify pass, walk down from the root while the target's token
 * at the current node equals one of its children's tokens.  [notes] "What broke
 * along the way": the bonus token is emitted, not accepted as a draft node.
 *   target_logits [n][T][V] (dt); argmax ties go to the lowest token id
 *   tok, parent [n][T] int32 from ddt_build_tree
 * outputs: acc_rows [n][L+1] int32 (root first, then accepted rows, -1 padded),
 *          acc_len [n] int32 (accepted non-root nodes a, 0..L; -1 if the tree is
 *          malformed: a parent row not before its child, or two siblings sharing the
 *          matched token), bonus [n] int32 (target argmax at the last accepted row).
 */
size_t ddt_tree_accept_workspace(int n, int B, int V);
int ddt_tree_accept(const void* target_logits, int dt, const int32_t* tok, const int32_t* parent,
                    int n, int B, int L, int V, int32_t* acc_rows, int32_t* acc_len,
                    int32_t* bonus, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- sampled walk
 * [notes] "What broke along the way": the walk compares sampled tokens (greedy-only
 * testing hid anomalies).  Same walk as ddt_tree_accept with each row's target token
 * drawn from softmax(z / t) instead of the argmax, by Gumbel-max:
 *   token(row) = argmax_v ( z[row][v] * (1/t) + gumbel[row][v] ),  ties to the lowest id
 * with t = temperature[s] of the row's sequence; 1/t, the product and the sum are each
 * one correctly rounded float32 operation (no fused multiply-add), so a host doing the
 * same float32 operations reproduces every decision.  t <= 0: greedy (argmax of z).
 * Every emitted token (accepted path and bonus) is then a draw of the target at its
 * own row, whatever the drafter proposed.
 *   gumbel      [n][T][V] f32 (device): the draws' noise, -log(-log U) of uniforms U,
 *               finite; supplied by the caller (one fresh array per round)
 *   temperature [n] f32 (device)
 *   other arguments and the workspace (ddt_tree_accept_workspace) as ddt_tree_accept.
 */
int ddt_tree_accept_sampled(const void* target_logits, int dt, const float* gumbel, const float* temperature,
                            const int32_t* tok, const int32_t* parent, int n, int B, int L, int V,
                            int32_t* acc_rows, int32_t* acc_len, int32_t* bonus, void* ws, size_t ws_bytes,
                            void* stream);

/* ---------------------------------------------------------------- commit
 * [notes] "Why hybrid attention makes it hard" and "Where the next step is": only
 * the accepted path is copied into the contiguous KV and recurrent buffers, through
 * an explicit commit keyed by node ids.  [arch]: the KV cache keeps only the
 * accepted path's entries.
 * For every sequence s with a = acc_len[s] in [0, L], P = prefix_len[s], P + a + 1 <= Pmax
 * and every accepted row acc_rows[s][0..a] a tree row in [0, T):
 *   every attention layer:  k_cache/v_cache[s][:][P+j] = k_tree/v_tree[s][:][acc_rows[s][j]], j = 0..a
 *   every GDN layer:        S[s] = S_scratch[s][r], conv_state[s] = conv_scratch[s][r],
 *                           r = acc_rows[s][a] (the deepest accepted row)
 *   prefix_len[s] += a + 1
 * Otherwise nothing of s is written and acc_len[s] becomes -1.  Copies are exact.
 * kv and gdn are HOST arrays of per-layer device pointers (n_kv, n_gdn entries; either
 * may be 0).  kv_dt is the element type of the KV buffers, act_dt of the conv buffers.
 */
typedef struct {
  const void* k_tree; /* [n][Hkv][T][D] */
  const void* v_tree;
  void* k_cache;      /* [n][Hkv][Pmax][D] */
  void* v_cache;
} ddt_kv_layer;

typedef struct {
  const float* S_scratch;   /* [n][T][H][dv][dk] */
  float* S;                 /* [n][H][dv][dk] */
  const void* conv_scratch; /* [n][T][W-1][C] */
  void* conv_state;         /* [n][W-1][C] */
} ddt_gdn_layer;

int ddt_commit(const int32_t* acc_rows, int32_t* acc_len, int32_t* prefix_len,
               const ddt_kv_layer* kv, int n_kv, int Hkv, int D, int Pmax, int kv_dt,
               const ddt_gdn_layer* gdn, int n_gdn, int H, int dk, int dv, int C, int W,
               int act_dt, int n, int B, int L, void* stream);
/* ddt_commit_paged: see "paged committed cache" above; kv[i].k_cache / v_cache are the
 * layer's page pools. */
int ddt_commit_paged(const int32_t* acc_rows, int32_t* acc_len, int32_t* prefix_len, const ddt_kv_layer* kv,
                     int n_kv, int Hkv, int D, const int32_t* block_table, int max_blocks, int page_size,
                     int num_pages, int kv_dt, const ddt_gdn_layer* gdn, int n_gdn, int H, int dk, int dv,
                     int C, int W, int act_dt, int n, int B, int L, void* stream);

/* ---------------------------------------------------------------- GDN replay on commit
 * [notes] "Where the next step is": scratch-buffer GDN and conv replay; [spec] "The
 * DDTree Integration Challenge": recompute or compact the recurrent state instead of
 * keeping a copy per branch.  For a round whose tree step stored no node state
 * (ddt_gdn_tree_step with S_scratch = conv_scratch = NULL), advance each GDN layer's
 * committed state along the accepted path.  Call it after ddt_commit of the same round
 * (which sets acc_len to -1 where nothing may be written); sequences with acc_len < 0,
 * or whose path rows are out of range, are left untouched.
 * For every sequence s with a = acc_len[s] >= 0 and path rows r_j = acc_rows[s][j]:
 *   for j = 0..a: window = [committed conv rows ..., x[r_0], ..., x[r_j]] (last W),
 *                 k = normalised SiLU(conv) of the k channels (as in the tree step),
 *                 S = g S + beta (v - g S k) k^T with the node's v, beta, g
 *   conv_state[s] = the last W-1 rows of the window of r_a (exact copies)
 * The result equals ddt_commit of stored states (S = S_scratch[r_a], conv_state =
 * conv_scratch[r_a]) up to fp32 rounding order of S.  layers is a HOST array of n_layers
 * entries of device pointers, each with the tree step's inputs of that layer.
 * Built: dk = dv in {32, 64, 128}; W in [2, 8]; C == 2*H*dk; L <= 63.
 */
typedef struct {
  const void* x;        /* [n][T][C] (act_dt), the tree step's input */
  const float* conv_w;  /* [C][W] */
  const void* v;        /* [n][T][H][dv] (act_dt) */
  const float* beta;    /* [n][T][H] */
  const float* g;       /* [n][T][H] */
  float* S;             /* [n][H][dv][dk] committed state, advanced in place (16-byte aligned) */
  void* conv_state;     /* [n][W-1][C] (act_dt) committed conv rows, replaced in place */
} ddt_gdn_replay_layer;

int ddt_gdn_replay(const int32_t* acc_rows, const int32_t* acc_len, const ddt_gdn_replay_layer* layers,
                   int n_layers, int H, int dk, int dv, int C, int W, int act_dt, int n, int B, int L,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DDT_H */
