/*
 * eagle3.h -- C-ABI of libeagle3.so: one EAGLE-3 draft-tree round and one
 * tree-verification round on an MI355X (gfx950) GPU.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The library never
 *    allocates or frees device memory; scratch space comes from a caller-provided device
 *    workspace whose size the matching *_workspace_size() function returns.
 *  - Every call is asynchronous on the caller's HIP stream, passed as `void* stream`
 *    (NULL = the default stream).  No call synchronises the host.
 *  - Tensors are dense, row-major, in the layouts stated per argument; float tensors start
 *    on a 16-byte boundary (kernels use 16-byte vector loads), else EAGLE3_EINVAL.  Float tensors are
 *    EAGLE3_F32 (IEEE fp32) or EAGLE3_BF16 (bfloat16) as the `dtype` argument says; ids and
 *    indices are int32; tree masks are uint64; log-sum-exp values and attention partials
 *    are always fp32 and use the natural logarithm.
 *  - Return value: EAGLE3_OK, or a negative status found on the host before any launch
 *    (nothing is enqueued then), or EAGLE3_EHIP if a launch failed.
 *  - Malformed DEVICE data (a parent index out of range, a token >= vocab) cannot be seen on
 *    the host: kernels clamp such indices so that no access leaves its buffer, and OR a
 *    flag into the optional caller-owned device word `dev_status` where one is taken.
 *  - The same inputs (and for sampling the same seed and round) give bit-identical outputs:
 *    every reduction runs in a fixed order and no floating-point atomics are used.
 *
 * Sources.  The pages that define each operation are cited per function:
 *  [P1] "EAGLE-3: Training-time Test 的投机推理加速" (paper deep-dive page).
 *  [P2] The EAGLE series evolution page (EAGLE-1 -> EAGLE-2 -> EAGLE-3, DFlash).
 *  [P3] "SpecForge：把 EAGLE3 从训练样本交付到 SGLang".
 *  [P4] "EAGLE-3 投机解码与 USP 长序列训练优化".
 *  [P5] The speculative-decoding thinking-budget page (tree verification steps).
 */
#ifndef EAGLE3_H
#define EAGLE3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EAGLE3_ABI_VERSION 1

#if defined(__GNUC__) || defined(__clang__)
#define EAGLE3_API __attribute__((visibility("default")))
#else
#define EAGLE3_API
#endif

/* status codes */
#define EAGLE3_OK 0
#define EAGLE3_EINVAL (-1)       /* null pointer, bad dtype, bad shape or size          */
#define EAGLE3_EUNSUPPORTED (-2) /* valid but outside what the kernels implement        */
#define EAGLE3_EWORKSPACE (-3)   /* workspace NULL or smaller than *_workspace_size()   */
#define EAGLE3_EHIP (-4)         /* a HIP launch or runtime call failed                 */

/* element types */
#define EAGLE3_F32 0
#define EAGLE3_BF16 1

/* bits OR-ed into the optional device status word */
#define EAGLE3_DEV_BAD_PARENT 1  /* parent[i] not in [0, i) (or root parent != -1)      */
#define EAGLE3_DEV_TOO_DEEP 2    /* a request has more nodes than the mask can hold     */
#define EAGLE3_DEV_BAD_TOKEN 4   /* a token id outside [0, vocab)                       */
#define EAGLE3_DEV_BAD_PATH 8    /* accept_len or a path node outside its request       */
#define EAGLE3_DEV_BAD_ROW 16    /* a destination row outside the cache                 */
#define EAGLE3_DEV_SYNC 32       /* a partial of another workgroup was not seen in time */

EAGLE3_API int eagle3_abi_version(void);
EAGLE3_API const char* eagle3_status_string(int status);

/* ====================================================================================
 * Drafter description.
 * One Llama-style decoder layer (the drafter is one decoder layer, [P1] 训练细节;
 * [P3] 多层特征融合到底融合了什么: a_{t+1} = D(e(x_t), g_t)) plus the feature-fusion
 * projection and the LM head.  Every projection is stored [out_features, in_features]
 * row-major; all tensors have element type `dtype`.
 * ==================================================================================== */
typedef struct eagle3_drafter {
  int32_t d;          /* hidden size of target features and drafter                      */
  int32_t n_heads_q;  /* Hq                                                              */
  int32_t n_heads_kv; /* Hkv (Hq % Hkv == 0; query head h uses KV head h / (Hq/Hkv))     */
  int32_t head_dim;   /* Dh: 64 or 128                                                   */
  int32_t ffn;        /* F: width of the SiLU-gated MLP                                  */
  int32_t vocab;      /* V                                                               */
  int32_t dtype;      /* EAGLE3_F32 or EAGLE3_BF16                                       */
  float eps;          /* RMSNorm epsilon (1e-5 for the Llama family)                     */
  float rope_theta;   /* RoPE base (500000 for the Llama-3.1 family)                     */
  const void* embed;     /* [V, d]           token embedding                             */
  const void* w_fuse;    /* [d, 3d]          W_f: g = W_f [h_low; h_mid; h_high]          */
  const void* g_embed;   /* [d]              RMSNorm gain on the token embedding          */
  const void* g_feat;    /* [d]              RMSNorm gain on the feature                  */
  const void* g_mlp;     /* [d]              RMSNorm gain before the MLP                  */
  const void* g_final;   /* [d]              RMSNorm gain before the LM head              */
  const void* w_qkv;     /* [(Hq+2Hkv)*Dh, 2d] rows: q heads, then k heads, then v heads */
  const void* w_o;       /* [d, Hq*Dh]                                                    */
  const void* w_gate_up; /* [2F, d]          rows 0..F-1 gate, F..2F-1 up                 */
  const void* w_down;    /* [d, F]                                                        */
  const void* w_lm;      /* [V, d]           LM head                                      */
} eagle3_drafter;

/* Draft-tree budget ([P1] Draft tree 配置: total draft tokens, depth, nodes selected per
 * expansion; [P2] 二、EAGLE-2动态草稿树: top-K children per expanded node).
 * depth D >= 1 evaluation steps, topk K >= 1 children per evaluated node, width W >= 1
 * nodes evaluated per depth, n_nodes N >= 1 draft nodes kept (the root is extra).
 * Limits: K <= 16, 1 + (D-1)*W <= 256, N <= 255. */
typedef struct eagle3_tree_cfg {
  int32_t depth;
  int32_t topk;
  int32_t width;
  int32_t n_nodes;
} eagle3_tree_cfg;

/* Optional per-evaluation-slot outputs of eagle3_draft_expand, for checking it.  Slot 0 is
 * the root; the j-th node evaluated at depth t >= 1 is slot 1 + (t-1)*W + j, so a request
 * has S = 1 + (D-1)*W slots.  Every pointer may be NULL (then that output is skipped). */
typedef struct eagle3_draft_debug {
  float* g;              /* [B, d]     fused feature g (fp32)                             */
  int32_t* slot_token;   /* [B, S]     token evaluated in the slot                        */
  int32_t* slot_parent;  /* [B, S]     parent slot; -1 for the root, -2 for an unused slot */
  float* slot_a;         /* [B, S, d]  drafter output a (fp32)                            */
  int32_t* slot_topk_id; /* [B, S, K]  top-K token ids (value desc, id asc)               */
  float* slot_topk_val;  /* [B, S, K]  their logits (fp32)                                */
  float* slot_lse;       /* [B, S]     ln sum_t e^{z_t} of the slot's logits              */
  float* slot_logits;    /* [B, S, V]  full logits (fp32), or NULL                        */
} eagle3_draft_debug;

/* ------------------------------------------------------------------------------------
 * eagle3_draft_expand -- one draft-tree round for B independent requests.
 * [P3] 多层特征融合到底融合了什么 and [P1] 推理流程: g = W_f [h_low; h_mid; h_high];
 * [P3] 第二步为什么没有“正确隐藏状态”可用: the root step uses (root token, g), every later
 * node uses (its token, the drafter output a of its parent); [P2] 二、EAGLE-2动态草稿树 and
 * [P1] Draft tree 配置: per-depth top-K expansion with a node budget.
 *
 * Per request: evaluate the root at position P_b; every evaluated node v creates its top-K
 * children (value desc, id asc) with score s = s_v + (z_v[t] - lse_v) in fp32; at each depth
 * t = 1..D-1 the W best depth-t candidates by (score desc, creation asc) are evaluated at
 * position P_b + t, attending to the drafter prefix KV and their evaluated ancestors; after
 * D steps the N best candidates overall are kept and relabelled by (depth asc, creation
 * asc), root = node 0.  Output is in level order with parent[i] < i.
 *
 *  h_low, h_mid, h_high : [B, d] dtype    target features of each request's root token
 *  root_tok             : [B] int32       root token ids
 *  kpre, vpre           : [sum P_b, Hkv, Dh] dtype  the drafter's own prefix KV, requests
 *                         concatenated; RoPE already applied to kpre
 *  cu_prefix            : [B+1] int32     prefix offsets (device); max_prefix >= every P_b
 *  tokens, parents, depth : [B, N+1] int32  the tree (padding -1)
 *  score                : [B, N+1] fp32   cumulative log-probability (root 0, padding -inf)
 *  n_nodes              : [B] int32       nodes written per request (root included)
 *  dbg                  : optional, see eagle3_draft_debug
 * ------------------------------------------------------------------------------------ */
EAGLE3_API size_t eagle3_draft_expand_workspace_size(const eagle3_drafter* w, const eagle3_tree_cfg* t,
                                          int B, int max_prefix);
EAGLE3_API int eagle3_draft_expand(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B,
                        const void* h_low, const void* h_mid, const void* h_high,
                        const int32_t* root_tok, const void* kpre, const void* vpre,
                        const int32_t* cu_prefix, int max_prefix, int32_t* tokens,
                        int32_t* parents, int32_t* depth, float* score, int32_t* n_nodes,
                        const eagle3_draft_debug* dbg, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ------------------------------------------------------------------------------------
 * eagle3_draft_expand_sampled -- the draft-tree round with sampled candidates.  [P1] 推理流程
 * and [P2] 三、EAGLE-3 (the draft head outputs a distribution over the vocabulary and the next
 * token is drawn from it); [P2] 四 DFlash (drafted tokens are later kept with probability
 * min(1, p_target / p_draft), which needs the drafter's distribution at every node).
 *
 * As eagle3_draft_expand, except that every evaluated node's children are K draws without
 * replacement from softmax(z / T) (the K best of z * invT + G, invT = 1/T in fp32, G Gumbel
 * noise from Philox4x32-10 with counter (t>>2, 0x80000000 | slot, b, round mod 2^32), key
 * (seed lo, seed hi), word t & 3; u and G as in eagle3_accept), listed in draw order; the
 * log-sum-exp is that of z * invT; a child's score is s_v + (z[t] * invT - lse), lowered to
 * the score of any sibling drawn before it (so the siblings a budget keeps are always the
 * first ones drawn, as eagle3_accept_sampled requires).
 *
 *  slot_logits : [B * S, V] fp32 (16-byte aligned)  every evaluated slot's logits (raw z)
 *  draft_row   : [B, N+1] int32  row of slot_logits holding node i's logits (the drafter's
 *                distribution at that node), -1 for a node that was not evaluated (it has no
 *                children); pass it, flattened like the tree, to eagle3_accept_sampled
 *  temperature > 0; other arguments, limits and the workspace as for eagle3_draft_expand.
 * ------------------------------------------------------------------------------------ */
EAGLE3_API int eagle3_draft_expand_sampled(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B,
                                           float temperature, uint64_t seed, uint64_t round,
                                           const void* h_low, const void* h_mid, const void* h_high,
                                           const int32_t* root_tok, const void* kpre, const void* vpre,
                                           const int32_t* cu_prefix, int max_prefix, int32_t* tokens,
                                           int32_t* parents, int32_t* depth, float* score,
                                           int32_t* n_nodes, float* slot_logits, int32_t* draft_row,
                                           const eagle3_draft_debug* dbg, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * eagle3_build_tree_mask -- pack flattened trees: ancestor bitmask, depth and position.
 * [P2] 二、EAGLE-2动态草稿树 (flatten the tree, add positions, build the 0/1 tree attention
 * mask so a node sees only itself and its ancestors); [P5] 一棵候选树怎样被验证 (assign each
 * node a position; mask so nodes see only their ancestors).
 *
 *  cu_nodes : [B+1] int32  node offsets per request (device); T = cu_nodes[B] (host copy)
 *  parents  : [T] int32    request-local parent index; root (node 0 of a request) = -1;
 *                          parent[i] < i is required (topological order)
 *  cu_prefix: [B+1] int32  prefix offsets; pos = P_b + depth
 *  mask     : [T, W64] uint64  bit j of word j/64 set iff node j is i or an ancestor of i
 *  depth    : [T] int32 (may be NULL)   pos : [T] int32 (may be NULL)
 *  dev_status: optional device int32; EAGLE3_DEV_BAD_PARENT / _TOO_DEEP are OR-ed in
 *  max_nodes: host upper bound on nodes per request, <= 64*W64
 * ------------------------------------------------------------------------------------ */
EAGLE3_API int eagle3_build_tree_mask(int B, int T, const int32_t* cu_nodes, const int32_t* parents,
                           const int32_t* cu_prefix, int max_nodes, uint64_t* mask, int W64,
                           int32_t* depth, int32_t* pos, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------------------
 * eagle3_tree_attention -- tree-masked attention of every tree node over the prefix KV
 * plus the tree KV.  [P3] 从序列到动态草稿树 (tree attention: each node attends only to its
 * ancestor path); [P5] 一棵候选树怎样被验证 steps 2-3; [P4] USP 核心设计 (attention results
 * carried as (Out, LSE) pairs).
 *
 * For node i of request b and query head h (KV head c = h / (Hq/Hkv)): softmax over the
 * prefix keys 0..P_b-1 (all visible) and the tree keys j with mask bit j set, scores
 * scale * q.k.  The prefix is cut into S splits, the tree keys form one more partial:
 *  o_part [S+1, T, Hq, Dh] fp32 and lse_part [S+1, T, Hq] fp32 receive the partials
 *  (with C_b = ceil(P_b/S) rounded up to a multiple of 128, partial s < S covers prefix
 *  keys [s*C_b, (s+1)*C_b) clipped to P_b; partial S covers the tree keys); an empty
 *  partial has O = 0, LSE = -inf.  If `o` is not NULL the partials
 *  are also merged (as eagle3_lse_merge) into o [T, Hq, Dh] (dtype) and lse [T, Hq] fp32;
 *  then o_part/lse_part may be NULL and the workspace holds them.
 *
 *  q [T, Hq, Dh], k_tree, v_tree [T, Hkv, Dh], kpre, vpre [sum P_b, Hkv, Dh]: dtype
 *  cu_nodes [B+1], cu_prefix [B+1]: int32 device; mask [T, W64] as built above
 *  max_nodes, max_prefix: host upper bounds per request; n_splits: S in 1..256 (0 =
 *  automatic: enough workgroups for the kernel shape chosen by the query rows per KV head,
 *  each split at least one key tile and three times as many keys as its row block has
 *  query rows; the same arguments give the same S in eagle3_tree_attention_num_splits).
 *  Dh must be 64 or 128.
 * ------------------------------------------------------------------------------------ */
EAGLE3_API int eagle3_tree_attention_num_splits(int B, int Hq, int Hkv, int max_nodes,
                                                int max_prefix, int n_splits);
EAGLE3_API size_t eagle3_tree_attention_workspace_size(int B, int T, int Hq, int Hkv, int Dh,
                                                      int max_nodes, int max_prefix, int n_splits);
EAGLE3_API int eagle3_tree_attention(int B, int T, int Hq, int Hkv, int Dh, int dtype, const void* q,
                          const void* k_tree, const void* v_tree, const int32_t* cu_nodes,
                          int max_nodes, const uint64_t* mask, int W64, const void* kpre,
                          const void* vpre, const int32_t* cu_prefix, int max_prefix,
                          float scale, int n_splits, float* o_part, float* lse_part, void* o,
                          float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * eagle3_lse_merge -- merge S attention partials by log-sum-exp.  [P4] USP 核心设计：三步走,
 * Step 3: fold Out_branch/LSE_branch into Out_main/LSE_main by streaming softmax with one
 * consistent normalisation.
 *
 * Per row r: m = max_s LSE_s; w_s = e^{LSE_s - m}; O = sum_s w_s O_s / sum_s w_s;
 * LSE = m + ln sum_s w_s.  Partials with LSE = -inf weigh 0; a row whose partials are all
 * -inf gives O = 0 and LSE = -inf.
 *  o_part [S, rows, Dh] fp32, lse_part [S, rows] fp32 -> o [rows, Dh] (out_dtype),
 *  lse [rows] fp32 (may be NULL).  1 <= S <= 512; Dh % 4 == 0 and Dh <= 128 (else
 *  EAGLE3_EUNSUPPORTED).
 * ------------------------------------------------------------------------------------ */
EAGLE3_API int eagle3_lse_merge(int S, int rows, int Dh, const float* o_part, const float* lse_part,
                     int out_dtype, void* o, float* lse, void* stream);

/* ------------------------------------------------------------------------------------
 * The training form of the long-context shape: [P4] USP 核心设计：三步走.  Every position of
 * a sequence is a query.
 * eagle3_causal_attention -- Step 1 (main): position t, query head h attends to keys
 *   0 .. t of its KV head h / (Hq/Hkv): Out_main and LSE_main.  bf16, head_dim 64 or 128.
 * eagle3_branch_attention -- Step 2 (branch): position t, query head h attends to its own
 *   TTT branch keys kb[j][t], j < n_steps (the unrolled draft steps' keys at position t),
 *   as per-position dot products: Out_branch and LSE_branch.  bf16 or fp32, head_dim 128,
 *   1 <= n_steps <= 8.
 * Step 3 (fusion) is eagle3_lse_merge with S = 2 over rows = L * Hq: place Out_main and
 * Out_branch as partials 0 and 1 of one [2, L*Hq, Dh] buffer (and the LSEs likewise).
 *
 *  q [L, Hq, Dh]; k, v [L, Hkv, Dh]; kb, vb [n_steps, L, Hkv, Dh] (dtype); scale > 0
 *  o [L, Hq, Dh] fp32 (normalised), lse [L, Hq] fp32 natural log.
 * ------------------------------------------------------------------------------------ */
EAGLE3_API int eagle3_causal_attention(int L, int Hq, int Hkv, int Dh, int dtype, const void* q,
                                       const void* k, const void* v, float scale, float* o,
                                       float* lse, void* stream);
EAGLE3_API int eagle3_branch_attention(int L, int n_steps, int Hq, int Hkv, int Dh, int dtype,
                                       const void* q, const void* kb, const void* vb, float scale,
                                       float* o, float* lse, void* stream);

/* ------------------------------------------------------------------------------------
 * eagle3_accept -- accept the longest draft path.  [P1] 论文位置 (accept the longest
 * correct prefix; the standard speculative-sampling rule keeps the target distribution);
 * [P2] 二、EAGLE-2动态草稿树 (accept the longest coherent path, roll back to its last node);
 * [P3] 先看 checkpoint 最终要参与什么计算 (accept the continuous prefix, correct at the
 * rejection); [P5] 一棵候选树怎样被验证 step 4.
 *
 * At every node i the target draw is y_i = argmax_t z_i[t] (temperature == 0) or
 * y_i = argmax_t (z_i[t] * invT + G_t), invT = 1/temperature in fp32, G_t Gumbel noise from
 * Philox4x32-10 with counter (t>>2, i, b, round mod 2^32), key (seed lo, seed hi), word
 * t & 3, u = ((x>>9)+0.5)*2^-23, G = -ln(-ln u) with a fixed float32 ln; ties go to the
 * lowest token id.  The accepted end node is the deepest node whose every non-root
 * ancestor-or-self j has tokens[j] == y_parent(j) (ties: lowest node index).
 *
 *  cu_nodes [B+1], tokens [T], parents [T] (request-local), mask [T, W64] (from
 *  eagle3_build_tree_mask), logits [T, V] dtype (target logits at every node).
 *  accept_len [B]; path [B, max_depth+1] accepted node indices, root first;
 *  out_tokens [B, max_depth+1] accepted draft tokens then the bonus token; bonus [B];
 *  padding -1.  max_depth >= the deepest node of any request.
 * ------------------------------------------------------------------------------------ */
EAGLE3_API size_t eagle3_accept_workspace_size(int T, int V);
EAGLE3_API int eagle3_accept(int B, int T, const int32_t* cu_nodes, const int32_t* tokens,
                  const int32_t* parents, const uint64_t* mask, int W64, const void* logits,
                  int V, int dtype, float temperature, uint64_t seed, uint64_t round,
                  int max_depth, int32_t* accept_len, int32_t* path, int32_t* out_tokens,
                  int32_t* bonus, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * eagle3_accept_noalloc -- eagle3_accept for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, rule and outputs as eagle3_accept, without the workspace: its scratch
 * (the per-(node, 4096-token chunk) winner list, 8 bytes per entry) is a fixed 1 MiB array
 * inside the library, one per GPU, held until the process ends.  Calls whose
 * T * ceil(V / 4096) exceeds eagle3_accept_noalloc_max_entries() (131008; e.g. T <= 4094 at
 * V = 128256) return EAGLE3_EUNSUPPORTED before anything is enqueued.  Every call on a GPU
 * shares that GPU's array, so calls that overlap on one GPU (other streams or host threads)
 * race; serialise them.  Nothing is allocated or freed.
 * ------------------------------------------------------------------------------------ */
EAGLE3_API size_t eagle3_accept_noalloc_max_entries(void);
EAGLE3_API int eagle3_accept_noalloc(int B, int T, const int32_t* cu_nodes, const int32_t* tokens,
                                     const int32_t* parents, const uint64_t* mask, int W64,
                                     const void* logits, int V, int dtype, float temperature,
                                     uint64_t seed, uint64_t round, int max_depth, int32_t* accept_len,
                                     int32_t* path, int32_t* out_tokens, int32_t* bonus, void* stream);

/* ------------------------------------------------------------------------------------
 * eagle3_accept_sampled -- acceptance of sampled candidates.  [P2] 四 DFlash (each drafted
 * token is kept with probability min(1, p_target / p_draft), dice thrown left to right, the
 * first rejection ends the kept prefix); [P3] 先看 checkpoint 最终要参与什么计算 (keep the
 * continuous prefix, correct at the rejection; the output then follows the target alone).
 * For a tree (the children of a node drawn without replacement from the drafter's
 * distribution at that node, in node-index order) the children are tested in that order:
 * child x is kept when u < p(x) / q(x); otherwise p becomes max(p - q, 0) normalised, x
 * leaves q and q is renormalised.  A kept child is the next node; when all are rejected (or
 * the node has none) the bonus token is a Gumbel-max draw from p as it then stands.
 *
 * At node i, p = softmax(logits_i / T) and q = softmax(draft_logits[draft_row[i]] / T), in
 * float64.  The uniform of child node j of request b is Philox4x32-10 with counter
 * (0x40000000, j, b, round mod 2^32), key (seed lo, seed hi), word 0, u = ((x>>9)+0.5)*2^-23;
 * the draw at node i uses the Gumbel noise of eagle3_accept at node i (token t: counter
 * (t>>2, i, b, round), word t & 3) and takes argmax_t ln p_t + G_t.  Children whose token is
 * outside [0, V) or repeats an earlier sibling's are skipped; only the first max_children
 * children of a node are tested (1 <= max_children <= 64, else EAGLE3_EUNSUPPORTED).
 *
 *  cu_nodes [B+1], tokens [T], parents [T] (request-local, parent < node; at most 256 nodes per
 *  request), logits [T, V] dtype (target logits at every node), draft_logits [n_draft_rows, V]
 *  draft_dtype (the drafter's logits; NULL when n_draft_rows == 0), draft_row [T] int32 (row of
 *  draft_logits at node i; outside [0, n_draft_rows) for a node without children).
 *  temperature > 0.  Outputs as for eagle3_accept (max_depth >= the deepest node).
 *  dev_status: EAGLE3_DEV_BAD_ROW (a node with children has no draft row: it draws from p),
 *  EAGLE3_DEV_BAD_TOKEN (a child token outside the vocabulary), EAGLE3_DEV_BAD_PATH (a request
 *  with more than 256 nodes: the later nodes are ignored), EAGLE3_DEV_SYNC (a partial result
 *  handed between workgroups was not visible within a bounded wait: the outputs of that call
 *  are not to be trusted).
 *  workspace: eagle3_accept_sampled_workspace_size(T, V, max_children) bytes.
 * ------------------------------------------------------------------------------------ */
EAGLE3_API size_t eagle3_accept_sampled_workspace_size(int T, int V, int max_children);
EAGLE3_API int eagle3_accept_sampled(int B, int T, const int32_t* cu_nodes, const int32_t* tokens,
                                     const int32_t* parents, const void* logits, int V, int dtype,
                                     const void* draft_logits, int draft_dtype, int n_draft_rows,
                                     const int32_t* draft_row, int max_children, float temperature,
                                     uint64_t seed, uint64_t round, int max_depth,
                                     int32_t* accept_len, int32_t* path, int32_t* out_tokens,
                                     int32_t* bonus, int32_t* dev_status, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * eagle3_commit_kv -- commit the accepted path's KV.  [P5] 一棵候选树怎样被验证, step 5
 * (commit only the KV on the accepted path, release the other branches); [P2]
 * 二、EAGLE-2动态草稿树 (fall back to the last accepted node, where the next round starts).
 * For request b the path nodes path[b * path_stride + i], i = 0 .. accept_len[b] (root
 * first, as eagle3_accept returns them), are tree rows cu_nodes[b] + node; their K and V
 * rows are copied to cache rows dst_row[b] + i.  No other cache row is written: the rows of
 * rejected branches are released by not being copied.
 *
 *  Hkv, Dh >= 1 with Hkv * Dh * element size a multiple of 16 bytes; path_stride >= 1
 *  cu_nodes [B+1], path [B, path_stride], accept_len [B], dst_row [B]: int32 (device)
 *  k_tree, v_tree [T, Hkv, Dh] dtype; k_cache, v_cache [cache_rows, Hkv, Dh] dtype, written
 *  in place (they must not overlap the tree rows).  Both caches must hold cache_rows rows
 *  of the tree's (Hkv, Dh): the kernel trusts cache_rows for its bounds, so a shorter cache
 *  is an out-of-bounds write (the Python binding refuses mismatched shapes).
 *  dev_status: EAGLE3_DEV_BAD_PATH (accept_len outside [0, path_stride) or a node outside
 *  its request: those rows are skipped), EAGLE3_DEV_BAD_ROW (destination outside
 *  [0, cache_rows): skipped).
 * ------------------------------------------------------------------------------------ */
EAGLE3_API int eagle3_commit_kv(int B, int Hkv, int Dh, int dtype, int path_stride,
                                const int32_t* cu_nodes, const int32_t* path,
                                const int32_t* accept_len, const void* k_tree, const void* v_tree,
                                const int32_t* dst_row, int64_t cache_rows, void* k_cache,
                                void* v_cache, int32_t* dev_status, void* stream);

/* ------------------------------------------------------------------------------------
 * eagle3_drafter_catchup -- the drafter's prefix KV of committed positions, from the
 * target's real features.  [P3] 第二步为什么没有“正确隐藏状态”可用 (a draft step reads the
 * real fused target feature only where the target has already run; drafted steps
 * substitute the drafter's own output), [P3] 多层特征融合到底融合了什么 (g = W_f [h_low;
 * h_mid; h_high]).  Row r (one committed position) is formed as the draft round's root:
 * g_r = W_f [h_low_r; h_mid_r; h_high_r], u_r = [rms(E[tokens_r]) g_e ; rms(g_r) g_f], and
 * its key (RoPE at pos_r) and value (the K and V rows of w_qkv) go to cache row dst_row[r].
 * g_r is returned in fp32: the last committed position's g is the next round's root
 * feature.  Rows may belong to different requests; n = P rows catch the drafter up over a
 * whole prompt (the fusion and K/V projections then run on the matrix-core tiles).
 *
 *  w: the drafter, as for eagle3_draft_expand; n >= 1
 *  tokens, pos, dst_row [n] int32 (device); h_low, h_mid, h_high [n, d] dtype
 *  k_cache, v_cache [cache_rows, Hkv, Dh] dtype (the drafter prefix KV), written in place;
 *  both must hold cache_rows rows of the drafter's (Hkv, Dh) (the kernel trusts cache_rows
 *  for its bounds; the Python binding refuses mismatched shapes)
 *  g_out [n, d] fp32, may be NULL
 *  dev_status: EAGLE3_DEV_BAD_TOKEN (token clamped into the vocabulary),
 *  EAGLE3_DEV_BAD_ROW (destination outside [0, cache_rows): row skipped)
 *  workspace: eagle3_drafter_catchup_workspace_size(w, n) bytes.
 *  bf16: any n (n > 160 needs d % 64 == 0); fp32: n <= 160; else EAGLE3_EUNSUPPORTED.
 * ------------------------------------------------------------------------------------ */
EAGLE3_API size_t eagle3_drafter_catchup_workspace_size(const eagle3_drafter* w, int n);
EAGLE3_API int eagle3_drafter_catchup(const eagle3_drafter* w, int n, const int32_t* tokens,
                                      const int32_t* pos, const void* h_low, const void* h_mid,
                                      const void* h_high, const int32_t* dst_row, int64_t cache_rows,
                                      void* k_cache, void* v_cache, float* g_out,
                                      int32_t* dev_status, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* ------------------------------------------------------------------------------------
 * eagle3_linear -- Y = X W^T through the GEMM kernels of the drafter's projections.
 * Every step of the drafter multiplies rows by a weight matrix stored [out_features,
 * in_features]: the fusion W_f ([P3] 多层特征融合到底融合了什么), the decoder layer's QKV, O and
 * MLP projections ([P1] 训练细节: a single decoder layer) and the LM head.  The kernel is
 * chosen by M: a few rows (M <= 32, bf16) stream W through LDS; up to 160 rows hold X in
 * registers; more rows (M > 160, bf16, K % 64 == 0) use 256 x 256 matrix-core tiles, with the
 * k-range split over workgroups when there are fewer tiles than compute units.
 *
 *  X [M, K] dtype, row stride ldx >= K elements; W [N, K] dtype; Y [M, N] fp32 (written
 *  whole).  N % 4 == 0, K % 8 == 0; M in 1..160 for any dtype, or M > 160 for bf16 with
 *  K % 64 == 0, N * K * 2 and M * ldx * 2 below 4 GiB (else EAGLE3_EUNSUPPORTED).  Pointers
 *  16-byte aligned (ldx * element size a multiple of 16).  workspace:
 *  eagle3_linear_workspace_size() bytes (split-K partial sums; 0 when none are needed, then
 *  workspace may be NULL).  Split-K sums are added in split order, so results are
 *  deterministic for a given shape.
 * ------------------------------------------------------------------------------------ */
EAGLE3_API size_t eagle3_linear_workspace_size(int M, int N, int K, int dtype);
EAGLE3_API int eagle3_linear(int M, int N, int K, int dtype, const void* X, int ldx, const void* W,
                             float* Y, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------
 * Speculative-budget controller (host code; no device memory, no stream).  [P5] 执行控制器:
 * adjust the draft-tree budget from what the rounds show -- committed tokens, drafter and
 * verify latency -- without touching the target's decoding: lower the budget when recent
 * accepted length is low or drafting is expensive, raise it cautiously when acceptance is
 * stable and verification has room, always bounded, cooled down and falling back rather
 * than oscillating.  The page gives the policy in words only; the thresholds are parameters.
 *
 * Per round the caller reports accept_len (committed tokens = accept_len + 1) and the
 * measured draft and verify times; the controller keeps the last `window` rounds at the
 * current level (cleared on every change) and, once the window is full and `cooldown` rounds
 * have passed since the last change, with c the committed tokens per round and D the
 * level's depth, frac = mean(c) / (D + 1), cv = std(c) / mean(c), goodput = mean(c) /
 * mean(draft + verify):
 *   1. the first full window after a raise whose goodput fell below (1 - revert_drop) of the
 *      goodput before the raise steps back down and blocks raises for 4 * cooldown rounds;
 *   2. frac < low_frac or mean(draft) / mean(draft + verify) > draft_share_max: one level down;
 *   3. frac >= high_frac, cv <= max_cv, mean(verify) < verify_ms_max, raises not blocked:
 *      one level up.
 * Statistics in double precision, sums in round order (decisions are reproducible).
 *  levels: tree budgets in increasing size (1 .. EAGLE3_BUDGET_MAX_LEVELS); start_level the
 *  baseline; cooldown >= 1; window 1 .. EAGLE3_BUDGET_MAX_WINDOW.
 * eagle3_budget_update returns the level to use for the next round (its tree in *next when
 * next != NULL) or a negative status.  The state is caller-owned; one per request stream.
 * ------------------------------------------------------------------------------------ */
#define EAGLE3_BUDGET_MAX_LEVELS 16
#define EAGLE3_BUDGET_MAX_WINDOW 256
typedef struct eagle3_budget_params {
  int32_t n_levels;
  eagle3_tree_cfg levels[EAGLE3_BUDGET_MAX_LEVELS];
  int32_t start_level;
  int32_t cooldown;
  int32_t window;
  float low_frac;
  float high_frac;
  float max_cv;
  float draft_share_max;
  float verify_ms_max;
  float revert_drop;
} eagle3_budget_params;

typedef struct eagle3_budget_state {
  int32_t level;       /* current level                                           */
  int32_t since;       /* rounds since the last change                            */
  int32_t block;       /* rounds during which raises stay blocked                 */
  int32_t check;       /* the last change was a raise: compare goodput next       */
  int32_t count;       /* rounds in the window                                    */
  int32_t head;        /* ring position of the oldest round                       */
  double g_before;     /* goodput measured before the last raise                  */
  double committed[EAGLE3_BUDGET_MAX_WINDOW];
  double draft_ms[EAGLE3_BUDGET_MAX_WINDOW];
  double verify_ms[EAGLE3_BUDGET_MAX_WINDOW];
} eagle3_budget_state;

EAGLE3_API int eagle3_budget_init(const eagle3_budget_params* p, eagle3_budget_state* s);
EAGLE3_API int eagle3_budget_update(const eagle3_budget_params* p, eagle3_budget_state* s,
                                    int32_t accept_len, float draft_ms, float verify_ms,
                                    eagle3_tree_cfg* next);

/* ------------------------------------------------------------------------------------
 * Launch timing.  While enabled, the library records a HIP event pair on the launch stream
 * around every kernel it enqueues whose name equals `only_kernel` (every kernel when
 * `only_kernel` is NULL).  eagle3_profile_read waits for the recorded events and reports
 * the summed device time and launch count of one kernel name (e.g. "gemm_lm_head").
 * eagle3_profile_reset drops all records.  Host-side bookkeeping only; not thread-safe
 * against concurrent launches from other threads beyond a global lock.
 * ------------------------------------------------------------------------------------ */
EAGLE3_API int eagle3_profile_enable(int on, const char* only_kernel);
EAGLE3_API int eagle3_profile_reset(void);
EAGLE3_API int eagle3_profile_read(const char* kernel, double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif
#endif /* EAGLE3_H */
