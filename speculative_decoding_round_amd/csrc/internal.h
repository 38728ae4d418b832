// Host-side launchers shared between the translation units of libeagle3.
#pragma once

#include "common.h"

namespace e3h {

// ---- attention -------------------------------------------------------------------------
// Query rows and tree keys of request b are either given by offset arrays (cu_* != null)
// or by a fixed per-request stride and count.
struct AttnArgs {
  int B, Hq, Hkv, Dh, dtype;
  const void* q;
  const int32_t* q_cu;
  int q_stride, q_rows_total;  // q_stride: rows per request when q_cu == null
  const void* kt;
  const void* vt;
  const int32_t* kt_cu;
  int kt_stride, kt_count;     // used when kt_cu == null
  const uint64_t* mask;        // [q_rows_total, W64], bits over the request's tree keys
  int W64;
  const void* kp;
  const void* vp;
  const int32_t* p_cu;         // [B+1] prefix offsets (may be null: no prefix)
  float scale;
  int S;                       // prefix splits; partial S is the tree
  int max_q_per_req;           // host bound on query rows (nodes) per request
  float* o_part;               // [S+1, q_rows_total, Hq, Dh]
  float* lse_part;             // [S+1, q_rows_total, Hq]
};
int launch_tree_attention(const AttnArgs& a, hipStream_t s, const char* tag);
int launch_lse_merge(int S, int rows, int Dh, const float* o_part, const float* lse_part,
                     int out_dtype, void* o, float* lse, hipStream_t s, const char* tag);
int attention_splits(int B, int Hkv, int rows_per_kv, int max_prefix, int n_splits);
int launch_causal_attention(int L, int Hq, int Hkv, int Dh, const void* q, const void* k, const void* v,
                            float scale, float* o, float* lse, hipStream_t s);
int launch_branch_attention(int L, int n_steps, int Hq, int Hkv, int Dh, int dtype, const void* q,
                            const void* kb, const void* vb, float scale, float* o, float* lse, hipStream_t s);

// ---- verify ----------------------------------------------------------------------------
int launch_build_mask(int B, int T, const int32_t* cu_nodes, const int32_t* parents,
                      const int32_t* cu_prefix, uint64_t* mask, int W64, int32_t* depth,
                      int32_t* pos, int32_t* dev_status, hipStream_t s);
int launch_accept(int B, int T, const int32_t* cu_nodes, const int32_t* tokens,
                  const int32_t* parents, const uint64_t* mask, int W64, const void* logits,
                  int V, int dtype, float temperature, uint64_t seed, uint64_t round,
                  int max_depth, int32_t* accept_len, int32_t* path, int32_t* out_tokens,
                  int32_t* bonus, float* part_v, int* part_i, hipStream_t s);
size_t accept_workspace(int T, int V);
size_t accept_sampled_workspace(int T, int V, int max_children);
int accept_sampled_max_children();
int launch_accept_sampled(int B, int T, const int32_t* cu_nodes, const int32_t* tokens,
                          const int32_t* parents, const void* logits, int V, int dtype,
                          const void* draft_logits, int draft_dtype, int n_draft_rows,
                          const int32_t* draft_row, int max_children, float temperature,
                          uint64_t seed, uint64_t round, int max_depth, int32_t* accept_len,
                          int32_t* path, int32_t* out_tokens, int32_t* bonus, int32_t* dev_status,
                          void* workspace, hipStream_t s);
int accept_chunks(int V);

// ---- GEMM ------------------------------------------------------------------------------
// Y_part[split][m][n] = sum over the split's k of X[m][k] * W[n][k]  (fp32 partials), or
// with silu: W = [gate; up] ([2F, K]) and act[m][j] = silu(gate) * up written in dtype.
struct GemmPlan {
  int M, N, K, MT, NT, n_blocks, splits, chunks_total, chunks_per_split, waves;
  bool silu;
  bool ring;   // bf16 LDS-ring kernel (one wave per workgroup)
  bool tile;   // bf16 tiled MFMA kernel for many rows (M > 160)
  bool wide;   // bf16 wide kernel (33 .. 160 rows: four waves split the rows, shared W ring)
};
// whole_k: no k-split, as the LM head's block statistics need (see launch_gemm).
GemmPlan plan_gemm(int M, int N, int K, int dtype, bool silu = false, bool whole_k = false);
// Whether a plan's kernel can emit the LM head's block statistics: the bf16 ring kernel, or
// the wide kernel at 16 or 32 tiles per block, without a k-split.
inline bool gemm_block_stats_ok(const GemmPlan& p) {
  return !p.silu && p.splits == 1 && (p.ring || (p.wide && (p.NT == 16 || p.NT == 32)));
}
// Row stride of the statistics planes: blocks of 128 columns, so N <= 131072.
constexpr int kLmStatsLd = 1024;
// stats (LM head only, tag "gemm_lm_head" or "gemm_lm_head_root", a plan with
// gemm_block_stats_ok): besides the logits, per row and block of 128 columns the best logit
// (value desc, column asc), its column and the sum of e^(z - best) over the block, in three
// planes of M x kLmStatsLd (fp32, int32, fp32; entry n / 128 for the block of column n).
int launch_gemm(const GemmPlan& p, int dtype, const void* X, int ldx, const void* W, float* Ypart,
                hipStream_t s, const char* tag, void* act = nullptr, float* stats = nullptr);

// out[m][n] = (resid ? resid[m][n] : 0) + sum_s part[s][m][n]  (split order)
int launch_epi_sum(const GemmPlan& p, const float* part, float* out, const float* resid,
                   hipStream_t s, const char* tag);

// ---- commit and drafter catch-up ------------------------------------------------------
int drafter_check(const eagle3_drafter* w);
int launch_commit_kv(int B, int row_elems, int dtype, int path_stride, const int32_t* cu_nodes,
                     const int32_t* path, const int32_t* accept_len, const void* k_tree,
                     const void* v_tree, const int32_t* dst_row, long cache_rows, void* k_cache,
                     void* v_cache, int32_t* dev_status, hipStream_t s);
size_t catchup_workspace(const eagle3_drafter* w, int n);
int catchup_supported(const eagle3_drafter* w, int n);
int launch_catchup(const eagle3_drafter* w, int n, const int32_t* tokens, const int32_t* pos,
                   const void* h_low, const void* h_mid, const void* h_high, const int32_t* dst_row,
                   long cache_rows, void* k_cache, void* v_cache, float* g_out, int32_t* dev_status,
                   void* ws, hipStream_t s);

}  // namespace e3h
