// C-ABI entry points of libeagle3: argument validation on the host, workspace sizing, and
// the launch-timing registry.  Every compute step runs in the kernels of the other units.
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "internal.h"

namespace e3h {
int draft_check(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B, int max_prefix);
size_t draft_workspace(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B, int max_prefix);
int draft_expand(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B, const void* h_low,
                 const void* h_mid, const void* h_high, const int32_t* root_tok, const void* kpre,
                 const void* vpre, const int32_t* cu_prefix, int max_prefix, int32_t* tokens,
                 int32_t* parents, int32_t* depth, float* score, int32_t* n_nodes,
                 const eagle3_draft_debug* dbg, void* ws, size_t ws_bytes, hipStream_t s);
int draft_expand_sampled(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B, float temperature,
                         uint64_t seed, uint64_t round, const void* h_low, const void* h_mid,
                         const void* h_high, const int32_t* root_tok, const void* kpre, const void* vpre,
                         const int32_t* cu_prefix, int max_prefix, int32_t* tokens, int32_t* parents,
                         int32_t* depth, float* score, int32_t* n_nodes, float* slot_logits,
                         int32_t* draft_row, const eagle3_draft_debug* dbg, void* ws, size_t ws_bytes,
                         hipStream_t s);

// ---------------------------------------------------------------------------------------
// Launch timing registry
// ---------------------------------------------------------------------------------------
namespace {
struct Rec {
  std::string name;
  hipEvent_t e0, e1;
};
std::mutex g_mu;
bool g_on = false;
std::string g_only;             // empty: every kernel
std::vector<Rec> g_recs;        // recorded pairs (events owned here)
std::vector<hipEvent_t> g_pool; // spare events
int g_open = -1;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : slot(-1), stream(s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || g_open >= 0) return;  // nested scopes are timed by the outermost one
  if (!g_only.empty() && g_only != name) return;
  Rec r;
  r.name = name;
  r.e0 = take_event();
  r.e1 = take_event();
  if (!r.e0 || !r.e1) return;
  if (hipEventRecord(r.e0, s) != hipSuccess) return;
  g_recs.push_back(r);
  slot = (int)g_recs.size() - 1;
  g_open = slot;
}

ProfScope::~ProfScope() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  (void)hipEventRecord(g_recs[slot].e1, stream);
  g_open = -1;
}

}  // namespace e3h

using namespace e3h;

extern "C" {

int eagle3_abi_version(void) { return EAGLE3_ABI_VERSION; }

const char* eagle3_status_string(int status) {
  switch (status) {
    case EAGLE3_OK: return "ok";
    case EAGLE3_EINVAL: return "invalid argument (null pointer, dtype, shape or size)";
    case EAGLE3_EUNSUPPORTED: return "unsupported shape or parameter";
    case EAGLE3_EWORKSPACE: return "workspace missing or too small";
    case EAGLE3_EHIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

// ---- draft ----------------------------------------------------------------------------
size_t eagle3_draft_expand_workspace_size(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B,
                                          int max_prefix) {
  return draft_workspace(w, t, B, max_prefix);
}

int eagle3_draft_expand(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B, const void* h_low,
                        const void* h_mid, const void* h_high, const int32_t* root_tok,
                        const void* kpre, const void* vpre, const int32_t* cu_prefix, int max_prefix,
                        int32_t* tokens, int32_t* parents, int32_t* depth, float* score,
                        int32_t* n_nodes, const eagle3_draft_debug* dbg, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return draft_expand(w, t, B, h_low, h_mid, h_high, root_tok, kpre, vpre, cu_prefix, max_prefix,
                      tokens, parents, depth, score, n_nodes, dbg, workspace, workspace_bytes,
                      (hipStream_t)stream);
}

int eagle3_draft_expand_sampled(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B,
                                float temperature, uint64_t seed, uint64_t round, const void* h_low,
                                const void* h_mid, const void* h_high, const int32_t* root_tok,
                                const void* kpre, const void* vpre, const int32_t* cu_prefix,
                                int max_prefix, int32_t* tokens, int32_t* parents, int32_t* depth,
                                float* score, int32_t* n_nodes, float* slot_logits, int32_t* draft_row,
                                const eagle3_draft_debug* dbg, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return draft_expand_sampled(w, t, B, temperature, seed, round, h_low, h_mid, h_high, root_tok, kpre,
                              vpre, cu_prefix, max_prefix, tokens, parents, depth, score, n_nodes,
                              slot_logits, draft_row, dbg, workspace, workspace_bytes, (hipStream_t)stream);
}

// ---- tree mask ------------------------------------------------------------------------
int eagle3_build_tree_mask(int B, int T, const int32_t* cu_nodes, const int32_t* parents,
                           const int32_t* cu_prefix, int max_nodes, uint64_t* mask, int W64,
                           int32_t* depth, int32_t* pos, int32_t* dev_status, void* stream) {
  if (B <= 0 || T < 0 || W64 < 1 || max_nodes < 0) return EAGLE3_EINVAL;
  if (!cu_nodes || (T > 0 && (!parents || !mask))) return EAGLE3_EINVAL;
  if (max_nodes > 64 * W64) return EAGLE3_EINVAL;
  if (W64 > 4) return EAGLE3_EUNSUPPORTED;
  if (T == 0) return EAGLE3_OK;
  return launch_build_mask(B, T, cu_nodes, parents, cu_prefix, mask, W64, depth, pos, dev_status,
                           (hipStream_t)stream);
}

// ---- attention ------------------------------------------------------------------------
int eagle3_tree_attention_num_splits(int B, int Hq, int Hkv, int max_nodes, int max_prefix,
                                     int n_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || max_nodes < 0 || max_prefix < 0 || n_splits < 0)
    return EAGLE3_EINVAL;
  if (n_splits > 256) return EAGLE3_EUNSUPPORTED;
  return attention_splits(B, Hkv, max_nodes * (Hq / Hkv), max_prefix, n_splits);
}

size_t eagle3_tree_attention_workspace_size(int B, int T, int Hq, int Hkv, int Dh, int max_nodes,
                                            int max_prefix, int n_splits) {
  const int S = eagle3_tree_attention_num_splits(B, Hq, Hkv, max_nodes, max_prefix, n_splits);
  if (S < 1 || T < 0 || Dh <= 0) return 0;
  Carve c(nullptr);
  c.take<float>((size_t)(S + 1) * T * Hq * Dh);
  c.take<float>((size_t)(S + 1) * T * Hq);
  return c.size();
}

int eagle3_tree_attention(int B, int T, int Hq, int Hkv, int Dh, int dtype, const void* q,
                          const void* k_tree, const void* v_tree, const int32_t* cu_nodes,
                          int max_nodes, const uint64_t* mask, int W64, const void* kpre,
                          const void* vpre, const int32_t* cu_prefix, int max_prefix, float scale,
                          int n_splits, float* o_part, float* lse_part, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (B <= 0 || T < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || max_nodes < 0 || max_prefix < 0 ||
      n_splits < 0 || W64 < 1)
    return EAGLE3_EINVAL;
  if (!dtype_ok(dtype)) return EAGLE3_EINVAL;
  if (Dh != 64 && Dh != 128) return EAGLE3_EUNSUPPORTED;
  if (W64 > 4 || max_nodes > 64 * W64 || n_splits > 256) return EAGLE3_EUNSUPPORTED;
  if (!(scale > 0.f)) return EAGLE3_EINVAL;
  if (T == 0) return EAGLE3_OK;
  if (!q || !k_tree || !v_tree || !cu_nodes || !mask) return EAGLE3_EINVAL;
  if (max_prefix > 0 && (!kpre || !vpre || !cu_prefix)) return EAGLE3_EINVAL;
  if (!o && (!o_part || !lse_part)) return EAGLE3_EINVAL;
  for (const void* ptr : {q, k_tree, v_tree, kpre, vpre, (const void*)o_part, (const void*)o})
    if ((uintptr_t)ptr % 16) return EAGLE3_EINVAL;
  const int S = attention_splits(B, Hkv, max_nodes * (Hq / Hkv), max_prefix, n_splits);
  if (!o_part || !lse_part) {
    const size_t need =
        eagle3_tree_attention_workspace_size(B, T, Hq, Hkv, Dh, max_nodes, max_prefix, n_splits);
    if (!workspace || workspace_bytes < need) return EAGLE3_EWORKSPACE;
    Carve c(workspace);
    o_part = c.take<float>((size_t)(S + 1) * T * Hq * Dh);
    lse_part = c.take<float>((size_t)(S + 1) * T * Hq);
  }
  AttnArgs a;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Dh = Dh;
  a.dtype = dtype;
  a.q = q;
  a.q_cu = cu_nodes;
  a.q_stride = 0;
  a.q_rows_total = T;
  a.kt = k_tree;
  a.vt = v_tree;
  a.kt_cu = cu_nodes;
  a.kt_stride = 0;
  a.kt_count = 0;
  a.mask = mask;
  a.W64 = W64;
  a.kp = kpre;
  a.vp = vpre;
  a.p_cu = max_prefix > 0 ? cu_prefix : nullptr;
  a.scale = scale;
  a.S = S;
  a.max_q_per_req = max_nodes;
  a.o_part = o_part;
  a.lse_part = lse_part;
  hipStream_t s = (hipStream_t)stream;
  int st = launch_tree_attention(a, s, "tree_attention");
  if (st || !o) return st;
  return launch_lse_merge(S + 1, T * Hq, Dh, o_part, lse_part, dtype, o, lse, s, "lse_merge");
}

int eagle3_lse_merge(int S, int rows, int Dh, const float* o_part, const float* lse_part,
                     int out_dtype, void* o, float* lse, void* stream) {
  if (S < 1 || rows < 0 || Dh <= 0 || Dh % 4) return EAGLE3_EINVAL;
  if (S > 512 || Dh > 128) return EAGLE3_EUNSUPPORTED;
  if (!dtype_ok(out_dtype)) return EAGLE3_EINVAL;
  if (rows == 0) return EAGLE3_OK;
  if (!o_part || !lse_part || !o) return EAGLE3_EINVAL;
  if ((uintptr_t)o_part % 16 || (uintptr_t)o % 16) return EAGLE3_EINVAL;
  return launch_lse_merge(S, rows, Dh, o_part, lse_part, out_dtype, o, lse, (hipStream_t)stream,
                          "lse_merge");
}

// ---- linear (the projections' GEMM) ----------------------------------------------------
namespace {
bool linear_shape_ok(int M, int N, int K, int dtype) {
  if (M <= 0 || N <= 0 || K <= 0 || !dtype_ok(dtype)) return false;
  return true;
}
}  // namespace

size_t eagle3_linear_workspace_size(int M, int N, int K, int dtype) {
  if (!linear_shape_ok(M, N, K, dtype)) return 0;
  const GemmPlan p = plan_gemm(M, N, K, dtype);
  if (p.splits <= 1) return 0;
  Carve c(nullptr);
  c.take<float>((size_t)p.splits * M * N);
  return c.size();
}

int eagle3_linear(int M, int N, int K, int dtype, const void* X, int ldx, const void* W, float* Y,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!linear_shape_ok(M, N, K, dtype) || ldx < K) return EAGLE3_EINVAL;
  if (N % 4 || K % 8) return EAGLE3_EUNSUPPORTED;
  if (!X || !W || !Y) return EAGLE3_EINVAL;
  if ((uintptr_t)X % 16 || (uintptr_t)W % 16 || (uintptr_t)Y % 16 || ((size_t)ldx * elem_size(dtype)) % 16)
    return EAGLE3_EINVAL;
  const GemmPlan p = plan_gemm(M, N, K, dtype);
  if (!p.tile && (p.MT == 0 || M > 160)) return EAGLE3_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  if (p.splits <= 1) return launch_gemm(p, dtype, X, ldx, W, Y, s, "linear");
  const size_t need = eagle3_linear_workspace_size(M, N, K, dtype);
  if (!workspace || workspace_bytes < need) return EAGLE3_EWORKSPACE;
  float* part = static_cast<float*>(workspace);
  int st = launch_gemm(p, dtype, X, ldx, W, part, s, "linear");
  if (st) return st;
  return launch_epi_sum(p, part, Y, nullptr, s, "linear_sum");
}

// ---- accept ---------------------------------------------------------------------------
int eagle3_commit_kv(int B, int Hkv, int Dh, int dtype, int path_stride, const int32_t* cu_nodes,
                     const int32_t* path, const int32_t* accept_len, const void* k_tree, const void* v_tree,
                     const int32_t* dst_row, int64_t cache_rows, void* k_cache, void* v_cache,
                     int32_t* dev_status, void* stream) {
  if (B <= 0 || Hkv <= 0 || Dh <= 0 || path_stride <= 0 || cache_rows < 0) return EAGLE3_EINVAL;
  if (!dtype_ok(dtype)) return EAGLE3_EINVAL;
  if (!cu_nodes || !path || !accept_len || !k_tree || !v_tree || !dst_row || !k_cache || !v_cache)
    return EAGLE3_EINVAL;
  const long row_bytes = (long)Hkv * Dh * elem_size(dtype);
  if (row_bytes % 16) return EAGLE3_EINVAL;
  if ((uintptr_t)k_tree % 16 || (uintptr_t)v_tree % 16 || (uintptr_t)k_cache % 16 || (uintptr_t)v_cache % 16)
    return EAGLE3_EINVAL;
  if (path_stride > 65535 || B > 65535) return EAGLE3_EUNSUPPORTED;
  return launch_commit_kv(B, Hkv * Dh, dtype, path_stride, cu_nodes, path, accept_len, k_tree, v_tree, dst_row,
                          (long)cache_rows, k_cache, v_cache, dev_status, (hipStream_t)stream);
}

size_t eagle3_drafter_catchup_workspace_size(const eagle3_drafter* w, int n) {
  if (drafter_check(w) != EAGLE3_OK || n <= 0) return 0;
  return catchup_workspace(w, n);
}

int eagle3_drafter_catchup(const eagle3_drafter* w, int n, const int32_t* tokens, const int32_t* pos,
                           const void* h_low, const void* h_mid, const void* h_high, const int32_t* dst_row,
                           int64_t cache_rows, void* k_cache, void* v_cache, float* g_out, int32_t* dev_status,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (const int st = drafter_check(w)) return st;
  if (n <= 0 || cache_rows < 0) return EAGLE3_EINVAL;
  if (!tokens || !pos || !h_low || !h_mid || !h_high || !dst_row || !k_cache || !v_cache) return EAGLE3_EINVAL;
  if ((uintptr_t)h_low % 16 || (uintptr_t)h_mid % 16 || (uintptr_t)h_high % 16 || (uintptr_t)k_cache % 16 ||
      (uintptr_t)v_cache % 16 || (uintptr_t)g_out % 16)
    return EAGLE3_EINVAL;
  if (!catchup_supported(w, n)) return EAGLE3_EUNSUPPORTED;
  const size_t need = catchup_workspace(w, n);
  if (!workspace || workspace_bytes < need) return EAGLE3_EWORKSPACE;
  return launch_catchup(w, n, tokens, pos, h_low, h_mid, h_high, dst_row, (long)cache_rows, k_cache, v_cache,
                        g_out, dev_status, workspace, (hipStream_t)stream);
}

int eagle3_causal_attention(int L, int Hq, int Hkv, int Dh, int dtype, const void* q, const void* k,
                            const void* v, float scale, float* o, float* lse, void* stream) {
  if (L <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || !(scale > 0.f)) return EAGLE3_EINVAL;
  if (!dtype_ok(dtype) || !q || !k || !v || !o || !lse) return EAGLE3_EINVAL;
  if ((uintptr_t)q % 16 || (uintptr_t)k % 16 || (uintptr_t)v % 16 || (uintptr_t)o % 16) return EAGLE3_EINVAL;
  if (dtype != EAGLE3_BF16 || (Dh != 64 && Dh != 128)) return EAGLE3_EUNSUPPORTED;
  if ((long)L * Hkv * Dh * 2 > 0xFFFFFFFFL) return EAGLE3_EUNSUPPORTED;   // 32-bit stream offsets
  return launch_causal_attention(L, Hq, Hkv, Dh, q, k, v, scale, o, lse, (hipStream_t)stream);
}

int eagle3_branch_attention(int L, int n_steps, int Hq, int Hkv, int Dh, int dtype, const void* q,
                            const void* kb, const void* vb, float scale, float* o, float* lse, void* stream) {
  if (L <= 0 || n_steps <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || !(scale > 0.f)) return EAGLE3_EINVAL;
  if (!dtype_ok(dtype) || !q || !kb || !vb || !o || !lse) return EAGLE3_EINVAL;
  if ((uintptr_t)q % 16 || (uintptr_t)kb % 16 || (uintptr_t)vb % 16 || (uintptr_t)o % 16) return EAGLE3_EINVAL;
  if (Dh != 128 || n_steps > 8 || (Hq / Hkv) * (Dh / 8) > 1024 || Hkv > 65535) return EAGLE3_EUNSUPPORTED;
  return launch_branch_attention(L, n_steps, Hq, Hkv, Dh, dtype, q, kb, vb, scale, o, lse, (hipStream_t)stream);
}

size_t eagle3_accept_workspace_size(int T, int V) {
  if (T < 0 || V <= 0) return 0;
  return accept_workspace(T, V);
}

int eagle3_accept(int B, int T, const int32_t* cu_nodes, const int32_t* tokens,
                  const int32_t* parents, const uint64_t* mask, int W64, const void* logits, int V,
                  int dtype, float temperature, uint64_t seed, uint64_t round, int max_depth,
                  int32_t* accept_len, int32_t* path, int32_t* out_tokens, int32_t* bonus,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (B <= 0 || T < B || V <= 0 || W64 < 1 || max_depth < 0) return EAGLE3_EINVAL;
  if (!dtype_ok(dtype)) return EAGLE3_EINVAL;
  if (!(temperature >= 0.f) || temperature == __builtin_huge_valf()) return EAGLE3_EINVAL;
  if (W64 > 4) return EAGLE3_EUNSUPPORTED;
  if (!cu_nodes || !tokens || !parents || !mask || !logits || !accept_len || !path || !out_tokens ||
      !bonus)
    return EAGLE3_EINVAL;
  const size_t need = accept_workspace(T, V);
  if (!workspace || workspace_bytes < need) return EAGLE3_EWORKSPACE;
  Carve c(workspace);
  const int n_chunks = accept_chunks(V);
  float* pv = c.take<float>((size_t)T * n_chunks);
  int* pi = c.take<int>((size_t)T * n_chunks);
  return launch_accept(B, T, cu_nodes, tokens, parents, mask, W64, logits, V, dtype, temperature,
                       seed, round, max_depth, accept_len, path, out_tokens, bonus, pv, pi,
                       (hipStream_t)stream);
}

size_t eagle3_accept_sampled_workspace_size(int T, int V, int max_children) {
  if (T < 1 || V <= 0 || max_children < 1 || max_children > accept_sampled_max_children()) return 0;
  return accept_sampled_workspace(T, V, max_children);
}

int eagle3_accept_sampled(int B, int T, const int32_t* cu_nodes, const int32_t* tokens,
                          const int32_t* parents, const void* logits, int V, int dtype,
                          const void* draft_logits, int draft_dtype, int n_draft_rows,
                          const int32_t* draft_row, int max_children, float temperature,
                          uint64_t seed, uint64_t round, int max_depth, int32_t* accept_len,
                          int32_t* path, int32_t* out_tokens, int32_t* bonus, int32_t* dev_status,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (B <= 0 || T < B || V <= 0 || max_depth < 0 || n_draft_rows < 0) return EAGLE3_EINVAL;
  if (!dtype_ok(dtype) || (n_draft_rows > 0 && !dtype_ok(draft_dtype))) return EAGLE3_EINVAL;
  if (!(temperature > 0.f) || temperature == __builtin_huge_valf()) return EAGLE3_EINVAL;
  if (!cu_nodes || !tokens || !parents || !logits || !draft_row || !accept_len || !path ||
      !out_tokens || !bonus || (n_draft_rows > 0 && !draft_logits))
    return EAGLE3_EINVAL;
  if (max_children < 1 || max_children > accept_sampled_max_children()) return EAGLE3_EUNSUPPORTED;
  const size_t need = accept_sampled_workspace(T, V, max_children);
  if (!workspace || workspace_bytes < need) return EAGLE3_EWORKSPACE;
  return launch_accept_sampled(B, T, cu_nodes, tokens, parents, logits, V, dtype,
                               n_draft_rows > 0 ? draft_logits : nullptr, draft_dtype, n_draft_rows,
                               draft_row, max_children, temperature, seed, round, max_depth,
                               accept_len, path, out_tokens, bonus, dev_status, workspace,
                               (hipStream_t)stream);
}

// ---- timing ---------------------------------------------------------------------------
int eagle3_profile_enable(int on, const char* only_kernel) {
  std::lock_guard<std::mutex> lk(e3h::g_mu);
  e3h::g_on = on != 0;
  e3h::g_only = only_kernel ? only_kernel : "";
  return EAGLE3_OK;
}

int eagle3_profile_reset(void) {
  std::lock_guard<std::mutex> lk(e3h::g_mu);
  for (auto& r : e3h::g_recs) {
    (void)hipEventSynchronize(r.e1);
    e3h::g_pool.push_back(r.e0);
    e3h::g_pool.push_back(r.e1);
  }
  e3h::g_recs.clear();
  e3h::g_open = -1;
  return EAGLE3_OK;
}

int eagle3_profile_read(const char* kernel, double* total_ms, int* launches) {
  if (!kernel || !total_ms || !launches) return EAGLE3_EINVAL;
  std::lock_guard<std::mutex> lk(e3h::g_mu);
  double tot = 0.0;
  int n = 0;
  for (auto& r : e3h::g_recs) {
    if (r.name != kernel) continue;
    if (hipEventSynchronize(r.e1) != hipSuccess) return EAGLE3_EHIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) return EAGLE3_EHIP;
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return EAGLE3_OK;
}

}  // extern "C"
