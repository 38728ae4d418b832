// Sampled-candidate acceptance: verification of drafted children that were drawn from the
// drafter's distribution (not taken as its top-K).
//
// At node i the target side is p = softmax(z_i / T) and the draft side q = softmax(zq_i / T),
// both in float64 (z / T formed as z * (1 / T)).  The children are tested in node-index order.
// After r rejections the target side is p_r(t) = max(p_t - lam q_t, 0) / N and the draft side
// q_r(t) = q_t / c for the tokens not yet rejected, with c = 1 - (q of the rejected tokens):
// rejecting x moves lam to lam + N / c and c to c - q_x, and the new N is
// sum_t max(p_t - lam q_t, 0).  (Induction: max(p_r - q_r, 0) = max(p - (lam + N / c) q, 0) / N
// on every token not yet rejected, and a rejected token x had p_r(x) < q_r(x), so p - lam' q is
// negative there from then on.)  Each rejection therefore costs one reduction over the
// vocabulary, the only sequential part.
//
// Launches: clear; stats (log-sum-exps of p and q at every node with a draft row, then the test
// of its first child); one pass per further child (N at the node's lam, then the test) over a
// device-side list of the nodes still undecided; the walk from each root through the kept
// children; the draw of the bonus token at each request's end node only.
//
// Within a pass, the workgroup that finishes a node's last chunk (a per-node counter) combines
// the node's partials in one fixed order.  Partials travel through agent-scope relaxed atomic
// stores and loads into per-pass slots preset to a sentinel: the reader waits (bounded) only
// for a store that its writer has issued but that is not visible yet, and no workgroup has to
// write back or invalidate the L2.
#include "common.h"
#include "internal.h"

using namespace e3;

namespace {

constexpr int SC = 4096;          // tokens per chunk, 16 per thread
constexpr int DC = 1024;          // tokens per chunk of the end-node draw, 4 per thread
constexpr int kMaxNodes = 256;    // nodes per request
constexpr int kMaxKids = 64;      // children tested per node
constexpr uint32_t kUniformC0 = 0x40000000u;   // counter word 0 of the acceptance uniforms
constexpr double kNegInfD = -__builtin_huge_val();
constexpr uint64_t kEmpty = 0x7FF4DEADBEEF0001ull;   // sentinel of an unwritten double slot
constexpr int kEmptyI = (int)0x80000000u;             // sentinel of an unwritten int slot
constexpr int kSpinMax = 1 << 16;

enum : int { ST_NEED = 0, ST_KEPT = 1, ST_DRAW = 2 };

struct NodeSt {
  double A, Bq;            // log-sum-exp of z / T and of zq / T
  double lam, lam_prev, N, c;
  int status;              // ST_NEED: candidate k waits for pass m
  int m, k, rej, npos, kept, nk, pad;
};

struct SArgs {
  const int32_t* cu_nodes;
  const int32_t* tokens;
  const int32_t* parents;
  const int32_t* draft_row;
  const void* logits;
  const void* dlogits;
  int B, T, V, nch, ndc, R, maxc, max_depth, az, aq;
  double invT;
  uint32_t seed_lo, seed_hi, rnd;
  NodeSt* st;         // [T]
  int* cnt;           // [T] chunks finished in the current pass
  int* lists;         // [maxc + 1][T]: list m (2 .. maxc) waits for pass m; list 0: end nodes to draw
  int* list_n;        // [maxc + 1]
  uint64_t* p_stats;  // [T][nch][4]        (max a, sum, max b, sum)
  uint64_t* p_n;      // [maxc - 1][T][nch] N partial of pass m
  int* p_pos;         // [T][nch]           tokens with q > 0 (pass 2)
  uint64_t* p_dv;     // [T][ndc]           draw: best value
  int* p_di;          // [T][ndc]           draw: its token
  int* kids_g;        // [T][maxc]          children of a node (written by the stats pass)
  int* toks_g;        // [T][maxc]          their tokens
  int32_t* accept_len;
  int32_t* path;
  int32_t* out_tokens;
  int32_t* bonus;
  int32_t* dev_status;
};

// ---- cross-workgroup slots -------------------------------------------------------------
__device__ __forceinline__ void put_d(uint64_t* p, double v) {
  __hip_atomic_store(p, (uint64_t)__double_as_longlong(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put_i(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A slot whose writer has already counted its chunk as finished: the store is issued, so it
// becomes visible; the wait is bounded all the same and a miss is flagged.
__device__ __forceinline__ double get_d(uint64_t* p, int32_t* dev_status) {
  uint64_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int it = 0; v == kEmpty && it < kSpinMax; ++it) {
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (v == kEmpty) {
    if (dev_status) atomicOr(dev_status, EAGLE3_DEV_SYNC);
    return 0.0;
  }
  return __longlong_as_double((long long)v);
}
__device__ __forceinline__ int get_i(int* p, int32_t* dev_status) {
  int v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int it = 0; v == kEmptyI && it < kSpinMax; ++it) {
    __builtin_amdgcn_s_sleep(1);
    v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (v == kEmptyI) {
    if (dev_status) atomicOr(dev_status, EAGLE3_DEV_SYNC);
    return 0;
  }
  return v;
}

// Count one finished chunk of node g; true (in every thread) in the workgroup that finished the
// node's last chunk.  Thread 0 has issued the chunk's partial store before this call.
__device__ __forceinline__ bool finish_chunk(const SArgs& a, int g, int* s_last, int n_chunks = -1) {
  if (threadIdx.x == 0) *s_last = atomicAdd(&a.cnt[g], 1) == (n_chunks < 0 ? a.nch : n_chunks) - 1;
  __syncthreads();
  return *s_last != 0;
}

// ---- loads and reductions --------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void load_chunk(const T* row, int tb, int V, int aligned, float* z) {
  constexpr int EPC = Vec<T>::N;
  if (aligned && tb + 16 <= V) {
#pragma unroll
    for (int q = 0; q < 16 / EPC; ++q) {
      const u32x4 v = ld16(row + tb + q * EPC);
#pragma unroll
      for (int e = 0; e < EPC; ++e) z[q * EPC + e] = chunk_elem<T>(v, e);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = tb + e < V ? to_f32(row[tb + e]) : 0.0f;
  }
}

// (m, s) pairs standing for s * exp(m); the combination is symmetric bit for bit, so a
// butterfly leaves every lane with the same result.
__device__ __forceinline__ void lse_add(double& m, double& s, double m2, double s2) {
#pragma clang fp contract(off)
  if (s2 == 0.0) return;
  if (s == 0.0) {
    m = m2;
    s = s2;
    return;
  }
  const double M = m > m2 ? m : m2;
  s = s * exp(m - M) + s2 * exp(m2 - M);
  m = M;
}

__device__ __forceinline__ void wave_lse(double& m, double& s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lse_add(m, s, __shfl_xor(m, off), __shfl_xor(s, off));
}

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma clang fp contract(off)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = x + __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Block-wide max / sum of two values (256 threads); every thread receives both results.
__device__ __forceinline__ void block_max2(double& x, double& y, double* sm) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    x = fmax(x, __shfl_xor(x, off));
    y = fmax(y, __shfl_xor(y, off));
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[w] = x;
    sm[4 + w] = y;
  }
  __syncthreads();
  x = fmax(fmax(sm[0], sm[1]), fmax(sm[2], sm[3]));
  y = fmax(fmax(sm[4], sm[5]), fmax(sm[6], sm[7]));
  __syncthreads();
}

__device__ __forceinline__ void block_sum2(double& x, double& y, double* sm) {
#pragma clang fp contract(off)
  x = wave_sum_d(x);
  y = wave_sum_d(y);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[w] = x;
    sm[4 + w] = y;
  }
  __syncthreads();
  x = (sm[0] + sm[1]) + (sm[2] + sm[3]);
  y = (sm[4] + sm[5]) + (sm[6] + sm[7]);
  __syncthreads();
}

// exp(x), x <= 0, by Tang's table-driven method (ACM TOMS 15(2), 1989): x = (64 k + j) ln2/64 + r
// with |r| <= ln2/128, exp(x) = 2^k * 2^(j/64) * exp(r), exp(r) by its degree-5 Taylor polynomial
// (truncation below 4e-17 relative on that interval).  ln2/64 is split in a float64 head and
// tail (from the series of ln 2) so that r is formed to within rounding; tab[j] = 2^(j/64) is
// filled per workgroup by exp2_table.  Below -1000 the result is 0.
constexpr double kExpInvStep = 0x1.71547652b82fep+6;   // 64 / ln 2
constexpr double kExpStepHi = 0x1.62e42fefa39efp-7;    // ln 2 / 64, head
constexpr double kExpStepLo = 0x1.abc9e3b39803fp-62;   // ln 2 / 64 - head
__device__ __forceinline__ void exp2_table(double* tab) {
  if (threadIdx.x < 64) tab[threadIdx.x] = exp2((double)threadIdx.x * 0.015625);
  __syncthreads();
}
__device__ __forceinline__ double exp_tab(double x, const double* tab) {
  const double xc = fmax(x, -1000.0);
  const double nd = __builtin_rint(xc * kExpInvStep);
  const int n = (int)nd;
  double r = __builtin_fma(-nd, kExpStepHi, xc);
  r = __builtin_fma(-nd, kExpStepLo, r);
  double p = __builtin_fma(r, 1.0 / 120.0, 1.0 / 24.0);
  p = __builtin_fma(p, r, 1.0 / 6.0);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  return __builtin_ldexp(tab[n & 63] * p, n >> 6);
}

__device__ __forceinline__ bool better_d(double va, int ia, double vb, int ib) {
  return (va > vb) | ((va == vb) & (ia < ib));
}

__device__ __forceinline__ void wave_argmax_d(double& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double ov = __shfl_xor(v, off);
    const int oi = __shfl_xor(i, off);
    if (better_d(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

__device__ __forceinline__ double accept_uniform(const SArgs& a, int b, int j) {
#pragma clang fp contract(off)
  uint32_t ctr[4] = {kUniformC0, (uint32_t)j, (uint32_t)b, a.rnd};
  philox4x32_10(ctr, a.seed_lo, a.seed_hi);
  return (double)(((float)(ctr[0] >> 9) + 0.5f) * 1.1920928955078125e-07f);  // 2^-23
}

// ---- the chain at one node -------------------------------------------------------------
// Children of request-local node i (nodes j > i with parent i, in index order, at most maxc)
// and their tokens, into LDS.  Whole block of 256 threads (one per possible node).
__device__ __forceinline__ int node_children(const SArgs& a, int n0, int n, int i, int* s_kids,
                                             int* s_tok, int* s_cnt) {
  const int j = threadIdx.x;
  const bool is = j > i && j < n && a.parents[n0 + j] == i;
  const uint64_t bal = __ballot(is);
  const int lane = j & 63, w = j >> 6;
  if (lane == 0) s_cnt[w] = __popcll(bal);
  __syncthreads();
  int before = __popcll(bal & ((1ull << lane) - 1ull));
  for (int q = 0; q < w; ++q) before += s_cnt[q];
  if (is && before < a.maxc) {
    s_kids[before] = j;
    s_tok[before] = a.tokens[n0 + j];
  }
  const int nk = min(s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3], a.maxc);
  __syncthreads();
  return nk;
}

// First candidate at or after k whose token is inside the vocabulary and differs from every
// earlier candidate's (an earlier equal token was tested and rejected already).
__device__ __forceinline__ int next_valid(const int* s_tok, int nk, int V, int k) {
  for (; k < nk; ++k) {
    const int x = s_tok[k];
    if (x < 0 || x >= V) continue;
    bool dup = false;
    for (int q = 0; q < k; ++q) dup |= s_tok[q] == x;
    if (!dup) return k;
  }
  return -1;
}

// Test the candidate waiting at s.k; from_pass: the pass that gives its N (and, for the second
// candidate, the count of tokens with q > 0) has just finished.
template <typename TZ, typename TQ>
__device__ void chain_step(const SArgs& a, NodeSt& s, const int* s_kids, const int* s_tok, int b,
                           const TZ* zrow, const TQ* qrow, bool from_pass, double N_new,
                           int npos_new, const float* pre = nullptr) {
#pragma clang fp contract(off)
  if (from_pass) {
    if (s.m == 2) s.npos = npos_new;
    if (s.rej >= s.npos) {  // every token the drafter could propose is rejected already
      s.status = ST_DRAW;
      return;
    }
    if (N_new > 0.0)
      s.N = N_new;
    else
      s.lam = s.lam_prev;
  }
  const int j = s_kids[s.k];
  const int x = s_tok[s.k];
  const float zx = pre ? pre[0] : to_f32(zrow[x]);
  const float qz = pre ? pre[1] : to_f32(qrow[x]);
  const double px = exp((double)zx * a.invT - s.A);
  const double qx = exp((double)qz * a.invT - s.Bq);
  bool keep = qx == 0.0;
  if (!keep) {
    const double pr = px - s.lam * qx;
    const double t = ((pr > 0.0 ? pr : 0.0) / s.N) / (qx / s.c);
    keep = accept_uniform(a, b, j) < t;
  }
  if (keep) {
    s.status = ST_KEPT;
    s.kept = j;
    return;
  }
  s.lam_prev = s.lam;
  s.lam = s.lam + s.N / s.c;
  s.c = s.c - qx;
  s.rej += 1;
  const int k2 = next_valid(s_tok, s.nk, a.V, s.k + 1);
  if (k2 < 0) {
    s.status = ST_DRAW;
    return;
  }
  s.k = k2;
  s.m += 1;
  s.status = ST_NEED;
}

__device__ __forceinline__ void enqueue_need(const SArgs& a, const NodeSt& s, int g) {
  if (s.status == ST_NEED) {
    const int at = atomicAdd(&a.list_n[s.m], 1);
    a.lists[(size_t)s.m * a.T + at] = g;
  }
}

// ---- kernels ---------------------------------------------------------------------------
__global__ void k_samp_clear(SArgs a, int n_stats, int n_n, int n_one, int n_draw) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < a.T) a.cnt[t] = 0;
  if (t <= a.maxc) a.list_n[t] = 0;
  if (t < n_stats) a.p_stats[t] = kEmpty;
  if (t < n_n) a.p_n[t] = kEmpty;
  if (t < n_one) a.p_pos[t] = kEmptyI;
  if (t < n_draw) {
    a.p_dv[t] = kEmpty;
    a.p_di[t] = kEmptyI;
  }
}

// Stats: log-sum-exps of p and q at every node with a draft row (the chunk's maximum first, so
// every element costs one exp); the last chunk tests the node's first child.  A node without a
// draft row is decided here (it draws from p) by its chunk-0 workgroup.
template <typename TZ, typename TQ>
__global__ __launch_bounds__(256) void k_samp_stats(SArgs a) {
#pragma clang fp contract(off)
  __shared__ double sm[8];
  __shared__ int s_kids[kMaxKids], s_tok[kMaxKids], s_cnt[4], s_last;
  const int g = blockIdx.x / a.nch, c = blockIdx.x % a.nch;
  const int b = find_request(a.cu_nodes, a.B, g);
  const int n0 = a.cu_nodes[b];
  const int n = min(a.cu_nodes[b + 1] - n0, kMaxNodes);
  const int i = g - n0;
  if (i >= kMaxNodes) {  // beyond what one request may hold: never reached by the walk
    if (c == 0 && threadIdx.x == 0 && a.dev_status) atomicOr(a.dev_status, EAGLE3_DEV_BAD_PATH);
    return;
  }
  const int r = a.draft_row[g];
  if (r < 0 || r >= a.R) {
    if (c != 0) return;
    const int nk = node_children(a, n0, n, i, s_kids, s_tok, s_cnt);
    if (threadIdx.x != 0) return;
    if (nk > 0 && a.dev_status) atomicOr(a.dev_status, EAGLE3_DEV_BAD_ROW);
    NodeSt s = {};
    s.status = ST_DRAW;
    s.kept = -1;
    a.st[g] = s;
    return;
  }
  __shared__ double s_exp[64];
  exp2_table(s_exp);
  const TZ* zrow = (const TZ*)a.logits + (size_t)g * a.V;
  const TQ* qrow = (const TQ*)a.dlogits + (size_t)r * a.V;
  const int tb = c * SC + 16 * threadIdx.x;
  const int ne = min(16, a.V - tb);      // <= 0 past the vocabulary
  double va[16], vb[16];
  {
    float z[16];
    load_chunk(zrow, tb, a.V, a.az, z);
#pragma unroll
    for (int e = 0; e < 16; ++e) va[e] = e < ne ? (double)z[e] * a.invT : kNegInfD;
    load_chunk(qrow, tb, a.V, a.aq, z);
#pragma unroll
    for (int e = 0; e < 16; ++e) vb[e] = e < ne ? (double)z[e] * a.invT : kNegInfD;
  }
  double ma = kNegInfD, mb = kNegInfD;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    ma = fmax(ma, va[e]);
    mb = fmax(mb, vb[e]);
  }
  block_max2(ma, mb, sm);
  double sa = 0.0, sb = 0.0;
  if (ma != kNegInfD) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sa = sa + exp_tab(va[e] - ma, s_exp);
  }
  if (mb != kNegInfD) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sb = sb + exp_tab(vb[e] - mb, s_exp);
  }
  block_sum2(sa, sb, sm);
  if (threadIdx.x == 0) {
    uint64_t* p = a.p_stats + ((size_t)g * a.nch + c) * 4;
    put_d(p + 0, ma);
    put_d(p + 1, sa);
    put_d(p + 2, mb);
    put_d(p + 3, sb);
  }
  if (!finish_chunk(a, g, &s_last)) return;
  const int nk = node_children(a, n0, n, i, s_kids, s_tok, s_cnt);
  if ((int)threadIdx.x < nk) {   // kept for the later passes of this node
    a.kids_g[(size_t)g * a.maxc + threadIdx.x] = s_kids[threadIdx.x];
    a.toks_g[(size_t)g * a.maxc + threadIdx.x] = s_tok[threadIdx.x];
  }
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  double MA = kNegInfD, SA = 0.0, MB = kNegInfD, SB = 0.0;
  for (int cc = lane; cc < a.nch; cc += 64) {
    uint64_t* p = a.p_stats + ((size_t)g * a.nch + cc) * 4;
    const double m0 = get_d(p + 0, a.dev_status), s0 = get_d(p + 1, a.dev_status);
    const double m1 = get_d(p + 2, a.dev_status), s1 = get_d(p + 3, a.dev_status);
    lse_add(MA, SA, m0, s0);
    lse_add(MB, SB, m1, s1);
  }
  wave_lse(MA, SA);
  wave_lse(MB, SB);
  if (lane != 0) return;
  NodeSt s;
  s.A = MA + log(SA);
  s.Bq = MB + log(SB);
  s.lam = 0.0;
  s.lam_prev = 0.0;
  s.N = 1.0;
  s.c = 1.0;
  s.m = 0;
  s.k = 0;
  s.rej = 0;
  s.npos = 0x7fffffff;
  s.kept = -1;
  s.nk = nk;
  s.pad = 0;
  s.status = ST_DRAW;
  for (int k = 0; k < nk; ++k)
    if ((s_tok[k] < 0 || s_tok[k] >= a.V) && a.dev_status) atomicOr(a.dev_status, EAGLE3_DEV_BAD_TOKEN);
  const int k0 = next_valid(s_tok, nk, a.V, 0);
  if (k0 >= 0) {
    s.k = k0;
    s.m = 1;
    chain_step(a, s, s_kids, s_tok, b, zrow, qrow, false, 0.0, 0);
  }
  a.st[g] = s;
  a.cnt[g] = 0;
  enqueue_need(a, s, g);
}

// Pass m (2 .. maxc): N at the node's current lam, for the nodes on list m; the last chunk
// tests the waiting candidate.
template <typename TZ, typename TQ>
__global__ __launch_bounds__(256) void k_samp_npass(SArgs a, int m) {
#pragma clang fp contract(off)
  __shared__ double sm[8];
  __shared__ int s_kids[kMaxKids], s_tok[kMaxKids], s_last;
  __shared__ float s_pre[2];
  __shared__ double s_exp[64];
  const int items = a.list_n[m] * a.nch;
  if ((int)blockIdx.x >= items) return;
  exp2_table(s_exp);
  const int lane = threadIdx.x & 63;
  uint64_t* pn = a.p_n + (size_t)(m - 2) * a.T * a.nch;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int g = a.lists[(size_t)m * a.T + it / a.nch];
    const int c = it % a.nch;
    const NodeSt s0 = a.st[g];
    const int r = a.draft_row[g];
    const TZ* zrow = (const TZ*)a.logits + (size_t)g * a.V;
    const TQ* qrow = (const TQ*)a.dlogits + (size_t)r * a.V;
    const int tb = c * SC + 16 * threadIdx.x;
    const int ne = min(16, a.V - tb);
    float pz = 0.f, pq = 0.f;
    if (threadIdx.x == 0) {   // the waiting candidate's logits, in case this chunk is the node's last
      const int x = a.toks_g[(size_t)g * a.maxc + s0.k];
      pz = to_f32(zrow[x]);
      pq = to_f32(qrow[x]);
    }
    double acc = 0.0, pos = 0.0;
    {
      float z[16], zq[16];
      load_chunk(zrow, tb, a.V, a.az, z);
      load_chunk(qrow, tb, a.V, a.aq, zq);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const double pe = e < ne ? exp_tab((double)z[e] * a.invT - s0.A, s_exp) : 0.0;
        const double qe = e < ne ? exp_tab((double)zq[e] * a.invT - s0.Bq, s_exp) : 0.0;
        const double d = pe - s0.lam * qe;
        acc = acc + (d > 0.0 ? d : 0.0);
        pos = pos + (qe > 0.0 ? 1.0 : 0.0);
      }
    }
    block_sum2(acc, pos, sm);
    if (threadIdx.x == 0) {
      put_d(pn + (size_t)g * a.nch + c, acc);
      if (m == 2) put_i(a.p_pos + (size_t)g * a.nch + c, (int)pos);
      s_pre[0] = pz;
      s_pre[1] = pq;
    }
    if (finish_chunk(a, g, &s_last)) {
      const int b = find_request(a.cu_nodes, a.B, g);
      if ((int)threadIdx.x < s0.nk) {
        s_kids[threadIdx.x] = a.kids_g[(size_t)g * a.maxc + threadIdx.x];
        s_tok[threadIdx.x] = a.toks_g[(size_t)g * a.maxc + threadIdx.x];
      }
      __syncthreads();
      if (threadIdx.x < 64) {
        double N = 0.0;
        int np = 0;
        for (int cc = lane; cc < a.nch; cc += 64) {
          N = N + get_d(pn + (size_t)g * a.nch + cc, a.dev_status);
          if (m == 2) np += get_i(a.p_pos + (size_t)g * a.nch + cc, a.dev_status);
        }
        N = wave_sum_d(N);
        np = wave_sum_i(np);
        if (lane == 0) {
          NodeSt s = s0;
          chain_step(a, s, s_kids, s_tok, b, zrow, qrow, true, N, np, s_pre);
          a.st[g] = s;
          a.cnt[g] = 0;
          enqueue_need(a, s, g);
        }
      }
    }
    __syncthreads();
  }
}

// Walk each request from its root through the kept children; its end node either ends on a
// kept child at max_depth (that child's token is the bonus) or is queued for the draw.
__global__ __launch_bounds__(64) void k_samp_walk(SArgs a) {
  if (threadIdx.x != 0) return;
  const int b = blockIdx.x;
  const int P = a.max_depth + 1;
  const int n0 = clampi(a.cu_nodes[b], 0, a.T);
  const int n1 = clampi(a.cu_nodes[b + 1], n0, a.T);
  int32_t* pth = a.path + (size_t)b * P;
  int32_t* out = a.out_tokens + (size_t)b * P;
  int s = 0;
  if (n1 > n0) {
    int i = 0;
    pth[0] = 0;
    for (;;) {
      const NodeSt st = a.st[n0 + i];
      if (st.status == ST_KEPT) {
        const int j = st.kept;
        if (s == a.max_depth) {     // deeper than the caller's bound: the kept child is the bonus
          out[s] = a.tokens[n0 + j];
          a.bonus[b] = a.tokens[n0 + j];
          break;
        }
        ++s;
        pth[s] = j;
        out[s - 1] = a.tokens[n0 + j];
        i = j;
        continue;
      }
      const int at = atomicAdd(&a.list_n[0], 1);
      a.lists[at] = n0 + i;
      break;
    }
  } else {
    a.bonus[b] = -1;
  }
  for (int k = n1 > n0 ? s + 1 : 0; k < P; ++k) {
    pth[k] = -1;
    out[k] = -1;
  }
  a.accept_len[b] = s;
}

// Draw at the end nodes: argmax over t of ln max(p_t - lam q_t, 0) + G_t, G the node's Gumbel
// noise; with no rejection (lam = 0) the argmax of z_t / T + G_t (ln p_t up to a constant).
template <typename TZ, typename TQ>
__global__ __launch_bounds__(256) void k_samp_draw(SArgs a) {
#pragma clang fp contract(off)
  __shared__ double sv[4];
  __shared__ int sx[4];
  __shared__ int s_last;
  __shared__ double s_exp[64];
  const int items = a.list_n[0] * a.ndc;
  if ((int)blockIdx.x >= items) return;
  exp2_table(s_exp);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int g = a.lists[it / a.ndc];
    const int c = it % a.ndc;
    const NodeSt s0 = a.st[g];
    const int b = find_request(a.cu_nodes, a.B, g);
    const uint32_t i_local = (uint32_t)(g - a.cu_nodes[b]);
    const bool plain = s0.lam == 0.0;
    const int r = plain ? 0 : a.draft_row[g];
    const TZ* zrow = (const TZ*)a.logits + (size_t)g * a.V;
    const TQ* qrow = (const TQ*)a.dlogits + (size_t)r * a.V;
    const int tb = c * DC + 4 * threadIdx.x;
    double best = kNegInfD;
    int bi = 0x7fffffff;
    if (tb < a.V) {
      float z[4], zq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[e] = tb + e < a.V ? to_f32(zrow[tb + e]) : 0.f;
        zq[e] = (!plain && tb + e < a.V) ? to_f32(qrow[tb + e]) : 0.f;
      }
      {
        const int q = 0;
        uint32_t ctr[4] = {(uint32_t)(tb >> 2), i_local, (uint32_t)b, a.rnd};
        philox4x32_10(ctr, a.seed_lo, a.seed_hi);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = 4 * q + u, t = tb + e;
          if (t >= a.V) continue;
          double v;
          if (plain) {
            v = (double)z[e] * a.invT;
          } else {
            const double d = exp_tab((double)z[e] * a.invT - s0.A, s_exp) -
                             s0.lam * exp_tab((double)zq[e] * a.invT - s0.Bq, s_exp);
            v = d > 0.0 ? log(d) : kNegInfD;
          }
          v = v + (double)gumbel_from_word(ctr[u]);
          if (better_d(v, t, best, bi)) {
            best = v;
            bi = t;
          }
        }
      }
    }
    wave_argmax_d(best, bi);
    if (lane == 0) {
      sv[w] = best;
      sx[w] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int q = 1; q < 4; ++q)
        if (better_d(sv[q], sx[q], best, bi)) {
          best = sv[q];
          bi = sx[q];
        }
      put_d(a.p_dv + (size_t)g * a.ndc + c, best);
      put_i(a.p_di + (size_t)g * a.ndc + c, bi);
    }
    if (finish_chunk(a, g, &s_last, a.ndc) && threadIdx.x < 64) {
      double bv = kNegInfD;
      int bx = 0x7fffffff;
      for (int cc = lane; cc < a.ndc; cc += 64) {
        const double v = get_d(a.p_dv + (size_t)g * a.ndc + cc, a.dev_status);
        const int x = get_i(a.p_di + (size_t)g * a.ndc + cc, a.dev_status);
        if (better_d(v, x, bv, bx)) {
          bv = v;
          bx = x;
        }
      }
      wave_argmax_d(bv, bx);
      if (lane == 0) {
        const int y = bx < a.V ? bx : 0;
        const int L = a.accept_len[b];
        a.out_tokens[(size_t)b * (a.max_depth + 1) + L] = y;
        a.bonus[b] = y;
        a.cnt[g] = 0;
      }
    }
    __syncthreads();
  }
}

struct SampLayout {
  NodeSt* st;
  int *cnt, *lists, *list_n, *p_pos, *p_di, *kids_g, *toks_g;
  uint64_t *p_stats, *p_n, *p_dv;
  size_t bytes;
};

SampLayout carve_sampled(void* ws, int T, int nch, int ndc, int maxc) {
  e3h::Carve c(ws);
  SampLayout L;
  L.st = c.take<NodeSt>((size_t)T);
  L.cnt = c.take<int>((size_t)T);
  L.lists = c.take<int>((size_t)(maxc + 1) * T);
  L.list_n = c.take<int>((size_t)(maxc + 1));
  L.p_stats = c.take<uint64_t>((size_t)T * nch * 4);
  L.p_n = c.take<uint64_t>((size_t)(maxc > 1 ? maxc - 1 : 1) * T * nch);
  L.p_pos = c.take<int>((size_t)T * nch);
  L.p_dv = c.take<uint64_t>((size_t)T * ndc);
  L.p_di = c.take<int>((size_t)T * ndc);
  L.kids_g = c.take<int>((size_t)T * maxc);
  L.toks_g = c.take<int>((size_t)T * maxc);
  L.bytes = c.size();
  return L;
}

template <typename TZ, typename TQ>
void launch_typed(const SArgs& a, hipStream_t s) {
  const int grid = (int)std::min<long>((long)a.T * a.nch, 4096);
  {
    e3h::ProfScope ps("sampled_stats", s);
    hipLaunchKernelGGL((k_samp_stats<TZ, TQ>), dim3((unsigned)((long)a.T * a.nch)), dim3(256), 0, s, a);
  }
  for (int m = 2; m <= a.maxc; ++m) {
    e3h::ProfScope ps("sampled_npass", s);
    hipLaunchKernelGGL((k_samp_npass<TZ, TQ>), dim3(grid), dim3(256), 0, s, a, m);
  }
  {
    e3h::ProfScope ps("sampled_walk", s);
    hipLaunchKernelGGL(k_samp_walk, dim3(a.B), dim3(64), 0, s, a);
  }
  e3h::ProfScope ps("sampled_draw", s);
  hipLaunchKernelGGL((k_samp_draw<TZ, TQ>), dim3((unsigned)std::min<long>((long)a.B * a.ndc, 4096)), dim3(256),
                     0, s, a);
}

}  // namespace

namespace e3h {

size_t accept_sampled_workspace(int T, int V, int max_children) {
  return carve_sampled(nullptr, T, (V + SC - 1) / SC, (V + DC - 1) / DC, max_children).bytes;
}

int accept_sampled_max_children() { return kMaxKids; }

int launch_accept_sampled(int B, int T, const int32_t* cu_nodes, const int32_t* tokens,
                          const int32_t* parents, const void* logits, int V, int dtype,
                          const void* draft_logits, int draft_dtype, int n_draft_rows,
                          const int32_t* draft_row, int max_children, float temperature,
                          uint64_t seed, uint64_t round, int max_depth, int32_t* accept_len,
                          int32_t* path, int32_t* out_tokens, int32_t* bonus, int32_t* dev_status,
                          void* workspace, hipStream_t s) {
  if (max_children < 1 || max_children > kMaxKids) return EAGLE3_EUNSUPPORTED;
  const int nch = (V + SC - 1) / SC, ndc = (V + DC - 1) / DC;
  const SampLayout L = carve_sampled(workspace, T, nch, ndc, max_children);
  SArgs a;
  a.cu_nodes = cu_nodes;
  a.tokens = tokens;
  a.parents = parents;
  a.draft_row = draft_row;
  a.logits = logits;
  a.dlogits = draft_logits ? draft_logits : logits;
  a.B = B;
  a.T = T;
  a.V = V;
  a.nch = nch;
  a.ndc = ndc;
  a.R = draft_logits ? n_draft_rows : 0;
  a.maxc = max_children;
  a.max_depth = max_depth;
  a.az = ((size_t)V * elem_size(dtype)) % 16 == 0 && (uintptr_t)logits % 16 == 0;
  a.aq = draft_logits && ((size_t)V * elem_size(draft_dtype)) % 16 == 0 && (uintptr_t)draft_logits % 16 == 0;
  a.invT = 1.0 / (double)temperature;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.rnd = (uint32_t)round;
  a.st = L.st;
  a.cnt = L.cnt;
  a.lists = L.lists;
  a.list_n = L.list_n;
  a.p_stats = L.p_stats;
  a.p_n = L.p_n;
  a.p_pos = L.p_pos;
  a.p_dv = L.p_dv;
  a.p_di = L.p_di;
  a.kids_g = L.kids_g;
  a.toks_g = L.toks_g;
  a.accept_len = accept_len;
  a.path = path;
  a.out_tokens = out_tokens;
  a.bonus = bonus;
  a.dev_status = dev_status;
  {
    e3h::ProfScope ps("sampled_clear", s);
    const int n_stats = T * nch * 4;
    const int n_n = (max_children > 1 ? max_children - 1 : 1) * T * nch;
    const int n_one = T * nch, n_draw = T * ndc;
    const int nthreads = std::max({T, max_children + 1, n_stats, n_n, n_one, n_draw});
    hipLaunchKernelGGL(k_samp_clear, dim3((nthreads + 255) / 256), dim3(256), 0, s, a, n_stats, n_n, n_one,
                       n_draw);
  }
  int st = launch_status();
  if (st) return st;
  const bool zb = dtype == EAGLE3_BF16;
  const bool qb = (draft_logits ? draft_dtype : dtype) == EAGLE3_BF16;
  if (zb && qb)
    launch_typed<bf16, bf16>(a, s);
  else if (zb)
    launch_typed<bf16, float>(a, s);
  else if (qb)
    launch_typed<float, bf16>(a, s);
  else
    launch_typed<float, float>(a, s);
  return launch_status();
}

}  // namespace e3h
