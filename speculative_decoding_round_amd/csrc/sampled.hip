// Sampled-candidate acceptance: verification of drafted children that were drawn from the
// drafter's distribution (not taken as its top-K).
//
// At node i the target side is p = softmax(z_i / T) and the draft side q = softmax(zq_i / T),
// both in float64.  The children are tested in node-index order.  After r rejections the
// target side is p_r(t) = max(p_t - lam q_t, 0) / N and the draft side q_r(t) = q_t / c for
// the tokens not yet rejected, with c = 1 - (q of the rejected tokens): rejecting x moves lam
// to lam + N / c and c to c - q_x, and the new N is sum_t max(p_t - lam q_t, 0).  (Induction:
// max(p_r - q_r, 0) = max(p - (lam + N / c) q, 0) / N on every token not yet rejected, and a
// rejected token x had p_r(x) < q_r(x), so p - lam' q is negative there from then on.)  Each
// rejection therefore costs one reduction over the vocabulary, the only sequential part.
//
// Every pass runs over (node, chunk of 4096 tokens) items.  The workgroup that finishes a
// node's last chunk (a per-node counter) combines the node's partials in one fixed order and
// advances its chain: the node is either decided (a child kept, or a draw from the residual
// target side) or queued on the list of the next pass.  The lists keep the grids of later
// passes to the nodes still undecided.
#include "common.h"
#include "internal.h"

using namespace e3;

namespace {

constexpr int SC = 4096;          // tokens per chunk, 16 per thread
constexpr int kMaxNodes = 256;    // nodes per request
constexpr int kMaxKids = 64;      // children tested per node
constexpr uint32_t kUniformC0 = 0x40000000u;   // counter word 0 of the acceptance uniforms
constexpr double kNegInfD = -__builtin_huge_val();
// p_t - lam q_t is exactly <= 0 in float64 when ln(p_t / (lam q_t)) is below this margin
constexpr double kSkipMargin = -1e-9;

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
  int B, T, V, nch, R, maxc, max_depth, az, aq;
  double temp;
  uint32_t seed_lo, seed_hi, rnd;
  NodeSt* st;       // [T]
  int* cnt;         // [T] chunks finished in the current pass
  int* lists;       // [maxc + 1][T]: list m (2 .. maxc) waits for pass m; list 0 draws
  int* list_n;      // [maxc + 1]
  double* part;     // [T][nch][4]
  int* part_i;      // [T][nch]
  int* ydraw;       // [T] residual draw of a node
  int32_t* dev_status;
};

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
                           int npos_new) {
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
  const double px = exp((double)to_f32(zrow[x]) / a.temp - s.A);
  const double qx = exp((double)to_f32(qrow[x]) / a.temp - s.Bq);
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

__device__ __forceinline__ void enqueue(const SArgs& a, const NodeSt& s, int g) {
  if (s.status == ST_NEED) {
    const int at = atomicAdd(&a.list_n[s.m], 1);
    a.lists[(size_t)s.m * a.T + at] = g;
  } else if (s.status == ST_DRAW) {
    const int at = atomicAdd(&a.list_n[0], 1);
    a.lists[at] = g;
  }
}

// Count one finished chunk of node g; true in the workgroup that finished the last one.
__device__ __forceinline__ bool finish_chunk(const SArgs& a, int g, int* s_last) {
  if (threadIdx.x == 0) {
    __threadfence();
    const int old = atomicAdd(&a.cnt[g], 1);
    *s_last = old == a.nch - 1;
  }
  __syncthreads();
  const bool last = *s_last != 0;
  if (last) __threadfence();
  return last;
}

__global__ void k_samp_clear(int* cnt, int T, int* list_n, int nl) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < T) cnt[t] = 0;
  if (t < nl) list_n[t] = 0;
}

// Pass 1: both log-sum-exps of every node; the last chunk starts the node's chain.
template <typename TZ, typename TQ>
__global__ __launch_bounds__(256) void k_samp_stats(SArgs a) {
#pragma clang fp contract(off)
  __shared__ double sm[4][4];
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
  const bool has_q = r >= 0 && r < a.R;
  const TZ* zrow = (const TZ*)a.logits + (size_t)g * a.V;
  const TQ* qrow = (const TQ*)a.dlogits + (size_t)(has_q ? r : 0) * a.V;
  const int tb = c * SC + 16 * threadIdx.x;
  double ma = kNegInfD, sa = 0.0, mb = kNegInfD, sb = 0.0;
  if (tb < a.V) {
    const int ne = min(16, a.V - tb);
    float z[16];
    double v[16];
    load_chunk(zrow, tb, a.V, a.az, z);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      v[e] = (double)z[e] / a.temp;
      if (e < ne && v[e] > ma) ma = v[e];
    }
    sa = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (e < ne) sa = sa + exp(v[e] - ma);
    if (has_q) {
      load_chunk(qrow, tb, a.V, a.aq, z);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        v[e] = (double)z[e] / a.temp;
        if (e < ne && v[e] > mb) mb = v[e];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (e < ne) sb = sb + exp(v[e] - mb);
    }
  }
  wave_lse(ma, sa);
  wave_lse(mb, sb);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    sm[w][0] = ma;
    sm[w][1] = sa;
    sm[w][2] = mb;
    sm[w][3] = sb;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int q = 1; q < 4; ++q) {
      lse_add(ma, sa, sm[q][0], sm[q][1]);
      lse_add(mb, sb, sm[q][2], sm[q][3]);
    }
    double* p = a.part + ((size_t)g * a.nch + c) * 4;
    p[0] = ma;
    p[1] = sa;
    p[2] = mb;
    p[3] = sb;
  }
  if (!finish_chunk(a, g, &s_last)) return;
  const int nk = node_children(a, n0, n, i, s_kids, s_tok, s_cnt);
  if (threadIdx.x >= 64) return;
  double MA = kNegInfD, SA = 0.0, MB = kNegInfD, SB = 0.0;
  for (int cc = lane; cc < a.nch; cc += 64) {
    const double* p = a.part + ((size_t)g * a.nch + cc) * 4;
    lse_add(MA, SA, p[0], p[1]);
    lse_add(MB, SB, p[2], p[3]);
  }
  wave_lse(MA, SA);
  wave_lse(MB, SB);
  if (lane != 0) return;
  NodeSt s;
  s.A = MA + log(SA);
  s.Bq = has_q ? MB + log(SB) : 0.0;
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
  if (nk > 0 && !has_q && a.dev_status) atomicOr(a.dev_status, EAGLE3_DEV_BAD_ROW);
  for (int k = 0; k < nk; ++k)
    if ((s_tok[k] < 0 || s_tok[k] >= a.V) && a.dev_status) atomicOr(a.dev_status, EAGLE3_DEV_BAD_TOKEN);
  const int k0 = has_q ? next_valid(s_tok, nk, a.V, 0) : -1;
  if (k0 >= 0) {
    s.k = k0;
    s.m = 1;
    chain_step(a, s, s_kids, s_tok, b, zrow, qrow, false, 0.0, 0);
  }
  a.st[g] = s;
  a.cnt[g] = 0;
  enqueue(a, s, g);
}

// Pass m (2 .. maxc): N at the node's current lam, for the nodes on list m; the last chunk
// tests the waiting candidate.
template <typename TZ, typename TQ>
__global__ __launch_bounds__(256) void k_samp_npass(SArgs a, int m) {
#pragma clang fp contract(off)
  __shared__ double sd[4];
  __shared__ int si[4];
  __shared__ int s_kids[kMaxKids], s_tok[kMaxKids], s_cnt[4], s_last;
  const int items = a.list_n[m] * a.nch;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int g = a.lists[(size_t)m * a.T + it / a.nch];
    const int c = it % a.nch;
    const NodeSt s0 = a.st[g];
    const int r = a.draft_row[g];
    const TZ* zrow = (const TZ*)a.logits + (size_t)g * a.V;
    const TQ* qrow = (const TQ*)a.dlogits + (size_t)r * a.V;
    const double ln_lam = log(s0.lam);
    const int tb = c * SC + 16 * threadIdx.x;
    double acc = 0.0;
    int pos = 0;
    if (tb < a.V) {
      const int ne = min(16, a.V - tb);
      float z[16], zq[16];
      load_chunk(zrow, tb, a.V, a.az, z);
      load_chunk(qrow, tb, a.V, a.aq, zq);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (e >= ne) continue;
        const double la = (double)z[e] / a.temp - s0.A;
        const double lb = (double)zq[e] / a.temp - s0.Bq;
        const bool skip = la - lb - ln_lam < kSkipMargin;
        if (skip && m != 2) continue;
        const double eb = exp(lb);
        pos += eb > 0.0;
        if (skip) continue;
        const double d = exp(la) - s0.lam * eb;
        if (d > 0.0) acc = acc + d;
      }
    }
    acc = wave_sum_d(acc);
    pos = wave_sum_i(pos);
    if (lane == 0) {
      sd[w] = acc;
      si[w] = pos;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double t = sd[0];
      int pt = si[0];
      for (int q = 1; q < 4; ++q) {
        t = t + sd[q];
        pt += si[q];
      }
      a.part[((size_t)g * a.nch + c) * 4] = t;
      a.part_i[(size_t)g * a.nch + c] = pt;
    }
    if (finish_chunk(a, g, &s_last)) {
      const int b = find_request(a.cu_nodes, a.B, g);
      const int n0 = a.cu_nodes[b];
      const int n = min(a.cu_nodes[b + 1] - n0, kMaxNodes);
      node_children(a, n0, n, g - n0, s_kids, s_tok, s_cnt);
      if (threadIdx.x < 64) {
        double N = 0.0;
        int np = 0;
        for (int cc = lane; cc < a.nch; cc += 64) {
          N = N + a.part[((size_t)g * a.nch + cc) * 4];
          np += a.part_i[(size_t)g * a.nch + cc];
        }
        N = wave_sum_d(N);
        np = wave_sum_i(np);
        if (lane == 0) {
          NodeSt s = s0;
          chain_step(a, s, s_kids, s_tok, b, zrow, qrow, true, N, np);
          a.st[g] = s;
          a.cnt[g] = 0;
          enqueue(a, s, g);
        }
      }
    }
    __syncthreads();
  }
}

// Residual draw for the nodes on list 0: argmax over t of ln max(p_t - lam q_t, 0) + G_t
// (for lam = 0: ln p_t = z_t / T - A), G the node's Gumbel noise.
template <typename TZ, typename TQ>
__global__ __launch_bounds__(256) void k_samp_draw(SArgs a) {
#pragma clang fp contract(off)
  __shared__ double sv[4];
  __shared__ int sx[4];
  __shared__ int s_last;
  const int items = a.list_n[0] * a.nch;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int g = a.lists[it / a.nch];
    const int c = it % a.nch;
    const NodeSt s0 = a.st[g];
    const int b = find_request(a.cu_nodes, a.B, g);
    const uint32_t i_local = (uint32_t)(g - a.cu_nodes[b]);
    const bool plain = s0.lam == 0.0;
    const int r = plain ? 0 : a.draft_row[g];
    const TZ* zrow = (const TZ*)a.logits + (size_t)g * a.V;
    const TQ* qrow = (const TQ*)a.dlogits + (size_t)r * a.V;
    const double ln_lam = plain ? 0.0 : log(s0.lam);
    const int tb = c * SC + 16 * threadIdx.x;
    double best = kNegInfD;
    int bi = 0x7fffffff;
    if (tb < a.V) {
      float z[16], zq[16];
      load_chunk(zrow, tb, a.V, a.az, z);
      if (!plain) load_chunk(qrow, tb, a.V, a.aq, zq);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t ctr[4] = {(uint32_t)((tb >> 2) + q), i_local, (uint32_t)b, a.rnd};
        philox4x32_10(ctr, a.seed_lo, a.seed_hi);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = 4 * q + u, t = tb + e;
          if (t >= a.V) continue;
          const double la = (double)z[e] / a.temp - s0.A;
          double v;
          if (plain) {
            v = la;
          } else {
            const double lb = (double)zq[e] / a.temp - s0.Bq;
            if (la - lb - ln_lam < kSkipMargin) continue;
            const double d = exp(la) - s0.lam * exp(lb);
            if (!(d > 0.0)) continue;
            v = log(d);
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
      a.part[((size_t)g * a.nch + c) * 4] = best;
      a.part_i[(size_t)g * a.nch + c] = bi;
    }
    if (finish_chunk(a, g, &s_last) && threadIdx.x < 64) {
      double bv = kNegInfD;
      int bx = 0x7fffffff;
      for (int cc = lane; cc < a.nch; cc += 64) {
        const double v = a.part[((size_t)g * a.nch + cc) * 4];
        const int x = a.part_i[(size_t)g * a.nch + cc];
        if (better_d(v, x, bv, bx)) {
          bv = v;
          bx = x;
        }
      }
      wave_argmax_d(bv, bx);
      if (lane == 0) {
        a.ydraw[g] = bx < a.V ? bx : 0;
        a.cnt[g] = 0;
      }
    }
    __syncthreads();
  }
}

// Walk each request from its root through the kept children.
__global__ __launch_bounds__(64) void k_samp_walk(SArgs a, int32_t* accept_len, int32_t* path,
                                                  int32_t* out_tokens, int32_t* bonus) {
  if (threadIdx.x != 0) return;
  const int b = blockIdx.x;
  const int P = a.max_depth + 1;
  const int n0 = clampi(a.cu_nodes[b], 0, a.T);
  const int n1 = clampi(a.cu_nodes[b + 1], n0, a.T);
  int32_t* pth = path + (size_t)b * P;
  int32_t* out = out_tokens + (size_t)b * P;
  int s = 0, y = -1;
  if (n1 > n0) {
    int i = 0;
    pth[0] = 0;
    for (;;) {
      const NodeSt st = a.st[n0 + i];
      if (st.status == ST_KEPT && s < a.max_depth) {
        const int j = st.kept;
        ++s;
        pth[s] = j;
        out[s - 1] = a.tokens[n0 + j];
        i = j;
        continue;
      }
      y = st.status == ST_KEPT ? a.tokens[n0 + st.kept] : a.ydraw[n0 + i];
      break;
    }
    out[s] = y;
  }
  for (int k = n1 > n0 ? s + 1 : 0; k < P; ++k) {
    pth[k] = -1;
    out[k] = -1;
  }
  accept_len[b] = s;
  bonus[b] = y;
}

struct SampLayout {
  NodeSt* st;
  int *cnt, *lists, *list_n, *part_i, *ydraw;
  double* part;
};

SampLayout carve_sampled(void* ws, int T, int nch, int maxc) {
  e3h::Carve c(ws);
  SampLayout L;
  L.st = c.take<NodeSt>((size_t)T);
  L.cnt = c.take<int>((size_t)T);
  L.lists = c.take<int>((size_t)(maxc + 1) * T);
  L.list_n = c.take<int>((size_t)(maxc + 1));
  L.part = c.take<double>((size_t)T * nch * 4);
  L.part_i = c.take<int>((size_t)T * nch);
  L.ydraw = c.take<int>((size_t)T);
  return L;
}

template <typename TZ, typename TQ>
void launch_typed(const SArgs& a, int32_t* accept_len, int32_t* path, int32_t* out_tokens,
                  int32_t* bonus, hipStream_t s) {
  const int grid = (int)std::min<long>((long)a.T * a.nch, 2048);
  {
    e3h::ProfScope ps("sampled_stats", s);
    hipLaunchKernelGGL((k_samp_stats<TZ, TQ>), dim3((unsigned)((long)a.T * a.nch)), dim3(256), 0, s, a);
  }
  for (int m = 2; m <= a.maxc; ++m) {
    e3h::ProfScope ps("sampled_npass", s);
    hipLaunchKernelGGL((k_samp_npass<TZ, TQ>), dim3(grid), dim3(256), 0, s, a, m);
  }
  {
    e3h::ProfScope ps("sampled_draw", s);
    hipLaunchKernelGGL((k_samp_draw<TZ, TQ>), dim3(grid), dim3(256), 0, s, a);
  }
  e3h::ProfScope ps("sampled_walk", s);
  hipLaunchKernelGGL(k_samp_walk, dim3(a.B), dim3(64), 0, s, a, accept_len, path, out_tokens, bonus);
}

}  // namespace

namespace e3h {

size_t accept_sampled_workspace(int T, int V, int max_children) {
  const int nch = (V + SC - 1) / SC;
  Carve c(nullptr);
  c.take<NodeSt>((size_t)T);
  c.take<int>((size_t)T);
  c.take<int>((size_t)(max_children + 1) * T);
  c.take<int>((size_t)(max_children + 1));
  c.take<double>((size_t)T * nch * 4);
  c.take<int>((size_t)T * nch);
  c.take<int>((size_t)T);
  return c.size();
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
  const int nch = (V + SC - 1) / SC;
  const SampLayout L = carve_sampled(workspace, T, nch, max_children);
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
  a.R = draft_logits ? n_draft_rows : 0;
  a.maxc = max_children;
  a.max_depth = max_depth;
  a.az = ((size_t)V * elem_size(dtype)) % 16 == 0 && (uintptr_t)logits % 16 == 0;
  a.aq = draft_logits && ((size_t)V * elem_size(draft_dtype)) % 16 == 0 && (uintptr_t)draft_logits % 16 == 0;
  a.temp = (double)temperature;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.rnd = (uint32_t)round;
  a.st = L.st;
  a.cnt = L.cnt;
  a.lists = L.lists;
  a.list_n = L.list_n;
  a.part = L.part;
  a.part_i = L.part_i;
  a.ydraw = L.ydraw;
  a.dev_status = dev_status;
  {
    e3h::ProfScope ps("sampled_clear", s);
    const int nthreads = std::max(T, max_children + 1);
    hipLaunchKernelGGL(k_samp_clear, dim3((nthreads + 255) / 256), dim3(256), 0, s, L.cnt, T, L.list_n,
                       max_children + 1);
  }
  int st = launch_status();
  if (st) return st;
  const bool zb = dtype == EAGLE3_BF16;
  const bool qb = (draft_logits ? draft_dtype : dtype) == EAGLE3_BF16;
  if (zb && qb)
    launch_typed<bf16, bf16>(a, accept_len, path, out_tokens, bonus, s);
  else if (zb)
    launch_typed<bf16, float>(a, accept_len, path, out_tokens, bonus, s);
  else if (qb)
    launch_typed<float, bf16>(a, accept_len, path, out_tokens, bonus, s);
  else
    launch_typed<float, float>(a, accept_len, path, out_tokens, bonus, s);
  return launch_status();
}

}  // namespace e3h
