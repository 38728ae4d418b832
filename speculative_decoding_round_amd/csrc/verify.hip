// Tree packing (ancestor bitmask, depth, position) and acceptance kernels.
#include "common.h"
#include "internal.h"

using namespace e3;

namespace {

// ---------------------------------------------------------------------------------------
// Tree mask.  One workgroup per request, one thread per node: walk the parent pointers to
// the root, setting one bit per node on the way.  parent[i] < i bounds every walk by i
// steps; a parent outside [0, i) is flagged and treated as the root so the walk ends.
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_build_mask(const int32_t* __restrict__ cu_nodes,
                                                    const int32_t* __restrict__ parents,
                                                    const int32_t* __restrict__ cu_prefix,
                                                    int T, uint64_t* __restrict__ mask, int W64,
                                                    int32_t* __restrict__ depth_out,
                                                    int32_t* __restrict__ pos_out,
                                                    int32_t* __restrict__ dev_status) {
  const int b = blockIdx.x;
  const int n0 = clampi(cu_nodes[b], 0, T);
  const int n1 = clampi(cu_nodes[b + 1], n0, T);
  const int n = n1 - n0;
  const int P = cu_prefix ? cu_prefix[b + 1] - cu_prefix[b] : 0;
  const int cap = 64 * W64;
  int flags = 0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    uint64_t* row = mask + (size_t)(n0 + i) * W64;
    for (int w = 0; w < W64; ++w) row[w] = 0ull;
    if (i >= cap) {
      flags |= EAGLE3_DEV_TOO_DEEP;
      if (depth_out) depth_out[n0 + i] = -1;
      if (pos_out) pos_out[n0 + i] = -1;
      continue;
    }
    int j = i, dep = 0;
    while (true) {
      row[j >> 6] |= 1ull << (j & 63);
      if (j == 0) break;
      int p = parents[n0 + j];
      if (p < 0 || p >= j) {
        flags |= EAGLE3_DEV_BAD_PARENT;
        p = 0;
      }
      ++dep;
      j = p;
    }
    if (i == 0 && parents[n0] != -1) flags |= EAGLE3_DEV_BAD_PARENT;
    if (depth_out) depth_out[n0 + i] = dep;
    if (pos_out) pos_out[n0 + i] = P + dep;
  }
  if (flags && dev_status) atomicOr(dev_status, flags);
}

// ---------------------------------------------------------------------------------------
// Acceptance pass 1: per (node, chunk of 4096 tokens) the best (value, token) of greedy z
// or z*invT + Gumbel.  Thread t takes 16 consecutive tokens (vector loads issued together
// when the row is 16-byte aligned); one Philox call yields the noise of four tokens.
//
// At T > 0 most of the Gumbel noise is never needed: G(u) = -ln(-ln u) rises with u, and a
// word whose 23-bit cell index k = x >> 9 has L leading ones has 1 - u >= 2^-(L+1), so
// -ln u > 1 - u >= 2^-(L+1) and G < (L+1) ln 2.  With a margin of 2^-10 over that (far above the
// rounding of the two logarithms), U = z*invT + G_bound(L) bounds the token's value (the same
// rounded addition, with a larger addend).  Each lane computes the exact value of its token
// with the largest bound; every token whose bound lies below the wave's best exact value
// cannot win the chunk (it stays strictly below a value the chunk attains), and the few
// remaining tokens are compacted across the wave (through LDS) so that their logarithms are
// evaluated by whole waves rather than by scattered lanes.  The winner is the same token as
// with every value computed.
// ---------------------------------------------------------------------------------------
constexpr int ACC_CHUNK = 4096;
constexpr int ACC_EXACT_CAP = 256;   // compacted tokens per wave; beyond, every token is evaluated

// Upper bound of gumbel_from_word(x) from the leading ones of x's top 23 bits.
__device__ __forceinline__ float gumbel_bound(uint32_t x) {
#pragma clang fp contract(off)
  const int ones = min(23, (int)__clz(~x));
  return (float)(ones + 1) * 0.693147182f + 0.0009765625f;
}

template <typename T>
__global__ __launch_bounds__(256) void k_accept_scan(const T* __restrict__ logits, int V, int n_chunks,
                                                     int aligned, const int32_t* __restrict__ cu_nodes,
                                                     int B, int greedy, float invT, uint32_t seed_lo,
                                                     uint32_t seed_hi, uint32_t rnd,
                                                     float* __restrict__ part_v,
                                                     int* __restrict__ part_i) {
#pragma clang fp contract(off)
  constexpr int EPC = Vec<T>::N;
  __shared__ float sv[8];
  __shared__ int si[8];
  __shared__ float s_xa[4][ACC_EXACT_CAP];
  __shared__ uint32_t s_xw[4][ACC_EXACT_CAP];
  __shared__ int s_xt[4][ACC_EXACT_CAP];
  const int node = blockIdx.x / n_chunks;
  const int c = blockIdx.x % n_chunks;
  const int tb = c * ACC_CHUNK + 16 * threadIdx.x;
  const T* row = logits + (size_t)node * V;
  float z[16];
  if (aligned && tb + 16 <= V) {
#pragma unroll
    for (int q = 0; q < 16 / EPC; ++q) {
      const u32x4 v = ld16(row + tb + q * EPC);
#pragma unroll
      for (int e = 0; e < EPC; ++e) z[q * EPC + e] = chunk_elem<T>(v, e);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = tb + e < V ? to_f32(row[tb + e]) : kNegInf;
  }
  float best = kNegInf;
  int bi = 0x7fffffff;
  if (greedy) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (tb + e < V && better(z[e], tb + e, best, bi)) {
        best = z[e];
        bi = tb + e;
      }
  } else {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint32_t wd[16] = {};
    float a[16], ub[16];
    if (tb < V) {
      const int b = find_request(cu_nodes, B, node);
      const uint32_t i_local = (uint32_t)(node - cu_nodes[b]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t ctr[4] = {(uint32_t)((tb >> 2) + q), i_local, (uint32_t)b, rnd};
        philox4x32_10(ctr, seed_lo, seed_hi);
#pragma unroll
        for (int w = 0; w < 4; ++w) wd[4 * q + w] = ctr[w];
      }
    }
    // the bounds, and the exact value of the lane's token with the largest one
    float utop = kNegInf, atop = 0.f;
    uint32_t wtop = 0;
    int etop = -1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const bool in = tb + e < V;
      a[e] = z[e] * invT;
      ub[e] = in ? a[e] + gumbel_bound(wd[e]) : kNegInf;
      if (in & (etop < 0 || ub[e] > utop)) {
        utop = ub[e];
        atop = a[e];
        wtop = wd[e];
        etop = e;
      }
    }
    if (etop >= 0) {
      best = atop + gumbel_from_word(wtop);
      bi = tb + etop;
    }
    const float th = wave_max(best);
    // tokens that may still reach th, compacted over the wave
    float* xa = s_xa[wv];
    uint32_t* xw = s_xw[wv];
    int* xt = s_xt[wv];
    const uint64_t below = (1ull << lane) - 1ull;
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const bool need = (tb + e < V) & (e != etop) & (ub[e] >= th);
      const uint64_t bal = __ballot(need);
      if (bal) {
        const int pos = cnt + __popcll(bal & below);
        if (need & (pos < ACC_EXACT_CAP)) {
          xa[pos] = a[e];
          xw[pos] = wd[e];
          xt[pos] = tb + e;
        }
        cnt += __popcll(bal);
      }
    }
    if (cnt <= ACC_EXACT_CAP) {
      __builtin_amdgcn_wave_barrier();
      for (int j = lane; j < cnt; j += 64) {
        const float val = xa[j] + gumbel_from_word(xw[j]);
        if (better(val, xt[j], best, bi)) {
          best = val;
          bi = xt[j];
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if ((tb + e < V) & (e != etop) & (ub[e] >= th)) {
          const float val = a[e] + gumbel_from_word(wd[e]);
          if (better(val, tb + e, best, bi)) {
            best = val;
            bi = tb + e;
          }
        }
      }
    }
  }
  block_argmax(best, bi, sv, si);
  if (threadIdx.x == 0) {
    part_v[(size_t)node * n_chunks + c] = best;
    part_i[(size_t)node * n_chunks + c] = bi;
  }
}

// ---------------------------------------------------------------------------------------
// Acceptance pass 2: one workgroup per request.  Reduce the chunk winners to y_i per node,
// form the match bits, find the deepest node whose ancestors-or-self all match, emit path.
// ---------------------------------------------------------------------------------------
constexpr int kMaxW64 = 4;

__global__ __launch_bounds__(256) void k_accept_path(
    const float* __restrict__ part_v, const int* __restrict__ part_i, int n_chunks,
    const int32_t* __restrict__ cu_nodes, int T, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ parents, const uint64_t* __restrict__ mask, int W64,
    int max_depth, int32_t* __restrict__ accept_len, int32_t* __restrict__ path,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ bonus) {
  __shared__ int y[64 * kMaxW64];
  __shared__ unsigned long long match[kMaxW64];
  __shared__ float sv[8];
  __shared__ int si[8];
  const int b = blockIdx.x;
  const int n0 = clampi(cu_nodes[b], 0, T);
  const int n1 = clampi(cu_nodes[b + 1], n0, T);
  const int n = min(n1 - n0, 64 * W64);
  if (n <= 0) {  // empty request: nothing accepted, no bonus
    for (int k = threadIdx.x; k <= max_depth; k += blockDim.x) {
      path[(size_t)b * (max_depth + 1) + k] = -1;
      out_tokens[(size_t)b * (max_depth + 1) + k] = -1;
    }
    if (threadIdx.x == 0) {
      accept_len[b] = 0;
      bonus[b] = -1;
    }
    return;
  }
  for (int w = threadIdx.x; w < W64; w += blockDim.x) match[w] = 0ull;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const float* pv = part_v + (size_t)(n0 + i) * n_chunks;
    const int* pi = part_i + (size_t)(n0 + i) * n_chunks;
    float bv = kNegInf;
    int bi = 0x7fffffff;
    for (int c0 = 0; c0 < n_chunks; c0 += 8) {
      float v8[8];
      int i8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        v8[u] = c0 + u < n_chunks ? pv[c0 + u] : kNegInf;
        i8[u] = c0 + u < n_chunks ? pi[c0 + u] : 0x7fffffff;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (better(v8[u], i8[u], bv, bi)) {
          bv = v8[u];
          bi = i8[u];
        }
    }
    y[i] = bi;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    bool m;
    if (i == 0) {
      m = true;
    } else {
      int p = parents[n0 + i];
      p = (p < 0 || p >= i) ? 0 : p;
      m = tokens[n0 + i] == y[p];
    }
    if (m) atomicOr(&match[i >> 6], 1ull << (i & 63));
  }
  __syncthreads();
  // deepest fully-matching node; ties to the lowest index
  float key = kNegInf;
  int idx = 0x7fffffff;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint64_t* row = mask + (size_t)(n0 + i) * W64;
    bool ok = true;
    int pc = 0;
    for (int w = 0; w < W64; ++w) {
      ok = ok && ((row[w] & ~match[w]) == 0ull);
      pc += __popcll(row[w]);
    }
    if (ok && better((float)(pc - 1), i, key, idx)) {
      key = (float)(pc - 1);
      idx = i;
    }
  }
  block_argmax(key, idx, sv, si);
  if (threadIdx.x == 0) {
    const int L = (int)key;
    const uint64_t* row = mask + (size_t)(n0 + idx) * W64;
    int s = 0;
    for (int w = 0; w < W64; ++w) {
      uint64_t bits = row[w];
      while (bits && s <= max_depth) {
        const int j = w * 64 + __ffsll((unsigned long long)bits) - 1;
        bits &= bits - 1;
        path[(size_t)b * (max_depth + 1) + s] = j;
        if (s >= 1) out_tokens[(size_t)b * (max_depth + 1) + s - 1] = tokens[n0 + j];
        ++s;
      }
    }
    for (int k = s; k <= max_depth; ++k) path[(size_t)b * (max_depth + 1) + k] = -1;
    const int Lc = min(L, max_depth);
    out_tokens[(size_t)b * (max_depth + 1) + Lc] = y[idx];
    for (int k = Lc + 1; k <= max_depth; ++k) out_tokens[(size_t)b * (max_depth + 1) + k] = -1;
    accept_len[b] = L;
    bonus[b] = y[idx];
  }
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------------------
namespace e3h {

int launch_build_mask(int B, int T, const int32_t* cu_nodes, const int32_t* parents,
                      const int32_t* cu_prefix, uint64_t* mask, int W64, int32_t* depth,
                      int32_t* pos, int32_t* dev_status, hipStream_t s) {
  ProfScope ps("build_tree_mask", s);
  hipLaunchKernelGGL(k_build_mask, dim3(B), dim3(64), 0, s, cu_nodes, parents, cu_prefix, T,
                     mask, W64, depth, pos, dev_status);
  return launch_status();
}

int accept_chunks(int V) { return (V + ACC_CHUNK - 1) / ACC_CHUNK; }

int launch_accept(int B, int T, const int32_t* cu_nodes, const int32_t* tokens,
                  const int32_t* parents, const uint64_t* mask, int W64, const void* logits,
                  int V, int dtype, float temperature, uint64_t seed, uint64_t round,
                  int max_depth, int32_t* accept_len, int32_t* path, int32_t* out_tokens,
                  int32_t* bonus, float* part_v, int* part_i, hipStream_t s) {
  if (W64 > kMaxW64) return EAGLE3_EUNSUPPORTED;
  const int n_chunks = accept_chunks(V);
  const int greedy = temperature == 0.0f;
  const float invT = greedy ? 1.0f : 1.0f / temperature;
  const uint32_t slo = (uint32_t)seed, shi = (uint32_t)(seed >> 32), rnd = (uint32_t)round;
  const int es = dtype == EAGLE3_BF16 ? 2 : 4;
  const int aligned = ((size_t)V * es) % 16 == 0 && ((uintptr_t)logits % 16) == 0;
  {
    ProfScope ps("accept_scan", s);
    dim3 grid((unsigned)((long)n_chunks * T));
    if (dtype == EAGLE3_BF16)
      hipLaunchKernelGGL(k_accept_scan<bf16>, grid, dim3(256), 0, s, (const bf16*)logits, V, n_chunks,
                         aligned, cu_nodes, B, greedy, invT, slo, shi, rnd, part_v, part_i);
    else
      hipLaunchKernelGGL(k_accept_scan<float>, grid, dim3(256), 0, s, (const float*)logits, V,
                         n_chunks, aligned, cu_nodes, B, greedy, invT, slo, shi, rnd, part_v, part_i);
  }
  int st = launch_status();
  if (st) return st;
  ProfScope ps("accept_path", s);
  hipLaunchKernelGGL(k_accept_path, dim3(B), dim3(256), 0, s, part_v, part_i, n_chunks, cu_nodes, T,
                     tokens, parents, mask, W64, max_depth, accept_len, path, out_tokens, bonus);
  return launch_status();
}

size_t accept_workspace(int T, int V) {
  const int n_chunks = accept_chunks(V);
  Carve c(nullptr);
  c.take<float>((size_t)T * n_chunks);
  c.take<int>((size_t)T * n_chunks);
  return c.size();
}

}  // namespace e3h
