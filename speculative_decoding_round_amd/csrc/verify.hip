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
// ---------------------------------------------------------------------------------------
constexpr int ACC_CHUNK = 4096;

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
  } else if (tb < V) {
    const int b = find_request(cu_nodes, B, node);
    const uint32_t i_local = (uint32_t)(node - cu_nodes[b]);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t ctr[4] = {(uint32_t)((tb >> 2) + q), i_local, (uint32_t)b, rnd};
      philox4x32_10(ctr, seed_lo, seed_hi);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int t = tb + 4 * q + w;
        if (t >= V) continue;
        const float val = z[4 * q + w] * invT + gumbel_from_word(ctr[w]);
        if (better(val, t, best, bi)) {
          best = val;
          bi = t;
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
