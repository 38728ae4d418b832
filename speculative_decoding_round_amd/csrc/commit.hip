// After acceptance: commit the accepted path's KV and rebuild the drafter's prefix KV of
// the committed positions from the target's real features.
//
//  * Commit ([P5] 一棵候选树怎样被验证, step 5: only the accepted path's KV is committed,
//    the other branches are released): for request b, tree rows cu_nodes[b] + path[b][i],
//    i = 0 .. accept_len[b] (root first), are copied to cache rows dst_row[b] + i.  Rows of
//    rejected branches are simply not copied.
//  * Drafter catch-up ([P3] 第二步为什么没有“正确隐藏状态”可用: a draft step reads the real
//    fused target feature only where the target has already run; once a position is
//    verified its real features exist): per committed position, the drafter's first-step
//    input is formed from the real features and its key (RoPE at the position) and value
//    are written into the drafter's prefix cache.  The arithmetic is the draft round's root
//    step: fusion GEMM, the same prep (RMSNorms in fp32, u in dtype), the K and V rows of
//    the QKV projection, the same RoPE.
#include "internal.h"

using namespace e3;

namespace {

// One workgroup per (path index i, request b): K and V rows of Hkv * Dh elements.
template <typename T>
__global__ __launch_bounds__(256) void k_commit_kv(int path_stride, int row_elems,
                                                   const int32_t* __restrict__ cu_nodes,
                                                   const int32_t* __restrict__ path,
                                                   const int32_t* __restrict__ accept_len,
                                                   const T* __restrict__ k_tree, const T* __restrict__ v_tree,
                                                   const int32_t* __restrict__ dst_row, long cache_rows,
                                                   T* __restrict__ k_cache, T* __restrict__ v_cache,
                                                   int32_t* __restrict__ dev_status) {
  const int i = blockIdx.x, b = blockIdx.y;
  int flags = 0;
  int a = accept_len[b];
  if (a < 0 || a >= path_stride) {
    flags |= EAGLE3_DEV_BAD_PATH;
    a = a < 0 ? -1 : path_stride - 1;
  }
  bool copy = i <= a;
  const int n0 = cu_nodes[b], nb = cu_nodes[b + 1] - n0;
  const int node = copy ? path[(size_t)b * path_stride + i] : 0;
  if (copy && (node < 0 || node >= nb)) {
    flags |= EAGLE3_DEV_BAD_PATH;
    copy = false;
  }
  const long dst = (long)dst_row[b] + i;
  if (copy && (dst < 0 || dst >= cache_rows)) {
    flags |= EAGLE3_DEV_BAD_ROW;
    copy = false;
  }
  if (flags && dev_status && threadIdx.x == 0) atomicOr(dev_status, flags);
  if (!copy) return;
  constexpr int EPC = Vec<T>::N;
  const size_t src = (size_t)(n0 + node) * row_elems, dr = (size_t)dst * row_elems;
  for (int e = threadIdx.x * EPC; e < row_elems; e += blockDim.x * EPC) {
    const u32x4 kv = ld16(k_tree + src + e);
    const u32x4 vv = ld16(v_tree + src + e);
    st16(k_cache + dr + e, kv);
    st16(v_cache + dr + e, vv);
  }
}

// xf[r] = [h_low[r]; h_mid[r]; h_high[r]]
template <typename T>
__global__ __launch_bounds__(256) void k_cu_concat(int d, const T* __restrict__ hl, const T* __restrict__ hm,
                                                   const T* __restrict__ hh, T* __restrict__ xf) {
  const size_t r = blockIdx.x;
  constexpr int EPC = Vec<T>::N;
  for (int k = threadIdx.x * EPC; k < d; k += blockDim.x * EPC) {
    st16(xf + r * 3 * d + k, ld16(hl + r * d + k));
    st16(xf + r * 3 * d + d + k, ld16(hm + r * d + k));
    st16(xf + r * 3 * d + 2 * d + k, ld16(hh + r * d + k));
  }
}

// Per row: g = sum of the fusion's k-split partials (split order), kept in fp32;
// u = [rms(E[x]) * g_e ; rms(g) * g_f] in dtype.  One thread per 8 elements.
template <typename T>
__global__ __launch_bounds__(1024) void k_cu_prep(int n, int d, int V, float eps, const int32_t* __restrict__ tok,
                                                  const T* __restrict__ embed, const T* __restrict__ g_e,
                                                  const T* __restrict__ g_f, const float* __restrict__ gpart,
                                                  int gsplits, float* __restrict__ g_out, T* __restrict__ u,
                                                  int32_t* __restrict__ dev_status) {
  __shared__ float red[32];
  const int r = blockIdx.x;
  const int t0 = tok[r];
  if (threadIdx.x == 0 && (t0 < 0 || t0 >= V) && dev_status) atomicOr(dev_status, EAGLE3_DEV_BAD_TOKEN);
  const int t = clampi(t0, 0, V - 1);
  const int k0 = threadIdx.x * 8;
  const bool act = k0 < d;
  float e[8], fv[8], ge[8], gf[8];
  float se = 0.f, sf = 0.f;
  if (act) {
    load8<T>(embed + (size_t)t * d + k0, e);
#pragma unroll
    for (int i = 0; i < 8; ++i) fv[i] = 0.f;
    for (int s = 0; s < gsplits; ++s) {
      float p[8];
      load8<float>(gpart + ((size_t)s * n + r) * d + k0, p);
#pragma unroll
      for (int i = 0; i < 8; ++i) fv[i] += p[i];
    }
    load8<T>(g_e + k0, ge);
    load8<T>(g_f + k0, gf);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      se += e[i] * e[i];
      sf += fv[i] * fv[i];
    }
  }
  block_sum2(se, sf, red);
  if (!act) return;
  const float ie = 1.f / sqrtf(se / d + eps);
  const float iff = 1.f / sqrtf(sf / d + eps);
  float o1[8], o2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    o1[i] = e[i] * ie * ge[i];
    o2[i] = fv[i] * iff * gf[i];
  }
  T* ur = u + (size_t)r * 2 * d;
  store8<T>(ur + k0, o1);
  store8<T>(ur + d + k0, o2);
  if (g_out) store8<float>(g_out + (size_t)r * d + k0, fv);
}

// Keys and values from the K/V rows of the QKV projection: sum of k-split partials, RoPE
// (half-split pairs, angle pos * theta^(-2i/Dh)) on the keys, written to the cache rows.
// One thread per (row, head, 4 consecutive pairs): 16-byte partial loads.
template <typename T>
__global__ __launch_bounds__(256) void k_cu_kv(const float* __restrict__ part, int splits, int n, int Hkv, int Dh,
                                               float theta, const int32_t* __restrict__ pos,
                                               const int32_t* __restrict__ dst_row, long cache_rows,
                                               T* __restrict__ k_cache, T* __restrict__ v_cache,
                                               int32_t* __restrict__ dev_status) {
  const int half = Dh / 2, q4 = half / 4;
  const int H = 2 * Hkv;
  const int N = H * Dh;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)n * H * q4) return;
  const int i0 = (int)(idx % q4) * 4;
  const int h = (int)((idx / q4) % H);
  const int m = (int)(idx / ((long)q4 * H));
  const long dst = dst_row[m];
  if (dst < 0 || dst >= cache_rows) {
    if (dev_status && i0 == 0 && h == 0) atomicOr(dev_status, EAGLE3_DEV_BAD_ROW);
    return;
  }
  floatx4 y1 = {0.f, 0.f, 0.f, 0.f}, y2 = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < splits; ++s) {
    const float* p = part + ((size_t)s * n + m) * N + h * Dh + i0;
    y1 += *reinterpret_cast<const floatx4*>(p);
    y2 += *reinterpret_cast<const floatx4*>(p + half);
  }
  if (h < Hkv) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double ang = (double)pos[m] * pow((double)theta, -2.0 * (i0 + e) / Dh);
      double sn, cn;
      sincos(ang, &sn, &cn);
      const float c = (float)cn, sv = (float)sn;
      const float o1 = y1[e] * c - y2[e] * sv;
      const float o2 = y1[e] * sv + y2[e] * c;
      y1[e] = o1;
      y2[e] = o2;
    }
  }
  T* base = h < Hkv ? k_cache : v_cache;
  T* out = base + ((size_t)dst * Hkv + (h < Hkv ? h : h - Hkv)) * Dh + i0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[e] = from_f32<T>(y1[e]);
    out[e + half] = from_f32<T>(y2[e]);
  }
}

struct CatchupPlan {
  e3h::GemmPlan gf, gk;
  void* xf;
  float* gpart;
  void* u;
  float* kvpart;
  size_t bytes;
};

CatchupPlan plan_catchup(const eagle3_drafter* w, int n, void* ws) {
  CatchupPlan p;
  const int d = w->d, dt = w->dtype, es = e3h::elem_size(dt);
  const int nkv = 2 * w->n_heads_kv * w->head_dim;
  p.gf = e3h::plan_gemm(n, d, 3 * d, dt);
  p.gk = e3h::plan_gemm(n, nkv, 2 * d, dt);
  e3h::Carve c(ws);
  p.xf = c.take<char>((size_t)n * 3 * d * es);
  p.gpart = c.take<float>((size_t)p.gf.splits * n * d);
  p.u = c.take<char>((size_t)n * 2 * d * es);
  p.kvpart = c.take<float>((size_t)p.gk.splits * n * nkv);
  p.bytes = c.size();
  return p;
}

bool gemm_supported(const e3h::GemmPlan& p) { return p.tile || (p.MT != 0 && p.M <= 160); }

}  // namespace

namespace e3h {

int launch_commit_kv(int B, int row_elems, int dtype, int path_stride, const int32_t* cu_nodes,
                     const int32_t* path, const int32_t* accept_len, const void* k_tree,
                     const void* v_tree, const int32_t* dst_row, long cache_rows, void* k_cache,
                     void* v_cache, int32_t* dev_status, hipStream_t s) {
  ProfScope ps("commit_kv", s);
  const dim3 grid(path_stride, B);
  if (dtype == EAGLE3_BF16)
    hipLaunchKernelGGL(k_commit_kv<bf16>, grid, dim3(256), 0, s, path_stride, row_elems, cu_nodes, path,
                       accept_len, (const bf16*)k_tree, (const bf16*)v_tree, dst_row, cache_rows,
                       (bf16*)k_cache, (bf16*)v_cache, dev_status);
  else
    hipLaunchKernelGGL(k_commit_kv<float>, grid, dim3(256), 0, s, path_stride, row_elems, cu_nodes, path,
                       accept_len, (const float*)k_tree, (const float*)v_tree, dst_row, cache_rows,
                       (float*)k_cache, (float*)v_cache, dev_status);
  return launch_status();
}

size_t catchup_workspace(const eagle3_drafter* w, int n) { return plan_catchup(w, n, nullptr).bytes; }

int catchup_supported(const eagle3_drafter* w, int n) {
  const CatchupPlan p = plan_catchup(w, n, nullptr);
  return gemm_supported(p.gf) && gemm_supported(p.gk);
}

template <typename T>
int run_catchup(const eagle3_drafter* w, int n, const int32_t* tokens, const int32_t* pos, const void* h_low,
                const void* h_mid, const void* h_high, const int32_t* dst_row, long cache_rows, void* k_cache,
                void* v_cache, float* g_out, int32_t* dev_status, void* ws, hipStream_t s) {
  const CatchupPlan p = plan_catchup(w, n, ws);
  const int d = w->d, dt = w->dtype;
  const int Hq = w->n_heads_q, Hkv = w->n_heads_kv, Dh = w->head_dim;
  int st;
  {
    ProfScope ps("catchup_concat", s);
    hipLaunchKernelGGL(k_cu_concat<T>, dim3(n), dim3(256), 0, s, d, (const T*)h_low, (const T*)h_mid,
                       (const T*)h_high, (T*)p.xf);
    if ((st = launch_status())) return st;
  }
  if ((st = launch_gemm(p.gf, dt, p.xf, 3 * d, w->w_fuse, p.gpart, s, "catchup_fuse"))) return st;
  {
    ProfScope ps("catchup_prep", s);
    hipLaunchKernelGGL(k_cu_prep<T>, dim3(n), dim3(((d / 8 + 63) / 64) * 64), 0, s, n, d, w->vocab, w->eps,
                       tokens, (const T*)w->embed, (const T*)w->g_embed, (const T*)w->g_feat, p.gpart,
                       p.gf.splits, g_out, (T*)p.u, dev_status);
    if ((st = launch_status())) return st;
  }
  const T* w_kv = (const T*)w->w_qkv + (size_t)Hq * Dh * 2 * d;   // the K rows, then the V rows
  if ((st = launch_gemm(p.gk, dt, p.u, 2 * d, w_kv, p.kvpart, s, "catchup_kv"))) return st;
  ProfScope ps("catchup_rope", s);
  const long total = (long)n * 2 * Hkv * (Dh / 8);
  hipLaunchKernelGGL(k_cu_kv<T>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p.kvpart, p.gk.splits,
                     n, Hkv, Dh, w->rope_theta, pos, dst_row, cache_rows, (T*)k_cache, (T*)v_cache,
                     dev_status);
  return launch_status();
}

int launch_catchup(const eagle3_drafter* w, int n, const int32_t* tokens, const int32_t* pos, const void* h_low,
                   const void* h_mid, const void* h_high, const int32_t* dst_row, long cache_rows, void* k_cache,
                   void* v_cache, float* g_out, int32_t* dev_status, void* ws, hipStream_t s) {
  if (w->dtype == EAGLE3_BF16)
    return run_catchup<bf16>(w, n, tokens, pos, h_low, h_mid, h_high, dst_row, cache_rows, k_cache, v_cache,
                             g_out, dev_status, ws, s);
  return run_catchup<float>(w, n, tokens, pos, h_low, h_mid, h_high, dst_row, cache_rows, k_cache, v_cache,
                            g_out, dev_status, ws, s);
}

}  // namespace e3h
