// Weight-streaming GEMM for the drafter's projections and LM head:
//   Y_part[split][m][n] = sum_{k in split} X[m][k] * W[n][k]
// X is [M, K] (a handful of rows: the nodes being evaluated), W is [N, K] row-major.
// The op is bound by streaming W from HBM once, so the layout puts W on the MFMA A operand
// (16 output features per tile), keeps every byte of W read exactly once, and spreads the
// work over (n-block, k-split) workgroups of four waves.  Each wave walks its own k-range,
// holding NT W-tiles and MT X-tiles per 16-byte chunk step; the four waves' partial tiles
// are summed in LDS in wave order, so results are deterministic.
#include "common.h"
#include "internal.h"

using namespace e3;

namespace {

constexpr int WAVES = 4;
constexpr int U = 4;  // chunk steps loaded ahead per iteration

template <typename T, int MT, int NT>
__global__ __launch_bounds__(256) void k_gemm(const T* __restrict__ X, int M, int ldx,
                                              const T* __restrict__ W, int N, int K,
                                              float* __restrict__ Y, int n_blocks,
                                              int chunks_total, int chunks_per_split) {
  constexpr int EPC = Vec<T>::N;
  constexpr int KPC = Mfma<T>::KPC;  // = 4 * EPC
  __shared__ floatx4 red[WAVES][NT * MT][64];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int nb = blockIdx.x % n_blocks, ks = blockIdx.x / n_blocks;
  const int cs0 = ks * chunks_per_split;
  const int cs1 = min(chunks_total, cs0 + chunks_per_split);
  const int per_wave = (cs1 - cs0 + WAVES - 1) / WAVES;
  const int c0 = cs0 + wid * per_wave;
  const int c1 = min(cs1, c0 + per_wave);

  const T* wrow[NT];
  bool wok[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = (nb * NT + nt) * 16 + r16;
    wok[nt] = n < N;
    wrow[nt] = W + (size_t)(wok[nt] ? n : 0) * K + g * EPC;
  }
  const T* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + r16;
    xok[mt] = m < M;
    xrow[mt] = X + (size_t)(xok[mt] ? m : 0) * ldx + g * EPC;
  }

  floatx4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  const u32x4 zero = {0, 0, 0, 0};
  for (int c = c0; c < c1; c += U) {
    u32x4 wv[U][NT], xv[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kc = c + u;
      const int koff = kc * KPC;
      const bool kin = kc < c1 && koff + g * EPC + EPC <= K;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) wv[u][nt] = (kin && wok[nt]) ? ld16(wrow[nt] + koff) : zero;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xv[u][mt] = (kin && xok[mt]) ? ld16(xrow[mt] + koff) : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = Mfma<T>::run(wv[u][nt], xv[u][mt], acc[nt][mt]);
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[wid][nt * MT + mt][lane] = acc[nt][mt];
  __syncthreads();
  // sum the four waves' tiles in wave order; write 4 consecutive n per (tile, lane)
  float* Ys = Y + (size_t)ks * M * N;
  for (int e = threadIdx.x; e < NT * MT * 64; e += 256) {
    const int tile = e / 64, ln = e % 64;
    const int nt = tile / MT, mt = tile % MT;
    floatx4 v = red[0][tile][ln];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) v += red[w][tile][ln];
    const int m = mt * 16 + (ln & 15);
    const int n = (nb * NT + nt) * 16 + 4 * (ln >> 4);
    if (m < M && n < N) *reinterpret_cast<floatx4*>(Ys + (size_t)m * N + n) = v;
  }
}

// out[m][n] = (resid ? resid[m][n] : 0) + sum_s part[s][m][n]
__global__ __launch_bounds__(256) void k_epi_sum(const float* __restrict__ part, int S, int M, int N,
                                                 float* __restrict__ out,
                                                 const float* __restrict__ resid) {
  const long i4 = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total = (long)M * N / 4;
  if (i4 >= total) return;
  floatx4 v = resid ? reinterpret_cast<const floatx4*>(resid)[i4] : floatx4{0.f, 0.f, 0.f, 0.f};
  floatx4 t = reinterpret_cast<const floatx4*>(part)[i4];
  for (int s = 1; s < S; ++s) t += reinterpret_cast<const floatx4*>(part + (size_t)s * M * N)[i4];
  v += t;
  reinterpret_cast<floatx4*>(out)[i4] = v;
}

// gate/up: N = 2F; out[m][j] = silu(y[m][j]) * y[m][F + j]
template <typename T>
__global__ __launch_bounds__(256) void k_epi_silu_mul(const float* __restrict__ part, int S, int M,
                                                      int N, T* __restrict__ out) {
  const int F = N / 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)M * F) return;
  const int m = (int)(idx / F), j = (int)(idx % F);
  float gt = 0.f, up = 0.f;
  for (int s = 0; s < S; ++s) {
    gt += part[((size_t)s * M + m) * N + j];
    up += part[((size_t)s * M + m) * N + F + j];
  }
  const float act = gt / (1.f + expf(-gt));
  out[(size_t)m * F + j] = from_f32<T>(act * up);
}

template <typename T, int MT, int NT>
void launch_gemm_t(const e3h::GemmPlan& p, const void* X, int ldx, const void* W, float* Y,
                   hipStream_t s) {
  dim3 grid(p.n_blocks * p.splits);
  hipLaunchKernelGGL((k_gemm<T, MT, NT>), grid, dim3(256), 0, s, (const T*)X, p.M, ldx,
                     (const T*)W, p.N, p.K, Y, p.n_blocks, p.chunks_total, p.chunks_per_split);
}

template <typename T>
int dispatch_gemm(const e3h::GemmPlan& p, const void* X, int ldx, const void* W, float* Y,
                  hipStream_t s) {
#define E3_CASE(mt, nt)                                   \
  if (p.MT == mt && p.NT == nt) {                         \
    launch_gemm_t<T, mt, nt>(p, X, ldx, W, Y, s);         \
    return e3h::launch_status();                          \
  }
  E3_CASE(1, 1) E3_CASE(1, 2) E3_CASE(2, 1) E3_CASE(2, 2) E3_CASE(3, 1) E3_CASE(4, 1)
  E3_CASE(6, 1) E3_CASE(8, 1) E3_CASE(10, 1)
#undef E3_CASE
  return EAGLE3_EUNSUPPORTED;
}

}  // namespace

namespace e3h {

GemmPlan plan_gemm(int M, int N, int K, int dtype) {
  GemmPlan p;
  p.M = M;
  p.N = N;
  p.K = K;
  const int mt_need = (M + 15) / 16;
  static const int mts[] = {1, 2, 3, 4, 6, 8, 10};
  p.MT = 0;
  for (int v : mts)
    if (v >= mt_need) {
      p.MT = v;
      break;
    }
  const int ntile = (N + 15) / 16;
  p.NT = (p.MT <= 2 && ntile >= 4096) ? 2 : 1;
  p.n_blocks = (ntile + p.NT - 1) / p.NT;
  const int kpc = dtype == EAGLE3_BF16 ? 32 : 16;
  p.chunks_total = (K + kpc - 1) / kpc;
  // enough workgroups to keep every CU streaming, but at least 8 chunk steps per wave
  const int target = 1024;
  int splits = (target + p.n_blocks - 1) / p.n_blocks;
  const int max_splits = p.chunks_total / (WAVES * 8) > 0 ? p.chunks_total / (WAVES * 8) : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  p.chunks_per_split = (p.chunks_total + splits - 1) / splits;
  p.splits = (p.chunks_total + p.chunks_per_split - 1) / p.chunks_per_split;
  p.waves = WAVES;
  return p;
}

int launch_gemm(const GemmPlan& p, int dtype, const void* X, int ldx, const void* W, float* Ypart,
                hipStream_t s, const char* tag) {
  if (p.MT == 0) return EAGLE3_EUNSUPPORTED;
  ProfScope ps(tag, s);
  if (dtype == EAGLE3_BF16) return dispatch_gemm<bf16>(p, X, ldx, W, Ypart, s);
  return dispatch_gemm<float>(p, X, ldx, W, Ypart, s);
}

int launch_epi_sum(const GemmPlan& p, const float* part, float* out, const float* resid,
                   hipStream_t s, const char* tag) {
  ProfScope ps(tag, s);
  const long total = (long)p.M * p.N / 4;
  hipLaunchKernelGGL(k_epi_sum, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part,
                     p.splits, p.M, p.N, out, resid);
  return launch_status();
}

int launch_epi_silu_mul(const GemmPlan& p, const float* part, int dtype, void* out, hipStream_t s,
                        const char* tag) {
  ProfScope ps(tag, s);
  const long total = (long)p.M * (p.N / 2);
  dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == EAGLE3_BF16)
    hipLaunchKernelGGL(k_epi_silu_mul<bf16>, grid, dim3(256), 0, s, part, p.splits, p.M, p.N,
                       (bf16*)out);
  else
    hipLaunchKernelGGL(k_epi_silu_mul<float>, grid, dim3(256), 0, s, part, p.splits, p.M, p.N,
                       (float*)out);
  return launch_status();
}

}  // namespace e3h
