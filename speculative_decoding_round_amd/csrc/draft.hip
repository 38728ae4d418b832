// One draft-tree round: feature fusion, D evaluation steps of the single-layer drafter
// over the growing tree, and on-device tree selection.  All shapes are static, so the
// host enqueues a fixed sequence of launches and never waits on the device.
//
// Row layout: at step 0 row b is request b's root; at step t >= 1 row b*W + j is the j-th
// node evaluated at depth t (evaluation slot 1 + (t-1)*W + j).  Slots that receive no node
// (fewer candidates than W) are computed as padding and ignored.
#include "common.h"
#include "internal.h"

using namespace e3;

namespace {

typedef int intx4 __attribute__((ext_vector_type(4)));

constexpr int KMAX = 16;     // largest top-K
constexpr int SMAX = 256;    // largest slot count (four mask words)

struct SlotState {
  int32_t* tok;      // [B*S]
  int32_t* parent;   // [B*S]  -1 root, -2 unused
  int32_t* valid;    // [B*S]
  float* score;      // [B*S]
  uint64_t* mask;    // [B*S, mw]  ancestors-or-self over slots, bit s of word s / 64
  int32_t* cand;     // [B*S]  candidate index of the slot's node (-1 root)
  int mw;            // mask words per slot: ceil(S / 64)
};
struct CandState {
  int32_t* tok;      // [B*PMAX]
  int32_t* pslot;    // [B*PMAX]
  int32_t* depth;    // [B*PMAX]
  float* score;      // [B*PMAX]
  int32_t* count;    // [B]
  int32_t* topn;     // [B*N]  the N best candidates so far (candidate index), best first
  float* topsc;      // [B*N]  their scores
  int32_t* ntop;     // [B]
};

// Sampled drafting: children are drawn without replacement from softmax(z / T) by ranking
// z * invT plus Gumbel noise (counter (t>>2, 0x80000000 | slot, b, round), word t & 3), the
// log-sum-exp is that of z * invT, and every evaluated slot's logits are kept for the
// verifier, with the node -> slot row map of the final tree.
struct SampCfg {
  int on;
  float invT;
  uint32_t seed_lo, seed_hi, rnd;
  int V;
  float* slot_logits;     // [B * S, V] fp32
  int32_t* draft_row;     // [B, N + 1]
};

// ---------------------------------------------------------------------------------------
// init: slot 0 = root, every other slot unused; concatenated fusion input.
// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_init(int /*B*/, int S, int d, int V, const int32_t* __restrict__ root_tok,
                                              SlotState st, CandState cs, const T* __restrict__ hl,
                                              const T* __restrict__ hm, const T* __restrict__ hh,
                                              T* __restrict__ xf, int32_t* dbg_tok, int32_t* dbg_par) {
  const int b = blockIdx.x;
  for (int s = threadIdx.x; s < S; s += blockDim.x) {
    const int i = b * S + s;
    const int rt = clampi(root_tok[b], 0, V - 1);
    st.tok[i] = s == 0 ? rt : -1;
    st.parent[i] = s == 0 ? -1 : -2;
    st.valid[i] = s == 0;
    st.score[i] = 0.f;
    for (int q = 0; q < st.mw; ++q) st.mask[(size_t)i * st.mw + q] = (s == 0 && q == 0) ? 1ull : 0ull;
    st.cand[i] = -1;
    if (dbg_tok) dbg_tok[i] = st.tok[i];
    if (dbg_par) dbg_par[i] = st.parent[i];
  }
  if (threadIdx.x == 0) {
    cs.count[b] = 0;
    cs.ntop[b] = 0;
  }
  constexpr int EPC = Vec<T>::N;
  for (int k = threadIdx.x * EPC; k < d; k += blockDim.x * EPC) {
    const u32x4 a = ld16(hl + (size_t)b * d + k);
    const u32x4 m = ld16(hm + (size_t)b * d + k);
    const u32x4 h = ld16(hh + (size_t)b * d + k);
    st16(xf + (size_t)b * 3 * d + k, a);
    st16(xf + (size_t)b * 3 * d + d + k, m);
    st16(xf + (size_t)b * 3 * d + 2 * d + k, h);
  }
}

// ---------------------------------------------------------------------------------------
// Row kernels.  One workgroup per row, one thread per 8-element chunk (d <= 8 * 1024), every
// load issued before any arithmetic so a row costs one memory round trip.
// ---------------------------------------------------------------------------------------
// prep: u = [rms(E[x]) * g_e ; rms(f) * g_f], f = g (root) or a of the parent slot.
template <typename T>
__global__ __launch_bounds__(1024) void k_prep(int R, int sb, int S, int d, int V, float eps, int step,
                                               SlotState st, const T* __restrict__ embed,
                                               const T* __restrict__ g_e, const T* __restrict__ g_f,
                                               const float* __restrict__ gpart, int gsplits, int B,
                                               const float* __restrict__ slot_a,
                                               float* __restrict__ f_rows, T* __restrict__ u,
                                               uint64_t* __restrict__ row_mask, float* __restrict__ g_dbg) {
  __shared__ float red[32];
  const int r = blockIdx.x;
  const int b = r / R, j = r % R;
  const int si = b * S + sb + j;
  const bool valid = st.valid[si] != 0;
  const int tok = valid ? clampi(st.tok[si], 0, V - 1) : 0;
  const int k0 = threadIdx.x * 8;
  const bool act = k0 < d;
  float e[8], fv[8], ge[8], gf[8];
  float se = 0.f, sf = 0.f;
  if (act) {
    load8<T>(embed + (size_t)tok * d + k0, e);
#pragma unroll
    for (int i = 0; i < 8; ++i) fv[i] = 0.f;
    if (step == 0) {
      // root: the fused feature g = W_f [h_low; h_mid; h_high], summed over its k-splits
      for (int s = 0; s < gsplits; ++s) {
        float t[8];
        load8<float>(gpart + ((size_t)s * B + b) * d + k0, t);
#pragma unroll
        for (int i = 0; i < 8; ++i) fv[i] += t[i];
      }
      if (g_dbg) store8<float>(g_dbg + (size_t)b * d + k0, fv);
      if (!valid)
#pragma unroll
        for (int i = 0; i < 8; ++i) fv[i] = 0.f;
    } else if (valid) {
      load8<float>(slot_a + ((size_t)b * S + clampi(st.parent[si], 0, S - 1)) * d + k0, fv);
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
  store8<float>(f_rows + (size_t)r * d + k0, fv);
  if ((int)threadIdx.x < st.mw)
    row_mask[(size_t)r * st.mw + threadIdx.x] = valid ? st.mask[(size_t)si * st.mw + threadIdx.x] : 0ull;
}

// Residual + RMSNorm over a projection's split-K partials:
//   y = resid + sum_s part[s] (split order), kept in fp32 as `out` (and per slot in `keep`),
//   outT = rms(y) * gamma in dtype.
template <typename T>
__global__ __launch_bounds__(1024) void k_resid_norm(const float* __restrict__ part, int splits, int M,
                                                     int d, const float* __restrict__ resid,
                                                     const T* __restrict__ gamma, float eps,
                                                     float* __restrict__ out, T* __restrict__ outT,
                                                     int R, int sb, int S, SlotState st,
                                                     float* __restrict__ keep, float* __restrict__ keep_dbg) {
  __shared__ float red[32];
  const int r = blockIdx.x;
  const int k0 = threadIdx.x * 8;
  const bool act = k0 < d;
  float x[8], gm[8];
  float ss = 0.f, dummy = 0.f;
  if (act) {
    load8<float>(resid + (size_t)r * d + k0, x);
    load8<T>(gamma + k0, gm);
    float acc[8];
    load8<float>(part + (size_t)r * d + k0, acc);
    for (int s = 1; s < splits; ++s) {
      float t[8];
      load8<float>(part + ((size_t)s * M + r) * d + k0, t);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += t[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] += acc[i];
      ss += x[i] * x[i];
    }
  }
  block_sum2(ss, dummy, red);
  if (!act) return;
  const float inv = 1.f / sqrtf(ss / d + eps);
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = x[i] * inv * gm[i];
  store8<float>(out + (size_t)r * d + k0, x);
  store8<T>(outT + (size_t)r * d + k0, o);
  if (keep) {
    const int b = r / R, j = r % R;
    const int si = b * S + sb + j;
    if (st.valid[si]) {
      store8<float>(keep + (size_t)si * d + k0, x);
      if (keep_dbg) store8<float>(keep_dbg + (size_t)si * d + k0, x);
    }
  }
}

// ---------------------------------------------------------------------------------------
// QKV epilogue: sum partials, RoPE on q and k (half-split pairs, angle pos*theta^(-2i/Dh)
// evaluated in fp64), scatter q to rows and k/v to the request's slot KV.
// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_epi_qkv(const float* __restrict__ part, int splits, int M, int Hq,
                                                 int Hkv, int Dh, int R, int sb, int S, int step,
                                                 float theta, const int32_t* __restrict__ cu_prefix,
                                                 SlotState /*st*/, T* __restrict__ q_rows,
                                                 T* __restrict__ kslot, T* __restrict__ vslot) {
  const int half = Dh / 2;
  const int H = Hq + 2 * Hkv;
  const int N = H * Dh;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)M * H * half) return;
  const int i = (int)(idx % half);
  const int h = (int)((idx / half) % H);
  const int m = (int)(idx / ((long)half * H));
  float y1 = 0.f, y2 = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float* p = part + ((size_t)s * M + m) * N + h * Dh;
    y1 += p[i];
    y2 += p[i + half];
  }
  const int b = m / R, j = m % R;
  const int si = b * S + sb + j;
  if (h < Hq + Hkv) {
    const int P = cu_prefix ? cu_prefix[b + 1] - cu_prefix[b] : 0;
    const double pos = (double)(P + step);
    const double ang = pos * pow((double)theta, -2.0 * i / Dh);
    double sn, cn;
    sincos(ang, &sn, &cn);
    const float c = (float)cn, s = (float)sn;
    const float o1 = y1 * c - y2 * s;
    const float o2 = y1 * s + y2 * c;
    y1 = o1;
    y2 = o2;
  }
  T* dst;
  if (h < Hq) {
    dst = q_rows + ((size_t)m * Hq + h) * Dh;
  } else {
    // padding rows (unused slots) are written too: their keys are masked out of every
    // row, but P = 0 times a non-finite stale value would still poison P.V
    const int c = h < Hq + Hkv ? h - Hq : h - Hq - Hkv;
    T* base = h < Hq + Hkv ? kslot : vslot;
    dst = base + ((size_t)si * Hkv + c) * Dh;
  }
  dst[i] = from_f32<T>(y1);
  dst[i + half] = from_f32<T>(y2);
}

// ---------------------------------------------------------------------------------------
// Exact top-K (value desc, id asc) over a wave, NV pairs per lane.
// The threshold tau is the K-th largest lane maximum (K rounds of wave max; the lanes that
// hold a round's maximum drop out), a lower bound on the K-th largest value, so the top K
// are among the pairs with value >= tau.  When at most TK_CAP pairs pass, they are
// compacted into this wave's LDS slots (positions from per-element ballots) and each is
// ranked against all of them; the pair of rank r < K goes to out(r, ...).  Otherwise (many
// ties at tau, or fewer than K finite lane maxima) K exact argmax rounds over all pairs are
// used.  Ids must be distinct across the wave, except for padding pairs (value -inf).
// `sv`, `si` hold TK_CAP entries of this wave's LDS, 16-byte aligned.
// ---------------------------------------------------------------------------------------
constexpr int TK_CAP = 64;

// Ranks the wave's compacted pairs sv/si[0 .. total), total <= TK_CAP, against each other
// by (value desc, id asc) (ids distinct); the pair of rank r < K goes to out(r, ...).  The
// list is padded to a multiple of four with (-inf, INT_MAX), which beats no entry, so each
// pair is ranked against four entries per LDS read.
template <typename Out>
__device__ __forceinline__ void rank_compacted(float* sv, int* si, int total, int K, Out out) {
  const int lane = threadIdx.x & 63;
  const int total4 = (total + 3) & ~3;
  if (lane >= total && lane < total4) {
    sv[lane] = kNegInf;
    si[lane] = 0x7fffffff;
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < total) {
    const float a = sv[lane];
    const int ia = si[lane];
    int r = 0;
    for (int j = 0; j < total4; j += 4) {
      const floatx4 bv = *reinterpret_cast<const floatx4*>(sv + j);
      const intx4 bi = *reinterpret_cast<const intx4*>(si + j);
#pragma unroll
      for (int q = 0; q < 4; ++q) r += (int)((bv[q] > a) | ((bv[q] == a) & (bi[q] < ia)));
    }
    if (r < K) out(r, a, ia);
  }
}

template <int NV, typename IdOf, typename Out>
__device__ __forceinline__ void wave_topk(const float* v, IdOf id_of, int K, float* sv, int* si, Out out) {
  const int lane = threadIdx.x & 63;
  float lm = kNegInf;
#pragma unroll
  for (int e = 0; e < NV; ++e) lm = fmaxf(lm, v[e]);
  float x = lm, tau = kNegInf;
  for (int k = 0; k < K; ++k) {
    tau = wave_max(x);
    if (x == tau) x = kNegInf;
  }
  uint64_t bal[NV];
  int total = 0;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    bal[e] = __ballot(v[e] >= tau);
    total += __popcll(bal[e]);
  }
  if (total <= TK_CAP) {
    int off = 0;
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      if (v[e] >= tau) {
        const int p = off + __popcll(bal[e] & below);
        sv[p] = v[e];
        si[p] = id_of(e);
      }
      off += __popcll(bal[e]);
    }
    rank_compacted(sv, si, total, K, out);
  } else {
    // a pair that won a round is taken out by its bit, so that when fewer than K finite
    // values exist the -inf padding is drawn in id order, each pair once
    uint32_t gone = 0;
    for (int k = 0; k < K; ++k) {
      float bv = kNegInf;
      int bi = 0x7fffffff;
#pragma unroll
      for (int e = 0; e < NV; ++e)
        if (!((gone >> e) & 1u)) argmax_pair(bv, bi, v[e], id_of(e));
      wave_argmax(bv, bi);
      if (lane == 0) out(k, bv, bi);
#pragma unroll
      for (int e = 0; e < NV; ++e)
        if (id_of(e) == bi && v[e] == bv) gone |= 1u << e;
    }
  }
}

// ---------------------------------------------------------------------------------------
// LM head top-K / log-sum-exp, pass 1: one workgroup per (row, chunk of 4096 logits).  Each
// wave takes 1024 logits, 16 per lane (four float4 loads issued together): its K winners
// from wave_topk and its (max, sum e^{z-max}) from wave reductions go to LDS; wave 0 then
// draws the chunk's K winners (best first) from the 4K wave winners, one per lane, and
// combines the four (max, sum) pairs in wave order.
// ---------------------------------------------------------------------------------------
constexpr int TK_CHUNK = 4096;

// Load one chunk's best-first list of K (padded to 16 with (-inf, max id)).
__device__ __forceinline__ void load_list(const float* cv, const int* ci, size_t base, int K, bool ok,
                                          float* v, int* id) {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const bool in = ok && k < K;
    v[k] = in ? cv[base + k] : kNegInf;
    id[k] = in ? ci[base + k] : 0x7fffffff;
  }
}

__global__ __launch_bounds__(256) void k_topk_chunk(const float* __restrict__ part, int splits, int M,
                                                    int V, int K, int n_chunks,
                                                    float* __restrict__ cv, int* __restrict__ ci,
                                                    float* __restrict__ cmax, float* __restrict__ csum,
                                                    float* __restrict__ dbg_logits, int R, int sb, int S,
                                                    SlotState st, SampCfg sc) {
  __shared__ __attribute__((aligned(16))) float sv[4][TK_CAP];
  __shared__ __attribute__((aligned(16))) int si[4][TK_CAP];
  __shared__ float wv[4 * KMAX];
  __shared__ int wi[4 * KMAX];
  __shared__ float wmax[4], wsum[4];
  const int m = blockIdx.y, c = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t0 = c * TK_CHUNK + w * 1024;
  float* dl = nullptr;
  const int rb = m / R, rj = m % R;
  float* lout = sc.on ? sc.slot_logits : dbg_logits;
  if (lout) {
    const int sidx = rb * S + sb + rj;
    if (st.valid[sidx]) dl = lout + (size_t)sidx * V;
  }
  // the four float4 loads of a split are issued together, splits summed in order
  float v[16];
  floatx4 z[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = t0 + 4 * (lane + 64 * q);
    z[q] = t < V ? *reinterpret_cast<const floatx4*>(part + (size_t)m * V + t) : floatx4{0.f, 0.f, 0.f, 0.f};
  }
  for (int s = 1; s < splits; ++s) {
    floatx4 y[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = t0 + 4 * (lane + 64 * q);
      y[q] = t < V ? *reinterpret_cast<const floatx4*>(part + ((size_t)s * M + m) * V + t)
                   : floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) z[q] += y[q];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = t0 + 4 * (lane + 64 * q);
    if (dl && t < V) *reinterpret_cast<floatx4*>(dl + t) = z[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * q + e] = t + e < V ? (sc.on ? __fmul_rn(z[q][e], sc.invT) : z[q][e]) : kNegInf;
  }
  float lm = kNegInf;
#pragma unroll
  for (int i = 0; i < 16; ++i) lm = fmaxf(lm, v[i]);
  const float bm = wave_max(lm);
  float ls = 0.f;
  if (bm != kNegInf)
#pragma unroll
    for (int i = 0; i < 16; ++i) ls += __builtin_amdgcn_exp2f((v[i] - bm) * kLog2e);
  const float tot = wave_sum(ls);
  if (sc.on) {   // the ranking values of sampled drafting: z * invT + Gumbel noise
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = t0 + 4 * (lane + 64 * q);
      if (t >= V) continue;
      uint32_t ctr[4] = {(uint32_t)(t >> 2), 0x80000000u | (uint32_t)(sb + rj), (uint32_t)rb, sc.rnd};
      philox4x32_10(ctr, sc.seed_lo, sc.seed_hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = __fadd_rn(v[4 * q + e], gumbel_from_word(ctr[e]));
    }
  }
  if (lane < K) {
    wv[w * K + lane] = kNegInf;   // a wave with fewer than K finite logits leaves padding
    wi[w * K + lane] = 0x7fffffff;
  }
  // a wave wholly past the vocabulary end keeps the padding written above (its list would be
  // K of its -inf pairs; with K <= V they never reach a row's top K)
  if (t0 < V)
    wave_topk<16>(v, [&](int e) { return t0 + 4 * (lane + 64 * (e >> 2)) + (e & 3); }, K, sv[w], si[w],
                  [&](int r, float val, int id) {
                    wv[w * K + r] = val;
                    wi[w * K + r] = id;
                  });
  if (lane == 0) {
    wmax[w] = bm;
    wsum[w] = tot;
  }
  __syncthreads();
  if (w != 0) return;
  const float x = lane < 4 * K ? wv[lane] : kNegInf;
  const int xi = lane < 4 * K ? wi[lane] : 0x7fffffff - lane;   // padding ids kept distinct
  const size_t base = ((size_t)m * n_chunks + c) * K;
  wave_topk<1>(&x, [&](int) { return xi; }, K, sv[0], si[0], [&](int r, float val, int id) {
    cv[base + r] = val;
    ci[base + r] = id;
  });
  if (lane == 0) {
    float mx = wmax[0];
    for (int i = 1; i < 4; ++i) mx = fmaxf(mx, wmax[i]);
    float sm = 0.f;
    for (int i = 0; i < 4; ++i)
      if (wmax[i] != kNegInf) sm += wsum[i] * __builtin_amdgcn_exp2f((wmax[i] - mx) * kLog2e);
    cmax[(size_t)m * n_chunks + c] = mx;
    csum[(size_t)m * n_chunks + c] = sm;
  }
}

// ---------------------------------------------------------------------------------------
// Tree selection for one request per workgroup (one wave per evaluated row).
// Phase 1: wave j merges row j's chunk winners into its top-K (each lane keeps a sorted
// list of 16 fed from its chunks, then K wave-argmax rounds) and its log-sum-exp (chunk
// maxima and sums combined in fixed order).
// Phase 2: children of the nodes evaluated at this step get s = s_parent + (z - lse) in
// fp32; then either the next depth's W best by (s desc, creation asc) become evaluation
// slots, or (last step) the N best candidates of the pool are kept and relabelled by
// (depth asc, creation asc).
// ---------------------------------------------------------------------------------------
constexpr int SEL_MAXR = 16;   // rows (W) per request handled by one workgroup

constexpr int SEL_MAXNEW = SEL_MAXR * KMAX;   // new candidates per step

// The LM head's output when it ran with block statistics (stats != nullptr): the logits z
// [M, V] and, per row and block of 128 columns, the best logit (value desc, column asc), its
// column and the sum of e^(z - best) over the block (three planes of M x e3h::kLmStatsLd).
struct LmBlocks {
  const float* stats;
  const float* z;
  float* dbg_z;      // per-slot copy of the logits [B * S, V] (optional)
  int M, nblk, V;    // nblk = ceil(V / 128)
};
constexpr int SEL_MAXTOP = 256;               // N <= 255

// Row top-K (value desc, column asc) and log-sum-exp from the LM head's statistics per block
// of 128 columns (one wave per row; an invalid row only issues its loads and returns 0).
// Fast path: tau, the value of the K-th of K rounds of wave maxima over the lanes' two best
// block bests (each lane holds 16 blocks), is at most the row's K-th best value (the rounds
// take at least K distinct entries at or above it), so every entry of the top K lies in a
// block whose best reaches tau; when at most 32 blocks do, their logits are scanned for the
// entries >= tau, which are ranked against each other when at most TK_CAP pass.  Otherwise (ties, or logits bunched at the top) the
// exact path: the K blocks with the best entries (a block whose best is not among them has K
// distinct entries above all of its own) are scanned for the entries at or above theta, the
// K-th of those block bests, and ranked, or (many ties at theta) K exact rounds over the K
// blocks each take the best entry below the previous round's.  The log-sum-exp combines the
// blocks' (best, sum) pairs.
template <typename Out>
__device__ __forceinline__ float row_topk_blocks(const LmBlocks& lb, int m, int K, bool valid, float* sv, int* si,
                                                 float* sbv, int* sblk, Out out) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  constexpr int LD = e3h::kLmStatsLd;
  const size_t plane = (size_t)lb.M * LD, row = (size_t)m * LD + 16 * lane;   // blocks 16 lane + i
  float bv[16], bs[16];
  int bi[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(lb.stats + row + 4 * q);
    const intx4 c = *reinterpret_cast<const intx4*>(reinterpret_cast<const int*>(lb.stats) + plane + row + 4 * q);
    const floatx4 d = *reinterpret_cast<const floatx4*>(lb.stats + 2 * plane + row + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = 16 * lane + 4 * q + e < lb.nblk;
      bv[4 * q + e] = ok ? a[e] : kNegInf;
      bi[4 * q + e] = ok ? c[e] : 0x7fffffff;
      bs[4 * q + e] = ok ? d[e] : 0.f;
    }
  }
  if (!valid) return 0.f;
  float lm = kNegInf;
#pragma unroll
  for (int i = 0; i < 16; ++i) lm = fmaxf(lm, bv[i]);
  const float mx = wave_max(lm);
  float ls = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ls += bv[i] != kNegInf ? bs[i] * __builtin_amdgcn_exp2f((bv[i] - mx) * kLog2e) : 0.f;
  const float lse = mx + logf(wave_sum(ls));
  const float* zr = lb.z + (size_t)m * lb.V;

  // ---- fast path
  {
    // tau: K rounds over the lanes' two best block bests (a round takes every lane's current
    // head that equals the wave maximum), at most the K-th best value
    float x = bv[0], x2 = kNegInf, tau = kNegInf;   // the lane's best and second best
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      x2 = fmaxf(x2, fminf(x, bv[i]));
      x = fmaxf(x, bv[i]);
    }
    for (int k = 0; k < K; ++k) {
      tau = wave_max(x);
      if (x == tau) {
        x = x2;
        x2 = kNegInf;
      }
    }
    int nb = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool in = bv[i] >= tau;
      const uint64_t bal = __ballot(in);
      const int pos = nb + __popcll(bal & below);
      if (in & (pos < 2 * KMAX)) sblk[pos] = 16 * lane + i;
      nb += __popcll(bal);
    }
    if (nb <= 2 * KMAX) {
      __builtin_amdgcn_wave_barrier();
      int total = 0;
      for (int r0 = 0; r0 < nb; r0 += KMAX) {   // up to 16 blocks per pass, two columns per lane each
        float z[2 * KMAX];
        int n[2 * KMAX];
#pragma unroll
        for (int r = 0; r < KMAX; ++r) {
          const int c = r0 + r < nb ? sblk[r0 + r] : -1;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int col = 128 * c + 64 * h + lane;
            n[2 * r + h] = (c >= 0) & (col < lb.V) ? col : lb.V;
            z[2 * r + h] = n[2 * r + h] < lb.V ? zr[n[2 * r + h]] : kNegInf;
          }
        }
#pragma unroll
        for (int i = 0; i < 2 * KMAX; ++i) {
          const bool keep = (n[i] < lb.V) & (z[i] >= tau);
          const uint64_t bal = __ballot(keep);
          if (bal) {
            const int pos = total + __popcll(bal & below);
            if (keep & (pos < TK_CAP)) {
              sv[pos] = z[i];
              si[pos] = n[i];
            }
            total += __popcll(bal);
          }
        }
      }
      if (total <= TK_CAP) {
        rank_compacted(sv, si, total, K, out);
        return lse;
      }
    }
  }

  // ---- exact path: the K best blocks (padding (-inf, INT_MAX) ranks last) and theta
  wave_topk<16>(bv, [&](int e) { return bi[e]; }, K, sv, si, [&](int r, float val, int idv) {
    sbv[r] = val;
    sblk[r] = idv;
  });
  __builtin_amdgcn_wave_barrier();
  const float tv = sbv[K - 1];
  const int ti = sblk[K - 1];
  int nsel = 0;
  for (int r = 0; r < K; ++r) nsel += sblk[r] != 0x7fffffff ? 1 : 0;
  const int tot = nsel * 128;   // the selected blocks' columns, block after block
  auto col_of = [&](int q) { return ((sblk[q >> 7] >> 7) << 7) + (q & 127); };
  int total = 0;
  for (int q0 = 0; q0 < tot; q0 += 64) {
    const int q = q0 + lane;
    const int col = q < tot ? col_of(q) : lb.V;
    const float zv = col < lb.V ? zr[col] : kNegInf;
    const bool keep = (col < lb.V) & ((zv > tv) | ((zv == tv) & (col <= ti)));
    const uint64_t bal = __ballot(keep);
    const int pos = total + __popcll(bal & below);
    if (keep & (pos < TK_CAP)) {
      sv[pos] = zv;
      si[pos] = col;
    }
    total += __popcll(bal);
  }
  if (total <= TK_CAP) {
    rank_compacted(sv, si, total, K, out);
  } else {
    float pv = __builtin_huge_valf();
    int pi = -1;
    for (int k = 0; k < K; ++k) {
      float v = kNegInf;
      int id = 0x7fffffff;
      for (int q = lane; q < tot; q += 64) {
        const int col = col_of(q);
        if (col < lb.V) {
          const float zv = zr[col];
          if (((zv < pv) | ((zv == pv) & (col > pi))) & better(zv, col, v, id)) {
            v = zv;
            id = col;
          }
        }
      }
      wave_argmax(v, id);
      if (lane == 0) out(k, v, id);
      pv = v;
      pi = id;
    }
  }
  return lse;
}

// Phase 2 keeps a running list of the N best candidates created so far: the N best of all
// candidates are the N best of (the previous list and the new candidates), so each step ranks
// at most N + W*K entries, and the last step relabels the final list.
__global__ __launch_bounds__(1024) void k_select(int step, int D, int K, int W, int N, int S, int PMAX,
                                                 int R, int n_chunks, const float* __restrict__ cv,
                                                 const int* __restrict__ ci,
                                                 const float* __restrict__ cmax,
                                                 const float* __restrict__ csum, SlotState st,
                                                 CandState cs, int32_t* __restrict__ out_tok,
                                                 int32_t* __restrict__ out_par,
                                                 int32_t* __restrict__ out_dep, float* __restrict__ out_score,
                                                 int32_t* __restrict__ out_n, int32_t* dbg_tok,
                                                 int32_t* dbg_par, int32_t* dbg_id, float* dbg_val,
                                                 float* dbg_lse, SampCfg sc, LmBlocks lb) {
#pragma clang fp contract(off)
  __shared__ float s_val[SEL_MAXR][KMAX];
  __shared__ float s_bv[SEL_MAXR][KMAX];
  __shared__ int s_blk[SEL_MAXR][2 * KMAX];
  __shared__ int s_id[SEL_MAXR][KMAX];
  __shared__ float s_lse[SEL_MAXR];
  __shared__ __attribute__((aligned(16))) float s_cv[SEL_MAXR][TK_CAP];
  __shared__ __attribute__((aligned(16))) int s_ci[SEL_MAXR][TK_CAP];
  __shared__ float nsc[SEL_MAXNEW];   // new candidates, creation order
  __shared__ int ntok[SEL_MAXNEW];
  __shared__ int nps[SEL_MAXNEW];
  __shared__ float msc[SEL_MAXTOP];   // the running list: scores, candidate indices
  __shared__ int midx[SEL_MAXTOP];
  __shared__ int ktop[SEL_MAXTOP];
  __shared__ float ktsc[SEL_MAXTOP];
  __shared__ int lab_of[1024];
  __shared__ int s_valid[SEL_MAXR];
  __shared__ float s_score[SEL_MAXR];
  __shared__ uint64_t s_mask[SEL_MAXR][SMAX / 64];
  __shared__ int s_cand[SEL_MAXR];
  __shared__ int fr_e[SEL_MAXR];
  __shared__ int s_rank[SEL_MAXNEW];   // ranks of the new candidates among themselves
  __shared__ int nord[SEL_MAXNEW];     // the new candidates in rank order
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int sb = step == 0 ? 0 : 1 + (step - 1) * W;
  const bool last = step + 1 == D;
  const int n_before = cs.count[b];
  const int ntop = cs.ntop[b];
  int32_t* ctok = cs.tok + (size_t)b * PMAX;
  int32_t* cps = cs.pslot + (size_t)b * PMAX;
  int32_t* cdep = cs.depth + (size_t)b * PMAX;
  float* csc = cs.score + (size_t)b * PMAX;
  int32_t* topn = cs.topn + (size_t)b * N;
  float* topsc = cs.topsc + (size_t)b * N;
  // ---- phase 1: each row's top-K and log-sum-exp, from the LM head's block statistics, or
  // from the chunk lists of k_topk_chunk (lane l holds chunk l's list; the chunks' (max, sum)
  // combined in lane order)
  if (w < R) {
    const int m = b * R + w;
    const int sidx = b * S + sb + w;
    const int valid = st.valid[sidx];
    const float score0 = st.score[sidx];
    const int cand0 = st.cand[sidx];
    if (lane < st.mw) s_mask[w][lane] = st.mask[(size_t)sidx * st.mw + lane];
    if (lane == 0) {
      s_valid[w] = valid;
      s_score[w] = score0;
      s_cand[w] = cand0;
    }
    auto out = [&](int r, float val, int idv) {
      // sampled drafting ranks by noisy values; the scores use the child's z * invT
      if (sc.on)
        val = (idv >= 0 && idv < sc.V) ? __fmul_rn(sc.slot_logits[(size_t)sidx * sc.V + idv], sc.invT) : kNegInf;
      s_val[w][r] = val;
      s_id[w][r] = idv;
      if (dbg_id) dbg_id[(size_t)sidx * K + r] = idv;
      if (dbg_val) dbg_val[(size_t)sidx * K + r] = val;
    };
    float row_lse = 0.f;
    if (lb.stats) {
      row_lse = row_topk_blocks(lb, m, K, valid != 0, s_cv[w], s_ci[w], s_bv[w], s_blk[w], out);
      if (valid && lb.dbg_z) {
        const floatx4* src = reinterpret_cast<const floatx4*>(lb.z + (size_t)m * lb.V);
        floatx4* dst = reinterpret_cast<floatx4*>(lb.dbg_z + (size_t)sidx * lb.V);
        for (int t = lane; t < lb.V / 4; t += 64) dst[t] = src[t];
      }
    } else {
      const bool ok = lane < n_chunks;
      const float cm = ok ? cmax[(size_t)m * n_chunks + lane] : kNegInf;
      const float cs_ = ok ? csum[(size_t)m * n_chunks + lane] : 0.f;
      float v[16];
      int id[16];
      load_list(cv, ci, ((size_t)m * n_chunks + lane) * K, K, ok, v, id);
      if (valid) {
        const float mx = wave_max(cm);
        const float tot = wave_sum(cm != kNegInf ? cs_ * expf(cm - mx) : 0.f);
        row_lse = mx + logf(tot);
        wave_topk<16>(v, [&](int e) { return id[e]; }, K, s_cv[w], s_ci[w], out);
      }
    }
    if (valid && lane == 0) {
      s_lse[w] = row_lse;
      if (dbg_lse) dbg_lse[sidx] = row_lse;
    }
  }
  // the running list into LDS, from the highest thread down: the top waves sit out phase 1
  // when R < 16, so these loads overlap its loads instead of preceding them
  for (int i = (int)(blockDim.x - 1 - threadIdx.x); i < ntop; i += blockDim.x) {
    msc[i] = topsc[i];
    midx[i] = topn[i];
  }
  __syncthreads();

  // ---- phase 2: children of this step's nodes, s = s_parent + (z - lse) in fp32, recorded in
  // creation order (evaluation rank of the parent, then child rank)
  int nE = 0;  // valid slots form a prefix of the step's slots
  for (int j = 0; j < R; ++j) nE += s_valid[j] ? 1 : 0;
  const int n_new = nE * K;
  const int n_total = n_before + n_new;
  const int m_total = ntop + n_new;
  for (int e = threadIdx.x; e < n_new; e += blockDim.x) {
    const int j = e / K, rk = e % K;
    // a child never scores above a sibling created before it: no change for a top-K list
    // (values fall with the rank); keeps sampled siblings a prefix of the draw order
    float sc = s_score[j] + (s_val[j][rk] - s_lse[j]);
    for (int r2 = 0; r2 < rk; ++r2) sc = fminf(sc, s_score[j] + (s_val[j][r2] - s_lse[j]));
    const int tk = s_id[j][rk];
    nsc[e] = sc;
    ntok[e] = tk;
    nps[e] = sb + j;
    s_rank[e] = rk;
  }
  for (int i = threadIdx.x; i < n_total; i += blockDim.x) lab_of[i] = -1;
  __syncthreads();
  // Ranks by (score desc, creation asc), a strict order (creation indices are distinct).  Each
  // evaluated row's children are sorted in it (scores fall with the child rank, creation
  // rises), and so is the running list of the N best so far.  So a candidate's rank among the
  // new ones is its child rank plus, for every other row, the length of that row's prefix that
  // beats it (a binary search); and in the union with the running list it is its rank in its
  // own sorted list plus the prefix of the other list that beats it.
  for (int pr = threadIdx.x; pr < n_new * nE; pr += blockDim.x) {
    const int e = pr / nE, j2 = pr - e * nE;
    if (j2 == e / K) continue;
    const float se = nsc[e];
    int lo = 0, hi = K;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1, f = j2 * K + mid;
      if ((nsc[f] > se) | ((nsc[f] == se) & (f < e))) lo = mid + 1;
      else hi = mid;
    }
    if (lo) atomicAdd(&s_rank[e], lo);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n_new; e += blockDim.x) nord[s_rank[e]] = e;
  __syncthreads();
  if (!last)
    for (int r = threadIdx.x; r < min(W, n_new); r += blockDim.x) fr_e[r] = nord[r];
  for (int x = threadIdx.x; x < m_total; x += blockDim.x) {
    float sx;
    int ix, own, lo = 0, hi;
    if (x < ntop) {   // a running-list entry against the new candidates in rank order
      sx = msc[x];
      ix = midx[x];
      own = x;
      hi = n_new;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1, f = nord[mid];
        if ((nsc[f] > sx) | ((nsc[f] == sx) & (n_before + f < ix))) lo = mid + 1;
        else hi = mid;
      }
    } else {          // the new candidate of rank x - ntop against the running list
      own = x - ntop;
      const int e = nord[own];
      sx = nsc[e];
      ix = n_before + e;
      hi = ntop;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((msc[mid] > sx) | ((msc[mid] == sx) & (midx[mid] < ix))) lo = mid + 1;
        else hi = mid;
      }
    }
    const int r = own + lo;
    if (r < N) {
      ktop[r] = ix;
      ktsc[r] = sx;
    }
  }
  __syncthreads();
  const int n_keep = min(N, m_total);
  // this step's candidates into the pool
  for (int e = threadIdx.x; e < n_new; e += blockDim.x) {
    ctok[n_before + e] = ntok[e];
    cps[n_before + e] = nps[e];
    cdep[n_before + e] = step + 1;
    csc[n_before + e] = nsc[e];
  }
  if (!last) {
    const int nsb = 1 + step * W;
    const int n_fr = min(W, n_new);
    for (int r = threadIdx.x; r < n_fr; r += blockDim.x) {
      const int e = fr_e[r];
      const int slot = nsb + r;
      const int i = b * S + slot;
      const int ps = nps[e];
      st.tok[i] = ntok[e];
      st.parent[i] = ps;
      st.valid[i] = 1;
      st.score[i] = nsc[e];
      st.cand[i] = n_before + e;
      for (int q = 0; q < st.mw; ++q)
        st.mask[(size_t)i * st.mw + q] = s_mask[ps - sb][q] | (q == (slot >> 6) ? 1ull << (slot & 63) : 0ull);
      if (dbg_tok) dbg_tok[i] = ntok[e];
      if (dbg_par) dbg_par[i] = ps;
    }
    for (int i = threadIdx.x; i < n_keep; i += blockDim.x) {
      topn[i] = ktop[i];
      topsc[i] = ktsc[i];
    }
    if (threadIdx.x == 0) {
      cs.ntop[b] = n_keep;
      cs.count[b] = n_total;
    }
    return;
  }
  // final: relabel the kept candidates by (depth asc, creation asc), which is creation order
  // since candidates are created depth by depth; root = 0
  for (int i = threadIdx.x; i < n_keep; i += blockDim.x) {
    const int idx = ktop[i];
    int lab = 1;
    for (int k = 0; k < n_keep; ++k) lab += (int)(ktop[k] < idx);
    lab_of[idx] = lab;
  }
  __syncthreads();
  const size_t ob = (size_t)b * (N + 1);
  if (sc.draft_row) {   // node -> row of its evaluation slot's logits, -1 for a node never evaluated
    int32_t* dr = sc.draft_row + ob;
    for (int l = threadIdx.x; l <= N; l += blockDim.x) dr[l] = -1;
    __syncthreads();
    if (threadIdx.x == 0) dr[0] = b * S;
    for (int sl = 1 + threadIdx.x; sl < sb + R; sl += blockDim.x) {
      const int i = b * S + sl;
      if (!st.valid[i]) continue;
      const int c = st.cand[i];
      const int lab = (c >= 0 && c < n_total) ? lab_of[c] : -1;
      if (lab > 0) dr[lab] = i;
    }
  }
  for (int i = threadIdx.x; i < n_keep; i += blockDim.x) {
    const int idx = ktop[i];
    const int lab = lab_of[idx];
    int tk, ps, dep;
    if (idx >= n_before) {
      tk = ntok[idx - n_before];
      ps = nps[idx - n_before];
      dep = step + 1;
    } else {
      tk = ctok[idx];
      ps = cps[idx];
      dep = cdep[idx];
    }
    int plab = 0;
    if (ps > 0) {
      // the parent slot's candidate: a slot of this step (LDS) or of an earlier one; it is kept
      // (a child's score never exceeds its parent's and a parent is created first)
      const int pc = (ps >= sb && ps < sb + R) ? s_cand[ps - sb] : st.cand[b * S + ps];
      plab = (pc >= 0 && pc < n_total) ? lab_of[pc] : -1;
    }
    out_tok[ob + lab] = tk;
    out_par[ob + lab] = plab;
    out_dep[ob + lab] = dep;
    out_score[ob + lab] = ktsc[i];
  }
  for (int l = n_keep + 1 + threadIdx.x; l <= N; l += blockDim.x) {
    out_tok[ob + l] = -1;
    out_par[ob + l] = -1;
    out_dep[ob + l] = -1;
    out_score[ob + l] = kNegInf;
  }
  if (threadIdx.x == 0) {
    out_tok[ob] = st.tok[b * S];
    out_par[ob] = -1;
    out_dep[ob] = 0;
    out_score[ob] = 0.f;
    out_n[b] = 1 + n_keep;
    cs.count[b] = n_total;
    cs.ntop[b] = n_keep;
  }
}

// ---------------------------------------------------------------------------------------
// Workspace plan
// ---------------------------------------------------------------------------------------
struct Plan {
  int B, d, Hq, Hkv, Dh, F, V, D, K, W, N, S, PMAX, Mmax, att_splits, lm_nchunk, row_threads;
  size_t gemm_part_elems;
  // pointers (null when measuring)
  SlotState st;
  CandState cs;
  float *gfuse, *slot_a, *f_rows, *h1, *a_rows, *gpart, *att_o, *att_lse, *cv, *cmax, *csum, *lmst;
  int* ci;
  uint64_t* row_mask;
  void *xf, *u, *q_rows, *kslot, *vslot, *attn, *mn, *act, *xl;
  size_t bytes;
};

Plan make_plan(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B, int max_prefix, void* ws) {
  Plan p;
  p.B = B;
  p.d = w->d;
  p.Hq = w->n_heads_q;
  p.Hkv = w->n_heads_kv;
  p.Dh = w->head_dim;
  p.F = w->ffn;
  p.V = w->vocab;
  p.D = t->depth;
  p.K = t->topk;
  p.W = t->width;
  p.N = t->n_nodes;
  p.S = 1 + (p.D - 1) * p.W;
  p.PMAX = p.K + (p.D - 1) * p.W * p.K;
  p.Mmax = B * (p.W > 1 ? p.W : 1);
  p.att_splits = e3h::attention_splits(B, p.Hkv, p.Mmax / B * (p.Hq / p.Hkv), max_prefix, 0);
  p.lm_nchunk = (p.V + TK_CHUNK - 1) / TK_CHUNK;
  p.row_threads = ((p.d / 8 + 63) / 64) * 64;
  const int es = e3h::elem_size(w->dtype);
  const int nqkv = (p.Hq + 2 * p.Hkv) * p.Dh;
  size_t gp = 0;
  auto upd = [&](int M, int N_, int K_) {
    e3h::GemmPlan gpl = e3h::plan_gemm(M, N_, K_, w->dtype);
    size_t e = (size_t)gpl.splits * M * N_;
    if (e > gp) gp = e;
  };
  for (int M : {B, p.Mmax}) {
    upd(M, nqkv, 2 * p.d);
    upd(M, p.d, p.Hq * p.Dh);
    upd(M, 2 * p.F, p.d);
    upd(M, p.d, p.F);
    upd(M, p.V, p.d);
  }
  p.gemm_part_elems = gp;
  e3h::Carve c(ws);
  const size_t BS = (size_t)B * p.S, BP = (size_t)B * p.PMAX;
  p.st.tok = c.take<int32_t>(BS);
  p.st.parent = c.take<int32_t>(BS);
  p.st.valid = c.take<int32_t>(BS);
  p.st.score = c.take<float>(BS);
  p.st.mw = (p.S + 63) / 64;
  p.st.mask = c.take<uint64_t>(BS * p.st.mw);
  p.st.cand = c.take<int32_t>(BS);
  p.cs.tok = c.take<int32_t>(BP);
  p.cs.pslot = c.take<int32_t>(BP);
  p.cs.depth = c.take<int32_t>(BP);
  p.cs.score = c.take<float>(BP);
  p.cs.count = c.take<int32_t>(B);
  p.cs.topn = c.take<int32_t>((size_t)B * p.N);
  p.cs.topsc = c.take<float>((size_t)B * p.N);
  p.cs.ntop = c.take<int32_t>(B);
  p.xf = c.take<char>((size_t)B * 3 * p.d * es);
  p.slot_a = c.take<float>(BS * p.d);
  p.kslot = c.take<char>(BS * p.Hkv * p.Dh * es);
  p.vslot = c.take<char>(BS * p.Hkv * p.Dh * es);
  const size_t M = p.Mmax;
  p.row_mask = c.take<uint64_t>(M * p.st.mw);
  p.f_rows = c.take<float>(M * p.d);
  p.u = c.take<char>(M * 2 * p.d * es);
  p.q_rows = c.take<char>(M * p.Hq * p.Dh * es);
  p.attn = c.take<char>(M * p.Hq * p.Dh * es);
  p.h1 = c.take<float>(M * p.d);
  p.mn = c.take<char>(M * p.d * es);
  p.act = c.take<char>(M * p.F * es);
  p.a_rows = c.take<float>(M * p.d);
  p.xl = c.take<char>(M * p.d * es);
  p.gpart = c.take<float>(gp);
  {
    e3h::GemmPlan gfp = e3h::plan_gemm(B, p.d, 3 * p.d, w->dtype);
    p.gfuse = c.take<float>((size_t)gfp.splits * B * p.d);
  }
  p.att_o = c.take<float>((size_t)(p.att_splits + 1) * M * p.Hq * p.Dh);
  p.att_lse = c.take<float>((size_t)(p.att_splits + 1) * M * p.Hq);
  p.cv = c.take<float>(M * p.lm_nchunk * p.K);
  p.ci = c.take<int>(M * p.lm_nchunk * p.K);
  p.cmax = c.take<float>(M * p.lm_nchunk);
  p.csum = c.take<float>(M * p.lm_nchunk);
  p.lmst = c.take<float>(3 * M * (size_t)e3h::kLmStatsLd);
  p.bytes = c.size();
  return p;
}

template <typename T>
int run_draft(const eagle3_drafter* w, const Plan& p, const void* h_low, const void* h_mid,
              const void* h_high, const int32_t* root_tok, const void* kpre, const void* vpre,
              const int32_t* cu_prefix, int32_t* tokens, int32_t* parents, int32_t* depth,
              float* score, int32_t* n_nodes, const eagle3_draft_debug* dbg, const SampCfg& sc,
              hipStream_t s) {
  using namespace e3h;
  const int B = p.B, d = p.d;
  const int dt = w->dtype;
  const int nqkv = (p.Hq + 2 * p.Hkv) * p.Dh;
  int32_t* dbg_tok = dbg ? dbg->slot_token : nullptr;
  int32_t* dbg_par = dbg ? dbg->slot_parent : nullptr;
  int st;
  GemmPlan gf = plan_gemm(B, d, 3 * d, dt);
  {
    {
      ProfScope ps("draft_init", s);
      hipLaunchKernelGGL(k_init<T>, dim3(B), dim3(256), 0, s, B, p.S, d, p.V, root_tok, p.st, p.cs,
                         (const T*)h_low, (const T*)h_mid, (const T*)h_high, (T*)p.xf, dbg_tok, dbg_par);
      if ((st = launch_status())) return st;
    }
    // feature fusion g = W_f [h_low; h_mid; h_high] (its k-splits are summed by the step-0 prep)
    if ((st = launch_gemm(gf, dt, p.xf, 3 * d, w->w_fuse, p.gfuse, s, "gemm_fuse"))) return st;
  }
  for (int step = 0; step < p.D; ++step) {
    const int R = step == 0 ? 1 : p.W;
    const int sb = step == 0 ? 0 : 1 + (step - 1) * p.W;
    const int M = B * R;
    {
      ProfScope ps("draft_prep", s);
      hipLaunchKernelGGL(k_prep<T>, dim3(M), dim3(p.row_threads), 0, s, R, sb, p.S, d, p.V, w->eps, step, p.st,
                         (const T*)w->embed, (const T*)w->g_embed, (const T*)w->g_feat, p.gfuse, gf.splits, B,
                         p.slot_a, p.f_rows, (T*)p.u, p.row_mask, dbg ? dbg->g : (float*)nullptr);
      if ((st = launch_status())) return st;
    }
    // QKV + RoPE
    {
      GemmPlan gp = plan_gemm(M, nqkv, 2 * d, dt);
      if ((st = launch_gemm(gp, dt, p.u, 2 * d, w->w_qkv, p.gpart, s, "gemm_qkv"))) return st;
      ProfScope ps("epi_qkv", s);
      const long n = (long)M * (p.Hq + 2 * p.Hkv) * (p.Dh / 2);
      hipLaunchKernelGGL(k_epi_qkv<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p.gpart,
                         gp.splits, M, p.Hq, p.Hkv, p.Dh, R, sb, p.S, step, w->rope_theta, cu_prefix,
                         p.st, (T*)p.q_rows, (T*)p.kslot, (T*)p.vslot);
      if ((st = launch_status())) return st;
    }
    // attention over the drafter prefix + evaluated ancestors-or-self
    {
      AttnArgs a;
      a.B = B;
      a.Hq = p.Hq;
      a.Hkv = p.Hkv;
      a.Dh = p.Dh;
      a.dtype = dt;
      a.q = p.q_rows;
      a.q_cu = nullptr;
      a.q_stride = R;
      a.q_rows_total = M;
      a.kt = p.kslot;
      a.vt = p.vslot;
      a.kt_cu = nullptr;
      a.kt_stride = p.S;
      a.kt_count = sb + R;
      a.mask = p.row_mask;
      a.W64 = p.st.mw;
      a.kp = kpre;
      a.vp = vpre;
      a.p_cu = cu_prefix;
      a.scale = (float)(1.0 / sqrt((double)p.Dh));
      a.S = p.att_splits;
      a.max_q_per_req = R;
      a.o_part = p.att_o;
      a.lse_part = p.att_lse;
      if ((st = launch_tree_attention(a, s, "draft_attention"))) return st;
      if ((st = launch_lse_merge(p.att_splits + 1, M * p.Hq, p.Dh, p.att_o, p.att_lse, dt, p.attn,
                                 nullptr, s, "draft_lse_merge")))
        return st;
    }
    // O projection + residual, RMSNorm
    {
      GemmPlan gp = plan_gemm(M, d, p.Hq * p.Dh, dt);
      if ((st = launch_gemm(gp, dt, p.attn, p.Hq * p.Dh, w->w_o, p.gpart, s, "gemm_o"))) return st;
      ProfScope ps("resid_norm", s);
      hipLaunchKernelGGL(k_resid_norm<T>, dim3(M), dim3(p.row_threads), 0, s, p.gpart, gp.splits, M, d,
                         p.f_rows, (const T*)w->g_mlp, w->eps, p.h1, (T*)p.mn, R, sb, p.S, p.st,
                         (float*)nullptr, (float*)nullptr);
      if ((st = launch_status())) return st;
    }
    // SiLU-gated MLP + residual, final RMSNorm
    {
      GemmPlan gp = plan_gemm(M, 2 * p.F, d, dt, true);
      if ((st = launch_gemm(gp, dt, p.mn, d, w->w_gate_up, p.gpart, s, "gemm_gate_up", p.act))) return st;
      GemmPlan gd = plan_gemm(M, d, p.F, dt);
      if ((st = launch_gemm(gd, dt, p.act, p.F, w->w_down, p.gpart, s, "gemm_down"))) return st;
      ProfScope ps("resid_norm", s);
      hipLaunchKernelGGL(k_resid_norm<T>, dim3(M), dim3(p.row_threads), 0, s, p.gpart, gd.splits, M, d, p.h1,
                         (const T*)w->g_final, w->eps, p.a_rows, (T*)p.xl, R, sb, p.S, p.st, p.slot_a,
                         dbg ? dbg->slot_a : (float*)nullptr);
      if ((st = launch_status())) return st;
    }
    // LM head, top-K and log-sum-exp, then the tree selection.  Drafting by top-K in bf16: the
    // LM head also emits per-block statistics, from which the selection takes each row's
    // top-K and log-sum-exp directly.  Otherwise (sampled drafting, fp32, a plan without the
    // statistics) k_topk_chunk first reduces chunks of 4096 logits to lists.
    {
      GemmPlan gp = plan_gemm(M, p.V, d, dt, false, !sc.on);
      const bool fused = !sc.on && gemm_block_stats_ok(gp) && (p.V + 127) / 128 <= kLmStatsLd;
      if (!fused) gp = plan_gemm(M, p.V, d, dt);
      LmBlocks lb{};
      if (fused) {
        lb.stats = p.lmst;
        lb.z = p.gpart;
        lb.dbg_z = dbg ? dbg->slot_logits : nullptr;
        lb.M = M;
        lb.nblk = (p.V + 127) / 128;
        lb.V = p.V;
      }
      // the root step's launch (B rows) carries its own tag, so timings of the depth steps'
      // LM head (B * W rows) are not averaged with it
      if ((st = launch_gemm(gp, dt, p.xl, d, w->w_lm, p.gpart, s, step == 0 ? "gemm_lm_head_root" : "gemm_lm_head",
                            nullptr, fused ? p.lmst : nullptr)))
        return st;
      if (!fused) {
        ProfScope ps("topk_chunk", s);
        hipLaunchKernelGGL(k_topk_chunk, dim3(p.lm_nchunk, M), dim3(256), 0, s, p.gpart,
                           gp.splits, M, p.V, p.K, p.lm_nchunk, p.cv, p.ci, p.cmax, p.csum,
                           dbg ? dbg->slot_logits : (float*)nullptr, R, sb, p.S, p.st, sc);
        if ((st = launch_status())) return st;
      }
      ProfScope ps("draft_select", s);
      hipLaunchKernelGGL(k_select, dim3(B), dim3(1024), 0, s, step, p.D, p.K, p.W, p.N, p.S, p.PMAX, R,
                         p.lm_nchunk, p.cv, p.ci, p.cmax, p.csum, p.st, p.cs, tokens, parents, depth,
                         score, n_nodes, dbg_tok, dbg_par, dbg ? dbg->slot_topk_id : (int32_t*)nullptr,
                         dbg ? dbg->slot_topk_val : (float*)nullptr, dbg ? dbg->slot_lse : (float*)nullptr,
                         sc, lb);
      if ((st = launch_status())) return st;
    }
  }
  return EAGLE3_OK;
}

}  // namespace

namespace e3h {

int drafter_check(const eagle3_drafter* w) {
  if (!w) return EAGLE3_EINVAL;
  if (!dtype_ok(w->dtype)) return EAGLE3_EINVAL;
  if (w->d <= 0 || w->n_heads_q <= 0 || w->n_heads_kv <= 0 || w->ffn <= 0 || w->vocab <= 0)
    return EAGLE3_EINVAL;
  if (w->n_heads_q % w->n_heads_kv) return EAGLE3_EINVAL;
  if (w->head_dim != 64 && w->head_dim != 128) return EAGLE3_EUNSUPPORTED;
  if (w->d % 8 || w->ffn % 8 || w->vocab % 4 || w->d > 8192) return EAGLE3_EUNSUPPORTED;
  if (!(w->eps > 0.f) || !(w->rope_theta > 0.f)) return EAGLE3_EINVAL;
  if (!w->embed || !w->w_fuse || !w->g_embed || !w->g_feat || !w->g_mlp || !w->g_final ||
      !w->w_qkv || !w->w_o || !w->w_gate_up || !w->w_down || !w->w_lm)
    return EAGLE3_EINVAL;
  return EAGLE3_OK;
}

int draft_check(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B, int max_prefix) {
  if (!w || !t || B <= 0 || max_prefix < 0) return EAGLE3_EINVAL;
  if (const int st = drafter_check(w)) return st;
  if (t->depth < 1 || t->topk < 1 || t->width < 1 || t->n_nodes < 1) return EAGLE3_EINVAL;
  if (t->topk > KMAX || t->topk > w->vocab) return EAGLE3_EUNSUPPORTED;
  if (1 + (long)(t->depth - 1) * t->width > SMAX) return EAGLE3_EUNSUPPORTED;
  if ((long)t->topk + (long)(t->depth - 1) * t->width * t->topk > 1024) return EAGLE3_EUNSUPPORTED;
  if (t->n_nodes > 255) return EAGLE3_EUNSUPPORTED;
  if ((long)B * (t->width > 1 ? t->width : 1) > 160) return EAGLE3_EUNSUPPORTED;
  if (t->width > SEL_MAXR) return EAGLE3_EUNSUPPORTED;
  if (w->vocab > 64 * TK_CHUNK) return EAGLE3_EUNSUPPORTED;
  return EAGLE3_OK;
}

size_t draft_workspace(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B, int max_prefix) {
  if (draft_check(w, t, B, max_prefix) != EAGLE3_OK) return 0;
  return make_plan(w, t, B, max_prefix, nullptr).bytes;
}

static int draft_common(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B, const void* h_low,
                        const void* h_mid, const void* h_high, const int32_t* root_tok, const void* kpre,
                        const void* vpre, const int32_t* cu_prefix, int max_prefix, int32_t* tokens,
                        int32_t* parents, int32_t* depth, float* score, int32_t* n_nodes,
                        const eagle3_draft_debug* dbg, const SampCfg& sc, void* ws, size_t ws_bytes,
                        hipStream_t s) {
  int st = draft_check(w, t, B, max_prefix);
  if (st) return st;
  if (!h_low || !h_mid || !h_high || !root_tok || !cu_prefix || !tokens || !parents || !depth ||
      !score || !n_nodes)
    return EAGLE3_EINVAL;
  if (max_prefix > 0 && (!kpre || !vpre)) return EAGLE3_EINVAL;
  for (const void* ptr : {h_low, h_mid, h_high, kpre, vpre, w->embed, w->w_fuse, w->g_embed, w->g_feat,
                          w->g_mlp, w->g_final, w->w_qkv, w->w_o, w->w_gate_up, w->w_down, w->w_lm})
    if ((uintptr_t)ptr % 16) return EAGLE3_EINVAL;
  Plan p = make_plan(w, t, B, max_prefix, nullptr);
  if (!ws || ws_bytes < p.bytes) return EAGLE3_EWORKSPACE;
  p = make_plan(w, t, B, max_prefix, ws);
  if (w->dtype == EAGLE3_BF16)
    return run_draft<bf16>(w, p, h_low, h_mid, h_high, root_tok, kpre, vpre, cu_prefix, tokens, parents,
                           depth, score, n_nodes, dbg, sc, s);
  return run_draft<float>(w, p, h_low, h_mid, h_high, root_tok, kpre, vpre, cu_prefix, tokens, parents,
                          depth, score, n_nodes, dbg, sc, s);
}

int draft_expand(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B, const void* h_low,
                 const void* h_mid, const void* h_high, const int32_t* root_tok, const void* kpre,
                 const void* vpre, const int32_t* cu_prefix, int max_prefix, int32_t* tokens,
                 int32_t* parents, int32_t* depth, float* score, int32_t* n_nodes,
                 const eagle3_draft_debug* dbg, void* ws, size_t ws_bytes, hipStream_t s) {
  SampCfg sc = {};
  return draft_common(w, t, B, h_low, h_mid, h_high, root_tok, kpre, vpre, cu_prefix, max_prefix, tokens,
                      parents, depth, score, n_nodes, dbg, sc, ws, ws_bytes, s);
}

int draft_expand_sampled(const eagle3_drafter* w, const eagle3_tree_cfg* t, int B, float temperature,
                         uint64_t seed, uint64_t round, const void* h_low, const void* h_mid,
                         const void* h_high, const int32_t* root_tok, const void* kpre, const void* vpre,
                         const int32_t* cu_prefix, int max_prefix, int32_t* tokens, int32_t* parents,
                         int32_t* depth, float* score, int32_t* n_nodes, float* slot_logits,
                         int32_t* draft_row, const eagle3_draft_debug* dbg, void* ws, size_t ws_bytes,
                         hipStream_t s) {
  if (!(temperature > 0.f) || temperature == __builtin_huge_valf()) return EAGLE3_EINVAL;
  if (!slot_logits || !draft_row || (uintptr_t)slot_logits % 16) return EAGLE3_EINVAL;
  if (!w) return EAGLE3_EINVAL;
  SampCfg sc;
  sc.on = 1;
  sc.invT = 1.0f / temperature;
  sc.seed_lo = (uint32_t)seed;
  sc.seed_hi = (uint32_t)(seed >> 32);
  sc.rnd = (uint32_t)round;
  sc.V = w->vocab;
  sc.slot_logits = slot_logits;
  sc.draft_row = draft_row;
  return draft_common(w, t, B, h_low, h_mid, h_high, root_tok, kpre, vpre, cu_prefix, max_prefix, tokens,
                      parents, depth, score, n_nodes, dbg, sc, ws, ws_bytes, s);
}

}  // namespace e3h
