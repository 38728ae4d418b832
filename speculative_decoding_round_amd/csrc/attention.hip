// Tree-masked attention over prefix KV + tree KV (split-KV partials) and the LSE merge.
//
// One workgroup = 4 waves = 64 query rows of one (request, KV head), where a row is a
// (node, query head) pair of that KV head's group, for one key split.  K and V tiles of
// 64 keys are staged through LDS (K row-major, V transposed), scores are formed as
// S^T = K Q^T with 16x16 MFMA so that every lane owns one query row, the online softmax
// runs in the log2 domain, and O^T += V^T P^T consumes the probabilities straight from the
// score registers.  Tree keys are masked per row by the ancestor bitmask.
#include "common.h"
#include "internal.h"

using namespace e3;

namespace {

constexpr int KT = 64;     // keys per tile
constexpr int ROWS = 64;   // query rows per workgroup (16 per wave)

template <typename T, int DH>
struct AttnSmem {
  static constexpr int EPC = Vec<T>::N;
  static constexpr int KPAD = EPC;           // one 16-byte chunk of padding per K row
  static constexpr int VPAD = 4;
  static constexpr int KROW = DH + KPAD;
  static constexpr int VROW = KT + VPAD;
  T k[KT * KROW];
  T vt[DH * VROW];
};

struct DevArgs {
  int B, Hq, Hkv, G;
  const void* q;
  const int32_t* q_cu;
  int q_stride, q_rows_total;
  const void* kt;
  const void* vt;
  const int32_t* kt_cu;
  int kt_stride, kt_count;
  const uint64_t* mask;
  int W64;
  const void* kp;
  const void* vp;
  const int32_t* p_cu;
  float scale_log2;
  int S;
  float* o_part;
  float* lse_part;
};

template <typename T, int DH>
__global__ __launch_bounds__(256) void k_tree_attn(DevArgs a) {
  constexpr int EPC = Vec<T>::N;
  constexpr int QCH = DH / (4 * EPC);          // 16-byte chunks per lane for one q row
  constexpr int CPR = DH / EPC;                // 16-byte chunks per key row
  constexpr int NDT = DH / 16;                 // output dim tiles
  using SM = AttnSmem<T, DH>;
  __shared__ SM sm;

  const int b = blockIdx.y / a.Hkv;
  const int c = blockIdx.y % a.Hkv;
  const int split = blockIdx.z;
  const int q0 = a.q_cu ? a.q_cu[b] : b * a.q_stride;
  const int nq = a.q_cu ? a.q_cu[b + 1] - q0 : a.q_stride;
  const int R = nq * a.G;
  const int rb0 = blockIdx.x * ROWS;
  if (rb0 >= R) return;

  // key range of this split
  const bool tree = split == a.S;
  int k_lo = 0, k_hi = 0;
  const T* kbase;
  const T* vbase;
  if (!tree) {
    const int p0 = a.p_cu ? a.p_cu[b] : 0;
    const int P = a.p_cu ? a.p_cu[b + 1] - p0 : 0;
    const int chunk = (P + a.S - 1) / a.S;
    k_lo = min(P, split * chunk);
    k_hi = min(P, k_lo + chunk);
    kbase = reinterpret_cast<const T*>(a.kp) + ((size_t)p0 * a.Hkv + c) * DH;
    vbase = reinterpret_cast<const T*>(a.vp) + ((size_t)p0 * a.Hkv + c) * DH;
  } else {
    const int t0 = a.kt_cu ? a.kt_cu[b] : b * a.kt_stride;
    k_hi = a.kt_cu ? a.kt_cu[b + 1] - t0 : a.kt_count;
    kbase = reinterpret_cast<const T*>(a.kt) + ((size_t)t0 * a.Hkv + c) * DH;
    vbase = reinterpret_cast<const T*>(a.vt) + ((size_t)t0 * a.Hkv + c) * DH;
  }
  const size_t kstride = (size_t)a.Hkv * DH;   // elements between consecutive keys

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int r = rb0 + wid * 16 + r16;
  const bool row_ok = r < R;
  const int node = row_ok ? r / a.G : 0;
  const int head = c * a.G + (row_ok ? r % a.G : 0);
  const size_t qrow = (size_t)(q0 + node);

  // this lane's query row (B operand of S^T = K Q^T)
  u32x4 qv[QCH];
  {
    const T* qp = reinterpret_cast<const T*>(a.q) + (qrow * a.Hq + head) * DH;
#pragma unroll
    for (int dc = 0; dc < QCH; ++dc)
      qv[dc] = row_ok ? ld16(qp + dc * 4 * EPC + g * EPC) : u32x4{0, 0, 0, 0};
  }
  uint64_t mrow[4] = {0, 0, 0, 0};
  if (tree && row_ok) {
    for (int w = 0; w < a.W64 && w < 4; ++w) mrow[w] = a.mask[qrow * a.W64 + w];
  }

  floatx4 acc[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  // cooperative tile loads: chunk id -> (key, 16-byte piece)
  constexpr int CHUNKS = KT * CPR;               // per tensor per tile
  constexpr int PER_T = CHUNKS / 256;            // per thread
  u32x4 kreg[PER_T], vreg[PER_T];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int id = threadIdx.x + u * 256;
      const int key = id / CPR, pc = id % CPR;
      const int kk = t0 + key;
      if (kk < k_hi) {
        kreg[u] = ld16(kbase + (size_t)kk * kstride + pc * EPC);
        vreg[u] = ld16(vbase + (size_t)kk * kstride + pc * EPC);
      } else {
        kreg[u] = u32x4{0, 0, 0, 0};
        vreg[u] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int id = threadIdx.x + u * 256;
      const int key = id / CPR, pc = id % CPR;
      st16(&sm.k[key * SM::KROW + pc * EPC], kreg[u]);
      const T* vv = reinterpret_cast<const T*>(&vreg[u]);
#pragma unroll
      for (int e = 0; e < EPC; ++e) sm.vt[(pc * EPC + e) * SM::VROW + key] = vv[e];
    }
  };

  if (k_lo < k_hi) load_tile(k_lo);
  for (int t0 = k_lo; t0 < k_hi; t0 += KT) {
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (t0 + KT < k_hi) load_tile(t0 + KT);  // prefetch next tile into registers

    // scores for 4 sub-tiles of 16 keys: lane holds keys st*16 + 4g + i of row r16
    floatx4 s[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      s[st] = floatx4{0.f, 0.f, 0.f, 0.f};
      const T* kr = &sm.k[(st * 16 + r16) * SM::KROW + g * EPC];
#pragma unroll
      for (int dc = 0; dc < QCH; ++dc) s[st] = Mfma<T>::run(ld16(kr + dc * 4 * EPC), qv[dc], s[st]);
    }
    float tmax = kNegInf;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = t0 + st * 16 + 4 * g + i;
        bool vis = key < k_hi;
        if (tree) vis = vis && ((mrow[(key >> 6) & 3] >> (key & 63)) & 1ull);
        const float v = vis ? s[st][i] * a.scale_log2 : kNegInf;
        s[st][i] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = row_reduce(tmax, OpMax());
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(s[st][i] - m_use);
        s[st][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;

    // O^T += V^T P^T
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int pc = 0; pc < 2; ++pc) {
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = static_cast<bf16>(s[2 * pc][i]);
          pb[4 + i] = static_cast<bf16>(s[2 * pc + 1][i]);
        }
        const u32x4 pbu = __builtin_bit_cast(u32x4, pb);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const T* vr = &sm.vt[(dt * 16 + r16) * SM::VROW];
          const uint2 lo = *reinterpret_cast<const uint2*>(vr + (2 * pc) * 16 + 4 * g);
          const uint2 hi = *reinterpret_cast<const uint2*>(vr + (2 * pc + 1) * 16 + 4 * g);
          acc[dt] = Mfma<T>::run(u32x4{lo.x, lo.y, hi.x, hi.y}, pbu, acc[dt]);
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4 pbu = u32x4{__float_as_uint(s[st][0]), __float_as_uint(s[st][1]),
                                __float_as_uint(s[st][2]), __float_as_uint(s[st][3])};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const T* vr = &sm.vt[(dt * 16 + r16) * SM::VROW];
          acc[dt] = Mfma<T>::run(ld16(vr + st * 16 + 4 * g), pbu, acc[dt]);
        }
      }
    }
  }

  const float l = row_reduce(l_run, OpAdd());
  if (!row_ok) return;
  const size_t orow = ((size_t)split * a.q_rows_total + qrow) * a.Hq + head;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = a.o_part + orow * DH;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    floatx4 v = acc[dt] * inv;
    *reinterpret_cast<floatx4*>(op + dt * 16 + 4 * g) = v;
  }
  if (g == 0) a.lse_part[orow] = l > 0.f ? (m_run + log2f(l)) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------------------------------
// LSE merge: one thread per (row, 4 dims); partials merged in split order.  The split
// LSEs are read first (independent loads), then the weighted partials, eight at a time.
// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_lse_merge(int S, int rows, int Dh,
                                                   const float* __restrict__ o_part,
                                                   const float* __restrict__ lse_part,
                                                   T* __restrict__ o, float* __restrict__ lse) {
  const int d4 = Dh / 4;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)rows * d4) return;
  const int row = (int)(idx / d4), q = (int)(idx % d4);
  float m = kNegInf;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float l8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) l8[u] = s0 + u < S ? lse_part[(size_t)(s0 + u) * rows + row] : kNegInf;
#pragma unroll
    for (int u = 0; u < 8; ++u) m = fmaxf(m, l8[u]);
  }
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != kNegInf) {
    for (int s0 = 0; s0 < S; s0 += 8) {
      float w8[8];
      floatx4 v8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = s0 + u < S;
        const float ls = ok ? lse_part[(size_t)(s0 + u) * rows + row] : kNegInf;
        w8[u] = ls == kNegInf ? 0.f : expf(ls - m);
        v8[u] = ok ? *reinterpret_cast<const floatx4*>(o_part + ((size_t)(s0 + u) * rows + row) * Dh + 4 * q)
                   : floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (w8[u] != 0.f) acc += v8[u] * w8[u];
        wsum += w8[u];
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  T* op = o + (size_t)row * Dh + 4 * q;
#pragma unroll
  for (int i = 0; i < 4; ++i) op[i] = from_f32<T>(acc[i] * inv);
  if (lse && q == 0) lse[row] = wsum > 0.f ? m + logf(wsum) : kNegInf;
}

template <typename T, int DH>
int launch_attn_t(const e3h::AttnArgs& h, hipStream_t s) {
  DevArgs a;
  a.B = h.B;
  a.Hq = h.Hq;
  a.Hkv = h.Hkv;
  a.G = h.Hq / h.Hkv;
  a.q = h.q;
  a.q_cu = h.q_cu;
  a.q_stride = h.q_stride;
  a.q_rows_total = h.q_rows_total;
  a.kt = h.kt;
  a.vt = h.vt;
  a.kt_cu = h.kt_cu;
  a.kt_stride = h.kt_stride;
  a.kt_count = h.kt_count;
  a.mask = h.mask;
  a.W64 = h.W64;
  a.kp = h.kp;
  a.vp = h.vp;
  a.p_cu = h.p_cu;
  a.scale_log2 = h.scale * kLog2e;
  a.S = h.S;
  a.o_part = h.o_part;
  a.lse_part = h.lse_part;
  const int rb = (h.max_q_per_req * a.G + ROWS - 1) / ROWS;
  dim3 grid(rb, h.B * h.Hkv, h.S + 1);
  hipLaunchKernelGGL((k_tree_attn<T, DH>), grid, dim3(256), 0, s, a);
  return e3h::launch_status();
}

}  // namespace

namespace e3h {

// Prefix splits: aim at ~1024 workgroups in total, but give every split at least
// 128 keys per 64-row block so that a split's fp32 partial (64 rows x Dh x 4 B per row
// block) stays at or below half of the bf16 K+V bytes it streams.
int attention_splits(int B, int Hkv, int rows_per_kv, int max_prefix, int n_splits) {
  if (n_splits > 0) return n_splits;
  if (max_prefix <= 0 || B <= 0 || Hkv <= 0) return 1;
  const int rb = rows_per_kv > 0 ? (rows_per_kv + ROWS - 1) / ROWS : 1;
  const long base = (long)B * Hkv * rb;
  long s = (1024 + base - 1) / base;
  const long min_keys = 128L * rb;
  const long max_s = (max_prefix + min_keys - 1) / min_keys;
  if (s > max_s) s = max_s;
  if (s > 256) s = 256;
  return s < 1 ? 1 : (int)s;
}

int launch_tree_attention(const AttnArgs& a, hipStream_t s, const char* tag) {
  if (a.W64 > 4) return EAGLE3_EUNSUPPORTED;
  if (a.max_q_per_req <= 0 || a.B <= 0) return EAGLE3_OK;
  ProfScope ps(tag, s);
  if (a.dtype == EAGLE3_BF16) {
    if (a.Dh == 128) return launch_attn_t<bf16, 128>(a, s);
    if (a.Dh == 64) return launch_attn_t<bf16, 64>(a, s);
  } else {
    if (a.Dh == 128) return launch_attn_t<float, 128>(a, s);
    if (a.Dh == 64) return launch_attn_t<float, 64>(a, s);
  }
  return EAGLE3_EUNSUPPORTED;
}

int launch_lse_merge(int S, int rows, int Dh, const float* o_part, const float* lse_part,
                     int out_dtype, void* o, float* lse, hipStream_t s, const char* tag) {
  if (rows <= 0) return EAGLE3_OK;
  ProfScope ps(tag, s);
  const long n = (long)rows * (Dh / 4);
  dim3 grid((unsigned)((n + 255) / 256));
  if (out_dtype == EAGLE3_BF16)
    hipLaunchKernelGGL(k_lse_merge<bf16>, grid, dim3(256), 0, s, S, rows, Dh, o_part, lse_part,
                       (bf16*)o, lse);
  else
    hipLaunchKernelGGL(k_lse_merge<float>, grid, dim3(256), 0, s, S, rows, Dh, o_part, lse_part,
                       (float*)o, lse);
  return launch_status();
}

}  // namespace e3h
