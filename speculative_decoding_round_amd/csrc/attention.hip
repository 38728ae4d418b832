// Tree-masked attention over prefix KV + tree KV (split-KV partials) and the LSE merge.
//
// One workgroup = 4 waves = 64 query rows of one (request, KV head), where a row is a
// (node, query head) pair of that KV head's group, for one key split.  K and V tiles of
// 64 keys are staged through LDS (K row-major, V transposed), scores are formed as
// S^T = K Q^T with 16x16 MFMA so that every lane owns one query row, the online softmax
// runs in the log2 domain, and O^T += V^T P^T consumes the probabilities straight from the
// score registers.  Tree keys are masked per row by the ancestor bitmask.
#include <algorithm>

#include "common.h"
#include "internal.h"

using namespace e3;

namespace {

constexpr int KT = 64;     // keys per tile

// Keys per prefix split: ceil(P / S) rounded up to a multiple of 128, so that every split
// but the last is a whole number of key tiles of either kernel.
__device__ __forceinline__ int split_keys(int P, int S) { return ((P + S - 1) / S + 127) / 128 * 128; }
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
  int n_rb;   // row blocks per (request, KV head) (bf16 kernel)
  int causal_len;   // causal mode: sequence length (request b = positions b * q_stride ..)
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
    const int chunk = split_keys(P, a.S);
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
// bf16 attention with LDS-DMA staged K/V (gfx950).
//
// K and V tiles go from HBM straight into LDS (global_load_lds, 16 bytes per lane, no
// register staging) through an NST-deep ring of stages, so several tiles are in flight
// per workgroup.  A stage holds WK sub-tiles of KTW keys, one per key group of waves;
// the WR = 4 / WK waves of a key group own disjoint query-row tiles and share its
// sub-tile.  With WK > 1 the key groups keep separate softmax states for the same rows,
// combined in LDS at the end.
//
// A key row's 16-byte chunks are stored XOR-swizzled (chunk c of key k at position
// c ^ swz(k)) so that both LDS read patterns are bank-conflict free: the 16 keys of one
// K operand read at a fixed chunk, and the 4 keys x 2 chunks of one transpose read.
// V is consumed through ds_read_b64_tr_b16: within each 16-lane group, the lane at
// (key row r, dim quad q) supplies the address of V[key0 + r][dim0 + 4q], and lane j of
// the group receives V[key0 .. key0+3][dim0 + j], which is the MFMA operand layout
// (4 consecutive keys of one dimension) without a transpose on store.
//
// Scores: S^T = K Q^T (16x16x32 MFMA, K from LDS as operand A, the wave's query rows
// stationary as operand B), so lane l holds row l % 16, keys 4*(l/16) + i of each 16-key
// block.  P^T feeds O^T += V^T P^T with the k-order {4g..4g+3, 16+4g..16+4g+3} on both
// operands.  The softmax runs in the log2 domain.
// ---------------------------------------------------------------------------------------
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const char lds_cchar;

// Byte address of a __shared__ object in the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_cchar*)p;
}

// One 16-byte-per-lane LDS DMA: lane l's 16 bytes land at LDS byte lds_base + 16 l.
// Non-temporal: the K/V stream is read once.  Written as inline assembly so that the
// compiler does not see an outstanding LDS write: it would otherwise drain every DMA
// (s_waitcnt vmcnt(0)) before each later LDS read, including the reads of stages whose
// data arrived long ago, and no stage could be in flight during the math.  Completion is
// ordered explicitly instead (wait_vm + barrier before a stage is read).
// s_waitcnt immediate (gfx9 encoding) for vmcnt(0) with expcnt and lgkmcnt left open.
constexpr int kWaitVm0 = 0x0F70;

// Address = wave-uniform base (SGPRs) + this lane's 32-bit byte offset.
// M0 is written by the asm and named as clobbered; the compiler does not preserve reserved
// registers across asm (hence its warning), which is harmless: nothing else in these
// kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_nt_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase),
               "s"(lds_base)
               : "memory", "m0");
}
// The same with the cache policy left at its default: for streams that other workgroups
// re-read through L2.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int CPR>
__device__ __forceinline__ int kv_swz(int key) {
  if constexpr (CPR == 16) return ((key & 7) << 1) | ((key >> 3) & 1);
  else return ((key & 3) << 1) | ((key >> 2) & 1);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// all of this wave's LDS reads done, then the workgroup barrier (no global-memory wait)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int DH, int QT, int WK, int KTW, int NST>
struct DmaCfg {
  static constexpr int CPR = DH / 8;                        // 16-byte chunks per key row
  static constexpr int WR = 4 / WK;                         // row waves per key group
  static constexpr int ROWS = WR * QT * 16;                 // query rows per workgroup
  static constexpr int KITER = WK * KTW;                    // keys per iteration
  static constexpr int SUB = KTW * CPR * 16;                // bytes of one K (or V) sub-tile
  static constexpr int STAGE = WK * 2 * SUB;                // bytes per stage
  static constexpr int PER = STAGE / 4096;                  // DMA instructions per thread per stage
  static constexpr int MERGE = (WK - 1) * WR * QT * (DH / 16) * 64 * 16 + 2 * (WK - 1) * WR * QT * 64 * 4;
  static constexpr int LDS = NST * STAGE > MERGE ? NST * STAGE : MERGE;
  static_assert(STAGE % 4096 == 0, "stage must be a whole number of 4 KB rounds");
  static_assert(KTW % 32 == 0, "sub-tile must hold whole 32-key PV steps");
  static_assert(PER <= 16 && PER * (NST - 1) <= 63, "outstanding DMA must fit the vmcnt counter");
  static_assert(NST >= 2 && NST <= 4, "the wait schedule covers 2..4 stages");
};

// Softmax reference: rows keep a reference max m (log2 domain) and exponentiate against
// it; m is raised (and O, l rescaled) only when some row of the wave sees a score more
// than 2^8 above its reference, so p <= 2^8 and the accumulator is rarely touched.
constexpr float kRescaleLog2 = 8.f;

// CAUSAL: every position of a sequence is a query row ([P4] USP step 1, the main causal
// attention).  Request b is the block of q_stride positions from b * q_stride; its rows see
// the keys 0 .. position (the sequence itself, from key 0), so a row block streams the keys
// up to its last position and masks the tiles that reach past a row's position; there is
// no tree split, and the output is split 0 = (Out_main, LSE_main).  Blocks are taken
// largest first (the work grows with the position), and K/V are read with the default
// cache policy: every block of a KV head re-reads the same keys.
template <int DH, int QT, int WK, int KTW, int NST, bool CAUSAL = false>
__global__ __launch_bounds__(256) void k_tree_attn_dma(DevArgs a) {
  using C = DmaCfg<DH, QT, WK, KTW, NST>;
  constexpr int CPR = C::CPR, WR = C::WR, NDT = DH / 16, NDC = DH / 32, NST16 = KTW / 16;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  __shared__ uint64_t smask[4][QT][16][4];

  // Workgroups that share K/V (the row blocks of one request, KV head and split) are
  // numbered so that they fall on the same XCD (workgroups go to XCDs round-robin), where
  // they share that XCD's L2.
  const int n_groups = a.B * a.Hkv * (CAUSAL ? 1 : a.S + 1);
  const int id = blockIdx.x, xcd = id % 8, t = id / 8;
  const int rbk = t % a.n_rb;
  const int grp = (t / a.n_rb) * 8 + xcd;
  if (grp >= n_groups) return;
  const int split = CAUSAL ? 0 : grp % (a.S + 1);
  const int bc = CAUSAL ? grp : grp / (a.S + 1);
  const int b = CAUSAL ? a.B - 1 - bc / a.Hkv : bc / a.Hkv;
  const int c = bc % a.Hkv;
  const int q0 = a.q_cu ? a.q_cu[b] : b * a.q_stride;
  const int nq = a.q_cu ? a.q_cu[b + 1] - q0 : (CAUSAL ? min(a.q_stride, a.causal_len - q0) : a.q_stride);
  const int R = nq * a.G;
  const int rb0 = rbk * C::ROWS;
  if (rb0 >= R) return;

  const bool tree = !CAUSAL && split == a.S;
  int k_lo = 0, k_hi = 0;
  const bf16* kbase;
  const bf16* vbase;
  if (CAUSAL) {
    // keys 0 .. the row block's last position
    k_hi = q0 + min(nq, (rb0 + C::ROWS - 1) / a.G + 1);
    kbase = reinterpret_cast<const bf16*>(a.kp) + (size_t)c * DH;
    vbase = reinterpret_cast<const bf16*>(a.vp) + (size_t)c * DH;
  } else if (!tree) {
    const int p0 = a.p_cu ? a.p_cu[b] : 0;
    const int P = a.p_cu ? a.p_cu[b + 1] - p0 : 0;
    const int chunk = split_keys(P, a.S);
    k_lo = min(P, split * chunk);
    k_hi = min(P, k_lo + chunk);
    kbase = reinterpret_cast<const bf16*>(a.kp) + ((size_t)p0 * a.Hkv + c) * DH;
    vbase = reinterpret_cast<const bf16*>(a.vp) + ((size_t)p0 * a.Hkv + c) * DH;
  } else {
    const int t0 = a.kt_cu ? a.kt_cu[b] : b * a.kt_stride;
    k_hi = a.kt_cu ? a.kt_cu[b + 1] - t0 : a.kt_count;
    kbase = reinterpret_cast<const bf16*>(a.kt) + ((size_t)t0 * a.Hkv + c) * DH;
    vbase = reinterpret_cast<const bf16*>(a.vt) + ((size_t)t0 * a.Hkv + c) * DH;
  }
  const int kstride = a.Hkv * DH;   // elements between consecutive keys
  const int n_it = k_hi > k_lo ? (k_hi - k_lo + C::KITER - 1) / C::KITER : 0;
  const float sc = a.scale_log2;    // > 0

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wk = w / WR, wr = w % WR;
  const int r16 = lane & 15, g = lane >> 4;

  // this wave's query rows (operand B of S^T = K Q^T); in the tree split, their mask words
  // go to this wave's own LDS slots (one word is read back per key tile)
  u32x4 qv[QT][NDC];
  int rowid[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = rb0 + (wr * QT + qt) * 16 + r16;
    const bool ok = r < R;
    rowid[qt] = ok ? r : -1;
    const int node = ok ? r / a.G : 0;
    const int head = c * a.G + (ok ? r % a.G : 0);
    const bf16* qp = reinterpret_cast<const bf16*>(a.q) + ((size_t)(q0 + node) * a.Hq + head) * DH;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) qv[qt][dc] = ok ? ld16(qp + dc * 32 + g * 8) : u32x4{0, 0, 0, 0};
    if (tree) smask[w][qt][r16][g] = (ok && g < a.W64) ? a.mask[(size_t)(q0 + node) * a.W64 + g] : 0ull;
  }

  // DMA: thread chunk q = (u*4 + w)*64 + lane of a stage, decoded as (key group, K|V,
  // key, position); position p holds the key's chunk p ^ swz(key).  A lane's byte offset
  // from the iteration's first key is the same in every iteration, and the K|V choice of
  // instruction u is the same for all lanes of a wave (CPR * KTW >= 64), so the stream
  // position lives in two scalar bases that advance by one iteration of keys; only the
  // last iteration clamps keys to the range end.
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t voff[C::PER], vpos[C::PER];
  int relk[C::PER];
  bool isv[C::PER];
#pragma unroll
  for (int u = 0; u < C::PER; ++u) {
    const int q = (u * 4 + wu) * 64 + lane;
    const int pos = q % CPR;
    const int key = (q / CPR) % KTW;
    isv[u] = ((u * 4 + wu) * 64 / (CPR * KTW)) % 2 != 0;
    const int kg = q / (2 * CPR * KTW);
    relk[u] = kg * KTW + key;
    vpos[u] = (uint32_t)(pos ^ kv_swz<CPR>(key)) * 16u;
    voff[u] = (uint32_t)relk[u] * (uint32_t)kstride * 2u + vpos[u];
  }
  const uint32_t smem_lds = lds_addr(smem);
  const char* kstream = reinterpret_cast<const char*>(kbase);
  const char* vstream = reinterpret_cast<const char*>(vbase);
  const size_t it_bytes = (size_t)C::KITER * kstride * 2;
  auto issue = [&](int it) {
    const uint32_t st = smem_lds + (it % NST) * C::STAGE;
    const int t0 = k_lo + it * C::KITER;
    const bool whole = t0 + C::KITER <= k_hi;
    const size_t adv = (size_t)k_lo * kstride * 2 + (size_t)it * it_bytes;
    const char* kb = kstream + adv;
    const char* vb = vstream + adv;
#pragma unroll
    for (int u = 0; u < C::PER; ++u) {
      uint32_t off = voff[u];
      if (!whole) off = (uint32_t)min(relk[u], k_hi - 1 - t0) * (uint32_t)kstride * 2u + vpos[u];
      if constexpr (CAUSAL) dma16_s(isv[u] ? vb : kb, off, st + (u * 4 + wu) * 1024);
      else dma16_nt_s(isv[u] ? vb : kb, off, st + (u * 4 + wu) * 1024);
    }
  };

  floatx4 acc[QT][NDT];
  // l_acc: each row's sum of P, formed by one more MFMA per 32 keys with a block of ones in
  // place of V^T (every element of the 16 x 16 result is the row's sum over those keys), so
  // the sum costs no vector adds and uses the same bf16 P as the output
  float m_ref[QT];
  floatx4 l_acc[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_ref[qt] = kNegInf;
    l_acc[qt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[qt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // per-lane LDS offsets (bytes within a sub-tile) of the K operand reads and V transpose reads
  int koff[NST16][NDC];
#pragma unroll
  for (int st = 0; st < NST16; ++st)
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      const int key = st * 16 + r16;
      koff[st][dc] = (key * CPR + ((dc * 4 + g) ^ kv_swz<CPR>(key))) * 16;
    }
  const int kr = (lane & 15) >> 2, dq = lane & 3;

  // The query rows (and mask words) are in registers / LDS before the stream starts.  This
  // wait is a real instruction the compiler accounts for: without it, the compiler (which
  // does not count the assembly DMAs) would keep the query loads pending and drain the
  // whole DMA ring (vmcnt(0)) before the first MFMA of every tile.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
#pragma unroll
  for (int s0 = 0; s0 < NST - 1; ++s0)
    if (s0 < n_it) issue(s0);

  const bool wave_active = rb0 + wr * QT * 16 < R;
  for (int it = 0; it < n_it; ++it) {
    if constexpr (NST >= 3) {
      if (it + NST - 2 < n_it) wait_vm<C::PER * (NST - 2)>();
      else if (it + 1 < n_it) wait_vm<C::PER * (NST - 3 > 0 ? NST - 3 : 0)>();
      else wait_vm<0>();
    } else {
      wait_vm<0>();
    }
    lds_barrier();  // stage it complete for every wave; stage it-1 fully consumed
    if (it + NST - 1 < n_it) issue(it + NST - 1);
    // a wave whose row tiles all lie past the last row only moves data and meets the barriers
    if (!wave_active) continue;

    const char* ks = smem + (it % NST) * C::STAGE + (wk * 2) * C::SUB;
    const char* vs = ks + C::SUB;
    const int kbase_it = k_lo + it * C::KITER + wk * KTW;

    // raw scores S^T for NST16 blocks of 16 keys
    floatx4 s[QT][NST16];
#pragma unroll
    for (int st = 0; st < NST16; ++st) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[qt][st] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(ks + koff[st][dc]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[qt][st] = Mfma<bf16>::run(kv, qv[qt][dc], s[qt][st]);
      }
    }
    // keys past the range end or outside the row's ancestor set -> -inf; whole prefix
    // tiles need no mask
    const int lim = k_hi - kbase_it;
    // causal: tiles reaching past the wave's first row position
    const bool cmask = CAUSAL && kbase_it + KTW - 1 > q0 + (rb0 + wr * QT * 16) / a.G;
    if (tree || lim < KTW || cmask) {
      const int word = (kbase_it >> 6) & 3, sh = kbase_it & 63;  // a sub-tile lies in one word
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const uint64_t bits = tree ? (smask[w][qt][r16][word] >> sh) >> (4 * g) : ~0ull;
        // keys visible to this lane's row: relative key < rlim (causal: key <= position)
        const int rlim = CAUSAL ? min(lim, q0 + max(rowid[qt], 0) / a.G + 1 - kbase_it) : lim;
#pragma unroll
        for (int st = 0; st < NST16; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool vis = st * 16 + 4 * g + i < rlim && ((bits >> (st * 16 + i)) & 1ull);
            if (!vis) s[qt][st][i] = kNegInf;
          }
      }
    }
    // online softmax against the reference max (scale > 0 is folded into the exponent)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float lmax = kNegInf;
#pragma unroll
      for (int st = 0; st < NST16; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, s[qt][st][i]);
      // the lane's maximum decides whether its row passes the reference (scaling by sc > 0
      // keeps the order), so the row maximum is reduced across lanes only when one does
      if (__any(lmax * sc > m_ref[qt] + kRescaleLog2)) {
        const float tmax = row_reduce(lmax, OpMax()) * sc;
        const float m_new = fmaxf(m_ref[qt], tmax);
        const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_ref[qt] - m_new);
        l_acc[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[qt][dt] *= alpha;
        m_ref[qt] = m_new;
      }
      const float nm = m_ref[qt] == kNegInf ? 0.f : -m_ref[qt];
#pragma unroll
      for (int st = 0; st < NST16; ++st)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[qt][st][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qt][st][i], sc, nm));
    }
    // O^T += V^T P^T, 32 keys per step
#pragma unroll
    for (int pc = 0; pc < KTW / 32; ++pc) {
      u32x4 pb[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        bf16x8 p8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p8[i] = static_cast<bf16>(s[qt][2 * pc][i]);
          p8[4 + i] = static_cast<bf16>(s[qt][2 * pc + 1][i]);
        }
        pb[qt] = __builtin_bit_cast(u32x4, p8);
      }
      const int ka = pc * 32 + 4 * g + kr, kb = ka + 16;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int gc = 2 * dt + (dq >> 1);
        const int off = (dq & 1) * 8;
        const char* pa = vs + (ka * CPR + (gc ^ kv_swz<CPR>(ka))) * 16 + off;
        const char* pbp = vs + (kb * CPR + (gc ^ kv_swz<CPR>(kb))) * 16 + off;
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(pa));
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(pbp));
        const uint2 lu = __builtin_bit_cast(uint2, lo), hu = __builtin_bit_cast(uint2, hi);
        const u32x4 va = u32x4{lu.x, lu.y, hu.x, hu.y};
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) acc[qt][dt] = Mfma<bf16>::run(va, pb[qt], acc[qt][dt]);
      }
      const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) l_acc[qt] = Mfma<bf16>::run(ones, pb[qt], l_acc[qt]);
    }
  }

  float l_tot[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) l_tot[qt] = l_acc[qt][0];

  if constexpr (WK > 1) {
    // key groups 1.. hand their (m, l, O) to group 0 through LDS
    __syncthreads();
    floatx4* mo = reinterpret_cast<floatx4*>(smem);
    float* ml = reinterpret_cast<float*>(smem + (WK - 1) * WR * QT * NDT * 64 * 16);
    if (wk > 0) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int slot = ((wk - 1) * WR + wr) * QT + qt;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) mo[(slot * NDT + dt) * 64 + lane] = acc[qt][dt];
        ml[(2 * slot) * 64 + lane] = m_ref[qt];
        ml[(2 * slot + 1) * 64 + lane] = l_tot[qt];
      }
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mm = m_ref[qt];
#pragma unroll
      for (int o = 1; o < WK; ++o) mm = fmaxf(mm, ml[(2 * (((o - 1) * WR + wr) * QT + qt)) * 64 + lane]);
      const float e0 = m_ref[qt] == kNegInf ? 0.f : exp2f(m_ref[qt] - mm);
      float lt = l_tot[qt] * e0;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[qt][dt] *= e0;
#pragma unroll
      for (int o = 1; o < WK; ++o) {
        const int slot = ((o - 1) * WR + wr) * QT + qt;
        const float mo_ = ml[(2 * slot) * 64 + lane];
        const float eo = mo_ == kNegInf ? 0.f : exp2f(mo_ - mm);
        lt += ml[(2 * slot + 1) * 64 + lane] * eo;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[qt][dt] += mo[(slot * NDT + dt) * 64 + lane] * eo;
      }
      m_ref[qt] = mm;
      l_tot[qt] = lt;
    }
  }

#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int r = rowid[qt];
    if (r < 0) continue;
    const int node = r / a.G;
    const int head = c * a.G + r % a.G;
    const size_t orow = ((size_t)split * a.q_rows_total + q0 + node) * a.Hq + head;
    const float l = l_tot[qt];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* op = a.o_part + orow * DH;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<floatx4*>(op + dt * 16 + 4 * g) = acc[qt][dt] * inv;
    if (g == 0) a.lse_part[orow] = l > 0.f ? (m_ref[qt] + log2f(l)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------------------
// LSE merge.  A row's split LSEs are read at once (one per lane or thread), giving
// m = max and the weights w_s = e^{LSE_s - m} in LDS; the weighted partials are then
// summed with eight loads in flight.  WPR = waves per row: with few splits one wave takes
// a row (four rows per workgroup; used when the head size has no thread-per-row kernel
// below); with many, the four waves of a workgroup take the splits s = w, w+4, ... of one
// row and their sums are added in wave order.  Every order is fixed, so the result is
// deterministic.
// ---------------------------------------------------------------------------------------
constexpr int MERGE_MAX_S = 512;
constexpr int MERGE_FEW_S = 16;   // up to this many splits: one wave per row

template <typename T, int WPR>
__global__ __launch_bounds__(256) void k_lse_merge(int S, int rows, int Dh,
                                                   const float* __restrict__ o_part,
                                                   const float* __restrict__ lse_part,
                                                   T* __restrict__ o, float* __restrict__ lse) {
  constexpr int SW = WPR == 1 ? MERGE_FEW_S : MERGE_MAX_S;
  __shared__ float sw[4 / WPR][SW];
  __shared__ float red[32];
  __shared__ floatx4 part[4][32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = WPR == 1 ? blockIdx.x * 4 + w : blockIdx.x;
  const int slot = WPR == 1 ? w : 0;
  float m, wsum;
  if constexpr (WPR == 1) {
    if (row >= rows) return;   // whole wave; no block barrier below
    const float l0 = lane < S ? lse_part[(size_t)lane * rows + row] : kNegInf;
    m = wave_max(l0);
    const float w0 = (m == kNegInf || l0 == kNegInf) ? 0.f : expf(l0 - m);
    if (lane < S) sw[slot][lane] = w0;
    wsum = wave_sum(w0);
  } else {
    const float l0 = tid < S ? lse_part[(size_t)tid * rows + row] : kNegInf;
    const float l1 = tid + 256 < S ? lse_part[(size_t)(tid + 256) * rows + row] : kNegInf;
    m = block_max(fmaxf(l0, l1), red);
    const float w0 = (m == kNegInf || l0 == kNegInf) ? 0.f : expf(l0 - m);
    const float w1 = (m == kNegInf || l1 == kNegInf) ? 0.f : expf(l1 - m);
    if (tid < S) sw[0][tid] = w0;
    if (tid + 256 < S) sw[0][tid + 256] = w1;
    wsum = block_sum(w0 + w1, red);   // its barriers also order the LDS weights
  }
  const int d4 = Dh / 4;                          // float4 columns of a row (<= 32)
  const int s_first = WPR == 1 ? 0 : w, s_step = WPR == 1 ? 1 : 4;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  if (lane < d4) {
    const float* base = o_part + (size_t)row * Dh + 4 * lane;
    for (int s0 = s_first; s0 < S; s0 += 8 * s_step) {
      floatx4 v[8];
      float ww[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sp = s0 + s_step * u;
        ww[u] = sp < S ? sw[slot][sp] : 0.f;
        v[u] = (sp < S && ww[u] != 0.f) ? *reinterpret_cast<const floatx4*>(base + (size_t)sp * rows * Dh)
                                        : floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u] * ww[u];
    }
  }
  if constexpr (WPR > 1) {
    if (lane < d4) part[w][lane] = acc;
    __syncthreads();
    if (w != 0) return;
    if (lane < d4) {
      acc = part[0][lane] + part[1][lane];
      acc += part[2][lane];
      acc += part[3][lane];
    }
  }
  if (lane >= d4) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  T* op = o + (size_t)row * Dh + 4 * lane;
#pragma unroll
  for (int i = 0; i < 4; ++i) op[i] = from_f32<T>(acc[i] * inv);
  if (lse && lane == 0) lse[row] = wsum > 0.f ? m + logf(wsum) : kNegInf;
}

// LSE merge with few partials (S <= MERGE_FEW_S): a thread owns 4 output dimensions of one
// row.  It reads the row's S split LSEs into registers (the same words for all threads of the
// row), forms m = max and the weights itself, issues all S partial loads at once and sums them
// in split order; nothing is exchanged between lanes.  S is a template argument: with a
// run-time count the guarded loads are issued one after another.
template <typename T, int DH, int S>
__global__ __launch_bounds__(256) void k_lse_merge_rows(int rows, const float* __restrict__ o_part,
                                                        const float* __restrict__ lse_part,
                                                        T* __restrict__ o, float* __restrict__ lse) {
  constexpr int TPR = DH / 4;   // threads per row
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid / TPR;
  const int c = (int)(gid % TPR);
  if (row >= rows) return;
  float l[S];
  floatx4 v[S];
#pragma unroll
  for (int sp = 0; sp < S; ++sp) {
    l[sp] = lse_part[(size_t)sp * rows + row];
    v[sp] = __builtin_nontemporal_load(
        reinterpret_cast<const floatx4*>(o_part + ((size_t)sp * rows + row) * DH + 4 * c));
  }
  float m = kNegInf;
#pragma unroll
  for (int sp = 0; sp < S; ++sp) m = fmaxf(m, l[sp]);
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != kNegInf) {
#pragma unroll
    for (int sp = 0; sp < S; ++sp) {
      const float w = l[sp] == kNegInf ? 0.f : expf(l[sp] - m);
      wsum += w;
      acc += v[sp] * w;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  T* op = o + (size_t)row * DH + 4 * c;
  if constexpr (sizeof(T) == 2) {
    typedef __bf16 bf16x4v __attribute__((ext_vector_type(4)));
    bf16x4v ov;
#pragma unroll
    for (int i = 0; i < 4; ++i) ov[i] = static_cast<bf16>(acc[i] * inv);
    *reinterpret_cast<bf16x4v*>(op) = ov;      // one 8-byte store
  } else {
    *reinterpret_cast<floatx4*>(op) = acc * inv;
  }
  if (lse && c == 0) lse[row] = wsum > 0.f ? m + logf(wsum) : kNegInf;
}

template <typename T, int DH, int S>
void launch_merge_rows(int S_rt, int rows, const float* o_part, const float* lse_part, void* o, float* lse,
                       hipStream_t st) {
  if constexpr (S > 1) {
    if (S_rt < S) return launch_merge_rows<T, DH, S - 1>(S_rt, rows, o_part, lse_part, o, lse, st);
  }
  const long threads = (long)rows * (DH / 4);
  hipLaunchKernelGGL((k_lse_merge_rows<T, DH, S>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     rows, o_part, lse_part, (T*)o, lse);
}

// Workgroup shape of the bf16 kernel by query rows per (request, KV head):
// 0: <= 32 rows: 32 rows per workgroup (one 16-row tile per wave), keys split over two wave
//    pairs, four 32 KB stages (one workgroup per CU, three stages in flight: these launches
//    only stream K/V, and a deeper ring beats the 64 KB stages of a four-way key split);
// 1: <= 256 rows: 64 rows per workgroup, one 16-row tile per wave, keys shared;
// 2: more: 128 rows per workgroup, two 16-row tiles per wave, keys shared.
// Shapes 1 and 2 take 64 keys per iteration in two 32 KB stages: half the barriers and
// per-tile softmax steps per key of 32-key tiles in four 16 KB stages, at the same 64 KB of
// LDS (their launches are bound by the math, not the stream).
// Workgroups aimed for per launch: one per CU for shape 0; for shape 1 four rounds of the two
// resident per CU, which evens out ragged requests, or two when each (request, KV head) has
// one row block (every workgroup then streams K/V no other one reads, and its fixed start and
// end costs weigh more: batch-16 drafter steps 3.28 -> 3.23 ms per round); for shape 2 one
// round (hundreds of rows, math-bound), or, with one row block per (request, KV head), a
// little under one round (the 70B-shaped drafter steps: 14 prefix splits and 480 workgroups
// beat 16 and 544 by ~50 us per round, and 15 and 512 by ~30 us).
// Workgroup shape by query rows per KV head: <= 32 rows, keys split over the waves; 65 .. 128
// rows (e.g. ten drafted nodes x 8 heads per KV head) in one 128-row block, so each K/V split
// is streamed by one workgroup and the splits stay few; other rows up to 256 in 64-row blocks;
// more in 128-row blocks.
inline int attn_cfg(int rows) {
  if (rows <= 32) return 0;
  if (rows > 64 && rows <= 128) return 2;
  return rows <= 256 ? 1 : 2;
}
inline int attn_cfg_rows(int cfg) { return cfg == 0 ? 32 : cfg == 1 ? 64 : 128; }
// keys per iteration, for split sizing (shape 0 streams 64 per iteration, but its splits keep
// at least 128 keys, two iterations)
inline int attn_cfg_keys(int cfg) { return cfg == 0 ? 128 : 64; }
inline int attn_cfg_wgs(int cfg, long row_blocks) {
  if (cfg == 0) return 256;
  if (cfg == 1) return row_blocks == 1 ? 1024 : 2048;
  return row_blocks == 1 ? 448 : 512;
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
  const int rows = h.max_q_per_req * a.G;
  if constexpr (sizeof(T) == 2) {
    auto go = [&](auto kern, int rows_wg) {
      a.n_rb = (rows + rows_wg - 1) / rows_wg;
      const long groups = (long)h.B * h.Hkv * (h.S + 1);
      const long n = (groups + 7) / 8 * 8 * a.n_rb;
      hipLaunchKernelGGL(kern, dim3((unsigned)n), dim3(256), 0, s, a);
    };
    switch (attn_cfg(rows)) {
      case 0: go(k_tree_attn_dma<DH, 1, 2, 32, 4>, DmaCfg<DH, 1, 2, 32, 4>::ROWS); break;
      case 1: go(k_tree_attn_dma<DH, 1, 1, 64, 2>, DmaCfg<DH, 1, 1, 64, 2>::ROWS); break;
      default: go(k_tree_attn_dma<DH, 2, 1, 64, 2>, DmaCfg<DH, 2, 1, 64, 2>::ROWS); break;
    }
  } else {
    const int rb = (rows + ROWS - 1) / ROWS;
    dim3 grid(rb, h.B * h.Hkv, h.S + 1);
    hipLaunchKernelGGL((k_tree_attn<T, DH>), grid, dim3(256), 0, s, a);
  }
  return e3h::launch_status();
}

// [P4] USP step 2, the TTT branch: position t, query head h attends to its own branch keys
// kb[j][t] (j < n_steps), computed as per-position dot products.  A workgroup takes
// positions of one KV head, G * DH/8 lanes each (16 lanes of 8 dimensions per query head);
// every key and value load is issued before the arithmetic, and a score is reduced over the
// 16 lanes of its head.
template <typename T, int DH>
__global__ __launch_bounds__(1024) void k_branch_attn(int L, int n_steps, int Hq, int Hkv, const T* __restrict__ q,
                                                      const T* __restrict__ kb, const T* __restrict__ vb,
                                                      float scale_log2, float* __restrict__ o,
                                                      float* __restrict__ lse) {
  constexpr int LPH = DH / 8;   // lanes per head
  constexpr int MAXS = 8;       // steps held in registers (host: n_steps <= MAXS)
  const int G = Hq / Hkv;
  const int per = G * LPH;      // lanes per position
  const int t = blockIdx.x * (blockDim.x / per) + threadIdx.x / per;
  const int c = blockIdx.y;
  if (t >= L) return;           // whole position groups only: a head's 16 lanes stay together
  const int li = threadIdx.x % per;
  const int hg = li / LPH, d8 = li % LPH;
  const int h = c * G + hg;
  float qv[8];
  load8<T>(q + ((size_t)t * Hq + h) * DH + d8 * 8, qv);
  float kv[MAXS][8], vv[MAXS][8];
#pragma unroll
  for (int j = 0; j < MAXS; ++j)
    if (j < n_steps) {
      load8<T>(kb + (((size_t)j * L + t) * Hkv + c) * DH + d8 * 8, kv[j]);
      load8<T>(vb + (((size_t)j * L + t) * Hkv + c) * DH + d8 * 8, vv[j]);
    }
  float sc[MAXS];
  float m = kNegInf;
#pragma unroll
  for (int j = 0; j < MAXS; ++j) {
    sc[j] = kNegInf;
    if (j < n_steps) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = __builtin_fmaf(qv[e], kv[j][e], d);
      d = row16_reduce(d, OpAdd()) * scale_log2;   // a head's 16 lanes (DH = 128)
      sc[j] = d;
      m = fmaxf(m, d);
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
#pragma unroll
  for (int j = 0; j < MAXS; ++j)
    if (j < n_steps) {
      const float p = __builtin_amdgcn_exp2f(sc[j] - m);
      tot += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(p, vv[j][e], acc[e]);
    }
  const float inv = 1.f / tot;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= inv;
  store8<float>(o + ((size_t)t * Hq + h) * DH + d8 * 8, acc);
  if (d8 == 0) lse[(size_t)t * Hq + h] = (m + log2f(tot)) * kLn2;
}

}  // namespace

namespace e3h {

// [P4] USP step 1: causal attention of every position over the sequence, bf16, positions in
// blocks of 128 (rows = 128 x G per block, 128 rows per workgroup, 64 keys per iteration).
int launch_causal_attention(int L, int Hq, int Hkv, int Dh, const void* q, const void* k, const void* v,
                            float scale, float* o, float* lse, hipStream_t s) {
  constexpr int CB = 128;
  DevArgs a{};
  a.B = (L + CB - 1) / CB;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.q = q;
  a.q_cu = nullptr;
  a.q_stride = CB;
  a.q_rows_total = L;
  a.kp = k;
  a.vp = v;
  a.p_cu = nullptr;
  a.mask = nullptr;
  a.W64 = 1;
  a.S = 0;
  a.causal_len = L;
  a.scale_log2 = scale * kLog2e;
  a.o_part = o;
  a.lse_part = lse;
  ProfScope ps("causal_attention", s);
  auto go = [&](auto kern, int rows_wg) {
    a.n_rb = (CB * a.G + rows_wg - 1) / rows_wg;
    const long groups = (long)a.B * Hkv;
    const long n = (groups + 7) / 8 * 8 * a.n_rb;
    hipLaunchKernelGGL(kern, dim3((unsigned)n), dim3(256), 0, s, a);
  };
  if (Dh == 128) go(k_tree_attn_dma<128, 2, 1, 64, 2, true>, DmaCfg<128, 2, 1, 64, 2>::ROWS);
  else if (Dh == 64) go(k_tree_attn_dma<64, 2, 1, 64, 2, true>, DmaCfg<64, 2, 1, 64, 2>::ROWS);
  else return EAGLE3_EUNSUPPORTED;
  return launch_status();
}

int launch_branch_attention(int L, int n_steps, int Hq, int Hkv, int Dh, int dtype, const void* q,
                            const void* kb, const void* vb, float scale, float* o, float* lse, hipStream_t s) {
  if (Dh != 128) return EAGLE3_EUNSUPPORTED;
  ProfScope ps("branch_attention", s);
  const int per = (Hq / Hkv) * (Dh / 8);        // lanes per position
  const int ppw = per >= 256 ? 1 : 256 / per;   // positions per workgroup
  const dim3 grid((L + ppw - 1) / ppw, Hkv), block(per * ppw);
  if (dtype == EAGLE3_BF16)
    hipLaunchKernelGGL((k_branch_attn<bf16, 128>), grid, block, 0, s, L, n_steps, Hq, Hkv, (const bf16*)q,
                       (const bf16*)kb, (const bf16*)vb, scale * kLog2e, o, lse);
  else
    hipLaunchKernelGGL((k_branch_attn<float, 128>), grid, block, 0, s, L, n_steps, Hq, Hkv, (const float*)q,
                       (const float*)kb, (const float*)vb, scale * kLog2e, o, lse);
  return launch_status();
}

// Prefix splits: enough workgroups for the launch target of the workgroup shape, but every
// split keeps at least one iteration of keys and at least three times as many keys as its
// row block has rows, so a split's fp32 partial stays at or below a third of the bf16 K+V
// bytes it streams.
int attention_splits(int B, int Hkv, int rows_per_kv, int max_prefix, int n_splits) {
  if (n_splits > 0) return n_splits;
  if (max_prefix <= 0 || B <= 0 || Hkv <= 0) return 1;
  const int rows = rows_per_kv > 0 ? rows_per_kv : 1;
  const int cfg = attn_cfg(rows);
  const int rows_wg = attn_cfg_rows(cfg), kiter = attn_cfg_keys(cfg);
  const long rb = (rows + rows_wg - 1) / rows_wg;
  const long base = (long)B * Hkv * rb;
  long s = (attn_cfg_wgs(cfg, rb) + base - 1) / base;
  const long min_keys = std::max<long>(kiter, 3L * std::min(rows, rows_wg));
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
  if (S > MERGE_MAX_S || Dh > 128 || Dh % 4) return EAGLE3_EUNSUPPORTED;
  ProfScope ps(tag, s);
  if (S <= MERGE_FEW_S && (Dh == 128 || Dh == 64)) {
    if (out_dtype == EAGLE3_BF16) {
      if (Dh == 128) launch_merge_rows<bf16, 128, MERGE_FEW_S>(S, rows, o_part, lse_part, o, lse, s);
      else launch_merge_rows<bf16, 64, MERGE_FEW_S>(S, rows, o_part, lse_part, o, lse, s);
    } else {
      if (Dh == 128) launch_merge_rows<float, 128, MERGE_FEW_S>(S, rows, o_part, lse_part, o, lse, s);
      else launch_merge_rows<float, 64, MERGE_FEW_S>(S, rows, o_part, lse_part, o, lse, s);
    }
    return launch_status();
  }
  const bool few = S <= MERGE_FEW_S;
  const dim3 grid(few ? (rows + 3) / 4 : rows);
  if (out_dtype == EAGLE3_BF16) {
    if (few) hipLaunchKernelGGL((k_lse_merge<bf16, 1>), grid, dim3(256), 0, s, S, rows, Dh, o_part, lse_part, (bf16*)o, lse);
    else hipLaunchKernelGGL((k_lse_merge<bf16, 4>), grid, dim3(256), 0, s, S, rows, Dh, o_part, lse_part, (bf16*)o, lse);
  } else {
    if (few) hipLaunchKernelGGL((k_lse_merge<float, 1>), grid, dim3(256), 0, s, S, rows, Dh, o_part, lse_part, (float*)o, lse);
    else hipLaunchKernelGGL((k_lse_merge<float, 4>), grid, dim3(256), 0, s, S, rows, Dh, o_part, lse_part, (float*)o, lse);
  }
  return launch_status();
}

}  // namespace e3h
