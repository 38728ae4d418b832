// Weight-streaming GEMM for the drafter's projections and LM head:
//   Y_part[split][m][n] = sum_{k in split} X[m][k] * W[n][k]
// X is [M, K] (the few rows being evaluated), W is [N, K] row-major.  The op is bound by
// streaming W from HBM exactly once, so W sits on the MFMA A operand (16 output features
// per tile) and X is kept stationary in registers: a wave loads KCB 16-byte chunks of its
// X rows once and streams NTB consecutive W tiles against them (X costs 1/(16 NTB) of the
// load traffic of W), with the next W tile in flight while the current one is multiplied.
// A workgroup is WK waves that split its k-range (summed in LDS in wave order, so results
// are deterministic); workgroups tile (n-block, k-split).
#include <cstring>
#include <type_traits>

#include "common.h"
#include "internal.h"

using namespace e3;

namespace {

// X-stationary variant: each wave keeps KCB chunks of its X rows in registers and streams
// NTB consecutive 16-row tiles of W against them (W tiles double-buffered), so the X rows
// cost 16*NTB times less load traffic than W.  The WK waves of a workgroup split the
// k-range and are summed in LDS in wave order.
// SILU: W is [2F, K] with the gate rows first and the up rows second.  A wave takes NTB/2
// gate tiles and the NTB/2 matching up tiles, and writes act[m][j] = silu(gate) * up in T
// (needs a single k-split).
template <int NTB, bool SILU>
__device__ __forceinline__ int tile_row0(int nb, int t, int F) {
  if constexpr (!SILU) {
    return (nb * NTB + t) * 16;
  } else {
    constexpr int H = NTB / 2;
    return t < H ? (nb * H + t) * 16 : F + (nb * H + t - H) * 16;
  }
}

template <typename T, bool SILU>
__device__ __forceinline__ void store_out(float* Ys, void* act, int M, int N, int F, int m, int n_gate,
                                          floatx4 g, floatx4 u) {
  if constexpr (!SILU) {
    if (m < M && n_gate < N) *reinterpret_cast<floatx4*>(Ys + (size_t)m * N + n_gate) = g;
  } else {
    if (m < M && n_gate < F) {
      T* o = reinterpret_cast<T*>(act) + (size_t)m * F + n_gate;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(g[e] / (1.f + expf(-g[e])) * u[e]);
    }
  }
}

template <typename T, int MT, int NTB, int KCB, int WK, bool SILU = false>
__global__ __launch_bounds__(WK * 64) void k_gemm(const T* __restrict__ X, int M, int ldx,
                                                     const T* __restrict__ W, int N, int K,
                                                     float* __restrict__ Y, int n_blocks,
                                                     int chunks_total, int chunks_per_split,
                                                     void* __restrict__ act, int F) {
  static_assert(NTB % 2 == 0, "NTB must be even");
  constexpr int EPC = Vec<T>::N;
  constexpr int KPC = Mfma<T>::KPC;
  __shared__ floatx4 red[WK][NTB * MT][64];
  const int lane = threadIdx.x & 63, wk = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int nb = blockIdx.x % n_blocks, ks = blockIdx.x / n_blocks;
  const int cs0 = ks * chunks_per_split;
  const int cs1 = min(chunks_total, cs0 + chunks_per_split);
  const int per_wave = (cs1 - cs0 + WK - 1) / WK;
  const int c0 = cs0 + wk * per_wave;
  const int c1 = min(cs1, c0 + per_wave);
  const u32x4 zero = {0, 0, 0, 0};

  const T* wbase[NTB];
  bool wok[NTB];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt) {
    const int n = tile_row0<NTB, SILU>(nb, nt, F) + r16;
    wok[nt] = n < N;
    wbase[nt] = W + (size_t)(wok[nt] ? n : 0) * K + g * EPC;
  }
  const T* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + r16;
    xok[mt] = m < M;
    xrow[mt] = X + (size_t)(xok[mt] ? m : 0) * ldx + g * EPC;
  }
  floatx4 acc[NTB][MT];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int cb = c0; cb < c1; cb += KCB) {
    bool kin[KCB];
#pragma unroll
    for (int u = 0; u < KCB; ++u) kin[u] = cb + u < c1 && (cb + u) * KPC + g * EPC + EPC <= K;
    u32x4 xv[KCB][MT];
#pragma unroll
    for (int u = 0; u < KCB; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xv[u][mt] = (kin[u] && xok[mt]) ? ld16(xrow[mt] + (cb + u) * KPC) : zero;
    u32x4 wa[KCB], wb[KCB];
#pragma unroll
    for (int u = 0; u < KCB; ++u) wa[u] = (kin[u] && wok[0]) ? ld16(wbase[0] + (cb + u) * KPC) : zero;
#pragma unroll
    for (int nt = 0; nt < NTB; nt += 2) {
#pragma unroll
      for (int u = 0; u < KCB; ++u)
        wb[u] = (kin[u] && wok[nt + 1]) ? ld16(wbase[nt + 1] + (cb + u) * KPC) : zero;
#pragma unroll
      for (int u = 0; u < KCB; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = Mfma<T>::run(wa[u], xv[u][mt], acc[nt][mt]);
      if (nt + 2 < NTB) {
#pragma unroll
        for (int u = 0; u < KCB; ++u)
          wa[u] = (kin[u] && wok[nt + 2]) ? ld16(wbase[nt + 2] + (cb + u) * KPC) : zero;
      }
#pragma unroll
      for (int u = 0; u < KCB; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt + 1][mt] = Mfma<T>::run(wb[u], xv[u][mt], acc[nt + 1][mt]);
    }
  }

  float* Ys = Y + (size_t)ks * M * N;
  constexpr int NOUT = SILU ? NTB / 2 : NTB;   // output tiles per wave
  if constexpr (WK == 1) {
#pragma unroll
    for (int nt = 0; nt < NOUT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r16;
        const int n = tile_row0<NTB, SILU>(nb, nt, F) + 4 * g;
        store_out<T, SILU>(Ys, act, M, N, F, m, n, acc[nt][mt], acc[SILU ? nt + NOUT : nt][mt]);
      }
  } else {
#pragma unroll
    for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[wk][nt * MT + mt][lane] = acc[nt][mt];
    __syncthreads();
    for (int e = threadIdx.x; e < NOUT * MT * 64; e += WK * 64) {
      const int tile = e / 64, ln = e % 64;
      const int nt = tile / MT, mt = tile % MT;
      const int tile2 = (SILU ? nt + NOUT : nt) * MT + mt;
      floatx4 v = red[0][tile][ln], u = red[0][tile2][ln];
#pragma unroll
      for (int w = 1; w < WK; ++w) {
        v += red[w][tile][ln];
        if constexpr (SILU) u += red[w][tile2][ln];
      }
      const int m = mt * 16 + (ln & 15);
      const int n = tile_row0<NTB, SILU>(nb, nt, F) + 4 * (ln >> 4);
      store_out<T, SILU>(Ys, act, M, N, F, m, n, v, u);
    }
  }
}

// LM-head statistics of one 16-row tile over 128 consecutive columns (eight 16-column tiles
// t of the accumulators, from column col0): for each row, the best logit by (value desc,
// column asc), its column, and the sum of e^(z - best) over the columns below N (the
// selection forms each row's top-K and log-sum-exp from these).  Lanes r16, r16 + 16, r16 + 32
// and r16 + 48 hold row r16 (4 columns of every tile each, ascending within a lane), so the
// reductions cross the four 16-lane rows only; the lanes of the first row write.  Layout:
// three planes of M x kLmStatsLd (best value fp32, its column int32, sum fp32), entry
// col0 / 128 of row m.  Kept lean: it runs once per workgroup, after the weight stream.
template <typename Tile>
__device__ __forceinline__ void lm_block_stats(Tile tile, int m, int M, int N, int col0,
                                               float* __restrict__ stats) {
  if (col0 >= N) return;   // a block wholly past the vocabulary end (uniform)
  const int g = (threadIdx.x & 63) >> 4;
  float v[32];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const floatx4 x = tile(t);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * t + e] = x[e];
  }
  if (col0 + 128 > N) {   // the vocabulary's last block: columns past N take no part
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (col0 + (i >> 2) * 16 + 4 * g + (i & 3) >= N) v[i] = kNegInf;
  }
  float mx = v[0];
#pragma unroll
  for (int i = 1; i + 1 < 32; i += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(v[i], v[i + 1]));
  mx = __builtin_fmaxf(mx, v[31]);
  mx = row_reduce(mx, OpMax());
  // the first column holding the maximum (columns ascend within the lane), then the
  // smallest over the row's four lanes
  int bi = 0x7fffffff;
#pragma unroll
  for (int i = 31; i >= 0; --i)
    if (v[i] == mx) bi = col0 + (i >> 2) * 16 + 4 * g + (i & 3);
  uint32_t ia, ib;
  swap16((uint32_t)bi, ia, ib);
  bi = min((int)ia, (int)ib);
  swap32((uint32_t)bi, ia, ib);
  bi = min((int)ia, (int)ib);
  float sum = 0.f;
  if (mx != kNegInf) {
    const float off = mx * kLog2e;
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(v[i], kLog2e, -off));
  }
  sum = row_reduce(sum, OpAdd());
  if (g == 0 && m < M) {
    const size_t plane = (size_t)M * e3h::kLmStatsLd, i = (size_t)m * e3h::kLmStatsLd + (col0 >> 7);
    stats[i] = mx;
    reinterpret_cast<int*>(stats)[plane + i] = bi;
    stats[2 * plane + i] = sum;
  }
}

// ---------------------------------------------------------------------------------------
// bf16 weight streaming through an LDS ring (one wave per workgroup).
//
// A tile is 16 rows x 8 chunks (a 512-byte row segment).  It moves from HBM to a slot of
// this wave's LDS ring by eight LDS-DMA instructions, each taking two whole 512-byte row
// segments (lanes 0-31 and 32-63), so every HBM line is fetched whole (W non-temporally;
// X, which every workgroup re-reads, with the default policy).  A row's 16-byte pieces are
// stored XOR-swizzled (piece p at position p ^ row), which keeps the MFMA operand reads (16
// rows at one piece) free of bank conflicts.  Per 8-chunk k-block
// the stream is MT tiles of X (the evaluated rows, kept in registers for the block) and then
// NTB tiles of W; NST slots are in flight.  W feeds operand A (16 output features), X
// operand B, accumulation in fp32.  Needs K % 32 == 0 and MT <= 2.
// ---------------------------------------------------------------------------------------
constexpr int RING_TILE = 16 * 512;

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// 16 bytes per lane into LDS at lds_base + 16 * lane, non-temporal (W: read once).  Issued
// as assembly so that the compiler does not see an outstanding LDS write (it would drain
// every DMA before each later LDS read); completion is ordered by the explicit vmcnt waits
// of the ring.  M0 is written by the asm and named as clobbered; the compiler does not
// preserve reserved registers across asm (hence its warning), which is harmless: nothing
// else in these kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void ring_dma(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(gptr), "s"(lds_base)
               : "memory", "m0");
}
// The same with the default cache policy, for X: every workgroup re-reads the same rows, which
// then come from L2 (non-temporal, they were fetched again from further out: 70B-shaped round
// 4.56 -> 4.50 ms, batch-16 round 3.46 -> 3.30 ms).
__device__ __forceinline__ void ring_dma_x(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void ring_wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ROLE names the projection (0 other, 1 LM head, 2 QKV, 3 O, 4 MLP down, 5 fusion, 6 MLP
// gate/up).  It does not change the code; each projection gets its own kernel symbol, so that
// profiles and hardware counters attribute launches to projections.
// WK waves share a workgroup's n-block: wave w streams the w-th part of the workgroup's
// k-range through its own ring, and the WK partial tiles are summed in LDS in wave order at
// the end (deterministic), so a k-split over WK waves costs no partial-sum traffic.
template <int MT, int NTB, int NST, bool SILU, int ROLE, int WK>
__global__ __launch_bounds__(64 * WK) void k_gemm_ring(const bf16* __restrict__ X, int M, int ldx,
                                                       const bf16* __restrict__ W, int N, int K,
                                                       float* __restrict__ Y, int n_blocks,
                                                       int chunks_total, int chunks_per_split,
                                                       void* __restrict__ act, int F,
                                                       float* __restrict__ stats) {
  static_assert(MT >= 1 && MT <= 2, "X is held in registers for one k-block");
  static_assert(NST >= 2 && 8 * (NST - 2) <= 63, "outstanding DMA must fit the vmcnt counter");
  static_assert((WK - 1) * NTB * MT * 64 * 16 <= WK * NST * RING_TILE, "reduction fits the rings");
  constexpr int SPK = MT + NTB;   // ring stages per k-block
  __shared__ __attribute__((aligned(16))) char ring[WK * NST * RING_TILE];
  const int lane = threadIdx.x & 63;
  const int wv_id = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int nb = blockIdx.x % n_blocks, ks = blockIdx.x / n_blocks;
  // this wave's chunk range: the workgroup's split, cut into WK parts of whole 8-chunk blocks
  const int ws0 = ks * chunks_per_split;
  const int ws1 = min(chunks_total, ws0 + chunks_per_split);
  const int wblocks = ws1 > ws0 ? (ws1 - ws0 + 7) / 8 : 0;
  const int per_wave = (wblocks + WK - 1) / WK;
  const int cs0 = min(ws1, ws0 + wv_id * per_wave * 8);
  const int cs1 = min(ws1, cs0 + per_wave * 8);
  const int n_kb = cs1 > cs0 ? (cs1 - cs0 + 7) / 8 : 0;
  const int total = n_kb * SPK;
  const uint32_t ring0 = lds_u32(ring) + (uint32_t)wv_id * (NST * RING_TILE);
  char* myring = ring + wv_id * (NST * RING_TILE);

  // DMA of stage s (k-block s / SPK; X tile, or W tile of this workgroup's n-block)
  auto issue = [&](int s) {
    const int j = s / SPK, r = s - j * SPK;
    const int c0 = cs0 + j * 8;
    const int lastp = min(8, cs1 - c0) * 4 - 1;
    const uint32_t slot = ring0 + (uint32_t)(s % NST) * RING_TILE;
    const bf16* base;
    int ld, row0, rmax;
    if (r < MT) {
      base = X;
      ld = ldx;
      row0 = r * 16;
      rmax = M - 1;
    } else {
      base = W;
      ld = K;
      row0 = tile_row0<NTB, SILU>(nb, r - MT, F);
      rmax = N - 1;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the slot's last reads are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rt = 2 * i + (lane >> 5);
      const int row = min(row0 + rt, rmax);
      const int pc = min((lane & 31) ^ rt, lastp);
      if (r < MT) ring_dma_x(base + (size_t)row * ld + c0 * 32 + pc * 8, slot + i * 1024);
      else ring_dma(base + (size_t)row * ld + c0 * 32 + pc * 8, slot + i * 1024);
    }
  };

  floatx4 acc[NTB][MT];
#pragma unroll
  for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  u32x4 xv[8][MT];

  // LDS byte offset of this lane's operand piece for chunk u: row r16, piece 4u + g
  auto opoff = [&](int u) { return (uint32_t)(r16 * 512 + (((4 * u + g) ^ r16) * 16)); };

#pragma unroll
  for (int s0 = 0; s0 < NST - 1; ++s0)
    if (s0 < total) issue(s0);

  int s = 0;
  for (int j = 0; j < n_kb; ++j) {
    const int nvalid = min(8, cs1 - (cs0 + j * 8));
#pragma unroll
    for (int r = 0; r < SPK; ++r, ++s) {
      if (s + NST - 2 < total) ring_wait_vm<8 * (NST - 2)>();
      else ring_wait_vm<0>();
      const char* slot = myring + (s % NST) * RING_TILE;
      if (r < MT) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(slot + opoff(u));
          xv[u][r] = u < nvalid ? v : u32x4{0, 0, 0, 0};
        }
      } else {
        u32x4 wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) wv[u] = *reinterpret_cast<const u32x4*>(slot + opoff(u));
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[r - MT][mt] = Mfma<bf16>::run(wv[u], xv[u][mt], acc[r - MT][mt]);
      }
      if (s + NST - 1 < total) issue(s + NST - 1);
    }
  }

  if constexpr (WK > 1) {
    // waves 1.. hand their tiles to wave 0 through LDS (the rings are drained: every wave's
    // last stage waited for vmcnt(0) before it was read)
    floatx4* red = reinterpret_cast<floatx4*>(ring);
    __syncthreads();
    if (wv_id > 0) {
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[(((wv_id - 1) * NTB + nt) * MT + mt) * 64 + lane] = acc[nt][mt];
    }
    __syncthreads();
    if (wv_id > 0) return;
#pragma unroll
    for (int w = 1; w < WK; ++w)
#pragma unroll
      for (int nt = 0; nt < NTB; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nt][mt] += red[(((w - 1) * NTB + nt) * MT + mt) * 64 + lane];
  }

  if constexpr (ROLE == 1 && !SILU && NTB == 8) {
    if (stats)   // the LM head without a k-split: statistics per 128 columns of the logits
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        lm_block_stats([&](int t) { return acc[t][mt]; }, mt * 16 + r16, M, N, nb * NTB * 16, stats);
  }
  float* Ys = Y + (size_t)ks * M * N;
  constexpr int NOUT = SILU ? NTB / 2 : NTB;
#pragma unroll
  for (int nt = 0; nt < NOUT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r16;
      const int n = tile_row0<NTB, SILU>(nb, nt, F) + 4 * g;
      store_out<bf16, SILU>(Ys, act, M, N, F, m, n, acc[nt][mt], acc[SILU ? nt + NOUT : nt][mt]);
    }
}

// ---------------------------------------------------------------------------------------
// bf16 weight streaming for 32 < M <= 192 rows (a batch of requests times the frontier).
// Past two row tiles a wave can no longer keep its X rows for a k-block in registers beside
// the accumulators of eight W tiles, and X re-read per wave would cost more load traffic
// than W itself.  So the four waves of a workgroup split the rows instead of the k-range:
// wave w owns row tiles w, w + 4, w + 8 (MT tiles of 16 rows in all), and every W tile is
// fetched once per workgroup into one shared LDS ring (two LDS-DMA instructions per wave,
// whole 512-byte row segments, non-temporal) and read by all four waves against their own
// rows.  The block's X (MT tiles x 8 chunks, fetched with the default cache policy: every
// workgroup reads the same rows, from L2) has an LDS buffer of its own; each wave copies
// its rows into registers at the block's first W tile, and the next block's X is fetched
// right after the barrier of the second W tile, when every wave has its copy.
// One barrier per W tile orders the ring: past it the tile's DMA has landed for every wave
// (each waited for its own two instructions by vmcnt), and every wave has finished reading
// the slot that the DMA issued next overwrites.  The vmcnt waits count the DMA instructions
// issued after the awaited ones, including the next block's X when it lies between them.
// Needs K % 32 == 0; MT <= 12; NT >= NS.
// ---------------------------------------------------------------------------------------
template <int MT, int NT, int NS, bool SILU, int ROLE>
__global__ __launch_bounds__(256) void k_gemm_wide(const bf16* __restrict__ X, int M, int ldx,
                                                   const bf16* __restrict__ W, int N, int K,
                                                   float* __restrict__ Y, int n_blocks,
                                                   int chunks_total, int chunks_per_split,
                                                   void* __restrict__ act, int F,
                                                   float* __restrict__ stats) {
  constexpr int MTW = (MT + 3) / 4;   // row tiles per wave (at most)
  static_assert(MT >= 1 && MT <= 12, "row tiles");
  static_assert(NS >= 3 && NT >= NS, "the next block's X is issued after W stage NS of a block");
  static_assert(2 * (NS - 1) <= 63 && 2 * (NS - 2) + 2 * MT <= 63, "outstanding DMA must fit the vmcnt counter");
  static_assert((MT + NS) * RING_TILE <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) char lds[(MT + NS) * RING_TILE];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int nb = blockIdx.x % n_blocks, ks = blockIdx.x / n_blocks;
  const int cs0 = ks * chunks_per_split;
  const int cs1 = min(chunks_total, cs0 + chunks_per_split);
  const int n_kb = cs1 > cs0 ? (cs1 - cs0 + 7) / 8 : 0;
  const int total = n_kb * NT;                     // W stages
  const uint32_t xbuf0 = lds_u32(lds);
  const uint32_t wring0 = xbuf0 + MT * RING_TILE;
  const char* wring = lds + MT * RING_TILE;

  // this wave's two DMA instructions of a 16-row tile: rows 4 wv .. 4 wv + 3
  auto dma_tile = [&](const bf16* base, int ld, int row0, int rmax, int c0, int lastp, uint32_t slot,
                      auto is_x) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 2 * wv + h;
      const int rt = 2 * i + (lane >> 5);
      const int row = min(row0 + rt, rmax);
      const int pc = min((lane & 31) ^ rt, lastp);
      if constexpr (decltype(is_x)::value) ring_dma_x(base + (size_t)row * ld + c0 * 32 + pc * 8, slot + i * 1024);
      else ring_dma(base + (size_t)row * ld + c0 * 32 + pc * 8, slot + i * 1024);
    }
  };
  auto issue_w = [&](int s) {      // stage s: k-block s / NT, W tile s % NT of this n-block
    const int j = s / NT, t = s - j * NT;
    const int c0 = cs0 + j * 8;
    dma_tile(W, K, tile_row0<NT, SILU>(nb, t, F), N - 1, c0, min(8, cs1 - c0) * 4 - 1,
             wring0 + (uint32_t)(s % NS) * RING_TILE, std::false_type{});
  };
  auto issue_x = [&](int j) {      // the MT row tiles of X for k-block j
    const int c0 = cs0 + j * 8;
    const int lastp = min(8, cs1 - c0) * 4 - 1;
#pragma unroll
    for (int t = 0; t < MT; ++t) dma_tile(X, ldx, t * 16, M - 1, c0, lastp, xbuf0 + t * RING_TILE, std::true_type{});
  };
  auto opoff = [&](int u) { return (uint32_t)(r16 * 512 + (((4 * u + g) ^ r16) * 16)); };

  floatx4 acc[NT][MTW];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mw = 0; mw < MTW; ++mw) acc[nt][mw] = floatx4{0.f, 0.f, 0.f, 0.f};
  u32x4 xv[8][MTW];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int mw = 0; mw < MTW; ++mw) xv[u][mw] = u32x4{0, 0, 0, 0};

  // this wave's X rows of block jb into registers; rows of tiles it does not own (past MT)
  // read tile 0 and are zeroed, so every wave runs MTW row tiles without a branch
  auto read_x = [&](int jb) {
    const int nvalid = min(8, cs1 - (cs0 + jb * 8));
#pragma unroll
    for (int mw = 0; mw < MTW; ++mw) {
      const bool own = mw * 4 + 3 < MT || mw * 4 + wv < MT;
      const char* xt = lds + (own ? mw * 4 + wv : 0) * RING_TILE;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(xt + opoff(u));
        xv[u][mw] = (own && u < nvalid) ? v : u32x4{0, 0, 0, 0};
      }
    }
  };
  u32x4 wf[2][8];
  auto read_w = [&](int st, u32x4 (&f)[8]) {
    const char* slot = wring + (st % NS) * RING_TILE;
#pragma unroll
    for (int u = 0; u < 8; ++u) f[u] = *reinterpret_cast<const u32x4*>(slot + opoff(u));
  };

  // Pipeline.  The ring holds NS W stages (stage s in slot s % NS).  Iteration s: wait for
  // W(s+1) and pass the barrier; refill the slot of W(s), whose reads every wave finished
  // before the barrier, with W(s+NS); read W(s+1)'s operands; then run stage s's MFMAs, so
  // the operand reads of the next stage overlap this stage's matrix work.  The next block's
  // X goes into the X buffer after the barrier of a block's first stage (every wave read
  // the block's X before it) and is read into registers after the block's last MFMAs.
  if (n_kb > 0) issue_x(0);
#pragma unroll
  for (int s0 = 0; s0 < NS; ++s0)
    if (s0 < total) issue_w(s0);
  if (total > 0) {
    if (NS - 1 < total) ring_wait_vm<2 * (NS - 1)>();
    else ring_wait_vm<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    read_x(0);
    read_w(0, wf[0]);
  }

  int s = 0;
  for (int j = 0; j < n_kb; ++j) {
    const bool next_x = j + 1 < n_kb;
    static_for<0, NT>([&](auto ntc) {
      constexpr int nt = decltype(ntc)::value;
      constexpr int cur = nt & 1;          // NT is even: stage parity is nt's
      // lgkmcnt(0) through the builtin, on every path, so that the compiler's own wait
      // tracking knows this stage's operand reads (issued one iteration earlier) are
      // complete and adds no waits on the next stage's reads before the MFMAs
      __builtin_amdgcn_s_waitcnt(0xC07F);
      if (s + 1 < total) {
        // own DMA of W(s+1) has landed.  Issued after it so far: W(s+2 .. s+NS-1), and the
        // next block's X when it follows W(s+1) (it was issued right after W(j NT + NS), at
        // this block's first stage).  At a block's last stage the next block's X must have
        // landed too: it precedes W(s+1), or (NT == NS) follows it directly, and the
        // 2 (NS - 2) instructions left in flight are W(s+2 ..).
        if (s + NS - 1 < total) {
          if constexpr (nt == NT - 1) {
            ring_wait_vm<2 * (NS - 2)>();
          } else if constexpr (nt >= 1 && nt <= NS - 1) {
            if (next_x) ring_wait_vm<2 * (NS - 2) + 2 * MT>();
            else ring_wait_vm<2 * (NS - 2)>();
          } else {
            ring_wait_vm<2 * (NS - 2)>();
          }
        } else {
          ring_wait_vm<0>();
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (s + NS < total) issue_w(s + NS);
        if constexpr (nt == 0) {
          if (next_x) issue_x(j + 1);
        }
        read_w(s + 1, wf[cur ^ 1]);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int mw = 0; mw < MTW; ++mw) acc[nt][mw] = Mfma<bf16>::run(wf[cur][u], xv[u][mw], acc[nt][mw]);
      if constexpr (nt == NT - 1) {
        if (next_x) read_x(j + 1);
      }
      ++s;
    });
  }

  if constexpr (ROLE == 1 && !SILU && NT % 8 == 0) {
    if (stats)   // the LM head without a k-split: statistics per 128 columns of the logits
#pragma unroll
      for (int mw = 0; mw < MTW; ++mw)
        if (mw * 4 + wv < MT)
#pragma unroll
          for (int h = 0; h < NT / 8; ++h)   // 128 columns at a time
            lm_block_stats([&](int t) { return acc[8 * h + t][mw]; }, (mw * 4 + wv) * 16 + r16, M, N,
                           nb * NT * 16 + 128 * h, stats);
  }
  float* Ys = Y + (size_t)ks * M * N;
  constexpr int NOUT = SILU ? NT / 2 : NT;
#pragma unroll
  for (int nt = 0; nt < NOUT; ++nt)
#pragma unroll
    for (int mw = 0; mw < MTW; ++mw)
      if (mw * 4 + wv < MT) {
        const int m = (mw * 4 + wv) * 16 + r16;
        const int n = tile_row0<NT, SILU>(nb, nt, F) + 4 * g;
        store_out<bf16, SILU>(Ys, act, M, N, F, m, n, acc[nt][mw], acc[SILU ? nt + NOUT : nt][mw]);
      }
}

// ---------------------------------------------------------------------------------------
// bf16 GEMM for many rows (M >= 256), bound by the matrix cores:
//   Y[m][n] = sum_k X[m][k] W[n][k], fp32 out.
// A workgroup owns a 256 (n) x 256 (m) output tile; its four waves (one per SIMD) each hold
// a 128 x 128 sub-tile in accumulators (4 x 4 tiles of v_mfma_f32_32x32x16_bf16, 256 fp32 per
// lane), which is the largest sub-tile the register file allows and so the fewest LDS operand
// reads per MFMA.  Both operands are k-major rows; a k-step of 64 brings 256 rows x 128 bytes
// of W and of X into LDS by LDS-DMA (one instruction moves eight 128-byte row pieces).
//
// Pipeline.  Two stages of 64 KB.  A k-step is four sub-steps of 16 MFMAs per wave; during
// each sub-step the wave reads the next sub-step's 8 operand fragments from LDS (one read
// after each of the first 8 MFMAs), so LDS latency hides under the MFMAs.  The DMA of stage
// s + 1 is issued during stage s, spread over its first two sub-steps (one instruction after
// every second MFMA): issued all at once behind the barrier, the 64 instructions of a stage
// back up in the CU's load path and hold every wave's MFMA issue for about half the stage.
// One barrier per stage, before the last sub-step, orders both hazards: stage s + 1 has
// landed for all waves (each waited for its own DMA), and every wave has finished reading
// stage s - 1's buffer, which the next DMA overwrites.
//
// LDS layout: the 16-byte piece p of row r sits at position p ^ (r & 7) ^ ((r >> 3) & 1) of
// the row's 128 bytes.  An operand read takes 16 rows at one piece per LDS cycle; the XOR
// places those 16 reads in distinct banks (two rows per 256-byte bank line).
//
// Tile order: consecutive workgroups go to different XCDs, so workgroup b is remapped to
// XCD-major order first, and each XCD walks its range in groups of 8 tile rows (m) per tile
// column (n), so the workgroups resident on one XCD share W and X tiles in its L2.
// With fewer tiles than CUs the k-range is split over workgroups (fp32 partial sums, added in
// split order by the sum epilogue).
// ---------------------------------------------------------------------------------------
constexpr int TILE_B = 256;                    // output rows (of W) and columns (rows of X) per tile
constexpr int TILE_K = 64;                     // k per stage
constexpr int TILE_RB = TILE_K * 2;            // bytes of one row per stage
constexpr int TILE_HALF = TILE_B * TILE_RB;    // bytes of the W (or X) part of a stage: 32 KB
constexpr int TILE_STAGE = 2 * TILE_HALF;      // 64 KB
constexpr int TILE_DPW = TILE_STAGE / 1024 / 4;   // DMA instructions per wave per stage: 16
constexpr int TILE_GROUP_M = 8;
constexpr int kTileCUs = 256;                  // MI355X compute units

typedef float floatx16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int tile_swz(int row) { return (row ^ ((row >> 3) & 1)) & 7; }

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from sbase + voff into LDS at lds_base + 16 * lane (cached: the tiles are
// re-read by other workgroups through L2).
__device__ __forceinline__ void tile_dma(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__global__ __launch_bounds__(256) void k_gemm_tile(const bf16* __restrict__ X, int M, int ldx,
                                                   const bf16* __restrict__ W, int N, int K,
                                                   float* __restrict__ Y, int tiles_n, int tiles_m,
                                                   int kps) {
  __shared__ __attribute__((aligned(16))) char lds[2 * TILE_STAGE];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int b = blockIdx.x;
  const int total = tiles_n * tiles_m;
  if (gridDim.x % 8 == 0) b = (b % 8) * (gridDim.x / 8) + b / 8;
  // split over k: workgroups total * ks .. hold k-steps [ks * kps, (ks + 1) * kps) of every
  // tile and write their partial sums to Y + ks * M * N
  const int ks = b / total;
  b -= ks * total;
  Y += (size_t)ks * M * N;
  const int gsz = TILE_GROUP_M * tiles_n;
  const int g = b / gsz, rem = b % gsz;
  const int gm = min(TILE_GROUP_M, tiles_m - g * TILE_GROUP_M);
  const int tm = g * TILE_GROUP_M + rem % gm, tn = rem / gm;
  const int n0 = tn * TILE_B, m0 = tm * TILE_B;
  const int wn = w & 1, wm = w >> 1;             // this wave: W rows n0 + 128 wn, X rows m0 + 128 wm
  const int k_first = ks * kps;
  const int n_k = min(kps, K / TILE_K - k_first);
  const uint32_t lds0 = lds_u32(lds);

  // DMA: a stage is 64 instructions of 1 KB (8 rows each): j < 32 cover W rows 8j .. 8j+7,
  // j >= 32 X rows; wave w issues j = 16 w .. 16 w + 15 (waves 0, 1: W; 2, 3: X).  Lane l:
  // row 8 (j % 32) + l / 8, LDS position l % 8, which holds piece (l % 8) ^ swz(row).
  const char* gb = reinterpret_cast<const char*>(w < 2 ? W : X) + (size_t)k_first * TILE_RB;
  uint32_t goff[TILE_DPW];
#pragma unroll
  for (int u = 0; u < TILE_DPW; ++u) {
    const int r = 8 * ((w * TILE_DPW + u) % 32) + (lane >> 3);
    const int p = (lane & 7) ^ tile_swz(r);
    goff[u] = (w < 2 ? (uint32_t)min(n0 + r, N - 1) * (uint32_t)K * 2u
                     : (uint32_t)min(m0 + r, M - 1) * (uint32_t)ldx * 2u) + p * 16;
  }
  auto dma_one = [&](int stage, int u) {
    tile_dma(gb + (size_t)stage * TILE_RB, goff[u],
             lds0 + (uint32_t)(stage & 1) * TILE_STAGE + (uint32_t)(w * TILE_DPW + u) * 1024);
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // operand fragments: lane l reads row rb + l % 32, piece 2 kk + l / 32 of k16 block kk
  // (swz(row) = swz(l % 32): fragment bases are multiples of 32 rows)
  const int lr = lane & 31, lh = lane >> 5;
  uint32_t ra[4], rx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = (uint32_t)(wn * 128 + i * 32 + lr) * TILE_RB;
    rx[i] = (uint32_t)(TILE_HALF + (wm * 128 + i * 32 + lr) * TILE_RB);
  }
  const int sw = tile_swz(lr);
  u32x4 fa[2][4], fb[2][4];
  auto read_one = [&](int nb, int t, int buf, int kk) {
    const char* st = lds + buf * TILE_STAGE + ((2 * kk + lh) ^ sw) * 16;
    if (t < 4) fa[nb][t] = *reinterpret_cast<const u32x4*>(st + ra[t]);
    else fb[nb][t - 4] = *reinterpret_cast<const u32x4*>(st + rx[t - 4]);
  };
  // sub-step: the 16 MFMAs of fragment set cb, with the reads of the next set (buf, kk) after
  // MFMAs 0..7 and DMA instructions lo.. of stage dstage after the odd MFMAs.  The explicit
  // order is kept by scheduling barriers.
  auto step = [&](int cb, int buf, int kk, bool dma_ok, int dstage, int lo, int hi) {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int i = t >> 2, j = t & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fa[cb][i]),
                                                          __builtin_bit_cast(bf16x8, fb[cb][j]), acc[i][j], 0, 0, 0);
      if (t < 8) read_one(cb ^ 1, t, buf, kk);
      if ((t & 1) && lo + (t >> 1) < hi && dma_ok) dma_one(dstage, lo + (t >> 1));
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no compiler-tracked load outstanding
#pragma unroll
  for (int u = 0; u < TILE_DPW; ++u) dma_one(0, u);
  ring_wait_vm<0>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int t = 0; t < 8; ++t) read_one(0, t, 0, 0);

  for (int kt = 0; kt < n_k; ++kt) {
    const int buf = kt & 1;
    const bool dma_ok = kt + 1 < n_k;            // stage kt + 1 goes to buffer buf ^ 1
    step(0, buf, 1, dma_ok, kt + 1, 0, 8);
    step(1, buf, 2, dma_ok, kt + 1, 8, 16);
    step(0, buf, 3, false, 0, 0, 0);
    if (dma_ok) {
      ring_wait_vm<0>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
    step(1, buf ^ 1, 0, false, 0, 0, 0);   // past the last stage these reads are unused
  }
  ring_wait_vm<0>();

  // D[n][m] of fragment (i, j): lane holds m = l % 32; register 4 q + e holds
  // n = 8 q + 4 (l / 32) + e
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 128 + j * 32 + lr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * 128 + i * 32 + 8 * q + 4 * lh;
        if (n < N)
          *reinterpret_cast<floatx4*>(Y + (size_t)m * N + n) =
              floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
      }
  }
}

// Ring kernel shape: 8 W tiles (128 output features) per workgroup, 4 ring slots of 8 KB per
// wave (five one-wave workgroups per CU).
constexpr int kRingNTB = 8, kRingNST = 3;   // three DMA stages measured faster than four (LM head)
// Waves aimed for by the k-split of the projections. ring launches (four per CU).
constexpr int kRingTargetWgs = 1024;

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

template <typename T, int MT, int NTB, int KCB, int WK, bool SILU>
void launch_gemm_t(const e3h::GemmPlan& p, const void* X, int ldx, const void* W, float* Y,
                   void* act, hipStream_t s) {
  dim3 grid(p.n_blocks * p.splits);
  hipLaunchKernelGGL((k_gemm<T, MT, NTB, KCB, WK, SILU>), grid, dim3(WK * 64), 0, s, (const T*)X, p.M,
                     ldx, (const T*)W, p.N, p.K, Y, p.n_blocks, p.chunks_total, p.chunks_per_split,
                     act, p.N / 2);
}

// Per row-tile count MT: (n-tiles per wave, X chunks held per lane).
constexpr int ntb_for(int mt) { return mt <= 4 ? 8 : 4; }
constexpr int kcb_for(int mt) { return mt <= 2 ? 8 : (mt <= 4 ? 4 : 2); }

template <typename T, int MT>
int dispatch_mt(const e3h::GemmPlan& p, const void* X, int ldx, const void* W, float* Y, void* act,
                hipStream_t s) {
  if (p.silu) {
    if (p.waves == 1)
      launch_gemm_t<T, MT, ntb_for(MT), kcb_for(MT), 1, true>(p, X, ldx, W, Y, act, s);
    else
      launch_gemm_t<T, MT, ntb_for(MT), kcb_for(MT), 4, true>(p, X, ldx, W, Y, act, s);
  } else {
    if (p.waves == 1)
      launch_gemm_t<T, MT, ntb_for(MT), kcb_for(MT), 1, false>(p, X, ldx, W, Y, act, s);
    else
      launch_gemm_t<T, MT, ntb_for(MT), kcb_for(MT), 4, false>(p, X, ldx, W, Y, act, s);
  }
  return e3h::launch_status();
}

template <int MT, int ROLE, int WK, bool SILU>
int launch_ring_r(const e3h::GemmPlan& p, const void* X, int ldx, const void* W, float* Y, void* act,
                  hipStream_t s, float* stats = nullptr) {
  hipLaunchKernelGGL((k_gemm_ring<MT, kRingNTB, kRingNST, SILU, ROLE, WK>), dim3(p.n_blocks * p.splits),
                     dim3(64 * WK), 0, s, (const bf16*)X, p.M, ldx, (const bf16*)W, p.N, p.K, Y, p.n_blocks,
                     p.chunks_total, p.chunks_per_split, act, p.N / 2, stats);
  return e3h::launch_status();
}

inline int gemm_role(const char* tag) {
  static const char* names[] = {"gemm_lm_head", "gemm_qkv", "gemm_o", "gemm_down", "gemm_fuse", "gemm_gate_up"};
  if (tag && strcmp(tag, "gemm_lm_head_root") == 0) return 1;
  for (int i = 0; i < 6; ++i)
    if (tag && strcmp(tag, names[i]) == 0) return i + 1;
  return 0;
}

// Instantiated shapes: the LM head one wave per workgroup (four when its vocabulary is too
// small to fill the chip and the k-range stays whole for the block statistics); the other
// projections two or four; the SiLU gate/up four.
template <int MT>
int launch_ring(const e3h::GemmPlan& p, const void* X, int ldx, const void* W, float* Y, void* act,
                hipStream_t s, int role, float* stats) {
  if (p.silu) return launch_ring_r<MT, 6, 4, true>(p, X, ldx, W, Y, act, s);
  if (p.waves == 1) return launch_ring_r<MT, 1, 1, false>(p, X, ldx, W, Y, act, s, stats);
  if (p.waves == 4) {
    switch (role) {
      case 1: return launch_ring_r<MT, 1, 4, false>(p, X, ldx, W, Y, act, s, stats);
      case 2: return launch_ring_r<MT, 2, 4, false>(p, X, ldx, W, Y, act, s);
      case 3: return launch_ring_r<MT, 3, 4, false>(p, X, ldx, W, Y, act, s);
      case 4: return launch_ring_r<MT, 4, 4, false>(p, X, ldx, W, Y, act, s);
      case 5: return launch_ring_r<MT, 5, 4, false>(p, X, ldx, W, Y, act, s);
      default: return launch_ring_r<MT, 0, 4, false>(p, X, ldx, W, Y, act, s);
    }
  }
  switch (role) {
    case 2: return launch_ring_r<MT, 2, 2, false>(p, X, ldx, W, Y, act, s);
    case 3: return launch_ring_r<MT, 3, 2, false>(p, X, ldx, W, Y, act, s);
    case 4: return launch_ring_r<MT, 4, 2, false>(p, X, ldx, W, Y, act, s);
    case 5: return launch_ring_r<MT, 5, 2, false>(p, X, ldx, W, Y, act, s);
    default: return launch_ring_r<MT, 0, 2, false>(p, X, ldx, W, Y, act, s);
  }
}

// Wide kernel shapes.  Row tiles MT in {3, 6, 10} (48, 96 or 160 rows).  NT W tiles per
// k-block (16 NT output features; X costs MT/NT of W's DMA traffic) is chosen by the planner
// from {8, 10, 12, 14, 16} so that the workgroups (one per CU) fill the 256 CUs; the ring is
// as deep as the X buffer leaves room for in 160 KB of LDS.  The 16-tile kernels get one
// symbol per projection (ROLE), the 8-tile ones one for the QKV, O and MLP-down projections,
// the others share role 0 (6 for the SiLU gate/up).  The LM
// head with block statistics at three row tiles may also take 32 tiles per k-block (512
// output features): its 128256 columns then fit one round of 251 workgroups instead of two
// rounds of 501, and X is half as large a share of each workgroup's stream (70B-shaped
// depth steps: 331.7 -> 315.7 us, 6.4 -> 6.7 TB/s).
constexpr int wide_ns(int mt, int nt) { return nt < 20 - mt ? nt : 20 - mt; }
constexpr int kWideMTs[] = {3, 6, 10};
constexpr int kWideNTs[] = {32, 16, 14, 12, 10, 8};

template <int MT, int NT, int ROLE, bool SILU>
int launch_wide_r(const e3h::GemmPlan& p, const void* X, int ldx, const void* W, float* Y, void* act,
                  hipStream_t s, float* stats = nullptr) {
  hipLaunchKernelGGL((k_gemm_wide<MT, NT, wide_ns(MT, NT), SILU, ROLE>), dim3(p.n_blocks * p.splits),
                     dim3(256), 0, s, (const bf16*)X, p.M, ldx, (const bf16*)W, p.N, p.K, Y, p.n_blocks,
                     p.chunks_total, p.chunks_per_split, act, p.N / 2, stats);
  return e3h::launch_status();
}

template <int MT>
int launch_wide(const e3h::GemmPlan& p, const void* X, int ldx, const void* W, float* Y, void* act,
                hipStream_t s, int role, float* stats) {
  if (p.silu) {
    switch (p.NT) {
      case 16: return launch_wide_r<MT, 16, 6, true>(p, X, ldx, W, Y, act, s);
      case 14: return launch_wide_r<MT, 14, 6, true>(p, X, ldx, W, Y, act, s);
      case 8: return launch_wide_r<MT, 8, 6, true>(p, X, ldx, W, Y, act, s);
      default: return EAGLE3_EUNSUPPORTED;
    }
  }
  switch (p.NT) {
    case 32:
      if constexpr (MT == 3) return launch_wide_r<MT, 32, 1, false>(p, X, ldx, W, Y, act, s, stats);
      return EAGLE3_EUNSUPPORTED;
    case 14: return launch_wide_r<MT, 14, 0, false>(p, X, ldx, W, Y, act, s);
    case 12: return launch_wide_r<MT, 12, 0, false>(p, X, ldx, W, Y, act, s);
    case 10: return launch_wide_r<MT, 10, 0, false>(p, X, ldx, W, Y, act, s);
    case 8:
      switch (role) {
        case 2: return launch_wide_r<MT, 8, 2, false>(p, X, ldx, W, Y, act, s);
        case 3: return launch_wide_r<MT, 8, 3, false>(p, X, ldx, W, Y, act, s);
        case 4: return launch_wide_r<MT, 8, 4, false>(p, X, ldx, W, Y, act, s);
        default: return launch_wide_r<MT, 8, 0, false>(p, X, ldx, W, Y, act, s);
      }
    case 16: break;
    default: return EAGLE3_EUNSUPPORTED;
  }
  switch (role) {
    case 1: return launch_wide_r<MT, 16, 1, false>(p, X, ldx, W, Y, act, s, stats);
    case 2: return launch_wide_r<MT, 16, 2, false>(p, X, ldx, W, Y, act, s);
    case 3: return launch_wide_r<MT, 16, 3, false>(p, X, ldx, W, Y, act, s);
    case 4: return launch_wide_r<MT, 16, 4, false>(p, X, ldx, W, Y, act, s);
    case 5: return launch_wide_r<MT, 16, 5, false>(p, X, ldx, W, Y, act, s);
    default: return launch_wide_r<MT, 16, 0, false>(p, X, ldx, W, Y, act, s);
  }
}

template <typename T>
int dispatch_gemm(const e3h::GemmPlan& p, const void* X, int ldx, const void* W, float* Y,
                  void* act, hipStream_t s, const char* tag, float* stats) {
  if constexpr (sizeof(T) == 2) {
    if (p.wide) {
      const int role = gemm_role(tag);
      switch (p.MT) {
        case 3: return launch_wide<3>(p, X, ldx, W, Y, act, s, role, stats);
        case 6: return launch_wide<6>(p, X, ldx, W, Y, act, s, role, stats);
        case 10: return launch_wide<10>(p, X, ldx, W, Y, act, s, role, stats);
        default: return EAGLE3_EUNSUPPORTED;
      }
    }
    if (p.ring) {
      const int role = gemm_role(tag);
      return p.MT == 1 ? launch_ring<1>(p, X, ldx, W, Y, act, s, role, stats)
                       : launch_ring<2>(p, X, ldx, W, Y, act, s, role, stats);
    }
  }
  switch (p.MT) {
    case 1: return dispatch_mt<T, 1>(p, X, ldx, W, Y, act, s);
    case 2: return dispatch_mt<T, 2>(p, X, ldx, W, Y, act, s);
    case 3: return dispatch_mt<T, 3>(p, X, ldx, W, Y, act, s);
    case 4: return dispatch_mt<T, 4>(p, X, ldx, W, Y, act, s);
    case 6: return dispatch_mt<T, 6>(p, X, ldx, W, Y, act, s);
    case 8: return dispatch_mt<T, 8>(p, X, ldx, W, Y, act, s);
    case 10: return dispatch_mt<T, 10>(p, X, ldx, W, Y, act, s);
    default: return EAGLE3_EUNSUPPORTED;
  }
}

}  // namespace

namespace e3h {

// Plan: single-wave workgroups when the n-blocks alone fill the chip (the LM head);
// otherwise four-wave workgroups and a k-split that brings the grid to about 256
// workgroups, keeping at least one X block of chunks per wave.
GemmPlan plan_gemm(int M, int N, int K, int dtype, bool silu, bool whole_k) {
  GemmPlan p;
  p.silu = silu;
  p.ring = false;
  p.tile = false;
  p.wide = false;
  p.M = M;
  p.N = N;
  p.K = K;
  const int mt_need = (M + 15) / 16;
  if (dtype == EAGLE3_BF16 && !silu && M > 160 && K % TILE_K == 0 && N % 4 == 0 &&
      (size_t)N * (size_t)K * 2 <= 0xFFFFFFFFull) {
    // many rows: the matrix cores bound it; 256 x 256 output tiles.  With fewer tiles than
    // CUs the k-range is split: pick the split count that minimises (rounds of workgroups over
    // the CUs) x (work per workgroup) + the partial sums' write and read, with the tile kernel
    // at ~1.2 PFLOP/s and the partial-sum traffic at ~5 TB/s.
    p.tile = true;
    p.MT = 0;
    p.NT = 0;
    p.n_blocks = (N + TILE_B - 1) / TILE_B;
    p.chunks_total = K / 32;
    p.waves = 4;
    const int n_k = K / TILE_K;
    const long tiles = (long)p.n_blocks * ((M + TILE_B - 1) / TILE_B);
    double best = 0;
    int best_s = 1;
    for (int sp = 1; sp <= 8 && sp <= n_k; ++sp) {
      const int kps = (n_k + sp - 1) / sp;
      const int s_eff = (n_k + kps - 1) / kps;
      const long wgs = tiles * s_eff;
      const long rounds = (wgs + kTileCUs - 1) / kTileCUs;
      const double t = (double)rounds * 2.0 * TILE_B * TILE_B * TILE_K * kps / (1.2e15 / kTileCUs) +
                       (s_eff > 1 ? 2.0 * s_eff * (double)M * N * 4 / 5e12 : 0.0);
      if (sp == 1 || t < best * 0.97) {
        best = t;
        best_s = s_eff;
      }
    }
    const int kps = (n_k + best_s - 1) / best_s;
    p.chunks_per_split = 2 * kps;
    p.splits = (n_k + kps - 1) / kps;
    return p;
  }
  if (dtype == EAGLE3_BF16 && mt_need <= 2 && K % 32 == 0 &&
      (!silu || (N / 2) % (16 * (kRingNTB / 2)) == 0)) {
    // LDS-ring kernel, 128 output features (or 64 gate + 64 up) per workgroup.  The LM head
    // has enough n-blocks for one wave per workgroup and no k-split; the SiLU gate/up needs
    // the whole k-range in one workgroup (four waves); the other projections use two waves
    // and a k-split in whole blocks to about kRingTargetWgs waves.
    p.ring = true;
    p.MT = mt_need < 1 ? 1 : mt_need;
    p.NT = kRingNTB;
    p.chunks_total = K / 32;
    int splits = 1;
    if (silu) {
      p.n_blocks = (N / 2) / (16 * (kRingNTB / 2));
      p.waves = 4;
    } else if (whole_k) {
      // no k-split (the LM head's block statistics need whole sums): four waves share a
      // workgroup's k-range unless the n-blocks alone fill the chip
      p.n_blocks = ((N + 15) / 16 + kRingNTB - 1) / kRingNTB;
      p.waves = p.n_blocks >= 512 ? 1 : 4;
    } else {
      p.n_blocks = ((N + 15) / 16 + kRingNTB - 1) / kRingNTB;
      p.waves = p.n_blocks >= 512 ? 1 : 2;
      // four waves per workgroup halve the split count (fewer fp32 partials for the
      // epilogue to read) when the workgroups, one per CU at 128 KB of LDS, still cover
      // three quarters of the CUs
      if (p.waves == 2 && p.n_blocks <= 64) {
        const int s4 = (kRingTargetWgs + p.n_blocks * 4 - 1) / (p.n_blocks * 4);
        const int c4 = ((p.chunks_total + s4 - 1) / s4 + 31) / 32 * 32;
        if ((long)p.n_blocks * ((p.chunks_total + c4 - 1) / c4) >= 192) p.waves = 4;
      }
      splits = (kRingTargetWgs + p.n_blocks * p.waves - 1) / (p.n_blocks * p.waves);
      if (p.waves == 1) splits = 1;   // >= 512 n-blocks cover the CUs: no fp32 partials to re-read
      // 65 .. 128 n-blocks (the 70B-shaped QKV of the root rows): two-wave workgroups over
      // kRingTargetWgs / 2 splits land unevenly on the CUs (two or three per CU); one four-wave
      // workgroup per CU over floor(256 / n_blocks) splits keeps the grid to one round
      // (measured 63 -> 55 us for 4 x 10240 x 16384)
      if (p.waves == 2 && p.n_blocks > 64 && p.n_blocks <= 128) {
        p.waves = 4;
        splits = 256 / p.n_blocks;
      }
    }
    int cps = (p.chunks_total + splits - 1) / splits;
    cps = (cps + 8 * p.waves - 1) / (8 * p.waves) * (8 * p.waves);
    p.chunks_per_split = cps;
    p.splits = (p.chunks_total + cps - 1) / cps;
    return p;
  }
  if (dtype == EAGLE3_BF16 && mt_need >= 3 && mt_need <= 10 && K % 32 == 0) {
    // 33 .. 160 rows: the wide kernel (waves split the rows, one shared W ring per
    // workgroup, one workgroup per CU).  For each tile count NT, a k-split in whole 8-chunk
    // blocks; the (NT, split) pair minimises (rounds of workgroups over the CUs) x (blocks per
    // workgroup) x (time of one block: NT W tiles from HBM at ~25 GB/s per CU, plus the MT X
    // tiles from L2) plus the fp32 partials' write and read.  Coefficients fitted to sweeps
    // of (NT, split) on this part: at three row tiles an X tile costs ~5% of a W tile and the
    // partials move at ~2.5 TB/s (eagle3_linear at the 70B-shaped O projection 34.3 -> 30.3 us
    // and MLP down 85.8 -> 82.2 us at 8 tiles x 4 splits instead of 16 x 8, sum pass included;
    // the drafter round, whose residual-norm launch reads the partials, measured the same); at
    // six and ten row tiles an X tile costs ~40% of a W tile and the partials move at ~6 TB/s.
    int mt = 0;
    for (int v : kWideMTs)
      if (v >= mt_need) {
        mt = v;
        break;
      }
    const int n_kb = (K / 32 + 7) / 8;
    double best = -1;
    for (int nt : kWideNTs) {
      if (silu && !(nt == 16 || nt == 14 || nt == 8)) continue;
      if (whole_k && nt != 16 && nt != 32) continue;   // the statistics epilogue takes 16 or 32 tiles
      if (nt == 32 && (mt != 3 || !whole_k)) continue;   // only the LM head at three row tiles
      if (silu && (N / 2) % (16 * (nt / 2))) continue;
      const int nbk = silu ? (N / 2) / (16 * (nt / 2)) : ((N + 15) / 16 + nt - 1) / nt;
      const double x_cost = mt == 3 ? 0.05 : 0.4, part_bw = mt == 3 ? 2.5e12 : 6e12;
      const double t_kb = (nt + x_cost * mt) * 8192.0 / 25e9;
      for (int kbps = n_kb; kbps >= 1; --kbps) {
        if ((silu || whole_k) && kbps != n_kb) break;   // the SiLU product needs the whole k-range
        const int sp = (n_kb + kbps - 1) / kbps;
        if (sp > 1 && (n_kb + sp - 1) / sp != kbps) continue;   // the same split count, fewer blocks
        const long wgs = (long)nbk * sp;
        const long rounds = (wgs + kTileCUs - 1) / kTileCUs;
        const double t = (double)rounds * kbps * t_kb + (sp > 1 ? 2.0 * sp * (double)M * N * 4 / part_bw : 0.0);
        if (best < 0 || t < best * 0.98) {
          best = t;
          p.wide = true;
          p.MT = mt;
          p.NT = nt;
          p.n_blocks = nbk;
          p.chunks_per_split = kbps * 8;
          p.splits = sp;
        }
      }
    }
    if (p.wide) {
      p.waves = 4;
      p.chunks_total = K / 32;
      return p;
    }
  }
  static const int mts[] = {1, 2, 3, 4, 6, 8, 10};
  p.MT = 0;
  for (int v : mts)
    if (v >= mt_need) {
      p.MT = v;
      break;
    }
  const int ntb = p.MT > 0 ? ntb_for(p.MT) : 8;
  const int kcb = p.MT > 0 ? kcb_for(p.MT) : 8;
  p.NT = ntb;
  const int ntile = (N + 15) / 16;
  p.n_blocks = (ntile + ntb - 1) / ntb;
  const int kpc = dtype == EAGLE3_BF16 ? 32 : 16;
  p.chunks_total = (K + kpc - 1) / kpc;
  int splits = 1;
  if (p.n_blocks >= 768) {
    p.waves = 1;
  } else {
    p.waves = 4;
    splits = 256 / p.n_blocks;
    const int max_splits = p.chunks_total / (p.waves * kcb);
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
  }
  if (silu) {
    // gate/up pairs: NTB/2 gate tiles per wave and one k-split
    p.n_blocks = (N / 2 + 16 * (ntb / 2) - 1) / (16 * (ntb / 2));
    p.waves = p.n_blocks >= 768 ? 1 : 4;
    splits = 1;
  }
  p.chunks_per_split = (p.chunks_total + splits - 1) / splits;
  p.splits = (p.chunks_total + p.chunks_per_split - 1) / p.chunks_per_split;
  return p;
}

int launch_gemm(const GemmPlan& p, int dtype, const void* X, int ldx, const void* W, float* Ypart,
                hipStream_t s, const char* tag, void* act, float* stats) {
  // the block statistics come from the LM head's ring or wide kernel without a k-split
  if (stats && (!gemm_block_stats_ok(p) || gemm_role(tag) != 1 || dtype != EAGLE3_BF16 ||
                (p.N + 127) / 128 > kLmStatsLd))
    return EAGLE3_EINVAL;
  if (p.tile) {
    if (dtype != EAGLE3_BF16) return EAGLE3_EUNSUPPORTED;
    // row offsets are 32-bit byte offsets from the operand base
    if ((size_t)p.M * (size_t)ldx * 2 > 0xFFFFFFFFull) return EAGLE3_EUNSUPPORTED;
    ProfScope ps(tag, s);
    const int tiles_m = (p.M + TILE_B - 1) / TILE_B;
    hipLaunchKernelGGL(k_gemm_tile, dim3(p.n_blocks * tiles_m * p.splits), dim3(256), 0, s, (const bf16*)X,
                       p.M, ldx, (const bf16*)W, p.N, p.K, Ypart, p.n_blocks, tiles_m,
                       p.chunks_per_split / 2);
    return launch_status();
  }
  if (p.MT == 0) return EAGLE3_EUNSUPPORTED;
  if (p.silu && (!act || (p.N / 2) % (16 * (p.NT / 2)))) return EAGLE3_EUNSUPPORTED;
  ProfScope ps(tag, s);
  if (dtype == EAGLE3_BF16) return dispatch_gemm<bf16>(p, X, ldx, W, Ypart, act, s, tag, stats);
  return dispatch_gemm<float>(p, X, ldx, W, Ypart, act, s, tag, nullptr);
}

int launch_epi_sum(const GemmPlan& p, const float* part, float* out, const float* resid,
                   hipStream_t s, const char* tag) {
  ProfScope ps(tag, s);
  const long total = (long)p.M * p.N / 4;
  hipLaunchKernelGGL(k_epi_sum, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part,
                     p.splits, p.M, p.N, out, resid);
  return launch_status();
}

}  // namespace e3h
