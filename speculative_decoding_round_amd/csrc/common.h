// Shared device/host helpers for libeagle3 (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "eagle3.h"

namespace e3 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// 16-byte vector load/store (addresses must be 16-byte aligned).
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Elements of T in one 16-byte chunk.
template <typename T>
struct Vec {
  static constexpr int N = 16 / sizeof(T);
};

// Unpack element e of a 16-byte chunk of T into fp32.
template <typename T>
__device__ __forceinline__ float chunk_elem(u32x4 v, int e);
template <>
__device__ __forceinline__ float chunk_elem<float>(u32x4 v, int e) {
  return __uint_as_float(v[e]);
}
template <>
__device__ __forceinline__ float chunk_elem<bf16>(u32x4 v, int e) {
  uint32_t w = v[e >> 1];
  uint32_t bits = (e & 1) ? (w & 0xffff0000u) : (w << 16);
  return __uint_as_float(bits);
}

// ---------------------------------------------------------------------------------------
// MFMA on one 16-byte operand chunk per lane (16x16 output tile, fp32 accumulate).
//
// Operand layout (16x16 MFMA family): lane l supplies row (A) / column (B) l % 16 and the
// k-group l / 16.  One 16-byte chunk per lane covers 4 * Vec<T>::N values of k across the
// four lane groups: group g holds k in [g*N, (g+1)*N) of the chunk.  A and B use the same
// k placement, so the product is the plain sum over k.  Output: lane l holds column l % 16,
// rows 4*(l/16) + i, i = 0..3.
// ---------------------------------------------------------------------------------------
template <typename T>
struct Mfma;

template <>
struct Mfma<bf16> {
  static constexpr int KPC = 32;  // k per chunk (8 per lane group)
  __device__ __forceinline__ static floatx4 run(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  static constexpr int KPC = 16;  // k per chunk (4 per lane group, one per MFMA)
  __device__ __forceinline__ static floatx4 run(u32x4 a, u32x4 b, floatx4 c) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j]), __uint_as_float(b[j]), c,
                                               0, 0, 0);
    return c;
  }
};

// ---------------------------------------------------------------------------------------
// Wave / block reductions (wave64), without LDS: quad_perm xor 1 and xor 2, then the
// half-row and row mirrors (DPP), then the gfx950 row-pair and half-wave swaps.  Every
// step combines a lane with a partner symmetrically, so all 64 lanes end with the same
// bits, and the order is fixed, so results are deterministic.
// ---------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// (own, partner) pairs for the cross-row steps: lanes l and l^16 (resp. l^32)
__device__ __forceinline__ void swap16(uint32_t v, uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap32(uint32_t v, uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  a = r[0];
  b = r[1];
}

template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, __uint_as_float(dpp_u<kDppXor1>(__float_as_uint(v))));
  v = op(v, __uint_as_float(dpp_u<kDppXor2>(__float_as_uint(v))));
  v = op(v, __uint_as_float(dpp_u<kDppHalfMirror>(__float_as_uint(v))));
  v = op(v, __uint_as_float(dpp_u<kDppMirror>(__float_as_uint(v))));
  uint32_t a, b;
  swap16(__float_as_uint(v), a, b);
  v = op(__uint_as_float(a), __uint_as_float(b));
  swap32(__float_as_uint(v), a, b);
  return op(__uint_as_float(a), __uint_as_float(b));
}

// Reduction within each 16-lane row (lanes 16r .. 16r+15); every lane of the row gets it.
template <typename Op>
__device__ __forceinline__ float row16_reduce(float v, Op op) {
  v = op(v, __uint_as_float(dpp_u<kDppXor1>(__float_as_uint(v))));
  v = op(v, __uint_as_float(dpp_u<kDppXor2>(__float_as_uint(v))));
  v = op(v, __uint_as_float(dpp_u<kDppHalfMirror>(__float_as_uint(v))));
  return op(v, __uint_as_float(dpp_u<kDppMirror>(__float_as_uint(v))));
}

// Reduction across the four 16-lane rows only (lanes l, l^16, l^32, l^48).
template <typename Op>
__device__ __forceinline__ float row_reduce(float v, Op op) {
  uint32_t a, b;
  swap16(__float_as_uint(v), a, b);
  v = op(__uint_as_float(a), __uint_as_float(b));
  swap32(__float_as_uint(v), a, b);
  return op(__uint_as_float(a), __uint_as_float(b));
}

struct OpAdd {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, OpAdd()); }
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, OpMax()); }

// Block-wide sum with a fixed reduction tree (deterministic for a given block size).
// `scratch` needs blockDim.x/64 floats.  All threads receive the result.
__device__ __forceinline__ float block_sum(float v, float* scratch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += scratch[i];
  return t;
}

// Block-wide max; scratch needs blockDim.x/64 floats.  All threads receive the result.
__device__ __forceinline__ float block_max(float v, float* scratch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  float t = scratch[0];
  for (int i = 1; i < nw; ++i) t = fmaxf(t, scratch[i]);
  return t;
}

// (value desc, index asc) ordering used by every argmax / top-K in the library.  Written with
// non-short-circuit operators: the short-circuit form compiles to exec-mask branches in loops.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return (va > vb) | ((va == vb) & (ia < ib));
}

__device__ __forceinline__ void argmax_pair(float& v, int& i, float ov, int oi) {
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// (value desc, index asc) argmax over the wave; every lane receives the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_pair(v, i, __uint_as_float(dpp_u<kDppXor1>(__float_as_uint(v))), (int)dpp_u<kDppXor1>((uint32_t)i));
  argmax_pair(v, i, __uint_as_float(dpp_u<kDppXor2>(__float_as_uint(v))), (int)dpp_u<kDppXor2>((uint32_t)i));
  argmax_pair(v, i, __uint_as_float(dpp_u<kDppHalfMirror>(__float_as_uint(v))),
              (int)dpp_u<kDppHalfMirror>((uint32_t)i));
  argmax_pair(v, i, __uint_as_float(dpp_u<kDppMirror>(__float_as_uint(v))), (int)dpp_u<kDppMirror>((uint32_t)i));
  uint32_t va, vb, ia, ib;
  swap16(__float_as_uint(v), va, vb);
  swap16((uint32_t)i, ia, ib);
  v = __uint_as_float(va);
  i = (int)ia;
  argmax_pair(v, i, __uint_as_float(vb), (int)ib);
  swap32(__float_as_uint(v), va, vb);
  swap32((uint32_t)i, ia, ib);
  v = __uint_as_float(va);
  i = (int)ia;
  argmax_pair(v, i, __uint_as_float(vb), (int)ib);
}

// Block argmax; scratch needs 2 * blockDim.x/64 words.  All threads receive the result.
__device__ __forceinline__ void block_argmax(float& v, int& i, float* sv, int* si) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  wave_argmax(v, i);
  __syncthreads();
  if (lane == 0) {
    sv[w] = v;
    si[w] = i;
  }
  __syncthreads();
  v = sv[0];
  i = si[0];
  for (int k = 1; k < nw; ++k)
    if (better(sv[k], si[k], v, i)) {
      v = sv[k];
      i = si[k];
    }
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Row helpers: 8 consecutive elements of a row as float (one or two 16-byte accesses).
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  const u32x4 a = ld16(p), b = ld16(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = __uint_as_float(a[i]);
    v[4 + i] = __uint_as_float(b[i]);
  }
}
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float* v) {
  const u32x4 a = ld16(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = chunk_elem<bf16>(a, i);
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* v);
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* v) {
  st16(p, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
  st16(p + 4, u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
}
template <>
__device__ __forceinline__ void store8<bf16>(bf16* p, const float* v) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = static_cast<bf16>(v[i]);
  st16(p, __builtin_bit_cast(u32x4, o));
}

// Sum of two values over the block (fixed order); scratch needs 2 * 16 floats.
__device__ __forceinline__ void block_sum2(float& a, float& b, float* scratch) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  a = wave_sum(a);
  b = wave_sum(b);
  if (lane == 0) {
    scratch[w] = a;
    scratch[16 + w] = b;
  }
  __syncthreads();
  a = 0.f;
  b = 0.f;
  for (int i = 0; i < nw; ++i) {
    a += scratch[i];
    b += scratch[16 + i];
  }
}

// ---------------------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11) and the fixed float32 natural log used for Gumbel
// noise.  Contraction is disabled so every multiply and add rounds on its own, as in the
// definition of the generator's output map.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// ln v for positive normal v: v = 2^e m, m in [sqrt(1/2), sqrt(2)); s = (m-1)/(m+1);
// ln v = e*ln2_hi + (e*ln2_lo + 2*(s + s^3 (1/3 + s^2 (1/5 + s^2 (1/7 + s^2/9))))).
__device__ __forceinline__ float ln_fixed(float v) {
#pragma clang fp contract(off)
  const uint32_t bits = __float_as_uint(v);
  int e = (int)((bits >> 23) & 0xffu) - 127;
  float m = __uint_as_float((bits & 0x7fffffu) | 0x3f800000u);
  if (m >= __uint_as_float(0x3fb504f3u)) {
    m = m * 0.5f;
    e += 1;
  }
  const float ef = (float)e;
  const float s = (m - 1.0f) / (m + 1.0f);
  const float t = s * s;
  float p = __uint_as_float(0x3de38e39u);           // 1/9
  p = p * t + __uint_as_float(0x3e124925u);         // 1/7
  p = p * t + __uint_as_float(0x3e4ccccdu);         // 1/5
  p = p * t + __uint_as_float(0x3eaaaaabu);         // 1/3
  const float r = s + (s * t) * p;
  return ef * __uint_as_float(0x3f317200u) + (ef * __uint_as_float(0x35bfbe8eu) + 2.0f * r);
}

__device__ __forceinline__ float gumbel_from_word(uint32_t x) {
#pragma clang fp contract(off)
  const float u = ((float)(x >> 9) + 0.5f) * 1.1920928955078125e-07f;  // 2^-23
  const float inner = -ln_fixed(u);
  return -ln_fixed(inner);
}

// Request of a flattened node: the b with cu[b] <= node < cu[b + 1] (binary search).
__device__ __forceinline__ int find_request(const int32_t* cu, int B, int node) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= node)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// fn(std::integral_constant<int, i>{}) for i = I .. N - 1, unrolled at compile time (for
// register arrays indexed by a loop counter).
template <int I, int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (I < N) {
    fn(std::integral_constant<int, I>{});
    static_for<I + 1, N>(fn);
  }
}

}  // namespace e3

// ---------------------------------------------------------------------------------------
// Host side: launch timing registry and workspace carving
// ---------------------------------------------------------------------------------------
namespace e3h {

// RAII: records an event pair around the launches in its scope when timing is enabled.
struct ProfScope {
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
  int slot;
  hipStream_t stream;
};

// Bump allocator over a workspace; with base == nullptr it only measures.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t n) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
  size_t size() const { return (off + 255) & ~size_t(255); }
};

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? EAGLE3_OK : EAGLE3_EHIP;
}

inline int elem_size(int dtype) { return dtype == EAGLE3_BF16 ? 2 : 4; }
inline bool dtype_ok(int dtype) { return dtype == EAGLE3_F32 || dtype == EAGLE3_BF16; }

}  // namespace e3h

#define E3_RETURN_IF(cond, code) \
  do {                           \
    if (cond) return (code);     \
  } while (0)
