// eagle3_accept_noalloc: the acceptance step for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid allocation).  It
// runs the kernels of eagle3_accept, whose only scratch memory is the per-(node, 4096-token
// chunk) winner list (value and token, 8 bytes per entry), in a fixed device array of this
// file instead of a caller workspace.
//
// The array is one per GPU (each device holds its own copy of a module's __device__
// variables) and lives until the process ends.  Its device address is looked up once per
// device, with that device current, by hipGetSymbolAddress; host code uses only that address.
// Every call on a GPU shares the array: calls that overlap on one GPU (several streams, or
// several host threads) race on it.  The scan writes every entry the path pass reads, so
// nothing needs clearing between calls.
#include <mutex>

#include "common.h"
#include "internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(1) << 20;   // 1 MiB: T * ceil(V / 4096) <= 131072
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array (looked up on first use per device).
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EAGLE3_EHIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return EAGLE3_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EAGLE3_OK;
}

}  // namespace

EAGLE3_API size_t eagle3_accept_noalloc_max_entries(void) { return kScratchBytes / 8 - 64; }

EAGLE3_API int eagle3_accept_noalloc(int B, int T, const int32_t* cu_nodes, const int32_t* tokens,
                                     const int32_t* parents, const uint64_t* mask, int W64,
                                     const void* logits, int V, int dtype, float temperature,
                                     uint64_t seed, uint64_t round, int max_depth, int32_t* accept_len,
                                     int32_t* path, int32_t* out_tokens, int32_t* bonus, void* stream) {
  if (B <= 0 || T < B || V <= 0 || W64 < 1 || max_depth < 0) return EAGLE3_EINVAL;
  if (dtype != EAGLE3_F32 && dtype != EAGLE3_BF16) return EAGLE3_EINVAL;
  if (!(temperature >= 0.f) || temperature == __builtin_huge_valf()) return EAGLE3_EINVAL;
  if (W64 > 4) return EAGLE3_EUNSUPPORTED;
  if (!cu_nodes || !tokens || !parents || !mask || !logits || !accept_len || !path || !out_tokens ||
      !bonus)
    return EAGLE3_EINVAL;
  // the winner list must fit the array: T * chunks entries of a float and an int, the int
  // part starting 256-byte aligned after the float part
  const size_t entries = (size_t)T * (size_t)e3h::accept_chunks(V);
  if (entries > eagle3_accept_noalloc_max_entries()) return EAGLE3_EUNSUPPORTED;
  void* base = nullptr;
  const int st = scratch_for_current_device(&base);
  if (st) return st;
  float* pv = static_cast<float*>(base);
  int* pi = reinterpret_cast<int*>(static_cast<unsigned char*>(base) + ((entries * 4 + 255) / 256) * 256);
  return e3h::launch_accept(B, T, cu_nodes, tokens, parents, mask, W64, logits, V, dtype, temperature,
                            seed, round, max_depth, accept_len, path, out_tokens, bonus, pv, pi,
                            (hipStream_t)stream);
}
