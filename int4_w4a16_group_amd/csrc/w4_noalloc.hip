// Context-free routing entry point that allocates nothing, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops): top-k softmax routing and the (stream, expert) bucketing of
// w4_route, with the bucketing's scratch (pair-to-slot map, used experts, the
// 16-row work units) in a file-scope device array instead of a context's
// workspace.  Same kernel, same results.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "w4_internal.h"

namespace w4 {
// Set by context-free entry points; w4_last_error(NULL) returns it.
thread_local std::string g_free_err;
}  // namespace w4

using namespace w4;

namespace {

// Largest routing problem: B <= 32 rows, top_k <= 16, n_experts <= 256.
constexpr int kNaMaxB = 32, kNaMaxK = 16, kNaMaxE = kRouteMaxE;
constexpr size_t kAlignNa = 256;
size_t na_align(size_t x) { return (x + kAlignNa - 1) / kAlignNa * kAlignNa; }

// Scratch of one call, carved from the array in this order.
struct NaLayout {
  size_t inv, used, n_used, units, unit_rows, n_units, total;
};
NaLayout na_layout(int B, int E, int k) {
  NaLayout l{};
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = na_align(cur + bytes);
    return at;
  };
  const size_t units_cap = (size_t)E + (size_t)B * k / 16 + 1;
  l.inv = take((size_t)B * k * 4);
  l.used = take((size_t)E * 4);
  l.n_used = take(4);
  l.units = take(units_cap * 16);
  l.unit_rows = take(units_cap * 16 * 4);
  l.n_units = take(4);
  l.total = cur;
  return l;
}

// 32 KiB holds the largest problem (about 26 KiB, checked below).  Each GPU
// holds its own copy until the process ends.
constexpr size_t kScratchBytes = 32 << 10;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of each GPU's copy of the array (hipGetSymbolAddress with
// that device current); in host code the array's name is not an address.
constexpr int kNaMaxDevices = 64;
std::mutex g_na_mu;
void* g_na_ptr[kNaMaxDevices] = {};

int na_fail(int code, const std::string& m) {
  g_free_err = m;
  return code;
}

}  // namespace

extern "C" int w4_route_noalloc(int32_t B, int32_t E, int32_t k, const float* logits_dev, int32_t* ids_dev,
                                float* w_dev, int32_t* counts_dev, int32_t* offsets_dev, int32_t* pair_stream_dev,
                                int32_t* pair_rank_dev, void* stream) {
  static_assert(kScratchBytes >= (size_t)kNaMaxB * kNaMaxK * 4 + 4 * kAlignNa + (size_t)kNaMaxE * 4 +
                                     (size_t)(kNaMaxE + kNaMaxB * kNaMaxK / 16 + 1) * 16 * 5,
                "scratch holds the largest routing problem");
  if (B < 1 || B > kNaMaxB || k < 1 || k > kNaMaxK || E < k || E > kNaMaxE)
    return na_fail(W4_E_UNSUPPORTED, "w4_route_noalloc: needs 1 <= B <= 32, 1 <= top_k <= 16, top_k <= n_experts <= 256");
  if (!logits_dev || !ids_dev || !w_dev) return na_fail(W4_E_INVALID, "w4_route_noalloc: null logits, ids or w");
  const NaLayout lay = na_layout(B, E, k);
  if (lay.total > kScratchBytes)
    return na_fail(W4_E_UNSUPPORTED, "w4_route_noalloc: the routing scratch (" + std::to_string(lay.total) +
                                         " bytes) exceeds the static array (" + std::to_string(kScratchBytes) + ")");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return na_fail(W4_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kNaMaxDevices) return na_fail(W4_E_UNSUPPORTED, "w4_route_noalloc: device index too large");
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_na_mu);
    if (!g_na_ptr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return na_fail(W4_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
      g_na_ptr[dev] = p;
    }
    base = g_na_ptr[dev];
  }
  char* s = static_cast<char*>(base);
  RouteOut r;
  r.ids = ids_dev;
  r.w = w_dev;
  r.counts = counts_dev;
  r.offsets = offsets_dev;
  r.pair_stream = pair_stream_dev;
  r.pair_rank = pair_rank_dev;
  r.inv = reinterpret_cast<int32_t*>(s + lay.inv);
  r.used = reinterpret_cast<int32_t*>(s + lay.used);
  r.n_used = reinterpret_cast<int32_t*>(s + lay.n_used);
  r.units = reinterpret_cast<int4*>(s + lay.units);
  r.unit_rows = reinterpret_cast<int32_t*>(s + lay.unit_rows);
  r.n_units = reinterpret_cast<int32_t*>(s + lay.n_units);
  r.units_cap = E + B * k / 16 + 1;
  // every scratch word the kernel reads back it has written first in the same
  // launch, so nothing needs clearing between calls
  e = launch_route(logits_dev, B, E, k, r, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return na_fail(W4_E_HIP, std::string("w4_route_noalloc launch: ") + hipGetErrorString(e));
  return W4_OK;
}
