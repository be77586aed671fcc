// dflash_op_linear_sk_noalloc: the stream-K projection of dflash_op_linear_sk with its scratch (partial
// tiles and tile counters) in a static device array instead of caller memory, for callers that cannot
// allocate device memory.  Every call on a GPU uses that GPU's copy of the array.
#include <mutex>

#include "../../include/dflash.h"
#include "kernels.h"

namespace {

constexpr int kStaticMaxN = 131072;  // output columns at most
constexpr size_t kStaticBytes = df::kSkPartBytes + (size_t)(kStaticMaxN / 16) * sizeof(int32_t);

// Held by each GPU the library runs on until the process ends.  In host code this name is a stand-in,
// not a device address: the per-device address below is what kernels receive.
static __device__ __align__(256) unsigned char scratch[kStaticBytes];

std::mutex g_mu;
void *g_ptr[64];  // per device ordinal: the device address of `scratch`, looked up on the first call

}  // namespace

extern "C" dflash_status dflash_op_linear_sk_noalloc(hipStream_t s, int32_t dtype, int32_t M, int32_t N, int32_t K,
                                                     const void *d_x, const void *d_w, float *d_y) {
  if (N < 1 || N > kStaticMaxN)
    return df::set_error(DFLASH_E_INVAL, "dflash_op_linear_sk_noalloc: N must be in [32, 131072]");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return df::set_error(DFLASH_E_DEVICE, "dflash_op_linear_sk_noalloc: no usable current device");
  void *ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {  // once per device, with that device current
      void *p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return df::set_error(DFLASH_E_DEVICE, "dflash_op_linear_sk_noalloc: device address of the static scratch");
      g_ptr[dev] = p;
    }
    ptr = g_ptr[dev];
  }
  return df::op_linear_sk(s, dtype, M, N, K, d_x, d_w, d_y, ptr);
}
