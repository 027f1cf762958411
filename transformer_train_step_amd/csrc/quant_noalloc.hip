// ll_fp8_quant_tensorwise_noalloc: the e4m3 tensorwise quantiser for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops): the same computation as
// ll_fp8_quant_tensorwise, with its scratch in a static device array.
#include "api.h"
#include "quant.h"

#include <mutex>

using namespace ll;

// ------------------------------------------------------------------ allocation-free variant
// The quantisation state (amax accumulator, scale, inverse scale) lives in a static device array
// instead of a caller workspace: one copy per GPU, kept until the process ends. In host code the
// array's name is only a host-side handle; its device address is looked up once per device with
// hipGetSymbolAddress and that address is what the kernels receive.
constexpr size_t kQuantStaticScratchBytes = 256;
static __device__ __align__(256) unsigned char scratch[kQuantStaticScratchBytes];
static_assert(sizeof(QScale) <= kQuantStaticScratchBytes, "the static scratch holds one quantisation state");

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch` per device ordinal (null: not looked up)

int static_scratch(void** out) {
  int dev = 0;
  LL_HIP(hipGetDevice(&dev));
  LL_CHECK(dev >= 0 && dev < kMaxDevices, LL_ERR_UNSUPPORTED, "device ordinal beyond the static scratch table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    LL_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    LL_CHECK(p, LL_ERR_HIP, "hipGetSymbolAddress returned a null address for the static scratch");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LL_OK;
}
}  // namespace

extern "C" int ll_fp8_quant_tensorwise_noalloc(int32_t in_dtype, const void* x, int64_t rows, int64_t cols,
                                               int64_t ld, uint8_t* q, uint8_t* q_t, float* scale,
                                               float* inv_scale, void* stream) {
  // the scratch this call needs is one quantisation state, whatever the tensor size
  static_assert(sizeof(QScale) <= kQuantStaticScratchBytes, "scratch too small");
  LL_CHECK(ll_fp8_quant_workspace_bytes() <= kQuantStaticScratchBytes, LL_ERR_WORKSPACE,
           "the quantiser needs more scratch than the static buffer holds");
  void* ws = nullptr;
  if (int st = static_scratch(&ws)) return st;
  return ll_fp8_quant_tensorwise(in_dtype, x, rows, cols, ld, q, q_t, scale, inv_scale, ws,
                                 kQuantStaticScratchBytes, stream);
}
