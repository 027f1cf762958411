// Host-side helpers shared by the entry points of libll: error text, argument checks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/ll.h"
#include "../../include/ll_testing.h"

namespace ll {

void set_error(const std::string& msg);
int fail(int status, const std::string& msg);   // records msg, returns status
void set_gemm_config_override(int cfg);

// Returns LL_ERR_HIP (with the HIP text recorded) if e is not hipSuccess.
#define LL_HIP(expr)                                                                           \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess)                                                                     \
      return ::ll::fail(LL_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));       \
  } while (0)

#define LL_CHECK(cond, status, msg)                                                            \
  do {                                                                                        \
    if (!(cond)) return ::ll::fail((status), (msg));                                          \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bump allocator over a caller-provided buffer (256-byte aligned sub-buffers). With base == null
// it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T> T* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
  size_t bytes() const { return (off + 255) & ~size_t(255); }
};

}  // namespace ll
