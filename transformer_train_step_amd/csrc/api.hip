// Status strings, last-error text and version of libll.
#include "api.h"

#include <mutex>
#include <vector>

namespace ll {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

// ------------------------------------------------------------------ launch trace
namespace {
struct TraceRec {
  const char* tag;
  int64_t m, n, k;
  int cfg, slices;
  hipEvent_t a, b;
};
std::mutex g_trace_mu;
std::vector<TraceRec> g_trace;
int g_trace_used = 0;
bool g_trace_on = false;
}  // namespace

bool trace_on() { return g_trace_on; }

static int g_gemm_cfg = 0;
int gemm_config_override() { return g_gemm_cfg; }
void set_gemm_config_override(int c) { g_gemm_cfg = c; }

int trace_open(const char* tag, hipStream_t s, int64_t m, int64_t n, int64_t k, int gemm_cfg, int slices) {
  std::lock_guard<std::mutex> lk(g_trace_mu);
  if (!g_trace_on || g_trace_used >= (int)g_trace.size()) return -1;
  const int slot = g_trace_used++;
  g_trace[slot].tag = tag;
  g_trace[slot].m = m;
  g_trace[slot].n = n;
  g_trace[slot].k = k;
  g_trace[slot].cfg = gemm_cfg;
  g_trace[slot].slices = slices;
  if (hipEventRecord(g_trace[slot].a, s) != hipSuccess) return -1;
  return slot;
}

void trace_close(int slot, hipStream_t s) { (void)hipEventRecord(g_trace[slot].b, s); }

}  // namespace ll

extern "C" {

int llt_trace_begin(int32_t capacity) {
  std::lock_guard<std::mutex> lk(ll::g_trace_mu);
  LL_CHECK(capacity > 0 && capacity <= (1 << 20), LL_ERR_INVALID_ARG, "capacity must be in [1, 2^20]");
  if ((int)ll::g_trace.size() != capacity) {
    for (auto& r : ll::g_trace) {
      (void)hipEventDestroy(r.a);
      (void)hipEventDestroy(r.b);
    }
    ll::g_trace.assign(capacity, ll::TraceRec{nullptr, 0, 0, 0, 0, 0, nullptr, nullptr});
    for (auto& r : ll::g_trace) {
      LL_HIP(hipEventCreate(&r.a));
      LL_HIP(hipEventCreate(&r.b));
    }
  }
  ll::g_trace_used = 0;
  ll::g_trace_on = true;
  return LL_OK;
}

int llt_trace_end(void) {
  std::lock_guard<std::mutex> lk(ll::g_trace_mu);
  ll::g_trace_on = false;
  return LL_OK;
}

int32_t llt_trace_count(void) {
  std::lock_guard<std::mutex> lk(ll::g_trace_mu);
  return ll::g_trace_used;
}

int llt_trace_get(int32_t i, const char** tag, float* ms, int64_t* mnk) {
  std::lock_guard<std::mutex> lk(ll::g_trace_mu);
  LL_CHECK(i >= 0 && i < ll::g_trace_used, LL_ERR_INVALID_ARG, "trace index out of range");
  LL_CHECK(tag && ms, LL_ERR_INVALID_ARG, "tag and ms must not be null");
  LL_HIP(hipEventSynchronize(ll::g_trace[i].b));
  LL_HIP(hipEventElapsedTime(ms, ll::g_trace[i].a, ll::g_trace[i].b));
  *tag = ll::g_trace[i].tag;
  if (mnk) {
    mnk[0] = ll::g_trace[i].m;
    mnk[1] = ll::g_trace[i].n;
    mnk[2] = ll::g_trace[i].k;
  }
  return LL_OK;
}

int llt_trace_get_gemm(int32_t i, int32_t* gemm_cfg, int32_t* slices) {
  std::lock_guard<std::mutex> lk(ll::g_trace_mu);
  LL_CHECK(i >= 0 && i < ll::g_trace_used, LL_ERR_INVALID_ARG, "trace index out of range");
  LL_CHECK(gemm_cfg && slices, LL_ERR_INVALID_ARG, "gemm_cfg and slices must not be null");
  *gemm_cfg = ll::g_trace[i].cfg;
  *slices = ll::g_trace[i].slices;
  return LL_OK;
}

const char* ll_status_string(int status) {
  switch (status) {
    case LL_OK: return "LL_OK";
    case LL_ERR_INVALID_ARG: return "LL_ERR_INVALID_ARG";
    case LL_ERR_UNSUPPORTED: return "LL_ERR_UNSUPPORTED";
    case LL_ERR_WORKSPACE: return "LL_ERR_WORKSPACE";
    case LL_ERR_HIP: return "LL_ERR_HIP";
    default: return "LL_ERR_UNKNOWN";
  }
}

const char* ll_last_error(void) { return ll::g_last_error.c_str(); }

int ll_version(void) { return 100; }

}  // extern "C"
