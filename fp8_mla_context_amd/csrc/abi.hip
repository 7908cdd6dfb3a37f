// ABI bookkeeping and host-only helpers of libmla_fp8.so.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "mla_internal.h"

namespace mla {

static thread_local char g_last_error[512] = {0};

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return MLA_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

int cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];  // zero: not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (dev < 0 ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;  // MI355X
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace mla

extern "C" {

int mla_abi_version(void) { return MLA_FP8_ABI_VERSION; }

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
  }
}

const char* mla_last_error(void) { return mla::g_last_error; }

int mla_check_descales_host(const float* descale, int32_t n) {
  if (descale == nullptr) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "descale is NULL");
  if (n < 0) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "n = %d < 0", n);
  const float lo = ldexpf(1.0f, -126), hi = ldexpf(1.0f, 126);
  for (int32_t i = 0; i < n; ++i) {
    float d = descale[i];
    if (!(isfinite(d) && d >= lo && d <= hi))
      return mla::fail(MLA_ERR_INVALID_ARGUMENT,
                       "descale[%d] = %g is not finite, positive and in [2^-126, 2^126]", i,
                       (double)d);
  }
  return mla::ok();
}

int mla_descale_from_amax_host(const float* amax, int32_t n, float* descale_out) {
  if (amax == nullptr || descale_out == nullptr)
    return mla::fail(MLA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (n < 0) return mla::fail(MLA_ERR_INVALID_ARGUMENT, "n = %d < 0", n);
  for (int32_t i = 0; i < n; ++i)
    if (!(isfinite(amax[i]) && amax[i] > 0.0f))
      return mla::fail(MLA_ERR_INVALID_ARGUMENT, "amax[%d] = %g is not finite and positive", i,
                       (double)amax[i]);
  // IEEE binary32 division is correctly rounded; volatile keeps it in fp32.
  for (int32_t i = 0; i < n; ++i) {
    volatile float a = amax[i];
    volatile float q = a / 448.0f;
    descale_out[i] = q;
  }
  return mla::ok();
}

}  // extern "C"
