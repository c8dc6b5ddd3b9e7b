// Status reporting and the gfx950 device check of the fp4moe C ABI.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "common.h"

namespace fp4moe {

static thread_local char g_last_error[512] = "";

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

// One verdict per device ordinal: 0 = unchecked, 1 = gfx950, 2 = other.
static int g_device_ok[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return set_error(FP4MOE_ERR_UNSUPPORTED, "no current HIP device");
  int v = __atomic_load_n(&g_device_ok[dev], __ATOMIC_ACQUIRE);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return set_error(FP4MOE_ERR_UNSUPPORTED, "hipGetDeviceProperties failed");
    v = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    __atomic_store_n(&g_device_ok[dev], v, __ATOMIC_RELEASE);
  }
  if (v != 1) return set_error(FP4MOE_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return FP4MOE_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(FP4MOE_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return FP4MOE_OK;
}

}  // namespace fp4moe

extern "C" const char* fp4moe_last_error(void) { return fp4moe::g_last_error; }

extern "C" int fp4moe_init(void) { return fp4moe::check_device(); }
