// Test-only stand-in for the HIP runtime calls and kernel launches of the C
// ABI layer (csrc/api.cpp), so that the layer's checks and failure paths run
// on a machine without a GPU: linked with api.cpp and plan.cpp into a host
// library by tests/test_abi_host.py.  Nothing here runs on the product path.
//
// Devices: hipGetDevice reports the device set by ea_stub_set; the device's
// architecture name comes from the table below.  Launches do nothing and
// return the error set by ea_stub_set; so does the scratch lookup.
#include <hip/hip_runtime.h>

#include <cstring>

#include "bwd_kernel.h"
#include "fwd_kernel.h"

namespace {
int g_device = 0;
hipError_t g_get_device_error = hipSuccess;
hipError_t g_launch_error = hipSuccess;
hipError_t g_symbol_error = hipSuccess;
int g_launches = 0;
int g_symbol_lookups = 0;
const char* arch_of(int dev) {
  switch (dev) {
    case 0: return "gfx950:sramecc+:xnack-";
    case 1: return "gfx942:sramecc+:xnack-";   // another CDNA GPU
    case 2: return "gfx9500";                   // a longer name sharing the prefix
    case 3: return "gfx950";                    // no feature suffix
    default: return "gfx1100";
  }
}
}  // namespace

extern "C" {

// Configure the stand-ins: the current device, and the errors that
// hipGetDevice, a launch and the scratch lookup return.
void ea_stub_set(int device, int get_device_error, int launch_error, int symbol_error) {
  g_device = device;
  g_get_device_error = (hipError_t)get_device_error;
  g_launch_error = (hipError_t)launch_error;
  g_symbol_error = (hipError_t)symbol_error;
}
int ea_stub_launches(void) { return g_launches; }
int ea_stub_symbol_lookups(void) { return g_symbol_lookups; }

hipError_t hipGetDevice(int* device) {
  *device = g_device;
  return g_get_device_error;
}

hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* prop, int device) {
  std::memset(prop, 0, sizeof(*prop));
  std::strncpy(prop->gcnArchName, arch_of(device), sizeof(prop->gcnArchName) - 1);
  return hipSuccess;
}

}  // extern "C"

namespace ea {

hipError_t launch_fwd(const FwdParams&, int, int, int, hipStream_t) {
  ++g_launches;
  return g_launch_error;
}

hipError_t launch_bwd(const BwdParams&, int, int, hipStream_t) {
  ++g_launches;
  return g_launch_error;
}

hipError_t scratch_address(int, void** ptr) {
  ++g_symbol_lookups;
  *ptr = g_symbol_error == hipSuccess ? reinterpret_cast<void*>(0x100000) : nullptr;
  return g_symbol_error;
}

}  // namespace ea
