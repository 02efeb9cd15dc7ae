// Host-only stand-ins for the kernel launchers, so that the C-ABI layer
// (fa_api.cpp) can be built with the address and undefined-behaviour
// sanitizers and driven on a machine without a GPU.  Each stub records the
// arguments it received and reports success; nothing touches a device.
#include "fa_decode.hpp"
#include "fa_launch.hpp"

namespace fa {

int g_launches = 0;
FwdArgs g_fwd;
BwdArgs g_bwd;
BwdArgs g_dq;
Fp8FwdArgs g_fp8;
DecodeArgs g_dec;

hipError_t launch_fwd(const FwdArgs& a) { ++g_launches; g_fwd = a; return hipSuccess; }
hipError_t launch_fwd_fp8(const Fp8FwdArgs& a) { ++g_launches; g_fp8 = a; return hipSuccess; }
hipError_t launch_bwd_preprocess(const BwdArgs& a) { ++g_launches; g_bwd = a; return hipSuccess; }
hipError_t launch_bwd_dkdv(const BwdArgs& a) { ++g_launches; g_bwd = a; return hipSuccess; }
hipError_t launch_bwd_dq(const BwdArgs& a) {
  ++g_launches; g_bwd = a; g_dq = a; return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs& a) { ++g_launches; g_dec = a; return hipSuccess; }

// The static scratch's device address: a fixed fake address here.
int g_scratch_lookups = 0;
hipError_t static_scratch(void** ptr) {
  ++g_scratch_lookups;
  *ptr = reinterpret_cast<void*>(0x7e0000000000ull);
  return hipSuccess;
}

}  // namespace fa
