// Stand-ins for the kernel launchers, for the host-only sanitizer build of the
// C ABI: the argument checks under test return before any launch, so reaching
// one of these is itself a failure.
#include <cstdio>
#include <cstdlib>

#include "fa2_kernels.h"

namespace {
[[noreturn]] void reached(const char* what) {
    std::fprintf(stderr, "launcher reached in a host-only check: %s\n", what);
    std::abort();
}
}  // namespace

namespace fa2 {
hipError_t launch_fwd(const FwdParams&, int, bool, hipStream_t) { reached("fa2::launch_fwd"); }
hipError_t launch_bwd(const BwdParams&, int, bool, unsigned, hipStream_t) { reached("fa2::launch_bwd"); }
}  // namespace fa2
namespace fa2_f16 {
hipError_t launch_fwd(const FwdParams&, int, bool, hipStream_t) { reached("fa2_f16::launch_fwd"); }
hipError_t launch_bwd(const BwdParams&, int, bool, unsigned, hipStream_t) { reached("fa2_f16::launch_bwd"); }
}  // namespace fa2_f16
