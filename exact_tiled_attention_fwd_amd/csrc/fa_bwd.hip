#include "fa_common.h"
#include "fa_kernels.h"
namespace fa {
hipError_t launch_bwd(const BwdArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
}
