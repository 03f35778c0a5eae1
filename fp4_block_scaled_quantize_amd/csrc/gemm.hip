// gemm.hip -- placeholder launchers (filled in with the GEMM kernels)
#include "fp4_internal.h"
namespace fp4 {
hipError_t launch_gemm_mx(const GemmLaunch&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gemm_dq(const GemmLaunch&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_wo_gemm(const WoGemmLaunch&, hipStream_t) { return hipErrorNotSupported; }
}
