// Stand-ins for the kernel launchers and kernel-side helpers, linked with
// the host-side sanitizer build of the C-ABI library (api.cpp) so that no
// device code is needed.  Every call the driver makes must be rejected
// before it reaches one of these; reaching one aborts the run.
#include <cstdio>
#include <cstdlib>

#include "fp4_internal.h"

namespace fp4 {

uint64_t g_exchange_wait_ticks = 20000000;
int64_t g_gemm_small_outputs = (int64_t)1 << 21;

[[noreturn]] static void reached(const char* what)
{
    std::fprintf(stderr, "abi sanitize driver: a rejected call reached %s\n", what);
    std::abort();
}

hipError_t launch_quantize(const QuantLaunch&, hipStream_t) { reached("launch_quantize"); }
hipError_t launch_quantize_t(const QuantLaunch&, hipStream_t, const RowOut*) { reached("launch_quantize_t"); }
hipError_t launch_dequantize(const DequantLaunch&, hipStream_t) { reached("launch_dequantize"); }
bool gemm_dq_supported(const ScaleFmtHost&, const ScaleFmtHost&, int) { reached("gemm_dq_supported"); }
hipError_t launch_gemm_mx(const GemmLaunch&, hipStream_t) { reached("launch_gemm_mx"); }
bool gemm_mx16_supported(const GemmLaunch&) { reached("gemm_mx16_supported"); }
hipError_t launch_gemm_mx16(const GemmLaunch&, hipStream_t) { reached("launch_gemm_mx16"); }
hipError_t launch_gemm_dq(const GemmLaunch&, hipStream_t) { reached("launch_gemm_dq"); }
bool gemm_small_supported(const GemmLaunch&) { reached("gemm_small_supported"); }
hipError_t launch_gemm_small(const GemmLaunch&, hipStream_t) { reached("launch_gemm_small"); }
hipError_t launch_wo_gemm(const WoGemmLaunch&, hipStream_t) { reached("launch_wo_gemm"); }
hipError_t launch_fill_zero_bf16(uint16_t*, int64_t, int64_t, int64_t, hipStream_t) { reached("fill_zero"); }

}  // namespace fp4
