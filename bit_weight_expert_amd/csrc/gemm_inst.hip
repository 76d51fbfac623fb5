// One (format, epilogue) pair of the W4A16 GEMM launchers and their kernels,
// chosen by MOE_FMT and MOE_EPI on the compiler's command line (the build
// compiles this file once per pair).
#include "gemm_impl.h"

#if !defined(MOE_FMT) || !defined(MOE_EPI)
#error "define MOE_FMT and MOE_EPI"
#endif

namespace moe {
template hipError_t launch_epi<MOE_FMT, MOE_EPI>(int, int, GemmArgs, const WeightArgs&, EpiArgs, int,
                                                 hipStream_t);
}  // namespace moe
