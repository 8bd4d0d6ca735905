// w12_gemm_inst.hip -- instantiates the GEMM kernel templates for one x
// height, chosen at compile time (-DW12_INST_M=1..8 for the GEMV, or
// -DW12_INST_MFMA for the 16- and 32-row MFMA tiles).  One object file per
// height keeps the build parallel.
#include "w12_gemm_kernels.hpp"

namespace w12 {

#if defined(W12_INST_M)
#define W12_CAT2(a, b) a##b
#define W12_CAT(a, b) W12_CAT2(a, b)
hipError_t W12_CAT(launch_gemv_m, W12_INST_M)(const GemmArgs& a, const Tiling& t, bool is_w12,
                                              hipStream_t s) {
    return is_w12 ? kern::dispatch<kern::FetchW12, false, W12_INST_M>(a, t, s)
                  : kern::dispatch<kern::FetchBF16, false, W12_INST_M>(a, t, s);
}
#elif defined(W12_INST_MFMA)
hipError_t launch_mfma_mt(int MT, const GemmArgs& a, const Tiling& t, bool is_w12, hipStream_t s) {
    switch (MT) {
        case 16: return is_w12 ? kern::dispatch<kern::FetchW12, true, 16>(a, t, s)
                               : kern::dispatch<kern::FetchBF16, true, 16>(a, t, s);
        case 32: return is_w12 ? kern::dispatch<kern::FetchW12, true, 32>(a, t, s)
                               : kern::dispatch<kern::FetchBF16, true, 32>(a, t, s);
        default: return hipErrorInvalidValue;
    }
}
#elif defined(W12_INST_MFMA8)
hipError_t launch_mfma8_mt(int MT, const GemmArgs& a, const Tiling& t, bool is_w12, hipStream_t s) {
    switch (MT) {
        case 16: return is_w12 ? kern::dispatch8<kern::FetchW12, 16>(a, t, s)
                               : kern::dispatch8<kern::FetchBF16, 16>(a, t, s);
        case 32: return is_w12 ? kern::dispatch8<kern::FetchW12, 32>(a, t, s)
                               : kern::dispatch8<kern::FetchBF16, 32>(a, t, s);
        default: return hipErrorInvalidValue;
    }
}
#else
#error "define W12_INST_M, W12_INST_MFMA or W12_INST_MFMA8"
#endif

}  // namespace w12
