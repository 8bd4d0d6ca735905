// w12_gemm_inst.hip -- instantiates the GEMM kernel templates for one x
// height, chosen at compile time (-DW12_INST_M=1..8 for the GEMV, or
// -DW12_INST_MFMA / -DW12_INST_MFMA8 / -DW12_INST_MFMA16 for the 16- and
// 32-row MFMA tiles in 256-, 512- and 1024-thread workgroups,
// -DW12_INST_MFMA8_BIG for 64 and 128 rows),
// for the weight fetches (BF16 control, W12-v1 without and with an exception
// list, W12-b).  One object file per height keeps the build
// parallel.
#include "w12_gemm_kernels.hpp"

namespace w12 {

#if defined(W12_INST_M)
#define W12_CAT2(a, b) a##b
#define W12_CAT(a, b) W12_CAT2(a, b)
hipError_t W12_CAT(launch_gemv_m, W12_INST_M)(const GemmArgs& a, const Tiling& t, int fetch,
                                              hipStream_t s) {
    switch (fetch) {
        case kFetchW12:
            return a.exc_off != nullptr ? kern::dispatch<kern::FetchW12X, false, W12_INST_M>(a, t, s)
                                        : kern::dispatch<kern::FetchW12, false, W12_INST_M>(a, t, s);
        case kFetchW12B: return kern::dispatch<kern::FetchW12B, false, W12_INST_M>(a, t, s);
        default: return kern::dispatch<kern::FetchBF16, false, W12_INST_M>(a, t, s);
    }
}
#elif defined(W12_INST_MFMA)
template <int MT>
static hipError_t mfma_fetch(const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s) {
    switch (fetch) {
        case kFetchW12:
            return a.exc_off != nullptr ? kern::dispatch<kern::FetchW12X, true, MT>(a, t, s)
                                        : kern::dispatch<kern::FetchW12, true, MT>(a, t, s);
        case kFetchW12B: return kern::dispatch<kern::FetchW12B, true, MT>(a, t, s);
        default: return kern::dispatch<kern::FetchBF16, true, MT>(a, t, s);
    }
}
hipError_t launch_mfma_mt(int MT, const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s) {
    switch (MT) {
        case 16: return mfma_fetch<16>(a, t, fetch, s);
        case 32: return mfma_fetch<32>(a, t, fetch, s);
        default: return hipErrorInvalidValue;
    }
}
#elif defined(W12_INST_MFMA8)
template <int MT>
static hipError_t mfma8_fetch(const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s) {
    switch (fetch) {
        case kFetchW12:
            return a.exc_off != nullptr ? kern::dispatch8<kern::FetchW12X, MT>(a, t, s)
                                        : kern::dispatch8<kern::FetchW12, MT>(a, t, s);
        case kFetchW12B: return kern::dispatch8<kern::FetchW12B, MT>(a, t, s);
        default: return kern::dispatch8<kern::FetchBF16, MT>(a, t, s);
    }
}
hipError_t launch_mfma8_mt(int MT, const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s) {
    switch (MT) {
        case 16: return mfma8_fetch<16>(a, t, fetch, s);
        case 32: return mfma8_fetch<32>(a, t, fetch, s);
        default: return hipErrorInvalidValue;
    }
}
#elif defined(W12_INST_MFMA16)
template <int MT>
static hipError_t mfma16_fetch(const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s) {
    switch (fetch) {
        case kFetchW12:
            return a.exc_off != nullptr ? kern::dispatch16<kern::FetchW12X, MT>(a, t, s)
                                        : kern::dispatch16<kern::FetchW12, MT>(a, t, s);
        case kFetchW12B: return kern::dispatch16<kern::FetchW12B, MT>(a, t, s);
        default: return kern::dispatch16<kern::FetchBF16, MT>(a, t, s);
    }
}
hipError_t launch_mfma16_mt(int MT, const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s) {
    switch (MT) {
        case 16: return mfma16_fetch<16>(a, t, fetch, s);
        case 32: return mfma16_fetch<32>(a, t, fetch, s);
        default: return hipErrorInvalidValue;
    }
}
#elif defined(W12_INST_MFMA8_BIG)
template <int MT>
static hipError_t mfma8_fetch(const GemmArgs& a, const Tiling& t, int fetch, hipStream_t s) {
    switch (fetch) {
        case kFetchW12:
            return a.exc_off != nullptr ? kern::dispatch8<kern::FetchW12X, MT>(a, t, s)
                                        : kern::dispatch8<kern::FetchW12, MT>(a, t, s);
        case kFetchW12B: return kern::dispatch8<kern::FetchW12B, MT>(a, t, s);
        default: return kern::dispatch8<kern::FetchBF16, MT>(a, t, s);
    }
}
hipError_t launch_mfma8_big_mt(int MT, const GemmArgs& a, const Tiling& t, int fetch,
                               hipStream_t s) {
    switch (MT) {
        case 64: return mfma8_fetch<64>(a, t, fetch, s);
        case 128: return mfma8_fetch<128>(a, t, fetch, s);
        default: return hipErrorInvalidValue;
    }
}
#else
#error "define W12_INST_M, W12_INST_MFMA, W12_INST_MFMA8, W12_INST_MFMA16 or W12_INST_MFMA8_BIG"
#endif

}  // namespace w12
