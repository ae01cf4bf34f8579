// na_m16.hip -- launches of the 16-bit MFMA kernels of na_mfma16.hpp.
//
// A translation unit of its own because it is compiled without IEEE-mode NaN
// handling (-fno-honor-nans, and the IEEE bit of the kernels' float mode
// cleared): the softmax maxima are then plain v_max / v_max3 instructions
// whose operands need no canonicalisation. The kernels never form NaNs from
// finite inputs (masked scores are -inf, empty windows are guarded), so the
// results are the same.
#include <hip/hip_runtime.h>

#include "na_mfma16.hpp"

namespace na {
namespace m16 {

template <typename T, int D, int W>
hipError_t launch_w(int kind, const Args<T> &a, hipStream_t s) {
    void (*kern)(Args<T>) = kind == 0   ? fwd_kernel<T, D, W>
                            : kind == 1 ? dq_kernel<T, D, W>
                                        : dkdv_kernel<T, D, W>;
    // static LDS only (two slab buffers sized for W): no dynamic-LDS attribute
    if (a.g.n_tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3(a.g.n_tiles), dim3(kTG), 0, s, a);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch(int kind, const Args<T> &a, hipStream_t s) {
    if (a.g.box_w > a.g.wmax) return hipErrorInvalidValue;
    switch (a.g.wmax) {
    case 24: return launch_w<T, D, 24>(kind, a, s);
    case 32: return launch_w<T, D, 32>(kind, a, s);
    case 48: return launch_w<T, D, 48>(kind, a, s);
    default: return hipErrorInvalidValue;
    }
}

template hipError_t launch<bf16, 32>(int, const Args<bf16> &, hipStream_t);
template hipError_t launch<bf16, 64>(int, const Args<bf16> &, hipStream_t);
template hipError_t launch<f16, 32>(int, const Args<f16> &, hipStream_t);
template hipError_t launch<f16, 64>(int, const Args<f16> &, hipStream_t);

}  // namespace m16
}  // namespace na
