// Vocabulary sweep kernel: one 256-thread workgroup per (row, chunk); the
// device code (sweep_dev.h) is described there.
#include "sweep_dev.h"

namespace dt {
namespace {

template <bool BF16>
__global__ void __launch_bounds__(kThreads) sweep_kernel(SweepArgs a) {
    __shared__ __align__(16) unsigned char lds[sweepdev::SweepLds<BF16>::bytes];
    const int64_t row = blockIdx.x / a.C;
    const int chunk = blockIdx.x - (int)(row * a.C);
    sweepdev::sweep_chunk<BF16>(a, row, chunk, a.lists == kWaves ? sweepdev::kOutWaveLists : sweepdev::kOutMergedList,
                                lds);
}

}  // namespace

hipError_t launch_sweep(const SweepArgs& a, int64_t rows, int dtype, bool take_turns, hipStream_t stream) {
    const int64_t grid = rows * a.C;
    if (grid <= 0) return hipSuccess;
    // taking turns: the workgroup holds kSweepLdsTurn bytes of LDS in all
    // (the rest as unused dynamic LDS)
    const size_t own = dtype == DT_DTYPE_BF16 ? sweepdev::SweepLds<true>::bytes : sweepdev::SweepLds<false>::bytes;
    const size_t pad = take_turns && own < (size_t)kSweepLdsTurn ? (size_t)kSweepLdsTurn - own : 0;
    if (dtype == DT_DTYPE_BF16)
        hipLaunchKernelGGL(sweep_kernel<true>, dim3((unsigned)grid), dim3(kThreads), pad, stream, a);
    else
        hipLaunchKernelGGL(sweep_kernel<false>, dim3((unsigned)grid), dim3(kThreads), pad, stream, a);
    return hipGetLastError();
}

}  // namespace dt
