// paged_decode_kernel (decode_kernel.hpp) built with VGPR-form MFMAs
// (build.py), for the short segments that launch_paged_decode sends here.
#include "decode_kernel.hpp"

namespace osc {

hipError_t launch_decode_kernel_vgpr(const DecodeArgs& a, bool bf16, int D, unsigned grid,
                                     hipStream_t stream) {
    return launch_decode_kernel_here(a, bf16, D, grid, stream);
}

}  // namespace osc
