// Kernel 2 instances: bf16 elements and bf16 G_x, W_hh slices in LDS.
#include "scan_kernel.hpp"

namespace rnnk {

hipError_t launch_scan_bf16gx_lds(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream) {
  return launch_scan_proj<bf16, false, true>(a, lds, grid, stream);
}

}  // namespace rnnk
