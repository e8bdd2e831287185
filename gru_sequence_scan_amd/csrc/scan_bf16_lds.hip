// Kernel 2 instances: bf16 elements and fp32 G_x, W_hh slices in LDS.
#include "scan_kernel.hpp"

namespace rnnk {

hipError_t launch_scan_bf16_lds(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream) {
  return launch_scan_proj<bf16, false, false>(a, lds, grid, stream);
}

}  // namespace rnnk
