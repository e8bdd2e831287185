// Kernel 2 instances: f32 elements, W_hh slices in registers.
#include "scan_kernel.hpp"

namespace rnnk {

hipError_t launch_scan_f32_reg(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream) {
  return launch_scan_proj<float, true, false>(a, lds, grid, stream);
}

}  // namespace rnnk
