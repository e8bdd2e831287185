// Kernel 2 instances for training: f32 elements, W_hh slices in registers,
// the gate values written to the reserve.
#include "scan_kernel.hpp"

namespace rnnk {

hipError_t launch_scan_f32t_reg(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream) {
  return launch_scan_proj<float, true, false, true>(a, lds, grid, stream);
}

}  // namespace rnnk
