// Kernel 2 dispatch: the launch shape and the instance of the scan kernel
// (scan_kernel.hpp) for the element type and where W_hh is kept.
#include "kernels.hpp"
#include "scan_kernel.hpp"

namespace rnnk {

int scan_lds_bytes(const ScanArgs& a, int esize) { return scan_lds(a, esize).total; }

hipError_t launch_scan_bf16_reg(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream);
hipError_t launch_scan_bf16_lds(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream);
hipError_t launch_scan_bf16gx_reg(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream);
hipError_t launch_scan_bf16gx_lds(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream);
hipError_t launch_scan_f32_reg(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream);
hipError_t launch_scan_f32_lds(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream);
hipError_t launch_scan_f32t_reg(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream);
hipError_t launch_scan_f32t_lds(const ScanArgs& a, int lds, dim3 grid, hipStream_t stream);

hipError_t launch_scan(const ScanArgs& a, int dtype_bf16, hipStream_t stream) {
  const int esize = dtype_bf16 ? 2 : 4;
  const int lds = scan_lds(a, esize).total;
  const dim3 grid(a.gpx > 0 ? a.nxcd * a.gpx * a.ns : a.nslot * a.D * a.nbb * a.ns);
  if (a.rsv) {  // training: fp32 only
    if (dtype_bf16 || a.gx_bf16) return hipErrorInvalidValue;
    return a.wreg ? launch_scan_f32t_reg(a, lds, grid, stream) : launch_scan_f32t_lds(a, lds, grid, stream);
  }
  if (dtype_bf16 && a.gx_bf16)
    return a.wreg ? launch_scan_bf16gx_reg(a, lds, grid, stream) : launch_scan_bf16gx_lds(a, lds, grid, stream);
  if (dtype_bf16)
    return a.wreg ? launch_scan_bf16_reg(a, lds, grid, stream) : launch_scan_bf16_lds(a, lds, grid, stream);
  if (a.gx_bf16) return hipErrorInvalidValue;  // bf16 G_x only with bf16 storage
  return a.wreg ? launch_scan_f32_reg(a, lds, grid, stream) : launch_scan_f32_lds(a, lds, grid, stream);
}

}  // namespace rnnk
