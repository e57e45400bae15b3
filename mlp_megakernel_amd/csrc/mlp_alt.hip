// The resident MLP megakernel's second launch configuration (fewer waves per
// SIMD with more registers each, see MlpCfg in mlp_kernel.hpp), for the
// inference forward only: a candidate of the per-shape autotuner.  Its own
// translation unit so that the two sets of instantiations compile in
// parallel.
#include "mlp_kernel.hpp"

namespace coalesce {

hipError_t launch_mlp_alt(const MlpParams& p, int D, int L, int act, bool pad, int num_workgroups, int num_cus,
                          hipStream_t stream) {
  if (D == 128)
    return pad ? launch_da<128, false, true, 1>(p, L, act, num_workgroups, num_cus, stream)
               : launch_da<128, false, false, 1>(p, L, act, num_workgroups, num_cus, stream);
  return pad ? launch_da<64, false, true, 1>(p, L, act, num_workgroups, num_cus, stream)
             : launch_da<64, false, false, 1>(p, L, act, num_workgroups, num_cus, stream);
}

}  // namespace coalesce
