// The resident MLP megakernel's default launch configuration (the kernels
// themselves are in mlp_kernel.hpp): inference forward and training forward,
// square and padded chains.
#include "mlp_kernel.hpp"

namespace coalesce {

hipError_t launch_mlp(const MlpParams& p, int D, int L, int act, bool store_acts, bool pad, int num_workgroups,
                      int num_cus, hipStream_t stream) {
  auto go = [&](auto d_tag) -> hipError_t {
    constexpr int D_ = decltype(d_tag)::value;
    if (pad)
      return store_acts ? launch_da<D_, true, true, 0>(p, L, act, num_workgroups, num_cus, stream)
                        : launch_da<D_, false, true, 0>(p, L, act, num_workgroups, num_cus, stream);
    return store_acts ? launch_da<D_, true, false, 0>(p, L, act, num_workgroups, num_cus, stream)
                      : launch_da<D_, false, false, 0>(p, L, act, num_workgroups, num_cus, stream);
  };
  if (D == 128) return go(std::integral_constant<int, 128>{});
  return go(std::integral_constant<int, 64>{});
}

}  // namespace coalesce
