// The resident MLP megakernel with 16-row wave tiles (one sub-tile per wave,
// see MlpCfg in mlp_kernel.hpp): inference and training forward.  A batch of
// few row tiles runs on few waves, each through the whole layer chain, so
// halving a wave's rows halves that chain's latency; the same arithmetic per
// row, so the same bits as the 32-row tiles.  Its own translation unit so
// that the instantiations compile in parallel with mlp.hip's.
#include "mlp_kernel.hpp"

namespace coalesce {

hipError_t launch_mlp_small(const MlpParams& p, int D, int L, int act, bool store_acts, bool pad, int num_workgroups,
                            int num_cus, hipStream_t stream) {
  auto go = [&](auto d_tag) -> hipError_t {
    constexpr int D_ = decltype(d_tag)::value;
    if (pad)
      return store_acts ? launch_da<D_, true, true, 2>(p, L, act, num_workgroups, num_cus, stream)
                        : launch_da<D_, false, true, 2>(p, L, act, num_workgroups, num_cus, stream);
    return store_acts ? launch_da<D_, true, false, 2>(p, L, act, num_workgroups, num_cus, stream)
                      : launch_da<D_, false, false, 2>(p, L, act, num_workgroups, num_cus, stream);
  };
  if (D == 128) return go(std::integral_constant<int, 128>{});
  return go(std::integral_constant<int, 64>{});
}

}  // namespace coalesce
