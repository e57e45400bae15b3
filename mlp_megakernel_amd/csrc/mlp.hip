// The resident MLP megakernel's launcher and its standard launch
// configuration, 32-row wave tiles (the kernels themselves are in
// mlp_kernel.hpp): inference forward and training forward, square and padded
// chains.
#include "mlp_kernel.hpp"

namespace coalesce {

int mlp_default_variant(int D, int64_t M, bool store_acts, int num_cus) {
  // 16-row wave tiles while a batch gives each wave of the grid at most ~96
  // rows: the chain of one tile through all layers is then the kernel's
  // latency, and halving a wave's rows halves it.  Measured per call (HIP
  // graph replays, 32-row -> 16-row tiles): 3 x 128, 32 / 4096 / 64K / 256K
  // rows 8.2 / 8.7 / 14.4 / 37.1 -> 6.9 / 7.4 / 13.9 / 35.8 us; 5 x 64 5.8 /
  // 6.1 / 9.4 / 24.2 -> 4.8 / 5.2 / 8.8 / 23.7 us.  From 512K rows on, 32-row
  // tiles are faster (their weight reads feed two MFMAs each): 3 x 128 on
  // 2^20 rows 135 against 141 us, 5 x 64 on 2^22 299 against 312 us.  The
  // width-128 training forward takes 16-row tiles at any size (2^20 rows of
  // 3 x 128: 0.400 -> 0.365 ms), the width-64 one keeps 32-row tiles for
  // large batches (2^22 rows of 5 x 64: 1.40 against 1.47 ms).
  const int64_t waves = (int64_t)num_cus * (D == 128 ? 12 : 16);
  if (store_acts && D == 128) return 2;
  return M <= 96 * waves ? 2 : 3;
}

hipError_t launch_mlp(const MlpParams& p, int D, int L, int act, bool store_acts, bool pad, int variant,
                      int num_workgroups, int num_cus, hipStream_t stream) {
  if (variant == 0) variant = mlp_default_variant(D, p.M, store_acts, num_cus);
  if (variant == 1 && !store_acts) return launch_mlp_alt(p, D, L, act, pad, num_workgroups, num_cus, stream);
  if (variant == 2) return launch_mlp_small(p, D, L, act, store_acts, pad, num_workgroups, num_cus, stream);
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
