// Instances of the backward kernels (fa_bwd.hpp): 16-bit dtypes, D in {64, 128},
// both masks.
#include "fa_bwd.hpp"
#include "fa_launch.hpp"

namespace {
template <int DT, int D, bool CAUSAL>
FaBwdLaunch make() {
  using C = fa::BwdCfg<D>;
  return {reinterpret_cast<const void *>(&fa::fa_bwd_dq_kernel<DT, D, CAUSAL>), C::Q_LDS,
          reinterpret_cast<const void *>(&fa::fa_bwd_dkdv_kernel<DT, D, CAUSAL>), C::K_LDS};
}
template <int DT>
FaBwdLaunch by_d(int d, bool causal) {
  if (d == 64) return causal ? make<DT, 64, true>() : make<DT, 64, false>();
  if (d == 128) return causal ? make<DT, 128, true>() : make<DT, 128, false>();
  return {nullptr, 0, nullptr, 0};
}
}  // namespace

FaBwdLaunch fa_bwd_instance(int dt, int d, bool causal) {
  switch (dt) {
    case fa::DT_FP16: return by_d<fa::DT_FP16>(d, causal);
    case fa::DT_BF16: return by_d<fa::DT_BF16>(d, causal);
    default: return {nullptr, 0, nullptr, 0};
  }
}
