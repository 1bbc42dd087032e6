// Instances of the two-group forward kernel (fa_kernel_pp.hpp): 16-bit inputs,
// D in {64, 128}, no causal mask.
#include "fa_kernel_pp.hpp"
#include "fa_launch.hpp"

namespace {
template <int DT, int D>
FaLaunch make() {
  using C = fa::PPCfg<D>;
  return {reinterpret_cast<const void *>(&fa::fa_fwd_pp_kernel<DT, D>), C::LDS_BYTES, C::BM, C::WAVES * 64, 0};
}
template <int DT>
FaLaunch by_d(int d) {
  if (d == 64) return make<DT, 64>();
  if (d == 128) return make<DT, 128>();
  return {nullptr, 0, 0, 0};
}
}  // namespace

FaLaunch fa_pp_instance(int dt, int d, bool causal) {
  if (causal) return {nullptr, 0, 0, 0};
  if (dt == 1) return by_d<fa::DT_FP16>(d);
  if (dt == 2) return by_d<fa::DT_BF16>(d);
  return {nullptr, 0, 0, 0};
}
