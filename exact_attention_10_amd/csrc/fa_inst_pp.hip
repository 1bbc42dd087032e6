// Instances of the two-group forward kernels (fa_kernel_pp.hpp on 32x32x16
// MFMAs, without a causal mask; fa_kernel_pp16.hpp on 16x16x32 MFMAs, with or
// without it): 16-bit inputs, D in {64, 128}.
#include "fa_kernel_pp16.hpp"
#include "fa_launch.hpp"

namespace {
template <int DT, int D, bool M16, bool CAUSAL>
FaLaunch make() {
  using C = fa::PPCfg<D>;
  const void *fn = M16 ? reinterpret_cast<const void *>(&fa::fa_fwd_pp16_kernel<DT, D, CAUSAL>)
                       : reinterpret_cast<const void *>(&fa::fa_fwd_pp_kernel<DT, D>);
  return {fn, C::LDS_BYTES, C::BM, C::WAVES * 64, CAUSAL ? 1 : 0};
}
template <int DT, bool M16, bool CAUSAL = false>
FaLaunch by_d(int d) {
  if (d == 64) return make<DT, 64, M16, CAUSAL>();
  if (d == 128) return make<DT, 128, M16, CAUSAL>();
  return {nullptr, 0, 0, 0};
}
}  // namespace

FaLaunch fa_pp_instance(int dt, int d, bool causal) {
  if (causal) return {nullptr, 0, 0, 0};
  if (dt == 1) return by_d<fa::DT_FP16, false>(d);
  if (dt == 2) return by_d<fa::DT_BF16, false>(d);
  return {nullptr, 0, 0, 0};
}

FaLaunch fa_pp16_instance(int dt, int d, bool causal) {
  if (dt == 1) return causal ? by_d<fa::DT_FP16, true, true>(d) : by_d<fa::DT_FP16, true>(d);
  if (dt == 2) return causal ? by_d<fa::DT_BF16, true, true>(d) : by_d<fa::DT_BF16, true>(d);
  return {nullptr, 0, 0, 0};
}
