// Instances of the simple schedule on 16x16x32 MFMAs (fa_kernel16.hpp) for
// 16-bit inputs: D in {64, 128}, both masks, 4 or 8 waves per workgroup.
#include "fa_kernel16.hpp"
#include "fa_launch.hpp"

namespace {
template <int DT, int D, bool CAUSAL, int W>
FaLaunch make() {
  using C = fa::Cfg<DT, D, CAUSAL, W>;
  return {reinterpret_cast<const void *>(&fa::fa_fwd16_kernel<DT, D, CAUSAL, W>), C::LDS_BYTES, C::BM, W * 64, CAUSAL ? 1 : 0};
}
template <int DT, int W>
FaLaunch by_d(int d, bool causal) {
  if (d == 64) return causal ? make<DT, 64, true, W>() : make<DT, 64, false, W>();
  if (d == 128) return causal ? make<DT, 128, true, W>() : make<DT, 128, false, W>();
  return {nullptr, 0, 0, 0};
}
template <int DT>
FaLaunch by_waves(int d, bool causal, int waves) {
  if (waves == 4) return by_d<DT, 4>(d, causal);
  if (waves == 8) return by_d<DT, 8>(d, causal);
  return {nullptr, 0, 0, 0};
}
}  // namespace

FaLaunch fa_simple16_instance(int dt, int d, bool causal, int waves) {
  if (dt == 1) return by_waves<fa::DT_FP16>(d, causal, waves);
  if (dt == 2) return by_waves<fa::DT_BF16>(d, causal, waves);
  return {nullptr, 0, 0, 0};
}
