// Instances of the two-group ping-pong schedule (fa_kernel_pingpong.hpp):
// 16-bit dtypes, D in {64, 128}, both masks.
#include "fa_kernel_pingpong.hpp"
#include "fa_launch.hpp"

namespace {
template <int DT, int D, bool CAUSAL>
FaLaunch make() {
  using C = fa::PPCfg<DT, D, CAUSAL>;
  return {reinterpret_cast<const void *>(&fa::fa_fwd_pingpong_kernel<DT, D, CAUSAL>), C::LDS_BYTES, C::BM, 512};
}
template <int DT>
FaLaunch by_d(int d, bool causal) {
  if (d == 64) return causal ? make<DT, 64, true>() : make<DT, 64, false>();
  if (d == 128) return causal ? make<DT, 128, true>() : make<DT, 128, false>();
  return {nullptr, 0, 0, 0};
}
}  // namespace

FaLaunch fa_pingpong_instance(int dt, int d, bool causal) {
  switch (dt) {
    case fa::DT_FP16: return by_d<fa::DT_FP16>(d, causal);
    case fa::DT_BF16: return by_d<fa::DT_BF16>(d, causal);
    default: return {nullptr, 0, 0, 0};
  }
}
