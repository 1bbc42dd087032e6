// Instances of the simple-schedule kernel (fa_kernel.hpp) for fp32 inputs: D in {64, 128},
// both masks, 4 waves per workgroup. One translation unit per dtype so the instances compile in parallel.
#include "fa_kernel.hpp"
#include "fa_launch.hpp"

namespace {
template <int D, bool CAUSAL>
FaLaunch make() {
  using C = fa::Cfg<fa::DT_FP32, D, CAUSAL>;
  return {reinterpret_cast<const void *>(&fa::fa_fwd_kernel<fa::DT_FP32, D, CAUSAL>), C::LDS_BYTES, C::BM, 256, CAUSAL ? 1 : 0};
}
}  // namespace

FaLaunch fa_simple_instance_fp32(int d, bool causal, int waves) {
  if (waves != 4) return {nullptr, 0, 0, 0};
  if (d == 64) return causal ? make<64, true>() : make<64, false>();
  if (d == 128) return causal ? make<128, true>() : make<128, false>();
  return {nullptr, 0, 0, 0};
}
