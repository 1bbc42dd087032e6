// Instances of the simple-schedule kernel (fa_kernel.hpp) for bf16 inputs: D in {64, 128},
// both masks, 4 or 8 waves per workgroup. One translation unit per dtype so the
// instances compile in parallel.
#include "fa_kernel.hpp"
#include "fa_launch.hpp"

namespace {
template <int D, bool CAUSAL, int W>
FaLaunch make() {
  using C = fa::Cfg<fa::DT_BF16, D, CAUSAL, W>;
  return {reinterpret_cast<const void *>(&fa::fa_fwd_kernel<fa::DT_BF16, D, CAUSAL, W>), C::LDS_BYTES, C::BM, W * 64, CAUSAL ? 1 : 0};
}
template <int W>
FaLaunch by_d(int d, bool causal) {
  if (d == 64) return causal ? make<64, true, W>() : make<64, false, W>();
  if (d == 128) return causal ? make<128, true, W>() : make<128, false, W>();
  return {nullptr, 0, 0, 0};
}
}  // namespace

FaLaunch fa_simple_instance_bf16(int d, bool causal, int waves) {
  if (waves == 4) return by_d<4>(d, causal);
  if (waves == 8) return by_d<8>(d, causal);
  return {nullptr, 0, 0, 0};
}
