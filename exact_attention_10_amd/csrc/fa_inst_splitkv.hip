// Instances of the split-KV forward: the simple-schedule kernel in split mode (4
// waves, fp32 partials) for every dtype, D in {64, 128} and both masks, and
// the combine kernel.
#include "fa_combine.hpp"
#include "fa_kernel.hpp"
#include "fa_launch.hpp"

namespace {
template <int DT, int D, bool CAUSAL>
FaLaunch make() {
  using C = fa::Cfg<DT, D, CAUSAL, 4>;
  return {reinterpret_cast<const void *>(&fa::fa_fwd_kernel<DT, D, CAUSAL, 4, true>), C::LDS_BYTES, C::BM, 256};
}
template <int DT>
FaLaunch by_d(int d, bool causal) {
  if (d == 64) return causal ? make<DT, 64, true>() : make<DT, 64, false>();
  if (d == 128) return causal ? make<DT, 128, true>() : make<DT, 128, false>();
  return {nullptr, 0, 0, 0};
}
template <int DT>
const void *combine_by_d(int d) {
  if (d == 64) return reinterpret_cast<const void *>(&fa::fa_splitkv_combine_kernel<DT, 64>);
  if (d == 128) return reinterpret_cast<const void *>(&fa::fa_splitkv_combine_kernel<DT, 128>);
  return nullptr;
}
}  // namespace

FaLaunch fa_splitkv_instance(int dt, int d, bool causal) {
  switch (dt) {
    case fa::DT_FP32: return by_d<fa::DT_FP32>(d, causal);
    case fa::DT_FP16: return by_d<fa::DT_FP16>(d, causal);
    case fa::DT_BF16: return by_d<fa::DT_BF16>(d, causal);
    default: return {nullptr, 0, 0, 0};
  }
}

const void *fa_combine_instance(int dt, int d) {
  switch (dt) {
    case fa::DT_FP32: return combine_by_d<fa::DT_FP32>(d);
    case fa::DT_FP16: return combine_by_d<fa::DT_FP16>(d);
    case fa::DT_BF16: return combine_by_d<fa::DT_BF16>(d);
    default: return nullptr;
  }
}
