// Kernel instance tables shared by the host API and the instance files.
//
// Each kernel family is instantiated in a translation unit of its own
// (fa_inst_*.hip), so the instances compile in parallel; the host API picks
// an instance through these functions.
#pragma once

struct FaLaunch {
  const void *fn;   // __global__ function, nullptr if the combination has no instance
  int lds;          // dynamic LDS bytes per workgroup
  int bm;           // query rows per workgroup
  int threads;      // threads per workgroup
  int paired = 0;   // causal grid of (head, pair of query tiles): one workgroup per pair
};

// dt: 0 fp32, 1 fp16, 2 bf16 (the values of the fa.h dtype codes); d: 64 or 128
// waves: 4 or 8 per workgroup (8 for 16-bit dtypes only)
FaLaunch fa_simple_instance_fp32(int d, bool causal, int waves);
FaLaunch fa_simple_instance_fp16(int d, bool causal, int waves);
FaLaunch fa_simple_instance_bf16(int d, bool causal, int waves);
// the same schedule on 16x16x32 MFMAs (16-bit inputs only; null otherwise)
FaLaunch fa_simple16_instance(int dt, int d, bool causal, int waves);
// two-group forward (16-bit inputs, non-causal only; null otherwise)
FaLaunch fa_pp_instance(int dt, int d, bool causal);
// the same schedule on 16x16x32 MFMAs (16-bit inputs, both masks; null otherwise)
FaLaunch fa_pp16_instance(int dt, int d, bool causal);
// split-KV: the simple-schedule kernel in split mode (4 waves) and the combine kernel
FaLaunch fa_splitkv_instance(int dt, int d, bool causal);
const void *fa_combine_instance(int dt, int d);

// backward: the dQ (and D) kernel and the dK/dV kernel, 256 threads each;
// both null for an unsupported combination (fp32 has no backward)
struct FaBwdLaunch {
  const void *dq_fn;
  int dq_lds;
  const void *dkdv_fn;
  int dkdv_lds;
};
FaBwdLaunch fa_bwd_instance(int dt, int d, bool causal);
