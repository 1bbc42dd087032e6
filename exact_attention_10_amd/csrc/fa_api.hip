// Host side of the gfx950 FlashAttention-2 forward library: argument
// validation, kernel selection and launch behind the C ABI of include/fa.h.
//
// Every argument is validated before the first HIP call, so the library can
// be loaded and its error paths exercised on a machine without a GPU. The
// library allocates no memory and keeps no per-call state; a launch is
// asynchronous on the caller's stream. The one piece of device memory it owns
// is the static scratch array of the no-allocation split-KV entry point.
#include "fa.h"
#include "fa_bwd.hpp"
#include "fa_combine.hpp"
#include "fa_kernel.hpp"
#include "fa_launch.hpp"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

namespace {

constexpr int kVersion = 100;  // 0.1.0

thread_local char g_hip_error[256] = "no HIP error recorded";

enum Family { kDefault = -1, kSimple = 0, kTwoGroup = 1, kTwoGroup16 = 2, kSimple16 = 3 };

struct Variant {
  const char *name;
  int family;      // kernel family
  int waves;       // waves per workgroup of the simple family (0 = per-shape default)
  int xcd_remap;
};

// Variants of the same computation; 0 is what fa_fwd runs.
const Variant kVariants[] = {
    {"default", kDefault, 0, 1},
    {"simple_bm128_xcd", kSimple, 4, 1},
    {"simple_bm128_linear", kSimple, 4, 0},
    {"simple_bm256_xcd", kSimple, 8, 1},
    {"simple_bm256_linear", kSimple, 8, 0},
    {"twogroup_bm256_xcd", kTwoGroup, 8, 1},
    {"twogroup16_bm256_xcd", kTwoGroup16, 8, 1},
    {"simple16_bm128_xcd", kSimple16, 4, 1},
    {"simple16_bm256_xcd", kSimple16, 8, 1},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

// The default. 16-bit D=128 runs the two-group kernel on 16x16x32 MFMAs, with
// or without the causal mask (3-5 % faster than the same schedule on 32x32x16
// MFMAs, which draw more power per FLOP at the board's power limit; causal
// 4-6 % faster than the simple schedule on 16x16x32). 16-bit D=64, whose
// softmax outweighs its matrix work, runs the simple schedule: on 16x16x32
// MFMAs with the causal mask (1-2 % faster there), on 32x32 ones without it.
// fp32 runs the simple schedule on 32x32 MFMAs. 16-bit D=128 uses 8 waves
// (256 query rows share each K/V tile), every other shape 4.
int default_family(int dtype, int64_t D, int causal) {
  if (dtype == FA_DTYPE_FP32) return kSimple;
  if (D == 128) return kTwoGroup16;
  return causal ? kSimple16 : kSimple;
}
int default_waves(int dtype, int64_t D, int causal) {
  (void)causal;
  return (dtype != FA_DTYPE_FP32 && D == 128) ? 8 : 4;
}

bool pick(int dtype, int64_t D, int causal, const Variant &var, FaLaunch *out) {
  if (dtype != FA_DTYPE_FP32 && dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return false;
  if (D != 64 && D != 128) return false;
  const int waves = var.waves ? var.waves : default_waves(dtype, D, causal);
  const int family = var.family == kDefault ? default_family(dtype, D, causal) : var.family;
  switch (family) {
    case kSimple:
      *out = dtype == FA_DTYPE_FP32   ? fa_simple_instance_fp32((int)D, causal != 0, waves)
             : dtype == FA_DTYPE_FP16 ? fa_simple_instance_fp16((int)D, causal != 0, waves)
                                      : fa_simple_instance_bf16((int)D, causal != 0, waves);
      break;
    case kTwoGroup:
      *out = fa_pp_instance(dtype, (int)D, causal != 0);
      break;
    case kTwoGroup16:
      *out = fa_pp16_instance(dtype, (int)D, causal != 0);
      break;
    case kSimple16:
      *out = fa_simple16_instance(dtype, (int)D, causal != 0, waves);
      break;
    default: return false;
  }
  return out->fn != nullptr;
}

int elem_bytes(int dtype) {
  return dtype == FA_DTYPE_FP32 ? 4 : (dtype == FA_DTYPE_FP16 || dtype == FA_DTYPE_BF16) ? 2 : 0;
}

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)bbytes && y < x + (uintptr_t)abytes;
}

int validate(const void *q, const void *k, const void *v, void *o, float *lse,
             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t n_kv, int64_t D,
             int causal_align, float scale, int dtype) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA_ERR_INVALID_ARG;
  if (n_kv < 0 || n_kv > Nk) return FA_ERR_INVALID_ARG;
  if (causal_align != FA_CAUSAL_TOP_LEFT && causal_align != FA_CAUSAL_BOTTOM_RIGHT) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  const int es = elem_bytes(dtype);
  if (es == 0) return FA_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  // one head of Q/O and of K/V must be addressable with 32-bit byte offsets
  // (this also keeps every row index and the causal offset within int range)
  if (Nq > (INT64_C(0x7fffffff) / (D * es)) || Nk > (INT64_C(0x7fffffff) / (D * es)))
    return FA_ERR_UNSUPPORTED;
  const int64_t tiles = (Nq + 127) / 128;
  if (B > INT64_C(0x7fffffff) / H || B * H > INT64_C(0x7fffffff) / tiles) return FA_ERR_UNSUPPORTED;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                        reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                        reinterpret_cast<uintptr_t>(lse);
  if (mis & 15) return FA_ERR_ALIGNMENT;
  const int64_t qbytes = B * H * Nq * D * es;  // < 2^62 given the limits above
  const int64_t kbytes = B * H * Nk * D * es;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) || overlaps(o, qbytes, v, kbytes))
    return FA_ERR_INVALID_ARG;
  if (lse) {
    const int64_t lbytes = B * H * Nq * (int64_t)sizeof(float);
    if (overlaps(lse, lbytes, q, qbytes) || overlaps(lse, lbytes, k, kbytes) ||
        overlaps(lse, lbytes, v, kbytes) || overlaps(lse, lbytes, o, qbytes))
      return FA_ERR_INVALID_ARG;
  }
  return FA_OK;
}

void opt_in_lds(const void *fn, int bytes);

// Compute units of the current device (cached per device).
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  static std::mutex mu;
  static int cache[64] = {0};
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

int launch(const void *q, const void *k, const void *v, void *o, float *lse,
           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t n_kv, int64_t D, int causal,
           int causal_align, float scale, int dtype, void *stream, int variant) {
  int rc = validate(q, k, v, o, lse, B, H, Nq, Nk, n_kv, D, causal_align, scale, dtype);
  if (rc != FA_OK) return rc;
  if (variant < 0 || variant >= kNumVariants) return FA_ERR_UNSUPPORTED;
  FaLaunch L;
  if (!pick(dtype, D, causal, kVariants[variant], &L)) return FA_ERR_UNSUPPORTED;
  if (L.lds > 65536) opt_in_lds(L.fn, L.lds);

  fa::Params p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.nq = Nq;
  p.nk = Nk;
  p.n_kv = n_kv;
  // top-left: query i sees keys j <= i; bottom-right: j <= i + (Nk - Nq)
  p.coff = causal_align == FA_CAUSAL_BOTTOM_RIGHT ? Nk - Nq : 0;
  p.nq_tiles = (int)((Nq + L.bm - 1) / L.bm);
  p.xcd_remap = kVariants[variant].xcd_remap;
  // scale * log2(e), formed in double and rounded once
  p.c = (float)((double)scale * 1.4426950408889634);

  // causal kernels that can pair query tiles take one workgroup per (head,
  // pair of tiles) when that grid still gives every CU a workgroup
  const int64_t pairs = (p.nq_tiles + 1) / 2;
  p.pair = (causal && L.paired && B * H * pairs >= cu_count()) ? 1 : 0;
  const int64_t per_head = p.pair ? pairs : p.nq_tiles;
  const dim3 grid((unsigned)(B * H * per_head));
  const dim3 block((unsigned)L.threads);
  void *args[] = {&p};
  hipError_t e = hipLaunchKernel(L.fn, grid, block, args, (size_t)L.lds,
                                 reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    std::snprintf(g_hip_error, sizeof(g_hip_error), "%s", hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// ---------------------------------------------------------------------------
// Split-KV: each (head, query tile) is split into n_splits shares of its key
// tiles, so a small grid still fills the chip; a second kernel combines the
// fp32 partials through their log-sum-exps.

constexpr int kSplitBM = 128;          // query rows per workgroup of the split kernel

int64_t split_grid(int64_t B, int64_t H, int64_t Nq) { return B * H * ((Nq + kSplitBM - 1) / kSplitBM); }

// Measured on MI355X: splitting pays only when the single-pass grid leaves
// most CUs idle and each split keeps enough key tiles to amortise the combine
// pass (8 tiles of 64 keys at D = 128, 16 at D = 64, whose tiles cost less).
// The splits then aim at about one workgroup per CU.
int auto_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D) {
  const int64_t g = split_grid(B, H, Nq);
  if (g <= 0 || g > 128) return 1;
  const int64_t tiles = (Nk + 63) / 64;
  int64_t ns = std::min<int64_t>((256 + g - 1) / g, tiles / (D == 64 ? 16 : 8));
  return (int)std::max<int64_t>(1, std::min<int64_t>(ns, fa::kMaxSplits));
}

// o_part at offset 0, lse_part at the next 256-byte boundary
struct SplitLayout {
  int64_t lse_off;
  int64_t bytes;
};
SplitLayout split_layout(int64_t B, int64_t H, int64_t Nq, int64_t D, int ns) {
  const int64_t rows = B * H * Nq;
  const int64_t o_bytes = (int64_t)ns * rows * D * (int64_t)sizeof(float);
  const int64_t lse_off = (o_bytes + 255) / 256 * 256;
  return {lse_off, lse_off + (int64_t)ns * rows * (int64_t)sizeof(float)};
}

int launch_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal,
                   int causal_align, float scale, int dtype, int num_splits, void *workspace,
                   size_t workspace_bytes, void *stream) {
  int rc = validate(q, k, v, o, lse, B, H, Nq, Nk, Nk, D, causal_align, scale, dtype);
  if (rc != FA_OK) return rc;
  if (num_splits < 0 || num_splits > fa::kMaxSplits) return FA_ERR_INVALID_ARG;
  const int ns = num_splits ? num_splits : auto_splits(B, H, Nq, Nk, D);
  if (ns == 1)   // nothing to split: the single-pass kernel, workspace untouched
    return launch(q, k, v, o, lse, B, H, Nq, Nk, Nk, D, causal, causal_align, scale, dtype, stream, 0);
  const SplitLayout lay = split_layout(B, H, Nq, D, ns);
  if (!workspace || (int64_t)workspace_bytes < lay.bytes) return FA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return FA_ERR_ALIGNMENT;
  const int es = elem_bytes(dtype);
  const int64_t qbytes = B * H * Nq * D * es, kbytes = B * H * Nk * D * es;
  if (overlaps(workspace, lay.bytes, q, qbytes) || overlaps(workspace, lay.bytes, k, kbytes) ||
      overlaps(workspace, lay.bytes, v, kbytes) || overlaps(workspace, lay.bytes, o, qbytes) ||
      (lse && overlaps(workspace, lay.bytes, lse, B * H * Nq * (int64_t)sizeof(float))))
    return FA_ERR_INVALID_ARG;
  if (split_grid(B, H, Nq) > INT64_C(0x7fffffff) / ns) return FA_ERR_UNSUPPORTED;

  const FaLaunch L = fa_splitkv_instance(dtype, (int)D, causal != 0);
  const void *comb = fa_combine_instance(dtype, (int)D);
  if (!L.fn || !comb) return FA_ERR_UNSUPPORTED;
  if (L.lds > 65536) opt_in_lds(L.fn, L.lds);

  fa::Params p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.nq = Nq;
  p.nk = Nk;
  p.n_kv = Nk;
  p.coff = causal_align == FA_CAUSAL_BOTTOM_RIGHT ? Nk - Nq : 0;
  p.nq_tiles = (int)((Nq + L.bm - 1) / L.bm);
  p.xcd_remap = 1;
  p.c = (float)((double)scale * 1.4426950408889634);
  p.n_splits = ns;
  p.n_heads = (int)(B * H);
  p.o_part = static_cast<float *>(workspace);
  p.lse_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + lay.lse_off);

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void *args[] = {&p};
  hipError_t e = hipLaunchKernel(L.fn, dim3((unsigned)(B * H * ns * p.nq_tiles)), dim3((unsigned)L.threads),
                                 args, (size_t)L.lds, st);
  if (e == hipSuccess) {
    fa::CombineParams cp;
    cp.o_part = p.o_part;
    cp.lse_part = p.lse_part;
    cp.o = o;
    cp.lse = lse;
    cp.rows = B * H * Nq;
    cp.n_splits = ns;
    void *cargs[] = {&cp};
    e = hipLaunchKernel(comb, dim3((unsigned)((cp.rows + 3) / 4)), dim3(256), cargs, 0, st);
  }
  if (e != hipSuccess) {
    std::snprintf(g_hip_error, sizeof(g_hip_error), "%s", hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// ---------------------------------------------------------------------------
// Split-KV without allocation: the fp32 partials go to a file-scope device
// array instead of a caller workspace. Each GPU holds its own copy of the
// array from the first use until the process ends; every call on one GPU
// reuses it, so calls that overlap on one GPU (different streams, no
// ordering) race on it. Nothing in it has to start at zero: every split
// writes all of its partial rows, including splits that see no key.

__device__ __attribute__((aligned(256))) char scratch[FA_SPLITKV_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device, looked up once per
// device with that device current. In host code the name `scratch` only
// stands for the array; kernels get this address.
int scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    std::snprintf(g_hip_error, sizeof(g_hip_error), "%s", hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  static std::mutex mu;
  static void *ptr[kMaxDevices] = {nullptr};
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      std::snprintf(g_hip_error, sizeof(g_hip_error), "scratch lookup: %s",
                    e != hipSuccess ? hipGetErrorString(e) : "null address");
      return FA_ERR_HIP;
    }
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return FA_OK;
}

int launch_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal,
                           int causal_align, float scale, int dtype, int num_splits,
                           void *stream) {
  int rc = validate(q, k, v, o, lse, B, H, Nq, Nk, Nk, D, causal_align, scale, dtype);
  if (rc != FA_OK) return rc;
  if (num_splits < 0 || num_splits > fa::kMaxSplits) return FA_ERR_INVALID_ARG;
  const int ns = num_splits ? num_splits : auto_splits(B, H, Nq, Nk, D);
  if (ns == 1)   // single pass: no partials, nothing of the scratch is used
    return launch(q, k, v, o, lse, B, H, Nq, Nk, Nk, D, causal, causal_align, scale, dtype, stream, 0);
  if (split_layout(B, H, Nq, D, ns).bytes > (int64_t)FA_SPLITKV_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void *ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != FA_OK) return rc;
  return launch_splitkv(q, k, v, o, lse, B, H, Nq, Nk, D, causal, causal_align, scale, dtype, ns,
                        ws, (size_t)FA_SPLITKV_SCRATCH_BYTES, stream);
}

// ---------------------------------------------------------------------------
// Backward: the dQ kernel (which also writes D = rowsum(dO * O)), then the
// dK/dV kernel, on the caller's stream.

int launch_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
               const float *lse, void *dq, void *dk, void *dv, float *delta, int64_t B, int64_t H,
               int64_t Nq, int64_t Nk, int64_t D, int causal, int causal_align, float scale,
               int dtype, void *stream) {
  if (!o || !dout || !lse || !dq || !dk || !dv || !delta) return FA_ERR_INVALID_ARG;
  // q, k, v, sizes, scale, dtype and alignment of q/k/v as in the forward
  // (dq stands in for the forward's output there)
  int rc = validate(q, k, v, dq, nullptr, B, H, Nq, Nk, Nk, D, causal_align, scale, dtype);
  if (rc != FA_OK) return rc;
  if (dtype == FA_DTYPE_FP32) return FA_ERR_UNSUPPORTED;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(o) | reinterpret_cast<uintptr_t>(dout) |
                        reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(dq) |
                        reinterpret_cast<uintptr_t>(dk) | reinterpret_cast<uintptr_t>(dv) |
                        reinterpret_cast<uintptr_t>(delta);
  if (mis & 15) return FA_ERR_ALIGNMENT;
  const int es = elem_bytes(dtype);
  const int64_t qb = B * H * Nq * D * es, kb = B * H * Nk * D * es, lb = B * H * Nq * (int64_t)sizeof(float);
  struct Span { const void *p; int64_t n; };
  const Span ins[] = {{q, qb}, {k, kb}, {v, kb}, {o, qb}, {dout, qb}, {lse, lb}};
  const Span outs[] = {{dq, qb}, {dk, kb}, {dv, kb}, {delta, lb}};
  for (const Span &a : outs) {
    for (const Span &b : ins)
      if (overlaps(a.p, a.n, b.p, b.n)) return FA_ERR_INVALID_ARG;
    for (const Span &b : outs)
      if (&a != &b && overlaps(a.p, a.n, b.p, b.n)) return FA_ERR_INVALID_ARG;
  }
  const int64_t nk_tiles = (Nk + 127) / 128;
  if (B * H > INT64_C(0x7fffffff) / nk_tiles) return FA_ERR_UNSUPPORTED;

  const FaBwdLaunch L = fa_bwd_instance(dtype, (int)D, causal != 0);
  if (!L.dq_fn || !L.dkdv_fn) return FA_ERR_UNSUPPORTED;
  if (L.dq_lds > 65536) opt_in_lds(L.dq_fn, L.dq_lds);
  if (L.dkdv_lds > 65536) opt_in_lds(L.dkdv_fn, L.dkdv_lds);

  fa::BwdParams p = {};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.delta = delta;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.nq = Nq;
  p.nk = Nk;
  p.coff = causal_align == FA_CAUSAL_BOTTOM_RIGHT ? Nk - Nq : 0;
  p.xcd_remap = 1;
  p.c = (float)((double)scale * 1.4426950408889634);
  p.scale = scale;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);

  p.n_tiles = (int)((Nq + 127) / 128);
  p.pair = (causal && B * H * ((p.n_tiles + 1) / 2) >= cu_count()) ? 1 : 0;
  void *args[] = {&p};
  hipError_t e = hipLaunchKernel(L.dq_fn, dim3((unsigned)(B * H * (p.pair ? (p.n_tiles + 1) / 2 : p.n_tiles))), dim3(256), args,
                                 (size_t)L.dq_lds, st);
  if (e == hipSuccess) {
    fa::BwdParams p2 = p;
    p2.n_tiles = (int)nk_tiles;
    p2.pair = (causal && B * H * ((p2.n_tiles + 1) / 2) >= cu_count()) ? 1 : 0;
    void *args2[] = {&p2};
    e = hipLaunchKernel(L.dkdv_fn, dim3((unsigned)(B * H * (p2.pair ? (p2.n_tiles + 1) / 2 : p2.n_tiles))), dim3(256), args2,
                        (size_t)L.dkdv_lds, st);
  }
  if (e != hipSuccess) {
    std::snprintf(g_hip_error, sizeof(g_hip_error), "%s", hipGetErrorString(e));
    return FA_ERR_HIP;
  }
  return FA_OK;
}

// Kernels that use more than 64 KB of LDS raise their limit once per process.
void opt_in_lds(const void *fn, int bytes) {
  static std::mutex mu;
  static const void *done[32];
  static int n_done = 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n_done; ++i)
    if (done[i] == fn) return;
  (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (n_done < 32) done[n_done++] = fn;
}

}  // namespace

extern "C" {

int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal,
              int causal_align, float scale, int dtype, void *stream) {
  return launch(q, k, v, o, lse, B, H, Nq, Nk, Nk, D, causal, causal_align, scale, dtype, stream, 0);
}

int fa_fwd_variant(const void *q, const void *k, const void *v, void *o, float *lse,
                   int64_t B, int64_t H, int64_t N, int64_t n_kv, int64_t D,
                   int causal, float scale, int dtype, void *stream, int variant) {
  return launch(q, k, v, o, lse, B, H, N, N, n_kv, D, causal, FA_CAUSAL_TOP_LEFT, scale, dtype,
                stream, variant);
}

int fa_fwd_nk(const void *q, const void *k, const void *v, void *o, float *lse,
              int64_t B, int64_t H, int64_t N, int64_t n_kv, int64_t D, int causal,
              float scale, int dtype, void *stream) {
  return fa_fwd_variant(q, k, v, o, lse, B, H, N, n_kv, D, causal, scale, dtype, stream, 0);
}

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int64_t B, int64_t H, int64_t N, int64_t D, int causal, float scale,
           int dtype, void *stream) {
  return fa_fwd_variant(q, k, v, o, lse, B, H, N, N, D, causal, scale, dtype, stream, 0);
}

int fa_splitkv_auto_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return 1;
  return auto_splits(B, H, Nq, Nk, D);
}

size_t fa_fwd_splitkv_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D,
                                     int num_splits) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || D < 1 || num_splits < 0 || num_splits > fa::kMaxSplits)
    return 0;
  const int ns = num_splits ? num_splits : auto_splits(B, H, Nq, Nk, D);
  return ns == 1 ? 0 : (size_t)split_layout(B, H, Nq, D, ns).bytes;
}

int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal,
                   int causal_align, float scale, int dtype, int num_splits, void *workspace,
                   size_t workspace_bytes, void *stream) {
  return launch_splitkv(q, k, v, o, lse, B, H, Nq, Nk, D, causal, causal_align, scale, dtype,
                        num_splits, workspace, workspace_bytes, stream);
}

int fa_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t D, int causal,
                           int causal_align, float scale, int dtype, int num_splits,
                           void *stream) {
  return launch_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, D, causal, causal_align, scale,
                                dtype, num_splits, stream);
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, void *dq, void *dk, void *dv, float *delta, int64_t B, int64_t H,
           int64_t Nq, int64_t Nk, int64_t D, int causal, int causal_align, float scale,
           int dtype, void *stream) {
  return launch_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, D, causal,
                    causal_align, scale, dtype, stream);
}

int fa_num_variants(void) { return kNumVariants; }

const char *fa_variant_name(int variant) {
  return (variant >= 0 && variant < kNumVariants) ? kVariants[variant].name : "";
}

const char *fa_strerror(int code) {
  switch (code) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dim, dtype, variant or size";
    case FA_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case FA_ERR_HIP: return g_hip_error;
    case FA_ERR_SCRATCH: return "split-KV partials larger than the library's static scratch";
    default: return "unknown status code";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
