// Two-group ("ping-pong") schedule of the FlashAttention-2 forward for
// gfx950, 16-bit inputs.
//
// The arithmetic per key tile is the one of fa_kernel.hpp (S^T = K Q^T on
// MFMA, online softmax with exp2 and a shared exponent reference, O^T +=
// V^T P^T on MFMA); what changes is who does it when. A workgroup has 8
// waves in two groups of 4; waves w and w+4 run on the same SIMD. Each tile
// step is split into two phases separated by workgroup barriers:
//
//   phase A: group 0 runs the matrix products of step j,
//            group 1 runs the softmax of tile j-1;
//   phase B: group 0 runs the softmax of tile j,
//            group 1 runs the matrix products of step j,
//
// where the matrix products of step j are PV(j-1) followed by QK(j). So on
// every SIMD one wave keeps the matrix core busy while the other works on
// exp/max/sum, instead of two waves drifting in and out of phase. Both
// groups run the same instruction stream (matrix products of step j,
// barrier, softmax of tile j, barrier); group 1 is offset by one phase by an
// extra barrier before its loop, group 0 by one after it.
//
// K_j and V_{j-1} (one "stage") are read in both phases of step j; group 0
// streams the stages by direct global->LDS loads through a ring of STAGES
// LDS buffers, STAGES-1 steps ahead. The loop is unrolled by STAGES so that
// every LDS address is a register plus an immediate offset.
//
// The online-softmax recurrence, masks, tile skipping and finalisation follow
// the same passages as fa_kernel.hpp ("A09 - Advanced Triton &
// FlashAttention", section 3; "Triton: FlashAttention-2 Forward Pass";
// "Building a Verifiable FlashAttention Forward from PyTorch to Triton",
// Part 3).
#pragma once

#include "fa_kernel.hpp"

#include <type_traits>

namespace fa {

template <int DT, int D, bool CAUSAL>
struct PPCfg {
  static constexpr int WAVES = 8;
  static constexpr int BM = WAVES * 32;                 // query rows per workgroup
  static constexpr int BN = 64;                         // keys per tile
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;     // one K or V tile
  static constexpr int STAGES = 4;
  static constexpr int AHEAD = STAGES - 1;              // stages in flight ahead of use
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;    // K_j then V_{j-1}
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  // stages are loaded by the 4 waves of group 0
  static constexpr int LOADS = TILE_BYTES / (4 * 64 * 16);   // per thread per matrix
  static_assert(TILE_BYTES % (4 * 64 * 16) == 0, "tile must split into 16-byte lane loads");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt_n() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int DT, int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) fa_fwd_pingpong_kernel(Params p) {
  static_assert(DT == DT_BF16 || DT == DT_FP16, "16-bit inputs only");
  using C = PPCfg<DT, D, CAUSAL>;
  constexpr int BN = C::BN, BM = C::BM, RB = C::ROW_BYTES;
  constexpr int NKC = D / 16;       // MFMAs along the head dim for S^T
  constexpr int NKB = BN / 32;      // 32-key blocks per tile
  constexpr int NDB = D / 32;       // 32-wide head-dim blocks of O^T
  constexpr int NPC = BN / 16;      // MFMAs along the keys for O^T
  constexpr int PER_STAGE = 2 * C::LOADS;

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if (p.xcd_remap && (nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int bh = bid / p.nq_tiles;
  int qt = bid - bh * p.nq_tiles;
  if (CAUSAL) qt = p.nq_tiles - 1 - qt;
  const int64_t Nq = p.nq;
  const int q0 = qt * BM;
  const int qw = q0 + wave * 32;
  const int my_q = qw + l32;
  const int coff = (int)p.coff;            // causal: key j visible to query i when j <= i + coff

  const int64_t q_head = Nq * (int64_t)D;      // elements per head of Q and O
  const int64_t k_head = p.nk * (int64_t)D;    // elements per head of K and V
  const char *qh = (const char *)p.q + (int64_t)bh * q_head * 2;
  const char *kh = (const char *)p.k + (int64_t)bh * k_head * 2;
  const char *vh = (const char *)p.v + (int64_t)bh * k_head * 2;
  const int n_kv = (int)p.n_kv;
  int kend = n_kv;
  if (CAUSAL) kend = min(kend, q0 + BM + coff);
  const int n_tiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  // ---- Q fragments of this wave's 32 rows ----
  uint32_t qf[NKC][4];
  {
    const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(qh, (uint32_t)(q_head * 2));
    const uint32_t row_off = (uint32_t)my_q * RB;
    const bool row_ok = my_q < Nq;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const uint32_t off = row_off + (uint32_t)((kc * 16 + half * 8) * 2);
      u32x4 x = row_ok ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off, 0, 0))
                       : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < 4; ++w) qf[kc][w] = x[w];
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- stage transfers (group 0): K_j and V_{j-1} into ring buffer j % STAGES ----
  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);
  uint32_t dma_off[C::LOADS];
#pragma unroll
  for (int u = 0; u < C::LOADS; ++u) {
    const int lds_off = ((wave & 3) * C::LOADS + u) * 1024 + lane * 16;
    const int row = lds_off / RB;
    dma_off[u] = (uint32_t)row * RB + (((lds_off % RB) / 16) ^ swz<RB>(row)) * 16;
  }
  // tile t of a matrix as a buffer resource: base at its first row, range
  // ending at key n_kv (rows past it, and tiles outside [0, n_tiles), read 0)
  auto tile_rsrc = [&](const char *base, int t) __attribute__((always_inline)) {
    const bool ok = t >= 0 && t < n_tiles;
    const int kstart = ok ? t * BN : 0;
    return make_rsrc_words(base + (int64_t)kstart * RB, ok ? (uint32_t)(n_kv - kstart) * RB : 0u);
  };
  auto issue_stage = [&](int j, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const i32x4 kr = tile_rsrc(kh, j), vr = tile_rsrc(vh, j - 1);
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const uint32_t lds = smem_base + buf * C::STAGE_BYTES + ((wave & 3) * C::LOADS + u) * 1024;
      lds_dma16(kr, dma_off[u], lds);
      lds_dma16(vr, dma_off[u], lds + C::TILE_BYTES);
    }
  };

  // ---- lane offsets of the MFMA operand fragments inside a tile ----
  uint32_t k_off[NKC], v_off[2][NDB];
  {
    const int g = lane >> 4, r = (lane & 15) >> 2, cq = lane & 3;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) k_off[kc] = l32 * RB + (((kc * 2 + half) ^ swz<RB>(l32)) * 16);
#pragma unroll
    for (int jg = 0; jg < 2; ++jg)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = db * 32 + (g & 1) * 16 + cq * 4;
        const int key = jg * 8 + (g >> 1) * 4 + r;
        v_off[jg][db] = key * RB + ((((col * 2) / 16) ^ swz<RB>(key)) * 16) + (col * 2) % 16;
      }
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  f32x16 s[NKB];
#pragma unroll
  for (int i = 0; i < NKB; ++i) s[i] = f32x16{};
  u32x4 pf[NPC];                 // P^T fragments (packed 16-bit) of the last softmaxed tile
#pragma unroll
  for (int i = 0; i < NPC; ++i) pf[i] = u32x4{0, 0, 0, 0};
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = p.c;

  // a tile is visible to this wave unless every key is in the wave's future
  auto visible = [&](int t) __attribute__((always_inline)) { return t >= 0 && t < n_tiles && (!CAUSAL || t * BN <= qw + 31 + coff); };

  auto mfma16 = [&](u32x4 a, u32x4 b, f32x16 cin) __attribute__((always_inline)) -> f32x16 {
    if constexpr (DT == DT_BF16)
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), cin, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), cin, 0, 0, 0);
  };

  // ---- matrix products of step j from the stage in buffer BUF ----
  auto gemm = [&](int j, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const char *kl = smem + buf * C::STAGE_BYTES;
    const char *vl = kl + C::TILE_BYTES;
    if (visible(j - 1)) {
      // all V^T fragments first, then the MFMAs: the reads stream while the
      // first products run
      u32x4 vf[NPC][NDB];
#pragma unroll
      for (int pc = 0; pc < NPC; ++pc)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int jg = 0; jg < 2; ++jg) {
            const char *addr = vl + v_off[jg][db] + pc * 16 * RB;
            const u32x2 xx = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4 *)addr));
            vf[pc][db][jg * 2] = xx[0];
            vf[pc][db][jg * 2 + 1] = xx[1];
          }
#pragma unroll
      for (int pc = 0; pc < NPC; ++pc)
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = mfma16(vf[pc][db], pf[pc], acc[db]);
    }
    if (visible(j)) {
      u32x4 kf[NKC][NKB];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) kf[kc][kb] = *(const FA_LDS u32x4 *)(kl + k_off[kc] + kb * 32 * RB);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const u32x4 b = {qf[kc][0], qf[kc][1], qf[kc][2], qf[kc][3]};
          s[kb] = mfma16(kf[kc][kb], b, kc == 0 ? f32x16{} : s[kb]);
        }
    }
  };

  // ---- softmax of tile t: scores in s -> packed P in pf, rescale of acc ----
  auto softmax = [&](int t) __attribute__((always_inline)) {
    if (!visible(t)) return;
    const int kstart = t * BN;
    if ((kstart + BN > n_kv) || (CAUSAL && kstart + BN - 1 > qw + coff)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kstart + kb * 32 + 8 * (i / 4) + half * 4 + (i % 4);
          if ((key >= n_kv) || (CAUSAL && key > my_q + coff)) s[kb][i] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = halves_max(mx) * c;
    // move the exponent reference only when a row max exceeds it by more than
    // 2^kRescaleSlack (see fa_kernel.hpp)
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
    const float neg = (m_run == -INFINITY) ? 0.f : -m_run;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, neg));
        s[kb][i] = e;
        rs += e;
      }
    l_run += rs;
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc) {
      const int kb = pc / 2, i0 = (pc % 2) * 8;
#pragma unroll
      for (int w = 0; w < 4; ++w) pf[pc][w] = pack2<DT>(s[kb][i0 + 2 * w], s[kb][i0 + 2 * w + 1]);
    }
  };

  // one step: phase with the products of step j, phase with the softmax of
  // tile j; BUF = j % STAGES is a compile-time constant
  auto step = [&](int j, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const bool more = j + C::AHEAD <= n_tiles;
    if (group == 0 && more) issue_stage(j + C::AHEAD, std::integral_constant<int, (buf + C::AHEAD) % C::STAGES>{});
    gemm(j, buf_c);
    __syncthreads();
    softmax(j);
    // (group 0) stage j+1 must be complete before the next step; later ones may fly
    if (group == 0) {
      if (j + C::AHEAD <= n_tiles) wait_vmcnt_n<(C::AHEAD - 1) * PER_STAGE>();
      else wait_vmcnt_n<0>();
    }
    __syncthreads();
  };

  // ---- prologue: group 0 puts stages 0 .. AHEAD-1 in flight; stage 0 complete ----
  if (group == 0) {
    issue_stage(0, std::integral_constant<int, 0>{});
    issue_stage(1, std::integral_constant<int, 1>{});
    if constexpr (C::AHEAD >= 3) issue_stage(2, std::integral_constant<int, 2>{});
    wait_vmcnt_n<(C::AHEAD - 1) * PER_STAGE>();
  }
  __syncthreads();

  // ---- steps 0 .. n_tiles; group 1 runs one phase behind group 0 ----
  if (group == 1) __syncthreads();
  for (int j = 0; j <= n_tiles; j += C::STAGES) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 <= n_tiles) step(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 <= n_tiles) step(j + 2, std::integral_constant<int, 2>{});
    if constexpr (C::STAGES >= 4)
      if (j + 3 <= n_tiles) step(j + 3, std::integral_constant<int, 3>{});
  }
  if (group == 0) __syncthreads();

  // ---- finalize ----
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (my_q < Nq) {
    char *orow = (char *)p.o + ((int64_t)bh * q_head + (int64_t)my_q * D) * 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = db * 32 + 8 * gq + half * 4;
        const uint32_t w0 = pack2<DT>(acc[db][gq * 4 + 0] * inv, acc[db][gq * 4 + 1] * inv);
        const uint32_t w1 = pack2<DT>(acc[db][gq * 4 + 2] * inv, acc[db][gq * 4 + 3] * inv);
        *(u32x2 *)(orow + d0 * 2) = u32x2{w0, w1};
      }
    if (p.lse && half == 0) {
      const float lse = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
      p.lse[(int64_t)bh * Nq + my_q] = lse;
    }
  }
}

}  // namespace fa
