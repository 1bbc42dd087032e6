// Two-group FlashAttention-2 forward for gfx950, 16-bit inputs, no mask other
// than the end of the keys.
//
// The arithmetic per key tile is that of fa_kernel.hpp (S^T = K Q^T on MFMA,
// online softmax with exp2 and a lazily moved exponent reference, O^T +=
// V^T P^T on MFMA; "A09 - Advanced Triton & FlashAttention", section 3, The
// kernel, in pseudocode). Only its placement in time differs. On gfx950 the
// MFMAs of one wave and the VALU work of another wave on the same SIMD
// overlap almost completely, while MFMAs and VALU work of one wave, or of two
// waves doing the same thing at the same time, largely take turns. So the
// 8 waves of a workgroup form two groups of 4 (waves w and w+4 share a SIMD),
// and every tile j of a wave has two phases:
//
//   matrix phase M(j):  S(j) = K_j Q^T, then PV(j-1) = V_{j-1}^T P_{j-1}^T;
//                       every LDS read and every tile transfer of the step
//   softmax phase X(j): row max, rebase, exponentials, row sums, packed P_j;
//                       VALU work only, on scores finished long before
//
// Both groups run M(0) X(0) M(1) X(1) ..., and one workgroup barrier per tile
// keeps them half a tile apart: group 0 reaches barrier j after X(j), group 1
// after M(j). So in period j (between barriers j-1 and j) group 0 runs M(j)
// X(j) while group 1 runs X(j-1) M(j): on every SIMD one wave issues MFMAs
// while the other runs the softmax.
//
// K and V tiles stream through two rings of four LDS stages by direct
// global->LDS loads, issued in softmax phases (a wave waiting on the address
// queue then holds up VALU work, not MFMAs): group 0 moves K_{j+3} at the
// start of X(j), in period j, into the stage of K_{j-1}; group 1 moves V_{j+2}
// at the end of X(j-1), in period j, into the stage of V_{j-2}. Both were last
// read in M(j-1), before barrier j-1. Before barrier j a group waits for the
// tile that period j+1 reads: K_{j+1} (group 0), V_j (group 1). Stages are
// compile-time constants (the loop is unrolled by four), so every LDS address
// is a register plus an immediate.
#pragma once

#include "fa_kernel.hpp"

#include <type_traits>

namespace fa {

template <int D>
struct PPCfg {
  static constexpr int WAVES = 8;
  static constexpr int BM = WAVES * 32;                 // query rows per workgroup
  static constexpr int BN = 64;                         // keys per tile
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;     // one K or V tile
  static constexpr int STAGES = 4;
  static constexpr int V_BASE = STAGES * TILE_BYTES;    // K stages, then V stages
  static constexpr int LDS_BYTES = 2 * STAGES * TILE_BYTES;
  static constexpr int LOADS = TILE_BYTES / (4 * 64 * 16);   // per thread of the moving group
  static_assert(TILE_BYTES % (4 * 64 * 16) == 0, "a tile splits into 16-byte lane loads");
  static_assert(STAGES * TILE_BYTES <= 65536, "immediate LDS offsets");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
};

template <int N>
__device__ __forceinline__ void pp_wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int DT, int D>
__global__ void __launch_bounds__(512, 2) fa_fwd_pp_kernel(Params p) {
  static_assert(DT == DT_BF16 || DT == DT_FP16, "16-bit inputs only");
  static_assert(D == 64 || D == 128, "head dim");
  using C = PPCfg<D>;
  constexpr int BN = C::BN, BM = C::BM, RB = C::ROW_BYTES, LOADS = C::LOADS;
  constexpr int NKC = D / 16;       // MFMAs along the head dim for S^T (per key block)
  constexpr int NDB = D / 32;       // 32-wide head-dim blocks of O^T
  constexpr int NPC = BN / 16;      // 16-key chunks of P^T

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int w4 = wave & 3;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if (p.xcd_remap && (nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int bh = bid / p.nq_tiles;
  const int qt = bid - bh * p.nq_tiles;
  const int64_t Nq = p.nq;
  const int my_q = qt * BM + wave * 32 + l32;

  const int64_t q_head = Nq * (int64_t)D;
  const int64_t k_head = p.nk * (int64_t)D;
  const char *qh = (const char *)p.q + (int64_t)bh * q_head * 2;
  const char *kh = (const char *)p.k + (int64_t)bh * k_head * 2;
  const char *vh = (const char *)p.v + (int64_t)bh * k_head * 2;
  const int n_kv = (int)p.n_kv;
  const int n = n_kv > 0 ? (n_kv + BN - 1) / BN : 0;     // key tiles

  // ---- Q fragments (B operand of S^T = K Q^T), straight from global ----
  // Requested here and waited for only after the first tile transfers have
  // been issued, so that the two memory round trips overlap. The loads are
  // inline asm, like the transfers, so that the compiler counts neither and
  // the explicit waits below are the only ones; rows at or past Nq lie
  // beyond the buffer's range and read as zeros.
  uint32_t qf[NKC][4];
  {
    const i32x4 qr = make_rsrc_words(qh, (uint32_t)(q_head * 2));
    i32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(qr[i]);
    const uint32_t row_off = (uint32_t)my_q * RB;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const uint32_t off = row_off + (uint32_t)((kc * 16 + half * 8) * 2);
      u32x4 x;
      asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(x) : "v"(off), "s"(r) : "memory");
#pragma unroll
      for (int w = 0; w < 4; ++w) qf[kc][w] = x[w];
    }
  }

  // ---- tile transfers: group 0 moves the K tiles, group 1 the V tiles ----
  // The LDS side is linear per wave; the global side reads the chunk that
  // the row swizzle puts there. Rows past n_kv read as zeros.
  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);
  uint32_t dma_off[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const int lds_off = (w4 * LOADS + u) * 1024 + lane * 16;
    const int row = lds_off / RB;
    dma_off[u] = (uint32_t)row * RB + (((lds_off % RB) / 16) ^ swz<RB>(row)) * 16;
  }
  const char *my_src = group == 0 ? kh : vh;
  const uint32_t my_lds = smem_base + (group == 0 ? 0u : (uint32_t)C::V_BASE) + (uint32_t)(w4 * LOADS * 1024);
  // instruction u of this group's transfer of tile t into stage st
  auto issue_part = [&](int t, int st, int u) __attribute__((always_inline)) {
    const int kstart = t * BN;
    const i32x4 r = make_rsrc_words(my_src + (int64_t)kstart * RB, (uint32_t)(n_kv - kstart) * RB);
    lds_dma16(r, dma_off[u], my_lds + (uint32_t)(st * C::TILE_BYTES + u * 1024));
  };
  auto issue_tile = [&](int t, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) issue_part(t, st, u);
  };

  // ---- lane offsets of the operand fragments in stage 0 ----
  uint32_t k_off[NKC], v_off[2][NDB];
  const FA_LDS char *k_ptr[NKC];
  const FA_LDS char *v_ptr[2][NDB];
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
        v_off[jg][db] = C::V_BASE + key * RB + ((((col * 2) / 16) ^ swz<RB>(key)) * 16) + (col * 2) % 16;
      }
    // LDS pointers formed once here. The empty asm hides the sum from the
    // compiler, which would otherwise add the (zero) base of the dynamic LDS
    // to each offset again inside the loop: eight adds per tile.
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      uint32_t a = smem_base + k_off[kc];
      asm volatile("" : "+v"(a));
      k_ptr[kc] = (const FA_LDS char *)(uintptr_t)a;
    }
#pragma unroll
    for (int jg = 0; jg < 2; ++jg)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        uint32_t a = smem_base + v_off[jg][db];
        asm volatile("" : "+v"(a));
        v_ptr[jg][db] = (const FA_LDS char *)(uintptr_t)a;
      }
  }

  auto mfma16 = [](u32x4 a, u32x4 b, f32x16 cin) __attribute__((always_inline)) -> f32x16 {
    if constexpr (DT == DT_BF16)
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), cin, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), cin, 0, 0, 0);
  };
  // An empty asm that claims to rewrite x: x is produced here, so the code
  // that computes it stays in this phase (the compiler would otherwise sink
  // the softmax past the barrier, next to the MFMAs that read P).
  auto pin = [](uint32_t &x) __attribute__((always_inline)) { asm volatile("" : "+v"(x)); };

  // ---- running state ----
  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;     // exponent reference (base-2 units), same in both halves
  float l_run = 0.f;           // this lane's partial row sum
  // derived from m_run, updated only where it moves: the threshold past which
  // a score moves the reference, and the exponent offset (0 for a row that
  // has seen no visible key, whose scores are all -inf: p = 0)
  float thr = -INFINITY;
  float neg = 0.f;
  const float c = p.c;
  f32x16 s[2];                 // S^T of the current tile: two 32-key blocks
  u32x4 pf[NPC];               // P^T of the last softmaxed tile, packed to 16 bits
#pragma unroll
  for (int i = 0; i < NPC; ++i) pf[i] = u32x4{0, 0, 0, 0};

  constexpr int KW = 3;                              // K chunks in flight in S

  // ---- matrix phase M(j): S(j) from K stage kst, then PV(j-1) from V
  // stage vst. K fragments stream KW chunks ahead of their MFMAs; the V^T
  // fragments of the first two 16-key chunks are requested during the second
  // half of S, the others two chunks ahead of their MFMAs. (At j = 0 the V
  // stage holds no tile yet; its reads are made but never used.) ----
  auto matrix = [&](int j, auto kst_c, auto vst_c) __attribute__((always_inline)) {
    constexpr int kst = decltype(kst_c)::value, vst = decltype(vst_c)::value;
    u32x4 vf[NPC][NDB];
    // transposing read r of chunk pc: head-dim block r / 2, half r % 2
    auto read_v1 = [&](int pc, int r) __attribute__((always_inline)) {
      const int db = r / 2, jg = r % 2;
      const FA_LDS char *addr = v_ptr[jg][db] + vst * C::TILE_BYTES + pc * 16 * RB;
      const u32x2 xx = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4 *)addr));
      vf[pc][db][jg * 2] = xx[0];
      vf[pc][db][jg * 2 + 1] = xx[1];
    };
    auto read_v = [&](int pc) __attribute__((always_inline)) {
#pragma unroll
      for (int r = 0; r < 2 * NDB; ++r) read_v1(pc, r);
    };
    __builtin_amdgcn_s_setprio(1);
    if (j < n) {
      constexpr int VR = 4 * NDB / (NKC / 2);        // V reads per S chunk, second half
      static_assert(VR * (NKC / 2) == 4 * NDB, "even spread of the V reads");
      u32x4 kf[NKC][2];
      auto read_k = [&](int kc) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) kf[kc][kb] = *(const FA_LDS u32x4 *)(k_ptr[kc] + kst * C::TILE_BYTES + kb * 32 * RB);
      };
#pragma unroll
      for (int kc = 0; kc < KW; ++kc) read_k(kc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const u32x4 b = {qf[kc][0], qf[kc][1], qf[kc][2], qf[kc][3]};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = mfma16(kf[kc][kb], b, kc == 0 ? f32x16{} : s[kb]);
        if (kc + KW < NKC) read_k(kc + KW);
        if (kc >= NKC / 2) {
#pragma unroll
          for (int q = 0; q < VR; ++q) {
            const int r = (kc - NKC / 2) * VR + q;     // 0 .. 4*NDB-1 over chunks 0, 1
            read_v1(r / (2 * NDB), r % (2 * NDB));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      read_v(0);
      read_v(1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (j >= 1) {
#pragma unroll
      for (int pc = 0; pc < NPC; ++pc) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = mfma16(vf[pc][db], pf[pc], acc[db]);
        if (pc + 2 < NPC) read_v(pc + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- softmax phase X(j): P_j from S_j (VALU only) ----
  auto softmax = [&](int j) __attribute__((always_inline)) {
    if (j < 0 || j >= n) return;
    const int kstart = j * BN;
    if (kstart + BN > n_kv) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kstart + kb * 32 + 8 * (i / 4) + half * 4 + (i % 4);
          if (key >= n_kv) s[kb][i] = -INFINITY;
        }
    }
    float lm = score_max(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = (kb == 0 ? 2 : 0); i < 16; ++i) lm = score_max(lm, s[kb][i]);
    // The reference moves only when a row max exceeds it by more than the
    // slack; acc and l are rescaled together ("A09", section 3, the
    // rebasing). A row max (scaled by c > 0, which keeps order) exceeds the
    // threshold exactly when the maximum of one of its two lanes does, so the
    // row max over both lanes is formed only when some row moves.
    if (__builtin_amdgcn_ballot_w64(lm * c > thr) != 0) {
      const float mx = halves_max(lm) * c;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      thr = m_new + kRescaleSlack;
      neg = (m_new == -INFINITY) ? 0.f : -m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
    float rs[4];
    // per 32-key block: exponentials, row-sum terms, then its packed P^T
    // chunks (chunk pc = keys pc*16 + 8*(w/2) + half*4 + ...: values
    // (pc%2)*8 .. +7 of block pc/2)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, neg));
        s[kb][i] = e;
        if (kb == 0 && i < 4) rs[i] = e;
        else rs[i % 4] += e;
      }
#pragma unroll
      for (int pc = 2 * kb; pc < 2 * kb + 2; ++pc)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t x = pack2<DT>(s[pc / 2][(pc % 2) * 8 + 2 * w], s[pc / 2][(pc % 2) * 8 + 2 * w + 1]);
          pin(x);
          pf[pc][w] = x;
        }
    }
    l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };

  // ---- end of period j: this group's transfer that period j+1 reads is
  // complete (K_{j+1} for group 0, V_j for group 1); later ones, up to
  // K_{j+3} and V_{j+2}, may still fly; then the barrier ----
  auto end_period = [&](int j) __attribute__((always_inline)) {
    const int need = group == 0 ? j + 1 : j;
    const int last = min(n - 1, group == 0 ? j + 3 : j + 2);
    const int later = max(0, last - max(need, 0));
    if (later >= 2) pp_wait_vmcnt<2 * LOADS>();
    else if (later == 1) pp_wait_vmcnt<LOADS>();
    else pp_wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: K_0 .. K_2 (group 0), V_0 .. V_2 (group 1) after the Q
  // loads; then Q complete in every wave and K_0 in LDS ----
#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (t < n) issue_tile(t, t);
  if (group == 0) {
    // K_0 (and Q before it) complete; K_1, K_2 may fly
    if (n >= 3) pp_wait_vmcnt<2 * LOADS>();
    else if (n == 2) pp_wait_vmcnt<LOADS>();
    else pp_wait_vmcnt<0>();
  } else {
    // Q complete; V_0 .. V_2 may fly
    if (n >= 3) pp_wait_vmcnt<3 * LOADS>();
    else if (n == 2) pp_wait_vmcnt<2 * LOADS>();
    else if (n == 1) pp_wait_vmcnt<LOADS>();
    else pp_wait_vmcnt<0>();
  }
  __syncthreads();

  // ---- periods j = 0 .. n; K_j sits in K stage j % 4, V_j in V stage j % 4 ----
  // Both groups run the same sequence M(j) X(j); only where the barrier sits
  // differs (one code path keeps the register allocation of a single group).
  auto period = [&](int j, auto st_c) __attribute__((always_inline)) {
    constexpr int st = decltype(st_c)::value;
    using KS = std::integral_constant<int, st>;
    using VS = std::integral_constant<int, (st + 3) % 4>;
    matrix(j, KS{}, VS{});
    if (group == 1) end_period(j);
    __builtin_amdgcn_sched_barrier(0);
    // Tile j+3 of this group's matrix is moved during its softmax phase:
    // K_{j+3} by group 0 at the start of X(j), while group 1 runs its softmax;
    // V_{j+3} by group 1 at the end of X(j), while group 0 issues the last
    // MFMAs of M(j+1), whose LDS reads are done. The transfers then meet few
    // LDS reads of the other group.
    if (group == 0 && j + 3 < n) issue_tile(j + 3, (st + 3) % 4);
    __builtin_amdgcn_sched_barrier(0);
    softmax(j);
    __builtin_amdgcn_sched_barrier(0);
    if (group == 1 && j + 3 < n) issue_tile(j + 3, (st + 3) % 4);

    if (group == 0) end_period(j);
  };
  static_assert(C::STAGES == 4, "the loop is unrolled by the stage count");
  for (int j = 0; j <= n; j += 4) {
    period(j, std::integral_constant<int, 0>{});
    if (j + 1 <= n) period(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 <= n) period(j + 2, std::integral_constant<int, 2>{});
    if (j + 3 <= n) period(j + 3, std::integral_constant<int, 3>{});
  }

  // ---- finalize: O = acc / l, LSE = (m + log2 l) ln 2 ----
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
