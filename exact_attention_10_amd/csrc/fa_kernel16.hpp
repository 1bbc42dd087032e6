// FlashAttention-2 forward on 16x16x32 MFMAs (gfx950), 16-bit inputs, with or
// without the causal mask: the schedule of fa_kernel.hpp (per key tile: wait
// for the tile and a barrier, S^T = K Q^T, the next tile's transfer, the V^T
// fragments, masks, online softmax, O^T += V^T P^T; K and V double-buffered
// in LDS; causal workgroups take query tiles longest first or in pairs
// T-1-i, i) with the operand layouts of fa_kernel_pp16.hpp: a wave's 32
// queries are two 16-query blocks, a lane holds 16 scores of each of its two
// queries, and a query's row statistics span four lanes. At the board's
// power limit the 16x16x32 form does more work per joule than 32x32x16.
//
// The arithmetic per score is that of fa_kernel.hpp ("A09 - Advanced Triton &
// FlashAttention", section 3, The kernel, in pseudocode; causal tile
// skipping and the masked diagonal as in its section 3).
#pragma once

#include "fa_kernel_pp16.hpp"

namespace fa {

template <int DT, int D, bool CAUSAL, int WAVES>
__global__ void __launch_bounds__(WAVES * 64, 2) fa_fwd16_kernel(Params p) {
  static_assert(DT == DT_BF16 || DT == DT_FP16, "16-bit inputs only");
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(WAVES == 4 || WAVES == 8, "4 or 8 waves");
  using C = Cfg<DT, D, CAUSAL, WAVES>;       // LDS: K and V tiles, two buffers
  constexpr int BN = C::BN, BM = C::BM, RB = C::ROW_BYTES;
  constexpr int NKC = D / 32;       // 32-wide head-dim chunks of S^T = K Q^T
  constexpr int NMB = BN / 16;      // 16-key blocks of S^T
  constexpr int NDB = D / 16;       // 16-wide head-dim blocks of O^T
  constexpr int NPC = BN / 32;      // 32-key chunks of P^T
  constexpr int NKF = NKC * NMB;    // K fragments per tile
  constexpr int KW = NKF < 6 ? NKF : 6;   // K fragments requested ahead of their MFMAs

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i16 = lane & 15;
  const int g = lane >> 4;

  // ---- which (head, query tile) this workgroup owns (fa_kernel.hpp) ----
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if (p.xcd_remap && (nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  int bh = bid / p.nq_tiles;
  int qt = bid - bh * p.nq_tiles;
  if (CAUSAL) qt = p.nq_tiles - 1 - qt;     // longest causal tiles first
  int second_qt = -1;
  if (CAUSAL && p.pair) {
    const int T = p.nq_tiles;
    const int npairs = (T + 1) / 2;
    int c = blockIdx.x;
    if (p.xcd_remap && (nblk & 7) == 0) c = (c & 7) * (nblk >> 3) + (c >> 3);
    bh = c / npairs;
    const int pr = c - bh * npairs;
    qt = T - 1 - pr;
    second_qt = (pr != T - 1 - pr) ? pr : -1;
  }
  const int64_t Nq = p.nq;
  const int coff = (int)p.coff;            // causal diagonal: key j visible when j <= i + coff
  const int64_t q_head = Nq * (int64_t)D;
  const int64_t k_head = p.nk * (int64_t)D;
  const char *qh = (const char *)p.q + (int64_t)bh * q_head * 2;
  const char *kh = (const char *)p.k + (int64_t)bh * k_head * 2;
  const char *vh = (const char *)p.v + (int64_t)bh * k_head * 2;
  const int n_kv = (int)p.n_kv;
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(qh, (uint32_t)(q_head * 2));

  // ---- K/V tile transfers, as in fa_kernel.hpp ----
  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);
  uint32_t dma_off[C::LOADS_PER_THREAD];
#pragma unroll
  for (int u = 0; u < C::LOADS_PER_THREAD; ++u) {
    const int lds_off = (wave * C::LOADS_PER_THREAD + u) * 1024 + lane * 16;
    const int row = lds_off / RB;
    dma_off[u] = (uint32_t)row * RB + (((lds_off % RB) / 16) ^ swz<RB>(row)) * 16;
  }
  auto issue_tile = [&](int t, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const int kstart = t * BN;
    const uint32_t valid = (uint32_t)(n_kv - kstart) * RB;      // kstart < n_kv here
    const i32x4 kr = make_rsrc_words(kh + (int64_t)kstart * RB, valid);
    const i32x4 vr = make_rsrc_words(vh + (int64_t)kstart * RB, valid);
#pragma unroll
    for (int u = 0; u < C::LOADS_PER_THREAD; ++u) {
      const uint32_t lds = smem_base + buf * (2 * C::TILE_BYTES) + (wave * C::LOADS_PER_THREAD + u) * 1024;
      lds_dma16(kr, dma_off[u], lds);
      lds_dma16(vr, dma_off[u], lds + C::TILE_BYTES);
    }
  };

  // ---- LDS addresses of the operand fragments in buffer 0 (fa_kernel_pp16.hpp):
  // K fragment (kc, mb) at k_ptr[kc] + 16 mb rows, V^T fragment (pc, db) by two
  // transposing reads at v_ptr[db] + 32 pc rows and + 16 rows more ----
  const FA_LDS char *k_ptr[NKC];
  const FA_LDS char *v_ptr[NDB];
  {
    const int r = i16 >> 2, cq = i16 & 3;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      uint32_t a = smem_base + (uint32_t)(i16 * RB + (((kc * 4 + g) ^ swz<RB>(i16)) * 16));
      asm volatile("" : "+v"(a));
      k_ptr[kc] = (const FA_LDS char *)(uintptr_t)a;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int key = 4 * g + r;
      const int col = db * 16 + cq * 4;
      uint32_t a = smem_base + (uint32_t)(C::TILE_BYTES + key * RB + ((((col * 2) / 16) ^ swz<RB>(key)) * 16) + (col * 2) % 16);
      asm volatile("" : "+v"(a));
      v_ptr[db] = (const FA_LDS char *)(uintptr_t)a;
    }
  }

  auto mfma = [](u32x4 a, u32x4 b, f32x4 cin) __attribute__((always_inline)) -> f32x4 {
    if constexpr (DT == DT_BF16)
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), cin, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), cin, 0, 0, 0);
  };

  for (int job = 0; job < 2; ++job) {
  if (job == 1) {
    if (second_qt < 0) break;
    qt = second_qt;
    __syncthreads();                       // every wave is done with the first tile's LDS
  }
  const int q0 = qt * BM;
  const int qw = q0 + wave * 32;           // first query row of this wave
  int kend = n_kv;
  if (CAUSAL) kend = min(kend, q0 + BM + coff);
  const int t_end = kend > 0 ? (kend + BN - 1) / BN : 0;

  // ---- Q fragments (B operand of S^T): query block nb, head-dim chunk kc:
  // row qw + 16 nb + i16, head dims 32 kc + 8 g .. +7; rows at or past Nq
  // lie beyond the buffer's range and read as zeros ----
  uint32_t qf[2][NKC][4];
  const int qln = fresh_lane_id();
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const uint32_t off = (uint32_t)(qw + nb * 16 + (qln & 15)) * RB + (uint32_t)((kc * 32 + (qln >> 4) * 8) * 2);
      const u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off, 0, 0));
#pragma unroll
      for (int w = 0; w < 4; ++w) qf[nb][kc][w] = x[w];
    }
  // Q is needed in every iteration: complete its loads here, so that no wait
  // for them is left inside the loop (where it would also wait for prefetches)
  wait_vmem();

  // ---- running state, per query block nb (fa_kernel_pp16.hpp) ----
  f32x4 acc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db][0] = acc[db][1] = f32x4{};
  float m_run[2] = {-INFINITY, -INFINITY};   // exponent reference (base 2), same in the query's four lanes
  float l_run[2] = {0.f, 0.f};               // this lane's partial row sums
  float thr[2] = {-INFINITY, -INFINITY};     // m_run + slack, updated where m_run moves
  float neg[2] = {0.f, 0.f};                 // -m_run, or 0 while a row has seen no visible key
  const float c = p.c;

  // one key tile; buf (0 or 1) is a compile-time constant so that every LDS
  // address is a register plus an immediate
  auto step = [&](int t, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    wait_vmem();
    __syncthreads();                        // tile t visible; the other buffer is free
    auto prefetch = [&]() __attribute__((always_inline)) {
      if (t + 1 < t_end) issue_tile(t + 1, std::integral_constant<int, buf ^ 1>{});
    };
    const int kstart = t * BN;

    // ---- S^T = K Q^T: K fragments stream KW ahead of their MFMAs ----
    f32x4 s[NMB][2];
    {
      u32x4 kf[NKF];
      auto read_k = [&](int f) __attribute__((always_inline)) {
        const int kc = f / NMB, mb = f % NMB;
        kf[f] = *(const FA_LDS u32x4 *)(k_ptr[kc] + buf * (2 * C::TILE_BYTES) + mb * 16 * RB);
      };
#pragma unroll
      for (int f = 0; f < KW; ++f) read_k(f);
#pragma unroll
      for (int f = 0; f < NKF; ++f) {
        if (f + KW < NKF) read_k(f + KW);
        __builtin_amdgcn_sched_barrier(0);
        const int kc = f / NMB, mb = f % NMB;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const u32x4 b = {qf[nb][kc][0], qf[nb][kc][1], qf[nb][kc][2], qf[nb][kc][3]};
          s[mb][nb] = mfma(kf[f], b, kc == 0 ? f32x4{} : s[mb][nb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // V^T fragments (pc, db): those of the first P^T chunk are read now, so
    // that they arrive while the softmax runs; each later one is read in
    // place of the fragment one chunk before it, while that chunk's products run
    u32x4 vf[NPC][NDB];
    auto read_v = [&](int pc, int db) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const FA_LDS char *addr = v_ptr[db] + buf * (2 * C::TILE_BYTES) + (pc * 32 + h * 16) * RB;
        const u32x2 xx = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4 *)addr));
        vf[pc][db][h * 2] = xx[0];
        vf[pc][db][h * 2 + 1] = xx[1];
      }
    };
#pragma unroll
    for (int db = 0; db < NDB; ++db) read_v(0, db);
    __builtin_amdgcn_sched_barrier(0);
    prefetch();

    // ---- masks: only on tiles past the end of the keys or on the diagonal ----
    if (kstart + BN > n_kv || (CAUSAL && kstart + BN - 1 > qw + coff)) {
      // score (mb, nb, i) holds key kstart + 4g + 16 mb + i of row
      // qw + 16 nb + i16: it is visible when 16 mb + i <= lim[nb]; one limit
      // per row and tile keeps every compare a register against an immediate.
      // (a reload from scratch here would wait for the tile transfer in flight)
      const int ln = fresh_lane_id();
      const int rel = kstart + ((ln >> 2) & ~3);
      int lim[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        lim[nb] = n_kv - 1 - rel;
        if (CAUSAL) lim[nb] = min(lim[nb], qw + coff + nb * 16 + (ln & 15) - rel);
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            if (mb * 16 + i > lim[nb]) s[mb][nb][i] = -INFINITY;
    }

    // ---- online softmax (fa_kernel_pp16.hpp): the rescale test on each
    // lane's own row maximum, the row max over four lanes only where a row
    // moves its reference ----
    float lm[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float m = score_max(s[0][nb][0], s[0][nb][1]);
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = (mb == 0 ? 2 : 0); i < 4; ++i) m = score_max(m, s[mb][nb][i]);
      lm[nb] = m;
    }
    if (__builtin_amdgcn_ballot_w64(lm[0] * c > thr[0] || lm[1] * c > thr[1]) != 0) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float mx = quad_max(lm[nb]) * c;
        const float m_new = score_max(m_run[nb], mx);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[nb] - m_new);
        m_run[nb] = m_new;
        thr[nb] = m_new + kRescaleSlack;
        neg[nb] = (m_new == -INFINITY) ? 0.f : -m_new;
        l_run[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[db][nb][i] *= alpha;
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      float rs[4];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mb][nb][i], c, neg[nb]));
          s[mb][nb][i] = e;
          if (mb == 0) rs[i] = e;
          else rs[i] += e;
        }
      l_run[nb] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    }

    // ---- O^T += V^T P^T, P^T packed chunk by chunk: the keys of S^T blocks
    // 2pc and 2pc+1 that this lane holds ----
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc) {
      u32x4 pf[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int mb = 2 * pc + w / 2, i = (w % 2) * 2;
          pf[nb][w] = pack2<DT>(s[mb][nb][i], s[mb][nb][i + 1]);
        }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[db][nb] = mfma(vf[pc][db], pf[nb], acc[db][nb]);
        if (pc + 1 < NPC) read_v(pc + 1, db);
      }
    }
  };

  // tiles past t_wave hold only keys in the future of every row of this wave:
  // there it only keeps the workgroup's barriers and transfers going
  const int t_wave = CAUSAL ? min(t_end, max(0, (qw + 31 + coff) / BN + 1)) : t_end;
  auto idle = [&](int t, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    wait_vmem();
    __syncthreads();
    if (t + 1 < t_end) issue_tile(t + 1, std::integral_constant<int, buf ^ 1>{});
  };
  if (0 < t_end) issue_tile(0, std::integral_constant<int, 0>{});
  int t = 0;
  for (; t + 1 < t_wave; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    step(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < t_wave) {
    step(t, std::integral_constant<int, 0>{});
    if (++t < t_end) idle(t++, std::integral_constant<int, 1>{});
  }
  for (; t < t_end; t += 2) {
    idle(t, std::integral_constant<int, 0>{});
    if (t + 1 < t_end) idle(t + 1, std::integral_constant<int, 1>{});
  }

  // ---- finalize: O = acc / l, LSE = (m + log2 l) ln 2 ----
  const int oln = fresh_lane_id();
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float l_tot = quad_sum(l_run[nb]);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const int64_t q = qw + nb * 16 + (oln & 15);
    if (q < Nq) {
      char *orow = (char *)p.o + ((int64_t)bh * q_head + q * D) * 2;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d0 = db * 16 + 4 * (oln >> 4);
        const uint32_t w0 = pack2<DT>(acc[db][nb][0] * inv, acc[db][nb][1] * inv);
        const uint32_t w1 = pack2<DT>(acc[db][nb][2] * inv, acc[db][nb][3] * inv);
        *(u32x2 *)(orow + d0 * 2) = u32x2{w0, w1};
      }
      if (p.lse && oln < 16) {
        const float lse = l_tot > 0.f ? (m_run[nb] + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
        p.lse[(int64_t)bh * Nq + q] = lse;
      }
    }
  }
  }   // job
}

}  // namespace fa
