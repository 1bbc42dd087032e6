// Intra-wave pipelined schedule of the FlashAttention-2 forward for gfx950,
// 16-bit inputs.
//
// Same arithmetic as fa_kernel.hpp (S^T = K Q^T and O^T += V^T P^T on MFMA,
// online softmax with exp2 and a shared exponent reference; "A09 - Advanced
// Triton & FlashAttention", section 3; "Triton: FlashAttention-2 Forward
// Pass"; "Building a Verifiable FlashAttention Forward from PyTorch to
// Triton", Part 3), scheduled so that one wave keeps the matrix core and the
// vector ALU busy at the same time. A workgroup has 4 waves (one per SIMD,
// 512 registers each) and 128 query rows. Iteration j of a wave runs
//
//   a stream of MFMA "slots": PV(j-1) then QK(j+1)   (matrix core)
//   the softmax of tile j, cut into short chunks    (vector ALU)
//
// with one softmax chunk and the LDS reads of a later slot placed between
// consecutive MFMAs, so the vector work and the LDS latency hide under the
// MFMAs. The two products never depend on the softmax of the same
// iteration: S_{j+1} and P_j live in a second register buffer (the loop is
// unrolled by two to swap them). The accumulator rescale, when the exponent
// reference moves, waits for PV(j-1) and is applied after the stream.
//
// Tiles outside the valid range, or in a wave's causal future, are still
// multiplied: their keys are masked to -inf, so P is 0 and PV adds zeros.
// K_{j+1} and V_{j-1} form the LDS stage of iteration j; stages stream
// through a ring of three buffers, two iterations ahead.
#pragma once

#include "fa_kernel.hpp"

namespace fa {

template <int DT, int D, bool CAUSAL>
struct IWCfg {
  static constexpr int WAVES = 4;
  static constexpr int BM = WAVES * 32;
  static constexpr int BN = 64;
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  static constexpr int STAGES = 3;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;       // K_{s+1}, then V_{s-1}
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int LOADS = TILE_BYTES / (WAVES * 64 * 16);   // per thread per matrix
  static_assert(TILE_BYTES % (WAVES * 64 * 16) == 0, "tile must split into 16-byte lane loads");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int DT, int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1) fa_fwd_interleaved_kernel(Params p) {
  static_assert(DT == DT_BF16 || DT == DT_FP16, "16-bit inputs only");
  using C = IWCfg<DT, D, CAUSAL>;
  constexpr int BN = C::BN, BM = C::BM, RB = C::ROW_BYTES;
  constexpr int NKC = D / 16, NKB = BN / 32, NDB = D / 32, NPC = BN / 16;
  constexpr int NPV = NPC * NDB;            // PV slots
  constexpr int NQK = NKC * NKB;            // QK slots
  constexpr int NS = NPV + NQK;             // MFMA slots per iteration
  constexpr int NV = NKB * 16;              // scores per lane per tile
  constexpr int kAhead = 6;                 // LDS reads run this many slots ahead
  constexpr int PER_STAGE = 2 * C::LOADS;   // LDS-direct loads per thread per stage

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if (p.xcd_remap && (nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  const int bh = bid / p.nq_tiles;
  int qt = bid - bh * p.nq_tiles;
  if (CAUSAL) qt = p.nq_tiles - 1 - qt;
  const int64_t N = p.N;
  const int q0 = qt * BM;
  const int qw = q0 + wave * 32;
  const int my_q = qw + l32;

  const int64_t head_elems = N * (int64_t)D;
  const char *qh = (const char *)p.q + (int64_t)bh * head_elems * 2;
  const char *kh = (const char *)p.k + (int64_t)bh * head_elems * 2;
  const char *vh = (const char *)p.v + (int64_t)bh * head_elems * 2;
  const int n_kv = (int)p.n_kv;
  int kend = n_kv;
  if (CAUSAL) kend = min(kend, q0 + BM);
  const int n_tiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  // ---- Q fragments ----
  uint32_t qf[NKC][4];
  {
    const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(qh, (uint32_t)(head_elems * 2));
    const uint32_t row_off = (uint32_t)my_q * RB;
    const bool row_ok = my_q < N;
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

  // ---- stages: stage s holds K_{s+1} and V_{s-1}, in ring buffer (s+1) % 3 ----
  const i32x4 k_rsrc = make_rsrc_words(kh, (uint32_t)((int64_t)n_kv * D * 2));
  const i32x4 v_rsrc = make_rsrc_words(vh, (uint32_t)((int64_t)n_kv * D * 2));
  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);
  auto stage_offset = [&](int s) __attribute__((always_inline)) { return (uint32_t)(((s + 1) % C::STAGES) * C::STAGE_BYTES); };
  auto issue_stage = [&](int s) __attribute__((always_inline)) {
    const uint32_t kl = smem_base + stage_offset(s);
    const uint32_t vl = kl + C::TILE_BYTES;
    const int kt = s + 1, vt = s - 1;
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const int inst = wave * C::LOADS + u;
      const int lds_off = inst * 1024 + lane * 16;
      const int row = lds_off / RB;
      const int lchunk = ((lds_off % RB) / 16) ^ swz<RB>(row);
      // tiles outside [0, n_tiles) read beyond the resource: zeros
      const uint32_t koff = (kt >= 0 && kt < n_tiles) ? (uint32_t)(kt * BN + row) * RB + lchunk * 16 : 0xFFFFFF00u;
      const uint32_t voff = (vt >= 0 && vt < n_tiles) ? (uint32_t)(vt * BN + row) * RB + lchunk * 16 : 0xFFFFFF00u;
      lds_dma16(k_rsrc, koff, kl + inst * 1024);
      lds_dma16(v_rsrc, voff, vl + inst * 1024);
    }
  };

  // ---- lane offsets of the MFMA operand fragments inside a tile ----
  uint32_t voff[2][NDB], koff[NKC];
  {
    const int tr_g = lane >> 4, tr_r = (lane & 15) >> 2, tr_cq = lane & 3;
#pragma unroll
    for (int jg = 0; jg < 2; ++jg)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = db * 32 + (tr_g & 1) * 16 + tr_cq * 4;
        const int key = jg * 8 + (tr_g >> 1) * 4 + tr_r;
        const int ch = ((col * 2) / 16) ^ swz<RB>(key);
        voff[jg][db] = key * RB + ch * 16 + (col * 2) % 16;
      }
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) koff[kc] = l32 * RB + (((kc * 2 + half) ^ swz<RB>(l32)) * 16);
  }
  // fragment of slot i: V^T (pc, db) for i < NPV, else K (kc, kb)
  auto frag = [&](uint32_t st, int slot) __attribute__((always_inline)) -> u32x4 {
    const char *kl = smem + st;
    const char *vl = kl + C::TILE_BYTES;
    if (slot < NPV) {
      const int pc = slot / NDB, db = slot % NDB;
      u32x4 a;
#pragma unroll
      for (int jg = 0; jg < 2; ++jg) {
        const char *addr = vl + voff[jg][db] + pc * 16 * RB;
        const u32x2 xx = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4 *)addr));
        a[jg * 2] = xx[0];
        a[jg * 2 + 1] = xx[1];
      }
      return a;
    }
    const int kc = (slot - NPV) / NKB, kb = (slot - NPV) % NKB;
    return *(const FA_LDS u32x4 *)(kl + koff[kc] + kb * 32 * RB);
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  f32x16 sA[NKB], sB[NKB];
  u32x4 pA[NPC], pB[NPC];
#pragma unroll
  for (int i = 0; i < NKB; ++i) { sA[i] = f32x16{}; sB[i] = f32x16{}; }
#pragma unroll
  for (int i = 0; i < NPC; ++i) { pA[i] = u32x4{0, 0, 0, 0}; pB[i] = u32x4{0, 0, 0, 0}; }
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float c = p.c;

  auto mfma16 = [&](u32x4 a, u32x4 b, f32x16 cin) __attribute__((always_inline)) -> f32x16 {
    if constexpr (DT == DT_BF16)
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), cin, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), cin, 0, 0, 0);
  };

  // QK of one tile as a plain pipelined stream (prologue)
  auto qk_only = [&](uint32_t st, f32x16 (&s)[NKB]) __attribute__((always_inline)) {
    u32x4 buf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) buf[i] = frag(st, NPV + i);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 a = buf[i % kAhead];
      if (i + kAhead < NQK) buf[i % kAhead] = frag(st, NPV + i + kAhead);
      const int kc = i / NKB, kb = i % NKB;
      const u32x4 b = {qf[kc][0], qf[kc][1], qf[kc][2], qf[kc][3]};
      s[kb] = mfma16(a, b, kc == 0 ? f32x16{} : s[kb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // PV of one tile as a plain pipelined stream (epilogue)
  auto pv_only = [&](uint32_t st, const u32x4 (&pp)[NPC]) __attribute__((always_inline)) {
    u32x4 buf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) buf[i] = frag(st, i);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 a = buf[i % kAhead];
      if (i + kAhead < NPV) buf[i % kAhead] = frag(st, i + kAhead);
      acc[i % NDB] = mfma16(a, pp[i / NDB], acc[i % NDB]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // masks of tile t on its scores (only tiles past the keys or on the diagonal)
  auto mask_tile = [&](int t, f32x16 (&s)[NKB]) __attribute__((always_inline)) {
    const int kstart = t * BN;
    if ((kstart + BN > n_kv) || (CAUSAL && kstart + BN - 1 > qw)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kstart + kb * 32 + 8 * (i / 4) + half * 4 + (i % 4);
          if ((key >= n_kv) || (CAUSAL && key > my_q)) s[kb][i] = -INFINITY;
        }
    }
  };

  // ---- one iteration: softmax(j) on sc -> pc_out, MFMAs PV(j-1) with pp and QK(j+1) into sn ----
  // Softmax work is cut into units spread evenly over the NS slots:
  //   [0, NV/2)           running max, two scores per unit (two chains)
  //   NV/2                new reference, rescale decision
  //   NV/2+1 ... +NV      exp2 and row sum, one score per unit
  //   then NPC*4 units    pack two probabilities into one 16-bit pair
  constexpr int U_MAX0 = 0, U_DEC = NV / 2, U_EXP0 = U_DEC + 1, U_PACK0 = U_EXP0 + NV;
  constexpr int U_TOTAL = U_PACK0 + NPC * 4;
  auto iteration = [&](int j, f32x16 (&sc)[NKB], f32x16 (&sn)[NKB], const u32x4 (&pp)[NPC],
                       u32x4 (&po)[NPC]) __attribute__((always_inline)) {
    const uint32_t st = stage_offset(j);
    mask_tile(j, sc);
    float mx0 = -INFINITY, mx1 = -INFINITY, rs0 = 0.f, rs1 = 0.f, neg = 0.f, alpha = 1.f;
    bool rescale = false;
    auto unit = [&](int u) __attribute__((always_inline)) {
      if (u < U_DEC) {
        const int e = 2 * u;
        const float x0 = sc[e / 16][e % 16], x1 = sc[(e + 1) / 16][(e + 1) % 16];
        if (u & 1) mx1 = fmaxf(mx1, fmaxf(x0, x1));
        else mx0 = fmaxf(mx0, fmaxf(x0, x1));
      } else if (u == U_DEC) {
        const float mx = halves_max(fmaxf(mx0, mx1)) * c;
        rescale = __builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0;
        if (rescale) {
          const float m_new = fmaxf(m_run, mx);
          alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
        }
        neg = (m_run == -INFINITY) ? 0.f : -m_run;
      } else if (u < U_PACK0) {
        const int e = u - U_EXP0;
        const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e / 16][e % 16], c, neg));
        sc[e / 16][e % 16] = x;
        if (e & 1) rs1 += x;
        else rs0 += x;
      } else if (u < U_TOTAL) {
        const int k = u - U_PACK0;
        const int pc = k / 4, w = k % 4, kb = pc / 2, i0 = (pc % 2) * 8 + 2 * w;
        po[pc][w] = pack2<DT>(sc[kb][i0], sc[kb][i0 + 1]);
      }
    };
    u32x4 buf[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) buf[i] = frag(st, i);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 a = buf[i % kAhead];
      if (i + kAhead < NS) buf[i % kAhead] = frag(st, i + kAhead);
      if (i < NPV) {
        acc[i % NDB] = mfma16(a, pp[i / NDB], acc[i % NDB]);
      } else {
        const int kc = (i - NPV) / NKB, kb = (i - NPV) % NKB;
        const u32x4 b = {qf[kc][0], qf[kc][1], qf[kc][2], qf[kc][3]};
        sn[kb] = mfma16(a, b, kc == 0 ? f32x16{} : sn[kb]);
      }
#pragma unroll
      for (int u = (i * U_TOTAL) / NS; u < ((i + 1) * U_TOTAL) / NS; ++u) unit(u);
    }
    __builtin_amdgcn_sched_barrier(0);
    l_run += rs0 + rs1;
    if (rescale) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
  };

  // ---- prologue: stages -1, 0, 1 in flight; S_0 = QK(0) from stage -1 ----
  issue_stage(-1);
  issue_stage(0);
  issue_stage(1);
  wait_vmcnt<2 * PER_STAGE>();
  __syncthreads();
  qk_only(stage_offset(-1), sA);
  wait_vmcnt<PER_STAGE>();
  __syncthreads();

  // ---- main loop, unrolled by two to swap the score / probability buffers ----
  int j = 0;
  for (; j + 1 < n_tiles; j += 2) {
    issue_stage(j + 2);
    iteration(j, sA, sB, pB, pA);
    wait_vmcnt<PER_STAGE>();
    __syncthreads();
    issue_stage(j + 3);
    iteration(j + 1, sB, sA, pA, pB);
    wait_vmcnt<PER_STAGE>();
    __syncthreads();
  }
  if (j < n_tiles) {
    // odd tile count: last softmax reads sA, its P goes to pA; PV(n-2) used pB
    issue_stage(j + 2);
    iteration(j, sA, sB, pB, pA);
    wait_vmcnt<PER_STAGE>();
    __syncthreads();
    pv_only(stage_offset(n_tiles), pA);
  } else if (n_tiles > 0) {
    pv_only(stage_offset(n_tiles), pB);
  }
  wait_vmcnt<0>();

  // ---- finalize ----
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (my_q < N) {
    char *orow = (char *)p.o + ((int64_t)bh * head_elems + (int64_t)my_q * D) * 2;
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
      p.lse[(int64_t)bh * N + my_q] = lse;
    }
  }
}

}  // namespace fa
