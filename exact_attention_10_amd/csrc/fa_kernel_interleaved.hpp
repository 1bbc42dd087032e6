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
//   the softmax of tile j, cut into short units      (vector ALU)
//
// with the softmax units placed between consecutive MFMAs in proportion to
// their issue cost, and the LDS reads of each slot issued several slots
// ahead, so the vector work and the LDS latency hide under the MFMAs. The two
// products never depend on the softmax of the same iteration: S_{j+1} and P_j
// live in a second register buffer. The accumulator rescale, when the
// exponent reference moves, waits for PV(j-1) and is applied after the stream.
//
// Tiles outside the valid range, or in a wave's causal future, are still
// multiplied: their keys are masked to -inf, so P is 0 and PV adds zeros.
// This includes up to three tiles past the end, which round the tile count up
// to the unroll factor of the main loop.
// K_{j+1} and V_{j-1} form the LDS stage of iteration j; stages stream
// through a ring of four buffers, three iterations ahead. The main loop is
// unrolled by four so that every buffer index, and with it every LDS address
// offset, is a compile-time constant.
#pragma once

#include "fa_kernel.hpp"

namespace fa {

template <int DT, int D, bool CAUSAL, int NWAVES>
struct IWCfg {
  static constexpr int WAVES = NWAVES;
  static constexpr int BM = WAVES * 32;
  static constexpr int BN = 64;
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  static constexpr int STAGES = 4;
  // K tiles of the four stages first, then their V tiles: every fragment
  // read is a per-lane base register plus an immediate below 64 KB
  static constexpr int V_REGION = STAGES * TILE_BYTES;
  static constexpr int LDS_BYTES = 2 * STAGES * TILE_BYTES;
  static constexpr int LOADS = TILE_BYTES / (WAVES * 64 * 16);   // per thread per matrix
  static_assert(TILE_BYTES % (WAVES * 64 * 16) == 0, "tile must split into 16-byte lane loads");
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Softmax work of one tile (NV scores per lane), as a sequence of units:
//   [0, NV/2)        running max, one 3-input maximum (two scores) per unit
//   NV/2             combine the chains, swap halves, rescale decision
//   then NV/2 times  exp2 of two scores (FMA, exp, add each) and their pack
// with the approximate VALU issue cycles of each unit, so that the units can
// be spread evenly over the MFMA slots of an iteration.
template <int NV>
struct IWUnits {
  static constexpr int DEC = NV / 2;
  static constexpr int EXP0 = DEC + 1;
  static constexpr int TOTAL = EXP0 + (NV / 2) * 3;
  static constexpr int cost(int u) {
    return u < DEC ? 4 : u == DEC ? 48 : ((u - EXP0) % 3 == 2 ? 4 : 16);
  }
  static constexpr int cum(int u) {
    int s = 0;
    for (int i = 0; i < u; ++i) s += cost(i);
    return s;
  }
  // first unit of slot i (of ns): the first unit whose cost starts at or
  // after the slot's even share of the total
  static constexpr int begin(int i, int ns) {
    int u = 0;
    while (u < TOTAL && cum(u) * ns < cum(TOTAL) * i) ++u;
    return u;
  }
};

// Calls f(std::integral_constant<int, i>) for i = B .. E-1, so that every
// index in f's body is a compile-time constant.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ float maxnum3(float a, float b, float c) {
  // NaN-propagating maximum (v_maximum3_f32): no canonicalisation needed
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

template <int DT, int D, bool CAUSAL, int NWAVES>
__global__ void __launch_bounds__(NWAVES * 64, 1) fa_fwd_interleaved_kernel(Params p) {
  static_assert(DT == DT_BF16 || DT == DT_FP16, "16-bit inputs only");
  using C = IWCfg<DT, D, CAUSAL, NWAVES>;
  constexpr int BN = C::BN, BM = C::BM, RB = C::ROW_BYTES;
  constexpr int NKC = D / 16, NKB = BN / 32, NDB = D / 32, NPC = BN / 16;
  constexpr int NPV = NPC * NDB;            // PV slots
  constexpr int NQK = NKC * NKB;            // QK slots
  constexpr int NS = NPV + NQK;             // MFMA slots per iteration
  constexpr int NV = NKB * 16;              // scores per lane per tile
  constexpr int kAhead = 4;                 // LDS reads run this many slots ahead
  constexpr int PER_STAGE = 2 * C::LOADS;   // LDS-direct loads per thread per stage
  using U = IWUnits<NV>;

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

  // ---- stages: stage s holds K_{s+1} and V_{s-1}, in ring slot (s+1) % 4 ----
  // A tile's loads use a buffer resource based at its first row whose range
  // ends at key n_kv (empty for tiles outside [0, n_tiles)), so each thread's
  // offsets are the same for every tile and rows past the keys read as zeros.
  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);
  uint32_t dma_off[C::LOADS];
#pragma unroll
  for (int u = 0; u < C::LOADS; ++u) {
    const int lds_off = (wave * C::LOADS + u) * 1024 + lane * 16;
    const int row = lds_off / RB;
    dma_off[u] = (uint32_t)row * RB + (((lds_off % RB) / 16) ^ swz<RB>(row)) * 16;
  }
  auto tile_rsrc = [&](const char *base, int t) __attribute__((always_inline)) {
    const bool ok = t >= 0 && t < n_tiles;
    const int start = ok ? t * BN : 0;
    return make_rsrc_words(base + (int64_t)start * RB, ok ? (uint32_t)(n_kv - start) * RB : 0u);
  };
  auto issue_stage = [&](int s, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const i32x4 kr = tile_rsrc(kh, s + 1);
    const i32x4 vr = tile_rsrc(vh, s - 1);
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
      const uint32_t lds = smem_base + buf * C::TILE_BYTES + (wave * C::LOADS + u) * 1024;
      lds_dma16(kr, dma_off[u], lds);
      lds_dma16(vr, dma_off[u], lds + C::V_REGION);
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
  // Absolute LDS addresses of the fragments in ring slot 0. They are made
  // opaque to the compiler so that the slot, key-chunk and region offsets
  // (all below 64 KB) stay in the instructions' immediate offset field
  // instead of being re-added to the lane address before every read.
  uint32_t kaddr[NKC], vaddr[2][NDB];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    kaddr[kc] = smem_base + koff[kc];
    asm volatile("" : "+v"(kaddr[kc]));
  }
#pragma unroll
  for (int jg = 0; jg < 2; ++jg)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      vaddr[jg][db] = smem_base + C::V_REGION + voff[jg][db];
      asm volatile("" : "+v"(vaddr[jg][db]));
    }
  // fragment of slot i in buffer buf: V^T (pc, db) for i < NPV, else K (kc, kb)
  auto frag = [&](auto buf_c, int slot) __attribute__((always_inline)) -> u32x4 {
    constexpr int buf = decltype(buf_c)::value;
    if (slot < NPV) {
      const int pc = slot / NDB, db = slot % NDB;
      u32x4 a;
#pragma unroll
      for (int jg = 0; jg < 2; ++jg) {
        FA_LDS char *addr = (FA_LDS char *)(uintptr_t)vaddr[jg][db] + (buf * C::TILE_BYTES + pc * 16 * RB);
        const u32x2 xx = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4 *)addr));
        a[jg * 2] = xx[0];
        a[jg * 2 + 1] = xx[1];
      }
      return a;
    }
    const int kc = (slot - NPV) / NKB, kb = (slot - NPV) % NKB;
    return *(const FA_LDS u32x4 *)((FA_LDS char *)(uintptr_t)kaddr[kc] + (buf * C::TILE_BYTES + kb * 32 * RB));
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
  auto qk_only = [&](auto buf_c, f32x16 (&s)[NKB]) __attribute__((always_inline)) {
    u32x4 fb[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) fb[i] = frag(buf_c, NPV + i);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 a = fb[i % kAhead];
      if (i + kAhead < NQK) fb[i % kAhead] = frag(buf_c, NPV + i + kAhead);
      const int kc = i / NKB, kb = i % NKB;
      const u32x4 b = {qf[kc][0], qf[kc][1], qf[kc][2], qf[kc][3]};
      s[kb] = mfma16(a, b, kc == 0 ? f32x16{} : s[kb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // PV of one tile as a plain pipelined stream (epilogue)
  auto pv_only = [&](auto buf_c, const u32x4 (&pp)[NPC]) __attribute__((always_inline)) {
    u32x4 fb[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) fb[i] = frag(buf_c, i);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 a = fb[i % kAhead];
      if (i + kAhead < NPV) fb[i % kAhead] = frag(buf_c, i + kAhead);
      acc[i % NDB] = mfma16(a, pp[i / NDB], acc[i % NDB]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // masks of tile t on its scores (only tiles past the keys or on the diagonal)
  // Score i of block kb is key kstart + half*4 + off(kb, i) with the
  // compile-time off = kb*32 + 8*(i/4) + i%4; it is masked when off reaches
  // lim, the first invisible key (past n_kv, or past this row's diagonal)
  // relative to kstart + half*4.
  auto mask_tile = [&](int t, f32x16 (&s)[NKB]) __attribute__((always_inline)) {
    const int kstart = t * BN;
    if ((kstart + BN > kend) || (CAUSAL && kstart + BN - 1 > qw)) {
      int lim = n_kv - kstart - half * 4;
      if (CAUSAL) lim = min(lim, my_q + 1 - kstart - half * 4);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 8 * (i / 4) + (i % 4) >= lim) s[kb][i] = -INFINITY;
    }
  };

  // ---- one iteration (phase ph = j % 4): softmax(j) on sc -> po,
  //      MFMAs PV(j-1) with pp and QK(j+1) into sn ----
  auto iteration = [&](int j, auto ph_c, f32x16 (&sc)[NKB], f32x16 (&sn)[NKB], const u32x4 (&pp)[NPC],
                       u32x4 (&po)[NPC]) __attribute__((always_inline)) {
    constexpr int ph = decltype(ph_c)::value;
    constexpr int buf = (ph + 1) % 4;          // stage j lives in buffer (j+1) % 4
    const auto bufc = std::integral_constant<int, buf>{};

    issue_stage(j + 3, std::integral_constant<int, ph>{});   // buffer (j+4) % 4
    mask_tile(j, sc);
    float mx0 = -INFINITY, mx1 = -INFINITY, rs0 = 0.f, rs1 = 0.f, neg = 0.f, alpha = 1.f;
    bool rescale = false;
    auto unit = [&](auto u_c) __attribute__((always_inline)) {
      constexpr int u = decltype(u_c)::value;
      if constexpr (u < U::DEC) {
        const int e = 2 * u;
        const float x0 = sc[e / 16][e % 16], x1 = sc[(e + 1) / 16][(e + 1) % 16];
        if constexpr (u & 1) mx1 = maxnum3(mx1, x0, x1);
        else mx0 = maxnum3(mx0, x0, x1);
      } else if constexpr (u == U::DEC) {
        const float m2 = __builtin_elementwise_maximum(mx0, mx1);
        const u32x2 r = __builtin_bit_cast(u32x2, __builtin_amdgcn_permlane32_swap(
            __float_as_uint(m2), __float_as_uint(m2), false, false));
        const float mx = __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1])) * c;
        rescale = __builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0;
        const float m_new = rescale ? __builtin_elementwise_maximum(m_run, mx) : m_run;
        // alpha = 0 on the first visible tile (m_run = -inf), 1 if unchanged
        alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        neg = (m_run == -INFINITY) ? 0.f : -m_run;
      } else {
        constexpr int k = (u - U::EXP0) / 3, part = (u - U::EXP0) % 3;
        constexpr int pc = k / 4, w = k % 4, kb = pc / 2, i0 = (pc % 2) * 8 + 2 * w;
        if constexpr (part < 2) {
          const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i0 + part], c, neg));
          sc[kb][i0 + part] = x;
          if constexpr (part) rs1 += x;
          else rs0 += x;
        } else {
          po[pc][w] = pack2<DT>(sc[kb][i0], sc[kb][i0 + 1]);
        }
      }
    };
    u32x4 fb[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) fb[i] = frag(bufc, i);
    static_for<0, NS>([&](auto i_c) __attribute__((always_inline)) {
      constexpr int i = decltype(i_c)::value;
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 a = fb[i % kAhead];
      if constexpr (i + kAhead < NS) fb[i % kAhead] = frag(bufc, i + kAhead);
      if constexpr (i < NPV) {
        acc[i % NDB] = mfma16(a, pp[i / NDB], acc[i % NDB]);
      } else {
        constexpr int kc = (i - NPV) / NKB, kb = (i - NPV) % NKB;
        const u32x4 b = {qf[kc][0], qf[kc][1], qf[kc][2], qf[kc][3]};
        sn[kb] = mfma16(a, b, kc == 0 ? f32x16{} : sn[kb]);
      }
      static_for<U::begin(i, NS), U::begin(i + 1, NS)>(unit);
    });
    // the probabilities are consumed in the next iteration only; pin them
    // here so that the compiler keeps their computation inside the stream
    // instead of sinking it past the rescale branch below
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc)
#pragma unroll
      for (int w = 0; w < 4; ++w) asm volatile("" : "+v"(po[pc][w]));
    __builtin_amdgcn_sched_barrier(0);
    l_run += rs0 + rs1;
    if (rescale) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
    }
    wait_vmcnt<2 * PER_STAGE>();          // stage j+1 has landed (j+2, j+3 may be in flight)
    __syncthreads();
  };

  // ---- prologue: stages -1 .. 2 in flight; S_0 = QK(0) from stage -1 ----
  issue_stage(-1, std::integral_constant<int, 0>{});
  issue_stage(0, std::integral_constant<int, 1>{});
  issue_stage(1, std::integral_constant<int, 2>{});
  issue_stage(2, std::integral_constant<int, 3>{});
  wait_vmcnt<3 * PER_STAGE>();
  __syncthreads();
  qk_only(std::integral_constant<int, 0>{}, sA);
  wait_vmcnt<2 * PER_STAGE>();
  __syncthreads();

  // ---- main loop, unrolled by four over the tile count rounded up to a
  //      multiple of four: the extra tiles lie past the visible keys, read as
  //      zeros and are masked, so they add nothing. The last PV(n-1) reads
  //      stage n, in slot (n+1) % 4 = 1, with the probabilities of phase 3 ----
  const int n_pad = (n_tiles + 3) & ~3;
  for (int j = 0; j < n_pad; j += 4) {
    iteration(j, std::integral_constant<int, 0>{}, sA, sB, pB, pA);
    iteration(j + 1, std::integral_constant<int, 1>{}, sB, sA, pA, pB);
    iteration(j + 2, std::integral_constant<int, 2>{}, sA, sB, pB, pA);
    iteration(j + 3, std::integral_constant<int, 3>{}, sB, sA, pA, pB);
  }
  pv_only(std::integral_constant<int, 1>{}, pB);
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
