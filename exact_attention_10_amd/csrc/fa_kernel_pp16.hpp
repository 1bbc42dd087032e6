// Two-group FlashAttention-2 forward on 16x16x32 MFMAs (gfx950), 16-bit
// inputs, with or without the causal mask.
//
// The schedule is that of fa_kernel_pp.hpp (two groups of four waves, a
// matrix phase M(j) = S(j) then PV(j-1) and a softmax phase X(j) per key
// tile, one barrier per tile that group 0 reaches after X(j) and group 1
// after M(j), K and V through two rings of four LDS stages). Only the matrix
// products use the 16x16x32 form instead of 32x32x16. On gfx950 that form
// does the same work per clock for less power: each product reads and writes
// a quarter of the accumulator registers of a 32x32x16 product for half its
// FLOPs. Every K and V fragment read from LDS feeds two products (the wave's
// two 16-query blocks), so the LDS traffic is that of the 32x32x16 kernel.
//
// Layouts (g = lane / 16, i16 = lane % 16):
//   S^T block (16 keys x 16 queries), accumulator: lane holds query i16 of
//     the block and keys 4g .. 4g+3 of it. A wave's 32 queries are two
//     blocks; a tile's 64 keys four, so a lane holds 16 scores of each of its
//     two queries and the four lanes with the same i16 hold all 64.
//   O^T block (16 head dims x 16 queries): lane holds query i16 and head
//     dims 4g .. 4g+3 of the block.
//   P^T operand (32 keys x 16 queries): lane holds query i16 and eight keys,
//     the four of S^T block 2c and the four of block 2c+1 that it holds; the
//     V^T operand reads its keys in the same order.
// The arithmetic per score is that of fa_kernel.hpp ("A09 - Advanced Triton &
// FlashAttention", section 3, The kernel, in pseudocode); the row max and
// the row sum take two lane swaps across the four lanes of a query. Under
// the causal mask ("A09", section 3, causal tile skipping) the workgroup
// streams the key tiles up to its last row's diagonal and every wave runs
// both phases on all of them, masking element by element the tiles that
// reach past one of its rows. On a tile wholly past its rows a wave skips the
// products and their LDS reads but still runs the (fully masked) softmax, so
// the two waves of a SIMD keep their phases in step near the diagonal and the
// overlap of one's matrix phase with the other's softmax holds there too.
// Causal workgroups take a pair of query tiles (T-1-i, i) when the grid of
// pairs still fills the chip, as fa_kernel.hpp does.
#pragma once

#include "fa_kernel_pp.hpp"

namespace fa {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The larger of x over the four lanes that hold a query (lanes l, l ^ 16,
// l ^ 32, l ^ 48).
__device__ __forceinline__ float quad_max(float x) {
  u32x2 r = __builtin_bit_cast(u32x2, __builtin_amdgcn_permlane16_swap(
      __float_as_uint(x), __float_as_uint(x), false, false));
  x = score_max(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_bit_cast(u32x2, __builtin_amdgcn_permlane32_swap(
      __float_as_uint(x), __float_as_uint(x), false, false));
  return score_max(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  u32x2 r = __builtin_bit_cast(u32x2, __builtin_amdgcn_permlane16_swap(
      __float_as_uint(x), __float_as_uint(x), false, false));
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_bit_cast(u32x2, __builtin_amdgcn_permlane32_swap(
      __float_as_uint(x), __float_as_uint(x), false, false));
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The lane index, formed by an mbcnt the compiler cannot merge with another:
// used where a value derived from it would otherwise stay live across the key
// loop, to be spilled to scratch and reloaded (a reload waits for every
// outstanding memory operation, the tile transfers included)
__device__ __forceinline__ int fresh_lane_id() {
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  return ln;
}

template <int DT, int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 2) fa_fwd_pp16_kernel(Params p) {
  static_assert(DT == DT_BF16 || DT == DT_FP16, "16-bit inputs only");
  static_assert(D == 64 || D == 128, "head dim");
  using C = PPCfg<D>;
  constexpr int BN = C::BN, BM = C::BM, RB = C::ROW_BYTES, LOADS = C::LOADS;
  constexpr int NKC = D / 32;       // 32-wide head-dim chunks of S^T = K Q^T
  constexpr int NMB = BN / 16;      // 16-key blocks of S^T
  constexpr int NDB = D / 16;       // 16-wide head-dim blocks of O^T
  constexpr int NPC = BN / 32;      // 32-key chunks of P^T
  constexpr int NKF = NKC * NMB;    // K fragments per tile
  constexpr int NVF = NPC * NDB;    // V^T fragments per tile
  constexpr int KW = 6;             // K fragments requested ahead of their MFMAs
  constexpr int VW = NVF < 12 ? NVF : 12;   // V^T fragments requested ahead (the first during S)
  static_assert(KW <= NKF && VW <= NVF, "look-ahead within a tile");

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int w4 = wave & 3;
  const int lane = tid & 63;
  const int i16 = lane & 15;
  const int g = lane >> 4;

  // ---- which (head, query tile) this workgroup owns: as fa_kernel.hpp,
  // with the causal grid's longest tiles first, or one workgroup per (head,
  // pair of query tiles T-1-i and i), which then runs both in turn ----
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if (p.xcd_remap && (nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  int bh = bid / p.nq_tiles;
  int qt = bid - bh * p.nq_tiles;
  if (CAUSAL) qt = p.nq_tiles - 1 - qt;
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

  // ---- tile transfers, as in fa_kernel_pp.hpp ----
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
  auto issue_tile = [&](int t, int st) __attribute__((always_inline)) {
    const int kstart = t * BN;
    const i32x4 r = make_rsrc_words(my_src + (int64_t)kstart * RB, (uint32_t)(n_kv - kstart) * RB);
#pragma unroll
    for (int u = 0; u < LOADS; ++u)
      lds_dma16(r, dma_off[u], my_lds + (uint32_t)(st * C::TILE_BYTES + u * 1024));
  };

  // ---- LDS addresses of the operand fragments in stage 0 ----
  // K fragment (kc, mb): key 16 mb + i16, head dims 32 kc + 8 g .. +7. The
  // swizzle of a row depends on its low four bits only, so block mb adds the
  // constant 16 mb rows. V^T fragment (pc, db): transposing reads in which
  // lane 4r + cq of group g addresses key 32 pc + 4 g + r (first read) or
  // that plus 16 (second read), head dims 16 db + 4 cq .. +3; pc and the
  // second read add constant rows. The pointers are formed once; the empty
  // asm keeps the compiler from adding the (zero) base of the dynamic LDS to
  // each offset again inside the loop.
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
      uint32_t a = smem_base + (uint32_t)(C::V_BASE + key * RB + ((((col * 2) / 16) ^ swz<RB>(key)) * 16) + (col * 2) % 16);
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
  // An empty asm that claims to rewrite x: x is produced here, so the code
  // that computes it stays in this phase (the compiler would otherwise sink
  // the softmax past the barrier, next to the MFMAs that read P).
  auto pin = [](uint32_t &x) __attribute__((always_inline)) { asm volatile("" : "+v"(x)); };

  for (int job = 0; job < 2; ++job) {
  if (job == 1) {
    if (second_qt < 0) break;
    qt = second_qt;
    pp_wait_vmcnt<0>();       // the first job's O stores are done: the counts below start from zero
    __syncthreads();          // every wave is done with the first job's LDS stages
  }
  const int q0 = qt * BM;
  const int q_wave = q0 + wave * 32;          // the wave's first query row
  int kend = n_kv;
  if (CAUSAL) kend = min(kend, q0 + BM + coff);
  const int n = kend > 0 ? (kend + BN - 1) / BN : 0;     // key tiles of the workgroup
  // tiles [t_live, n) hold only keys past every row of this wave: their
  // products and fragment reads are skipped; the softmax still runs on them,
  // and its causal mask sets every score of such a tile to -inf
  const int t_live = CAUSAL ? (q_wave + 31 + coff >= 0 ? (q_wave + 31 + coff) / BN + 1 : 0) : n;

  // ---- Q fragments (B operand of S^T = K Q^T): query block nb, head-dim
  // chunk kc: row q_wave + 16 nb + i16, head dims 32 kc + 8 g .. +7. Inline
  // asm like the transfers, so that the compiler counts neither and the
  // explicit waits below are the only ones; rows at or past Nq lie beyond the
  // buffer's range and read as zeros. ----
  uint32_t qf[2][NKC][4];
  {
    const int qln = fresh_lane_id();
    const i32x4 qr = make_rsrc_words(qh, (uint32_t)(q_head * 2));
    i32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(qr[i]);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const uint32_t off = (uint32_t)(q_wave + nb * 16 + (qln & 15)) * RB + (uint32_t)((kc * 32 + (qln >> 4) * 8) * 2);
        u32x4 x;
        asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(x) : "v"(off), "s"(r) : "memory");
#pragma unroll
        for (int w = 0; w < 4; ++w) qf[nb][kc][w] = x[w];
      }
  }

  // ---- running state: per query block nb ----
  f32x4 acc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db][0] = acc[db][1] = f32x4{};
  float m_run[2] = {-INFINITY, -INFINITY};   // exponent reference (base 2), same in the query's four lanes
  float l_run[2] = {0.f, 0.f};               // this lane's partial row sums
  // derived from m_run, updated only where it moves: the threshold past which
  // a score moves the reference, and the exponent offset (0 for a row that
  // has seen no visible key, whose scores are all -inf: p = 0)
  float thr[2] = {-INFINITY, -INFINITY};
  float neg[2] = {0.f, 0.f};
  const float c = p.c;
  // S^T of the current tile (zero until a matrix phase writes it: the
  // softmax of a tile whose products this wave skips reads it, all masked)
  f32x4 s[NMB][2];
  u32x4 pf[NPC][2];            // P^T of the last softmaxed tile, packed to 16 bits
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) s[mb][0] = s[mb][1] = f32x4{};
#pragma unroll
  for (int pc = 0; pc < NPC; ++pc) pf[pc][0] = pf[pc][1] = u32x4{0, 0, 0, 0};

  // ---- matrix phase M(j): S(j) from K stage kst, then PV(j-1) from V
  // stage vst. K fragments stream KW ahead of their MFMAs; the first VW V^T
  // fragments are requested during the second half of S, the others VW ahead
  // of their MFMAs. (At j = 0 the V stage holds no tile yet; its reads are
  // made but never used.) ----
  auto matrix = [&](int j, auto kst_c, auto vst_c) __attribute__((always_inline)) {
    constexpr int kst = decltype(kst_c)::value, vst = decltype(vst_c)::value;
    u32x4 vf[NVF];
    // V^T fragment f = pc * NDB + db
    auto read_v = [&](int f) __attribute__((always_inline)) {
      const int pc = f / NDB, db = f % NDB;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const FA_LDS char *addr = v_ptr[db] + vst * C::TILE_BYTES + (pc * 32 + h * 16) * RB;
        const u32x2 xx = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4 *)addr));
        vf[f][h * 2] = xx[0];
        vf[f][h * 2 + 1] = xx[1];
      }
    };
    __builtin_amdgcn_s_setprio(1);
    if (j < n && j < t_live) {
      u32x4 kf[NKF];
      // K fragment f = kc * NMB + mb
      auto read_k = [&](int f) __attribute__((always_inline)) {
        const int kc = f / NMB, mb = f % NMB;
        kf[f] = *(const FA_LDS u32x4 *)(k_ptr[kc] + kst * C::TILE_BYTES + mb * 16 * RB);
      };
      constexpr int VPER = (VW + NKF / 2 - 1) / (NKF / 2);   // V reads per K fragment, second half
#pragma unroll
      for (int f = 0; f < KW; ++f) read_k(f);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < NKF; ++f) {
        const int kc = f / NMB, mb = f % NMB;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const u32x4 b = {qf[nb][kc][0], qf[nb][kc][1], qf[nb][kc][2], qf[nb][kc][3]};
          s[mb][nb] = mfma(kf[f], b, kc == 0 ? f32x4{} : s[mb][nb]);
        }
        if (f + KW < NKF) read_k(f + KW);
        if (f >= NKF / 2) {
#pragma unroll
          for (int q = 0; q < VPER; ++q) {
            const int v = (f - NKF / 2) * VPER + q;
            if (v < VW) read_v(v);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if (j >= 1 && j - 1 < t_live) {
#pragma unroll
      for (int f = 0; f < VW; ++f) read_v(f);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (j >= 1 && j - 1 < t_live) {
#pragma unroll
      for (int f = 0; f < NVF; ++f) {
        const int pc = f / NDB, db = f % NDB;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[db][nb] = mfma(vf[f], pf[pc][nb], acc[db][nb]);
        if (f + VW < NVF) read_v(f + VW);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- softmax phase X(j): P_j from S_j (VALU only) ----
  auto softmax = [&](int j) __attribute__((always_inline)) {
    if (j < 0 || j >= n) return;
    const int kstart = j * BN;
    // masks only on the tile past the end of the keys and, under the causal
    // mask, on tiles that reach past a row of the wave
    if (kstart + BN > n_kv || (CAUSAL && kstart + BN - 1 > q_wave + coff)) {
      const int ln = fresh_lane_id();
      const int rel = kstart + ((ln >> 2) & ~3);
      int lim[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        lim[nb] = n_kv - 1 - rel;
        if (CAUSAL) lim[nb] = min(lim[nb], q_wave + coff + nb * 16 + (ln & 15) - rel);
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            if (mb * 16 + i > lim[nb]) s[mb][nb][i] = -INFINITY;
    }
    // this lane's maximum of each row (a quarter of the row's keys)
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
    // The reference moves only when a row max exceeds it by more than the
    // slack; acc and l are rescaled together ("A09", section 3, the
    // rebasing). A row max (scaled by c > 0, which keeps order) exceeds the
    // threshold exactly when one of its four lanes' maxima does, so the row
    // max over the lanes is formed only when some row moves.
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
      // P^T chunk pc for this query block: the keys of S^T blocks 2pc, 2pc+1
#pragma unroll
      for (int pc = 0; pc < NPC; ++pc)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int mb = 2 * pc + w / 2, i = (w % 2) * 2;
          uint32_t x = pack2<DT>(s[mb][nb][i], s[mb][nb][i + 1]);
          pin(x);
          pf[pc][nb][w] = x;
        }
    }
  };

  // ---- end of period j, as in fa_kernel_pp.hpp ----
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

  // ---- prologue, as in fa_kernel_pp.hpp (the Q loads are 2 * NKC = 8 or 4
  // instructions, all issued before the transfers) ----
#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (t < n) issue_tile(t, t);
  if (group == 0) {
    if (n >= 3) pp_wait_vmcnt<2 * LOADS>();
    else if (n == 2) pp_wait_vmcnt<LOADS>();
    else pp_wait_vmcnt<0>();
  } else {
    if (n >= 3) pp_wait_vmcnt<3 * LOADS>();
    else if (n == 2) pp_wait_vmcnt<2 * LOADS>();
    else if (n == 1) pp_wait_vmcnt<LOADS>();
    else pp_wait_vmcnt<0>();
  }
  __syncthreads();

  auto period = [&](int j, auto st_c) __attribute__((always_inline)) {
    constexpr int st = decltype(st_c)::value;
    using KS = std::integral_constant<int, st>;
    using VS = std::integral_constant<int, (st + 3) % 4>;
    matrix(j, KS{}, VS{});
    if (group == 1) end_period(j);
    __builtin_amdgcn_sched_barrier(0);
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
  const int oln = fresh_lane_id();
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float l_tot = quad_sum(l_run[nb]);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const int64_t q = q_wave + nb * 16 + (oln & 15);
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
  }  // job
}

}  // namespace fa
