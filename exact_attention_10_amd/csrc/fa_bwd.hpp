// FlashAttention-2 backward for gfx950 (CDNA4), 16-bit inputs, hand-written HIP.
//
// The backward recomputes the probabilities tile by tile from the stored row
// log-sum-exp, P = exp(S - L), and needs the row vector D = rowsum(dO * O);
// the key gradients are built by a kernel that walks the query tiles for each
// key tile, and dQ by a second pass instead of atomics ("FlashAttention 2 from
// PyTorch to Triton", What is wrong with this kernel, item 5; What I am
// building, on recovering P from L). With S = scale * Q K^T:
//   dP = dO V^T,  dS = P * (dP - D),  dV = P^T dO,  dQ = scale dS K,
//   dK = scale dS^T Q.
//
// Two kernels, no atomics, deterministic:
//  * fa_bwd_dq_kernel: one workgroup per (batch*head, 128-row query tile), 4
//    waves of 32 query rows, streaming 64-key K/V tiles through LDS exactly as
//    the forward does. It first computes D for its rows from dO and O and
//    stores it, then per key tile S^T = K Q^T and dP^T = V dO^T (a lane owns a
//    query column, so L and D are per-lane scalars), dS^T, and
//    dQ^T += K^T dS^T with K read transposed from LDS.
//  * fa_bwd_dkdv_kernel: one workgroup per (batch*head, 128-key tile), 4
//    waves of 32 keys, streaming 64-row Q/dO tiles (and their L and D) through
//    LDS. Per query tile S = Q K^T and dP = dO V^T with the wave's K and V
//    held in registers (a lane owns a key column), dS, then
//    dV^T += dO^T P and dK^T += Q^T dS with Q and dO read transposed.
// Scores are fp32; P and dS are rounded to the input type for the MFMAs that
// consume them; all gradients accumulate in fp32 and are rounded once.
#pragma once

#include "fa_kernel.hpp"

namespace fa {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct BwdParams {
  const void *q, *k, *v, *o, *dout;   // q, o, dout [BH][nq][D]; k, v [BH][nk][D]
  const float *lse;                   // [BH][nq], natural log, from the forward
  float *delta;                       // [BH][nq]: D = rowsum(dO * O), written by the dq kernel
  void *dq, *dk, *dv;                 // like q, k, v
  int64_t nq, nk;
  int64_t coff;                       // causal: query i sees keys j <= i + coff
  int n_tiles;                        // query tiles (dq) or key tiles (dkdv) per head
  int xcd_remap;
  int pair;                           // causal: one workgroup per (head, pair of tiles)
  float c;                            // scale * log2(e)
  float scale;
};

// Direct global->LDS load of 4 bytes per lane (lane i lands at lds_base + 4*i).
__device__ __forceinline__ void lds_dma4(i32x4 rsrc, uint32_t voffset, uint32_t lds_base) {
  i32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  // the LDS base goes to m0 through an operand constraint, so the compiler
  // knows that m0 is written here
  asm volatile("buffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(r), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

template <int DT>
__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int D>
struct BwdCfg {
  static constexpr int RB = D * 2;                 // bytes per row
  static constexpr int NKC = D / 16;               // 16-wide head-dim chunks (MFMA K for S)
  static constexpr int NDB = D / 32;               // 32-wide head-dim blocks of the d-major accumulators
  // dq kernel: 128 query rows per workgroup, 64-key tiles
  static constexpr int Q_BN = 64;
  static constexpr int Q_TILE = Q_BN * RB;         // one K or V tile
  static constexpr int Q_LDS = 4 * Q_TILE;         // K, V x 2 buffers
  static constexpr int Q_LOADS = Q_TILE / (4 * 64 * 16);
  // dkdv kernel: 128 keys per workgroup, 64-row query tiles
  static constexpr int K_BQ = 64;
  static constexpr int K_TILE = K_BQ * RB;         // one Q or dO tile
  static constexpr int K_STAT = K_BQ * 4;          // L or D of one tile
  static constexpr int K_BUF = 2 * K_TILE + 2 * K_STAT;   // Q, dO, L, D of one stage
  static constexpr int K_LDS = 2 * K_BUF;
  static constexpr int K_LOADS = K_TILE / (4 * 64 * 16);
};

// lane offsets inside a tile of 16-bit rows: the b128 row fragment of chunk kc
// (rows l32 of a 32-row block) and the transposing read of 4 rows x 4 columns
// (the same swizzled layout and offsets the forward uses for K and V)
template <int D>
struct TileOffsets {
  uint32_t row[D / 16];
  uint32_t tr[2][D / 32];
  __device__ __forceinline__ TileOffsets(int lane) {
    constexpr int RB = D * 2;
    const int l32 = lane & 31, half = lane >> 5;
    const int g = lane >> 4, r = (lane & 15) >> 2, cq = lane & 3;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) row[kc] = l32 * RB + (((kc * 2 + half) ^ swz<RB>(l32)) * 16);
#pragma unroll
    for (int jg = 0; jg < 2; ++jg)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int col = db * 32 + (g & 1) * 16 + cq * 4;
        const int key = jg * 8 + (g >> 1) * 4 + r;
        tr[jg][db] = key * RB + ((((col * 2) / 16) ^ swz<RB>(key)) * 16) + (col * 2) % 16;
      }
  }
};

template <int D>
__device__ __forceinline__ u32x4 lds_row_frag(const char *tile, const TileOffsets<D> &off, int kc, int blk) {
  return *(const FA_LDS u32x4 *)(tile + off.row[kc] + blk * 32 * D * 2);
}

// A operand of a d-major product over 16 rows of a tile (the rows of chunk pc
// in the permuted order the score accumulator imposes), columns db*32 ...
template <int D>
__device__ __forceinline__ u32x4 lds_tr_frag(const char *tile, const TileOffsets<D> &off, int pc, int db) {
  u32x4 a;
#pragma unroll
  for (int jg = 0; jg < 2; ++jg) {
    const u32x2 xx = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (FA_LDS s16x4 *)(tile + off.tr[jg][db] + pc * 16 * D * 2)));
    a[jg * 2] = xx[0];
    a[jg * 2 + 1] = xx[1];
  }
  return a;
}

// Row fragments of one 16-bit row held in registers: lane (l32, half) holds
// row[kc*16 + half*8 .. +7] for every chunk kc (the B operand layout).
template <int D>
__device__ __forceinline__ void load_row_frags(u32x4 (&f)[D / 16], const __amdgpu_buffer_rsrc_t rs,
                                               int row, bool ok, int half) {
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    const uint32_t off = (uint32_t)row * (D * 2) + (uint32_t)((kc * 16 + half * 8) * 2);
    f[kc] = ok ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0)) : u32x4{0, 0, 0, 0};
  }
}

template <int DT>
__device__ __forceinline__ float dot_pairs(uint32_t a, uint32_t b) {
  if constexpr (DT == DT_BF16) {
    const bf16x2 x = __builtin_bit_cast(bf16x2, a), y = __builtin_bit_cast(bf16x2, b);
    return (float)x[0] * (float)y[0] + (float)x[1] * (float)y[1];
  } else {
    const f16x2 x = __builtin_bit_cast(f16x2, a), y = __builtin_bit_cast(f16x2, b);
    return (float)x[0] * (float)y[0] + (float)x[1] * (float)y[1];
  }
}

// Store a d-major fp32 accumulator (lane owns row `row`, d = db*32 + 8*gq +
// half*4 + 0..3) times `mul`, rounded to the 16-bit type.
template <int DT, int D>
__device__ __forceinline__ void store_rows(void *base, int64_t row, const f32x16 (&acc)[D / 32], float mul, int half) {
  char *dst = (char *)base + row * (D * 2);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d0 = db * 32 + 8 * gq + half * 4;
      const uint32_t w0 = pack2<DT>(acc[db][gq * 4 + 0] * mul, acc[db][gq * 4 + 1] * mul);
      const uint32_t w1 = pack2<DT>(acc[db][gq * 4 + 2] * mul, acc[db][gq * 4 + 3] * mul);
      *(u32x2 *)(dst + d0 * 2) = u32x2{w0, w1};
    }
}

__device__ __forceinline__ int remap_block(int bid, int nblk, int xcd_remap) {
  return (xcd_remap && (nblk & 7) == 0) ? (bid & 7) * (nblk >> 3) + (bid >> 3) : bid;
}

// The (head, tile) jobs of a workgroup. Causal work per tile grows (dQ: with
// the query tile) or shrinks (dK/dV: with the key tile) linearly, so with
// p.pair a workgroup takes tiles i and n_tiles-1-i, the longer first, and
// every workgroup does the same work; otherwise one tile per workgroup.
struct BwdJobs {
  int bh, first, second;   // second < 0: a single job
};
__device__ __forceinline__ BwdJobs bwd_jobs(const BwdParams &p, bool causal, bool work_grows) {
  const int T = p.n_tiles;
  const int c = remap_block(blockIdx.x, gridDim.x, p.xcd_remap);
  BwdJobs j;
  if (causal && p.pair) {
    const int npairs = (T + 1) / 2;
    j.bh = c / npairs;
    const int pr = c - j.bh * npairs;
    const int lo = pr, hi = T - 1 - pr;
    j.first = work_grows ? hi : lo;
    j.second = (lo != hi) ? (work_grows ? lo : hi) : -1;
  } else {
    j.bh = c / T;
    j.first = c - j.bh * T;
    if (causal && work_grows) j.first = T - 1 - j.first;   // longest first
    j.second = -1;
  }
  return j;
}

// ---------------------------------------------------------------------------
// dQ (and D) kernel

template <int DT, int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1) fa_bwd_dq_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  constexpr int RB = C::RB, NKC = C::NKC, NDB = C::NDB, BN = C::Q_BN, TB = C::Q_TILE;
  constexpr int BM = 128, NKB = BN / 32, NPC = BN / 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const BwdJobs jobs = bwd_jobs(p, CAUSAL, true);
  const int bh = jobs.bh;
  for (int job = 0; job < 2; ++job) {
  if (job == 1) {
    if (jobs.second < 0) break;
    __syncthreads();                     // every wave is done with the first tile's LDS
  }
  const int qt = job == 0 ? jobs.first : jobs.second;
  const int64_t Nq = p.nq;
  const int Nk = (int)p.nk, coff = (int)p.coff;
  const int q0 = qt * BM, qw = q0 + wave * 32, my_q = qw + l32;
  const bool row_ok = my_q < Nq;

  const int64_t q_head = Nq * D, k_head = (int64_t)Nk * D;
  const char *kh = (const char *)p.k + (int64_t)bh * k_head * 2;
  const char *vh = (const char *)p.v + (int64_t)bh * k_head * 2;
  int kend = Nk;
  if (CAUSAL) kend = min(kend, q0 + BM + coff);
  const int n_tiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  // Q and dO rows of this lane (B operands), O only for D = rowsum(dO * O)
  u32x4 qf[NKC], df[NKC];
  float delta, nlse;
  {
    const uint32_t bytes = (uint32_t)(q_head * 2);
    const __amdgpu_buffer_rsrc_t qr = make_rsrc((const char *)p.q + (int64_t)bh * q_head * 2, bytes);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc((const char *)p.dout + (int64_t)bh * q_head * 2, bytes);
    const __amdgpu_buffer_rsrc_t orr = make_rsrc((const char *)p.o + (int64_t)bh * q_head * 2, bytes);
    load_row_frags<D>(qf, qr, my_q, row_ok, half);
    load_row_frags<D>(df, dr, my_q, row_ok, half);
    u32x4 of[NKC];
    load_row_frags<D>(of, orr, my_q, row_ok, half);
    float part = 0.f;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int w = 0; w < 4; ++w) part += dot_pairs<DT>(df[kc][w], of[kc][w]);
    delta = halves_sum(part);
    const float L = row_ok ? p.lse[(int64_t)bh * Nq + my_q] : 0.f;
    // a row that saw no key in the forward (L = -inf) has every key masked
    // here too; its exponent reference only has to stay finite
    nlse = (L == -INFINITY) ? 0.f : -L * 1.4426950408889634f;
    if (row_ok && half == 0) p.delta[(int64_t)bh * Nq + my_q] = delta;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);
  uint32_t dma_off[C::Q_LOADS];
#pragma unroll
  for (int u = 0; u < C::Q_LOADS; ++u) {
    const int lds_off = (wave * C::Q_LOADS + u) * 1024 + lane * 16;
    const int row = lds_off / RB;
    dma_off[u] = (uint32_t)row * RB + (((lds_off % RB) / 16) ^ swz<RB>(row)) * 16;
  }
  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    const int kstart = t * BN;
    const uint32_t valid = (uint32_t)(Nk - kstart) * RB;
    const i32x4 kr = make_rsrc_words(kh + (int64_t)kstart * RB, valid);
    const i32x4 vr = make_rsrc_words(vh + (int64_t)kstart * RB, valid);
#pragma unroll
    for (int u = 0; u < C::Q_LOADS; ++u) {
      const uint32_t lds = smem_base + buf * (2 * TB) + (wave * C::Q_LOADS + u) * 1024;
      lds_dma16(kr, dma_off[u], lds);
      lds_dma16(vr, dma_off[u], lds + TB);
    }
  };
  const TileOffsets<D> off(lane);

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  const float c = p.c;

  auto step = [&](int t, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    wait_vmem();
    __syncthreads();
    if (t + 1 < n_tiles) issue_tile(t + 1, buf ^ 1);
    const int kstart = t * BN;
    if (CAUSAL && kstart > qw + 31 + coff) return;
    const char *kl = smem + buf * (2 * TB);
    const char *vl = kl + TB;

    // S^T = K Q^T and dP^T = V dO^T (keys x queries; a lane owns one query)
    f32x16 s[NKB], dp[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{}, dp[kb] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = mfma16<DT>(lds_row_frag<D>(kl, off, kc, kb), qf[kc], s[kb]);
        dp[kb] = mfma16<DT>(lds_row_frag<D>(vl, off, kc, kb), df[kc], dp[kb]);
      }
    const bool need_mask = (kstart + BN > Nk) || (CAUSAL && kstart + BN - 1 > qw + coff);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kstart + kb * 32 + 8 * (i / 4) + half * 4 + (i % 4);
          if ((key >= Nk) || (CAUSAL && key > my_q + coff)) s[kb][i] = -INFINITY;
        }
    }
    // dS^T = P^T (dP^T - D), P^T = exp2(S^T c - L log2 e), packed as B operands
#pragma unroll
    for (int pc = 0; pc < NPC; ++pc) {
      const int kb = pc / 2, i0 = (pc % 2) * 8;
      u32x4 b;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int i = i0 + 2 * w;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, nlse));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i + 1], c, nlse));
        b[w] = pack2<DT>(p0 * (dp[kb][i] - delta), p1 * (dp[kb][i + 1] - delta));
      }
      // dQ^T += K^T dS^T over the 16 keys of chunk pc
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = mfma16<DT>(lds_tr_frag<D>(kl, off, pc, db), b, acc[db]);
    }
  };

  if (n_tiles > 0) issue_tile(0, 0);
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < n_tiles) step(t + 1, std::integral_constant<int, 1>{});
  }
  if (row_ok) store_rows<DT, D>(p.dq, (int64_t)bh * Nq + my_q, acc, p.scale, half);
  }   // job
}

// ---------------------------------------------------------------------------
// dK and dV kernel

template <int DT, int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 1) fa_bwd_dkdv_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  constexpr int RB = C::RB, NKC = C::NKC, NDB = C::NDB, BQ = C::K_BQ, TB = C::K_TILE;
  constexpr int BKEYS = 128, NQB = BQ / 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const BwdJobs jobs = bwd_jobs(p, CAUSAL, false);
  const int bh = jobs.bh;
  for (int job = 0; job < 2; ++job) {
  if (job == 1) {
    if (jobs.second < 0) break;
    __syncthreads();                     // every wave is done with the first tile's LDS
  }
  const int kt = job == 0 ? jobs.first : jobs.second;
  const int Nq = (int)p.nq, Nk = (int)p.nk, coff = (int)p.coff;
  const int k0 = kt * BKEYS, kw = k0 + wave * 32, my_key = kw + l32;
  const bool key_ok = my_key < Nk;

  const int64_t q_head = (int64_t)Nq * D, k_head = (int64_t)Nk * D;
  const char *qh = (const char *)p.q + (int64_t)bh * q_head * 2;
  const char *dh = (const char *)p.dout + (int64_t)bh * q_head * 2;
  const float *lh = p.lse + (int64_t)bh * Nq;
  const float *deh = p.delta + (int64_t)bh * Nq;

  // query tiles that can see some key of this workgroup: i + coff >= k0
  int qbegin = 0;
  if (CAUSAL) qbegin = max(0, (k0 - coff) / BQ * BQ);
  const int t_first = qbegin / BQ;
  const int n_qt = (Nq + BQ - 1) / BQ;

  // K and V rows of this lane's key (B operands of S = Q K^T and dP = dO V^T)
  u32x4 kf[NKC], vf[NKC];
  {
    const uint32_t bytes = (uint32_t)(k_head * 2);
    load_row_frags<D>(kf, make_rsrc((const char *)p.k + (int64_t)bh * k_head * 2, bytes), my_key, key_ok, half);
    load_row_frags<D>(vf, make_rsrc((const char *)p.v + (int64_t)bh * k_head * 2, bytes), my_key, key_ok, half);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);

  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);
  uint32_t dma_off[C::K_LOADS];
#pragma unroll
  for (int u = 0; u < C::K_LOADS; ++u) {
    const int lds_off = (wave * C::K_LOADS + u) * 1024 + lane * 16;
    const int row = lds_off / RB;
    dma_off[u] = (uint32_t)row * RB + (((lds_off % RB) / 16) ^ swz<RB>(row)) * 16;
  }
  // stage layout: Q tile, dO tile, the exponent offsets -L log2(e) (64 floats),
  // D (64 floats). Wave 0 loads a tile's L into a register when the tile is
  // requested and, once the loads have landed, stores -L log2(e) (-inf for a
  // row that saw no key) into the stage just before the barrier that
  // publishes it, so the per-row conversion is done once per tile, not by
  // every lane that reads the row.
  float l_next = 0.f;
  auto issue_tile = [&](int t, int buf) __attribute__((always_inline)) {
    const int qstart = t * BQ;
    const uint32_t valid = (uint32_t)(Nq - qstart) * RB;
    const i32x4 qr = make_rsrc_words(qh + (int64_t)qstart * RB, valid);
    const i32x4 dr = make_rsrc_words(dh + (int64_t)qstart * RB, valid);
    const uint32_t stage = smem_base + buf * C::K_BUF;
#pragma unroll
    for (int u = 0; u < C::K_LOADS; ++u) {
      const uint32_t lds = stage + (wave * C::K_LOADS + u) * 1024;
      lds_dma16(qr, dma_off[u], lds);
      lds_dma16(dr, dma_off[u], lds + TB);
    }
    if (wave == 0) {
      const uint32_t svalid = (uint32_t)(Nq - qstart) * 4;
      // rows past the queries read L = 0 (their Q and dO rows are zero too)
      l_next = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(lh + qstart, svalid), (uint32_t)lane * 4, 0, 0));
      lds_dma4(make_rsrc_words(deh + qstart, svalid), (uint32_t)lane * 4, stage + 2 * TB + C::K_STAT);
    }
  };
  // called by every wave after wait_vmem() and before the barrier that
  // publishes stage `buf`
  auto publish_offsets = [&](int buf) __attribute__((always_inline)) {
    if (wave == 0) {
      const float nl = (l_next == -INFINITY) ? -INFINITY : -l_next * 1.4426950408889634f;
      *(FA_LDS float *)(smem + buf * C::K_BUF + 2 * TB + lane * 4) = nl;
    }
  };
  const TileOffsets<D> off(lane);

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dk[i] = f32x16{}, dv[i] = f32x16{};
  const float c = p.c;

  auto step = [&](int t, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    wait_vmem();
    publish_offsets(buf);
    __syncthreads();
    if (t + 1 < n_qt) issue_tile(t + 1, buf ^ 1);
    const int qstart = t * BQ;
    // every query of this tile is before the wave's first visible diagonal
    if (CAUSAL && qstart + BQ - 1 + coff < kw) return;
    const char *stage = smem + buf * C::K_BUF;
    const char *ql = stage, *dl = stage + TB;
    const float *ls = (const float *)(stage + 2 * TB);
    const float *ds_ = (const float *)(stage + 2 * TB + C::K_STAT);
    const bool need_mask = CAUSAL && (qstart + coff < kw + 31);

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // S = Q K^T and dP = dO V^T (queries x keys; a lane owns one key)
      // every row fragment of the block is requested before the first MFMA
      // (one wave per SIMD: nothing else hides the LDS latency)
      f32x16 s = f32x16{}, dp = f32x16{};
      u32x4 qr[NKC], dr[NKC];
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        qr[kc] = lds_row_frag<D>(ql, off, kc, qb);
        dr[kc] = lds_row_frag<D>(dl, off, kc, qb);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        s = mfma16<DT>(qr[kc], kf[kc], s);
        dp = mfma16<DT>(dr[kc], vf[kc], dp);
      }
      // L and D of the 16 query rows this lane holds: rows 8*g + half*4 + 0..3
      float nl[16], dd[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = qb * 32 + 8 * g + half * 4;
        const f32x4 lvv = *(const FA_LDS f32x4 *)(ls + r0);
        const f32x4 dvv = *(const FA_LDS f32x4 *)(ds_ + r0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // rows past the queries have offset 0, D = 0 and zero Q and dO, so
          // they contribute nothing; a row that saw no key has offset -inf: P = 0
          nl[4 * g + j] = lvv[j];
          dd[4 * g + j] = dvv[j];
        }
      }
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int q = qstart + qb * 32 + 8 * (i / 4) + half * 4 + (i % 4);
          if (my_key > q + coff) s[i] = -INFINITY;
        }
      }
      // P and dS as B operands (a lane owns a key; 8 query rows per half)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int pc = qb * 2 + h, i0 = h * 8;
        u32x4 bp, bs;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int i = i0 + 2 * w;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, nl[i]));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i + 1], c, nl[i + 1]));
          bp[w] = pack2<DT>(p0, p1);
          bs[w] = pack2<DT>(p0 * (dp[i] - dd[i]), p1 * (dp[i + 1] - dd[i + 1]));
        }
        // dV^T += dO^T P and dK^T += Q^T dS over the 16 query rows of chunk pc
        u32x4 ta[NDB], tb[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          ta[db] = lds_tr_frag<D>(dl, off, pc, db);
          tb[db] = lds_tr_frag<D>(ql, off, pc, db);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dv[db] = mfma16<DT>(ta[db], bp, dv[db]);
          dk[db] = mfma16<DT>(tb[db], bs, dk[db]);
        }
      }
    }
  };

  if (t_first < n_qt) issue_tile(t_first, 0);
  for (int t = t_first; t < n_qt; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < n_qt) step(t + 1, std::integral_constant<int, 1>{});
  }
  if (key_ok) {
    store_rows<DT, D>(p.dk, (int64_t)bh * Nk + my_key, dk, p.scale, half);
    store_rows<DT, D>(p.dv, (int64_t)bh * Nk + my_key, dv, 1.0f, half);
  }
  }   // job
}

}  // namespace fa
