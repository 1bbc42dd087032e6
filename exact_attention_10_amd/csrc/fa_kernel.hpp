// FlashAttention-2 forward kernel for gfx950 (CDNA4), hand-written HIP.
//
// One workgroup owns one (batch*head, query tile) pair: 4 or 8 waves, 32 query
// rows per wave, 128 or 256 rows per tile. The workgroup streams the head's key/value tiles
// (64 keys each) through LDS, double-buffered, with direct global->LDS buffer
// loads; each wave keeps the online-softmax state of its 32 rows in registers
// and never writes a score to memory ("A09 - Advanced Triton &
// FlashAttention", section 3, The kernel, in pseudocode; "Triton:
// FlashAttention-2 Forward Pass", Decomposition).
//
// Matrix products run on MFMA with fp32 accumulation. Scores are computed
// transposed, S^T = K Q^T, so that a lane owns one query column of the 32x32
// accumulator: row max and row sum are in-lane plus one swap between the two
// 32-lane halves, and the per-row rescale factor is a per-lane scalar. The
// output is accumulated transposed as well, O^T += V^T P^T, so P goes from the
// score accumulator to the MFMA B operand without leaving registers; the key
// order that the accumulator layout imposes on P is applied to V when it is
// read from LDS with the transposing LDS read.
//
// Online softmax ("A09", section 3, The rescaling update, written out;
// "Building a Verifiable FlashAttention Forward from PyTorch to Triton",
// Part 3 Step 4): with c = scale*log2(e), the running max m is kept in base-2
// units, p = exp2(s*c - m) is one FMA and one exp, alpha = exp2(m_old - m_new)
// rescales l and the accumulator, and O = acc / l once at the end. LSE is
// (m + log2 l) * ln 2. A row that has seen no visible key keeps m = -inf; the
// exponent reference is then taken as 0 so no NaN can arise, and such a row
// ends with O = 0, LSE = -inf ("Triton: FlashAttention-2 Forward Pass", The
// rescale direction).
//
// Causal attention stops the key loop after the tile's last query row and
// applies the element mask only on tiles that straddle the diagonal or the
// end of the keys ("A09", section 3, Causal masking: skipping beats masking).
// The diagonal is shifted by coff: 0 aligns it top-left, nk - nq bottom-right
// ("How to profile and optimise kernels", Round 4, on non-square causal
// attention).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((vector_size(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

enum { DT_FP32 = 0, DT_FP16 = 1, DT_BF16 = 2 };

// The exponent reference of a row is moved only when the row max exceeds it
// by more than this many powers of two (so every p is at most 2^8).
constexpr float kRescaleSlack = 8.0f;

struct Params {
  const void *q, *k, *v;
  void *o;
  float *lse;          // may be null
  int64_t nq;          // query (and output) rows per head
  int64_t nk;          // key and value rows per head
  int64_t n_kv;        // keys j >= n_kv are masked (n_kv <= nk)
  int64_t coff;        // causal: query i sees keys j <= i + coff
  int nq_tiles;        // ceil(nq / BM)
  int xcd_remap;       // 1: map workgroups so that one XCD works on few heads
  float c;             // scale * log2(e)
  // split-KV partials (split kernels only): each workgroup covers a share of
  // its query tile's key tiles and writes a normalised fp32 O partial and its
  // LSE; a second kernel combines the splits
  int n_splits;        // 1 .. kMaxSplits
  int n_heads;         // B*H
  float *o_part;       // [n_splits][BH][nq][D]
  float *lse_part;     // [n_splits][BH][nq]
  // causal single pass: 1 = one workgroup per (head, pair of query tiles)
  int pair;
};

constexpr int kMaxSplits = 32;

// ---------------------------------------------------------------------------
// Element traits. 16-bit types use the 32x32x16 MFMA (8 elements per lane per
// operand); fp32 uses the 32x32x2 MFMA (1 element per lane per operand).

template <int DT> struct Elem;
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; static constexpr int k_step = 16; };
template <> struct Elem<DT_FP16> { static constexpr int bytes = 2; static constexpr int k_step = 16; };
template <> struct Elem<DT_FP32> { static constexpr int bytes = 4; static constexpr int k_step = 2; };

// ---------------------------------------------------------------------------
// Small device helpers

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  // Raw buffer resource: base address, stride 0, num_records = bytes, gfx9
  // data-format word. Reads at byte offsets >= bytes return 0.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// vmcnt(0): wait until this wave's outstanding vector-memory operations,
// including LDS-direct loads, have completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Direct global->LDS load of 16 bytes per lane: lane i's bytes land at
// lds_base + 16*i; reads at offsets beyond the resource's range return 0.
// Issued as inline asm so that the compiler does not treat the transfer as an
// outstanding LDS write that every later LDS read must wait for: the kernel
// orders these transfers itself (wait_vmem + barrier before a tile is read).
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, uint32_t voffset, uint32_t lds_base) {
  // the resource and the LDS base are wave-uniform; make that explicit so
  // they live in scalar registers as the instruction requires
  i32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  // the LDS base goes to m0 through an operand constraint, so the compiler
  // knows that m0 is written here
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(r), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}

__device__ __forceinline__ i32x4 make_rsrc_words(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)(uint32_t)(a >> 32);   // stride 0
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// Max over the two 32-lane halves: both halves end with the same value.
// The larger of two scores. IEEE 754-2019 maximum (NaN-propagating) rather
// than fmaxf (maxNum): the scores hold no NaN, so the two agree here, but
// fmaxf must quiet each operand the compiler cannot prove canonical (MFMA
// results, lane swaps) with an extra instruction, while gfx950 has
// v_maximum3_f32, which needs none.
__device__ __forceinline__ float score_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float halves_max(float x) {
  u32x2 r = __builtin_bit_cast(u32x2, __builtin_amdgcn_permlane32_swap(
      __float_as_uint(x), __float_as_uint(x), false, false));
  return score_max(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  u32x2 r = __builtin_bit_cast(u32x2, __builtin_amdgcn_permlane32_swap(
      __float_as_uint(x), __float_as_uint(x), false, false));
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 values rounded to nearest-even into one packed 16-bit pair
// (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float x0, float x1) {
  const f32x2 v = {x0, x1};
  if constexpr (DT == DT_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// LDS row swizzle: the 16-byte chunk c of tile row r is stored at chunk
// c ^ swz(r). Chosen so that (a) 16 consecutive rows read at the same chunk
// (K operand reads) fall in 16 different chunks, and (b) the 4-row x 64-byte
// blocks of the transposing V reads of one half-wave cover all 64 banks.
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int r) {
  if constexpr (ROW_BYTES >= 256) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// ---------------------------------------------------------------------------
// The kernel

template <int DT, int D, bool CAUSAL, int WAVES_ = 4>
struct Cfg {
  static constexpr int WAVES = WAVES_;      // 4 or 8 (two per SIMD with 8)
  static constexpr int BM = WAVES * 32;     // query rows per workgroup
  static constexpr int BN = 64;             // keys per tile
  static constexpr int ES = Elem<DT>::bytes;
  static constexpr int ROW_BYTES = D * ES;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;            // one K or V tile
  static constexpr int LDS_BYTES = 4 * TILE_BYTES;             // K,V x 2 buffers
  static constexpr int LOADS_PER_THREAD = TILE_BYTES / (WAVES * 64 * 16);
  static_assert(TILE_BYTES % (WAVES * 64 * 16) == 0, "tile must split into 16-byte lane loads");
};

// Register budget: two waves per SIMD (256 VGPRs) for 16-bit inputs, one wave
// per SIMD for fp32, whose Q fragments are twice as wide. With 8 waves the
// workgroup holds both waves of every SIMD and shares each K/V tile between
// 256 query rows, halving the global->LDS traffic per query row.
template <int DT, int D, bool CAUSAL, int WAVES = 4, bool SPLIT = false>
__global__ void __launch_bounds__(WAVES * 64, (DT == DT_FP32 ? 1 : 2)) fa_fwd_kernel(Params p) {
  static_assert(WAVES == 4 || (WAVES == 8 && DT != DT_FP32), "4 waves, or 8 for 16-bit inputs");
  using C = Cfg<DT, D, CAUSAL, WAVES>;
  constexpr int ES = C::ES, BN = C::BN, BM = C::BM, RB = C::ROW_BYTES;
  constexpr int KSTEP = Elem<DT>::k_step;
  constexpr int NKC = D / KSTEP;           // MFMAs along the head dim for S^T
  constexpr int NKB = BN / 32;             // 32-key blocks per tile
  constexpr int NDB = D / 32;              // 32-wide head-dim blocks of O^T
  constexpr int NPC = BN / KSTEP;          // MFMAs along the keys for O^T

  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // ---- which (head, query tile) this workgroup owns ----
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  if (p.xcd_remap && (nblk & 7) == 0) {
    // Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
    // contiguous range of (head, tile) pairs so the tiles of one head share
    // that XCD's L2.
    bid = (bid & 7) * (nblk >> 3) + (bid >> 3);
  }
  int rest = bid / p.nq_tiles;
  int qt = bid - rest * p.nq_tiles;
  int split = 0;
  if (SPLIT) {
    split = rest % p.n_splits;
    rest /= p.n_splits;
  }
  int bh = rest;
  if (CAUSAL) qt = p.nq_tiles - 1 - qt;    // longest causal tiles first
  // Causal, single pass, with p.pair: the grid has one workgroup per (head,
  // pair of query tiles) and each workgroup runs the long tile T-1-i, then
  // the short tile i, so every workgroup does the same T+1 tile-rows of work
  // (the middle tile of an odd T runs alone). Equal work per workgroup removes
  // the tail of unequal ones and spreads the short tiles' fixed costs; the
  // host pairs only grids that still fill the chip.
  int second_qt = -1;
  if (CAUSAL && !SPLIT && p.pair) {
    const int T = p.nq_tiles;
    const int npairs = (T + 1) / 2;
    const int nvalid = (int)gridDim.x;     // heads x pairs
    int c = blockIdx.x;
    if (p.xcd_remap && (nvalid & 7) == 0) c = (c & 7) * (nvalid >> 3) + (c >> 3);
    bh = c / npairs;
    const int pr = c - bh * npairs;
    qt = T - 1 - pr;
    second_qt = (pr != T - 1 - pr) ? pr : -1;
  }
  for (int job = 0; job < 2; ++job) {
  if (job == 1) {
    if (second_qt < 0) break;
    qt = second_qt;
    __syncthreads();                       // every wave is done with the first tile's LDS
  }
  // Query and key lengths are separate ("Triton: FlashAttention-2 Forward
  // Pass", Masks and sentinels): Q rows, the output and LSE use nq; the key
  // loop and the K/V rows use nk (and the key-length mask n_kv).
  const int64_t Nq = p.nq;
  const int q0 = qt * BM;
  const int qw = q0 + wave * 32;           // first query row of this wave
  const int my_q = qw + l32;               // the query row this lane owns
  const int coff = (int)p.coff;            // causal diagonal: key j visible when j <= i + coff

  const int64_t q_head = Nq * (int64_t)D;      // elements per head of Q and O
  const int64_t k_head = p.nk * (int64_t)D;    // elements per head of K and V
  const char *qh = (const char *)p.q + (int64_t)bh * q_head * ES;
  const char *kh = (const char *)p.k + (int64_t)bh * k_head * ES;
  const char *vh = (const char *)p.v + (int64_t)bh * k_head * ES;

  const int n_kv = (int)p.n_kv;
  int kend = n_kv;
  if (CAUSAL) kend = min(kend, q0 + BM + coff);
  const int n_tiles = kend > 0 ? (kend + BN - 1) / BN : 0;
  // key tiles [t_begin, t_end) of this workgroup: all of them, or this
  // split's even share of them (a split may be empty)
  int t_begin = 0, t_end = n_tiles;
  if (SPLIT) {
    t_begin = (int)(((int64_t)split * n_tiles) / p.n_splits);
    t_end = (int)(((int64_t)(split + 1) * n_tiles) / p.n_splits);
  }

  // ---- Q fragments (B operand of S^T = K Q^T), straight from global ----
  // lane (q = l32, half) holds Q[my_q][kc*KSTEP + half*KSTEP/2 ...]
  constexpr int QE = KSTEP / 2;             // elements per lane per fragment
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(qh, (uint32_t)(q_head * ES));
  const uint32_t smem_base = (uint32_t)reinterpret_cast<uintptr_t>(smem);

  // fragments stored as raw 32-bit words
  constexpr int QW = (QE * ES) / 4;          // 32-bit words per Q fragment
  uint32_t qf[NKC][QW];
  {
    const uint32_t row_off = (uint32_t)my_q * RB;
    const bool row_ok = my_q < Nq;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const uint32_t off = row_off + (uint32_t)((kc * KSTEP + half * QE) * ES);
      if constexpr (QW == 4) {
        u32x4 x = row_ok ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(q_rsrc, off, 0, 0))
                         : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < 4; ++w) qf[kc][w] = x[w];
      } else {
        qf[kc][0] = row_ok ? __builtin_amdgcn_raw_buffer_load_b32(q_rsrc, off, 0, 0) : 0u;
      }
    }
  }

  // Q is needed in every iteration: complete its loads here, so that no wait
  // for them is left inside the loop (where it would also wait for prefetches).
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- K/V tile staging: direct global->LDS loads into a swizzled layout ----
  // Each thread moves LOADS_PER_THREAD fixed 16-byte pieces of the K tile and
  // of the V tile. A piece's offset relative to the tile's first row does not
  // change from tile to tile, so per tile only the (scalar) buffer resource
  // moves: its base is the tile's first row and its range ends at key n_kv,
  // so rows past the keys read as zeros.
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

  // Lane offsets of the 16-bit MFMA operand fragments inside a tile. The
  // swizzle of a row depends only on its low 4 bits, so the fragment of key
  // block kb (K) or key chunk pc (V) is the offset of block 0 plus a
  // compile-time constant, and every LDS read is one register plus an
  // immediate offset.
  constexpr int NKO = (DT == DT_FP32) ? 1 : NKC;
  constexpr int NVO = (DT == DT_FP32) ? 1 : NDB;
  uint32_t k_off[NKO], v_off[2][NVO];
  const FA_LDS char *k_ptr[NKO];
  const FA_LDS char *v_ptr[2][NVO];
  if constexpr (DT != DT_FP32) {
    const int g = lane >> 4, r = (lane & 15) >> 2, cq = lane & 3;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) k_off[kc] = l32 * RB + (((kc * 2 + half) ^ swz<RB>(l32)) * 16);
#pragma unroll
    for (int jg = 0; jg < 2; ++jg)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        // V^T operand for lane (d = db*32 + l32, half): V[k0 + 0..3][d] and
        // V[k0 + 8 + 0..3][d], k0 = pc*16 + half*4, via the transposing read:
        // within each 16-lane group, lane 4*r + cq addresses row k + r,
        // head-dim columns 4*cq .. 4*cq+3 of the group's 16 columns.
        const int col = db * 32 + (g & 1) * 16 + cq * 4;
        const int key = jg * 8 + (g >> 1) * 4 + r;
        v_off[jg][db] = key * RB + ((((col * 2) / 16) ^ swz<RB>(key)) * 16) + (col * 2) % 16;
      }
    // LDS pointers formed once here. The empty asm hides the sum from the
    // compiler, which would otherwise add the (zero) base of the dynamic LDS
    // to each offset again inside the loop, once per fragment read group.
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

  // ---- running state ----
  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY;     // exponent reference (base-2 units), same in both halves
  float l_run = 0.f;           // this lane's partial row sum (its half's keys)
  // derived from m_run, updated only where it moves: the threshold past which
  // a score moves the reference, and the exponent offset (0 for a row that
  // has seen no visible key, whose scores are all -inf: p = 0)
  float thr = -INFINITY;
  float neg = 0.f;
  const float c = p.c;

  // one key tile; buf (0 or 1) is a compile-time constant so that every LDS
  // address is a register plus an immediate
  auto step = [&](int t, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    wait_vmem();
    __syncthreads();                        // tile t visible; the other buffer is free
    // the next tile's loads go out after this tile's S MFMAs have been issued,
    // so that they do not hold up the wave's first LDS reads and MFMAs
    auto prefetch = [&]() __attribute__((always_inline)) {
      if (t + 1 < t_end) issue_tile(t + 1, std::integral_constant<int, buf ^ 1>{});
    };

    const int kstart = t * BN;
    if (CAUSAL && kstart > qw + 31 + coff) {   // every key of this tile is in this wave's future
      prefetch();
      return;
    }

    const char *kl = smem + buf * (2 * C::TILE_BYTES);
    const char *vl = kl + C::TILE_BYTES;

    // ---- S^T = K Q^T : NKB blocks of 32 keys x 32 queries ----
    // head-dim chunks outer, key blocks inner, so consecutive MFMAs feed
    // independent accumulators. For 16-bit inputs all K fragments are read
    // up front so the MFMAs wait only for the first one.
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    if constexpr (DT == DT_FP32) {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int row = kb * 32 + l32;
          const int col = kc * 2 + half;                       // element
          const int ch = (col / 4) ^ swz<RB>(row);
          const float a = *(const FA_LDS float *)(kl + row * RB + ch * 16 + (col % 4) * 4);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, __uint_as_float(qf[kc][0]), s[kb], 0, 0, 0);
        }
    } else {
      // The K fragments stream through a window of KPIPE head-dim chunks:
      // chunk kc + KPIPE is requested before chunk kc's MFMAs are issued, so
      // each MFMA finds its operand already in registers. Scheduling fences
      // keep this order; left alone, the compiler sinks every read next to
      // its MFMA, and each pair of MFMAs then waits a full LDS round trip
      // unless the other wave of the SIMD has work to fill it.
      constexpr int KPIPE = NKC < 4 ? NKC : 4;
      u32x4 kf[NKC][NKB];
      auto read_k = [&](int kc) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          kf[kc][kb] = *(const FA_LDS u32x4 *)(k_ptr[kc] + buf * (2 * C::TILE_BYTES) + kb * 32 * RB);
      };
#pragma unroll
      for (int kc = 0; kc < KPIPE; ++kc) read_k(kc);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        if (kc + KPIPE < NKC) read_k(kc + KPIPE);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const u32x4 b = {qf[kc][0], qf[kc][1], qf[kc][2], qf[kc][3]};
          if constexpr (DT == DT_BF16)
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[kc][kb]), __builtin_bit_cast(bf16x8, b), s[kb], 0, 0, 0);
          else
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kf[kc][kb]), __builtin_bit_cast(f16x8, b), s[kb], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // V^T fragments for this tile's PV, read now so that they arrive while
    // the softmax runs (16-bit inputs)
    constexpr int NVF = (DT == DT_FP32) ? 1 : NPC;
    u32x4 vf[NVF][NVO];
    if constexpr (DT != DT_FP32) {
#pragma unroll
      for (int pc = 0; pc < NPC; ++pc)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int jg = 0; jg < 2; ++jg) {
            const FA_LDS char *addr = v_ptr[jg][db] + (buf * 2 + 1) * C::TILE_BYTES + pc * 16 * RB;
            const u32x2 xx = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4 *)addr));
            vf[pc][db][jg * 2] = xx[0];
            vf[pc][db][jg * 2 + 1] = xx[1];
          }
      __builtin_amdgcn_sched_barrier(0);
    }
    prefetch();

    // ---- masks: only on tiles past the end of the keys or on the diagonal ----
    const bool need_mask = (kstart + BN > n_kv) || (CAUSAL && kstart + BN - 1 > qw + coff);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kstart + kb * 32 + 8 * (i / 4) + half * 4 + (i % 4);
          const bool bad = (key >= n_kv) || (CAUSAL && key > my_q + coff);
          if (bad) s[kb][i] = -INFINITY;
        }
    }

    // ---- online softmax ----
    // m_run is the exponent reference shared by l and acc (base-2 units).
    // It moves to the running max only when some row of the wave has a new
    // max more than kRescaleSlack above it; until then the stale reference
    // is kept and p = exp2(s*c - m_run) stays below 2^kRescaleSlack. Any
    // common reference gives the same acc / l and m_run + log2 l ("A09",
    // section 3: rebasing multiplies every accumulated term by one common
    // factor), so this skips most accumulator rescales without changing the
    // result beyond rounding.
    // A row max (scaled by c > 0, which keeps order) exceeds the threshold
    // exactly when the maximum of one of its two lanes does, so the row max
    // over both lanes is formed only when some row moves.
    float lm = score_max(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = (kb == 0 ? 2 : 0); i < 16; ++i) lm = score_max(lm, s[kb][i]);
    if (__builtin_amdgcn_ballot_w64(lm * c > thr) != 0) {
      const float mx = halves_max(lm) * c;
      const float m_new = fmaxf(m_run, mx);
      // alpha = 0 on the first visible tile (m_run = -inf), 1 if unchanged
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
    // row sum in four interleaved partial sums (short dependency chains)
    float rs[4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c, neg));
        s[kb][i] = e;
        if (kb == 0 && i < 4) rs[i] = e;
        else rs[i % 4] += e;
      }
    l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);

    // ---- O^T += V^T P^T ----
    if constexpr (DT == DT_FP32) {
#pragma unroll
      for (int pc = 0; pc < NPC; ++pc) {
        const int kb = pc / 16, i = pc % 16;
        const int key = kb * 32 + 8 * (i / 4) + half * 4 + (i % 4);   // tile-local
        const float pv = s[kb][i];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int col = db * 32 + l32;
          const int ch = (col / 4) ^ swz<RB>(key);
          const float a = *(const FA_LDS float *)(vl + key * RB + ch * 16 + (col % 4) * 4);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pv, acc[db], 0, 0, 0);
        }
      }
    } else {
      // P^T chunk pc = 16 keys: this lane's values i = (pc%2)*8 .. +7 of block pc/2,
      // i.e. keys pc*16 + 8*(j/4) + half*4 + (j%4), j = 0..7, rounded to the input type.
#pragma unroll
      for (int pc = 0; pc < NPC; ++pc) {
        const int kb = pc / 2, i0 = (pc % 2) * 8;
        u32x4 b;
#pragma unroll
        for (int w = 0; w < 4; ++w) b[w] = pack2<DT>(s[kb][i0 + 2 * w], s[kb][i0 + 2 * w + 1]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4 a = vf[pc][db];
          if constexpr (DT == DT_BF16)
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc[db], 0, 0, 0);
          else
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc[db], 0, 0, 0);
        }
      }
    }
  };

  if (t_begin < t_end) issue_tile(t_begin, std::integral_constant<int, 0>{});
  for (int t = t_begin; t < t_end; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < t_end) step(t + 1, std::integral_constant<int, 1>{});
  }

  // ---- finalize: O = acc / l, LSE = (m + log2 l) ln 2 ----
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (SPLIT) {
    // this split's normalised partial in fp32 and its LSE (-inf if it saw no key)
    if (my_q < Nq) {
      const int64_t prow = ((int64_t)split * p.n_heads + bh) * Nq + my_q;
      float *orow = p.o_part + prow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d0 = db * 32 + 8 * gq + half * 4;
          *(float4 *)(orow + d0) = float4{acc[db][gq * 4 + 0] * inv, acc[db][gq * 4 + 1] * inv,
                                          acc[db][gq * 4 + 2] * inv, acc[db][gq * 4 + 3] * inv};
        }
      if (half == 0)
        p.lse_part[prow] = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
    return;
  }
  if (my_q < Nq) {
    char *orow = (char *)p.o + ((int64_t)bh * q_head + (int64_t)my_q * D) * ES;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = db * 32 + 8 * gq + half * 4;
        if constexpr (DT == DT_FP32) {
          float4 w = {acc[db][gq * 4 + 0] * inv, acc[db][gq * 4 + 1] * inv,
                      acc[db][gq * 4 + 2] * inv, acc[db][gq * 4 + 3] * inv};
          *(float4 *)(orow + d0 * 4) = w;
        } else {
          const uint32_t w0 = pack2<DT>(acc[db][gq * 4 + 0] * inv, acc[db][gq * 4 + 1] * inv);
          const uint32_t w1 = pack2<DT>(acc[db][gq * 4 + 2] * inv, acc[db][gq * 4 + 3] * inv);
          *(u32x2 *)(orow + d0 * 2) = u32x2{w0, w1};
        }
      }
    if (p.lse && half == 0) {
      const float lse = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : -INFINITY;
      p.lse[(int64_t)bh * Nq + my_q] = lse;
    }
  }
  }   // job
}

}  // namespace fa
