// C[M, N] = A[M, K] W[N, K]^T on bf16 MFMA (16x16x32, f32 accumulate), with the stage's epilogues.
// A is an activation plane buffer (bf16 hi + lo, or hi + mid + lo for the QKV projection); every W
// tile meets every plane, so the product keeps the activations' ~16 (~24) significant bits.
//
// Prefill projections (M = T tokens) and batched decode (M = B rows) both land here.  Both
// operands are K-contiguous, the layout the MFMA operands want: lane l takes 8 consecutive k of
// row l%16.  A work-group of 4 waves owns a BM x BN tile; BK = 64 slices of A and W are staged
// global -> registers -> LDS (16-byte chunks XOR-swizzled by row so the ds_read_b128 of 16 rows
// hits distinct banks), the next slices' loads in flight while the current slice feeds the MFMAs.
// STAGES = LDS buffers (1: a barrier separates the last reads from the next store), DEPTH =
// register staging sets (loads issued DEPTH slices ahead).
// Small tile counts (skinny decode GEMMs) split K: every split writes an f32 partial and a second
// kernel sums them in split order -- a fixed order, so results never depend on timing -- and
// applies the epilogue.
#include "kernels.h"
#include "norm.h"

namespace {

constexpr int BK = 64;
constexpr int kGroupM = 8;   // M-tiles per group of the tile order

// Tile order.  Work-groups are dealt to the 8 XCDs round-robin (block i runs on XCD i % 8), and
// each XCD has its own L2; so block i first maps to the logical index that gives every XCD one
// contiguous range of logical tiles.  Logical tiles then walk groups of kGroupM M-tiles, column by
// column, so a group's A panels and each W panel are reused from L2 instead of HBM.
PSD_DEV void tile_coords(int block, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn) {
  int logical = block;
  if (nblocks % 8 == 0) logical = (block % 8) * (nblocks / 8) + block / 8;
  const int per_group = kGroupM * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = logical - group * per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// Store a wave's accumulators acc[i][j] (rows r0 + i*16 .., columns c0 + j*16 ..; MFMA C layout):
// the split's f32 partial when K is split, else the epilogue.  Column pairs (c, c + 16) with
// c % 32 < 16 meet in one lane for the SwiGLU and RoPE epilogues.
template <int TM, int TN, int WTM, int WTN, int EPI>
PSD_DEV void gemm_store(const GemmArgs& g, const f32x4_t (&acc)[TM][TN], int r0, int c0, int lane, int split) {
  const int M = g.M, N = g.N;
  // ---- split-K: write this split's partial; k_splitk_reduce sums them in split order ------------
  if (g.splitk > 1) {
    float* part = g.part + (size_t)split * M * N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = r0 + i * 16 + (lane >> 4) * 4 + jj;
          const int c = c0 + j * 16 + (lane & 15);
          if (r < M && c < N) part[(size_t)r * N + c] = acc[i][j][jj];
        }
    return;
  }

  // ---- epilogue ----------------------------------------------------------------------------------
  const EpiArgs& e = g.e;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = r0 + i * 16 + (lane >> 4) * 4 + jj;
      if (r >= M) continue;
      if (EPI == EPI_F32 || EPI == EPI_RESID) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int c = c0 + j * 16 + (lane & 15);
          if (c >= N) continue;
          float v = acc[i][j][jj];
          if (EPI == EPI_RESID) v += e.resid[(size_t)r * e.ldo + c];
          e.out[(size_t)r * e.ldo + c] = v;
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; j += 2) {
          const int c = c0 + j * 16 + (lane & 15);   // c % 32 < 16, partner c + 16
          if (c >= N) continue;
          const float x0 = acc[i][j][jj], x1 = acc[i][j + 1][jj];
          if (EPI == EPI_SWIGLU) {
            store_pair(e.act, e.act_ps, (size_t)r * e.ldo + (c >> 5) * 16 + (c & 15), silu_mul(x0, x1));
          } else {
            int slot, pos;
            if (!row_slot_pos(e, r, slot, pos)) {
              if (c + e.col_off == 0) atomicAdd(e.err, 1u);
            } else {
              qkv_epilogue_pair(e, r, c, x0, x1);
            }
          }
        }
      }
    }
}

template <int BM, int BN, int WM, int WN, int NP, int EPI, int STAGES, int DEPTH>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  static_assert(DEPTH == 1 || DEPTH == 2, "register staging sets");
  static_assert(WM * WN == 4, "4 waves");
  static_assert(STAGES == 1 || STAGES == 2, "LDS buffers");
  constexpr int WTM = BM / WM, WTN = BN / WN;       // wave tile
  constexpr int TM = WTM / 16, TN = WTN / 16;       // MFMA tiles per wave
  static_assert(WTN % 32 == 0, "paired epilogues need 32-aligned wave columns");
  constexpr int A_ITERS = (BM * 8 + 255) / 256, B_ITERS = (BN * 8 + 255) / 256;
  __shared__ uint4 As[STAGES][NP][BM * 8];  // [buffer][plane][row * 8 + swizzled chunk]
  __shared__ uint4 Bs[STAGES][BN * 8];

  const int M = g.M, N = g.N, K = g.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  const int tile = blockIdx.x;
  int tm, tn;
  tile_coords(tile, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int split = blockIdx.y;
  const int kper = ((K + g.splitk - 1) / g.splitk + BK - 1) / BK * BK;
  const int kbeg = split * kper;
  const int kend = min(K, kbeg + kper);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  // Global -> register staging, two sets: the loads of step it + 2 are issued while step it is
  // computed, so each load has two steps of MFMA work to arrive.  Rows past M / N are clamped to
  // the last row (their results are never stored) and k past the split's end reads as zero, so
  // every load is unconditional and in bounds.
  typedef uint4 ASet[NP][A_ITERS];
  typedef uint4 BSet[B_ITERS];
  ASet ra0, ra1;
  BSet rb0, rb1;
  auto gload = [&](ASet& ra, BSet& rb, int k0) {
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
      const int q = tid + i * 256, row = (q >> 3) % BM, c8 = q & 7;
      const int gm = min(m0 + row, M - 1), gk = k0 + c8 * 8;
      const bool ok = gk < kend;
      const uint16_t* src = g.a + (size_t)gm * K + (ok ? gk : kbeg);
#pragma unroll
      for (int pl = 0; pl < NP; ++pl) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + pl * g.a_ps);
        ra[pl][i] = ok ? v : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
      const int q = tid + i * 256, row = (q >> 3) % BN, c8 = q & 7;
      const int gn = min(n0 + row, N - 1), gk = k0 + c8 * 8;
      const bool ok = gk < kend;
      const uint4 v = *reinterpret_cast<const uint4*>(g.w + (size_t)gn * K + (ok ? gk : kbeg));
      rb[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf, const ASet& ra, const BSet& rb) {
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
      const int q = tid + i * 256, row = q >> 3, c8 = q & 7;
      if (q < BM * 8) {
#pragma unroll
        for (int pl = 0; pl < NP; ++pl) As[buf][pl][row * 8 + (c8 ^ (row & 7))] = ra[pl][i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
      const int q = tid + i * 256, row = q >> 3, c8 = q & 7;
      if (q < BN * 8) Bs[buf][row * 8 + (c8 ^ (row & 7))] = rb[i];
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int cur) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c8 = kk * 4 + (lane >> 4);
      bf16x8_t af[NP][TM], bw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WTM + i * 16 + (lane & 15);
#pragma unroll
        for (int pl = 0; pl < NP; ++pl) af[pl][i] = as_bf16x8(As[cur][pl][row * 8 + (c8 ^ (row & 7))]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WTN + j * 16 + (lane & 15);
        bw[j] = as_bf16x8(Bs[cur][row * 8 + (c8 ^ (row & 7))]);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) acc[i][j] = mfma16(af[pl][i], bw[j], acc[i][j]);
        }
    }
  };

  if (DEPTH == 1) {
    // one staging set: step it + 1's loads are issued while step it is computed
    if (nk > 0) {
      gload(ra0, rb0, kbeg);
      sstore(0, ra0, rb0);
      __syncthreads();
    }
    for (int it = 0; it < nk; ++it) {
      const int cur = STAGES == 2 ? (it & 1) : 0;
      if (it + 1 < nk) gload(ra0, rb0, kbeg + (it + 1) * BK);
      compute(cur);
      if (STAGES == 1) __syncthreads();
      if (it + 1 < nk) sstore(STAGES == 2 ? cur ^ 1 : 0, ra0, rb0);
      __syncthreads();
    }
  } else {
  if (nk > 0) {
    gload(ra0, rb0, kbeg);
    if (nk > 1) gload(ra1, rb1, kbeg + BK);
    sstore(0, ra0, rb0);
    __syncthreads();
  }
  // step it computes LDS buffer it & 1 (buffer 0 with one buffer); register set it & 1 is free
  // (stored during step it - 1) and receives step it + 2; set (it + 1) & 1 holds step it + 1 and goes
  // to LDS after the MFMAs -- with one LDS buffer, after a barrier that ends every wave's reads
  constexpr int B1 = STAGES == 2 ? 1 : 0;
  for (int it = 0; it < nk; it += 2) {
    if (it + 2 < nk) gload(ra0, rb0, kbeg + (it + 2) * BK);
    compute(0);
    if (STAGES == 1) __syncthreads();
    if (it + 1 < nk) sstore(B1, ra1, rb1);
    __syncthreads();
    if (it + 1 >= nk) break;
    if (it + 3 < nk) gload(ra1, rb1, kbeg + (it + 3) * BK);
    compute(B1);
    if (STAGES == 1) __syncthreads();
    if (it + 2 < nk) sstore(0, ra0, rb0);
    __syncthreads();
  }
  }

  gemm_store<TM, TN, WTM, WTN, EPI>(g, acc, m0 + wm * WTM, n0 + wn * WTN, lane, split);
}

// ------------------------------------------------------------------------------------------------
// LDS-direct tiles.  When K is a multiple of 64 (every benchmarked projection) 8 waves own a
// 128 x 256 tile, each wave 32 x 128 (two waves per SIMD), K in 64-deep stages so that every row
// segment a load instruction fetches is a whole 128-byte line: two activation-plane buffers and
// three weight buffers (STB = 3) for two planes, two of each for three; the batched decode at
// M <= 64 takes 64 x 128 tiles.  Otherwise 32-deep stages in a ring of ST buffers, on 256 x 256
// tiles (waves of 64 x 128) or 128 x 256, with the ping-pong schedule (PP) on grids of several
// rounds.  Tiles go from global memory straight into LDS (global_load_lds_dwordx4), so no registers
// stage them and no ds_write is issued: the accumulators, one step's fragments and the addresses
// fit the 256 registers of two waves per SIMD.  ST LDS buffers form a ring: while stage t feeds the
// MFMAs the loads of stages t + 1 .. t + ST - 2 are in flight, and stage t + ST - 1 is issued into
// the buffer stage t - 1 has just left.
// Rows of a stage are BK / 8 chunks of 16 bytes, XOR-swizzled by row (dma_swz) so that the 8 rows
// one ds_read_b128 phase reads land in distinct banks.  One load instruction writes 64 consecutive
// chunks -- lane l's 16 bytes at position l -- so the swizzle is applied on the global side: lane
// l fetches the chunk that belongs at position l.
// The loads are issued from inline assembly and waited for by hand: each wave waits (vmcnt) for
// its own loads of stage t before the barrier that hands the stage to the other waves.  (Through
// the compiler builtin, every LDS read would also wait for the loads still in flight.)  The
// kernel uses no other instruction that reads M0.
// Per 32-k step each accumulator takes the hi-plane product and then the lo-plane product(s), the
// same sequence as k_gemm, so both kernels give identical sums.
// PP (ping-pong, 8 waves, 32-deep stages): the waves on one SIMD are split into two groups that
// run half a step apart, with two barriers per step; while one group reads its fragments and
// issues its loads, the other issues its MFMAs, so the matrix core takes both waves' products
// back to back instead of both waves reading LDS at once after one barrier.  The same products
// in the same order: identical sums.
// ------------------------------------------------------------------------------------------------
constexpr int kDmaBK = 32;

// 16 bytes per lane from global memory (wave-uniform base + the lane's byte offset) into LDS at
// lds_wave_base + 16 * lane (wave-uniform)
PSD_DEV void dma16(const uint16_t* base, uint32_t lane_off, uint32_t lds_wave_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(lane_off), "s"(base), "s"(lds_wave_base)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// the same load, non-temporal: for weights that no other work-group reads (a single row of
// M-tiles), streamed past the caches
PSD_DEV void dma16_nt(const uint16_t* base, uint32_t lane_off, uint32_t lds_wave_base) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(lane_off), "s"(base), "s"(lds_wave_base)
               : "memory", "m0");
#pragma clang diagnostic pop
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8)
template <int n>
PSD_DEV void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
}

// workgroup barrier that the compiler may not move memory accesses across
PSD_DEV void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Position of logical 16-byte chunk c of stage row r: rows of 4 chunks (BK = 32) XOR (r >> 1) & 3,
// rows of 8 chunks (BK = 64) XOR r & 7 -- either way the 8 rows one ds_read_b128 phase reads land in
// distinct banks.
template <int CH>
PSD_DEV int dma_swz(int r, int c) {
  return CH == 4 ? c ^ ((r >> 1) & 3) : c ^ (r & 7);
}

template <int NP, int EPI, int BM, int BN, int WM, int WN, int ST, int BK = kDmaBK, bool PP = false, int STB = 0>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm_dma(GemmArgs g) {
  constexpr int NT = WM * WN * 64;
  // weight (B) stages in LDS: ST like the activations, or STB > ST with the activations double-
  // buffered, so that the weight stream runs STB - 2 stages ahead of the activation stream
  constexpr int SB = STB > 0 ? STB : ST;
  static_assert(SB == ST || (ST == 2 && SB >= 3 && !PP), "deeper weight ring: two activation buffers");
  static_assert(BK == 32 || BK == 64, "stage depth");
  constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 16, TN = WTN / 16;
  static_assert(WTN % 32 == 0, "paired epilogues need 32-aligned wave columns");
  constexpr int CH = BK / 8;                               // chunks per row
  constexpr int A_DMA = BM * CH / NT, B_DMA = BN * CH / NT;     // load instructions per thread
  static_assert(A_DMA * NT == BM * CH && B_DMA * NT == BN * CH, "whole load instructions");
  constexpr int PER_STAGE = NP * A_DMA + B_DMA;
  static_assert(ST >= 2 && ST <= 8 && (ST - 2) * PER_STAGE < 64, "ring depth within vmcnt");
  __shared__ uint4 As[ST][NP][BM * CH];
  __shared__ uint4 Bs[SB][BN * CH];

  const int M = g.M, N = g.N, K = g.K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int split = blockIdx.y;
  const int kper = ((K + g.splitk - 1) / g.splitk + BK - 1) / BK * BK;
  const int kbeg = split * kper;
  const int kend = min(K, kbeg + kper);
  const int nk = kend > kbeg ? (kend - kbeg) / BK : 0;    // K and the split ranges are multiples of BK

  // lane's source of load instruction i: row (64 / CH) * (wave * n + i) + lane / CH (past M / N: the
  // last row, never stored), the logical chunk stored at position lane % CH; a byte offset from the
  // operand's column kbeg (A and W are under 4 GiB)
  auto src_off = [&](int row0, int rows_max, int i, int n) {
    const int row = (wave * n + i) * (64 / CH) + lane / CH;
    const int c = dma_swz<CH>(row, lane % CH);
    return (uint32_t)(((size_t)min(row0 + row, rows_max - 1) * K + c * 8) * 2);
  };
  uint32_t a_off[A_DMA], b_off[B_DMA];
#pragma unroll
  for (int i = 0; i < A_DMA; ++i) a_off[i] = src_off(m0, M, i, A_DMA);
#pragma unroll
  for (int i = 0; i < B_DMA; ++i) b_off[i] = src_off(n0, N, i, B_DMA);
  // LDS byte addresses of this wave's destination blocks in stage buffer 0 (wave-uniform)
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t a_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&As[0][0][0] +
                         (uint32_t)(wave_s * A_DMA * 64 * 16);
  const uint32_t b_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)&Bs[0][0] +
                         (uint32_t)(wave_s * B_DMA * 64 * 16);

  auto issue_a = [&](int t) {   // activation stage t -> buffer t % ST
    const int buf = t % ST;
    const size_t k0 = (size_t)kbeg + (size_t)t * BK;
#pragma unroll
    for (int pl = 0; pl < NP; ++pl)
#pragma unroll
      for (int i = 0; i < A_DMA; ++i)
        dma16(g.a + pl * g.a_ps + k0, a_off[i], a_lds + (uint32_t)((buf * NP + pl) * BM * CH * 16 + i * 64 * 16));
  };
  const bool w_nt = g.w_stream != 0;
  auto issue_b = [&](int t) {   // weight stage t -> buffer t % SB
    const int buf = t % SB;
    const size_t k0 = (size_t)kbeg + (size_t)t * BK;
    if (w_nt) {
#pragma unroll
      for (int i = 0; i < B_DMA; ++i)
        dma16_nt(g.w + k0, b_off[i], b_lds + (uint32_t)(buf * BN * CH * 16 + i * 64 * 16));
    } else {
#pragma unroll
      for (int i = 0; i < B_DMA; ++i) dma16(g.w + k0, b_off[i], b_lds + (uint32_t)(buf * BN * CH * 16 + i * 64 * 16));
    }
  };
  auto issue = [&](int t) {
    issue_a(t);
    issue_b(t);
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int kc = lane >> 4;   // logical k chunk of this lane's MFMA operands
  // s_waitcnt vmcnt(n * PER_STAGE) for n = 0 .. ST - 2 later stages left in flight
  auto wait_stages = [&](int n) {
    switch (n) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<PER_STAGE>(); break;
      case 2: wait_vmcnt<(ST > 3 ? 2 : 1) * PER_STAGE>(); break;
      case 3: wait_vmcnt<(ST > 4 ? 3 : 1) * PER_STAGE>(); break;
      case 4: wait_vmcnt<(ST > 5 ? 4 : 1) * PER_STAGE>(); break;
      case 5: wait_vmcnt<(ST > 6 ? 5 : 1) * PER_STAGE>(); break;
      default: wait_vmcnt<(ST > 7 ? 6 : 1) * PER_STAGE>(); break;
    }
  };

  if constexpr (SB != ST) {
    // Issue order: B0 .. B(SB-3), then per stage j the pair A(j), B(j + SB - 2).  When stage t is
    // consumed, the only loads issued after A(t) are those of B(t + SB - 2), so waiting for all but
    // B_DMA loads lands both A(t) and B(t).  Iteration t refills the buffers of stage t - 1.
    for (int j = 0; j < SB - 2; ++j)
      if (j < nk) issue_b(j);
    if (nk > 0) issue_a(0);
    if (SB - 2 < nk) issue_b(SB - 2);
    for (int t = 0; t < nk; ++t) {
      if (t + SB - 2 < nk) wait_vmcnt<B_DMA>();
      else wait_vmcnt<0>();
      lds_barrier();
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        const int ch = ks * 4 + kc;
        bf16x8_t af[NP][TM], bw[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = wm * WTM + i * 16 + (lane & 15);
#pragma unroll
          for (int pl = 0; pl < NP; ++pl) af[pl][i] = as_bf16x8(As[t % ST][pl][row * CH + dma_swz<CH>(row, ch)]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int row = wn * WTN + j * 16 + (lane & 15);
          bw[j] = as_bf16x8(Bs[t % SB][row * CH + dma_swz<CH>(row, ch)]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pl = 0; pl < NP; ++pl) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(af[pl][i], bw[j], acc[i][j]);
          if (pl == 0 && ks == 0) {
            __builtin_amdgcn_sched_barrier(0);
            if (t + 1 < nk) issue_a(t + 1);
            if (t + SB - 1 < nk) issue_b(t + SB - 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
  } else {
#pragma unroll
  for (int t = 0; t < ST - 1; ++t)
    if (t < nk) issue(t);
  if constexpr (PP) {
    static_assert(BK == 32 && WM * WN == 8, "ping-pong: 32-deep stages, two waves per SIMD");
    bf16x8_t af[NP][TM], bw[TN];
    auto read_frags = [&](int t) {   // this wave's fragments of stage t, landed in registers
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WTM + i * 16 + (lane & 15);
#pragma unroll
        for (int pl = 0; pl < NP; ++pl) af[pl][i] = as_bf16x8(As[t % ST][pl][row * CH + dma_swz<CH>(row, kc)]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WTN + j * 16 + (lane & 15);
        bw[j] = as_bf16x8(Bs[t % ST][row * CH + dma_swz<CH>(row, kc)]);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
    };
    auto products = [&]() {   // at raised issue priority, so the other wave's reads do not delay them
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int pl = 0; pl < NP; ++pl)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(af[pl][i], bw[j], acc[i][j]);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    };
    // Waves 0-3 and 4-7 (one of each per SIMD) run half a step apart: between two barriers one
    // group reads its fragments from LDS while the other issues its MFMAs, so each SIMD's matrix
    // core takes the two waves' products back to back.  Barrier 2t: every wave's loads of stage t
    // have landed and every read of stage t - 1 has completed (its buffer takes stage t + ST - 1).
    if (wave_s < 4) {   // wave-uniform branch: both sides take 2 nk + 1 barriers
      for (int t = 0; t < nk; ++t) {
        wait_stages(min(ST - 2, nk - 1 - t));
        lds_barrier();
        if (t + ST - 1 < nk) issue(t + ST - 1);
        read_frags(t);
        lds_barrier();
        products();
      }
      lds_barrier();
    } else {
      for (int t = 0; t < nk; ++t) {
        wait_stages(min(ST - 2, nk - 1 - t));
        lds_barrier();
        if (t + ST - 1 < nk) issue(t + ST - 1);
        if (t > 0) products();
        lds_barrier();
        read_frags(t);
      }
      lds_barrier();
      if (nk > 0) products();
    }
  } else
  for (int t = 0; t < nk; ++t) {
    // stage t's own loads done (later stages' may stay in flight); after the barrier every wave's
    // loads of stage t are in LDS and no wave still reads stage t - 1's buffer
    wait_stages(min(ST - 2, nk - 1 - t));
    lds_barrier();
    // per 32-k step: all of this wave's fragment reads, then the hi-plane MFMAs, (in the first
    // step) the loads of stage t + ST - 1 into the freed buffer, and the MFMAs of the other planes
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int ch = ks * 4 + kc;
      bf16x8_t af[NP][TM], bw[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WTM + i * 16 + (lane & 15);
#pragma unroll
        for (int pl = 0; pl < NP; ++pl) af[pl][i] = as_bf16x8(As[t % ST][pl][row * CH + dma_swz<CH>(row, ch)]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wn * WTN + j * 16 + (lane & 15);
        bw[j] = as_bf16x8(Bs[t % ST][row * CH + dma_swz<CH>(row, ch)]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int pl = 0; pl < NP; ++pl) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(af[pl][i], bw[j], acc[i][j]);
        if (pl == 0 && ks == 0) {
          __builtin_amdgcn_sched_barrier(0);
          if (t + ST - 1 < nk) issue(t + ST - 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  }

  gemm_store<TM, TN, WTM, WTN, EPI>(g, acc, m0 + wm * WTM, n0 + wn * WTN, lane, split);
}

// Sum the split-K partials of column pairs (c, c + 16), c % 32 < 16, in split order and apply the
// epilogue.  A separate launch: combining partials inside the GEMM would need device-scope
// release/acquire fences, which on gfx950 write back and invalidate the XCD's L2 per work-group.
template <int EPI>
__global__ __launch_bounds__(256) void k_splitk_reduce(GemmArgs g) {
  const int M = g.M, N = g.N;
  if constexpr (EPI == EPI_QKV) {
    // two adjacent pairs per thread, (c0, c0 + 16) and (c0 + 1, c0 + 17) with c0 even: 8-byte
    // partial loads (the fused QKV width is a multiple of 32), each element summed in split order
    const int quads_per_row = N >> 2;
    const size_t total = (size_t)M * quads_per_row, plane = (size_t)M * N;
    const EpiArgs& e = g.e;
    for (size_t t = (size_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (size_t)gridDim.x * 256) {
      const int r = (int)(t / quads_per_row), pp = 2 * (int)(t - (size_t)r * quads_per_row);
      const int c0 = ((pp >> 4) << 5) + (pp & 15);
      float2 x0 = make_float2(0.0f, 0.0f), x1 = make_float2(0.0f, 0.0f);
      for (int sp = 0; sp < g.splitk; ++sp) {
        const float* p = g.part + sp * plane + (size_t)r * N;
        const float2 a = *reinterpret_cast<const float2*>(p + c0);
        const float2 b = *reinterpret_cast<const float2*>(p + c0 + 16);
        x0.x += a.x;
        x0.y += a.y;
        x1.x += b.x;
        x1.y += b.y;
      }
      int slot, pos;
      const int s0 = c0 + e.col_off;   // stored row of the fused weight
      if (!row_slot_pos(e, r, slot, pos)) {
        if (s0 == 0) atomicAdd(e.err, 1u);
      } else {
        qkv_store_pair(e, r, slot, pos, s0, x0.x, x1.x, qkv_rope_cs(e, pos, s0));
        qkv_store_pair(e, r, slot, pos, s0 + 1, x0.y, x1.y, qkv_rope_cs(e, pos, s0 + 1));
      }
    }
    return;
  }
  const int pairs_per_row = ((N + 31) >> 5) << 4;
  const size_t total = (size_t)M * pairs_per_row;
  const size_t plane = (size_t)M * N;
  for (size_t t = (size_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (size_t)gridDim.x * 256) {
    const int r = (int)(t / pairs_per_row), pp = (int)(t - (size_t)r * pairs_per_row);
    const int c0 = ((pp >> 4) << 5) + (pp & 15), c1 = c0 + 16;
    const bool v0 = c0 < N, v1 = c1 < N;
    float x0 = 0.0f, x1 = 0.0f;
    for (int sp = 0; sp < g.splitk; ++sp) {
      const float* p = g.part + sp * plane + (size_t)r * N;
      if (v0) x0 += p[c0];
      if (v1) x1 += p[c1];
    }
    const EpiArgs& e = g.e;
    if (EPI == EPI_F32 || EPI == EPI_RESID) {
      if (v0) e.out[(size_t)r * e.ldo + c0] = (EPI == EPI_RESID ? e.resid[(size_t)r * e.ldo + c0] : 0.0f) + x0;
      if (v1) e.out[(size_t)r * e.ldo + c1] = (EPI == EPI_RESID ? e.resid[(size_t)r * e.ldo + c1] : 0.0f) + x1;
    } else if (v1) {
      if (EPI == EPI_SWIGLU) {
        store_pair(e.act, e.act_ps, (size_t)r * e.ldo + (c0 >> 5) * 16 + (c0 & 15), silu_mul(x0, x1));
      } else {
        int slot, pos;
        if (!row_slot_pos(e, r, slot, pos)) {
          if (c0 + e.col_off == 0) atomicAdd(e.err, 1u);
        } else {
          qkv_epilogue_pair(e, r, c0, x0, x1);
        }
      }
    }
  }
}

// Split-K sum with the residual epilogue, fused with the RMSNorm of the result (the operand of
// the next projection): one work-group per row.  x = ((0 + p0) + p1) + ..., out = resid + x, as
// k_splitk_reduce; then the row's RMS scale and the normalised bf16 planes exactly as k_rmsnorm
// computes them from out (same element order, same f64 reduction).  N % 4 == 0, N <= 8192.
constexpr int kReduceNormMaxN = 8192;

// PER float4 per thread (rows of up to 1024 PER).  With PER = 4 the residual row and the gain are
// loaded before the partials so that all loads are in flight together; at PER = 8 the extra
// registers would leave one wave per SIMD, so they are loaded after the sum.
template <int PER>
__global__ __launch_bounds__(256) void k_splitk_reduce_norm(GemmArgs g, NormArgs nrm) {
  constexpr bool kEarly = PER <= 4;
  constexpr int SB = 4;                          // splits whose loads are in flight together
  __shared__ double red[4];
  const int r = blockIdx.x, N = g.N;
  const size_t plane = (size_t)g.M * N;
  const EpiArgs& e = g.e;
  // the residual row and the gain (first when kEarly, so that their loads are in flight with the
  // partials'; out may be resid itself: each thread reads its own elements before it writes them)
  float4 res[PER], gn[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x * 4 + j * 1024;
    res[j] = gn[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (kEarly && i < N) {
      res[j] = *(const float4*)(e.resid + (size_t)r * e.ldo + i);
      gn[j] = *(const float4*)(nrm.gain + i);
    }
  }
  // the row's split partials, SB splits per round trip (a few rows only fill few CUs, so each
  // work-group needs its loads in flight at once); summed per element in split order
  float4 x[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) x[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp0 = 0; sp0 < g.splitk; sp0 += SB) {
    float4 p[SB][PER];
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = threadIdx.x * 4 + j * 1024;
        p[u][j] = (sp0 + u < g.splitk && i < N) ? *(const float4*)(g.part + (sp0 + u) * plane + (size_t)r * N + i)
                                                : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int u = 0; u < SB; ++u)
      if (sp0 + u < g.splitk) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          x[j].x += p[u][j].x;
          x[j].y += p[u][j].y;
          x[j].z += p[u][j].z;
          x[j].w += p[u][j].w;
        }
      }
  }
  float4 v[PER];
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x * 4 + j * 1024;
    if (i < N) {
      if (!kEarly) res[j] = *(const float4*)(e.resid + (size_t)r * e.ldo + i);
      v[j] = make_float4(res[j].x + x[j].x, res[j].y + x[j].y, res[j].z + x[j].z, res[j].w + x[j].w);
      *(float4*)(e.out + (size_t)r * e.ldo + i) = v[j];
      ss = sumsq4(v[j], ss);
    }
  }
  const double rs = block_rms_finish(ss, N, nrm.eps, red);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x * 4 + j * 1024;
    if (i < N)
      store_norm_planes4(nrm.out_pair + (size_t)r * N + i, nrm.pair_ps, v[j], rs,
                         kEarly ? gn[j] : *(const float4*)(nrm.gain + i));
  }
}

// The same sum and norm for a few rows (batched decode): 1024 threads per row, each owning PER
// float4 columns (i = 4 t + 4096 j), so that every split's partials of the row, its residual and
// its gains are in flight in one round trip (up to 8 splits).  The summed row goes to LDS and
// threads 0..255 take its sum of squares over exactly the elements, order and wave combination of
// block_rms_scale (thread t: i = 4 t + 1024 j, j ascending; waves 0..3), so the RMS scale -- and
// every output bit -- equals k_rmsnorm's and the 256-thread kernel's.
template <int PER>
__global__ __launch_bounds__(1024) void k_splitk_reduce_norm_w(GemmArgs g, NormArgs nrm) {
  constexpr int SB = 8;
  __shared__ double red[16];
  __shared__ float4 vrow[kReduceNormMaxN / 4];
  const int r = blockIdx.x, N = g.N;
  const size_t plane = (size_t)g.M * N;
  const EpiArgs& e = g.e;
  float4 res[PER], gn[PER], x[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x * 4 + j * 4096;
    res[j] = gn[j] = x[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < N) {
      res[j] = *(const float4*)(e.resid + (size_t)r * e.ldo + i);
      gn[j] = *(const float4*)(nrm.gain + i);
    }
  }
  for (int sp0 = 0; sp0 < g.splitk; sp0 += SB) {
    float4 p[SB][PER];
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = threadIdx.x * 4 + j * 4096;
        p[u][j] = (sp0 + u < g.splitk && i < N) ? *(const float4*)(g.part + (sp0 + u) * plane + (size_t)r * N + i)
                                                : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int u = 0; u < SB; ++u)
      if (sp0 + u < g.splitk) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          x[j].x += p[u][j].x;
          x[j].y += p[u][j].y;
          x[j].z += p[u][j].z;
          x[j].w += p[u][j].w;
        }
      }
  }
  float4 v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x * 4 + j * 4096;
    if (i < N) {
      v[j] = make_float4(res[j].x + x[j].x, res[j].y + x[j].y, res[j].z + x[j].z, res[j].w + x[j].w);
      *(float4*)(e.out + (size_t)r * e.ldo + i) = v[j];
      vrow[i / 4] = v[j];
    }
  }
  __syncthreads();
  double ss = 0.0;
  if (threadIdx.x < 256)
    for (int i = threadIdx.x * 4; i < N; i += 1024) ss = sumsq4(vrow[i / 4], ss);
  const double rs = block_rms_finish(ss, N, nrm.eps, red);   // waves 4..15 add nothing it reads
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x * 4 + j * 4096;
    if (i < N) store_norm_planes4(nrm.out_pair + (size_t)r * N + i, nrm.pair_ps, v[j], rs, gn[j]);
  }
}

struct Cfg {
  int bm, bn;
};
// cfg 8 (a 64 x 256 batched-decode tile) is no longer planned; its slot keeps the numbering
constexpr Cfg kCfgs[] = {{128, 128}, {64, 256}, {64, 128}, {32, 128}, {16, 128}, {256, 256}, {128, 256}, {128, 256}, {64, 256}, {64, 128}, {128, 256}, {128, 256}};

}  // namespace

// K splits of a batched-decode projection: its tiles take one work-group per CU (the LDS-direct
// tiles hold 128-160 KB), so the most splits that keep the grid within one round of 256
// work-groups, each split at least 512 deep (any count: the split-K sum runs in split order)
static int decode_splits(int tiles, int K) {
  if (tiles >= 190) return 1;
  int sk = 256 / tiles;
  if (sk > 16) sk = 16;
  while (sk > 1 && K / sk < 512) --sk;
  return sk;
}

GemmPlan gemm_plan(int M, int N, int K, int planes, bool qkv) {
  // Tile shapes from sweeps on MI355X over the prefill and batched-decode projections.
  //  * M >= 256 with K a multiple of 64: 128 x 256 LDS-direct tiles with 64-deep stages in two
  //    LDS buffers (two or three activation planes; three planes fill exactly 160 KB), K split
  //    until the grid holds ~190 work-groups as long as each split keeps >= 1024 of K.  Every row
  //    segment a load instruction fetches is then a whole 128-byte line, which measured faster
  //    than the 32-deep rings of 256 x 256 and 128 x 256 tiles at every prefill projection (70B
  //    shape at M = 4096: gate/up 6.27 -> 5.91 ms, down 3.16 -> 3.04, O 0.96 -> 0.90, three-plane
  //    QKV 1.78 -> 1.52; 8B shape at M = 512: down 113 -> 98 us, O 48 -> 42, QKV 85 -> 75, gate/up
  //    equal).
  //  * M >= 256 otherwise: 256 x 256 (two planes) when at most 4 splits fill the chip, else
  //    128 x 256, both in 32-deep stages.  The QKV epilogue (RoPE in f64 and the cache stores)
  //    never takes 256 x 256: on that tile it needed more registers than two waves per SIMD leave
  //    and spilled 528 bytes per lane.
  //  * Batched decode (32 < M <= 128) splits K as many ways as keep the grid within one round of
  //    256 work-groups (each split >= 512 deep), not in powers of two: the three-plane QKV at
  //    M = 128 runs 40 x 6 work-groups instead of 40 x 4 (70B decode step: QKV 1.73 -> 1.47 ms).
  //  * 32 < M <= 64 (batched decode): 64 x 128 LDS-direct tiles with 64-deep stages (8B-shaped
  //    projections at M = 64: gate/up 55 -> 50 us, down 37 -> 31 us, O 17.5 -> 16 us, against
  //    32-deep stages).  With every weight read cold (the 8B gate/up, 235 MB, otherwise stays in
  //    the 256 MB memory-side cache between repetitions), 224 unsplit 64 x 128 tiles beat 112
  //    64 x 256 tiles in two K splits plus their split-K sum: gate/up 59.8 -> 55.5 us; readout equal.
  //  * 64 < M <= 128 (batched decode): 128 x 256 with 64-deep stages in two LDS buffers (K a
  //    multiple of 64), so each row segment a load instruction fetches is a whole 128-byte line
  //    of the activation or weight row (M = 128: 70B gate/up 324 -> 280 us, O 46.5 -> 41 us, 8B O
  //    25.7 -> 23 us, readout 337 -> 309 us; bit-identical); three planes fill exactly 160 KB
  //    (70B QKV 74.6 -> 67.9 us against 32-deep stages in a 3-deep ring).  Otherwise 32-deep
  //    stages in a ring, 8 waves of 64 x 64.
  //  * The two-plane 128 x 256 tile keeps a third weight buffer in the 32 KB that two planes leave
  //    free, so the weight stream runs two stages ahead of the activations (bit-identical; M = 128:
  //    70B gate/up 259 -> 240 us, down 144 -> 133 us, O and QKV equal; M = 4096: 70B down 3.04 ->
  //    2.98 ms, O 0.88 -> 0.86 ms, gate/up 0.7% slower; 8B M = 512 gate/up 194 -> 187 us).  With
  //    32-deep stages and up to 8 weight buffers it was 10-20% slower.
  //  * otherwise 128 x 128 up to M = 512 and 64 x 256 above, one LDS buffer and one register
  //    staging set so that two work-groups fit a CU (the second hides the first's barrier, LDS and
  //    load waits), each wave owning a 64 x 64 tile; the 64 x 256 tile's 4 MB weight panels keep
  //    the long-K projections 1.5x faster than 128 x 128.  Skinny M uses 64 / 32 / 16 x 128
  //    tiles.  Split K until the grid holds ~400 work-groups (256 for skinny tiles), each split
  //    >= 256 deep.
  GemmPlan p{};
  const bool dma_ok = K % kDmaBK == 0 && (uint64_t)(M > N ? M : N) * K * 2 < (1ull << 32);
  if (dma_ok && K % 64 == 0 && M > 32 && M <= 64) {
    // batched decode rows: 64 x 128 tiles with 64-deep stages, so that every weight row segment a
    // load instruction touches is a whole 128-byte line; K split to fill one round of work-groups
    const int cfg = 9;
    const int tiles = (N + kCfgs[cfg].bn - 1) / kCfgs[cfg].bn;
    const int sk = decode_splits(tiles, K);
    p.cfg = cfg;
    p.bm = kCfgs[cfg].bm;
    p.bn = kCfgs[cfg].bn;
    p.tiles_m = 1;
    p.tiles_n = tiles;
    p.splitk = sk;
    return p;
  }
  if (dma_ok && M > 64 && M <= 128) {
    // batched decode rows: 128 x 256 with 64-deep stages in two buffers (8 waves of 32 x 128),
    // two or three planes; K not a multiple of 64: 64 x 64 wave tiles and a 3-deep (two planes:
    // 4-deep) ring of 32-deep stages; K split until the grid holds ~150 work-groups
    const int tiles = (N + 255) / 256;
    const int sk = decode_splits(tiles, K);
    p.cfg = K % 64 == 0 ? (planes == 2 ? 10 : 11) : 7;
    p.bm = kCfgs[p.cfg].bm;
    p.bn = kCfgs[p.cfg].bn;
    p.tiles_m = 1;
    p.tiles_n = tiles;
    p.splitk = sk;
    return p;
  }
  if (dma_ok && M >= 256 && K % 64 == 0) {
    // cfg 10 (two planes) / 11 (three planes): 128 x 256 with 64-deep stages in two buffers
    const int cfg = planes == 2 ? 10 : 11;
    const int tiles = ((M + 127) / 128) * ((N + 255) / 256);
    int sk = 1;
    while (tiles * sk < 190 && K / (sk * 2) >= 1024 && sk < 8) sk *= 2;
    p.cfg = cfg;
    p.bm = kCfgs[cfg].bm;
    p.bn = kCfgs[cfg].bn;
    p.tiles_m = (M + 127) / 128;
    p.tiles_n = (N + 255) / 256;
    p.splitk = sk;
    return p;
  }
  if (dma_ok && M >= 256) {
    // cfg 5 (256 x 256, two planes) when it fills the chip, else cfg 6 (128 x 256)
    for (int cfg = planes == 2 && !qkv ? 5 : 6; cfg <= 6; ++cfg) {
      const int bm = kCfgs[cfg].bm, bn = kCfgs[cfg].bn;
      const int tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
      const int want = cfg == 5 ? 200 : 190, least = cfg == 5 ? 200 : 128, most = cfg == 5 ? 4 : 8;
      int sk = 1;
      while (tiles * sk < want && K / (sk * 2) >= 1024 && sk < most) sk *= 2;
      if (tiles * sk >= least) {
        p.cfg = cfg;
        p.bm = bm;
        p.bn = bn;
        p.tiles_m = (M + bm - 1) / bm;
        p.tiles_n = (N + bn - 1) / bn;
        p.splitk = sk;
        return p;
      }
    }
  }
  p.cfg = M > 512 ? 1 : (M > 64 ? 0 : (M > 32 ? 2 : (M > 16 ? 3 : 4)));
  p.bm = kCfgs[p.cfg].bm;
  p.bn = kCfgs[p.cfg].bn;
  p.tiles_m = (M + p.bm - 1) / p.bm;
  p.tiles_n = (N + p.bn - 1) / p.bn;
  const int tiles = p.tiles_m * p.tiles_n;
  const int target = M > 64 ? 400 : 256;
  p.splitk = 1;
  while (tiles * p.splitk < target && K / (p.splitk * 2) >= 4 * BK && p.splitk < 16) p.splitk *= 2;
  return p;
}

namespace {

// Grids of at least kPingPongMinGroups work-groups (several per CU) run the 8-wave tiles with the
// two wave groups half a step apart; on single-round grids and short split-K ranges the lock-step
// schedule measured faster.  Both give identical sums.
constexpr int kPingPongMinGroups = 512;

template <int NP, int EPI>
void launch_cfg(const GemmArgs& a, const GemmPlan& p, dim3 grid, hipStream_t s) {
  const bool pp = (int)(grid.x * grid.y) >= kPingPongMinGroups;
  switch (p.cfg) {
    case 0: k_gemm<128, 128, 2, 2, NP, EPI, 1, 1><<<grid, 256, 0, s>>>(a); break;
    case 1: k_gemm<64, 256, 1, 4, NP, EPI, 1, 1><<<grid, 256, 0, s>>>(a); break;
    case 2: k_gemm<64, 128, 1, 4, NP, EPI, 2, 1><<<grid, 256, 0, s>>>(a); break;
    case 3: k_gemm<32, 128, 1, 4, NP, EPI, 2, 2><<<grid, 256, 0, s>>>(a); break;
    case 5:   // the planner gives it two planes and no QKV epilogue only
      if constexpr (EPI != EPI_QKV) {
        if (pp) k_gemm_dma<2, EPI, 256, 256, 4, 2, 3, kDmaBK, true><<<grid, 512, 0, s>>>(a);
        else k_gemm_dma<2, EPI, 256, 256, 4, 2, 3><<<grid, 512, 0, s>>>(a);
      }
      break;
    case 6:
      if (pp) k_gemm_dma<NP, EPI, 128, 256, 4, 2, 3, kDmaBK, true><<<grid, 512, 0, s>>>(a);
      else k_gemm_dma<NP, EPI, 128, 256, 4, 2, 3><<<grid, 512, 0, s>>>(a);
      break;
    case 7:
      k_gemm_dma<NP, EPI, 128, 256, 2, 4, NP == 2 ? 4 : 3><<<grid, 512, 0, s>>>(a);
      break;
    case 9: k_gemm_dma<NP, EPI, 64, 128, 1, 4, NP == 2 ? 4 : 3, 64><<<grid, 256, 0, s>>>(a); break;
    case 10:   // two planes only: 2 x 32 KB of activations + 3 x 32 KB of weights = 160 KB of LDS
      k_gemm_dma<2, EPI, 128, 256, 4, 2, 2, 64, false, 3><<<grid, 512, 0, s>>>(a);
      break;
    case 11:   // three planes only: 2 x (3 x 32 KB + 32 KB) = 160 KB of LDS
      if constexpr (NP == 3) k_gemm_dma<3, EPI, 128, 256, 4, 2, 2, 64><<<grid, 512, 0, s>>>(a);
      break;

    default: k_gemm<16, 128, 1, 4, NP, EPI, 2, 2><<<grid, 256, 0, s>>>(a); break;
  }
}

}  // namespace

template <int EPI>
void launch_reduce(const GemmArgs& a, hipStream_t s) {
  const size_t pairs = (size_t)a.M * ((((size_t)a.N + 31) >> 5) << 4);
  size_t grid = ((EPI == EPI_QKV ? pairs / 2 : pairs) + 255) / 256;   // QKV: two pairs per thread
  if (grid > 2048) grid = 2048;
  k_splitk_reduce<EPI><<<(unsigned)grid, 256, 0, s>>>(a);
}

hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& p, hipStream_t s, const NormArgs* then_norm,
                       bool* normed) {
  if (normed) *normed = false;
  // the LDS-direct tile takes two planes, K in whole 32-deep stages and operands under 4 GiB
  if (((p.cfg == 5 || p.cfg == 10) && a.planes != 2) || (p.cfg == 11 && a.planes != 3) ||
      (p.cfg >= 5 && (a.K % kDmaBK != 0 || (uint64_t)(a.M > a.N ? a.M : a.N) * a.K * 2 >= (1ull << 32))))
    return hipErrorInvalidValue;
  if (p.cfg == 5 && a.e.kind == EPI_QKV) return hipErrorInvalidValue;   // not instantiated (see gemm_plan)
  if (p.cfg == 8) return hipErrorInvalidValue;                           // retired tile: no launch
  if (p.cfg >= 8 && a.K % 64 != 0) return hipErrorInvalidValue;   // 64-deep stages
  dim3 grid(p.tiles_m * p.tiles_n, p.splitk);
  // one row of M-tiles (batched decode): every weight byte is read by one work-group, so the
  // LDS-direct tiles stream the weights with non-temporal loads
  GemmArgs g = a;
  g.w_stream = p.tiles_m == 1;
  switch (a.e.kind) {
    case EPI_QKV:
      // whole head-dim groups (Dh 64 or 128), from a stored row that starts a group
      if (a.N % 32 != 0 || a.e.col_off % 32 != 0 || a.e.col_off < 0) return hipErrorInvalidValue;
      if (a.planes == 3) launch_cfg<3, EPI_QKV>(g, p, grid, s);
      else launch_cfg<2, EPI_QKV>(g, p, grid, s);
      if (p.splitk > 1) launch_reduce<EPI_QKV>(a, s);
      break;
    case EPI_SWIGLU:
      launch_cfg<2, EPI_SWIGLU>(g, p, grid, s);
      if (p.splitk > 1) launch_reduce<EPI_SWIGLU>(a, s);
      break;
    case EPI_RESID:
      launch_cfg<2, EPI_RESID>(g, p, grid, s);
      if (p.splitk > 1) {
        // one work-group per row, every split's loads of a row in flight together
        if (then_norm && a.N % 4 == 0 && a.N <= kReduceNormMaxN && a.e.ldo == a.N) {
          if (a.M < 256) {   // few rows: a 1024-thread work-group per row, one round of loads
            if (a.N <= 4096) k_splitk_reduce_norm_w<1><<<a.M, 1024, 0, s>>>(a, *then_norm);
            else k_splitk_reduce_norm_w<kReduceNormMaxN / 4096><<<a.M, 1024, 0, s>>>(a, *then_norm);
          } else if (a.N <= 4096) {
            k_splitk_reduce_norm<4><<<a.M, 256, 0, s>>>(a, *then_norm);
          } else {
            k_splitk_reduce_norm<kReduceNormMaxN / 1024><<<a.M, 256, 0, s>>>(a, *then_norm);
          }
          if (normed) *normed = true;
        } else {
          launch_reduce<EPI_RESID>(a, s);
        }
      }
      break;
    default:
      launch_cfg<2, EPI_F32>(g, p, grid, s);
      if (p.splitk > 1) launch_reduce<EPI_F32>(a, s);
      break;
  }
  return hipGetLastError();
}
