// LDS-tiled bf16 MFMA GEMM for large token counts (prefill-sized batches),
// where the layer is bound by matrix-core throughput.
//
// Work-group tile: BM token rows x BN weight rows, k in steps of BK.  Eight
// waves (2 along tokens x 4 along weights) each own a (BM/2) x (BN/4)
// sub-tile of MFMA 16x16x32 tiles; with two waves per SIMD a wave has 256
// registers, so its sub-tile is 64 x 128 accumulators.  Four-wave variants
// with 128 x 128 accumulators per wave (one wave per SIMD, which can keep the
// matrix cores ~95% busy on its own) were measured and were not faster on the
// expert GEMMs: their time goes to the global -> LDS stream, not MFMA issue.
//
// Operands move global -> LDS with gfx950's direct 16-byte loads
// (global_load_lds_dwordx4), NS stages in flight and no staging registers;
// the LDS rows are XOR-swizzled so the 16 rows of an MFMA fragment read
// fall in distinct banks (measured: zero bank conflicts).  Each k tile: wait
// for this tile's loads, one barrier, the next stage's loads, all fragment
// reads, then the MFMAs.
//
// Work order is XCD-aware (see work_item).  Grouped mode (experts) takes the
// m tiles from the expert tile list built by the dispatch kernel; a tile
// never spans two experts.
#include <type_traits>

#include "gemm_problems.h"
#include "kernels.h"
#include "mxfp4_device.h"

namespace lmoe {

// s_waitcnt with only the vector-memory counter set to N (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt and lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence: the direct-to-LDS loads are
// waited for explicitly (wait_vmcnt) so that later stages stay in flight.
// The signal fences keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(3))) void lds_void;

// Work-item order.  Work-groups are dealt to the 8 XCDs round-robin by id,
// and each XCD has its own L2, so XCD x is given the contiguous chunk x of
// the work list: the work-groups resident on one XCD at a time are then
// neighbours in the list and share operand panels in that XCD's L2 while
// they walk k in step.  List order: for the grouped expert GEMMs, expert by
// expert, n block by n block, the expert's m tiles fastest (they share the
// weight panel); for dense GEMMs, groups of kDenseGroupM m tiles, m fastest
// (8: measured on the prefill batch's dense GEMMs, 1-3% faster than 4 and
// within noise of 16).
constexpr int kXcds = 8;
constexpr int kDenseGroupM = 8;

template <bool GROUPED>
__device__ __forceinline__ bool work_item(int nblocks, int mrows, int bm, const Tile* tiles,
                                          const int* ntiles, int& tm, int& nb) {
  const int mtiles = GROUPED ? *ntiles : (mrows + bm - 1) / bm;
  const int total = mtiles * nblocks;
  const int chunk = (total + kXcds - 1) / kXcds;
  const int local = blockIdx.x / kXcds;
  const int item = (blockIdx.x % kXcds) * chunk + local;
  if (local >= chunk || item >= total) return false;
  if (GROUPED) {
    const Tile t = tiles[item / nblocks];
    const int i = item - t.first * nblocks;
    nb = i / t.count;
    tm = t.first + i % t.count;
  } else {
    const int gsz = kDenseGroupM * nblocks;
    const int g = item / gsz;
    const int gm = min(kDenseGroupM, mtiles - g * kDenseGroupM);
    const int r = item - g * gsz;
    tm = g * kDenseGroupM + r % gm;
    nb = r / gm;
  }
  return true;
}

// Multi-stage variant: global -> LDS with gfx950's 16-byte direct loads
// (global_load_lds_dwordx4), NS stages in flight, no staging registers.
// A stage holds BM token rows then BN weight rows of BK bf16 each.  One wave
// instruction moves 1 KB = 1024 / (2 BK) rows; lane l fills slot l % CPR of
// row l / CPR and fetches the global chunk (slot ^ swz(row)) so the stage is
// already swizzled.  Token rows past the tile's count are loaded from the
// tile's first row instead (their outputs are never stored, and each output
// row depends only on its own token row).
template <class P, bool GROUPED, int BM, int BN, int BK, int NS, int WGN>
__global__ __launch_bounds__(128 * WGN) void tiled_gemm_kernel(P p, int mrows, const Tile* tiles,
                                                               const int* ntiles) {
  constexpr int NW = 2 * WGN;            // waves: 2 along tokens x WGN along weights
  constexpr int TM = BM / 32;            // 16-row token groups per wave
  constexpr int TN = BN / (16 * WGN);    // 16-row weight groups per wave
  constexpr int CPR = BK / 8;            // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;          // rows per wave instruction
  constexpr int RPB = 256 / (BK * 2);    // rows per 256-byte bank window
  constexpr int NIA = BM / RPI / NW;     // A instructions per wave per stage
  constexpr int NIB = BN / RPI / NW;
  constexpr int NI = NIA + NIB;
  constexpr int SROWS = BM + BN;
  static_assert((BM / RPI) % NW == 0 && (BN / RPI) % NW == 0, "rows per stage");
  static_assert((NS - 2) * NI < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS][SROWS * BK];

  int tm, nb;
  if (!work_item<GROUPED>(p.N() / BN, mrows, BM, tiles, ntiles, tm, nb)) return;
  int e = 0, m0, mcount;
  if (GROUPED) {
    const Tile t = tiles[tm];
    e = t.expert;
    m0 = t.row0;
    mcount = t.nrows;
  } else {
    m0 = tm * BM;
    mcount = min(BM, mrows - m0);
  }
  const int n0 = nb * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int K = p.K(), K0 = p.K0();
  const int nk = K / BK;

  auto swz = [](int row) { return (row / RPB) & (CPR - 1); };

  // Per-lane source rows: instruction j of wave w covers stage rows
  // RPI * (w + NW j) .. + RPI - 1; this lane takes row RPI * (w + NW j) + l / CPR.
  // The swizzled chunk depends only on w and the lane (NW j RPI rows is a
  // multiple of the swizzle period), so one chunk offset serves every j.
  // Gathered token rows keep one pointer per instruction; strided rows are
  // recomputed in issue() (no extra registers, no extra memory reads).
  const int lr = lane / CPR;
  const int chunk8 = ((lane % CPR) ^ swz(RPI * w + lr)) * 8;
  constexpr bool GA = P::kGatherA;
  const uint16_t* pa[GA ? NIA : 1];
  if constexpr (GA) {
#pragma unroll
    for (int j = 0; j < NIA; ++j) {
      const int row = RPI * (w + NW * j) + lr;
      pa[j] = p.a_row0(m0 + (row < mcount ? row : 0)) + chunk8;
    }
  }
  const uint16_t* pb0 = p.b_row0(e, n0 + RPI * w + lr) + chunk8;
  const uint16_t* qb = p.b_row1(e, n0 + RPI * w + lr);
  const uint16_t* pb1 = qb ? qb + chunk8 : nullptr;
  const long sb0 = (long)RPI * NW * p.ldb0(), sb1 = (long)RPI * NW * p.ldb1();
  // The second source as byte offsets from the first: issue() selects it by
  // adding, since a choice between two captured pointers was compiled into
  // a private-memory table in one instantiation.
  const long db = pb1 ? (long)((intptr_t)pb1 - (intptr_t)pb0) : 0, dsb = sb1 - sb0;

  auto issue = [&](int kt) {
    const int k = kt * BK;
    const bool s0 = k < K0;
    const int kk = s0 ? k : k - K0;
    uint16_t* stage = &smem[kt % NS][0];
    const uint16_t* abase = s0 ? p.a_base0() : p.a_base1();
    const long lda = s0 ? p.lda0() : p.lda1();
#pragma unroll
    for (int j = 0; j < NIA; ++j) {
      // With two stages every wait is vmcnt(0), so instructions whose rows
      // all lie past the tile's count can be skipped (with more stages the
      // waits count a fixed number of loads per stage).
      if (NS == 2 && RPI * (w + NW * j) >= mcount) continue;
      const uint16_t* src;
      if constexpr (GA) {
        src = pa[j];
      } else {
        int row = RPI * (w + NW * j) + lr;
        row = row < mcount ? row : 0;
        src = abase + (long)(m0 + row) * lda + chunk8;
      }
      __builtin_amdgcn_global_load_lds((const void*)(src + kk),
                                       (lds_void*)(stage + RPI * (w + NW * j) * BK), 16, 0, 0);
    }
    const uint16_t* b =
        reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(pb0) + (s0 ? 0 : db));
    const long sb = sb0 + (s0 ? 0 : dsb);
#pragma unroll
    for (int j = 0; j < NIB; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(b + j * sb + kk),
                                       (lds_void*)(stage + RPI * (w + NW * (NIA + j)) * BK), 16,
                                       0, 0);
  };

  const int wm = w / WGN, wn = w % WGN;
  const int r16 = lane & 15, kq = lane >> 4;
  f32x4 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s);

  // Per k tile: wait for this tile's stage (own loads, then everyone's via
  // the barrier, which also frees the stage written next: its last reads were
  // the previous tile's, consumed by that tile's MFMAs), issue the DMA of
  // tile kt + NS - 1 first (issued before the fragment reads, the expert
  // GEMMs of the prefill batch run 6-7% faster; the dense ones are
  // unchanged), read every MFMA fragment of the tile from LDS, then run the
  // MFMAs.
  constexpr int KS = BK / 32;
  // Partial tiles skip token groups wholly past the tile's count (uniform
  // branches; ~2% of the expert GEMMs' MFMA work at the prefill batch, and a
  // third of a 192-row batch's dense tile).  Full dense tiles take a copy of
  // the loop without those branches: across them the compiler waits for
  // every fragment read before the first MFMA, without them for each read
  // as it is needed, and the dense GEMMs run 4-9% faster.  (Full expert tiles
  // measured no different, so grouped GEMMs keep one copy.)
  auto kloop = [&](auto full_tile) {
    constexpr bool FULL = decltype(full_tile)::value;
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + NS - 2 < nk)
        wait_vmcnt<(NS - 2) * NI>();
      else
        wait_vmcnt<0>();
      stage_barrier();
      if (kt + NS - 1 < nk) issue(kt + NS - 1);
      const uint16_t* st = &smem[kt % NS][0];
      bf16x8 xf[KS][TM], wf[KS][TN];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int q = ks * 4 + kq;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          const int row = wm * (BM / 2) + t * 16 + r16;
          if (FULL || wm * (BM / 2) + t * 16 < mcount)
            xf[ks][t] = *reinterpret_cast<const bf16x8*>(st + row * BK + ((q ^ swz(row)) << 3));
        }
#pragma unroll
        for (int gi = 0; gi < TN; ++gi) {
          const int row = BM + wn * (BN / WGN) + gi * 16 + r16;
          wf[ks][gi] = *reinterpret_cast<const bf16x8*>(st + row * BK + ((q ^ swz(row)) << 3));
        }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < TM; ++t)
          if (FULL || wm * (BM / 2) + t * 16 < mcount)
#pragma unroll
            for (int gi = 0; gi < TN; ++gi)
              acc[gi][t] = mfma_bf16(wf[ks][gi], xf[ks][t], acc[gi][t]);
    }
  };
  if constexpr (!GROUPED) {
    if (mcount == BM)
      kloop(std::true_type{});
    else
      kloop(std::false_type{});
  } else {
    kloop(std::false_type{});
  }

  const int ncol = (lane >> 4) * 4;
#pragma unroll
  for (int gi = 0; gi < TN; ++gi)
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int i = wm * (BM / 2) + t * 16 + r16;
      if (i < mcount) p.store(e, m0 + i, n0 + wn * (BN / WGN) + gi * 16 + ncol, acc[gi][t]);
    }
}

// Grouped expert GEMM with MXFP4 weights for large batches: the main loop of
// tiled_gemm_kernel (NS = 2 stages of 64 k), with each stage's weight rows
// decoded from FP4 codes instead of copied.  Every lane owns whole 32-k code
// blocks (16 code bytes and a scale byte each; BN / 256 blocks per stage),
// loads them into registers two stages ahead, decodes them exactly to bf16
// and writes them into the stage's swizzled weight rows; the token rows keep
// the direct global -> LDS copy.  The codes cut the weight bytes moved to a
// quarter; the MFMA part is unchanged.
template <class P, int BM, int BN, int WGN>
__global__ __launch_bounds__(128 * WGN) void tiled_mx_kernel(P p, const Tile* tiles, const int* ntiles) {
  constexpr int BK = 64, NS = 2;
  constexpr int NW = 2 * WGN;
  constexpr int TM = BM / 32, TN = BN / (16 * WGN);
  constexpr int CPR = BK / 8, RPI = 64 / CPR, RPB = 256 / (BK * 2);
  constexpr int NIA = BM / RPI / NW;      // token DMA instructions per wave per stage
  constexpr int NBL = BN / (32 * NW);     // weight blocks (32 k of a row) per lane per stage
  static_assert(NBL >= 1 && NBL * 32 * NW == BN, "BN");
  constexpr int NCL = 2 * NBL;            // code + scale loads per lane per stage
  constexpr int SROWS = BM + BN;
  static_assert((BM / RPI) % NW == 0, "rows per stage");
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS][SROWS * BK];

  int tm, nb;
  if (!work_item<true>(p.N() / BN, 0, BM, tiles, ntiles, tm, nb)) return;
  const Tile t = tiles[tm];
  const int e = __builtin_amdgcn_readfirstlane(t.expert);
  const int m0 = __builtin_amdgcn_readfirstlane(t.row0);
  const int mcount = __builtin_amdgcn_readfirstlane(t.nrows);
  const int n0 = nb * BN;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nk = p.K() / BK;
  auto swz = [](int row) { return (row / RPB) & (CPR - 1); };

  const int lr = lane / CPR;
  const int chunk8 = ((lane % CPR) ^ swz(RPI * w + lr)) * 8;
  const uint16_t* pa[NIA];
#pragma unroll
  for (int j = 0; j < NIA; ++j) {
    const int row = RPI * (w + NW * j) + lr;
    pa[j] = p.a_row(m0 + (row < mcount ? row : 0)) + chunk8;
  }
  auto issue_a = [&](int kt) {
    uint16_t* stage = &smem[kt % NS][0];
#pragma unroll
    for (int j = 0; j < NIA; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(pa[j] + kt * BK),
                                       (lds_void*)(stage + RPI * (w + NW * j) * BK), 16, 0, 0);
  };
  // weight block i of this lane: stage row w * (BN / NW) + 32 i + lane / 2, k half lane % 2
  const int half = lane & 1;
  const uint8_t* cp[NBL];
  const uint8_t* sp[NBL];
  int brow[NBL];
#pragma unroll
  for (int i = 0; i < NBL; ++i) {
    brow[i] = w * (BN / NW) + 32 * i + (lane >> 1);
    cp[i] = p.codes_row(e, n0 + brow[i]) + half * 16;
    sp[i] = p.scales_row(e, n0 + brow[i]) + half;
  }
  struct Codes { u32x4 c[NBL]; uint32_t s[NBL]; };
  auto load_codes = [&](Codes& C, int kt) {
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
      C.c[i] = *reinterpret_cast<const u32x4*>(cp[i] + kt * (BK / 2));
      C.s[i] = sp[i][kt * (BK / 32)];
    }
  };
  // decode this lane's blocks of stage kt and write them as bf16 into the stage's weight rows
  auto store_b = [&](const Codes& C, int kt) {
    uint16_t* stage = &smem[kt % NS][0];
#pragma unroll
    for (int i = 0; i < NBL; ++i) {
      const int row = BM + brow[i];
      const float sc = mx_scale(C.s[i]);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int ch = half * 4 + d;
        *reinterpret_cast<bf16x8*>(stage + row * BK + ((ch ^ swz(row)) << 3)) = mx_decode8(C.c[i][d], sc);
      }
    }
  };

  const int wm = w / WGN, wn = w % WGN;
  const int r16 = lane & 15, kq = lane >> 4;
  f32x4 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // prologue: codes 0 and 1 in flight, stage 0 (tokens by DMA, weights decoded)
  Codes C0, C1;
  issue_a(0);
  load_codes(C0, 0);
  if (nk > 1) load_codes(C1, 1);
  store_b(C0, 0);
  if (nk > 2) load_codes(C0, 2);

  constexpr int KS = BK / 32;
  auto iter = [&](int kt, Codes& Cn) {
    // this stage's token rows (own DMA, issued before the last code loads) and
    // weight rows (own LDS writes), then everyone's via the barrier
    if (kt + 2 < nk || (kt == 0 && nk > 2)) wait_vmcnt<NCL>(); else wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's weight writes
    stage_barrier();
    // the next stage's token DMA first (its buffer's last reads were the
    // previous stage's): 2-4% faster than issuing it after the reads
    if (kt + 1 < nk) issue_a(kt + 1);
    const uint16_t* st = &smem[kt % NS][0];
    bf16x8 xf[KS][TM], wf[KS][TN];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int q = ks * 4 + kq;
#pragma unroll
      for (int tt = 0; tt < TM; ++tt) {
        const int row = wm * (BM / 2) + tt * 16 + r16;
        if (wm * (BM / 2) + tt * 16 < mcount)
          xf[ks][tt] = *reinterpret_cast<const bf16x8*>(st + row * BK + ((q ^ swz(row)) << 3));
      }
#pragma unroll
      for (int gi = 0; gi < TN; ++gi) {
        const int row = BM + wn * (BN / WGN) + gi * 16 + r16;
        wf[ks][gi] = *reinterpret_cast<const bf16x8*>(st + row * BK + ((q ^ swz(row)) << 3));
      }
    }
    if (kt + 1 < nk) {
      store_b(Cn, kt + 1);                 // codes kt + 1, loaded two iterations ago
      if (kt + 3 < nk) load_codes(Cn, kt + 3);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int tt = 0; tt < TM; ++tt)
        if (wm * (BM / 2) + tt * 16 < mcount)
#pragma unroll
          for (int gi = 0; gi < TN; ++gi) acc[gi][tt] = mfma_bf16(wf[ks][gi], xf[ks][tt], acc[gi][tt]);
  };
  for (int kt = 0; kt < nk; kt += 2) {
    iter(kt, C1);
    if (kt + 1 < nk) iter(kt + 1, C0);
  }

  const int ncol = (lane >> 4) * 4;
#pragma unroll
  for (int gi = 0; gi < TN; ++gi)
#pragma unroll
    for (int tt = 0; tt < TM; ++tt) {
      const int i = wm * (BM / 2) + tt * 16 + r16;
      if (i < mcount) p.store(e, m0 + i, n0 + wn * (BN / WGN) + gi * 16 + ncol, acc[gi][tt]);
    }
}

// Tile shapes used per problem (token rows x weight rows), from a sweep on
// the full-shape prefill problems.  Expert GEMMs use 128-row token tiles
// (with ~352 rows per expert at the prefill batch a 256-row tile would pad
// 45% of the rows) and 512 weight rows where N allows (fewer bytes moved per
// flop: measured, the vector-memory data path, not the MFMAs, limits these
// GEMMs), else 256.
constexpr int kExpBM = 128, kExpBK = 64;
constexpr int kDenseBM = 256, kDenseBN = 256, kDenseBK = 64, kDenseNS = 2;
constexpr int kWGN = 4;

static long xcd_grid(long items) { return (items + kXcds - 1) / kXcds * kXcds; }

template <class P, int BM, int BN, int BK, int NS>
static hipError_t launch_dense(const P& p, int T, hipStream_t s) {
  const long grid = xcd_grid((long)((T + BM - 1) / BM) * (p.N() / BN));
  if (grid <= 0) return hipSuccess;
  tiled_gemm_kernel<P, false, BM, BN, BK, NS, kWGN><<<grid, 128 * kWGN, 0, s>>>(p, T, nullptr,
                                                                                nullptr);
  return hipGetLastError();
}

template <class P, int BM, int BN, int BK, int NS>
static hipError_t launch_grouped(const P& p, const Tile* tiles, const int* ntiles, int max_tiles,
                                 hipStream_t s) {
  const long grid = xcd_grid((long)max_tiles * (p.N() / BN));
  if (grid <= 0) return hipSuccess;
  tiled_gemm_kernel<P, true, BM, BN, BK, NS, kWGN><<<grid, 128 * kWGN, 0, s>>>(p, 0, tiles,
                                                                               ntiles);
  return hipGetLastError();
}

int tiled_block_m() { return kExpBM; }
int tiled_block_n() { return 256; }

// Sum of the split partial sums in split order (deterministic), then P's own
// epilogue; one thread per four consecutive columns.
template <class P>
__global__ __launch_bounds__(256) void split_reduce_kernel(P p, const float* __restrict__ part,
                                                           int nsplit, int mrows) {
  const int N = p.N();
  const long i = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= (long)mrows * N) return;
  const int m = i / N, n = i % N;
  f32x4 v = *reinterpret_cast<const f32x4*>(part + i);
  for (int q = 1; q < nsplit; ++q)
    v += *reinterpret_cast<const f32x4*>(part + (size_t)q * mrows * N + i);
  p.store(0, m, n, v);
}

template <class P, int BM, int BN, int NS>
static hipError_t launch_split(const P& p, int T, float* part, int nsplit, hipStream_t s) {
  const long gx = xcd_grid((long)((T + BM - 1) / BM) * (p.N() / BN));
  if (gx <= 0) return hipSuccess;
  const SplitK<P> sp{p, p.K() / nsplit, part, T};
  tiled_gemm_kernel<SplitK<P>, false, BM, BN, kDenseBK, NS, kWGN>
      <<<dim3(gx, nsplit), 128 * kWGN, 0, s>>>(sp, T, nullptr, nullptr);
  const long n4 = (long)T * p.N() / 4;
  split_reduce_kernel<<<(n4 + 255) / 256, 256, 0, s>>>(p, part, nsplit, T);
  return hipGetLastError();
}

// Largest split count <= want (a power of two) whose k range is a whole
// number of k tiles.
static int pick_splits(int K, int want) {
  for (int n = want; n > 1; n /= 2)
    if (K % (n * kDenseBK) == 0) return n;
  return 1;
}

// Tile shapes and split counts measured on the full-shape problems at
// T = 192 (speculative-verify batch): output projection 256x256 in 8 splits
// (62 us vs 145 us for the best weight-streaming shape), latent 128x256 with
// 3 stages in 8 splits (28 vs 39 us), shared up 256x256 in 4 splits
// (69 vs 96 us).
hipError_t split_proj_in(const ProjIn& p, float* part, hipStream_t s) {
  if (p.N() <= 4096)
    return launch_split<ProjIn, 128, 256, 3>(p, p.T, part, pick_splits(p.K(), kSplitMax), s);
  return launch_split<ProjIn, 256, 256, 2>(p, p.T, part, pick_splits(p.K(), 4), s);
}
hipError_t split_proj_out(const ProjOut& p, float* part, hipStream_t s) {
  return launch_split<ProjOut, 256, 256, 2>(p, p.T, part, pick_splits(p.K(), kSplitMax), s);
}

hipError_t tiled_proj_in(const ProjIn& p, hipStream_t s) {
  return launch_dense<ProjIn, kDenseBM, kDenseBN, kDenseBK, kDenseNS>(p, p.T, s);
}
hipError_t tiled_proj_out(const ProjOut& p, hipStream_t s) {
  return launch_dense<ProjOut, kDenseBM, kDenseBN, kDenseBK, kDenseNS>(p, p.T, s);
}
template <class P>
static hipError_t launch_expert(const P& p, const Tile* tiles, const int* ntiles, int max_tiles,
                                hipStream_t s) {
  if (p.N() % 512 == 0)
    return launch_grouped<P, kExpBM, 512, kExpBK, 2>(p, tiles, ntiles, max_tiles, s);
  return launch_grouped<P, kExpBM, 256, kExpBK, 3>(p, tiles, ntiles, max_tiles, s);
}

hipError_t tiled_exp_up(const ExpUp& p, const Tile* tiles, const int* ntiles, int max_tiles,
                        hipStream_t s) {
  return launch_expert(p, tiles, ntiles, max_tiles, s);
}
hipError_t tiled_exp_down(const ExpDown& p, const Tile* tiles, const int* ntiles, int max_tiles,
                          hipStream_t s) {
  return launch_expert(p, tiles, ntiles, max_tiles, s);
}

// MXFP4 weights: 128 x 256 tiles (128 x 512 needs more than the 256
// registers two waves per SIMD allow, and spills).
template <class P>
static hipError_t launch_expert_mx(const P& p, const Tile* tiles, const int* ntiles,
                                   int max_tiles, hipStream_t s) {
  constexpr int BN = 256;
  const long grid = xcd_grid((long)max_tiles * (p.N() / BN));
  if (grid <= 0) return hipSuccess;
  tiled_mx_kernel<P, kExpBM, BN, kWGN><<<grid, 128 * kWGN, 0, s>>>(p, tiles, ntiles);
  return hipGetLastError();
}
hipError_t tiled_mx_exp_up(const ExpUpMx& p, const Tile* tiles, const int* ntiles, int max_tiles,
                           hipStream_t s) {
  return launch_expert_mx(p, tiles, ntiles, max_tiles, s);
}
hipError_t tiled_mx_exp_down(const ExpDownMx& p, const Tile* tiles, const int* ntiles,
                             int max_tiles, hipStream_t s) {
  return launch_expert_mx(p, tiles, ntiles, max_tiles, s);
}

}  // namespace lmoe
