// LDS-tiled bf16 MFMA GEMM for large token counts (prefill-sized batches),
// where the layer is bound by matrix-core throughput, and its MXFP4 forms
// (expert weights as FP4 codes decoded before the MFMAs: lds_mx_kernel, and
// tiled_mx_kernel for the shapes that one does not take).
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
// reads, then the MFMAs.  lds_pipe_kernel (the whole-k dense projections and
// the expert down projection) splits each k tile into two half-steps and
// keeps two copy units in flight across the waits.
//
// Work order is XCD-aware (see work_item).  Grouped mode (experts) takes the
// m tiles from the expert tile list built by the dispatch kernel; a tile
// never spans two experts, and its output goes out through LDS as whole row
// pieces (staged_store).
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

// Output of one wave's block of 16 TM rows, written through LDS.  In the
// MFMA result layout lane (r, q) (r = lane % 16, q = lane / 16) of tile
// (g, t) holds columns 16 g + 4 q .. + 3 of row 16 t + r, so a direct store
// instruction writes 16 pieces of 32 bytes.  Here tiles G0 .. G0 + GN - 1
// are packed (p.pack4: the stored bits of four columns) into `reg`, the
// wave's own LDS region of 16 TM rows x 32 GN bytes (16-byte chunks XOR-
// swizzled by row), and read back as 16 contiguous bytes per lane, so that
// each store instruction (p.store8) writes whole 32 GN-byte row pieces.
// Rows from `rows` on are not stored; row i goes to slot m0 + i, columns
// from n0.  Only this wave touches `reg`, and a wave's LDS accesses stay in
// order, so no barrier is needed inside.  Measured on the prefill batch's
// expert GEMMs (bitwise equal): MXFP4 up projection 3.41 against 3.45-3.56
// ms with direct stores, down projection 3.18 against 3.30-3.33 ms.
template <int GN, int G0, int TN, int TM, class P>
__device__ __forceinline__ void staged_store(const P& p, char* reg, int lane,
                                             const f32x4 (&acc)[TN][TM], int m0, int rows, int n0) {
  constexpr int RB = GN * 32, CH = RB / 16, RPI = 64 / CH;
  static_assert(G0 + GN <= TN && (CH & (CH - 1)) == 0 && CH <= 64, "staged store");
  const int r16 = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int g = 0; g < GN; ++g)
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int row = t * 16 + r16;
      const int chunk = 2 * g + (kq >> 1);
      *reinterpret_cast<u16x4*>(reg + row * RB + ((chunk ^ (row & (CH - 1))) << 4) +
                                (kq & 1) * 8) = p.pack4(acc[G0 + g][t]);
    }
  const int c = lane & (CH - 1);
#pragma unroll
  for (int j = 0; j < 16 * TM / RPI; ++j) {
    const int row = j * RPI + lane / CH;
    const u16x8 v = *reinterpret_cast<const u16x8*>(reg + row * RB + ((c ^ (row & (CH - 1))) << 4));
    if (row < rows) p.store8(m0 + row, n0 + c * 8, v);
  }
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

  if constexpr (GROUPED && P::kStagedStore && NS == 2 && TN == 8 && TM == 4) {
    // through the stage buffer the last k tile did not read (its last
    // reader, tile nk - 2, finished before every wave passed tile nk - 1's
    // barrier; no copy targets it any more): 8 KB per wave, two passes of
    // 64 columns
    char* const reg = reinterpret_cast<char*>(&smem[nk % 2][0]) + w * (64 * 128);
    const int wr = wm * (BM / 2), wc = n0 + wn * (BN / WGN);
    staged_store<4, 0>(p, reg, lane, acc, m0 + wr, mcount - wr, wc);
    staged_store<4, 4>(p, reg, lane, acc, m0 + wr, mcount - wr, wc + 64);
    return;
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

// ---- Two-stage LDS GEMM with scalar addressing -----------------------------
//
// The same tiling and results as tiled_gemm_kernel with NS = 2 (eight waves,
// 2 along tokens x 4 along weights, BK = 64, both operands copied global ->
// LDS with 16-byte direct loads, the same swizzle, the same MFMA order, so
// the outputs are bit for bit those of tiled_gemm_kernel), written so that
// the compiler sees what is uniform:
//  - the wave index, the tile's row count and its expert are read into
//    scalar registers (readfirstlane), so the per-wave "rows left" tests are
//    scalar branches, not exec-mask regions (inside those regions the
//    compiler had waited for every LDS read before the first MFMA);
//  - copies are buffer loads: a per-lane 32-bit offset (fixed for the whole
//    tile) plus the k offset in a scalar register, so a k step costs no
//    vector address arithmetic;
//  - the k loop is unrolled over the two stage buffers, so every LDS address
//    is a register plus an immediate, and its last step is peeled (no copy);
//  - a wave whose token rows all lie past the tile's count only copies.
// Measured on the prefill batch's problems (standalone, same inputs): expert
// up 4.60 -> 4.43 ms, shared up 1.13 -> 1.03 ms (with the directed MFMA /
// LDS-read interleave, SCHED = 1); expert down 4.50 -> 4.60 ms at first, and
// 4.54 -> 4.46 ms once both kernels wrote their outputs through LDS
// (staged_store), so both expert projections now take it.  Launched when
// the k range is an even number of 64-wide k tiles (every full-shape
// problem).

// Problems whose k range has two segments (the output projection's [r | Hs]).
template <class P>
struct TwoSegments : std::false_type {};
template <>
struct TwoSegments<ProjOut> : std::true_type {};
template <>
struct TwoSegments<SplitK<ProjOut>> : std::true_type {};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  // raw buffer over 2 GiB from `base`: offsets are checked against this
  // bound by the hardware (reads past it return 0)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFF0,
                                           0x00020000);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A barrier that is also a hard scheduling boundary: no LDS read of the
// stage may be hoisted above it (its data is not there yet) and no read of
// the previous stage sunk below it (other waves overwrite that buffer next).
__device__ __forceinline__ void stage_barrier_hard() {
  __builtin_amdgcn_sched_barrier(0);
  stage_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// work_item with the tile list's fields read into scalar registers.
template <bool GROUPED>
__device__ __forceinline__ bool work_item_uniform(int nblocks, int mrows, int bm,
                                                  const Tile* tiles, const int* ntiles, int& tm,
                                                  int& nb) {
  const int mtiles = GROUPED ? uniform(*ntiles) : (mrows + bm - 1) / bm;
  const int total = mtiles * nblocks;
  const int chunk = (total + kXcds - 1) / kXcds;
  const int local = blockIdx.x / kXcds;
  const int item = (blockIdx.x % kXcds) * chunk + local;
  if (local >= chunk || item >= total) return false;
  if (GROUPED) {
    const int first = uniform(tiles[item / nblocks].first);
    const int count = uniform(tiles[item / nblocks].count);
    const int i = item - first * nblocks;
    nb = i / count;
    tm = first + i % count;
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

template <class P, bool GROUPED, int BM, int BN, int SCHED>
__device__ __forceinline__ void lds_gemm_body(const P& p, int mrows, const Tile* tiles,
                                              const int* ntiles) {
  constexpr int WM = 2, WN = 4, NW = WM * WN, BK = 64;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int RPI = 8;                      // rows per copy instruction (8 x 128 B)
  constexpr int NIA = BM / RPI / NW, NIB = BN / RPI / NW, NI = NIA + NIB;
  static_assert(NIA * RPI * NW == BM && NIB * RPI * NW == BN, "rows per stage");
  constexpr int ROWB = BK * 2;                // bytes per LDS row
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr bool SEG2 = TwoSegments<P>::value;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  int tm, nb;
  if (!work_item_uniform<GROUPED>(p.N() / BN, mrows, BM, tiles, ntiles, tm, nb)) return;
  int e = 0, m0, mcount;
  if (GROUPED) {
    e = uniform(tiles[tm].expert);
    m0 = uniform(tiles[tm].row0);
    mcount = uniform(tiles[tm].nrows);
  } else {
    m0 = tm * BM;
    mcount = min(BM, mrows - m0);
  }
  const int n0 = nb * BN;
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int wm = w / WN, wn = w % WN;
  const int nk = p.K() / BK;
  const int nk0 = SEG2 ? p.K0() / BK : nk;

  // Copy instruction j of wave w fills stage rows RPI (w + NW j) .. + 7; lane
  // l takes row + l / 8 and the global 16-byte chunk (l % 8) ^ swz with
  // swz = (row / 2) % 8, which for these rows is (4 (w % 2) + (l / 8) / 2) % 8
  // for every j: the stage is written already swizzled.
  const int lr = lane >> 3;
  const int sw = ((4 * (w & 1)) + (lr >> 1)) & 7;
  const uint32_t chunk = (uint32_t)(((lane & 7) ^ sw) * 16);
  // One k segment's copy sources.  A: a per-lane byte offset per instruction
  // from the tile's first row (strided A) or the array (gathered A); rows
  // past the tile's count read its first row (never stored).  B: one
  // per-lane offset (row l / 8 of the instruction, its chunk) from the
  // tile's first weight row plus a uniform offset per instruction.
  struct Seg {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t ao[NIA];
    uint32_t bo;
    int b0, bstep;  // uniform bytes to instruction 0's rows, between instructions
  };
  auto make_seg = [&](int seg) __attribute__((always_inline)) {
    Seg g;
    const char* pa = GROUPED && P::kGatherA
                         ? reinterpret_cast<const char*>(seg ? p.a_base1() : p.a_base0())
                         : reinterpret_cast<const char*>(seg ? p.a_row1(m0) : p.a_row0(m0));
#pragma unroll
    for (int j = 0; j < NIA; ++j) {
      const int row = RPI * (w + NW * j) + lr;
      const int m = m0 + (row < mcount ? row : 0);
      g.ao[j] = (uint32_t)(reinterpret_cast<const char*>(seg ? p.a_row1(m) : p.a_row0(m)) - pa) +
                chunk;
    }
    const char* pb = reinterpret_cast<const char*>(seg ? p.b_row1(e, n0) : p.b_row0(e, n0));
    const int ldb = (int)(seg ? p.ldb1() : p.ldb0()) * 2;
    g.bo = (uint32_t)(lr * ldb) + chunk;
    g.b0 = RPI * w * ldb;
    g.bstep = RPI * NW * ldb;
    g.ra = buffer_rsrc(pa);
    g.rb = buffer_rsrc(pb);
    return g;
  };
  // copy one k tile (byte offset kb within the rows) of segment g into stage
  // buffer buf
  auto issue = [&](const Seg& g, int kb, int buf) __attribute__((always_inline)) {
    char* st = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < NIA; ++j) {
      // expert tiles: no copy of token rows wholly past the tile's count
      // (their LDS rows keep stale values; the outputs of such rows are
      // never stored, and every wait here is for all copies); at the
      // prefill batch about 1% faster on both expert projections
      if (GROUPED && RPI * (w + NW * j) >= mcount) continue;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(g.ra, (lds_void*)(st + (w + NW * j) * RPI * ROWB),
                                               16, g.ao[j], kb, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NIB; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          g.rb, (lds_void*)(st + BM * ROWB + (w + NW * j) * RPI * ROWB), 16, g.bo,
          kb + g.b0 + j * g.bstep, 0, 0);
  };
  const Seg seg0 = make_seg(0);
  auto copy0 = [&](int kt, int buf) { issue(seg0, kt * ROWB, buf); };

  // Fragment reads: lane (r16, kq) of k half ks reads row base + r16, 16-byte
  // chunk (4 ks + kq) ^ swz(row), and swz(row) = r16 / 2 for these rows.
  const int r16 = lane & 15, kq = lane >> 4;
  const uint32_t l0 = r16 * ROWB + (((0 + kq) ^ (r16 >> 1)) << 4);
  const uint32_t l1 = r16 * ROWB + (((4 + kq) ^ (r16 >> 1)) << 4);
  const uint32_t aw = (uint32_t)(wm * (BM / WM)) * ROWB;
  const uint32_t bw = (uint32_t)(BM + wn * (BN / WN)) * ROWB;
  const bool has_rows = wm * (BM / WM) < mcount;
  // 16-row token groups of this wave that hold rows (uniform): expert tiles
  // skip the MFMAs of the others (scalar branches; the fragment reads stay
  // unconditional).  At the prefill batch, where padding rows are 8.7% of
  // the MFMA work otherwise: expert up 4.22-4.24 -> 4.14-4.16 ms, down
  // 4.43-4.44 -> 4.36 ms standalone, same bits.  (lds_mx_kernel, where the
  // same branch was slower, takes one of four copies of its k loop instead.)
  const int tlim = uniform(min(TM, max(0, (mcount - wm * (BM / WM) + 15) / 16)));

  f32x4 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One k step on stage buffer BUF: wait for this wave's copies of the stage,
  // barrier (everyone's copies landed; everyone is done with the other
  // buffer), copy the next k tile into the other buffer, then the fragment
  // reads and MFMAs (k half 0 then 1, the order of tiled_gemm_kernel).
  // `copy` copies k tile kt + 1 into the other buffer (nullptr: nothing left)
  auto body = [&](auto buf_c, auto copy, int kt) {
    constexpr int BUF = decltype(buf_c)::value;
    constexpr bool COPY = !std::is_same<decltype(copy), std::nullptr_t>::value;
    wait_vmcnt<0>();
    stage_barrier_hard();
    if constexpr (COPY) copy(kt + 1, BUF ^ 1);
    const char* st = smem + BUF * STAGE;
    bf16x8 xf[2][TM], wf[2][TN];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t l = ks ? l1 : l0;
#pragma unroll
      for (int t = 0; t < TM; ++t)
        xf[ks][t] = *reinterpret_cast<const bf16x8*>(st + aw + l + t * 16 * ROWB);
#pragma unroll
      for (int g = 0; g < TN; ++g)
        wf[ks][g] = *reinterpret_cast<const bf16x8*>(st + bw + l + g * 16 * ROWB);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int t = 0; t < TM; ++t)
        if (!GROUPED || t < tlim)
#pragma unroll
          for (int g = 0; g < TN; ++g) acc[g][t] = mfma_bf16(wf[ks][g], xf[ks][t], acc[g][t]);
    if constexpr (SCHED == 1) {
      // directed order: the first half's fragment reads, the copies spread
      // over the first MFMAs, the second half's reads under the rest of the
      // first half's MFMAs, then the second half's MFMAs
      constexpr int R = TM + TN, M = TM * TN, D = COPY ? NI : 0;
      constexpr int rest = M - (D < M ? D : M);
      constexpr int per = rest / R > 0 ? rest / R : 1;
#pragma unroll
      for (int i = 0; i < R; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int i = 0; i < D; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, per, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * M, 0);
    }
  };
  // a wave whose token rows all lie past the tile's count only copies
  auto copy_only = [&](auto buf_c, auto copy, int kt) {
    constexpr int BUF = decltype(buf_c)::value;
    wait_vmcnt<0>();
    stage_barrier_hard();
    if constexpr (!std::is_same<decltype(copy), std::nullptr_t>::value) copy(kt + 1, BUF ^ 1);
  };

  // k tiles 2i use buffer 0, 2i + 1 buffer 1; each step copies the next k
  // tile from its segment and the last step copies nothing.  The k tile
  // counts of the whole range and of the first segment are even (checked by
  // the launchers and implied by the tile sizes): an odd tail as a third copy
  // of the step made the compiler spill the accumulators.
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // k tiles [k0, k1) of one segment through `copy`; `last_copy` copies the
  // tile after the segment's last (the next segment's first, or nullptr)
  auto segment = [&](auto step, int k0, int k1, auto copy, auto last_copy) {
    int kt = k0;
    for (; kt + 2 < k1; kt += 2) {
      step(B0{}, copy, kt);
      step(B1{}, copy, kt + 1);
    }
    step(B0{}, copy, kt);
    step(B1{}, last_copy, kt + 1);
  };
  auto run = [&](auto step) {
    if constexpr (SEG2) {
      // segment 0: tiles [0, nk0); segment 1: [nk0, nk)
      if (nk0 == nk) {
        segment(step, 0, nk, copy0, nullptr);
      } else {
        const Seg seg1 = make_seg(1);
        auto copy1 = [&](int kt, int buf) { issue(seg1, (kt - nk0) * ROWB, buf); };
        if (nk0 > 0) segment(step, 0, nk0, copy0, copy1);
        segment(step, nk0, nk, copy1, nullptr);
      }
    } else {
      segment(step, 0, nk, copy0, nullptr);
    }
  };
  // the first k tile
  if (!SEG2 || nk0 > 0) {
    copy0(0, 0);
  } else {
    const Seg seg1 = make_seg(1);
    issue(seg1, 0, 0);
  }
  if (!has_rows) {
    run(copy_only);
    return;
  }
  run(body);

  if constexpr (GROUPED && P::kStagedStore && TN == 8 && TM == 4) {
    // through stage buffer 0, which the last k tile (buffer 1) does not read
    // and whose last reader finished before every wave passed that tile's
    // barrier: 8 KB per wave, two passes of 64 columns
    char* const reg = smem + w * (64 * 128);
    const int wr = wm * (BM / WM), wc = n0 + wn * (BN / WN);
    staged_store<4, 0>(p, reg, lane, acc, m0 + wr, mcount - wr, wc);
    staged_store<4, 4>(p, reg, lane, acc, m0 + wr, mcount - wr, wc + 64);
    return;
  }
  const int ncol = (lane >> 4) * 4;
#pragma unroll
  for (int g = 0; g < TN; ++g)
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int i = wm * (BM / WM) + t * 16 + r16;
      if (i < mcount) p.store(e, m0 + i, n0 + wn * (BN / WN) + g * 16 + ncol, acc[g][t]);
    }
}

template <class P, bool GROUPED, int BM, int BN, int SCHED>
__global__ __launch_bounds__(512) void lds_gemm_kernel(P p, int mrows, const Tile* tiles,
                                                       const int* ntiles) {
  lds_gemm_body<P, GROUPED, BM, BN, TwoSegments<P>::value ? 0 : SCHED>(p, mrows, tiles, ntiles);
}

// Half-step pipelined LDS GEMM: the tiles and the 2 x 4 wave layout of
// lds_gemm_body (expert down projection: 128 x 512 tiles; whole-k dense
// projections: 256 x 256, the output projection's two k segments included),
// with the copies in half-steps.  Half-step s = 2 kt + h multiplies k tile kt
// of the token rows with weight rows BN/2 h .. BN/2 h + BN/2 - 1 of the
// block; each wave owns BM/2 token rows x BN/8 weight rows of each half
// (BN/4 weight rows in all, as in lds_gemm_body, in two pieces).  The copy
// unit of half-step s is weight half h of k tile kt, plus kt's token rows
// when h = 0.  Units are issued L half-steps ahead into a ring of L + 1
// weight-half buffers and two token buffers, so the wait at the top of a
// half-step leaves the next L - 1 units in flight: the copy stream never
// drains, where one stage ahead drained it at every k tile.  Token fragments
// are read at h = 0 and kept in registers for h = 1.  Each output element
// sees the MFMAs in the order of lds_gemm_body (k tiles ascending, k halves
// 0 then 1), so the bits match.
// Every wave copies its token rows whole (rows past the tile's count read
// its first row): the wait counts below assume a fixed number of copies per
// unit.  Every wave also runs all its MFMAs, those of token rows past the
// count included (their outputs are not stored): measured on the prefill and
// skewed batches, skipping the 16-row groups past the count made the down
// projection 3% slower (4.28-4.36 against 4.15-4.24 ms, same bits), since
// partly filled tiles then run ahead of the full tiles that share their
// weight panel and stop meeting them in L2.
template <class P, bool GROUPED, int BM, int BN, int L>
__device__ __forceinline__ void lds_pipe_body(const P& p, int mrows, const Tile* tiles,
                                              const int* ntiles) {
  constexpr int BH = BN / 2, WM = 2, WN = 4, NW = WM * WN, BK = 64;
  constexpr int TM = BM / WM / 16, TH = BH / WN / 16;
  constexpr int RPI = 8, ROWB = BK * 2;
  constexpr int NIA = BM / RPI / NW, NIH = BH / RPI / NW;
  constexpr int ABUF = BM * ROWB, HBUF = BH * ROWB, NB = L + 1;
  constexpr bool SEG2 = TwoSegments<P>::value;
  static_assert(NIA * RPI * NW == BM && NIH * RPI * NW == BH, "rows per unit");
  static_assert(L == 2 || L == 3, "lookahead");
  static_assert(2 * ABUF + NB * HBUF <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char smem[2 * ABUF + NB * HBUF];

  int tm, nb;
  if (!work_item_uniform<GROUPED>(p.N() / BN, mrows, BM, tiles, ntiles, tm, nb)) return;
  int e = 0, m0, mcount;
  if (GROUPED) {
    e = uniform(tiles[tm].expert);
    m0 = uniform(tiles[tm].row0);
    mcount = uniform(tiles[tm].nrows);
  } else {
    m0 = tm * BM;
    mcount = min(BM, mrows - m0);
  }
  const int n0 = nb * BN;
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int wm = w / WN, wn = w % WN;
  const int nk = p.K() / BK;
  const int nk0 = SEG2 ? p.K0() / BK : nk;
  const int nsub = 2 * nk;

  // copy sources of one k segment, as in lds_gemm_body: instruction j of
  // wave w fills rows RPI (w + NW j) .. + 7 of its buffer, already swizzled;
  // token rows past the tile's count read its first row
  const int lr = lane >> 3;
  const int sw = ((4 * (w & 1)) + (lr >> 1)) & 7;
  const uint32_t chunk = (uint32_t)(((lane & 7) ^ sw) * 16);
  struct Seg {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t ao[NIA];
    uint32_t bo;
    int b0, bstep, bhalf;
  };
  auto make_seg = [&](int seg) __attribute__((always_inline)) {
    Seg g;
    const char* pa = GROUPED && P::kGatherA
                         ? reinterpret_cast<const char*>(seg ? p.a_base1() : p.a_base0())
                         : reinterpret_cast<const char*>(seg ? p.a_row1(m0) : p.a_row0(m0));
#pragma unroll
    for (int j = 0; j < NIA; ++j) {
      const int row = RPI * (w + NW * j) + lr;
      const int m = m0 + (row < mcount ? row : 0);
      g.ao[j] = (uint32_t)(reinterpret_cast<const char*>(seg ? p.a_row1(m) : p.a_row0(m)) - pa) +
                chunk;
    }
    const char* pb = reinterpret_cast<const char*>(seg ? p.b_row1(e, n0) : p.b_row0(e, n0));
    const int ldb = (int)(seg ? p.ldb1() : p.ldb0()) * 2;
    g.bo = (uint32_t)(lr * ldb) + chunk;
    g.b0 = RPI * w * ldb;
    g.bstep = RPI * NW * ldb;
    g.bhalf = BH * ldb;
    g.ra = buffer_rsrc(pa);
    g.rb = buffer_rsrc(pb);
    return g;
  };
  const Seg g0 = make_seg(0);
  const Seg g1 = SEG2 && nk0 < nk ? make_seg(1) : g0;
  char* const sa0 = smem;
  char* const sb0 = smem + 2 * ABUF;

  // issue copy unit u (its half H = u % 2 known here) from segment g, k
  // tile kt at byte offset kb within that segment's rows
  auto issue_seg = [&](auto h_c, const Seg& g, int u, int kb) __attribute__((always_inline)) {
    constexpr int H = decltype(h_c)::value;
    if constexpr (H == 0) {
      char* st = sa0 + ((u >> 1) & 1) * ABUF;
#pragma unroll
      for (int j = 0; j < NIA; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(g.ra, (lds_void*)(st + (w + NW * j) * RPI * ROWB),
                                                 16, g.ao[j], kb, 0, 0);
    }
    char* st = sb0 + (u % NB) * HBUF;
#pragma unroll
    for (int j = 0; j < NIH; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(g.rb, (lds_void*)(st + (w + NW * j) * RPI * ROWB),
                                               16, g.bo, kb + g.b0 + j * g.bstep + H * g.bhalf, 0,
                                               0);
  };
  // both segments issue the same copies, so the wait counts hold across the
  // boundary
  auto issue = [&](auto h_c, int u) __attribute__((always_inline)) {
    const int kt = u >> 1;
    if (SEG2 && kt >= nk0) issue_seg(h_c, g1, u, (kt - nk0) * ROWB);
    else issue_seg(h_c, g0, u, kt * ROWB);
  };
  // wait until unit s has landed: the later units in flight are s + 1 ..
  // min(s + L - 1, nsub - 1), NIH copies each plus NIA for even ones
  auto wait_unit = [&](auto h_c, int s) __attribute__((always_inline)) {
    constexpr int H = decltype(h_c)::value;
    if constexpr (L == 3) {
      if (s + 2 < nsub) wait_vmcnt<2 * NIH + NIA>();
      else if (H == 0 && s + 1 < nsub) wait_vmcnt<NIH>();
      else wait_vmcnt<0>();
    } else {
      if (s + 1 < nsub) wait_vmcnt<H == 0 ? NIH : NIH + NIA>();
      else wait_vmcnt<0>();
    }
  };
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  using HL0 = std::integral_constant<int, (L & 1)>;      // half of unit s + L, s even
  using HL1 = std::integral_constant<int, (L & 1) ^ 1>;  // s odd

#pragma unroll
  for (int u = 0; u < L; ++u) {
    if (u & 1) issue(H1{}, u);
    else issue(H0{}, u);
  }

  const int r16 = lane & 15, kq = lane >> 4;
  const uint32_t l0 = r16 * ROWB + (((0 + kq) ^ (r16 >> 1)) << 4);
  const uint32_t l1 = r16 * ROWB + (((4 + kq) ^ (r16 >> 1)) << 4);
  const uint32_t aw = (uint32_t)(wm * (BM / WM)) * ROWB;
  const uint32_t bw = (uint32_t)(wn * (BH / WN)) * ROWB;
  f32x4 acc[2 * TH][TM];
#pragma unroll
  for (int a = 0; a < 2 * TH; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 xf[2][TM];  // token fragments of the current k tile

  auto half_step = [&](auto h_c, auto hl_c, int s) __attribute__((always_inline)) {
    constexpr int H = decltype(h_c)::value;
    wait_unit(h_c, s);
    stage_barrier_hard();
    if (s + L < nsub) issue(hl_c, s + L);
    if constexpr (H == 0) {
      const char* st = sa0 + ((s >> 1) & 1) * ABUF + aw;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int t = 0; t < TM; ++t)
          xf[ks][t] = *reinterpret_cast<const bf16x8*>(st + (ks ? l1 : l0) + t * 16 * ROWB);
    }
    const char* st = sb0 + (s % NB) * HBUF + bw;
    bf16x8 wf[2][TH];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int g = 0; g < TH; ++g)
        wf[ks][g] = *reinterpret_cast<const bf16x8*>(st + (ks ? l1 : l0) + g * 16 * ROWB);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int g = 0; g < TH; ++g)
          acc[H * TH + g][t] = mfma_bf16(wf[ks][g], xf[ks][t], acc[H * TH + g][t]);
  };
  for (int s = 0; s < nsub; s += 2) {
    half_step(H0{}, HL0{}, s);
    half_step(H1{}, HL1{}, s + 1);
  }

  const int wr = wm * (BM / WM);
  if constexpr (GROUPED && P::kStagedStore && TH == 4 && TM == 4) {
    // through LDS away from the weight-half buffer of the last half-step
    // (rows past the tile's count are not stored): every wave passed that
    // half-step's barrier, so every other buffer's last reader is done, and
    // every copy has landed (vmcnt(0) above)
    const int last = (nsub - 1) % NB;
    char* const reg = smem + (last == 0 ? 2 * ABUF + HBUF : 0) + w * (64 * 128);
    staged_store<4, 0>(p, reg, lane, acc, m0 + wr, mcount - wr, n0 + wn * (BH / WN));
    staged_store<4, 4>(p, reg, lane, acc, m0 + wr, mcount - wr, n0 + BH + wn * (BH / WN));
    return;
  }
  const int ncol = (lane >> 4) * 4;
#pragma unroll
  for (int g = 0; g < 2 * TH; ++g)
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int i = wr + t * 16 + r16;
      const int n = n0 + (g / TH) * BH + wn * (BH / WN) + (g % TH) * 16 + ncol;
      if (i < mcount) p.store(e, m0 + i, n, acc[g][t]);
    }
}

template <class P, bool GROUPED, int BM, int BN, int L>
__global__ __launch_bounds__(512) void lds_pipe_kernel(P p, int mrows, const Tile* tiles,
                                                       const int* ntiles) {
  lds_pipe_body<P, GROUPED, BM, BN, L>(p, mrows, tiles, ntiles);
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

// ---- MXFP4 expert GEMM with the codes staged in LDS --------------------------
//
// Large batches with MXFP4 expert weights: the weight side of each stage is
// copied into LDS as FP4 codes and scale bytes (a quarter of the bf16 bytes)
// and decoded to bf16 in registers right before the MFMAs, so the copy
// stream into LDS per flop is 2.4x smaller than with bf16 weights (the
// stream that bounds the bf16 expert GEMMs).  Tile: 128 token rows x 512
// weight rows, eight waves in WM x (8 / WM) (WM = 2: 64 x 128 accumulators
// each; WM = 1: 128 x 64, each decoded weight fragment then feeding eight
// MFMAs instead of four), k in stages of 128, two stages in LDS (2 x 64 KB)
// plus the scale bytes of two groups of four stages (2 x 8 KB), everything
// copied with 16-byte direct loads.
//
// k assignment inside a stage: MFMA lane (r, q) (q = lane / 16) covers the
// 32 consecutive k of block q of the stage (one scale byte) and step s of
// the four MFMAs per stage takes its k q*32 + 8s .. + 7; the token
// fragment of that lane and step is loaded at the same k, so both operands
// agree on which 32 k one MFMA sums over (any such bijection gives the same
// dot products, rounded in a different order).  A lane's codes for a stage
// are then one 16-byte LDS read per row group and its scale one byte.
//
// LDS rows are XOR-swizzled: token row t (256 bytes) keeps its 16-byte chunk
// c at c ^ (t % 16); code row n (64 bytes) its chunk q at q ^ ((n / 4) % 4).
template <class P, int BM, int BN, int WM = 2>
__device__ __forceinline__ void lds_mx_body(const P& p, const Tile* tiles, const int* ntiles) {
  constexpr int WN = 8 / WM, NW = WM * WN, BK = 128;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int AROW = BK * 2, CROW = BK / 2;   // bytes per token row, per code row
  constexpr int AST = BM * AROW, CST = BN * CROW;
  constexpr int STAGE = AST + CST;
  constexpr int SGRP = BN * 16;                 // scale bytes of 4 stages (16 per row)
  constexpr int NIA = BM / 4 / NW;              // token copies per wave: 4 rows of 256 B each
  constexpr int NIC = BN / 16 / NW;             // code copies per wave: 16 rows of 64 B each
  static_assert(NIA * 4 * NW == BM && NIC * 16 * NW == BN && BN == 64 * NW, "tile");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE + 2 * SGRP];

  int tm, nb;
  if (!work_item_uniform<true>(p.N() / BN, 0, BM, tiles, ntiles, tm, nb)) return;
  const int e = uniform(tiles[tm].expert);
  const int m0 = uniform(tiles[tm].row0);
  const int mcount = uniform(tiles[tm].nrows);
  const int n0 = nb * BN;
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int wm = w / WN, wn = w % WN;
  const int K = p.K();
  const int nk = K / BK;

  // token copies: instruction j of wave w fills rows 4 (w + NW j) .. + 3,
  // lane l row + l / 16, LDS slot l % 16 holding chunk (l % 16) ^ (row % 16).
  // Offsets are taken from the tile's first row; they are not negative, as
  // the dispatch keeps an expert's rows in token order (gathered rows) and
  // rows read in place follow each other.
  const char* abase = reinterpret_cast<const char*>(p.a_row(m0));
  uint32_t aoff[NIA];
#pragma unroll
  for (int j = 0; j < NIA; ++j) {
    const int row = 4 * (w + NW * j) + (lane >> 4);
    const int m = m0 + (row < mcount ? row : 0);
    const uint32_t chunk = (uint32_t)(((lane & 15) ^ (row & 15)) * 16);
    aoff[j] = (uint32_t)(reinterpret_cast<const char*>(p.a_row(m)) - abase) + chunk;
  }
  // code copies: instruction j of wave w fills rows 16 (w + NW j) .. + 15,
  // lane l row + l / 4, slot l % 4 holding chunk (l % 4) ^ ((row / 4) % 4);
  // rows of different j differ by a uniform stride
  const char* cbase = reinterpret_cast<const char*>(p.codes_row(e, n0));
  const int crow_bytes = K / 2;
  const uint32_t coff =
      (uint32_t)((lane >> 2) * crow_bytes + (((lane & 3) ^ ((lane >> 4) & 3)) * 16));
  // scale copies, once per 4 stages into one of two buffers: one per wave,
  // lane l row 64 w + l, 16 bytes (the 16 blocks of 32 k of those stages);
  // per stage a 4-byte copy would make 512 row requests for 2 KB
  const char* sbase = reinterpret_cast<const char*>(p.scales_row(e, n0));
  const int srow_bytes = K / 32;
  const uint32_t soff = (uint32_t)((64 * w + lane) * srow_bytes);
  char* const sbuf = smem + 2 * STAGE;
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(abase);
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(cbase);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(sbase);

  auto issue = [&](int kt, int buf, bool scales) __attribute__((always_inline)) {
    char* st = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < NIA; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + (w + NW * j) * 4 * AROW), 16,
                                               aoff[j], kt * AROW, 0, 0);
#pragma unroll
    for (int j = 0; j < NIC; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rc, (lds_void*)(st + AST + (w + NW * j) * 16 * CROW), 16, coff,
          kt * CROW + 16 * (w + NW * j) * crow_bytes, 0, 0);
    if (scales)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (lds_void*)(sbuf + ((kt >> 2) & 1) * SGRP + 64 * w * 16), 16, soff, kt * 4, 0, 0);
  };

  // fragment reads (see the k assignment above)
  const int r16 = lane & 15, kq = lane >> 4;
  const uint32_t ard = (uint32_t)((wm * (BM / WM) + r16) * AROW);   // + t * 16 rows
  const uint32_t crd =
      (uint32_t)(AST + (wn * (BN / WN) + r16) * CROW + ((kq ^ ((r16 >> 2) & 3)) << 4));
  const uint32_t srd = (uint32_t)((wn * (BN / WN) + r16) * 16 + kq);   // + 4 (stage % 4)
  const bool has_rows = wm * (BM / WM) < mcount;

  f32x4 acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // step kt (buffer BUF = kt % 2, Q = kt % 4): copy stage kt + 1 (and, when
  // it starts a group of 4, that group's scales) unless COPY is false
  auto body_ta = [&](auto q_c, auto copy_c, int kt, auto ta_c) __attribute__((always_inline)) {
    constexpr int Q = decltype(q_c)::value, BUF = Q & 1;
    constexpr int TA = decltype(ta_c)::value;  // token groups computed
    wait_vmcnt<0>();
    stage_barrier_hard();
    if constexpr (decltype(copy_c)::value) issue(kt + 1, BUF ^ 1, Q == 3);
    const char* ss = sbuf + ((kt >> 2) & 1) * SGRP + Q * 4;
    const char* st = smem + BUF * STAGE;
    u32x4 code[TN];
    float sc[TN];
#pragma unroll
    for (int g = 0; g < TN; ++g) {
      code[g] = *reinterpret_cast<const u32x4*>(st + crd + g * 16 * CROW);
      sc[g] = mx_scale(*reinterpret_cast<const uint8_t*>(ss + srd + g * 16 * 16));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 xf[TA];
#pragma unroll
      for (int t = 0; t < TA; ++t)
        xf[t] = *reinterpret_cast<const bf16x8*>(st + ard + t * 16 * AROW +
                                                 ((((kq << 2) + s) ^ r16) << 4));
#pragma unroll
      for (int g = 0; g < TN; ++g) {
        const bf16x8 wf = mx_decode8(code[g][s], sc[g]);
#pragma unroll
        for (int t = 0; t < TA; ++t) acc[g][t] = mfma_bf16(wf, xf[t], acc[g][t]);
      }
    }
  };
  // the step computing the first TA token groups only (the wave's rows past
  // them are padding of the tile)
  auto body_of = [&](auto ta_c) __attribute__((always_inline)) {
    return [&, ta_c](auto q_c, auto copy_c, int kt) __attribute__((always_inline)) {
      body_ta(q_c, copy_c, kt, ta_c);
    };
  };
  auto copy_only = [&](auto q_c, auto copy_c, int kt) __attribute__((always_inline)) {
    constexpr int Q = decltype(q_c)::value, BUF = Q & 1;
    wait_vmcnt<0>();
    stage_barrier_hard();
    if constexpr (decltype(copy_c)::value) issue(kt + 1, BUF ^ 1, Q == 3);
  };
  // the stage count is a multiple of 4 (checked by the launcher); the last
  // step copies nothing
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
  using Yes = std::true_type;
  using No = std::false_type;
  auto run = [&](auto step) __attribute__((always_inline)) {
    int kt = 0;
    for (; kt + 4 < nk; kt += 4) {
      step(Q0{}, Yes{}, kt);
      step(Q1{}, Yes{}, kt + 1);
      step(Q2{}, Yes{}, kt + 2);
      step(Q3{}, Yes{}, kt + 3);
    }
    step(Q0{}, Yes{}, kt);
    step(Q1{}, Yes{}, kt + 1);
    step(Q2{}, Yes{}, kt + 2);
    step(Q3{}, No{}, kt + 3);
  };
  issue(0, 0, true);
  if (!has_rows) {  // no token rows for this wave: copies only
    run(copy_only);
    return;
  }
  // With one wave along the tokens every wave computes all BM rows, so a
  // partly filled tile takes one of four copies of the k loop: the first
  // quarter, half, three quarters or all of its token groups.  Measured at
  // the prefill batch (same bits): up projection 3.40-3.41 -> 3.19-3.22 ms,
  // down 3.24-3.26 -> 3.13-3.14 ms (halves only: 3.24-3.25 and 3.14-3.18).
  // (Skipping each padding group's MFMAs by a branch inside the step
  // instead was slower than computing them: 3.55-3.61 and 3.61 ms.)
  if constexpr (WM == 1 && TM % 4 == 0) {
    if (mcount <= BM / 4)
      run(body_of(std::integral_constant<int, TM / 4>{}));
    else if (mcount <= BM / 2)
      run(body_of(std::integral_constant<int, TM / 2>{}));
    else if (mcount <= 3 * BM / 4)
      run(body_of(std::integral_constant<int, 3 * TM / 4>{}));
    else
      run(body_of(std::integral_constant<int, TM>{}));
  } else {
    run(body_of(std::integral_constant<int, TM>{}));
  }

  if constexpr (P::kStagedStore && WM == 1) {
    // 16 KB per wave over both stage buffers, after a barrier (every wave
    // is done reading them; with WM = 1 every wave has rows, so every wave
    // of the work-group reaches it)
    static_assert(BN / WN == 64 && TN == 4 && BM * 128 * NW <= 2 * STAGE, "staged store");
    stage_barrier_hard();
    staged_store<4, 0>(p, smem + w * (BM * 128), lane, acc, m0, mcount, n0 + wn * 64);
    return;
  }
  const int ncol = (lane >> 4) * 4;
#pragma unroll
  for (int g = 0; g < TN; ++g)
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int i = wm * (BM / WM) + t * 16 + r16;
      if (i < mcount) p.store(e, m0 + i, n0 + wn * (BN / WN) + g * 16 + ncol, acc[g][t]);
    }
}

template <class P, int BM, int BN, int WM = 2>
__global__ __launch_bounds__(512) void lds_mx_kernel(P p, const Tile* tiles, const int* ntiles) {
  lds_mx_body<P, BM, BN, WM>(p, tiles, ntiles);
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
  static_assert(NS == 2 && BK == 64, "dense tiles");
  // the half-step kernel, three units ahead: on the prefill batch (same bits)
  // the output projection 1.463-1.468 -> 1.430-1.433 ms and the latent
  // projection 0.245 -> 0.236 ms against lds_gemm_kernel, the forward
  // 11.37-11.38 -> 11.29-11.30 ms (two A/B rounds on one box)
  if (p.K() % 128 == 0)
    lds_pipe_kernel<P, false, BM, BN, 3><<<grid, 512, 0, s>>>(p, T, nullptr, nullptr);
  else
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
  bool done = false;
  if constexpr (NS == 2) {
    if (sp.K() % 128 == 0) {
      lds_gemm_kernel<SplitK<P>, false, BM, BN, 1>
          <<<dim3(gx, nsplit), 512, 0, s>>>(sp, T, nullptr, nullptr);
      done = true;
    }
  }
  if (!done)
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
// T = 192 (speculative-verify batch), reduction included: output projection
// 192x128 with four stages in 4 splits (52-53 us against 61-63 for 256x256
// in 8 splits and 145 for the best weight-streaming shape: one tile covers
// the batch's rows, and three stages are in flight), latent 128x128 in 8
// splits (20.5 us against 26.5-27.1 for 128x256 with 3 stages; 192-row tiles
// within 1 us), shared up 128x128 in 4 splits (56.5-57.4 us against
// 58.1-59.8 for 256x256, 56-63 for 192x128).  With the same split count the
// tile shape leaves every output bit unchanged.
hipError_t split_proj_in(const ProjIn& p, float* part, hipStream_t s) {
  if (p.N() <= 4096)
    return launch_split<ProjIn, 128, 128, 2>(p, p.T, part, pick_splits(p.K(), kSplitMax), s);
  return launch_split<ProjIn, 128, 128, 2>(p, p.T, part, pick_splits(p.K(), 4), s);
}
hipError_t split_proj_out(const ProjOut& p, float* part, hipStream_t s) {
  if (p.T <= 192 && p.N() % 128 == 0)
    return launch_split<ProjOut, 192, 128, 4>(p, p.T, part, pick_splits(p.K(), 4), s);
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

// Expert up projection: lds_gemm_kernel when N allows 512-row weight tiles
// and every gathered latent row lies within the 2 GiB its buffer offsets
// reach from the latent array's start (a row index is below the token
// count).
hipError_t tiled_exp_up(const ExpUp& p, const Tile* tiles, const int* ntiles, int max_tiles,
                        int tokens, hipStream_t s) {
  if (p.N() % 512 == 0 && p.K() % 128 == 0 && (long)tokens * p.K() * 2 < (1L << 31)) {
    const long grid = xcd_grid((long)max_tiles * (p.N() / 512));
    if (grid <= 0) return hipSuccess;
    lds_gemm_kernel<ExpUp, true, kExpBM, 512, 0><<<grid, 512, 0, s>>>(p, 0, tiles, ntiles);
    return hipGetLastError();
  }
  return launch_expert(p, tiles, ntiles, max_tiles, s);
}
// Expert down projection: the half-step kernel (lds_pipe_kernel, three
// units ahead) when N allows 512-row weight tiles (its token rows are read in
// place, within the tile's 128).  Measured on the prefill and skewed batches
// against lds_gemm_kernel on one box, same bits: 4.20-4.26 against 4.42-4.59
// ms (two units ahead: 4.32), and 4.15-4.24 once it ran the MFMAs of partly
// filled tiles' padding rows too.  The up projection (32 k tiles of 2048
// against the down projection's 80) was slower on it either way, 4.51-4.66
// against 4.47-4.53 ms, and keeps lds_gemm_kernel.
hipError_t tiled_exp_down(const ExpDown& p, const Tile* tiles, const int* ntiles, int max_tiles,
                          hipStream_t s) {
  if (p.N() % 512 == 0 && p.K() % 128 == 0) {
    const long grid = xcd_grid((long)max_tiles * (p.N() / 512));
    if (grid <= 0) return hipSuccess;
    lds_pipe_kernel<ExpDown, true, kExpBM, 512, 3><<<grid, 512, 0, s>>>(p, 0, tiles, ntiles);
    return hipGetLastError();
  }
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
// lds_mx_kernel where its shape conditions hold: N a multiple of 512, K a
// multiple of 512 (whole groups of four 128-k stages, whose 16 scale bytes
// per row are then one aligned 16-byte piece), the scales 16-byte aligned,
// and the token rows' byte offsets from the tile's first row within the
// 2 GiB its buffer offsets reach, which holds while `a_rows` rows do:
// gathered rows (up projection; `a_rows` = the token count) are one expert's
// tokens in ascending order, so they lie after the tile's first row by less
// than the token count; rows read in place (down projection) lie within the
// tile's 128.  Wave layout 1 x 8, whose 128 x 64 blocks go out through LDS
// (staged_store).  Measured at the prefill batch (T = 8192, all three give the
// same bits), with direct stores 1 x 8 took the down projection from 3.38 to
// 3.28 ms and left the up projection within run-to-run noise (3.44 to 3.51
// ms for both layouts).
template <class P>
static hipError_t launch_lds_mx(const P& p, const Tile* tiles, const int* ntiles, int max_tiles,
                                long a_rows, hipStream_t s) {
  const long a_span = a_rows * p.K() * 2;
  if (p.N() % 512 == 0 && p.K() % 512 == 0 && (reinterpret_cast<uintptr_t>(p.scales) & 15) == 0 &&
      a_span < (1L << 31)) {
    const long grid = xcd_grid((long)max_tiles * (p.N() / 512));
    if (grid <= 0) return hipSuccess;
    lds_mx_kernel<P, kExpBM, 512, 1><<<grid, 512, 0, s>>>(p, tiles, ntiles);
    return hipGetLastError();
  }
  return launch_expert_mx(p, tiles, ntiles, max_tiles, s);
}

hipError_t tiled_mx_exp_up(const ExpUpMx& p, const Tile* tiles, const int* ntiles, int max_tiles,
                           int tokens, hipStream_t s) {
  return launch_lds_mx(p, tiles, ntiles, max_tiles, tokens, s);
}
hipError_t tiled_mx_exp_down(const ExpDownMx& p, const Tile* tiles, const int* ntiles,
                             int max_tiles, hipStream_t s) {
  return launch_lds_mx(p, tiles, ntiles, max_tiles, kExpBM, s);
}

}  // namespace lmoe
