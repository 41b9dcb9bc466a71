// LDS-tiled bf16 MFMA GEMM for large token counts (prefill-sized batches),
// where the layer is bound by matrix-core throughput.
//
// Work-group tile: 128 token rows x 128 weight rows, k in steps of 64.  Four
// waves in a 2 x 2 arrangement each own a 64 x 64 sub-tile (4 x 4 MFMA
// 16x16x32 tiles, 64 fp32 accumulators per lane).  Global -> register
// prefetch of the next k tile overlaps the MFMAs of the current one; tiles
// are double-buffered in LDS, one barrier per k tile.  LDS rows are padded
// by 16 bytes so the 16 rows read by one MFMA fragment land in distinct banks.
//
// Grouped mode (experts): the m tiles come from the expert tile list built by
// the dispatch kernel; a tile never spans two experts, rows past the tile's
// count are zero-filled on load and masked on store.
#include "gemm_problems.h"
#include "kernels.h"

namespace lmoe {

constexpr int kBM = 128, kBN = 128, kBK = 64, kLDK = kBK + 8;

template <class P, bool GROUPED>
__global__ __launch_bounds__(256) void tiled_gemm_kernel(P p, int mrows, const Tile* tiles,
                                                         const int* ntiles) {
  __shared__ uint16_t sA[2][kBM * kLDK];
  __shared__ uint16_t sB[2][kBN * kLDK];

  const int nblocks = p.N() / kBN;
  const int nb = blockIdx.x % nblocks;
  const int tm = blockIdx.x / nblocks;
  int e = 0, m0, mcount;
  if (GROUPED) {
    if (tm >= *ntiles) return;
    const Tile t = tiles[tm];
    e = t.expert;
    m0 = t.row0;
    mcount = t.nrows;
  } else {
    m0 = tm * kBM;
    mcount = min(kBM, mrows - m0);
  }
  const int n0 = nb * kBN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int K = p.K(), K0 = p.K0();
  const int nk = K / kBK;

  // Global load assignment: 16-byte chunk c = tid + 256 j, row c / 8,
  // k offset (c % 8) * 8; eight lanes cover one 128-byte row segment.
  const int lrow = tid >> 3;
  const int lk = (tid & 7) * 8;
  const uint16_t* ga0[4];
  const uint16_t* ga1[4];
  const uint16_t* gb0[4];
  const uint16_t* gb1[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = lrow + 32 * j;
    const bool ok = row < mcount;
    ga0[j] = ok ? p.a_row0(m0 + row) + lk : nullptr;
    const uint16_t* q = ok ? p.a_row1(m0 + row) : nullptr;
    ga1[j] = q ? q + lk : nullptr;
    gb0[j] = p.b_row0(e, n0 + row) + lk;
    q = p.b_row1(e, n0 + row);
    gb1[j] = q ? q + lk : nullptr;
  }

  bf16x8 ra[4], rb[4];
  auto gload = [&](int kt) {
    const int k = kt * kBK;
    const bool s0 = k < K0;
    const int kk = s0 ? k : k - K0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ra[j] = ga0[j] ? load8((s0 ? ga0[j] : ga1[j]) + kk) : zero8();
      rb[j] = load8((s0 ? gb0[j] : gb1[j]) + kk);
    }
  };
  auto sstore = [&](int st) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = lrow + 32 * j;
      *reinterpret_cast<bf16x8*>(&sA[st][row * kLDK + lk]) = ra[j];
      *reinterpret_cast<bf16x8*>(&sB[st][row * kLDK + lk]) = rb[j];
    }
  };

  const int wm = w >> 1, wn = w & 1;
  const int r16 = lane & 15, kq = (lane >> 4) * 8;
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      bf16x8 wf[4], xf[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        wf[g] = *reinterpret_cast<const bf16x8*>(
            &sB[st][(wn * 64 + g * 16 + r16) * kLDK + ks * 32 + kq]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        xf[t] = *reinterpret_cast<const bf16x8*>(
            &sA[st][(wm * 64 + t * 16 + r16) * kLDK + ks * 32 + kq]);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[g][t] = mfma_bf16(wf[g], xf[t], acc[g][t]);
    }
    if (kt + 1 < nk) sstore(st ^ 1);
    __syncthreads();
  }

  const int ncol = (lane >> 4) * 4;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = wm * 64 + t * 16 + r16;
      if (i < mcount) p.store(e, m0 + i, n0 + wn * 64 + g * 16 + ncol, acc[g][t]);
    }
}

template <class P>
static hipError_t launch_dense(const P& p, int N, int T, hipStream_t s) {
  const long grid = (long)((T + kBM - 1) / kBM) * (N / kBN);
  if (grid <= 0) return hipSuccess;
  tiled_gemm_kernel<P, false><<<grid, 256, 0, s>>>(p, T, nullptr, nullptr);
  return hipGetLastError();
}

template <class P>
static hipError_t launch_grouped(const P& p, int N, const Tile* tiles, const int* ntiles,
                                 int max_tiles, hipStream_t s) {
  const long grid = (long)max_tiles * (N / kBN);
  if (grid <= 0) return hipSuccess;
  tiled_gemm_kernel<P, true><<<grid, 256, 0, s>>>(p, 0, tiles, ntiles);
  return hipGetLastError();
}

int tiled_block_m() { return kBM; }
int tiled_block_n() { return kBN; }

hipError_t tiled_proj_in(const ProjIn& p, hipStream_t s) { return launch_dense(p, p.ncount, p.T, s); }
hipError_t tiled_proj_out(const ProjOut& p, hipStream_t s) { return launch_dense(p, p.D, p.T, s); }
hipError_t tiled_exp_up(const ExpUp& p, const Tile* tiles, const int* ntiles, int max_tiles,
                        hipStream_t s) {
  return launch_grouped(p, p.F, tiles, ntiles, max_tiles, s);
}
hipError_t tiled_exp_down(const ExpDown& p, const Tile* tiles, const int* ntiles, int max_tiles,
                          hipStream_t s) {
  return launch_grouped(p, p.R, tiles, ntiles, max_tiles, s);
}

}  // namespace lmoe
