// Weight-streaming GEMM for small token counts (decode-sized batches).
//
// With few tokens every GEMM of the layer is bound by reading its weights
// from HBM once; the page's own accounting puts decode on weight I/O and
// prefill on compute ("Nemotron 3 架构解读", the decode/prefill discussion).
// So this kernel is built around one thing: every weight byte is read
// exactly once, with many 16-byte loads in flight per wave, and turned into
// MFMA operands straight from registers (no LDS staging of weights).
//
// Work-group = NW waves on one block of 64 weight rows (4 MFMA row groups of
// 16) and MT*16 token rows.  The k range is split evenly over the NW waves
// (so many waves stream disjoint parts of the same rows); each wave keeps a
// double-buffered register pipeline of 2 x (4 weight + MT activation)
// fragments per 32-wide k step, then the waves' partial sums are added in
// LDS in a fixed order (deterministic) and the problem's epilogue stores.
//
// Weights are the MFMA A operand (rows = output columns n), activations the
// B operand (columns = tokens), so each lane ends with four consecutive
// output columns of one token: an 8- or 16-byte store.
#include "gemm_problems.h"
#include "kernels.h"

namespace lmoe {

constexpr int kRG = 4;   // 16-row groups of weights per work-group (64 rows)
constexpr int kU = 2;    // k steps of 32 per pipeline stage

template <class P, bool GROUPED, int NW, int MT>
__global__ __launch_bounds__(NW * 64) void stream_gemm_kernel(P p, int mrows, const Tile* tiles,
                                                              const int* ntiles) {
  constexpr int J = kRG * MT;
  __shared__ f32x4 red[NW > 1 ? NW : 1][J][64];

  const int nblocks = p.N() / (16 * kRG);
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
    m0 = tm * (16 * MT);
    mcount = min(16 * MT, mrows - m0);
  }
  const int n0 = nb * (16 * kRG);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int K = p.K(), K0 = p.K0();
  const int kw = K / NW;
  const int kbeg = w * kw;
  const int nit = kw / (32 * kU);

  const uint16_t* b0[kRG];
  const uint16_t* b1[kRG];
#pragma unroll
  for (int g = 0; g < kRG; ++g) {
    b0[g] = p.b_row0(e, n0 + g * 16 + r16) + kq;
    const uint16_t* q = p.b_row1(e, n0 + g * 16 + r16);
    b1[g] = q ? q + kq : nullptr;
  }
  const uint16_t* a0[MT];
  const uint16_t* a1[MT];
  bool av[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int i = t * 16 + r16;
    av[t] = i < mcount;
    a0[t] = av[t] ? p.a_row0(m0 + i) + kq : nullptr;
    const uint16_t* q = av[t] ? p.a_row1(m0 + i) : nullptr;
    a1[t] = q ? q + kq : nullptr;
  }

  f32x4 acc[kRG][MT];
#pragma unroll
  for (int g = 0; g < kRG; ++g)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 wA[kU][kRG], xA[kU][MT], wB[kU][kRG], xB[kU][MT];

  auto load = [&](bf16x8(&wf)[kU][kRG], bf16x8(&xf)[kU][MT], int it) {
    const int k = kbeg + it * (32 * kU);
    const bool s0 = k < K0;
    const int kk = s0 ? k : k - K0;
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int g = 0; g < kRG; ++g) wf[u][g] = load8_stream((s0 ? b0[g] : b1[g]) + kk + u * 32);
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t)
        xf[u][t] = av[t] ? load8((s0 ? a0[t] : a1[t]) + kk + u * 32) : zero8();
  };
  auto compute = [&](const bf16x8(&wf)[kU][kRG], const bf16x8(&xf)[kU][MT]) {
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int g = 0; g < kRG; ++g)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[g][t] = mfma_bf16(wf[u][g], xf[u][t], acc[g][t]);
  };

  if (nit > 0) load(wA, xA, 0);
  for (int it = 0; it < nit; it += 2) {
    if (it + 1 < nit) load(wB, xB, it + 1);
    compute(wA, xA);
    if (it + 1 < nit) {
      if (it + 2 < nit) load(wA, xA, it + 2);
      compute(wB, xB);
    }
  }

  const int ncol = (lane >> 4) * 4;
  if constexpr (NW == 1) {
#pragma unroll
    for (int g = 0; g < kRG; ++g)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int i = t * 16 + r16;
        if (i < mcount) p.store(e, m0 + i, n0 + g * 16 + ncol, acc[g][t]);
      }
  } else {
#pragma unroll
    for (int g = 0; g < kRG; ++g)
#pragma unroll
      for (int t = 0; t < MT; ++t) red[w][g * MT + t][lane] = acc[g][t];
    __syncthreads();
    for (int j = w; j < J; j += NW) {
      f32x4 s = red[0][j][lane];
#pragma unroll
      for (int v = 1; v < NW; ++v) s += red[v][j][lane];
      const int g = j / MT, t = j % MT;
      const int i = t * 16 + r16;
      if (i < mcount) p.store(e, m0 + i, n0 + g * 16 + ncol, s);
    }
  }
}

// Waves per work-group: the fewest that still give about two waves per
// SIMD over the whole launch, subject to the k range splitting evenly into
// 64-wide pipeline stages (and the segment boundary falling on one).
static int pick_nw(int K, int K0, long blocks) {
  const int opts[4] = {1, 2, 4, 8};
  int best = 1;
  for (int i = 0; i < 4; ++i) {
    const int nw = opts[i];
    if (K % (nw * 32 * kU) != 0) continue;
    best = nw;
    if (blocks * nw >= 2048) break;
  }
  (void)K0;
  return best;
}

template <class P, bool GROUPED, int MT>
static hipError_t launch_mt(const P& p, int nw, long grid, int mrows, const Tile* tiles,
                            const int* ntiles, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  switch (nw) {
    case 1: stream_gemm_kernel<P, GROUPED, 1, MT><<<grid, 64, 0, s>>>(p, mrows, tiles, ntiles); break;
    case 2: stream_gemm_kernel<P, GROUPED, 2, MT><<<grid, 128, 0, s>>>(p, mrows, tiles, ntiles); break;
    case 4: stream_gemm_kernel<P, GROUPED, 4, MT><<<grid, 256, 0, s>>>(p, mrows, tiles, ntiles); break;
    default: stream_gemm_kernel<P, GROUPED, 8, MT><<<grid, 512, 0, s>>>(p, mrows, tiles, ntiles); break;
  }
  return hipGetLastError();
}

template <class P>
static hipError_t launch_dense(const P& p, int N, int K, int K0, int T, hipStream_t s) {
  const int mt = T <= 16 ? 1 : (T <= 32 ? 2 : 4);
  const long mtiles = (T + 16 * mt - 1) / (16 * mt);
  const long nblocks = N / (16 * kRG);
  const long grid = mtiles * nblocks;
  const int nw = pick_nw(K, K0, grid);
  switch (mt) {
    case 1: return launch_mt<P, false, 1>(p, nw, grid, T, nullptr, nullptr, s);
    case 2: return launch_mt<P, false, 2>(p, nw, grid, T, nullptr, nullptr, s);
    default: return launch_mt<P, false, 4>(p, nw, grid, T, nullptr, nullptr, s);
  }
}

template <class P>
static hipError_t launch_grouped(const P& p, int N, int K, const Tile* tiles, const int* ntiles,
                                 int max_tiles, hipStream_t s) {
  const long nblocks = N / (16 * kRG);
  const long grid = (long)max_tiles * nblocks;
  const int nw = pick_nw(K, K, grid);
  return launch_mt<P, true, 1>(p, nw, grid, 0, tiles, ntiles, s);
}

hipError_t stream_proj_in(const ProjIn& p, hipStream_t s) {
  return launch_dense(p, p.R + p.S, p.D, p.D, p.T, s);
}
hipError_t stream_proj_out(const ProjOut& p, hipStream_t s) {
  return launch_dense(p, p.D, p.R + p.S, p.R, p.T, s);
}
hipError_t stream_exp_up(const ExpUp& p, const Tile* tiles, const int* ntiles, int max_tiles,
                         hipStream_t s) {
  return launch_grouped(p, p.F, p.R, tiles, ntiles, max_tiles, s);
}
hipError_t stream_exp_down(const ExpDown& p, const Tile* tiles, const int* ntiles, int max_tiles,
                           hipStream_t s) {
  return launch_grouped(p, p.R, p.F, tiles, ntiles, max_tiles, s);
}

}  // namespace lmoe
