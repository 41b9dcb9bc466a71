// Weight-streaming GEMM for small token counts (decode-sized batches).
//
// With few tokens every GEMM of the layer is bound by reading its weights
// from HBM once; the page's own accounting puts decode on weight I/O and
// prefill on compute ("Nemotron 3 架构解读", the decode/prefill discussion).
// So this kernel is built around one thing: every weight byte is read
// exactly once, with many 16-byte loads in flight per wave, and turned into
// MFMA operands straight from registers (no LDS staging of weights).
//
// Work-group = NW waves on one block of RG*16 weight rows (RG MFMA row
// groups of 16) and MT*16 token rows.  The k range is split evenly over the
// NW waves (so many waves stream disjoint parts of the same rows); each wave
// keeps a double-buffered register pipeline of U k steps of (RG weight + MT
// activation) fragments, then the waves' partial sums are added in LDS in a
// fixed order (deterministic) and the problem's epilogue stores.
//
// Weights are the MFMA A operand (rows = output columns n), activations the
// B operand (columns = tokens), so each lane ends with four consecutive
// output columns of one token: an 8- or 16-byte store.
#include "gemm_problems.h"
#include "kernels.h"

namespace lmoe {

// NT: load weights with the non-temporal hint (kept for measurement; the
// launch shapes below use plain loads).
template <class P, bool GROUPED, int NW, int MT, int kRG, int kU, bool NT>
__global__ __launch_bounds__(NW * 64) void stream_gemm_kernel(P p, int mrows, const Tile* tiles,
                                                              const int* ntiles) {
  constexpr int J = kRG * MT;
  __shared__ f32x4 red[NW > 1 ? NW : 1][J][64];

  const int nblocks = p.N() / (16 * kRG);
  int nb, tm;
  if (GROUPED) {
    nb = blockIdx.x % nblocks;
    tm = blockIdx.x / nblocks;
  } else {
    // Dense: the m tiles that share a weight block run back to back on one
    // XCD (work-groups are dealt to the 8 XCDs round-robin by id), so the
    // block is fetched from HBM once and re-read from that XCD's L2.
    const int mtiles = (mrows + 16 * MT - 1) / (16 * MT);
    const int local = blockIdx.x / 8;
    tm = local % mtiles;
    nb = (local / mtiles) * 8 + blockIdx.x % 8;
    if (nb >= nblocks) return;
  }
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
      for (int g = 0; g < kRG; ++g) {
        const uint16_t* q = (s0 ? b0[g] : b1[g]) + kk + u * 32;
        wf[u][g] = NT ? load8_stream(q) : load8(q);
      }
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

// Launch shapes.  Measured on MI355X with the full-shape decode problems
// (T = 32, ~400 touched experts): plain loads beat the non-temporal hint for
// this access pattern (each wave instruction touches half of 16 cache lines,
// and the other half is wanted by the next instruction), and the shapes
// below were the fastest of a sweep over waves/work-group, row groups and
// pipeline depth.  A shape is used only if it divides the problem; the
// chain ends in one that always does (dimensions are multiples of 64).
struct Shape {
  int nw, rg, u;
};

static bool fits(const Shape& c, int N, int K, int K0) {
  return K % (c.nw * 32 * c.u) == 0 && K0 % (32 * c.u) == 0 && N % (16 * c.rg) == 0;
}

static Shape pick(const Shape& pref, int N, int K, int K0) {
  const Shape chain[] = {pref, {4, 2, 2}, {2, 2, 2}, {1, 2, 2}, {1, 1, 2}};
  for (const Shape& c : chain)
    if (fits(c, N, K, K0)) return c;
  return {1, 1, 2};
}

template <class P, bool GROUPED, int MT>
static hipError_t launch_shape(const P& p, const Shape& c, long mtiles, int mrows, const Tile* tiles,
                               const int* ntiles, hipStream_t s) {
  const long nblocks = p.N() / (16 * c.rg);
  const long grid = GROUPED ? mtiles * nblocks : 8 * mtiles * ((nblocks + 7) / 8);
  if (grid <= 0) return hipSuccess;
#define LMOE_SG(NW_, RG_, U_)                                                              \
  if (c.nw == NW_ && c.rg == RG_ && c.u == U_) {                                           \
    stream_gemm_kernel<P, GROUPED, NW_, MT, RG_, U_, false>                                \
        <<<grid, NW_ * 64, 0, s>>>(p, mrows, tiles, ntiles);                               \
    return hipGetLastError();                                                              \
  }
  LMOE_SG(4, 4, 2)
  LMOE_SG(4, 4, 4)
  LMOE_SG(8, 2, 4)
  LMOE_SG(4, 2, 2)
  LMOE_SG(2, 2, 2)
  LMOE_SG(1, 2, 2)
  LMOE_SG(1, 1, 2)
#undef LMOE_SG
  return hipErrorInvalidConfiguration;
}

template <class P>
static hipError_t launch_dense(const P& p, const Shape& pref, int T, hipStream_t s) {
  const int mt = T <= 16 ? 1 : (T <= 32 ? 2 : 4);
  const long mtiles = (T + 16 * mt - 1) / (16 * mt);
  const Shape c = pick(pref, p.N(), p.K(), p.K0());
  switch (mt) {
    case 1: return launch_shape<P, false, 1>(p, c, mtiles, T, nullptr, nullptr, s);
    case 2: return launch_shape<P, false, 2>(p, c, mtiles, T, nullptr, nullptr, s);
    default: return launch_shape<P, false, 4>(p, c, mtiles, T, nullptr, nullptr, s);
  }
}

template <class P>
static hipError_t launch_grouped(const P& p, const Shape& pref, const Tile* tiles,
                                 const int* ntiles, int max_tiles, hipStream_t s) {
  const Shape c = pick(pref, p.N(), p.K(), p.K0());
  return launch_shape<P, true, 1>(p, c, max_tiles, 0, tiles, ntiles, s);
}

hipError_t stream_proj_in(const ProjIn& p, hipStream_t s) {
  return launch_dense(p, Shape{4, 4, 2}, p.T, s);
}
hipError_t stream_proj_out(const ProjOut& p, hipStream_t s) {
  return launch_dense(p, Shape{4, 2, 2}, p.T, s);
}
hipError_t stream_exp_up(const ExpUp& p, const Tile* tiles, const int* ntiles, int max_tiles,
                         hipStream_t s) {
  return launch_grouped(p, Shape{4, 4, 4}, tiles, ntiles, max_tiles, s);
}
hipError_t stream_exp_down(const ExpDown& p, const Tile* tiles, const int* ntiles, int max_tiles,
                           hipStream_t s) {
  return launch_grouped(p, Shape{8, 2, 4}, tiles, ntiles, max_tiles, s);
}

}  // namespace lmoe
