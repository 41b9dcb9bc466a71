// Weight-streaming GEMM for small token counts (decode-sized batches).
//
// With few tokens every GEMM of the layer is bound by reading its weights
// from HBM once; the page's own accounting puts decode on weight I/O and
// prefill on compute ("Nemotron 3 架构解读", the decode/prefill discussion).
// So this kernel is built around one thing: every weight byte is read
// exactly once, as whole cache lines, with many loads in flight per wave.
//
// Work-group = NW waves on one block of RG*16 weight rows and MT*16 token
// rows; the k range is split evenly over the waves, whose partial sums are
// added in LDS in a fixed order (deterministic).  Weights are the MFMA A
// operand (rows = output columns), activations the B operand (columns =
// tokens), so each lane ends with four consecutive output columns of one
// token.
//
// Weight loads: one wave instruction reads 8 rows x 128 bytes (64 k), i.e.
// whole cache lines, with the non-temporal hint; two such loads (rows 0-7
// and 8-15 of a row group) hold the two 16x32 MFMA fragments of that 64-k
// chunk, and ds_bpermute moves each 16-byte piece to the lane the MFMA
// layout wants (lane (r, q) of step s takes row r, k chunk 4s + q).
// Measured on MI355X (decode expert GEMMs, ~400 experts): 6.9 TB/s, against
// 6.2-6.4 TB/s for loading the fragments directly (16 rows x 64 bytes per
// instruction, where the nt hint makes it worse, not better).
#include "gemm_problems.h"
#include "kernels.h"

namespace lmoe {

// Fragment for MFMA step s from the two 8-row loads a (rows 0-7) and b
// (rows 8-15): the lane reads byte offset src4 of the other lanes' data and
// keeps a's value for rows 0-7, b's for rows 8-15.
__device__ __forceinline__ bf16x8 permute_frag(const bf16x8& a, const bf16x8& b, int src4,
                                               bool lo) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 ai = __builtin_bit_cast(i32x4, a), bi = __builtin_bit_cast(i32x4, b);
  i32x4 r;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int va = __builtin_amdgcn_ds_bpermute(src4, ai[d]);
    const int vb = __builtin_amdgcn_ds_bpermute(src4, bi[d]);
    r[d] = lo ? va : vb;
  }
  return __builtin_bit_cast(bf16x8, r);
}

template <class P, bool GROUPED, int NW, int MT, int RG, int U>
__global__ __launch_bounds__(NW * 64) void stream_gemm_kernel(P p, int mrows, const Tile* tiles,
                                                              const int* ntiles) {
  constexpr int J = RG * MT;
  __shared__ f32x4 red[NW > 1 ? NW : 1][J][64];

  const int nblocks = p.N() / (16 * RG);
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
  const int n0 = nb * (16 * RG);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int kq = lane >> 4;
  const int K = p.K(), K0 = p.K0();
  const int kw = K / NW;
  const int kbeg = w * kw;
  const int nit = kw / (64 * U);

  // Weight load layout: lane -> row lane / 8 (+8 for the second load), k
  // chunk lane % 8.  Pointers for both k segments (segment 1 only exists for
  // the K-concatenated output projection).
  const int lrow = lane >> 3, lch = (lane & 7) * 8;
  const uint16_t* wa0[RG];
  const uint16_t* wb0[RG];
  const uint16_t* wa1[RG];
  const uint16_t* wb1[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    wa0[g] = p.b_row0(e, n0 + g * 16 + lrow) + lch;
    wb0[g] = p.b_row0(e, n0 + g * 16 + 8 + lrow) + lch;
    const uint16_t* qa = p.b_row1(e, n0 + g * 16 + lrow);
    const uint16_t* qb = p.b_row1(e, n0 + g * 16 + 8 + lrow);
    wa1[g] = qa ? qa + lch : nullptr;
    wb1[g] = qb ? qb + lch : nullptr;
  }
  // Activation rows past the tile's count read the tile's first row (their
  // outputs are never stored).
  const uint16_t* x0[MT];
  const uint16_t* x1[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int i = t * 16 + r16;
    const int row = m0 + (i < mcount ? i : 0);
    x0[t] = p.a_row0(row) + kq * 8;
    const uint16_t* q = p.a_row1(row);
    x1[t] = q ? q + kq * 8 : nullptr;
  }
  const int src0 = (((r16 & 7) << 3) | kq) * 4;
  const int src1 = (((r16 & 7) << 3) | (4 + kq)) * 4;
  const bool lo = r16 < 8;

  f32x4 acc[RG][MT];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 LA[U][RG][2], XA[U][MT][2], LB[U][RG][2], XB[U][MT][2];
  auto load = [&](bf16x8(&L)[U][RG][2], bf16x8(&X)[U][MT][2], int it) {
    const int k = kbeg + it * (64 * U);
    const bool s0 = k < K0;
    const int kk = s0 ? k : k - K0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        L[u][g][0] = load8_stream((s0 ? wa0[g] : wa1[g]) + kk + u * 64);
        L[u][g][1] = load8_stream((s0 ? wb0[g] : wb1[g]) + kk + u * 64);
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const uint16_t* x = (s0 ? x0[t] : x1[t]) + kk + u * 64;
        X[u][t][0] = load8(x);
        X[u][t][1] = load8(x + 32);
      }
    }
  };
  auto compute = [&](const bf16x8(&L)[U][RG][2], const bf16x8(&X)[U][MT][2]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const bf16x8 f0 = permute_frag(L[u][g][0], L[u][g][1], src0, lo);
        const bf16x8 f1 = permute_frag(L[u][g][0], L[u][g][1], src1, lo);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          acc[g][t] = mfma_bf16(f0, X[u][t][0], acc[g][t]);
          acc[g][t] = mfma_bf16(f1, X[u][t][1], acc[g][t]);
        }
      }
  };

  if (nit > 0) load(LA, XA, 0);
  for (int it = 0; it < nit; it += 2) {
    if (it + 1 < nit) load(LB, XB, it + 1);
    compute(LA, XA);
    if (it + 1 < nit) {
      if (it + 2 < nit) load(LA, XA, it + 2);
      compute(LB, XB);
    }
  }

  const int ncol = (lane >> 4) * 4;
  // Expert outputs are stored with the non-temporal hint: a tile's few rows
  // are scattered 32 bytes at a time over a large array while the weights
  // stream past.  Measured in the forward: decode 2.364 vs 2.376 ms,
  // speculative verify 3.372 vs 3.424 ms (standalone at T = 192, the up
  // projection takes 1582 us with plain stores, 1548 with these, 1483-1503
  // with none at all).
  auto store = [&](int m, int n, f32x4 v) __attribute__((always_inline)) {
    if constexpr (GROUPED) p.store_nt(e, m, n, v);
    else p.store(e, m, n, v);
  };
  if constexpr (NW == 1) {
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int i = t * 16 + r16;
        if (i < mcount) store(m0 + i, n0 + g * 16 + ncol, acc[g][t]);
      }
  } else if constexpr (GROUPED && MT == 1 && (RG == 2 || RG == 4) && P::kStagedStore) {
    // Wave 0 adds the waves' partial sums of all RG tiles and writes the
    // tile's 16 rows x 16 RG columns through LDS (red[0], already read), so
    // that each lane stores 16 contiguous bytes and each instruction whole
    // 32 RG-byte row pieces (in the MFMA layout a store instruction writes
    // 16 pieces of 32 bytes).
#pragma unroll
    for (int g = 0; g < RG; ++g) red[w][g][lane] = acc[g][0];
    __syncthreads();
    if (w == 0) {
      constexpr int RB = 32 * RG, CH = RB / 16, RPI = 64 / CH;
      f32x4 sm[RG];
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        sm[g] = red[0][g][lane];
#pragma unroll
        for (int v = 1; v < NW; ++v) sm[g] += red[v][g][lane];
      }
      char* const reg = reinterpret_cast<char*>(&red[0][0][0]);
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const int chunk = 2 * g + (kq >> 1);
        *reinterpret_cast<u16x4*>(reg + r16 * RB + ((chunk ^ (r16 & (CH - 1))) << 4) +
                                  (kq & 1) * 8) = p.pack4(sm[g]);
      }
      const int c = lane & (CH - 1);
#pragma unroll
      for (int j = 0; j < 16 / RPI; ++j) {
        const int i = j * RPI + lane / CH;
        const u16x8 v =
            *reinterpret_cast<const u16x8*>(reg + i * RB + ((c ^ (i & (CH - 1))) << 4));
        if (i < mcount) p.store8_nt(m0 + i, n0 + c * 8, v);
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int t = 0; t < MT; ++t) red[w][g * MT + t][lane] = acc[g][t];
    __syncthreads();
    for (int j = w; j < J; j += NW) {
      f32x4 sm = red[0][j][lane];
#pragma unroll
      for (int v = 1; v < NW; ++v) sm += red[v][j][lane];
      const int g = j / MT, t = j % MT;
      const int i = t * 16 + r16;
      if (i < mcount) store(m0 + i, n0 + g * 16 + ncol, sm);
    }
  }
}

// Launch shapes (waves per work-group, row groups, 64-k chunks per pipeline
// stage), from a sweep on the full-shape decode problems.  A shape is used
// only if it divides the problem; the chain ends in one that always does
// (dimensions are multiples of 64).
struct Shape {
  int nw, rg, u;
};

static bool fits(const Shape& c, int N, int K, int K0) {
  return K % (c.nw * 64 * c.u) == 0 && K0 % (64 * c.u) == 0 && N % (16 * c.rg) == 0;
}

static Shape pick(const Shape& pref, int N, int K, int K0) {
  const Shape chain[] = {pref, {4, 4, 1}, {4, 2, 1}, {2, 2, 1}, {1, 2, 1}, {1, 1, 1}};
  for (const Shape& c : chain)
    if (fits(c, N, K, K0)) return c;
  return {1, 1, 1};
}

template <class P, bool GROUPED, int MT>
static hipError_t launch_shape(const P& p, const Shape& c, long mtiles, int mrows, const Tile* tiles,
                               const int* ntiles, hipStream_t s) {
  const long nblocks = p.N() / (16 * c.rg);
  const long grid = GROUPED ? mtiles * nblocks : 8 * mtiles * ((nblocks + 7) / 8);
  if (grid <= 0) return hipSuccess;
#define LMOE_SG(NW_, RG_, U_)                                                      \
  if (c.nw == NW_ && c.rg == RG_ && c.u == U_) {                                   \
    stream_gemm_kernel<P, GROUPED, NW_, MT, RG_, U_>                               \
        <<<grid, NW_ * 64, 0, s>>>(p, mrows, tiles, ntiles);                       \
    return hipGetLastError();                                                      \
  }
  LMOE_SG(8, 1, 2)
  LMOE_SG(8, 2, 1)
  LMOE_SG(8, 4, 1)
  LMOE_SG(4, 4, 1)
  LMOE_SG(4, 2, 1)
  LMOE_SG(4, 2, 2)
  LMOE_SG(2, 2, 1)
  LMOE_SG(1, 2, 1)
  LMOE_SG(1, 1, 1)
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
  // the latent part (few rows) wants many short waves; the shared part wider blocks
  return launch_dense(p, p.N() <= 4096 ? Shape{8, 1, 2} : Shape{8, 4, 1}, p.T, s);
}
hipError_t stream_proj_out(const ProjOut& p, hipStream_t s) {
  return launch_dense(p, Shape{8, 2, 1}, p.T, s);
}
// Expert GEMMs, measured on the decode (T = 32, ~380 experts touched, 1.4
// rows each on average) and speculative-verify (T = 192, all 512, 8.3 rows)
// problems: up projection 8 waves x 2 row groups (1117 / 1575 us against
// 1151 / 1618 us for 4 x 4); down projection 8 waves x 1 row group x 2 k
// chunks per stage where experts average at most 2 rows (1113 against 1140 us
// for 4 x 4 at T = 32), else 4 x 4 (1584 us at T = 192, against 1632 for
// 8 x 2 and 1732 for 8 x 1 x 2).
hipError_t stream_exp_up(const ExpUp& p, const Tile* tiles, const int* ntiles, int max_tiles,
                         hipStream_t s) {
  return launch_grouped(p, Shape{8, 2, 1}, tiles, ntiles, max_tiles, s);
}
hipError_t stream_exp_down(const ExpDown& p, const Tile* tiles, const int* ntiles, int max_tiles,
                           int rows_per_expert, hipStream_t s) {
  return launch_grouped(p, rows_per_expert <= 2 ? Shape{8, 1, 2} : Shape{4, 4, 1}, tiles, ntiles,
                        max_tiles, s);
}

}  // namespace lmoe
