// Router of the LatentMoE layer: fp32 logits of the latent against the gate,
// sigmoid, correction bias, top-K and renormalisation.
//
// Page "Nemotron 3 Ultra 架构深度拆解报告", CH5 §5.6 Steps 1-4: the gate is
// an fp32 linear layer, scores are sigmoid(logit), the selection uses
// score + e_score_correction_bias, the weights use the unbiased scores of
// the selected experts, divided by (their sum + 1e-20) and multiplied by
// routed_scaling_factor.  One routing group (n_group = 1, §5.5).  This
// implementation reads the fp32 latent (the router is on the latent).
//
// Two kernels: the logits GEMM (fp32 MFMA, weight-streaming layout like the
// bf16 streaming GEMM) and one wavefront per token for everything after it.
// With few tokens the GEMM also splits k over work-groups (the 4 MB gate is
// otherwise streamed by a few dozen work-groups); the selection kernel adds
// the split partial logits in a fixed order.
#include "kernels.h"
#include "lmoe_device.h"

namespace lmoe {

// logits[t][e] = sum_k z[t][k] * Wg[e][k].  Work-group: RG*16 experts x
// MT*16 tokens, the k range split over NW waves, partial sums added in LDS in
// a fixed order.  Each lane loads 4 consecutive floats of its row per 16-wide
// k step and feeds them to 4 MFMAs (16x16x4): MFMA j takes component j, so
// lane group q = l/16 covers k = 4q + j -- the same for both operands.  Few
// tokens: RG = 1 (many work-groups to stream the 4 MB gate); many tokens:
// RG = 4, so each latent row loaded serves 64 experts.
// Work-group b: k split b / (mtiles * eblocks) of `nsplit` (each R / nsplit
// long), writing partial logits to logits + split * T * E.
template <int NW, int MT, int RG>
__global__ __launch_bounds__(NW * 64) void router_logits_kernel(const float* __restrict__ z,
                                                                const float* __restrict__ wg,
                                                                float* __restrict__ logits, int T,
                                                                int E, int R, int nsplit) {
  constexpr int J = RG * MT;
  __shared__ f32x4 red[NW > 1 ? NW : 1][J][64];
  const int eblocks = E / (16 * RG);
  const int mtiles = (T + 16 * MT - 1) / (16 * MT);
  const int split = blockIdx.x / (eblocks * mtiles);
  const int bid = blockIdx.x % (eblocks * mtiles);
  const int eb = bid % eblocks;
  const int m0 = (bid / eblocks) * (16 * MT);
  const int e0 = eb * 16 * RG;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r16 = lane & 15, kq = (lane >> 4) * 4;
  const int rs = R / nsplit;
  const int kw = rs / NW, kbeg = split * rs + w * kw;
  logits += (size_t)split * T * E;
  constexpr int KS = 32;  // k per pipeline stage (2 loads of 16 k)
  const int nit = kw / KS;

  const float* brow = wg + (size_t)(e0 + r16) * R + kbeg + kq;
  const long gstride = 16L * R;
  const float* arow[MT];
  bool av[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m0 + t * 16 + r16;
    av[t] = m < T;
    arow[t] = av[t] ? z + (size_t)m * R + kbeg + kq : nullptr;
  }
  f32x4 acc[RG][MT];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[g][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  f32x4 wA[2][RG], xA[2][MT], wB[2][RG], xB[2][MT];
  auto load = [&](f32x4(&wf)[2][RG], f32x4(&xf)[2][MT], int it) {
    const int k = it * KS;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int g = 0; g < RG; ++g)
        wf[u][g] = *reinterpret_cast<const f32x4*>(brow + g * gstride + k + u * 16);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        xf[u][t] = av[t] ? *reinterpret_cast<const f32x4*>(arow[t] + k + u * 16)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto compute = [&](const f32x4(&wf)[2][RG], const f32x4(&xf)[2][MT]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
          for (int t = 0; t < MT; ++t) acc[g][t] = mfma_f32(wf[u][g][j], xf[u][t][j], acc[g][t]);
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
  const int ecol = e0 + (lane >> 4) * 4;
  if constexpr (NW == 1) {
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int t = 0; t < MT; ++t)
        if (av[t])
          *reinterpret_cast<f32x4*>(logits + (size_t)(m0 + t * 16 + r16) * E + ecol + g * 16) =
              acc[g][t];
  } else {
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int t = 0; t < MT; ++t) red[w][g * MT + t][lane] = acc[g][t];
    __syncthreads();
    for (int jj = w; jj < J; jj += NW) {
      f32x4 s = red[0][jj][lane];
#pragma unroll
      for (int v = 1; v < NW; ++v) s += red[v][jj][lane];
      const int g = jj / MT, t = jj % MT;
      const int m = m0 + t * 16 + r16;
      if (m < T) *reinterpret_cast<f32x4*>(logits + (size_t)m * E + ecol + g * 16) = s;
    }
  }
}

// Order-preserving map of a finite float onto uint32 (larger float ->
// larger integer); -0 is first turned into +0 so the two compare equal.
__device__ __forceinline__ uint32_t ordered_bits(float b) {
  if (b == 0.0f) b = 0.0f;
  const uint32_t u = __float_as_uint(b);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Largest key v such that at least n of the wave's keys (NS slots per lane)
// are >= v: built bit by bit from the top, each candidate kept if at least n
// keys reach it, counted with one ballot per slot (no cross-lane data
// movement).  With keys of 0 for empty slots and n <= the number of nonzero
// keys, v is the n-th largest key.
template <int NS>
__device__ __forceinline__ uint32_t nth_largest_key(const uint32_t (&key)[NS], int n) {
  uint32_t v = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = v | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < NS; ++j) cnt += __popcll(__ballot(key[j] >= c));
    if (cnt >= n) v = c;
  }
  return v;
}

// One wavefront per token.  Expert e = 64 j + lane lives in slot j of lane
// `lane`; its key is the ordered bit pattern of its biased score (0 for slots
// past E, below every finite score).  The K-th largest key v comes from
// nth_largest_key; the selected set is every key above v plus the lowest-id
// experts whose key equals v (equal scores go to the lower expert id).
// Output order is ascending expert id, the renormalising sum is a plain
// float32 sum in that order, then w = (s / (sum + 1e-20)) * rho.
//
// Routing groups (n_group > 1; page "Nemotron 3 Ultra 架构深度拆解报告",
// CH5 §5.5): the token's biased scores go to LDS, lane g < n_group takes the
// two largest of group g (experts [g G, (g + 1) G)) and their float32 sum is
// the group score; the topk_group best groups are kept the same way as the
// experts (equal group scores to the lower group index), and the keys of the
// experts of the other groups are set to 0, so they cannot be selected.
template <int NJ>
__global__ __launch_bounds__(256) void router_select_kernel(const float* __restrict__ logits,
                                                           int nsplit,
                                                           const float* __restrict__ bias, int T,
                                                           int E, int K, int n_group,
                                                           int topk_group, float rho,
                                                           int32_t* __restrict__ idx_out,
                                                           float* __restrict__ w_out) {
  __shared__ float ssel[4][64];
  __shared__ float sb[4][NJ * 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  const size_t pstride = (size_t)T * E;
  // logit = partial 0 + partial 1 + ... (split order); all slots' loads of a
  // batch of partials are issued before any is added
  const float* lp = logits + (size_t)t * E + lane;
  float l[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) l[j] = (j * 64 + lane < E) ? lp[j * 64] : 0.f;
  for (int q0 = 1; q0 < nsplit; q0 += 4) {
    float pv[4][NJ];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        pv[q][j] = (q0 + q < nsplit && j * 64 + lane < E) ? lp[(q0 + q) * pstride + j * 64] : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q0 + q < nsplit)
#pragma unroll
        for (int j = 0; j < NJ; ++j) l[j] += pv[q][j];
  }
  float s[NJ];
  uint32_t key[NJ];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = j * 64 + lane;
    if (e < E) {
      s[j] = 1.0f / (1.0f + expf(-l[j]));
      const float b = s[j] + bias[e];
      key[j] = ordered_bits(b);
      sb[wv][e] = b;
    } else {
      s[j] = 0.f;
      key[j] = 0u;
    }
  }
  if (n_group > 1) {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int G = E / n_group;
    uint32_t gkey[1] = {0u};
    if (lane < n_group) {
      float t1 = -INFINITY, t2 = -INFINITY;
      for (int i = 0; i < G; ++i) {
        const float b = sb[wv][lane * G + i];
        if (b > t1) {
          t2 = t1;
          t1 = b;
        } else if (b > t2) {
          t2 = b;
        }
      }
      gkey[0] = ordered_bits(t1 + t2);
    }
    const uint32_t gv = nth_largest_key(gkey, topk_group);
    const int groom = topk_group - __popcll(__ballot(gkey[0] > gv));
    const uint64_t geq = __ballot(gkey[0] == gv);
    const bool kept = gkey[0] > gv || (gkey[0] == gv && __popcll(geq & below) < groom);
    const uint64_t kept_mask = __ballot(kept);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int e = j * 64 + lane;
      if (e < E && !((kept_mask >> (e / G)) & 1ull)) key[j] = 0u;
    }
  }
  const uint32_t v = nth_largest_key(key, K);
  int above = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) above += __popcll(__ballot(key[j] > v));
  int room = K - above;  // experts with key == v still to take, lowest ids first
  int base = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint64_t eq = __ballot(key[j] == v);
    bool on = key[j] > v;
    if (key[j] == v && __popcll(eq & below) < room) on = true;
    const int took = __popcll(eq);
    room -= took < room ? took : room;
    const uint64_t m = __ballot(on);
    if (on) {
      const int pos = base + __popcll(m & below);
      idx_out[(size_t)t * K + pos] = j * 64 + lane;
      ssel[wv][pos] = s[j];
    }
    base += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float denom = 0.f;
  if (lane == 0) {
    float acc = 0.f;
    for (int k = 0; k < K; ++k) acc = acc + ssel[wv][k];
    denom = acc + 1e-20f;
  }
  denom = __shfl(denom, 0, 64);
  if (lane < K) w_out[(size_t)t * K + lane] = (ssel[wv][lane] / denom) * rho;
}

// Launch geometry of the logits GEMM for T tokens.
struct RouterGeom {
  int mt, rg, nsplit, nw;
  long grid;
};

static RouterGeom router_geom(int T, int E, int R) {
  RouterGeom g;
  g.mt = T <= 16 ? 1 : (T <= 32 ? 2 : 4);
  g.rg = (T > 256 && E % 64 == 0) ? 4 : 1;
  const long base = (long)((T + 16 * g.mt - 1) / (16 * g.mt)) * (E / (16 * g.rg));
  // split k until about 512 work-groups, keeping each split a multiple of 64
  g.nsplit = 1;
  while (g.nsplit < router_max_splits() && base * g.nsplit * 2 <= 512 &&
         R % (g.nsplit * 2 * 64) == 0 && T <= router_split_max_tokens())
    g.nsplit *= 2;
  g.grid = base * g.nsplit;
  const int rs = R / g.nsplit;
  g.nw = 1;
  const int opts[4] = {1, 2, 4, 8};
  for (int i = 0; i < 4; ++i) {
    if (rs % (opts[i] * 64) != 0) continue;
    g.nw = opts[i];
    if (g.grid * g.nw >= 2048) break;
  }
  return g;
}

int router_splits(int T, int E, int R) { return T > 0 ? router_geom(T, E, R).nsplit : 1; }

hipError_t router_logits(const float* z, const float* wg, float* logits, int T, int E, int R,
                         hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const RouterGeom g = router_geom(T, E, R);
  const long grid = g.grid;
  const int nsplit = g.nsplit, mt = g.mt, rg = g.rg;
#define LMOE_RL(NW_, MT_, RG_)                                        \
  router_logits_kernel<NW_, MT_, RG_><<<grid, NW_ * 64, 0, s>>>(z, wg, logits, T, E, R, nsplit)
#define LMOE_RL_MT(NW_)                 \
  do {                                  \
    if (rg == 4) LMOE_RL(NW_, 4, 4);    \
    else if (mt == 1) LMOE_RL(NW_, 1, 1); \
    else if (mt == 2) LMOE_RL(NW_, 2, 1); \
    else LMOE_RL(NW_, 4, 1);            \
  } while (0)
  switch (g.nw) {
    case 1: LMOE_RL_MT(1); break;
    case 2: LMOE_RL_MT(2); break;
    case 4: LMOE_RL_MT(4); break;
    default: LMOE_RL_MT(8); break;
  }
#undef LMOE_RL_MT
#undef LMOE_RL
  return hipGetLastError();
}

hipError_t router_select(const float* logits, const float* bias, int T, int E, int R, int K,
                         int n_group, int topk_group, float rho, int32_t* idx, float* w,
                         hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int grid = (T + 3) / 4;
  const int nj = (E + 63) / 64;
  const int nsplit = router_splits(T, E, R);
#define LMOE_RS(NJ_) \
  router_select_kernel<NJ_><<<grid, 256, 0, s>>>(logits, nsplit, bias, T, E, K, n_group, \
                                                  topk_group, rho, idx, w)
  if (nj <= 1) LMOE_RS(1);
  else if (nj <= 2) LMOE_RS(2);
  else if (nj <= 4) LMOE_RS(4);
  else if (nj <= 8) LMOE_RS(8);
  else LMOE_RS(16);
#undef LMOE_RS
  return hipGetLastError();
}

}  // namespace lmoe
