// C ABI of the LatentMoE layer: argument checks, workspace carving and the
// launch sequence of one forward pass.  See include/lmoe.h for the contract.
//
// Launch sequence (no host synchronisation; page "Nemotron 3 Ultra 架构深度
// 拆解报告", CH5 §5.6 Steps 1-7).  On the caller's stream:
//  [prenorm        h -> bf16(gamma h), 1/rms   (block pre-norm, CH9 §9.3)]
//   proj_latent    x -> z (fp32 + bf16)                        (Step 5)
//   router_logits  z (fp32) -> logits                          (Step 1)
//   router_select  logits -> top-K experts and weights         (Steps 2-4)
//   dispatch       experts -> expert-sorted rows + tile list   (Step 6 grouping)
//   expert_up      relu(z16 Wup[e]^T)^2                        (Step 6)
//   expert_down    H Wdn[e]^T                                  (Step 6)
//   combine        r = sum_k w O                               (Step 6 index_add_)
//   proj_out       y = r W2^T + Hs Wsd^T  [+ h, block residual] (Step 7)
// and, forked onto the handle's auxiliary stream (before proj_latent for
// weight-streaming batches, after it otherwise) and joined before proj_out
// (the shared expert only needs x):
//   shared_up      x -> Hs = relu(x Wsu^T)^2                   (Step 7)
//                  [weight-streaming batches: then ys = Hs Wsd^T in fp32,
//                   and proj_out computes r W2^T + ys]
// The latent projection and the router/dispatch chain are latency-bound and
// leave HBM idle; the shared expert's weight stream fills that time.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/lmoe.h"
#include "gemm_problems.h"
#include "kernels.h"

using namespace lmoe;

namespace {

// Stages 0..7 run back to back on the caller's stream (stage i is timed
// between events i and i + 1; proj_out's interval includes the wait for the
// auxiliary stream); stage 8 runs on the auxiliary stream between its own
// pair of events.
constexpr int kNumStages = 9;
constexpr int kMainStages = 8;
constexpr int kEventsPerForward = kMainStages + 1 + 2;
const char* const kStageNames[kNumStages] = {
    "proj_latent", "router_logits", "router_select", "dispatch", "expert_up",
    "expert_down", "combine",       "proj_out",      "shared_up"};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool tiled_dims_ok(const lmoe_config& c) {
  const int bn = tiled_block_n();
  return c.moe_shared_expert_intermediate_size % bn == 0 && c.hidden_size % bn == 0 &&
         c.moe_intermediate_size % bn == 0 && c.moe_latent_size % bn == 0;
}

lmoe_status check_config(const lmoe_config* c) {
  if (!c) return LMOE_ERR_INVALID_ARG;
  if (c->hidden_size <= 0 || c->moe_latent_size <= 0 || c->n_routed_experts <= 0 ||
      c->num_experts_per_tok <= 0 || c->moe_intermediate_size <= 0 ||
      c->moe_shared_expert_intermediate_size <= 0 || c->max_tokens <= 0 ||
      !std::isfinite(c->routed_scaling_factor))
    return LMOE_ERR_INVALID_ARG;
  if (c->path < LMOE_PATH_AUTO || c->path > LMOE_PATH_TILED) return LMOE_ERR_INVALID_ARG;
  if (c->expert_format != LMOE_EXPERTS_BF16 && c->expert_format != LMOE_EXPERTS_MXFP4)
    return LMOE_ERR_INVALID_ARG;
  if (c->hidden_size % 64 || c->moe_latent_size % 64 || c->moe_intermediate_size % 64 ||
      c->moe_shared_expert_intermediate_size % 64)
    return LMOE_ERR_UNSUPPORTED;
  if (c->n_routed_experts > 1024 || c->n_routed_experts % 16) return LMOE_ERR_UNSUPPORTED;
  if (c->num_experts_per_tok > c->n_routed_experts || c->num_experts_per_tok > 64)
    return LMOE_ERR_UNSUPPORTED;
  // routing groups (page §5.5): n_group equal contiguous groups of at least
  // two experts, 1 <= topk_group <= n_group, enough experts in the kept
  // groups for the top-K; the selection kernel holds one group per lane
  if (c->n_group < 1 || c->topk_group < 1 || c->topk_group > c->n_group)
    return LMOE_ERR_INVALID_ARG;
  if (c->n_routed_experts <= 0 || c->n_routed_experts % c->n_group) return LMOE_ERR_INVALID_ARG;
  if (c->n_group > 1 && c->n_routed_experts / c->n_group < 2) return LMOE_ERR_INVALID_ARG;
  if (c->num_experts_per_tok > c->topk_group * (c->n_routed_experts / c->n_group))
    return LMOE_ERR_INVALID_ARG;
  if (c->n_group > 64) return LMOE_ERR_UNSUPPORTED;
  // MXFP4 experts: the streaming kernel covers 128 k per step (4 blocks)
  if (c->expert_format == LMOE_EXPERTS_MXFP4 &&
      (c->moe_latent_size % 128 || c->moe_intermediate_size % 128))
    return LMOE_ERR_UNSUPPORTED;
  // block steps: known bits; the pre-norm's epsilon finite and >= 0
  if (c->fuse & ~(LMOE_FUSE_PRENORM | LMOE_FUSE_RESIDUAL)) return LMOE_ERR_INVALID_ARG;
  if ((c->fuse & LMOE_FUSE_PRENORM) && !(std::isfinite(c->norm_eps) && c->norm_eps >= 0.f))
    return LMOE_ERR_INVALID_ARG;
  if (c->max_tokens > (1 << 22)) return LMOE_ERR_UNSUPPORTED;
  if (c->path == LMOE_PATH_TILED && !tiled_dims_ok(*c)) return LMOE_ERR_UNSUPPORTED;
  return LMOE_OK;
}

// Upper bound on the tile count of the expert tile list for T tokens.
long max_tiles(const lmoe_config& c, long T, int tile_m) {
  const long slots = T * c.num_experts_per_tok;
  return std::min<long>(c.n_routed_experts, slots) + slots / tile_m + 1;
}

struct Layout {
  size_t xt, rn, z32, z16, hs, ys, part, logits, idx, tw, counts, offsets, blockcnt, rows_tok,
      inv, tiles, ntiles, h, o, r16, total;
};

Layout make_layout(const lmoe_config& c) {
  const size_t T = c.max_tokens, R = c.moe_latent_size, S = c.moe_shared_expert_intermediate_size;
  const size_t E = c.n_routed_experts, K = c.num_experts_per_tok, F = c.moe_intermediate_size;
  const size_t slots = T * K;
  const size_t ntile = std::max(max_tiles(c, T, kStreamTileM), max_tiles(c, T, tiled_block_m()));
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  const bool prenorm_fused = (c.fuse & LMOE_FUSE_PRENORM) != 0;
  L.xt = take(prenorm_fused ? T * c.hidden_size * 2 : 0);
  L.rn = take(prenorm_fused ? T * 4 : 0);
  L.z32 = take(T * R * 4);
  L.z16 = take(T * R * 2);
  L.hs = take(T * S * 2);
  // fp32 shared-expert output of weight-streaming batches (at most
  // kStreamDenseMaxTokens tokens), computed on the auxiliary stream
  L.ys = take(std::min<size_t>(T, kStreamDenseMaxTokens) * c.hidden_size * 4);
  // split-k partial sums of the dense GEMMs (any batch of at most
  // kSplitMaxTokens tokens may take the split path when the tiled GEMMs apply)
  const size_t D = c.hidden_size;
  L.part = take(tiled_dims_ok(c) ? static_cast<size_t>(kSplitMax) *
                                       std::min<size_t>(T, kSplitMaxTokens) *
                                       std::max({R, S, D}) * 4
                                 : 0);
  L.logits = take(std::max(T, std::min<size_t>(T, router_split_max_tokens()) *
                                  static_cast<size_t>(router_max_splits())) *
                  E * 4);
  L.idx = take(slots * 4);
  L.tw = take(slots * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.blockcnt = take(((T + 63) / 64) * E * 4);
  L.rows_tok = take(slots * 4);
  L.inv = take(slots * 4);
  L.tiles = take(ntile * sizeof(Tile));
  L.ntiles = take(16);
  L.h = take(slots * F * 2);
  L.o = take(slots * R * 2);
  L.r16 = take(T * R * 2);
  L.total = off;
  return L;
}

lmoe_status check_weights(const lmoe_config& c, const lmoe_weights* w) {
  if (!w || !w->fc1_latent || !w->router || !w->router_bias || !w->fc2_latent ||
      !w->shared_up || !w->shared_down)
    return LMOE_ERR_INVALID_ARG;
  const void* ptrs[6] = {w->fc1_latent, w->router,    w->router_bias,
                         w->fc2_latent, w->shared_up, w->shared_down};
  for (const void* p : ptrs)
    if (!aligned16(p)) return LMOE_ERR_INVALID_ARG;
  if (c.expert_format == LMOE_EXPERTS_MXFP4) {
    if (!w->expert_up_mxfp4 || !w->expert_up_scale || !w->expert_down_mxfp4 ||
        !w->expert_down_scale || !aligned16(w->expert_up_mxfp4) ||
        !aligned16(w->expert_down_mxfp4))
      return LMOE_ERR_INVALID_ARG;
  } else if (!w->expert_up || !w->expert_down || !aligned16(w->expert_up) ||
             !aligned16(w->expert_down)) {
    return LMOE_ERR_INVALID_ARG;
  }
  if ((c.fuse & LMOE_FUSE_PRENORM) && (!w->norm_weight || !aligned16(w->norm_weight)))
    return LMOE_ERR_INVALID_ARG;
  return LMOE_OK;
}

// Host-side checks of one forward's x, y and taps.
lmoe_status check_io(const lmoe_config& c, const uint16_t* x, int32_t T, const uint16_t* y,
                     const lmoe_taps* taps) {
  if (!x || !y || !aligned16(x) || !aligned16(y)) return LMOE_ERR_INVALID_ARG;
  const size_t xb = static_cast<size_t>(T) * c.hidden_size * 2;
  const char* xc = reinterpret_cast<const char*>(x);
  const char* yc = reinterpret_cast<const char*>(y);
  if (xc < yc + xb && yc < xc + xb) return LMOE_ERR_INVALID_ARG;
  if (taps) {
    const void* tp[5] = {taps->z_f32, taps->topk_idx, taps->topk_w, taps->expert_counts,
                         taps->r_latent};
    for (const void* p : tp)
      if (p && !aligned16(p)) return LMOE_ERR_INVALID_ARG;
  }
  return LMOE_OK;
}

}  // namespace

struct lmoe_handle {
  lmoe_config cfg;
  lmoe_weights w;
  char* ws;
  Layout L;
  // auxiliary stream and its fork/join events, created by lmoe_create
  hipStream_t aux = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  // profiling
  int prof_max = 0, prof_n = 0;
  std::vector<hipEvent_t> events;
  // LMOE_DEBUG set (and not "0") at creation: synchronise after every stage
  bool debug = false;

  template <class T>
  T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
};

namespace {

// The launch sequence of one forward of T tokens (1 <= T <= the layout's
// max_tokens) on the workspace `ws` carved by `L`.  `aux` (with its fork and
// join events) runs the shared expert concurrently; without it everything
// runs on `s`.  `ev`: profiling events of this forward, or null.
lmoe_status run_forward(const lmoe_config& c, const lmoe_weights& w, const Layout& L, char* ws,
                        bool debug, hipStream_t aux, hipEvent_t fork, hipEvent_t join,
                        hipEvent_t* ev, const uint16_t* x, int32_t T, uint16_t* y, hipStream_t s,
                        const lmoe_taps* taps) {
  const int D = c.hidden_size, R = c.moe_latent_size, E = c.n_routed_experts;
  const int K = c.num_experts_per_tok, F = c.moe_intermediate_size;
  const int S = c.moe_shared_expert_intermediate_size;
  const bool tiled_ok = tiled_dims_ok(c);
  // Dense GEMMs: weight streaming for few tokens; LDS-tiled above that,
  // split over k while the batch is too small to fill the GPU with tiles.
  enum class Dense { kStream, kSplit, kTiled };
  Dense dense = Dense::kStream;
  if (tiled_ok && (c.path == LMOE_PATH_TILED ||
                   (c.path == LMOE_PATH_AUTO && T > kStreamDenseMaxTokens)))
    dense = T <= kSplitMaxTokens ? Dense::kSplit : Dense::kTiled;
  const bool mxfp4 = c.expert_format == LMOE_EXPERTS_MXFP4;
  const bool expert_tiled =
      tiled_ok && (c.path == LMOE_PATH_TILED ||
                   (c.path == LMOE_PATH_AUTO && static_cast<long>(T) * K > 32L * E));
  const int tile_m = expert_tiled ? tiled_block_m() : kStreamTileM;
  const int ntile_max = static_cast<int>(max_tiles(c, T, tile_m));

  // Block pre-norm: the projections read bf16(gamma h) and scale by 1/rms.
  const bool prenorm_fused = (c.fuse & LMOE_FUSE_PRENORM) != 0;
  uint16_t* xt = reinterpret_cast<uint16_t*>(ws + L.xt);
  float* rn = reinterpret_cast<float*>(ws + L.rn);
  const uint16_t* xin = prenorm_fused ? xt : x;
  const float* rscale = prenorm_fused ? rn : nullptr;
  const uint16_t* resid = (c.fuse & LMOE_FUSE_RESIDUAL) ? x : nullptr;
  float* z32 = reinterpret_cast<float*>(ws + L.z32);
  uint16_t* z16 = reinterpret_cast<uint16_t*>(ws + L.z16);
  uint16_t* hs = reinterpret_cast<uint16_t*>(ws + L.hs);
  float* part = reinterpret_cast<float*>(ws + L.part);
  auto proj_in = [&](const ProjIn& p, hipStream_t st) {
    switch (dense) {
      case Dense::kStream: return stream_proj_in(p, st);
      case Dense::kSplit: return split_proj_in(p, part, st);
      default: return tiled_proj_in(p, st);
    }
  };
  auto proj_out = [&](const ProjOut& p, hipStream_t st) {
    switch (dense) {
      case Dense::kStream: return stream_proj_out(p, st);
      case Dense::kSplit: return split_proj_out(p, part, st);
      default: return tiled_proj_out(p, st);
    }
  };
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + L.idx);
  float* tw = reinterpret_cast<float*>(ws + L.tw);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* blockcnt = reinterpret_cast<int32_t*>(ws + L.blockcnt);
  int32_t* rows_tok = reinterpret_cast<int32_t*>(ws + L.rows_tok);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
  Tile* tiles = reinterpret_cast<Tile*>(ws + L.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(ws + L.ntiles);
  uint16_t* H = reinterpret_cast<uint16_t*>(ws + L.h);
  uint16_t* O = reinterpret_cast<uint16_t*>(ws + L.o);
  uint16_t* r16 = reinterpret_cast<uint16_t*>(ws + L.r16);

  int stage = 0;
  auto mark = [&]() -> bool {
    if (!ev) return true;
    return hipEventRecord(ev[stage++], s) == hipSuccess;
  };
  auto ok = [](hipError_t e) { return e == hipSuccess; };
  // Debug mode: wait for the stage just launched (and the auxiliary stream)
  // and report the first failure with the stage's name.
  auto done = [&](const char* stage_name) -> bool {
    if (!debug) return true;
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess && aux) e = hipStreamSynchronize(aux);
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) return true;
    std::fprintf(stderr, "lmoe: stage %s failed: %s\n", stage_name, hipGetErrorString(e));
    return false;
  };

  // Weight-streaming batches: the shared expert's down projection also runs
  // on the auxiliary stream (its weight stream fills HBM time the router and
  // dispatch leave idle), into fp32 ys; proj_out then streams only W2 and
  // adds ys before its single rounding.
  const bool split_out = dense == Dense::kStream && T <= kStreamDenseMaxTokens;
  float* ys = reinterpret_cast<float*>(ws + L.ys);
  // Shared expert's up projection on the auxiliary stream, forked from `s`
  // at the current point and joined before proj_out.
  // Without an auxiliary stream the same kernels run in the same order on
  // `s`.
  hipStream_t sh_stream = aux ? aux : s;
  auto fork_shared = [&]() -> bool {
    if (aux &&
        (!ok(hipEventRecord(fork, s)) || !ok(hipStreamWaitEvent(aux, fork, 0))))
      return false;
    if (ev && !ok(hipEventRecord(ev[kMainStages + 1], sh_stream))) return false;
    ProjIn pshared{xin, w.fc1_latent, w.shared_up, z32, z16, hs, T, D, R, S, R, S, rscale};
    if (!ok(proj_in(pshared, sh_stream))) return false;
    if (split_out) {
      ProjOut pdown{r16, hs, w.fc2_latent, w.shared_down, y, T, D, R, S, nullptr, 1, ys};
      if (!ok(stream_proj_out(pdown, sh_stream))) return false;
    }
    if (ev && !ok(hipEventRecord(ev[kMainStages + 2], sh_stream))) return false;
    return !aux || ok(hipEventRecord(join, aux));
  };
  // Weight streaming: fork first, so that the shared weight stream also uses
  // the bandwidth the short latent projection leaves idle.  Otherwise fork
  // after the latent projection (the split-k path's partial sums are one
  // buffer, and the tiled GEMMs would only compete for the same CUs).
  const bool fork_first = dense == Dense::kStream;
  if (!mark()) return LMOE_ERR_HIP;
  if (prenorm_fused && !ok(prenorm(x, w.norm_weight, T, D, c.norm_eps, xt, rn, s)))
    return LMOE_ERR_HIP;
  if (prenorm_fused && !done("prenorm")) return LMOE_ERR_HIP;
  if (fork_first && !(fork_shared() && done("shared_up"))) return LMOE_ERR_HIP;
  ProjIn platent{xin, w.fc1_latent, w.shared_up, z32, z16, hs, T, D, R, S, 0, R, rscale};
  if (!ok(proj_in(platent, s)) || !done("proj_latent")) return LMOE_ERR_HIP;
  if (!fork_first && !(fork_shared() && done("shared_up"))) return LMOE_ERR_HIP;
  if (!mark()) return LMOE_ERR_HIP;
  if (!ok(router_logits(z32, w.router, logits, T, E, R, s)) || !done("router_logits"))
    return LMOE_ERR_HIP;
  if (!mark()) return LMOE_ERR_HIP;
  if (!ok(router_select(logits, w.router_bias, T, E, R, K, c.n_group, c.topk_group,
                        c.routed_scaling_factor, idx, tw, s)) ||
      !done("router_select"))
    return LMOE_ERR_HIP;
  if (!mark()) return LMOE_ERR_HIP;
  if (!ok(dispatch(idx, T, K, E, blockcnt, counts, offsets, rows_tok, inv, tiles, ntiles, tile_m,
                   s)) ||
      !done("dispatch"))
    return LMOE_ERR_HIP;
  if (!mark()) return LMOE_ERR_HIP;
  if (mxfp4) {
    ExpUpMx pup{z16, rows_tok, w.expert_up_mxfp4, w.expert_up_scale, H, R, F};
    if (!ok(expert_tiled ? tiled_mx_exp_up(pup, tiles, ntiles, ntile_max, T, s)
                         : stream_mx_exp_up(pup, tiles, ntiles, ntile_max, T,
                                            static_cast<int>((T * K + E - 1) / E), s)))
      return LMOE_ERR_HIP;
  } else {
    ExpUp pup{z16, rows_tok, w.expert_up, H, R, F};
    if (!ok(expert_tiled ? tiled_exp_up(pup, tiles, ntiles, ntile_max, T, s)
                         : stream_exp_up(pup, tiles, ntiles, ntile_max, s)))
      return LMOE_ERR_HIP;
  }
  if (!done("expert_up") || !mark()) return LMOE_ERR_HIP;
  if (mxfp4) {
    ExpDownMx pdn{H, w.expert_down_mxfp4, w.expert_down_scale, O, R, F};
    if (!ok(expert_tiled ? tiled_mx_exp_down(pdn, tiles, ntiles, ntile_max, s)
                         : stream_mx_exp_down(pdn, tiles, ntiles, ntile_max, s)))
      return LMOE_ERR_HIP;
  } else {
    ExpDown pdn{H, w.expert_down, O, R, F};
    if (!ok(expert_tiled ? tiled_exp_down(pdn, tiles, ntiles, ntile_max, s)
                         : stream_exp_down(pdn, tiles, ntiles, ntile_max,
                                           static_cast<int>((T * K + E - 1) / E), s)))
      return LMOE_ERR_HIP;
  }
  if (!done("expert_down") || !mark()) return LMOE_ERR_HIP;
  if (!ok(combine(O, inv, tw, T, K, R, r16, taps ? taps->r_latent : nullptr, s)) ||
      !done("combine"))
    return LMOE_ERR_HIP;
  if (!mark()) return LMOE_ERR_HIP;
  // join, then y = r W2^T + Hs Wsd^T (+ h with the block residual fused)
  if (aux && !ok(hipStreamWaitEvent(s, join, 0))) return LMOE_ERR_HIP;
  ProjOut pout{r16, hs, w.fc2_latent, w.shared_down, y, T, D, R, S, resid,
               split_out ? 2 : 0, ys};
  if (!ok(proj_out(pout, s)) || !done("proj_out")) return LMOE_ERR_HIP;
  if (!mark()) return LMOE_ERR_HIP;

  if (taps) {
    if (taps->z_f32 &&
        !ok(hipMemcpyAsync(taps->z_f32, z32, sizeof(float) * T * R, hipMemcpyDeviceToDevice, s)))
      return LMOE_ERR_HIP;
    if (taps->topk_idx && !ok(hipMemcpyAsync(taps->topk_idx, idx, sizeof(int32_t) * T * K,
                                             hipMemcpyDeviceToDevice, s)))
      return LMOE_ERR_HIP;
    if (taps->topk_w &&
        !ok(hipMemcpyAsync(taps->topk_w, tw, sizeof(float) * T * K, hipMemcpyDeviceToDevice, s)))
      return LMOE_ERR_HIP;
    if (taps->expert_counts && !ok(hipMemcpyAsync(taps->expert_counts, counts,
                                                  sizeof(int32_t) * E, hipMemcpyDeviceToDevice, s)))
      return LMOE_ERR_HIP;
  }
  return LMOE_OK;
}

// Scratch of the allocation-free forward: one static device array, which
// every GPU the library runs on holds (its own copy, at its own address)
// until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host it names a host-side stand-in); it looks up the
// device address once per device and keeps it.
constexpr size_t kScratchBytes = LMOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on
// that device, with that device current).
lmoe_status device_scratch(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return LMOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return LMOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return LMOE_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return LMOE_OK;
}

}  // namespace

extern "C" {

size_t lmoe_workspace_size(const lmoe_config* cfg) {
  if (check_config(cfg) != LMOE_OK) return 0;
  return make_layout(*cfg).total;
}

lmoe_status lmoe_create(const lmoe_config* cfg, const lmoe_weights* w, void* workspace,
                        size_t workspace_bytes, lmoe_handle** out) {
  if (!out) return LMOE_ERR_INVALID_ARG;
  *out = nullptr;
  lmoe_status st = check_config(cfg);
  if (st != LMOE_OK) return st;
  st = check_weights(*cfg, w);
  if (st != LMOE_OK) return st;
  const Layout L = make_layout(*cfg);
  if (!workspace || workspace_bytes < L.total) return LMOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return LMOE_ERR_WORKSPACE;
  lmoe_handle* h = new (std::nothrow) lmoe_handle();
  if (!h) return LMOE_ERR_INVALID_ARG;
  h->cfg = *cfg;
  h->w = *w;
  h->ws = static_cast<char*>(workspace);
  h->L = L;
  const char* dbg = std::getenv("LMOE_DEBUG");
  h->debug = dbg && *dbg && std::strcmp(dbg, "0") != 0;
  // The auxiliary stream and its fork/join events, created here so that
  // every lmoe_forward (the first included) can be captured into a graph.
  if (hipStreamCreateWithFlags(&h->aux, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&h->fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->join, hipEventDisableTiming) != hipSuccess) {
    lmoe_destroy(h);
    return LMOE_ERR_HIP;
  }
  *out = h;
  return LMOE_OK;
}

void lmoe_destroy(lmoe_handle* h) {
  if (!h) return;
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  if (h->fork) (void)hipEventDestroy(h->fork);
  if (h->join) (void)hipEventDestroy(h->join);
  if (h->aux) (void)hipStreamDestroy(h->aux);
  delete h;
}

const char* lmoe_status_string(lmoe_status s) {
  switch (s) {
    case LMOE_OK: return "ok";
    case LMOE_ERR_INVALID_ARG: return "invalid argument";
    case LMOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case LMOE_ERR_TOO_MANY_TOKENS: return "token count exceeds max_tokens";
    case LMOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case LMOE_ERR_HIP: return "HIP runtime error";
    case LMOE_ERR_SCRATCH: return "input too large for the allocation-free forward's scratch";
  }
  return "unknown status";
}

int32_t lmoe_num_stages(void) { return kNumStages; }

const char* lmoe_stage_name(int32_t i) {
  return (i >= 0 && i < kNumStages) ? kStageNames[i] : nullptr;
}

lmoe_status lmoe_profile_begin(lmoe_handle* h, int32_t max_forwards) {
  if (!h || max_forwards <= 0 || max_forwards > 4096) return LMOE_ERR_INVALID_ARG;
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  h->events.assign(static_cast<size_t>(max_forwards) * kEventsPerForward, nullptr);
  for (auto& e : h->events)
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      return LMOE_ERR_HIP;
    }
  h->prof_max = max_forwards;
  h->prof_n = 0;
  return LMOE_OK;
}

lmoe_status lmoe_profile_end(lmoe_handle* h, float* ms, int32_t n_stages, int32_t* n_forwards) {
  if (!h || !ms || n_stages < kNumStages || !n_forwards) return LMOE_ERR_INVALID_ARG;
  for (int i = 0; i < kNumStages; ++i) ms[i] = 0.f;
  lmoe_status st = LMOE_OK;
  for (int f = 0; f < h->prof_n && st == LMOE_OK; ++f) {
    hipEvent_t* ev = &h->events[static_cast<size_t>(f) * kEventsPerForward];
    if (hipEventSynchronize(ev[kMainStages]) != hipSuccess ||
        hipEventSynchronize(ev[kEventsPerForward - 1]) != hipSuccess) {
      st = LMOE_ERR_HIP;
      break;
    }
    for (int i = 0; i < kNumStages; ++i) {
      float t = 0.f;
      hipEvent_t a = i < kMainStages ? ev[i] : ev[kMainStages + 1];
      hipEvent_t b = i < kMainStages ? ev[i + 1] : ev[kMainStages + 2];
      if (hipEventElapsedTime(&t, a, b) != hipSuccess) {
        st = LMOE_ERR_HIP;
        break;
      }
      ms[i] += t;
    }
  }
  *n_forwards = h->prof_n;
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  h->events.clear();
  h->prof_max = h->prof_n = 0;
  return st;
}

lmoe_status lmoe_quantize_mxfp4(const uint16_t* w, int64_t rows, int32_t cols, uint8_t* codes,
                                uint8_t* scales, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32) return LMOE_ERR_INVALID_ARG;
  if (rows == 0) return LMOE_OK;
  if (!w || !codes || !scales || !aligned16(w) || !aligned16(codes)) return LMOE_ERR_INVALID_ARG;
  if (rows > (int64_t{1} << 40) / cols) return LMOE_ERR_INVALID_ARG;
  return mxfp4_quantize(w, static_cast<long>(rows), cols, codes, scales,
                        static_cast<hipStream_t>(stream)) == hipSuccess
             ? LMOE_OK
             : LMOE_ERR_HIP;
}

lmoe_status lmoe_route(lmoe_handle* h, const float* z_f32, int32_t T, int32_t* topk_idx,
                       float* topk_w, void* stream) {
  if (!h) return LMOE_ERR_INVALID_ARG;
  if (T < 0) return LMOE_ERR_INVALID_ARG;
  if (T > h->cfg.max_tokens) return LMOE_ERR_TOO_MANY_TOKENS;
  if (T == 0) return LMOE_OK;
  if (!z_f32 || !topk_idx || !topk_w || !aligned16(z_f32) || !aligned16(topk_idx) ||
      !aligned16(topk_w))
    return LMOE_ERR_INVALID_ARG;
  const lmoe_config& c = h->cfg;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = h->at<float>(h->L.logits);
  if (router_logits(z_f32, h->w.router, logits, T, c.n_routed_experts, c.moe_latent_size, s) !=
      hipSuccess)
    return LMOE_ERR_HIP;
  if (router_select(logits, h->w.router_bias, T, c.n_routed_experts, c.moe_latent_size,
                    c.num_experts_per_tok, c.n_group, c.topk_group, c.routed_scaling_factor,
                    topk_idx, topk_w, s) != hipSuccess)
    return LMOE_ERR_HIP;
  if (h->debug) {
    hipError_t e = hipStreamSynchronize(s);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) {
      std::fprintf(stderr, "lmoe: route failed: %s\n", hipGetErrorString(e));
      return LMOE_ERR_HIP;
    }
  }
  return LMOE_OK;
}

lmoe_status lmoe_forward(lmoe_handle* h, const uint16_t* x, int32_t T, uint16_t* y, void* stream,
                         const lmoe_taps* taps) {
  if (!h) return LMOE_ERR_INVALID_ARG;
  if (T < 0) return LMOE_ERR_INVALID_ARG;
  if (T > h->cfg.max_tokens) return LMOE_ERR_TOO_MANY_TOKENS;
  if (T == 0) return LMOE_OK;
  const lmoe_status st = check_io(h->cfg, x, T, y, taps);
  if (st != LMOE_OK) return st;
  hipEvent_t* ev = nullptr;
  if (h->prof_n < h->prof_max)
    ev = &h->events[static_cast<size_t>(h->prof_n++) * kEventsPerForward];
  return run_forward(h->cfg, h->w, h->L, h->ws, h->debug, h->aux, h->fork, h->join, ev, x, T, y,
                     static_cast<hipStream_t>(stream), taps);
}

lmoe_status lmoe_forward_noalloc(const lmoe_config* cfg, const lmoe_weights* w,
                                 const uint16_t* x, int32_t T, uint16_t* y, void* stream) {
  lmoe_status st = check_config(cfg);
  if (st != LMOE_OK) return st;
  st = check_weights(*cfg, w);
  if (st != LMOE_OK) return st;
  if (T < 0) return LMOE_ERR_INVALID_ARG;
  if (T > cfg->max_tokens) return LMOE_ERR_TOO_MANY_TOKENS;
  if (T == 0) return LMOE_OK;
  st = check_io(*cfg, x, T, y, nullptr);
  if (st != LMOE_OK) return st;
  // the workspace of a handle made for exactly T tokens, carved from the
  // static scratch instead of caller memory
  lmoe_config c = *cfg;
  c.max_tokens = T;
  const Layout L = make_layout(c);
  if (L.total > kScratchBytes) return LMOE_ERR_SCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cur = -1, sdev = -1;
  if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(s, &sdev) != hipSuccess)
    return LMOE_ERR_HIP;
  if (sdev != cur) return LMOE_ERR_INVALID_ARG;
  char* ws = nullptr;
  st = device_scratch(&ws);
  if (st != LMOE_OK) return st;
  // Every scratch byte a forward reads is written earlier in the same
  // forward (LDS-only atomics, no accumulation into device memory), so
  // nothing is cleared first.  One stream: no auxiliary stream or event.
  return run_forward(c, *w, L, ws, false, nullptr, nullptr, nullptr, nullptr, x, T, y, s,
                     nullptr);
}

}  // extern "C"
