#!/usr/bin/env python3
"""Benchmark of the LatentMoE layer forward pass on one MI355X.

One step = one whole forward of the layer (every kernel of the path) over one
batch of synthetic tokens, weights and inputs resident in HBM.  Prints ONE
JSON line: tokens/s of the layer (K timed forwards with nothing else on the
stream), the roofline of its dominant kernel (timed live with HIP events
around every stage, on the stream the stage runs on, over K further
forwards), the layer-level roofline fraction, and the CPU oracle timed on a
bounded sample of the same workload on the host's cores.

Default run: the full-shape decode batch (T = 32 tokens; hidden 8192, latent
2048, 512 experts top-22, expert MLP 2048->5120->2048, shared expert
8192->10240->8192; bf16 weights and activations, fp32 router) is the headline,
and the line also carries one block per benchmark configuration (tiny T = 64,
decode T = 32, MTP verify T = 192, prefill T = 8192, skewed routing
T = 8192), each timed the same way on one set of full-shape weights.
``--workload NAME`` runs one workload alone.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LatentMoE layer tokens/s; % HBM roofline (decode) / % bf16 MFMA peak (prefill)"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
HBM_BOUND = {"tiny", "decode", "mtp_verify", "decode_grouped", "decode_mxfp4",
             "mtp_verify_mxfp4"}
MXFP4_BYTES = 0.5 + 1.0 / 32
# Batches of at most this many tokens stream the dense weights, and run the
# shared expert's down projection on the auxiliary stream (timed with
# shared_up); the output projection then covers fc2_latent only.
STREAM_DENSE_MAX_TOKENS = 64


def stage_work(sh, T, U, expert_weight_bytes=2.0, block=False):
    """Algorithmic bytes and flops of each stage for T tokens touching U
    distinct experts (weights read once, activations read/written once);
    expert weights take ``expert_weight_bytes`` per element (2 for bf16,
    0.5 + 1/32 for MXFP4: half a byte per element plus a scale byte per 32).
    ``block``: the block's pre-norm (timed inside proj_latent: h and gamma
    read, bf16(gamma h) and 1/rms written) and residual (h read by proj_out)
    are fused in.  For weight-streaming batches (T <= STREAM_DENSE_MAX_TOKENS)
    the shared expert's down projection (Wsd and Hs read) is counted in the
    stage it runs in, shared_up; the fp32 hand-over between the two launches
    is not algorithmic traffic and is not counted."""
    D, R, E = sh.hidden_size, sh.moe_latent_size, sh.n_routed_experts
    K, F, S = sh.num_experts_per_tok, sh.moe_intermediate_size, sh.moe_shared_expert_intermediate_size
    slots = T * K
    b = {
        "proj_latent": R * D * 2 + T * D * 2 + T * R * 6,
        "shared_up": S * D * 2 + T * D * 2 + T * S * 2,
        "router_logits": E * R * 4 + T * R * 4 + T * E * 4,
        "router_select": T * E * 4 + E * 4 + slots * 8,
        "dispatch": slots * 4 * 4 + E * 12,
        "expert_up": int(U * F * R * expert_weight_bytes) + slots * R * 2 + slots * F * 2,
        "expert_down": int(U * R * F * expert_weight_bytes) + slots * F * 2 + slots * R * 2,
        "combine": slots * R * 2 + slots * 8 + T * R * 2,
        "proj_out": D * (R + S) * 2 + T * (R + S) * 2 + T * D * 2,
    }
    if block:
        b["proj_latent"] += T * D * 2 + D * 2 + T * D * 2 + T * 4
        b["proj_out"] += T * D * 2
    split = T <= STREAM_DENSE_MAX_TOKENS
    if split:
        moved = D * S * 2 + T * S * 2
        b["shared_up"] += moved
        b["proj_out"] -= moved
    f = {
        "proj_latent": 2 * T * D * R,
        "shared_up": 2 * T * D * S,
        "router_logits": 2 * T * R * E,
        "router_select": 0, "dispatch": 0,
        "expert_up": 2 * slots * R * F,
        "expert_down": 2 * slots * F * R,
        "combine": 2 * slots * R,
        "proj_out": 2 * T * D * (R + S),
    }
    if split:
        f["shared_up"] += 2 * T * D * S
        f["proj_out"] -= 2 * T * D * S
    return b, f


# Device code each stored counter measurement depends on: the kernel sources
# and device headers the workload runs (decode: weight streaming only; MTP
# verify also takes the LDS-tiled split-k GEMMs for its dense projections).
DECODE_SOURCES = ("gemm_stream.hip", "router.hip", "dispatch.hip", "gemm_problems.h",
                  "lmoe_device.h")
TRAFFIC_PROFILES = {
    "decode": ("traffic_decode_T32.json", DECODE_SOURCES),
    "mtp_verify": ("traffic_mtp_verify_T192.json", DECODE_SOURCES + ("gemm_tiled.hip",)),
    "prefill": ("traffic_prefill_T8192.json", DECODE_SOURCES + ("gemm_tiled.hip",)),
}


def source_sha256(device=DECODE_SOURCES):
    """Hash of the device code a workload runs (the kernel sources and the
    device headers, not the host-side launch code), to tell whether stored
    counter data still describes the kernels being run."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "sparse_moe_layer_latentmoe_amd", "csrc", "*"))):
        if os.path.basename(f) not in device:
            continue
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` (calibrated FETCH_SIZE + WRITE_SIZE
    from the rocprofv3 counter runs kept under profiles/), or None when no
    such measurement exists for this workload or the kernels have changed
    since it was taken."""
    if workload not in TRAFFIC_PROFILES:
        return None
    fname, sources = TRAFFIC_PROFILES[workload]
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    st = d.get("stages", {}).get(stage)
    if st is None or d.get("source_sha256") != source_sha256(sources):
        return None
    return int(st["fetch_bytes"] + st["write_bytes"])


def bf16_flops(sh, T):
    D, R, K, F, S = (sh.hidden_size, sh.moe_latent_size, sh.num_experts_per_tok,
                     sh.moe_intermediate_size, sh.moe_shared_expert_intermediate_size)
    return 2 * T * (2 * D * R + 2 * K * R * F + 2 * D * S)


def blas_info():
    """The BLAS library NumPy calls (name, version, threads), from threadpoolctl."""
    try:
        from threadpoolctl import threadpool_info
        libs = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception:
        libs = []
    if not libs:
        return {"library": "unknown", "version": None,
                "threads": len(os.sched_getaffinity(0))}
    p = max(libs, key=lambda q: q.get("num_threads", 1))
    return {"library": p.get("internal_api", "unknown"), "version": p.get("version"),
            "threads": int(p.get("num_threads", 1))}


class HostExperts:
    """``obj[e]``: expert e's bf16 bits, copied to the host before the timer
    for the experts in ``experts``, on demand for any other (none, unless
    the oracle routes a tie token differently)."""

    def __init__(self, t, experts):
        import lmoe_inputs as li
        self.t = t
        self.cache = {int(e): li.bf16_bits(t[int(e)]) for e in experts}

    def __getitem__(self, e):
        import lmoe_inputs as li
        e = int(e)
        if e not in self.cache:
            self.cache[e] = li.bf16_bits(self.t[e])
        return self.cache[e]


def oracle_flops(sh, T):
    """Algorithmic flops of the layer for T tokens: the bf16 GEMMs and the
    fp32 gate (the oracle computes both)."""
    return bf16_flops(sh, T) + 2 * T * sh.moe_latent_size * sh.n_routed_experts


def cpu_baseline(inp, sh, experts, tiny_inp, tiny_reps=3):
    """The CPU oracle, as it stands, on the host's cores: once on the whole
    full-shape batch ``inp`` (the touched experts ``experts`` copied to the
    host before the timer; the timed region is the oracle forward, which
    upcasts each expert it visits), and ``tiny_reps`` times on the tiny
    configuration's batch ``tiny_inp``."""
    import numpy as np
    import lmoe_inputs as li
    from oracle import lmoe_oracle as O

    def ocfg(s):
        return O.OracleConfig(s.hidden_size, s.moe_latent_size, s.n_routed_experts,
                              s.num_experts_per_tok, s.moe_intermediate_size,
                              s.moe_shared_expert_intermediate_size, s.routed_scaling_factor)

    blas = blas_info()
    hw = li.HostWeights(inp)                       # dense weights copied to the host
    hw.expert_up = HostExperts(inp.expert_up, experts)
    hw.expert_down = HostExperts(inp.expert_down, experts)
    x = li.bf16_bits(inp.x)
    T = x.shape[0]
    t0 = time.perf_counter()
    O.forward(x, hw, ocfg(sh))
    dt = time.perf_counter() - t0
    del hw
    tsh = tiny_inp.workload.shape
    thw = li.HostWeights(tiny_inp, eager_experts=True)
    tx = li.bf16_bits(tiny_inp.x)
    tt = []
    for _ in range(tiny_reps):
        t1 = time.perf_counter()
        O.forward(tx, thw, ocfg(tsh))
        tt.append(time.perf_counter() - t1)
    tmed = float(np.median(tt))
    Tt = tx.shape[0]
    return {"value": round(T / dt, 3), "unit": "tokens/s", "cores": blas["threads"],
            "kind": "oracle",
            "sample": (f"the whole decode batch ({T} tokens, full shape) once through the "
                       f"float64 NumPy oracle; the {len(experts)} touched experts copied to "
                       f"the host before the timer, their upcast inside it; "
                       f"{blas['library']} {blas['version']} with {blas['threads']} threads, "
                       f"{len(os.sched_getaffinity(0))} host cpus"),
            "s_per_layer": round(dt, 4),
            "gflops": round(oracle_flops(sh, T) / dt / 1e9, 2),
            "blas": blas, "host_cpus": len(os.sched_getaffinity(0)),
            "tiny": {"tokens": Tt, "reps": tiny_reps, "s_per_layer": [round(v, 5) for v in tt],
                     "median_s_per_layer": round(tmed, 5),
                     "tokens_per_s": round(Tt / tmed, 1),
                     "gflops": round(oracle_flops(tsh, Tt) / tmed / 1e9, 3)}}


def library_ceiling(inp, sh, T, stage_ms, reps=5):
    """torch's bf16 matmul (the vendor GEMM library) on the layer's GEMM
    shapes, timed like the layer's stages: a yardstick for the hand-written
    GEMMs, never part of the layer.  Dense: the latent and shared-expert up
    projections (x against W1, Wsu) and the output projection ([r | Hs]
    against [W2 | Wsd]).  Experts: a batched stand-in with every expert
    given the mean row count T K / E, contiguous rows (no gather, no fused
    relu^2) and weights copied to [E, in, out]; the layer's own expert GEMMs
    run on the real, uneven per-expert counts."""
    import torch
    import torch.nn.functional as Fn
    D, R, S = sh.hidden_size, sh.moe_latent_size, sh.moe_shared_expert_intermediate_size
    E, K, F = sh.n_routed_experts, sh.num_experts_per_tok, sh.moe_intermediate_size

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    res = {}
    x = inp.x
    res["proj_latent"] = (timed(lambda: Fn.linear(x, inp.fc1_latent)), 2.0 * T * D * R)
    res["shared_up"] = (timed(lambda: Fn.linear(x, inp.shared_up)), 2.0 * T * D * S)
    a_out = torch.randn(T, R + S, device=x.device, dtype=torch.bfloat16)
    w_out = torch.cat([inp.fc2_latent, inp.shared_down], dim=1).contiguous()
    res["proj_out"] = (timed(lambda: Fn.linear(a_out, w_out)), 2.0 * T * D * (R + S))
    del a_out, w_out
    M = max(1, round(T * K / E))
    for name, w, kin, kout in (("expert_up", inp.expert_up, R, F),
                               ("expert_down", inp.expert_down, F, R)):
        wt = w.transpose(1, 2).contiguous()           # [E, in, out]
        act = torch.randn(E, M, kin, device=x.device, dtype=torch.bfloat16)
        res[name] = (timed(lambda: torch.bmm(act, wt)), 2.0 * E * M * kin * kout)
        del wt, act
    torch.cuda.empty_cache()
    return {"what": "torch bf16 matmul on the same GEMM shapes (experts: batched stand-in, "
                    f"{M} rows per expert)",
            "library_ms": {k: round(v[0], 4) for k, v in res.items()},
            "library_tflops": {k: round(v[1] / v[0] / 1e9, 1) for k, v in res.items()},
            "layer_ms": {k: round(stage_ms[k], 4) for k in res if k in stage_ms}}


def near_ties(z32, wg, bias, sh, eps=1e-6):
    """Tokens whose K-th and (K+1)-th selection scores (sigmoid(z Wg^T) + bias,
    from the layer's own fp32 latent, evaluated in float64) differ by less
    than eps: where rounding may decide which expert is chosen.  Reported
    only for ungrouped routing (None otherwise); a diagnostic computed after
    the first forward, outside the timed region."""
    import torch
    K = sh.num_experts_per_tok
    if sh.n_group != 1 or K >= sh.n_routed_experts:
        return None
    sel = torch.sigmoid(z32.double() @ wg.double().t()) + bias.double()
    top = torch.topk(sel, K + 1, dim=1).values
    gap = top[:, K - 1] - top[:, K]
    return {"count": int((gap < eps).sum().item()), "min_gap": float(gap.min().item()),
            "eps": eps}


def copy_calibration(torch, nbytes=4 << 30, launches=3):
    """Read and write nbytes per launch with one elementwise kernel (int32 negation: 16-byte
    vector loads and stores), so that a counter run over it shows what FETCH_SIZE and
    WRITE_SIZE read for a known number of bytes."""
    dev = torch.device("cuda:0")
    a = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(launches):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": nbytes,
                                           "bytes_written_per_launch": nbytes,
                                           "launches": launches,
                                           "check": int(b[-1].item())}}))


FULL_CONFIGS = ("decode", "mtp_verify", "prefill", "skewed")
ALL_CONFIGS = ("tiny",) + FULL_CONFIGS
WORKLOADS = ["all", "tiny", "decode", "mtp_verify", "prefill", "skewed", "decode_grouped",
             "decode_mxfp4", "mtp_verify_mxfp4", "decode_block", "mtp_verify_block",
             "prefill_block", "decode_mxfp4_block", "prefill_mxfp4"]


def parse_workload(name):
    """(layer workload, MXFP4 experts?, block steps fused?) of a --workload name."""
    import lmoe_inputs as li
    block = name.endswith("_block")
    base = name[:-len("_block")] if block else name
    mxfp4 = base.endswith("_mxfp4")
    return li.workload(base[:-len("_mxfp4")] if mxfp4 else base), mxfp4, block


def build_layer(torch, pkg, li, name, dev, weights=None):
    """Inputs and a layer for the --workload ``name``; full-shape workloads
    reuse ``weights`` (the skewed one with its own correction bias)."""
    wl, mxfp4, block = parse_workload(name)
    if weights is not None and wl.bias_recipe == "zipf":
        weights = dict(weights)
        weights["router_bias"] = torch.from_numpy(
            li.zipf_bias(wl.shape, wl.seed + 3, wl.zipf_s, wl.zipf_dead_frac,
                         x_std=wl.x_std, w_std=wl.w_std)).to(dev)
    inp = li.make_inputs(wl, dev, weights=weights)
    lw = {k: getattr(inp, k) for k in (
        "fc1_latent", "router", "router_bias", "expert_up", "expert_down",
        "fc2_latent", "shared_up", "shared_down")}
    if block:
        # the block's pre-norm and residual fused: x is the residual stream
        lw["norm_weight"] = li.make_norm_weight(wl, dev)
    if mxfp4:
        # routed experts stored as MXFP4, quantised by the library's kernel
        up_c, up_s = pkg.quantize_mxfp4(inp.expert_up)
        dn_c, dn_s = pkg.quantize_mxfp4(inp.expert_down)
        lw.update(expert_up=None, expert_down=None, expert_up_mxfp4=up_c,
                  expert_up_scale=up_s, expert_down_mxfp4=dn_c, expert_down_scale=dn_s)
    layer = pkg.LatentMoE(wl.shape, lw, max_tokens=wl.tokens,
                          expert_format=pkg.EXPERTS_MXFP4 if mxfp4 else pkg.EXPERTS_BF16,
                          fuse=pkg.FUSE_BLOCK if block else 0)
    return inp, layer


def describe(name, sh, T, mxfp4, block):
    return (f"{name}: LatentMoE layer forward, T={T} tokens, hidden {sh.hidden_size}, latent "
            f"{sh.moe_latent_size}, {sh.n_routed_experts} experts top-{sh.num_experts_per_tok}, "
            f"expert MLP {sh.moe_intermediate_size}, shared "
            f"{sh.moe_shared_expert_intermediate_size}, "
            + ("MXFP4 routed-expert weights (decoded to bf16), other weights bf16"
               if mxfp4 else "bf16 weights")
            + ", fp32 router"
            + (", block pre-norm RMSNorm and residual add fused" if block else ""))


def measure(torch, pkg, name, inp, layer, steps, warmup, use_graph=False):
    """Time one workload: K forwards with nothing else on the stream (the
    value), then K more with per-stage HIP events (the per-kernel times the
    rooflines use).  Returns the workload's result block."""
    wl, mxfp4, block = parse_workload(name)
    sh, T = wl.shape, wl.tokens
    dev = inp.x.device
    y = torch.empty_like(inp.x)
    counts = torch.empty(sh.n_routed_experts, dtype=torch.int32, device=dev)
    z_tap = torch.empty(T, sh.moe_latent_size, dtype=torch.float32, device=dev)
    layer.forward_into(inp.x, y, pkg.Taps(expert_counts=counts, z_f32=z_tap))
    torch.cuda.synchronize()
    ties = near_ties(z_tap, inp.router, inp.router_bias, sh)
    del z_tap
    U = int((counts > 0).sum().item())
    # load balance of the batch: busiest expert over the mean load, idle experts
    max_vio = float(counts.max().item()) / (T * sh.num_experts_per_tok / sh.n_routed_experts)
    empty = sh.n_routed_experts - U
    for _ in range(warmup):
        layer.forward_into(inp.x, y)
    torch.cuda.synchronize()

    graph = None
    if use_graph:
        # one forward captured into a HIP graph (the forward has no memset and
        # no host synchronisation); its replays are the timed steps
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            layer.forward_into(inp.x, y)
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()

    # Timed region: K forwards with nothing else on the stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if graph is not None:
            graph.replay()
        else:
            layer.forward_into(inp.x, y)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps

    # Per-kernel durations: K more forwards with a HIP event pair around every
    # stage, recorded on the stream each stage runs on.  The events cost a few
    # microseconds each, so they stay out of the region timed above.
    layer.profile_begin(steps)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(steps):
        layer.forward_into(inp.x, y)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    stages, nf = layer.profile_end()
    ms_events = (t3 - t2) * 1e3 / steps
    stage_ms = {k: v / max(nf, 1) for k, v in stages.items()}

    sb, sf = stage_work(sh, T, U, MXFP4_BYTES if mxfp4 else 2.0, block)
    hbm = parse_workload(name)[0].name in HBM_BOUND
    dom = max(stage_ms, key=stage_ms.get)
    if hbm:
        ach = sb[dom] / (stage_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(name, dom), "kernel": dom,
                "algorithmic_bytes_per_launch": sb[dom], "avg_launch_ms": round(stage_ms[dom], 5)}
        layer_bytes = sum(sb.values())
        layer_ach = layer_bytes / (ms * 1e-3) / 1e9
        layer_roof = {"bound": "hbm", "achieved": round(layer_ach, 1), "unit": "GB/s",
                      "frac": round(layer_ach / HBM_PEAK_GBS, 4), "algorithmic_bytes": layer_bytes}
        # HBM bytes the counters measured for one whole forward (every stage),
        # over the forward's wall time; null without a current measurement
        measured = [measured_traffic(name, st) for st in sb]
        if measured and all(m is not None for m in measured):
            mb = sum(measured)
            layer_roof["measured_bytes"] = mb
            layer_roof["measured_achieved"] = round(mb / (ms * 1e-3) / 1e9, 1)
            layer_roof["measured_frac"] = round(mb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        else:
            layer_roof["measured_bytes"] = None
    else:
        ach = sf[dom] / (stage_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(name, dom),
                "kernel": dom, "algorithmic_flops_per_launch": sf[dom],
                "avg_launch_ms": round(stage_ms[dom], 5)}
        fl = bf16_flops(sh, T)
        layer_ach = fl / (ms * 1e-3) / 1e12
        layer_roof = {"bound": "mfma", "achieved": round(layer_ach, 1), "unit": "TFLOP/s",
                      "frac": round(layer_ach / BF16_PEAK_TFLOPS, 4), "algorithmic_bf16_flops": fl}
    return {
        "workload": describe(name, sh, T, mxfp4, block),
        "tokens": T, "seed": wl.seed,
        "ms_per_step": round(ms, 5), "us_per_layer": round(ms * 1e3, 2),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "unique_experts": U, "empty_experts": empty, "max_violation": round(max_vio, 3),
        "near_ties": ties,
        "roofline": roof, "layer_roofline": layer_roof,
        "stages_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "launch": "replays of one captured HIP graph" if graph is not None else "direct calls",
        "stage_timing": f"{nf} further forwards with per-stage HIP events "
                        f"({ms_events:.4f} ms/step with the events)",
        "touched_experts": torch.nonzero(counts > 0).flatten().tolist(),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all", choices=WORKLOADS,
                    help="one workload, or 'all' (default): the decode batch as the headline "
                         "and every benchmark configuration (tiny, decode, MTP verify, "
                         "prefill, skewed) in a block of its own, on one set of full-shape "
                         "weights")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--library-ceiling", action="store_true",
                    help="also time torch's bf16 matmul (the vendor GEMM library) on the "
                         "layer's GEMM shapes, as a throughput yardstick (not the layer)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one captured HIP graph of the forward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain elementwise copy of 4 GiB three times (torch.neg "
                         "on int32), the known traffic that scales the FETCH_SIZE and "
                         "WRITE_SIZE counters")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import lmoe_inputs as li
    import sparse_moe_layer_latentmoe_amd as pkg

    dev = torch.device("cuda:0")
    names = ALL_CONFIGS if args.workload == "all" else (args.workload,)
    head_name = "decode" if args.workload == "all" else args.workload
    full_w = None
    if any(parse_workload(n)[0].shape == li.FULL for n in names):
        # one set of full-shape weights for every full-shape workload
        full_w = li.make_weights(li.workload("decode"), dev)
    blocks, keep = {}, {}
    for n in names:
        wl = parse_workload(n)[0]
        inp, layer = build_layer(torch, pkg, li, n, dev,
                                 full_w if wl.shape == li.FULL else None)
        print(f"[bench {n} T={wl.tokens}]", file=sys.stderr, flush=True)
        blocks[n] = measure(torch, pkg, n, inp, layer, args.steps, args.warmup, args.graph)
        if n == head_name and args.library_ceiling:
            blocks[n]["library_ceiling"] = library_ceiling(inp, wl.shape, wl.tokens,
                                                           blocks[n]["stages_ms"])
        layer.close()
        del layer
        if n in (head_name, "tiny"):
            keep[n] = inp
        else:
            del inp
        torch.cuda.empty_cache()

    head = blocks[head_name]
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"], "tokens": head["tokens"], "seed": head["seed"],
                   "unique_experts": head["unique_experts"],
                   "empty_experts": head["empty_experts"],
                   "max_violation": head["max_violation"], "near_ties": head["near_ties"],
                   "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "layer_roofline": head["layer_roofline"],
        "us_per_layer": head["us_per_layer"],
        "stages_ms": head["stages_ms"],
        "launch": head["launch"],
        "stage_timing": head["stage_timing"],
    }
    if "library_ceiling" in head:
        out["library_ceiling"] = head["library_ceiling"]
    if len(blocks) > 1:
        out["configs"] = {n: {k: v for k, v in b.items() if k != "touched_experts"}
                          for n, b in blocks.items()}
    wl_head, mx_head, blk_head = parse_workload(head_name)
    if not args.no_cpu_baseline and not mx_head and not blk_head and wl_head.shape == li.FULL:
        tiny_inp = keep.get("tiny") or li.make_inputs(li.workload("tiny"), dev)
        out["cpu_baseline"] = cpu_baseline(keep[head_name], wl_head.shape,
                                           head["touched_experts"], tiny_inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
