"""The benchmark's roofline accounting on the CPU: the algorithmic bytes and
flops that every roofline fraction divides by, pinned to the page's layer
totals ("Nemotron 3 Ultra 架构深度拆解报告", §2.3.4 / §3.1.3: 10.74 G expert
parameters per MoE layer, 20.97 M per expert) and to counts done by hand for
the benchmark batches."""

import bench
import lmoe_inputs as li


def test_weights_read_once_add_up_to_the_layer():
    sh = li.FULL
    E = sh.n_routed_experts
    b, _ = bench.stage_work(sh, 0, E)          # no tokens: weights only
    # every expert touched: the page's 10.74 G expert parameters, 2 bytes each, per GEMM half
    assert b["expert_up"] + b["expert_down"] == 2 * 10_737_418_240
    assert b["expert_up"] == 2 * 20_971_520 // 2 * E
    # fc1_latent + fc2_latent + shared up + shared down in bf16, the gate in fp32
    D, R, S = sh.hidden_size, sh.moe_latent_size, sh.moe_shared_expert_intermediate_size
    assert b["proj_latent"] + b["proj_out"] + b["shared_up"] == 2 * (2 * D * R + 2 * D * S)
    assert b["router_logits"] == 4 * E * R


def test_decode_batch_expert_bytes_by_hand():
    # T = 32 tokens, 22 experts each: 704 slots; 375 distinct experts touched
    b, f = bench.stage_work(li.FULL, 32, 375)
    weights = 375 * 5120 * 2048 * 2
    acts = 704 * 2048 * 2 + 704 * 5120 * 2       # gathered latent rows in, expert hidden out
    assert b["expert_up"] == weights + acts == 7_874_412_544
    assert f["expert_up"] == 2 * 704 * 2048 * 5120
    # MXFP4: half a byte per weight plus one scale byte per 32
    bm, _ = bench.stage_work(li.FULL, 32, 375, bench.MXFP4_BYTES)
    assert bm["expert_up"] == 375 * 5120 * 2048 // 2 + 375 * 5120 * 2048 // 32 + acts


def test_prefill_flops_per_token():
    sh = li.FULL
    _, f = bench.stage_work(sh, 8192, 512)
    # the MFMA GEMMs (the fp32 gate and the combine's vector adds are not bf16 MFMA work)
    gemms = ("proj_latent", "shared_up", "expert_up", "expert_down", "proj_out")
    assert sum(f[k] for k in gemms) == bench.bf16_flops(sh, 8192)
    # 2 (2 D R + 2 K R F + 2 D S) per token: the page's ~1.33 GFLOP less the gate
    assert round(bench.bf16_flops(sh, 1) / 1e9, 4) == 1.3254


def test_block_fusion_adds_its_activation_bytes():
    sh = li.FULL
    b0, _ = bench.stage_work(sh, 32, 375)
    b1, _ = bench.stage_work(sh, 32, 375, block=True)
    D = sh.hidden_size
    # pre-norm: h and gamma read, bf16(gamma h) written, 1/rms written; residual: h read
    assert b1["proj_latent"] - b0["proj_latent"] == 32 * D * 2 + D * 2 + 32 * D * 2 + 32 * 4
    assert b1["proj_out"] - b0["proj_out"] == 32 * D * 2


def test_near_ties_counts_boundary_ties_only():
    """The benchmark's tie diagnostic on a hand-made router: four experts,
    K = 2, one latent coordinate.  Logits 3, 2, 2, 1 put the 2nd and 3rd
    scores level (a tie at the selection boundary); logits 3, 3, 1, 0 put
    the tie inside the selected set (no tie at the boundary); a bias that
    separates the two level experts by 1e-3 removes the tie."""
    import torch
    from dataclasses import replace
    sh = replace(li.FULL, n_routed_experts=4, num_experts_per_tok=2, moe_latent_size=1)
    z = torch.ones(1, 1)
    zero = torch.zeros(4, dtype=torch.float64)
    t = bench.near_ties(z, torch.tensor([[3.0], [2.0], [2.0], [1.0]]), zero, sh)
    assert t["count"] == 1 and t["min_gap"] == 0.0
    t = bench.near_ties(z, torch.tensor([[3.0], [3.0], [1.0], [0.0]]), zero, sh)
    assert t["count"] == 0 and t["min_gap"] > 0.1
    bias = torch.tensor([0.0, 1e-3, 0.0, 0.0], dtype=torch.float64)
    t = bench.near_ties(z, torch.tensor([[3.0], [2.0], [2.0], [1.0]]), bias, sh)
    assert t["count"] == 0 and abs(t["min_gap"] - 1e-3) < 1e-12
    # group-limited routing: not reported
    assert bench.near_ties(z, torch.ones(4, 1), zero, replace(sh, n_group=2, topk_group=1)) is None


def test_more_than_one_gpu_is_refused():
    """The benchmark runs on one GPU: --gpus above 1 exits with status 2 and
    a one-line JSON message, before touching torch or the library."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60, cwd=root)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_stored_traffic_profiles_use_the_benchmark_accounting():
    """Each committed HBM-traffic profile records, per stage, the algorithmic
    bytes that the benchmark's own accounting gives for the experts the
    profiled batch touched, and its source list is the one the benchmark
    checks its hash against."""
    import json
    import os
    for workload, (fname, sources) in bench.TRAFFIC_PROFILES.items():
        path = os.path.join(bench.ROOT, "profiles", fname)
        d = json.load(open(path))
        wl = li.workload(workload)
        sb, _ = bench.stage_work(wl.shape, wl.tokens, d["unique_experts"])
        assert set(d["stages"]) == set(sb)
        for st, rec in d["stages"].items():
            assert rec["algorithmic_bytes"] == int(sb[st]), (workload, st)
            assert rec["fetch_bytes"] > 0
        if "sources" in d:
            assert tuple(d["sources"]) == tuple(sources)


def test_streaming_batches_count_the_shared_down_projection_where_it_runs():
    """At T <= 64 the shared expert's down projection runs on the auxiliary
    stream with its up projection: its weight bytes and flops move from
    proj_out to shared_up, and the layer's totals do not change."""
    import re
    sh = li.FULL
    D, R, S = sh.hidden_size, sh.moe_latent_size, sh.moe_shared_expert_intermediate_size
    b, f = bench.stage_work(sh, 32, 375)
    assert b["proj_out"] == D * R * 2 + 32 * R * 2 + 32 * D * 2
    assert b["shared_up"] == S * D * 2 + 32 * D * 2 + 32 * S * 2 + D * S * 2 + 32 * S * 2
    assert f["proj_out"] == 2 * 32 * D * R and f["shared_up"] == 4 * 32 * D * S
    b65, f65 = bench.stage_work(sh, 65, 375)
    assert b65["proj_out"] == D * (R + S) * 2 + 65 * (R + S) * 2 + 65 * D * 2
    assert f["proj_out"] + f["shared_up"] == 2 * 32 * D * (R + S) + 2 * 32 * D * S
    # the threshold is the library's own
    src = open(bench.ROOT + "/sparse_moe_layer_latentmoe_amd/csrc/kernels.h").read()
    assert int(re.search(r"kStreamDenseMaxTokens = (\d+)", src).group(1)) == bench.STREAM_DENSE_MAX_TOKENS
