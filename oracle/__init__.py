"""CPU oracle for the LatentMoE feed-forward layer (forward pass).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or
calls this package: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg do.  It shares no code, header, table or
helper with the HIP library; both sides only consume the same seeded
inputs.

Every function here is plain NumPy on the host, written so that it can be
checked against the definition by eye:

* floating point is IEEE float64 everywhere the pages do not fix the
  precision (the latent projections, the experts, the shared expert, the
  combine);
* the router runs in float32 where the pages fix it: the gate is an fp32
  linear layer and the correction bias is kept in fp32 ("Nemotron 3 Ultra
  架构深度拆解报告", CH5 §5.4 and §5.6 Step 1), so logits, sigmoid scores
  and biased scores are float32 values (the dot products are accumulated
  in float64 and rounded once to float32).

Parity status of each function is listed in ``oracle.lmoe_oracle``'s
module docstring.
"""

from .lmoe_oracle import (  # noqa: F401
    OracleConfig,
    bf16_bits_to_f64,
    latent_projection,
    router_scores,
    select_experts,
    renormalize,
    expert_mlp,
    routed_experts,
    shared_expert,
    latent_up_projection,
    forward,
)
