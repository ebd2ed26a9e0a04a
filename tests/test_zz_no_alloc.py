"""prism_forward_static, the entry point that allocates nothing (its workspace is the
library's static scratch), against prism_plan + prism_attn_fwd with a caller-owned
workspace, through the C ABI: two calls in a row, the second on a smaller grid; outputs
must be bit-identical (same kernels, same inputs)."""
import pytest
import torch

import dynamic_block_sparse_stats_amd as P
from dynamic_block_sparse_stats_amd import synth

pytestmark = pytest.mark.gpu


def _with_workspace(cfg, inp):
    att = P.PrismAttention(cfg)
    att.plan(inp["q"], inp["k"], inp["v"], inp["a2v"])
    return att.forward()


def test_static_forward_matches_workspace_path():
    cases = [synth.custom(16, 16, 24, 3, 128, "bf16", top_k=4, top_p=0.8, seed=7),
             synth.custom(8, 16, 16, 2, 128, "bf16", top_k=3, top_p=0.5, seed=8)]
    assert cases[1].N * cases[1].heads < cases[0].N * cases[0].heads
    for wl in cases:
        inp = {k: v.cuda() for k, v in synth.make_inputs(wl, device="cpu").items()}
        cfg = P.config_for(wl)
        assert P.workspace_bytes(cfg) <= 128 << 20
        o = torch.full((wl.N, wl.heads, wl.head_dim), float("nan"), dtype=torch.bfloat16,
                       device="cuda")
        lse = torch.full((wl.heads, wl.N), float("nan"), dtype=torch.float32, device="cuda")
        P.forward_static(cfg, inp["q"], inp["k"], inp["v"], inp["a2v"], o, lse)
        ref_o, ref_lse = _with_workspace(cfg, inp)
        torch.cuda.synchronize()
        print(f"{wl.name}: {wl.heads} heads, workspace {P.workspace_bytes(cfg)} bytes",
              flush=True)
        assert torch.equal(o, ref_o), wl.name
        assert torch.equal(lse, ref_lse), wl.name
