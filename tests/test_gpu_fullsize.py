"""HIP path vs CPU oracle at the full workload sizes (720p, 1080p, 2K; 24 heads), in the
launch configuration the benchmark times.  The oracle recomputes the plan of every head in
full (zone shapes, permutation, block table, selection lists) and, for the first and last
head, a seeded sample of output rows one by one; gradients are checked
element by element with an upstream gradient that is zero except on a sample of query
rows (then every dK/dV row the oracle sums is exact, and all others must be zero)."""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_stats_amd as P
from dynamic_block_sparse_stats_amd import synth
import oracle
from parity import (check_close, check_grads, compare_plan, compare_selection, describe,
                    rows_of_exact_blocks, to_np)

pytestmark = pytest.mark.gpu


def _head_inputs(inp, h):
    return {n: inp[n][:, h].double().cpu().numpy() for n in ("q", "k", "v")}


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("cid,policy,fixed", [(1, None, None), (2, None, None), (4, None, None),
                                              (4, "pages", None), (4, "pages", (4, 4, 4))],
                         ids=["720p", "1080p", "2k", "2k-pages-operating-point",
                              "2k-pages-all-64-token-blocks"])
def test_fullsize(cid, policy, fixed):
    """With every block of 64 tokens (13,312 blocks per head) the forward and dQ walk query
    tiles of four blocks and dK/dV runs only its 64-key launch; there the oracle's plan is
    recomputed for the first and last head only (about half a minute each)."""
    wl = synth.workload(cid)
    print(f"\n== {wl.name} {policy or ''} {fixed or ''}: generating inputs", flush=True)
    inp = synth.make_inputs(wl, device="cuda", with_dout=False)
    over = dict(P.POLICIES[policy]) if policy else {}
    if fixed:
        over["fixed_shape"] = P.shape_code(*fixed)
    cfg = P.config_for(wl, **over)
    sel = dict(top_k=cfg.top_k, top_p=cfg.top_p, top_k_frac=cfg.top_k_frac,
               fixed_shape=cfg.fixed_shape)
    att = P.PrismAttention(cfg)
    att.plan(inp["q"], inp["k"], inp["v"], inp["a2v"])
    o, lse = att.forward()
    torch.cuda.synchronize()
    print("   plan + forward done", flush=True)
    rng = np.random.default_rng(100 + cid)
    a2v = inp["a2v"].double().cpu().numpy()
    # every head's plan and selection lists against the oracle; sampled attention rows
    # (and gradients) on the first and last head
    heads = [0, wl.heads - 1]
    samples = {}
    views = att.views()
    for h in (heads if fixed else range(wl.heads)):
        hi = _head_inputs(inp, h)
        op = oracle.plan_head(wl.T, wl.H, wl.W, hi["q"], hi["k"], hi["v"], a2v,
                              min_edge_log2=wl.min_edge_log2, **sel)
        rep = compare_plan(views, h, op)
        assert not rep.get("downstream_skipped"), rep
        exact, excl, nnz = compare_selection(views, h, op, cfg.top_p)
        if h not in heads:
            print(f"   head {h}: plan and selection match (nb {op.nb} nnz {nnz} excluded "
                  f"{excl} near-tie zones {rep['near_tie_zones']})", flush=True)
            continue
        ok_rows = np.nonzero(rows_of_exact_blocks(op, exact))[0]
        rows = np.sort(rng.choice(ok_rows, size=64, replace=False))
        oo, ol = oracle.attn_fwd(op, hi["q"], hi["k"], hi["v"], rows=rows)
        e_o, r_o, _ = check_close(o[rows, h].float().cpu().numpy(), oo[rows], "bf16", f"h{h} O")
        e_l, r_l, _ = check_close(lse[h, rows].cpu().numpy(), ol[rows], "bf16", f"h{h} lse")
        print(f"   head {h}: nb {op.nb} nnz {nnz} excluded {excl} near-tie zones "
              f"{rep['near_tie_zones']} | O err {e_o:.2e} (bound use {r_o:.2f}) "
              f"lse err {e_l:.2e}", flush=True)
        samples[h] = (op, hi, rows)
    if not wl.backward:
        return
    # gradients: upstream gradient nonzero on 16 sampled rows of each checked head
    dout = torch.zeros(wl.N, wl.heads, wl.head_dim, dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(7 + cid)
    brows = {}
    for h in heads:
        br = samples[h][2][::4][:16]
        brows[h] = br
        idx = torch.from_numpy(br).cuda()
        dout[idx, h] = torch.randn(len(br), wl.head_dim, generator=g, device="cuda").bfloat16()
    dq, dk, dv = att.backward(dout)
    torch.cuda.synchronize()
    print("   backward done", flush=True)
    for h in heads:
        op, hi, _ = samples[h]
        br = brows[h]
        d_np = dout[:, h].double().cpu().numpy()
        rq, rk, rv, mq, mk, mv = oracle.attn_bwd(op, hi["q"], hi["k"], hi["v"], d_np, rows=br,
                                                 with_mag=True)
        res = check_grads({n: t[:, h].float().cpu().numpy() for n, t in
                           (("dq", dq), ("dk", dk), ("dv", dv))},
                          dict(dq=rq, dk=rk, dv=rv), dict(dq=mq, dk=mk, dv=mv), "bf16", f"h{h}")
        nz = int((np.abs(rv).sum(1) > 0).sum())
        print(f"   head {h}: " + "; ".join(describe(n, c) for n, c in res.items())
              + f" ({nz} key rows with nonzero gradient)", flush=True)
