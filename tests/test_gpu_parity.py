"""HIP path vs CPU oracle on small grids that span several tiles and ragged tails
(called through the C ABI; the oracle never sees anything the GPU produced)."""
import math

import numpy as np
import pytest
import torch

import dynamic_block_sparse_stats_amd as P
from dynamic_block_sparse_stats_amd import synth
import oracle
from parity import (TOL, check_close, compare_plan, compare_selection, oracle_plan,
                    rows_of_exact_blocks, run_plan, to_np)

pytestmark = pytest.mark.gpu


def _inputs(wl, with_dout=False):
    inp = synth.make_inputs(wl, device="cpu", with_dout=with_dout)
    return inp, {k: v.cuda() for k, v in inp.items()}


def _check_head(wl, cfg, att, inp_cpu, h, o, lse, a2v=True, **over):
    op = oracle_plan(wl, inp_cpu, h, a2v=a2v, **over)
    views = att.views()
    rep = compare_plan(views, h, op)
    assert not rep.get("downstream_skipped"), rep
    exact, excl, nnz = compare_selection(views, h, op, cfg.top_p, to_np(views["scores"])
                                         if h == cfg.num_heads - 1 else None)
    oo, ol, mo = oracle.attn_fwd(op, inp_cpu["q"][:, h], inp_cpu["k"][:, h],
                                 inp_cpu["v"][:, h], with_mag=True)
    rows = rows_of_exact_blocks(op, exact)
    go = o[:, h].float().cpu().numpy()
    gl = lse[h].cpu().numpy()
    err_o, r_o = check_close(go[rows], oo[rows], wl.dtype, f"head {h} O", mo[rows])
    err_l, r_l = check_close(gl[rows], ol[rows], "f32" if wl.dtype == "f32" else "bf16",
                             f"head {h} lse")
    print(f"head {h}: nb {op.nb} nnz {nnz} excluded {excl} near-tie zones "
          f"{rep['near_tie_zones']} max|O| {np.abs(oo).max():.2f} max|dO| {err_o:.2e} "
          f"(bound use {r_o:.2f}) max|dlse| {err_l:.2e}", flush=True)
    return op, exact


@pytest.mark.parametrize("use_a2v", [True, False])
def test_tiny_fp32_plan_and_forward(use_a2v):
    wl = synth.workload(0)
    inp_cpu, inp = _inputs(wl)
    cfg = P.config_for(wl)
    att = run_plan(cfg, inp, a2v=use_a2v)
    o, lse = att.forward()
    torch.cuda.synchronize()
    for h in range(wl.heads):
        _check_head(wl, cfg, att, inp_cpu, h, o, lse, a2v=use_a2v)


def test_tiny_fp32_topk_all_is_dense():
    """Top-k = all blocks: the sparse path reduces to dense softmax attention."""
    wl = synth.workload(0)
    inp_cpu, inp = _inputs(wl)
    cfg = P.config_for(wl, top_k=wl.N // 64)
    att = run_plan(cfg, inp)
    o, lse = att.forward()
    torch.cuda.synchronize()
    cnt = att.views()["sel_count"]
    for h in range(wl.heads):
        nb = int(att.views()["zone_block"][h, -1])
        assert torch.all(cnt[h, :nb] == nb)
        q, k, v = (inp_cpu[n][:, h].double().numpy() for n in ("q", "k", "v"))
        s = q @ k.T / math.sqrt(wl.head_dim)
        m = s.max(1, keepdims=True)
        e = np.exp(s - m)
        od = (e / e.sum(1, keepdims=True)) @ v
        ld = (m + np.log(e.sum(1, keepdims=True)))[:, 0]
        assert np.abs(o[:, h].cpu().numpy() - od).max() <= 1e-4
        assert np.abs(lse[h].cpu().numpy() - ld).max() <= 1e-4


def test_tiny_fp32_backward():
    wl = synth.workload(0)
    inp_cpu, inp = _inputs(wl, with_dout=True)
    cfg = P.config_for(wl)
    att = run_plan(cfg, inp)
    o, lse = att.forward()
    dq, dk, dv = att.backward(inp["dout"])
    torch.cuda.synchronize()
    for h in range(wl.heads):
        op, exact = _check_head(wl, cfg, att, inp_cpu, h, o, lse)
        assert exact.all()
        g = oracle.attn_bwd(op, inp_cpu["q"][:, h], inp_cpu["k"][:, h], inp_cpu["v"][:, h],
                            inp_cpu["dout"][:, h])
        for name, gpu, ref in (("dq", dq, g[0]), ("dk", dk, g[1]), ("dv", dv, g[2])):
            err, _ = check_close(gpu[:, h].cpu().numpy(), ref, "f32", f"head {h} {name}")
            print(f"head {h} {name}: max abs err {err:.3e}", flush=True)


@pytest.mark.parametrize("T,H,W,heads,mel,k,p", [
    (8, 24, 40, 2, 1, 8, 0.9),     # 15 zones: ragged score tiles and bitmask words
    (16, 16, 16, 3, 0, 4, 0.5),    # 19-shape pool
    (8, 16, 32, 2, 1, 1, 0.2),     # the pages' p with k = 1
])
def test_bf16_small_forward(T, H, W, heads, mel, k, p):
    wl = synth.custom(T, H, W, heads, 128, "bf16", top_k=k, top_p=p, min_edge_log2=mel,
                      seed=T + H + W)
    inp_cpu, inp = _inputs(wl)
    cfg = P.config_for(wl)
    att = run_plan(cfg, inp)
    o, lse = att.forward()
    torch.cuda.synchronize()
    for h in range(heads):
        _check_head(wl, cfg, att, inp_cpu, h, o, lse)


@pytest.mark.parametrize("T,H,W,bg,seed,need256", [
    (8, 16, 24, 1.0, 5, False),
    (16, 32, 32, 0.15, 3, True),   # near-uniform field: 256-token blocks (two key tiles each)
])
def test_bf16_small_backward(T, H, W, bg, seed, need256):
    wl = synth.custom(T, H, W, 2, 128, "bf16", top_k=4, top_p=0.8, bg_amp=bg, seed=seed)
    inp_cpu, inp = _inputs(wl, with_dout=True)
    cfg = P.config_for(wl)
    att = run_plan(cfg, inp)
    codes = att.views()["zone_shape"].cpu().numpy()
    log2vol = ((codes >> 4) & 3) + ((codes >> 2) & 3) + (codes & 3)
    sizes = {b: int((log2vol == lb).sum()) for b, lb in ((64, 6), (128, 7), (256, 8))}
    print(f"zones by block size: {sizes}", flush=True)
    if need256:
        assert sizes[256] > 0
    o, lse = att.forward()
    dq, dk, dv = att.backward(inp["dout"])
    torch.cuda.synchronize()
    for h in range(wl.heads):
        op, exact = _check_head(wl, cfg, att, inp_cpu, h, o, lse)
        if not exact.all():
            pytest.skip("selection differs at a near-threshold block; gradient rows excluded")
        g = oracle.attn_bwd(op, inp_cpu["q"][:, h], inp_cpu["k"][:, h], inp_cpu["v"][:, h],
                            inp_cpu["dout"][:, h], with_mag=True)
        for name, gpu, ref, mag in (("dq", dq, g[0], g[3]), ("dk", dk, g[1], g[4]),
                                    ("dv", dv, g[2], g[5])):
            err, ratio = check_close(gpu[:, h].float().cpu().numpy(), ref, "bf16",
                                     f"head {h} {name}", mag)
            print(f"head {h} {name}: max|ref| {np.abs(ref).max():.2f} max abs err {err:.3e} "
                  f"(bound use {ratio:.2f})", flush=True)


def _unit_list_lengths(views, h):
    """Per query block, the units of its selected key blocks; per key block selected by at
    least one query block, the units of those query blocks; and the key blocks nobody
    selected."""
    nb = int(views["zone_block"][h, -1])  # the head's block count
    bsz = views["block_size"][h, :nb].cpu().numpy() // 64
    cnt = views["sel_count"][h, :nb].cpu().numpy()
    col = views["csr_col"][h, :nb].cpu().numpy()
    ccnt = views["csc_count"][h, :nb].cpu().numpy()
    crow = views["csc_row"][h, :nb].cpu().numpy()
    q_units = [int(bsz[col[i, :cnt[i]]].sum()) for i in range(nb)]
    k_units = [int(bsz[crow[j, :ccnt[j]]].sum()) for j in range(nb) if ccnt[j] > 0]
    return q_units, k_units, int((ccnt == 0).sum())


def test_bf16_short_lists():
    """Pure Top-k with k = 1, 2, 3 (Top-p off): selection lists of a few units, so the
    unrolled unit loops of the three attention kernels end at every stage position, and
    key blocks that no query block selected get zero dK and dV."""
    fwd_res, kv_res, unselected = set(), set(), 0
    for k in (1, 2, 3):
        wl = synth.custom(8, 16, 24, 2, 128, "bf16", top_k=k, top_p=0.0, bg_amp=1.0, seed=5)
        inp_cpu, inp = _inputs(wl, with_dout=True)
        cfg = P.config_for(wl)
        att = run_plan(cfg, inp)
        o, lse = att.forward()
        dq, dk, dv = att.backward(inp["dout"])
        torch.cuda.synchronize()
        views = att.views()
        for h in range(wl.heads):
            q_units, k_units, unsel = _unit_list_lengths(views, h)
            fwd_res |= {u % 4 for u in q_units}
            kv_res |= {u % 3 for u in k_units}
            unselected += unsel
            print(f"k={k} head {h}: query lists {sorted(set(q_units))} units, key lists "
                  f"{sorted(set(k_units))} units, unselected key blocks {unsel}", flush=True)
            op, exact = _check_head(wl, cfg, att, inp_cpu, h, o, lse)
            if not exact.all():
                print(f"k={k} head {h}: a near-threshold block differs; gradients not compared")
                continue
            g = oracle.attn_bwd(op, inp_cpu["q"][:, h], inp_cpu["k"][:, h],
                                inp_cpu["v"][:, h], inp_cpu["dout"][:, h], with_mag=True)
            for name, gpu, ref, mag in (("dq", dq, g[0], g[3]), ("dk", dk, g[1], g[4]),
                                        ("dv", dv, g[2], g[5])):
                err, ratio = check_close(gpu[:, h].float().cpu().numpy(), ref, "bf16",
                                         f"k={k} head {h} {name}", mag)
                print(f"k={k} head {h} {name}: max abs err {err:.3e} (bound use {ratio:.2f})",
                      flush=True)
    # the forward and dQ loops are unrolled by four stages, dK/dV by three
    assert fwd_res == {0, 1, 2, 3}, fwd_res
    assert kv_res == {0, 1, 2}, kv_res
    assert unselected > 0


def test_deterministic_rerun():
    """Two runs of plan, forward and backward give bit-identical results."""
    wl = synth.custom(8, 16, 24, 2, 128, "bf16", seed=9)
    _, inp = _inputs(wl, with_dout=True)
    cfg = P.config_for(wl)
    outs = []
    for _ in range(2):
        att = run_plan(cfg, inp)
        o, lse = att.forward()
        g = att.backward(inp["dout"])
        torch.cuda.synchronize()
        v = att.views()
        lists = []
        for h in range(cfg.num_heads):
            nb = int(v["zone_block"][h, -1])
            c = v["sel_count"][h, :nb]
            lists.append(c.clone())
            lists += [v["csr_col"][h, i, :int(c[i])].clone() for i in range(nb)]
        outs.append([o.clone(), lse.clone(), *[x.clone() for x in g], v["perm"].clone(),
                     *lists])
    assert len(outs[0]) == len(outs[1])
    names = ["o", "lse", "dq", "dk", "dv", "perm"]
    for i, (a, b) in enumerate(zip(*outs)):
        if not torch.equal(a, b):
            bad = (a != b).nonzero()
            d = (a.float() - b.float()).abs().max().item()
            what = names[i] if i < len(names) else f"selection list {i - len(names)}"
            raise AssertionError(f"{what} differs between runs at {bad.shape[0]} places "
                                 f"(first {bad[:4].tolist()}), max difference {d:.3e}")


# The pages' operating point and sparsity policies, the fixed-shape baseline and the mapping
# and density ablation settings: plan, selection and forward against the oracle.
SETTINGS = [
    ("pages", P.POLICIES["pages"]),
    ("topk85", P.POLICIES["topk85"]),
    ("topp0.3", P.POLICIES["topp0.3"]),
    ("fixed-4x8x8", dict(fixed_shape=P.shape_code(4, 8, 8))),
    ("fixed-4x4x4", dict(fixed_shape=P.shape_code(4, 4, 4))),
    ("map-1.0", dict(map_exponent=1.0)),
    ("map-0.3", dict(map_exponent=0.3)),
    ("density-spatial", dict(density_mode=1)),
    ("density-temporal", dict(density_mode=2)),
    ("density-audio", dict(density_mode=3)),
]


@pytest.mark.parametrize("name,over", SETTINGS, ids=[s[0] for s in SETTINGS])
def test_bf16_settings(name, over):
    wl = synth.custom(8, 24, 40, 2, 128, "bf16", seed=11)
    inp_cpu, inp = _inputs(wl)
    cfg = P.config_for(wl, **over)
    att = run_plan(cfg, inp)
    o, lse = att.forward()
    torch.cuda.synchronize()
    oover = dict(over)
    if "map_exponent" in oover:  # the library receives a float32
        oover["map_exponent"] = float(np.float32(oover["map_exponent"]))
    for h in range(wl.heads):
        _check_head(wl, cfg, att, inp_cpu, h, o, lse, **oover)


@pytest.mark.parametrize("shape", [(4, 4, 4), (4, 4, 8), (4, 8, 8)],
                         ids=["64", "128", "256"])
def test_bf16_fixed_shape_backward(shape):
    """Every zone cut into one block shape: 64-token blocks (64-key dK/dV tiles with half the
    wave pairs idle, 64-row forward/dQ tiles), 128-token blocks (one key tile per block),
    256-token blocks (two key tiles per block, placed on one XCD)."""
    wl = synth.custom(8, 16, 24, 2, 128, "bf16", top_k=3, top_p=0.5, seed=5)
    over = dict(fixed_shape=P.shape_code(*shape))
    inp_cpu, inp = _inputs(wl, with_dout=True)
    cfg = P.config_for(wl, **over)
    att = run_plan(cfg, inp)
    o, lse = att.forward()
    dq, dk, dv = att.backward(inp["dout"])
    torch.cuda.synchronize()
    compared = 0
    for h in range(wl.heads):
        op, exact = _check_head(wl, cfg, att, inp_cpu, h, o, lse, **over)
        if not exact.all():
            print(f"head {h}: a near-threshold block differs; gradients not compared")
            continue
        g = oracle.attn_bwd(op, inp_cpu["q"][:, h], inp_cpu["k"][:, h], inp_cpu["v"][:, h],
                            inp_cpu["dout"][:, h], with_mag=True)
        for name, gpu, ref, mag in (("dq", dq, g[0], g[3]), ("dk", dk, g[1], g[4]),
                                    ("dv", dv, g[2], g[5])):
            err, ratio = check_close(gpu[:, h].float().cpu().numpy(), ref, "bf16",
                                     f"{shape} head {h} {name}", mag)
            print(f"{shape} head {h} {name}: max abs err {err:.3e} (bound use {ratio:.2f})",
                  flush=True)
        compared += 1
    assert compared > 0


@pytest.mark.parametrize("layout", ["fused_qkv", "head_major"])
def test_bf16_strided_inputs_match_dense(layout):
    """q, k, v passed as strided views (slices of a fused [N, 3, heads, D] QKV projection, or
    [heads, N, D] tensors seen as [N, heads, D]) give the same plan and bit-identical
    outputs and gradients as the dense tensors."""
    wl = synth.custom(8, 16, 24, 2, 128, "bf16", top_k=4, top_p=0.8, seed=5)
    _, inp = _inputs(wl, with_dout=True)
    cfg = P.config_for(wl)
    dense = P.PrismAttention(cfg)
    dense.plan(inp["q"], inp["k"], inp["v"], inp["a2v"])
    ref = (*dense.forward(), *dense.backward(inp["dout"]))
    if layout == "fused_qkv":
        fused = torch.stack([inp["q"], inp["k"], inp["v"]], dim=1).contiguous()
        q, k, v = fused[:, 0], fused[:, 1], fused[:, 2]
    else:
        q, k, v = (inp[n].transpose(0, 1).contiguous().transpose(0, 1) for n in "qkv")
    assert not q.is_contiguous() and q.stride(2) == 1
    att = P.PrismAttention(cfg)
    att.plan(q, k, v, inp["a2v"])
    got = (*att.forward(), *att.backward(inp["dout"]))
    torch.cuda.synchronize()
    va, vd = att.views(), dense.views()
    for name in ("zone_shape", "zone_block", "perm"):
        assert torch.equal(va[name], vd[name]), name
    for h in range(wl.heads):  # the selection lists (entries past them are not written)
        nb = int(vd["zone_block"][h, -1])
        cnt = vd["sel_count"][h, :nb]
        assert torch.equal(va["sel_count"][h, :nb], cnt)
        keep = torch.arange(nb, device=cnt.device)[None, :] < cnt[:, None]
        assert torch.equal(va["csr_col"][h, :nb, :nb][keep], vd["csr_col"][h, :nb, :nb][keep])
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name
