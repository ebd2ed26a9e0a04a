"""HIP path vs CPU oracle on small grids that span several tiles and ragged tails
(called through the C ABI; the oracle never sees anything the GPU produced)."""
import ctypes
import math

import numpy as np
import pytest
import torch

import dynamic_block_sparse_stats_amd as P
from dynamic_block_sparse_stats_amd import synth
import oracle
from parity import (TOL, check_close, check_grads, compare_plan, compare_selection, describe,
                    oracle_plan, rows_of_exact_blocks, run_plan, to_np)

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
    oo, ol = oracle.attn_fwd(op, inp_cpu["q"][:, h], inp_cpu["k"][:, h], inp_cpu["v"][:, h])
    rows = rows_of_exact_blocks(op, exact)
    go = o[:, h].float().cpu().numpy()
    gl = lse[h].cpu().numpy()
    err_o, r_o, _ = check_close(go[rows], oo[rows], wl.dtype, f"head {h} O")
    err_l, r_l, _ = check_close(gl[rows], ol[rows], "f32" if wl.dtype == "f32" else "bf16",
                                f"head {h} lse")
    print(f"head {h}: nb {op.nb} nnz {nnz} excluded {excl} near-tie zones "
          f"{rep['near_tie_zones']} max|O| {np.abs(oo).max():.2f} max|dO| {err_o:.2e} "
          f"(bound use {r_o:.2f}) max|dlse| {err_l:.2e}", flush=True)
    return op, exact


def _grads_vs_oracle(op, inp_cpu, h, dq, dk, dv, what):
    """Head h's dQ, dK, dV against the oracle's backward (bfloat16 bounds of check_grads)."""
    g = oracle.attn_bwd(op, inp_cpu["q"][:, h], inp_cpu["k"][:, h], inp_cpu["v"][:, h],
                        inp_cpu["dout"][:, h], with_mag=True)
    refs = dict(dq=g[0], dk=g[1], dv=g[2])
    res = check_grads({n: t[:, h].float().cpu().numpy() for n, t in
                       (("dq", dq), ("dk", dk), ("dv", dv))},
                      refs, dict(dq=g[3], dk=g[4], dv=g[5]), "bf16", what)
    for name, c in res.items():
        print(f"{what} max|{name}| {np.abs(refs[name]).max():.2f} " + describe(name, c),
              flush=True)
    return res


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
            err = check_close(gpu[:, h].cpu().numpy(), ref, "f32", f"head {h} {name}").err
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
        _grads_vs_oracle(op, inp_cpu, h, dq, dk, dv, f"head {h}")


def _unit_list_lengths(views, h):
    """The unit counts the attention kernels walk: per query tile (256 rows: one block of
    256, two of 128 or four of 64 tokens; the forward and dQ walk the union of the tile's
    blocks' selections), the units of the union; per key block selected by at least one
    query block, the units of those query blocks (dK/dV); and the key blocks nobody
    selected."""
    nb = int(views["zone_block"][h, -1])  # the head's block count
    bsz = views["block_size"][h, :nb].cpu().numpy() // 64
    zb = views["zone_block"][h].cpu().numpy()
    col = P.csr_rows(views, h, "csr")
    crow = P.csr_rows(views, h, "csc")
    q_units = []
    for m in range(len(zb) - 1):
        g = 4 // int(bsz[zb[m]])     # blocks per query tile
        for i in range(2):
            first = zb[m] + i * g
            union = set().union(*(col[first + b].tolist() for b in range(g)))
            q_units.append(int(bsz[sorted(union)].sum()))
    k_units = [int(bsz[r].sum()) for r in crow if len(r) > 0]
    return q_units, k_units, sum(len(r) == 0 for r in crow)


def test_bf16_short_lists():
    """Pure Top-k with k = 1, 2, 3 (Top-p off): selection lists of a few units, so the
    unrolled unit loops of the three attention kernels end at every stage position (the
    forward and dQ walk the query tiles' union lists), and key blocks that no query block
    selected get zero dK and dV."""
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
            print(f"k={k} head {h}: query tile lists {sorted(set(q_units))} units, key lists "
                  f"{sorted(set(k_units))} units, unselected key blocks {unsel}", flush=True)
            op, exact = _check_head(wl, cfg, att, inp_cpu, h, o, lse)
            if not exact.all():
                print(f"k={k} head {h}: a near-threshold block differs; gradients not compared")
                continue
            _grads_vs_oracle(op, inp_cpu, h, dq, dk, dv, f"k={k} head {h}")
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
            lists += [torch.from_numpy(x) for x in P.csr_rows(v, h, "csr")]
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
    """Every zone cut into one block shape: 64-token blocks (the 64-key dK/dV launch, where
    the wave pairs split keys and query halves: 96 tiles, one full group of 64 placed by zone
    on the XCDs and a tail of 32; forward/dQ query tiles of four blocks), 128-token blocks
    (one key tile per block), 256-token blocks (two key tiles per block, placed on one XCD)."""
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
        _grads_vs_oracle(op, inp_cpu, h, dq, dk, dv, f"{shape} head {h}")
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
        for a, b in zip(P.csr_rows(va, h, "csr"), P.csr_rows(vd, h, "csr")):
            assert np.array_equal(a, b)
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name


def test_call_order_is_enforced():
    """A re-plan invalidates the forward state: a backward after it, with no forward, is
    refused (by the binding and by the C ABI itself), as is a forward whose configuration
    differs from the plan's (the padding bytes of the struct do not count); after a forward
    the backward runs again and gives the same gradients."""
    wl = synth.custom(8, 16, 24, 2, 128, "bf16", top_k=4, top_p=0.8, seed=5)
    _, inp = _inputs(wl, with_dout=True)
    cfg = P.config_for(wl)
    att = run_plan(cfg, inp)
    o, lse = att.forward()
    ref = att.backward(inp["dout"])
    att.plan(inp["q"], inp["k"], inp["v"], inp["a2v"])
    with pytest.raises(P.PrismError, match="forward"):
        att.backward(inp["dout"])
    dq, dk, dv = (torch.empty_like(inp["q"]) for _ in range(3))
    with pytest.raises(P.PrismError, match="out of order"):
        P.attn_bwd(cfg, att.ws, inp["dout"], dq, dk, dv)
    other = P.config_for(wl, top_k=2)
    with pytest.raises(P.PrismError, match="out of order"):
        P.attn_fwd(other, att.ws, o, lse)
    # the same configuration with other bytes in the struct's padding (before eps) is the
    # same configuration
    pad0 = P.PrismConfig.tau256.offset + 4
    assert P.PrismConfig.eps.offset - pad0 == 4
    raw = bytearray(ctypes.string_at(ctypes.addressof(att.cfg), ctypes.sizeof(att.cfg)))
    raw[pad0:pad0 + 4] = b"\xab\xcd\xef\x01"
    padded = P.PrismConfig.from_buffer_copy(bytes(raw))
    P.attn_fwd(padded, att.ws, o, lse)
    P.attn_bwd(att.cfg, att.ws, inp["dout"], dq, dk, dv)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv), ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("T,H,W,bg", [(8, 16, 24, 1.0), (16, 32, 32, 0.15)],
                         ids=["mixed-blocks", "near-uniform"])
def test_bf16_head_dim_64(T, H, W, bg):
    """bfloat16 with head_dim 64: the permuted float16 operands are zero-padded to 128
    channels; plan, forward and backward against the oracle (small blocks of a varied
    field, and the 256-token blocks of a near-uniform one)."""
    wl = synth.custom(T, H, W, 2, 64, "bf16", top_k=4, top_p=0.8, bg_amp=bg, seed=5)
    inp_cpu, inp = _inputs(wl, with_dout=True)
    cfg = P.config_for(wl)
    att = run_plan(cfg, inp)
    o, lse = att.forward()
    dq, dk, dv = att.backward(inp["dout"])
    torch.cuda.synchronize()
    assert att.check() == [0] * wl.heads
    for h in range(wl.heads):
        op, exact = _check_head(wl, cfg, att, inp_cpu, h, o, lse)
        if not exact.all():
            print(f"head {h}: a near-threshold block differs; gradients not compared")
            continue
        _grads_vs_oracle(op, inp_cpu, h, dq, dk, dv, f"D=64 head {h}")


def _all_nan(t):
    return bool(torch.isnan(t.float()).all())


def _all_finite(t):
    return bool(torch.isfinite(t.float()).all())


def test_out_of_range_inputs_are_flagged():
    """bfloat16 q/k/v values beyond the float16 range of the attention operands: the head
    gets PRISM_FLAG_QKV_RANGE, its outputs are NaN, and prism_check_flags reports it; the
    other head is unaffected and still matches the oracle."""
    wl = synth.custom(8, 16, 24, 2, 128, "bf16", top_k=4, top_p=0.8, seed=5)
    inp_cpu, inp = _inputs(wl, with_dout=True)
    for name, big in (("q", 7.0e4), ("k", -1.0e5), ("v", 3.0e38)):
        bad = {n: t.clone() for n, t in inp.items()}
        bad[name][100, 1, 5] = big          # head 1 only
        cfg = P.config_for(wl)
        att = run_plan(cfg, bad)
        o, lse = att.forward()
        dq, dk, dv = att.backward(bad["dout"])
        torch.cuda.synchronize()
        flags = att.check()
        assert flags[0] == 0 and flags[1] & P.FLAG_QKV_RANGE, (name, flags)
        with pytest.raises(P.PrismError, match="float16 range"):
            P._check(P.lib().prism_check_flags(ctypes.byref(cfg), P._ws(att.ws)[0], None,
                                               P._stream(None)), "check")
        for t in (o[:, 1], lse[1], dq[:, 1], dk[:, 1], dv[:, 1]):
            assert _all_nan(t), name
        for t in (o[:, 0], lse[0], dq[:, 0], dk[:, 0], dv[:, 0]):
            assert _all_finite(t), name
    # head 0 of the last run still matches the oracle
    _check_head(wl, cfg, att, inp_cpu, 0, o, lse)


def test_out_of_range_gradients_are_flagged():
    """An upstream gradient beyond the float16 range, or one large enough that the bound on
    the float16 dS reaches it: the backward flags the head and its gradients are NaN; a
    later backward with a normal gradient clears the flags."""
    wl = synth.custom(8, 16, 24, 2, 128, "bf16", top_k=4, top_p=0.8, seed=5)
    _, inp = _inputs(wl, with_dout=True)
    cfg = P.config_for(wl)
    att = run_plan(cfg, inp)
    att.forward()
    for scale, flag in ((1e5, P.FLAG_DOUT_RANGE), (3e3, P.FLAG_DS_RANGE)):
        dout = inp["dout"].clone()
        dout[:, 0] = (dout[:, 0].float() * scale).bfloat16()
        dq, dk, dv = att.backward(dout)
        flags = att.check()
        assert flags[0] & flag and flags[1] == 0, (scale, flags)
        for t in (dq[:, 0], dk[:, 0], dv[:, 0]):
            assert _all_nan(t), scale
        for t in (dq[:, 1], dk[:, 1], dv[:, 1]):
            assert _all_finite(t), scale
    dq, dk, dv = att.backward(inp["dout"])
    assert att.check() == [0, 0]
    assert _all_finite(dq) and _all_finite(dk) and _all_finite(dv)


def test_selection_overflow_is_flagged():
    """A selection-list capacity (max_pairs) below what the plan selects: the lists stay
    inside the capacity, the heads are flagged and their outputs are NaN; with room for
    every pair the same plan is unflagged and its lists are the full ones."""
    wl = synth.custom(8, 16, 24, 2, 128, "bf16", top_k=4, top_p=0.8, seed=5)
    _, inp = _inputs(wl, with_dout=True)
    full = run_plan(P.config_for(wl), inp)
    full.forward()
    assert full.check() == [0, 0]
    nnz = [int(full.views()["csr_ptr"][h, int(full.views()["zone_block"][h, -1])])
           for h in range(wl.heads)]
    cap = min(nnz) - 1
    small = P.config_for(wl, max_pairs=cap)
    att = run_plan(small, inp)
    o, lse = att.forward()
    dq, dk, dv = att.backward(inp["dout"])
    flags = att.check()
    assert all(f & P.FLAG_SELECTION_OVERFLOW for f in flags), flags
    v = att.views()
    for h in range(wl.heads):
        nb = int(v["zone_block"][h, -1])
        assert int(v["csr_ptr"][h, nb]) <= cap and int(v["csc_ptr"][h, nb]) <= cap
        assert int(v["sel_count"][h, :nb].sum()) <= cap
    for t in (o, lse, dq, dk, dv):
        assert _all_nan(t)
    exact = P.config_for(wl, max_pairs=max(nnz))
    ok = run_plan(exact, inp)
    ok.forward()
    assert ok.check() == [0, 0]
    for h in range(wl.heads):
        for a, b in zip(P.csr_rows(ok.views(), h), P.csr_rows(full.views(), h)):
            assert np.array_equal(a, b)
