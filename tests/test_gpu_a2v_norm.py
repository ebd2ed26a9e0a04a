"""The A2V norm producer (prism_a2v_norm) against the oracle's float64 row norms, on the same
stored values, at small ragged sizes and at the 2K size of a 24 x 128 hidden width (sampled
rows).  Bar: |got - ref| <= 1e-6 |ref|: the kernel sums in float64 and rounds the root to
float32 once (half an ulp, 6e-8 relative), so 1e-6 leaves room only for summation order."""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_stats_amd as P
from dynamic_block_sparse_stats_amd import synth
import oracle

pytestmark = pytest.mark.gpu
REL = 1e-6


def _check(got, ref, what):
    err = np.abs(got - ref)
    bound = REL * np.abs(ref) + 1e-44   # float32 keeps norms down to its subnormal range
    worst = int(np.argmax(err / bound))
    assert np.all(err <= bound), f"{what}: row {worst} got {got[worst]!r} ref {ref[worst]!r}"
    return float((err / np.maximum(np.abs(ref), 1e-30)).max())


@pytest.mark.parametrize("dtype,N,C,ld", [
    ("f32", 1001, 3072, 3072), ("bf16", 1001, 3072, 3072), ("bf16", 517, 20, 24),
    ("f32", 263, 5, 8), ("bf16", 64, 128, 256), ("f32", 3, 1, 4),
])
def test_row_norms_small(dtype, N, C, ld):
    g = torch.Generator().manual_seed(N + C)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    full = (torch.randn(N, ld, generator=g) * 3.0).to(tdt)
    x = full.cuda()[:, :C]
    got = P.a2v_norm(x).cpu().numpy()
    ref = oracle.row_norms(full[:, :C].double().numpy())
    r = _check(got, ref, f"{dtype} {N}x{C} ld {ld}")
    print(f"{dtype} N {N} C {C} ld {ld}: max relative error {r:.2e}", flush=True)


def test_row_norms_zero_rows():
    x = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    assert torch.equal(P.a2v_norm(x), torch.zeros(8, device="cuda"))


@pytest.mark.timeout(600)
def test_row_norms_2k_and_field_roundtrip():
    """The 2K grid (851,968 tokens) with a hidden width of 24 heads x 128: a synthetic
    cross-attention output whose rows are directions scaled by the workload's A2V field;
    sampled rows against the oracle, and the produced field against the field itself."""
    wl = synth.workload(4)
    inp = synth.make_inputs(wl, device="cuda", with_dout=False)
    a = inp["a2v"]
    del inp
    x = synth.a2v_output(a, 3072, "bf16", seed=4)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = P.a2v_norm(x)
    s.record()
    P.a2v_norm(x, out=out)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    rows = np.sort(np.random.default_rng(4).choice(wl.N, size=4096, replace=False))
    idx = torch.from_numpy(rows).cuda()
    ref = oracle.row_norms(x[idx].double().cpu().numpy())
    r = _check(out[idx].cpu().numpy(), ref, "2K rows")
    # the stored rows are bf16 roundings of a[n] u_n: their length is a[n] to ~2^-9
    da = (out - a).abs().max().item()
    assert da <= 4e-3 * a.max().item()
    gbs = x.numel() * 2 / (ms * 1e-3) / 1e9
    print(f"2K: {ms:.3f} ms for {x.numel() * 2 / 1e9:.2f} GB ({gbs:.0f} GB/s); max relative "
          f"error {r:.2e}; max |norm - a2v| {da:.2e}", flush=True)
