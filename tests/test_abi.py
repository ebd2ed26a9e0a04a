"""The C ABI of libprism.so: it loads, exports every entry point include/prism.h declares,
and rejects bad configurations with status codes before touching a GPU."""
import ctypes
import os
import re

import pytest

import dynamic_block_sparse_stats_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "prism.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(prism_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(P.LIB_PATH):
        pytest.skip("libprism.so not built")
    return P.lib()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(P.EXPORTS)
    handle = ctypes.CDLL(P.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n


def test_layout_and_workspace(lib):
    cfg = P.make_config(8, 16, 16, 2, 64, "f32", min_edge_log2=0, top_k=4, top_p=0.9)
    L = P.plan_layout(cfg)
    assert L.N == 2048 and L.Z == 4 and L.nb_max == 32
    offs = [getattr(L, f) for f in P._LAYOUT_FIELDS if f != "total"]
    assert all(o % 256 == 0 for o in offs)
    assert len(set(offs)) == len(offs)
    assert P.workspace_bytes(cfg) == L.total >= max(offs)


@pytest.mark.parametrize("over,code", [
    (dict(T=12), -2), (dict(H=0), -1), (dict(head_dim=96), -2), (dict(dtype=7), -2),
    (dict(min_edge_log2=2), -1), (dict(top_k=-1), -1), (dict(top_p=float("nan")), -1),
    (dict(T=4096, H=1024, W=1024), -2),
    (dict(top_k_frac=1.5), -1), (dict(top_k_frac=-0.1), -1), (dict(density_mode=4), -1),
    (dict(map_exponent=float("inf")), -1),
    (dict(fixed_shape=(1 << 4) | (1 << 2) | 1), -1),     # 2x2x2: 8 tokens
    (dict(fixed_shape=(3 << 4) | (3 << 2) | 3), -1),     # 8x8x8: 512 tokens
    (dict(fixed_shape=(0 << 4) | (3 << 2) | 3), -1),     # edge 1 with min_edge_log2 = 1
    (dict(fixed_shape=-1), -1),
    (dict(T=1 << 30, H=1 << 30, W=1 << 30), -2),          # T * H * W beyond 64 bits
    (dict(max_pairs=-1), -1),
])
def test_rejected_configs(lib, over, code):
    base = dict(T=8, H=16, W=16, num_heads=2, head_dim=128, dtype=P.BF16, min_edge_log2=1,
                top_k=8, top_p=0.9, tau128=0.5, tau256=0.25, eps=1e-6, score_scale=0.0,
                softmax_scale=0.0, top_k_frac=0.0, fixed_shape=0, map_exponent=0.0,
                density_mode=0)
    base.update(over)
    cfg = P.PrismConfig(**base)
    assert lib.prism_workspace_bytes(ctypes.byref(cfg)) == 0
    out = P.PrismLayout()
    assert lib.prism_plan_layout(ctypes.byref(cfg), ctypes.byref(out)) == code
    # the same check runs first in every entry point: nothing is launched
    dummy = ctypes.c_void_p(16)
    assert lib.prism_plan(ctypes.byref(cfg), dummy, dummy, dummy, 0, 0, None, dummy, 1 << 40,
                          None) == code
    assert lib.prism_attn_fwd(ctypes.byref(cfg), dummy, 1 << 40, dummy, dummy, None) == code
    assert lib.prism_last_error().decode() != ""


@pytest.mark.parametrize("W,code", [(8 * 8191, 0), (8 * 8192, -2)])
def test_largest_grid(lib, W, code):
    """A head holds at most 65535 64-token units.  With 8x8x8 zones the largest grid has
    8191 zones (65528 units) and is accepted; one zone more is refused before any launch."""
    cfg = P.make_config(8, 8, W, 1, 128, "bf16", top_k=8, top_p=0.9)
    out = P.PrismLayout()
    assert lib.prism_plan_layout(ctypes.byref(cfg), ctypes.byref(out)) == code
    if code == 0:
        assert out.N == 8 * 8 * W and out.Z == 8191 and out.nb_max == 8 * 8191
        assert lib.prism_workspace_bytes(ctypes.byref(cfg)) == out.total > 0
    else:
        assert lib.prism_workspace_bytes(ctypes.byref(cfg)) == 0


def test_null_and_small_workspace(lib):
    cfg = P.make_config(8, 16, 16, 2, 128, "bf16")
    d = ctypes.c_void_p(256)
    assert lib.prism_plan(ctypes.byref(cfg), None, d, d, 0, 0, None, d, 1 << 40, None) == -1
    need = lib.prism_workspace_bytes(ctypes.byref(cfg))
    assert lib.prism_plan(ctypes.byref(cfg), d, d, d, 0, 0, None, d, need - 1, None) == -3
    assert lib.prism_attn_fwd(ctypes.byref(cfg), d, need - 1, d, d, None) == -3
    assert lib.prism_attn_bwd(ctypes.byref(cfg), d, need, d, d, None, d, None) == -1
    assert lib.prism_attn_bwd(ctypes.byref(cfg), d, need - 1, d, d, d, d, None) == -3
    assert lib.prism_status_string(-3) == b"workspace too small"


def test_plan_rejects_bad_strides(lib):
    cfg = P.make_config(8, 16, 16, 2, 128, "bf16")
    d = ctypes.c_void_p(256)
    need = lib.prism_workspace_bytes(ctypes.byref(cfg))
    for tok, head in ((-256, 0), (0, -1), (2 * 128 + 4, 128), (3 * 2 * 128, 132)):
        # negative, or a row not starting on a 16-byte boundary (bf16: 8 elements)
        assert lib.prism_plan(ctypes.byref(cfg), d, d, d, tok, head, None, d, need,
                              None) == -1, (tok, head)
    assert lib.prism_plan(ctypes.byref(cfg), ctypes.c_void_p(264), d, d, 0, 0, None, d, need,
                          None) == -1  # q not 16-byte aligned


def test_entry_points_reject_misaligned_buffers(lib):
    cfg = P.make_config(8, 16, 16, 2, 128, "bf16")
    need = lib.prism_workspace_bytes(ctypes.byref(cfg))
    d, ws, bad_ws = ctypes.c_void_p(4096), ctypes.c_void_p(8192), ctypes.c_void_p(8192 + 16)
    assert lib.prism_plan(ctypes.byref(cfg), d, d, d, 0, 0, None, bad_ws, need, None) == -1
    assert lib.prism_attn_fwd(ctypes.byref(cfg), bad_ws, need, d, d, None) == -1
    assert lib.prism_attn_fwd(ctypes.byref(cfg), ws, need, ctypes.c_void_p(4104), d,
                              None) == -1                                  # o
    assert lib.prism_attn_fwd(ctypes.byref(cfg), ws, need, d, ctypes.c_void_p(4098),
                              None) == -1                                  # lse
    assert lib.prism_attn_bwd(ctypes.byref(cfg), bad_ws, need, d, d, d, d, None) == -1
    for i in range(4):
        args = [d] * 4
        args[i] = ctypes.c_void_p(4104)
        assert lib.prism_attn_bwd(ctypes.byref(cfg), ws, need, *args, None) == -1, i


def test_plan_view_matches_layout(lib):
    cfg = P.make_config(8, 16, 16, 2, 128, "bf16")
    a, b = P.PrismLayout(), P.PrismLayout()
    assert lib.prism_plan_layout(ctypes.byref(cfg), ctypes.byref(a)) == 0
    assert lib.prism_plan_view(ctypes.byref(cfg), ctypes.c_void_p(256), ctypes.byref(b)) == 0
    assert bytes(a) == bytes(b)
    assert lib.prism_plan_view(ctypes.byref(cfg), None, ctypes.byref(b)) == -1


def test_accepted_ablation_configs(lib):
    for over in (dict(top_k_frac=0.05, top_p=0.2), dict(fixed_shape=P.shape_code(4, 8, 8)),
                 dict(fixed_shape=P.shape_code(4, 4, 4)), dict(map_exponent=1.0),
                 dict(density_mode=3)):
        cfg = P.make_config(8, 16, 16, 2, 128, "bf16", **over)
        assert lib.prism_workspace_bytes(ctypes.byref(cfg)) > 0, over


def test_a2v_norm_rejects_bad_arguments(lib):
    d = ctypes.c_void_p(256)
    assert lib.prism_a2v_norm(None, 10, 8, 8, P.BF16, d, None) == -1
    assert lib.prism_a2v_norm(d, 0, 8, 8, P.BF16, d, None) == -1
    assert lib.prism_a2v_norm(d, 10, 8, 4, P.BF16, d, None) == -1      # ld < channels
    assert lib.prism_a2v_norm(d, 10, 8, 12, P.BF16, d, None) == -1     # rows not 16-B aligned
    assert lib.prism_a2v_norm(ctypes.c_void_p(8), 10, 8, 8, P.BF16, d, None) == -1
    assert lib.prism_a2v_norm(d, 10, 8, 8, 5, d, None) == -2


def test_forward_and_backward_refused_without_plan(lib):
    """A workspace that no prism_plan has written: the forward and the backward are refused
    with PRISM_ERR_STATE before any launch (nothing here touches a GPU)."""
    cfg = P.make_config(8, 16, 16, 2, 128, "bf16")
    need = lib.prism_workspace_bytes(ctypes.byref(cfg))
    d, ws = ctypes.c_void_p(4096), ctypes.c_void_p(1 << 20)
    assert lib.prism_attn_fwd(ctypes.byref(cfg), ws, need, d, d, None) == -5
    assert b"no prism_plan" in lib.prism_last_error()
    assert lib.prism_attn_bwd(ctypes.byref(cfg), ws, need, d, d, d, d, None) == -5
    assert lib.prism_status_string(-5) == b"call out of order for this workspace"


def test_pair_capacity_sizes_the_lists(lib):
    """max_pairs bounds the selection lists of each head (CSR, CSC and the query tiles'
    union lists): the 2K grid with 24 heads needs half the workspace at the named
    workloads' capacity that it needs at the worst case."""
    full = P.make_config(64, 104, 128, 24, 128, "bf16", top_k=8, top_p=0.95)
    capped = P.make_config(64, 104, 128, 24, 128, "bf16", top_k=8, top_p=0.95,
                           max_pairs=P.default_max_pairs(64 * 104 * 128))
    a, b = P.plan_layout(full), P.plan_layout(capped)
    assert a.pair_cap == a.nb_max ** 2 and b.pair_cap == (851968 // 128) ** 2
    list_bytes = lambda L: 3 * 24 * L.pair_cap * 4
    assert a.total - b.total == list_bytes(a) - list_bytes(b)
    assert a.total > 80e9 and b.total < 0.55 * a.total
    big = P.make_config(8, 16, 16, 2, 128, "bf16", max_pairs=10 ** 12)   # clamped to Nb_max^2
    assert P.plan_layout(big).pair_cap == 32 ** 2


def test_bf16_head_dim_64_accepted(lib):
    cfg = P.make_config(8, 16, 16, 2, 64, "bf16")
    L = P.plan_layout(cfg)
    assert L.total > 0 and P.workspace_bytes(cfg) == L.total


def test_check_flags_rejects_bad_arguments(lib):
    cfg = P.make_config(8, 16, 16, 2, 128, "bf16")
    assert lib.prism_check_flags(ctypes.byref(cfg), None, None, None) == -1
    bad = P.make_config(12, 16, 16, 2, 128, "bf16")
    assert lib.prism_check_flags(ctypes.byref(bad), ctypes.c_void_p(256), None, None) == -2


def test_static_forward_refuses_what_exceeds_its_scratch(lib):
    """prism_forward_static checks the workspace its configuration needs against its static
    scratch before touching the GPU: the 720p workload (24 heads) is refused."""
    cfg = P.make_config(24, 48, 80, 24, 128, "bf16", top_k=8, top_p=0.9)
    assert lib.prism_workspace_bytes(ctypes.byref(cfg)) > 128 << 20
    d = ctypes.c_void_p(4096)
    assert lib.prism_forward_static(ctypes.byref(cfg), d, d, d, 0, 0, None, d, d, None) == -3
    assert b"static scratch" in lib.prism_last_error()
    assert lib.prism_forward_static(ctypes.byref(cfg), None, d, d, 0, 0, None, d, d,
                                    None) == -1
