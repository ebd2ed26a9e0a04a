"""Prism dynamic block-sparse video self-attention on AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libprism.so`` (the C ABI in ``include/prism.h``): it checks
tensor shapes and dtypes and passes device pointers and the current HIP stream; every step
of the method runs in the library's HIP kernels.  PyTorch only provides device memory and
streams.  There is no fallback: if the library is missing or was built for another target,
calls raise.

Entry points (same names as the C ABI):
  workspace_bytes(cfg), plan_layout(cfg), plan_view(cfg, ws), plan(cfg, q, k, v, a2v, ws),
  attn_fwd(cfg, ws, o, lse), attn_bwd(cfg, ws, dout, dq, dk, dv), a2v_norm(x)
and ``PrismAttention``, which owns a workspace and chains them.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libprism.so")

F32, BF16 = 0, 1
_DTYPES = {F32: torch.float32, BF16: torch.bfloat16}


class PrismConfig(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int), ("H", ctypes.c_int), ("W", ctypes.c_int),
                ("num_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
                ("dtype", ctypes.c_int), ("min_edge_log2", ctypes.c_int),
                ("top_k", ctypes.c_int), ("top_p", ctypes.c_float),
                ("tau128", ctypes.c_float), ("tau256", ctypes.c_float),
                ("eps", ctypes.c_double), ("score_scale", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("top_k_frac", ctypes.c_float),
                ("fixed_shape", ctypes.c_int), ("map_exponent", ctypes.c_float),
                ("density_mode", ctypes.c_int), ("max_pairs", ctypes.c_longlong)]

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def torch_dtype(self):
        return _DTYPES[self.dtype]


_LAYOUT_FIELDS = ["zone_stats", "audio_stats", "zone_diag", "zone_shape", "zone_block",
                  "block_start", "block_size", "unit_block", "perm", "inv_perm", "qbar",
                  "kbar", "sel_count", "csr_ptr", "csr_col", "csc_count", "csc_ptr", "csc_row",
                  "scores", "flags", "total"]


class PrismLayout(ctypes.Structure):
    _fields_ = [(f, ctypes.c_size_t) for f in _LAYOUT_FIELDS] + [
        ("N", ctypes.c_int), ("Z", ctypes.c_int), ("nb_max", ctypes.c_int),
        ("pair_cap", ctypes.c_longlong)]


# status flags of a head (include/prism.h, PRISM_FLAG_*)
FLAG_QKV_RANGE, FLAG_SELECTION_OVERFLOW, FLAG_DOUT_RANGE, FLAG_DS_RANGE = 1, 2, 4, 8


class PrismError(RuntimeError):
    pass


_lib = None
EXPORTS = ["prism_workspace_bytes", "prism_plan_layout", "prism_plan_view", "prism_plan",
           "prism_attn_fwd", "prism_attn_bwd", "prism_a2v_norm", "prism_check_flags",
           "prism_forward_static",
           "prism_status_string", "prism_last_error", "prism_trace_enable", "prism_trace_read",
           "prism_stage_name"]
STAGES = ["audio_stats", "zone_stats", "quantize", "gather", "tiles", "scores", "select",
          "attn_fwd", "bwd_prep", "bwd_dkdv", "bwd_dq"]


def lib():
    """The loaded libprism.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise PrismError(f"{LIB_PATH} is missing: build it with "
                             "`python -m dynamic_block_sparse_stats_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, cfgp = ctypes.c_void_p, ctypes.POINTER(PrismConfig)
        L.prism_workspace_bytes.argtypes = [cfgp]
        L.prism_workspace_bytes.restype = ctypes.c_size_t
        L.prism_plan_layout.argtypes = [cfgp, ctypes.POINTER(PrismLayout)]
        L.prism_plan_layout.restype = ctypes.c_int
        L.prism_plan_view.argtypes = [cfgp, vp, ctypes.POINTER(PrismLayout)]
        L.prism_plan_view.restype = ctypes.c_int
        L.prism_plan.argtypes = [cfgp, vp, vp, vp, ctypes.c_int64, ctypes.c_int64, vp, vp,
                                 ctypes.c_size_t, vp]
        L.prism_plan.restype = ctypes.c_int
        L.prism_attn_fwd.argtypes = [cfgp, vp, ctypes.c_size_t, vp, vp, vp]
        L.prism_attn_fwd.restype = ctypes.c_int
        L.prism_attn_bwd.argtypes = [cfgp, vp, ctypes.c_size_t, vp, vp, vp, vp, vp]
        L.prism_attn_bwd.restype = ctypes.c_int
        L.prism_a2v_norm.argtypes = [vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                     ctypes.c_int, vp, vp]
        L.prism_a2v_norm.restype = ctypes.c_int
        L.prism_forward_static.argtypes = [cfgp, vp, vp, vp, ctypes.c_int64, ctypes.c_int64,
                                           vp, vp, vp, vp]
        L.prism_forward_static.restype = ctypes.c_int
        L.prism_check_flags.argtypes = [cfgp, vp, vp, vp]
        L.prism_check_flags.restype = ctypes.c_int
        L.prism_status_string.argtypes = [ctypes.c_int]
        L.prism_status_string.restype = ctypes.c_char_p
        L.prism_last_error.argtypes = []
        L.prism_last_error.restype = ctypes.c_char_p
        L.prism_trace_enable.argtypes = [ctypes.c_int]
        L.prism_trace_enable.restype = ctypes.c_int
        L.prism_trace_read.argtypes = [vp, vp]
        L.prism_trace_read.restype = ctypes.c_int
        L.prism_stage_name.argtypes = [ctypes.c_int]
        L.prism_stage_name.restype = ctypes.c_char_p
        _lib = L
    return _lib


def make_config(T, H, W, num_heads, head_dim, dtype="bf16", min_edge_log2=1, top_k=8,
                top_p=0.9, tau128=0.5, tau256=0.25, eps=1e-6, score_scale=0.0,
                softmax_scale=0.0, top_k_frac=0.0, fixed_shape=0, map_exponent=0.0,
                density_mode=0, max_pairs=0) -> PrismConfig:
    dt = {"f32": F32, "bf16": BF16, F32: F32, BF16: BF16, torch.float32: F32,
          torch.bfloat16: BF16}[dtype]
    return PrismConfig(T, H, W, num_heads, head_dim, dt, min_edge_log2, int(top_k),
                       float(top_p), float(tau128), float(tau256), float(eps),
                       float(score_scale), float(softmax_scale), float(top_k_frac),
                       int(fixed_shape), float(map_exponent), int(density_mode),
                       int(max_pairs))


def shape_code(bT: int, bH: int, bW: int) -> int:
    """The packed shape code (log2 edges, lT*16 + lH*4 + lW) of a block of bT x bH x bW."""
    lg = [int(x).bit_length() - 1 for x in (bT, bH, bW)]
    if any(1 << l != x for l, x in zip(lg, (bT, bH, bW))):
        raise ValueError("block edges must be powers of two")
    return lg[0] * 16 + lg[1] * 4 + lg[2]


# Selection policies of the pages' sparsity ablation (digest, ablation table of per-query
# sparsity strategies): Top-k as a sparsity (k = ceil((1 - s) * Nb)), Top-p thresholds,
# and their union; "pages" is the default configuration (95% + 0.2).
POLICIES = {
    "pages": dict(top_k=0, top_k_frac=0.05, top_p=0.2),
    "topk75": dict(top_k=0, top_k_frac=0.25, top_p=0.0),
    "topk85": dict(top_k=0, top_k_frac=0.15, top_p=0.0),
    "topk95": dict(top_k=0, top_k_frac=0.05, top_p=0.0),
    "topp0.1": dict(top_k=0, top_k_frac=0.0, top_p=0.1),
    "topp0.2": dict(top_k=0, top_k_frac=0.0, top_p=0.2),
    "topp0.3": dict(top_k=0, top_k_frac=0.0, top_p=0.3),
    "topk95+p0.1": dict(top_k=0, top_k_frac=0.05, top_p=0.1),
    "topk95+p0.3": dict(top_k=0, top_k_frac=0.05, top_p=0.3),
}


def default_max_pairs(n_tokens: int) -> int:
    """Selection-list capacity per head for the named workload grids: (N/128)^2 block
    pairs, i.e. every pair of a head whose blocks average 128 tokens or more, or a
    selection density up to 1/4 of the finest (all-64) partition."""
    return (n_tokens // 128) ** 2


def config_for(wl, **over) -> PrismConfig:
    """Configuration of a synth.Workload.  The named 720p-2K workloads bound their
    selection lists at default_max_pairs(N); other grids keep the worst case."""
    kw = dict(dtype=wl.dtype, min_edge_log2=wl.min_edge_log2, top_k=wl.top_k,
              top_p=wl.top_p, max_pairs=default_max_pairs(wl.N) if wl.cid in (1, 2, 3, 4)
              else 0)
    kw.update(over)
    return make_config(wl.T, wl.H, wl.W, wl.heads, wl.head_dim, **kw)


def _check(st: int, what: str):
    if st != 0:
        L = lib()
        raise PrismError(f"{what}: {L.prism_status_string(st).decode()} "
                         f"({L.prism_last_error().decode()})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _tok(cfg, t, name, dtype=None, strided=False):
    dtype = dtype or cfg.torch_dtype
    shape = (cfg.N, cfg.num_heads, cfg.head_dim)
    layout_ok = t.stride(2) == 1 and min(t.stride()) >= 0 if strided else t.is_contiguous()
    if t.dtype != dtype or tuple(t.shape) != shape or not layout_ok or not t.is_cuda:
        what = "unit channel stride" if strided else "contiguous"
        raise ValueError(f"{name}: expected {what} {dtype} {shape} on the GPU, got "
                         f"{t.dtype} {tuple(t.shape)} strides {t.stride()} on {t.device}")


def _ws(ws):
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace: expected a contiguous GPU tensor")
    return _ptr(ws), ws.numel() * ws.element_size()


def workspace_bytes(cfg: PrismConfig) -> int:
    n = lib().prism_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise PrismError("configuration rejected: " + lib().prism_last_error().decode())
    return n


def plan_layout(cfg: PrismConfig) -> PrismLayout:
    out = PrismLayout()
    _check(lib().prism_plan_layout(ctypes.byref(cfg), ctypes.byref(out)), "prism_plan_layout")
    return out


def plan(cfg, q, k, v, a2v, ws, stream=None):
    """q, k, v: [N, heads, D] GPU tensors, dense or strided views with unit channel stride
    and the same strides (e.g. slices of a fused [N, 3, heads, D] QKV projection)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _tok(cfg, t, name, strided=True)
    if not (q.stride() == k.stride() == v.stride()):
        raise ValueError("q, k, v must share their strides")
    if a2v is not None and (a2v.dtype != torch.float32 or a2v.numel() != cfg.N
                            or not a2v.is_contiguous() or not a2v.is_cuda):
        raise ValueError("a2v: expected a contiguous float32 [N] GPU tensor")
    _check(lib().prism_plan(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), q.stride(0),
                            q.stride(1), _ptr(a2v), *_ws(ws), _stream(stream)), "prism_plan")


def attn_fwd(cfg, ws, o, lse, stream=None):
    _tok(cfg, o, "o")
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (cfg.num_heads, cfg.N)
            or not lse.is_contiguous() or not lse.is_cuda):
        raise ValueError("lse: expected a contiguous float32 [heads, N] GPU tensor")
    _check(lib().prism_attn_fwd(ctypes.byref(cfg), *_ws(ws), _ptr(o), _ptr(lse),
                                _stream(stream)), "prism_attn_fwd")


def attn_bwd(cfg, ws, dout, dq, dk, dv, stream=None):
    """Needs prism_attn_fwd to have run on ws since the last plan (it keeps O and lse)."""
    for name, t in (("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _tok(cfg, t, name)
    _check(lib().prism_attn_bwd(ctypes.byref(cfg), *_ws(ws), _ptr(dout), _ptr(dq), _ptr(dk),
                                _ptr(dv), _stream(stream)), "prism_attn_bwd")


def a2v_norm(x, out=None, stream=None):
    """The A2V norm field of an audio-to-video cross-attention output x [N, C] (float32 or
    bfloat16, rows 16-byte aligned): out[n] = ||x[n, :]||_2 as float32 [N]."""
    if x.dim() != 2 or x.dtype not in (torch.float32, torch.bfloat16) or not x.is_cuda:
        raise ValueError("x: expected a CUDA float32 or bfloat16 [N, C] tensor")
    if x.stride(1) != 1:
        raise ValueError("x: rows must be contiguous")
    n = x.shape[0]
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=x.device)
    if (out.shape != (n,) or out.dtype != torch.float32 or not out.is_contiguous()
            or not out.is_cuda):
        raise ValueError("out: expected a contiguous float32 [N] GPU tensor")
    dt = BF16 if x.dtype == torch.bfloat16 else F32
    _check(lib().prism_a2v_norm(_ptr(x), n, x.shape[1], x.stride(0), dt, _ptr(out),
                                _stream(stream)), "prism_a2v_norm")
    return out


def forward_static(cfg, q, k, v, a2v, o, lse, stream=None):
    """prism_forward_static: plan and forward with the library's static scratch as the
    workspace (no device allocation; small configurations only)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _tok(cfg, t, name, strided=True)
    if not (q.stride() == k.stride() == v.stride()):
        raise ValueError("q, k, v must share their strides")
    _tok(cfg, o, "o")
    if (lse.dtype != torch.float32 or tuple(lse.shape) != (cfg.num_heads, cfg.N)
            or not lse.is_contiguous() or not lse.is_cuda):
        raise ValueError("lse: expected a contiguous float32 [heads, N] GPU tensor")
    _check(lib().prism_forward_static(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v),
                                      q.stride(0), q.stride(1), _ptr(a2v), _ptr(o), _ptr(lse),
                                      _stream(stream)), "prism_forward_static")


def check_flags(cfg, ws, stream=None):
    """Waits for the stream, then returns the per-head status flags (a list of ints; see
    FLAG_*) of the workspace; prism_check_flags."""
    flags = (ctypes.c_uint32 * cfg.num_heads)()
    st = lib().prism_check_flags(ctypes.byref(cfg), _ws(ws)[0], ctypes.addressof(flags),
                                 _stream(stream))
    if st not in (0, -6):
        _check(st, "prism_check_flags")
    return list(flags)


def trace_enable(on: bool = True):
    """Per-stage HIP-event tracing inside the library (see prism_trace_enable)."""
    _check(lib().prism_trace_enable(1 if on else 0), "prism_trace_enable")


def trace_read() -> dict:
    """{stage: (milliseconds, launches)} accumulated since the last read."""
    n = len(STAGES)
    ms = (ctypes.c_double * n)()
    calls = (ctypes.c_int * n)()
    _check(lib().prism_trace_read(ctypes.addressof(ms), ctypes.addressof(calls)),
           "prism_trace_read")
    return {lib().prism_stage_name(i).decode(): (ms[i], calls[i]) for i in range(n)}


def plan_view(cfg: PrismConfig, ws) -> PrismLayout:
    """Byte offsets of the plan's arrays inside the workspace ws (prism_plan_view)."""
    out = PrismLayout()
    _check(lib().prism_plan_view(ctypes.byref(cfg), _ws(ws)[0], ctypes.byref(out)),
           "prism_plan_view")
    return out


def plan_views(cfg, ws) -> dict:
    """Typed views of the plan's arrays inside the workspace (see prism_layout)."""
    L = plan_view(cfg, ws)
    Hh, Z, nb, N, D, cap = cfg.num_heads, L.Z, L.nb_max, L.N, cfg.head_dim, L.pair_cap

    def view(off, dtype, shape):
        n = int(math.prod(shape))
        esz = torch.empty((), dtype=dtype).element_size()
        return ws[off: off + n * esz].view(dtype).view(*shape)

    return {
        "zone_stats": view(L.zone_stats, torch.float64, (Hh, Z, 4)),
        "audio_stats": view(L.audio_stats, torch.float64, (Z, 4)),
        "zone_diag": view(L.zone_diag, torch.float64, (Hh, Z, 4)),
        "zone_shape": view(L.zone_shape, torch.int32, (Hh, Z)),
        "zone_block": view(L.zone_block, torch.int32, (Hh, Z + 1)),
        "block_start": view(L.block_start, torch.int32, (Hh, nb)),
        "block_size": view(L.block_size, torch.int32, (Hh, nb)),
        "unit_block": view(L.unit_block, torch.int32, (Hh, N // 64)),
        "perm": view(L.perm, torch.int32, (Hh, N)),
        "inv_perm": view(L.inv_perm, torch.int32, (Hh, N)),
        "qbar": view(L.qbar, torch.float32, (Hh, nb, D)),
        "kbar": view(L.kbar, torch.float32, (Hh, nb, D)),
        "sel_count": view(L.sel_count, torch.int32, (Hh, nb)),
        "csr_ptr": view(L.csr_ptr, torch.int32, (Hh, nb + 1)),
        "csr_col": view(L.csr_col, torch.int32, (Hh, cap)),
        "csc_count": view(L.csc_count, torch.int32, (Hh, nb)),
        "csc_ptr": view(L.csc_ptr, torch.int32, (Hh, nb + 1)),
        "csc_row": view(L.csc_row, torch.int32, (Hh, cap)),
        "scores": view(L.scores, torch.float32, (nb, nb)),
        "flags": view(L.flags, torch.int32, (Hh,)),
    }


def csr_rows(views, h, which="csr"):
    """The selection lists of head h as a list of numpy arrays: which = "csr" (key blocks
    of each query block) or "csc" (query blocks of each key block), for its nb blocks."""
    nb = int(views["zone_block"][h, -1])
    cnt = views[f"{which}_count" if which == "csc" else "sel_count"][h, :nb].cpu().numpy()
    ptr = views[f"{which}_ptr"][h, :nb + 1].cpu().numpy()
    flat = views["csr_col" if which == "csr" else "csc_row"][h, :int(ptr[nb])].cpu().numpy()
    return [flat[ptr[i]:ptr[i] + cnt[i]] for i in range(nb)]


@dataclass
class PrismAttention:
    """Owns a workspace for one configuration and chains plan -> forward -> backward."""
    cfg: PrismConfig
    device: str = "cuda"

    def __post_init__(self):
        self.ws_bytes = workspace_bytes(self.cfg)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.o = None
        self.lse = None

    def plan(self, q, k, v, a2v=None, stream=None):
        # a new plan invalidates the forward state of the previous one
        self.o = None
        self.lse = None
        plan(self.cfg, q, k, v, a2v, self.ws, stream)

    def forward(self, o=None, lse=None, stream=None):
        cfg = self.cfg
        if o is None:
            o = torch.empty(cfg.N, cfg.num_heads, cfg.head_dim, dtype=cfg.torch_dtype,
                            device=self.device)
        if lse is None:
            lse = torch.empty(cfg.num_heads, cfg.N, dtype=torch.float32, device=self.device)
        attn_fwd(cfg, self.ws, o, lse, stream)
        self.o, self.lse = o, lse
        return o, lse

    def backward(self, dout, dq=None, dk=None, dv=None, stream=None):
        cfg = self.cfg
        if self.o is None:
            raise PrismError("backward needs a forward on this workspace since its last plan")
        mk = lambda: torch.empty(cfg.N, cfg.num_heads, cfg.head_dim, dtype=cfg.torch_dtype,
                                 device=self.device)
        dq = mk() if dq is None else dq
        dk = mk() if dk is None else dk
        dv = mk() if dv is None else dv
        attn_bwd(cfg, self.ws, dout, dq, dk, dv, stream)
        return dq, dk, dv

    def views(self):
        return plan_views(self.cfg, self.ws)

    def check(self, stream=None):
        """Per-head status flags (waits for the stream); all zero on a valid result."""
        return check_flags(self.cfg, self.ws, stream)
