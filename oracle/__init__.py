"""CPU oracle for Prism's dynamic block-sparse video self-attention (float64).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and its
binding) never imports this package, and this package never imports the product.

The arithmetic lives in ``prism_oracle.c`` (plain C loops, one head at a time); this
module compiles it with gcc and marshals numpy arrays.  Every function cites the page
passage it follows in the C source.

Parity status of each function (what pins it; see tests/test_oracle_pins.py):
  zone_stats, audio_stats  -- closed forms on ramps, separable fields, constant zones
  zone_plan                -- l* invariants, continuous optimality of J, brute-force
                              enumeration of the pool, ordering invariant, hand-derived
                              shapes (tests/golden/shape_cases.json)
  permutation              -- bijection, box structure, 64-aligned offsets
  block_means, block_probs -- brute force, softmax rows sum to one
  select                   -- brute-force sort, p = 0 / k = 1 / k = all special cases
  attn_fwd                 -- Top-k = all equals textbook dense attention; any plan equals
                              dense attention under the plan's block mask
  attn_bwd                 -- central finite differences of attn_fwd
  with_mag outputs         -- bound the change of o, dq, dk, dv under relative
                              perturbations of the weights and dS (dense masked
                              formulation, random and worst-case signs; tight for o, dv)
  row_norms                -- closed forms (unit vectors, constant rows, Pythagorean rows)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "prism_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

ZONE = 8


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", _LIB + ".tmp",
               _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _dp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def _f64(x):
    """Exact conversion of a torch tensor / numpy array to contiguous float64."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu").to(torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def zone_stats(T, H, W, v, density_mode=0):
    v = _f64(v)
    N, D = v.shape
    assert N == T * H * W
    Z = N // ZONE ** 3
    out = np.zeros((Z, 4))
    rc = _load().orc_zone_stats(T, H, W, D, _dp(v), int(density_mode), _dp(out))
    if rc:
        raise ValueError("grid not divisible by the zone edge")
    return out


def audio_stats(T, H, W, a):
    a = _f64(a).reshape(-1)
    Z = a.size // ZONE ** 3
    out = np.zeros((Z, 4))
    rc = _load().orc_audio_stats(T, H, W, _dp(a), _dp(out))
    if rc:
        raise ValueError("grid not divisible by the zone edge")
    return out


def shape_pool(S, min_edge_log2):
    cand = np.zeros((64, 3), dtype=np.int32)
    n = _load().orc_shape_pool(int(S), int(min_edge_log2), _ip(cand))
    return cand[:n].copy()


def zone_plan(vstats, astats=None, tau128=0.5, tau256=0.25, eps=1e-6, min_edge_log2=1,
              map_exponent=0.5, fixed_shape=0, density_mode=0):
    lib = _load()
    lib.orc_zone_plan.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                  ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_void_p]
    vstats = np.ascontiguousarray(vstats, dtype=np.float64)
    Z = vstats.shape[0]
    shape = np.zeros(Z, dtype=np.int32)
    diag = np.zeros((Z, 12))
    ap = None
    if astats is not None:
        astats = np.ascontiguousarray(astats, dtype=np.float64)
        ap = astats.ctypes.data
    rc = lib.orc_zone_plan(Z, vstats.ctypes.data, ap, tau128, tau256, eps, min_edge_log2,
                           float(map_exponent), int(fixed_shape), int(density_mode),
                           shape.ctypes.data, diag.ctypes.data)
    if rc:
        raise ValueError("bad zone_plan arguments")
    return shape, diag


def unpack_shape(code):
    code = np.asarray(code)
    return np.stack([(code >> 4) & 3, (code >> 2) & 3, code & 3], axis=-1)


def permutation(T, H, W, shape):
    N = T * H * W
    shape = np.ascontiguousarray(shape, dtype=np.int32)
    perm = np.zeros(N, dtype=np.int32)
    inv = np.zeros(N, dtype=np.int32)
    bstart = np.zeros(N // 64 + 1, dtype=np.int32)
    bsize = np.zeros(N // 64 + 1, dtype=np.int32)
    bof = np.zeros(N, dtype=np.int32)
    nb = _load().orc_permutation(T, H, W, _ip(shape), _ip(perm), _ip(inv), _ip(bstart),
                                 _ip(bsize), _ip(bof))
    if nb < 0:
        raise ValueError("grid not divisible by the zone edge")
    return perm, inv, bstart[:nb].copy(), bsize[:nb].copy(), bof


def block_means(x, perm, bstart, bsize):
    x = _f64(x)
    D = x.shape[1]
    nb = len(bstart)
    out = np.zeros((nb, D))
    _load().orc_block_means(D, _dp(x), _ip(perm), nb, _ip(np.ascontiguousarray(bstart)),
                            _ip(np.ascontiguousarray(bsize)), _dp(out))
    return out


def block_probs(qbar, kbar, scale):
    lib = _load()
    lib.orc_block_probs.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
                                    ctypes.c_void_p]
    qbar = np.ascontiguousarray(qbar, dtype=np.float64)
    kbar = np.ascontiguousarray(kbar, dtype=np.float64)
    nb, D = qbar.shape
    s = np.zeros((nb, nb))
    P = np.zeros((nb, nb))
    lib.orc_block_probs(nb, D, qbar.ctypes.data, kbar.ctypes.data, float(scale),
                        s.ctypes.data, P.ctypes.data)
    return s, P


def select(P, top_k, top_p):
    lib = _load()
    lib.orc_select.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    P = np.ascontiguousarray(P, dtype=np.float64)
    nb = P.shape[0]
    count = np.zeros(nb, dtype=np.int32)
    cols = np.zeros((nb, nb), dtype=np.int32)
    diag = np.zeros((nb, 4))
    lib.orc_select(nb, P.ctypes.data, int(top_k), float(top_p), count.ctypes.data,
                   cols.ctypes.data, diag.ctypes.data)
    return count, cols, diag


@dataclass
class HeadPlan:
    """Everything the oracle decides for one head."""
    shape: np.ndarray        # [Z] packed log2 edges
    zone_diag: np.ndarray    # [Z][12]
    vstats: np.ndarray       # [Z][4]
    perm: np.ndarray         # [N] permuted position -> token
    inv: np.ndarray          # [N] token -> permuted position
    bstart: np.ndarray       # [nb]
    bsize: np.ndarray        # [nb]
    bof: np.ndarray          # [N] permuted position -> block
    qbar: np.ndarray         # [nb][D]
    kbar: np.ndarray         # [nb][D]
    s: np.ndarray            # [nb][nb] block logits
    P: np.ndarray            # [nb][nb] block relevance
    count: np.ndarray        # [nb]
    cols: np.ndarray         # [nb][nb] (row i: first count[i] entries, ascending)
    sel_diag: np.ndarray     # [nb][4]

    @property
    def nb(self):
        return len(self.bstart)

    def lists(self):
        return [self.cols[i, :self.count[i]].copy() for i in range(self.nb)]


def topk_of(nb, top_k, top_k_frac):
    """Top-k of a head with nb blocks: ceil(frac * nb) when a fraction is given (the
    fraction taken as the float32 the library receives), else the count."""
    if top_k_frac and top_k_frac > 0:
        return int(np.ceil(float(np.float32(top_k_frac)) * nb))
    return int(top_k)


def plan_head(T, H, W, q, k, v, a=None, top_k=8, top_p=0.9, tau128=0.5, tau256=0.25,
              eps=1e-6, min_edge_log2=1, score_scale=None, astats=None, top_k_frac=0.0,
              map_exponent=0.5, fixed_shape=0, density_mode=0):
    """The full plan for one head: q, k, v are [N, D] for that head; a is [N] or None."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    D = q.shape[1]
    if score_scale is None:
        score_scale = 1.0 / np.sqrt(D)
    vs = zone_stats(T, H, W, v, density_mode)
    if astats is None and a is not None:
        astats = audio_stats(T, H, W, a)
    shape, zd = zone_plan(vs, astats, tau128, tau256, eps, min_edge_log2, map_exponent,
                          fixed_shape, density_mode)
    perm, inv, bstart, bsize, bof = permutation(T, H, W, shape)
    qbar = block_means(q, perm, bstart, bsize)
    kbar = block_means(k, perm, bstart, bsize)
    s, P = block_probs(qbar, kbar, score_scale)
    count, cols, sd = select(P, topk_of(len(bsize), top_k, top_k_frac), top_p)
    return HeadPlan(shape, zd, vs, perm, inv, bstart, bsize, bof, qbar, kbar, s, P, count,
                    cols, sd)


def attn_fwd(plan: HeadPlan, q, k, v, scale=None, rows=None, with_mag=False):
    """o [N, D], lse [N] (only listed rows are written when rows is given); with_mag also
    returns mo [N, D], the first-order size of the change in o under a relative
    perturbation of at most 1 of every attention weight (see orc_attn_fwd)."""
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.zeros((N, D))
    lse = np.full(N, np.nan)
    mo = np.zeros((N, D)) if with_mag else None
    lib.orc_attn_fwd.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 8 + [
        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    lib.orc_attn_fwd(N, D, q.ctypes.data, k.ctypes.data, v.ctypes.data, plan.perm.ctypes.data,
                     plan.inv.ctypes.data, plan.bstart.ctypes.data, plan.bsize.ctypes.data,
                     plan.bof.ctypes.data, plan.nb, plan.count.ctypes.data,
                     plan.cols.ctypes.data, float(scale),
                     None if rws is None else rws.ctypes.data,
                     0 if rws is None else len(rws), o.ctypes.data, lse.ctypes.data,
                     None if mo is None else mo.ctypes.data)
    return (o, lse, mo) if with_mag else (o, lse)


def attn_bwd(plan: HeadPlan, q, k, v, dout, scale=None, rows=None, with_mag=False):
    """dq, dk, dv [N, D]; with rows given, only those query tokens' terms are summed.
    with_mag also returns mq, mk, mv [N, D]: the first-order size of the change in each
    gradient under a relative perturbation of at most 1 of every attention weight and
    every dS (see orc_attn_bwd)."""
    lib = _load()
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    N, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.zeros((N, D))
    dk = np.zeros((N, D))
    dv = np.zeros((N, D))
    mags = [np.zeros((N, D)) for _ in range(3)] if with_mag else [None] * 3
    lib.orc_attn_bwd.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 9 + [
        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p,
        ctypes.c_int] + [ctypes.c_void_p] * 6
    rws = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    if rws is not None and len(np.unique(rws)) != len(rws):
        raise ValueError("attn_bwd: rows must not repeat a token")
    lib.orc_attn_bwd(N, D, q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                     plan.perm.ctypes.data, plan.inv.ctypes.data, plan.bstart.ctypes.data,
                     plan.bsize.ctypes.data, plan.bof.ctypes.data, plan.nb,
                     plan.count.ctypes.data, plan.cols.ctypes.data, float(scale),
                     None if rws is None else rws.ctypes.data,
                     0 if rws is None else len(rws), dq.ctypes.data, dk.ctypes.data,
                     dv.ctypes.data, *[None if m is None else m.ctypes.data for m in mags])
    return (dq, dk, dv, *mags) if with_mag else (dq, dk, dv)


def row_norms(x, rows=None):
    """The A2V norm field sqrt(sum_c x[n, c]^2) of rows `rows` (default: all) of x [N, C]."""
    x = _f64(x)
    N, C = x.shape
    rows = np.arange(N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros(len(rows))
    lib = _load()
    lib.orc_row_norms.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_void_p]
    if lib.orc_row_norms(C, x.ctypes.data, rows.ctypes.data, len(rows), out.ctypes.data):
        raise ValueError("bad row_norms arguments")
    return out
