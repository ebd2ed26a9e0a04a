"""Seeded synthetic inputs shaped like the Prism paper's video self-attention workloads.

This module holds no step of the method: it only draws random fields. Both the HIP
path and the CPU oracle read the tensors it returns (the oracle after an exact
conversion to float64), so the two never disagree about their inputs.

Field recipe (one video latent grid T x H x W, hidden width D):
  X[t,h,w,:] = background + blobs + noise
  * background: per channel, a sum of 4 separable products of low-frequency cosines
    (integer wavenumbers <= 2 periods per axis, random phases), times ``bg_amp``;
  * blob b: Gaussian envelope e_b (spatial sigma 3 tokens, temporal sigma 4 frames,
    centre moving with a constant velocity) times (u_b + 2 xi), u_b a random
    per-channel direction, xi ~ N(0,1) per token and channel; a "flip" blob
    multiplies its content by (-1)^t;
  * noise: N(0, 0.1^2) per element.
  Q/K/V for head h are X @ W_{q,k,v,h} (seeded Gaussian D x D, scaled 1/sqrt(D)),
  each channel then standardised (zero mean, unit variance over tokens).
  The audio-to-video norm field is a[t,h,w] = max_b (audio_b * e_b), in [0, 1].
  The upstream gradient dO is N(0, 1).

Token order is raster over (t, h, w), w fastest; tensors are [N, heads, D].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, asdict

import numpy as np
import torch

BASE_SEED = 20261203


@dataclass
class Blob:
    t0: float            # temporal centre (frames)
    h0: float            # spatial centre at t = t0
    w0: float
    vt_h: float = 0.0    # velocity, tokens per frame
    vt_w: float = 0.0
    audio: float = 0.0   # weight in the A2V norm field, [0, 1]
    flip: bool = False   # sign-flipping content per frame (fast in T)
    sigma_s: float = 3.0
    sigma_t: float = 4.0


@dataclass
class Workload:
    name: str
    T: int
    H: int
    W: int
    heads: int
    head_dim: int
    dtype: str                 # "f32" | "bf16"
    top_k: int
    top_p: float
    min_edge_log2: int         # 0: edges {1,2,4,8} (19 shapes); 1: {2,4,8} (16 shapes)
    bg_amp: float
    blobs: list = field(default_factory=list)
    backward: bool = False
    cid: int = 0
    tensor_cid: int = -1       # workload whose seeded tensors this one reads (-1: its own)

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    def describe(self) -> dict:
        d = asdict(self)
        d["N"] = self.N
        return d


def _blobs_for(cid: int, T: int, H: int, W: int, rng: np.random.Generator) -> list:
    """Blob layout per workload; positions drawn from ``rng``."""
    def pos():
        return (float(rng.uniform(0.2, 0.8) * T), float(rng.uniform(0.2, 0.8) * H),
                float(rng.uniform(0.2, 0.8) * W))
    if cid == 0:
        # one sounding blob whose motion runs along T only: fixed in H and W, it rises and
        # fades over the frames around t0 (the tiny grid's one zone row along T sees it
        # change from frame to frame)
        t0, h0, w0 = T / 2.0, H / 2.0, W / 4.0
        return [Blob(t0, h0, w0, vt_h=0.0, vt_w=0.0, audio=1.0)]
    if cid == 1:
        out = []
        for b in range(3):
            t0, h0, w0 = pos()
            ang = rng.uniform(0, 2 * math.pi)
            out.append(Blob(t0, h0, w0, vt_h=0.5 * math.sin(ang), vt_w=0.5 * math.cos(ang),
                            audio=1.0 if b == 0 else 0.0))
        return out
    if cid == 2:
        b_static = Blob(*pos(), audio=0.3)
        b_fast_w = Blob(*pos(), vt_w=2.0)
        b_fast_t = Blob(*pos(), flip=True)
        b_audio = Blob(*pos(), vt_h=0.25, audio=1.0)
        return [b_static, b_fast_w, b_fast_t, b_audio]
    # 2K grids: six blobs, two of them sounding
    out = []
    for b in range(6):
        t0, h0, w0 = pos()
        ang = rng.uniform(0, 2 * math.pi)
        sp = [0.0, 0.5, 1.0, 2.0, 0.5, 0.25][b]
        out.append(Blob(t0, h0, w0, vt_h=sp * math.sin(ang), vt_w=sp * math.cos(ang),
                        audio=[1.0, 0.5, 0, 0, 0, 0][b], flip=(b == 3)))
    return out


def workload(cid: int) -> Workload:
    """The five workloads: tiny (fp32), 720p, 1080p, 2K forward, 2K training step."""
    # the 2K training step runs on the 2K forward workload's tensors (same blobs, same
    # seeds): only the pass differs
    tcid = 3 if cid == 4 else cid
    ss = np.random.SeedSequence(BASE_SEED + tcid)
    rng = np.random.default_rng(ss.spawn(1)[0])
    if cid == 0:
        T, H, W, heads, D, dt, k, p, mel, amp = 8, 16, 16, 2, 64, "f32", 4, 0.9, 0, 1.0
        name, bwd = "tiny-8x16x16", False
    elif cid == 1:
        T, H, W, heads, D, dt, k, p, mel, amp = 24, 48, 80, 24, 128, "bf16", 8, 0.9, 1, 1.0
        name, bwd = "720p-24x48x80", False
    elif cid == 2:
        T, H, W, heads, D, dt, k, p, mel, amp = 24, 72, 120, 24, 128, "bf16", 8, 0.9, 1, 1.0
        name, bwd = "1080p-24x72x120", True
    elif cid in (3, 4):
        T, H, W, heads, D, dt, k, p, mel, amp = 64, 104, 128, 24, 128, "bf16", 8, 0.95, 1, 0.15
        name, bwd = ("2k-fwd-64x104x128", False) if cid == 3 else ("2k-train-64x104x128", True)
    else:
        raise ValueError(f"unknown workload {cid}")
    blobs = _blobs_for(tcid, T, H, W, rng)
    return Workload(name, T, H, W, heads, D, dt, k, p, mel, amp, blobs, bwd, cid, tcid)


def custom(T: int, H: int, W: int, heads: int, head_dim: int, dtype: str = "bf16",
           top_k: int = 8, top_p: float = 0.9, min_edge_log2: int = 1, bg_amp: float = 1.0,
           nblobs: int = 2, seed: int = 0, backward: bool = True) -> Workload:
    """A smaller grid with the same field recipe (parity cases between the named sizes)."""
    rng = np.random.default_rng(np.random.SeedSequence(BASE_SEED + 1000 + seed).spawn(1)[0])
    blobs = []
    for b in range(nblobs):
        blobs.append(Blob(float(rng.uniform(0.2, 0.8) * T), float(rng.uniform(0.2, 0.8) * H),
                          float(rng.uniform(0.2, 0.8) * W), vt_w=float(rng.uniform(-1, 1)),
                          audio=1.0 if b == 0 else 0.0, flip=(b == 2)))
    return Workload(f"custom-{T}x{H}x{W}-s{seed}", T, H, W, heads, head_dim, dtype, top_k,
                    top_p, min_edge_log2, bg_amp, blobs, backward, 1000 + seed)


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(wl: Workload, device="cpu", with_dout: bool | None = None, seed_offset: int = 0):
    """Draw q, k, v [N, heads, D], a2v [N] (float32) and optionally dout [N, heads, D]."""
    if with_dout is None:
        with_dout = wl.backward
    tcid = wl.tensor_cid if wl.tensor_cid >= 0 else wl.cid
    ss = np.random.SeedSequence(BASE_SEED + tcid + 7919 * seed_offset)
    c_bg, c_blob, c_w, c_bulk, c_do = ss.spawn(5)
    T, H, W, D, Hh = wl.T, wl.H, wl.W, wl.head_dim, wl.heads
    N = T * H * W
    dev = torch.device(device)

    # background: 4 separable cosine products per channel
    rbg = np.random.default_rng(c_bg)
    tt = torch.arange(T, dtype=torch.float32, device=dev)
    hh = torch.arange(H, dtype=torch.float32, device=dev)
    ww = torch.arange(W, dtype=torch.float32, device=dev)
    X = torch.zeros(T, H, W, D, dtype=torch.float32, device=dev)
    for _ in range(4):
        kt, kh, kw = (rbg.integers(0, 3, size=(3, D))).astype(np.float32)
        ph = rbg.uniform(0, 2 * np.pi, size=(3, D)).astype(np.float32)
        amp = rbg.normal(0, 1, size=D).astype(np.float32)
        ft = torch.cos(2 * math.pi * tt[:, None] * torch.from_numpy(kt).to(dev) / T
                       + torch.from_numpy(ph[0]).to(dev))
        fh = torch.cos(2 * math.pi * hh[:, None] * torch.from_numpy(kh).to(dev) / H
                       + torch.from_numpy(ph[1]).to(dev))
        fw = torch.cos(2 * math.pi * ww[:, None] * torch.from_numpy(kw).to(dev) / W
                       + torch.from_numpy(ph[2]).to(dev))
        X += (wl.bg_amp * torch.from_numpy(amp).to(dev)) * (
            ft[:, None, None, :] * fh[None, :, None, :] * fw[None, None, :, :])

    gen = torch.Generator(device=dev)
    gen.manual_seed(int(c_bulk.generate_state(1)[0]))
    xi = torch.randn(T, H, W, D, generator=gen, device=dev)
    rblob = np.random.default_rng(c_blob)
    a2v = torch.zeros(T, H, W, dtype=torch.float32, device=dev)
    for b in wl.blobs:
        u = torch.from_numpy(rblob.normal(0, 1, size=D).astype(np.float32)).to(dev)
        ch = b.h0 + b.vt_h * (tt - b.t0)
        cw = b.w0 + b.vt_w * (tt - b.t0)
        d2 = ((hh[None, :, None] - ch[:, None, None]) ** 2
              + (ww[None, None, :] - cw[:, None, None]) ** 2)
        env = torch.exp(-d2 / (2 * b.sigma_s ** 2)
                        - ((tt - b.t0) ** 2)[:, None, None] / (2 * b.sigma_t ** 2))
        content = u[None, None, None, :] + 2.0 * xi
        if b.flip:
            sign = 1.0 - 2.0 * (torch.arange(T, device=dev) % 2).float()
            content = content * sign[:, None, None, None]
        X += env[..., None] * content
        if b.audio > 0:
            a2v = torch.maximum(a2v, b.audio * env)
    X += 0.1 * torch.randn(T, H, W, D, generator=gen, device=dev)
    X = X.reshape(N, D)
    del xi

    rw = np.random.default_rng(c_w)
    out = {}
    tdt = _torch_dtype(wl.dtype)
    for name in ("q", "k", "v"):
        t = torch.empty(N, Hh, D, dtype=tdt, device=dev)
        for h in range(Hh):
            Wm = torch.from_numpy((rw.normal(0, 1, size=(D, D)) / math.sqrt(D))
                                  .astype(np.float32)).to(dev)
            y = X @ Wm
            y = (y - y.mean(0, keepdim=True)) / y.std(0, keepdim=True).clamp_min(1e-12)
            t[:, h, :] = y.to(tdt)
            del y
        out[name] = t
    out["a2v"] = a2v.reshape(N).contiguous()
    if with_dout:
        gdo = torch.Generator(device=dev)
        gdo.manual_seed(int(c_do.generate_state(1)[0]))
        out["dout"] = torch.randn(N, Hh, D, generator=gdo, device=dev).to(tdt)
    return out


def a2v_output(a2v, channels: int, dtype: str = "bf16", seed: int = 0):
    """A synthetic audio-to-video cross-attention output [N, channels] whose rows are seeded
    random directions scaled by the A2V intensity field a2v [N]: each row has length a2v[n]
    (up to the rounding of the stored dtype).  Stands in for the previous layer's output,
    which needs the model; the norm producer reads it back into an A2V field."""
    dev = a2v.device
    g = torch.Generator(device=dev)
    g.manual_seed(BASE_SEED + 31 * seed + 17)
    out = torch.empty(a2v.shape[0], channels, dtype=_torch_dtype(dtype), device=dev)
    step = max(1, (1 << 28) // max(channels, 1))
    for i0 in range(0, a2v.shape[0], step):
        u = torch.randn(min(step, a2v.shape[0] - i0), channels, generator=g, device=dev)
        u = u / u.norm(dim=1, keepdim=True).clamp_min(1e-30)
        out[i0:i0 + u.shape[0]] = (u * a2v[i0:i0 + u.shape[0], None]).to(out.dtype)
    return out
