"""Pins for the CPU oracle: each check uses a fact fixed by the pages or by the mathematics
(closed forms, brute force, textbook attention, finite differences), never the oracle's own
formula retyped."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
rng0 = np.random.default_rng(12345)


def coords(T, H, W):
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return t.reshape(-1), h.reshape(-1), w.reshape(-1)


# ----------------------------------------------------------------------------- zone stats

@pytest.mark.parametrize("axis", [0, 1, 2])
def test_zone_stats_ramp(axis):
    T, H, W, D = 16, 8, 16, 5
    alpha = rng0.normal(size=D)
    c = coords(T, H, W)[axis].astype(float)
    v = c[:, None] * alpha[None, :]
    st = oracle.zone_stats(T, H, W, v)
    a2 = np.mean(alpha ** 2)
    var8 = (8 ** 2 - 1) / 12.0          # population variance of 0..7
    exp = np.zeros(3)
    exp[axis] = var8 * a2
    for m in range(st.shape[0]):
        np.testing.assert_allclose(st[m, :3], exp, atol=1e-12)
        # T ramp: no spatial spread, frame differences of alpha; H/W ramp: spatial only
        rho = a2 if axis == 0 else var8 * a2
        assert st[m, 3] == pytest.approx(rho, rel=1e-12)


def test_zone_stats_separable():
    """V = f(t) + g(h) + u(w): directional variances are those of f, g, u inside the zone;
    the spatial term is Var(g) + Var(u); the temporal term is the mean squared step of f."""
    T, H, W, D = 8, 16, 8, 3
    f = rng0.normal(size=(T, D))
    g = rng0.normal(size=(H, D))
    u = rng0.normal(size=(W, D))
    t, h, w = coords(T, H, W)
    v = f[t] + g[h] + u[w]
    st = oracle.zone_stats(T, H, W, v)
    for m, zh in enumerate(range(2)):
        gz = g[8 * zh: 8 * zh + 8]
        exp_t = np.mean(np.var(f, axis=0))
        exp_h = np.mean(np.var(gz, axis=0))
        exp_w = np.mean(np.var(u, axis=0))
        spatial = exp_h + exp_w
        temporal = np.mean(np.sum(np.diff(f, axis=0) ** 2, axis=0) / 7.0)
        np.testing.assert_allclose(st[m], [exp_t, exp_h, exp_w, spatial + temporal], rtol=1e-12)


def test_zone_stats_constant_zone():
    st = oracle.zone_stats(8, 8, 8, np.full((512, 4), 3.25))
    assert np.all(st == 0)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_audio_stats_ramp(axis):
    T, H, W = 8, 16, 8
    c = coords(T, H, W)[axis].astype(float)
    a = 0.01 * c + 0.2
    st = oracle.audio_stats(T, H, W, a)
    for m in range(st.shape[0]):
        sl = [slice(None)] * 3
        zone = a.reshape(T, H, W)[:, 8 * m: 8 * m + 8, :]
        assert st[m, 0] == pytest.approx(zone.mean(), rel=1e-13)
        exp = np.zeros(3)
        exp[axis] = 1e-4 * (63 / 12.0)
        np.testing.assert_allclose(st[m, 1:], exp, atol=1e-15)


# ----------------------------------------------------------------------------- shapes

def test_pool_sizes():
    # pages: 16 candidates with edges in {2,4,8}; edges {1,2,4,8}: 19
    n16 = sum(len(oracle.shape_pool(S, 1)) for S in (6, 7, 8))
    n19 = sum(len(oracle.shape_pool(S, 0)) for S in (6, 7, 8))
    assert (n16, n19) == (16, 19)
    for S in (6, 7, 8):
        for c in oracle.shape_pool(S, 0):
            assert 2 ** c.sum() == 2 ** S and c.max() <= 3


def _brute_shape(lstar, B, min_edge):
    """Enumerate every edge triple of {1,2,4,8} with product B and edges >= min_edge."""
    best, arg = None, None
    cands = [c for c in itertools.product([1, 2, 4, 8], repeat=3)
             if c[0] * c[1] * c[2] == B and min(c) >= min_edge]
    dists = [sum((lstar[d] - math.log2(c[d])) ** 2 for d in range(3)) for c in cands]
    m = min(dists)
    tied = sorted(c for c, dd in zip(cands, dists) if dd <= m + 1e-9)
    return tied[0]


@pytest.mark.parametrize("mel", [0, 1])
def test_golden_shapes(mel):
    cases = json.load(open(os.path.join(HERE, "golden", "shape_cases.json")))["cases"]
    for cs in cases:
        vstats = np.array([[1.0, 1.0, 1.0, 1.0], cs["sigma2"] + [cs["rho"]]])
        shape, diag = oracle.zone_plan(vstats, None, min_edge_log2=mel)
        edges = tuple(int(2 ** e) for e in oracle.unpack_shape(shape[1]))
        assert edges == tuple(cs["expect"][str(mel)]), cs["name"]


def _random_stats(n, seed):
    r = np.random.default_rng(seed)
    vs = np.zeros((n, 4))
    vs[:, :3] = r.gamma(0.7, size=(n, 3)) * r.uniform(0.01, 3, size=(n, 1))
    vs[:, 3] = r.uniform(0, 5, size=n)
    ast = np.zeros((n, 4))
    ast[:, 0] = r.uniform(0, 1, size=n)
    ast[:, 1:] = r.gamma(0.5, size=(n, 3))
    return vs, ast


@pytest.mark.parametrize("mel", [0, 1])
@pytest.mark.parametrize("use_audio", [False, True])
def test_plan_invariants_random(mel, use_audio):
    vs, ast = _random_stats(400, 7 + mel)
    shape, diag = oracle.zone_plan(vs, ast if use_audio else None, min_edge_log2=mel)
    edges = oracle.unpack_shape(shape)
    rho = vs[:, 3] / vs[:, 3].max()
    B = 2 ** edges.sum(1)
    # tiers: rho >= 0.5 -> 64, [0.25, 0.5) -> 128, else 256
    np.testing.assert_array_equal(B, np.where(rho >= 0.5, 64, np.where(rho >= 0.25, 128, 256)))
    assert np.all(edges >= mel) and np.all(edges <= 3)
    g = diag[:, 2:5]
    ls = diag[:, 5:8]
    S = np.log2(B)
    # sum of l* is S; differences follow -1/2 log2 of the g ratio
    np.testing.assert_allclose(ls.sum(1), S, atol=1e-10)
    np.testing.assert_allclose(ls[:, 0] - ls[:, 1], -0.5 * np.log2(g[:, 0] / g[:, 1]), atol=1e-10)
    np.testing.assert_allclose(ls[:, 1] - ls[:, 2], -0.5 * np.log2(g[:, 1] / g[:, 2]), atol=1e-10)
    if not use_audio:
        # without audio the shares sum to one (zones with any variance), so sum g = 1 + 3 eps
        nz = vs[:, :3].sum(1) > 0
        np.testing.assert_allclose(g[nz].sum(1), 1 + 3e-6, rtol=1e-12)
    r = np.random.default_rng(3)
    for m in range(len(shape)):
        # brute-force enumeration of the pool
        got = tuple(int(2 ** e) for e in edges[m])
        assert got == _brute_shape(ls[m], int(B[m]), 2 ** mel)
        # l* minimises J = sum g_d (b_d^2 - 1) on the surface prod b_d = B
        J = lambda l: float(np.sum(g[m] * (4.0 ** l - 1)))
        j0 = J(ls[m])
        for _ in range(20):
            d = r.normal(size=3) * r.uniform(1e-3, 1)
            d -= d.mean()
            assert J(ls[m] + d) >= j0 * (1 - 1e-12)
        # ordering invariant: the axis that varies more never gets the longer edge
        if diag[m, 10] > 1e-9:
            for a, b in itertools.permutations(range(3), 2):
                if g[m, a] > g[m, b]:
                    assert edges[m, a] <= edges[m, b]


def test_audio_zero_equals_first_layer():
    """An all-zero A2V norm field and no field at all (first layer) give the same plan."""
    T, H, W, D = 16, 16, 8, 4
    v = rng0.normal(size=(T * H * W, D))
    vs = oracle.zone_stats(T, H, W, v)
    ast = oracle.audio_stats(T, H, W, np.zeros(T * H * W))
    s1, _ = oracle.zone_plan(vs, None)
    s2, _ = oracle.zone_plan(vs, ast)
    np.testing.assert_array_equal(s1, s2)


def test_audio_guidance_moves_shape():
    """A strong A2V field varying only along W (a-bar = 1 gates the audio term fully)
    shortens the W edge of an isotropic B = 128 zone: without audio l* = (7/3)^3 and the
    tie rule gives (4,4,8); with g_W raised by one, l* = (8/3, 8/3, 5/3) and (2,3,2)/(3,2,2)
    tie at 2/3, giving (4,8,4)."""
    vs = np.array([[1.0, 1.0, 1.0, 1.0], [1.0, 1.0, 1.0, 0.3]])
    ast = np.array([[1.0, 0.0, 0.0, 1.0], [1.0, 0.0, 0.0, 1.0]])
    s0, _ = oracle.zone_plan(vs, None)
    s1, d1 = oracle.zone_plan(vs, ast)
    e0, e1 = oracle.unpack_shape(s0[1]), oracle.unpack_shape(s1[1])
    assert tuple(e0) == (2, 2, 3)
    assert tuple(e1) == (2, 3, 2)
    np.testing.assert_allclose(d1[1, 2:5], [1 / 3 + 1e-6, 1 / 3 + 1e-6, 4 / 3 + 1e-6], rtol=1e-12)


# ----------------------------------------------------------------------------- permutation

def _grid_plan(T, H, W, seed, mel=1):
    r = np.random.default_rng(seed)
    Z = (T // 8) * (H // 8) * (W // 8)
    codes = []
    for m in range(Z):
        S = r.integers(6, 9)
        pool = oracle.shape_pool(S, mel)
        c = pool[r.integers(len(pool))]
        codes.append(c[0] * 16 + c[1] * 4 + c[2])
    return np.array(codes, dtype=np.int32)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_permutation_structure(seed):
    T, H, W = 16, 24, 16
    shape = _grid_plan(T, H, W, seed, mel=seed % 2)
    perm, inv, bstart, bsize, bof = oracle.permutation(T, H, W, shape)
    N = T * H * W
    assert np.array_equal(np.sort(perm), np.arange(N))
    assert np.array_equal(inv[perm], np.arange(N))
    assert np.array_equal(perm[inv], np.arange(N))
    edges = 2 ** oracle.unpack_shape(shape)
    assert len(bstart) == int(np.sum(512 // edges.prod(1)))
    assert np.all(bstart % 64 == 0) and np.all(np.isin(bsize, [64, 128, 256]))
    t, h, w = coords(T, H, W)
    nzh, nzw = H // 8, W // 8
    for b in range(len(bstart)):
        toks = perm[bstart[b]: bstart[b] + bsize[b]]
        assert np.all(bof[bstart[b]: bstart[b] + bsize[b]] == b)
        zt, zh, zw = t[toks] // 8, h[toks] // 8, w[toks] // 8
        assert len(set(zip(zt, zh, zw))) == 1
        m = (zt[0] * nzh + zh[0]) * nzw + zw[0]
        ext = [np.ptp(t[toks]) + 1, np.ptp(h[toks]) + 1, np.ptp(w[toks]) + 1]
        assert tuple(ext) == tuple(edges[m]) and bsize[b] == edges[m].prod()
        # raster order inside the block
        assert np.all(np.diff(toks) > 0)


# ----------------------------------------------------------------------------- pooling, scores

def test_block_means_and_probs():
    T, H, W, D = 8, 16, 16, 8
    shape = _grid_plan(T, H, W, 5, mel=0)
    perm, inv, bstart, bsize, bof = oracle.permutation(T, H, W, shape)
    x = rng0.normal(size=(T * H * W, D))
    y = rng0.normal(size=(T * H * W, D))
    xb = oracle.block_means(x, perm, bstart, bsize)
    yb = oracle.block_means(y, perm, bstart, bsize)
    for b in range(len(bstart)):
        np.testing.assert_allclose(xb[b], x[perm[bstart[b]:bstart[b] + bsize[b]]].mean(0),
                                   rtol=1e-12)
    s, P = oracle.block_probs(xb, yb, 0.3)
    np.testing.assert_allclose(s, 0.3 * xb @ yb.T, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(P.sum(1), 1.0, rtol=1e-13)
    assert np.all(np.argmax(P, 1) == np.argmax(s, 1))


# ----------------------------------------------------------------------------- selection

def _brute_select(P, k, p):
    nb = P.shape[0]
    out = []
    for i in range(nb):
        order = np.lexsort((np.arange(nb), -P[i]))
        cum = np.cumsum(P[i][order])
        hit = np.nonzero(cum >= p)[0]
        n_p = hit[0] + 1 if len(hit) else nb
        n = min(nb, max(k, n_p, 1))
        out.append(np.sort(order[:n]))
    return out


@pytest.mark.parametrize("k,p", [(4, 0.9), (1, 0.5), (8, 0.95), (3, 0.0), (50, 0.2), (1, 1.0)])
def test_select_brute_force(k, p):
    nb = 37
    s = rng0.normal(size=(nb, nb)) * 2
    s[3, 5] = s[3, 6]          # exact tie
    P = np.exp(s - s.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    count, cols, _ = oracle.select(P, k, p)
    exp = _brute_select(P, k, p)
    for i in range(nb):
        np.testing.assert_array_equal(cols[i, :count[i]], exp[i])


def test_select_special_cases():
    nb = 29
    s = rng0.normal(size=(nb, nb)) * 3
    P = np.exp(s - s.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    c, _, _ = oracle.select(P, 5, 0.0)            # p = 0: exactly k
    assert np.all(c == 5)
    c, cols, _ = oracle.select(P, nb, 0.5)        # k = all: every block
    assert np.all(c == nb)
    c, cols, _ = oracle.select(P, 1, 0.7)         # k = 1: the minimal Top-p prefix
    for i in range(nb):
        sel = cols[i, :c[i]]
        mass = P[i, sel].sum()
        assert mass >= 0.7
        assert mass - P[i, sel].min() < 0.7
        rest = np.setdiff1d(np.arange(nb), sel)
        if len(rest):
            assert P[i, rest].max() <= P[i, sel].min()


# ----------------------------------------------------------------------------- attention

def _small_problem(seed, T=8, H=16, W=16, D=16, k=3, p=0.6, mel=0, scale_inputs=1.0):
    r = np.random.default_rng(seed)
    N = T * H * W
    q = r.normal(size=(N, D)) * scale_inputs
    kk = r.normal(size=(N, D)) * scale_inputs
    v = r.normal(size=(N, D))
    a = r.uniform(size=N)
    plan = oracle.plan_head(T, H, W, q, kk, v, a, top_k=k, top_p=p, min_edge_log2=mel)
    return q, kk, v, plan


def _dense(q, k, v, scale, mask=None):
    s = scale * q @ k.T
    if mask is not None:
        s = np.where(mask, s, -np.inf)
    m = s.max(1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(1, keepdims=True)
    return (e / z) @ v, (m + np.log(z))[:, 0]


def test_attn_topk_all_is_dense():
    T, H, W, D = 8, 16, 16, 64
    r = np.random.default_rng(1)
    N = T * H * W
    q, k, v = (r.normal(size=(N, D)) for _ in range(3))
    plan = oracle.plan_head(T, H, W, q, k, v, None, top_k=N, top_p=0.9, min_edge_log2=0)
    assert np.all(plan.count == plan.nb)
    o, lse = oracle.attn_fwd(plan, q, k, v)
    od, lsed = _dense(q, k, v, 1 / 8.0)
    np.testing.assert_allclose(o, od, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, atol=1e-12)


def _block_mask(plan, N):
    blk_tok = np.empty(N, dtype=np.int64)
    blk_tok[plan.perm] = plan.bof          # token -> block
    sel = np.zeros((plan.nb, plan.nb), dtype=bool)
    for i, l in enumerate(plan.lists()):
        sel[i, l] = True
    return sel[blk_tok][:, blk_tok]


@pytest.mark.parametrize("seed", [0, 1])
def test_attn_equals_masked_dense(seed):
    q, k, v, plan = _small_problem(seed, D=32)
    N = q.shape[0]
    assert plan.count.min() < plan.nb     # a genuinely sparse plan
    o, lse = oracle.attn_fwd(plan, q, k, v)
    od, lsed = _dense(q, k, v, 1 / math.sqrt(32), _block_mask(plan, N))
    np.testing.assert_allclose(o, od, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, atol=1e-12)
    rows = np.array([0, 17, 300, N - 1])
    o2, l2 = oracle.attn_fwd(plan, q, k, v, rows=rows)
    np.testing.assert_array_equal(o2[rows], o[rows])


def test_attn_bwd_finite_differences():
    T, H, W, D = 8, 8, 8, 16
    q, k, v, plan = _small_problem(3, T, H, W, D, k=2, p=0.5, scale_inputs=0.7)
    N = q.shape[0]
    r = np.random.default_rng(9)
    do = r.normal(size=(N, D))
    dq, dk, dv = oracle.attn_bwd(plan, q, k, v, do)

    def loss(q, k, v):
        o, _ = oracle.attn_fwd(plan, q, k, v)
        return float(np.sum(o * do))

    h = 1e-5
    for name, X, G in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            x, c = r.integers(N), r.integers(D)
            Xp, Xm = X.copy(), X.copy()
            Xp[x, c] += h
            Xm[x, c] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = Xp, Xm
            fd = (loss(**args_p) - loss(**args_m)) / (2 * h)
            assert G[x, c] == pytest.approx(fd, rel=1e-6, abs=1e-8), (name, x, c)


def test_attn_bwd_rows_subset():
    """With an upstream gradient that vanishes off a row sample, summing only those rows'
    terms gives the full gradient."""
    q, k, v, plan = _small_problem(4, D=16)
    N = q.shape[0]
    r = np.random.default_rng(2)
    rows = r.choice(N, 40, replace=False)
    do = np.zeros((N, 16))
    do[rows] = r.normal(size=(40, 16))
    full = oracle.attn_bwd(plan, q, k, v, do)
    part = oracle.attn_bwd(plan, q, k, v, do, rows=rows)
    for a, b in zip(full, part):
        np.testing.assert_allclose(a, b, atol=1e-13)
    # sum over keys of dV equals the sum of dO; dK sums to zero
    np.testing.assert_allclose(full[2].sum(0), do.sum(0), atol=1e-10)
    np.testing.assert_allclose(full[1].sum(0), 0, atol=1e-10)
    # a row listed twice would count its terms twice: refused
    with pytest.raises(ValueError):
        oracle.attn_bwd(plan, q, k, v, do, rows=np.concatenate([rows, rows[:1]]))


def _dense_grads(q, k, v, do, scale, mask, wf=None, wb=None, wd=None):
    """Dense masked attention gradients with optional relative perturbations: wf of the
    forward's weights (renormalised; it moves o and so delta), wb of the weights in the
    dV product, wd of dS.  Returns o, dq, dk, dv."""
    s = np.where(mask, scale * q @ k.T, -np.inf)
    P = np.exp(s - s.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    Pf = P if wf is None else P * (1 + wf)
    o = (Pf / Pf.sum(1, keepdims=True)) @ v
    delta = np.sum(do * o, 1, keepdims=True)
    dS = P * (do @ v.T - delta)
    if wd is not None:
        dS = dS * (1 + wd)
    Pb = P if wb is None else P * (1 + wb)
    return o, scale * dS @ k, scale * dS.T @ q, Pb.T @ do


def test_rounding_magnitudes_bound_perturbed_weights():
    """The oracle's magnitude outputs bound, to first order, how far o, dq, dk and dv move
    when every attention weight and every dS is perturbed by a relative amount of at most
    u (checked on the dense masked formulation with random and with worst-case signs), are
    reached by the worst case (o, dv), and are never below the results' own sizes."""
    q, k, v, plan = _small_problem(6, D=16, scale_inputs=1.5)
    N, D = q.shape
    scale = 1 / math.sqrt(D)
    r = np.random.default_rng(8)
    do = r.normal(size=(N, D))
    mask = _block_mask(plan, N)
    o0, mo = oracle.attn_fwd(plan, q, k, v, with_mag=True)[0::2]
    dq0, dk0, dv0, mq, mk, mv = oracle.attn_bwd(plan, q, k, v, do, with_mag=True)
    od, dqd, dkd, dvd = _dense_grads(q, k, v, do, scale, mask)
    np.testing.assert_allclose(od, o0, atol=1e-12)
    for g, m in ((dq0, mq), (dk0, mk), (dv0, mv)):
        assert np.all(np.abs(g) <= m * (1 + 1e-12) + 1e-15)
    u = 2.0 ** -11
    slack = 1 + 8 * u   # second-order terms
    for seed in range(3):
        rr = np.random.default_rng(100 + seed)
        wf, wb, wd = (u * rr.uniform(-1, 1, size=(N, N)) for _ in range(3))
        o1, dq1, dk1, dv1 = _dense_grads(q, k, v, do, scale, mask, wf, wb, wd)
        for a, b, m in ((o1, od, mo), (dq1, dqd, mq), (dk1, dkd, mk), (dv1, dvd, mv)):
            assert np.all(np.abs(a - b) <= u * m * slack + 1e-14)
    # worst case for channel c: weights moved toward the sign of (v - o) and of do
    for c in (0, 7):
        wf = u * np.sign(v[None, :, c] - od[:, None, c])
        o1 = _dense_grads(q, k, v, do, scale, mask, wf=wf)[0]
        ratio = np.abs(o1[:, c] - od[:, c]) / (u * mo[:, c])
        assert ratio.max() <= slack and ratio.max() >= 0.99
        wb = u * np.sign(do[:, None, c]) * np.ones((1, N))
        dv1 = _dense_grads(q, k, v, do, scale, mask, wb=wb)[3]
        hit = mv[:, c] > 0
        ratio = np.abs(dv1[hit, c] - dvd[hit, c]) / (u * mv[hit, c])
        assert ratio.max() <= slack and ratio.min() >= 1 - 1e-9


# ----------------------------------------------------------------------------- ablation settings

def test_density_terms_separable():
    """Density ablation: mode 1 keeps Var(g) + Var(u) (spatial spread at a fixed time),
    mode 2 the mean squared frame step of f, mode 0 their sum (same separable field as
    test_zone_stats_separable, closed forms from numpy)."""
    T, H, W, D = 8, 8, 8, 3
    f = rng0.normal(size=(T, D))
    g = rng0.normal(size=(H, D))
    u = rng0.normal(size=(W, D))
    t, h, w = coords(T, H, W)
    v = f[t] + g[h] + u[w]
    spatial = np.mean(np.var(g, axis=0)) + np.mean(np.var(u, axis=0))
    temporal = np.mean(np.sum(np.diff(f, axis=0) ** 2, axis=0) / 7.0)
    for mode, exp in ((0, spatial + temporal), (1, spatial), (2, temporal)):
        st = oracle.zone_stats(T, H, W, v, density_mode=mode)
        assert st[0, 3] == pytest.approx(exp, rel=1e-12)
        # the directional variances do not depend on the density terms
        np.testing.assert_allclose(st[0, :3], oracle.zone_stats(T, H, W, v)[0, :3], rtol=0)


def test_density_from_audio_intensity():
    """Density mode 3: the tier follows the zone-mean A2V intensity normalised by its maximum
    (1.0 -> 64, 0.4 -> 128, 0.1 -> 256 with the pages' thresholds 0.5 and 0.25), whatever
    rho_raw says."""
    vs = np.array([[1.0, 1.0, 1.0, 0.0], [1.0, 1.0, 1.0, 5.0], [1.0, 1.0, 1.0, 1.0]])
    ast = np.array([[2.0, 0, 0, 0], [0.8, 0, 0, 0], [0.2, 0, 0, 0]])
    shape, diag = oracle.zone_plan(vs, ast, density_mode=3)
    assert list(diag[:, 8]) == [64.0, 128.0, 256.0]
    np.testing.assert_allclose(diag[:, 0], [1.0, 0.4, 0.1], rtol=1e-15)


@pytest.mark.parametrize("alpha", [0.25, 0.5, 1.0, 2.0])
def test_mapping_exponent(alpha):
    """Mapping ablation b_d ~ g_d^-alpha: sum_d l*_d = S for every alpha, and
    l*_d - l*_d' = -alpha log2(g_d / g_d')."""
    vs = np.array([[0.6, 0.3, 0.1, 0.2]])   # shares r = (0.6, 0.3, 0.1), rho = 1 -> B = 64
    shape, diag = oracle.zone_plan(vs, None, eps=0.0, map_exponent=alpha)
    ls = diag[0, 5:8]
    assert ls.sum() == pytest.approx(6.0, abs=1e-12)
    assert ls[0] - ls[1] == pytest.approx(-alpha * math.log2(0.6 / 0.3), abs=1e-12)
    assert ls[1] - ls[2] == pytest.approx(-alpha * math.log2(0.3 / 0.1), abs=1e-12)


def test_mapping_exponent_extremes():
    """A vanishing exponent maps every zone to the isotropic optimum S/3 per axis, so a
    64-token block is 4 x 4 x 4; a large one drives the fast axis to the shortest edge."""
    vs = np.array([[0.9, 0.05, 0.05, 1.0]])
    shape, diag = oracle.zone_plan(vs, None, eps=0.0, map_exponent=1e-9)
    assert list(oracle.unpack_shape(shape)[0]) == [2, 2, 2]
    shape, _ = oracle.zone_plan(vs, None, eps=0.0, map_exponent=4.0)
    assert oracle.unpack_shape(shape)[0][0] == 1          # T edge 2, the pool's minimum


@pytest.mark.parametrize("edges", [(4, 8, 8), (4, 4, 4), (2, 8, 8), (8, 4, 4)])
def test_fixed_shape(edges):
    """Fixed-shape baseline: every zone takes the given shape; the permutation is then the
    regular tiling of each zone into bT x bH x bW boxes."""
    T, H, W = 16, 16, 8
    code = (int(math.log2(edges[0])) << 4) | (int(math.log2(edges[1])) << 2) | int(
        math.log2(edges[2]))
    v = rng0.normal(size=(T * H * W, 4))
    vs = oracle.zone_stats(T, H, W, v)
    shape, diag = oracle.zone_plan(vs, None, fixed_shape=code)
    assert np.all(shape == code)
    assert np.all(diag[:, 10] == 1e300)
    perm, inv, bstart, bsize, bof = oracle.permutation(T, H, W, shape)
    B = edges[0] * edges[1] * edges[2]
    assert np.all(bsize == B) and len(bsize) == T * H * W // B
    t, h, w = coords(T, H, W)
    for b in range(len(bsize)):
        toks = perm[bstart[b]:bstart[b] + B]
        for ax, e in zip((t, h, w), edges):
            c = ax[toks]
            assert c.max() - c.min() == e - 1 and c.min() % e == 0


def test_fixed_shape_rejects_bad_codes():
    vs = np.ones((1, 4))
    for bad in ((1 << 4) | (1 << 2) | 1, (3 << 4) | (3 << 2) | 3):   # 8 tokens; 512 tokens
        with pytest.raises(ValueError):
            oracle.zone_plan(vs, None, fixed_shape=bad)


@pytest.mark.parametrize("frac", [0.05, 0.15, 0.25])
def test_topk_as_fraction(frac):
    """Top-k as a sparsity: with p = 0 every row keeps exactly ceil(frac * Nb) blocks, the
    ones a brute-force sort ranks first (relevance descending, index ascending)."""
    nb = 57
    P = rng0.dirichlet(np.ones(nb), size=nb)
    k = oracle.topk_of(nb, 0, frac)
    assert k == math.ceil(np.float32(frac) * nb)
    count, cols, _ = oracle.select(P, k, 0.0)
    for i in range(nb):
        order = sorted(range(nb), key=lambda j: (-P[i, j], j))
        assert count[i] == k
        assert sorted(cols[i, :k]) == sorted(order[:k])


# ----------------------------------------------------------------------------- A2V norm field

def test_row_norms_closed_forms():
    C = 12
    x = np.zeros((4, C))
    x[0, 5] = -2.5                       # one nonzero entry: its magnitude
    x[1, :] = 3.0                        # constant row: |c| sqrt(C)
    x[2, 0], x[2, 7] = 3.0, 4.0          # Pythagorean pair
    u = rng0.normal(size=C)
    x[3] = 7.0 * u / np.sqrt(np.sum(u * u))  # scaled unit vector
    np.testing.assert_allclose(oracle.row_norms(x), [2.5, 3.0 * math.sqrt(C), 5.0, 7.0],
                               rtol=1e-14)
    np.testing.assert_allclose(oracle.row_norms(x, rows=[2, 0]), [5.0, 2.5], rtol=1e-14)
