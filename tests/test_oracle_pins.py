"""Pins for the CPU oracle against things other than itself (runs on CPU).

Each check ties the oracle to an independent source of truth:
  - library routines for the same operation: torch CPU conv2d in float64 and
    its autograd gradients (any stride/pad/dilation/groups), scipy's 2-D
    correlation (groups=1, stride 1), numpy matmul for the Linear cases;
  - brute force on tiny inputs: the dense unfold matrix A of x -> y, with
    y = A x and gradInput = A^T dy, and the matrix of w -> y for gradWeight;
  - closed forms and values the pages fix (tests/golden/*.json);
  - identities: per-group narrowing, bias closed forms, adjoints, fp64 central
    differences, one-hot probes, integer probes (exact).
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from cases import asym_descs, conv_kwargs, random_descs, tensors
from grouped_convolution_amd.workloads import draw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_all(x, w, b, dy, kw):
    """y, gradInput, gradWeight, gradBias from torch CPU float64."""
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    bt = None if b is None else torch.tensor(b, dtype=torch.float64, requires_grad=True)
    y = F.conv2d(xt, wt, bt, **kw)
    if dy is None:
        return y.detach().numpy(), None, None, None
    g = torch.autograd.grad(y, [t for t in (xt, wt, bt) if t is not None],
                            grad_outputs=torch.tensor(dy, dtype=torch.float64))
    gb = g[2].numpy() if bt is not None else None
    return y.detach().numpy(), g[0].numpy(), g[1].numpy(), gb


def close(val, ref, mag, rel=1e-12, abs_=1e-15):
    return np.all(np.abs(val - ref) <= rel * mag + abs_)


def run_oracle_all(x, w, b, dy, kw):
    y, ya = oracle.fwd(x, w, b, **kw)
    dx, dxa = oracle.bwd_data(dy, w, x.shape, **kw)
    dw, dwa = oracle.bwd_filter(x, dy, w.shape, **kw)
    db, dba = oracle.bwd_bias(dy)
    return (y, ya), (dx, dxa), (dw, dwa), (db, dba)


# --------------------------------------------------------------------------- library pins

def check_against_torch(d, seed, dist=("normal", 1.0)):
    kw = conv_kwargs(d)
    x, w, b = tensors(d, seed, dist)
    y_t, _, _, _ = torch_all(x, w, b, None, kw)
    dy = draw(dist, y_t.shape, seed + 3)
    y_t, dx_t, dw_t, db_t = torch_all(x, w, b, dy, kw)
    assert oracle.output_dims(d["N"], d["C"], d["H"], d["W"], d["K"], d["kh"], d["kw"], **kw) \
        == y_t.shape[2:]
    (y, ya), (dx, dxa), (dw, dwa), (db, dba) = run_oracle_all(x, w, b, dy, kw)
    ok = {"fwd": close(y, y_t, ya), "bwd_data": close(dx, dx_t, dxa),
          "bwd_filter": close(dw, dw_t, dwa), "bwd_bias": close(db, db_t, dba)}
    return ok


@pytest.mark.parametrize("seed", range(6))
def test_oracle_matches_torch_conv2d_random(seed):
    for d in random_descs(100 + seed, 12):
        ok = check_against_torch(d, 7000 + seed)
        assert all(ok.values()), (d, ok)


def test_oracle_matches_scipy_correlate():
    from scipy.signal import correlate2d
    rng = np.random.default_rng(5)
    for (C, H, W, kh, kw, p) in [(1, 7, 5, 3, 2, 0), (3, 6, 6, 3, 3, 1), (2, 5, 8, 2, 4, 2)]:
        x = rng.standard_normal((1, C, H, W))
        w = rng.standard_normal((2, C, kh, kw))
        y, _ = oracle.fwd(x, w, padding=p)
        xp = np.pad(x[0], ((0, 0), (p, p), (p, p)))
        for k in range(2):
            ref = sum(correlate2d(xp[c], w[k, c], mode="valid") for c in range(C))
            np.testing.assert_allclose(y[0, k], ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- brute force

def unfold_matrix(d, w):
    """Dense A with y.ravel() = A @ x.ravel() (bias-free), built tap by tap."""
    N, C, H, W, K = d["N"], d["C"], d["H"], d["W"], d["K"]
    G = d["G"]
    Cg, Kg = C // G, K // G
    Ho = (H + 2 * d["ph"] - d["dh"] * (d["kh"] - 1) - 1) // d["sh"] + 1
    Wo = (W + 2 * d["pw"] - d["dw"] * (d["kw"] - 1) - 1) // d["sw"] + 1
    A = np.zeros((N * K * Ho * Wo, N * C * H * W))
    wmap = np.zeros((N * K * Ho * Wo, w.size))   # y.ravel() = wmap(x) @ w.ravel()
    return A, wmap, (Ho, Wo), (Cg, Kg)


def brute_force_matrices(d, x, w):
    A, B, (Ho, Wo), (Cg, Kg) = unfold_matrix(d, w)
    N, C, H, W, K = d["N"], d["C"], d["H"], d["W"], d["K"]
    for n in range(N):
        for k in range(K):
            for oh in range(Ho):
                for ow in range(Wo):
                    row = ((n * K + k) * Ho + oh) * Wo + ow
                    for c in range(Cg):
                        cin = (k // Kg) * Cg + c
                        for i in range(d["kh"]):
                            for j in range(d["kw"]):
                                ih = oh * d["sh"] + i * d["dh"] - d["ph"]
                                iw = ow * d["sw"] + j * d["dw"] - d["pw"]
                                if 0 <= ih < H and 0 <= iw < W:
                                    col = ((n * C + cin) * H + ih) * W + iw
                                    widx = ((k * Cg + c) * d["kh"] + i) * d["kw"] + j
                                    A[row, col] += w.ravel()[widx]
                                    B[row, widx] += x.ravel()[col]
    return A, B, (Ho, Wo)


@pytest.mark.parametrize("seed", range(4))
def test_oracle_matches_unfold_brute_force(seed):
    for d in random_descs(300 + seed, 6, max_hw=6, max_k=3, max_cg=2, max_kg=2, max_n=2):
        x, w, b = tensors(d, 9000 + seed, bias=False)
        A, B, (Ho, Wo) = brute_force_matrices(d, x.astype(np.float64), w.astype(np.float64))
        dy = draw(("normal", 1.0), (d["N"], d["K"], Ho, Wo), 9100 + seed)
        kw = conv_kwargs(d)
        (y, ya), (dx, dxa), (dw, dwa), _ = run_oracle_all(x, w, None, dy, kw)
        assert close(y.ravel(), A @ x.ravel().astype(np.float64), ya.ravel())
        assert close(dx.ravel(), A.T @ dy.ravel().astype(np.float64), dxa.ravel())
        assert close(dw.ravel(), B.T @ dy.ravel().astype(np.float64), dwa.ravel())


# --------------------------------------------------------------------------- what the pages fix

def test_golden_shapes():
    g = json.load(open(os.path.join(GOLDEN, "shapes.json")))
    for e in g["output_dims"]:
        assert oracle.output_dims(e["N"], e["C"], e["H"], e["W"], e["K"], e["kh"], e["kw"],
                                  e["stride"], e["pad"], e["dil"], e["groups"]) \
            == (e["Ho"], e["Wo"]), e
    for e in g["weight_planes"]:
        # A weight of K x (C/G) planes is accepted; the full K x C count is not (G > 1).
        C, K, G = e["C"], e["K"], e["groups"]
        w = np.zeros((K, C // G, 1, 1))
        assert w.shape[0] * w.shape[1] == e["planes"]
        oracle.fwd(np.zeros((1, C, 2, 2)), w, groups=G)
        if G > 1:
            with pytest.raises(oracle.OracleError):
                oracle.fwd(np.zeros((1, C, 2, 2)), np.zeros((K, C, 1, 1)), groups=G)


def test_golden_output_dims_more():
    # stride / dilation / invalid cases (floor rule; kernel larger than the padded input).
    assert oracle.output_dims(1, 1, 7, 7, 1, 3, 3, 2, 1, 1) == (4, 4)
    assert oracle.output_dims(1, 1, 7, 7, 1, 3, 3, 1, 0, 2) == (3, 3)
    assert oracle.output_dims(1, 1, 8, 5, 1, 2, 3, (3, 2), (1, 0), (1, 2)) == (3, 1)
    for bad in [dict(kh=8), dict(stride=0), dict(dilation=0), dict(padding=-1),
                dict(groups=3), dict(N=-1)]:
        args = dict(N=1, C=4, H=7, W=7, K=4, kh=3, kw=3, stride=1, padding=0, dilation=1,
                    groups=2)
        args.update(bad)
        with pytest.raises(oracle.OracleError):
            oracle.output_dims(**args)


def test_golden_fc_all_ones_closed_form():
    """The all-ones fully-connected problem of the cudnn.torch issue, at full size,
    on sampled elements: every value is the integer closed form, exactly."""
    g = json.load(open(os.path.join(GOLDEN, "fc_all_ones.json")))
    x = np.ones(g["x_shape"])
    w = np.ones(g["w_shape"])
    b = np.ones(g["w_shape"][0])
    dy = np.ones(g["dy_shape"])
    rng = np.random.default_rng(0)
    ex = g["expected"]
    y, _ = oracle.fwd(x, w, b, idx=rng.integers(0, dy.size, 64))
    assert np.all(y == ex["output"])
    dx, _ = oracle.bwd_data(dy, w, x.shape, idx=rng.integers(0, x.size, 64))
    assert np.all(dx == ex["gradInput"])
    dw, _ = oracle.bwd_filter(x, dy, w.shape, idx=rng.integers(0, w.size, 64))
    assert np.all(dw == ex["gradWeight"])
    db, _ = oracle.bwd_bias(dy)
    assert np.all(db == ex["gradBias"])


def test_golden_linear_1x1():
    """1x1 convolution on a 1x1 input equals Linear on the flattened input."""
    g = json.load(open(os.path.join(GOLDEN, "linear_1x1.json")))
    rng = np.random.default_rng(1)
    x = rng.standard_normal(g["x_shape"])
    w = rng.standard_normal(g["w_shape"])
    b = rng.standard_normal(g["w_shape"][0])
    y, _ = oracle.fwd(x, w, b)
    lin = x.reshape(x.shape[0], -1) @ w.reshape(w.shape[0], -1).T + b
    assert np.max(np.abs(y.reshape(lin.shape) - lin)) <= g["bound_max_abs_diff"]


def test_fc_mode_equals_linear_at_full_shape():
    """Kernel == input (the fully-connected problem shape, random data): the
    convolution and its gradients equal the Linear layer's, on sampled elements."""
    rng = np.random.default_rng(2)
    N, C, H, W, K = 1600, 256, 6, 6, 4096
    x = rng.standard_normal((N, C, H, W)).astype(np.float32)
    w = (rng.standard_normal((K, C, H, W)) * (1 / 96)).astype(np.float32)
    b = rng.standard_normal(K).astype(np.float32)
    dy = rng.standard_normal((N, K, 1, 1)).astype(np.float32)
    X = x.reshape(N, -1).astype(np.float64)
    Wm = w.reshape(K, -1).astype(np.float64)
    D = dy.reshape(N, K).astype(np.float64)
    iy = rng.integers(0, N * K, 48)
    y, ya = oracle.fwd(x, w, b, idx=iy)
    n, k = np.divmod(iy, K)
    ref = np.einsum("ij,ij->i", X[n], Wm[k]) + b[k]
    assert close(y, ref, ya)
    ix = rng.integers(0, x.size, 48)
    dx, dxa = oracle.bwd_data(dy, w, x.shape, idx=ix)
    n, dd = np.divmod(ix, C * H * W)
    assert close(dx, np.einsum("ij,ji->i", D[n], Wm[:, dd]), dxa)
    iw = rng.integers(0, w.size, 48)
    dw, dwa = oracle.bwd_filter(x, dy, w.shape, idx=iw)
    k, dd = np.divmod(iw, C * H * W)
    assert close(dw, np.einsum("ji,ji->i", D[:, k], X[:, dd]), dwa)


# --------------------------------------------------------------------------- identities

def test_group_narrowing_equals_per_group_convs():
    """Every op on a grouped problem equals G independent groups=1 problems on
    narrowed slices (the clnn issue's narrow() draft, with the weight rows of
    group g being output planes g*Kg..(g+1)*Kg-1)."""
    for d in random_descs(500, 10, max_g=4):
        if d["G"] == 1:
            continue
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 600)
        G, Cg, Kg = d["G"], d["C"] // d["G"], d["K"] // d["G"]
        y, _ = oracle.fwd(x, w, b, **kw)
        dy = draw(("normal", 1.0), y.shape, 601)
        dx, _ = oracle.bwd_data(dy, w, x.shape, **kw)
        dw, _ = oracle.bwd_filter(x, dy, w.shape, **kw)
        kw1 = dict(kw, groups=1)
        for g in range(G):
            xs, ws, bs = x[:, g * Cg:(g + 1) * Cg], w[g * Kg:(g + 1) * Kg], b[g * Kg:(g + 1) * Kg]
            dys = dy[:, g * Kg:(g + 1) * Kg]
            assert np.array_equal(oracle.fwd(xs, ws, bs, **kw1)[0], y[:, g * Kg:(g + 1) * Kg])
            assert np.array_equal(oracle.bwd_data(dys, ws, xs.shape, **kw1)[0],
                                  dx[:, g * Cg:(g + 1) * Cg])
            assert np.array_equal(oracle.bwd_filter(xs, dys, ws.shape, **kw1)[0],
                                  dw[g * Kg:(g + 1) * Kg])


def test_bias_closed_forms():
    for d in random_descs(700, 8):
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 701)
        y1, _ = oracle.fwd(x, w, b, **kw)
        y0, _ = oracle.fwd(x, w, None, **kw)
        diff = y1 - y0
        np.testing.assert_allclose(diff, np.broadcast_to(b[None, :, None, None], y1.shape),
                                   rtol=0, atol=1e-12 * (1 + np.abs(y0).max()))
        dy = draw(("normal", 1.0), y1.shape, 702)
        db, dba = oracle.bwd_bias(dy)
        assert close(db, dy.astype(np.float64).sum(axis=(0, 2, 3)), dba)


def test_adjoint_identities():
    """<fwd(x,w), dy> = <x, bwd_data(dy,w)> = <w, bwd_filter(x,dy)> (bias-free)."""
    for d in random_descs(800, 16):
        kw = conv_kwargs(d)
        x, w, _ = tensors(d, 801, bias=False)
        y, _ = oracle.fwd(x, w, **kw)
        dy = draw(("normal", 1.0), y.shape, 802)
        dx, _ = oracle.bwd_data(dy, w, x.shape, **kw)
        dw, _ = oracle.bwd_filter(x, dy, w.shape, **kw)
        a = np.vdot(y, dy)
        bnd = 1e-12 * (np.vdot(np.abs(y), np.abs(dy)) + 1e-300) + 1e-13
        scale = np.abs(x).ravel() @ np.abs(dx).ravel() + np.abs(w).ravel() @ np.abs(dw).ravel()
        bnd = max(bnd, 1e-12 * scale)
        assert abs(a - np.vdot(x.astype(np.float64), dx)) <= bnd, d
        assert abs(a - np.vdot(w.astype(np.float64), dw)) <= bnd, d


def test_finite_differences_fp64():
    """L(x, w, b) = <fwd(x, w, b), dy> is linear in each argument, so fp64
    central differences equal the gradients up to rounding."""
    rng = np.random.default_rng(900)
    for d in random_descs(901, 4):
        kw = conv_kwargs(d)
        x, w, b = (a.astype(np.float64) for a in tensors(d, 902))
        y, _ = oracle.fwd(x, w, b, **kw)
        dy = rng.standard_normal(y.shape)
        dx, _ = oracle.bwd_data(dy, w, x.shape, **kw)
        dw, _ = oracle.bwd_filter(x, dy, w.shape, **kw)
        db, _ = oracle.bwd_bias(dy)

        def L(xx, ww, bb):
            return np.vdot(oracle.fwd(xx, ww, bb, **kw)[0], dy)

        h = 0.5
        for arr, grad, which in ((x, dx, 0), (w, dw, 1), (b, db, 2)):
            for _ in range(24):
                t = tuple(int(rng.integers(0, s)) for s in arr.shape)
                args_p = [x.copy(), w.copy(), b.copy()]
                args_m = [x.copy(), w.copy(), b.copy()]
                args_p[which][t] += h
                args_m[which][t] -= h
                fd = (L(*args_p) - L(*args_m)) / (2 * h)
                assert abs(fd - grad[t]) <= 1e-9 * (1 + abs(grad[t]) + np.abs(y).sum()), \
                    (d, which, t, fd, grad[t])


def test_one_hot_probes_and_group_isolation():
    """A single 1 in x and a single 1 in w give y = 1 exactly where that tap
    reads that pixel and 0 everywhere else; a probe in group g leaves all
    other groups' outputs zero."""
    for d in random_descs(1000, 20, max_g=3):
        kw = conv_kwargs(d)
        rng = np.random.default_rng(1001)
        G, Cg, Kg = d["G"], d["C"] // d["G"], d["K"] // d["G"]
        x = np.zeros((d["N"], d["C"], d["H"], d["W"]))
        w = np.zeros((d["K"], Cg, d["kh"], d["kw"]))
        n, ca, h, ww = (int(rng.integers(0, s)) for s in x.shape)
        k, c, i, j = (int(rng.integers(0, s)) for s in w.shape)
        x[n, ca, h, ww] = 1
        w[k, c, i, j] = 1
        y, _ = oracle.fwd(x, w, **kw)
        expect = np.zeros_like(y)
        if k // Kg == ca // Cg and c == ca % Cg:
            for oh in range(y.shape[2]):
                for ow in range(y.shape[3]):
                    if oh * d["sh"] - d["ph"] + i * d["dh"] == h and \
                            ow * d["sw"] - d["pw"] + j * d["dw"] == ww:
                        expect[n, k, oh, ow] = 1
        assert np.array_equal(y, expect), d
        other = [kk for kk in range(d["K"]) if kk // Kg != ca // Cg]
        assert np.all(y[:, other] == 0)


def test_integer_probes_exact():
    """Integer data in [-3, 3]: all products and partial sums are exact, so the
    oracle equals torch's float64 conv and gradients bit for bit."""
    for d in random_descs(1100, 16, max_cg=4, max_kg=4):
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 1101, dist=("int", -3, 3))
        y_t, _, _, _ = torch_all(x, w, b, None, kw)
        dy = draw(("int", -3, 3), y_t.shape, 1102)
        y_t, dx_t, dw_t, db_t = torch_all(x, w, b, dy, kw)
        (y, _), (dx, _), (dw, _), (db, _) = run_oracle_all(x, w, b, dy, kw)
        assert np.array_equal(y, y_t) and np.array_equal(dx, dx_t)
        assert np.array_equal(dw, dw_t) and np.array_equal(db, db_t)


def test_sampled_indices_match_full():
    d = random_descs(1200, 1)[0]
    kw = conv_kwargs(d)
    x, w, b = tensors(d, 1201)
    y, ya = oracle.fwd(x, w, b, **kw)
    idx = np.arange(y.size)[::3]
    v, a = oracle.fwd(x, w, b, idx=idx, **kw)
    assert np.array_equal(v, y.ravel()[idx]) and np.array_equal(a, ya.ravel()[idx])
    with pytest.raises(oracle.OracleError):
        oracle.fwd(x, w, b, idx=[y.size], **kw)


def test_abs_sum_is_sum_of_abs_products():
    """A_e with all-nonnegative data equals the value itself."""
    d = dict(N=2, C=4, H=5, W=6, K=6, kh=3, kw=2, sh=1, sw=2, ph=1, pw=0, dh=1, dw=1, G=2)
    kw = conv_kwargs(d)
    x, w, b = tensors(d, 1300, dist=("uniform",))
    y, ya = oracle.fwd(x, w, b, **kw)
    np.testing.assert_allclose(ya, y, rtol=1e-14)
    # and flips sign-insensitively
    y2, ya2 = oracle.fwd(-x, w, b, **kw)
    np.testing.assert_allclose(ya2, ya, rtol=1e-14)


def torch_abs_sums(x, w, b, dy, d):
    """Per-element sums of |product| from torch CPU float64, independently of the
    oracle: each op's terms with every factor replaced by its absolute value.
    The forward map is linear in x and in w, so
      fwd:        conv2d(|x|, |w|) + |b|
      bwd_data:   d<conv2d(x, |w|), |dy|>/dx   (= sum of |w|*|dy| over the taps that read x)
      bwd_filter: d<conv2d(|x|, w), |dy|>/dw   (= sum of |dy|*|x| over the pixels)
      bwd_bias:   |dy| summed over images and pixels.
    The padding is applied to the input explicitly (F.pad), so the end pads may
    differ from the start pads."""
    pad = (d["pw"], d.get("pr", d["pw"]), d["ph"], d.get("pb", d["ph"]))
    conv = dict(stride=(d["sh"], d["sw"]), dilation=(d["dh"], d["dw"]), groups=d["G"])
    f64 = lambda a: torch.tensor(np.abs(a), dtype=torch.float64)
    xa, wa, dya = f64(x), f64(w), f64(dy)
    ya = F.conv2d(F.pad(xa, pad), wa, None if b is None else f64(b), **conv)
    xv = torch.zeros_like(xa, requires_grad=True)
    (dxa,) = torch.autograd.grad((F.conv2d(F.pad(xv, pad), wa, **conv) * dya).sum(), [xv])
    wv = torch.zeros_like(wa, requires_grad=True)
    (dwa,) = torch.autograd.grad((F.conv2d(F.pad(xa, pad), wv, **conv) * dya).sum(), [wv])
    return ya.numpy(), dxa.numpy(), dwa.numpy(), dya.sum(dim=(0, 2, 3)).numpy()


@pytest.mark.parametrize("seed", range(3))
def test_abs_sums_match_torch(seed):
    """A_e, the scale of every tolerance bound, is pinned for all four ops: the
    oracle's per-element sums of |product| (forward with |bias|, as the bias add
    rounds too) equal torch float64 on absolute values, on random descriptors
    with symmetric and asymmetric padding, strides and dilations, and the bias
    sum of |dy| ("Pointwise Broadcast Reduce", DLPrimitives Blog: gradBias sums
    dy over images and pixels)."""
    descs = random_descs(60 + seed, 10) + asym_descs(70 + seed, 6)
    for t, d in enumerate(descs):
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 8000 + 10 * seed + t)
        pad = (d["pw"], d.get("pr", d["pw"]), d["ph"], d.get("pb", d["ph"]))
        y_shape = F.conv2d(F.pad(torch.tensor(x, dtype=torch.float64), pad),
                           torch.tensor(w, dtype=torch.float64), stride=kw["stride"],
                           dilation=kw["dilation"], groups=d["G"]).shape
        dy = draw(("normal", 1.0), tuple(y_shape), 8500 + 10 * seed + t)
        ya_t, dxa_t, dwa_t, dba_t = torch_abs_sums(x, w, b, dy, d)
        (_, ya), (_, dxa), (_, dwa), (_, dba) = run_oracle_all(x, w, b, dy, kw)
        for name, got, want in (("fwd", ya, ya_t), ("bwd_data", dxa, dxa_t),
                                ("bwd_filter", dwa, dwa_t), ("bwd_bias", dba, dba_t)):
            assert got.shape == want.shape, (name, d)
            assert np.allclose(got, want, rtol=1e-12, atol=1e-14), (name, d)


def test_empty_batch():
    """N = 0 is a valid descriptor: empty y and gradInput, zero gradWeight and
    gradBias (sums over no terms), as torch's float64 conv gives."""
    d = dict(N=0, C=6, H=5, W=4, K=4, kh=3, kw=2, sh=1, sw=1, ph=1, pw=0, dh=1, dw=1, G=2)
    kw = conv_kwargs(d)
    x, w, b = tensors(d, 1400)
    y_t, _, _, _ = torch_all(x, w, b, None, kw)
    dy = np.zeros(y_t.shape, np.float32)
    _, dx_t, dw_t, db_t = torch_all(x, w, b, dy, kw)
    (y, _), (dx, _), (dw, _), (db, _) = run_oracle_all(x, w, b, dy, kw)
    assert y.shape == y_t.shape and dx.shape == dx_t.shape == x.shape
    assert np.array_equal(dw, dw_t) and np.all(dw == 0)
    assert np.array_equal(db, db_t) and np.all(db == 0)


@pytest.mark.parametrize("seed", range(3))
def test_relu_epilogue_matches_torch(seed):
    """The forward pass with the ReLU epilogue equals torch's relu(conv2d(x, w, b))
    in float64 on random descriptors (bias added before the activation)."""
    for d in random_descs(40 + seed, 6):
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 4000 + seed)
        want = torch.relu(F.conv2d(torch.tensor(x, dtype=torch.float64),
                                   torch.tensor(w, dtype=torch.float64),
                                   torch.tensor(b, dtype=torch.float64), **kw)).numpy()
        got, _ = oracle.fwd(x, w, b, relu=True, **kw)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12), d


def test_relu_epilogue_invariants():
    """relu(y) - relu(-y) = y exactly (the negated output comes from negating w
    and b, the forward pass being linear in them); nonnegative inputs leave the
    output unchanged; nonnegative x with nonpositive w and b gives exact zeros."""
    for d in random_descs(50, 6):
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 4100)
        y, _ = oracle.fwd(x, w, b, **kw)
        pos, _ = oracle.fwd(x, w, b, relu=True, **kw)
        neg, _ = oracle.fwd(x, -w, -b, relu=True, **kw)
        assert np.array_equal(pos - neg, y), d
        ax, aw, ab = np.abs(x), np.abs(w), np.abs(b)
        assert np.array_equal(oracle.fwd(ax, aw, ab, relu=True, **kw)[0], oracle.fwd(ax, aw, ab, **kw)[0])
        assert not np.any(oracle.fwd(ax, -aw, -ab, relu=True, **kw)[0])


# --------------------------------------------------------------------------- asymmetric padding

def _pad_input(x, d):
    return np.pad(x, ((0, 0), (0, 0), (d["ph"], d["pb"]), (d["pw"], d["pr"])))


@pytest.mark.parametrize("seed", range(3))
def test_asymmetric_padding_equals_explicit_zero_pad(seed):
    """Start and end padding that differ (DLPrimitives Blog, "TensorFlow": what
    TensorFlow does by padding the input by hand) equal the unpadded convolution of
    the input padded with those zero rows and columns: same forward output (and
    magnitudes), same gradWeight, and gradInput is the padded input's gradInput
    with the padding cut away. Skipped taps and added zeros leave every fp64 sum
    unchanged, so the equality is exact."""
    for d in asym_descs(300 + seed, 12):
        kw = conv_kwargs(d)
        kw0 = dict(kw, padding=0)
        x, w, b = tensors(d, 5000 + seed)
        xp = _pad_input(x, d)
        y, ya = oracle.fwd(x, w, b, **kw)
        y0, y0a = oracle.fwd(xp, w, b, **kw0)
        assert np.array_equal(y, y0) and np.array_equal(ya, y0a), d
        dy = draw(("normal", 1.0), y.shape, 5003 + seed)
        dx, _ = oracle.bwd_data(dy, w, x.shape, **kw)
        dx0, _ = oracle.bwd_data(dy, w, xp.shape, **kw0)
        assert np.array_equal(dx, dx0[:, :, d["ph"]:d["ph"] + d["H"], d["pw"]:d["pw"] + d["W"]]), d
        dw, _ = oracle.bwd_filter(x, dy, w.shape, **kw)
        dw0, _ = oracle.bwd_filter(xp, dy, w.shape, **kw0)
        assert np.array_equal(dw, dw0), d


@pytest.mark.parametrize("seed", range(2))
def test_asymmetric_padding_matches_torch(seed):
    """torch CPU float64: conv2d of F.pad(x, (left, right, top, bottom)) and its
    autograd gradients (through the pad) against the oracle with end padding."""
    for d in asym_descs(400 + seed, 10):
        kw = conv_kwargs(d)
        x, w, b = tensors(d, 6000 + seed)
        xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        wt = torch.tensor(w, dtype=torch.float64, requires_grad=True)
        bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
        yt = F.conv2d(F.pad(xt, (d["pw"], d["pr"], d["ph"], d["pb"])), wt, bt, stride=kw["stride"],
                      dilation=kw["dilation"], groups=d["G"])
        dy = draw(("normal", 1.0), tuple(yt.shape), 6003 + seed)
        gx, gw, gb = torch.autograd.grad(yt, [xt, wt, bt], torch.tensor(dy, dtype=torch.float64))
        (y, ya), (dx, dxa), (dw, dwa), (db, dba) = run_oracle_all(x, w, b, dy, kw)
        assert y.shape == tuple(yt.shape), d
        assert close(y, yt.detach().numpy(), ya) and close(dx, gx.numpy(), dxa), d
        assert close(dw, gw.numpy(), dwa) and close(db, gb.numpy(), dba), d


def test_asymmetric_padding_output_extents():
    """Ho = floor((H + top + bottom - d(k-1) - 1)/s) + 1 by counting, for every
    start and end padding up to 3: the number of window origins h0 = ho*s - top
    whose last tap h0 + d(k-1) stays below H + bottom."""
    for H in range(1, 12):
        for k in range(1, 5):
            for s_ in (1, 2, 3):
                for dil in (1, 2):
                    for top in range(4):
                        for bot in range(4):
                            count = sum(1 for ho in range(64)
                                        if ho * s_ - top + dil * (k - 1) < H + bot)
                            try:
                                got = oracle.output_dims(1, 1, H, 1, 1, k, 1, (s_, 1),
                                                         (top, bot, 0, 0), (dil, 1), 1)[0]
                            except oracle.OracleError:
                                got = 0
                            assert got == count, (H, k, s_, dil, top, bot)
