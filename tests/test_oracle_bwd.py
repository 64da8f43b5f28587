"""Pins for the oracle's backward (gradients of L = sum(dout * out)).

* central finite differences of an independent NumPy fp64 forward (written
  here, per slot: g = G x, u = U x, h = SiLU(g) u, y = W2 h, out = sum w y)
  for entries of x, the top-k weights, gate, up and w2, against the oracle
  with the h rounding off (the smooth function);
* torch autograd on the dense special case E = 1, k = 1, w = 1 (a SwiGLU MLP)
  in fp64;
* exact invariants: a weight-0 slot adds nothing to dx or the weight
  gradients (its dw is still <dout, y>), a skipped slot has dw = 0, doubling
  dout doubles every gradient, and a transposed x equals the contiguous copy.
"""
import numpy as np
import pytest
import torch

from conftest import bits


def _case(T=3, H=16, I=8, E=3, k=2, seed=0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    gate = (torch.randn(E, I, H, generator=g) / 4).to(torch.bfloat16)
    up = (torch.randn(E, I, H, generator=g) / 4).to(torch.bfloat16)
    w2 = (torch.randn(E, H, I, generator=g) / 3).to(torch.bfloat16)
    dout = torch.randn(T, H, generator=g).to(torch.bfloat16)
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    w = (torch.rand(T, k, generator=g) + 0.1).to(torch.float32)
    return x, gate, up, w2, dout, ids.numpy(), w.numpy()


def _f64(t):
    return t.to(torch.float64).numpy()


def _np_loss(x, G, U, W2, dout, ids, w):
    """Independent forward: sum(dout * out), everything in float64."""
    L = 0.0
    for t in range(x.shape[0]):
        out = np.zeros(x.shape[1])
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if not 0 <= e < G.shape[0]:
                continue
            gg = G[e] @ x[t]
            uu = U[e] @ x[t]
            h = gg / (1.0 + np.exp(-gg)) * uu
            out += float(w[t, j]) * (W2[e] @ h)
        L += float(dout[t] @ out)
    return L


def _oracle(orc, x, gate, up, w2, dout, ids, w, round_h=False, exps=None):
    E = gate.shape[0]
    return orc.ffn_bwd(bits(x), ids, w, bits(dout), num_experts=E, gate=bits(gate), up=bits(up),
                       w2=bits(w2), exps=np.arange(E) if exps is None else exps, round_h=round_h)


def test_finite_differences_of_an_independent_forward(orc):
    x, gate, up, w2, dout, ids, w = _case()
    dx, _, dw, dG, dU, dW2 = _oracle(orc, x, gate, up, w2, dout, ids, w)
    X, G, U, W, D = _f64(x), _f64(gate), _f64(up), _f64(w2), _f64(dout)
    wf = w.astype(np.float64)
    d = 1e-5

    def fd(arr, idx, loss):
        a = arr.copy()
        a[idx] += d
        lp = loss(a)
        a[idx] -= 2 * d
        lm = loss(a)
        return (lp - lm) / (2 * d)

    rng = np.random.default_rng(0)
    for _ in range(6):
        t, c = rng.integers(0, X.shape[0]), rng.integers(0, X.shape[1])
        num = fd(X, (t, c), lambda a: _np_loss(a, G, U, W, D, ids, wf))
        assert abs(num - dx[t, c]) <= 1e-6 * (1 + abs(num))
    for t in range(X.shape[0]):
        for j in range(ids.shape[1]):
            num = fd(wf, (t, j), lambda a: _np_loss(X, G, U, W, D, ids, a))
            assert abs(num - dw[t, j]) <= 1e-6 * (1 + abs(num))
    for _ in range(6):
        e, i, c = (rng.integers(0, s) for s in G.shape)
        num = fd(G, (e, i, c), lambda a: _np_loss(X, a, U, W, D, ids, wf))
        assert abs(num - dG[e, i, c]) <= 1e-6 * (1 + abs(num))
        num = fd(U, (e, i, c), lambda a: _np_loss(X, G, a, W, D, ids, wf))
        assert abs(num - dU[e, i, c]) <= 1e-6 * (1 + abs(num))
        e, n, i = (rng.integers(0, s) for s in W.shape)
        num = fd(W, (e, n, i), lambda a: _np_loss(X, G, U, a, D, ids, wf))
        assert abs(num - dW2[e, n, i]) <= 1e-6 * (1 + abs(num))


def test_dense_swiglu_matches_torch_autograd(orc):
    x, gate, up, w2, dout, _, _ = _case(T=5, H=32, I=16, E=1, k=1, seed=3)
    ids = np.zeros((5, 1), dtype=np.int32)
    w = np.ones((5, 1), dtype=np.float32)
    dx, _, dw, dG, dU, dW2 = _oracle(orc, x, gate, up, w2, dout, ids, w)
    X = torch.tensor(_f64(x), requires_grad=True)
    G = torch.tensor(_f64(gate[0]), requires_grad=True)
    U = torch.tensor(_f64(up[0]), requires_grad=True)
    W = torch.tensor(_f64(w2[0]), requires_grad=True)
    out = (torch.nn.functional.silu(X @ G.T) * (X @ U.T)) @ W.T
    (out * torch.tensor(_f64(dout))).sum().backward()
    assert np.allclose(dx, X.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dG[0], G.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dU[0], U.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dW2[0], W.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dw[:, 0], (out * torch.tensor(_f64(dout))).sum(1).detach().numpy(), rtol=1e-12)


def test_exact_invariants(orc):
    x, gate, up, w2, dout, ids, w = _case(T=4, H=32, I=16, E=4, k=2, seed=5)
    base = _oracle(orc, x, gate, up, w2, dout, ids, w, round_h=True)
    w0 = w.copy()
    w0[1, 0] = 0.0
    zero = _oracle(orc, x, gate, up, w2, dout, ids, w0, round_h=True)
    ids_s = ids.copy()
    ids_s[1, 0] = -1
    skip = _oracle(orc, x, gate, up, w2, dout, ids_s, w0, round_h=True)
    assert np.array_equal(zero[0], skip[0])                       # dx
    for a, b in zip(zero[3:], skip[3:]):                          # weight gradients
        assert np.array_equal(a, b)
    assert zero[2][1, 0] == base[2][1, 0] != 0.0                  # dw of the weight-0 slot
    assert skip[2][1, 0] == 0.0
    twice = _oracle(orc, x, gate, up, w2, (dout.float() * 2).to(torch.bfloat16), ids, w, round_h=True)
    for a, b in zip(twice[:1] + twice[2:], base[:1] + base[2:]):
        assert np.array_equal(a, 2 * b)
    xt = x.t().contiguous().t()
    tr = _oracle(orc, xt, gate, up, w2, dout, ids, w, round_h=True)
    for a, b in zip(tr, base):
        assert np.array_equal(a, b)
