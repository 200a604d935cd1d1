"""Pins that tie the oracle's backward pass (oracle.attention_bwd) to facts
that do not come from the oracle itself.

The pages print no formula for the gradients (page "解释FlashAttention的显存
优化原理" §一.2(2) only says the backward pass recomputes the forward's
blocks), so the gradients are fixed by the forward pass they differentiate:

  * central finite differences of the (separately pinned) forward oracle;
  * closed forms: one key (dQ = dK = 0, dV = sum of dO), two keys (logistic
    weights), constant values (dQ = dK = 0);
  * sum rules implied by invariances of the forward pass: rows of P sum to
    one (sum_j dV_j = sum_i dO_i), a shift added to every key leaves O
    unchanged (sum_j dK_j = 0), and q -> t q, k -> k / t leaves O unchanged
    (sum_i <q_i, dQ_i> = sum_j <k_j, dK_j>);
  * an independent formulation (torch fp64 autograd through softmax on the
    CPU), row sampling, and the magnitude sums as upper bounds.

Each ``pin_*`` takes a loaded oracle library and raises AssertionError on a
mismatch; test_oracle_mutations.py runs the battery against planted mistakes.
"""
from __future__ import annotations

import numpy as np

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"


def _inputs(seed, B, H, Nq, Nk, D, std=1.0):
    r = _rng(seed)
    q = r.standard_normal((B, H, Nq, D)) * std
    k = r.standard_normal((B, H, Nk, D)) * std
    v = r.standard_normal((B, H, Nk, D))
    g = r.standard_normal((B, H, Nq, D))
    return q, k, v, g


# ---------------------------------------------------------------------------
def pin_bwd_finite_differences(lib):
    """Every gradient entry against a central difference of sum(dO * O)."""
    h = 1e-5
    for seed, (B, H, Nq, Nk, D, causal, scale) in enumerate([
            (1, 2, 5, 5, 3, False, 0.7), (1, 1, 6, 6, 4, True, 0.45),
            (2, 1, 3, 7, 2, False, -0.9), (1, 1, 7, 4, 3, True, 1.3),
            (1, 1, 4, 9, 2, True, 0.6)]):
        q, k, v, g = _inputs(100 + seed, B, H, Nq, Nk, D)
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal, lib=lib)
        base = {"q": q, "k": k, "v": v}

        def loss(**kw):
            a = dict(base)
            a.update(kw)
            o, _ = oracle.attention(a["q"], a["k"], a["v"], scale, causal, lib=lib)
            return float((o * g).sum())

        for name, grad in (("q", dq), ("k", dk), ("v", dv)):
            x = base[name]
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp = x.copy()
                xp[idx] += h
                xm = x.copy()
                xm[idx] -= h
                num[idx] = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * h)
            _close(grad, num, 1e-7, f"finite differences d{name} case {seed}")


def pin_bwd_one_key(lib):
    """Nk = 1: O_i = v_0 for every row, so dQ = dK = 0 and dV_0 = sum_i dO_i."""
    for causal in (False, True):
        q, k, v, g = _inputs(7, 2, 2, 9, 1, 5)
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.4, causal, lib=lib)
        _close(dq, np.zeros_like(dq), 1e-13, "one key dQ")
        _close(dk, np.zeros_like(dk), 1e-13, "one key dK")
        _close(dv, g.sum(axis=2, keepdims=True), 1e-12, "one key dV")


def pin_bwd_two_keys(lib):
    """Nk = 2, non-causal: O_i = a_i v_0 + (1 - a_i) v_1 with a_i the logistic
    function of scale <q_i, k_0 - k_1>; differentiate by hand."""
    q, k, v, g = _inputs(8, 1, 1, 6, 2, 4)
    scale = 0.8
    q0, k0, k1, v0, v1, g0 = q[0, 0], k[0, 0, 0], k[0, 0, 1], v[0, 0, 0], v[0, 0, 1], g[0, 0]
    a = 1.0 / (1.0 + np.exp(-scale * (q0 @ (k0 - k1))))
    c = a * (1 - a) * (g0 @ (v0 - v1))                   # d loss / d (score gap)
    dq_ref = scale * c[:, None] * (k0 - k1)[None, :]
    dk0 = scale * (c[:, None] * q0).sum(axis=0)
    dv0 = (a[:, None] * g0).sum(axis=0)
    dv1 = ((1 - a)[:, None] * g0).sum(axis=0)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, False, lib=lib)
    _close(dq[0, 0], dq_ref, 1e-12, "two keys dQ")
    _close(dk[0, 0], np.stack([dk0, -dk0]), 1e-12, "two keys dK")
    _close(dv[0, 0], np.stack([dv0, dv1]), 1e-12, "two keys dV")


def pin_bwd_constant_values(lib):
    """All v_j equal: O does not depend on q or k, so dQ = dK = 0."""
    for causal in (False, True):
        q, k, _, g = _inputs(9, 1, 2, 8, 11, 6)
        v = np.broadcast_to(_rng(10).standard_normal(6), k.shape).copy()
        dq, dk, _ = oracle.attention_bwd(q, k, v, g, 0.5, causal, lib=lib)
        _close(dq, np.zeros_like(dq), 1e-12, "constant V dQ")
        _close(dk, np.zeros_like(dk), 1e-12, "constant V dK")


def pin_bwd_sum_rules(lib):
    """Invariances of the forward pass seen through its gradients."""
    for causal, (Nq, Nk) in ((False, (13, 9)), (True, (12, 12)), (True, (9, 15)),
                             (True, (15, 9))):
        q, k, v, g = _inputs(11 + Nq, 2, 1, Nq, Nk, 8)
        scale = 0.35
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal, lib=lib)
        # keys no row can see get no gradient; the rest obey the rules
        seen = Nk if not causal else min(Nk, Nq)
        _close(dv[:, :, seen:], np.zeros_like(dv[:, :, seen:]), 0.0, "unseen keys dV")
        _close(dk[:, :, seen:], np.zeros_like(dk[:, :, seen:]), 0.0, "unseen keys dK")
        _close(dv.sum(axis=2), g.sum(axis=2), 1e-11, "sum_j dV_j = sum_i dO_i")
        _close(dk.sum(axis=2), np.zeros_like(dk.sum(axis=2)), 1e-11, "sum_j dK_j = 0")
        lhs = np.einsum("bhnd,bhnd->bh", q, dq)
        rhs = np.einsum("bhnd,bhnd->bh", k, dk)
        _close(lhs, rhs, 1e-11, "sum <q, dQ> = sum <k, dK>")


def pin_bwd_autograd_witness(lib):
    """torch fp64 autograd through softmax(scale q k^T, masked) v on the CPU."""
    import torch

    for causal, (Nq, Nk) in ((False, (10, 14)), (True, (16, 16)), (True, (11, 6))):
        q, k, v, g = _inputs(20 + Nk, 2, 2, Nq, Nk, 8)
        scale = 0.3
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        s = scale * torch.matmul(tq, tk.transpose(-1, -2).contiguous())
        if causal:
            keep = torch.arange(Nq)[:, None] >= torch.arange(Nk)[None, :]
            s = s.masked_fill(~keep, float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), tv)
        o.backward(torch.tensor(g))
        dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal, lib=lib)
        _close(dq, tq.grad.numpy(), 1e-12, "autograd dQ")
        _close(dk, tk.grad.numpy(), 1e-12, "autograd dK")
        _close(dv, tv.grad.numpy(), 1e-12, "autograd dV")


def pin_bwd_row_sampling(lib):
    """Sampled query and key rows equal the same rows of the full result."""
    B, H, Nq, Nk, D = 2, 3, 17, 13, 4
    q, k, v, g = _inputs(30, B, H, Nq, Nk, D)
    for causal in (False, True):
        full = oracle.attention_bwd(q, k, v, g, 0.5, causal, magnitudes=True, lib=lib)
        qr = np.array([0, 5, B * H * Nq - 1, 40, 17])
        kr = np.array([B * H * Nk - 1, 3, 0, 27])
        part = oracle.attention_bwd(q, k, v, g, 0.5, causal, qrows=qr, krows=kr,
                                    magnitudes=True, lib=lib)
        _close(part[0], full[0].reshape(-1, D)[qr], 0.0, "sampled dQ")
        _close(part[3], full[3].reshape(-1, D)[qr], 0.0, "sampled bQ")
        for t in (1, 2, 4, 5):
            _close(part[t], full[t].reshape(-1, D)[kr], 0.0, f"sampled key output {t}")


def pin_bwd_magnitudes(lib):
    """The magnitude sums bound the gradients and follow their definition."""
    import torch

    for causal in (False, True):
        B, H, Nq, Nk, D = 1, 2, 12, 10, 6
        q, k, v, g = _inputs(40, B, H, Nq, Nk, D)
        scale = 0.6
        dq, dk, dv, bq, bk, bv = oracle.attention_bwd(q, k, v, g, scale, causal,
                                                      magnitudes=True, lib=lib)
        for grad, bound, what in ((dq, bq, "Q"), (dk, bk, "K"), (dv, bv, "V")):
            assert np.all(bound >= np.abs(grad) - 1e-12), f"b{what} below |d{what}|"
        s = torch.tensor(scale * np.einsum("bhid,bhjd->bhij", q, k))
        if causal:
            keep = torch.arange(Nq)[:, None] >= torch.arange(Nk)[None, :]
            s = s.masked_fill(~keep, float("-inf"))
        p = torch.softmax(s, dim=-1).numpy()
        dp = np.einsum("bhid,bhjd->bhij", g, v)
        o = np.einsum("bhij,bhjd->bhid", p, v)
        rowterm = (g * o).sum(-1, keepdims=True)
        e = (np.abs(g) * np.einsum("bhij,bhjd->bhid", p, np.abs(v))).sum(-1, keepdims=True)
        w = np.abs(p * (dp - rowterm)) + p * e
        _close(bv, np.einsum("bhij,bhid->bhjd", p, np.abs(g)), 1e-12, "bV definition")
        _close(bq, scale * np.einsum("bhij,bhjd->bhid", w, np.abs(k)), 1e-12,
               "bQ definition")
        _close(bk, scale * np.einsum("bhij,bhid->bhjd", w, np.abs(q)), 1e-12,
               "bK definition")


ALL_BWD_PINS = [
    pin_bwd_finite_differences,
    pin_bwd_one_key,
    pin_bwd_two_keys,
    pin_bwd_constant_values,
    pin_bwd_sum_rules,
    pin_bwd_autograd_witness,
    pin_bwd_row_sampling,
    pin_bwd_magnitudes,
]
