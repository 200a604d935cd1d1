"""Pins of the oracle's variable-length attention (oracle.attention_varlen).

Variable-length batches are named as an extension on page
"FlashAttention-2实现与优化：高效注意力机制详解" §7 (ragged input sequences)
without a definition; the reading used here: S sequences packed along the
token axis, each attending only to its own keys with the forward's
definition (and its top-left causal rule) inside the sequence.  Pins:

  * equal lengths reduce to the dense batched oracle ([B,H,N,D] with B = S);
  * a pure-Python brute force (math.fsum) on tiny mixed lengths;
  * isolation: changing one sequence's keys and values leaves every other
    sequence's output bit-identical;
  * empty sequences (no queries, or no keys: O = 0, L = -inf).
"""
from __future__ import annotations

import math

import numpy as np

import oracle


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    fin = np.isfinite(b)
    assert np.array_equal(fin, np.isfinite(a)), f"{what}: finiteness differs"
    err = float(np.max(np.abs(a[fin] - b[fin]))) if fin.any() else 0.0
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: non-finite values differ"
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"


def _packed(seed, H, lq, lk, D):
    r = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    q = r.standard_normal((H, int(cu_q[-1]), D))
    k = r.standard_normal((H, int(cu_k[-1]), D))
    v = r.standard_normal((H, int(cu_k[-1]), D))
    return q, k, v, cu_q, cu_k


def pin_varlen_equal_lengths_is_dense(lib):
    S, H, N, D = 3, 2, 11, 5
    q, k, v, cu_q, cu_k = _packed(1, H, [N] * S, [N] * S, D)
    for causal in (False, True):
        o, l = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.4, causal, lib=lib)
        qd = q.reshape(H, S, N, D).transpose(1, 0, 2, 3)
        kd = k.reshape(H, S, N, D).transpose(1, 0, 2, 3)
        vd = v.reshape(H, S, N, D).transpose(1, 0, 2, 3)
        od, ld = oracle.attention(qd, kd, vd, 0.4, causal, lib=lib)
        _close(o, od.transpose(1, 0, 2, 3).reshape(H, S * N, D), 0.0, "equal lengths O")
        _close(l, ld.transpose(1, 0, 2).reshape(H, S * N), 0.0, "equal lengths L")


def pin_varlen_brute_force(lib):
    lq, lk = [3, 1, 5, 2], [4, 2, 5, 1]
    H, D, scale = 2, 3, 0.7
    q, k, v, cu_q, cu_k = _packed(2, H, lq, lk, D)
    for causal in (False, True):
        o, l = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale, causal, lib=lib)
        for h in range(H):
            for s in range(len(lq)):
                for i in range(lq[s]):
                    row = int(cu_q[s]) + i
                    keys = [int(cu_k[s]) + j for j in range(lk[s]) if not causal or j <= i]
                    sc = [scale * math.fsum(q[h, row] * k[h, j]) for j in keys]
                    m = max(sc)
                    w = [math.exp(x - m) for x in sc]
                    tot = math.fsum(w)
                    ref = [math.fsum(wj * v[h, j, d] for wj, j in zip(w, keys)) / tot
                           for d in range(D)]
                    _close(o[h, row], ref, 1e-12, "brute force O")
                    _close([l[h, row]], [m + math.log(tot)], 1e-12, "brute force L")


def pin_varlen_isolation(lib):
    lq, lk = [7, 4, 9], [5, 8, 6]
    H, D = 1, 4
    q, k, v, cu_q, cu_k = _packed(3, H, lq, lk, D)
    o, l = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.5, True, lib=lib)
    k2, v2 = k.copy(), v.copy()
    k2[:, cu_k[1]:cu_k[2]] += 3.0
    v2[:, cu_k[1]:cu_k[2]] *= -2.0
    o2, l2 = oracle.attention_varlen(q, k2, v2, cu_q, cu_k, 0.5, True, lib=lib)
    for s in (0, 2):
        a, b = cu_q[s], cu_q[s + 1]
        assert np.array_equal(o[:, a:b], o2[:, a:b]), "isolation: O changed"
        assert np.array_equal(l[:, a:b], l2[:, a:b]), "isolation: L changed"
    a, b = cu_q[1], cu_q[2]
    assert not np.allclose(o[:, a:b], o2[:, a:b]), "isolation: the changed sequence must change"


def pin_varlen_empty_sequences(lib):
    lq, lk = [0, 3, 2, 4], [2, 0, 3, 4]
    H, D = 1, 3
    q, k, v, cu_q, cu_k = _packed(4, H, lq, lk, D)
    o, l = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.5, False, lib=lib)
    a, b = cu_q[1], cu_q[2]  # queries without keys
    assert np.array_equal(o[:, a:b], np.zeros_like(o[:, a:b])), "no keys: O = 0"
    assert np.all(np.isneginf(l[:, a:b])), "no keys: L = -inf"
    od, ld = oracle.attention(q[None, :, cu_q[3]:], k[None, :, cu_k[3]:], v[None, :, cu_k[3]:],
                              0.5, False, lib=lib)
    _close(o[:, cu_q[3]:], od[0], 0.0, "last sequence O")


def pin_varlen_bwd_equal_lengths_is_dense(lib):
    S, H, N, D = 3, 2, 9, 4
    q, k, v, cu_q, cu_k = _packed(5, H, [N] * S, [N] * S, D)
    g = np.random.default_rng(6).standard_normal(q.shape)
    for causal in (False, True):
        got = oracle.attention_bwd_varlen(q, k, v, g, cu_q, cu_k, 0.4, causal, lib=lib)
        dense = [x.reshape(H, S, N, D).transpose(1, 0, 2, 3) for x in (q, k, v, g)]
        ref = oracle.attention_bwd(*dense, 0.4, causal, lib=lib)
        for a, b in zip(got, ref):
            _close(a, b.transpose(1, 0, 2, 3).reshape(H, S * N, D), 0.0, "bwd equal lengths")


def pin_varlen_bwd_finite_differences(lib):
    """Gradients of sum(dO * O_varlen) against central differences."""
    lq, lk, H, D, scale = [3, 0, 2, 4], [2, 3, 3, 0], 1, 2, 0.8
    q, k, v, cu_q, cu_k = _packed(7, H, lq, lk, D)
    g = np.random.default_rng(8).standard_normal(q.shape)
    h = 1e-5
    for causal in (False, True):
        grads = oracle.attention_bwd_varlen(q, k, v, g, cu_q, cu_k, scale, causal, lib=lib)
        base = {"q": q, "k": k, "v": v}

        def loss(**kw):
            a = dict(base)
            a.update(kw)
            o, _ = oracle.attention_varlen(a["q"], a["k"], a["v"], cu_q, cu_k, scale, causal,
                                           lib=lib)
            return float((o * g).sum())

        for name, grad in zip(("q", "k", "v"), grads):
            x = base[name]
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                num[idx] = (loss(**{name: xp}) - loss(**{name: xm})) / (2 * h)
            _close(grad, num, 1e-7, f"varlen finite differences d{name}")


ALL_VARLEN_PINS = [
    pin_varlen_bwd_equal_lengths_is_dense,
    pin_varlen_bwd_finite_differences,
    pin_varlen_equal_lengths_is_dense,
    pin_varlen_brute_force,
    pin_varlen_isolation,
    pin_varlen_empty_sequences,
]
