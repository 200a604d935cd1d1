"""Pins of the oracle's local-window + global-token attention
(oracle.attention_masked).  The pages name the pattern without defining it
(page "FlashAttention-2实现与优化：高效注意力机制详解" §7); the reading is
stated in fa_oracle.c.  Pins:

  * a window covering every key and no global tokens reduces to the dense
    oracle (causal and not); so does nglobal >= Nq, Nk;
  * window 1 without global tokens leaves only the diagonal: O_i = v_i
    exactly and L_i = scale <q_i, k_i>;
  * a pure-Python brute force (math.fsum) over a visibility set written
    independently, on tiny shapes, Nq != Nk both ways;
  * keys a row cannot see do not matter: changing them leaves the row's
    output bit-identical;
  * rows with no visible key (Nq > Nk) get O = 0 and L = -inf;
  * backward: reduction to the dense backward (gradients and magnitude
    sums), the diagonal window, central finite differences of the masked
    forward, the magnitude sums against their definition written with numpy
    on an independently built visibility matrix, and row sampling.
"""
from __future__ import annotations

import math

import numpy as np

import oracle


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.isfinite(err) and err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"


def _qkv(seed, B, H, Nq, Nk, D):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, H, Nq, D)), r.standard_normal((B, H, Nk, D)),
            r.standard_normal((B, H, Nk, D)))


def pin_masked_reduces_to_dense(lib):
    q, k, v = _qkv(1, 2, 2, 13, 11, 4)
    for causal in (False, True):
        ref = oracle.attention(q, k, v, 0.6, causal, lib=lib)
        for window, ng in ((13, 0), (100, 3), (1, 13), (2, 50)):
            got = oracle.attention_masked(q, k, v, 0.6, causal, window, ng, lib=lib)
            _close(got[0], ref[0], 0.0, f"dense O (window {window}, global {ng})")
            _close(got[1], ref[1], 0.0, f"dense L (window {window}, global {ng})")


def pin_masked_diagonal_only(lib):
    q, k, v = _qkv(2, 1, 2, 9, 9, 5)
    for causal in (False, True):
        o, l = oracle.attention_masked(q, k, v, 0.7, causal, 1, 0, lib=lib)
        _close(o, v, 0.0, "window 1: O = V")
        _close(l, 0.7 * np.einsum("bhnd,bhnd->bhn", q, k), 1e-12, "window 1: L = s_ii")


def _visible(i, j, causal, window, ng):
    if causal and j > i:
        return False
    if abs(i - j) < window:
        return True
    return j < ng or i < ng


def pin_masked_brute_force(lib):
    for (Nq, Nk, window, ng) in ((7, 7, 2, 1), (9, 5, 3, 2), (4, 10, 2, 0), (6, 6, 4, 6)):
        q, k, v = _qkv(3 + Nq, 1, 1, Nq, Nk, 3)
        for causal in (False, True):
            o, l = oracle.attention_masked(q, k, v, 0.9, causal, window, ng, lib=lib)
            for i in range(Nq):
                keys = [j for j in range(Nk) if _visible(i, j, causal, window, ng)]
                if not keys:
                    assert np.all(o[0, 0, i] == 0) and np.isneginf(l[0, 0, i])
                    continue
                s = [0.9 * math.fsum(q[0, 0, i] * k[0, 0, j]) for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = math.fsum(w)
                ref = [math.fsum(wj * v[0, 0, j, d] for wj, j in zip(w, keys)) / tot
                       for d in range(3)]
                _close(o[0, 0, i], ref, 1e-12, "brute force O")
                _close([l[0, 0, i]], [m + math.log(tot)], 1e-12, "brute force L")


def pin_masked_hidden_keys_do_not_matter(lib):
    q, k, v = _qkv(4, 1, 1, 40, 40, 4)
    window, ng = 5, 2
    o, l = oracle.attention_masked(q, k, v, 0.5, True, window, ng, lib=lib)
    k2, v2 = k.copy(), v.copy()
    k2[..., 10:20, :] += 5.0   # hidden from rows 25.. (not global, out of window)
    v2[..., 10:20, :] *= -3.0
    o2, l2 = oracle.attention_masked(q, k2, v2, 0.5, True, window, ng, lib=lib)
    assert np.array_equal(o[..., 25:, :], o2[..., 25:, :]), "hidden keys changed O"
    assert np.array_equal(l[..., 25:], l2[..., 25:]), "hidden keys changed L"
    assert not np.allclose(o[..., 12, :], o2[..., 12, :]), "visible keys must matter"


def pin_masked_rows_without_keys(lib):
    q, k, v = _qkv(5, 1, 1, 12, 4, 3)
    o, l = oracle.attention_masked(q, k, v, 0.5, True, 3, 0, lib=lib)
    # rows i >= Nk + window - 1 = 6 see no key (window [i-2, i] past Nk)
    assert np.all(o[0, 0, 6:] == 0) and np.all(np.isneginf(l[0, 0, 6:]))
    assert np.all(np.isfinite(l[0, 0, :6]))


def pin_masked_bwd_reduces_to_dense(lib):
    """A window covering every key: gradients and magnitude sums are the
    dense oracle's."""
    q, k, v = _qkv(6, 1, 2, 12, 9, 3)
    g = np.random.default_rng(7).standard_normal(q.shape)
    for causal in (False, True):
        ref = oracle.attention_bwd(q, k, v, g, 0.5, causal, magnitudes=True, lib=lib)
        got = oracle.attention_bwd_masked(q, k, v, g, 0.5, causal, 100, 0, magnitudes=True,
                                          lib=lib)
        for a, b in zip(got, ref):
            _close(a, b, 1e-12, "masked bwd reduces to dense")


def _visible_matrix(Nq, Nk, causal, window, ng):
    """The visibility matrix, written from the rule's two parts on index
    grids (independently of the oracle's per-pair test)."""
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    band = (i - j >= 0) & (i - j < window) if causal else np.abs(i - j) < window
    glob = (j < ng) | (i < ng)
    if causal:
        glob &= j <= i
    return band | glob


def pin_masked_bwd_magnitudes(lib):
    """The magnitude sums bound the gradients and follow their definition
    over the visible pairs (written here with numpy on the visibility matrix;
    rows without a visible key contribute nothing)."""
    B, H, Nq, Nk, D = 1, 2, 13, 9, 5
    q, k, v = _qkv(50, B, H, Nq, Nk, D)
    g = np.random.default_rng(51).standard_normal(q.shape)
    scale = -0.7
    for causal, window, ng in ((False, 3, 1), (True, 2, 2), (True, 4, 0), (False, 1, 0)):
        dq, dk, dv, bq, bk, bv = oracle.attention_bwd_masked(q, k, v, g, scale, causal, window,
                                                             ng, magnitudes=True, lib=lib)
        for grad, bound, what in ((dq, bq, "Q"), (dk, bk, "K"), (dv, bv, "V")):
            assert np.all(bound >= np.abs(grad) - 1e-12), f"b{what} below |d{what}|"
        vis = _visible_matrix(Nq, Nk, causal, window, ng)
        s = scale * np.einsum("bhid,bhjd->bhij", q, k)
        s = np.where(vis, s, -np.inf)
        mx = s.max(-1, keepdims=True)
        mx = np.where(np.isfinite(mx), mx, 0.0)
        e = np.where(vis, np.exp(s - mx), 0.0)
        tot = e.sum(-1, keepdims=True)
        p = np.divide(e, tot, out=np.zeros_like(e), where=tot > 0)
        dp = np.einsum("bhid,bhjd->bhij", g, v)
        o = np.einsum("bhij,bhjd->bhid", p, v)
        rowterm = (g * o).sum(-1, keepdims=True)
        ee = (np.abs(g) * np.einsum("bhij,bhjd->bhid", p, np.abs(v))).sum(-1, keepdims=True)
        w = np.abs(p * (dp - rowterm)) + p * ee
        _close(bv, np.einsum("bhij,bhid->bhjd", p, np.abs(g)), 1e-12, "masked bV definition")
        _close(bq, abs(scale) * np.einsum("bhij,bhjd->bhid", w, np.abs(k)), 1e-12,
               "masked bQ definition")
        _close(bk, abs(scale) * np.einsum("bhij,bhid->bhjd", w, np.abs(q)), 1e-12,
               "masked bK definition")
        _close(dv, np.einsum("bhij,bhid->bhjd", p, g), 1e-12, "masked dV (numpy)")


def pin_masked_bwd_row_sampling(lib):
    """Sampled query and key rows equal the same rows of the full result,
    gradients and magnitude sums alike."""
    B, H, Nq, Nk, D = 2, 2, 15, 11, 3
    q, k, v = _qkv(60, B, H, Nq, Nk, D)
    g = np.random.default_rng(61).standard_normal(q.shape)
    for causal, window, ng in ((False, 4, 2), (True, 3, 1)):
        full = oracle.attention_bwd_masked(q, k, v, g, 0.4, causal, window, ng,
                                           magnitudes=True, lib=lib)
        qr = np.array([0, 7, B * H * Nq - 1, 33, 16])
        kr = np.array([B * H * Nk - 1, 2, 0, 25])
        part = oracle.attention_bwd_masked(q, k, v, g, 0.4, causal, window, ng, qrows=qr,
                                           krows=kr, magnitudes=True, lib=lib)
        _close(part[0], full[0].reshape(-1, D)[qr], 0.0, "sampled masked dQ")
        _close(part[3], full[3].reshape(-1, D)[qr], 0.0, "sampled masked bQ")
        for t in (1, 2, 4, 5):
            _close(part[t], full[t].reshape(-1, D)[kr], 0.0, f"sampled masked key output {t}")


def pin_masked_bwd_diagonal(lib):
    """window 1: each row sees only its own key, so dQ = dK = 0, dV_i = dO_i."""
    q, k, v = _qkv(8, 1, 1, 7, 7, 4)
    g = np.random.default_rng(9).standard_normal(q.shape)
    for causal in (False, True):
        dq, dk, dv = oracle.attention_bwd_masked(q, k, v, g, 0.8, causal, 1, 0, lib=lib)
        _close(dq, np.zeros_like(dq), 1e-14, "diagonal dQ")
        _close(dk, np.zeros_like(dk), 1e-14, "diagonal dK")
        _close(dv, g, 1e-14, "diagonal dV")


def pin_masked_bwd_finite_differences(lib):
    h = 1e-5
    for Nq, Nk, window, ng, causal in ((6, 6, 2, 1, True), (5, 7, 3, 2, False),
                                       (7, 4, 2, 0, True)):
        q, k, v = _qkv(10 + Nq, 1, 1, Nq, Nk, 2)
        g = np.random.default_rng(11).standard_normal(q.shape)
        grads = oracle.attention_bwd_masked(q, k, v, g, 0.7, causal, window, ng, lib=lib)
        base = {"q": q, "k": k, "v": v}

        def loss(**kw):
            a = dict(base)
            a.update(kw)
            o, _ = oracle.attention_masked(a["q"], a["k"], a["v"], 0.7, causal, window, ng,
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
            _close(grad, num, 1e-7, f"masked finite differences d{name}")


ALL_MASKED_PINS = [
    pin_masked_bwd_reduces_to_dense,
    pin_masked_bwd_magnitudes,
    pin_masked_bwd_row_sampling,
    pin_masked_bwd_diagonal,
    pin_masked_bwd_finite_differences,
    pin_masked_reduces_to_dense,
    pin_masked_diagonal_only,
    pin_masked_brute_force,
    pin_masked_hidden_keys_do_not_matter,
    pin_masked_rows_without_keys,
]
