"""Pins that tie the CPU oracle to what the pages and mathematics fix.

Each ``pin_*`` function takes a loaded oracle library handle (see
``oracle.load``) and raises AssertionError when the oracle disagrees with a
fact that does not come from the oracle itself:

  * closed forms (identical keys, causal row 0, one and two keys,
    hand-derived worked examples under tests/golden/);
  * invariants of the definition (key permutation, a shift added to every
    key, an affine map of the values, constant values, rows of the softmax
    summing to one);
  * independent formulations (pure-Python brute force with math.fsum, a numpy
    log-sum-exp formulation, torch's fp64 CPU scaled_dot_product_attention);
  * the pages' tiled recurrence reaching the two-pass result
    (page "FlashAttention-2实现与优化：高效注意力机制详解" §3.1).

The same battery runs against deliberately broken builds of the oracle in
test_oracle_mutations.py, to show that a plausible mistake fails a pin.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "worked_examples.json")

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max-abs error {err:.3e} > {tol:.1e}"


def _eval_expr(s: str) -> float:
    return float(eval(s, {"__builtins__": {}}, {"e": math.e, "ln": math.log}))


# ---------------------------------------------------------------------------
def pin_worked_examples(lib):
    """Hand-derived examples (tests/golden/worked_examples.json)."""
    with open(GOLDEN) as f:
        examples = json.load(f)["examples"]
    for ex in examples:
        q = np.array(ex["q"])[None]
        k = np.array(ex["k"])[None]
        v = np.array(ex["v"])[None]
        o, lse = oracle.attention(q, k, v, ex["scale"], ex["causal"], lib=lib)
        want_o = np.array([[_eval_expr(s) for s in row] for row in ex["o"]])
        want_l = np.array([_eval_expr(s) for s in ex["lse"]])
        _close(o[0], want_o, 1e-13, ex["name"] + " o")
        _close(lse[0], want_l, 1e-13, ex["name"] + " lse")


def pin_rows_sum_to_one(lib):
    """With D = Nk and V = I the output rows are the softmax rows themselves:
    non-negative, summing to 1, and exactly 0 on causally hidden keys."""
    for (nq, nk, causal, seed) in [(5, 5, False, 1), (7, 7, True, 2), (6, 4, True, 3),
                                   (3, 9, True, 4), (9, 3, False, 5)]:
        r = _rng(seed)
        d = nk
        q = r.standard_normal((2, nq, d))
        k = r.standard_normal((2, nk, d))
        v = np.broadcast_to(np.eye(nk), (2, nk, nk)).copy()
        o, _ = oracle.attention(q, k, v, 0.7, causal, lib=lib)
        assert np.all(o >= 0), "softmax weights must be non-negative"
        _close(o.sum(-1), np.ones((2, nq)), 1e-13, "row sums")
        if causal:
            hidden = np.triu(np.ones((nq, nk), dtype=bool), k=1)
            assert np.all(o[:, hidden] == 0.0), "hidden keys must get weight 0"
            assert np.all(o[:, ~hidden] > 0.0), "visible keys must get weight > 0"


def pin_online_matches_two_pass(lib):
    """The pages' tiled recurrence reaches the two-pass result, for tile
    sizes that are ragged, a single key, and larger than the problem."""
    for n in (1, 2, 5, 17, 64):
        r = _rng(100 + n)
        q = r.standard_normal((2, n, 8))
        k = r.standard_normal((2, n, 8))
        v = r.standard_normal((2, n, 8))
        tiles = sorted({1, 3, 7, 16, max(n - 1, 1), n, n + 5})
        for causal in (False, True):
            o2, l2 = oracle.attention(q, k, v, 0.5, causal, lib=lib)
            for bq in tiles:
                for bk in tiles:
                    o1, l1 = oracle.attention_online(q, k, v, 0.5, causal, bq, bk,
                                                     lib=lib)
                    _close(o1, o2, TOL, f"online o n={n} bq={bq} bk={bk} c={causal}")
                    _close(l1, l2, TOL, f"online lse n={n} bq={bq} bk={bk} c={causal}")
    # unequal query / key counts
    r = _rng(7)
    for nq, nk in [(5, 13), (13, 5)]:
        q = r.standard_normal((1, nq, 4))
        k = r.standard_normal((1, nk, 4))
        v = r.standard_normal((1, nk, 4))
        for causal in (False, True):
            o2, l2 = oracle.attention(q, k, v, 0.9, causal, lib=lib)
            o1, l1 = oracle.attention_online(q, k, v, 0.9, causal, 4, 3, lib=lib)
            _close(o1, o2, TOL, "online nq!=nk o")
            _close(l1, l2, TOL, "online nq!=nk lse")


def pin_identical_keys(lib):
    """All keys equal to one vector kk: every visible score of row i is
    scale*q_i.kk, so o_i is the mean of the visible values and
    L_i = scale*q_i.kk + ln(#visible)."""
    r = _rng(11)
    n, d, scale = 19, 6, 0.37
    q = r.standard_normal((2, n, d))
    kk = r.standard_normal(d)
    k = np.broadcast_to(kk, (2, n, d)).copy()
    v = r.standard_normal((2, n, d))
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, scale, causal, lib=lib)
        cnt = np.arange(1, n + 1) if causal else np.full(n, n)
        if causal:
            want_o = np.cumsum(v, axis=1) / cnt[None, :, None]
        else:
            want_o = np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape)
        want_l = scale * (q @ kk) + np.log(cnt)[None]
        _close(o, want_o, 1e-12, f"identical keys o causal={causal}")
        _close(lse, want_l, 1e-12, f"identical keys lse causal={causal}")


def pin_causal_row_zero(lib):
    """Under the causal mask row 0 sees only key 0: o_0 = v_0 exactly and
    L_0 = scale*q_0.k_0."""
    r = _rng(12)
    q = r.standard_normal((3, 10, 5))
    k = r.standard_normal((3, 10, 5))
    v = r.standard_normal((3, 10, 5))
    o, lse = oracle.attention(q, k, v, 1.3, True, lib=lib)
    assert np.array_equal(o[:, 0], v[:, 0]), "causal row 0 must equal v_0"
    _close(lse[:, 0], 1.3 * np.einsum("bd,bd->b", q[:, 0], k[:, 0]), 1e-14,
           "causal row 0 lse")


def pin_one_and_two_keys(lib):
    """Nk = 1: o = v_0, L = s_0.  Nk = 2: o = sig(s0-s1) v_0 + (1-sig) v_1 with
    the logistic function sig, and L = logaddexp(s0, s1)."""
    r = _rng(13)
    q = r.standard_normal((4, 6, 3))
    k1 = r.standard_normal((4, 1, 3))
    v1 = r.standard_normal((4, 1, 3))
    o, lse = oracle.attention(q, k1, v1, 0.8, False, lib=lib)
    _close(o, np.broadcast_to(v1, o.shape), 0.0, "one key o")
    _close(lse, 0.8 * np.einsum("bid,bd->bi", q, k1[:, 0]), 1e-14, "one key lse")

    k2 = r.standard_normal((4, 2, 3))
    v2 = r.standard_normal((4, 2, 3))
    o, lse = oracle.attention(q, k2, v2, 0.8, False, lib=lib)
    s = 0.8 * np.einsum("bid,bjd->bij", q, k2)
    sig = 1.0 / (1.0 + np.exp(-(s[..., 0] - s[..., 1])))
    want_o = sig[..., None] * v2[:, None, 0] + (1 - sig)[..., None] * v2[:, None, 1]
    _close(o, want_o, 1e-13, "two keys o")
    _close(lse, np.logaddexp(s[..., 0], s[..., 1]), 1e-13, "two keys lse")


def pin_invariants(lib):
    """Structural facts of the definition:
      * permuting keys (with their values) changes nothing, unmasked;
      * adding u to every key shifts L_i by scale*q_i.u, o unchanged;
      * v -> v A + b gives o -> o A + b;
      * constant values give that constant."""
    r = _rng(14)
    B, nq, nk, d, sc = 2, 11, 13, 5, 0.45
    q = r.standard_normal((B, nq, d))
    k = r.standard_normal((B, nk, d))
    v = r.standard_normal((B, nk, d))
    o, lse = oracle.attention(q, k, v, sc, False, lib=lib)

    perm = r.permutation(nk)
    o_p, l_p = oracle.attention(q, k[:, perm], v[:, perm], sc, False, lib=lib)
    _close(o_p, o, 1e-13, "key permutation o")
    _close(l_p, lse, 1e-13, "key permutation lse")

    u = r.standard_normal(d)
    for causal in (False, True):
        o0, l0 = oracle.attention(q, k, v, sc, causal, lib=lib)
        o_s, l_s = oracle.attention(q, k + u, v, sc, causal, lib=lib)
        _close(o_s, o0, 1e-12, f"key shift o causal={causal}")
        _close(l_s, l0 + sc * (q @ u), 1e-12, f"key shift lse causal={causal}")

        A = r.standard_normal((d, d))
        b = r.standard_normal(d)
        o_a, l_a = oracle.attention(q, k, v @ A + b, sc, causal, lib=lib)
        _close(o_a, o0 @ A + b, 1e-12, f"value affine o causal={causal}")
        _close(l_a, l0, 0.0, f"value affine lse causal={causal}")

        c = r.standard_normal(d)
        o_c, _ = oracle.attention(q, k, np.broadcast_to(c, v.shape).copy(), sc, causal,
                                  lib=lib)
        _close(o_c, np.broadcast_to(c, o_c.shape), 1e-14, f"constant v causal={causal}")


def pin_bruteforce(lib):
    """Pure-Python loops with math.fsum on tiny inputs (an independent
    formulation: normalise first, then take the weighted sum)."""
    r = _rng(15)
    for (nq, nk, d, causal) in [(4, 4, 3, False), (5, 5, 2, True), (3, 6, 4, True),
                                (6, 3, 2, True), (1, 7, 3, False)]:
        q = r.standard_normal((1, nq, d))
        k = r.standard_normal((1, nk, d))
        v = r.standard_normal((1, nk, d))
        sc = 0.6
        o, lse = oracle.attention(q, k, v, sc, causal, lib=lib)
        for i in range(nq):
            js = [j for j in range(nk) if (not causal) or j <= i]
            s = [sc * math.fsum(q[0, i, t] * k[0, j, t] for t in range(d)) for j in js]
            m = max(s)
            z = math.fsum(math.exp(x - m) for x in s)
            L = m + math.log(z)
            for t in range(d):
                want = math.fsum(math.exp(s[a] - L) * v[0, j, t] for a, j in enumerate(js))
                assert abs(o[0, i, t] - want) <= 1e-13, f"brute force o[{i},{t}]"
            assert abs(lse[0, i] - L) <= 1e-13, f"brute force lse[{i}]"


def pin_numpy_witness(lib):
    """Vectorised numpy formulation p = exp(S - logsumexp(S)), masked with -inf,
    on multi-head shapes including unequal query / key counts."""
    r = _rng(16)
    for (B, H, nq, nk, d) in [(2, 3, 33, 33, 16), (1, 2, 40, 17, 8), (2, 1, 17, 40, 8)]:
        q = r.standard_normal((B, H, nq, d))
        k = r.standard_normal((B, H, nk, d))
        v = r.standard_normal((B, H, nk, d))
        for causal in (False, True):
            S = 0.25 * (q @ np.swapaxes(k, -1, -2))
            if causal:
                S = np.where(np.tril(np.ones((nq, nk), dtype=bool)), S, -np.inf)
            mx = S.max(-1, keepdims=True)
            L = (mx + np.log(np.exp(S - mx).sum(-1, keepdims=True)))
            want_o = np.exp(S - L) @ v
            o, lse = oracle.attention(q, k, v, 0.25, causal, lib=lib)
            _close(o, want_o, 1e-12, f"numpy witness o causal={causal}")
            _close(lse, L[..., 0], 1e-12, f"numpy witness lse causal={causal}")


def pin_torch_witness(lib):
    """torch's fp64 CPU scaled_dot_product_attention (test-only witness);
    its causal mask is the same top-left alignment for Nq == Nk."""
    import torch
    r = _rng(17)
    for causal in (False, True):
        q = r.standard_normal((2, 3, 29, 16))
        k = r.standard_normal((2, 3, 29, 16))
        v = r.standard_normal((2, 3, 29, 16))
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=0.3).numpy()
        o, _ = oracle.attention(q, k, v, 0.3, causal, lib=lib)
        _close(o, want, 1e-12, f"torch witness causal={causal}")


def pin_row_sampling(lib):
    """Selecting rows returns exactly the corresponding rows of the full run."""
    r = _rng(18)
    q = r.standard_normal((2, 3, 21, 8))
    k = r.standard_normal((2, 3, 21, 8))
    v = r.standard_normal((2, 3, 21, 8))
    o, lse = oracle.attention(q, k, v, 0.5, True, lib=lib)
    rows = np.array([0, 5, 20, 21, 62, 125])
    o_s, l_s = oracle.attention(q, k, v, 0.5, True, rows=rows, lib=lib)
    assert np.array_equal(o_s, o.reshape(-1, 8)[rows])
    assert np.array_equal(l_s, lse.reshape(-1)[rows])


def pin_gaussian_statistics(lib):
    """Not a tight pin: with i.i.d. N(0,1) inputs and scale 1/sqrt(D) the
    scores are ~N(0,1), so L_i - ln(n_keys) averages about 1/2
    (ln E[e^s] = 1/2 for s ~ N(0,1)).  Catches a gross scale or log-base slip."""
    r = _rng(19)
    d = 64
    q = r.standard_normal((1, 256, d))
    k = r.standard_normal((1, 4096, d))
    v = r.standard_normal((1, 4096, d))
    _, lse = oracle.attention(q, k, v, 1.0 / math.sqrt(d), False, lib=lib)
    mean = float(np.mean(lse - math.log(4096)))
    assert 0.35 < mean < 0.6, f"mean L - ln N = {mean:.3f}, expected about 0.5"


ALL_PINS = [
    pin_worked_examples,
    pin_rows_sum_to_one,
    pin_online_matches_two_pass,
    pin_identical_keys,
    pin_causal_row_zero,
    pin_one_and_two_keys,
    pin_invariants,
    pin_bruteforce,
    pin_numpy_witness,
    pin_torch_witness,
    pin_row_sampling,
    pin_gaussian_statistics,
]
