"""GPU parity of variable-length batches (fa_fwd_varlen, and fa_fwd_varlen_ws
with its stream schedule over (head, sequence) pairs or, past 512 pairs,
its key-split tiles; through the C ABI)
against the fp64 oracle (oracle.attention_varlen), with the forward's
tolerances: fp32 O <= 1e-2 and L <= 1e-3 for 16-bit inputs, 16-bit O the
exact rounding of the fp32 O and within 1e-2 plus half an ulp.  Each
sequence must also be bit-identical to the same per-tile code run on that
sequence alone (no cross-talk between packed sequences)."""
import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_07_amd as fa
from workloads import gen_qkv, sample_rows, varlen_lengths

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _log(msg):
    print(f"[varlen] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()
    oracle.load()


def _half_ulp(x, dtype):
    mant = {torch.bfloat16: 7, torch.float16: 10}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return 2.0 ** (e - mant - 1)


def packed(lq, lk, H, D, seed, dtype="bf16"):
    Tq, Tk = sum(lq), sum(lk)
    q, _, _ = gen_qkv(1, H, Tq, 1, D, seed=seed, dtype=dtype)
    _, k, v = gen_qkv(1, H, 1, Tk, D, seed=seed + 1, dtype=dtype)
    cu_q = torch.tensor([0] + list(np.cumsum(lq)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(lk)), dtype=torch.int32)
    return q[0], k[0], v[0], cu_q, cu_k


def run(q, k, v, cu_q, cu_k, maxq, causal, scale, out_dtype, maxk=None):
    o, lse = fa.fwd_varlen(q.to(DEV), k.to(DEV), v.to(DEV), cu_q.to(DEV), cu_k.to(DEV), maxq,
                           causal=causal, scale=scale, out_dtype=out_dtype, max_seqlen_k=maxk)
    torch.cuda.synchronize()
    return o.float().cpu(), lse.cpu()


def compare(lq, lk, H, D, causal, seed, dtype="bf16", scale=None, rows=None, solo=True,
            maxk=None):
    """maxk: run fa_fwd_varlen_ws with this max_seqlen_k (the stream
    schedule at H * S <= 512 pairs, key-split tiles above)."""
    q, k, v, cu_q, cu_k = packed(lq, lk, H, D, seed, dtype)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    maxq = max(lq) if max(lq) > 0 else 1
    _log(f"S={len(lq)} H={H} D={D} causal={causal} dtype={dtype} Tq={sum(lq)} Tk={sum(lk)} "
         f"max_q={maxq} max_k={maxk} rows={'all' if rows is None else len(rows)}")
    if maxk is not None:
        st, nb = fa.fa_fwd_varlen_workspace_size(len(lq), H, sum(lq), sum(lk), maxq, maxk, D,
                                                 causal, fa._dtype_code(torch, q.dtype, q.dtype))
        assert st == 0 and nb > 0, "the split case must split"
        solo = False  # split tiles sum their chunks in another order than fa_fwd
    o32, l32 = run(q, k, v, cu_q, cu_k, maxq, causal, scale, torch.float32, maxk)
    o16, l16 = run(q, k, v, cu_q, cu_k, maxq, causal, scale, q.dtype, maxk)
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    if rows is None:
        ro, rl = oracle.attention_varlen(qn, kn, vn, cu_q.numpy(), cu_k.numpy(), scale, causal)
        sel = slice(None)
        ro, rl = ro.reshape(-1, D), rl.reshape(-1)
    else:
        # sampled rows, each from the oracle on its own sequence
        ro, rl = [], []
        cq, ck = cu_q.numpy(), cu_k.numpy()
        for r in rows:
            h, t = divmod(int(r), sum(lq))
            s = int(np.searchsorted(cq, t, side="right") - 1)
            a, b, ka, kb = cq[s], cq[s + 1], ck[s], ck[s + 1]
            oo, ll = oracle.attention(qn[None, h:h + 1, a:b], kn[None, h:h + 1, ka:kb],
                                      vn[None, h:h + 1, ka:kb], scale, causal, rows=[t - a])
            ro.append(oo[0])
            rl.append(ll[0])
        ro, rl = np.array(ro), np.array(rl)
        sel = torch.as_tensor(rows)
    g_o = o32.reshape(-1, D)[sel].double().numpy()
    g_l = l32.reshape(-1)[sel].double().numpy()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(g_l), fin), "lse finiteness differs"
    assert np.all(np.isneginf(g_l[~fin])), "rows without keys must have lse = -inf"
    assert np.all(g_o[~fin] == 0), "rows without keys must have O = 0"
    err_o = float(np.abs(g_o - ro).max()) if g_o.size else 0.0
    err_l = float(np.abs(g_l[fin] - rl[fin]).max()) if fin.any() else 0.0
    _log(f"  fp32-O max-abs O {err_o:.3e} L {err_l:.3e}")
    assert err_o <= 1e-2 and err_l <= 1e-3
    x16 = o16.reshape(-1, D)[sel].double().numpy()
    rnd = torch.from_numpy(g_o).to(q.dtype).double().numpy()
    assert np.array_equal(rnd, x16), "16-bit O is not the rounding of the fp32 O"
    assert (np.abs(x16 - ro) <= 1e-2 + _half_ulp(ro, q.dtype)).all()
    assert torch.equal(l16.reshape(-1)[sel], l32.reshape(-1)[sel])
    if solo and rows is None:
        # every sequence bit-identical to the same computation on that
        # sequence alone: fa_fwd's one-workgroup-per-tile grid (the same
        # 256-row per-tile code), or at D = 128, where few packed tiles select
        # the pair-split 128-row layout, fa_fwd_varlen with that one sequence
        for s in range(len(lq)):
            a, b, ka, kb = (int(x) for x in (cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]))
            if b == a or kb == ka:
                continue
            qs = q[:, a:b].contiguous()
            ks, vs = k[:, ka:kb].contiguous(), v[:, ka:kb].contiguous()
            if D == 128:
                one = torch.tensor([0, b - a], dtype=torch.int32)
                onek = torch.tensor([0, kb - ka], dtype=torch.int32)
                so, sl = run(qs, ks, vs, one, onek, b - a, causal, scale, torch.float32)
            else:
                so, sl = fa.fwd(qs[None].to(DEV), ks[None].to(DEV), vs[None].to(DEV),
                                causal=causal, scale=scale, out_dtype=torch.float32,
                                split=False)
                torch.cuda.synchronize()
                so, sl = so[0].cpu(), sl[0].cpu()
            assert torch.equal(so, o32[:, a:b]), f"sequence {s}: O differs when run alone"
            assert torch.equal(sl, l32[:, a:b]), f"sequence {s}: L differs when run alone"


MIXED = [1, 31, 256, 257, 700, 64, 1000, 5]


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_mixed_lengths(D, causal):
    compare(MIXED, MIXED, 2, D, causal, seed=1200 + D)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_unequal_query_key_lengths(causal):
    compare([100, 3, 513, 40], [7, 300, 200, 41], 2, 128, causal, seed=1300)


def test_varlen_fp16():
    compare(MIXED, MIXED, 1, 64, True, seed=1400, dtype="f16")


def test_varlen_empty_sequences():
    """A sequence without queries, one without keys (O = 0, L = -inf)."""
    compare([5, 0, 300, 17, 9], [5, 12, 300, 0, 30], 2, 64, False, seed=1500)
    compare([5, 0, 300, 17, 9], [5, 12, 300, 0, 30], 2, 64, True, seed=1501)


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_varlen_scales(scale):
    compare([70, 300, 1], [70, 300, 1], 1, 128, True, seed=1600, scale=scale)


def test_varlen_larger_bound():
    """max_seqlen_q above every length: the extra workgroups exit at once."""
    q, k, v, cu_q, cu_k = packed([40, 90], [40, 90], 1, 64, 1700)
    a = run(q, k, v, cu_q, cu_k, 90, True, 0.125, torch.float32)
    b = run(q, k, v, cu_q, cu_k, 5000, True, 0.125, torch.float32)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_varlen_32k_tokens_sampled():
    """Eight sequences with seeded lengths summing to 32768 tokens, D=128,
    causal bf16 (the shape bench.py --varlen times): 512 sampled rows."""
    lens = varlen_lengths(32768, 8, seed=77, min_len=64)
    rows = sample_rows(32768, 512, 7700).numpy()
    compare(lens, lens, 1, 128, True, seed=1800, rows=rows)


# --- work split over the keys (fa_fwd_varlen_ws) ------------------------------
# Lengths with long sequences next to short ones.  At these head counts the
# stream schedule runs: the call's units are dealt evenly over the compute
# units, so the long sequences' tiles are cut between workgroups and merged.
SPLIT = [1, 2000, 31, 700, 1500, 64, 5]


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_split_mixed_lengths(D, causal):
    compare(SPLIT, SPLIT, 2, D, causal, seed=2100 + D, maxk=max(SPLIT))


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_split_unequal_and_empty(causal):
    """Nq != Nk per sequence, a sequence without queries and one without keys."""
    compare([100, 0, 1300, 40, 9], [7, 900, 2000, 0, 41], 2, 128, causal, seed=2200,
            maxk=2000)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_split_pair_layout(causal):
    """Long sequences on average (>= 2048 tokens): the pair-split 128-row
    tiles, cut over their keys."""
    compare([3000, 1200], [3000, 1200], 2, 128, causal, seed=2250, maxk=3000)


def test_varlen_split_fp16_negative_scale():
    compare(SPLIT, SPLIT, 1, 64, True, seed=2300, dtype="f16", scale=-0.2, maxk=max(SPLIT))


def test_varlen_split_underestimated_keys():
    """max_seqlen_k below the real longest key range: the chunks of a tile
    grow (at most the planned count per tile) and every key is still seen."""
    compare(SPLIT, SPLIT, 2, 128, True, seed=2400, maxk=1500)
    compare(SPLIT, SPLIT, 2, 128, False, seed=2401, maxk=1500)


def test_varlen_split_32k_tokens_sampled():
    """The shape bench.py --varlen 32 --split times (32768 tokens in 32
    sequences, D=128, causal bf16): 512 sampled rows against the oracle."""
    lens = varlen_lengths(32768, 32, seed=77, min_len=64)
    rows = sample_rows(32768, 512, 7832).numpy()
    compare(lens, lens, 1, 128, True, seed=1832, rows=rows, maxk=max(lens))


def test_varlen_split_one_long_sequence_sampled():
    """One 16384-token sequence beside three short ones (pair-split tiles,
    the longest cut into many chunks): 512 sampled rows."""
    lens = [16384, 100, 1000, 3000]
    rows = sample_rows(sum(lens), 512, 7900).numpy()
    compare(lens, lens, 1, 128, True, seed=1900, rows=rows, maxk=max(lens))


def test_varlen_stream_8_sequences_and_many_heads():
    """The stream schedule over (head, sequence) pairs: 8 sequences of the
    32768-token mix (the shape bench.py --varlen 8 --split times), and 48
    short sequences over 3 heads with empty ones between them (sampled
    rows against the oracle)."""
    lens = varlen_lengths(32768, 8, seed=77, min_len=64)
    st, nb = fa.fa_fwd_varlen_workspace_size(8, 1, 32768, 32768, max(lens), max(lens), 128,
                                             True, fa.FA_BF16)
    assert st == 0 and nb > 0
    rows = sample_rows(32768, 384, 7700).numpy()
    compare(lens, lens, 1, 128, True, seed=1700, rows=rows, maxk=max(lens))
    r = np.random.default_rng(7701)
    lq = [int(x) for x in r.integers(0, 300, 48)]
    lk = [int(x) if i % 7 else 0 for i, x in enumerate(r.integers(0, 300, 48))]
    lq[5] = 0
    compare(lq, lk, 3, 64, False, seed=1710, maxk=max(lk))
    compare(lq, lq, 3, 128, True, seed=1720, maxk=max(lq))


def test_varlen_stream_computes_rows_past_max_seqlen_q():
    """Under the stream schedule the offsets alone decide the work: with
    max_seqlen_q and max_seqlen_k far below the real lengths every row is
    still computed, bit-identical to the call with true bounds of the same
    tile height (both below the pair-split bound here: D = 64)."""
    lq, lk = [1000, 50, 700], [1000, 50, 900]
    q, k, v, cu_q, cu_k = packed(lq, lk, 2, 64, 3450)
    scale = 0.125
    full = run(q, k, v, cu_q, cu_k, 1000, True, scale, torch.float32, maxk=1000)
    short = run(q, k, v, cu_q, cu_k, 100, True, scale, torch.float32, maxk=60)
    assert torch.isfinite(short[0]).all() and torch.isfinite(short[1]).all()
    assert torch.equal(short[0], full[0]) and torch.equal(short[1], full[1])


def test_varlen_split_graph_capture_replays_match_eager():
    """Both kernels of fa_fwd_varlen_ws are plain launches on the caller's
    stream (no allocation, no memset), so a HIP graph captured around the
    call replays it: every replay, with eager work on the same buffers in
    between and stale workspace contents, gives the eager result bit for
    bit."""
    lens = [3000, 700, 1, 1200, 64]
    H, D, T = 2, 128, sum(lens)
    q, k, v, cu_q, cu_k = (t.to(DEV) for t in packed(lens, lens, H, D, 3100))
    st, nb = fa.fa_fwd_varlen_workspace_size(len(lens), H, T, T, max(lens), max(lens), D, True,
                                             fa.FA_BF16)
    assert st == fa.FA_OK and nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=DEV)

    def call():
        r = fa.fa_fwd_varlen_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), cu_q.data_ptr(), cu_k.data_ptr(), len(lens), H,
                                T, T, max(lens), max(lens), D, 0.125, True, fa.FA_BF16,
                                ws.data_ptr(), nb, torch.cuda.current_stream().cuda_stream)
        assert r == fa.FA_OK, fa.fa_status_str(r)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    want_o, want_l = o.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(i + 1)  # stale partials must not leak into a replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want_o), f"replay {i}: O differs from the eager call"
        assert torch.equal(lse, want_l), f"replay {i}: L differs from the eager call"
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o, want_o) and torch.equal(lse, want_l)


# --- backward over variable-length batches (fa_bwd_varlen) ------------------
def compare_bwd(lq, lk, H, D, causal, seed, dtype="bf16"):
    """Gradients against the oracle (per sequence, with the backward's
    derived bound 2u*b, u the input type's unit roundoff), 16-bit gradients
    the exact rounding of the fp32 ones, and each sequence matching fa_bwd on
    that sequence alone: bit for bit at D = 16 and 32, where both run the same
    kernels; at D = 64 and 128 fa_bwd runs the pipelined kernels (other tile
    shapes and summation orders, and P and dS can round to the neighbouring
    16-bit value), so there within u*b, half of each side's own bound."""
    from workloads import gen_grad_out

    q, k, v, cu_q, cu_k = packed(lq, lk, H, D, seed, dtype)
    g = gen_grad_out(1, H, sum(lq), D, seed=seed + 2, dtype=dtype)[0]
    scale = 1.0 / math.sqrt(D)
    maxq, maxk = max(max(lq), 1), max(lk)
    _log(f"bwd S={len(lq)} H={H} D={D} causal={causal} Tq={sum(lq)} Tk={sum(lk)}")
    qd, kd, vd, gd, cqd, ckd = (t.to(DEV) for t in (q, k, v, g, cu_q, cu_k))
    o, lse = fa.fwd_varlen(qd, kd, vd, cqd, ckd, maxq, causal=causal, scale=scale)
    g32 = fa.bwd_varlen(qd, kd, vd, o, lse, gd, cqd, ckd, maxq, maxk, causal=causal,
                        scale=scale, grad_dtype=torch.float32)
    g16 = fa.bwd_varlen(qd, kd, vd, o, lse, gd, cqd, ckd, maxq, maxk, causal=causal,
                        scale=scale)
    torch.cuda.synchronize()
    g32 = [x.cpu() for x in g32]
    g16 = [x.cpu() for x in g16]
    u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    qn, kn, vn, gn = (t.double().numpy() for t in (q, k, v, g))
    cq, ck = cu_q.tolist(), cu_k.tolist()
    for s in range(len(lq)):
        a, b, ka, kb = cq[s], cq[s + 1], ck[s], ck[s + 1]
        rows = (slice(a, b), slice(ka, kb), slice(ka, kb))
        if b == a or kb == ka:
            for n in range(3):
                assert torch.all(g32[n][:, rows[n]] == 0), f"sequence {s}: expected zeros"
            continue
        ref = oracle.attention_bwd(qn[None, :, a:b], kn[None, :, ka:kb], vn[None, :, ka:kb],
                                   gn[None, :, a:b], scale, causal, magnitudes=True)
        for n, name in enumerate(("dQ", "dK", "dV")):
            x = g32[n][:, rows[n]].double().numpy()
            r, bd = ref[n][0], ref[n + 3][0]
            bound = 2 * u * bd + 1e-6 * float(bd.max()) + 1e-30
            ratio = float((np.abs(x - r) / bound).max())
            assert ratio <= 1.0, f"sequence {s} {name}: error/bound {ratio:.3f}"
            rnd = g32[n][:, rows[n]].to(q.dtype)
            assert torch.equal(rnd, g16[n][:, rows[n]]), f"sequence {s} {name}: rounding"
        # the same sequence through the dense entry point
        so, sl = fa.fwd(qd[None, :, a:b].contiguous(), kd[None, :, ka:kb].contiguous(),
                        vd[None, :, ka:kb].contiguous(), causal=causal, scale=scale)
        one = fa.bwd(qd[None, :, a:b].contiguous(), kd[None, :, ka:kb].contiguous(),
                     vd[None, :, ka:kb].contiguous(), o[None, :, a:b].contiguous(),
                     lse[None, :, a:b].contiguous(), gd[None, :, a:b].contiguous(),
                     causal=causal, scale=scale, grad_dtype=torch.float32)
        torch.cuda.synchronize()
        for n in range(3):
            if D <= 32:
                assert torch.equal(one[n][0].cpu(), g32[n][:, rows[n]]), \
                    f"sequence {s}: gradient {n} differs from fa_bwd on the sequence alone"
            else:
                bd = ref[n + 3][0]
                d = np.abs(one[n][0].cpu().double().numpy() - g32[n][:, rows[n]].double().numpy())
                lim = u * bd + 1e-6 * float(bd.max()) + 1e-30
                assert (d <= lim).all(), \
                    f"sequence {s}: gradient {n} differs from fa_bwd on the sequence alone"


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_bwd_mixed_lengths(D, causal):
    compare_bwd(MIXED, MIXED, 2, D, causal, seed=1900 + D)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_bwd_unequal_and_empty(causal):
    compare_bwd([100, 0, 513, 40, 17], [7, 30, 200, 41, 0], 2, 128, causal, seed=2000)


def test_varlen_bwd_fp16():
    compare_bwd(MIXED, MIXED, 1, 64, True, seed=2100, dtype="f16")


def test_varlen_bwd_32k_tokens_sampled():
    """The shape bench.py --varlen 8 --pass bwd times: 32768 tokens in 8
    sequences of seeded lengths, one head, D=128, causal bf16.  Sampled query
    rows (dQ) and key rows (dK, dV) of every sequence against the oracle's
    backward on that sequence, with the backward's bound (2u times the
    oracle's magnitude sums), and 16-bit gradients the rounding of the fp32
    ones."""
    from workloads import gen_grad_out

    lens = varlen_lengths(32768, 8, seed=77, min_len=64)
    D, T = 128, 32768
    q, k, v, cu_q, cu_k = packed(lens, lens, 1, D, 3200)
    g = gen_grad_out(1, 1, T, D, seed=3202, dtype="bf16")[0]
    scale = 1.0 / math.sqrt(D)
    _log(f"bwd sampled S=8 T={T} lens={lens}")
    qd, kd, vd, gd, cqd, ckd = (t.to(DEV) for t in (q, k, v, g, cu_q, cu_k))
    o, lse = fa.fwd_varlen(qd, kd, vd, cqd, ckd, max(lens), causal=True, scale=scale)
    g32 = fa.bwd_varlen(qd, kd, vd, o, lse, gd, cqd, ckd, max(lens), max(lens), causal=True,
                        scale=scale, grad_dtype=torch.float32)
    g16 = fa.bwd_varlen(qd, kd, vd, o, lse, gd, cqd, ckd, max(lens), max(lens), causal=True,
                        scale=scale)
    torch.cuda.synchronize()
    g32 = [x.cpu()[0] for x in g32]
    g16 = [x.cpu()[0] for x in g16]
    qn, kn, vn, gn = (t.double().numpy() for t in (q, k, v, g))
    u = 2.0 ** -8
    r = np.random.default_rng(3203)
    cq = cu_q.tolist()
    for s in range(8):
        a, b = cq[s], cq[s + 1]
        n = b - a
        pick = np.unique(np.concatenate([r.integers(0, n, 32), [0, n - 1]]))
        ref = oracle.attention_bwd(qn[None, :, a:b], kn[None, :, a:b], vn[None, :, a:b],
                                   gn[None, :, a:b], scale, True, qrows=pick, krows=pick,
                                   magnitudes=True)
        for m, name in enumerate(("dQ", "dK", "dV")):
            x = g32[m][a + pick].double().numpy()
            bd = ref[m + 3]
            bound = 2 * u * bd + 1e-6 * float(bd.max()) + 1e-30
            ratio = float((np.abs(x - ref[m]) / bound).max())
            assert ratio <= 1.0, f"sequence {s} {name}: error/bound {ratio:.3f}"
            assert torch.equal(g32[m][a + pick].to(torch.bfloat16), g16[m][a + pick]), \
                f"sequence {s} {name}: rounding"
        _log(f"  sequence {s} ({n} tokens): {len(pick)} rows ok")


def test_varlen_split_chunk_cap_leaves_no_chunk_empty():
    """One 128-row sequence against 8256 keys, non-causal, with
    max_seqlen_k = 8256: the split plan caps the tile at 16 chunks of 9 key
    tiles, which cover its 129 key tiles with 15, so the 16th must neither
    run nor be merged.  The workspace is filled with NaN bytes first, so a
    merged empty chunk would show."""
    lq, lk = [128], [8256]
    H, D = 1, 128
    q, k, v, cu_q, cu_k = (t.to(DEV) for t in packed(lq, lk, H, D, 3300))
    code = fa._dtype_code(torch, q.dtype, torch.float32)
    st, nb = fa.fa_fwd_varlen_workspace_size(1, H, 128, 8256, 128, 8256, D, False, code)
    assert st == fa.FA_OK and nb > 0
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=DEV)
    o = torch.empty((H, 128, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((H, 128), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(D)
    st = fa.fa_fwd_varlen_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), cu_q.data_ptr(), cu_k.data_ptr(), 1, H, 128, 8256,
                             128, 8256, D, scale, False, code, ws.data_ptr(), nb,
                             torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_str(st)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(q.cpu().double().numpy()[None], k.cpu().double().numpy()[None],
                              v.cpu().double().numpy()[None], scale, False)
    err_o = float(np.abs(o.cpu().double().numpy() - ro[0]).max())
    err_l = float(np.abs(lse.cpu().double().numpy() - rl[0]).max())
    _log(f"chunk cap: O {err_o:.3e} L {err_l:.3e}")
    assert err_o <= 1e-2 and err_l <= 1e-3
    # and the same through the Python binding
    compare(lq, lk, H, D, False, seed=3300, maxk=8256)


def test_varlen_rows_past_max_seqlen_q_are_nan():
    """A sequence longer than max_seqlen_q: rows up to the end of the query
    tile holding row max_seqlen_q - 1 (256-row tiles at D = 64) are computed
    exactly, the rest get O = NaN and lse = NaN; the other sequence is
    unaffected."""
    lq, lk = [1000, 50], [1000, 50]
    q, k, v, cu_q, cu_k = packed(lq, lk, 1, 64, 3400)
    scale = 0.125
    full = run(q, k, v, cu_q, cu_k, 1000, True, scale, torch.float32)
    short = run(q, k, v, cu_q, cu_k, 100, True, scale, torch.float32)
    assert torch.equal(short[0][:, :256], full[0][:, :256])
    assert torch.equal(short[1][:, :256], full[1][:, :256])
    assert torch.isnan(short[0][:, 256:1000]).all() and torch.isnan(short[1][:, 256:1000]).all()
    assert torch.equal(short[0][:, 1000:], full[0][:, 1000:])
    assert torch.equal(short[1][:, 1000:], full[1][:, 1000:])


def test_varlen_bwd_rows_past_bounds_are_nan():
    """Sequences longer than max_seqlen_q / max_seqlen_k in the backward:
    dq rows past the 64-row tile holding row max_seqlen_q - 1, and dk, dv
    rows past the tile holding key max_seqlen_k - 1, are NaN; every other row
    equals the run with true bounds bit for bit."""
    lq, lk = [300, 20], [400, 30]
    H, D = 1, 64
    q, k, v, cu_q, cu_k = (t.to(DEV) for t in packed(lq, lk, H, D, 3500))
    from workloads import gen_grad_out

    g = gen_grad_out(1, H, sum(lq), D, seed=3501, dtype="bf16")[0].to(DEV)
    o, lse = fa.fwd_varlen(q, k, v, cu_q, cu_k, 300, causal=False, scale=0.125)
    full = fa.bwd_varlen(q, k, v, o, lse, g, cu_q, cu_k, 300, 400, causal=False, scale=0.125,
                         grad_dtype=torch.float32)
    short = fa.bwd_varlen(q, k, v, o, lse, g, cu_q, cu_k, 100, 70, causal=False, scale=0.125,
                          grad_dtype=torch.float32)
    torch.cuda.synchronize()
    full = [x.cpu() for x in full]
    short = [x.cpu() for x in short]
    # dq: rows 0..127 computed, 128..299 NaN, the second sequence (300..319) whole
    assert torch.equal(short[0][:, :128], full[0][:, :128])
    assert torch.isnan(short[0][:, 128:300]).all()
    assert torch.equal(short[0][:, 300:], full[0][:, 300:])
    for m in (1, 2):  # dk, dv: keys 0..127 computed, 128..399 NaN, 400..429 whole
        assert torch.equal(short[m][:, :128], full[m][:, :128])
        assert torch.isnan(short[m][:, 128:400]).all()
        assert torch.equal(short[m][:, 400:], full[m][:, 400:])
