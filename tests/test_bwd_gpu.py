"""GPU parity of the backward pass (fa_bwd, through the C ABI) against the
fp64 CPU oracle's chain-rule gradients.

The forward pass runs first on the GPU (fa_fwd_ws, 16-bit O as the pages
store it), and its O and L are what fa_bwd consumes; the oracle
differentiates the exact forward from q, k, v and dO alone.

Tolerance (no figure is given for gradients, so it is derived from the
arithmetic).  Every product on the GPU has 16-bit operands and an fp32 sum;
one factor of each product is rounded from fp32 (P for dV, dS for dQ and
dK), and the row term <dO_i, O_i> uses the forward's O, whose error from
rounding P is at most a unit roundoff u times sum_j P_ij |v_j| per element.
That bounds every gradient element by u times the oracle's magnitude sum of
the same element (bq, bk, bv: the gradient's sum taken over absolute values,
with the row term's sensitivity included), so the test requires

    |grad_gpu - grad_ref| <= 2 u b + 1e-6 max(b)      (fp32 gradients)

with u = 2^-8 for bf16 and 2^-11 for fp16 inputs; the factor 2 covers the
fp32 sums and the second-order terms.  16-bit gradients must be exactly the
round-to-nearest-even of the fp32 gradients of the same call inputs (the
same kernels, another store) and within that bound plus half an ulp of the
storage type.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_07_amd as fa
from workloads import gen_grad_out, gen_qkv, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
UNIT = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def _log(msg):
    print(f"[bwd] {msg}", flush=True)


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


def gpu_grads(q, k, v, g, causal, scale, grad_dtype):
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, gd, causal=causal, scale=scale,
                        grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return [t.double().cpu().numpy() for t in (dq, dk, dv)]


def compare(q, k, v, g, causal, scale, qrows=None, krows=None, what=""):
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    _log(f"{what} B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} scale={scale:.4g} "
         f"dtype={q.dtype} rows={'all' if qrows is None else (len(qrows), len(krows))}")
    ref = oracle.attention_bwd(*(t.double().numpy() for t in (q, k, v, g)), scale, causal,
                               qrows=qrows, krows=krows, magnitudes=True)
    u = UNIT[q.dtype]
    g32 = gpu_grads(q, k, v, g, causal, scale, torch.float32)
    g16 = gpu_grads(q, k, v, g, causal, scale, q.dtype)
    sels = (qrows, krows, krows)
    for n, name in enumerate(("dQ", "dK", "dV")):
        r, b = ref[n].reshape(-1, D), ref[n + 3].reshape(-1, D)
        sel = slice(None) if sels[n] is None else np.asarray(sels[n])
        x32 = g32[n].reshape(-1, D)[sel]
        x16 = g16[n].reshape(-1, D)[sel]
        assert np.isfinite(x32).all(), f"{name}: non-finite gradient"
        bound = 2 * u * b + 1e-6 * float(b.max()) + 1e-30
        err = np.abs(x32 - r)
        ratio = float((err / bound).max())
        _log(f"  {name}: max-abs {float(err.max()):.3e}  max |ref| "
             f"{float(np.abs(r).max()):.3e}  worst error/bound {ratio:.3f}")
        assert ratio <= 1.0, f"{name}: error exceeds 2u*b (worst ratio {ratio:.3f})"
        rounded = torch.from_numpy(x32).to(q.dtype).double().numpy()
        mism = int((rounded != x16).sum())
        assert mism == 0, f"{name}: {mism} 16-bit gradients differ from RNE of fp32 ones"
        err16 = np.abs(x16 - r)
        assert (err16 <= bound + _half_ulp(r, q.dtype)).all(), f"{name}: 16-bit bound"


def inputs(B, H, Nq, Nk, D, seed, dtype=torch.bfloat16, q_mult=1.0, std=1.0):
    name = {torch.bfloat16: "bf16", torch.float16: "f16"}[dtype]
    q, k, v = gen_qkv(B, H, Nq, Nk, D, seed=seed, dtype=name, q_mult=q_mult, std=std)
    g = gen_grad_out(B, H, Nq, D, seed=seed + 10000, dtype=name)
    return q, k, v, g


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_bwd_ragged_tiles(D, causal, dtype):
    """Several 128-row tiles and a ragged tail in both sequences."""
    q, k, v, g = inputs(2, 3, 300, 300, D, seed=600 + D, dtype=dtype)
    compare(q, k, v, g, causal, 1.0 / math.sqrt(D), what="ragged")


@pytest.mark.parametrize("Nq,Nk", [(129, 400), (400, 129), (500, 77), (33, 1000)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_unequal_lengths(Nq, Nk, causal):
    q, k, v, g = inputs(1, 2, Nq, Nk, 64, seed=700 + Nq)
    compare(q, k, v, g, causal, 0.125, what="Nq!=Nk")


@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 7), (5, 3), (31, 33), (32, 32), (65, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_tiny(Nq, Nk, causal):
    """Single rows and keys, partial 32-row blocks, a single key (dQ = dK = 0)."""
    q, k, v, g = inputs(2, 1, Nq, Nk, 32, seed=800 + 10 * Nq + Nk)
    compare(q, k, v, g, causal, 1.0 / math.sqrt(32), what="tiny")


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.3])
def test_bwd_scales(scale):
    """scale 0 (uniform P over the visible keys), a negative and a large scale."""
    q, k, v, g = inputs(1, 2, 200, 200, 128, seed=900)
    compare(q, k, v, g, True, scale, what="scale")


def test_bwd_large_logits():
    """q scaled by 8: near one-hot rows, P close to 0 or 1."""
    q, k, v, g = inputs(1, 2, 256, 256, 128, seed=901, q_mult=8.0)
    compare(q, k, v, g, True, 1.0 / math.sqrt(128), what="q x 8")


@pytest.mark.parametrize("q_mult", [1.0, 8.0])
def test_bwd_headline_sampled(q_mult):
    """B8 N4096 D128 causal bf16, the forward's headline shape: 256 sampled
    query rows (dQ) and 256 sampled key rows (dK, dV) against the oracle."""
    B, N, D = 8, 4096, 128
    q, k, v, g = inputs(B, 1, N, N, D, seed=3, q_mult=q_mult)
    qrows = sample_rows(B * N, 256, 6000).numpy()
    krows = sample_rows(B * N, 256, 6001).numpy()
    compare(q, k, v, g, True, 1.0 / math.sqrt(D), qrows=qrows, krows=krows,
            what="headline sampled")


def test_bwd_multihead_sampled():
    """B1 H64 N8192 D128 causal, N(0, 0.5^2): sampled rows."""
    B, H, N, D = 1, 64, 8192, 128
    q, k, v, g = inputs(B, H, N, N, D, seed=5, std=0.5)
    heads = np.array([3, 17, 42, 63])  # rows from four heads keep the oracle short
    qrows = (heads[:, None] * N + sample_rows(N, 32, 6002).numpy()[None]).reshape(-1)
    krows = (heads[:, None] * N + sample_rows(N, 32, 6003).numpy()[None]).reshape(-1)
    compare(q, k, v, g, True, 1.0 / math.sqrt(D), qrows=qrows, krows=krows,
            what="64 heads sampled")


def test_bwd_deterministic():
    """Two calls give bit-identical gradients (plain stores, no atomics)."""
    q, k, v, g = inputs(2, 2, 700, 700, 128, seed=902)
    a = gpu_grads(q, k, v, g, True, 0.088, torch.float32)
    b = gpu_grads(q, k, v, g, True, 0.088, torch.float32)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("shape", [(2, 2, 700, 700, 128), (8, 1, 1024, 1024, 64),
                                   (1, 3, 300, 1300, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_dq_stream_and_grid(shape, causal):
    """dQ at D = 64 and 128 runs the stream-K schedule of 128-row tiles when
    the workspace holds its partial sums (the size fa_bwd_workspace_size
    reports) and one workgroup per tile when it holds only the row terms;
    so do dK and dV where their schedule applies (non-causal, or causal with
    Nq = Nk a multiple of 128), else both runs take the 64-key kernel: both
    against the oracle's bound, and within a few fp32 roundings of each
    other (the sums run in a different order)."""
    B, H, Nq, Nk, D = shape
    q, k, v, g = inputs(B, H, Nq, Nk, D, seed=950 + Nq)
    scale = 1.0 / math.sqrt(D)
    st, full = fa.fa_bwd_workspace_size(B, H, Nq, Nk, D, causal, fa.FA_BF16_OF32)
    assert st == fa.FA_OK and full > B * H * Nq * 4, "no stream schedule for dQ"
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale)
    res = []
    for nbytes in (full, B * H * Nq * 4):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        grads = [torch.empty(t.shape, dtype=torch.float32, device=DEV) for t in (qd, kd, vd)]
        st = fa.fa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       gd.data_ptr(), *(t.data_ptr() for t in grads), B, H, Nq, Nk, D, scale,
                       int(causal), fa.FA_BF16_OF32, ws.data_ptr(), nbytes,
                       torch.cuda.current_stream().cuda_stream)
        assert st == fa.FA_OK, fa.fa_status_str(st)
        torch.cuda.synchronize()
        res.append([t.double().cpu().numpy() for t in grads])
    ref = oracle.attention_bwd(*(t.double().numpy() for t in (q, k, v, g)), scale, causal,
                               magnitudes=True)
    u = UNIT[q.dtype]
    for which, grads in zip(("stream", "grid"), res):
        for n, name in enumerate(("dQ", "dK", "dV")):
            r, b = ref[n].reshape(-1, D), ref[n + 3].reshape(-1, D)
            err = np.abs(grads[n].reshape(-1, D) - r)
            ratio = float((err / (2 * u * b + 1e-6 * float(b.max()) + 1e-30)).max())
            _log(f"  {which} {name}: max-abs {float(err.max()):.3e} worst error/bound {ratio:.3f}")
            assert ratio <= 1.0, f"{which} {name}: error exceeds 2u*b ({ratio:.3f})"
    for n in range(3):
        d = np.abs(res[0][n] - res[1][n])
        assert float(d.max()) <= 1e-5 * max(1.0, float(np.abs(res[1][n]).max())), float(d.max())
    if causal and (Nq != Nk or Nq % 128):  # the same dK/dV kernel both times
        assert np.array_equal(res[0][1], res[1][1]) and np.array_equal(res[0][2], res[1][2])


@pytest.mark.parametrize("shape,causal", [
    ((2, 3, 1024, 1024, 128), True),   # 48 tiles over 256 chunks: most cut many times
    ((1, 1, 128, 128, 64), True),      # one tile, two pieces
    ((1, 2, 640, 640, 64), True),
    ((1, 2, 77, 333, 64), False),      # ragged keys and queries
    ((3, 1, 500, 300, 128), False),
])
def test_bwd_dkv_stream_shapes(shape, causal):
    """dK and dV on the stream-K schedule of 128-key tiles (fewer than two
    per compute unit): key tiles split into pieces over query tiles, each
    cut tile's partial sums added in piece order by the merge kernel; every
    row against the oracle."""
    B, H, Nq, Nk, D = shape
    q, k, v, g = inputs(B, H, Nq, Nk, D, seed=990 + Nq + D)
    compare(q, k, v, g, causal, 1.0 / math.sqrt(D), what="dK/dV stream")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_many_key_tiles(D, causal):
    """B2 H128, Nq = 200 against Nk = 250: 512 tiles of 128 keys, so dK and
    dV run one workgroup per 128-key tile of the pipelined kernel (Q, dO and
    their row terms streamed through the DMA ring), ragged query and key
    tails, every row against the oracle."""
    q, k, v, g = inputs(2, 128, 200, 250, D, seed=970 + D)
    compare(q, k, v, g, causal, 1.0 / math.sqrt(D), what="512 key tiles")


def test_bwd_rejects_fp32_and_odd_head_dims():
    q = torch.zeros(1, 1, 64, 48, device=DEV, dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 64, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.bwd(q, q, q, q, lse, q, causal=True)
    assert e.value.status == fa.FA_ERR_HEAD_DIM
    x = torch.zeros(1, 1, 64, 64, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.bwd(x, x, x, x, lse, x)  # fp32 inputs: not supported by the backward pass
    assert e.value.status == fa.FA_ERR_DTYPE


def test_bwd_d16_sweep_shape_sampled():
    """B8 N8192 D16 causal bf16 (a head dim of the pages' sweep): sampled rows."""
    B, N, D = 8, 8192, 16
    q, k, v, g = inputs(B, 1, N, N, D, seed=40)
    qrows = sample_rows(B * N, 128, 6010).numpy()
    krows = sample_rows(B * N, 128, 6011).numpy()
    compare(q, k, v, g, True, 1.0 / math.sqrt(D), qrows=qrows, krows=krows,
            what="D16 sampled")


@pytest.mark.parametrize("entry", ["bwd", "bwd_stream", "bwd_masked", "fwd_varlen",
                                   "fwd_masked"])
def test_graph_capture_replays_match_eager(entry):
    """fa_bwd, fa_bwd_masked, fa_fwd_varlen and fa_fwd_masked are plain
    launches on the caller's stream (no allocation, no memset), so a HIP
    graph captured around one call replays it: every replay, with eager work
    between replays and stale outputs and workspace, gives the eager result
    bit for bit."""
    B, H, N, D = 2, 2, 333, 64
    q, k, v, g = inputs(B, H, N, N, D, seed=903)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    scale = 0.125
    o, lse = fa.fwd(qd, kd, vd, causal=True, scale=scale)
    outs = [torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)]
    nws = B * H * N * 4
    if entry == "bwd_stream":  # room for the stream schedule's dQ partial sums
        nws = fa.fa_bwd_workspace_size(B, H, N, N, D, 1, fa.FA_BF16)[1]
        assert nws > B * H * N * 4
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    cu = torch.tensor([0, 100, 333, 2 * N], dtype=torch.int32, device=DEV)
    stream = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
    if entry in ("bwd", "bwd_stream", "bwd_masked"):
        if entry == "bwd_masked":
            o, lse = fa.fwd_masked(qd, kd, vd, 40, 5, causal=True, scale=scale)

        def call():
            base = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                    lse.data_ptr(), gd.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(),
                    outs[2].data_ptr(), B, H, N, N, D, scale, 1)
            if entry in ("bwd", "bwd_stream"):
                st = fa.fa_bwd(*base, fa.FA_BF16, ws.data_ptr(), ws.numel(), stream())
            else:
                st = fa.fa_bwd_masked(*base, 40, 5, fa.FA_BF16, ws.data_ptr(), ws.numel(),
                                      stream())
            assert st == fa.FA_OK, fa.fa_status_str(st)
    else:
        outs = [torch.empty_like(qd), torch.empty(qd.shape[:-1], dtype=torch.float32,
                                                  device=DEV)]

        def call():
            if entry == "fwd_varlen":
                # q viewed as [2, 666, D]: two heads of 666 packed tokens, three sequences
                st = fa.fa_fwd_varlen(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                      outs[0].data_ptr(), outs[1].data_ptr(), cu.data_ptr(),
                                      cu.data_ptr(), 3, B * H // 2, 2 * N, 2 * N, 333, D, scale,
                                      1, fa.FA_BF16, stream())
            else:
                st = fa.fa_fwd_masked(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                      outs[0].data_ptr(), outs[1].data_ptr(), B, H, N, N, D,
                                      scale, 1, 40, 5, fa.FA_BF16, stream())
            assert st == fa.FA_OK, fa.fa_status_str(st)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    want = [x.clone() for x in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(3):
        for x in outs:
            x.fill_(float("nan"))
        ws.fill_(i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip(outs, want):
            assert torch.equal(x, y), f"replay {i} differs from the eager call"
        call()
        torch.cuda.synchronize()
