"""GPU parity of the FP8 forward (fa_fwd_fp8 and fa_fwd_fp8_ws, the
pipelined kernel, through the C ABI; every case runs both).  The
operation is fa_fwd's on the dequantized inputs (e4m3 values times their
per-tensor factors), so the oracle is the dense fp64 oracle applied to
those real values, and the tolerance is the 16-bit path's: the products of
e4m3 values are exact in fp32 and V widens exactly to bf16, leaving P's
rounding to bf16 and fp32 sums: fp32 O <= 1e-2, L <= 1e-3; bf16 O the
exact rounding of the fp32 O and within 1e-2 plus half an ulp."""
import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_07_amd as fa
from workloads import gen_qkv_fp8, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()
    oracle.load()


def compare(B, H, Nq, Nk, D, causal, seed, rows=None, q_mult=1.0, scale=None,
            descales=None):
    q8, k8, v8, (sq, sk, sv) = gen_qkv_fp8(B, H, Nq, Nk, D, seed, q_mult=q_mult)
    if descales is not None:
        sq, sk, sv = descales
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    real = [t.double().numpy() * s for t, s in ((q8, sq), (k8, sk), (v8, sv))]
    ro, rl = oracle.attention(*real, scale, causal, rows=rows)
    sel = slice(None) if rows is None else torch.as_tensor(rows)
    ro, rl = ro.reshape(-1, D), rl.reshape(-1)
    qd, kd, vd = q8.to(DEV), k8.to(DEV), v8.to(DEV)
    for ws in (False, True):
        print(f"[fp8] B={B} H={H} Nq={Nq} Nk={Nk} D={D} causal={causal} ws={ws} "
              f"rows={'all' if rows is None else len(rows)}", flush=True)
        o32, l32 = fa.fwd_fp8(qd, kd, vd, sq, sk, sv, causal=causal, scale=scale,
                              out_dtype=torch.float32, ws=ws)
        o16, l16 = fa.fwd_fp8(qd, kd, vd, sq, sk, sv, causal=causal, scale=scale, ws=ws)
        torch.cuda.synchronize()
        g_o = o32.reshape(-1, D)[sel].double().cpu().numpy()
        g_l = l32.reshape(-1)[sel].double().cpu().numpy()
        err_o = float(np.abs(g_o - ro).max())
        err_l = float(np.abs(g_l - rl).max())
        print(f"[fp8]   fp32-O max-abs O {err_o:.3e} L {err_l:.3e}", flush=True)
        assert err_o <= 1e-2 and err_l <= 1e-3
        x16 = o16.reshape(-1, D)[sel].double().cpu().numpy()
        assert np.array_equal(torch.from_numpy(g_o).to(torch.bfloat16).double().numpy(), x16)
        mant = 7
        e = np.floor(np.log2(np.maximum(np.abs(ro), 2.0 ** -14)))
        assert (np.abs(x16 - ro) <= 1e-2 + 2.0 ** (e - mant - 1)).all()
        assert torch.equal(l16.reshape(-1)[sel], l32.reshape(-1)[sel])


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_ragged(D, causal):
    compare(2, 2, 700, 700, D, causal, seed=3000 + D)


@pytest.mark.parametrize("Nq,Nk", [(1, 1), (129, 400), (400, 129), (31, 33)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_shapes(Nq, Nk, causal):
    compare(1, 2, Nq, Nk, 128, causal, seed=3100 + Nq)


def test_fp8_large_logits():
    compare(1, 2, 512, 512, 128, True, seed=3200, q_mult=8.0)


def test_fp8_headline_shape_sampled():
    """B8 N4096 D128 causal (the headline shape, FP8 inputs): 512 sampled rows."""
    rows = sample_rows(8 * 4096, 512, 3300).numpy()
    compare(8, 1, 4096, 4096, 128, True, seed=3, rows=rows)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_many_tiles_sampled(causal):
    """B1 H64 N1024 D128: 512 tiles of 128 rows, enough to fill every
    workgroup slot, so the 128-row layout runs (smaller grids take the
    pair-split 64-row layout): 512 sampled rows."""
    rows = sample_rows(64 * 1024, 512, 3400 + int(causal)).numpy()
    compare(1, 64, 1024, 1024, 128, causal, seed=3401, rows=rows)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_negative_scale_and_descales(causal):
    """A negative scale (the pipelined kernel flips Q's e4m3 sign bits) and
    negative descale factors (q and v) against the oracle on the same real
    inputs."""
    compare(1, 2, 300, 520, 128, causal, seed=3500, scale=-0.07,
            descales=(-0.011, 0.013, -0.021))


@pytest.mark.parametrize("shape", [(2, 3, 777, 1300, 64), (1, 1, 2048, 2048, 128),
                                   (3, 1, 129, 4000, 128)])
def test_fp8_stream_schedule_shapes(shape):
    """Shapes that take the stream-K schedule on the pipelined kernel (cut
    query tiles combined by the merge): both masks, every row."""
    B, H, Nq, Nk, D = shape
    st, nb = fa.fa_fwd_fp8_workspace_size(B, H, Nq, Nk, D, 1, 0)
    assert st == fa.FA_OK and nb > ((B * H * Nk * D * 2 + 255) // 256) * 256, "no schedule"
    for causal in (False, True):
        compare(B, H, Nq, Nk, D, causal, seed=3600 + Nq)


def test_fp8_ws_contract():
    """Missing, short, misaligned or overlapping scratch is refused before
    any launch; D outside {64, 128} is refused by the size query too."""
    B, H, N, D = 1, 2, 512, 128
    q8, k8, v8, (sq, sk, sv) = gen_qkv_fp8(B, H, N, N, D, 1)
    qd, kd, vd = q8.to(DEV), k8.to(DEV), v8.to(DEV)
    o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    st, need = fa.fa_fwd_fp8_workspace_size(B, H, N, N, D, 1, 0)
    assert st == fa.FA_OK and need >= B * H * N * D * 2
    assert fa.fa_fwd_fp8_workspace_size(B, H, N, N, 32, 1, 0)[0] == fa.FA_ERR_HEAD_DIM
    ws = torch.empty(need + 64, dtype=torch.uint8, device=DEV)
    sp = torch.cuda.current_stream().cuda_stream
    args = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N,
            N, D, 0.1, sq, sk, sv, 1, 0)
    assert fa.fa_fwd_fp8_ws(*args, None, 0, sp) == fa.FA_ERR_WORKSPACE
    assert fa.fa_fwd_fp8_ws(*args, ws.data_ptr(), need - 1, sp) == fa.FA_ERR_WORKSPACE
    assert fa.fa_fwd_fp8_ws(*args, ws.data_ptr() + 8, need, sp) == fa.FA_ERR_ALIGN
    assert fa.fa_fwd_fp8_ws(*args, o.data_ptr(), need, sp) == fa.FA_ERR_OVERLAP
    assert fa.fa_fwd_fp8_ws(*args, ws.data_ptr(), need, sp) == fa.FA_OK
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_grid_path_sampled(D):
    """B1 H64 N2048: four 128-row tiles per compute unit of a 256-unit
    device, so fa_fwd_fp8_ws takes one workgroup per 256-row tile (no
    stream-K schedule): 512 sampled rows, both masks."""
    st, nb = fa.fa_fwd_fp8_workspace_size(1, 64, 2048, 2048, D, 1, 0)
    assert st == fa.FA_OK
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    if cus == 256:
        assert nb == ((64 * 2048 * D * 2 + 255) // 256) * 256, "expected the grid path"
    rows = sample_rows(64 * 2048, 512, 3700 + D).numpy()
    for causal in (False, True):
        compare(1, 64, 2048, 2048, D, causal, seed=3701 + D, rows=rows)
