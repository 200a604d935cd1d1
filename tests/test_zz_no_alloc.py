"""GPU test of fa_fwd_noalloc (the entry point that allocates nothing: its
stream-K partials live in a scratch array inside the library), through the
C ABI.  Two calls in a row, the second on a smaller problem, each checked
bit for bit against fa_fwd_ws (the same kernels with a caller workspace)
and against the fp64 oracle at the forward's tolerance; the scratch keeps
the first call's contents when the second runs."""
import math

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_07_amd as fa
from workloads import gen_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run_both(B, H, N, D, causal, seed):
    q, k, v = gen_qkv(B, H, N, N, D, seed=seed, dtype="bf16")
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    scale = 1.0 / math.sqrt(D)
    code = fa.FA_BF16_OF32
    stream = torch.cuda.current_stream().cuda_stream
    st, nb = fa.fa_fwd_workspace_size(B, H, N, N, D, causal, code)
    assert st == fa.FA_OK
    assert 0 < nb <= fa.FA_NOALLOC_SCRATCH_BYTES, "the case must use the stream-K scratch"
    o1 = torch.full((B, H, N, D), float("nan"), dtype=torch.float32, device=DEV)
    l1 = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
    st = fa.fa_fwd_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o1.data_ptr(),
                           l1.data_ptr(), B, H, N, N, D, scale, causal, code, stream)
    assert st == fa.FA_OK, fa.fa_status_str(st)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    st = fa.fa_fwd_ws(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                      B, H, N, N, D, scale, causal, code, ws.data_ptr(), nb, stream)
    assert st == fa.FA_OK, fa.fa_status_str(st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), "O differs from fa_fwd_ws"
    assert torch.equal(l1, l2), "L differs from fa_fwd_ws"
    rows = np.arange(0, B * H * N, max(1, B * H * N // 512))
    ro, rl = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale,
                              causal, rows=rows)
    err_o = float(np.abs(o1.cpu().double().numpy().reshape(-1, D)[rows] - ro).max())
    err_l = float(np.abs(l1.cpu().double().numpy().reshape(-1)[rows] - rl).max())
    print(f"[noalloc] B={B} H={H} N={N} D={D} causal={causal} scratch {nb} bytes: "
          f"O {err_o:.2e} L {err_l:.2e}", flush=True)
    assert err_o <= 1e-2 and err_l <= 1e-3


def test_noalloc_two_calls_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.library()
    # the B8 N4096 D128 causal workload (34.6 MB of scratch), then a smaller
    # ragged one (15.1 MB): the second call runs over the first one's contents
    _run_both(8, 1, 4096, 128, True, seed=4100)
    _run_both(1, 1, 1000, 128, True, seed=4101)
