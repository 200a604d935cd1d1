"""CPU tests of the C ABI: libfa.so loads without a GPU, exports every symbol
include/fa.h declares, its constants match the header, and every validation
error is returned before any device work (the pointers below are never
dereferenced: each call fails validation first)."""
import math
import os
import re

import pytest

import transformer_attention_07_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# Fake, 256-byte aligned, never-dereferenced device addresses.
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def _header_text():
    with open(HEADER) as f:
        return f.read()


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def _header_enums():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return {name: int(val) for name, val in re.findall(r"\b(FA_[A-Z0-9_]+)\s*=\s*(\d+)", text)}


def call(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Nq=100, Nk=90, D=64, scale=0.125,
             causal=1, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                     a["Nk"], a["D"], a["scale"], a["causal"], a["dtype"], a["stream"])


def test_library_loads_and_exports_every_declared_symbol():
    lib = fa.library()
    declared = _declared_functions()
    assert set(declared) == set(fa.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), f"libfa.so does not export {name}"


def test_constants_match_header():
    enums = _header_enums()
    for name, val in enums.items():
        assert getattr(fa, name) == val, name
    assert len(enums) == 15


def test_version_and_status_strings():
    assert fa.fa_version() >= 100
    for s in range(10):
        assert fa.fa_status_str(s)
    assert fa.fa_status_str(1234) == "unknown status"
    assert fa.fa_last_hip_error() == ""


@pytest.mark.parametrize("field", ["q", "k", "v", "o", "lse"])
def test_null_pointer(field):
    assert call(**{field: None}) == fa.FA_ERR_NULLPTR


@pytest.mark.parametrize("field,val", [("B", 0), ("H", 0), ("Nq", 0), ("Nk", 0),
                                       ("B", -1), ("Nk", -5)])
def test_bad_shape(field, val):
    assert call(**{field: val}) == fa.FA_ERR_SHAPE


def test_too_large_for_32bit_slice_offsets():
    assert call(Nq=1 << 22, D=128) == fa.FA_ERR_SHAPE
    assert call(Nk=1 << 22, D=128) == fa.FA_ERR_SHAPE


@pytest.mark.parametrize("d", [0, 8, 48, 96, 256, -16])
def test_bad_head_dim(d):
    assert call(D=d) == fa.FA_ERR_HEAD_DIM


@pytest.mark.parametrize("dt", [-1, 5, 99])
def test_bad_dtype(dt):
    assert call(dtype=dt) == fa.FA_ERR_DTYPE


@pytest.mark.parametrize("s", [math.inf, -math.inf, math.nan])
def test_bad_scale(s):
    assert call(scale=s) == fa.FA_ERR_SCALE


@pytest.mark.parametrize("field,val", [("q", Q + 8), ("k", K + 2), ("v", V + 4),
                                       ("o", O + 12), ("lse", L + 2)])
def test_misaligned(field, val):
    assert call(**{field: val}) == fa.FA_ERR_ALIGN


def test_lse_needs_only_four_byte_alignment_check_passes_to_overlap():
    # lse at +4 is aligned enough; make it overlap o so the call stops before
    # any launch and the status proves the alignment check was passed.
    assert call(lse=O + 4) == fa.FA_ERR_OVERLAP


@pytest.mark.parametrize("o,lse", [(Q, L), (Q + 4096, L), (O, K + 64), (O, V),
                                   (K - 16, L)])
def test_outputs_must_not_overlap(o, lse):
    assert call(o=o, lse=lse) == fa.FA_ERR_OVERLAP


def call_ws(ws=O + (1 << 24), ws_bytes=1 << 20, **kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Nq=100, Nk=90, D=64, scale=0.125,
             causal=1, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd_ws(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                        a["Nk"], a["D"], a["scale"], a["causal"], a["dtype"], ws, ws_bytes,
                        a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), "FA_ERR_NULLPTR"), (dict(Nq=0), "FA_ERR_SHAPE"),
    (dict(D=48), "FA_ERR_HEAD_DIM"), (dict(dtype=7), "FA_ERR_DTYPE"),
    (dict(scale=math.nan), "FA_ERR_SCALE"), (dict(k=K + 2), "FA_ERR_ALIGN"),
    (dict(lse=O + 4), "FA_ERR_OVERLAP"),
])
def test_ws_entry_validates_like_fa_fwd(kw, want):
    assert call_ws(**kw) == getattr(fa, want)


@pytest.mark.parametrize("ws,want", [(O + (1 << 24) + 8, "FA_ERR_ALIGN"),
                                     (Q + 256, "FA_ERR_OVERLAP"), (L - 64, "FA_ERR_OVERLAP"),
                                     (V - 16, "FA_ERR_OVERLAP")])
def test_workspace_alignment_and_overlap(ws, want):
    assert call_ws(ws=ws) == getattr(fa, want)


@pytest.mark.parametrize("kw,want", [(dict(B=0), "FA_ERR_SHAPE"), (dict(Nk=-1), "FA_ERR_SHAPE"),
                                     (dict(D=80), "FA_ERR_HEAD_DIM"),
                                     (dict(dtype=5), "FA_ERR_DTYPE")])
def test_workspace_size_validation(kw, want):
    a = dict(B=2, H=3, Nq=100, Nk=90, D=64, causal=1, dtype=fa.FA_BF16)
    a.update(kw)
    st, n = fa.fa_fwd_workspace_size(**a)
    assert st == getattr(fa, want) and n == 0


def test_workspace_size_null_output():
    lib = fa.library()
    assert lib.fa_fwd_workspace_size(1, 1, 64, 64, 64, 0, fa.FA_BF16, None) == \
        fa.FA_ERR_NULLPTR


# --- fa_bwd: every validation error precedes device work -------------------
DO, DQ, DK, DV, WS = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000


def call_bwd(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, B=2, H=3, Nq=100,
             Nk=90, D=64, scale=0.125, causal=1, dtype=fa.FA_BF16, ws=WS, ws_bytes=1 << 20,
             stream=None)
    a.update(kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                     a["dv"], a["B"], a["H"], a["Nq"], a["Nk"], a["D"], a["scale"],
                     a["causal"], a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("arg", ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"])
def test_bwd_null_pointers(arg):
    assert call_bwd(**{arg: None}) == fa.FA_ERR_NULLPTR


@pytest.mark.parametrize("kw,status", [
    ({"B": 0}, "FA_ERR_SHAPE"), ({"Nq": 0}, "FA_ERR_SHAPE"), ({"Nk": -1}, "FA_ERR_SHAPE"),
    ({"D": 8}, "FA_ERR_HEAD_DIM"), ({"D": 96}, "FA_ERR_HEAD_DIM"),
    ({"dtype": 0}, "FA_ERR_DTYPE"), ({"dtype": 5}, "FA_ERR_DTYPE"),
    ({"scale": math.inf}, "FA_ERR_SCALE"), ({"scale": math.nan}, "FA_ERR_SCALE"),
    ({"dq": DQ + 8}, "FA_ERR_ALIGN"), ({"do": DO + 2}, "FA_ERR_ALIGN"),
    ({"lse": L + 2}, "FA_ERR_ALIGN"), ({"ws": WS + 4}, "FA_ERR_ALIGN"),
    ({"ws": None}, "FA_ERR_WORKSPACE"), ({"ws_bytes": 2 * 3 * 100 * 4 - 1}, "FA_ERR_WORKSPACE"),
    ({"dq": Q}, "FA_ERR_OVERLAP"), ({"dk": DV}, "FA_ERR_OVERLAP"),
    ({"ws": L}, "FA_ERR_OVERLAP"), ({"dv": O + 1024}, "FA_ERR_OVERLAP"),
])
def test_bwd_validation(kw, status):
    assert call_bwd(**kw) == getattr(fa, status)


def test_bwd_workspace_size():
    """The row terms (B*H*Nq fp32), plus at D = 64 and 128 the partial sums
    of the stream schedules past them (rounded up to 256 bytes): the larger
    of dQ's (two slots of 128 rows x D fp32 per chunk) and dK/dV's (two
    slots of 2 x 128 keys x D per chunk), at most 256 chunks.  The query
    needs no device."""
    st, n = fa.fa_bwd_workspace_size(2, 3, 100, 90, 32, 1, fa.FA_BF16)
    assert (st, n) == (fa.FA_OK, 2 * 3 * 100 * 4)
    # causal with Nq != Nk: the dQ schedule only
    st, n = fa.fa_bwd_workspace_size(2, 3, 100, 90, 64, 1, fa.FA_BF16)
    assert st == fa.FA_OK and n > 2 * 3 * 100 * 4 and (n - 2560) % (2 * 128 * 64 * 4) == 0
    assert n - 2560 <= 2 * 256 * 128 * 64 * 4
    # causal, Nq = Nk = 256: dK/dV's plan has 6 heads x (2 + 4 query-tile
    # units and 2 x 2 lead units) = 60 chunks (two slots of 2 x 128 x 64
    # floats each), dQ's 6 x (2 + 4 key-tile units and 2 x 3 lead units) =
    # 72 chunks (two slots of 128 x 64 floats)
    st, n = fa.fa_bwd_workspace_size(2, 3, 256, 256, 64, 1, fa.FA_BF16)
    assert (st, n) == (fa.FA_OK, 6 * 256 * 4 + 2 * 60 * 2 * 128 * 64 * 4)
    # a workspace of that size is written in full: the part past the row
    # terms counts in the overlap check
    assert call_bwd(Nq=256, Nk=256, ws=DQ - 8192, ws_bytes=n) == fa.FA_ERR_OVERLAP
    # 512 or more query tiles of 128 rows: one workgroup per tile, row terms only
    assert fa.fa_bwd_workspace_size(1, 32, 2048, 2048, 128, 1, fa.FA_BF16)[1] == 32 * 2048 * 4
    assert fa.fa_bwd_workspace_size(2, 3, 100, 90, 48, 1, fa.FA_BF16)[0] == fa.FA_ERR_HEAD_DIM
    assert fa.fa_bwd_workspace_size(2, 3, 100, 90, 64, 1, fa.FA_F32)[0] == fa.FA_ERR_DTYPE


def test_fwd_masked_workspace_size():
    """Non-causal masks with global tokens: the 256-row tiles holding global
    queries, ceil(min(G, Nq)/256) per (batch, head), each cut into
    ceil(key tiles / cap) parts of 256 x (D + 4) fp32, cap the band tile's
    key-tile count ((G key tiles) + (255 + 2 (W - 1)) // 64 + 2), at least
    32.  Causal masks and G = 0 need nothing.  No device."""
    ws = fa.fa_fwd_masked_workspace_size
    # B1 H8 N32768 D128, window 512 + 32 global: 512 key tiles, band 1 + 19 +
    # 2 = 22 -> cap 32 -> 16 parts of one tile per head
    assert ws(1, 8, 32768, 32768, 128, 0, 512, 32, fa.FA_BF16) == (
        fa.FA_OK, 8 * 16 * 256 * 132 * 4)
    # 300 global tokens: two split tiles; 79 key tiles -> 3 parts
    assert ws(1, 2, 5000, 5000, 64, 0, 64, 300, fa.FA_BF16) == (
        fa.FA_OK, 2 * 2 * 3 * 256 * 68 * 4)
    assert ws(1, 8, 32768, 32768, 128, 1, 512, 32, fa.FA_BF16) == (fa.FA_OK, 0)
    assert ws(1, 8, 32768, 32768, 128, 0, 512, 0, fa.FA_BF16) == (fa.FA_OK, 0)
    assert ws(1, 2, 2048, 2048, 128, 0, 64, 16, fa.FA_BF16) == (fa.FA_OK, 0)
    assert ws(1, 2, 4096, 4096, 64, 0, 0, 3, fa.FA_BF16)[0] == fa.FA_ERR_SHAPE
    assert ws(1, 2, 4096, 4096, 48, 0, 5, 3, fa.FA_BF16)[0] == fa.FA_ERR_HEAD_DIM
    assert ws(1, 2, 4096, 4096, 64, 0, 5, 3, fa.FA_F32)[0] == fa.FA_ERR_DTYPE


def test_bwd_masked_workspace_size():
    """The row terms, plus (rounded up to 256 bytes) the parts of the key
    tiles that hold global keys: B*H*ceil(min(G, Nk)/128) tiles, each cut
    into ceil(query tiles / cap) parts of two 128 x D fp32 blocks, cap being
    a band tile's query-tile count (causal: (127 + W - 1) // 64 + 2), at
    least 32.  No device."""
    ws = fa.fa_bwd_masked_workspace_size
    lb = 8 * 32768 * 4
    # B1 H8 N32768 D128 causal, window 512 + 32 global: 512 query tiles,
    # cap 32 -> 16 parts of one tile per head
    assert ws(1, 8, 32768, 32768, 128, 1, 512, 32, fa.FA_BF16) == (
        fa.FA_OK, lb + 8 * 16 * 2 * 128 * 128 * 4)
    # window 2048 + 128 global: cap (127 + 2047) // 64 + 2 = 35 -> 15 parts
    assert ws(1, 8, 32768, 32768, 128, 1, 2048, 128, fa.FA_BF16) == (
        fa.FA_OK, lb + 8 * 15 * 2 * 128 * 128 * 4)
    # 300 global keys: three split tiles; D = 64
    assert ws(1, 2, 4096, 4096, 64, 1, 100, 300, fa.FA_BF16) == (
        fa.FA_OK, 2 * 4096 * 4 + 2 * 3 * 2 * 2 * 128 * 64 * 4)
    # non-causal: the band cap counts both sides and the global query tiles
    # (1 + (127 + 126) // 64 + 2 = 6 -> 32); the dK/dV parts (larger than
    # the dQ split's) set the size
    assert ws(1, 2, 4096, 4096, 64, 0, 64, 40, fa.FA_BF16) == (
        fa.FA_OK, 2 * 4096 * 4 + 2 * 2 * 2 * 128 * 64 * 4)
    # at D = 128 non-causal dK/dV runs whole; the dQ split's query tile (40
    # global queries: one 128-row tile, 2 parts of 128 x D fp32) is what counts
    assert ws(1, 2, 4096, 4096, 128, 0, 64, 40, fa.FA_BF16) == (
        fa.FA_OK, 2 * 4096 * 4 + 2 * 1 * 2 * 128 * 128 * 4)
    # no global key, a short sequence, or a band as long as the sequence:
    # nothing to split
    assert ws(1, 8, 32768, 32768, 128, 1, 512, 0, fa.FA_BF16) == (fa.FA_OK, lb)
    assert ws(1, 2, 2048, 2048, 128, 1, 64, 16, fa.FA_BF16) == (fa.FA_OK, 2 * 2048 * 4)
    assert ws(1, 2, 8192, 8192, 128, 1, 8192, 16, fa.FA_BF16) == (fa.FA_OK, 2 * 8192 * 4)
    # D = 16 and 32 run the earlier kernels
    assert ws(1, 2, 4096, 4096, 32, 1, 100, 300, fa.FA_BF16) == (fa.FA_OK, 2 * 4096 * 4)
    assert ws(1, 2, 4096, 4096, 64, 1, 0, 3, fa.FA_BF16)[0] == fa.FA_ERR_SHAPE
    assert ws(1, 2, 4096, 4096, 64, 1, 5, -1, fa.FA_BF16)[0] == fa.FA_ERR_SHAPE
    assert ws(1, 2, 4096, 4096, 48, 1, 5, 3, fa.FA_BF16)[0] == fa.FA_ERR_HEAD_DIM


# --- fa_fwd_varlen: validation precedes device work --------------------------
CQ, CK = 0xB0000000, 0xC0000000


def call_varlen(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, cq=CQ, ck=CK, S=3, H=2, Tq=500, Tk=400, mq=300,
             D=64, scale=0.125, causal=1, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"],
                            a["S"], a["H"], a["Tq"], a["Tk"], a["mq"], a["D"], a["scale"],
                            a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    ({"q": None}, "FA_ERR_NULLPTR"), ({"cq": None}, "FA_ERR_NULLPTR"),
    ({"ck": None}, "FA_ERR_NULLPTR"), ({"S": 0}, "FA_ERR_SHAPE"), ({"Tq": 0}, "FA_ERR_SHAPE"),
    ({"Tk": -1}, "FA_ERR_SHAPE"), ({"mq": 0}, "FA_ERR_SHAPE"), ({"D": 48}, "FA_ERR_HEAD_DIM"),
    ({"dtype": fa.FA_F32}, "FA_ERR_DTYPE"), ({"scale": math.nan}, "FA_ERR_SCALE"),
    ({"o": O + 8}, "FA_ERR_ALIGN"), ({"cq": CQ + 2}, "FA_ERR_ALIGN"),
    ({"o": Q}, "FA_ERR_OVERLAP"), ({"lse": CK}, "FA_ERR_OVERLAP"),
])
def test_varlen_validation(kw, status):
    assert call_varlen(**kw) == getattr(fa, status)


def call_varlen_ws(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, cq=CQ, ck=CK, S=3, H=2, Tq=500, Tk=400, mq=300, mk=300,
             D=64, scale=0.125, causal=1, dtype=fa.FA_BF16, ws=None, nb=0, stream=None)
    a.update(kw)
    return fa.fa_fwd_varlen_ws(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"],
                               a["S"], a["H"], a["Tq"], a["Tk"], a["mq"], a["mk"], a["D"],
                               a["scale"], a["causal"], a["dtype"], a["ws"], a["nb"],
                               a["stream"])


@pytest.mark.parametrize("kw,status", [
    ({"q": None}, "FA_ERR_NULLPTR"), ({"ck": None}, "FA_ERR_NULLPTR"),
    ({"S": 0}, "FA_ERR_SHAPE"), ({"mk": -1}, "FA_ERR_SHAPE"), ({"mq": 0}, "FA_ERR_SHAPE"),
    ({"D": 8}, "FA_ERR_HEAD_DIM"), ({"dtype": fa.FA_F32}, "FA_ERR_DTYPE"),
    ({"scale": math.inf}, "FA_ERR_SCALE"), ({"lse": L + 2}, "FA_ERR_ALIGN"),
    ({"o": K}, "FA_ERR_OVERLAP"), ({"lse": O}, "FA_ERR_OVERLAP"),
])
def test_varlen_ws_validation(kw, status):
    """fa_fwd_varlen_ws checks its arguments before it looks at the device."""
    assert call_varlen_ws(**kw) == getattr(fa, status)


@pytest.mark.parametrize("args,status", [
    ((0, 1, 100, 100, 100, 100, 64, 1, 1), "FA_ERR_SHAPE"),
    ((1, 1, 100, 100, 100, -1, 64, 1, 1), "FA_ERR_SHAPE"),
    ((1, 1, 100, 100, 100, 100, 24, 1, 1), "FA_ERR_HEAD_DIM"),
    ((1, 1, 100, 100, 100, 100, 64, 1, 0), "FA_ERR_DTYPE"),
])
def test_varlen_workspace_size_validation(args, status):
    st, nb = fa.fa_fwd_varlen_workspace_size(*args)
    assert st == getattr(fa, status) and nb == 0


def call_bwd_varlen(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, cq=CQ, ck=CK, S=3, H=2,
             Tq=500, Tk=400, mq=300, mk=200, D=64, scale=0.125, causal=1, dtype=fa.FA_BF16,
             ws=WS, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return fa.fa_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                            a["dk"], a["dv"], a["cq"], a["ck"], a["S"], a["H"], a["Tq"],
                            a["Tk"], a["mq"], a["mk"], a["D"], a["scale"], a["causal"],
                            a["dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    ({"cq": None}, "FA_ERR_NULLPTR"), ({"dv": None}, "FA_ERR_NULLPTR"),
    ({"S": 0}, "FA_ERR_SHAPE"), ({"Tq": 0}, "FA_ERR_SHAPE"), ({"mk": -1}, "FA_ERR_SHAPE"),
    ({"D": 48}, "FA_ERR_HEAD_DIM"), ({"dtype": fa.FA_F32}, "FA_ERR_DTYPE"),
    ({"scale": math.inf}, "FA_ERR_SCALE"), ({"ck": CK + 1}, "FA_ERR_ALIGN"),
    ({"ws_bytes": 2 * 500 * 4 - 4}, "FA_ERR_WORKSPACE"), ({"dq": CQ}, "FA_ERR_OVERLAP"),
])
def test_bwd_varlen_validation(kw, status):
    assert call_bwd_varlen(**kw) == getattr(fa, status)


def call_masked(**kw):
    a = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Nq=100, Nk=90, D=64, scale=0.125, causal=1,
             window=16, nglobal=4, dtype=fa.FA_BF16, stream=None)
    a.update(kw)
    return fa.fa_fwd_masked(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                            a["Nk"], a["D"], a["scale"], a["causal"], a["window"],
                            a["nglobal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    ({"lse": None}, "FA_ERR_NULLPTR"), ({"Nk": 0}, "FA_ERR_SHAPE"),
    ({"window": 0}, "FA_ERR_SHAPE"), ({"nglobal": -1}, "FA_ERR_SHAPE"),
    ({"D": 48}, "FA_ERR_HEAD_DIM"), ({"dtype": fa.FA_F32}, "FA_ERR_DTYPE"),
    ({"scale": math.inf}, "FA_ERR_SCALE"), ({"v": V + 4}, "FA_ERR_ALIGN"),
    ({"o": K}, "FA_ERR_OVERLAP"),
])
def test_masked_validation(kw, status):
    assert call_masked(**kw) == getattr(fa, status)


def test_bwd_masked_validation():
    def call(**kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, B=2, H=3, Nq=100,
                 Nk=90, D=64, scale=0.125, causal=1, window=8, nglobal=2, dtype=fa.FA_BF16,
                 ws=WS, ws_bytes=1 << 20, stream=None)
        a.update(kw)
        return fa.fa_bwd_masked(*(a[x] for x in ("q", "k", "v", "o", "lse", "do", "dq", "dk",
                                                  "dv", "B", "H", "Nq", "Nk", "D", "scale",
                                                  "causal", "window", "nglobal", "dtype",
                                                  "ws", "ws_bytes", "stream")))
    assert call(window=0) == fa.FA_ERR_SHAPE
    assert call(nglobal=-1) == fa.FA_ERR_SHAPE
    assert call(dk=None) == fa.FA_ERR_NULLPTR
    assert call(D=48) == fa.FA_ERR_HEAD_DIM
    assert call(dq=Q) == fa.FA_ERR_OVERLAP
    assert call(ws=None) == fa.FA_ERR_WORKSPACE


def test_fp8_validation():
    def call(**kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Nq=100, Nk=90, D=128, scale=0.1, dq=0.01,
                 dk=0.01, dv=0.01, causal=1, out_f32=0, stream=None)
        a.update(kw)
        return fa.fa_fwd_fp8(*(a[x] for x in ("q", "k", "v", "o", "lse", "B", "H", "Nq", "Nk",
                                               "D", "scale", "dq", "dk", "dv", "causal",
                                               "out_f32", "stream")))
    assert call(q=None) == fa.FA_ERR_NULLPTR
    assert call(Nq=0) == fa.FA_ERR_SHAPE
    assert call(D=32) == fa.FA_ERR_HEAD_DIM
    assert call(dk=math.inf) == fa.FA_ERR_SCALE
    assert call(scale=3e38, dq=1e10) == fa.FA_ERR_SCALE
    assert call(o=O + 4) == fa.FA_ERR_ALIGN
    assert call(lse=Q) == fa.FA_ERR_OVERLAP


# --- extreme sizes: rejected, with no overflow in the size arithmetic ------
BIG = [1 << 31, 1 << 40, 1 << 62, (1 << 63) - 1]


@pytest.mark.parametrize("big", BIG)
@pytest.mark.parametrize("entry,field", [
    (call, "B"), (call, "H"), (call, "Nq"), (call, "Nk"),
    (call_ws, "B"), (call_ws, "H"), (call_ws, "Nq"), (call_ws, "Nk"),
    (call_bwd, "B"), (call_bwd, "H"), (call_bwd, "Nq"), (call_bwd, "Nk"),
    (call_varlen, "S"), (call_varlen, "H"), (call_varlen, "Tq"), (call_varlen, "Tk"),
    (call_varlen_ws, "S"), (call_varlen_ws, "H"), (call_varlen_ws, "Tq"),
    (call_varlen_ws, "Tk"),
    (call_bwd_varlen, "S"), (call_bwd_varlen, "H"), (call_bwd_varlen, "Tq"),
    (call_bwd_varlen, "Tk"),
    (call_masked, "B"), (call_masked, "H"), (call_masked, "Nq"), (call_masked, "Nk"),
], ids=lambda x: getattr(x, "__name__", x))
def test_extreme_sizes_rejected(entry, field, big):
    assert entry(**{field: big}) == fa.FA_ERR_SHAPE


@pytest.mark.parametrize("big", BIG)
@pytest.mark.parametrize("pos", [0, 1, 2, 3])
def test_extreme_sizes_workspace_queries(pos, big):
    a = [2, 3, 100, 90]
    a[pos] = big
    assert fa.fa_fwd_workspace_size(*a, 64, 1, fa.FA_BF16)[0] == fa.FA_ERR_SHAPE
    assert fa.fa_bwd_workspace_size(*a, 64, 1, fa.FA_BF16)[0] == fa.FA_ERR_SHAPE
    v = [3, 2, 500, 400]
    v[pos] = big
    assert fa.fa_fwd_varlen_workspace_size(*v, 300, 300, 64, 1, fa.FA_BF16)[0] == \
        fa.FA_ERR_SHAPE


def test_debug_library_exports_the_same_symbols_and_its_check():
    """libfa_debug.so (the build with ring-barrier checks, include/fa_debug.h)
    exports every symbol of include/fa.h plus fa_debug_barrier_faults, which
    the release library does not."""
    dbg = fa.debug_library()
    for name in _declared_functions():
        assert hasattr(dbg, name), f"libfa_debug.so does not export {name}"
    assert hasattr(dbg, "fa_debug_barrier_faults")
    assert not hasattr(fa.library(), "fa_debug_barrier_faults")
    assert dbg.fa_debug_barrier_faults(None, 0) == fa.FA_ERR_NULLPTR
