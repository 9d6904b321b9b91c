"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status codes
before launching anything (every call below fails validation or is a no-op)."""
import ctypes
import os
import re

import pytest

import group_circulant_linear_p4_amd as eql

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eqlinear.h")

A16 = 0x10000          # fake, 16-byte aligned device addresses (never dereferenced:
A16B = 0x20000         # every call that receives them fails validation first)
MIS = 0x10008          # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(eqlinear_\w+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_function():
    L = eql.lib()
    names = declared_functions()
    assert len(names) == 19
    for n in names:
        assert hasattr(L, n), "missing export %s" % n
        assert hasattr(eql, n), "binding lacks %s" % n


def test_version_and_status_strings():
    assert eql.eqlinear_abi_version() == 205
    for s in range(5):
        assert eql.eqlinear_status_string(s)
    assert eql.eqlinear_status_string(99) == "unknown status"


def test_packed_weight_bytes():
    # Opad * Jin * 16 * T bytes: Opad = out rounded up to a multiple of 32, Jin =
    # ceil(in / G) rounded up to a multiple of 4, G = 16 / sizeof(elt)
    assert eql.eqlinear_packed_weight_bytes(3, 5, 4, eql.EQL_F16) == 32 * 4 * 16 * 4
    assert eql.eqlinear_packed_weight_bytes(3, 33, 4, eql.EQL_F16) == 32 * 8 * 16 * 4
    assert eql.eqlinear_packed_weight_bytes(1024, 1024, 4, eql.EQL_F16) == 1024 * 1024 * 4 * 2
    assert eql.eqlinear_packed_weight_bytes(64, 64, 8, eql.EQL_F32) == 64 * 64 * 8 * 4
    assert eql.eqlinear_packed_weight_bytes(7, 3, 3, eql.EQL_F32) == 32 * 4 * 16 * 3
    assert eql.eqlinear_packed_weight_bytes(33, 3, 3, eql.EQL_F32) == 64 * 4 * 16 * 3
    assert eql.eqlinear_packed_weight_bytes(3, 3, 0, eql.EQL_F32) == 0
    assert eql.eqlinear_packed_weight_bytes(3, 3, 17, eql.EQL_F32) == 0
    assert eql.eqlinear_packed_weight_bytes(3, 3, 4, 7) == 0


def bwdw_fused(N, Cp, Dp, T, elt):
    """The weight gradient's path rule as documented in the header: the fused path for
    T in {1, 2, 4}, 16-byte dy rows and fewer than 400 actual FLOPs per algorithmic byte."""
    if N == 0 or T not in (1, 2, 4) or (Dp * T * elt) % 16 or N * Dp * T * elt >= 2**32:
        return False
    planes = {1: 1, 2: 2, 4: 6}[T]
    return 2 * planes * N * Dp * Cp / (elt * T * N * (Cp + Dp)) < 400


def test_workspace_bytes():
    assert eql.eqlinear_bwd_w_workspace_bytes(0, 4, 4, 4, eql.EQL_F16) == 0
    # Separate path: dy and x half spectra as 16-byte units (2G rows per k-step, G = 8
    # for fp16 and 4 for fp32; channels padded to the GEMM tile width, 256 unless that
    # pads more than a third of the channels, else 64; each section 256-byte aligned),
    # then fp32 partial spectra: whole [D'][C'] planes, at least one set of T planes
    # and at most one set per k-step.  Fused path: x's spectrum only, channels padded
    # to a multiple of a column tile of 32 nb channels (nb in 4, 3, 2 with T nb a
    # multiple of 4, the least padding, ties to the wider), then the partials.
    def padded(ch):
        w = 256 if -(-ch // 256) * 256 * 3 <= ch * 4 else 64
        return -(-ch // w) * w

    def fused_padded(ch, T):
        widths = [32 * nb for nb in (4, 3, 2) if (T * nb) % 4 == 0]
        return min((-(-ch // w) * w for w in widths))

    paths = set()
    for (N, Cp, Dp, G, code) in ((65536, 1024, 1024, 8, eql.EQL_F16), (37, 5, 3, 4, eql.EQL_F32),
                                 (100352, 192, 768, 8, eql.EQL_F16), (1000, 96, 200, 8, eql.EQL_F16)):
        T = 4
        elt = 16 // G
        n = eql.eqlinear_bwd_w_workspace_bytes(N, Cp, Dp, T, code)
        steps = -(-N // (2 * G))
        fused = bwdw_fused(N, Cp, Dp, T, elt)
        paths.add(fused)
        if fused:
            spec = -(-(steps * T * 2 * fused_padded(Cp, T) * 16) // 256) * 256
        else:
            spec = sum(-(-(steps * T * 2 * padded(K) * 16) // 256) * 256 for K in (Dp, Cp))
        part = n - spec
        plane = Dp * Cp * 4
        assert T * plane <= part <= steps * T * plane + 256
    assert paths == {True, False}
    assert eql.eqlinear_bwd_w_workspace_bytes(10, 4, 4, 0, eql.EQL_F16) == 0


def raw(fn, *args):
    return getattr(eql.lib(), fn)(*args)


@pytest.mark.parametrize("fn", ["eqlinear_fwd", "eqlinear_bwd_x"])
def test_fwd_validation(fn):
    F16, F32 = eql.EQL_F16, eql.EQL_F32
    ok = (A16, A16B, A16 + 0x1000)
    assert raw(fn, *ok, 8, 4, 4, 4, 5, None) == eql.EQL_EINVAL            # dtype
    assert raw(fn, *ok, 8, 4, 4, 0, F16, None) == eql.EQL_EINVAL          # T < 1
    assert raw(fn, *ok, 8, 4, 4, 17, F16, None) == eql.EQL_EUNSUPPORTED   # T > 16
    assert raw(fn, *ok, -1, 4, 4, 4, F16, None) == eql.EQL_EINVAL         # N < 0
    assert raw(fn, *ok, 8, 0, 4, 4, F16, None) == eql.EQL_EINVAL          # C' < 1
    assert raw(fn, *ok, 8, 4, 0, 4, F32, None) == eql.EQL_EINVAL          # D' < 1
    assert raw(fn, *ok, 8, 1 << 22, 4, 4, F32, None) == eql.EQL_EINVAL    # C'T >= 2^24
    assert raw(fn, *ok, 1 << 31, 4, 4, 4, F32, None) == eql.EQL_EINVAL   # N >= 2^31
    assert raw(fn, *ok, (1 << 31) - (1 << 20) + 1, 4, 4, 4, F32, None) == eql.EQL_EINVAL  # N > 2^31 - 2^20
    assert raw(fn, None, A16B, A16, 8, 4, 4, 4, F16, None) == eql.EQL_EINVAL
    assert raw(fn, A16, None, A16B, 8, 4, 4, 4, F16, None) == eql.EQL_EINVAL
    assert raw(fn, A16, A16B, None, 8, 4, 4, 4, F16, None) == eql.EQL_EINVAL
    assert raw(fn, MIS, A16B, A16, 8, 4, 4, 4, F16, None) == eql.EQL_EALIGN
    assert raw(fn, A16, MIS, A16B, 8, 4, 4, 4, F16, None) == eql.EQL_EALIGN
    assert raw(fn, A16, A16B, MIS, 8, 4, 4, 4, F32, None) == eql.EQL_EALIGN
    # N == 0 is a no-op that launches nothing, even with null buffers.
    assert raw(fn, None, None, None, 0, 4, 4, 4, F16, None) == eql.EQL_OK


def test_fwd_fused_validation():
    F16, F32 = eql.EQL_F16, eql.EQL_F32
    GELU = eql.EQL_ACT_GELU
    x, wp, y = A16, A16B, A16 + 0x1000
    fn = "eqlinear_fwd_fused"
    assert raw(fn, x, wp, None, None, y, None, 8, 4, 4, 4, F16, 2, None) == eql.EQL_EINVAL       # act
    assert raw(fn, x, wp, None, None, y, None, 8, 4, 4, 4, F16, -1, None) == eql.EQL_EINVAL      # act
    assert raw(fn, x, wp, None, None, y, None, 8, 4, 4, 4, 5, GELU, None) == eql.EQL_EINVAL      # dtype
    assert raw(fn, x, wp, None, None, y, None, 8, 4, 4, 17, F16, GELU, None) == eql.EQL_EUNSUPPORTED
    assert raw(fn, None, wp, None, None, y, None, 8, 4, 4, 4, F16, GELU, None) == eql.EQL_EINVAL
    assert raw(fn, x, wp, A16 + 1, None, y, None, 8, 4, 4, 4, F16, GELU, None) == eql.EQL_EALIGN  # bias
    assert raw(fn, x, wp, A16 + 2, None, y, None, 8, 4, 4, 4, F32, GELU, None) == eql.EQL_EALIGN  # bias
    assert raw(fn, x, wp, None, MIS, y, None, 8, 4, 4, 4, F16, GELU, None) == eql.EQL_EALIGN     # residual
    assert raw(fn, x, wp, None, None, y, MIS, 8, 4, 4, 4, F16, GELU, None) == eql.EQL_EALIGN     # pre_out
    assert raw(fn, MIS, wp, None, None, y, None, 8, 4, 4, 4, F16, GELU, None) == eql.EQL_EALIGN
    assert raw(fn, None, None, None, None, None, None, 0, 4, 4, 4, F16, GELU, None) == eql.EQL_OK


def test_fused_epilogue_bwd_validation():
    F16, F32 = eql.EQL_F16, eql.EQL_F32
    GELU, NONE = eql.EQL_ACT_GELU, eql.EQL_ACT_NONE
    fn = "eqlinear_fused_epilogue_bwd"
    dy, pre, dpre, db, ws = A16, A16B, A16 + 0x1000, A16 + 0x2000, A16 + 0x3000
    need = eql.eqlinear_fused_epilogue_bwd_workspace_bytes(300, 5, 4, F16)
    # fp32 column sums of each block of rows: 300 rows of D'T = 20 elements (one 64-chunk
    # block across) take the smallest row block, 16 rows: 19 blocks.
    assert need == 19 * 20 * 4
    # Large enough for 2048 workgroups at 1024 rows a block: 65536 rows of 16384 fp16
    # elements (32 blocks of 64 16-byte chunks across) give 64 row blocks.
    assert eql.eqlinear_fused_epilogue_bwd_workspace_bytes(65536, 4096, 4, F16) == 64 * 16384 * 4
    assert eql.eqlinear_fused_epilogue_bwd_workspace_bytes(0, 5, 4, F16) == 0
    assert raw(fn, dy, pre, dpre, db, ws, need, 300, 5, 4, F16, 3, None) == eql.EQL_EINVAL      # act
    assert raw(fn, dy, None, dpre, db, ws, need, 300, 5, 4, F16, GELU, None) == eql.EQL_EINVAL  # pre needed
    assert raw(fn, dy, pre, dpre, db, ws, need - 1, 300, 5, 4, F16, GELU, None) == eql.EQL_EINVAL   # short ws
    assert raw(fn, dy, pre, dpre, db, None, need, 300, 5, 4, F16, GELU, None) == eql.EQL_EINVAL  # no ws
    assert raw(fn, None, pre, dpre, db, ws, need, 300, 5, 4, F16, GELU, None) == eql.EQL_EINVAL
    assert raw(fn, dy, pre, None, db, ws, need, 300, 5, 4, F16, GELU, None) == eql.EQL_EINVAL
    assert raw(fn, dy, pre, dpre, db, ws, need, 300, 5, 17, F16, GELU, None) == eql.EQL_EUNSUPPORTED
    assert raw(fn, MIS, pre, dpre, db, ws, need, 300, 5, 4, F16, GELU, None) == eql.EQL_EALIGN
    assert raw(fn, dy, pre, dpre, A16 + 2, ws, need, 300, 5, 4, F32, NONE, None) == eql.EQL_EALIGN
    assert raw(fn, dy, pre, dpre, db, ws, need, 300, 0, 4, F16, GELU, None) == eql.EQL_EINVAL   # D' < 1


def test_fused_epilogue_bwd_noalloc_validation():
    """The no-allocation variant validates like eqlinear_fused_epilogue_bwd, and refuses a
    shape whose bias partials exceed its static scratch before anything is launched."""
    F16, F32 = eql.EQL_F16, eql.EQL_F32
    GELU, NONE = eql.EQL_ACT_GELU, eql.EQL_ACT_NONE
    fn = "eqlinear_fused_epilogue_bwd_noalloc"
    dy, pre, dpre, db = A16, A16B, A16 + 0x1000, A16 + 0x2000
    cap = eql.EQL_NOALLOC_SCRATCH_BYTES
    assert cap == 16 << 20
    assert raw(fn, dy, pre, dpre, db, 300, 5, 4, F16, 3, None) == eql.EQL_EINVAL      # act
    assert raw(fn, dy, None, dpre, db, 300, 5, 4, F16, GELU, None) == eql.EQL_EINVAL  # pre needed
    assert raw(fn, None, pre, dpre, db, 300, 5, 4, F16, GELU, None) == eql.EQL_EINVAL
    assert raw(fn, dy, pre, None, db, 300, 5, 4, F16, GELU, None) == eql.EQL_EINVAL
    assert raw(fn, dy, pre, dpre, db, 300, 5, 17, F16, GELU, None) == eql.EQL_EUNSUPPORTED
    assert raw(fn, MIS, pre, dpre, db, 300, 5, 4, F16, GELU, None) == eql.EQL_EALIGN
    assert raw(fn, dy, pre, dpre, A16 + 2, 300, 5, 4, F32, NONE, None) == eql.EQL_EALIGN
    assert raw(fn, dy, pre, dpre, db, 300, 0, 4, F16, GELU, None) == eql.EQL_EINVAL   # D' < 1
    assert raw(fn, None, None, None, None, 0, 4, 4, F16, NONE, None) == eql.EQL_OK    # N = 0, no dbias
    # 2^21 rows of D'T = 4096 fp16 elements: 2048 row blocks of 1024 rows, 32 MiB of fp32
    # partials; 2^20 rows need exactly the scratch.
    assert eql.eqlinear_fused_epilogue_bwd_workspace_bytes(1 << 21, 1024, 4, F16) == 2 * cap
    assert eql.eqlinear_fused_epilogue_bwd_workspace_bytes(1 << 20, 1024, 4, F16) == cap
    assert raw(fn, dy, pre, dpre, db, 1 << 21, 1024, 4, F16, GELU, None) == eql.EQL_ESCRATCH
    assert raw(fn, dy, pre, dpre, db, (1 << 20) + 1024, 1024, 4, F16, NONE, None) == eql.EQL_ESCRATCH
    assert "scratch" in eql.eqlinear_status_string(eql.EQL_ESCRATCH)


def test_p4m_map_validation():
    """The p4m weight expansion and gradient fold validate like the other entry points,
    with the size rules of the C_4 view (2C' inputs, 2D' outputs, T = 4)."""
    F16, F32 = eql.EQL_F16, eql.EQL_F32
    for fn in ("eqlinear_p4m_expand_weight", "eqlinear_p4m_fold_weight_grad"):
        assert raw(fn, A16, A16B, 4, 4, 7, None) == eql.EQL_EINVAL               # dtype
        assert raw(fn, A16, A16B, 0, 4, F16, None) == eql.EQL_EINVAL             # D' < 1
        assert raw(fn, A16, A16B, 4, -3, F32, None) == eql.EQL_EINVAL            # C' < 1
        assert raw(fn, A16, A16B, 4, 1 << 62, F32, None) == eql.EQL_EINVAL       # C' far too large
        assert raw(fn, A16, A16B, 4, (1 << 20) + 1, F32, None) == eql.EQL_EINVAL  # 2C' x 4 x 4 B > 2^23
        assert raw(fn, None, A16B, 4, 4, F16, None) == eql.EQL_EINVAL
        assert raw(fn, A16, None, 4, 4, F16, None) == eql.EQL_EINVAL
        assert raw(fn, MIS, A16B, 4, 4, F16, None) == eql.EQL_EALIGN
        assert raw(fn, A16, MIS, 4, 4, F32, None) == eql.EQL_EALIGN


def test_pack_validation():
    F16 = eql.EQL_F16
    assert raw("eqlinear_pack_weight", A16, A16B, 4, 4, 4, F16, 2, None) == eql.EQL_EINVAL   # mode
    assert raw("eqlinear_pack_weight", None, A16B, 4, 4, 4, F16, 0, None) == eql.EQL_EINVAL
    assert raw("eqlinear_pack_weight", A16, None, 4, 4, 4, F16, 1, None) == eql.EQL_EINVAL
    assert raw("eqlinear_pack_weight", MIS, A16B, 4, 4, 4, F16, 0, None) == eql.EQL_EALIGN
    assert raw("eqlinear_pack_weight", A16, A16B, 4, 4, 20, F16, 0, None) == eql.EQL_EUNSUPPORTED
    assert raw("eqlinear_pack_weight", A16, A16B, 0, 4, 4, F16, 0, None) == eql.EQL_EINVAL


def test_bwd_w_validation():
    F16 = eql.EQL_F16
    need = eql.eqlinear_bwd_w_workspace_bytes(64, 4, 4, 4, F16)
    f = "eqlinear_bwd_w"
    assert raw(f, A16, A16B, A16 + 0x100, A16 + 0x200, need - 1, 64, 4, 4, 4, F16, None) == eql.EQL_EINVAL
    assert raw(f, None, A16B, A16 + 0x100, A16 + 0x200, need, 64, 4, 4, 4, F16, None) == eql.EQL_EINVAL
    assert raw(f, A16, A16B, None, A16 + 0x200, need, 64, 4, 4, 4, F16, None) == eql.EQL_EINVAL
    assert raw(f, A16, A16B, A16 + 0x100, None, need, 64, 4, 4, 4, F16, None) == eql.EQL_EINVAL
    assert raw(f, A16, MIS, A16 + 0x100, A16 + 0x200, need, 64, 4, 4, 4, F16, None) == eql.EQL_EALIGN
    assert raw(f, A16, A16B, A16 + 0x100, A16 + 0x208, need, 64, 4, 4, 4, F16, None) == eql.EQL_EALIGN
    assert raw(f, A16, A16B, A16 + 0x100, A16 + 0x200, need, 64, 4, 4, 0, F16, None) == eql.EQL_EINVAL
    assert raw(f, A16, A16B, A16 + 0x100, A16 + 0x200, need, 64, 4, 4, 4, 9, None) == eql.EQL_EINVAL


def test_binding_raises_on_error_and_rejects_host_tensors():
    import torch
    with pytest.raises(eql.EqlError) as ei:
        eql.eqlinear_fwd(MIS, A16, A16B, 8, 4, 4, 4, eql.EQL_F16, stream=0)
    assert ei.value.status == eql.EQL_EALIGN
    with pytest.raises(ValueError):
        eql.eqlinear_fwd(torch.zeros(8, 16), A16, A16B, 8, 4, 4, 4, eql.EQL_F32, stream=0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(eql, "_lib", None)
    monkeypatch.setattr(eql, "_LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        eql.lib()


@pytest.mark.parametrize("shape", [(12,), (2,), (1, 3)], ids=["per_feature", "short", "two_dim"])
def test_fused_layer_rejects_a_bias_of_the_wrong_shape(shape):
    """The fused layer's bias holds one value per output channel (D' = 3 here); a
    per-feature bias of D'*T values, a short one or a 2-D one is refused before any
    buffer reaches the library (CPU tensors: nothing is launched)."""
    import torch
    from group_circulant_linear_p4_amd.layer import eqlinear_fused
    x = torch.zeros(5, 2 * 4)
    w = torch.zeros(3, 2, 4)
    b = torch.zeros(*shape)
    with pytest.raises(ValueError, match="bias"):
        eqlinear_fused(x, w, bias=b, act="gelu")
