"""The C ABI library loads, exports every function include/moe.h declares, and rejects
invalid arguments on the host before any launch (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from combine_top_router_amd import lib as L
    if not os.path.exists(L.lib_path()):
        pytest.skip("libmoe.so not built")
    return L


def _declared():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("moe_route_topk", "moe_dispatch", "moe_fwd", "moe_bwd", "moe_combine"):
        assert n in names
    assert set(names) == set(_lib().EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib()
    raw = ctypes.CDLL(L.lib_path())
    for n in _declared():
        assert hasattr(raw, n), n
    assert L.moe_abi_version() == 3


def _shape(L, **kw):
    base = dict(T=64, H=128, I=64, E=8, k=2, e_begin=0, e_local=8, dtype=L.MOE_BF16, bwd=0, renorm=1)
    base.update(kw)
    return L.MoeShape(**base)


BAD = [
    (dict(T=-1), -1), (dict(H=0), -1), (dict(E=0), -1), (dict(E=2000), -1), (dict(k=0), -1),
    (dict(k=9), -1), (dict(k=17, E=32), -1), (dict(e_local=0), -1), (dict(e_begin=5, e_local=4), -1),
    (dict(e_begin=-1), -1), (dict(dtype=7), -1), (dict(bwd=3), -1), (dict(renorm=2), -1),
    # valid sizes the kernels do not support: bf16 H or I off a multiple of 64, fp32 H of 4
    (dict(H=100), -2), (dict(I=96), -2), (dict(dtype=0, H=130), -2),
    (dict(H=(1 << 20) + 64), -1), (dict(I=(1 << 20) + 64), -1),
    (dict(dtype=0, bwd=1), -2),
    # MXFP8 backward whose padded row space (R_cap plus 127 rows per expert) passes 2^31 - 1
    (dict(T=(2 ** 31 - 1) // 8, k=8, E=1024, e_local=1024, bwd=1), -2),
    # MXFP8 forward: an unknown value, fp32 data, H or I not a multiple of 128
    (dict(fwd=2), -1), (dict(dtype=0, fwd=1), -2), (dict(fwd=1), -2), (dict(fwd=1, I=128, H=192), -2),
    # recompute: an unknown value, fp32 data
    (dict(recompute=2), -1), (dict(dtype=0, recompute=1), -2),
    # row tile height: neither automatic (0) nor one of the two builds
    (dict(row_tile=128), -1), (dict(row_tile=-1), -1),
]


@pytest.mark.parametrize("kw,code", BAD, ids=[str(b[0]) for b in BAD])
def test_invalid_shapes_are_rejected(kw, code):
    L = _lib()
    with pytest.raises(L.MoeError) as ei:
        L.moe_workspace_bytes(_shape(L, **kw))
    assert ei.value.code == code
    assert L.moe_last_error()


def test_null_pointers_are_rejected_before_launch():
    L = _lib()
    s = _shape(L)
    with pytest.raises(L.MoeError) as ei:
        L.moe_route_topk(s, 0, 0, 0)
    assert ei.value.code == L.MOE_EINVAL
    with pytest.raises(L.MoeError) as ei:
        L.moe_dispatch(s, 8, 0, 8, 8, 8, 8, 0, 0)      # scratch is NULL
    assert ei.value.code == L.MOE_EWORKSPACE
    with pytest.raises(L.MoeError) as ei:
        L.moe_fwd(s, 8, 0, 8, 8, 8, 8, 8, 8, 8, 0, 8)  # saved is NULL
    assert ei.value.code == L.MOE_EWORKSPACE
    with pytest.raises(L.MoeError) as ei:
        L.moe_bwd(s, 8, 8, 0, 8, 8, 8, 8, 8, 8, 8, 8, 8, 0, 8, 8, 8, 8)  # dw_gate is NULL
    assert ei.value.code == L.MOE_EINVAL
    with pytest.raises(L.MoeError) as ei:
        L.moe_route_topk_bwd(_shape(L, renorm=0), 0, 8, 8, 8, 8)  # renorm 0 needs logits
    assert ei.value.code == L.MOE_EINVAL


def test_workspace_sizes_grow_with_the_layer():
    L = _lib()
    small = L.moe_workspace_bytes(_shape(L))
    big = L.moe_workspace_bytes(_shape(L, T=4096, H=2048, I=768, E=128, k=8, e_local=128))
    assert all(b > a > 0 for a, b in zip(small, big))
    # saved holds G|U and A for every possible row
    R = 4096 * 8
    assert big[0] >= R * 3 * 768 * 2
    # recompute keeps nothing between the calls; the backward's recomputed G|U and A live
    # in scratch instead
    ck = L.moe_workspace_bytes(_shape(L, T=4096, H=2048, I=768, E=128, k=8, e_local=128, recompute=1))
    assert ck[0] == 0 and ck[1] >= big[1] + R * 3 * 768 * 2
    # mxfp8: saved also holds the backward's row-wise weight codes (with their scales),
    # unless recompute is on
    mx = dict(T=4096, H=2048, I=768, E=128, k=8, e_local=128, fwd=1, bwd=1)
    wcodes = 128 * 3 * 2048 * 768 * (1 + 1 / 32)
    assert L.moe_workspace_bytes(_shape(L, **mx))[0] >= big[0] + wcodes
    assert L.moe_workspace_bytes(_shape(L, **mx, recompute=1))[0] == 0
    # fp8_bwd: the forward writes the weight codes only where an expert's rows fill three
    # or more row tiles (the 235B-A22B share: about 1024 rows), not at 30B (about 256 rows)
    fp8 = dict(mx, fwd=0)
    assert L.moe_workspace_bytes(_shape(L, **fp8))[0] == big[0]
    share = dict(T=16384, H=4096, I=1536, E=128, k=8, e_local=16)
    plain = L.moe_workspace_bytes(_shape(L, **share))
    fused = L.moe_workspace_bytes(_shape(L, **share, bwd=1))
    assert fused[0] >= plain[0] + 16 * 3 * 4096 * 1536 * (1 + 1 / 32)
    assert L.moe_workspace_bytes(_shape(L, **share, bwd=1, recompute=1))[0] == 0


def test_quantizer_arguments_are_checked_before_launch():
    L = _lib()
    bad = [
        dict(N=64, groups=0, Rp=128),      # no groups
        dict(N=64, groups=1025, Rp=128),   # more than 1024 groups
        dict(N=12, groups=2, Rp=128),      # N not a multiple of 8
        dict(N=64, groups=2, Rp=100),      # Rp not a multiple of 128
        dict(N=64, groups=2, Rp=-128),
        dict(N=72, groups=2, Rp=128, rows=True),   # row-wise output needs N % 32 == 0
        dict(N=64, groups=2, Rp=128, half=True),   # row codes without row scales
    ]
    for kw in bad:
        with pytest.raises(L.MoeError) as ei:
            rows = 8 if kw.get("rows") or kw.get("half") else 0
            L.moe_mx_quantize_cols(8, kw["N"], 8, kw["groups"], kw["Rp"], 8, 8, 8, rows, 0 if kw.get("half") else rows)
        assert ei.value.code == L.MOE_EINVAL, kw
    with pytest.raises(L.MoeError) as ei:
        L.moe_mx_quantize_cols(8, 64, 0, 2, 128, 8, 8, 8)     # offsets NULL
    assert ei.value.code == L.MOE_EINVAL
    with pytest.raises(L.MoeError) as ei:
        L.moe_mx_quantize(8, 4, 48, 8, 8)                     # K not a multiple of 32
    assert ei.value.code == L.MOE_EINVAL


def test_quotient_by_top_k_through_double_is_exact():
    """The kernels divide a row_src entry x (0 <= x < 2^31) by k (1..16) as
    trunc((x + 0.5) * (1.0 / k)) in double precision; check it against integer division on
    the residues next to every multiple of k near the ends of the range."""
    for k in range(1, 17):
        inv = 1.0 / k
        base = np.concatenate([np.arange(0, 4096), np.arange(2**31 - 4096 * k, 2**31 - 1, k)])
        x = np.unique(np.clip((base[:, None] // k * k + np.arange(-1, k + 1)[None, :]).ravel(), 0, 2**31 - 1))
        q = np.trunc((x.astype(np.float64) + 0.5) * inv).astype(np.int64)
        assert np.array_equal(q, x // k), k


def test_router_arguments_are_checked_before_launch():
    L = _lib()
    cases = [
        (dict(dtype=0), L.MOE_EUNSUPPORTED),   # fp32 data
        (dict(E=12, k=2), L.MOE_EUNSUPPORTED),  # E not a multiple of 8
    ]
    for kw, code in cases:
        for call in (lambda s: L.moe_router_fwd(s, 8, 8, 8, 8, 8, 8),
                     lambda s: L.moe_router_bwd(s, 8, 8, 8, 0, 8, 8, 8)):
            with pytest.raises(L.MoeError) as ei:
                call(_shape(L, **kw))
            assert ei.value.code == code
    s = _shape(L)
    with pytest.raises(L.MoeError) as ei:
        L.moe_router_fwd(s, 8, 0, 8, 8, 8, 8)       # w_r is NULL
    assert ei.value.code == L.MOE_EINVAL
    with pytest.raises(L.MoeError) as ei:
        L.moe_router_bwd(s, 8, 8, 8, 0, 8, 8, 0)    # scratch is NULL
    assert ei.value.code == L.MOE_EWORKSPACE
    with pytest.raises(L.MoeError) as ei:
        L.moe_router_bwd(s, 8, 8, 0, 0, 8, 8, 8)    # d_logits is NULL
    assert ei.value.code == L.MOE_EINVAL

