"""The C-ABI library loads without a GPU, exports every declared entry point, and rejects
bad arguments on the host before anything is launched."""
import ctypes as C
import os
import re

import pytest
import torch

import sparse_attention_sagesla_amd as S
from sparse_attention_sagesla_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sagesla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sagesla_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = C.CDLL(_lib.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.EXPORTS) == names


def test_version_and_status_strings():
    assert S.lib().sagesla_version() >= 100
    for s in range(5):
        assert len(S.status_string(s)) > 0


def test_ksel_matches_rule():
    assert S.ksel(2048, 0.1) == 4
    assert S.ksel(32760, 0.1) == 52
    assert S.ksel(75600, 0.1) == 119
    assert S.ksel(75600, 0.15) == 178
    assert S.ksel(75600, 1.0) == 1182
    assert S.ksel(1920, 0.1) == 3
    assert S.ksel(37, 0.1) == 1


@pytest.mark.parametrize("args,status", [
    (dict(N=0), _lib.ERR_INVALID_ARGUMENT),
    (dict(N=(1 << 20) + 1), _lib.ERR_INVALID_ARGUMENT),
    (dict(d=64), _lib.ERR_UNSUPPORTED),
    (dict(block=128), _lib.ERR_UNSUPPORTED),
    (dict(topk=0.0), _lib.ERR_INVALID_ARGUMENT),
    (dict(topk=1.5), _lib.ERR_INVALID_ARGUMENT),
    (dict(topk=float("nan")), _lib.ERR_INVALID_ARGUMENT),
    (dict(B=0), _lib.ERR_INVALID_ARGUMENT),
])
def test_workspace_size_rejects(args, status):
    kw = dict(B=1, H=2, N=2048, d=128, block=64, topk=0.1)
    kw.update(args)
    out = C.c_size_t()
    st = S.lib().sagesla_workspace_size(kw["B"], kw["H"], kw["N"], kw["d"], kw["block"], kw["topk"], 1,
                                        C.byref(out))
    assert st == status


def test_workspace_layout_regions():
    lay = S.workspace_layout(1, 4, 1000, topk=0.2, linear=True)
    total = S.workspace_size(1, 4, 1000, topk=0.2, linear=True)
    assert lay["keys"] == total  # the score keys are the adaptive forward's alone
    offs = sorted(o for name, o in lay.items() if name != "keys")
    assert all(o % 256 == 0 for o in offs)
    assert len(set(offs)) == len(offs)  # every region present and distinct
    assert max(offs) < total
    no_lin = S.workspace_size(1, 4, 1000, topk=0.2, linear=False)
    assert no_lin < total
    lay0 = S.workspace_layout(1, 4, 1000, topk=0.2, linear=False)
    assert lay0["hs"] == no_lin and lay0["y"] == no_lin
    # topk = 1 keeps every block: the linear branch has nothing to do
    assert S.workspace_size(1, 4, 1000, topk=1.0, linear=True) == S.workspace_size(1, 4, 1000, topk=1.0,
                                                                                    linear=False)


def _fwd_status(q=0x10000, k=0x20000, v=0x30000, proj=None, B=1, H=2, N=2048, d=128, topk=0.1, block=64,
                out=0x40000, ws=0x50000, wsbytes=1 << 40):
    return S.lib().sagesla_fwd(q, k, v, proj, B, H, N, d, topk, block, out, ws, wsbytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.ERR_INVALID_ARGUMENT),
    (dict(out=None), _lib.ERR_INVALID_ARGUMENT),
    (dict(ws=None), _lib.ERR_INVALID_ARGUMENT),
    (dict(k=0x20008), _lib.ERR_INVALID_ARGUMENT),     # misaligned
    (dict(proj=0x60004), _lib.ERR_INVALID_ARGUMENT),  # misaligned optional pointer
    (dict(d=96), _lib.ERR_UNSUPPORTED),
    (dict(block=32), _lib.ERR_UNSUPPORTED),
    (dict(topk=-0.1), _lib.ERR_INVALID_ARGUMENT),
    (dict(N=-5), _lib.ERR_INVALID_ARGUMENT),
    (dict(wsbytes=100), _lib.ERR_WORKSPACE),
])
def test_fwd_rejects_before_launch(kw, status):
    # the pointers are never dereferenced: validation fails on the host first
    assert _fwd_status(**kw) == status


def test_stage_entry_points_reject_bad_arguments():
    L = S.lib()
    p = 0x10000
    assert L.sagesla_pool(None, p, p, 1, 1, 64, 128, 64, p, p, p, p, p, p, None) == _lib.ERR_INVALID_ARGUMENT
    assert L.sagesla_select(p, p, 1, 1, 64, 128, 64, 2.0, p, None) == _lib.ERR_INVALID_ARGUMENT
    assert L.sagesla_sparse_attn(p, p, p, p, p, p, p, 0x7, 1, 1, 64, 128, 64, 0.5, p, None) == \
        _lib.ERR_INVALID_ARGUMENT
    assert L.sagesla_quant_kv(p, p, p, p, 1, 1, 64, 128, 64, p, p, p, None, p, None) == \
        _lib.ERR_INVALID_ARGUMENT
    assert L.sagesla_linear_complement(p, p, p, p, None, 1, 1, 64, 128, 64, 0.1, p, p, p, p, p, None) == \
        _lib.ERR_INVALID_ARGUMENT
    assert L.sagesla_linear_total(p, 1, 1, 64, 128, 64, None, None) == _lib.ERR_INVALID_ARGUMENT


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path; a GPU is present")
def test_valid_arguments_without_device_report_hip_error():
    # all arguments valid: validation passes, the device check fails, nothing is launched
    assert _fwd_status() in (_lib.ERR_HIP, _lib.ERR_UNSUPPORTED)


def test_python_binding_rejects_cpu_tensors():
    q = torch.zeros(1, 1, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        S.fwd(q, q, q)


@pytest.mark.parametrize("M,N,K", [(0, 256, 128), (1, 128, 128), (1, 384, 128), (1, 256, 100), (1, 256, 0),
                                   ((1 << 24) + 1, 256, 128), (1, 256, 1 << 17)])
def test_w8a8_sizes_rejects(M, N, K):
    out = [C.c_size_t() for _ in range(4)]
    st = S.lib().sagesla_w8a8_sizes(M, N, K, *[C.byref(o) for o in out])
    assert st == _lib.ERR_INVALID_ARGUMENT


def test_w8a8_sizes():
    sz = S.w8a8_sizes(300, 512, 384)
    assert sz == {"x8": 512 * 384, "sx": 3 * 512 * 4, "w8": 512 * 384, "sw": 4 * 3 * 4}
    sz = S.w8a8_sizes(75600, 5120, 5120)
    assert sz["x8"] == 75776 * 5120 and sz["sx"] == 40 * 75776 * 4


def test_sla_workspace_regions():
    lay = S.sla_workspace_layout(1, 4, 1000, topk=0.2, linear=True)
    total = S.sla_workspace_size(1, 4, 1000, topk=0.2, linear=True)
    offs = sorted(o for name, o in lay.items() if name != "keys")  # no score keys in training
    assert all(o % 256 == 0 for o in offs)
    assert len(set(offs)) == len(offs) and max(offs) < total
    # the training workspace holds the forward's regions at the same offsets
    fwd = S.workspace_layout(1, 4, 1000, topk=0.2, linear=True)
    assert all(lay[n] == fwd[n] for n in fwd)
    assert S.sla_workspace_size(1, 4, 1000, topk=0.2, linear=False) < total


def test_sla_bwd_rejects_on_host():
    L = S.lib()
    p = C.c_void_p(1 << 20)  # never dereferenced: the checks fail first
    # proj given without dproj (and the reverse)
    st = L.sagesla_sla_bwd(p, p, p, p, p, 1, 2, 256, 128, 0.2, 64, p, p, p, None, p, 1 << 30, None)
    assert st == _lib.ERR_INVALID_ARGUMENT
    st = L.sagesla_sla_bwd(p, p, p, None, p, 1, 2, 256, 128, 0.2, 64, p, p, p, p, p, 1 << 30, None)
    assert st == _lib.ERR_INVALID_ARGUMENT
    # unsupported head dimension; workspace too small
    st = L.sagesla_sla_bwd(p, p, p, None, p, 1, 2, 256, 64, 0.2, 64, p, p, p, None, p, 1 << 30, None)
    assert st == _lib.ERR_UNSUPPORTED
    st = L.sagesla_sla_fwd(p, p, p, None, 1, 2, 256, 128, 0.2, 64, p, p, 1024, None)
    assert st == _lib.ERR_WORKSPACE


def test_prepare_rejects_on_host():
    L = S.lib()
    p = C.c_void_p(1 << 20)
    for eps in (-1.0, float("nan"), float("inf")):
        st = L.sagesla_prepare(p, p, p, eps, 1, 2, 256, 128, 0.1, 64, 1, p, p, p, p, 1 << 30, None)
        assert st == _lib.ERR_INVALID_ARGUMENT
    st = L.sagesla_prepare(p, p, p, 1e-6, 1, 2, 256, 128, 0.1, 64, 1, p, p, p, p, 16, None)
    assert st == _lib.ERR_WORKSPACE
    unaligned = C.c_void_p((1 << 20) + 2)
    st = L.sagesla_prepare(unaligned, p, p, 1e-6, 1, 2, 256, 128, 0.1, 64, 1, p, p, p, p, 1 << 30, None)
    assert st == _lib.ERR_INVALID_ARGUMENT


def test_export_list_is_the_documented_boundary():
    # the boundary: the whole forward (plain and with tensor descriptors), the grouped
    # stages, every single stage, the workspace queries, and the next-step workloads
    want = {"sagesla_fwd", "sagesla_fwd_tensors", "sagesla_workspace_size", "sagesla_workspace_layout",
            "sagesla_pool_select", "sagesla_quantize", "sagesla_linear_states", "sagesla_linear_complement",
            "sagesla_sparse_attn", "sagesla_pool", "sagesla_head_stats", "sagesla_select", "sagesla_quant_kv",
            "sagesla_linear_total", "sagesla_ksel", "sagesla_version", "sagesla_status_string"}
    assert want <= set(declared_functions())


def _desc(shape, dtype=_lib.DT_BF16, data=0x10000, stride=None):
    d = _lib.Tensor()
    d.data, d.dtype, d.ndim = data, dtype, len(shape)
    st, acc = [0] * len(shape), 1
    for a in range(len(shape) - 1, -1, -1):
        st[a] = acc
        acc *= shape[a]
    for a in range(len(shape)):
        d.shape[a] = shape[a]
        d.stride[a] = (stride or st)[a]
    return d


def _fwd_tensors(q=None, k=None, v=None, proj=None, out=None, ws=None, topk=0.1, block=64):
    shp = (1, 2, 2048, 128)
    q = q or _desc(shp)
    k = k or _desc(shp)
    v = v or _desc(shp)
    out = out or _desc(shp)
    ws = ws or _desc((1 << 30,), _lib.DT_U8)
    P = C.byref
    return S.lib().sagesla_fwd_tensors(P(q), P(k), P(v), P(proj) if proj is not None else None, topk, block, P(out),
                                       P(ws), None)


@pytest.mark.parametrize("case", ["dtype", "rank", "stride", "shape", "proj-shape", "proj-dtype", "ws-dtype", "null"])
def test_fwd_tensors_rejects_descriptors_on_host(case):
    shp = (1, 2, 2048, 128)
    kw = {}
    if case == "dtype":
        kw["q"] = _desc(shp, _lib.DT_F32)
    elif case == "rank":
        kw["k"] = _desc((2, 2048, 128))
    elif case == "stride":  # a transposed (non-contiguous) view
        kw["v"] = _desc(shp, stride=[2 * 2048 * 128, 2048 * 128, 1, 2048])
    elif case == "shape":
        kw["out"] = _desc((1, 2, 2047, 128))
    elif case == "proj-shape":
        kw["proj"] = _desc((128, 64))
    elif case == "proj-dtype":
        kw["proj"] = _desc((128, 128), _lib.DT_F32)
    elif case == "ws-dtype":
        kw["ws"] = _desc((1 << 30,), _lib.DT_BF16)
    elif case == "null":
        kw["q"] = _desc(shp, data=0)
    assert _fwd_tensors(**kw) == _lib.ERR_INVALID_ARGUMENT


def test_fwd_tensors_size_rules_match_fwd():
    # sizes pass the descriptor checks and then meet the same rules as sagesla_fwd
    assert _fwd_tensors(q=_desc((1, 2, 2048, 64)), k=_desc((1, 2, 2048, 64)), v=_desc((1, 2, 2048, 64)),
                        out=_desc((1, 2, 2048, 64))) == _lib.ERR_UNSUPPORTED
    assert _fwd_tensors(ws=_desc((100,), _lib.DT_U8)) == _lib.ERR_WORKSPACE
    assert _fwd_tensors(topk=0.0) == _lib.ERR_INVALID_ARGUMENT


def test_grouped_stage_entry_points_reject_bad_arguments():
    L = S.lib()
    p = 0x10000
    assert L.sagesla_pool_select(p, p, p, 1, 1, 64, 128, 64, 0.0, *([p] * 9), None) == _lib.ERR_INVALID_ARGUMENT
    assert L.sagesla_pool_select(p, p, p, 1, 1, 64, 128, 64, 0.5, *([p] * 8), None, None) == \
        _lib.ERR_INVALID_ARGUMENT
    assert L.sagesla_quantize(p, p, p, p, 1, 1, 64, 64, 64, p, p, p, None) == _lib.ERR_UNSUPPORTED
    assert L.sagesla_quantize(p, p, p, p, 1, 1, 64, 128, 64, p, 0x3, p, None) == _lib.ERR_INVALID_ARGUMENT
    assert L.sagesla_linear_states(p, p, p, p, 1, 1, 64, 128, 64, p, p, p, p, p, None, None) == \
        _lib.ERR_INVALID_ARGUMENT


def test_header_documents_the_kept_list_order():
    text = open(HEADER).read()
    assert "best first" in text and "stored ascending" not in text


def test_adaptive_entry_points_reject_on_host():
    L = S.lib()
    p = 0x10000
    sz = C.c_size_t()
    # topk_min <= topk_max within (0, 1]; tau within (0, 1]
    for tmin, tmax, tau in [(0.0, 0.5, 0.5), (0.6, 0.5, 0.5), (0.1, 1.5, 0.5), (0.1, 0.5, 0.0), (0.1, 0.5, 1.01)]:
        assert L.sagesla_adaptive_ksel(p, p, 1, 1, 4096, 128, 64, tmin, tmax, tau, p, p, None) == \
            _lib.ERR_INVALID_ARGUMENT
        assert L.sagesla_fwd_adaptive(p, p, p, None, 1, 1, 4096, 128, tmin, tmax, tau, 64, p, p, p, p, 1 << 30,
                                      None) == _lib.ERR_INVALID_ARGUMENT
    # more than 8192 key blocks is not supported; 8192 is
    assert L.sagesla_adaptive_workspace_size(1, 1, 8193 * 64, 128, 64, 0.1, 0.2, 1, C.byref(sz)) == \
        _lib.ERR_UNSUPPORTED
    assert L.sagesla_fwd_adaptive(p, p, p, None, 1, 1, 8193 * 64, 128, 0.1, 0.2, 0.5, 64, p, p, p, p, 1 << 40,
                                  None) == _lib.ERR_UNSUPPORTED
    assert L.sagesla_adaptive_workspace_size(1, 1, 8192 * 64, 128, 64, 0.1, 0.2, 1, C.byref(sz)) == _lib.OK
    # missing outputs, small workspace
    assert L.sagesla_fwd_adaptive(p, p, p, None, 1, 1, 4096, 128, 0.1, 0.2, 0.5, 64, p, None, p, p, 1 << 30,
                                  None) == _lib.ERR_INVALID_ARGUMENT
    assert L.sagesla_fwd_adaptive(p, p, p, None, 1, 1, 4096, 128, 0.1, 0.2, 0.5, 64, p, p, p, p, 100, None) == \
        _lib.ERR_WORKSPACE


def test_adaptive_workspace_is_the_fixed_layout_at_the_largest_count():
    # the same regions as the fixed-count forward at topk_max, with the linear regions
    # whenever some head may leave blocks out, plus the score keys [BH][Nb][Nb] at the end
    B, H, N = 1, 3, 5000
    Nb = (N + 63) // 64
    ada = S.adaptive_workspace_layout(B, H, N, topk_min=0.05, topk_max=0.25)
    fix = S.workspace_layout(B, H, N, topk=0.25)
    fixed_total = S.workspace_size(B, H, N, topk=0.25)
    assert fix["keys"] == fixed_total
    assert {k: v for k, v in ada.items() if k != "keys"} == {k: v for k, v in fix.items() if k != "keys"}
    assert ada["keys"] == fixed_total
    keys_bytes = B * H * Nb * Nb * 8
    assert S.adaptive_workspace_size(B, H, N, topk_min=0.05, topk_max=0.25) == fixed_total + (keys_bytes + 255) // 256 * 256
    lay = S.adaptive_workspace_layout(1, 2, 1000, topk_min=0.1, topk_max=1.0)
    assert lay["hs"] < lay["keys"] < S.adaptive_workspace_size(1, 2, 1000, topk_min=0.1, topk_max=1.0)
