"""sagesla_fwd_noalloc: the forward with its workspace in the library's fixed device array.

Called through the C ABI twice in a row, the second time on a smaller input, each result
must equal sagesla_fwd's (with a caller-allocated workspace) on the same inputs: the same
kernels run, and the array's leftover contents from the first call must not leak into the
second. A shape whose workspace exceeds the array is rejected on the host."""
import pytest
import torch

import sparse_attention_sagesla_amd as S
from sparse_attention_sagesla_amd import _lib, synth

pytestmark = pytest.mark.gpu


def _noalloc(x, topk, out):
    B, H, N, d = x["q"].shape
    proj = x["proj"]
    return S.lib().sagesla_fwd_noalloc(x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(),
                                       proj.data_ptr() if proj is not None else None, B, H, N, d, topk, 64,
                                       out.data_ptr(), torch.cuda.current_stream().cuda_stream)


def test_noalloc_matches_fwd_on_two_calls():
    big = synth.scaled(synth.CONFIGS["wan14b-720p"], H=3, grid=(4, 20, 33), seed=61, name="noalloc-big")
    small = synth.scaled(synth.CONFIGS["wan1.3b-480p"], H=1, grid=(2, 9, 40), topk=0.2, seed=62, name="noalloc-small")
    assert S.workspace_size(small.B, small.H, small.N, topk=small.topk) < S.workspace_size(
        big.B, big.H, big.N, topk=big.topk) <= _lib_scratch_bytes()
    for cfg in (big, small):
        x = synth.make_inputs(cfg, device="cuda")
        out = torch.full_like(x["q"], float("nan"))
        assert _noalloc(x, cfg.topk, out) == 0
        ref = S.fwd(x["q"], x["k"], x["v"], x["proj"], topk=cfg.topk)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), cfg.name
        # and once more without the linear branch
        out2 = torch.empty_like(x["q"])
        assert _noalloc(dict(x, proj=None), cfg.topk, out2) == 0
        ref2 = S.fwd(x["q"], x["k"], x["v"], None, topk=cfg.topk)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref2), cfg.name


def _lib_scratch_bytes():
    return 256 << 20


def test_noalloc_rejects_shapes_beyond_its_array():
    # 40 heads of 75,600 tokens need about 5 GiB of workspace: rejected before any launch
    q = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    p = q.data_ptr()
    st = S.lib().sagesla_fwd_noalloc(p, p, p, p, 1, 40, 75600, 128, 0.1, 64, p, None)
    assert st == _lib.ERR_WORKSPACE
