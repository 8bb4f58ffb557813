"""The no-allocation forward (rope_attn_fwd_noalloc, workspace in the
library's fixed device array) against the forward with a caller workspace:
bit-identical outputs, on two calls in a row, the second smaller."""
import numpy as np
import pytest

from bwd_rope_apply_amd import workloads as W
import harness as Hn

pytestmark = pytest.mark.gpu


def _ref_and_noalloc(wl):
    import torch
    from bwd_rope_apply_amd import _lib, fwd
    inp = W.make_inputs(wl)
    q, k, v = (Hn.to_device(getattr(inp, n)) for n in ("q", "k", "v"))
    a = Hn.to_device(inp.alpha)
    o_ref, lse_ref = fwd(q, k, v, wl.base, a, wl.causal)
    B, H, N, D = q.shape
    o = torch.full((B, H, N, D), float("nan"), device="cuda")
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    lib = _lib.load()
    st = lib.rope_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), B, H, N, D,
                                   _lib.BF16 if wl.dtype == "bf16" else _lib.FP32, float(wl.base),
                                   a.data_ptr(), int(wl.causal),
                                   torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    torch.cuda.synchronize()
    return (o_ref, lse_ref), (o, lse), inp


def test_noalloc_forward_matches_forward_twice():
    import torch
    for wl in (W.get("layer_2k", B=2, H=4, N=1500, seed=31), W.get("long_8k", B=1, H=2, N=300, seed=32)):
        print(wl.name, flush=True)
        (o_ref, lse_ref), (o, lse), inp = _ref_and_noalloc(wl)
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        ref = Hn.run_oracle(inp)
        assert Hn.err_rms(o.double().cpu().numpy(), ref["O"]) <= 2e-2


def test_noalloc_fp32_and_too_large():
    import torch
    from bwd_rope_apply_amd import _lib
    (o_ref, lse_ref), (o, lse), _ = _ref_and_noalloc(W.get("tiny_fp32"))
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    q = torch.zeros((1, 32, 8192, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(_lib.RopeAttnError) as e:
        _lib.fwd_noalloc(q, q, q, 1e4)
    assert e.value.status == -5
