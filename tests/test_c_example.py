"""The C ABI from a plain C++ program (bwd_rope_apply_amd/examples/
rope_attn_example.cpp, built by the package build): no Python or torch in
the process that calls the library.  Its outputs must equal, bit for bit,
those of the same calls made through the Python binding, and meet the bf16
bar against the float64 oracle."""
import os
import subprocess

import numpy as np
import pytest

from bwd_rope_apply_amd import workloads as W
import harness as Hn

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXAMPLE = os.path.join(ROOT, "bwd_rope_apply_amd", "rope_attn_example")


def test_c_caller_matches_binding_and_oracle(tmp_path):
    import torch
    from bwd_rope_apply_amd import _lib
    if not os.path.exists(EXAMPLE):
        pytest.fail(f"{EXAMPLE} is not built: run `python -m bwd_rope_apply_amd.build`")
    wl = W.get("layer_2k", B=2, H=2, N=333, seed=21)
    inp = W.make_inputs(wl)
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    fin = tmp_path / "in.bin"
    with open(fin, "wb") as f:
        np.array([B, H, N, D, int(wl.causal)], dtype=np.int32).tofile(f)
        np.array([wl.base], dtype=np.float64).tofile(f)
        for n in ("q", "k", "v", "do"):
            np.ascontiguousarray(getattr(inp, n)).tofile(f)
        inp.alpha.astype(np.float32).tofile(f)
    fout = tmp_path / "out.bin"
    r = subprocess.run([EXAMPLE, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(fout, dtype=np.float32)
    n, nr = B * H * N * D, B * H * N
    sizes = [n, nr, n, n, n, D // 2]
    assert raw.size == sum(sizes)
    parts, off = [], 0
    for s in sizes:
        parts.append(raw[off:off + s])
        off += s
    c_out = dict(O=parts[0].reshape(B, H, N, D), LSE=parts[1].reshape(B, H, N),
                 dQ=parts[2].reshape(B, H, N, D), dK=parts[3].reshape(B, H, N, D),
                 dV=parts[4].reshape(B, H, N, D), dalpha=parts[5])

    # the same calls through the binding (shared workspace, backward reusing the forward)
    q, k, v, do = (Hn.to_device(getattr(inp, nm)) for nm in ("q", "k", "v", "do"))
    a = Hn.to_device(inp.alpha)
    ws = torch.empty(_lib.workspace_bytes("bwd", B, H, N, D, _lib.BF16, wl.causal), dtype=torch.uint8,
                     device="cuda")
    o, lse = _lib.fwd(q, k, v, wl.base, a, wl.causal, workspace=ws)
    st = _lib.STAGE_ALL & ~_lib.STAGE_PREP | _lib.STAGE_PREP_GRAD
    dq, dk, dv, da = _lib.bwd(q, k, v, o, do, lse, wl.base, a, wl.causal, workspace=ws, stages=st)
    torch.cuda.synchronize()
    py_out = dict(O=o, LSE=lse, dQ=dq, dK=dk, dV=dv, dalpha=da)
    for name, t in py_out.items():
        assert np.array_equal(c_out[name], t.cpu().numpy()), name

    ref = Hn.run_oracle(inp)
    for name in ("O", "dQ", "dK", "dV", "dalpha"):
        e = Hn.err_rms(c_out[name].astype(np.float64), ref[name])
        print(name, e)
        assert e <= 2e-2, (name, e)
