"""GPU parity of block-list attention (each 128-row query block attends its
own key block plus listed key blocks: the exact part of Multipole Semantic
Attention, "Retrieval-augmented approximation") against the float64 oracle
restricted to the same blocks.

Lists are seeded (workloads.block_lists) and, where marked, carry entries the
library must ignore or merge (duplicates, out-of-range indices, later blocks
under the causal mask).  Bars as for dense attention: fp32 max-rel <= 1e-4,
bf16 max |err| / rms(ref) <= 2e-2 per tensor, LSE within 2e-2 absolute.
"""
import numpy as np
import pytest

from bwd_rope_apply_amd import workloads as W
import harness as Hn
from test_parity import _check, BF16_TOL, NAMES

pytestmark = pytest.mark.gpu


def _lists(wl, retrieved, causal=None, noise=True, seed=5):
    causal = wl.causal if causal is None else causal
    return W.block_lists(wl.B, wl.H, wl.N, retrieved, causal, seed, noise=noise)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("D", [64, 128])
def test_bf16_block_lists(causal, D):
    """N = 700 (five full blocks and a 60-row tail), two retrieved blocks per
    query block plus noise entries."""
    wl = W.Workload("bf16_blocks", 2, 2, 700, D, "bf16", 1e4, causal, ("normal", 1.0, 1.0),
                    ("normal", 1.0, 1.0), ("normal", 1.0, 1.0), ("normal", 0.2, 1.0), seed=31)
    print(wl.name, causal, D, flush=True)
    _check(W.make_inputs(wl), causal=causal, opts=dict(block_lists=_lists(wl, 2, causal)))


@pytest.mark.parametrize("N,causal", [(790, True), (790, False), (850, True), (850, False),
                                      (1, True), (128, True), (129, False), (300, True)])
def test_bf16_block_list_lengths(N, causal):
    """Last blocks of 22 and 82 rows (the step that starts past N is cut),
    one row, exactly one block, one block plus a row."""
    wl = W.get("long_8k", B=1, H=2, N=N, seed=900 + N)
    print(wl.name, causal, flush=True)
    _check(W.make_inputs(wl), causal=causal, opts=dict(block_lists=_lists(wl, 3, causal)))


@pytest.mark.parametrize("causal", [True, False])
def test_bf16_diagonal_only(causal):
    """Empty lists: block-diagonal attention (each query block sees only its
    own block)."""
    wl = W.get("layer_2k", B=1, H=3, N=500)
    print(wl.name, causal, flush=True)
    _check(W.make_inputs(wl), causal=causal,
           opts=dict(block_lists=_lists(wl, 0, causal, noise=False)))


@pytest.mark.parametrize("N,causal", [(700, True), (832, True), (700, False), (832, False)])
def test_full_lists_match_dense(N, causal):
    """Lists naming every block give dense attention.  Under the causal mask
    the kernels walk the same tiles in the same order as the dense path that
    recomputes the scores for dQ (the smallest workspace; block lists never
    use the dS panels), and the exact corner is one block in both at
    N <= 8192, so the results are bit-identical; without it the ragged block
    may take the masked tile body where the dense path does not, which
    changes no value but is compared to 1e-6 of the RMS.  128 heads keep the
    dense dK/dV launch large enough (>= 512 workgroups) that it does not
    split its query range between two wave groups, which would sum dK, dV
    in another order."""
    import torch
    wl = W.get("layer_2k", B=1, H=128, N=N, seed=N)
    inp = W.make_inputs(wl)
    nb = (N + 127) // 128
    full = [[[list(range(nb))] * nb for _ in range(wl.H)] for _ in range(wl.B)]
    print(wl.name, causal, flush=True)
    a = Hn.run_gpu(inp, causal, ws="bwd_min")
    b = Hn.run_gpu(inp, causal, opts=dict(block_lists=full))
    for n in NAMES + ("LSE",):
        d = float(np.max(np.abs(a[n] - b[n])))
        print(n, d)
        if causal:
            assert d == 0.0, (n, d)
        else:
            assert d <= 1e-6 * float(np.sqrt(np.mean(np.square(a[n])))), (n, d)


@pytest.mark.parametrize("causal", [True, False])
def test_fp32_block_lists(causal):
    """The exact float32 path with block lists (fp32 bar)."""
    wl = W.get("tiny_fp32", B=1, H=2, N=300)
    print(wl.name, causal, flush=True)
    _check(W.make_inputs(wl), causal=causal, opts=dict(block_lists=_lists(wl, 1, causal)))


def test_bf16_block_lists_with_frequency_options():
    """Block lists combined with partial RoPE, a softmax scale and an offset."""
    wl = W.get("long_8k", B=1, H=2, N=600)
    opts = dict(block_lists=_lists(wl, 2), unrotated_pairs=16, scale=0.13, pos_offset=4096)
    _check(W.make_inputs(wl), opts=opts)


@pytest.mark.parametrize("name,N", [("long_8k", 700), ("tiny_fp32", 260)])
def test_block_lists_backward_reusing_forward_workspace(name, N):
    """PREP_GRAD on the forward's workspace reuses its visibility mask:
    bit-identical to a standalone backward."""
    import torch
    from bwd_rope_apply_amd import _lib, fwd, bwd
    wl = W.get(name, B=1, H=2, N=N)
    inp = W.make_inputs(wl)
    q, k, v, do = (Hn.to_device(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    a = Hn.to_device(inp.alpha)
    opts = Hn.device_opts(dict(block_lists=_lists(wl, 2)))
    dt = _lib.BF16 if wl.dtype == "bf16" else _lib.FP32
    ws = torch.empty(_lib.workspace_bytes("bwd", 1, 2, N, wl.D, dt, wl.causal), dtype=torch.uint8,
                     device="cuda")
    o, lse = fwd(q, k, v, wl.base, a, wl.causal, workspace=ws, opts=opts)
    ref = bwd(q, k, v, o, do, lse, wl.base, a, wl.causal, opts=opts)
    st = _lib.STAGE_ALL & ~_lib.STAGE_PREP | _lib.STAGE_PREP_GRAD
    got = bwd(q, k, v, o, do, lse, wl.base, a, wl.causal, workspace=ws, stages=st, opts=opts)
    torch.cuda.synchronize()
    for x, y in zip(ref, got):
        assert torch.equal(x, y)


def test_block_lists_full_size_long_8k():
    """long_8k at full size (B1 H32 N8192 D128) with eight retrieved blocks
    per query block, in the launch configuration the benchmark's block-list
    mode times: two complete heads against the oracle; dalpha against its
    definition, theta_hat_m * sum_p p * wedge(x_p, g_p), on the GPU's own dQ
    and dK (which the two heads pin), and rotational balance on every head."""
    from oracle import ref
    wl = W.get("long_8k")
    inp = W.make_inputs(wl)
    lists = W.block_lists(wl.B, wl.H, wl.N, 8, True, 8192)
    print(wl.name, "block lists", flush=True)
    got = Hn.run_gpu(inp, opts=dict(block_lists=lists))
    q, k, v, do = (inp.f64(n) for n in ("q", "k", "v", "do"))
    refs, gots = {n: [] for n in ("O", "dQ", "dK", "dV")}, {n: [] for n in ("O", "dQ", "dK", "dV")}
    for h in (0, wl.H - 1):
        sl = (slice(0, 1), slice(h, h + 1))
        sel = [[lists[0][h]]]
        o, lse = ref.ref_fwd(q[sl], k[sl], v[sl], wl.base, inp.alpha, True, blocks=sel)
        dq, dk, dv, _ = ref.ref_bwd(q[sl], k[sl], v[sl], o, do[sl], lse, wl.base, inp.alpha, True,
                                    blocks=sel)
        for n, r in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
            refs[n].append(r[0, 0])
            gots[n].append(got[n][0, h])
        assert float(np.abs(got["LSE"][0, h] - lse[0, 0]).max()) <= BF16_TOL
    errs = {n: Hn.err_rms(np.stack(gots[n]), np.stack(refs[n])) for n in refs}
    print(errs, flush=True)
    for n, e in errs.items():
        assert e <= BF16_TOL, (n, e)

    wq = (q[..., 0::2] * got["dQ"][..., 1::2] - q[..., 1::2] * got["dQ"][..., 0::2])
    wk = (k[..., 0::2] * got["dK"][..., 1::2] - k[..., 1::2] * got["dK"][..., 0::2])
    scale = np.abs(wq).sum(axis=2).max()
    assert np.abs(wq.sum(axis=2) + wk.sum(axis=2)).max() <= 1e-3 * scale
    pos = np.arange(wl.N, dtype=np.float64)[:, None]
    th = ref.theta_hat(wl.base, inp.alpha, wl.D)
    prop = th * ((pos * wq).sum(axis=(0, 1, 2)) + (pos * wk).sum(axis=(0, 1, 2)))
    e = Hn.err_rms(got["dalpha"], prop)
    print("dalpha vs its definition on the GPU's dQ, dK:", e, flush=True)
    assert e <= 1e-3
