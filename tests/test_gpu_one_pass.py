"""The one-pass chunk-parallel forward (bf16, d = 64, no content projection)
against the two-launch schedule and the float64 oracle, through the C ABI.

Both schedules evaluate the same per-block expressions with the same operand
roundings and the same MFMA order (the per-block affine map of the
gist.science technical summary, §2 and §2.1; Theorem 11 of §3), so o, the
final state and the final mean must agree bit for bit. The one-pass
workspace's sticky error word must stay zero (no bounded wait ran out, no
L2 exchange crossed an XCD), and its ready flags must be left clear, which
repeated calls on one workspace check.
"""
import numpy as np
import pytest

from chunk_gated_delta_carve_amd.workloads import WORKLOADS, make_inputs, to_f64, to_torch
from oracle import carve_forward

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from chunk_gated_delta_carve_amd import _lib
    _lib.lib()
    return torch


def rel_err(x, ref):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


def fwd(torch, t, L, two_pass, ws, S_in=None, m_in=None, **kw):
    from chunk_gated_delta_carve_amd import chunk_fwd
    o, S, m = chunk_fwd(*(t[k] for k in ("q", "k", "v", "g", "bx", "w")), L=L, state_in=S_in, mean_in=m_in,
                        return_state=True, workspace=ws, two_pass=two_pass, **kw)
    torch.cuda.synchronize()
    return o, S, m


def workspace(torch, B, H, T, L, two_pass, **kw):
    from chunk_gated_delta_carve_amd.api import make_config
    from chunk_gated_delta_carve_amd import _lib
    n = int(_lib.ref_shapes(make_config(B, H, T, 64, 64, L, 0, torch.bfloat16, two_pass=two_pass, **kw))
            .workspace_bytes)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")


SHAPES = [
    # name, B, H, T, L, with state_in / mean_in
    ("headline", 4, 12, 2048, 64, False),
    ("state-in", 2, 12, 1024, 64, True),
    ("T1", 1, 2, 1, 32, True),
    ("T64", 1, 1, 64, 64, False),
    ("ragged-100-L16", 1, 3, 100, 16, True),
    ("ragged-200-L128", 2, 2, 200, 128, True),     # the last chunk spans two 64-token blocks
    ("L128-T256", 1, 3, 256, 128, False),
    ("BH15", 3, 5, 256, 64, True),                 # head groups of eight end part-full
    ("nblk13", 2, 3, 832, 64, False),
    ("BH1-long", 1, 1, 4096, 64, True),
]


@pytest.mark.parametrize("name,B,H,T,L,with_state", SHAPES, ids=[s[0] for s in SHAPES])
def test_one_pass_bitwise_two_pass(torch_cuda, name, B, H, T, L, with_state):
    torch = torch_cuda
    from chunk_gated_delta_carve_amd.api import workspace_error
    wl = WORKLOADS["init_equiv"].with_(B=B, H=H, T=T, L=L, seed=4100 + T)
    say("case", name, wl)
    inp = make_inputs(wl)
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    S_in = m_in = None
    if with_state:
        g = torch.Generator().manual_seed(T)
        S_in = (0.3 * torch.randn(B, H, 64, 64, generator=g)).cuda()
        m_in = (0.3 * torch.randn(B, H, 64, generator=g)).cuda()
    ws1 = workspace(torch, B, H, T, L, False)
    ws2 = workspace(torch, B, H, T, L, True)
    a = fwd(torch, t, L, False, ws1, S_in, m_in)
    b = fwd(torch, t, L, True, ws2, S_in, m_in)
    assert workspace_error(ws1) == 0
    for n, x, y in zip(("o", "state", "mean"), a, b):
        assert torch.isfinite(x.float()).all(), f"{name}: non-finite {n}"
        assert torch.equal(x, y), f"{name}: {n} differs from the two-pass schedule"
    # the same workspace again (its flags must have been left clear)
    c = fwd(torch, t, L, False, ws1, S_in, m_in)
    assert workspace_error(ws1) == 0
    for x, y in zip(a, c):
        assert torch.equal(x, y)


@pytest.mark.parametrize("flags", [dict(decay_logits=True), dict(qk_l2norm=True),
                                   dict(decay_logits=True, qk_l2norm=True)],
                         ids=["logits", "l2norm", "logits+l2norm"])
def test_one_pass_input_modes_bitwise_two_pass(torch_cuda, flags):
    torch = torch_cuda
    from chunk_gated_delta_carve_amd.api import workspace_error
    wl = WORKLOADS["init_equiv"].with_(B=2, H=6, T=640, seed=4200)
    inp = make_inputs(wl, decay_logits=flags.get("decay_logits", False))
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    if flags.get("qk_l2norm"):
        t["q"] = (3.0 * t["q"].float()).to(torch.bfloat16)
        t["k"] = (0.5 * t["k"].float()).to(torch.bfloat16)
    ws1 = workspace(torch, 2, 6, 640, 64, False, **flags)
    ws2 = workspace(torch, 2, 6, 640, 64, True, **flags)
    a = fwd(torch, t, 64, False, ws1, **flags)
    b = fwd(torch, t, 64, True, ws2, **flags)
    assert workspace_error(ws1) == 0
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_one_pass_headline_oracle_sampled(torch_cuda):
    """The headline shape against the oracle on every (batch, head) pair of
    two batches' worth of heads (parity bar 2e-2 for bf16)."""
    torch = torch_cuda
    wl = WORKLOADS["init_equiv"]
    inp = make_inputs(wl)
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    o, S, m = fwd(torch, t, wl.L, False, workspace(torch, wl.B, wl.H, wl.T, wl.L, False))
    f = lambda k: to_f64(inp[k][:2], wl.dtype)
    ro, rS, rm = carve_forward(f("q"), f("k"), f("v"), f("g"), f("bx"), f("w"), wl.L)
    for n, x, r in (("o", o[:2], ro), ("state", S[:2], rS), ("mean", m[:2], rm)):
        e = rel_err(x.float().cpu().numpy(), r)
        say(f"one-pass headline {n}: {e:.2e}")
        assert e <= 2e-2


def test_default_workspace_survives_other_schedules(torch_cuda):
    """The binding hands its cached, zeroed one-pass workspace to one-pass
    calls only: calls of the two-launch pair and of the d = 128 pair in between
    (which use their workspace as scratch) leave it intact."""
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_fwd
    from chunk_gated_delta_carve_amd.api import forward_workspace, workspace_error
    wl = WORKLOADS["init_equiv"].with_(B=2, H=6, T=512, seed=4300)
    inp = make_inputs(wl)
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    args = [t[k] for k in ("q", "k", "v", "g", "bx", "w")]
    ref = [x.clone() for x in chunk_fwd(*args, L=64, return_state=True)]
    chunk_fwd(*args, L=64, return_state=True, two_pass=True)
    wide = WORKLOADS["init_equiv"].with_(B=1, H=2, T=256, dk=128, dv=128, seed=4301)
    winp = make_inputs(wide)
    chunk_fwd(*(to_torch(winp[k], wide.dtype) for k in ("q", "k", "v", "g", "bx", "w")), L=64)
    again = chunk_fwd(*args, L=64, return_state=True)
    torch.cuda.synchronize()
    for x, y in zip(ref, again):
        assert torch.equal(x, y)
    ws = forward_workspace(1, torch.device("cuda", torch.cuda.current_device()), torch.cuda.current_stream().cuda_stream)
    assert workspace_error(ws) == 0


def test_default_workspace_across_shapes(torch_cuda):
    """The flag layout depends on the shape and the rest of the workspace is
    scratch, so a shape change on the cached workspace must re-zero its flag
    prefix: a sequence of shapes, each repeated, all bit for bit the two-pass
    results."""
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_fwd
    from chunk_gated_delta_carve_amd.api import forward_workspace, workspace_error
    seq = [(1, 3, 100), (2, 3, 832), (2, 3, 832), (1, 3, 100), (4, 12, 2048), (1, 1, 64), (2, 3, 832)]
    for B, H, T in seq:
        wl = WORKLOADS["init_equiv"].with_(B=B, H=H, T=T, seed=4400 + T)
        inp = make_inputs(wl)
        t = [to_torch(inp[k], wl.dtype) for k in ("q", "k", "v", "g", "bx", "w")]
        a = chunk_fwd(*t, L=64, return_state=True)
        b = chunk_fwd(*t, L=64, return_state=True, two_pass=True)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), (B, H, T)
    ws = forward_workspace(1, torch.device("cuda", torch.cuda.current_device()), torch.cuda.current_stream().cuda_stream)
    assert workspace_error(ws) == 0
