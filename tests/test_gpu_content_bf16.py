"""bf16 parity of the content-gated path where the content projection matters.

The content bias z = U_up (U_down m_{c-1}) moves the erase gate of every
chunk (gist.science technical summary, §2.1 "Content-Aware Erase via Output
Reuse"). On the standard workloads it moves o by about 1e-5 relative, far
below the bf16 bar of 2e-2, so parity there cannot show that the bf16 content
bias is right. Here the recipe makes erasing matter: a long memory (the
log-decay g scaled by 0.02), an erase logit b_x = 0 (b = 1/2 without the
bias), rank-16 factors with standard deviation 2 and a nonzero mean_in (so
chunk 0 is gated too). Each case first checks with the oracle alone that the
projection moves o by at least ten times the bar, then checks the GPU against
the oracle. The cases cover the eight-wave layout (d = 64, blocks of 32 and
64 tokens) and the one-wave-per-slice layout (d = 128, blocks of 16 and 64
tokens, and L = 128 as two 64-token blocks per chunk).
"""
import numpy as np
import pytest

from chunk_gated_delta_carve_amd.workloads import WORKLOADS, bf16_bits_from_f32, make_inputs, to_f64, to_torch
from oracle import carve_forward

pytestmark = pytest.mark.gpu
TOL = 2e-2

CASES = [
    # name, d, L, seed
    ("d64-L32", 64, 32, 9196),
    ("d64-L64", 64, 64, 9228),
    ("d128-L16", 128, 16, 9300),
    ("d128-L64", 128, 64, 9292),
    ("d128-L128", 128, 128, 9356),
]


def say(*a):
    print(*a, flush=True)


def rel_err(x, ref):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


def content_inputs(d, L, seed):
    wl = WORKLOADS["tiny"].with_(name="content-bf16", dtype="bf16", B=1, H=2, T=512, dk=d, dv=d, L=L, rank=16,
                                 ub_std=2.0, seed=seed)
    inp = make_inputs(wl)
    g = to_f64(inp["g"], "bf16") * 0.02
    inp["g"] = bf16_bits_from_f32(g.astype(np.float32))
    inp["bx"] = bf16_bits_from_f32(np.zeros(inp["bx"].shape, np.float32))
    m_in = np.random.default_rng(seed).standard_normal((1, 2, d)).astype(np.float32)
    return wl, inp, m_in


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from chunk_gated_delta_carve_amd import _lib
    _lib.lib()
    return torch


@pytest.mark.parametrize("name,d,L,seed", CASES, ids=[c[0] for c in CASES])
def test_content_bf16_moves_output_and_matches(torch_cuda, name, d, L, seed):
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_fwd
    wl, inp, m_in = content_inputs(d, L, seed)
    say("case", name, wl)
    f = lambda k: to_f64(inp[k], "bf16")
    m64 = m_in.astype(np.float64)
    ref = carve_forward(f("q"), f("k"), f("v"), f("g"), f("bx"), f("w"), L, f("U_down"), f("U_up"), mean_in=m64)
    ref0 = carve_forward(f("q"), f("k"), f("v"), f("g"), f("bx"), f("w"), L, mean_in=m64)
    effect = rel_err(ref0[0], ref[0])
    say(f"{name}: the projection moves o by {effect:.3f} (bar {TOL})")
    assert effect >= 10 * TOL
    t = {k: to_torch(v, "bf16") for k, v in inp.items()}
    o, S, m = chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["bx"], t["w"], L=L, ub_down=t["U_down"], ub_up=t["U_up"],
                        mean_in=torch.from_numpy(m_in).cuda(), return_state=True)
    torch.cuda.synchronize()
    got = (o.float().cpu().numpy(), S.cpu().numpy(), m.cpu().numpy())
    errs = [rel_err(x, r) for x, r in zip(got, ref)]
    say(f"{name}: o {errs[0]:.2e}, state {errs[1]:.2e}, mean {errs[2]:.2e}")
    for n, x in zip(("o", "state", "mean"), got):
        assert np.all(np.isfinite(x)), f"{name}: non-finite {n}"
    for n, e in zip(("o", "state", "mean"), errs):
        assert e <= TOL, f"{name}: {n} rel err {e:.3e} > {TOL}"
