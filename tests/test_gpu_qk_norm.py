"""Parity of in-kernel q, k normalisation (CARVE_QK_L2NORM): q and k are raw,
and the kernels divide each token's q and k by their L2 norms over d_k. Every
case is checked against the float64 oracle run on l2_normalize of the same
stored raw values (and, for gradients, taken back through
l2_normalize_backward), with the bars of the forward pass (1e-4 for fp32
inputs, 2e-2 for bf16), through the C ABI: both forward schedules and widths,
the pairwise fallback, the decode step, and the backward pass's kernels.
"""
import numpy as np
import pytest

from chunk_gated_delta_carve_amd.workloads import WORKLOADS, bf16_bits_from_f32, make_inputs, to_f64, to_torch
from oracle import (carve_backward, carve_forward, carve_step, decay_from_logits, l2_normalize,
                    l2_normalize_backward, sigmoid)

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
KEYS = ("q", "k", "v", "g", "bx", "w")


def say(*a):
    print(*a, flush=True)


def rel_err(x, ref):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from chunk_gated_delta_carve_amd import _lib
    _lib.lib()                                   # loud failure if the library is missing
    return torch


def raw_inputs(name, dtype, B, H, T, d, L, rank, seed, logits=False):
    """The generator's inputs with q and k scaled by seeded per-token factors
    in [0.2, 5], stored again in the dtype: raw rows the kernels must normalise."""
    wl = WORKLOADS["tiny"].with_(name=name, dtype=dtype, B=B, H=H, T=T, dk=d, dv=d, L=L, rank=rank,
                                 ub_std=0.5, seed=seed)
    inp = make_inputs(wl, decay_logits=logits)
    rng = np.random.default_rng(seed + 1)
    for key in ("q", "k"):
        x = to_f64(inp[key], dtype) * rng.uniform(0.2, 5.0, size=(B, T, H, 1))
        inp[key] = x.astype(np.float32) if dtype == "f32" else bf16_bits_from_f32(x.astype(np.float32))
    return wl, inp


def start_state(B, H, d, seed):
    rng = np.random.default_rng(seed)
    return ((0.3 * rng.standard_normal((B, H, d, d))).astype(np.float32),
            (0.3 * rng.standard_normal((B, H, d))).astype(np.float32))


def oracle_inputs(inp, dtype, logits=False):
    f = {k: to_f64(v, dtype) for k, v in inp.items()}
    f["q"], f["k"] = l2_normalize(f["q"]), l2_normalize(f["k"])
    if logits:
        f["g"] = decay_from_logits(f["g"])
    return f


def assert_parity(got, ref, tol, what, names):
    errs = {n: rel_err(g, r) for n, g, r in zip(names, got, ref)}
    say(f"{what}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, g in zip(names, got):
        assert np.all(np.isfinite(g)), f"{what}: non-finite {n}"
    for n, e in errs.items():
        assert e <= tol, f"{what}: {n} rel err {e:.3e} > {tol}"


FWD_CASES = [
    # name, dtype, B, H, T, d, L, rank
    ("par-d64-ragged-300", "bf16", 2, 3, 300, 64, 64, 0),
    ("par-d128-ragged-200-L128", "bf16", 1, 2, 200, 128, 128, 0),
    ("ser-f32-d64-L64-r8", "f32", 1, 2, 256, 64, 64, 8),
    ("ser-bf16-d128-L32-r8-ragged-150", "bf16", 1, 2, 150, 128, 32, 8),
    ("ser-f32-d128-L16-r4", "f32", 1, 2, 96, 128, 16, 4),
    # the chunk-serial kernel's lean 64-token blocks (bf16, d = 64), ragged tail
    ("lean-bf16-d64-L64-r16-ragged-200", "bf16", 2, 2, 200, 64, 64, 16),
]


@pytest.mark.parametrize("name,dtype,B,H,T,d,L,rank", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_normalises_q_and_k(torch_cuda, name, dtype, B, H, T, d, L, rank):
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_fwd
    wl, inp = raw_inputs(name, dtype, B, H, T, d, L, rank, 7000 + T)
    say("case", wl)
    S_in, m_in = start_state(B, H, d, T)
    t = {k: to_torch(v, dtype) for k, v in inp.items()}
    o, S, m = chunk_fwd(*(t[k] for k in KEYS), L=L, ub_down=t.get("U_down"), ub_up=t.get("U_up"),
                        state_in=torch.from_numpy(S_in).cuda(), mean_in=torch.from_numpy(m_in).cuda(),
                        return_state=True, qk_l2norm=True)
    torch.cuda.synchronize()
    f = oracle_inputs(inp, dtype)
    ref = carve_forward(*(f[k] for k in KEYS), L, f.get("U_down"), f.get("U_up"),
                        state_in=S_in.astype(np.float64), mean_in=m_in.astype(np.float64))
    assert_parity((o.float().cpu().numpy(), S.cpu().numpy(), m.cpu().numpy()), ref, TOL[dtype], name,
                  ("o", "state_out", "mean_out"))


@pytest.mark.parametrize("dtype,rank", [("bf16", 0), ("f32", 8)], ids=["parallel-bf16", "serial-f32"])
def test_normalised_steep_decay_with_logits(torch_cuda, dtype, rank):
    """Both flags at once, with half the channels' logits at +10 (decay e^-10
    per token), so the pairwise Gram rebuild runs and normalises its rows."""
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_fwd
    wl, inp = raw_inputs(f"steep-{dtype}", dtype, 1, 3, 192, 64, 64, rank, 7100, logits=True)
    a = np.empty(inp["g"].shape, np.float32)
    a[..., :32] = 10.0
    a[..., 32:] = -4.0
    inp["g"] = a if dtype == "f32" else bf16_bits_from_f32(a)
    t = {k: to_torch(v, dtype) for k, v in inp.items()}
    o, S, m = chunk_fwd(*(t[k] for k in KEYS), L=64, ub_down=t.get("U_down"), ub_up=t.get("U_up"),
                        return_state=True, qk_l2norm=True, decay_logits=True)
    torch.cuda.synchronize()
    f = oracle_inputs(inp, dtype, logits=True)
    ref = carve_forward(*(f[k] for k in KEYS), 64, f.get("U_down"), f.get("U_up"))
    assert_parity((o.float().cpu().numpy(), S.cpu().numpy(), m.cpu().numpy()), ref, TOL[dtype],
                  f"steep, logits and norm ({dtype})", ("o", "state_out", "mean_out"))


def test_fused_norm_agrees_with_normalised_inputs(torch_cuda):
    """fp32: normalising inside the kernels equals handing them q and k that
    torch normalised, to fp32 rounding."""
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_fwd
    wl, inp = raw_inputs("agree", "f32", 2, 2, 256, 64, 64, 8, 7200)
    t = {k: to_torch(v, "f32") for k, v in inp.items()}
    ub = dict(ub_down=t["U_down"], ub_up=t["U_up"])
    fused = chunk_fwd(*(t[k] for k in KEYS), L=64, return_state=True, qk_l2norm=True, **ub)
    nq = torch.nn.functional.normalize(t["q"], dim=-1, eps=1e-12)
    nk = torch.nn.functional.normalize(t["k"], dim=-1, eps=1e-12)
    plain = chunk_fwd(nq, nk, t["v"], t["g"], t["bx"], t["w"], L=64, return_state=True, **ub)
    torch.cuda.synchronize()
    errs = [rel_err(x.cpu().numpy(), y.cpu().numpy()) for x, y in zip(fused, plain)]
    say("fused vs pre-normalised: " + ", ".join(f"{e:.2e}" for e in errs))
    assert max(errs) <= 1e-5


@pytest.mark.parametrize("dtype,d,L,rank", [("f32", 64, 16, 8), ("bf16", 128, 64, 16)], ids=["f32-d64", "bf16-d128"])
def test_step_normalises_q_and_k(torch_cuda, dtype, d, L, rank):
    torch = torch_cuda
    from chunk_gated_delta_carve_amd.api import recurrent_step
    B, H, T = 2, 2, 40
    wl, inp = raw_inputs(f"step-{dtype}", dtype, B, H, T, d, L, rank, 7300 + d)
    S_in, m_in = start_state(B, H, d, 9)
    t = {k: to_torch(v, dtype) for k, v in inp.items()}
    S, m = torch.from_numpy(S_in.copy()).cuda(), torch.from_numpy(m_in.copy()).cuda()
    acc = torch.zeros_like(m)
    outs = []
    for s_ in range(T):
        tok = {k: t[k][:, s_].clone() for k in KEYS}
        outs.append(recurrent_step(*(tok[k] for k in KEYS), S, m, acc, s_ % L, L, t["U_down"], t["U_up"],
                                   qk_l2norm=True).float())
    torch.cuda.synchronize()
    f = oracle_inputs(inp, dtype)
    Sr, mr, accr = S_in.astype(np.float64), m_in.astype(np.float64), np.zeros((B, H, d))
    ro = []
    for s_ in range(T):
        o_, Sr, mr, accr = carve_step(Sr, mr, accr, s_ % L, *(f[k][:, s_] for k in KEYS), L, f["U_down"], f["U_up"])
        ro.append(o_)
    got = (torch.stack(outs, 1).cpu().numpy(), S.cpu().numpy(), m.cpu().numpy(), acc.cpu().numpy())
    assert_parity(got, (np.stack(ro, 1), Sr, mr, accr), TOL[dtype], f"step {dtype} d{d}",
                  ("o", "state", "mean_prev", "chunk_acc"))


BWD_CASES = [
    # name, dtype, B, H, T, d, L, rank: the chunk-parallel kernel (bf16, d = 64,
    # rank 0), the row-lane kernels (rank 0; d = 64 with a projection) and the
    # per-head kernel (d = 128 with a projection)
    ("bwd-bf16-d64-r0-ragged-150", "bf16", 2, 2, 150, 64, 64, 0),
    ("bwd-bf16-d64-r0-L128-ragged-200", "bf16", 1, 3, 200, 64, 128, 0),
    ("bwd-f32-d128-r0", "f32", 1, 2, 96, 128, 32, 0),
    ("bwd-f32-d64-r8-ragged-75", "f32", 1, 2, 75, 64, 16, 8),
    ("bwd-f32-d128-r4", "f32", 1, 2, 64, 128, 32, 4),
]


@pytest.mark.parametrize("name,dtype,B,H,T,d,L,rank", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_through_the_normalisation(torch_cuda, name, dtype, B, H, T, d, L, rank):
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_bwd
    wl, inp = raw_inputs(name, dtype, B, H, T, d, L, rank, 7400 + T, logits=(rank == 8))
    say("case", wl)
    rng = np.random.default_rng(7500 + T)
    do = rng.standard_normal((B, T, H, d)).astype(np.float32)
    do = do if dtype == "f32" else bf16_bits_from_f32(do)
    dSo = (0.3 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    dmo = (0.3 * rng.standard_normal((B, H, d))).astype(np.float32)
    S_in, m_in = start_state(B, H, d, T)
    t = {k: to_torch(v, dtype) for k, v in inp.items()}
    cu = lambda x: torch.from_numpy(x).cuda()
    logits = rank == 8
    got = chunk_bwd(*(t[k] for k in KEYS), to_torch(do, dtype), L=L, ub_down=t.get("U_down"), ub_up=t.get("U_up"),
                    state_in=cu(S_in), mean_in=cu(m_in), d_state_out=cu(dSo), d_mean_out=cu(dmo),
                    decay_logits=logits, qk_l2norm=True)
    torch.cuda.synchronize()
    f = oracle_inputs(inp, dtype, logits=logits)
    ref = carve_backward(*(f[k] for k in KEYS), L, to_f64(do, dtype), f.get("U_down"), f.get("U_up"),
                         S_in.astype(np.float64), m_in.astype(np.float64), dSo.astype(np.float64),
                         dmo.astype(np.float64))
    ref["dq"] = l2_normalize_backward(to_f64(inp["q"], dtype), ref["dq"])
    ref["dk"] = l2_normalize_backward(to_f64(inp["k"], dtype), ref["dk"])
    if logits:
        ref["dg"] = ref["dg"] * -sigmoid(to_f64(inp["g"], dtype))
    names = ["dq", "dk", "dv", "dg", "dbx", "dw", "d_state_in", "d_mean_in"]
    rnames = ["dq", "dk", "dv", "dg", "dbx", "dw", "dstate_in", "dmean_in"]
    if rank:
        names += ["dub_down", "dub_up"]
        rnames += ["dU_down", "dU_up"]
    assert_parity([got[n].float().cpu().numpy() for n in names], [ref[n] for n in rnames], TOL[dtype], name, names)
