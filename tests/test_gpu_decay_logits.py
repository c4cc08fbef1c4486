"""Parity of the in-kernel decay activation (CARVE_DECAY_LOGITS): the g input
holds raw decay logits a and the kernels form g = -softplus(a) themselves.
Every case is checked against the float64 oracle run on decay_from_logits(a)
of the same stored logits, with the bars of the forward pass (1e-4 for fp32
inputs, 2e-2 for bf16), through the C ABI: both forward schedules (the
chunk-parallel pair and the chunk-serial kernel), both widths, ragged tails,
decays steep enough for the pairwise fallback, and the decode step.
"""
import numpy as np
import pytest

from chunk_gated_delta_carve_amd.workloads import WORKLOADS, bf16_bits_from_f32, make_inputs, to_f64, to_torch
from oracle import carve_forward, carve_step, decay_from_logits

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


def workload(name, dtype, B, H, T, d, L, rank, seed):
    return WORKLOADS["tiny"].with_(name=name, dtype=dtype, B=B, H=H, T=T, dk=d, dv=d, L=L, rank=rank,
                                   ub_std=0.5, seed=seed)


def start_state(B, H, d, seed):
    rng = np.random.default_rng(seed)
    return ((0.3 * rng.standard_normal((B, H, d, d))).astype(np.float32),
            (0.3 * rng.standard_normal((B, H, d))).astype(np.float32))


def fwd_gpu(torch, inp, dtype, L, S_in, m_in, logits=True, g_override=None):
    from chunk_gated_delta_carve_amd import chunk_fwd
    t = {k: to_torch(v, dtype) for k, v in inp.items()}
    g = t["g"] if g_override is None else g_override
    o, S, m = chunk_fwd(t["q"], t["k"], t["v"], g, t["bx"], t["w"], L=L,
                        ub_down=t.get("U_down"), ub_up=t.get("U_up"),
                        state_in=torch.from_numpy(S_in).cuda(), mean_in=torch.from_numpy(m_in).cuda(),
                        return_state=True, decay_logits=logits)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), m.cpu().numpy()


def fwd_oracle(inp, dtype, L, S_in, m_in):
    f = lambda key: to_f64(inp[key], dtype)
    return carve_forward(f("q"), f("k"), f("v"), decay_from_logits(f("g")), f("bx"), f("w"), L,
                         f("U_down") if "U_down" in inp else None, f("U_up") if "U_up" in inp else None,
                         state_in=S_in.astype(np.float64), mean_in=m_in.astype(np.float64))


def assert_parity(got, ref, tol, what, names=("o", "state_out", "mean_out")):
    errs = {n: rel_err(g, r) for n, g, r in zip(names, got, ref)}
    say(f"{what}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, g in zip(names, got):
        assert np.all(np.isfinite(g)), f"{what}: non-finite {n}"
    for n, e in errs.items():
        assert e <= tol, f"{what}: {n} rel err {e:.3e} > {tol}"


FWD_CASES = [
    # name, dtype, B, H, T, d, L, rank
    # no content projection in bf16: the chunk-parallel pair (intra + state kernels)
    ("par-d64-ragged-1000", "bf16", 2, 3, 1000, 64, 64, 0),
    ("par-d128-ragged-200-L128", "bf16", 1, 2, 200, 128, 128, 0),
    # the chunk-serial kernel at its block lengths 64, 32 and 16
    ("ser-f32-d64-L64-r8", "f32", 1, 2, 256, 64, 64, 8),
    ("ser-bf16-d64-L32-r16-ragged-300", "bf16", 2, 2, 300, 64, 32, 16),
    ("ser-f32-d128-L16-r4-ragged-150", "f32", 1, 2, 150, 128, 16, 4),
    ("ser-bf16-d128-L64-r8", "bf16", 1, 2, 256, 128, 64, 8),
    # the chunk-serial kernel's lean 64-token blocks (bf16, d = 64), ragged tail
    ("lean-bf16-d64-L64-r16-ragged-200", "bf16", 2, 2, 200, 64, 64, 16),
]


@pytest.mark.parametrize("name,dtype,B,H,T,d,L,rank", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_with_decay_logits(torch_cuda, name, dtype, B, H, T, d, L, rank):
    wl = workload(name, dtype, B, H, T, d, L, rank, 5000 + T)
    say("case", wl)
    inp = make_inputs(wl, decay_logits=True)
    S_in, m_in = start_state(B, H, d, T)
    assert_parity(fwd_gpu(torch_cuda, inp, dtype, L, S_in, m_in), fwd_oracle(inp, dtype, L, S_in, m_in),
                  TOL[dtype], name)


@pytest.mark.parametrize("dtype,rank", [("bf16", 0), ("f32", 8)], ids=["parallel-bf16", "serial-f32"])
def test_steep_logits_take_the_pairwise_path(torch_cuda, dtype, rank):
    """Half the key channels get logit +10 (a decay of about e^-10 per token, too
    steep for the factorised Grams, so the pairwise rebuild runs and forms
    -softplus itself); the other half get -4 (a long memory)."""
    wl = workload(f"steep-{dtype}", dtype, 1, 3, 320, 64, 64, rank, 5100)
    inp = make_inputs(wl, decay_logits=True)
    a = np.empty(inp["g"].shape, np.float32)
    a[..., :32] = 10.0
    a[..., 32:] = -4.0
    inp["g"] = a if dtype == "f32" else bf16_bits_from_f32(a)
    say("case steep logits", wl)
    S_in, m_in = start_state(1, 3, 64, 5)
    assert_parity(fwd_gpu(torch_cuda, inp, dtype, 64, S_in, m_in), fwd_oracle(inp, dtype, 64, S_in, m_in),
                  TOL[dtype], f"steep logits ({dtype})")


def test_hard_decay_logits_are_memoryless(torch_cuda):
    """Logits of 1e4: g = -1e4, so every token wipes the state; the result
    must stay finite and match the oracle."""
    wl = workload("hard", "f32", 1, 2, 128, 64, 64, 8, 5200)
    inp = make_inputs(wl, decay_logits=True)
    inp["g"] = np.full_like(inp["g"], 1e4)
    S_in, m_in = start_state(1, 2, 64, 6)
    assert_parity(fwd_gpu(torch_cuda, inp, "f32", 64, S_in, m_in), fwd_oracle(inp, "f32", 64, S_in, m_in),
                  TOL["f32"], "hard decay logits")


@pytest.mark.parametrize("rank", [0, 8])
def test_logits_agree_with_materialised_decay(torch_cuda, rank):
    """fp32: the fused activation equals handing the kernels g = -softplus(a)
    computed by torch, to fp32 rounding (both runs use the same schedule)."""
    torch = torch_cuda
    wl = workload(f"agree-{rank}", "f32", 2, 2, 300, 64, 64, rank, 5300 + rank)
    inp = make_inputs(wl, decay_logits=True)
    S_in, m_in = start_state(2, 2, 64, 8)
    fused = fwd_gpu(torch, inp, "f32", 64, S_in, m_in)
    g = -torch.nn.functional.softplus(to_torch(inp["g"], "f32"))
    plain = fwd_gpu(torch, inp, "f32", 64, S_in, m_in, logits=False, g_override=g.contiguous())
    errs = [rel_err(x, y) for x, y in zip(fused, plain)]
    say(f"fused vs materialised decay, rank {rank}: " + ", ".join(f"{e:.2e}" for e in errs))
    assert max(errs) <= 1e-5


# ------------------------------------------------------------------ decode step

def step_gpu(torch, inp, dtype, L, S_in, m_in, T):
    from chunk_gated_delta_carve_amd.api import recurrent_step
    t = {k: to_torch(v, dtype) for k, v in inp.items()}
    S = torch.from_numpy(S_in.copy()).cuda()
    m = torch.from_numpy(m_in.copy()).cuda()
    acc = torch.zeros_like(m)
    outs = []
    for s in range(T):
        tok = {k: t[k][:, s].clone() for k in KEYS}
        outs.append(recurrent_step(*(tok[k] for k in KEYS), S, m, acc, s % L, L, t.get("U_down"), t.get("U_up"),
                                   decay_logits=True).float())
    torch.cuda.synchronize()
    return torch.stack(outs, dim=1).cpu().numpy(), S.cpu().numpy(), m.cpu().numpy(), acc.cpu().numpy()


STEP_CASES = [
    ("f32-d64-L16-r8", "f32", 2, 3, 40, 64, 16, 8),
    ("bf16-d128-L64-r16", "bf16", 1, 2, 70, 128, 64, 16),
    ("bf16-d64-L32-r0", "bf16", 2, 2, 45, 64, 32, 0),
]


@pytest.mark.parametrize("name,dtype,B,H,T,d,L,rank", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_step_with_decay_logits(torch_cuda, name, dtype, B, H, T, d, L, rank):
    wl = workload(name, dtype, B, H, T, d, L, rank, 5400 + T)
    say("case step", wl)
    inp = make_inputs(wl, decay_logits=True)
    S_in, m_in = start_state(B, H, d, T)
    got = step_gpu(torch_cuda, inp, dtype, L, S_in, m_in, T)
    f = lambda key: to_f64(inp[key], dtype)
    q, k, v, a, bx, w = (f(n) for n in KEYS)
    g = decay_from_logits(a)
    Ud = f("U_down") if rank else None
    Uu = f("U_up") if rank else None
    S, m, acc = S_in.astype(np.float64), m_in.astype(np.float64), np.zeros((B, H, d))
    outs = []
    for s in range(T):
        o, S, m, acc = carve_step(S, m, acc, s % L, q[:, s], k[:, s], v[:, s], g[:, s], bx[:, s], w[:, s], L, Ud, Uu)
        outs.append(o)
    assert_parity(got, (np.stack(outs, axis=1), S, m, acc), TOL[dtype], f"step {name}",
                  names=("o", "state", "mean_prev", "chunk_acc"))


def test_steps_agree_with_forward_under_logits(torch_cuda):
    """Stepping a sequence with raw logits reproduces carve_chunk_fwd with raw
    logits on the same GPU: outputs, final state and the last chunk's mean."""
    torch = torch_cuda
    B, H, T, d, L = 2, 3, 150, 64, 64
    wl = workload("agree-steps", "bf16", B, H, T, d, L, 16, 5500)
    inp = make_inputs(wl, decay_logits=True)
    S_in, m_in = start_state(B, H, d, 9)
    o_f, S_f, m_f = fwd_gpu(torch, inp, "bf16", L, S_in, m_in)
    o_s, S_s, _, acc_s = step_gpu(torch, inp, "bf16", L, S_in, m_in, T)
    e = (rel_err(o_s, o_f), rel_err(S_s, S_f), rel_err(acc_s / (T % L), m_f))
    say("steps vs forward under logits: " + ", ".join(f"{x:.2e}" for x in e))
    assert max(e) <= TOL["bf16"]
