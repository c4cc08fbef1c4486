"""Parity of the HIP decode step (carve_recurrent_step) against the float64
oracle's step, through the C ABI, and agreement with the GPU forward pass.

Error metric (per tensor): max |x - ref| / max |ref|, with the bars of the
forward pass (1e-4 for fp32 inputs, 2e-2 for bf16 inputs). The step computes
in fp32 throughout, so its errors sit far below both bars.
"""
import numpy as np
import pytest

from chunk_gated_delta_carve_amd.workloads import WORKLOADS, make_inputs, to_f64, to_torch
from oracle import carve_step

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


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
    S = (0.3 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    m = (0.3 * rng.standard_normal((B, H, d))).astype(np.float32)
    return S, m


def step_gpu(torch, inp, dtype, L, S_in, m_in, T):
    """Step t = 0 .. T-1 on the GPU; returns (o [B,T,H,d], S, mean_prev, chunk_acc)."""
    from chunk_gated_delta_carve_amd.api import recurrent_step
    t = {k: to_torch(v, dtype) for k, v in inp.items()}
    S = torch.from_numpy(S_in.copy()).cuda()
    m = torch.from_numpy(m_in.copy()).cuda()
    acc = torch.zeros_like(m)
    ud, uu = t.get("U_down"), t.get("U_up")
    outs = []
    for s in range(T):
        tok = {k: t[k][:, s].clone() for k in ("q", "k", "v", "g", "bx", "w")}   # fresh, aligned copies
        outs.append(recurrent_step(tok["q"], tok["k"], tok["v"], tok["g"], tok["bx"], tok["w"], S, m, acc,
                                   s % L, L, ud, uu).float())
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=1).cpu().numpy()
    return o, S.cpu().numpy(), m.cpu().numpy(), acc.cpu().numpy()


def step_oracle(inp, dtype, L, S_in, m_in, T):
    f = lambda key: to_f64(inp[key], dtype)
    q, k, v, g, bx, w = (f(n) for n in ("q", "k", "v", "g", "bx", "w"))
    Ud = f("U_down") if "U_down" in inp else None
    Uu = f("U_up") if "U_up" in inp else None
    S, m = S_in.astype(np.float64), m_in.astype(np.float64)
    acc = np.zeros_like(m)
    outs = []
    for s in range(T):
        o, S, m, acc = carve_step(S, m, acc, s % L, q[:, s], k[:, s], v[:, s], g[:, s], bx[:, s], w[:, s],
                                  L, Ud, Uu)
        outs.append(o)
    return np.stack(outs, axis=1), S, m, acc


STEP_CASES = [
    # name, dtype, B, H, T, d, L, rank: T crosses chunk ends and stops inside a chunk
    ("f32-d64-L16-r8", "f32", 2, 3, 40, 64, 16, 8),
    ("f32-d128-L32-r4", "f32", 1, 2, 37, 128, 32, 4),
    ("bf16-d64-L64-r0", "bf16", 2, 2, 70, 64, 64, 0),
    ("bf16-d128-L64-r16", "bf16", 1, 2, 70, 128, 64, 16),
    ("bf16-d64-L128-r64", "bf16", 1, 1, 130, 64, 128, 64),
]


@pytest.mark.parametrize("name,dtype,B,H,T,d,L,rank", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_step_matches_oracle(torch_cuda, name, dtype, B, H, T, d, L, rank):
    wl = workload(name, dtype, B, H, T, d, L, rank, 3000 + T)
    say("case", wl)
    inp = make_inputs(wl)
    S_in, m_in = start_state(B, H, d, T)
    got = step_gpu(torch_cuda, inp, dtype, L, S_in, m_in, T)
    ref = step_oracle(inp, dtype, L, S_in, m_in, T)
    errs = {n: rel_err(x, r) for n, x, r in zip(("o", "state", "mean_prev", "chunk_acc"), got, ref)}
    say(f"{name}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, x in zip(("o", "state", "mean_prev", "chunk_acc"), got):
        assert np.all(np.isfinite(x)), f"{name}: non-finite {n}"
    for n, e in errs.items():
        assert e <= TOL[dtype], f"{name}: {n} rel err {e:.3e} > {TOL[dtype]}"


@pytest.mark.parametrize("rank", [0, 16])
def test_steps_agree_with_gpu_forward(torch_cuda, rank):
    """Stepping a sequence reproduces carve_chunk_fwd on the same GPU (the
    chunk-parallel schedule without a projection, the chunk-serial one with it):
    outputs, final state and the last chunk's mean."""
    from chunk_gated_delta_carve_amd import chunk_fwd
    torch = torch_cuda
    B, H, T, d, L = 2, 3, 150, 64, 64
    wl = workload(f"agree-r{rank}", "bf16", B, H, T, d, L, rank, 4000 + rank)
    inp = make_inputs(wl)
    S_in, m_in = start_state(B, H, d, 7)
    t = {k: to_torch(v, "bf16") for k, v in inp.items()}
    o_f, S_f, m_f = chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["bx"], t["w"], L=L,
                              ub_down=t.get("U_down"), ub_up=t.get("U_up"),
                              state_in=torch.from_numpy(S_in).cuda(), mean_in=torch.from_numpy(m_in).cuda(),
                              return_state=True)
    o_s, S_s, m_s, acc_s = step_gpu(torch, inp, "bf16", L, S_in, m_in, T)
    tail = T % L
    e_o = rel_err(o_s, o_f.float().cpu().numpy())
    e_S = rel_err(S_s, S_f.cpu().numpy())
    e_m = rel_err(acc_s / tail, m_f.cpu().numpy())
    say(f"steps vs forward, rank {rank}: o {e_o:.2e}, state {e_S:.2e}, last mean {e_m:.2e}")
    assert max(e_o, e_S, e_m) <= TOL["bf16"]


def test_step_chunk_end_many_heads(torch_cuda):
    """One step at a chunk's last position for 96 (batch, head) pairs: the mean
    is replaced and the running sum restarts from zero."""
    torch = torch_cuda
    from chunk_gated_delta_carve_amd.api import recurrent_step
    B, H, d, L = 8, 12, 64, 64
    wl = workload("chunk-end", "bf16", B, H, 1, d, L, 16, 4100)
    inp = make_inputs(wl)
    S_in, m_in = start_state(B, H, d, 11)
    acc_in = (np.random.default_rng(12).standard_normal((B, H, d)) * 2).astype(np.float32)
    t = {k: to_torch(v, "bf16") for k, v in inp.items()}
    S, m, acc = (torch.from_numpy(x.copy()).cuda() for x in (S_in, m_in, acc_in))
    o = recurrent_step(*(t[k][:, 0].clone() for k in ("q", "k", "v", "g", "bx", "w")), S, m, acc,
                       L - 1, L, t["U_down"], t["U_up"])
    torch.cuda.synchronize()
    f = lambda key: to_f64(inp[key], "bf16")
    o_r, S_r, m_r, acc_r = carve_step(S_in.astype(np.float64), m_in.astype(np.float64), acc_in.astype(np.float64),
                                      L - 1, *(f(k)[:, 0] for k in ("q", "k", "v", "g", "bx", "w")), L,
                                      f("U_down"), f("U_up"))
    assert not acc.cpu().numpy().any() and not acc_r.any()
    for n, x, r in (("o", o.float().cpu().numpy(), o_r), ("state", S.cpu().numpy(), S_r), ("mean", m.cpu().numpy(), m_r)):
        e = rel_err(x, r)
        say(f"chunk end {n}: {e:.2e}")
        assert e <= TOL["bf16"]


def test_step_graph_replays_match_eager(torch_cuda):
    """A chunk of steps captured in a HIP graph and replayed (with eager work
    on the stream between replays) gives bit for bit what the same steps give
    launched one at a time."""
    torch = torch_cuda
    from chunk_gated_delta_carve_amd.api import recurrent_step
    B, H, d, L = 3, 4, 64, 16
    wl = workload("graph", "bf16", B, H, L, d, L, 8, 4200)
    inp = make_inputs(wl)
    t = {k: to_torch(v, "bf16") for k, v in inp.items()}
    toks = [{k: t[k][:, s].clone() for k in ("q", "k", "v", "g", "bx", "w")} for s in range(L)]
    S_in, m_in = start_state(B, H, d, 13)

    def fresh():
        S = torch.from_numpy(S_in.copy()).cuda()
        m = torch.from_numpy(m_in.copy()).cuda()
        return S, m, torch.zeros_like(m), torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")

    def chunk(S, m, acc, o, outs=None):
        for s in range(L):
            x = toks[s]
            recurrent_step(x["q"], x["k"], x["v"], x["g"], x["bx"], x["w"], S, m, acc, s, L,
                           t["U_down"], t["U_up"], out=o)
            if outs is not None:
                outs.append(o.clone())

    S_e, m_e, acc_e, o_e = fresh()
    eager = []
    for _ in range(3):
        outs = []
        chunk(S_e, m_e, acc_e, o_e, outs)
        eager.append((S_e.clone(), m_e.clone(), outs[-1]))
    S_g, m_g, acc_g, o_g = fresh()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            chunk(S_g, m_g, acc_g, o_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture does not run the work: start the replays from the initial state
    S_g.copy_(torch.from_numpy(S_in)); m_g.copy_(torch.from_numpy(m_in)); acc_g.zero_()
    for i in range(3):
        graph.replay()
        scratch = torch.ones(1 << 20, device="cuda").sum()      # eager work between replays
        torch.cuda.synchronize()
        S_ref, m_ref, o_ref = eager[i]
        assert torch.equal(S_g, S_ref), f"replay {i}: state"
        assert torch.equal(m_g, m_ref), f"replay {i}: mean"
        assert torch.equal(o_g, o_ref), f"replay {i}: output"
        assert float(scratch) == float(1 << 20)
