"""Parity of the HIP forward pass against the float64 oracle, through the C ABI.

Error metric (per tensor): max |x - ref| / max |ref|. Bars: 1e-4 for fp32
inputs, 2e-2 for bf16 inputs with fp32 accumulation. (Batch, head) pairs are
independent, so for the large workloads the oracle runs on a sample of pairs
over the full sequence length and those pairs are compared exactly.
"""
import numpy as np
import pytest

from chunk_gated_delta_carve_amd.workloads import (WORKLOADS, LSWEEP_CHUNKS, bf16_bits_from_f32, make_inputs, to_f64,
                                                   to_torch)
from oracle import carve_forward

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


def run_gpu(torch, inp, dtype, L, use_ub=True, state_in=None, mean_in=None, zero_ub=False):
    from chunk_gated_delta_carve_amd import chunk_fwd
    t = {k: to_torch(v, dtype) for k, v in inp.items()}
    ud = t.get("U_down") if use_ub else None
    uu = t.get("U_up") if use_ub else None
    if zero_ub:
        ud, uu = torch.zeros_like(ud), torch.zeros_like(uu)
    si = None if state_in is None else torch.from_numpy(np.ascontiguousarray(state_in, np.float32)).cuda()
    mi = None if mean_in is None else torch.from_numpy(np.ascontiguousarray(mean_in, np.float32)).cuda()
    o, S, m = chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["bx"], t["w"], L=L, ub_down=ud, ub_up=uu,
                        state_in=si, mean_in=mi, return_state=True)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), S.cpu().numpy(), m.cpu().numpy()


def run_oracle(inp, dtype, L, pairs=None, use_ub=True, state_in=None, mean_in=None):
    """Oracle on all pairs, or on the listed (b, h) pairs stacked along the head axis."""
    f = lambda key: to_f64(inp[key], dtype)
    ub = use_ub and "U_down" in inp
    if pairs is None:
        return carve_forward(f("q"), f("k"), f("v"), f("g"), f("bx"), f("w"), L,
                             f("U_down") if ub else None, f("U_up") if ub else None,
                             state_in=state_in, mean_in=mean_in)
    hs = [h for _, h in pairs]
    sel = {}
    for key in ("q", "k", "v", "g", "bx"):
        sel[key] = to_f64(np.stack([inp[key][b, :, h] for b, h in pairs], axis=1)[None], dtype)
    sel["w"] = to_f64(np.stack([inp["w"][b, :, h] for b, h in pairs], axis=1)[None], dtype)
    Ud = to_f64(inp["U_down"][hs], dtype) if ub else None
    Uu = to_f64(inp["U_up"][hs], dtype) if ub else None
    return carve_forward(sel["q"], sel["k"], sel["v"], sel["g"], sel["bx"], sel["w"], L, Ud, Uu)


def gather(o, S, m, pairs):
    return (np.stack([o[b, :, h] for b, h in pairs], axis=1)[None],
            np.stack([S[b, h] for b, h in pairs])[None],
            np.stack([m[b, h] for b, h in pairs])[None])


def assert_parity(got, ref, tol, what):
    names = ("o", "state_out", "mean_out")
    errs = {n: rel_err(g, r) for n, g, r in zip(names, got, ref)}
    say(f"{what}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, g in zip(names, got):
        assert np.all(np.isfinite(g)), f"{what}: non-finite {n}"
    for n, e in errs.items():
        assert e <= tol, f"{what}: {n} rel err {e:.3e} > {tol}"


# ------------------------------------------------------------------ the workloads

def test_tiny_f32(torch_cuda):
    wl = WORKLOADS["tiny"]
    say("case tiny", wl)
    inp = make_inputs(wl)
    assert_parity(run_gpu(torch_cuda, inp, wl.dtype, wl.L), run_oracle(inp, wl.dtype, wl.L), TOL["f32"], "tiny")


def test_content_path_is_exercised_f32(torch_cuda):
    """U_b moves the output far beyond the tolerance, and the GPU still matches."""
    wl = WORKLOADS["content_test"]
    say("case content_test", wl)
    inp = make_inputs(wl)
    ref = run_oracle(inp, wl.dtype, wl.L)
    ref0 = run_oracle(inp, wl.dtype, wl.L, use_ub=False)
    effect = rel_err(ref0[0], ref[0])
    say(f"content effect on o: {effect:.2e}")
    assert effect >= 30 * TOL["f32"]
    assert_parity(run_gpu(torch_cuda, inp, wl.dtype, wl.L), ref, TOL["f32"], "content_test")


def test_init_equiv_bf16_full(torch_cuda):
    wl = WORKLOADS["init_equiv"]
    say("case init_equiv", wl)
    inp = make_inputs(wl)
    got = run_gpu(torch_cuda, inp, wl.dtype, wl.L)
    assert_parity(got, run_oracle(inp, wl.dtype, wl.L), TOL["bf16"], "init_equiv")


def test_zero_projection_is_bitwise_absent_projection(torch_cuda):
    """A zero-filled content projection leaves the layer exactly the
    memory-blind rule: with fp32 inputs both calls run the same kernel, and
    the content bias it adds is exactly zero."""
    wl = WORKLOADS["init_equiv"].with_(B=2, T=512, rank=16, ub_std=0.05, dtype="f32")
    say("case zero U_b vs absent U_b (f32)", wl)
    inp = make_inputs(wl)
    a = run_gpu(torch_cuda, inp, wl.dtype, wl.L, use_ub=False)
    b = run_gpu(torch_cuda, inp, wl.dtype, wl.L, zero_ub=True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("T", [2048, 2000])
def test_zero_projection_is_bitwise_parallel_schedule(torch_cuda, T):
    """bf16 at the B4 H12 d64 L64 shape: a zero-filled rank-16 projection runs
    the chunk-serial kernel, an absent one the chunk-parallel pair. The serial
    kernel's 64-token blocks form the affine maps from the solve's registers
    with the pair's products, apply them in the pair's order and sum the final
    mean in the state pass's order, and a zero projection adds a content bias
    of exactly zero, so o, the final state and the final mean are equal bit
    for bit (the layer at initialisation is the memory-blind rule exactly;
    shd-paper.top English abstract, and gist.science technical summary §2.1).
    T = 2000 ends in a ragged block."""
    wl = WORKLOADS["init_equiv"].with_(T=T, rank=16, ub_std=0.05)
    say("case zero U_b (serial) vs absent U_b (parallel)", wl)
    inp = make_inputs(wl)
    a = run_gpu(torch_cuda, inp, wl.dtype, wl.L, use_ub=False)
    b = run_gpu(torch_cuda, inp, wl.dtype, wl.L, zero_ub=True)
    for name, x, y in zip(("o", "state", "mean"), a, b):
        say(name, "differing elements:", int(np.count_nonzero(x != y)))
        assert np.array_equal(x, y), name


def test_content_bf16_sampled(torch_cuda):
    wl = WORKLOADS["content"]
    say("case content", wl)
    inp = make_inputs(wl)
    got = run_gpu(torch_cuda, inp, wl.dtype, wl.L)
    pairs = [(0, 0), (3, 5), (7, 11)]
    assert_parity(gather(*got, pairs), run_oracle(inp, wl.dtype, wl.L, pairs), TOL["bf16"], "content")


@pytest.mark.parametrize("L", LSWEEP_CHUNKS)
def test_lsweep_bf16_sampled(torch_cuda, L):
    wl = WORKLOADS["lsweep"]
    say("case lsweep L =", L, wl)
    inp = make_inputs(wl)
    got = run_gpu(torch_cuda, inp, wl.dtype, L)
    pairs = [(0, 3), (3, 14)]
    assert_parity(gather(*got, pairs), run_oracle(inp, wl.dtype, L, pairs), TOL["bf16"], f"lsweep L={L}")


def test_long_bf16_sampled(torch_cuda):
    wl = WORKLOADS["long"]
    say("case long", wl)
    inp = make_inputs(wl)
    got = run_gpu(torch_cuda, inp, wl.dtype, wl.L)
    pairs = [(0, 0), (0, 9)]
    assert_parity(gather(*got, pairs), run_oracle(inp, wl.dtype, wl.L, pairs), TOL["bf16"], "long")


# ------------------------------------------------------------------ edge cases

EDGE = [
    # name, dtype, B, H, T, d, L, rank
    ("ragged-1", "f32", 1, 2, 1, 64, 64, 4),
    ("ragged-15", "bf16", 2, 2, 15, 64, 16, 4),
    ("ragged-100", "f32", 1, 3, 100, 64, 32, 8),
    ("ragged-129", "bf16", 1, 2, 129, 128, 128, 8),
    ("ragged-200-L16", "f32", 1, 2, 200, 64, 16, 8),
    ("f32-d128-L64", "f32", 1, 2, 256, 128, 64, 8),
    ("f32-d128-L128", "f32", 1, 2, 384, 128, 128, 8),
    ("bf16-d64-L32", "bf16", 2, 2, 320, 64, 32, 8),
    ("bf16-d128-L16", "bf16", 1, 2, 160, 128, 16, 8),
    # the lean 64-token blocks of the chunk-serial kernel, ending in a ragged block
    ("lean-ragged-200", "bf16", 2, 2, 200, 64, 64, 8),
    ("no-ub-L16", "f32", 1, 2, 192, 64, 16, 0),
    # no content projection in bf16: the chunk-parallel schedule
    ("par-T1", "bf16", 1, 2, 1, 64, 32, 0),
    ("par-T64", "bf16", 1, 1, 64, 64, 64, 0),
    ("par-ragged-100-L16", "bf16", 1, 3, 100, 64, 16, 0),
    ("par-d128-ragged-200-L128", "bf16", 2, 2, 200, 128, 128, 0),
    ("par-d128-L64", "bf16", 1, 3, 512, 128, 64, 0),
    # 13 blocks: the state pass's prefetch loops end in partial rounds
    ("par-nblk13", "bf16", 2, 3, 832, 64, 64, 0),
    # 15 (batch, head) pairs: the state pass's placement groups of eight end part-full
    ("par-BH15", "bf16", 3, 5, 256, 64, 64, 0),
]


@pytest.mark.parametrize("name,dtype,B,H,T,d,L,rank", EDGE, ids=[e[0] for e in EDGE])
def test_edge_shapes(torch_cuda, name, dtype, B, H, T, d, L, rank):
    wl = WORKLOADS["tiny"].with_(name=name, dtype=dtype, B=B, H=H, T=T, dk=d, dv=d, L=L, rank=rank,
                                 ub_std=0.5, seed=2000 + T)
    say("case", wl)
    inp = make_inputs(wl)
    rng = np.random.default_rng(7)
    S_in = 0.3 * rng.standard_normal((B, H, d, d))
    m_in = 0.3 * rng.standard_normal((B, H, d))
    S_in32, m_in32 = S_in.astype(np.float32), m_in.astype(np.float32)
    got = run_gpu(torch_cuda, inp, dtype, L, state_in=S_in32, mean_in=m_in32)
    ref = run_oracle(inp, dtype, L, state_in=S_in32.astype(np.float64), mean_in=m_in32.astype(np.float64))
    assert_parity(got, ref, TOL[dtype], name)


def test_empty_sequence_passes_state(torch_cuda):
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_fwd
    B, H, d = 2, 3, 64
    z = lambda *s: torch.zeros(*s, device="cuda", dtype=torch.bfloat16)
    S_in = torch.randn(B, H, d, d, device="cuda")
    m_in = torch.randn(B, H, d, device="cuda")
    o, S, m = chunk_fwd(z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d),
                        z(B, 0, H), L=64, state_in=S_in, mean_in=m_in, return_state=True)
    torch.cuda.synchronize()
    assert o.shape == (B, 0, H, d)
    assert torch.equal(S, S_in) and torch.equal(m, m_in)


def test_chaining_on_gpu(torch_cuda):
    """Two calls with state and mean carried equal one call."""
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_fwd
    wl = WORKLOADS["content_test"].with_(T=512)
    say("case chaining", wl)
    inp = make_inputs(wl)
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    args = lambda sl: [t[k][:, sl].contiguous() for k in ("q", "k", "v", "g", "bx", "w")]
    o, S, m = chunk_fwd(*args(slice(None)), L=64, ub_down=t["U_down"], ub_up=t["U_up"], return_state=True)
    oa, Sa, ma = chunk_fwd(*args(slice(0, 256)), L=64, ub_down=t["U_down"], ub_up=t["U_up"], return_state=True)
    ob, Sb, mb = chunk_fwd(*args(slice(256, 512)), L=64, ub_down=t["U_down"], ub_up=t["U_up"],
                           state_in=Sa, mean_in=ma, return_state=True)
    torch.cuda.synchronize()
    assert rel_err(torch.cat([oa, ob], 1).cpu().numpy(), o.cpu().numpy()) < 1e-5
    assert rel_err(Sb.cpu().numpy(), S.cpu().numpy()) < 1e-5
    assert rel_err(mb.cpu().numpy(), m.cpu().numpy()) < 1e-5


def test_state_out_may_alias_state_in(torch_cuda):
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import _lib
    from chunk_gated_delta_carve_amd.api import make_config
    import ctypes
    wl = WORKLOADS["tiny"].with_(T=128)
    inp = make_inputs(wl)
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    S = 0.1 * torch.randn(1, 2, 64, 64, device="cuda")
    S0 = S.clone()
    o = torch.empty(1, 128, 2, 64, device="cuda")
    cfg = make_config(1, 2, 128, 64, 64, 64, 8, torch.float32)
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    code = _lib.lib().carve_chunk_fwd(ctypes.byref(cfg), p(t["q"]), p(t["k"]), p(t["v"]), p(t["g"]), p(t["bx"]),
                                      p(t["w"]), p(t["U_down"]), p(t["U_up"]), p(S), None, p(o), p(S), None,
                                      None, ctypes.c_size_t(0), None)
    torch.cuda.synchronize()
    assert code == 0
    ref = run_oracle(inp, wl.dtype, 64, state_in=S0.cpu().double().numpy())
    assert rel_err(o.cpu().numpy(), ref[0]) < TOL["f32"]
    assert rel_err(S.cpu().numpy(), ref[1]) < TOL["f32"]


def test_hard_decay_memoryless_and_finite(torch_cuda):
    """g = -1e4 wipes the state every token; the kernel must stay finite (the
    factorised exponents would overflow, so this exercises the pairwise path)."""
    wl = WORKLOADS["tiny"].with_(T=128, seed=3001)
    inp = make_inputs(wl)
    inp["g"] = np.full_like(inp["g"], -1e4)
    got = run_gpu(torch_cuda, inp, wl.dtype, wl.L)
    ref = run_oracle(inp, wl.dtype, wl.L)
    assert_parity(got, ref, TOL["f32"], "hard decay")


def test_steep_decay_chunk_parallel(torch_cuda):
    """bf16 without a projection (the chunk-parallel pair): half the key
    channels decay by e^-10 per token, so a 16-token sub-block spans far more
    than the factorised Grams allow and the pairwise rebuild runs; the other
    half keep a long memory, so the result is far from trivial."""
    wl = WORKLOADS["init_equiv"].with_(B=1, H=3, T=320, seed=3003)
    inp = make_inputs(wl)
    g = np.empty(inp["g"].shape, np.float32)
    g[..., : wl.dk // 2] = -10.0
    g[..., wl.dk // 2:] = -0.02
    inp["g"] = bf16_bits_from_f32(g)
    say("case steep decay, chunk-parallel", wl)
    got = run_gpu(torch_cuda, inp, wl.dtype, wl.L)
    ref = run_oracle(inp, wl.dtype, wl.L)
    assert_parity(got, ref, TOL["bf16"], "steep decay (parallel)")


def test_deterministic_chunk_parallel(torch_cuda):
    wl = WORKLOADS["init_equiv"].with_(B=2, T=1024)
    inp = make_inputs(wl)
    a = run_gpu(torch_cuda, inp, wl.dtype, wl.L)
    b = run_gpu(torch_cuda, inp, wl.dtype, wl.L)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_delta_rule_special_case(torch_cuda):
    """b = 1, g = 0, w = 1: the plain delta rule; a query equal to the previous
    key reads back the previous value."""
    wl = WORKLOADS["tiny"].with_(T=64, rank=0, seed=3002)
    inp = make_inputs(wl)
    inp["g"] = np.zeros_like(inp["g"])
    inp["bx"] = np.full_like(inp["bx"], 40.0)
    inp["w"] = np.ones_like(inp["w"])
    inp["q"][:, 1:] = inp["k"][:, :-1]
    o, _, _ = run_gpu(torch_cuda, inp, wl.dtype, wl.L)
    assert rel_err(o[:, 1:], inp["v"][:, :-1].astype(np.float64)) < 1e-4


def test_deterministic(torch_cuda):
    """Repeated chunk-serial calls agree bit for bit in o, the state and the
    mean (48 heads, four calls: a race between two writers of the final mean
    once showed here as last-bit differences in a few heads per call)."""
    wl = WORKLOADS["content"].with_(B=4, T=2048)
    inp = make_inputs(wl)
    a = run_gpu(torch_cuda, inp, wl.dtype, wl.L)
    for _ in range(3):
        b = run_gpu(torch_cuda, inp, wl.dtype, wl.L)
        for name, x, y in zip(("o", "state", "mean"), a, b):
            assert np.array_equal(x, y), name


@pytest.mark.parametrize("rank", [0, 8], ids=["chunk-parallel", "chunk-serial"])
def test_forward_graph_replays_match_eager(torch_cuda, rank):
    """carve_chunk_fwd captured in a HIP graph (output, state buffers and
    workspace allocated before the capture) and replayed, with eager work on
    the stream between replays, gives bit for bit the eager call's results."""
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_fwd, recurrent_ref_shapes
    wl = WORKLOADS["init_equiv"].with_(B=2, H=3, T=320, rank=rank, ub_std=0.05, seed=3100 + rank)
    inp = make_inputs(wl)
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    ub = dict(ub_down=t["U_down"], ub_up=t["U_up"]) if rank else {}
    ws = torch.empty(max(16, int(recurrent_ref_shapes(2, 3, 320, 64, 64, 64, rank, torch.bfloat16).workspace_bytes)),
                     dtype=torch.uint8, device="cuda")
    args = [t[k] for k in ("q", "k", "v", "g", "bx", "w")]
    ref = [x.clone() for x in chunk_fwd(*args, L=64, return_state=True, workspace=ws, **ub)]
    o = torch.empty_like(ref[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            chunk_fwd(*args, L=64, out=o, workspace=ws, stream=side.cuda_stream, **ub)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(3):
        o.fill_(7.0)                                       # the replay must rewrite the output
        graph.replay()
        scratch = torch.ones(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]), f"replay {i}"
        assert float(scratch) == float(1 << 20)


def test_steep_blocks_between_lean_blocks(torch_cuda):
    """bf16 with a projection at d = 64, L = 64 (the chunk-serial kernel's
    lean blocks): in blocks 1 and 3 half the key channels decay by e^-10 per
    token, too steep for the factorised Grams, so those blocks take the
    general stages with the pairwise rebuild while blocks 0, 2 and 4 stay
    lean; the state, the content bias and the chunk means pass between the
    two kinds of block."""
    wl = WORKLOADS["init_equiv"].with_(B=1, H=3, T=320, rank=16, ub_std=0.5, seed=3005)
    inp = make_inputs(wl)
    g = np.full(inp["g"].shape, -0.02, np.float32)
    for blk in (1, 3):
        g[:, 64 * blk: 64 * (blk + 1), :, : wl.dk // 2] = -10.0
    inp["g"] = bf16_bits_from_f32(g)
    say("case steep blocks between lean blocks", wl)
    rng = np.random.default_rng(11)
    m_in = (0.3 * rng.standard_normal((wl.B, wl.H, wl.dv))).astype(np.float32)
    got = run_gpu(torch_cuda, inp, wl.dtype, wl.L, mean_in=m_in)
    ref = run_oracle(inp, wl.dtype, wl.L, mean_in=m_in.astype(np.float64))
    assert_parity(got, ref, TOL["bf16"], "steep blocks between lean blocks")
