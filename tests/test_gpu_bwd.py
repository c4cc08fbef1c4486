"""Parity of the HIP backward pass (carve_chunk_bwd) against the float64
oracle's adjoint (carve_backward, itself pinned by finite differences of the
forward pass), through the C ABI.

Error metric (per gradient tensor): max |x - ref| / max |ref|, with the bars
of the forward pass (1e-4 for fp32 inputs, 2e-2 for bf16 inputs). The
kernels compute in fp32 throughout; bf16 gradients are rounded once on store.
"""
import numpy as np
import pytest

from chunk_gated_delta_carve_amd.workloads import WORKLOADS, make_inputs, to_f64, to_torch
from oracle import carve_backward, decay_from_logits, sigmoid

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
KEYS = ("q", "k", "v", "g", "bx", "w")
NAMES = {"dq": "dq", "dk": "dk", "dv": "dv", "dg": "dg", "dbx": "dbx", "dw": "dw", "dub_down": "dU_down",
         "dub_up": "dU_up", "d_state_in": "dstate_in", "d_mean_in": "dmean_in"}


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


def cotangents(B, H, T, d, dtype, seed, with_state=True):
    """Seeded output gradients: d_o in the input dtype, d_state_out and
    d_mean_out in fp32 (None without state), and the initial state and mean."""
    from chunk_gated_delta_carve_amd.workloads import bf16_bits_from_f32
    rng = np.random.default_rng(seed)
    do = rng.standard_normal((B, T, H, d)).astype(np.float32)
    do = do if dtype == "f32" else bf16_bits_from_f32(do)
    if not with_state:
        return do, None, None, None, None
    f = lambda *s: (0.3 * rng.standard_normal(s)).astype(np.float32)
    return do, f(B, H, d, d), f(B, H, d), f(B, H, d, d), f(B, H, d)


def bwd_gpu(torch, inp, dtype, L, do, dSo, dmo, S_in, m_in, logits=False, alias=False, detach=False):
    from chunk_gated_delta_carve_amd import chunk_bwd
    t = {k: to_torch(v, dtype) for k, v in inp.items()}
    cu = lambda x: None if x is None else torch.from_numpy(x).cuda()
    dSo_t, dmo_t = cu(dSo), cu(dmo)
    out = chunk_bwd(*(t[k] for k in KEYS), to_torch(do, dtype), L=L, ub_down=t.get("U_down"), ub_up=t.get("U_up"),
                    state_in=cu(S_in), mean_in=cu(m_in), d_state_out=dSo_t, d_mean_out=dmo_t, decay_logits=logits,
                    d_state_in=dSo_t if alias else None, d_mean_in=dmo_t if alias else None, detach_mean=detach)
    torch.cuda.synchronize()
    return {n: None if x is None else x.float().cpu().numpy() for n, x in out.items()}


def bwd_oracle(inp, dtype, L, do, dSo, dmo, S_in, m_in, logits=False, detach=False):
    f = lambda key: to_f64(inp[key], dtype)
    g = f("g")
    if logits:
        g = decay_from_logits(g)
    ref = carve_backward(f("q"), f("k"), f("v"), g, f("bx"), f("w"), L, to_f64(do, dtype),
                         f("U_down") if "U_down" in inp else None, f("U_up") if "U_up" in inp else None,
                         None if S_in is None else S_in.astype(np.float64),
                         None if m_in is None else m_in.astype(np.float64),
                         None if dSo is None else dSo.astype(np.float64),
                         None if dmo is None else dmo.astype(np.float64), detach_mean=detach)
    if logits:                                   # d/da of g = -softplus(a) is -sigmoid(a)
        ref["dg"] = ref["dg"] * -sigmoid(f("g"))
    return ref


def assert_grads(got, ref, tol, what):
    errs = {}
    for n, rn in NAMES.items():
        if ref[rn] is None:
            assert got[n] is None, f"{what}: {n} should be absent"
            continue
        x = got[n]
        assert np.all(np.isfinite(x)), f"{what}: non-finite {n}"
        errs[n] = rel_err(x, ref[rn])
    say(f"{what}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= tol, f"{what}: {n} rel err {e:.3e} > {tol}"


BWD_CASES = [
    # name, dtype, B, H, T, d, L, rank
    ("f32-d64-L16-r8-ragged-75", "f32", 1, 2, 75, 64, 16, 8),
    ("f32-d128-L32-r4", "f32", 1, 2, 64, 128, 32, 4),
    ("f32-d64-L64-r0-ragged-130", "f32", 2, 2, 130, 64, 64, 0),
    ("bf16-d64-L64-r0", "bf16", 2, 3, 192, 64, 64, 0),
    ("bf16-d128-L128-r16-ragged-150", "bf16", 1, 2, 150, 128, 128, 16),
    ("bf16-d64-L32-r64-ragged-100", "bf16", 2, 1, 100, 64, 32, 64),
    ("f32-T1", "f32", 2, 2, 1, 64, 64, 8),
    # without a projection: the row-sliced schedule (D / 16 workgroups per head)
    ("bf16-d128-L64-r0-ragged-200", "bf16", 1, 2, 200, 128, 64, 0),
    ("f32-d128-L16-r0-T1", "f32", 2, 1, 1, 128, 16, 0),
    ("f32-d64-L32-r0-ragged-47", "f32", 3, 1, 47, 64, 32, 0),
    # bf16 without a projection: chunk-start states from the forward pair when
    # L is a multiple of its 64-token blocks (every block or every other one),
    # from the backward's own sweep otherwise
    ("bf16-d64-L128-r0-ragged-300", "bf16", 2, 2, 300, 64, 128, 0),
    ("bf16-d128-L128-r0-ragged-129", "bf16", 1, 2, 129, 128, 128, 0),
    ("bf16-d64-L32-r0-ragged-100", "bf16", 2, 2, 100, 64, 32, 0),
]


@pytest.mark.parametrize("name,dtype,B,H,T,d,L,rank", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_matches_oracle(torch_cuda, name, dtype, B, H, T, d, L, rank):
    wl = workload(name, dtype, B, H, T, d, L, rank, 6000 + T)
    say("case", wl)
    inp = make_inputs(wl)
    do, dSo, dmo, S_in, m_in = cotangents(B, H, T, d, dtype, 6100 + T)
    got = bwd_gpu(torch_cuda, inp, dtype, L, do, dSo, dmo, S_in, m_in)
    assert_grads(got, bwd_oracle(inp, dtype, L, do, dSo, dmo, S_in, m_in), TOL[dtype], name)


def test_backward_without_state_gradients(torch_cuda):
    """No incoming state or mean and no state or mean gradients (the usual
    training call): absent tensors are zeros on both sides."""
    wl = workload("plain", "bf16", 2, 2, 256, 64, 64, 8, 6200)
    inp = make_inputs(wl)
    do = cotangents(2, 2, 256, 64, "bf16", 6201, with_state=False)[0]
    got = bwd_gpu(torch_cuda, inp, "bf16", 64, do, None, None, None, None)
    assert_grads(got, bwd_oracle(inp, "bf16", 64, do, None, None, None, None), TOL["bf16"], "no state")


CHUNK_CASES = [
    # bf16, d 64, no projection: the chunk-parallel schedule (one workgroup per
    # (batch, head, 64-token block) on the matrix cores, whatever L is; L
    # only decides which tokens d_mean_out reaches)
    ("one-short-chunk-40", 2, 2, 40, 64, True),
    ("whole-chunks-256", 1, 3, 256, 64, True),
    ("ragged-150", 2, 1, 150, 64, True),
    ("no-state-gradients-200", 2, 2, 200, 64, False),
    ("L16-ragged-90", 1, 2, 90, 16, True),
    ("L32-ragged-170", 2, 1, 170, 32, True),
    ("L128-ragged-200", 1, 2, 200, 128, True),
    ("L128-one-chunk-100", 2, 1, 100, 128, True),
]


@pytest.mark.parametrize("name,B,H,T,L,with_state", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_backward_chunk_parallel(torch_cuda, name, B, H, T, L, with_state):
    wl = workload("chunk-" + name, "bf16", B, H, T, 64, L, 0, 6900 + T)
    say("case chunk", wl)
    inp = make_inputs(wl)
    do, dSo, dmo, S_in, m_in = cotangents(B, H, T, 64, "bf16", 6950 + T, with_state=with_state)
    got = bwd_gpu(torch_cuda, inp, "bf16", L, do, dSo, dmo, S_in, m_in)
    assert_grads(got, bwd_oracle(inp, "bf16", L, do, dSo, dmo, S_in, m_in), TOL["bf16"], "chunk " + name)


def test_backward_chunk_parallel_steep_decay(torch_cuda):
    """Sub-blocks whose decay falls by more than 2^96 over 16 tokens in some
    channel (log-decays of about -6 and -30 per token) take their diagonal
    terms pairwise from the raw inputs; the rest of the chunk is factorised."""
    from chunk_gated_delta_carve_amd.workloads import bf16_bits_from_f32
    wl = workload("chunk-steep", "bf16", 1, 2, 150, 64, 64, 0, 7000)
    inp = make_inputs(wl)
    g = to_f64(inp["g"], "bf16")
    g[:, :, 0, :8] *= 10.0                       # head 0: eight steep channels
    g[:, 40:90, 1, 8:12] = -30.0                 # head 1: near-total forgetting in the middle
    inp["g"] = bf16_bits_from_f32(g.astype(np.float32))
    do, dSo, dmo, S_in, m_in = cotangents(1, 2, 150, 64, "bf16", 7001)
    got = bwd_gpu(torch_cuda, inp, "bf16", 64, do, dSo, dmo, S_in, m_in)
    assert_grads(got, bwd_oracle(inp, "bf16", 64, do, dSo, dmo, S_in, m_in), TOL["bf16"], "chunk steep")


def test_backward_chunk_parallel_in_place(torch_cuda):
    """The chunk-parallel schedule with d_state_in and d_mean_in written over
    d_state_out and d_mean_out (several chunks, so other workgroups still
    need the last chunk's mean gradient when chunk 0's is written)."""
    wl = workload("chunk-alias", "bf16", 2, 2, 200, 64, 64, 0, 7100)
    inp = make_inputs(wl)
    do, dSo, dmo, S_in, m_in = cotangents(2, 2, 200, 64, "bf16", 7101)
    ref = bwd_oracle(inp, "bf16", 64, do, dSo, dmo, S_in, m_in)
    got = bwd_gpu(torch_cuda, inp, "bf16", 64, do, dSo.copy(), dmo.copy(), S_in, m_in, alias=True)
    assert_grads(got, ref, TOL["bf16"], "chunk in place")


CONTENT_CHUNK_CASES = [
    # bf16, d 64, 64-token chunks, with a projection: one workgroup per head
    # walks the chunks from the last with the chunk-parallel products
    # name, B, H, T, rank, with_state, detach, alias
    ("r16-ragged-150", 2, 2, 150, 16, True, False, False),
    ("r64-one-chunk-64", 1, 3, 64, 64, True, False, False),
    ("r4-short-40", 2, 1, 40, 4, True, False, False),
    ("r8-no-state-gradients-256", 2, 2, 256, 8, False, False, False),
    ("r8-detached-200", 1, 2, 200, 8, True, True, False),
    ("r16-in-place-190", 2, 2, 190, 16, True, False, True),
]


@pytest.mark.parametrize("name,B,H,T,rank,with_state,detach,alias", CONTENT_CHUNK_CASES,
                         ids=[c[0] for c in CONTENT_CHUNK_CASES])
def test_backward_content_chunk_walk(torch_cuda, name, B, H, T, rank, with_state, detach, alias):
    wl = workload("content-chunk-" + name, "bf16", B, H, T, 64, 64, rank, 7200 + T)
    say("case content chunk", wl)
    inp = make_inputs(wl)
    do, dSo, dmo, S_in, m_in = cotangents(B, H, T, 64, "bf16", 7250 + T, with_state=with_state)
    ref = bwd_oracle(inp, "bf16", 64, do, dSo, dmo, S_in, m_in, detach=detach)
    if alias:
        got = bwd_gpu(torch_cuda, inp, "bf16", 64, do, dSo.copy(), dmo.copy(), S_in, m_in, alias=True)
    else:
        got = bwd_gpu(torch_cuda, inp, "bf16", 64, do, dSo, dmo, S_in, m_in, detach=detach)
    assert_grads(got, ref, TOL["bf16"], "content chunk " + name)


def test_backward_content_chunk_walk_steep_decay(torch_cuda):
    """The content walk through sub-blocks whose decay is too steep for the
    factorised diagonal products (pairwise path, with the gate bias)."""
    from chunk_gated_delta_carve_amd.workloads import bf16_bits_from_f32
    wl = workload("content-chunk-steep", "bf16", 1, 2, 150, 64, 64, 16, 7300)
    inp = make_inputs(wl)
    g = to_f64(inp["g"], "bf16")
    g[:, :, 0, :8] *= 10.0
    g[:, 40:90, 1, 8:12] = -30.0
    inp["g"] = bf16_bits_from_f32(g.astype(np.float32))
    do, dSo, dmo, S_in, m_in = cotangents(1, 2, 150, 64, "bf16", 7301)
    got = bwd_gpu(torch_cuda, inp, "bf16", 64, do, dSo, dmo, S_in, m_in)
    assert_grads(got, bwd_oracle(inp, "bf16", 64, do, dSo, dmo, S_in, m_in), TOL["bf16"], "content chunk steep")


@pytest.mark.parametrize("dtype,L,rank", [("f32", 32, 0), ("f32", 32, 8), ("bf16", 64, 0)],
                         ids=["f32-r0", "f32-r8", "bf16-r0-forward-checkpoints"])
def test_backward_with_decay_logits(torch_cuda, dtype, L, rank):
    """Raw decay logits: dg is the gradient of the logit a, dg_g * (-sigmoid(a)).
    In bf16 without a projection the forward pair forms the chunk-start states
    from the same raw logits."""
    wl = workload("logits", dtype, 1, 2, 96 if dtype == "f32" else 200, 64, L, rank, 6300)
    T = wl.T
    inp = make_inputs(wl, decay_logits=True)
    do, dSo, dmo, S_in, m_in = cotangents(1, 2, T, 64, dtype, 6301)
    got = bwd_gpu(torch_cuda, inp, dtype, L, do, dSo, dmo, S_in, m_in, logits=True)
    assert_grads(got, bwd_oracle(inp, dtype, L, do, dSo, dmo, S_in, m_in, logits=True), TOL[dtype], "logits")


DETACH_CASES = [
    # both content schedules (one workgroup per head at d 64, the per-head
    # kernel at d 128) and the projection-free one, where the bit changes nothing
    ("f32-d64-L16-r8-ragged-75", "f32", 1, 2, 75, 64, 16, 8),
    ("bf16-d128-L32-r4-ragged-90", "bf16", 1, 2, 90, 128, 32, 4),
    ("bf16-d64-L64-r0", "bf16", 1, 2, 130, 64, 64, 0),
]


@pytest.mark.parametrize("name,dtype,B,H,T,d,L,rank", DETACH_CASES, ids=[c[0] for c in DETACH_CASES])
def test_backward_with_detached_means(torch_cuda, name, dtype, B, H, T, d, L, rank):
    """CARVE_DETACH_MEAN: gradients with the gate's chunk means held constant
    match the oracle's detached gradients; with a projection they differ from
    the full ones (so the bit took effect), without one they are the same."""
    wl = workload("detach-" + name, dtype, B, H, T, d, L, rank, 6600 + T)
    say("case detach", wl)
    inp = make_inputs(wl)
    do, dSo, dmo, S_in, m_in = cotangents(B, H, T, d, dtype, 6700 + T)
    got = bwd_gpu(torch_cuda, inp, dtype, L, do, dSo, dmo, S_in, m_in, detach=True)
    ref = bwd_oracle(inp, dtype, L, do, dSo, dmo, S_in, m_in, detach=True)
    assert_grads(got, ref, TOL[dtype], "detached " + name)
    full = bwd_oracle(inp, dtype, L, do, dSo, dmo, S_in, m_in)
    moved = rel_err(full["dq"], ref["dq"])
    say(f"full vs detached oracle dq: {moved:.2e}")
    if not rank:
        assert moved == 0
        return
    assert not got["d_mean_in"].any() and np.abs(full["dmean_in"]).max() > 0.02
    if dtype == "f32":
        assert moved > 10 * TOL[dtype]


def test_backward_in_place_state_gradients(torch_cuda):
    """d_state_in and d_mean_in written over d_state_out and d_mean_out."""
    wl = workload("alias", "f32", 2, 2, 80, 64, 16, 4, 6400)
    inp = make_inputs(wl)
    do, dSo, dmo, S_in, m_in = cotangents(2, 2, 80, 64, "f32", 6401)
    ref = bwd_oracle(inp, "f32", 16, do, dSo, dmo, S_in, m_in)
    got = bwd_gpu(torch_cuda, inp, "f32", 16, do, dSo.copy(), dmo.copy(), S_in, m_in, alias=True)
    assert_grads(got, ref, TOL["f32"], "in place")


@pytest.mark.parametrize("r", [0, 4])
def test_backward_empty_sequence(torch_cuda, r):
    """T = 0: the state and mean gradients pass through; the projection gets zeros."""
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_bwd
    B, H, d = 2, 3, 64
    z = lambda *s: torch.zeros(*s, device="cuda", dtype=torch.bfloat16)
    dSo = torch.randn(B, H, d, d, device="cuda")
    dmo = torch.randn(B, H, d, device="cuda")
    out = chunk_bwd(z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H, d), z(B, 0, H),
                    z(B, 0, H, d), L=64, ub_down=z(H, r, d) if r else None, ub_up=z(H, d, r) if r else None,
                    d_state_out=dSo, d_mean_out=dmo)
    torch.cuda.synchronize()
    assert torch.equal(out["d_state_in"], dSo) and torch.equal(out["d_mean_in"], dmo)
    if r:
        assert not out["dub_down"].any() and not out["dub_up"].any()


@pytest.mark.parametrize("rank", [0, 16])
def test_backward_deterministic(torch_cuda, rank):
    wl = workload("det", "bf16", 2, 2, 200, 64, 64, rank, 6500)
    inp = make_inputs(wl)
    do, dSo, dmo, S_in, m_in = cotangents(2, 2, 200, 64, "bf16", 6501)
    a = bwd_gpu(torch_cuda, inp, "bf16", 64, do, dSo, dmo, S_in, m_in)
    b = bwd_gpu(torch_cuda, inp, "bf16", 64, do, dSo, dmo, S_in, m_in)
    for n in a:
        if a[n] is not None:
            assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("wlname,rank", [("init_equiv", 0), ("init_equiv", 16)], ids=["headline-r0", "headline-r16"])
def test_backward_full_size_sampled(torch_cuda, wlname, rank):
    """The benchmarked shape (B4 H12 T2048 d64 L64 bf16) in the launch bench.py
    times, from N(0,1) output gradients; the oracle recomputes sampled
    (batch, head) pairs over the full sequence (the pairs are independent, so
    their gradients need no other pair). With a projection the factors'
    gradients sum over the batch and are not compared here."""
    torch = torch_cuda
    from chunk_gated_delta_carve_amd.workloads import bf16_bits_from_f32
    wl = WORKLOADS[wlname].with_(rank=rank, ub_std=0.05)
    say("case full size", wl)
    inp = make_inputs(wl)
    B, T, H, d = wl.B, wl.T, wl.H, wl.dv
    do = bf16_bits_from_f32(np.random.default_rng(6600 + rank).standard_normal((B, T, H, d)).astype(np.float32))
    got = bwd_gpu(torch, inp, "bf16", wl.L, do, None, None, None, None)
    for b, h in ((0, 0), (3, 11)):
        sub = {k: (v[b:b + 1, :, h:h + 1] if k not in ("U_down", "U_up") else v[h:h + 1]) for k, v in inp.items()}
        sub["w"] = inp["w"][b:b + 1, :, h:h + 1]
        ref = bwd_oracle(sub, "bf16", wl.L, do[b:b + 1, :, h:h + 1], None, None, None, None)
        pick = {n: (None if x is None or n in ("dub_down", "dub_up") else
                    (x[b:b + 1] if n in ("d_state_in", "d_mean_in") else x[b:b + 1, :, h:h + 1]))
                for n, x in got.items()}
        pick["d_state_in"] = got["d_state_in"][b:b + 1, h:h + 1]
        pick["d_mean_in"] = got["d_mean_in"][b:b + 1, h:h + 1]
        ref["dU_down"] = ref["dU_up"] = None
        assert_grads(pick, ref, TOL["bf16"], f"full size rank {rank} pair ({b}, {h})")


@pytest.mark.parametrize("rank", [0, 8])
def test_backward_graph_replays_match_eager(torch_cuda, rank):
    """carve_chunk_bwd captured in a HIP graph (outputs and workspace
    allocated before the capture) and replayed, with eager work on the
    stream between replays, gives bit for bit the eager call's gradients."""
    torch = torch_cuda
    from chunk_gated_delta_carve_amd import chunk_bwd, recurrent_ref_shapes
    wl = workload("graph", "bf16", 2, 2, 160, 64, 64, rank, 6700 + rank)
    inp = make_inputs(wl)
    t = {k: to_torch(v, "bf16") for k, v in inp.items()}
    do = to_torch(cotangents(2, 2, 160, 64, "bf16", 6701, with_state=False)[0], "bf16")
    ws = torch.empty(int(recurrent_ref_shapes(2, 2, 160, 64, 64, 64, rank, torch.bfloat16).bwd_workspace_bytes),
                     dtype=torch.uint8, device="cuda")
    ub = dict(ub_down=t["U_down"], ub_up=t["U_up"]) if rank else {}
    args = [t[k] for k in KEYS] + [do]
    eager = chunk_bwd(*args, L=64, workspace=ws, **ub)
    eager = {n: None if x is None else x.clone() for n, x in eager.items()}
    out = chunk_bwd(*args, L=64, workspace=ws, **ub)              # buffers the graph writes
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            chunk_bwd(*args, L=64, workspace=ws, out=out, stream=side.cuda_stream, **ub)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(3):
        for x in out.values():
            if x is not None:
                x.fill_(7.0)                                    # the replay must rewrite every output
        graph.replay()
        scratch = torch.ones(1 << 20, device="cuda").sum()      # eager work between replays
        torch.cuda.synchronize()
        for n, x in eager.items():
            if x is not None:
                assert torch.equal(out[n], x), f"replay {i}: {n}"
        assert float(scratch) == float(1 << 20)
