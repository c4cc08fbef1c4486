"""carve_chunk_fwd_noalloc (the forward entry point that allocates nothing and
keeps its workspace in a fixed device array) against carve_chunk_fwd, through
the C ABI: two calls in a row, the second with a smaller input, then a call
that needs no workspace. The same kernels run, so the results must agree bit
for bit."""
import ctypes

import numpy as np
import pytest

from chunk_gated_delta_carve_amd.workloads import WORKLOADS, make_inputs, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from chunk_gated_delta_carve_amd import _lib
    _lib.lib()
    return torch


def both(torch, wl, seed):
    from chunk_gated_delta_carve_amd import _lib
    from chunk_gated_delta_carve_amd.api import make_config
    inp = make_inputs(wl.with_(seed=seed))
    t = {k: to_torch(v, wl.dtype) for k, v in inp.items()}
    dt = t["q"].dtype
    B, T, H, d = wl.B, wl.T, wl.H, wl.dk
    cfg = make_config(B, H, T, d, d, wl.L, wl.rank, dt)
    sh = _lib.ref_shapes(cfg)
    g = torch.Generator().manual_seed(seed)
    S_in = (0.3 * torch.randn(B, H, d, d, generator=g)).cuda()
    m_in = (0.3 * torch.randn(B, H, d, generator=g)).cuda()
    p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
    ub = (t["U_down"], t["U_up"]) if wl.rank else (None, None)
    outs = []
    for noalloc in (False, True):
        o = torch.full((B, T, H, d), float("nan"), dtype=dt, device="cuda")
        S = torch.full((B, H, d, d), float("nan"), device="cuda")
        m = torch.full((B, H, d), float("nan"), device="cuda")
        args = [ctypes.byref(cfg)] + [p(t[k]) for k in ("q", "k", "v", "g", "bx", "w")] + \
               [p(ub[0]), p(ub[1]), p(S_in), p(m_in), p(o), p(S), p(m)]
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if noalloc:
            code = _lib.lib().carve_chunk_fwd_noalloc(*args, stream)
        else:
            ws = torch.empty(max(int(sh.workspace_bytes), 16), dtype=torch.uint8, device="cuda")
            code = _lib.lib().carve_chunk_fwd(*args, p(ws), ctypes.c_size_t(ws.numel()), stream)
        assert code == 0, _lib.error_string(code)
        torch.cuda.synchronize()
        outs.append((o, S, m))
    return sh, outs


@pytest.mark.parametrize("shapes", [
    # (B, H, T, d, L, rank, dtype): the first two use the fixed scratch, the second smaller
    [(4, 12, 2048, 64, 64, 0, "bf16"), (1, 3, 320, 64, 64, 0, "bf16"), (2, 2, 256, 64, 64, 8, "f32")],
    [(2, 4, 512, 128, 64, 0, "bf16"), (1, 2, 200, 128, 128, 0, "bf16"), (1, 2, 128, 64, 32, 4, "bf16")],
], ids=["d64", "d128"])
def test_noalloc_matches_fwd(torch_cuda, shapes):
    torch = torch_cuda
    for i, (B, H, T, d, L, rank, dtype) in enumerate(shapes):
        wl = WORKLOADS["tiny"].with_(B=B, H=H, T=T, dk=d, dv=d, L=L, rank=rank, dtype=dtype, ub_std=0.5)
        sh, (a, b) = both(torch, wl, 7000 + i)
        print(f"call {i}: B{B} H{H} T{T} d{d} L{L} rank{rank} {dtype}, workspace {sh.workspace_bytes} B", flush=True)
        if i < 2:
            assert sh.workspace_bytes > 0
        for n, x, y in zip(("o", "state", "mean"), a, b):
            assert torch.isfinite(x.float()).all(), n
            assert torch.equal(x, y), f"call {i}: {n} differs"


def test_noalloc_rejects_oversize(torch_cuda):
    from chunk_gated_delta_carve_amd import _lib
    from chunk_gated_delta_carve_amd.api import make_config
    cfg = make_config(8, 16, 4096, 64, 64, 64, 0, torch_cuda.bfloat16)   # 64 MiB of block images and more
    assert _lib.ref_shapes(cfg).workspace_bytes > 64 << 20
    fake = ctypes.c_void_p(1 << 32)
    args = [ctypes.byref(cfg)] + [fake] * 6 + [None] * 4 + [ctypes.c_void_p((1 << 32) + (1 << 30)), None, None, None]
    assert _lib.lib().carve_chunk_fwd_noalloc(*args) == _lib.CARVE_EWORKSPACE
