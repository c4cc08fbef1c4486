"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/carve.h, reports the shape contract, and rejects invalid
arguments before making any HIP call."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from chunk_gated_delta_carve_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from chunk_gated_delta_carve_amd.build import build_library
        build_library(verbose=False)
    return _lib.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "carve.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(carve_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def cfg(**kw):
    base = dict(B=2, H=3, T=100, dk=64, dv=64, L=64, rank=4, dtype=_lib.CARVE_BF16, flags=0)
    base.update(kw)
    return _lib.CarveConfig(*(base[n] for n in ("B", "H", "T", "dk", "dv", "L", "rank", "dtype", "flags")))


def test_shape_contract(L):
    sh = _lib.ref_shapes(cfg())
    assert sh.q == sh.k == sh.g == sh.bx == 2 * 100 * 3 * 64
    assert sh.v == sh.o == 2 * 100 * 3 * 64
    assert sh.w == 2 * 100 * 3
    assert sh.ub_down == 3 * 4 * 64 and sh.ub_up == 3 * 64 * 4
    assert sh.state == 2 * 3 * 64 * 64 and sh.mean == 2 * 3 * 64
    assert sh.workspace_bytes >= 0
    sh = _lib.ref_shapes(cfg(rank=0, dk=128, dv=128, L=128, dtype=_lib.CARVE_F32))
    assert sh.ub_down == 0 and sh.ub_up == 0 and sh.state == 2 * 3 * 128 * 128


@pytest.mark.parametrize("kw,code", [
    (dict(dk=32, dv=32), _lib.CARVE_EUNSUPPORTED),
    (dict(dk=64, dv=128), _lib.CARVE_EUNSUPPORTED),
    (dict(dk=96, dv=96), _lib.CARVE_EUNSUPPORTED),
    (dict(L=48), _lib.CARVE_EUNSUPPORTED),
    (dict(L=256), _lib.CARVE_EUNSUPPORTED),
    (dict(rank=65), _lib.CARVE_EUNSUPPORTED),
    # 64 token rows of one head exceed 32-bit byte offsets (the 16-row output
    # limit alone would still pass)
    (dict(B=1, H=300000, dk=128, dv=128, dtype=_lib.CARVE_BF16), _lib.CARVE_EUNSUPPORTED),
    (dict(B=1, H=60000, dk=128, dv=128, dtype=_lib.CARVE_BF16), _lib.CARVE_OK),
    (dict(T=-1), _lib.CARVE_EINVAL),
    (dict(B=-2), _lib.CARVE_EINVAL),
    (dict(rank=-1), _lib.CARVE_EINVAL),
    (dict(dtype=7), _lib.CARVE_EINVAL),
    (dict(flags=_lib.CARVE_DECAY_LOGITS), _lib.CARVE_OK),
    (dict(flags=_lib.CARVE_QK_L2NORM), _lib.CARVE_OK),
    (dict(flags=_lib.CARVE_DECAY_LOGITS | _lib.CARVE_QK_L2NORM), _lib.CARVE_OK),
    (dict(flags=_lib.CARVE_DETACH_MEAN), _lib.CARVE_OK),
    (dict(flags=7), _lib.CARVE_OK),
    (dict(flags=8), _lib.CARVE_EINVAL),
    (dict(flags=-1), _lib.CARVE_EINVAL),
])
def test_config_rejected(L, kw, code):
    out = _lib.CarveShapes()
    assert L.carve_recurrent_ref_shapes(ctypes.byref(cfg(**kw)), ctypes.byref(out)) == code


def test_null_config_and_output(L):
    out = _lib.CarveShapes()
    assert L.carve_recurrent_ref_shapes(None, ctypes.byref(out)) == _lib.CARVE_EINVAL
    assert L.carve_recurrent_ref_shapes(ctypes.byref(cfg()), None) == _lib.CARVE_EINVAL


FAKE = 0x10000000   # never dereferenced: validation fails before any use


def call_fwd(L, c, **ptrs):
    names = ["q", "k", "v", "g", "bx", "w", "ub_down", "ub_up", "state_in", "mean_in",
             "o", "state_out", "mean_out", "workspace"]
    base = {n: None for n in names}
    step = 1 << 24
    for i, n in enumerate(["q", "k", "v", "g", "bx", "w", "ub_down", "ub_up", "o"]):
        base[n] = FAKE + i * step
    base.update(ptrs)
    args = [ctypes.c_void_p(base[n]) if base[n] is not None else None for n in names]
    return L.carve_chunk_fwd(ctypes.byref(c) if c is not None else None, *args,
                             ctypes.c_size_t(ptrs.get("ws_bytes", 0) if False else 0), None)


def test_fwd_argument_errors(L):
    c = cfg()
    assert call_fwd(L, None) == _lib.CARVE_EINVAL
    assert call_fwd(L, c, q=None) == _lib.CARVE_EINVAL
    assert call_fwd(L, c, o=None) == _lib.CARVE_EINVAL
    assert call_fwd(L, c, ub_down=None) == _lib.CARVE_EINVAL          # rank > 0 needs U_b
    assert call_fwd(L, c, k=FAKE + 0x1000 + 4) == _lib.CARVE_EALIGN
    assert call_fwd(L, c, state_in=FAKE - 8) == _lib.CARVE_EALIGN
    assert call_fwd(L, c, o=FAKE + 64) == _lib.CARVE_EINVAL           # o overlaps q
    assert call_fwd(L, cfg(dk=96, dv=96)) == _lib.CARVE_EUNSUPPORTED
    # nothing to do: no HIP call is made and the call succeeds
    assert call_fwd(L, cfg(B=0)) == _lib.CARVE_OK
    assert call_fwd(L, cfg(T=0)) == _lib.CARVE_OK


def test_workspace_contract(L):
    """Without a content projection (bf16) the chunk-parallel schedule needs a
    workspace; a smaller one is rejected before any HIP call."""
    c = cfg(rank=0)
    sh = _lib.ref_shapes(c)
    assert sh.workspace_bytes > 0
    assert _lib.ref_shapes(cfg(rank=4)).workspace_bytes == 0
    assert _lib.ref_shapes(cfg(rank=0, dtype=_lib.CARVE_F32)).workspace_bytes == 0
    assert call_fwd(L, c, ub_down=None, ub_up=None) == _lib.CARVE_EWORKSPACE
    assert call_fwd(L, cfg(rank=0, B=0)) == _lib.CARVE_OK


def test_error_strings(L):
    for code in range(6):
        assert len(_lib.error_string(code)) > 0
    assert "unknown" in _lib.error_string(99)


def call_step(L, c, pos=0, **ptrs):
    names = ["q", "k", "v", "g", "bx", "w", "ub_down", "ub_up", "state", "mean_prev", "chunk_acc", "o"]
    step = 1 << 24
    base = {n: FAKE + i * step for i, n in enumerate(names)}
    base.update(ptrs)
    args = [ctypes.c_void_p(base[n]) if base[n] is not None else None for n in names]
    return L.carve_recurrent_step(ctypes.byref(c) if c is not None else None, ctypes.c_int32(pos), *args, None)


def test_step_argument_errors(L):
    c = cfg(T=1)
    assert call_step(L, None) == _lib.CARVE_EINVAL
    assert call_step(L, cfg(T=2)) == _lib.CARVE_EINVAL               # one token per call
    assert call_step(L, c, pos=-1) == _lib.CARVE_EINVAL
    assert call_step(L, c, pos=64) == _lib.CARVE_EINVAL               # pos < L
    assert call_step(L, cfg(T=1, L=16), pos=16) == _lib.CARVE_EINVAL
    for n in ("q", "w", "o", "state", "mean_prev", "chunk_acc", "ub_up"):
        assert call_step(L, c, **{n: None}) == _lib.CARVE_EINVAL, n
    assert call_step(L, c, v=FAKE + 2 * (1 << 24) + 8) == _lib.CARVE_EALIGN
    assert call_step(L, c, chunk_acc=FAKE + 4) == _lib.CARVE_EALIGN
    assert call_step(L, c, o=FAKE + 64) == _lib.CARVE_EINVAL          # o overlaps q
    assert call_step(L, c, state=FAKE + 3 * (1 << 24)) == _lib.CARVE_EINVAL    # state overlaps g
    assert call_step(L, c, mean_prev=FAKE + 8 * (1 << 24) + 16) == _lib.CARVE_EINVAL   # inside state
    assert call_step(L, cfg(T=1, dk=96, dv=96)) == _lib.CARVE_EUNSUPPORTED
    # rank 0 needs no projection factors; nothing to do without heads
    assert call_step(L, cfg(T=1, rank=0, B=0), ub_down=None, ub_up=None) == _lib.CARVE_OK
    assert call_step(L, cfg(T=1, B=0)) == _lib.CARVE_OK


BWD_NAMES = ["q", "k", "v", "g", "bx", "w", "ub_down", "ub_up", "state_in", "mean_in", "d_o", "d_state_out",
             "d_mean_out", "dq", "dk", "dv", "dg", "dbx", "dw", "d_ub_down", "d_ub_up", "d_state_in", "d_mean_in",
             "workspace"]


def call_bwd(L, c, ws_bytes=None, **ptrs):
    step = 1 << 24
    base = {n: FAKE + i * step for i, n in enumerate(BWD_NAMES)}
    base.update(ptrs)
    if ws_bytes is None:
        out = _lib.CarveShapes()
        ok = c is not None and L.carve_recurrent_ref_shapes(ctypes.byref(c), ctypes.byref(out)) == _lib.CARVE_OK
        ws_bytes = out.bwd_workspace_bytes if ok else 0
    args = [ctypes.c_void_p(base[n]) if base[n] is not None else None for n in BWD_NAMES]
    return L.carve_chunk_bwd(ctypes.byref(c) if c is not None else None, *args, ctypes.c_size_t(ws_bytes), None)


def test_bwd_workspace_size():
    """The backward workspace holds, per (batch, head), the fp32 state at every
    chunk start and one chunk's recomputed states (every token's for the
    one-workgroup-per-head kernel at d = 128 with a projection, every 8-token
    sub-block start for the row-lane kernel), small per-chunk vectors, and
    every token's column sums per row slice (one slice of all rows with a
    projection at d = 64, d / 16 slices without one, none at d = 128 with one);
    in bf16 without a projection and with L a multiple of 64, also the
    forward pair's block images and output."""
    sh = _lib.ref_shapes(cfg(dtype=_lib.CARVE_F32))  # B2 H3 T100 d64 L64 rank 4: two chunks
    vecs = 2 * 2 * 64 + 2 * 4 + 2 * 4 * 64           # z and m per chunk, U_down m per chunk, dU partials
    per_bh = 2 * 64 * 64 + 8 * 64 * 64 + vecs
    per_bh = (per_bh + 3) // 4 * 4 + 100 * 1 * (4 * 64 + 1)
    assert sh.bwd_workspace_bytes == 6 * 4 * ((per_bh + 3) // 4 * 4)
    # in bf16 at d 64 with 64-token chunks, the per-head chunk walk: the state,
    # gate bias and gate mean of every chunk, one carried state gradient, the
    # factor gradients' partial sums and a d_mean_out share; then a scratch
    # output for the checkpointing forward
    shc = _lib.ref_shapes(cfg())
    per_bh_c = 2 * 64 * 64 + 64 * 64 + 2 * 2 * 64 + 2 * 4 * 64 + 64
    own_c = 6 * 4 * ((per_bh_c + 3) // 4 * 4)
    assert shc.bwd_workspace_bytes == (own_c + 255) // 256 * 256 + 2 * 100 * 3 * 64 * 2
    sh128 = _lib.ref_shapes(cfg(dk=128, dv=128))
    per_bh128 = 2 * 128 * 128 + 64 * 128 * 128 + 2 * 2 * 128 + 2 * 4 + 2 * 4 * 128
    assert sh128.bwd_workspace_bytes == 6 * 4 * ((per_bh128 + 3) // 4 * 4)
    assert _lib.ref_shapes(cfg(B=0)).bwd_workspace_bytes == 0
    # without a projection the rows of a head are split into d / 16 slices, and
    # each token keeps every slice's four column sums and its dw share
    per_bh0 = 2 * 64 * 64 + 8 * 64 * 64 + 2 * 2 * 64 + 100 * 4 * (4 * 64 + 1)
    own0 = 6 * 4 * ((per_bh0 + 3) // 4 * 4)
    assert _lib.ref_shapes(cfg(rank=0, dtype=_lib.CARVE_F32)).bwd_workspace_bytes == own0
    per_bh32 = 4 * 64 * 64 + 4 * 64 * 64 + 4 * 2 * 64 + 100 * 4 * (4 * 64 + 1)   # L = 32: four chunks
    assert _lib.ref_shapes(cfg(rank=0, L=32, dtype=_lib.CARVE_F32)).bwd_workspace_bytes == 6 * 4 * per_bh32
    # in bf16 at d 64 with 64-token chunks the chunk-parallel schedule keeps
    # the state at every chunk start (written by the forward pair), the state
    # gradient at every chunk end and each row's share of d_mean_out; the
    # pair's block images and an output follow, 256-byte aligned
    sh0 = _lib.ref_shapes(cfg(rank=0))
    fwd = sh0.workspace_bytes
    assert fwd > 0
    own_ch = 6 * 4 * (2 * 2 * 64 * 64 + 64)
    assert sh0.bwd_workspace_bytes == (own_ch + 255) // 256 * 256 + fwd + 2 * 100 * 3 * 64 * 2
    long_ch = _lib.ref_shapes(cfg(rank=0, T=2560))
    own_long_ch = 6 * 4 * (2 * 40 * 64 * 64 + 64)
    assert long_ch.bwd_workspace_bytes == ((own_long_ch + 255) // 256 * 256 + long_ch.workspace_bytes
                                           + 2 * 2560 * 3 * 64 * 2)
    # the schedule works on 64-token blocks whatever L is (L only decides
    # which tokens d_mean_out reaches)
    for L in (16, 32, 128):
        assert _lib.ref_shapes(cfg(rank=0, L=L)).bwd_workspace_bytes == sh0.bwd_workspace_bytes
        assert _lib.ref_shapes(cfg(rank=0, T=2560, L=L)).bwd_workspace_bytes == long_ch.bwd_workspace_bytes
    # at d = 128 with 128-token chunks (a multiple of the pair's 64-token
    # blocks) the row-lane walk runs in chunk groups: one chunk's sub-block
    # start states per group and the state gradient at every chunk end; at
    # most sixteen groups (20 chunks here)
    long_pre = _lib.ref_shapes(cfg(rank=0, T=2560, L=128, dk=128, dv=128))
    DD = 128 * 128
    per_bh_long = 20 * DD + 16 * 16 * DD + 20 * DD + 20 * 2 * 128 + 2560 * 8 * (4 * 128 + 1)
    own_long = 6 * 4 * ((per_bh_long + 3) // 4 * 4)
    assert long_pre.bwd_workspace_bytes == ((own_long + 255) // 256 * 256 + long_pre.workspace_bytes
                                            + 2 * 2560 * 3 * 128 * 2)
    # d = 128 in bf16 keeps the grouped row-lane walk (two chunks, two groups)
    sh128_0 = _lib.ref_shapes(cfg(rank=0, dk=128, dv=128))
    per_bh128_0 = 2 * 128 * 128 + 2 * 8 * 128 * 128 + 2 * 128 * 128 + 2 * 2 * 128 + 100 * 8 * (4 * 128 + 1)
    own128_0 = 6 * 4 * ((per_bh128_0 + 3) // 4 * 4)
    assert sh128_0.bwd_workspace_bytes == ((own128_0 + 255) // 256 * 256 + sh128_0.workspace_bytes
                                           + 2 * 100 * 3 * 128 * 2)

def test_bwd_argument_errors(L):
    c = cfg()
    assert call_bwd(L, None) == _lib.CARVE_EINVAL
    for n in ("q", "d_o", "dq", "dk", "dv", "dg", "dbx", "dw", "d_ub_down", "d_ub_up", "ub_up"):
        assert call_bwd(L, c, **{n: None}) == _lib.CARVE_EINVAL, n
    assert call_bwd(L, c, dk=FAKE + 14 * (1 << 24) + 4) == _lib.CARVE_EALIGN
    assert call_bwd(L, c, d_mean_in=FAKE + 22 * (1 << 24) + 8) == _lib.CARVE_EALIGN
    assert call_bwd(L, c, ws_bytes=_lib.ref_shapes(c).bwd_workspace_bytes - 16) == _lib.CARVE_EWORKSPACE
    assert call_bwd(L, c, dq=FAKE + 64) == _lib.CARVE_EINVAL                        # dq overlaps q
    assert call_bwd(L, c, dk=FAKE + 23 * (1 << 24) + 4096) == _lib.CARVE_EINVAL     # dk inside the workspace
    assert call_bwd(L, c, dv=FAKE + 10 * (1 << 24) + 16) == _lib.CARVE_EINVAL       # dv overlaps d_o
    # d_state_in may be d_state_out itself, but not a shifted view of it
    assert call_bwd(L, c, d_state_in=FAKE + 11 * (1 << 24) + 16) == _lib.CARVE_EINVAL
    assert call_bwd(L, cfg(dk=96, dv=96)) == _lib.CARVE_EUNSUPPORTED
    # within the forward's index limits, but one thread per gradient element
    # would exceed a one-dimensional grid
    big = cfg(B=64, H=1, T=1 << 30, dk=128, dv=128, L=64, rank=0)
    assert L.carve_recurrent_ref_shapes(ctypes.byref(big), ctypes.byref(_lib.CarveShapes())) == _lib.CARVE_OK
    assert call_bwd(L, big, ws_bytes=0, ub_down=None, ub_up=None, d_ub_down=None, d_ub_up=None) \
        == _lib.CARVE_EUNSUPPORTED
    assert call_bwd(L, cfg(flags=8)) == _lib.CARVE_EINVAL
    # nothing to compute and no projection: no HIP call, success
    assert call_bwd(L, cfg(B=0, rank=0), ub_down=None, ub_up=None, d_ub_down=None, d_ub_up=None) == _lib.CARVE_OK


def test_missing_library_fails_loudly(tmp_path):
    """Without the compiled library the binding raises at first use; no path
    of the package falls back to another implementation (checked in a fresh
    interpreter whose library path points at nothing)."""
    code = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from chunk_gated_delta_carve_amd import _lib\n"
        f"_lib.LIB_PATH = {str(tmp_path / 'absent.so')!r}\n"
        "try:\n"
        "    _lib.lib()\n"
        "except ImportError as e:\n"
        "    print('raised', 'no fallback' in str(e))\n"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.stdout.strip() == "raised True", r.stdout + r.stderr


def test_noalloc_argument_errors(L):
    """carve_chunk_fwd_noalloc checks its arguments as carve_chunk_fwd does,
    before any HIP call, and rejects a problem whose workspace would exceed
    its fixed 64 MiB scratch."""
    def call(c, **ptrs):
        names = ["q", "k", "v", "g", "bx", "w", "ub_down", "ub_up", "state_in", "mean_in", "o", "state_out",
                 "mean_out"]
        base = {n: None for n in names}
        for i, n in enumerate(["q", "k", "v", "g", "bx", "w", "ub_down", "ub_up", "o"]):
            base[n] = FAKE + i * (1 << 24)
        base.update(ptrs)
        args = [ctypes.c_void_p(base[n]) if base[n] is not None else None for n in names]
        return L.carve_chunk_fwd_noalloc(ctypes.byref(c) if c is not None else None, *args, None)
    assert call(None) == _lib.CARVE_EINVAL
    assert call(cfg(), q=None) == _lib.CARVE_EINVAL
    assert call(cfg(), k=FAKE + 4) == _lib.CARVE_EALIGN
    assert call(cfg(), o=FAKE + 64) == _lib.CARVE_EINVAL
    assert call(cfg(dk=96, dv=96)) == _lib.CARVE_EUNSUPPORTED
    assert call(cfg(B=0)) == _lib.CARVE_OK
    assert call(cfg(T=0)) == _lib.CARVE_OK
    # 2048 (batch, head, 64-token block) triples of 32 KiB images fill the scratch exactly
    fits = cfg(B=1, H=16, T=128 * 64, rank=0)
    assert _lib.ref_shapes(fits).workspace_bytes == 64 << 20
    over = cfg(B=1, H=16, T=128 * 64 + 1, rank=0)
    assert _lib.ref_shapes(over).workspace_bytes > 64 << 20
    assert call(over, ub_down=None, ub_up=None, o=FAKE + 12 * (1 << 24) + (1 << 30)) == _lib.CARVE_EWORKSPACE
