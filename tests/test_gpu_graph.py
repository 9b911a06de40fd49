"""The forward captured once in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library enqueues kernels and device-to-device copies only (no memset, no
host synchronisation, no allocation), so a serving loop can capture a whole
forward and replay it without launch overhead.  Each replay must give the
eager forward's bits; between replays the test runs other eager work on the
same buffers (a fill of the output and an eager forward into another buffer)
and synchronises, so a replay cannot lean on state an earlier run left behind.
"""
import numpy as np
import pytest
import torch

from gpu_util import DEV, say
from transformer_encoder_forward_amd import binding as B
from transformer_encoder_forward_amd import model as M
from transformer_encoder_forward_amd import workloads as wl

pytestmark = pytest.mark.gpu

DIT_SMALL = dict(d=1024, nq=8, nkv=8, ff=2560)

CASES = [
    ("vit_layer_f32", dict()),
    # key-split attention (partials and merge) on every layer
    ("lfm2_vit_f32", dict(layers=2)),
    # windowed f32 attention over several sequences, final RMS + mean pool
    ("gemma_text_f32", dict(layers=2, lengths=[600, 37, 1100, 5, 130])),
    # the int8 path: f16 sites, gated SwiGLU epilogue, two-range items
    ("zimage_dit_cfg_8448", dict(layers=2, grid=8, ncap=8, overrides=DIT_SMALL)),
    # column fields, guards, adaLN modulation and the amax reduction
    ("zimage_dit_mod_1056", dict(layers=2, grid=8, ncap=8, overrides=DIT_SMALL)),
]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    B.context(0)


def _replays_match(fwd, out, ref, other):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(out)  # warm-up outside the capture, as torch asks
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(out)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(out, ref)
        say(f"  replay {i}: {'bit-identical' if same else 'DIFFERS'}")
        assert same, f"replay {i} differs from the eager forward"
        fwd(other)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, ref)


@pytest.mark.parametrize("name,kw", CASES, ids=[n for n, _ in CASES])
def test_forward_graph_replay_equals_eager(name, kw):
    w = wl.make(name, **kw)
    say(f"graph replay {name} rows={w.rows} layers={w.cfg['layers']}")
    dm = M.DeviceModel(w, DEV)
    db = M.DeviceBatch(w, DEV)
    X = torch.from_numpy(np.ascontiguousarray(w.x)).to(DEV)
    ws = dm.workspace(db, DEV)
    shape = (M.out_rows(w), w.cfg["d"])

    def fwd(o):
        M.encoder_forward(dm, db, X, o, ws)

    ref = torch.empty(shape, dtype=torch.float32, device=DEV)
    fwd(ref)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    _replays_match(fwd, torch.empty_like(ref), ref, torch.empty_like(ref))


def test_staged_program_graph_replay_equals_eager():
    """The DiT step program (refiners, then the stack) updates its rows in
    place: each replay starts from a fresh copy of the input made inside the
    graph."""
    w = wl.make("zimage_dit_step_1056", layers=2, grid=8, ncap=8, cfg_pair=True, overrides=DIT_SMALL)
    say(f"graph replay staged program rows={w.rows}")
    prog = M.DeviceProgram(w, DEV)
    X = torch.from_numpy(np.ascontiguousarray(w.x)).to(DEV)
    ws = prog.workspace(DEV)

    def fwd(o):
        M.stages_forward(prog, X, o, ws)

    ref = torch.empty_like(X)
    fwd(ref)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    _replays_match(fwd, torch.empty_like(X), ref, torch.empty_like(X))
