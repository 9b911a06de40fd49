"""GPU parity of the whole forward (encoder_forward / encoder_layer_forward)
against the f64 oracle, per workload, plus the invariants that hold at any
size: packed == separate, the CFG pair == two singles, the fused layer chain ==
layer-by-layer, determinism."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, TOL_F32, TOL_I8F16, host, row_rel_err, say
from transformer_encoder_forward_amd import binding as B
from transformer_encoder_forward_amd import model as M
from transformer_encoder_forward_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    B.context(0)


def run(w, layers=None, x=None):
    dm = M.DeviceModel(w, DEV, layers=layers)
    db = M.DeviceBatch(w, DEV)
    X = torch.from_numpy(np.ascontiguousarray(w.x if x is None else x)).to(DEV)
    out = torch.empty((M.out_rows(w), w.cfg["d"]), dtype=torch.float32, device=DEV)
    ws = dm.workspace(db, DEV)
    M.encoder_forward(dm, db, X, out, ws)
    torch.cuda.synchronize()
    return out


def tol(w):
    return TOL_I8F16 if w.cfg["path"] == wl.PATH_I8F16 else TOL_F32


DIT_SMALL = dict(d=1024, nq=8, nkv=8, ff=2560)

CASES = [
    ("vit_layer_f32", dict()),
    ("gemma_text_f32", dict(layers=2, lengths=[600, 37, 1100, 5, 130])),
    ("lfm2_vit_f32", dict(layers=2)),
    ("zimage_dit_1056", dict(layers=2, grid=8, ncap=8, overrides=DIT_SMALL)),
    ("zimage_dit_1056", dict(layers=1, grid=4, ncap=4)),
    ("zimage_dit_cfg_8448", dict(layers=2, grid=6, ncap=5, overrides=DIT_SMALL)),
    # GQA 8:2, v-norm, windowed / global layers with their own RoPE tables, layer
    # scalars, per-layer input
    ("gemma_text_ple_f32", dict(layers=3, lengths=[600, 37, 1100, 5, 130],
                                overrides=dict(global_every=2))),
    # the vision tower: images of 20x20, 12x12, 9x9 and 3x3 patches (the first
    # two take the key split)
    ("gemma_vision_f32", dict(layers=2, lengths=[20, 12, 9, 3])),
    # adaLN modulation, q8_2f column fields, the Turbo guards
    ("zimage_dit_mod_1056", dict(layers=2, grid=8, ncap=8, overrides=DIT_SMALL)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_forward_vs_oracle(name, kw):
    w = wl.make(name, **kw)
    say(f"forward {name} rows={w.rows} layers={w.cfg['layers']} d={w.cfg['d']}")
    got = host(run(w))
    ref = O.forward(w)
    err = row_rel_err(got, ref)
    say(f"  max row-relative error {err:.3e} (tolerance {tol(w):.0e})")
    if w.cfg["path"] == wl.PATH_I8F16:
        err64 = row_rel_err(got, O.forward(w, f16_sites=False))
        say(f"  vs the pure-f64 diagnostic (no f16 sites): {err64:.3e}")
    assert np.isfinite(got).all()
    assert err <= tol(w)


@pytest.mark.parametrize("name,kw", [
    ("gemma_text_f32", dict(layers=3, lengths=[300, 77, 700])),
    ("lfm2_vit_f32", dict(layers=2, overrides=dict(), lengths=[200])),
    ("zimage_dit_cfg_8448", dict(layers=2, grid=4, ncap=8, overrides=DIT_SMALL)),
    ("gemma_text_ple_f32", dict(layers=3, lengths=[300, 77, 700], overrides=dict(global_every=2))),
    ("zimage_dit_mod_1056", dict(layers=2, grid=4, ncap=8, overrides=DIT_SMALL)),
])
def test_fused_chain_equals_layer_by_layer(name, kw):
    """encoder_forward (each layer's last row op writes the next pre-norm) gives
    the same bits as encoder_layer_forward called per layer, both with each layer
    computing its own pre-norm and as a chain that hands the next layer's input
    over in `a` (written by the last row op of the layer before)."""
    w = wl.make(name, **kw)
    w.cfg["final"] = wl.FINAL_NONE
    fused = run(w)
    dm = M.DeviceModel(w, DEV)
    db = M.DeviceBatch(w, DEV)
    x0 = torch.from_numpy(w.x.copy()).to(DEV)
    db.batch.ple_x = x0.data_ptr()  # the rows the per-layer inputs project
    ws = dm.workspace(db, DEV)
    nl = w.cfg["layers"]
    h = torch.from_numpy(w.x.copy()).to(DEV)
    for li in range(nl):
        M.encoder_layer_forward(dm, li, db, h, ws)
    torch.cuda.synchronize()
    assert torch.equal(fused, h)
    # the chain: layer 0 computes its pre-norm; each call writes the next one's
    copies = 3 if w.cfg.get("col_fields") else 1
    esz = torch.float16 if w.cfg["path"] == wl.PATH_I8F16 else torch.float32
    a = torch.full((copies * w.rows * w.cfg["d"],), float("nan"), dtype=esz, device=DEV)
    h = torch.from_numpy(w.x.copy()).to(DEV)
    M.layer_input(dm, 0, h, a)
    for li in range(nl):
        M.encoder_layer_forward(dm, li, db, h, ws, a=a, next_layer=li + 1 if li + 1 < nl else None)
    torch.cuda.synchronize()
    assert torch.equal(fused, h)


@pytest.mark.parametrize("name", ["gemma_text_f32", "gemma_text_ple_f32"])
def test_packed_equals_separate_stack(name):
    lengths = [513, 40, 1030]
    kw = dict(overrides=dict(global_every=2)) if name == "gemma_text_ple_f32" else {}
    w = wl.make(name, layers=2, lengths=lengths, **kw)
    packed = run(w)
    r = 0
    for i, n in enumerate(lengths):
        ws_ = wl.make(name, layers=2, lengths=[n], **kw)
        alone = run(ws_, x=w.x[r:r + n])
        assert torch.equal(alone[0], packed[i]), f"sequence {i}"
        r += n


def test_packed_images_equal_separate():
    """Vision tower: each packed image gets the bits of its forward alone."""
    sides = [20, 7, 12]
    w = wl.make("gemma_vision_f32", layers=2, lengths=sides)
    packed = run(w)
    r = 0
    for i, g in enumerate(sides):
        alone = run(wl.make("gemma_vision_f32", layers=2, lengths=[g]), x=w.x[r:r + g * g])
        assert torch.equal(alone, packed[r:r + g * g]), f"image {i}"
        r += g * g


@pytest.mark.parametrize("name,grid,ncap", [("zimage_dit_cfg_8448", 4, 8), ("zimage_dit_mod_1056", 4, 8),
                                            ("zimage_dit_cfg_8448", 32, 32), ("zimage_dit_pad_cfg", 7, 5)])
def test_cfg_pair_equals_two_singles(name, grid, ncap):
    """The CFG batch-2 program gives each item the bits of its single forward
    (at 32x32 + 32 rows per item the attention takes key splits)."""
    kw = dict(layers=2, grid=grid, ncap=ncap, overrides=DIT_SMALL)
    w = wl.make(name, cfg_pair=True, **kw)
    pair = run(w)
    for i, rr in enumerate(w.items):
        idx = np.concatenate([np.arange(r0, r0 + n) for r0, n in rr])
        single = wl.make(name, cfg_pair=False, **kw)
        alone = run(single, x=w.x[idx])
        assert torch.equal(alone, pair[torch.from_numpy(idx).to(DEV)]), f"item {i}"


def test_padded_dit_pair_vs_oracle():
    """The CFG pair with padded lengths (zimage.rs `prepare`: image and caption
    ranges padded to 32 rows, the image's with the learned pad row): a 7x7 image
    (49 rows + 15 pad rows) and 5 captions (+ 27 pad rows) per item, two layers;
    the oracle takes the same positions (pad rows at (0, 0)) from the rule
    written out in tests/positions_ref.py."""
    from positions_ref import dit_positions
    w = wl.make("zimage_dit_pad_cfg", layers=2, grid=7, ncap=5, overrides=DIT_SMALL)
    assert w.items == [[(0, 64), (128, 32)], [(64, 64), (160, 32)]]
    pos = dit_positions(w.rows, w.items, w.grids)
    assert np.array_equal(B.positions(w.rows, w.items, w.grids, 2), pos)
    got = host(run(w))
    err = row_rel_err(got, O.forward(w, pos=pos))
    say(f"padded DiT pair: rows {w.rows}, error {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= TOL_I8F16


def test_amax_per_site_vs_oracle():
    """The guard calibration: each layer's max |stored half| at the five sites
    (q/k/v input, panel, attention output, w1/w3 input, hidden), after the
    column fields and guards, against the oracle's."""
    w = wl.make("zimage_dit_mod_1056", layers=2, grid=8, ncap=8, overrides=DIT_SMALL)
    dm = M.DeviceModel(w, DEV)
    db = M.DeviceBatch(w, DEV)
    am = torch.zeros((2, 5), dtype=torch.float32, device=DEV)
    db.batch.amax = am.data_ptr()
    X = torch.from_numpy(w.x).to(DEV)
    out = torch.empty((w.rows, w.cfg["d"]), dtype=torch.float32, device=DEV)
    ws = dm.workspace(db, DEV)
    M.encoder_forward(dm, db, X, out, ws)
    torch.cuda.synchronize()
    ref = np.zeros((2, 5))
    O.forward(w, amax=ref)
    got = host(am)
    say(f"amax gpu {got.tolist()}\n     oracle {ref.tolist()}")
    assert np.all(np.abs(got - ref) <= TOL_I8F16 * ref)
    # the same forward without recording gives the same output bits
    assert torch.equal(out, run(w))


def _program(w, x=None):
    prog = M.DeviceProgram(w, DEV)
    X = torch.from_numpy(np.ascontiguousarray(w.x if x is None else x)).to(DEV)
    h = torch.empty_like(X)
    ws = prog.workspace(DEV)
    M.stages_forward(prog, X, h, ws)
    torch.cuda.synchronize()
    return h


def test_refiner_program_vs_oracle():
    """The DiT step program with its refiners (context refiner on the caption
    rows, noise refiner on the image rows, then the stack), CFG pair, in place."""
    w = wl.make("zimage_dit_step_1056", layers=2, grid=8, ncap=8, cfg_pair=True, overrides=DIT_SMALL)
    got = host(_program(w))
    joint = O.positions(w.rows, w.items, w.grids, 2)
    ref = O.forward_stages([(st, r0, joint[r0:r0 + st.rows]) for _, st, r0 in w.stages], w.x)
    err = row_rel_err(got, ref)
    say(f"  refiner program error {err:.2e}")
    assert err <= TOL_I8F16
    # each CFG item's rows equal the program of that item alone, bit for bit
    for i, rr in enumerate(w.items):
        idx = np.concatenate([np.arange(r0, r0 + n) for r0, n in rr])
        single = wl.make("zimage_dit_step_1056", layers=2, grid=8, ncap=8, cfg_pair=False,
                         overrides=DIT_SMALL)
        alone = _program(single, x=w.x[idx])
        assert np.array_equal(host(alone), got[idx]), f"item {i}"


def test_deterministic():
    w = wl.make("gemma_text_f32", layers=2, lengths=[333, 64])
    assert torch.equal(run(w), run(w))


def test_nonfinite_input_flagged():
    w = wl.make("gemma_text_f32", layers=1, lengths=[50, 60])
    w.cfg["final"] = wl.FINAL_NONE
    x = w.x.copy()
    x[3, 5] = np.inf
    out = host(run(w, x=x))
    assert not np.isfinite(out[:50]).all()
    assert np.isfinite(out[50:]).all()


def test_empty_and_one_row_sequences():
    """A packed batch with a one-row sequence and an empty one: every row matches
    the oracle (final RMS, no pool); with the mean pool the empty sequence is
    refused (its mean is undefined) before anything runs."""
    w = wl.make("gemma_text_f32", layers=2, lengths=[40, 1, 0, 25])
    w.cfg["final"] = wl.FINAL_NONE
    assert row_rel_err(host(run(w)), O.forward(w)) <= TOL_F32
    w.cfg["final"] = wl.FINAL_RMS_MEANPOOL
    with pytest.raises(RuntimeError, match="empty"):
        run(w)


def test_many_sequences_pooled():
    """More sequences than one pool launch takes (64): 150 short sequences."""
    lengths = [1 + (7 * i) % 13 for i in range(150)]
    w = wl.make("gemma_text_f32", layers=1, lengths=lengths)
    got = host(run(w))
    assert got.shape == (150, w.cfg["d"])
    assert row_rel_err(got, O.forward(w)) <= TOL_F32
