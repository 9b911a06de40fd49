"""Parity at the full sizes the benchmark runs, through the same C ABI and the same
launch configurations: sampled outputs against the oracle where the oracle can
compute them one by one (GEMM rows, attention query rows, whole short items),
whole outputs where a layer fits the oracle's budget, and the invariants that hold
at any size (the CFG pair == two singles) where it does not."""
import dataclasses
import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, TOL_F32, TOL_I8F16, host, row_rel_err, say, to_dev
from transformer_encoder_forward_amd import binding as B
from transformer_encoder_forward_amd import model as M
from transformer_encoder_forward_amd import workloads as wl

pytestmark = pytest.mark.gpu

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import full_depth  # noqa: E402  (stored oracle outputs, written by tests/golden/full_depth.py)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    B.context(0)


def sample_rows(n, seed, extra=6):
    """Row 0 and 1, tile edges, the last rows, and a few seeded draws."""
    fixed = [0, 1, 127, 128, 255, 256, n // 2, n - 2, n - 1]
    rng = np.random.default_rng(seed)
    return np.unique(np.clip(np.concatenate([fixed, rng.integers(0, n, extra)]), 0, n - 1))


# ----------------------------------------------------------------- GEMMs

# (label, path, rows, out features, in features) at the workloads' sizes
FULL_GEMMS = [
    ("C2 q|k|v", B.ENC_F32, 16057, 1536, 512),
    ("C2 O", B.ENC_F32, 16057, 512, 512),
    ("C2 down", B.ENC_F32, 16057, 512, 2048),
    ("C3 up", B.ENC_F32, 1024, 3072, 768),
    ("C5 q|k|v", B.ENC_I8F16, 8448, 11520, 3840),
    ("C5 O", B.ENC_I8F16, 8448, 3840, 3840),
    ("C5 W2", B.ENC_I8F16, 8448, 3840, 10240),
]


def _gemm_inputs(rng, path, n, m, k):
    if path == B.ENC_F32:
        x = rng.standard_normal((n, k), dtype=np.float32)
        w = (0.02 * rng.standard_normal((m, k), dtype=np.float32)).astype(np.float32)
        return x, w, None
    x = rng.standard_normal((n, k), dtype=np.float32).astype(np.float16)
    q = rng.integers(-127, 128, (m, k), dtype=np.int8)
    rs = (0.002 * np.exp(0.25 * rng.standard_normal(m))).astype(np.float32)
    return x, q, rs


@pytest.mark.parametrize("label,path,n,m,k", FULL_GEMMS, ids=[g[0] for g in FULL_GEMMS])
def test_gemm_full_size_sampled_rows(label, path, n, m, k):
    say(f"full-size GEMM {label}: {n} x {m} x {k}")
    rng = np.random.default_rng(n + m + k)
    x, w, rs = _gemm_inputs(rng, path, n, m, k)
    Y = torch.empty((n, m), dtype=torch.float32, device=DEV)
    B.gemm_items(to_dev(x), Y, [to_dev(w)], [(n, m, k, k, m, 0, 0, 0)], path=path,
                 row_scale=None if rs is None else [to_dev(rs)])
    rows = sample_rows(n, m)
    xd = x[rows].astype(np.float64)
    ref = O.linear(xd, w) if path == B.ENC_F32 else O.linear_q8(xd, w, rs)
    err = row_rel_err(host(Y)[rows], ref)
    say(f"  {len(rows)} sampled rows, error {err:.2e}")
    assert err <= (TOL_F32 if path == B.ENC_F32 else TOL_I8F16)


# the gated MLP GEMMs at full size: C2 (GELU-tanh gating, f32) and C5 (SwiGLU, f16 out)
@pytest.mark.parametrize("label,path,n,ff,d", [("C2 gate/up", B.ENC_F32, 16057, 2048, 512),
                                               ("C5 W1/W3", B.ENC_I8F16, 8448, 10240, 3840)])
def test_gated_gemm_full_size_sampled_rows(label, path, n, ff, d):
    say(f"full-size gated GEMM {label}: {n} x {ff} x {d}")
    rng = np.random.default_rng(n + ff)
    i8 = path == B.ENC_I8F16
    x, wg, rg = _gemm_inputs(rng, path, n, ff, d)
    _, wu, ru = _gemm_inputs(rng, path, 1, ff, d)
    odt = torch.float16 if i8 else torch.float32
    Y = torch.empty((n, ff), dtype=odt, device=DEV)
    flags = (B.ENC_EPI_GATE_SILU | B.ENC_Y_F16) if i8 else B.ENC_EPI_GATE_GELU_TANH
    B.gemm_items(to_dev(x), Y, [to_dev(wg), to_dev(wu)], [(n, ff, d, d, ff, 0, 0, 0)], path=path,
                 row_scale=[to_dev(rg), to_dev(ru)] if i8 else None, flags=flags)
    rows = sample_rows(n, ff, extra=2)
    xd = x[rows].astype(np.float64)
    if i8:
        g, u = O.linear_q8(xd, wg, rg), O.linear_q8(xd, wu, ru)
        ref = np.vectorize(O.round_f16)(np.vectorize(O.silu)(g) * u)
    else:
        g, u = O.linear(xd, wg), O.linear(xd, wu)
        ref = np.vectorize(O.gelu_tanh)(g) * u
    err = row_rel_err(host(Y)[rows], ref)
    say(f"  {len(rows)} sampled rows, error {err:.2e}")
    assert err <= (TOL_I8F16 if i8 else TOL_F32)


# -------------------------------------------------------------- attention

def _attn_case(name):
    cfg = wl.CONFIGS[name]
    rows, items, _ = wl.layout(cfg)
    return cfg, rows, items


@pytest.mark.parametrize("name", ["gemma_text_f32", "lfm2_vit_f32", "zimage_dit_cfg_8448"])
def test_attention_full_size_sampled_queries(name):
    """The workload's own item table, heads, window and scale; q and k unit-scale
    as after qk-norm; sampled query rows from every item (and every range)."""
    cfg, rows, items = _attn_case(name)
    f16 = cfg["path"] == wl.PATH_I8F16
    nq, nkv, hd = cfg["nq"], cfg["nkv"], cfg["hd"]
    ld = (nq + 2 * nkv) * hd
    say(f"full-size attention {name}: rows {rows}, {len(items)} items, {nq}x{hd}, "
        f"window {cfg['window']}")
    rng = np.random.default_rng(len(name))
    p = rng.standard_normal((rows, ld), dtype=np.float32)
    p = p.astype(np.float16) if f16 else p
    out = torch.empty((rows, nq * hd), dtype=torch.float16 if f16 else torch.float32, device=DEV)
    B.attention_items(to_dev(p), out, items, nq, nkv, hd, cfg["attn_scale"], cfg["window"],
                      path=cfg["path"])
    sel = []
    for rr in items:
        for r0, n in rr:
            sel += [r0, r0 + n // 2, r0 + n - 1]
    sel = np.unique(np.concatenate([sel, sample_rows(rows, rows, extra=4)]))
    pd = p.astype(np.float64)
    q, k, v = pd[:, :nq * hd], pd[:, nq * hd:(nq + nkv) * hd], pd[:, (nq + nkv) * hd:]
    ref = O.attention(items, q, k, v, nq, nkv, hd, cfg["attn_scale"], cfg["window"],
                      query_rows=sel)[sel]
    if f16:
        ref = np.vectorize(O.round_f16)(ref)
    err = row_rel_err(host(out)[sel], ref)
    say(f"  {len(sel)} sampled queries, error {err:.2e}")
    assert err <= (TOL_I8F16 if f16 else TOL_F32)


# ------------------------------------------------------------ whole stacks

def run(w, x=None, layers=None):
    dm = M.DeviceModel(w, DEV, layers=layers)
    db = M.DeviceBatch(w, DEV)
    X = torch.from_numpy(np.ascontiguousarray(w.x if x is None else x)).to(DEV)
    out = torch.empty((M.out_rows(w), w.cfg["d"]), dtype=torch.float32, device=DEV)
    ws = dm.workspace(db, DEV)
    M.encoder_forward(dm, db, X, out, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["gemma_text_f32", "gemma_text_ple_f32"])
def test_text_encoder_full_batch_shortest_sequences(name):
    """The benchmark batch (16 sequences, 16 057 rows, 24 layers, pooled output):
    the pooled rows of the three shortest sequences against the oracle run on
    each sequence alone (packed == separate is pinned in the oracle), and the GPU
    packed result against the GPU run of each sequence alone, bit for bit.  Also
    with every text-encoder option on (GQA, v-norm, window pattern, two RoPE
    tables, layer scalars, per-layer input)."""
    w = wl.make(name)
    say(f"full text encoder: rows {w.rows}, layers {w.cfg['layers']}")
    pooled = host(run(w))
    assert np.isfinite(pooled).all()
    lens = [rr[0][1] for rr in w.items]
    starts = [rr[0][0] for rr in w.items]
    for i in np.argsort(lens, kind="stable")[:3]:
        r0, n = starts[i], lens[i]
        x = np.ascontiguousarray(w.x[r0:r0 + n])
        # the same model over this one sequence
        alone = dataclasses.replace(w, rows=n, items=[[(0, n)]], grids=[0], x=x)
        ref = O.forward(alone, x=x)
        err = row_rel_err(pooled[i:i + 1], ref)
        say(f"  sequence {i} (length {n}): error {err:.2e}")
        assert err <= TOL_F32
        assert np.array_equal(host(run(alone, x=x)), pooled[i:i + 1])


@pytest.mark.parametrize("name", ["gemma_text_f32", "gemma_text_ple_f32"])
def test_text_encoder_full_batch_every_sequence_vs_stored_oracle(name):
    """The benchmark batch whole (16 sequences, 16 057 rows, 24 layers): every
    pooled row, the two sequences longer than 1024 rows (where the 512-key
    window masks) included, against the oracle's forward of the same packed
    batch, stored by tests/golden/full_depth.py under a key of its inputs."""
    w = wl.make(name)
    rows, ref = full_depth.load(name, w)
    pooled = host(run(w))
    lens = [rr[0][1] for rr in w.items]
    assert max(lens) > 1024
    err = row_rel_err(pooled[rows], ref)
    say(f"full text encoder {name}: {len(rows)} pooled rows, lengths {min(lens)}..{max(lens)}, "
        f"error {err:.2e}")
    assert err <= TOL_F32


def test_vit_encoder_full_stack_vs_oracle():
    """C3 whole: 1024 rows, 16 pre-LN layers, post-LN; every output row."""
    w = wl.make("lfm2_vit_f32")
    got = host(run(w))
    err = row_rel_err(got, O.forward(w))
    say(f"full ViT encoder: error {err:.2e}")
    assert err <= TOL_F32


def test_vision_tower_full_stack_vs_oracle():
    """The vision tower whole: five images (2176 rows), 16 layers; every row."""
    w = wl.make("gemma_vision_f32")
    got = host(run(w))
    err = row_rel_err(got, O.forward(w))
    say(f"full vision tower: error {err:.2e}")
    assert err <= TOL_F32


def test_dit_1056_full_width_layer_vs_oracle():
    """C4 at full width and rows (1056 x 3840, 30 heads of 128, SwiGLU 10240), one
    layer; every output row against the oracle with its f16 sites."""
    w = wl.make("zimage_dit_1056", layers=1)
    got = host(run(w))
    err = row_rel_err(got, O.forward(w))
    say(f"DiT 1056 full-width layer: error {err:.2e}")
    assert np.isfinite(got).all()
    assert err <= TOL_I8F16


@pytest.mark.parametrize("name", ["zimage_dit_1056", "zimage_dit_cfg_8448", "zimage_dit_mod_1056",
                                  "zimage_dit_pad_cfg"])
def test_dit_full_stack_vs_stored_oracle(name):
    """The DiT stack whole (every layer, every row of the batch), its output rows
    sampled (each range's first, middle and last rows, tile edges, seeded draws)
    against the oracle's forward of the same batch with its f16 sites, stored by
    tests/golden/full_depth.py under a key of its inputs: the plain 1056-row
    stack, the 8448-row CFG pair, the modulated q8_2f stack with the Turbo
    guards and the padded CFG pair (pad rows at position (0, 0)).  For the CFG
    pairs the stored rows are the first item's (the oracle ran that item alone;
    the second item equals its own single forward bit for bit, tested below and
    in the stack tests)."""
    w = wl.make(name, lazy_int8=True)
    rows, ref = full_depth.load(name, w)
    got = host(run(w))
    assert np.isfinite(got).all()
    err = row_rel_err(got[rows], ref)
    say(f"DiT {name} full stack ({w.cfg['layers']} layers, {w.rows} rows): {len(rows)} rows, error {err:.2e}")
    assert err <= TOL_I8F16


def test_dit_step_program_full_vs_stored_oracle():
    """The DiT step program whole, through encoder_stages_forward: the context
    refiner (2 unmodulated blocks) on the 32 caption rows, the noise refiner (2
    modulated blocks) on the 1024 image rows, then the 30-block modulated stack
    on all 1056 rows, in place; sampled output rows against the oracle's
    forward_stages stored by tests/golden/full_depth.py."""
    name = "zimage_dit_step_1056"
    w = wl.make(name, lazy_int8=True)
    rows, ref = full_depth.load(name, w)
    prog = M.DeviceProgram(w, DEV)
    X = torch.from_numpy(np.ascontiguousarray(w.x)).to(DEV)
    h = torch.empty_like(X)
    ws = prog.workspace(DEV)
    M.stages_forward(prog, X, h, ws)
    torch.cuda.synchronize()
    got = host(h)
    assert np.isfinite(got).all()
    err = row_rel_err(got[rows], ref)
    say(f"DiT step program ({len(w.stages)} stages, {w.rows} rows): {len(rows)} rows, error {err:.2e}")
    assert err <= TOL_I8F16


def test_dit_padded_pair_full_width_layer_vs_oracle():
    """The padded CFG pair at full width and rows (2 x (928 + 32) = 1920 rows:
    30x30 images padded to 928 rows, 20 captions padded to 32), one layer; every
    output row against the oracle with the same positions."""
    from positions_ref import dit_positions
    w = wl.make("zimage_dit_pad_cfg", layers=1)
    pos = dit_positions(w.rows, w.items, w.grids)
    got = host(run(w))
    err = row_rel_err(got, O.forward(w, pos=pos))
    say(f"padded DiT pair full-width layer: error {err:.2e}")
    assert np.isfinite(got).all()
    assert err <= TOL_I8F16


def test_dit_modulated_full_width_layer_vs_oracle():
    """The modulated q8_2f DiT block with the Turbo guards at full width and rows
    (1056 x 3840), one layer; every output row against the oracle."""
    w = wl.make("zimage_dit_mod_1056", layers=1)
    got = host(run(w))
    err = row_rel_err(got, O.forward(w))
    say(f"modulated DiT 1056 full-width layer: error {err:.2e}")
    assert np.isfinite(got).all()
    assert err <= TOL_I8F16


def test_dit_cfg_pair_full_stack_equals_singles():
    """C5 whole (8448 rows, 30 layers): each item of the CFG pair gets the bits of
    its own single forward (4224 rows); outputs finite."""
    w = wl.make("zimage_dit_cfg_8448", lazy_int8=True)
    pair = run(w)
    assert torch.isfinite(pair).all()
    for i, rr in enumerate(w.items):
        idx = np.concatenate([np.arange(r0, r0 + n) for r0, n in rr])
        single = wl.make("zimage_dit_cfg_8448", cfg_pair=False, lazy_int8=True)
        alone = run(single, x=w.x[idx])
        say(f"  item {i}: {len(idx)} rows")
        assert torch.equal(alone, pair[torch.from_numpy(idx).to(DEV)]), f"item {i}"
        del alone
        torch.cuda.empty_cache()
