"""Host-side checks of the C ABI that need no GPU: exports, validation, tables."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from transformer_encoder_forward_amd import binding as B
from transformer_encoder_forward_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "enc.h")).read()
    declared = set(re.findall(r"^ENC_API[^(]*?\b(\w+)\(", hdr, re.M))
    assert declared == set(B.EXPORTS)
    lib = C.CDLL(B.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_create_without_gfx950_fails_cleanly():
    # no GPU here: enc_create must report an error, not crash
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = C.c_void_p()
    st = B.lib().enc_create(0, C.byref(h))
    assert st in (B.ENC_EDEVICE, B.ENC_EUNSUPPORTED)
    assert not h.value
    assert B.lib().enc_last_error(None)


# fake, aligned device addresses: validation never dereferences them
X, Y, W0, W1, RS, BIAS = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000


def _gemm(path=B.ENC_F32, flags=0):
    d = B.GemmDesc()
    d.path, d.x, d.y = path, X, Y
    d.w[0], d.w[1] = W0, W1
    d.row_scale[0] = d.row_scale[1] = RS
    d.alpha, d.flags = 1.0, flags
    return d


def test_check_gemm_accepts_qkv_panel():
    items = [(100, 64, 128, 128, 192, 0, 0, 0), (100, 64, 128, 128, 192, 1, 0, 64),
             (100, 64, 128, 128, 192, 1, 0, 128)]
    st, msg = B.check_gemm(_gemm(), items)
    assert st == B.ENC_OK, msg


@pytest.mark.parametrize("mutate,items,want", [
    (lambda d: None, [], B.ENC_EINVAL),                                         # no items
    (lambda d: None, [(4, 8, 8, 8, 8, 0, 0, 0)] * 5, B.ENC_EINVAL),             # > 4 items
    (lambda d: setattr(d, "x", 0), [(4, 8, 8, 8, 8, 0, 0, 0)], B.ENC_EINVAL),  # null x
    (lambda d: None, [(4, 8, 6, 8, 8, 0, 0, 0)], B.ENC_EUNSUPPORTED),           # k % 4
    (lambda d: None, [(4, 8, 8, 4, 8, 0, 0, 0)], B.ENC_ESHAPE),                 # ldx < k
    (lambda d: None, [(4, 8, 8, 8, 8, 2, 0, 0)], B.ENC_EINVAL),                 # empty slot
    (lambda d: None, [(4, 8, 8, 8, 16, 0, 0, 0), (4, 8, 8, 8, 16, 1, 0, 4)],
     B.ENC_EINVAL),                                                             # overlapping Y
    (lambda d: setattr(d, "flags", B.ENC_Y_F16 | B.ENC_Y_ACCUMULATE),
     [(4, 8, 8, 8, 8, 0, 0, 0)], B.ENC_EUNSUPPORTED),
    (lambda d: setattr(d, "x", X + 4), [(4, 8, 8, 8, 8, 0, 0, 0)], B.ENC_EUNSUPPORTED),
])
def test_check_gemm_rejects(mutate, items, want):
    d = _gemm()
    mutate(d)
    st, msg = B.check_gemm(d, items)
    assert st == want, msg
    assert msg


def test_check_gemm_gated():
    d = _gemm(flags=B.ENC_EPI_GATE_GELU_TANH)
    assert B.check_gemm(d, [(4, 8, 8, 8, 8, 0, 0, 0)])[0] == B.ENC_OK
    assert B.check_gemm(d, [(4, 8, 8, 8, 8, 1, 0, 0)])[0] == B.ENC_EINVAL  # no slot 2
    d = _gemm(flags=B.ENC_EPI_GATE_SILU | B.ENC_Y_ACCUMULATE)
    assert B.check_gemm(d, [(4, 8, 8, 8, 8, 0, 0, 0)])[0] == B.ENC_EUNSUPPORTED
    d = _gemm(flags=B.ENC_EPI_GATE_SILU | B.ENC_EPI_GATE_GELU_TANH)
    assert B.check_gemm(d, [(4, 8, 8, 8, 8, 0, 0, 0)])[0] == B.ENC_EINVAL
    d = _gemm(flags=B.ENC_EPI_GATE_SILU)
    d.bias[0] = BIAS
    assert B.check_gemm(d, [(4, 8, 8, 8, 8, 0, 0, 0)])[0] == B.ENC_EUNSUPPORTED


def test_check_gemm_int8_needs_scales_and_k16():
    d = _gemm(B.ENC_I8F16)
    assert B.check_gemm(d, [(4, 8, 32, 32, 8, 0, 0, 0)])[0] == B.ENC_OK
    assert B.check_gemm(d, [(4, 8, 24, 24, 8, 0, 0, 0)])[0] == B.ENC_EUNSUPPORTED
    d.row_scale[0] = None
    assert B.check_gemm(d, [(4, 8, 32, 32, 8, 0, 0, 0)])[0] == B.ENC_EINVAL


def _attn(hd=64, nq=4, nkv=2):
    d = B.AttnDesc()
    d.path, d.qkv, d.out = B.ENC_F32, X, Y
    d.ld = (nq + 2 * nkv) * hd
    d.q_col, d.k_col, d.v_col = 0, nq * hd, (nq + nkv) * hd
    d.ldo = nq * hd
    d.nq, d.nkv, d.hd = nq, nkv, hd
    d.scale, d.window, d.rows = 0.125, 0, 100
    return d


def test_check_attention():
    ok = [[(0, 40)], [(40, 30), (90, 10)]]
    assert B.check_attention(_attn(), ok)[0] == B.ENC_OK
    assert B.check_attention(_attn(hd=96), ok)[0] == B.ENC_EUNSUPPORTED
    assert B.check_attention(_attn(nq=3, nkv=2), ok)[0] == B.ENC_EINVAL
    assert B.check_attention(_attn(), [[(0, 40)], [(39, 5)]])[0] == B.ENC_EINVAL  # overlap
    assert B.check_attention(_attn(), [[(90, 20)]])[0] == B.ENC_EINVAL            # past rows
    d = _attn()
    d.ld = 100
    assert B.check_attention(d, ok)[0] != B.ENC_OK


def _fake_model(name, **kw):
    w = wl.make(name, layers=2, **kw)
    layers = (B.Layer * 2)()
    p = 0x10000000
    for li in range(2):
        L = layers[li]
        for n in B._LAYER_U32:
            setattr(L, n, int(w.cfg[n]))
        L.eps, L.attn_scale = w.cfg["eps"], w.cfg["attn_scale"]
        for n in B._LAYER_PTRS:
            key = n
            if key in w.layers[li] or (w.cfg["path"] == 1 and key in wl.weight_shapes(w.cfg)):
                setattr(L, n, p)
                p += 0x100000
        L.window = int(w.layers[li].get("window", w.cfg["window"]))
        L.v_norm = 1 if w.cfg.get("v_norm") else 0
        L.scalar = float(w.layers[li].get("scalar", 0.0))
        L.n_ple, L.ple_scale = int(w.cfg.get("n_ple", 0)), float(w.cfg.get("ple_scale", 1.0))
        if L.n_ple:
            for n in B._LAYER_PLE_PTRS:
                setattr(L, n, p)
                p += 0x100000
    m = B.Model()
    m.nlayers, m.layers, m.final_kind = 2, layers, w.cfg["final"]
    m.final_w = 0x7000000 if w.final_w is not None else None
    m.final_eps = 1e-6
    items = B.make_items(w.items)
    b = B.Batch()
    b.rows, b.items, b.nitems = w.rows, items, len(w.items)
    b.rope_cos[0] = b.rope_sin[0] = 0x8000000 if w.cfg["rope_sections"] else None
    return w, m, b, (layers, items)


@pytest.mark.parametrize("name,kw", [("vit_layer_f32", {}),
                                     ("gemma_text_f32", dict(lengths=[5, 7])),
                                     ("zimage_dit_1056", dict(grid=2, ncap=2, lazy_int8=True))])
def test_check_model_accepts_workloads(name, kw):
    w, m, b, keep = _fake_model(name, **kw)
    st, msg = B.check_model(m, b)
    assert st == B.ENC_OK, msg
    assert B.lib().enc_workspace_bytes(C.byref(m), C.byref(b)) > 0


def test_check_model_rejects():
    w, m, b, keep = _fake_model("gemma_text_f32", lengths=[5, 7])
    b.rows = 13  # items cover 12
    assert B.check_model(m, b)[0] == B.ENC_ESHAPE
    b.rows = 12
    b.rope_cos[0] = None
    assert B.check_model(m, b)[0] == B.ENC_EINVAL
    b.rope_cos[0] = 0x8000000
    m.layers[1].hd = 96
    assert B.check_model(m, b)[0] == B.ENC_EUNSUPPORTED
    m.layers[1].hd = 64
    m.layers[1].d = 256
    assert B.check_model(m, b)[0] == B.ENC_EUNSUPPORTED
    m.layers[1].d = 512
    m.layers[0].q_norm_w = None
    assert B.check_model(m, b)[0] == B.ENC_EINVAL


def test_validate_model_gives_check_model_status():
    w, m, b, keep = _fake_model("gemma_text_f32", lengths=[5, 7])
    V = lambda: B.lib().enc_validate_model(C.byref(m), C.byref(b))  # noqa: E731
    assert V() == B.ENC_OK
    b.rows = 13
    assert V() == B.check_model(m, b)[0] == B.ENC_ESHAPE
    b.rows = 12
    m.layers[1].hd = 96
    assert V() == B.check_model(m, b)[0] == B.ENC_EUNSUPPORTED
    assert B.lib().enc_validate_model(None, None) == B.check_model(None, None)[0] != B.ENC_OK


def test_check_model_text_encoder_options():
    w, m, b, keep = _fake_model("gemma_text_ple_f32", lengths=[5, 7])
    st, msg = B.check_model(m, b)
    assert st == B.ENC_OK, msg
    base = B.lib().enc_workspace_bytes(C.byref(m), C.byref(b))
    # the branch's two [rows][n_ple] f32 buffers
    assert base >= 2 * 12 * 256 * 4
    L = m.layers[1]
    L.rope_table = 1                      # no second table in the batch
    assert B.check_model(m, b)[0] == B.ENC_EINVAL
    b.rope_cos[1] = b.rope_sin[1] = 0x9000000
    assert B.check_model(m, b)[0] == B.ENC_OK
    L.rope_table = B.MAX_ROPE_TABLES
    assert B.check_model(m, b)[0] == B.ENC_EINVAL
    L.rope_table = 0
    L.n_ple = 96                          # not a multiple of 64
    assert B.check_model(m, b)[0] == B.ENC_EUNSUPPORTED
    L.n_ple = 256
    L.ple_gate = None
    assert B.check_model(m, b)[0] == B.ENC_EINVAL
    L.ple_gate = 0x6000000
    L.scalar = float("nan")
    assert B.check_model(m, b)[0] == B.ENC_EINVAL
    L.scalar = 1.0
    L.path = m.layers[0].path = 1         # per-layer input on the int8 path
    assert B.check_model(m, b)[0] != B.ENC_OK
    w2, m2, b2, keep2 = _fake_model("vit_layer_f32")
    m2.layers[0].v_norm = 1               # a sandwich option on a pre-LN layer
    assert B.check_model(m2, b2)[0] == B.ENC_EUNSUPPORTED


def test_workspace_grows_with_rows():
    w, m, b, keep = _fake_model("gemma_text_f32", lengths=[5, 7])
    b.rows = 1000
    a = B.lib().enc_workspace_bytes(C.byref(m), C.byref(b))
    b.rows = 2000
    c = B.lib().enc_workspace_bytes(C.byref(m), C.byref(b))
    assert c > a > 0 and a % 256 == 0
    # A, panel, attention out, T, m, H in f32 at d 512, ff 2048, 8x64 heads
    per_row = 4 * (512 + 1536 + 512 + 512 + 2048 + 512)
    assert a >= 1000 * per_row


def _up256(v):
    return (v + 255) // 256 * 256


def _split_bytes(records, hd):
    return _up256(records * hd * 4) + _up256(records * 8) if records else 0


def test_attention_key_split_workspace_rule():
    """Key splits: windowless f32 items whose 128-query tiles times heads stay
    under 768 blocks are cut into min(8, 768 // blocks, L // 128) chunks of whole
    32-key blocks; one record (hd + 2 floats) per chunk, item row and head."""
    def ws(items, nq=12, hd=64, window=0, path=B.ENC_F32):
        d = B.attention_desc(None, None, nq, nq, hd, 0.125, window, ld=3 * nq * hd,
                             ldo=nq * hd, path=path, rows=1 << 20)
        return B.attention_workspace_bytes(d, items)
    # 1024 rows, 12 heads: 96 blocks -> 8 chunks of 128 keys
    assert ws([[(0, 1024)]]) == _split_bytes(8 * 1024 * 12, 64)
    # 1000 rows: min(8, 8, 7) = 7 -> chunk ceil(1000/7) = 143 -> 160 -> 7 chunks
    assert ws([[(0, 1000)]]) == _split_bytes(7 * 1000 * 12, 64)
    # 30 heads of 128 at 1056 rows: 9 tiles x 30 = 270 blocks -> 2 chunks
    assert ws([[(0, 1056)]], nq=30, hd=128) == _split_bytes(2 * 1056 * 30, 128)
    # no split: a window, the f16 path, short items, items that fill the GPU alone
    assert ws([[(0, 1024)]], window=512) == 0
    assert ws([[(0, 1024)]], path=B.ENC_I8F16) == 0
    assert ws([[(0, 255)]]) == 0
    assert ws([[(0, 8192)]]) == 0
    # items are planned one by one and their records add up (same launch)
    assert ws([[(0, 1024)], [(1024, 1024)], [(2048, 100)]]) == _split_bytes(2 * 8 * 1024 * 12, 64)


def test_attention_workspace_checked():
    d = B.attention_desc(None, None, 12, 12, 64, 0.125, 0, ld=3 * 768, ldo=768, rows=1024)
    d.qkv = d.out = 0x10000
    items = B.make_items([[(0, 1024)]])
    need = B.attention_workspace_bytes(d, [[(0, 1024)]])
    msg = C.create_string_buffer(256)
    d.ws, d.ws_bytes = 0x100000, need - 1
    assert B.lib().enc_check_attention(C.byref(d), items, 1, msg, 256) == B.ENC_ESHAPE
    d.ws_bytes = need
    assert B.lib().enc_check_attention(C.byref(d), items, 1, msg, 256) == B.ENC_OK
    d.ws = 0x100010
    assert B.lib().enc_check_attention(C.byref(d), items, 1, msg, 256) == B.ENC_EUNSUPPORTED
    d.ws, d.ws_bytes = None, 0  # no workspace: nothing is split, always valid
    assert B.lib().enc_check_attention(C.byref(d), items, 1, msg, 256) == B.ENC_OK


def test_model_workspace_holds_key_splits():
    w, m, b, keep = _fake_model("vit_layer_f32")
    small = B.lib().enc_workspace_bytes(C.byref(m), C.byref(b))  # 64 rows: no split
    items = B.make_items([[(0, 1024)]])
    b.rows, b.items, b.nitems = 1024, items, 1
    big = B.lib().enc_workspace_bytes(C.byref(m), C.byref(b))
    # vit_layer_f32: 2 heads of 64 -> 16 blocks -> 8 chunks of 128 keys
    # A, attention out, T, H at d 128; the panel (384); the GELU hidden (512)
    dense = _up256(1024 * 128 * 4) * 4 + _up256(1024 * 384 * 4) + _up256(1024 * 512 * 4)
    assert big == dense + _split_bytes(8 * 1024 * 2, 64) > small


# --------------------------------------------------- tables vs the oracle

@pytest.mark.parametrize("name,kw", [
    ("gemma_text_f32", {}),
    ("zimage_dit_1056", dict(lazy_int8=True, layers=0)),
    ("zimage_dit_cfg_8448", dict(lazy_int8=True, layers=0)),
    ("zimage_dit_cfg_8448", dict(lazy_int8=True, layers=0, grid=5, ncap=3)),
])
def test_positions_bit_exact_vs_oracle(oracle, name, kw):
    kw.setdefault("layers", 0)
    w = wl.make(name, **kw)
    sec = w.cfg["rope_sections"]
    got = B.positions(w.rows, w.items, w.grids, sec)
    ref = oracle.positions(w.rows, w.items, w.grids, sec)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("sections,hd", [(1, 64), (2, 128), (2, 64), (1, 128)])
def test_rope_table_is_rounded_f64(sections, hd):
    rng = np.random.default_rng(sections * 7 + hd)
    pos = rng.integers(0, 4200, (300, sections)).astype(np.int32)
    cos, sin = B.rope_table(pos, hd, sections, 10000.0)
    S = hd // sections
    i = np.arange(S // 2)
    ang = np.concatenate([pos[:, s:s + 1] * 10000.0 ** (-2.0 * i / S) for s in range(sections)], 1)
    # one rounding of the f64 value: within half an f32 ulp of it
    for got, ref in ((cos, np.cos(ang)), (sin, np.sin(ang))):
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got.astype(np.float64) - ref) <= 0.5 * ulp + 1e-300)


def test_check_model_pool_needs_nonempty_items():
    w, m, b, keep = _fake_model("gemma_text_f32", lengths=[5, 7])
    items = B.make_items([[(0, 5)], [(5, 0)], [(5, 7)]])
    b.items, b.nitems = items, 3
    st, msg = B.check_model(m, b)
    assert st == B.ENC_EINVAL and "empty" in msg
    m.final_kind = 0  # no pool: an empty sequence is fine
    assert B.check_model(m, b)[0] == B.ENC_OK


def test_positions_padded_dit_items():
    """Padded CFG items ([img0 | img1 | cap0 | cap1], each range padded to 32):
    image rows on the grid, image pad rows at (0, 0), captions on the diagonal
    counted from the start of their range; unpadded items keep their tables."""
    from positions_ref import dit_positions
    for name, kw in [("zimage_dit_pad_cfg", {}), ("zimage_dit_pad_cfg", dict(grid=5, ncap=3)),
                     ("zimage_dit_cfg_8448", dict(grid=6, ncap=5)), ("zimage_dit_1056", {})]:
        w = wl.make(name, layers=1, lazy_int8=True, **kw)
        got = B.positions(w.rows, w.items, w.grids, 2)
        assert np.array_equal(got, dit_positions(w.rows, w.items, w.grids)), (name, kw)
    w = wl.make("zimage_dit_pad_cfg", layers=1, lazy_int8=True)
    assert w.items == [[(0, 928), (1856, 32)], [(928, 928), (1888, 32)]]
