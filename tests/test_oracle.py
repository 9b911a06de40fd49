"""Pins of the f64 oracle against facts fixed outside it (CPU only).

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a wrong mask edge) fails it:
closed forms and hand values (tests/golden), library routines on special cases
(numpy float16 rounding, integer matmul, torch's scaled-dot-product attention
and TransformerEncoderLayer in f64), invariants (norm preservation, relative
positions, packed == separate) and brute force on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from transformer_encoder_forward_amd import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- binary16

def test_round_f16_matches_numpy_half(oracle):
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.normal(0, 1, 2000), rng.normal(0, 1e3, 2000), rng.normal(0, 1e-5, 2000),
        rng.uniform(-70000, 70000, 500),
        # exact ties between neighbouring halves: odd multiples of half an ulp
        (np.arange(1, 200, 2) * 2.0 ** -11) + 1.0, (np.arange(1, 200, 2) * 2.0 ** -25),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
         6.1e-5, 1e9, -1e9]])
    ref = vals.astype(np.float16).astype(np.float64)
    got = np.array([oracle.round_f16(v) for v in vals])
    assert np.array_equal(got, ref) or np.array_equal(np.nan_to_num(got), np.nan_to_num(ref))
    assert np.array_equal(np.signbit(got), np.signbit(ref))


# ------------------------------------------------------------------- norms

def test_norm_hand_values(oracle):
    g = _gold("norms.json")
    y = oracle.rms_norm(np.array([g["rms"]["x"]]), np.ones(2, np.float32), 0.0)[0]
    assert np.allclose(y, g["rms"]["y"], rtol=0, atol=1e-15)
    y = oracle.layer_norm(np.array([g["layernorm"]["x"]]), np.ones(4, np.float32),
                          np.zeros(4, np.float32), 0.0)[0]
    assert np.allclose(y, g["layernorm"]["y"], rtol=0, atol=1e-15)
    assert abs(oracle.gelu_tanh(1.0) - g["gelu_tanh"]["y"][0]) < 1e-15


def test_norms_match_torch_f64(oracle):
    rng = np.random.default_rng(2)
    x = rng.normal(0, 3, (7, 96))
    w = rng.normal(1, 0.1, 96).astype(np.float32)
    b = rng.normal(0, 0.1, 96).astype(np.float32)
    tx = torch.from_numpy(x)
    ref = torch.nn.functional.rms_norm(tx, (96,), torch.from_numpy(w.astype(np.float64)), eps=1e-6)
    assert np.allclose(oracle.rms_norm(x, w, 1e-6), ref.numpy(), rtol=1e-13, atol=1e-13)
    ref = torch.nn.functional.layer_norm(tx, (96,), torch.from_numpy(w.astype(np.float64)),
                                         torch.from_numpy(b.astype(np.float64)), eps=1e-6)
    assert np.allclose(oracle.layer_norm(x, w, b, 1e-6), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_rms_gain_multiplies_directly(oracle):
    # w = 0 must give 0 (a 1 + w convention would give the normed row)
    x = np.array([[1.0, -2.0, 3.0, 0.5]])
    assert np.all(oracle.rms_norm(x, np.zeros(4, np.float32), 1e-6) == 0.0)


# ------------------------------------------------------------- activations

@pytest.mark.parametrize("x", [0.1, 0.7, 1.3, 2.9, 5.0, 11.0])
def test_activation_identities(oracle, x):
    # f(x) - f(-x) = x for both gelu_tanh and silu; f(0) = 0
    assert abs(oracle.gelu_tanh(x) - oracle.gelu_tanh(-x) - x) < 1e-14 * max(1, x)
    assert abs(oracle.silu(x) - oracle.silu(-x) - x) < 1e-14 * max(1, x)
    ref = torch.nn.functional.gelu(torch.tensor(x, dtype=torch.float64), approximate="tanh")
    assert abs(oracle.gelu_tanh(x) - ref.item()) < 1e-15 * max(1, x)
    ref = torch.nn.functional.silu(torch.tensor(x, dtype=torch.float64))
    assert abs(oracle.silu(x) - ref.item()) < 1e-15 * max(1, x)
    assert oracle.gelu_tanh(0.0) == 0.0 and oracle.silu(0.0) == 0.0


# ------------------------------------------------------------------ linear

def test_linear_integer_exact(oracle):
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, (13, 200))
    w = rng.integers(-8, 9, (37, 200))
    b = rng.integers(-5, 6, 37)
    y = oracle.linear(x.astype(np.float64), w.astype(np.float32), b.astype(np.float32))
    assert np.array_equal(y, (x @ w.T + b).astype(np.float64))


def test_linear_q8_integer_exact(oracle):
    rng = np.random.default_rng(4)
    x = rng.integers(-16, 17, (9, 320))
    q = rng.integers(-127, 128, (21, 320)).astype(np.int8)
    rs = (2.0 ** -rng.integers(3, 12, 21)).astype(np.float32)
    y = oracle.linear_q8(x.astype(np.float64), q, rs)
    assert np.array_equal(y, (x @ q.astype(np.int64).T) * rs.astype(np.float64))


def test_linear_not_transposed(oracle):
    # y = x W^T with W [out][in]: a W (not W^T) product has the wrong shape,
    # and on a square W the asymmetric case tells them apart
    w = np.array([[1, 2], [0, 1]], np.float32)
    y = oracle.linear(np.array([[1.0, 0.0]]), w)
    assert np.array_equal(y, [[1.0, 0.0]])


# --------------------------------------------------------------- positions

def test_positions_1d_restart(oracle):
    items = [[(0, 3)], [(3, 5)], [(8, 1)]]
    pos = oracle.positions(9, items, [0, 0, 0], 1)[:, 0]
    assert pos.tolist() == [0, 1, 2, 0, 1, 2, 3, 4, 0]


def test_positions_2d_grid_and_captions(oracle):
    # CFG pair, grid 2, 2 caption rows each: rows [img0|img1|cap0|cap1]
    rows, items, grids = wl.layout(wl.CONFIGS["zimage_dit_1056"], grid=2, ncap=2, cfg_pair=True)
    assert rows == 12 and items == [[(0, 4), (8, 2)], [(4, 4), (10, 2)]]
    pos = oracle.positions(rows, items, grids, 2)
    img = [[0, 0], [1, 0], [0, 1], [1, 1]]  # (column, row) in row-major order
    cap = [[2, 2], [3, 3]]
    assert pos.tolist() == img + img + cap + cap


# -------------------------------------------------------------------- RoPE

def test_rope_closed_form(oracle):
    # hd 4, one section: x = e0 at position p -> (cos p, 0, sin p, 0); e1 uses
    # theta = p * base^(-1/2)
    base, p = 100.0, 3
    x = np.array([[1.0, 0, 0, 0, 0, 1.0, 0, 0]])  # two heads
    w = np.ones(4, np.float32)
    y = oracle.qk_norm_rope(x, 2, 4, w, 0.0, 1, np.array([[p]], np.int32), base)
    s = math.sqrt(4.0)  # rms of a unit vector in 4 channels = 1/2
    th1 = p * base ** -0.5
    ref = np.array([[math.cos(p), 0, math.sin(p), 0, 0, math.cos(th1), 0, math.sin(th1)]]) * s
    assert np.allclose(y, ref, atol=1e-14)


def test_rope_2d_sections(oracle):
    # hd 8, two sections of 4: first rotated by the column, second by the row
    x = np.array([[1.0, 0, 0, 0, 1.0, 0, 0, 0]])
    w = np.ones(8, np.float32)
    y = oracle.qk_norm_rope(x, 1, 8, w, 0.0, 2, np.array([[2, 5]], np.int32), 10000.0)
    r = 2.0  # 1 / rms of two unit entries in 8 channels
    ref = np.array([[math.cos(2), 0, math.sin(2), 0, math.cos(5), 0, math.sin(5), 0]]) * r
    assert np.allclose(y, ref, atol=1e-14)


def test_rope_invariants(oracle):
    rng = np.random.default_rng(5)
    hd, n = 64, 6
    q = rng.normal(0, 1, (n, hd))
    k = rng.normal(0, 1, (n, hd))
    w = np.ones(hd, np.float32)
    pos = rng.integers(0, 2000, (n, 1)).astype(np.int32)
    qr = oracle.qk_norm_rope(q, 1, hd, w, 0.0, 1, pos, 1e4)
    kr = oracle.qk_norm_rope(k, 1, hd, w, 0.0, 1, pos, 1e4)
    qn = oracle.rms_norm(q, w, 0.0)
    kn = oracle.rms_norm(k, w, 0.0)
    # norm preserved
    assert np.allclose(np.linalg.norm(qr, axis=1), np.linalg.norm(qn, axis=1), rtol=1e-13)
    # position 0 is the identity
    q0 = oracle.qk_norm_rope(q, 1, hd, w, 0.0, 1, np.zeros((n, 1), np.int32), 1e4)
    assert np.allclose(q0, qn, atol=1e-15)
    # scores depend only on relative positions
    s1 = qr @ kr.T
    q2 = oracle.qk_norm_rope(q, 1, hd, w, 0.0, 1, pos + 77, 1e4)
    k2 = oracle.qk_norm_rope(k, 1, hd, w, 0.0, 1, pos + 77, 1e4)
    assert np.allclose(q2 @ k2.T, s1, atol=1e-11)


# --------------------------------------------------------------- attention

def _sdpa(q, k, v, scale, mask):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], attn_mask=torch.from_numpy(mask)[None, None],
        scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("window", [0, 1, 3, 7, 40])
def test_attention_vs_sdpa_bruteforce(oracle, window):
    rng = np.random.default_rng(6 + window)
    L, hd, nq, nkv = 23, 8, 4, 2
    q = rng.normal(0, 1, (L, nq * hd))
    k = rng.normal(0, 1, (L, nkv * hd))
    v = rng.normal(0, 1, (L, nkv * hd))
    o = oracle.attention([[(0, L)]], q, k, v, nq, nkv, hd, 0.37, window)
    i = np.arange(L)
    mask = (np.abs(i[:, None] - i[None, :]) <= window) if window else np.ones((L, L), bool)
    for h in range(nq):
        kvh = h // (nq // nkv)
        ref = _sdpa(q[:, h * hd:(h + 1) * hd], k[:, kvh * hd:(kvh + 1) * hd],
                    v[:, kvh * hd:(kvh + 1) * hd], 0.37, mask)
        assert np.allclose(o[:, h * hd:(h + 1) * hd], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,W", [(40, 0), (40, 5), (40, 39), (17, 16), (33, 1)])
def test_attention_mask_probe(oracle, L, W):
    # Q = 0 and one-hot V per key: o_i[j] = 1/|V(i)| for visible j, else 0
    hd = 64
    q = np.zeros((L, hd))
    k = np.random.default_rng(7).normal(0, 1, (L, hd))
    v = np.eye(L, hd)
    o = oracle.attention([[(0, L)]], q, k, v, 1, 1, hd, 1.0, W)[:, :L]
    i = np.arange(L)
    pred = (np.abs(i[:, None] - i[None, :]) <= W) if W else np.ones((L, L), bool)
    assert np.array_equal(o > 0, pred)
    nvis = (np.minimum(i + W, L - 1) - np.maximum(i - W, 0) + 1) if W else np.full(L, L)
    assert np.array_equal(pred.sum(1), nvis)
    assert np.allclose(o[pred], np.repeat(1.0 / nvis, nvis), rtol=1e-15)


def test_attention_two_range_item_and_packing(oracle):
    rng = np.random.default_rng(8)
    hd, nq = 16, 3
    rows = 20
    q = rng.normal(0, 1, (rows, nq * hd))
    k = rng.normal(0, 1, (rows, nq * hd))
    v = rng.normal(0, 1, (rows, nq * hd))
    # item A = rows [0,6) ++ [14,17); item B = [6,14) ++ [17,20)
    items = [[(0, 6), (14, 3)], [(6, 8), (17, 3)]]
    o = oracle.attention(items, q, k, v, nq, nq, hd, 0.5, 0)
    for rr in items:
        idx = np.concatenate([np.arange(r0, r0 + n) for r0, n in rr])
        alone = oracle.attention([[(0, len(idx))]], q[idx], k[idx], v[idx], nq, nq, hd, 0.5, 0)
        assert np.array_equal(o[idx], alone)  # packed == separate, bit for bit
    # a two-range item with a window: t is the concatenated index
    ow = oracle.attention([[(0, 6), (14, 3)]], q, k, v, nq, nq, hd, 0.5, 2)
    idx = np.concatenate([np.arange(0, 6), np.arange(14, 17)])
    alone = oracle.attention([[(0, 9)]], q[idx], k[idx], v[idx], nq, nq, hd, 0.5, 2)
    assert np.array_equal(ow[idx], alone)


def test_attention_closed_forms(oracle):
    rng = np.random.default_rng(9)
    L, hd = 12, 8
    v = rng.normal(0, 1, (L, hd))
    k = rng.normal(0, 1, (L, hd))
    o = oracle.attention([[(0, L)]], np.zeros((L, hd)), k, v, 1, 1, hd, 1.0, 0)
    assert np.allclose(o, np.tile(v.mean(0), (L, 1)), atol=1e-15)
    # one key far larger than the rest: every query returns that key's value
    q = np.ones((L, hd))
    k2 = np.zeros((L, hd))
    k2[5] = 100.0
    o = oracle.attention([[(0, L)]], q, k2, v, 1, 1, hd, 1.0, 0)
    assert np.allclose(o, np.tile(v[5], (L, 1)), atol=1e-12)
    # window >= L-1 is full attention
    o1 = oracle.attention([[(0, L)]], q + k, k, v, 1, 1, hd, 0.3, 0)
    o2 = oracle.attention([[(0, L)]], q + k, k, v, 1, 1, hd, 0.3, L - 1)
    assert np.array_equal(o1, o2)


# ------------------------------------------------------------------ layers

def _zero_layer_weights(w):
    for t in w.layers:
        for n in list(t):
            if (n.startswith(("w", "b", "q_")) and n not in ("q_norm_w", "window")) or \
                    n in ("ple_in", "ple_gate", "ple_proj"):
                t[n] = np.zeros_like(t[n])
    return w


@pytest.mark.parametrize("name", ["vit_layer_f32", "gemma_text_f32", "zimage_dit_1056",
                                  "gemma_text_ple_f32"])
def test_zero_weights_layer_is_identity(oracle, name):
    """All projection weights zero: every residual update adds rms(0) = 0, so the
    layer is the identity, times the layer scalar where there is one."""
    kw = dict(layers=2)
    if name.startswith("gemma_text"):
        kw["lengths"] = [5, 9]
    if name == "zimage_dit_1056":
        kw.update(grid=2, ncap=2, overrides=dict(d=256, nq=2, nkv=2, ff=512))
    w = _zero_layer_weights(wl.make(name, **kw))
    w.cfg["final"] = wl.FINAL_NONE
    out = oracle.forward(w, f16_sites=False)
    ref = w.x.astype(np.float64)
    for t in w.layers:
        ref = ref * t.get("scalar", 1.0)
    assert np.array_equal(out, ref)
    if name == "gemma_text_ple_f32":
        assert not np.array_equal(ref, w.x.astype(np.float64)), "the scalars must act"


def test_pre_ln_layer_matches_torch_encoder_layer(oracle):
    """One pre-LN ViT layer == torch.nn.TransformerEncoderLayer(norm_first) in f64."""
    w = wl.make("vit_layer_f32")
    c, t = w.cfg, w.layers[0]
    d = c["d"]
    layer = torch.nn.TransformerEncoderLayer(
        d, c["nq"], dim_feedforward=c["ff"], dropout=0.0,
        activation=lambda x: torch.nn.functional.gelu(x, approximate="tanh"),
        layer_norm_eps=c["eps"], batch_first=True, norm_first=True, dtype=torch.float64)
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    with torch.no_grad():
        layer.self_attn.in_proj_weight.copy_(T(np.concatenate([t["wq"], t["wk"], t["wv"]])))
        layer.self_attn.in_proj_bias.copy_(T(np.concatenate([t["bq"], t["bk"], t["bv"]])))
        layer.self_attn.out_proj.weight.copy_(T(t["wo"]))
        layer.self_attn.out_proj.bias.copy_(T(t["bo"]))
        layer.linear1.weight.copy_(T(t["w_up"]))
        layer.linear1.bias.copy_(T(t["b_up"]))
        layer.linear2.weight.copy_(T(t["w_down"]))
        layer.linear2.bias.copy_(T(t["b_down"]))
        layer.norm1.weight.copy_(T(t["norm1_w"]))
        layer.norm1.bias.copy_(T(t["norm1_b"]))
        layer.norm2.weight.copy_(T(t["norm2_w"]))
        layer.norm2.bias.copy_(T(t["norm2_b"]))
        ref = layer(T(w.x)[None])[0].numpy()
    out = oracle.forward(w)
    assert np.abs(out - ref).max() / np.abs(ref).max() < 1e-13


F16_SITES = ("A", "panel", "qk", "att", "A2", "hidden")


def _torch_sandwich_layer(c, t, x, pos_cos_sin, items, f16, x0=None, skip=()):
    """Composition of torch f64 library ops in the sandwich order (independent check).
    GQA by repeating each kv head over its query group; the text-encoder options
    (v-norm, per-layer window, per-layer input from x0, layer scalar) as written
    on the page.  With f16, the half sites round to binary16, except those named
    in `skip` (used to show that the comparison notices a missing site)."""
    F = torch.nn.functional
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    eps, hd, nq, nkv = c["eps"], c["hd"], c["nq"], c["nkv"]

    def r16(a, site):
        return a if (not f16 or site in skip) else a.to(torch.float16).to(torch.float64)
    H = T(x)
    d = H.shape[1]

    def lin(a, name):
        if c["path"] == wl.PATH_F32:
            return a @ T(t[name]).T
        return (a @ T(t[name].astype(np.float64)).T) * T(t["s" + name[1:]])

    A = r16(F.rms_norm(H, (d,), T(t["norm1_w"]), eps), "A")
    q, k, v = r16(lin(A, "wq"), "panel"), r16(lin(A, "wk"), "panel"), r16(lin(A, "wv"), "panel")
    cos, sin = pos_cos_sin

    def qk(z, wn, nh):
        z = z.view(z.shape[0], nh, hd)
        z = F.rms_norm(z, (hd,), T(wn), eps)
        S = hd // c["rope_sections"]
        parts = []
        for s in range(c["rope_sections"]):
            zz = z[..., s * S:(s + 1) * S]
            cs, sn = cos[s][:, None, :], sin[s][:, None, :]
            a, b = zz[..., :S // 2], zz[..., S // 2:]
            parts += [a * cs - b * sn, b * cs + a * sn]
        return r16(torch.cat(parts, -1).reshape(z.shape[0], nh * hd), "qk")

    q, k = qk(q, t["q_norm_w"], nq), qk(k, t["k_norm_w"], nkv)
    if c.get("v_norm"):
        v = r16(F.rms_norm(v.view(-1, nkv, hd), (hd,), None, eps).reshape(v.shape[0], nkv * hd),
                "qk")
    att = torch.zeros_like(q)
    W = t.get("window", c["window"])
    for rr in items:
        idx = torch.cat([torch.arange(r0, r0 + n) for r0, n in rr])
        L = len(idx)
        i = torch.arange(L)
        mask = (i[:, None] - i[None, :]).abs() <= W if W else torch.ones(L, L, dtype=torch.bool)
        qh = q[idx].view(L, nq, hd).transpose(0, 1)
        kh = k[idx].view(L, nkv, hd).transpose(0, 1).repeat_interleave(nq // nkv, 0)
        vh = v[idx].view(L, nkv, hd).transpose(0, 1).repeat_interleave(nq // nkv, 0)
        o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=c["attn_scale"])
        att[idx] = o.transpose(0, 1).reshape(L, nq * hd)
    att = r16(att, "att")
    H = H + F.rms_norm(lin(att, "wo"), (d,), T(t["post_attn_w"]), eps)
    A = r16(F.rms_norm(H, (d,), T(t["norm2_w"]), eps), "A2")
    g, u = lin(A, "w_gate"), lin(A, "w_up")
    act = F.gelu(g, approximate="tanh") if c["mlp"] == wl.MLP_GELU_GATED else F.silu(g)
    m = r16(act * u, "hidden")
    H = H + F.rms_norm(lin(m, "w_down"), (d,), T(t["post_ff_w"]), eps)
    if c.get("n_ple"):
        P = F.rms_norm(c["ple_scale"] * (T(x0) @ T(t["ple_in"]).T), (c["n_ple"],),
                       T(t["ple_in_norm_w"]), eps)
        Z = F.gelu(H @ T(t["ple_gate"]).T, approximate="tanh") * P
        H = H + F.rms_norm(Z @ T(t["ple_proj"]).T, (d,), T(t["ple_post_w"]), eps)
    return (H * t.get("scalar", 1.0)).numpy()


def _angles(pos, sections, hd, base):
    S = hd // sections
    i = np.arange(S // 2)
    cos, sin = [], []
    for s in range(sections):
        th = pos[:, s:s + 1].astype(np.float64) * base ** (-2.0 * i / S)
        cos.append(torch.from_numpy(np.cos(th)))
        sin.append(torch.from_numpy(np.sin(th)))
    return cos, sin


@pytest.mark.parametrize("name,kw", [
    ("gemma_text_f32", dict(lengths=[9, 30, 4], overrides=dict(window=6))),
    ("zimage_dit_1056", dict(grid=3, ncap=4, cfg_pair=True,
                             overrides=dict(d=256, nq=2, nkv=2, ff=384))),
    # the vision tower: several images (3x3, 4x4, 2x2 grids), 2-D RoPE, no captions
    ("gemma_vision_f32", dict(lengths=[3, 4, 2], overrides=dict(d=128, nq=2, nkv=2, ff=256))),
])
def test_sandwich_layer_matches_torch_composition(oracle, name, kw):
    w = wl.make(name, layers=1, **kw)
    w.cfg["final"] = wl.FINAL_NONE
    c = w.cfg
    pos = oracle.positions(w.rows, w.items, w.grids, c["rope_sections"])
    ang = _angles(pos, c["rope_sections"], c["hd"], c["rope_base"])
    f16 = c["path"] == wl.PATH_I8F16
    ref = _torch_sandwich_layer(c, w.layers[0], w.x, ang, w.items, f16)
    out = oracle.forward(w)
    err = lambda a: np.abs(out - a).max() / np.abs(a).max()
    # both sides round the same f64 values to half at the same six sites; where
    # the two summation orders put a value on either side of a half rounding
    # point (one row of the DiT case) the result moves by ~1e-8
    assert err(ref) < (1e-6 if f16 else 1e-12)
    if f16:
        # each site matters: leaving any one out moves the result by > 1e-4
        for site in F16_SITES:
            alt = _torch_sandwich_layer(c, w.layers[0], w.x, ang, w.items, True, skip=(site,))
            assert err(alt) > 1e-5, site
        out64 = oracle.forward(w, f16_sites=False)
        ref64 = _torch_sandwich_layer(c, w.layers[0], w.x, ang, w.items, False)
        assert np.abs(out64 - ref64).max() / np.abs(ref64).max() < 1e-12


def test_text_encoder_options_match_torch_composition(oracle):
    """GQA (8 q / 2 kv heads), v-norm, a windowed then a global layer with their
    own RoPE bases, layer scalars and the per-layer input, two layers deep."""
    w = wl.make("gemma_text_ple_f32", layers=2, lengths=[9, 30, 4],
                overrides=dict(window=6, global_every=2, n_ple=64))
    w.cfg["final"] = wl.FINAL_NONE
    c = w.cfg
    assert [t["window"] for t in w.layers] == [6, 0]
    assert w.layers[0]["rope_base"] != w.layers[1]["rope_base"]
    pos = oracle.positions(w.rows, w.items, w.grids, 1)
    H = w.x
    for t in w.layers:
        H = _torch_sandwich_layer(c, t, H, _angles(pos, 1, c["hd"], t["rope_base"]), w.items,
                                  False, x0=w.x)
    out = oracle.forward(w)
    assert np.abs(out - H).max() / np.abs(H).max() < 1e-12
    # each option changes the result (none of them is silently dropped)
    for key, val in (("v_norm", False), ("n_ple", 0)):
        ov = dict(window=6, global_every=2, n_ple=64)
        ov[key] = val
        w2 = wl.make("gemma_text_ple_f32", layers=2, lengths=[9, 30, 4], overrides=ov)
        w2.cfg["final"] = wl.FINAL_NONE
        assert np.abs(oracle.forward(w2) - out).max() > 1e-3 * np.abs(out).max(), key


DIT_MOD_SMALL = dict(layers=1, grid=3, ncap=4, overrides=dict(d=256, nq=2, nkv=2, ff=384))


def _dit_mod(**kw):
    args = dict(DIT_MOD_SMALL)
    args.update(kw)
    w = wl.make("zimage_dit_mod_1056", **args)
    w.cfg["final"] = wl.FINAL_NONE
    return w


def _torch_dit_mod_layer(c, t, x, pos_cos_sin, items):
    """The modulated int8 block in exact arithmetic (torch f64), with the column
    fields folded into the weights, W_eff = diag(rs) q diag(col), and no guards
    (they cancel exactly): an independent form of what the half-site chain
    computes when nothing is rounded; also returns each site's max |value|
    (as stored, after the column field and the guard)."""
    F = torch.nn.functional
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    eps, hd, nq = c["eps"], c["hd"], c["nq"]
    ga, gq, gao, gf, gh = c["guards"]
    H = T(x)
    d = H.shape[1]
    W = lambda n: (T(t["s" + n[1:]])[:, None] * T(t[n].astype(np.float64))
                   * T(t["col_" + n[1:].lstrip("_")])[None, :])
    amax = np.zeros(5)
    def site(i, v, colname, g):
        amax[i] = max(amax[i], float((v * T(t[colname]) * 2.0 ** -g).abs().max()) if colname
                      else float((v * 2.0 ** -g).abs().max()))
    A = F.rms_norm(H, (d,), T(t["norm1_w"]), eps) * (1 + T(t["mod_s_attn"]))
    for n in ("col_q", "col_k", "col_v"):
        site(0, A, n, ga)
    q, k, v = A @ W("wq").T, A @ W("wk").T, A @ W("wv").T
    for z in (q, k, v):
        site(1, z, None, gq)
    cos, sin = pos_cos_sin

    def qk(z, wn):
        z = F.rms_norm(z.view(z.shape[0], nq, hd), (hd,), T(wn), eps)
        S = hd // 2
        parts = []
        for s_ in range(2):
            zz = z[..., s_ * S:(s_ + 1) * S]
            cs, sn = cos[s_][:, None, :], sin[s_][:, None, :]
            a, b = zz[..., :S // 2], zz[..., S // 2:]
            parts += [a * cs - b * sn, b * cs + a * sn]
        return torch.cat(parts, -1).reshape(z.shape[0], nq * hd)

    q, k = qk(q, t["q_norm_w"]), qk(k, t["k_norm_w"])
    att = torch.zeros_like(q)
    for rr in items:
        idx = torch.cat([torch.arange(r0, r0 + n) for r0, n in rr])
        L = len(idx)
        qh, kh, vh = (z[idx].view(L, nq, hd).transpose(0, 1) for z in (q, k, v))
        att[idx] = F.scaled_dot_product_attention(qh, kh, vh, scale=c["attn_scale"]).transpose(0, 1).reshape(L, nq * hd)
    site(2, att, "col_o", gao)
    H = H + T(t["mod_g_attn"]) * F.rms_norm(att @ W("wo").T, (d,), T(t["post_attn_w"]), eps)
    A = F.rms_norm(H, (d,), T(t["norm2_w"]), eps) * (1 + T(t["mod_s_ff"]))
    for n in ("col_gate", "col_up"):
        site(3, A, n, gf)
    m = F.silu(A @ W("w_gate").T) * (A @ W("w_up").T)
    site(4, m, "col_down", gh)
    H = H + T(t["mod_g_ff"]) * F.rms_norm(m @ W("w_down").T, (d,), T(t["post_ff_w"]), eps)
    return H.numpy(), amax


def test_dit_modulated_layer_matches_torch_composition(oracle):
    """adaLN modulation, q8_2f column fields and guards: the oracle's half-site
    chain without rounding equals the folded-weight form in exact arithmetic,
    and so do its per-site maxima."""
    w = _dit_mod()
    c = w.cfg
    pos = oracle.positions(w.rows, w.items, w.grids, 2)
    ref, ref_amax = _torch_dit_mod_layer(c, w.layers[0], w.x, _angles(pos, 2, c["hd"], c["rope_base"]),
                                         w.items)
    amax = np.zeros((1, 5))
    out = oracle.forward(w, f16_sites=False, amax=amax)
    assert np.abs(out - ref).max() / np.abs(ref).max() < 1e-12
    assert np.allclose(amax[0], ref_amax, rtol=1e-12)
    # with the f16 sites: within the int8 path's tolerance of the exact result
    out16 = oracle.forward(w)
    assert np.abs(out16 - ref).max() / np.abs(ref).max() < 3e-3


def test_guards_cancel_exactly_without_rounding(oracle):
    """A guard multiplies by 2^-s at a half site and 2^s at its consumer, and
    the qk-norm's eps is scaled by 2^-2s: in f64 these are exact, so without
    the f16 rounding every guard set gives the same bits."""
    outs = []
    for g in ([0, 0, 0, 0, 0], [0, 1, 0, 0, 6], [6, 8, 6, 6, 11]):
        w = _dit_mod(layers=2, overrides=dict(DIT_MOD_SMALL["overrides"], guards=g))
        outs.append(oracle.forward(w, f16_sites=False))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_guard_keeps_the_hidden_in_half_range(oracle):
    """Up/gate row scales raised until the SwiGLU hidden passes 65504: the
    stored half overflows to infinity without a guard; with the hidden guard
    (2^-6) it stays finite and within the int8 tolerance of the exact result."""
    res = {}
    for gh in (0, 6):
        w = _dit_mod(overrides=dict(DIT_MOD_SMALL["overrides"], guards=[0, 1, 0, 0, gh]))
        for n in ("s_gate", "s_up"):
            w.layers[0][n] = w.layers[0][n] * np.float32(150.0)
        amax = np.zeros((1, 5))
        res[gh] = (oracle.forward(w, amax=amax), amax[0, 4], oracle.forward(w, f16_sites=False))
    out0, am0, exact = res[0]
    out6, am6, _ = res[6]
    assert not np.isfinite(out0).all() and am0 == np.inf
    assert np.isfinite(out6).all() and 65504 / 64 < am6 <= 65504
    assert np.abs(out6 - exact).max() / np.abs(exact).max() < 3e-3


def test_unit_modulation_is_unmodulated(oracle):
    """s = 0, g = 1 (the context refiner's form) gives the unmodulated bits."""
    w = _dit_mod(layers=2)
    for t in w.layers:
        for n in ("mod_s_attn", "mod_s_ff"):
            t[n] = np.zeros_like(t[n])
        for n in ("mod_g_attn", "mod_g_ff"):
            t[n] = np.ones_like(t[n])
    a = oracle.forward(w)
    for t in w.layers:
        for n in ("mod_s_attn", "mod_s_ff", "mod_g_attn", "mod_g_ff"):
            del t[n]
    assert np.array_equal(a, oracle.forward(w))


def test_refiner_program_stages(oracle):
    """The staged DiT program: the noise refiner's rows carry their own grid
    positions (the joint table's image slice), the two refiners touch disjoint
    rows so their order does not change a bit, a program of the main stage
    alone is the plain forward, and the refiners do act."""
    w = wl.make("zimage_dit_step_1056", layers=1, grid=3, ncap=4, cfg_pair=True,
                overrides=dict(d=256, nq=2, nkv=2, ff=384))
    joint = oracle.positions(w.rows, w.items, w.grids, 2)
    stages = [(st, r0, joint[r0:r0 + st.rows]) for _, st, r0 in w.stages]
    assert [lab for lab, _, _ in w.stages] == ["context refiner", "noise refiner", "main"]
    nr = w.stages[1][1]
    assert np.array_equal(joint[:nr.rows], oracle.positions(nr.rows, nr.items, nr.grids, 2))
    out = oracle.forward_stages(stages, w.x)
    assert np.array_equal(oracle.forward_stages([stages[1], stages[0], stages[2]], w.x), out)
    main_only = oracle.forward_stages([stages[2]], w.x)
    assert np.array_equal(main_only, oracle.forward(w))
    assert np.abs(main_only - out).max() > 1e-2 * np.abs(out).max()


def test_packed_equals_separate_forward(oracle):
    w = wl.make("gemma_text_f32", layers=2, lengths=[7, 12, 3], overrides=dict(window=4))
    out = oracle.forward(w)
    r = 0
    for i, n in enumerate([7, 12, 3]):
        ws = wl.make("gemma_text_f32", layers=2, lengths=[n], overrides=dict(window=4))
        ws.x = w.x[r:r + n].copy()
        alone = oracle.forward(ws)
        assert np.array_equal(out[i], alone[0])
        r += n


def test_cfg_pair_equals_two_singles(oracle):
    kw = dict(layers=1, grid=2, ncap=3, overrides=dict(d=256, nq=2, nkv=2, ff=256))
    w = wl.make("zimage_dit_cfg_8448", cfg_pair=True, **kw)
    out = oracle.forward(w)
    for i, rr in enumerate(w.items):
        idx = np.concatenate([np.arange(r0, r0 + n) for r0, n in rr])
        ws = wl.make("zimage_dit_cfg_8448", cfg_pair=False, **kw)
        ws.x = w.x[idx].copy()
        alone = oracle.forward(ws)
        assert np.array_equal(out[idx], alone)


def test_meanpool_of_identical_rows(oracle):
    w = wl.make("gemma_text_f32", layers=0, lengths=[4, 2])
    w.x[:4] = w.x[0]
    w.x[4:] = w.x[4]
    out = oracle.forward(w)
    d = w.cfg["d"]
    assert np.allclose(out[0], oracle.rms_norm(w.x[:1], w.final_w, 1e-6)[0], rtol=1e-15)
    assert np.allclose(out[1], oracle.rms_norm(w.x[4:5], w.final_w, 1e-6)[0], rtol=1e-15)
    assert out.shape == (2, d)


class _Tiny:
    """A workload-like object with no layers: only the final stage acts."""

    def __init__(self, rows, items, w, b=None, final=wl.FINAL_RMS_MEANPOOL, eps=0.0):
        x = np.asarray(rows, np.float32)
        self.cfg = dict(d=x.shape[1], final=final, eps=eps)
        self.rows, self.items, self.grids = x.shape[0], items, [0] * len(items)
        self.x, self.layers = x, []
        self.final_w = np.asarray(w, np.float32)
        self.final_b = None if b is None else np.asarray(b, np.float32)


def test_final_rms_then_pool_hand_values(oracle):
    """The text encoder's output: each row RMS-normed with the final weight, then the
    mean over the item's rows (two-range items, unequal lengths).  Norming the pooled
    mean instead gives other values (tests/golden/final_stage.json)."""
    g = _gold("final_stage.json")["rms_then_pool"]
    items = [[tuple(r) for r in it] for it in g["items"]]
    out = oracle.forward(_Tiny(g["rows"], items, g["w"]), layers=0)
    assert np.allclose(out, np.asarray(g["out"]), rtol=0, atol=1e-15)


def test_final_rms_then_pool_matches_torch_f64(oracle):
    """Random rows and items of unequal length: torch rms_norm per row, then the mean."""
    rng = np.random.default_rng(11)
    lens = [3, 17, 1, 40]
    rows = rng.standard_normal((sum(lens), 24)).astype(np.float32) * 3
    w = (1 + 0.1 * rng.standard_normal(24)).astype(np.float32)
    items, r = [], 0
    for n in lens:
        items.append([(r, n)])
        r += n
    out = oracle.forward(_Tiny(rows, items, w, eps=1e-6), layers=0)
    R = torch.nn.functional.rms_norm(torch.from_numpy(rows.astype(np.float64)), (24,),
                                     torch.from_numpy(w.astype(np.float64)), 1e-6)
    ref = np.stack([R[r0:r0 + n].mean(0).numpy() for (r0, n), in items])
    assert np.abs(out - ref).max() < 1e-14


def test_post_ln_stack_matches_torch_encoder(oracle):
    """Two pre-LN layers and the final LayerNorm == torch.nn.TransformerEncoder with
    norm=LayerNorm in f64 (the ViT's post-LN after the blocks)."""
    w = wl.make("lfm2_vit_f32", layers=2, lengths=[40],
                overrides=dict(d=128, nq=2, nkv=2, ff=256))
    c = w.cfg
    d = c["d"]
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    proto = torch.nn.TransformerEncoderLayer(
        d, c["nq"], dim_feedforward=c["ff"], dropout=0.0,
        activation=lambda x: torch.nn.functional.gelu(x, approximate="tanh"),
        layer_norm_eps=c["eps"], batch_first=True, norm_first=True, dtype=torch.float64)
    norm = torch.nn.LayerNorm(d, eps=c["eps"], dtype=torch.float64)
    enc = torch.nn.TransformerEncoder(proto, 2, norm=norm, enable_nested_tensor=False)
    with torch.no_grad():
        for layer, t in zip(enc.layers, w.layers):
            layer.self_attn.in_proj_weight.copy_(T(np.concatenate([t["wq"], t["wk"], t["wv"]])))
            layer.self_attn.in_proj_bias.copy_(T(np.concatenate([t["bq"], t["bk"], t["bv"]])))
            layer.self_attn.out_proj.weight.copy_(T(t["wo"]))
            layer.self_attn.out_proj.bias.copy_(T(t["bo"]))
            layer.linear1.weight.copy_(T(t["w_up"]))
            layer.linear1.bias.copy_(T(t["b_up"]))
            layer.linear2.weight.copy_(T(t["w_down"]))
            layer.linear2.bias.copy_(T(t["b_down"]))
            layer.norm1.weight.copy_(T(t["norm1_w"]))
            layer.norm1.bias.copy_(T(t["norm1_b"]))
            layer.norm2.weight.copy_(T(t["norm2_w"]))
            layer.norm2.bias.copy_(T(t["norm2_b"]))
        enc.norm.weight.copy_(T(w.final_w))
        enc.norm.bias.copy_(T(w.final_b))
        ref = enc(T(w.x)[None])[0].numpy()
    out = oracle.forward(w)
    assert np.abs(out - ref).max() / np.abs(ref).max() < 1e-13
    # the final LN acts: without it the rows are not normalised
    bare = dict(w.cfg, final=wl.FINAL_NONE)
    w.cfg = bare
    assert np.abs(oracle.forward(w) - out).max() > 1e-3


def test_padded_pair_equals_singles_and_pads_attend(oracle):
    """Padded items (image and caption ranges padded to 32 with pad rows) are
    ordinary rows of their item: the CFG pair still equals two singles bit for
    bit, and a pad row is a key the real rows attend to (changing the pad row
    changes them) while leaving the other item alone."""
    from positions_ref import dit_positions
    kw = dict(layers=1, grid=3, ncap=2, overrides=dict(d=128, nq=2, nkv=2, ff=256))
    w = wl.make("zimage_dit_pad_cfg", **kw)
    assert w.items == [[(0, 32), (64, 32)], [(32, 32), (96, 32)]]
    pos = dit_positions(w.rows, w.items, w.grids)
    pair = oracle.forward(w, pos=pos)
    for rr in w.items:
        idx = np.concatenate([np.arange(r0, r0 + n) for r0, n in rr])
        single = wl.make("zimage_dit_pad_cfg", cfg_pair=False, **kw)
        spos = dit_positions(single.rows, single.items, single.grids)
        assert np.array_equal(oracle.forward(single, x=w.x[idx], pos=spos), pair[idx])
    x2 = w.x.copy()
    x2[20:32] += 1.0  # item 0's image pad rows
    moved = oracle.forward(w, x=x2, pos=pos)
    assert np.abs(moved[:9] - pair[:9]).max() > 1e-6  # item 0's image rows
    assert np.array_equal(moved[32:64], pair[32:64]) and np.array_equal(moved[96:], pair[96:])


def test_nonfinite_input_propagates(oracle):
    w = wl.make("gemma_text_f32", layers=1, lengths=[5, 6])
    w.cfg["final"] = wl.FINAL_NONE
    w.x[2, 7] = np.inf
    out = oracle.forward(w)
    assert not np.isfinite(out[:5]).all()
    assert np.isfinite(out[5:]).all()


def test_attention_query_subset_equals_full(oracle):
    """The query-row-subset entry returns the full attention's bits on the chosen
    rows and leaves every other row untouched (it is the same computation)."""
    rng = np.random.default_rng(10)
    hd, nq, nkv, rows = 16, 4, 2, 30
    q = rng.normal(0, 1, (rows, nq * hd))
    k = rng.normal(0, 1, (rows, nkv * hd))
    v = rng.normal(0, 1, (rows, nkv * hd))
    items = [[(0, 10), (25, 5)], [(10, 15)]]
    for window in (0, 3):
        full = oracle.attention(items, q, k, v, nq, nkv, hd, 0.4, window)
        sel = [0, 9, 11, 24, 27]
        part = oracle.attention(items, q, k, v, nq, nkv, hd, 0.4, window, query_rows=sel)
        assert np.array_equal(part[sel], full[sel])
        rest = np.setdiff1d(np.arange(rows), sel)
        assert not part[rest].any()
