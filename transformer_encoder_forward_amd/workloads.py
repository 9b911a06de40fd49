"""Synthetic workloads of the packed encoder forward: shapes, items and seeded tensors.

Nine workloads, each the shape of one of the encoders on the reference pages,
with random weights (no trained checkpoint is available):

  vit_layer_f32        one pre-LN ViT layer: 64 tokens, d 128, 2x64 heads, MLP 512
  gemma_text_f32       EmbeddingGemma-style text encoder: 24 sandwich layers, d 512,
                       8x64 heads, qk-norm + 1-D RoPE, window 512, gated GELU 2048,
                       16 packed sequences of 32..2048 rows, final RMS + mean pool
  lfm2_vit_f32         LFM2-VL-style ViT: 16 pre-LN layers, 1024 patches, d 768,
                       12x64 heads, MLP 3072, final LayerNorm
  zimage_dit_1056      Z-Image-style DiT stack: 30 sandwich layers, d 3840, 30x128
                       heads, int8 row-scaled weights x f16 activations, qk-norm +
                       2-D RoPE over a 32x32 grid + 32 caption rows, SwiGLU 10240
  zimage_dit_cfg_8448  the same stack at a 64x64 grid + 128 caption rows as a CFG
                       batch-2 program: rows [img0|img1|cap0|cap1]
  gemma_text_ple_f32   the text encoder's full layer spec on the gemma_text_f32 batch:
                       8 q / 2 kv heads, v-norm, 5 windowed : 1 global layers with
                       RoPE bases 1e4 / 1e6, layer scalars, per-layer input (256 wide)
  zimage_dit_mod_1056  zimage_dit_1056 with adaLN modulation, q8_2f column fields and
                       the Turbo power-of-two guards of the five half sites
  zimage_dit_step_1056 zimage_dit_mod_1056 as the page's staged program: context
                       refiner (2 unmodulated blocks, caption rows), noise refiner
                       (2 blocks, image rows), then the 30-block stack
  gemma_vision_f32     the text model's vision tower: 16 sandwich layers, d 768, 12x64
                       heads, qk-norm + 2-D RoPE, gated GELU 3072, five images of
                       32x32, 24x24, 16x16, 16x16 and 8x8 patches packed back to back

Only draws and shapes live here; the forward itself is computed by the HIP
library (and, independently, by the oracle).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from . import synth

MASTER_SEED = 0xE1C0DE00

BLOCK_PRE_LN, BLOCK_SANDWICH = 0, 1
PATH_F32, PATH_I8F16 = 0, 1
MLP_GELU, MLP_GELU_GATED, MLP_SWIGLU = 0, 1, 2
FINAL_NONE, FINAL_LN, FINAL_RMS_MEANPOOL = 0, 1, 2

CONFIGS = {
    "vit_layer_f32": dict(
        num=1, block=BLOCK_PRE_LN, path=PATH_F32, mlp=MLP_GELU, d=128, nq=2, nkv=2, hd=64,
        ff=512, layers=1, window=0, rope_sections=0, final=FINAL_NONE, eps=1e-6,
        attn_scale=1.0 / 8.0, rope_base=10000.0, x_scale=1.0, biases=True,
        lengths=[64]),
    "gemma_text_f32": dict(
        num=2, block=BLOCK_SANDWICH, path=PATH_F32, mlp=MLP_GELU_GATED, d=512, nq=8, nkv=8,
        hd=64, ff=2048, layers=24, window=512, rope_sections=1, final=FINAL_RMS_MEANPOOL,
        eps=1e-6, attn_scale=1.0, rope_base=10000.0, x_scale=math.sqrt(512.0), biases=False,
        nseq=16, len_lo=32, len_hi=2048),
    # the same packed batch (lengths drawn from the stream of workload 2) through
    # the full option set of the text encoder's layer spec: GQA, v-norm, a
    # sliding/global window pattern with one RoPE table per kind, layer scalars
    # and the per-layer-input branch
    "gemma_text_ple_f32": dict(
        num=6, block=BLOCK_SANDWICH, path=PATH_F32, mlp=MLP_GELU_GATED, d=512, nq=8, nkv=2,
        hd=64, ff=2048, layers=24, window=512, global_every=6, rope_sections=1,
        final=FINAL_RMS_MEANPOOL, eps=1e-6, attn_scale=1.0, rope_base=10000.0,
        rope_base_global=1000000.0, x_scale=math.sqrt(512.0), biases=False, nseq=16, len_lo=32,
        len_hi=2048, len_stream=2, v_norm=True, layer_scalar=True, n_ple=256,
        ple_scale=1.0 / math.sqrt(2.0)),
    "lfm2_vit_f32": dict(
        num=3, block=BLOCK_PRE_LN, path=PATH_F32, mlp=MLP_GELU, d=768, nq=12, nkv=12, hd=64,
        ff=3072, layers=16, window=0, rope_sections=0, final=FINAL_LN, eps=1e-6,
        attn_scale=1.0 / 8.0, rope_base=10000.0, x_scale=1.0, biases=True,
        lengths=[1024]),
    # the text model's vision tower: sandwich RMS blocks, qk-norm + 2-D RoPE
    # (column half, row half) over several images packed back to back, hd-64
    # flash per image with scale 1, gated GELU; H out (no final norm).  The
    # q/k norm gains are drawn around hd^-1/4 (they carry the softmax
    # temperature at scale 1): with gains near 1 the logits have a standard
    # deviation of 8, attention is nearly one-hot and 16 random layers amplify
    # f32 rounding several thousand times
    "gemma_vision_f32": dict(
        num=7, block=BLOCK_SANDWICH, path=PATH_F32, mlp=MLP_GELU_GATED, d=768, nq=12, nkv=12,
        hd=64, ff=3072, layers=16, window=0, rope_sections=2, final=FINAL_NONE, eps=1e-6,
        attn_scale=1.0, rope_base=10000.0, x_scale=1.0, biases=False,
        image_grids=[32, 24, 16, 16, 8], qk_gain=64 ** -0.25),
    "zimage_dit_1056": dict(
        num=4, block=BLOCK_SANDWICH, path=PATH_I8F16, mlp=MLP_SWIGLU, d=3840, nq=30, nkv=30,
        hd=128, ff=10240, layers=30, window=0, rope_sections=2, final=FINAL_NONE, eps=1e-6,
        attn_scale=1.0 / math.sqrt(128.0), rope_base=10000.0, x_scale=1.0, biases=False,
        grid=32, ncap=32, cfg_pair=False),
    # the 1056-row DiT stack with the rest of the int8 block's row-op contract:
    # adaLN modulation per layer, q8_2f column fields folded into the half
    # producers, and the power-of-two guards of the five half sites (the
    # pages' Turbo set: q/k/v input 0, panel 1, attention out 0, FFN input 0,
    # hidden 6)
    "zimage_dit_mod_1056": dict(
        num=8, block=BLOCK_SANDWICH, path=PATH_I8F16, mlp=MLP_SWIGLU, d=3840, nq=30, nkv=30,
        hd=128, ff=10240, layers=30, window=0, rope_sections=2, final=FINAL_NONE, eps=1e-6,
        attn_scale=1.0 / math.sqrt(128.0), rope_base=10000.0, x_scale=1.0, biases=False,
        grid=32, ncap=32, cfg_pair=False, modulated=True, col_fields=True,
        guards=[0, 1, 0, 0, 6]),
    # one DiT step of the 1056-row program with its refiner stages: two noise
    # refiner blocks on the image rows, then the 30-block stack (both modulated);
    # before them, once per prompt, two unmodulated context refiner blocks on
    # the caption rows
    "zimage_dit_step_1056": dict(
        num=9, block=BLOCK_SANDWICH, path=PATH_I8F16, mlp=MLP_SWIGLU, d=3840, nq=30, nkv=30,
        hd=128, ff=10240, layers=30, window=0, rope_sections=2, final=FINAL_NONE, eps=1e-6,
        attn_scale=1.0 / math.sqrt(128.0), rope_base=10000.0, x_scale=1.0, biases=False,
        grid=32, ncap=32, cfg_pair=False, modulated=True, col_fields=True,
        guards=[0, 1, 0, 0, 6], noise_refiner=2, context_refiner=2),
    # the CFG pair with the page's padded lengths: a 30x30 image (900 rows) and
    # 20 caption rows per item, each range padded to a multiple of 32 (928 and
    # 32 rows) with one learned pad row (image) and one caption pad row
    "zimage_dit_pad_cfg": dict(
        num=10, block=BLOCK_SANDWICH, path=PATH_I8F16, mlp=MLP_SWIGLU, d=3840, nq=30, nkv=30,
        hd=128, ff=10240, layers=30, window=0, rope_sections=2, final=FINAL_NONE, eps=1e-6,
        attn_scale=1.0 / math.sqrt(128.0), rope_base=10000.0, x_scale=1.0, biases=False,
        grid=30, ncap=20, cfg_pair=True, pad_to=32),
    "zimage_dit_cfg_8448": dict(
        num=5, block=BLOCK_SANDWICH, path=PATH_I8F16, mlp=MLP_SWIGLU, d=3840, nq=30, nkv=30,
        hd=128, ff=10240, layers=30, window=0, rope_sections=2, final=FINAL_NONE, eps=1e-6,
        attn_scale=1.0 / math.sqrt(128.0), rope_base=10000.0, x_scale=1.0, biases=False,
        grid=64, ncap=128, cfg_pair=True),
}


@dataclass
class Workload:
    """One packed batch and its model, as host arrays.

    items: per item, a list of (first row, row count) ranges (one or two);
    grids: per item the image grid side G for 2-D positions, else 0.
    layers[i]: tensor name -> array (float32 weights/norms/biases, or int8
    weights with float32 row scales s_* on the int8 path); int8 weights may be
    absent (lazy) and are then drawn by `int8_weight` on demand.
    """
    name: str
    cfg: dict
    rows: int
    items: list
    grids: list
    x: np.ndarray
    layers: list = field(default_factory=list)
    final_w: np.ndarray | None = None
    final_b: np.ndarray | None = None
    seed: int = 0
    prefix: str = "L"   # tensor-name prefix of the layers' draws
    # a staged program: (label, stage workload over rows [row0, row0 + rows),
    # row0); the stage's items are relative to row0
    stages: list = field(default_factory=list)

    @property
    def ld(self):
        c = self.cfg
        return (c["nq"] + 2 * c["nkv"]) * c["hd"]


def weight_shapes(cfg: dict) -> dict:
    d, q, kv, ff = cfg["d"], cfg["nq"] * cfg["hd"], cfg["nkv"] * cfg["hd"], cfg["ff"]
    s = {"wq": (q, d), "wk": (kv, d), "wv": (kv, d), "wo": (d, q),
         "w_up": (ff, d), "w_down": (d, ff)}
    if cfg["mlp"] != MLP_GELU:
        s["w_gate"] = (ff, d)
    return s


def _normal(seed, name, shape, std, mean=0.0):
    n = int(np.prod(shape))
    z = synth.normal_np(synth.tensor_key(seed, name), 0, n)
    return (mean + std * z).astype(np.float32).reshape(shape)


def int8_weight_rows(seed: int, layer: int, name: str, shape, r0: int, r1: int,
                     prefix: str = "L") -> np.ndarray:
    """Rows r0..r1-1 of an int8 weight (host draw of just those rows)."""
    k = synth.tensor_key(seed, f"{prefix}{layer}.{name}")
    cols = shape[1]
    return synth.int8_np(k, r0 * cols, (r1 - r0) * cols).reshape(r1 - r0, cols)


def int8_weight_torch(seed: int, layer: int, name: str, shape, device, prefix: str = "L"):
    k = synth.tensor_key(seed, f"{prefix}{layer}.{name}")
    return synth.int8_torch(k, 0, shape[0] * shape[1], device).view(shape[0], shape[1])


def _layer(cfg: dict, seed: int, li: int, lazy_int8: bool, prefix: str = "L") -> dict:
    t = {}
    d, hd = cfg["d"], cfg["hd"]
    for name, shape in weight_shapes(cfg).items():
        if cfg["path"] == PATH_F32:
            t[name] = _normal(seed, f"{prefix}{li}.{name}", shape, 0.02)
        else:
            if not lazy_int8:
                t[name] = int8_weight_rows(seed, li, name, shape, 0, shape[0], prefix)
            sname = "s" + name[1:]
            z = synth.normal_np(synth.tensor_key(seed, f"{prefix}{li}.{sname}"), 0, shape[0])
            t[sname] = (0.002 * np.exp(0.25 * z)).astype(np.float32)
    if cfg["biases"]:
        for name, width in (("bq", cfg["nq"] * hd), ("bk", cfg["nkv"] * hd),
                            ("bv", cfg["nkv"] * hd), ("bo", d), ("b_up", cfg["ff"]),
                            ("b_down", d)):
            t[name] = _normal(seed, f"{prefix}{li}.{name}", (width,), 0.01)
    if cfg["block"] == BLOCK_PRE_LN:
        for name in ("norm1_w", "norm2_w"):
            t[name] = _normal(seed, f"{prefix}{li}.{name}", (d,), 0.02, 1.0)
        for name in ("norm1_b", "norm2_b"):
            t[name] = _normal(seed, f"{prefix}{li}.{name}", (d,), 0.01)
    else:
        for name in ("norm1_w", "post_attn_w", "norm2_w", "post_ff_w"):
            t[name] = _normal(seed, f"{prefix}{li}.{name}", (d,), 0.02, 1.0)
        for name in ("q_norm_w", "k_norm_w"):
            g = cfg.get("qk_gain", 1.0)
            t[name] = _normal(seed, f"{prefix}{li}.{name}", (hd,), 0.02 * g, g)
    # per-layer values: every global_every-th layer attends globally (window 0)
    # with its own RoPE base; the rest keep the config's window and base
    ge = cfg.get("global_every", 0)
    if ge and (li + 1) % ge == 0:
        t["window"] = 0
        t["rope_base"] = cfg["rope_base_global"]
    else:
        t["window"] = cfg["window"]
        t["rope_base"] = cfg["rope_base"]
    if cfg.get("modulated"):
        # [s_msa | g_msa | s_mlp | g_mlp]: scales near 0, gates near 1
        for name, mean in (("mod_s_attn", 0.0), ("mod_g_attn", 1.0), ("mod_s_ff", 0.0),
                           ("mod_g_ff", 1.0)):
            t[name] = _normal(seed, f"{prefix}{li}.{name}", (d,), 0.1, mean)
    if cfg.get("col_fields"):
        # q8_2f column fields: positive, lognormal around 1, one per input column
        q = cfg["nq"] * hd
        for name, width in (("col_q", d), ("col_k", d), ("col_v", d), ("col_o", q),
                            ("col_gate", d), ("col_up", d), ("col_down", cfg["ff"])):
            z = synth.normal_np(synth.tensor_key(seed, f"{prefix}{li}.{name}"), 0, width)
            t[name] = np.exp(0.25 * z).astype(np.float32)
    if cfg.get("layer_scalar"):
        t["scalar"] = float(1.0 + 0.05 * synth.normal_np(synth.tensor_key(seed, f"{prefix}{li}.scalar"), 0, 1)[0])
    if cfg.get("n_ple"):
        np_ = cfg["n_ple"]
        t["ple_in"] = _normal(seed, f"{prefix}{li}.ple_in", (np_, d), 0.02)
        t["ple_gate"] = _normal(seed, f"{prefix}{li}.ple_gate", (np_, d), 0.02)
        t["ple_proj"] = _normal(seed, f"{prefix}{li}.ple_proj", (d, np_), 0.02)
        t["ple_in_norm_w"] = _normal(seed, "ple_in_norm_w", (np_,), 0.02, 1.0)  # model-wide
        t["ple_post_w"] = _normal(seed, f"{prefix}{li}.ple_post_w", (d,), 0.02, 1.0)
    return t


def layout(cfg: dict, lengths=None, grid=None, ncap=None, cfg_pair=None):
    """(rows, items, grids) of a workload.

    Images (2-D, no captions): one single-range item of G*G rows per grid side
    in `image_grids` (or `lengths` read as grid sides), back to back.
    Sequences (1-D): `lengths` back to back, one single-range item each.
    DiT (2-D): one item = G*G image rows + ncap caption rows; the CFG pair is two
    items over rows [img0 | img1 | cap0 | cap1], each item = its image range then
    its caption range.
    """
    if cfg["rope_sections"] == 2 and "image_grids" in cfg:
        sides = cfg["image_grids"] if lengths is None else lengths
        items, r = [], 0
        for g in sides:
            items.append([(r, g * g)])
            r += g * g
        return r, items, [int(g) for g in sides]
    if cfg["rope_sections"] == 2:
        g = cfg["grid"] if grid is None else grid
        nc = cfg["ncap"] if ncap is None else ncap
        pair = cfg["cfg_pair"] if cfg_pair is None else cfg_pair
        ni = g * g
        pad = cfg.get("pad_to", 0)
        if pad:
            # each range padded to a multiple of `pad` rows
            ni, nc = -(-ni // pad) * pad, -(-nc // pad) * pad
        if not pair:
            return ni + nc, [[(0, ni), (ni, nc)] if nc else [(0, ni)]], [g]
        items = [[(0, ni), (2 * ni, nc)] if nc else [(0, ni)],
                 [(ni, ni), (2 * ni + nc, nc)] if nc else [(ni, ni)]]
        return 2 * ni + 2 * nc, items, [g, g]
    if lengths is None:
        if "lengths" in cfg:
            lengths = cfg["lengths"]
        else:
            k = synth.tensor_key(MASTER_SEED + cfg.get("len_stream", cfg["num"]), "lengths")
            lengths = [int(v) for v in synth.ints_np(k, cfg["nseq"], cfg["len_lo"], cfg["len_hi"])]
    items, r = [], 0
    for n in lengths:
        items.append([(r, int(n))])
        r += int(n)
    return r, items, [0] * len(items)


def make(name: str, layers=None, lengths=None, grid=None, ncap=None, cfg_pair=None,
         lazy_int8=False, overrides=None) -> Workload:
    """Build workload `name`, optionally reduced (fewer layers, other lengths/grid)."""
    cfg = dict(CONFIGS[name])
    if overrides:
        cfg.update(overrides)
    if layers is not None:
        cfg["layers"] = layers
    seed = MASTER_SEED + cfg["num"]
    rows, items, grids = layout(cfg, lengths, grid, ncap, cfg_pair)
    d = cfg["d"]
    if cfg["rope_sections"] == 2 and "image_grids" not in cfg:
        # image rows are one draw shared by every item (one latent, CFG pair);
        # each item's caption rows are its own draw
        x = np.empty((rows, d), np.float32)
        g = cfg["grid"] if grid is None else grid
        nc_real = cfg["ncap"] if ncap is None else ncap
        for i, rr in enumerate(items):
            (r0, ni) = rr[0]
            nimg = min(ni, g * g)
            x[r0:r0 + nimg] = _normal(seed, "x.img", (nimg, d), cfg["x_scale"])
            if ni > nimg:  # image padding: the learned pad row
                x[r0 + nimg:r0 + ni] = _normal(seed, "x.pad", (d,), cfg["x_scale"])
            if len(rr) > 1:
                (c0, nc) = rr[1]
                ncr = min(nc, nc_real)
                x[c0:c0 + ncr] = _normal(seed, f"x.cap{i}", (ncr, d), cfg["x_scale"])
                if nc > ncr:  # caption padding: the caption pad row
                    x[c0 + ncr:c0 + nc] = _normal(seed, "x.cap_pad", (d,), cfg["x_scale"])
    else:
        x = _normal(seed, "x", (rows, d), cfg["x_scale"])
    w = Workload(name=name, cfg=cfg, rows=rows, items=items, grids=grids, x=x, seed=seed)
    w.layers = [_layer(cfg, seed, li, lazy_int8) for li in range(cfg["layers"])]
    if cfg["final"] != FINAL_NONE:
        w.final_w = _normal(seed, "final_w", (d,), 0.02, 1.0)
        if cfg["final"] == FINAL_LN:
            w.final_b = _normal(seed, "final_b", (d,), 0.01)
    if cfg.get("noise_refiner") or cfg.get("context_refiner"):
        w.stages = _dit_stages(w, lazy_int8)
    return w


def _dit_stages(w: Workload, lazy_int8: bool) -> list:
    """The DiT step program with its refiners: the context refiner (its own
    unmodulated blocks) on each item's caption rows, the noise refiner (the
    first step blocks) on the image rows of every item, then the main stack on
    all rows.  Rows stay where the packed batch has them, so a refiner stage
    is a contiguous slice: [img0 | img1 | cap0 | cap1]."""
    cfg, seed = w.cfg, w.seed
    img = [rr[0] for rr in w.items]
    caps = [rr[1] for rr in w.items if len(rr) > 1]
    stages = []
    nc = cfg.get("context_refiner", 0)
    if nc and caps:
        ccfg = dict(cfg, layers=nc, modulated=False)
        r0 = caps[0][0]
        rows = sum(n for _, n in caps)
        sub = Workload(name=w.name + ".context_refiner", cfg=ccfg, rows=rows,
                       items=[[(c0 - r0, n)] for c0, n in caps], grids=[0] * len(caps),
                       x=w.x[r0:r0 + rows], seed=seed, prefix="CR")
        sub.layers = [_layer(ccfg, seed, li, lazy_int8, "CR") for li in range(nc)]
        stages.append(("context refiner", sub, r0))
    nn = cfg.get("noise_refiner", 0)
    if nn:
        ncfg = dict(cfg, layers=nn)
        rows = sum(n for _, n in img)
        sub = Workload(name=w.name + ".noise_refiner", cfg=ncfg, rows=rows, items=[[r] for r in img],
                       grids=list(w.grids), x=w.x[:rows], seed=seed, prefix="NR")
        sub.layers = [_layer(ncfg, seed, li, lazy_int8, "NR") for li in range(nn)]
        stages.append(("noise refiner", sub, 0))
    stages.append(("main", w, 0))
    return stages


def gemm_flops(w: Workload) -> float:
    """Algorithmic GEMM flops of the whole forward (2 per multiply-add)."""
    c = w.cfg
    d, q, kv, ff = c["d"], c["nq"] * c["hd"], c["nkv"] * c["hd"], c["ff"]
    per_row = d * (q + 2 * kv) + q * d + ff * d * (1 if c["mlp"] == MLP_GELU else 2) + ff * d
    per_row += 3 * c.get("n_ple", 0) * d  # per-layer input: ple_in, ple_gate, ple_proj
    return 2.0 * per_row * w.rows * c["layers"]


def layer_windows(w: Workload) -> list:
    return [int(t.get("window", w.cfg["window"])) for t in w.layers]


def visible_pairs(w: Workload, window=None) -> int:
    """Sum over items of the (query, key) pairs the attention mask lets through."""
    W = w.cfg["window"] if window is None else window
    tot = 0
    for rr in w.items:
        L = sum(n for _, n in rr)
        if W == 0 or W >= L - 1:
            tot += L * L
        else:
            i = np.arange(L)
            tot += int((np.minimum(i + W, L - 1) - np.maximum(i - W, 0) + 1).sum())
    return tot


def attn_flops(w: Workload) -> float:
    """Algorithmic attention flops: 4*hd per visible pair per head per layer."""
    c = w.cfg
    pairs = {W: visible_pairs(w, W) for W in set(layer_windows(w))}
    return 4.0 * c["hd"] * c["nq"] * sum(pairs[W] for W in layer_windows(w))
