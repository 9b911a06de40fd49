"""Device-resident model and batch for encoder_forward: marshalling only.

Weights are uploaded once as torch tensors on the device (PyTorch supplies the
memory); the C structs hold their addresses.  RoPE positions and tables come
from the library's host helpers (enc_positions, enc_rope_table).
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import binding as B
from . import workloads as wl

_F32_NAMES = ["bq", "bk", "bv", "bo", "b_up", "b_down", "norm1_w", "norm1_b", "norm2_w",
              "norm2_b", "post_attn_w", "post_ff_w", "q_norm_w", "k_norm_w",
              "sq", "sk", "sv", "so", "s_gate", "s_up", "s_down"]
_W_NAMES = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]
_PLE_NAMES = ["ple_in", "ple_gate", "ple_proj", "ple_in_norm_w", "ple_post_w"]
_MOD_COL_NAMES = ["mod_s_attn", "mod_g_attn", "mod_s_ff", "mod_g_ff",
                  "col_q", "col_k", "col_v", "col_o", "col_gate", "col_up", "col_down"]


def rope_bases(w: wl.Workload) -> list:
    """Distinct RoPE bases of the layers, in order of first use: table i of the
    batch holds base i."""
    bases = []
    for t in w.layers:
        b = float(t.get("rope_base", w.cfg["rope_base"]))
        if b not in bases:
            bases.append(b)
    assert len(bases) <= B.MAX_ROPE_TABLES
    return bases


class DeviceModel:
    def __init__(self, w: wl.Workload, device="cuda", layers=None):
        self.cfg = cfg = w.cfg
        self.keep = []
        nl = len(w.layers) if layers is None else layers
        self.nlayers = nl
        self.layers = (B.Layer * max(1, nl))()
        shapes = wl.weight_shapes(cfg)
        bases = rope_bases(w)
        for li in range(nl):
            t = w.layers[li]
            L = self.layers[li]
            for n in B._LAYER_U32:
                setattr(L, n, int(cfg[n]))
            L.window = int(t.get("window", cfg["window"]))
            L.eps = cfg["eps"]
            L.attn_scale = cfg["attn_scale"]
            L.v_norm = 1 if cfg.get("v_norm") else 0
            L.rope_table = bases.index(float(t.get("rope_base", cfg["rope_base"])))
            L.scalar = float(t.get("scalar", 1.0))
            L.n_ple = int(cfg.get("n_ple", 0))
            L.ple_scale = float(cfg.get("ple_scale", 1.0))
            for n in _W_NAMES:
                if n not in shapes:
                    continue
                if cfg["path"] == wl.PATH_I8F16 and n not in t:
                    dev = wl.int8_weight_torch(w.seed, li, n, shapes[n], device, w.prefix)
                else:
                    arr = t[n]
                    dev = torch.from_numpy(np.ascontiguousarray(arr)).to(device)
                self.keep.append(dev)
                setattr(L, n, dev.data_ptr())
            guards = t.get("guards", cfg.get("guards"))
            if guards:
                for n, g in zip(B._LAYER_GUARDS, guards):
                    setattr(L, n, int(g))
            for n in _F32_NAMES + _PLE_NAMES + _MOD_COL_NAMES:
                if t.get(n) is not None:
                    dev = torch.from_numpy(np.ascontiguousarray(t[n], np.float32)).to(device)
                    self.keep.append(dev)
                    setattr(L, n, dev.data_ptr())
        self.model = B.Model()
        self.model.nlayers = nl
        self.model.layers = self.layers
        self.model.final_kind = int(cfg["final"])
        self.model.final_eps = cfg["eps"]
        for n in ("final_w", "final_b"):
            a = getattr(w, n)
            if a is not None:
                dev = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
                self.keep.append(dev)
                setattr(self.model, n, dev.data_ptr())

    def workspace_bytes(self, batch: "DeviceBatch"):
        return B.lib().enc_workspace_bytes(C.byref(self.model), C.byref(batch.batch))

    def workspace(self, batch: "DeviceBatch", device="cuda"):
        return torch.empty(self.workspace_bytes(batch), dtype=torch.uint8, device=device)


class DeviceBatch:
    """The batch struct of a workload; `pos` gives the rows' RoPE positions
    (default: from its items, enc_positions) -- a stage of a larger program
    passes the positions its rows have in that program."""

    def __init__(self, w: wl.Workload, device="cuda", pos=None):
        cfg = w.cfg
        self.rows = w.rows
        self.items_py = w.items
        self.items = B.make_items(w.items)
        self.batch = B.Batch()
        self.batch.rows = w.rows
        self.batch.items = self.items
        self.batch.nitems = len(w.items)
        self.cos = self.sin = None
        sec = cfg["rope_sections"]
        self.tables = []
        if sec:
            self.pos = B.positions(w.rows, w.items, w.grids, sec) if pos is None else pos
            for i, base in enumerate(rope_bases(w)):
                cos, sin = B.rope_table(self.pos, cfg["hd"], sec, base)
                cos, sin = torch.from_numpy(cos).to(device), torch.from_numpy(sin).to(device)
                self.tables.append((cos, sin))
                self.batch.rope_cos[i] = cos.data_ptr()
                self.batch.rope_sin[i] = sin.data_ptr()
            self.cos, self.sin = self.tables[0]


def encoder_forward(model: DeviceModel, batch: DeviceBatch, x, out, ws, ctx=None, stream=None):
    ctx = ctx or B.context()
    ctx.check(B.lib().encoder_forward(ctx.h, C.byref(model.model), C.byref(batch.batch),
                                      x.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(),
                                      B._stream(stream)))


def encoder_layer_forward(model: DeviceModel, layer: int, batch: DeviceBatch, h, ws, ctx=None,
                          stream=None, a=None, next_layer=None):
    """Layer `layer` in place on h.  a: the layer's pre-normed input (None: the
    layer computes it); next_layer: the index of the layer whose input the call
    then writes into a (needs a)."""
    ctx = ctx or B.context()
    nxt = C.byref(model.layers[next_layer]) if next_layer is not None else None
    ctx.check(B.lib().encoder_layer_forward(ctx.h, C.byref(model.layers[layer]), nxt,
                                            C.byref(batch.batch), h.data_ptr(),
                                            a.data_ptr() if a is not None else None,
                                            ws.data_ptr(), ws.numel(), B._stream(stream)))


def layer_input(model: DeviceModel, layer: int, h, a, ctx=None, stream=None):
    """The pre-normed input of layer `layer` from the rows h, into a: the first
    call of a chain of encoder_layer_forward calls that hand each next layer's
    input over in a.  Sandwich: enc_add_norm without a residual (rms(h) w (1 + s),
    one copy per column field, times 2^-guard); pre-LN: enc_layer_norm."""
    ctx = ctx or B.context()
    L = model.layers[layer]
    f16 = L.path == wl.PATH_I8F16
    if L.block == wl.BLOCK_PRE_LN:
        d = B.NormDesc()
        d.rows, d.d, d.x, d.ldx = h.shape[0], h.shape[1], h.data_ptr(), h.stride(0)
        d.w, d.b, d.eps = L.norm1_w, L.norm1_b, L.eps
        d.y, d.ldy, d.flags = a.data_ptr(), h.shape[1], B.ENC_Y_F16 if f16 else 0
        ctx.check(B.lib().enc_layer_norm(ctx.h, C.byref(d), B._stream(stream)))
        return
    d = B.AddNormDesc()
    d.rows, d.d, d.h, d.t = h.shape[0], h.shape[1], h.data_ptr(), None
    d.w_next, d.eps, d.a = L.norm1_w, L.eps, a.data_ptr()
    d.flags = B.ENC_Y_F16 if f16 else 0
    d.scale = L.mod_s_attn
    cols = (L.col_q, L.col_k, L.col_v)
    if any(cols):
        for z, c in enumerate(cols):
            d.col[z] = c
        d.nout = 3
    d.oscale = 2.0 ** -int(L.guard_attn)
    ctx.check(B.lib().enc_add_norm(ctx.h, C.byref(d), B._stream(stream)))


def out_rows(w: wl.Workload):
    return len(w.items) if w.cfg["final"] == wl.FINAL_RMS_MEANPOOL else w.rows


class DeviceProgram:
    """A staged program (w.stages: context refiner, noise refiner, main stack)
    as an enc_stage array; `skip` leaves out stages by label (the context
    refiner runs once per prompt, not per step)."""

    def __init__(self, w: wl.Workload, device="cuda", skip=()):
        sec = w.cfg["rope_sections"]
        joint = B.positions(w.rows, w.items, w.grids, sec) if sec else None
        self.rows, self.d = w.rows, w.cfg["d"]
        self.parts = []
        for label, st, row0 in w.stages:
            if label in skip:
                continue
            pos = joint[row0:row0 + st.rows] if joint is not None else None
            self.parts.append((label, DeviceModel(st, device), DeviceBatch(st, device, pos=pos), row0))
        self.stages = (B.Stage * len(self.parts))()
        for i, (_, dm, db, row0) in enumerate(self.parts):
            self.stages[i].model = C.pointer(dm.model)
            self.stages[i].batch = db.batch
            self.stages[i].row0 = row0

    def workspace_bytes(self):
        return B.lib().enc_stages_workspace_bytes(self.stages, len(self.parts))

    def workspace(self, device="cuda"):
        return torch.empty(self.workspace_bytes(), dtype=torch.uint8, device=device)


def stages_forward(prog: DeviceProgram, x, h, ws, ctx=None, stream=None):
    ctx = ctx or B.context()
    ctx.check(B.lib().encoder_stages_forward(ctx.h, prog.stages, len(prog.parts), prog.rows,
                                             x.data_ptr(), h.data_ptr(), ws.data_ptr(), ws.numel(),
                                             B._stream(stream)))
