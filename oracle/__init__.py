"""Python marshalling for the f64 oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY.  Callers: tests/, __graft_entry__.smoke() and the
bench's cpu_baseline leg.  The HIP library never imports, links or runs this.
This module only converts numpy arrays and plain values into the C structs;
every step of the forward is computed in oracle.c.  It imports nothing from the
library package: a workload is read through its attributes (cfg, rows, items,
grids, x, layers, final_w, final_b).

Parity pins: every function here is pinned by tests/test_oracle.py.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain -O2, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        _lib = C.CDLL(LIB)
        _setup(_lib)
    return _lib


class Item(C.Structure):
    _fields_ = [("nr", C.c_int32), ("r0", C.c_int32 * 2), ("n", C.c_int32 * 2),
                ("grid", C.c_int32)]


_LAYER_PTRS_F = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]
_LAYER_PTRS_Q = ["qq", "qk", "qv", "qo", "q_gate", "q_up", "q_down"]
_LAYER_PTRS_S = ["sq", "sk", "sv", "so", "s_gate", "s_up", "s_down"]
_LAYER_PTRS_B = ["bq", "bk", "bv", "bo", "b_up", "b_down"]
_LAYER_PTRS_N = ["norm1_w", "norm1_b", "norm2_w", "norm2_b", "post_attn_w", "post_ff_w",
                 "q_norm_w", "k_norm_w"]
_LAYER_PTRS_PLE = ["ple_in", "ple_gate", "ple_proj", "ple_in_norm_w", "ple_post_w"]
_LAYER_PTRS_MOD = ["mod_s_attn", "mod_g_attn", "mod_s_ff", "mod_g_ff"]
_LAYER_PTRS_COL = ["col_q", "col_k", "col_v", "col_o", "col_gate", "col_up", "col_down"]
_LAYER_GUARDS = ["guard_attn", "guard_qkv", "guard_ao", "guard_ffn", "guard_hid"]


class Layer(C.Structure):
    _fields_ = ([(n, C.c_int32) for n in ("block", "path", "mlp", "d", "nq", "nkv", "hd", "ff",
                                          "window", "rope_sections")]
                + [(n, C.c_double) for n in ("eps", "attn_scale", "rope_base")]
                + [(n, C.POINTER(C.c_float)) for n in _LAYER_PTRS_F]
                + [(n, C.POINTER(C.c_int8)) for n in _LAYER_PTRS_Q]
                + [(n, C.POINTER(C.c_float)) for n in _LAYER_PTRS_S + _LAYER_PTRS_B
                   + _LAYER_PTRS_N]
                + [("v_norm", C.c_int32), ("n_ple", C.c_int32), ("scalar", C.c_double),
                   ("ple_scale", C.c_double)]
                + [(n, C.POINTER(C.c_float)) for n in _LAYER_PTRS_PLE + _LAYER_PTRS_MOD
                   + _LAYER_PTRS_COL]
                + [(n, C.c_int32) for n in _LAYER_GUARDS])


class Model(C.Structure):
    _fields_ = [("d", C.c_int32), ("nlayers", C.c_int32), ("layers", C.POINTER(Layer)),
                ("final_kind", C.c_int32),
                ("final_w", C.POINTER(C.c_float)), ("final_b", C.POINTER(C.c_float)),
                ("final_eps", C.c_double)]


_D = C.POINTER(C.c_double)
_F = C.POINTER(C.c_float)
_I32 = C.POINTER(C.c_int32)
_I8 = C.POINTER(C.c_int8)


def _setup(L):
    L.or_threads.argtypes = []
    L.or_threads.restype = C.c_int
    L.or_round_f16.argtypes = [C.c_double]
    L.or_round_f16.restype = C.c_double
    L.or_gelu_tanh.argtypes = [C.c_double]
    L.or_gelu_tanh.restype = C.c_double
    L.or_silu.argtypes = [C.c_double]
    L.or_silu.restype = C.c_double
    L.or_rms_norm.argtypes = [C.c_int64, C.c_int, _D, _F, C.c_double, _D]
    L.or_layer_norm.argtypes = [C.c_int64, C.c_int, _D, _F, _F, C.c_double, _D]
    L.or_linear.argtypes = [C.c_int64, C.c_int, C.c_int, _D, _F, _F, _D]
    L.or_linear_q8.argtypes = [C.c_int64, C.c_int, C.c_int, _D, _I8, _F, _D]
    L.or_positions.argtypes = [C.c_int, C.POINTER(Item), C.c_int, _I32]
    L.or_qk_norm_rope.argtypes = [C.c_int64, C.c_int, C.c_int, _D, _F, C.c_double, C.c_int, _I32,
                                  C.c_double]
    L.or_attention.argtypes = [C.c_int, C.POINTER(Item), C.c_int, C.c_int, C.c_int, _D, C.c_int,
                               _D, C.c_int, _D, C.c_int, _D, C.c_int, C.c_double, C.c_int]
    L.or_attention_rows.argtypes = L.or_attention.argtypes + [_I8]
    L.or_encoder_forward.argtypes = [C.POINTER(Model), C.c_int64, C.c_int, C.POINTER(Item), _D,
                                     _D, C.c_int, _D]
    L.or_encoder_forward_pos.argtypes = [C.POINTER(Model), C.c_int64, C.c_int, C.POINTER(Item),
                                         _I32, _D, _D, C.c_int, _D]
    L.or_encoder_forward_pos.restype = None
    for f in ("or_rms_norm", "or_layer_norm", "or_linear", "or_linear_q8", "or_positions",
              "or_qk_norm_rope", "or_attention", "or_attention_rows", "or_encoder_forward"):
        getattr(L, f).restype = None


def _d(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_D)


def _f(a):
    if a is None:
        return None, None
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(_F)


def _items(items, grids=None):
    arr = (Item * max(1, len(items)))()
    for i, rr in enumerate(items):
        arr[i].nr = len(rr)
        for r, (r0, n) in enumerate(rr):
            arr[i].r0[r] = r0
            arr[i].n[r] = n
        arr[i].grid = grids[i] if grids else 0
    return arr


# --------------------------------------------------------------------------- ops

def threads() -> int:
    return lib().or_threads()


def round_f16(x: float) -> float:
    return lib().or_round_f16(float(x))


def gelu_tanh(x: float) -> float:
    return lib().or_gelu_tanh(float(x))


def silu(x: float) -> float:
    return lib().or_silu(float(x))


def rms_norm(x, w, eps):
    x, xp = _d(x)
    w, wp = _f(w)
    y = np.empty_like(x)
    lib().or_rms_norm(x.shape[0], x.shape[1], xp, wp, eps, y.ctypes.data_as(_D))
    return y


def layer_norm(x, w, b, eps):
    x, xp = _d(x)
    w, wp = _f(w)
    b, bp = _f(b)
    y = np.empty_like(x)
    lib().or_layer_norm(x.shape[0], x.shape[1], xp, wp, bp, eps, y.ctypes.data_as(_D))
    return y


def linear(x, w, b=None):
    x, xp = _d(x)
    w, wp = _f(w)
    b, bp = _f(b)
    y = np.empty((x.shape[0], w.shape[0]))
    lib().or_linear(x.shape[0], x.shape[1], w.shape[0], xp, wp, bp, y.ctypes.data_as(_D))
    return y


def linear_q8(x, q, rs):
    x, xp = _d(x)
    q = np.ascontiguousarray(q, dtype=np.int8)
    rs, rp = _f(rs)
    y = np.empty((x.shape[0], q.shape[0]))
    lib().or_linear_q8(x.shape[0], x.shape[1], q.shape[0], xp, q.ctypes.data_as(_I8), rp,
                       y.ctypes.data_as(_D))
    return y


def positions(rows, items, grids, sections):
    pos = np.zeros((rows, max(1, sections)), np.int32)
    it = _items(items, grids)
    lib().or_positions(len(items), it, sections, pos.ctypes.data_as(_I32))
    return pos


def qk_norm_rope(x, nh, hd, w, eps, sections, pos, base):
    """x [rows][nh*hd] -> normed + rotated copy."""
    y, yp = _d(np.array(x, dtype=np.float64, copy=True))
    w, wp = _f(w)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    lib().or_qk_norm_rope(y.shape[0], nh, hd, yp, wp, eps, sections, pos.ctypes.data_as(_I32),
                          base)
    return y


def attention(items, q, k, v, nq, nkv, hd, scale, window, rows=None, query_rows=None):
    """Per-item softmax attention; q [rows][nq*hd], k/v [rows][nkv*hd] -> o [rows][nq*hd].
    With `query_rows`, only those output rows are computed (the others stay 0)."""
    q, qp = _d(q)
    k, kp = _d(k)
    v, vp = _d(v)
    o = np.zeros((q.shape[0], nq * hd))
    it = _items(items)
    if query_rows is None:
        lib().or_attention(len(items), it, nq, nkv, hd, qp, q.shape[1], kp, k.shape[1], vp,
                           v.shape[1], o.ctypes.data_as(_D), nq * hd, scale, window)
    else:
        sel = np.zeros(q.shape[0], np.int8)
        sel[np.asarray(query_rows)] = 1
        lib().or_attention_rows(len(items), it, nq, nkv, hd, qp, q.shape[1], kp, k.shape[1], vp,
                                v.shape[1], o.ctypes.data_as(_D), nq * hd, scale, window,
                                sel.ctypes.data_as(_I8))
    return o


# ----------------------------------------------------------------------- forward

def _layer_struct(cfg, t, keep):
    """A layer from the workload config and the layer's dict; per-layer values
    (window, rope_base, scalar) in the dict override the config's."""
    L = Layer()
    for n in ("block", "path", "mlp", "d", "nq", "nkv", "hd", "ff", "rope_sections"):
        setattr(L, n, int(cfg[n]))
    L.window = int(t.get("window", cfg["window"]))
    L.eps = cfg["eps"]
    L.attn_scale = cfg["attn_scale"]
    L.rope_base = float(t.get("rope_base", cfg["rope_base"]))
    L.v_norm = 1 if cfg.get("v_norm") else 0
    L.scalar = float(t.get("scalar", 1.0))
    L.n_ple = int(cfg.get("n_ple", 0))
    L.ple_scale = float(cfg.get("ple_scale", 1.0))
    for n in _LAYER_PTRS_PLE + _LAYER_PTRS_MOD + _LAYER_PTRS_COL:
        if t.get(n) is not None:
            a, p = _f(t[n])
            keep.append(a)
            setattr(L, n, p)
    guards = t.get("guards", cfg.get("guards"))
    if guards:
        for n, g in zip(_LAYER_GUARDS, guards):
            setattr(L, n, int(g))
    for fn, qn, sn in zip(_LAYER_PTRS_F, _LAYER_PTRS_Q, _LAYER_PTRS_S):
        if fn not in t:
            continue
        if cfg["path"] == 0:
            a, p = _f(t[fn])
            keep.append(a)
            setattr(L, fn, p)
        else:
            a = np.ascontiguousarray(t[fn], dtype=np.int8)
            keep.append(a)
            setattr(L, qn, a.ctypes.data_as(_I8))
            s, sp = _f(t[sn])
            keep.append(s)
            setattr(L, sn, sp)
    for n in _LAYER_PTRS_B + _LAYER_PTRS_N:
        if t.get(n) is not None:
            a, p = _f(t[n])
            keep.append(a)
            setattr(L, n, p)
    return L


def forward(w, layers=None, f16_sites: bool = True, x=None, amax=None, pos=None):
    """The oracle forward of a workload-like object (first `layers` layers).
    amax: an optional float64 array [layers][5] that receives the per-site
    max |stored value| of the int8 path's half sites.  pos: the rows' RoPE
    positions [rows][sections] (default: from the items, as or_positions)."""
    cfg = w.cfg
    nl = len(w.layers) if layers is None else layers
    keep = []
    arr = (Layer * max(1, nl))()
    for i in range(nl):
        arr[i] = _layer_struct(cfg, w.layers[i], keep)
    M = Model()
    M.d = int(cfg["d"])
    M.nlayers = nl
    M.layers = arr
    M.final_kind = int(cfg["final"])
    M.final_eps = cfg["eps"]
    fw, fwp = _f(w.final_w)
    fb, fbp = _f(w.final_b)
    M.final_w = fwp
    M.final_b = fbp
    x, xp = _d(w.x if x is None else x)
    d = x.shape[1]
    nout = len(w.items) if cfg["final"] == 2 else w.rows
    out = np.zeros((nout, d))
    it = _items(w.items, w.grids)
    if amax is not None:
        assert amax.dtype == np.float64 and amax.shape == (nl, 5) and amax.flags.c_contiguous
        amax[:] = 0.0
    am = amax.ctypes.data_as(_D) if amax is not None else None
    if pos is None:
        lib().or_encoder_forward(C.byref(M), w.rows, len(w.items), it, xp, out.ctypes.data_as(_D),
                                 1 if f16_sites else 0, am)
    else:
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        assert pos.shape[0] == w.rows
        lib().or_encoder_forward_pos(C.byref(M), w.rows, len(w.items), it, pos.ctypes.data_as(_I32),
                                     xp, out.ctypes.data_as(_D), 1 if f16_sites else 0, am)
    del keep, fw, fb
    return out


def forward_stages(stages, x, f16_sites: bool = True):
    """A staged program: each stage (a workload-like object over rows
    [row0, row0 + rows), its items relative to row0, its positions, final NONE)
    runs its layers in place on those rows of the residual, in order."""
    H = np.array(x, dtype=np.float64, copy=True)
    for st, row0, pos in stages:
        assert st.cfg["final"] == 0
        H[row0:row0 + st.rows] = forward(st, f16_sites=f16_sites, x=H[row0:row0 + st.rows], pos=pos)
    return H
