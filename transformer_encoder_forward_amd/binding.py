"""ctypes binding of libenc.so (include/enc.h): argument marshalling only.

Every function here converts torch tensors / Python values into the C structs
and calls the library; no step of the forward runs in Python.  Importing this
module never falls back to anything: if libenc.so is missing or cannot be
loaded, `lib()` raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libenc.so")

ENC_OK, ENC_EINVAL, ENC_ESHAPE, ENC_EUNSUPPORTED, ENC_EDEVICE = range(5)
ENC_F32, ENC_I8F16 = 0, 1
ENC_Y_F16, ENC_Y_ACCUMULATE, ENC_EPI_GELU_TANH = 1, 2, 4
ENC_EPI_GATE_GELU_TANH, ENC_EPI_GATE_SILU = 8, 16
ENC_ACT_GELU_TANH_GATED, ENC_ACT_SWIGLU = 1, 2
STATUS_NAMES = {0: "ENC_OK", 1: "ENC_EINVAL", 2: "ENC_ESHAPE", 3: "ENC_EUNSUPPORTED",
                4: "ENC_EDEVICE"}

# every symbol include/enc.h declares
EXPORTS = ["enc_create", "enc_destroy", "enc_last_error", "gemm_items", "attention_items",
           "attention_items_static", "enc_rms_norm", "enc_layer_norm", "enc_add_norm", "enc_qk_norm_rope", "enc_gated_act",
           "enc_mean_pool", "enc_workspace_bytes", "encoder_layer_forward", "encoder_forward",
           "enc_check_gemm", "enc_check_attention", "enc_check_model", "enc_validate_model", "enc_positions",
           "enc_rope_table", "enc_prof_enable", "enc_prof_read", "enc_mfma_peak",
           "enc_attention_workspace_bytes", "encoder_stages_forward", "enc_stages_workspace_bytes"]
CLASS_NAMES = ["gemm", "attn", "rows"]


class EncError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


# ------------------------------------------------------------------ structs

class GemmItem(C.Structure):
    _fields_ = [("n", C.c_uint32), ("m", C.c_uint32), ("k", C.c_uint32), ("ldx", C.c_uint32),
                ("ldy", C.c_uint32), ("slot", C.c_uint32), ("x_off", C.c_uint64),
                ("y_off", C.c_uint64)]


class GemmDesc(C.Structure):
    _fields_ = [("path", C.c_uint32), ("x", C.c_void_p), ("y", C.c_void_p),
                ("w", C.c_void_p * 4), ("row_scale", C.c_void_p * 4), ("bias", C.c_void_p * 4),
                ("alpha", C.c_float), ("flags", C.c_uint32), ("y_col", C.c_void_p),
                ("y_scale", C.c_float)]


class Range(C.Structure):
    _fields_ = [("r0", C.c_uint32), ("n", C.c_uint32)]


class Item(C.Structure):
    _fields_ = [("r", Range * 2), ("nr", C.c_uint32)]


class AttnDesc(C.Structure):
    _fields_ = [("path", C.c_uint32), ("qkv", C.c_void_p), ("ld", C.c_uint32),
                ("q_col", C.c_uint32), ("k_col", C.c_uint32), ("v_col", C.c_uint32),
                ("out", C.c_void_p), ("ldo", C.c_uint32), ("nq", C.c_uint32),
                ("nkv", C.c_uint32), ("hd", C.c_uint32), ("scale", C.c_float),
                ("window", C.c_uint32), ("rows", C.c_uint32), ("ws", C.c_void_p),
                ("ws_bytes", C.c_size_t), ("out_col", C.c_void_p), ("out_scale", C.c_float)]


class NormDesc(C.Structure):
    _fields_ = [("rows", C.c_uint32), ("d", C.c_uint32), ("x", C.c_void_p), ("ldx", C.c_uint32),
                ("w", C.c_void_p), ("b", C.c_void_p), ("eps", C.c_float), ("y", C.c_void_p),
                ("ldy", C.c_uint32), ("flags", C.c_uint32), ("pre", C.c_float)]


class AddNormDesc(C.Structure):
    _fields_ = [("rows", C.c_uint32), ("d", C.c_uint32), ("h", C.c_void_p), ("t", C.c_void_p),
                ("w_post", C.c_void_p), ("w_next", C.c_void_p), ("eps", C.c_float),
                ("a", C.c_void_p), ("flags", C.c_uint32), ("post", C.c_float),
                ("gate", C.c_void_p), ("scale", C.c_void_p), ("col", C.c_void_p * 3),
                ("nout", C.c_uint32), ("oscale", C.c_float)]


class QkDesc(C.Structure):
    _fields_ = [("path", C.c_uint32), ("panel", C.c_void_p), ("rows", C.c_uint32),
                ("ld", C.c_uint32), ("q_col", C.c_uint32), ("k_col", C.c_uint32),
                ("nq", C.c_uint32), ("nkv", C.c_uint32), ("hd", C.c_uint32),
                ("q_norm_w", C.c_void_p), ("k_norm_w", C.c_void_p), ("eps", C.c_float),
                ("cos", C.c_void_p), ("sin", C.c_void_p), ("sections", C.c_uint32),
                ("v_col", C.c_uint32), ("v_norm", C.c_uint32)]


class ActDesc(C.Structure):
    _fields_ = [("kind", C.c_uint32), ("rows", C.c_uint32), ("ff", C.c_uint32),
                ("g", C.c_void_p), ("ldg", C.c_uint32), ("u", C.c_void_p), ("ldu", C.c_uint32),
                ("out", C.c_void_p), ("ldo", C.c_uint32), ("flags", C.c_uint32),
                ("out_col", C.c_void_p), ("out_scale", C.c_float)]


_LAYER_U32 = ["block", "path", "mlp", "d", "nq", "nkv", "hd", "ff", "window", "rope_sections"]
_LAYER_PTRS = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down",
               "sq", "sk", "sv", "so", "s_gate", "s_up", "s_down",
               "bq", "bk", "bv", "bo", "b_up", "b_down",
               "norm1_w", "norm1_b", "norm2_w", "norm2_b",
               "post_attn_w", "post_ff_w", "q_norm_w", "k_norm_w"]


_LAYER_PLE_PTRS = ["ple_in", "ple_gate", "ple_proj", "ple_in_norm_w", "ple_post_w"]
_LAYER_MOD_PTRS = ["mod_s_attn", "mod_g_attn", "mod_s_ff", "mod_g_ff"]
_LAYER_COL_PTRS = ["col_q", "col_k", "col_v", "col_o", "col_gate", "col_up", "col_down"]
_LAYER_GUARDS = ["guard_attn", "guard_qkv", "guard_ao", "guard_ffn", "guard_hid"]


class Layer(C.Structure):
    _fields_ = ([(n, C.c_uint32) for n in _LAYER_U32]
                + [("eps", C.c_float), ("attn_scale", C.c_float)]
                + [(n, C.c_void_p) for n in _LAYER_PTRS]
                + [("v_norm", C.c_uint32), ("rope_table", C.c_uint32), ("scalar", C.c_float),
                   ("n_ple", C.c_uint32), ("ple_scale", C.c_float)]
                + [(n, C.c_void_p) for n in _LAYER_PLE_PTRS + _LAYER_MOD_PTRS + _LAYER_COL_PTRS]
                + [(n, C.c_uint32) for n in _LAYER_GUARDS])


class ProfStat(C.Structure):
    _fields_ = [("launches", C.c_uint64), ("ms", C.c_double), ("flops", C.c_double),
                ("bytes", C.c_double)]


MAX_ROPE_TABLES = 4


class Batch(C.Structure):
    _fields_ = [("rows", C.c_uint32), ("items", C.POINTER(Item)), ("nitems", C.c_uint32),
                ("rope_cos", C.c_void_p * MAX_ROPE_TABLES), ("rope_sin", C.c_void_p * MAX_ROPE_TABLES),
                ("ple_x", C.c_void_p), ("amax", C.c_void_p)]


class Model(C.Structure):
    _fields_ = [("nlayers", C.c_uint32), ("layers", C.POINTER(Layer)),
                ("final_kind", C.c_uint32), ("final_w", C.c_void_p), ("final_b", C.c_void_p),
                ("final_eps", C.c_float)]


class Stage(C.Structure):
    _fields_ = [("model", C.POINTER(Model)), ("batch", Batch), ("row0", C.c_uint32)]


# ------------------------------------------------------------------ loading

_lib = None


def lib():
    """The loaded libenc.so; raises if it is not built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                           "(python -m transformer_encoder_forward_amd.build)")
    L = C.CDLL(LIB_PATH)
    P = C.c_void_p
    S = C.c_int
    L.enc_create.argtypes = [C.c_int, C.POINTER(P)]
    L.enc_create.restype = S
    L.enc_destroy.argtypes = [P]
    L.enc_destroy.restype = None
    L.enc_last_error.argtypes = [P]
    L.enc_last_error.restype = C.c_char_p
    L.gemm_items.argtypes = [P, C.POINTER(GemmDesc), C.POINTER(GemmItem), C.c_uint32, P]
    L.attention_items.argtypes = [P, C.POINTER(AttnDesc), C.POINTER(Item), C.c_uint32, P]
    L.attention_items_static.argtypes = [P, C.POINTER(AttnDesc), C.POINTER(Item), C.c_uint32, P]
    L.enc_rms_norm.argtypes = [P, C.POINTER(NormDesc), P]
    L.enc_layer_norm.argtypes = [P, C.POINTER(NormDesc), P]
    L.enc_add_norm.argtypes = [P, C.POINTER(AddNormDesc), P]
    L.enc_qk_norm_rope.argtypes = [P, C.POINTER(QkDesc), P]
    L.enc_gated_act.argtypes = [P, C.POINTER(ActDesc), P]
    L.enc_mean_pool.argtypes = [P, C.c_uint32, C.c_uint32, P, C.POINTER(Item), C.c_uint32, P, P]
    L.enc_workspace_bytes.argtypes = [C.POINTER(Model), C.POINTER(Batch)]
    L.enc_workspace_bytes.restype = C.c_size_t
    L.enc_attention_workspace_bytes.argtypes = [C.POINTER(AttnDesc), C.POINTER(Item), C.c_uint32]
    L.enc_attention_workspace_bytes.restype = C.c_size_t
    L.encoder_layer_forward.argtypes = [P, C.POINTER(Layer), C.POINTER(Layer), C.POINTER(Batch), P,
                                        P, P, C.c_size_t, P]
    L.encoder_forward.argtypes = [P, C.POINTER(Model), C.POINTER(Batch), P, P, P, C.c_size_t, P]
    L.encoder_stages_forward.argtypes = [P, C.POINTER(Stage), C.c_uint32, C.c_uint32, P, P, P,
                                         C.c_size_t, P]
    L.enc_stages_workspace_bytes.argtypes = [C.POINTER(Stage), C.c_uint32]
    L.enc_stages_workspace_bytes.restype = C.c_size_t
    L.enc_check_gemm.argtypes = [C.POINTER(GemmDesc), C.POINTER(GemmItem), C.c_uint32,
                                 C.c_char_p, C.c_size_t]
    L.enc_check_attention.argtypes = [C.POINTER(AttnDesc), C.POINTER(Item), C.c_uint32,
                                      C.c_char_p, C.c_size_t]
    L.enc_check_model.argtypes = [C.POINTER(Model), C.POINTER(Batch), C.c_char_p, C.c_size_t]
    L.enc_validate_model.argtypes = [C.POINTER(Model), C.POINTER(Batch)]
    L.enc_positions.argtypes = [C.c_uint32, C.POINTER(Item), P, C.c_uint32, C.c_uint32, P]
    L.enc_rope_table.argtypes = [C.c_uint32, C.c_uint32, C.c_uint32, P, C.c_double, P, P]
    L.enc_prof_enable.argtypes = [P, C.c_int]
    L.enc_prof_read.argtypes = [P, C.POINTER(ProfStat)]
    L.enc_mfma_peak.argtypes = [P, C.c_uint32, C.c_uint32, C.c_uint32, P, C.POINTER(C.c_double), P]
    for f in ("gemm_items", "attention_items", "attention_items_static", "enc_rms_norm", "enc_layer_norm", "enc_add_norm",
              "enc_qk_norm_rope", "enc_gated_act", "enc_mean_pool", "encoder_layer_forward",
              "encoder_forward", "encoder_stages_forward", "enc_check_gemm", "enc_check_attention", "enc_check_model",
              "enc_validate_model",
              "enc_positions", "enc_rope_table", "enc_prof_enable", "enc_prof_read",
              "enc_mfma_peak"):
        getattr(L, f).restype = S
    _lib = L
    return L


# ------------------------------------------------------------------ helpers

def _ptr(t):
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def make_items(items):
    """[[ (r0, n), ... ], ...] -> ctypes array of Item."""
    arr = (Item * max(1, len(items)))()
    for i, rr in enumerate(items):
        arr[i].nr = len(rr)
        for r, (r0, n) in enumerate(rr):
            arr[i].r[r].r0 = r0
            arr[i].r[r].n = n
    return arr


class Context:
    """One enc_ctx on a HIP device."""

    def __init__(self, device: int = 0):
        h = C.c_void_p()
        st = lib().enc_create(device, C.byref(h))
        if st != ENC_OK:
            raise EncError(st, lib().enc_last_error(None).decode())
        self.h = h
        self.device = device

    def check(self, st):
        if st != ENC_OK:
            raise EncError(st, lib().enc_last_error(self.h).decode())

    def __del__(self):
        if getattr(self, "h", None) and _lib is not None:
            _lib.enc_destroy(self.h)
            self.h = None


_ctx = {}


def context(device: int = 0) -> Context:
    if device not in _ctx:
        _ctx[device] = Context(device)
    return _ctx[device]


# ------------------------------------------------------------------ ops

def gemm_items(x, y, w, items, path=ENC_F32, row_scale=None, bias=None, alpha=1.0, flags=0,
               y_col=None, y_scale=1.0, ctx=None, stream=None):
    """items: list of dicts/tuples (n, m, k, ldx, ldy, slot, x_off, y_off); w: list of tensors."""
    ctx = ctx or context()
    d = GemmDesc()
    d.path = path
    d.x = _ptr(x)
    d.y = _ptr(y)
    for s in range(4):
        d.w[s] = _ptr(w[s]) if s < len(w) else None
        d.row_scale[s] = _ptr(row_scale[s]) if row_scale and s < len(row_scale) else None
        d.bias[s] = _ptr(bias[s]) if bias and s < len(bias) else None
    d.alpha = alpha
    d.flags = flags
    d.y_col = _ptr(y_col)
    d.y_scale = y_scale
    arr = (GemmItem * len(items))(*[GemmItem(*it) for it in items])
    ctx.check(lib().gemm_items(ctx.h, C.byref(d), arr, len(items), _stream(stream)))


def attention_desc(qkv, out, nq, nkv, hd, scale, window=0, ld=None, q_col=0, k_col=None,
                   v_col=None, ldo=None, path=ENC_F32, rows=None):
    d = AttnDesc()
    d.path = path
    d.qkv = _ptr(qkv)
    d.ld = ld if ld is not None else qkv.shape[1]
    d.q_col = q_col
    d.k_col = k_col if k_col is not None else nq * hd
    d.v_col = v_col if v_col is not None else nq * hd + nkv * hd
    d.out = _ptr(out)
    d.ldo = ldo if ldo is not None else out.shape[1]
    d.nq, d.nkv, d.hd = nq, nkv, hd
    d.scale = scale
    d.window = window
    d.rows = rows if rows is not None else qkv.shape[0]
    return d


def attention_workspace_bytes(desc, items):
    return lib().enc_attention_workspace_bytes(C.byref(desc), make_items(items), len(items))


def attention_items(qkv, out, items, nq, nkv, hd, scale, window=0, ld=None, q_col=0,
                    k_col=None, v_col=None, ldo=None, path=ENC_F32, rows=None, ws="auto",
                    out_col=None, out_scale=1.0, ctx=None, stream=None):
    """ws: "auto" (a torch buffer of the size the key splits need), None (no
    split) or a uint8 device tensor."""
    ctx = ctx or context()
    d = attention_desc(qkv, out, nq, nkv, hd, scale, window, ld, q_col, k_col, v_col, ldo, path,
                       rows)
    d.out_col, d.out_scale = _ptr(out_col), out_scale
    if isinstance(ws, str):
        import torch
        n = attention_workspace_bytes(d, items)
        ws = torch.empty(n, dtype=torch.uint8, device=qkv.device) if n else None
        if ws is not None and stream is not None and hasattr(stream, "cuda_stream"):
            ws.record_stream(stream)
    if ws is not None:
        d.ws, d.ws_bytes = ws.data_ptr(), ws.numel()
    arr = make_items(items)
    ctx.check(lib().attention_items(ctx.h, C.byref(d), arr, len(items), _stream(stream)))


def attention_items_static(qkv, out, items, nq, nkv, hd, scale, window=0, ld=None, q_col=0,
                           k_col=None, v_col=None, ldo=None, path=ENC_F32, rows=None,
                           out_col=None, out_scale=1.0, ctx=None, stream=None):
    """attention_items with the key-split partials in the library's static
    per-GPU scratch (no workspace, nothing allocated)."""
    ctx = ctx or context()
    d = attention_desc(qkv, out, nq, nkv, hd, scale, window, ld, q_col, k_col, v_col, ldo, path,
                       rows)
    d.out_col, d.out_scale = _ptr(out_col), out_scale
    arr = make_items(items)
    ctx.check(lib().attention_items_static(ctx.h, C.byref(d), arr, len(items), _stream(stream)))


STATIC_SCRATCH_BYTES = 32 << 20  # ENC_STATIC_SCRATCH_BYTES


def _norm(fn, x, w, b, eps, y, f16, ctx, stream, pre=1.0):
    ctx = ctx or context()
    d = NormDesc()
    d.pre = pre
    d.rows, d.d = x.shape[0], x.shape[1]
    d.x, d.ldx = _ptr(x), x.stride(0)
    d.w, d.b = _ptr(w), _ptr(b)
    d.eps = eps
    d.y, d.ldy = _ptr(y), y.stride(0)
    d.flags = ENC_Y_F16 if f16 else 0
    ctx.check(fn(ctx.h, C.byref(d), _stream(stream)))


def rms_norm(x, w, eps, y, f16=False, pre=1.0, ctx=None, stream=None):
    _norm(lib().enc_rms_norm, x, w, None, eps, y, f16, ctx, stream, pre)


def layer_norm(x, w, b, eps, y, f16=False, ctx=None, stream=None):
    _norm(lib().enc_layer_norm, x, w, b, eps, y, f16, ctx, stream)


def add_norm(h, t, w_post, eps, w_next=None, a=None, f16=False, post=1.0, gate=None, scale=None,
             cols=None, nout=1, oscale=1.0, ctx=None, stream=None):
    """h = (h + gate rms(t) w_post) post (t may be None: no update); then with
    w_next, `nout` copies a_z = rms(h) w_next (1 + scale) cols[z] oscale."""
    ctx = ctx or context()
    d = AddNormDesc()
    d.post = post
    d.gate, d.scale = _ptr(gate), _ptr(scale)
    for z, c in enumerate(cols or []):
        d.col[z] = _ptr(c)
    d.nout, d.oscale = nout, oscale
    d.rows, d.d = h.shape[0], h.shape[1]
    d.h, d.t, d.w_post, d.w_next, d.a = _ptr(h), _ptr(t), _ptr(w_post), _ptr(w_next), _ptr(a)
    d.eps = eps
    d.flags = ENC_Y_F16 if f16 else 0
    ctx.check(lib().enc_add_norm(ctx.h, C.byref(d), _stream(stream)))


def qk_norm_rope(panel, nq, nkv, hd, q_norm_w, k_norm_w, eps, cos, sin, sections, q_col=0,
                 k_col=None, path=ENC_F32, v_col=None, v_norm=False, ctx=None, stream=None):
    ctx = ctx or context()
    d = QkDesc()
    d.path = path
    d.panel = _ptr(panel)
    d.rows, d.ld = panel.shape[0], panel.stride(0)
    d.q_col = q_col
    d.k_col = k_col if k_col is not None else nq * hd
    d.nq, d.nkv, d.hd = nq, nkv, hd
    d.q_norm_w, d.k_norm_w = _ptr(q_norm_w), _ptr(k_norm_w)
    d.eps = eps
    d.cos, d.sin = _ptr(cos), _ptr(sin)
    d.sections = sections
    d.v_col = v_col if v_col is not None else d.k_col + nkv * hd
    d.v_norm = 1 if v_norm else 0
    ctx.check(lib().enc_qk_norm_rope(ctx.h, C.byref(d), _stream(stream)))


def gated_act(g, u, out, kind, f16=False, out_col=None, out_scale=1.0, ctx=None, stream=None):
    ctx = ctx or context()
    d = ActDesc()
    d.out_col, d.out_scale = _ptr(out_col), out_scale
    d.kind, d.rows, d.ff = kind, g.shape[0], g.shape[1]
    d.g, d.ldg, d.u, d.ldu = _ptr(g), g.stride(0), _ptr(u), u.stride(0)
    d.out, d.ldo = _ptr(out), out.stride(0)
    d.flags = ENC_Y_F16 if f16 else 0
    ctx.check(lib().enc_gated_act(ctx.h, C.byref(d), _stream(stream)))


def prof_enable(on=True, ctx=None):
    ctx = ctx or context()
    ctx.check(lib().enc_prof_enable(ctx.h, 1 if on else 0))


def prof_read(ctx=None):
    """{class: dict(launches, ms, flops, bytes)} since the previous read."""
    ctx = ctx or context()
    st = (ProfStat * 3)()
    ctx.check(lib().enc_prof_read(ctx.h, st))
    return {CLASS_NAMES[i]: dict(launches=st[i].launches, ms=st[i].ms, flops=st[i].flops,
                                 bytes=st[i].bytes) for i in range(3)}


def mfma_peak(path, blocks=2048, iters=2000, reps=3, ctx=None):
    """Measured MFMA ceiling in TFLOP/s (best of `reps` launches, timed with events)."""
    import torch
    ctx = ctx or context()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    fl = C.c_double()
    s = torch.cuda.current_stream()
    best = 0.0
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        ctx.check(lib().enc_mfma_peak(ctx.h, path, blocks, iters, _ptr(out), C.byref(fl),
                                      s.cuda_stream))
        e1.record(s)
        torch.cuda.synchronize()
        best = max(best, fl.value / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def mean_pool(a, items, out, ctx=None, stream=None):
    ctx = ctx or context()
    arr = make_items(items)
    ctx.check(lib().enc_mean_pool(ctx.h, a.shape[0], a.shape[1], _ptr(a), arr, len(items),
                                  _ptr(out), _stream(stream)))


# ------------------------------------------------------------------ host helpers

def positions(rows, items, grids, sections):
    pos = np.zeros((rows, sections), np.int32)
    g = np.ascontiguousarray(grids if grids is not None else [0] * len(items), np.uint32)
    st = lib().enc_positions(rows, make_items(items), g.ctypes.data, len(items), sections,
                             pos.ctypes.data)
    if st != ENC_OK:
        raise EncError(st, "enc_positions")
    return pos


def rope_table(pos, hd, sections, base):
    rows = pos.shape[0]
    pos = np.ascontiguousarray(pos, np.int32)
    cos = np.zeros((rows, hd // 2), np.float32)
    sin = np.zeros((rows, hd // 2), np.float32)
    st = lib().enc_rope_table(rows, hd, sections, pos.ctypes.data, base, cos.ctypes.data,
                              sin.ctypes.data)
    if st != ENC_OK:
        raise EncError(st, "enc_rope_table")
    return cos, sin


def check_gemm(desc, items):
    msg = C.create_string_buffer(512)
    arr = (GemmItem * max(1, len(items)))(*[GemmItem(*it) for it in items])
    st = lib().enc_check_gemm(C.byref(desc) if desc is not None else None, arr, len(items), msg,
                              512)
    return st, msg.value.decode()


def check_attention(desc, items):
    msg = C.create_string_buffer(512)
    st = lib().enc_check_attention(C.byref(desc) if desc is not None else None,
                                   make_items(items), len(items), msg, 512)
    return st, msg.value.decode()


def check_model(model, batch):
    msg = C.create_string_buffer(512)
    st = lib().enc_check_model(C.byref(model) if model is not None else None,
                               C.byref(batch) if batch is not None else None, msg, 512)
    return st, msg.value.decode()
