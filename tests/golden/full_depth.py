"""Stored oracle outputs of whole stacks too slow to run inside a GPU test.

The full-depth parity tests compare the GPU forward of a benchmark workload
(every layer, every row of the packed batch) with the f64 oracle.  For the
DiT stacks and the full text-encoder batch one oracle forward takes from
minutes (the 16-sequence text batch, the 30-layer 1056-row DiT) to hours (the
30-layer 8448-row CFG pair), so this script runs the oracle once on the host
and stores the outputs of sampled rows (or every pooled row) under
`tests/golden/full_depth_<workload>.npz`.

Only the oracle and the seeded input draws are called: no expected value comes
from the HIP library.  Each file carries a key, the SHA-256 of the oracle
source, of the draw module, of the workload's configuration and item table, and
of the inputs themselves (the input rows, every float tensor of every layer,
and the first, middle and last rows of every int8 weight, drawn on their own).
A test recomputes the key from the workload it builds and refuses a stale file.
The DiT step program (`zimage_dit_step_1056`: context refiner on the caption
rows, noise refiner on the image rows, then the stack) runs its stages in place
as the oracle's `forward_stages` does, and its key covers every stage's inputs.

    python tests/golden/full_depth.py gemma_text_f32 zimage_dit_1056 ...

Rows stored: for a pooled output every item's row; otherwise, per item and
range, its first two, middle and last two rows, the rows at offsets 127, 128,
255 and 256 of a range (the edges of the GEMM and attention tiles) and four
seeded draws per item.

The CFG pairs (8448 rows; the padded pair) store their first item only, and
the oracle runs that item alone (its rows, as the single-item layout orders
them, with the pair's positions of those rows where they are explicit): a packed
item shares no row with another in attention and every other step is
row-local, so by the definition of a packed batch the item's rows of the pair's
forward are the forward of the item alone.  That halves an oracle run of
hours.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from transformer_encoder_forward_amd import workloads as wl  # noqa: E402  (draws and shapes only)

ORACLE_SRC = os.path.join(ROOT, "oracle", "oracle.c")
SYNTH_SRC = os.path.join(ROOT, "transformer_encoder_forward_amd", "synth.py")

WORKLOADS = ("gemma_text_f32", "gemma_text_ple_f32", "zimage_dit_1056", "zimage_dit_cfg_8448",
             "zimage_dit_pad_cfg", "zimage_dit_mod_1056", "zimage_dit_step_1056")
FIRST_ITEM_ONLY = ("zimage_dit_cfg_8448", "zimage_dit_pad_cfg")  # the oracle runs item 0 alone (module doc)


def positions(w):
    """The rows' positions when the workload needs the padded-item rule stated in
    tests/positions_ref.py (pad rows at (0, 0)), else None (the oracle's own)."""
    if not w.cfg.get("pad_to"):
        return None
    tests_dir = os.path.dirname(HERE)
    if tests_dir not in sys.path:
        sys.path.insert(0, tests_dir)
    from positions_ref import dit_positions
    return dit_positions(w.rows, w.items, w.grids)


def path_for(name: str) -> str:
    return os.path.join(HERE, f"full_depth_{name}.npz")


def _file_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def key(w, pos=None) -> str:
    """SHA-256 identifying the oracle source, the draw module and every input of
    workload `w` (built with or without its int8 weights in host memory), and
    the positions when they are given explicitly."""
    h = hashlib.sha256()
    if pos is not None:
        h.update(np.ascontiguousarray(pos, np.int32).tobytes())
    h.update(_file_sha(ORACLE_SRC).encode())
    h.update(_file_sha(SYNTH_SRC).encode())
    h.update(json.dumps(w.cfg, sort_keys=True).encode())
    h.update(json.dumps([w.rows, w.items, w.grids]).encode())
    h.update(np.ascontiguousarray(w.x, np.float32).tobytes())
    _hash_layers(h, w)
    for a in (w.final_w, w.final_b):
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    # a staged program: each refiner stage's rows, items, config and weights
    for label, st, row0 in w.stages:
        if st is w:
            continue
        h.update(f"{label}@{row0}".encode())
        h.update(json.dumps(st.cfg, sort_keys=True).encode())
        h.update(json.dumps([st.rows, st.items, st.grids]).encode())
        _hash_layers(h, st)
    return h.hexdigest()


def _hash_layers(h, w) -> None:
    """The layers' float tensors and scalars whole; int8 weights by three rows
    each (drawn by the seeded generator, so a row pins the draw)."""
    shapes = wl.weight_shapes(w.cfg)
    for li, t in enumerate(w.layers):
        for name in sorted(t):
            v = t[name]
            if isinstance(v, np.ndarray):
                if v.dtype == np.int8:
                    continue  # present only when not lazy; fingerprinted below
                h.update(name.encode())
                h.update(np.ascontiguousarray(v).tobytes())
            else:
                h.update(f"{name}={v!r}".encode())
        if w.cfg["path"] == wl.PATH_I8F16:
            for name, shape in sorted(shapes.items()):
                m = shape[0]
                for r in (0, m // 2, m - 1):
                    h.update(wl.int8_weight_rows(w.seed, li, name, shape, r, r + 1,
                                                 w.prefix).tobytes())


def item_rows(rr) -> np.ndarray:
    """The rows of an item, its ranges in order."""
    return np.concatenate([np.arange(r0, r0 + n) for r0, n in rr])


def sample_rows(w) -> np.ndarray:
    """The output rows a file stores (see the module doc)."""
    if w.cfg["final"] == wl.FINAL_RMS_MEANPOOL:
        return np.arange(len(w.items))
    items = w.items[:1] if w.name in FIRST_ITEM_ONLY else w.items
    rows = []
    for ii, rr in enumerate(items):
        for r0, n in rr:
            for o in (0, 1, n // 2, n - 2, n - 1, 127, 128, 255, 256):
                if 0 <= o < n:
                    rows.append(r0 + o)
        rng = np.random.default_rng(ii + 1)
        rows += [int(v) for v in rng.choice(item_rows(rr), 4, replace=False)]
    return np.unique(np.asarray(rows, np.int64))


def load(name: str, w):
    """(rows, expected outputs of those rows) for workload `w`; raises when the
    file is missing or was written for other inputs or another oracle."""
    p = path_for(name)
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} is missing: run python tests/golden/full_depth.py {name}")
    z = np.load(p, allow_pickle=False)
    k = key(w, positions(w))
    if str(z["key"]) != k:
        raise ValueError(f"{p} is stale (inputs or oracle changed): rerun "
                         f"python tests/golden/full_depth.py {name}")
    return z["rows"], z["out"]


def write(name: str) -> None:
    import oracle as O

    O.build(force=False)
    w = wl.make(name)
    pos = positions(w)
    k = key(w, pos)
    rows = sample_rows(w)
    print(f"{name}: {w.rows} rows, {w.cfg['layers']} layers, {len(rows)} stored rows, "
          f"oracle threads {O.threads()}", flush=True)
    t0 = time.time()
    if name in FIRST_ITEM_ONLY:
        # item 0 alone, in the single-item layout of the same model (with the
        # pair's positions of its rows, when they are explicit)
        idx = item_rows(w.items[0])
        srows, sitems, sgrids = wl.layout(w.cfg, cfg_pair=False)
        assert srows == len(idx)
        single = wl.Workload(name=w.name, cfg=w.cfg, rows=srows, items=sitems, grids=sgrids,
                             x=w.x[idx], seed=w.seed)
        single.layers, single.final_w, single.final_b = w.layers, w.final_w, w.final_b
        out = np.zeros((w.rows, w.cfg["d"]))
        out[idx] = O.forward(single, pos=None if pos is None else pos[idx])
        assert np.isin(rows, idx).all()
    elif w.stages:
        # the staged program: each stage in place on its rows, with its rows'
        # positions in the joint table of the whole batch
        joint = O.positions(w.rows, w.items, w.grids, w.cfg["rope_sections"])
        out = O.forward_stages([(st, r0, joint[r0:r0 + st.rows]) for _, st, r0 in w.stages], w.x)
    else:
        out = O.forward(w, pos=pos)
    dt = time.time() - t0
    print(f"{name}: oracle forward {dt:.1f} s", flush=True)
    np.savez_compressed(path_for(name), key=np.array(k), rows=rows, out=out[rows],
                        oracle_seconds=np.array(dt), oracle_threads=np.array(O.threads()))


if __name__ == "__main__":
    names = sys.argv[1:] or list(WORKLOADS)
    for n in names:
        if n not in WORKLOADS:
            raise SystemExit(f"unknown workload {n}; one of {WORKLOADS}")
    for n in names:
        write(n)
