"""GPU parity of each op behind the C ABI against the f64 oracle.

Integer-valued operands make every partial sum exact in f32 and f64, so those
GEMM cases must match the oracle bit for bit (this pins offsets, strides, the
weight slot, the MFMA output layout, bias and accumulate).  Random operands are
held to the path's tolerance.  Attention is checked against brute force, with
the one-hot mask probe bit-exact, and packed == separate bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, TOL_F32, TOL_I8F16, host, row_rel_err, say, to_dev
from transformer_encoder_forward_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    B.context(0)


# ---------------------------------------------------------------- GEMM f32

@pytest.mark.parametrize("n,m,k", [(1, 1, 4), (37, 70, 36), (130, 257, 128), (257, 128, 512),
                                   (64, 384, 128), (300, 96, 2048),
                                   (8001, 1000, 96),    # 256 x 128 tiles, ragged rows and columns
                                   (4100, 4000, 64),    # 128 x 128 tiles
                                   # K split four ways inside the block (m <= 768, K >= 3072)
                                   (300, 700, 3200), (1024, 768, 3072)])
def test_gemm_f32_integer_exact(n, m, k):
    say(f"gemm f32 integer n={n} m={m} k={k}")
    rng = np.random.default_rng(n * 31 + m * 7 + k)
    x = rng.integers(-8, 9, (n, k)).astype(np.float32)
    w = rng.integers(-8, 9, (m, k)).astype(np.float32)
    b = rng.integers(-5, 6, m).astype(np.float32)
    y0 = rng.integers(-100, 100, (n, m)).astype(np.float32)
    ref = O.linear(x, w, b)
    X, Wd, Bd = to_dev(x), to_dev(w), to_dev(b)
    Y = torch.zeros((n, m), dtype=torch.float32, device=DEV)
    B.gemm_items(X, Y, [Wd], [(n, m, k, k, m, 0, 0, 0)], bias=[Bd])
    assert np.array_equal(host(Y), ref)
    Y = to_dev(y0)
    B.gemm_items(X, Y, [Wd], [(n, m, k, k, m, 0, 0, 0)], bias=[Bd], flags=B.ENC_Y_ACCUMULATE)
    assert np.array_equal(host(Y), ref + y0)


def test_gemm_f32_qkv_items_one_launch():
    """q|k|v as three items of one launch into one panel at column offsets,
    rows offset and strided input (x_off, ldx > k)."""
    rng = np.random.default_rng(11)
    n, d, qw, kw = 150, 128, 128, 64
    ldx = d + 8
    xfull = rng.integers(-8, 9, (n + 3, ldx)).astype(np.float32)
    ws = [rng.integers(-8, 9, (mm, d)).astype(np.float32) for mm in (qw, kw, kw)]
    ld = qw + 2 * kw
    Y = torch.full((n, ld), -7.0, dtype=torch.float32, device=DEV)
    items = [(n, qw, d, ldx, ld, 0, 3 * ldx, 0), (n, kw, d, ldx, ld, 1, 3 * ldx, qw),
             (n, kw, d, ldx, ld, 2, 3 * ldx, qw + kw)]
    B.gemm_items(to_dev(xfull), Y, [to_dev(w) for w in ws], items)
    x = xfull[3:, :d]
    ref = np.concatenate([O.linear(x, w) for w in ws], 1)
    assert np.array_equal(host(Y), ref)


@pytest.mark.parametrize("n,m,k", [(64, 384, 128), (1000, 1536, 512), (333, 512, 2048),
                                   (1024, 3072, 768), (1024, 768, 3072), (77, 300, 4096),
                                   # more tiles than resident blocks: blocks loop over tiles
                                   (9001, 1536, 256), (4099, 1536, 512)])
def test_gemm_f32_random(n, m, k):
    say(f"gemm f32 random n={n} m={m} k={k}")
    rng = np.random.default_rng(n + m + k)
    x = rng.normal(0, 1, (n, k)).astype(np.float32)
    w = (0.02 * rng.normal(0, 1, (m, k))).astype(np.float32)
    Y = torch.empty((n, m), dtype=torch.float32, device=DEV)
    B.gemm_items(to_dev(x), Y, [to_dev(w)], [(n, m, k, k, m, 0, 0, 0)])
    err = row_rel_err(host(Y), O.linear(x, w))
    say(f"  err {err:.2e}")
    assert err <= TOL_F32


def test_gemm_f32_items_of_different_k_many_tiles():
    """Two items of different K in one launch with more tiles than resident
    blocks, so that blocks work through tiles of both items in turn."""
    rng = np.random.default_rng(12)
    n, k0, k1, m0, m1 = 6000, 512, 2048, 1536, 512
    x = rng.integers(-8, 9, (n, k1)).astype(np.float32)
    w0 = rng.integers(-8, 9, (m0, k0)).astype(np.float32)
    w1 = rng.integers(-8, 9, (m1, k1)).astype(np.float32)
    ld = m0 + m1
    Y = torch.full((n, ld), -7.0, dtype=torch.float32, device=DEV)
    items = [(n, m0, k0, k1, ld, 0, 0, 0), (n, m1, k1, k1, ld, 1, 0, m0)]
    B.gemm_items(to_dev(x), Y, [to_dev(w0), to_dev(w1)], items)
    ref = np.concatenate([O.linear(x[:, :k0], w0), O.linear(x, w1)], 1)
    assert np.array_equal(host(Y), ref)


def test_gemm_f32_split_and_plain_items_one_launch():
    """A launch mixing an item whose K is split inside the block (768 outputs,
    K 3072) with plain items gives each item the bits it gets alone."""
    rng = np.random.default_rng(21)
    n, k = 700, 3072
    x = rng.normal(0, 1, (n, k)).astype(np.float32)
    ws = [rng.normal(0, 0.02, (768, k)).astype(np.float32), rng.normal(0, 0.02, (512, 512)).astype(np.float32)]
    ld = 768 + 512
    X, Wd = to_dev(x), [to_dev(w) for w in ws]
    Y = torch.empty((n, ld), dtype=torch.float32, device=DEV)
    items = [(n, 768, k, k, ld, 0, 0, 0), (n, 512, 512, k, ld, 1, 0, 768)]
    B.gemm_items(X, Y, Wd, items)
    for it in items:
        alone = torch.empty((n, ld), dtype=torch.float32, device=DEV)
        B.gemm_items(X, alone, Wd, [it])
        c0, m = it[7], it[1]
        assert torch.equal(alone[:, c0:c0 + m], Y[:, c0:c0 + m])
    ref = np.concatenate([O.linear(x, ws[0]), O.linear(x[:, :512], ws[1])], 1)
    assert row_rel_err(host(Y), ref) <= TOL_F32


def test_gemm_f32_gelu_epilogue():
    rng = np.random.default_rng(5)
    n, m, k = 77, 200, 64
    x = rng.normal(0, 1, (n, k)).astype(np.float32)
    w = (0.3 * rng.normal(0, 1, (m, k))).astype(np.float32)
    b = (0.1 * rng.normal(0, 1, m)).astype(np.float32)
    Y = torch.empty((n, m), dtype=torch.float32, device=DEV)
    B.gemm_items(to_dev(x), Y, [to_dev(w)], [(n, m, k, k, m, 0, 0, 0)], bias=[to_dev(b)],
                 flags=B.ENC_EPI_GELU_TANH)
    ref = np.vectorize(O.gelu_tanh)(O.linear(x, w, b))
    assert row_rel_err(host(Y), ref) <= TOL_F32


@pytest.mark.parametrize("n,m,k,gated", [
    (900, 300, 512, False),      # small launches only (64 x 64, direct loads)
    (8192, 1536, 512, False),    # 256 x 128 direct-loaded tiles vs the 64 x 64 ones
    (8192, 1536, 100, False),    # K % 32 != 0: the register-staged 256 x 128 vs 64 x 64
    (8192, 2048, 512, True),     # gated: 256 x (128 + 128) direct vs 64 x (64 + 64) direct
    (8192, 2048, 100, True),     # gated, register-staged tiles
    (1100, 768, 3072, False)])   # K split inside the block at every launch size
def test_gemm_f32_packed_rows_bit_identical(n, m, k, gated):
    """A row's output bits do not depend on how many rows share the launch, so
    not on which tile shape or staging the launch size selects."""
    rng = np.random.default_rng(6 + k)
    x = rng.normal(0, 1, (n, k)).astype(np.float32)
    ws = [to_dev(rng.normal(0, 0.02, (m, k)).astype(np.float32)) for _ in range(1 + gated)]
    flags = B.ENC_EPI_GATE_GELU_TANH if gated else 0
    Yall = torch.empty((n, m), dtype=torch.float32, device=DEV)
    B.gemm_items(to_dev(x), Yall, ws, [(n, m, k, k, m, 0, 0, 0)], flags=flags)
    for r0, r1 in ((0, 1), (129, 200), (700, 900)):
        Y = torch.empty((r1 - r0, m), dtype=torch.float32, device=DEV)
        B.gemm_items(to_dev(x[r0:r1]), Y, ws, [(r1 - r0, m, k, k, m, 0, 0, 0)], flags=flags)
        assert torch.equal(Y, Yall[r0:r1])


@pytest.mark.parametrize("path,act,n,ff,d", [
    (B.ENC_F32, "gelu", 1000, 2048, 512), (B.ENC_F32, "gelu", 37, 200, 128),
    (B.ENC_I8F16, "silu", 300, 1280, 256), (B.ENC_I8F16, "silu", 45, 96, 64),
    (B.ENC_I8F16, "silu", 520, 12800, 128), (B.ENC_I8F16, "gelu", 300, 25600, 192),
    (B.ENC_I8F16, "silu", 77, 160, 80), (B.ENC_F32, "gelu", 8001, 2048, 512),
    (B.ENC_I8F16, "silu", 1300, 11000, 128),    # >= 512 tiles: the 256 x (128 + 128) int8 tile
    (B.ENC_I8F16, "silu", 200, 2560, 320), (B.ENC_I8F16, "silu", 200, 2560, 448)])
def test_gemm_gated_equals_unfused(path, act, n, ff, d):
    """act(gate) * up formed in the GEMM epilogue == gate/up GEMM + enc_gated_act,
    bit for bit, and == the oracle within tolerance."""
    rng = np.random.default_rng(n + ff)
    i8 = path == B.ENC_I8F16
    if i8:
        x = rng.normal(0, 1, (n, d)).astype(np.float16)
        ws = [rng.integers(-127, 128, (ff, d)).astype(np.int8) for _ in range(2)]
        rss = [(0.002 * np.exp(0.25 * rng.normal(0, 1, ff))).astype(np.float32) for _ in range(2)]
        rs = [to_dev(r) for r in rss]
    else:
        x = rng.normal(0, 1, (n, d)).astype(np.float32)
        ws = [rng.normal(0, 0.05, (ff, d)).astype(np.float32) for _ in range(2)]
        rs = None
    X, W = to_dev(x), [to_dev(w) for w in ws]
    odt = torch.float16 if i8 else torch.float32
    gflag = B.ENC_EPI_GATE_GELU_TANH if act == "gelu" else B.ENC_EPI_GATE_SILU
    fused = torch.empty((n, ff), dtype=odt, device=DEV)
    B.gemm_items(X, fused, W, [(n, ff, d, d, ff, 0, 0, 0)], path=path, row_scale=rs,
                 flags=gflag | (B.ENC_Y_F16 if i8 else 0))
    gu = torch.empty((n, 2 * ff), dtype=torch.float32, device=DEV)
    B.gemm_items(X, gu, W, [(n, ff, d, d, 2 * ff, 0, 0, 0), (n, ff, d, d, 2 * ff, 1, 0, ff)],
                 path=path, row_scale=rs)
    unfused = torch.empty((n, ff), dtype=odt, device=DEV)
    kind = B.ENC_ACT_GELU_TANH_GATED if act == "gelu" else B.ENC_ACT_SWIGLU
    B.gated_act(gu[:, :ff], gu[:, ff:], unfused, kind, f16=i8)
    assert torch.equal(fused, unfused)
    # the oracle's scalar activations: every row of small cases, sampled rows of large ones
    rows = np.arange(n) if n * ff <= 2_000_000 else np.array([0, 1, 255, 256, n - 1])
    xd = x[rows].astype(np.float64)
    if i8:
        g, u = O.linear_q8(xd, ws[0], rss[0]), O.linear_q8(xd, ws[1], rss[1])
    else:
        g, u = O.linear(xd, ws[0]), O.linear(xd, ws[1])
    ref = np.vectorize(O.gelu_tanh if act == "gelu" else O.silu)(g) * u
    if i8:
        ref = np.vectorize(O.round_f16)(ref)
    assert row_rel_err(host(fused)[rows], ref) <= (TOL_I8F16 if i8 else TOL_F32)


# ------------------------------------------------------------- GEMM int8 x f16

@pytest.mark.parametrize("n,m,k", [(1, 1, 16), (45, 70, 48), (130, 257, 256), (300, 128, 3840)])
def test_gemm_i8f16_integer_exact(n, m, k):
    say(f"gemm i8f16 integer n={n} m={m} k={k}")
    rng = np.random.default_rng(n * 3 + m + k)
    x = rng.integers(-16, 17, (n, k)).astype(np.float16)
    q = rng.integers(-127, 128, (m, k)).astype(np.int8)
    rs = (2.0 ** -rng.integers(0, 10, m)).astype(np.float32)
    ref = O.linear_q8(x.astype(np.float64), q, rs)
    Y = torch.empty((n, m), dtype=torch.float32, device=DEV)
    B.gemm_items(to_dev(x), Y, [to_dev(q)], [(n, m, k, k, m, 0, 0, 0)], path=B.ENC_I8F16,
                 row_scale=[to_dev(rs)])
    assert np.array_equal(host(Y), ref)


# shapes that take the direct-to-LDS kernel (K % 64 == 0): 256 x 256 tiles (>= 256
# of them), 128 x 256 tiles (the 520- and 513-row launches: more than 512 tiles of
# 64 x 256) and 64 x 256 tiles; one K stage, exactly the LDS ring, ring
# wrap-around; ragged rows and columns
@pytest.mark.parametrize("n,m,k", [(1300, 11000, 64), (1300, 11000, 192), (1283, 11000, 320),
                                   (520, 17000, 64), (513, 17000, 320),
                                   (130, 1000, 64), (257, 3000, 192), (1, 300, 320),
                                   # small launches, K stages 2 and 6 to 8 (deeper rings)
                                   (130, 1000, 128), (200, 900, 384), (77, 1000, 448),
                                   (257, 700, 512)])
def test_gemm_i8f16_wide_tiles_integer_exact(n, m, k):
    say(f"gemm i8f16 wide integer n={n} m={m} k={k}")
    rng = np.random.default_rng(n + m + k)
    x = rng.integers(-16, 17, (n, k)).astype(np.float16)
    q = rng.integers(-127, 128, (m, k)).astype(np.int8)
    rs = (2.0 ** -rng.integers(0, 10, m)).astype(np.float32)
    ref = O.linear_q8(x.astype(np.float64), q, rs)
    Y = torch.empty((n, m), dtype=torch.float32, device=DEV)
    B.gemm_items(to_dev(x), Y, [to_dev(q)], [(n, m, k, k, m, 0, 0, 0)], path=B.ENC_I8F16,
                 row_scale=[to_dev(rs)])
    assert np.array_equal(host(Y), ref)


def test_gemm_i8f16_kernel_choice_bit_identical():
    """Rows computed in a launch of 256 x 256 tiles (1600 rows), a 1300-row
    launch of 128 x 256 tiles, an 800-row launch of 96 x 256 tiles (both
    two-stage rings, two blocks per CU) and small launches of 64 x 256 tiles
    give the same bits (one K order for every int8 kernel)."""
    rng = np.random.default_rng(77)
    n, m, k = 1600, 11000, 256
    x = rng.normal(0, 1, (n, k)).astype(np.float16)
    W = to_dev(rng.integers(-127, 128, (m, k)).astype(np.int8))
    rs = [to_dev((0.002 * np.exp(0.25 * rng.normal(0, 1, m))).astype(np.float32))]
    Yall = torch.empty((n, m), dtype=torch.float32, device=DEV)
    B.gemm_items(to_dev(x), Yall, [W], [(n, m, k, k, m, 0, 0, 0)], path=B.ENC_I8F16, row_scale=rs)
    for r0, r1 in ((0, 1), (250, 300), (450, 520), (1100, 1600), (100, 1400), (300, 1100)):
        Y = torch.empty((r1 - r0, m), dtype=torch.float32, device=DEV)
        B.gemm_items(to_dev(x[r0:r1]), Y, [W], [(r1 - r0, m, k, k, m, 0, 0, 0)], path=B.ENC_I8F16,
                     row_scale=rs)
        assert torch.equal(Y, Yall[r0:r1])


def test_gemm_i8f16_beyond_31_bit_offsets_bit_identical():
    """An item whose X spans more than 2^31 bytes (300 000 rows of K 3840) takes
    the register-staged kernel (the direct loads address by 32-bit offsets);
    its first and last rows equal the same rows computed alone by the
    direct-loaded kernel, bit for bit."""
    n, m, k = 300_000, 128, 3840
    assert (n - 1) * k * 2 >= 2 ** 31
    g = torch.Generator(device=DEV).manual_seed(5)
    x = torch.randn((n, k), generator=g, device=DEV).to(torch.float16)
    rng = np.random.default_rng(78)
    W = to_dev(rng.integers(-127, 128, (m, k)).astype(np.int8))
    rs = [to_dev((0.002 * np.exp(0.25 * rng.normal(0, 1, m))).astype(np.float32))]
    Y = torch.empty((n, m), dtype=torch.float32, device=DEV)
    B.gemm_items(x, Y, [W], [(n, m, k, k, m, 0, 0, 0)], path=B.ENC_I8F16, row_scale=rs)
    for r0, r1 in ((0, 64), (n - 100, n)):
        Ys = torch.empty((r1 - r0, m), dtype=torch.float32, device=DEV)
        B.gemm_items(x[r0:r1].contiguous(), Ys, [W], [(r1 - r0, m, k, k, m, 0, 0, 0)], path=B.ENC_I8F16,
                     row_scale=rs)
        assert torch.equal(Ys, Y[r0:r1]), (r0, r1)
    del x, Y
    torch.cuda.empty_cache()


def test_gemm_i8f16_gated_kernel_choice_bit_identical():
    """Gated int8 rows computed in a launch of 256 x (128 + 128) tiles (1300
    rows), of 192 x (128 + 128) tiles (1000 and 390 rows, ragged last tiles)
    and of 128 x (128 + 128) tiles (200 rows and fewer) give the same bits."""
    rng = np.random.default_rng(79)
    n, ff, d = 1300, 10240, 256
    x = rng.normal(0, 1, (n, d)).astype(np.float16)
    W = [to_dev(rng.integers(-127, 128, (ff, d)).astype(np.int8)) for _ in range(2)]
    rs = [to_dev((0.002 * np.exp(0.25 * rng.normal(0, 1, ff))).astype(np.float32)) for _ in range(2)]
    flags = B.ENC_EPI_GATE_SILU | B.ENC_Y_F16
    Yall = torch.empty((n, ff), dtype=torch.float16, device=DEV)
    B.gemm_items(to_dev(x), Yall, W, [(n, ff, d, d, ff, 0, 0, 0)], path=B.ENC_I8F16, row_scale=rs, flags=flags)
    for r0, r1 in ((0, 1000), (300, 500), (1299, 1300), (100, 490)):
        Y = torch.empty((r1 - r0, ff), dtype=torch.float16, device=DEV)
        B.gemm_items(to_dev(x[r0:r1]), Y, W, [(r1 - r0, ff, d, d, ff, 0, 0, 0)], path=B.ENC_I8F16,
                     row_scale=rs, flags=flags)
        assert torch.equal(Y, Yall[r0:r1]), (r0, r1)


def test_gemm_i8f16_gated_last_row_tile_peel_bit_identical():
    """A one-item gated launch of 8448 rows (33 x 80 tiles of 256 x (128 + 128):
    ten rounds of 256 CUs and 80 tiles) issues its last 256 rows as a second
    launch of 128-row tiles; its rows equal those of the same rows as two items
    of one launch (no peel), bit for bit."""
    rng = np.random.default_rng(83)
    n, ff, d = 8448, 10240, 256
    x = to_dev(rng.normal(0, 1, (n, d)).astype(np.float16))
    W = [to_dev(rng.integers(-127, 128, (ff, d)).astype(np.int8)) for _ in range(2)]
    rs = [to_dev((0.002 * np.exp(0.25 * rng.normal(0, 1, ff))).astype(np.float32)) for _ in range(2)]
    flags = B.ENC_EPI_GATE_SILU | B.ENC_Y_F16
    Y1 = torch.empty((n, ff), dtype=torch.float16, device=DEV)
    B.gemm_items(x, Y1, W, [(n, ff, d, d, ff, 0, 0, 0)], path=B.ENC_I8F16, row_scale=rs, flags=flags)
    Y2 = torch.empty((n, ff), dtype=torch.float16, device=DEV)
    h = n // 2
    B.gemm_items(x, Y2, W, [(h, ff, d, d, ff, 0, 0, 0), (n - h, ff, d, d, ff, 0, h * d, h * ff)],
                 path=B.ENC_I8F16, row_scale=rs, flags=flags)
    assert torch.equal(Y1, Y2)
    assert torch.isfinite(Y1.float()).all()
    del Y1, Y2
    torch.cuda.empty_cache()


def test_gemm_i8f16_f16_output_and_items():
    rng = np.random.default_rng(12)
    n, d, f = 96, 256, 384
    x = rng.normal(0, 1, (n, d)).astype(np.float16)
    qs = [rng.integers(-127, 128, (f, d)).astype(np.int8) for _ in range(2)]
    rss = [(0.002 * np.exp(0.25 * rng.normal(0, 1, f))).astype(np.float32) for _ in range(2)]
    Y = torch.empty((n, 2 * f), dtype=torch.float16, device=DEV)
    items = [(n, f, d, d, 2 * f, 0, 0, 0), (n, f, d, d, 2 * f, 1, 0, f)]
    B.gemm_items(to_dev(x), Y, [to_dev(q) for q in qs], items, path=B.ENC_I8F16,
                 row_scale=[to_dev(r) for r in rss], flags=B.ENC_Y_F16)
    ref = np.concatenate([O.linear_q8(x.astype(np.float64), q, r) for q, r in zip(qs, rss)], 1)
    ref16 = np.vectorize(O.round_f16)(ref)
    assert row_rel_err(host(Y), ref16) <= TOL_I8F16


@pytest.mark.parametrize("m,k", [(11520, 3840), (3840, 3840), (10240, 3840), (3840, 10240)])
def test_gemm_i8f16_dit_shapes_sampled(m, k):
    """The DiT's four GEMM shapes at 1056 rows; sampled rows vs the oracle."""
    say(f"gemm i8f16 dit n=1056 m={m} k={k}")
    rng = np.random.default_rng(m + k)
    n = 1056
    x = (rng.normal(0, 1, (n, k))).astype(np.float16)
    q = rng.integers(-127, 128, (m, k)).astype(np.int8)
    rs = (0.002 * np.exp(0.25 * rng.normal(0, 1, m))).astype(np.float32)
    Y = torch.empty((n, m), dtype=torch.float32, device=DEV)
    B.gemm_items(to_dev(x), Y, [to_dev(q)], [(n, m, k, k, m, 0, 0, 0)], path=B.ENC_I8F16,
                 row_scale=[to_dev(rs)])
    rows = np.array([0, 1, 127, 128, 511, 1000, 1023, 1024, 1055])
    ref = O.linear_q8(x[rows].astype(np.float64), q, rs)
    err = row_rel_err(host(Y)[rows], ref)
    say(f"  err {err:.2e}")
    assert err <= 1e-5


# ------------------------------------------------------------------ attention

def _panel(rng, rows, nq, nkv, hd, f16=False, qscale=1.0):
    q = rng.normal(0, qscale, (rows, nq * hd))
    k = rng.normal(0, 1, (rows, nkv * hd))
    v = rng.normal(0, 1, (rows, nkv * hd))
    p = np.concatenate([q, k, v], 1)
    p = p.astype(np.float16 if f16 else np.float32)
    return p


def _split(p, nq, nkv, hd):
    p = p.astype(np.float64)
    return p[:, :nq * hd], p[:, nq * hd:(nq + nkv) * hd], p[:, (nq + nkv) * hd:]


ATTN_CASES = [
    ("single", [[(0, 64)]], 0),
    ("ragged", [[(0, 1)], [(1, 37)], [(38, 130)], [(168, 300)], [(468, 5)]], 0),
    ("window", [[(0, 700)], [(700, 33)], [(733, 260)]], 96),
    ("window_big", [[(0, 1100)]], 512),
    ("two_range", [[(0, 200), (420, 20)], [(200, 200), (440, 20)], [(400, 20)]], 0),
    # the range seam inside a key block of the split f16 kernel's first key half
    # (block 1 of 11 and of 5; "two_range" has it in the second half)
    ("two_range_seams", [[(0, 40), (100, 300)], [(40, 60), (400, 90)]], 0),
]


@pytest.mark.parametrize("name,items,window", ATTN_CASES)
@pytest.mark.parametrize("hd,nq,nkv", [(64, 4, 4), (64, 4, 2), (128, 2, 1)])
def test_attention_f32(name, items, window, hd, nq, nkv):
    say(f"attention f32 {name} hd={hd} nq={nq} nkv={nkv} W={window}")
    rows = max(r0 + n for rr in items for r0, n in rr)
    rng = np.random.default_rng(hd + nq + rows)
    p = _panel(rng, rows, nq, nkv, hd, qscale=0.5)
    out = torch.full((rows, nq * hd), 0.0, dtype=torch.float32, device=DEV)
    scale = 1.0 / np.sqrt(hd)
    B.attention_items(to_dev(p), out, items, nq, nkv, hd, scale, window)
    q, k, v = _split(p, nq, nkv, hd)
    ref = O.attention(items, q, k, v, nq, nkv, hd, scale, window)
    err = row_rel_err(host(out), ref)
    say(f"  err {err:.2e}")
    assert err <= TOL_F32


@pytest.mark.parametrize("name,items,window", ATTN_CASES)
@pytest.mark.parametrize("hd,nq,nkv", [(128, 4, 4), (64, 4, 2)])
def test_attention_f16(name, items, window, hd, nq, nkv):
    say(f"attention f16 {name} hd={hd} nq={nq} nkv={nkv} W={window}")
    rows = max(r0 + n for rr in items for r0, n in rr)
    rng = np.random.default_rng(hd * 3 + nq + rows)
    p = _panel(rng, rows, nq, nkv, hd, f16=True, qscale=0.5)
    out = torch.zeros((rows, nq * hd), dtype=torch.float16, device=DEV)
    scale = 1.0 / np.sqrt(hd)
    B.attention_items(to_dev(p), out, items, nq, nkv, hd, scale, window, path=B.ENC_I8F16)
    q, k, v = _split(p, nq, nkv, hd)
    ref = np.vectorize(O.round_f16)(O.attention(items, q, k, v, nq, nkv, hd, scale, window))
    err = row_rel_err(host(out), ref)
    say(f"  err {err:.2e}")
    assert err <= TOL_I8F16


def test_attention_f16_wide_launch_two_range_sampled():
    """A launch wide enough for the 256-query f16 blocks (nq 24, GQA 3:1), with
    two-range items whose first range ends inside a 32-key block, a ragged last
    block and a one-row item; sampled query rows of every range against the
    oracle."""
    items = [[(0, 3001), (6100, 37)], [(3001, 3099), (6137, 50)], [(6187, 1)]]
    rows, nq, nkv, hd = 6188, 24, 8, 128
    rng = np.random.default_rng(11)
    p = _panel(rng, rows, nq, nkv, hd, f16=True, qscale=0.5)
    out = torch.zeros((rows, nq * hd), dtype=torch.float16, device=DEV)
    scale = 1.0 / np.sqrt(hd)
    B.attention_items(to_dev(p), out, items, nq, nkv, hd, scale, 0, path=B.ENC_I8F16)
    sel = []
    for rr in items:
        for r0, n in rr:
            sel += [r0, r0 + 1, r0 + n // 2, r0 + n - 2, r0 + n - 1]
    sel = np.unique(np.clip(sel + list(rng.integers(0, rows, 24)), 0, rows - 1))
    q, k, v = _split(p, nq, nkv, hd)
    ref = O.attention(items, q, k, v, nq, nkv, hd, scale, 0, query_rows=sel)[sel]
    ref = np.vectorize(O.round_f16)(ref)
    err = row_rel_err(host(out)[sel], ref)
    say(f"  {len(sel)} sampled queries, err {err:.2e}")
    assert err <= TOL_I8F16


def test_attention_f16_split_keys_short_items():
    """Items of 1 to 10 key blocks, which take the kernel that splits each
    query's keys two ways inside the block (every count of blocks per half,
    an empty second half at one block, ragged last blocks, GQA 4:1): every row
    against the oracle, and three items alone give the packed rows' bits."""
    lens = [1, 31, 32, 33, 64, 65, 96, 97, 128, 160, 161, 192, 193, 224, 255, 256, 257, 300]
    items, r = [], 0
    for n in lens:
        items.append([(r, n)])
        r += n
    rows, nq, nkv, hd = r, 32, 8, 128
    rng = np.random.default_rng(21)
    p = _panel(rng, rows, nq, nkv, hd, f16=True, qscale=0.5)
    P = to_dev(p)
    out = torch.zeros((rows, nq * hd), dtype=torch.float16, device=DEV)
    scale = 1.0 / np.sqrt(hd)
    B.attention_items(P, out, items, nq, nkv, hd, scale, 0, path=B.ENC_I8F16)
    q, k, v = _split(p, nq, nkv, hd)
    ref = O.attention(items, q, k, v, nq, nkv, hd, scale, 0)  # f64; the output's f16 rounding is in the bar
    err = row_rel_err(host(out), ref)
    say(f"  {len(items)} items, err {err:.2e}")
    assert err <= TOL_I8F16
    for i in (0, 9, 17):
        (r0, n), = items[i]
        o1 = torch.zeros((n, nq * hd), dtype=torch.float16, device=DEV)
        B.attention_items(to_dev(p[r0:r0 + n]), o1, [[(0, n)]], nq, nkv, hd, scale, 0, path=B.ENC_I8F16)
        assert torch.equal(o1, out[r0:r0 + n]), f"item {i} ({n} rows)"


def test_attention_f16_long_items_ring_and_split_boundary():
    """At nq 32 items of more than 1024 rows (more than 16 blocks of 64
    queries per head) take the pipelined kernel: 33 and 50 to 55 key blocks
    (every count modulo its six-stage ring, ragged last blocks) in a launch
    wide enough for 256-query blocks (GQA 4:1), next to a 1024-row item that
    takes the split-key kernel; sampled query rows of every item against the
    oracle, and items alone give the packed rows' bits (the 1025-row one alone
    runs 128-query blocks)."""
    lens = [1024, 1025, 1569, 1601, 1664, 1665, 1727, 1760]
    items, r = [], 0
    for n in lens:
        items.append([(r, n)])
        r += n
    rows, nq, nkv, hd = r, 32, 8, 128
    rng = np.random.default_rng(23)
    p = _panel(rng, rows, nq, nkv, hd, f16=True, qscale=0.5)
    out = torch.zeros((rows, nq * hd), dtype=torch.float16, device=DEV)
    scale = 1.0 / np.sqrt(hd)
    B.attention_items(to_dev(p), out, items, nq, nkv, hd, scale, 0, path=B.ENC_I8F16)
    sel = []
    for (r0, n), in items:
        sel += [r0, r0 + 31, r0 + 32, r0 + n // 2, r0 + n - 33, r0 + n - 1]
    sel = np.unique(np.array(sel + list(rng.integers(0, rows, 16))))
    q, k, v = _split(p, nq, nkv, hd)
    ref = O.attention(items, q, k, v, nq, nkv, hd, scale, 0, query_rows=sel)[sel]
    err = row_rel_err(host(out)[sel], ref)
    say(f"  {len(sel)} sampled queries, err {err:.2e}")
    assert err <= TOL_I8F16
    for i in (0, 1, 7):
        (r0, n), = items[i]
        o1 = torch.zeros((n, nq * hd), dtype=torch.float16, device=DEV)
        B.attention_items(to_dev(p[r0:r0 + n]), o1, [[(0, n)]], nq, nkv, hd, scale, 0, path=B.ENC_I8F16)
        assert torch.equal(o1, out[r0:r0 + n]), f"item {i} ({n} rows)"


@pytest.mark.parametrize("nq", [4, 128])
def test_attention_f16_panel_beyond_31_bit_offsets(nq):
    """Items at the end of a q/k/v panel of more than 2^31 bytes are staged by
    64-bit per-lane addresses instead of raw buffer loads (nq 4: the last item
    takes 128-query blocks, the others the split-key kernel; nq 128: the 33-
    and 256-row items the split-key kernel, the others 256-query blocks with
    the six-stage ring); their rows equal the same items in a small panel, bit
    for bit."""
    hd = 128
    ld = 3 * nq * hd
    lens = [300, 257, 33, 256, 8300 if nq == 4 else 1600]
    rows = (2 ** 31) // (ld * 2) + sum(lens) + 300
    r0 = rows - sum(lens)
    items, r = [], r0
    for n in lens:
        items.append([(r, n)])
        r += n
    g = torch.Generator(device=DEV).manual_seed(9)
    P = (torch.randn((rows, ld), generator=g, device=DEV) * 0.5).to(torch.float16)
    out = torch.zeros((rows, nq * hd), dtype=torch.float16, device=DEV)
    B.attention_items(P, out, items, nq, nq, hd, hd ** -0.5, 0, path=B.ENC_I8F16)
    small = P[r0:].contiguous()
    o1 = torch.zeros((rows - r0, nq * hd), dtype=torch.float16, device=DEV)
    B.attention_items(small, o1, [[(a - r0, n)] for (a, n), in items], nq, nq, hd, hd ** -0.5, 0,
                      path=B.ENC_I8F16)
    assert torch.equal(o1, out[r0:])
    assert torch.isfinite(o1.float()).all()
    del P, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", [B.ENC_F32, B.ENC_I8F16])
@pytest.mark.parametrize("L,W", [(64, 0), (64, 5), (64, 31), (40, 39), (64, 1)])
def test_attention_mask_probe(path, L, W):
    """Q = 0, V = one-hot per key: o_i[j] > 0 exactly for visible keys j."""
    hd = 64
    f16 = path == B.ENC_I8F16
    rng = np.random.default_rng(L + W)
    k = rng.normal(0, 1, (L, hd))
    v = np.eye(L, hd)
    p = np.concatenate([np.zeros((L, hd)), k, v], 1).astype(np.float16 if f16 else np.float32)
    out = torch.zeros((L, hd), dtype=torch.float16 if f16 else torch.float32, device=DEV)
    B.attention_items(to_dev(p), out, [[(0, L)]], 1, 1, hd, 1.0, W, path=path)
    got = host(out)[:, :L] > 0
    i = np.arange(L)
    pred = (np.abs(i[:, None] - i[None, :]) <= W) if W else np.ones((L, L), bool)
    assert np.array_equal(got, pred)


@pytest.mark.parametrize("path", [B.ENC_F32, B.ENC_I8F16])
def test_attention_packed_equals_separate(path):
    f16 = path == B.ENC_I8F16
    nq, hd = 2, 128 if f16 else 64
    items = [[(0, 150)], [(150, 37)], [(187, 300)]]
    rows = 487
    rng = np.random.default_rng(3)
    p = _panel(rng, rows, nq, nq, hd, f16=f16)
    dt = torch.float16 if f16 else torch.float32
    out = torch.zeros((rows, nq * hd), dtype=dt, device=DEV)
    B.attention_items(to_dev(p), out, items, nq, nq, hd, 0.1, 64, path=path)
    for rr in items:
        (r0, n), = rr
        o1 = torch.zeros((n, nq * hd), dtype=dt, device=DEV)
        B.attention_items(to_dev(p[r0:r0 + n]), o1, [[(0, n)]], nq, nq, hd, 0.1, 64, path=path)
        assert torch.equal(o1, out[r0:r0 + n])


WINDOW_ITEM_CASES = [
    # (window, item lengths): windowed f32 launches over many items of mixed
    # lengths; every row of every item must be written once, as alone
    (128, [5, 130, 300, 1, 700, 129, 257, 90]),          # one q-tile of keys each side
    (512, [1856, 194, 1100, 640, 37, 900, 385]),         # the text encoder's window
    (2500, [2600, 300, 1500, 20]),                       # window beyond 15 q-tiles
    (64, [int(n) for n in np.random.default_rng(5).integers(1, 200, 70)]),  # 64 items + a second launch
]


@pytest.mark.parametrize("window,lens", WINDOW_ITEM_CASES)
def test_attention_f32_windowed_many_items(window, lens):
    nq, nkv, hd = 2, 1, 64
    say(f"attention f32 windowed items W={window} items={len(lens)} rows={sum(lens)}")
    r0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(int)
    items = [[(int(a), int(n))] for a, n in zip(r0, lens)]
    rows = int(sum(lens))
    rng = np.random.default_rng(window + rows)
    p = _panel(rng, rows, nq, nkv, hd, qscale=0.5)
    P = to_dev(p)
    out = torch.full((rows, nq * hd), 7.0, dtype=torch.float32, device=DEV)
    scale = 1.0 / np.sqrt(hd)
    B.attention_items(P, out, items, nq, nkv, hd, scale, window)
    q, k, v = _split(p, nq, nkv, hd)
    ref = O.attention(items, q, k, v, nq, nkv, hd, scale, window)
    err = row_rel_err(host(out), ref)
    say(f"  err {err:.2e}")
    assert err <= TOL_F32
    for (a, n), in items[:12]:
        o1 = torch.full((n, nq * hd), 7.0, dtype=torch.float32, device=DEV)
        B.attention_items(to_dev(p[a:a + n]), o1, [[(0, n)]], nq, nkv, hd, scale, window)
        assert torch.equal(o1, out[a:a + n])


KEY_SPLIT_CASES = [
    # (path, items, nq, nkv, hd): each windowless item too short to fill the GPU alone
    (B.ENC_F32, [[(0, 1024)]], 12, 12, 64),             # the 1024-row ViT: 8 chunks of 128 keys
    (B.ENC_F32, [[(0, 1000)]], 12, 4, 64),              # 7 chunks, the last one ragged (40 keys)
    (B.ENC_F32, [[(0, 600), (700, 300)]], 4, 4, 64),    # two ranges, chunks across the seam
    (B.ENC_F32, [[(0, 800)], [(800, 100)], [(900, 300)]], 4, 2, 128),  # split and unsplit items
]


@pytest.mark.parametrize("path,items,nq,nkv,hd", KEY_SPLIT_CASES)
def test_attention_key_split(path, items, nq, nkv, hd):
    f16 = path == B.ENC_I8F16
    say(f"attention key split path={path} items={items} nq={nq} nkv={nkv} hd={hd}")
    rows = max(r0 + n for rr in items for r0, n in rr)
    rng = np.random.default_rng(rows + nq + hd)
    p = _panel(rng, rows, nq, nkv, hd, f16=f16, qscale=0.5)
    scale = 1.0 / np.sqrt(hd)
    d = B.attention_desc(None, None, nq, nkv, hd, scale, 0, ld=p.shape[1], ldo=nq * hd,
                         rows=rows, path=path)
    assert B.attention_workspace_bytes(d, items) > 0, "the case must take the split path"
    P = to_dev(p)
    dt = torch.float16 if f16 else torch.float32
    out = torch.full((rows, nq * hd), 7.0, dtype=dt, device=DEV)
    B.attention_items(P, out, items, nq, nkv, hd, scale, 0, path=path)
    q, k, v = _split(p, nq, nkv, hd)
    ref = O.attention(items, q, k, v, nq, nkv, hd, scale, 0)
    if f16:
        ref = np.vectorize(O.round_f16)(ref)
    covered = np.zeros(rows, bool)
    for rr in items:
        for r0, n in rr:
            covered[r0:r0 + n] = True
    got = host(out)
    assert np.all(got[~covered] == 7.0), "rows outside every item were written"
    err = row_rel_err(got[covered], ref[covered])
    # the unsplit kernel (no workspace) computes the same softmax in one pass
    out1 = torch.full_like(out, 7.0)
    B.attention_items(P, out1, items, nq, nkv, hd, scale, 0, ws=None, path=path)
    err1 = row_rel_err(got[covered], host(out1)[covered].astype(np.float64))
    tol = TOL_I8F16 if f16 else TOL_F32
    say(f"  err vs oracle {err:.2e}, vs unsplit {err1:.2e}")
    assert err <= tol and err1 <= tol
    out2 = torch.full_like(out, 7.0)
    B.attention_items(P, out2, items, nq, nkv, hd, scale, 0, path=path)
    assert torch.equal(out, out2), "key-split attention is not deterministic"


@pytest.mark.parametrize("path,hd,nq", [(B.ENC_F32, 64, 4), (B.ENC_I8F16, 128, 32)])
def test_attention_packed_equals_separate_long_items(path, hd, nq):
    """Items long enough for the f32 key split across blocks; on the f16 path
    (nq 32) the 1800-row item takes the unsplit kernel and the others the
    split-key one, in two launches."""
    f16 = path == B.ENC_I8F16
    items = [[(0, 1800)], [(1800, 700)], [(2500, 90)]]
    rows = 2590
    rng = np.random.default_rng(11)
    p = _panel(rng, rows, nq, nq, hd, f16=f16)
    dt = torch.float16 if f16 else torch.float32
    out = torch.zeros((rows, nq * hd), dtype=dt, device=DEV)
    B.attention_items(to_dev(p), out, items, nq, nq, hd, 0.125, 0, path=path)
    for rr in items:
        (r0, n), = rr
        o1 = torch.zeros((n, nq * hd), dtype=dt, device=DEV)
        B.attention_items(to_dev(p[r0:r0 + n]), o1, [[(0, n)]], nq, nq, hd, 0.125, 0, path=path)
        assert torch.equal(o1, out[r0:r0 + n])


# ------------------------------------------------------------------ row ops

@pytest.mark.parametrize("d", [4, 128, 512, 768, 3840, 4096])
@pytest.mark.parametrize("f16", [False, True])
def test_norms(d, f16):
    rng = np.random.default_rng(d)
    rows = 203
    x = rng.normal(0, 3, (rows, d)).astype(np.float32)
    w = rng.normal(1, 0.02, d).astype(np.float32)
    b = rng.normal(0, 0.01, d).astype(np.float32)
    dt = torch.float16 if f16 else torch.float32
    tol = TOL_I8F16 if f16 else TOL_F32
    Y = torch.empty((rows, d), dtype=dt, device=DEV)
    B.rms_norm(to_dev(x), to_dev(w), 1e-6, Y, f16=f16)
    assert row_rel_err(host(Y), O.rms_norm(x, w, 1e-6)) <= tol
    B.layer_norm(to_dev(x), to_dev(w), to_dev(b), 1e-6, Y, f16=f16)
    assert row_rel_err(host(Y), O.layer_norm(x, w, b, 1e-6)) <= tol


@pytest.mark.parametrize("d", [512, 3840])
@pytest.mark.parametrize("f16", [False, True])
def test_add_norm_fused_equals_unfused(d, f16):
    rng = np.random.default_rng(d + 1)
    rows = 130
    h = rng.normal(0, 3, (rows, d)).astype(np.float32)
    t = rng.normal(0, 1, (rows, d)).astype(np.float32)
    wp = rng.normal(1, 0.02, d).astype(np.float32)
    wn = rng.normal(1, 0.02, d).astype(np.float32)
    dt = torch.float16 if f16 else torch.float32
    H, T = to_dev(h), to_dev(t)
    A = torch.empty((rows, d), dtype=dt, device=DEV)
    B.add_norm(H, T, to_dev(wp), 1e-6, to_dev(wn), A, f16=f16)
    ref_h = h.astype(np.float64) + O.rms_norm(t, wp, 1e-6)
    assert row_rel_err(host(H), ref_h) <= TOL_F32
    assert row_rel_err(host(A), O.rms_norm(ref_h, wn, 1e-6)) <= (TOL_I8F16 if f16 else TOL_F32)
    A2 = torch.empty_like(A)
    B.rms_norm(H, to_dev(wn), 1e-6, A2, f16=f16)
    assert torch.equal(A, A2)  # the fused next pre-norm gives the same bits


@pytest.mark.parametrize("hd,sections,f16,nq,nkv", [
    (64, 1, False, 3, 2), (64, 2, False, 3, 2), (128, 2, True, 3, 2), (128, 1, True, 3, 2),
    (64, 1, True, 3, 2), (128, 2, False, 3, 2),
    # several head groups per row, the last one partial
    (128, 2, True, 30, 30), (64, 1, False, 13, 5), (128, 1, False, 7, 3), (64, 2, True, 21, 4)])
def test_qk_norm_rope(hd, sections, f16, nq, nkv):
    rng = np.random.default_rng(hd + sections + nq)
    rows = 97
    ld = (nq + 2 * nkv) * hd
    p = rng.normal(0, 2, (rows, ld)).astype(np.float16 if f16 else np.float32)
    qw = rng.normal(1, 0.02, hd).astype(np.float32)
    kw = rng.normal(1, 0.02, hd).astype(np.float32)
    pos = rng.integers(0, 2048, (rows, sections)).astype(np.int32)
    cos, sin = B.rope_table(pos, hd, sections, 10000.0)
    P = to_dev(p)
    B.qk_norm_rope(P, nq, nkv, hd, to_dev(qw), to_dev(kw), 1e-6, to_dev(cos), to_dev(sin),
                   sections, path=B.ENC_I8F16 if f16 else B.ENC_F32)
    got = host(P)
    pp = p.astype(np.float64)
    refq = O.qk_norm_rope(pp[:, :nq * hd], nq, hd, qw, 1e-6, sections, pos, 10000.0)
    refk = O.qk_norm_rope(pp[:, nq * hd:(nq + nkv) * hd], nkv, hd, kw, 1e-6, sections, pos, 10000.0)
    tol = TOL_I8F16 if f16 else TOL_F32
    assert row_rel_err(got[:, :nq * hd], refq) <= tol
    assert row_rel_err(got[:, nq * hd:(nq + nkv) * hd], refk) <= tol
    assert np.array_equal(got[:, (nq + nkv) * hd:], pp[:, (nq + nkv) * hd:])  # v untouched


@pytest.mark.parametrize("hd,f16,sections", [(128, True, 2), (64, False, 1)])
def test_qk_norm_rope_head_grouping_bit_identical(hd, f16, sections):
    """Few rows split each row's heads over several waves, many rows take one wave
    per row: a row's bits do not depend on which."""
    rng = np.random.default_rng(17 + hd)
    rows, nq, nkv = 9000, 30 if f16 else 8, 30 if f16 else 8
    ld = (nq + 2 * nkv) * hd
    p = rng.normal(0, 2, (rows, ld)).astype(np.float16 if f16 else np.float32)
    qw = rng.normal(1, 0.02, hd).astype(np.float32)
    kw = rng.normal(1, 0.02, hd).astype(np.float32)
    pos = rng.integers(0, 2048, (rows, sections)).astype(np.int32)
    cos, sin = B.rope_table(pos, hd, sections, 10000.0)
    path = B.ENC_I8F16 if f16 else B.ENC_F32
    Pall = to_dev(p)
    B.qk_norm_rope(Pall, nq, nkv, hd, to_dev(qw), to_dev(kw), 1e-6, to_dev(cos), to_dev(sin),
                   sections, path=path)
    for r0, r1 in ((0, 500), (4321, 4400), (8999, 9000)):
        P = to_dev(p[r0:r1])
        B.qk_norm_rope(P, nq, nkv, hd, to_dev(qw), to_dev(kw), 1e-6, to_dev(cos[r0:r1]),
                       to_dev(sin[r0:r1]), sections, path=path)
        assert torch.equal(P, Pall[r0:r1])


def test_rms_norm_prescale_and_add_norm_scalar():
    """rms(pre x) w (the per-layer input's norm) and h = (h + rms(t) w) post (the
    layer scalar) against the oracle's norms; pre = post = 1 is bit-identical to
    the plain calls."""
    rng = np.random.default_rng(5)
    n, d = 300, 512
    x = rng.normal(0, 3, (n, d)).astype(np.float32)
    w = (1 + 0.02 * rng.normal(0, 1, d)).astype(np.float32)
    y = torch.empty((n, d), dtype=torch.float32, device=DEV)
    B.rms_norm(to_dev(x), to_dev(w), 1e-6, y, pre=0.7071)
    ref = O.rms_norm(x.astype(np.float64) * np.float64(np.float32(0.7071)), w, 1e-6)
    assert row_rel_err(host(y), ref) <= TOL_F32
    y1 = torch.empty_like(y)
    B.rms_norm(to_dev(x), to_dev(w), 1e-6, y1, pre=1.0)
    y0 = torch.empty_like(y)
    B.rms_norm(to_dev(x), to_dev(w), 1e-6, y0)
    assert torch.equal(y1, y0)
    h = rng.normal(0, 20, (n, d)).astype(np.float32)
    t = rng.normal(0, 1, (n, d)).astype(np.float32)
    H = to_dev(h)
    B.add_norm(H, to_dev(t), to_dev(w), 1e-6, post=0.93)
    ref = (h.astype(np.float64) + O.rms_norm(t, w, 1e-6)) * np.float64(np.float32(0.93))
    assert row_rel_err(host(H), ref) <= TOL_F32


@pytest.mark.parametrize("f16", [False, True])
@pytest.mark.parametrize("with_t", [True, False])
def test_row_op_modulation_column_fields_guard(f16, with_t):
    """The int8 block's row op: h = h + gate * rms(t) w_post, then three copies
    a_z = rms(h) w (1 + scale) col_z 2^-6 (the q/k/v inputs of a modulated
    q8_2f block with its guard); with t = None only the pre-norm runs."""
    rng = np.random.default_rng(21 + f16)
    n, d = 130, 3840
    h = rng.normal(0, 5, (n, d)).astype(np.float32)
    t = rng.normal(0, 1, (n, d)).astype(np.float32)
    vec = lambda m, sd: (m + sd * rng.normal(0, 1, d)).astype(np.float32)
    w_post, w_next, gate, scale = vec(1, 0.02), vec(1, 0.02), vec(1, 0.1), vec(0, 0.1)
    cols = [np.exp(0.25 * rng.normal(0, 1, d)).astype(np.float32) for _ in range(3)]
    H = to_dev(h)
    A = torch.empty((3, n, d), dtype=torch.float16 if f16 else torch.float32, device=DEV)
    B.add_norm(H, to_dev(t) if with_t else None, to_dev(w_post) if with_t else None, 1e-6,
               w_next=to_dev(w_next), a=A, f16=f16, gate=to_dev(gate) if with_t else None,
               scale=to_dev(scale), cols=[to_dev(c) for c in cols], nout=3, oscale=2.0 ** -6)
    hr = h.astype(np.float64)
    if with_t:
        hr = hr + O.rms_norm(t, w_post, 1e-6) * gate.astype(np.float64)
    assert row_rel_err(host(H), hr) <= TOL_F32
    base = O.rms_norm(hr, w_next, 1e-6) * (1.0 + scale.astype(np.float64))
    for z in range(3):
        ref = base * cols[z].astype(np.float64) * 2.0 ** -6
        if f16:
            ref = np.vectorize(O.round_f16)(ref)
        assert row_rel_err(host(A[z]), ref) <= (TOL_I8F16 if f16 else TOL_F32), z


@pytest.mark.parametrize("path,n,ff,d", [(B.ENC_I8F16, 520, 12800, 128), (B.ENC_I8F16, 77, 160, 80),
                                         (B.ENC_F32, 300, 512, 256)])
def test_gated_epilogue_column_field_and_guard(path, n, ff, d):
    """The gated GEMM's y_col / y_scale (w2's column field, the hidden's guard)
    equal the unfused gate/up GEMM + enc_gated_act with out_col / out_scale, bit
    for bit, on the 256 x 256 direct-to-LDS, the register-staged and the f32
    gated kernels."""
    rng = np.random.default_rng(n + ff)
    i8 = path == B.ENC_I8F16
    if i8:
        x = rng.normal(0, 1, (n, d)).astype(np.float16)
        ws = [rng.integers(-127, 128, (ff, d)).astype(np.int8) for _ in range(2)]
        rs = [to_dev((0.002 * np.exp(0.25 * rng.normal(0, 1, ff))).astype(np.float32)) for _ in range(2)]
    else:
        x = rng.normal(0, 1, (n, d)).astype(np.float32)
        ws = [rng.normal(0, 0.05, (ff, d)).astype(np.float32) for _ in range(2)]
        rs = None
    col = to_dev(np.exp(0.25 * rng.normal(0, 1, ff)).astype(np.float32))
    X, W = to_dev(x), [to_dev(w) for w in ws]
    odt = torch.float16 if i8 else torch.float32
    fused = torch.empty((n, ff), dtype=odt, device=DEV)
    B.gemm_items(X, fused, W, [(n, ff, d, d, ff, 0, 0, 0)], path=path, row_scale=rs, alpha=2.0,
                 flags=B.ENC_EPI_GATE_SILU | (B.ENC_Y_F16 if i8 else 0), y_col=col, y_scale=2.0 ** -6)
    gu = torch.empty((n, 2 * ff), dtype=torch.float32, device=DEV)
    B.gemm_items(X, gu, W, [(n, ff, d, d, 2 * ff, 0, 0, 0), (n, ff, d, d, 2 * ff, 1, 0, ff)],
                 path=path, row_scale=rs, alpha=2.0)
    unfused = torch.empty((n, ff), dtype=odt, device=DEV)
    B.gated_act(gu[:, :ff], gu[:, ff:], unfused, B.ENC_ACT_SWIGLU, f16=i8, out_col=col,
                out_scale=2.0 ** -6)
    assert torch.equal(fused, unfused)


@pytest.mark.parametrize("path,items,nq,hd,window", [
    (B.ENC_I8F16, [[(0, 300), (400, 40)], [(300, 100)]], 4, 128, 0),
    # unsplit f16 kernels: 128-query blocks; 256-query blocks; windowed
    (B.ENC_I8F16, [[(0, 1100)]], 32, 128, 0),
    (B.ENC_I8F16, [[(0, 500), (1100, 100)], [(500, 600)]], 128, 128, 0),
    (B.ENC_I8F16, [[(0, 700)]], 4, 128, 96),
    (B.ENC_I8F16, [[(0, 200)]], 4, 64, 0),
    (B.ENC_F32, [[(0, 1024)]], 12, 64, 0),
    (B.ENC_F32, [[(0, 100)], [(100, 50)]], 2, 128, 0)])
def test_attention_output_column_field_and_scale(path, items, nq, hd, window):
    """out = o * out_scale * out_col (the O projection's column field and the
    guards), in the attention epilogue of every kernel (f16: the split-key one,
    the unsplit 128- and 256-query ones, the windowed one, hd 64; f32) and in
    the key-split merge."""
    f16 = path == B.ENC_I8F16
    rows = max(r0 + n for rr in items for r0, n in rr)
    rng = np.random.default_rng(rows)
    p = _panel(rng, rows, nq, nq, hd, f16=f16, qscale=0.5)
    dt = torch.float16 if f16 else torch.float32
    col = np.exp(0.25 * rng.normal(0, 1, nq * hd)).astype(np.float32)
    out = torch.zeros((rows, nq * hd), dtype=dt, device=DEV)
    B.attention_items(to_dev(p), out, items, nq, nq, hd, 0.1, window, path=path, out_col=to_dev(col),
                      out_scale=2.0)
    q, k, v = _split(p, nq, nq, hd)
    ref = O.attention(items, q, k, v, nq, nq, hd, 0.1, window) * col.astype(np.float64) * 2.0
    if f16:
        ref = np.vectorize(O.round_f16)(ref)
    got = host(out)
    idx = np.concatenate([np.arange(r0, r0 + n) for rr in items for r0, n in rr])
    assert row_rel_err(got[idx], ref[idx]) <= (TOL_I8F16 if f16 else TOL_F32)


@pytest.mark.parametrize("hd,f16", [(64, False), (128, True)])
def test_qk_norm_rope_with_v_norm(hd, f16):
    """With v_norm the v heads are RMS-normed without gain and not rotated; q and
    k get exactly the bits they get without it."""
    rng = np.random.default_rng(hd)
    rows, nq, nkv = 200, 8, 2
    ld = (nq + 2 * nkv) * hd
    p = rng.normal(0, 2, (rows, ld)).astype(np.float16 if f16 else np.float32)
    qw = (1 + 0.02 * rng.normal(0, 1, hd)).astype(np.float32)
    kw = (1 + 0.02 * rng.normal(0, 1, hd)).astype(np.float32)
    pos = O.positions(rows, [[(0, rows)]], [0], 1)
    th = pos.astype(np.float64) * 10000.0 ** (-2.0 * np.arange(hd // 2) / hd)
    cos, sin = to_dev(np.cos(th).astype(np.float32)), to_dev(np.sin(th).astype(np.float32))
    path = B.ENC_I8F16 if f16 else B.ENC_F32
    P1, P2 = to_dev(p), to_dev(p)
    B.qk_norm_rope(P1, nq, nkv, hd, to_dev(qw), to_dev(kw), 1e-6, cos, sin, 1, path=path, v_norm=True)
    B.qk_norm_rope(P2, nq, nkv, hd, to_dev(qw), to_dev(kw), 1e-6, cos, sin, 1, path=path)
    vc = (nq + nkv) * hd
    assert torch.equal(P1[:, :vc], P2[:, :vc])
    assert torch.equal(P2[:, vc:], to_dev(p)[:, vc:])  # untouched without v_norm
    v = p[:, vc:].astype(np.float64).reshape(rows * nkv, hd)
    ref = O.rms_norm(v, None, 1e-6).reshape(rows, nkv * hd)
    if f16:
        ref = np.vectorize(O.round_f16)(ref)
    assert row_rel_err(host(P1)[:, vc:], ref) <= (TOL_I8F16 if f16 else TOL_F32)


@pytest.mark.parametrize("kind,f16", [(B.ENC_ACT_GELU_TANH_GATED, False), (B.ENC_ACT_SWIGLU, True),
                                      (B.ENC_ACT_SWIGLU, False)])
def test_gated_act(kind, f16):
    rng = np.random.default_rng(kind)
    rows, ff = 77, 2048
    gu = rng.normal(0, 2, (rows, 2 * ff)).astype(np.float32)
    GU = to_dev(gu)
    out = torch.empty((rows, ff), dtype=torch.float16 if f16 else torch.float32, device=DEV)
    B.gated_act(GU[:, :ff], GU[:, ff:], out, kind, f16=f16)
    g, u = gu[:, :ff].astype(np.float64), gu[:, ff:].astype(np.float64)
    act = np.vectorize(O.gelu_tanh if kind == B.ENC_ACT_GELU_TANH_GATED else O.silu)
    assert row_rel_err(host(out), act(g) * u) <= (TOL_I8F16 if f16 else TOL_F32)


@pytest.mark.parametrize("f16", [False, True])
def test_swiglu_far_negative_gate(f16):
    """silu at gates from -92 to -80, where 1 + e^-x passes 2^126 and the
    reciprocal leaves the normal range: the outputs (below 1e-30 in magnitude)
    stay within 1e-30 of the oracle's, and the rows' normal values within the
    path's tolerance."""
    rows, ff = 8, 512
    g = np.linspace(-92.0, -80.0, rows * ff).reshape(rows, ff).astype(np.float32)
    g[:, ::64] = 3.0  # a normal value per 64 so the row errors are relative to it
    u = np.ones((rows, ff), np.float32)
    out = torch.empty((rows, ff), dtype=torch.float16 if f16 else torch.float32, device=DEV)
    B.gated_act(to_dev(g), to_dev(u), out, B.ENC_ACT_SWIGLU, f16=f16)
    ref = np.vectorize(O.silu)(g.astype(np.float64))
    if f16:
        ref = np.vectorize(O.round_f16)(ref)
    got = host(out)
    tiny = g < 0
    assert np.abs(got[tiny] - ref[tiny]).max() <= 1e-30
    assert row_rel_err(got, ref) <= (TOL_I8F16 if f16 else TOL_F32)


def test_mean_pool():
    rng = np.random.default_rng(9)
    rows, d = 300, 512
    a = rng.normal(0, 1, (rows, d)).astype(np.float32)
    items = [[(0, 100)], [(100, 1)], [(101, 150), (290, 10)], [(251, 39)]]
    out = torch.empty((len(items), d), dtype=torch.float32, device=DEV)
    B.mean_pool(to_dev(a), items, out)
    ref = np.stack([np.concatenate([a[r0:r0 + n] for r0, n in rr]).astype(np.float64).mean(0)
                    for rr in items])
    assert row_rel_err(host(out), ref) <= TOL_F32


# ------------------------------------------------------------- edge cases

def test_gemm_empty_items():
    """Items with no rows are no-ops beside non-empty ones; a launch of empty items
    leaves Y untouched."""
    rng = np.random.default_rng(31)
    n, m, k = 70, 96, 64
    x = rng.integers(-8, 9, (n, k)).astype(np.float32)
    w = rng.integers(-8, 9, (m, k)).astype(np.float32)
    Y = torch.full((n, 2 * m), 7.0, device=DEV)
    B.gemm_items(to_dev(x), Y, [to_dev(w)], [(0, m, k, k, 2 * m, 0, 0, 0), (n, m, k, k, 2 * m, 0, 0, m)])
    got = host(Y)
    assert np.array_equal(got[:, m:], O.linear(x, w))
    assert (got[:, :m] == 7.0).all()
    B.gemm_items(to_dev(x), Y, [to_dev(w)], [(0, m, k, k, 2 * m, 0, 0, 0)])
    assert np.array_equal(host(Y), got)


@pytest.mark.parametrize("path", [B.ENC_F32, B.ENC_I8F16])
def test_attention_empty_and_one_row_items(path):
    f16 = path == B.ENC_I8F16
    rng = np.random.default_rng(32)
    rows, nq, nkv, hd = 50, 2, 2, 64
    items = [[(0, 0)], [(0, 1)], [(1, 0), (1, 0)], [(1, 49)]]
    p = _panel(rng, rows, nq, nkv, hd, f16=f16)
    out = torch.full((rows, nq * hd), 5.0, dtype=torch.float16 if f16 else torch.float32, device=DEV)
    B.attention_items(to_dev(p), out, items, nq, nkv, hd, 0.125, 0, path=path)
    q, k, v = _split(p, nq, nkv, hd)
    ref = O.attention(items, q, k, v, nq, nkv, hd, 0.125, 0)
    assert row_rel_err(host(out), ref) <= (TOL_I8F16 if f16 else TOL_F32)
    assert np.array_equal(host(out)[0], v[0])  # a one-row item returns its own value


def test_row_ops_zero_rows():
    w = to_dev(np.ones(256, np.float32))
    x = torch.empty((0, 256), dtype=torch.float32, device=DEV)
    y = torch.empty((0, 256), dtype=torch.float32, device=DEV)
    B.rms_norm(x, w, 1e-6, y)
    B.layer_norm(x, w, w, 1e-6, y)
    torch.cuda.synchronize()


def test_mean_pool_many_items_and_empty_refused():
    """More items than one launch takes (64); an empty item is refused."""
    rows, d = 1000, 40
    a = torch.arange(rows * d, dtype=torch.float32, device=DEV).reshape(rows, d) % 1000.0
    items = [[(2 * i, 2)] for i in range(rows // 2)]
    out = torch.empty((rows // 2, d), dtype=torch.float32, device=DEV)
    B.mean_pool(a, items, out)
    assert torch.equal(out, (a[0::2] + a[1::2]) / 2)
    with pytest.raises(RuntimeError, match="empty"):
        B.mean_pool(a, [[(0, 3)], [(3, 0)]], out)
