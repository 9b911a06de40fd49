"""The allocation-free attention entry point (attention_items_static) against
attention_items with a workspace: the same kernels and split plan, so the same
bits, on two calls in a row, the second with a smaller input; and a clear error
for items whose key splits need more than the static scratch."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, say, to_dev
from transformer_encoder_forward_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.lib()
    B.context(0)


def _case(rows, items, nq, hd, seed, path=B.ENC_F32):
    rng = np.random.default_rng(seed)
    ld = 3 * nq * hd
    p = rng.standard_normal((rows, ld), dtype=np.float32)
    dt = torch.float16 if path == B.ENC_I8F16 else torch.float32
    panel = to_dev(p).to(dt)
    return panel, dt


@pytest.mark.parametrize("path", [B.ENC_F32, B.ENC_I8F16])
def test_static_scratch_attention_equals_workspace_attention(path):
    # first call: a 1024-row item of 12 heads (the f32 path cuts its keys into
    # 8 chunks: 26 MB of partials), then a smaller two-item launch
    calls = [(1024, [[(0, 1024)]], 12, 64, 0.125),
             (700, [[(0, 300)], [(300, 260), (620, 80)]], 4, 128 if path == B.ENC_I8F16 else 64, 0.2)]
    for k, (rows, items, nq, hd, scale) in enumerate(calls):
        panel, dt = _case(rows, items, nq, hd, 10 + k, path)
        # rows outside every item are not written: both outputs start equal
        want = torch.zeros((rows, nq * hd), dtype=dt, device=DEV)
        got = torch.zeros((rows, nq * hd), dtype=dt, device=DEV)
        desc = B.attention_desc(panel, want, nq, nq, hd, scale, path=path)
        need = B.attention_workspace_bytes(desc, items)
        say(f"call {k}: rows {rows}, {len(items)} items, {nq}x{hd}, split scratch {need} bytes")
        assert need <= B.STATIC_SCRATCH_BYTES
        B.attention_items(panel, want, items, nq, nq, hd, scale, path=path)
        B.attention_items_static(panel, got, items, nq, nq, hd, scale, path=path)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"call {k}"


def test_static_scratch_refuses_oversized_splits():
    # 4 items of 2048 rows x 16 heads of 64, f32, no window: each is cut into
    # key chunks whose partials together need far more than the static scratch
    rows, nq, hd = 8192, 16, 64
    items = [[(2048 * i, 2048)] for i in range(4)]
    panel = torch.zeros((rows, 3 * nq * hd), dtype=torch.float32, device=DEV)
    out = torch.zeros((rows, nq * hd), dtype=torch.float32, device=DEV)
    need = B.attention_workspace_bytes(B.attention_desc(panel, out, nq, nq, hd, 0.125), items)
    say(f"oversized case needs {need} bytes")
    if need <= B.STATIC_SCRATCH_BYTES:
        pytest.skip("the split plan of this case fits the scratch")
    with pytest.raises(B.EncError) as ei:
        B.attention_items_static(panel, out, items, nq, nq, hd, 0.125)
    assert ei.value.status == 3 and "static scratch" in str(ei.value)
