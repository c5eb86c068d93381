"""Two forwards in flight at once, on two streams with their own workspaces.

The C ABI promises that calls with distinct workspaces are independent: all
per-call state lives in the caller's workspace, and the only library-wide
state (the per-device CU count and the GEMMs' occupancy, filled at first use)
is read-only afterwards.  Two forwards of different shapes, one using the
256-row GEMM tiles and the two-pass sort, the other the 64-row tiles and the
one-launch permute, are enqueued alternately on two default-priority streams
and must give, bit for bit, what each gives alone on the current stream.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from moe_expert_ffn_amd import inputs as W  # noqa: E402
from moe_expert_ffn_amd import megamoe as MM  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    MM.load()


def _setup(w, seed):
    inp = W.generate(w, seed=seed)
    dev = H.to_dev(inp)
    d = MM.dims(w.M, w.K, w.E, w.top_k, w.I)
    w1p, w2p = H.prepack(d, dev)
    ws = torch.empty(MM.megamoe_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.M, w.K), dtype=torch.bfloat16, device="cuda")
    return d, dev, w1p, w2p, ws, out


def _forward(case, stream=None):
    d, dev, w1p, w2p, ws, out = case
    MM.megamoe_forward(d, dev["x"], dev["expert_idx"], dev["probs"], w1p, dev["scale1"], w2p,
                       dev["scale2"], out, ws, stream=stream)


def test_two_streams_distinct_workspaces():
    wa = W.custom(2400, 512, 8, 4, 256, routing="zipf", name="streams_256_rows")  # R > 8192
    wb = W.custom(96, 1024, 32, 6, 384, name="streams_64_rows")                    # R <= 8192
    print(f"[streams] {wa.describe()} | {wb.describe()}", flush=True)
    a, b = _setup(wa, 21), _setup(wb, 22)
    # each alone, on the current stream
    _forward(a)
    _forward(b)
    torch.cuda.synchronize()
    ref_a, ref_b = a[5].clone(), b[5].clone()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for rep in range(3):
        a[5].fill_(float("nan"))
        b[5].fill_(float("nan"))
        torch.cuda.synchronize()
        for _ in range(4):  # alternate launches so the two forwards overlap
            _forward(a, sa)
            _forward(b, sb)
        torch.cuda.synchronize()
        assert torch.equal(a[5].view(torch.int16), ref_a.view(torch.int16)), f"stream a, rep {rep}"
        assert torch.equal(b[5].view(torch.int16), ref_b.view(torch.int16)), f"stream b, rep {rep}"
    assert np.all(np.isfinite(H.bf16_f32(ref_a))) and np.all(np.isfinite(H.bf16_f32(ref_b)))
