"""megamoe_forward captured into a HIP graph and replayed.

Serving loops replay the MoE layer from a captured graph, so the forward must
enqueue nothing that a capture cannot hold (no allocation, no memset node, no
host synchronisation).  Each case runs the forward eagerly, captures it, then
replays it several times with eager work and synchronisations in between (the
output is overwritten with garbage before every replay) and checks every
replay bit for bit against the eager output.  The eager output itself is
checked against the oracle by the parity tests; here it is also compared with
the oracle's tolerance once, so a capture that silently ran nothing fails.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from moe_expert_ffn_amd import inputs as W  # noqa: E402
from moe_expert_ffn_amd import megamoe as MM  # noqa: E402
from oracle import oracle as O  # noqa: E402
from tests import gpu_helpers as H  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = [
    W.custom(96, 1024, 8, 4, 256, name="graph_fused_permute"),      # R <= 8192: one-launch permute
    W.custom(2500, 256, 16, 4, 128, name="graph_two_pass_sort"),     # R > 8192: two-pass sort
    W.custom(256, 1024, 8, 4, 256, name="graph_mid_rows"),           # 128 rows per expert
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    MM.load()


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_forward_graph_replay(w):
    inp = W.generate(w, 3)
    dev = H.to_dev(inp)
    d = MM.dims(w.M, w.K, w.E, w.top_k, w.I)
    w1p, w2p = H.prepack(d, dev)
    ws = torch.empty(MM.megamoe_workspace_bytes(d), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.M, w.K), dtype=torch.bfloat16, device="cuda")

    def fwd():
        MM.megamoe_forward(d, dev["x"], dev["expert_idx"], dev["probs"], w1p, dev["scale1"],
                           w2p, dev["scale2"], out, ws)

    fwd()
    torch.cuda.synchronize()
    eager = out.clone()
    ref = O.forward(inp, E=w.E)
    ref_out = ref["out_f32"]
    err = np.abs(eager.float().cpu().numpy() - ref_out).max()
    assert err <= 2e-2 * np.abs(ref_out).max(), f"eager forward off the oracle: {err}"

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fwd()  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            fwd()
    torch.cuda.synchronize()

    for rep in range(4):
        out.fill_(float("nan"))          # eager work between replays
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert MM.megamoe_last_error(ws) == 0
