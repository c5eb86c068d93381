"""megamoe_permute_noalloc (no workspace; the sort's count table in a static
device array) against megamoe_permute through the C ABI.

Two calls in a row on the two-pass sort, which is the path that uses the
static table, the second with fewer routes and experts than the first (so the
second call's table is smaller than what the first left behind), then one call
on the one-launch permute.  Every output -- indices, counts, prefix, the
quantised rows, the scales and the dropped-route count -- must equal the
workspace variant's bit for bit."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from moe_expert_ffn_amd import inputs as W  # noqa: E402
from moe_expert_ffn_amd import megamoe as MM  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = [
    # R = 24000: two-pass sort, 94 blocks x 64 experts of counts; 2% of routes dropped
    (W.custom(3000, 256, 64, 8, 128, routing="zipf", name="noalloc_first"), 0.02),
    # R = 9600: two-pass sort, 38 blocks x 32 experts
    (W.custom(1200, 512, 32, 8, 128, name="noalloc_second_smaller"), 0.0),
    # R = 400: the one-launch permute (no count table)
    (W.custom(100, 256, 16, 4, 128, name="noalloc_one_launch"), 0.01),
]


def _outputs(w):
    cu = dict(device="cuda")
    R = w.R
    return dict(gmA=torch.zeros((R, w.K), dtype=torch.int8, **cu),
                pts1=torch.zeros(R, dtype=torch.float32, **cu),
                eri=torch.empty(R, dtype=torch.int32, **cu),
                srt=torch.empty(R, dtype=torch.int32, **cu),
                cnt=torch.empty(w.E, dtype=torch.int32, **cu),
                cum=torch.empty(w.E, dtype=torch.int32, **cu))


def test_noalloc_permute_matches_workspace_variant():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    MM.load()
    runs = []
    for i, (w, drop) in enumerate(CASES):
        inp = W.generate(w, seed=30 + i)
        if drop:
            rng = np.random.default_rng(40 + i)
            hit = rng.random(inp["expert_idx"].shape) < drop
            inp["expert_idx"] = np.where(hit, -1, inp["expert_idx"]).astype(np.int32)
        x = torch.from_numpy(inp["x"]).cuda()
        ei = torch.from_numpy(inp["expert_idx"]).cuda()
        d = MM.dims(w.M, w.K, w.E, w.top_k, w.I)
        ref = _outputs(w)
        ws = torch.empty(MM.megamoe_permute_workspace_bytes(d), dtype=torch.uint8, device="cuda")
        MM.megamoe_permute(d, x, ei, ref["gmA"], ref["pts1"], ref["eri"], ref["srt"], ref["cnt"],
                           ref["cum"], ws)
        ref_dropped = MM.megamoe_last_error(ws)
        assert ref_dropped == int((inp["expert_idx"] < 0).sum())
        runs.append((w, d, x, ei, ref, ref_dropped))
    torch.cuda.synchronize()
    # the allocation-free calls, back to back: larger, smaller, one-launch
    got = []
    for w, d, x, ei, _, _ in runs:
        o = _outputs(w)
        o["dropped"] = torch.full((4,), -7, dtype=torch.int32, device="cuda")
        print(f"[noalloc] {w.describe()}", flush=True)
        MM.megamoe_permute_noalloc(d, x, ei, o["gmA"], o["pts1"], o["eri"], o["srt"], o["cnt"],
                                   o["cum"], o["dropped"])
        got.append(o)
    torch.cuda.synchronize()
    for (w, _, _, _, ref, ref_dropped), o in zip(runs, got):
        for k in ("eri", "srt", "cnt", "cum", "gmA", "pts1"):
            assert torch.equal(o[k].view(torch.int8) if o[k].dtype == torch.float32 else o[k],
                               ref[k].view(torch.int8) if ref[k].dtype == torch.float32 else ref[k]), \
                f"{w.name}: {k}"
        assert int(o["dropped"][0].item()) == ref_dropped, w.name
