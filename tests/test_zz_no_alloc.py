"""The entry point that allocates nothing, bra_forward_static (the library's
static device scratch instead of a workspace), against bra_forward_ws on the
same inputs: the same output bits, on two calls in a row whose second has a
smaller input, so that it runs over the first call's leftover scratch."""

import pytest
import torch

import vision_transformer_dynamic_amd as bra
from vision_transformer_dynamic_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

PAIRS = [
    # (first call, second call with a smaller input)
    (wl.WORKLOADS[3], wl.WORKLOADS[2]),    # stage-3 then stage-2 shape (image-resident attention)
    (wl.WORKLOADS[1], wl.custom(2, 14, 14, 64, 2, 7, 4, "bf16", seed=95)),  # stage-1 shape then a 2-image map
    (wl.WORKLOADS[4], wl.WORKLOADS[0]),    # dense map (chunked attention) then the tiny fp32 map
]


def _with_workspace(w, q, k, v):
    ws = torch.empty(bra.workspace_bytes(w.B, w.H, w.W, w.C, w.S, w.topk), dtype=torch.uint8, device=DEV)
    return bra.forward_ws(q, k, v, w.heads, w.S, w.topk, ws)


@pytest.mark.parametrize("first,second", PAIRS, ids=lambda w: w.name)
def test_static_scratch_forward_matches_workspace_form(first, second):
    for w in (first, second):
        print(f"\n[no-alloc] {w.name}", flush=True)
        q, k, v = (t.to(DEV) for t in wl.make_inputs(w))
        got = bra.forward_static(q, k, v, w.heads, w.S, w.topk)
        ref = _with_workspace(w, q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), w.name
