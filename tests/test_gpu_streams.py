"""The whole path on a non-default stream and inside a captured HIP graph.

Every entry point enqueues its kernels on the stream it is given and does
nothing else on the device: no host synchronisation, no allocation, no memset
(the quantizers' absmax accumulators are cleared by a one-workgroup kernel).
So the step (input step, then attention) gives the same bits on a side stream
as on the default one, and it can be captured once and replayed. Each replay
is compared bit for bit with the same step run eagerly, with eager work and
synchronisations between the replays.
"""

import numpy as np
import pytest
import torch

from bf16_causal_prefill_fwd_amd import ops
from bf16_causal_prefill_fwd_amd.workloads import Workload, make_inputs

from .test_gpu_parity import dev

pytestmark = pytest.mark.gpu

CASES = {
    "fp8": Workload("stream_gqa_fp8", 1, 1000, 8, 2, 128, 128, "fp8", "outlier"),
    "fp8_mla": Workload("stream_mla_fp8", 1, 700, 4, 4, 192, 128, "fp8", "mla"),
    "bf16": Workload("stream_gqa_bf16", 1, 1000, 8, 2, 128, 128, "bf16", "gauss"),
}


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(_bits(a), _bits(b))


def _same_step(r1, r2) -> bool:
    (o1, l1, x1), (o2, l2, x2) = r1, r2
    ok = _same(o1, o2) and _same(l1, l2)
    ok = ok and all(torch.equal(x1[n].view(torch.uint8), x2[n].view(torch.uint8)) for n in ("q", "k", "v"))
    if x1["scales"] is not None:
        ok = ok and _same(x1["scales"], x2["scales"])
    return ok


@pytest.mark.parametrize("case", list(CASES))
def test_side_stream_matches_default_stream(case):
    w = CASES[case]
    q, k, v = (dev(x) for x in make_inputs(w, seed=5))
    print(f"case {w.name} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk}/{w.d_v} on a side stream", flush=True)
    ref = ops.prefill(q, k, v, w.dtype)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        r1 = ops.prefill(q, k, v, w.dtype)           # the current stream is s
    r2 = ops.prefill(q, k, v, w.dtype, stream=s)     # s given explicitly
    s.synchronize()
    torch.cuda.synchronize()
    assert _same_step(r1, ref) and _same_step(r2, ref)


@pytest.mark.parametrize("case", list(CASES))
def test_captured_graph_replays_match_eager(case):
    w = CASES[case]
    inputs = [tuple(dev(x) for x in make_inputs(w, seed=s)) for s in (6, 7, 8)]
    sq, sk, sv = (t.clone() for t in inputs[0])      # the graph's static inputs
    print(f"case {w.name} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d_qk}/{w.d_v} captured", flush=True)
    # warm-up on a side stream before the capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ops.prefill(sq, sk, sv, w.dtype)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = ops.prefill(sq, sk, sv, w.dtype)
    torch.cuda.synchronize()
    for rep in range(6):
        q, k, v = inputs[rep % 3]
        sq.copy_(q)
        sk.copy_(k)
        sv.copy_(v)
        g.replay()
        torch.cuda.synchronize()
        eager = ops.prefill(q, k, v, w.dtype)
        torch.cuda.synchronize()
        assert _same_step(captured, eager), f"replay {rep} differs from the eager step"
        if rep == 0:
            o = captured[0].float().cpu().numpy()
            assert np.all(np.isfinite(o))
