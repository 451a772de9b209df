"""The no-allocation entry point: cq_quantize_groups_noalloc, whose scratch is the library's fixed
per-GPU array, against cq_quantize_groups with a caller workspace, through the C ABI: every
method, two calls in a row on the same array, the second smaller than the first."""
import numpy as np
import pytest
import torch

import post_weight_quantization_group_amd as cq
import workloads as W
from parity import dev, say

pytestmark = pytest.mark.gpu

METHODS = [("exhaustive", cq.EXHAUSTIVE, True), ("bounded", cq.BOUNDED, True), ("candidate", cq.CANDIDATE, False)]


def _outputs(n, pooled):
    o = {"scales": torch.empty(n, dtype=torch.int16, device="cuda"),
         "codes": torch.empty((n, 128), dtype=torch.int8, device="cuda"),
         "objective": torch.empty(n, dtype=torch.float64, device="cuda"),
         "flags": torch.empty(n, dtype=torch.uint8, device="cuda")}
    if pooled:
        o["pooled_scales"] = torch.empty(n, dtype=torch.int16, device="cuda")
        o["pooled_objective"] = torch.empty(n, dtype=torch.float64, device="cuda")
    return o


def _call(fn, wt, dt, p, E, n, m, o, **kw):
    fn(wt, dt, p, E, n, m, o["scales"], o["codes"], o["objective"], o["flags"], o.get("pooled_scales"),
       o.get("pooled_objective"), **kw)


def _same(a, b, label):
    for k in a:
        assert torch.equal(a[k], b[k]), f"{label}: {k} differs"


@pytest.mark.parametrize("name,m,pooled", METHODS, ids=[x[0] for x in METHODS])
def test_noalloc_matches_workspace_call_twice(name, m, pooled):
    """A config-1 matrix (28,672 groups), then 700 groups (the bounded search slices a group over
    several workgroups below 1,024, using the slice parts of the scratch): both calls equal the
    workspace entry point's results bit for bit."""
    w, d, p = W.matrix_groups(*W.make_matrix(1, 0))
    E = d.shape[1]
    for n in (w.shape[0], 700):
        say(f"no-alloc {name}: {n} groups")
        wt, dt = dev(w[:n]), dev(d)
        a, b = _outputs(n, pooled), _outputs(n, pooled)
        ws = torch.empty(cq.cq_workspace_size(m, E, n), dtype=torch.uint8, device="cuda")
        _call(cq.cq_quantize_groups, wt, dt, p, E, n, m, a, workspace=ws)
        _call(cq.cq_quantize_groups_noalloc, wt, dt, p, E, n, m, b)
        torch.cuda.synchronize()
        _same(a, b, f"{name}, {n} groups")


def test_noalloc_after_a_tie_heavy_call():
    """Groups that fill the binary64 queue and the candidate solver's tie list (all-zero and
    symmetric-pair groups), then ordinary groups on the same scratch: the queue counters start at
    zero again."""
    rng = np.random.default_rng(3)
    n = 64
    w = np.zeros((n, 128), np.float32)
    c = 2.0 ** -6
    for j in range(0, n, 2):
        mult = np.array([1, 2, 3] + list(rng.integers(1, 4, 61)), np.float64)
        w[j] = np.concatenate([mult * c, -mult * c]).astype(np.float32)
    d = rng.lognormal(0, 1, (n, 4, 128)).astype(np.float32)
    w[1] = rng.normal(0, 0.02, 128).astype(np.float32)
    d[1, 1, 3] = 1e-38  # outside the binary32 screen's range: the binary64 queue
    w2, d2, p2 = W.matrix_groups(*W.make_matrix(0, 0))
    for m in (cq.CANDIDATE, cq.EXHAUSTIVE):
        for ww, dd, p in ((w, d, n), (w2, d2, p2)):
            k = ww.shape[0]
            a, b = _outputs(k, False), _outputs(k, False)
            ws = torch.empty(cq.cq_workspace_size(m, 4, k), dtype=torch.uint8, device="cuda")
            wt, dt = dev(ww), dev(dd)
            _call(cq.cq_quantize_groups, wt, dt, p, 4, k, m, a, workspace=ws)
            _call(cq.cq_quantize_groups_noalloc, wt, dt, p, 4, k, m, b)
            torch.cuda.synchronize()
            _same(a, b, f"method {m}, {k} groups")


def test_noalloc_rejects_more_groups_than_its_scratch():
    lib = cq.load()
    fake = 1 << 20
    assert lib.cq_quantize_groups_noalloc(fake, fake, 1, 4, (1 << 20) + 1, 0, fake, None, None, None, None, None,
                                          None) == -5
    assert lib.cq_quantize_groups_noalloc(None, None, 1, 4, 0, 0, None, None, None, None, None, None, None) == 0
    assert "no-allocation" in cq.cq_status_string(-5)
