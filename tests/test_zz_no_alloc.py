"""The allocation-free sparsified all-reduce against the workspace form.

rsx_sparse_all_reduce_noalloc (through the C ABI, via the binding's
``noalloc=True``) must give the same bits as rsx_sparse_all_reduce on the same
inputs: results on every rank, residuals, message lengths and every message
entry.  Two calls in a row share the library's scratch array, the second on a
smaller input, so contents left by the first must not matter.
"""
import numpy as np
import pytest
import torch

import collective_reduction_ring_amd as rsx
from parity_util import say

pytestmark = pytest.mark.gpu

f32 = np.float32


def _inputs(seed, w, n):
    rng = np.random.default_rng(seed)
    grads = [(rng.standard_normal(n) * 1e-3).astype(f32) for _ in range(w)]
    accs = [(rng.standard_normal(n) * 1e-3).astype(f32) for _ in range(w)]
    return grads, accs


def _run(grads, accs, mode, kw, noalloc):
    w, n = len(grads), len(grads[0])
    g = [torch.from_numpy(x).to("cuda:0") for x in grads]
    a = [torch.from_numpy(x).to("cuda:0") for x in accs]
    outs = [torch.full((n,), 7.0, device="cuda:0") for _ in range(w)]
    plan = rsx.SparseAllReduce(g, a, outs, mode, noalloc=noalloc, **kw)
    plan()
    torch.cuda.synchronize()
    nnz = plan.nnz_host()
    msgs = [(plan.msg_idx[r][:nnz[r]].cpu().numpy(), plan.msg_val[r][:nnz[r]].cpu().numpy())
            for r in range(w)]
    return [o.cpu().numpy() for o in outs], [t.cpu().numpy() for t in a], nnz, msgs


def _same_bits(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, what
    bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    if got.dtype == np.float32:
        bad = bad[~(np.isnan(got[bad]) & np.isnan(want[bad]))]
    assert bad.size == 0, f"{what}: {bad.size} differ, first at {bad[:5].tolist()}"


@pytest.mark.parametrize("mode", ["threshold", "topk"])
def test_noalloc_matches_workspace_form_on_two_calls(mode):
    kw = {"fraction": 0.01} if mode == "topk" else {"threshold": 1.8e-3}
    # first call near the scratch limit (W = 8, 1.9 M per rank: about 122 MiB
    # of workspace), then a smaller one (W = 3, 50,000 per rank)
    for seed, (w, n) in enumerate([(8, 1_900_000), (3, 50_000)]):
        grads, accs = _inputs(100 + seed, w, n)
        say(f"noalloc {mode}: call {seed + 1}, W={w} n={n}")
        got = _run(grads, accs, mode, kw, noalloc=True)
        want = _run(grads, accs, mode, kw, noalloc=False)
        assert got[2] == want[2], (mode, w, n)
        for r in range(w):
            _same_bits(got[0][r], want[0][r], f"{mode} W={w} rank {r} result")
            _same_bits(got[1][r], want[1][r], f"{mode} W={w} rank {r} residual")
            _same_bits(got[3][r][0], want[3][r][0], f"{mode} W={w} rank {r} message indices")
            _same_bits(got[3][r][1], want[3][r][1], f"{mode} W={w} rank {r} message values")


def test_noalloc_refuses_sizes_beyond_the_scratch_array():
    w, n = 8, 2_200_000
    g = [torch.zeros(n, device="cuda:0") for _ in range(w)]
    with pytest.raises(rsx.RsxError) as e:
        rsx.SparseAllReduce(g, None, None, "threshold", threshold=1.0, noalloc=True)()
    assert e.value.status == 4
