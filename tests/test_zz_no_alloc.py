"""bcq_gemm_skinny_noalloc through the C ABI: the same results as
bcq_gemm_skinny with a caller's workspace, bit for bit, on two calls in a row
(the second smaller, so it runs on scratch the first left dirty), plus a call
that needs no scratch; each also against the float64 oracle per request."""

import sys

import numpy as np
import pytest

import bcq_synth
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import binary_coded_precision_amd as bcq  # noqa: E402


def say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry_point(order):
    cases = [(4096, 4096, 64, 4, 11), (1024, 4096, 32, 3, 12), (2048, 4096, 8, 2, 13)]
    for M, K, b, p, seed in cases:
        w = bcq_synth.make(M, K, 4, b=b, dtype=np.float16, seed=seed, outlier_frac=0.01)
        st = bcq.Store.from_host(w.signs, w.alpha, w.zero)
        X = torch.from_numpy(np.ascontiguousarray(w.x)).cuda()
        need = bcq.bcq_workspace_bytes(st, b)
        say("noalloc", M, K, b, p, need)
        assert need <= bcq.BCQ_NOALLOC_SCRATCH_BYTES
        Yw = torch.full((b, M), 9.0, dtype=torch.float16, device="cuda")
        Yn = torch.full((b, M), 7.0, dtype=torch.float16, device="cuda")
        ws = bcq.new_workspace(st, b)
        bcq.bcq_gemm_skinny(st, p, X, Yw, workspace=ws)
        bcq.bcq_gemm_skinny_noalloc(st, p, X, Yn)
        torch.cuda.synchronize()
        assert torch.equal(Yw.view(torch.int16), Yn.view(torch.int16)), (M, K, b)
        rows = np.unique(np.concatenate([np.random.default_rng(seed).choice(M, 64, replace=False),
                                         [0, M - 1]]))
        ref = oracle.gemv_requests(w.signs[:, rows], w.x, [p] * b,
                                   lambda q: w.alpha_for(q)[:, rows], lambda q: w.zero_for(q)[rows])
        got = Yn.cpu().numpy()[:, rows]
        for r in range(b):
            assert rel_l2(got[r], ref[r]) <= 2e-3, (M, K, b, r)
