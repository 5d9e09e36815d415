"""bcq_quantize (the HIP progressive-precision quantizer) against the float64
reference quantizer oracle/quantize.py: sign planes bit-exact, fp64 scales
and offsets bit-exact (both take every decision on the same exactly rounded
values), fp16/fp32 tables equal to the reference's values rounded once; then
a quantized store served through bcq_gemv_mixed_p at per-request precisions."""

import sys

import numpy as np
import pytest

import bcq_synth
import oracle
from oracle import quantize as qref

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import binary_coded_precision_amd as bcq  # noqa: E402


def say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    return float(np.linalg.norm(got - ref) / np.linalg.norm(ref))


def run(W, P, p_low, iters, out=torch.float64, pad=0):
    M, K = W.shape
    Wd = torch.zeros((M, K + pad), dtype=torch.float16 if W.dtype == np.float16 else torch.float32,
                     device="cuda")
    Wd[:, :K] = torch.from_numpy(W).cuda()
    signs, alpha, zero = bcq.bcq_quantize(Wd[:, :K] if pad else Wd, P, p_low, iters, out_dtype=out)
    torch.cuda.synchronize()
    return (signs.cpu().numpy().view(np.uint32), {p: a.cpu().numpy() for p, a in alpha.items()},
            {p: z.cpu().numpy() for p, z in zero.items()})


@pytest.mark.parametrize("M,K,P,p_low,iters,dt,pad", [
    (64, 512, 4, 2, 20, np.float16, 0),   # the pages' recipe: base 2 bits, 20 rounds, up to 4
    (37, 384, 4, 2, 20, np.float16, 8),   # ragged rows, padded leading dimension
    (48, 256, 3, 1, 5, np.float32, 0),    # fp32 weights, base precision 1
    (16, 128, 2, 2, 0, np.float16, 0),    # no refinement round
    (40, 640, 4, 4, 3, np.float16, 0),    # no expansion
])
def test_quantizer_bit_exact_against_reference(M, K, P, p_low, iters, dt, pad):
    W = bcq_synth.weights(M, K, dtype=dt, seed=M + K + P)
    say("quantize", M, K, P, p_low, iters, np.dtype(dt).name, pad)
    signs, alpha, zero = run(W, P, p_low, iters, pad=pad)
    rs, ra, rz = qref.quantize(W, P, p_low, iters)
    assert np.array_equal(signs, rs)
    assert sorted(alpha) == list(range(p_low, P + 1))
    for p in range(p_low, P + 1):
        assert np.array_equal(alpha[p], ra[p]), p
        assert np.array_equal(zero[p], rz[p]), p


def test_quantizer_tables_rounded_once_to_fp16_and_fp32():
    W = bcq_synth.weights(32, 512, seed=3)
    _, ra, rz = qref.quantize(W, 4, 2, 20)
    for out, npdt in ((torch.float16, np.float16), (torch.float32, np.float32)):
        say("quantize rounding", npdt.__name__)
        _, alpha, zero = run(W, 4, 2, 20, out=out)
        for p in range(2, 5):
            assert np.array_equal(alpha[p].view(np.uint8), ra[p].astype(npdt).view(np.uint8)), p
            assert np.array_equal(zero[p].view(np.uint8), rz[p].astype(npdt).view(np.uint8)), p


def test_fp16_rounding_of_halfway_and_subnormal_scales():
    """Groups of +-a (fp32 weights, half of each sign): offset 0 and scale a
    exactly, so the fp16 table shows the rounding of a itself -- halfway cases
    go to the even neighbour, tiny values to subnormals or zero."""
    vals = [1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2.0 ** -25, 3 * 2.0 ** -26, 65520.0,
            65519.0, 2.0 ** -14 * (1 - 2.0 ** -11), float(np.float32(0.1)), 2.0 ** -24 * 1.5]
    rng = np.random.default_rng(0)
    W = np.empty((len(vals), 128), np.float32)
    for m, a in enumerate(vals):
        s = np.array([1.0] * 64 + [-1.0] * 64)[rng.permutation(128)]
        W[m] = (s * a).astype(np.float32)
    assert all(np.float32(a) == a for a in vals)
    say("quantize fp16 ties")
    _, alpha, zero = run(W, 1, 1, 2, out=torch.float16)
    with np.errstate(over="ignore"):  # 65520 rounds to infinity, as it must
        want = np.array(vals, np.float64).astype(np.float16)
    assert np.array_equal(alpha[1][0, :, 0].view(np.uint16), want.view(np.uint16))
    assert np.all(zero[1] == 0)


def test_quantizer_full_layer_sampled_rows():
    """4096x4096 (one q_proj-shaped layer): every sign word and fp64 table of
    sampled rows (rows are quantized independently) against the reference."""
    M, K = 4096, 4096
    W = bcq_synth.weights(M, K, seed=44)
    say("quantize 4096x4096")
    signs, alpha, zero = run(W, 4, 2, 20)
    rows = np.array([0, 1, 777, 2048, 4095])
    rs, ra, rz = qref.quantize(W[rows], 4, 2, 20)
    assert np.array_equal(signs[:, rows], rs)
    for p in range(2, 5):
        assert np.array_equal(alpha[p][:, rows], ra[p]) and np.array_equal(zero[p][rows], rz[p])


def test_quantized_store_serves_every_precision():
    """Quantize on the GPU (fp16 tables), pack, and run per-request
    precisions 2, 3, 4 through bcq_gemv_mixed_p: each request against the
    float64 product of the same store; the reconstruction error of the store
    falls as precision rises (AnyBCQ paper notes: accuracy rises monotonically
    as bits are added)."""
    M, K = 1024, 2048
    W = bcq_synth.weights(M, K, seed=9)
    Wd = torch.from_numpy(W).cuda()
    say("quantized store")
    signs, alpha, zero = bcq.bcq_quantize(Wd, 4, 2, 20)
    st = bcq.Store.from_quantized(signs, alpha, zero)
    ps = [2, 3, 4, 4, 2, 3]
    X = np.random.default_rng(1).standard_normal((len(ps), K)).astype(np.float16)
    Y = torch.empty((len(ps), M), dtype=torch.float16, device="cuda")
    bcq.bcq_gemv_mixed_p(st, ps, torch.from_numpy(X).cuda(), Y)
    sg = signs.cpu().numpy().view(np.uint32)
    a_h = {p: alpha[p].cpu().numpy() for p in alpha}
    z_h = {p: zero[p].cpu().numpy() for p in zero}
    ref = oracle.gemv_requests(sg, X, ps, lambda p: a_h[p], lambda p: z_h[p])
    got = Y.cpu().numpy()
    for r in range(len(ps)):
        assert rel_l2(got[r], ref[r]) <= 2e-3, r
    err = [np.linalg.norm(oracle.dequant(sg, a_h[p], z_h[p], p, K) - W.astype(np.float64))
           for p in (2, 3, 4)]
    assert err[0] > err[1] > err[2], err
