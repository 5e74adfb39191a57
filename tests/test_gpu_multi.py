"""GPU parity of the multi-projection launch (several projections of one x).

aqg_gemv_bf16_multi / aqg_gemv_affine_q{b}_multi compute y_p = x . W_p^T for
up to four projections in one call.  Bars: every output within the GEMV
bound of the oracle; when the launch is fused (one kernel with a projection
table), every output bit-equal to the same row of a single call on the
concatenated matrix; ragged and unaligned row counts (the latter launched
one projection at a time); canary guards around every output.  Shapes: the
q/k/v projections of the hidden-1536 decode set (dense) and of the ~0.8B
decoder (4-bit 1024 x 1024), M = 1..32.
"""
import numpy as np
import pytest
import torch

import affine_quantized_gemv_amd as aqg
import oracle
import synth
from gpu_helpers import Guarded, assert_within, bf16_dev, u32_dev

pytestmark = pytest.mark.gpu
FUSED = {"piece", "mfma_split", "affine_split"}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aqg.load()
    yield


def _guarded(M, Ns, dtype):
    gs = [Guarded(M, n, dtype) for n in Ns]
    return gs, [g.out for g in gs]


def _run_dense(xd, Ws, Wd, M, Ns):
    g32, outs = _guarded(M, Ns, torch.float32)
    aqg.gemv_bf16_multi(xd[:M], Wd, out=outs)
    g16, outs16 = _guarded(M, Ns, torch.bfloat16)
    aqg.gemv_bf16_multi(xd[:M], Wd, out=outs16)
    torch.cuda.synchronize()
    for a, b in zip(g32, g16):
        a.check()
        b.check()
        assert np.array_equal(b.numpy(), oracle.f32_to_bf16(a.numpy())), "bf16 != RNE(fp32)"
    return [g.numpy().astype(np.float64) for g in g32]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 16, 17, 32])
def test_dense_qkv_fused(M):
    K = 1536
    x = synth.activations(synth.CFG_DENSE_DECODE, K)
    Ws = [synth.dense_weight(synth.CFG_DENSE_DECODE, n, 1536, K) for n in ("q_proj", "k_proj", "v_proj")]
    Ns = [1536, 1536, 1536]
    xd, Wd = bf16_dev(x), [bf16_dev(W) for W in Ws]
    path = aqg.dispatch_path(0, M, sum(Ns), K)[0]
    assert path in FUSED, path
    ys = _run_dense(xd, Ws, Wd, M, Ns)
    cat = aqg.gemv_bf16(xd[:M], torch.cat(Wd), out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    r0 = 0
    for y, W, n in zip(ys, Ws, Ns):
        ref, A = oracle.gemv_bf16(x[:M], W)
        assert_within(y, ref, oracle.tolerance(A), "q/k/v M=%d (%s)" % (M, path))
        assert np.array_equal(y, cat[:, r0:r0 + n]), "fused output differs from the concatenated call"
        r0 += n


@pytest.mark.parametrize("Ns", [[1024, 512, 300], [16, 4096], [2048, 1024, 1024, 1000], [100, 200, 3]],
                         ids=lambda n: "x".join(map(str, n)))
@pytest.mark.parametrize("M", [1, 4, 12, 32])
def test_dense_ragged_and_unaligned(Ns, M):
    K = 1024
    x = synth.normal_bf16((M, K), 1.0, 64, "mu/x")
    Ws = [synth.dense_weight(64, "mu/%d/%d" % (i, n), n, K) for i, n in enumerate(Ns)]
    xd, Wd = bf16_dev(x), [bf16_dev(W) for W in Ws]
    ys = _run_dense(xd, Ws, Wd, M, Ns)
    for y, W in zip(ys, Ws):
        ref, A = oracle.gemv_bf16(x, W)
        assert_within(y, ref, oracle.tolerance(A), "dense multi %s M=%d" % (Ns, M))


@pytest.mark.parametrize("bits,Ns,K", [(4, [1024, 1024, 1024], 1024), (4, [2048, 512, 512], 1024),
                                       (8, [1024, 256, 256], 1024), (2, [4096, 1024], 2048),
                                       (3, [1024, 1024, 1024], 1024), (4, [1000, 24], 1024)])
@pytest.mark.parametrize("M", [1, 4, 5, 16, 32])
def test_affine_qkv(bits, Ns, K, M):
    x = synth.activations(synth.CFG_AFFINE4_08B, K)[:M]
    aws = [synth.affine_weight(synth.CFG_AFFINE4_08B, "mq/%d/%d" % (i, n), bits, n, K) for i, n in enumerate(Ns)]
    xd = bf16_dev(x)
    mats = [(u32_dev(a.words), bf16_dev(a.scales), bf16_dev(a.biases)) for a in aws]
    g32, outs = _guarded(M, Ns, torch.float32)
    aqg.gemv_affine_multi(xd, mats, bits, out=outs)
    torch.cuda.synchronize()
    path = aqg.dispatch_path(bits, M, sum(Ns), K)[0]
    fused = path in FUSED and all(n % 16 == 0 for n in Ns[:-1])
    if fused:
        cat = aqg.gemv_affine(xd, torch.cat([m[0] for m in mats]), torch.cat([m[1] for m in mats]),
                              torch.cat([m[2] for m in mats]), bits, out_dtype=torch.float32).cpu().numpy()
    r0 = 0
    for g, a, n in zip(g32, aws, Ns):
        g.check()
        y = g.numpy().astype(np.float64)
        ref, A = oracle.gemv_affine(x, a.words, a.scales, a.biases, bits)
        assert_within(y, ref, oracle.tolerance(A), "q%d multi %s M=%d (%s)" % (bits, Ns, M, path))
        if fused:
            assert np.array_equal(y, cat[:, r0:r0 + n].astype(np.float64))
        r0 += n
