"""GPU parity of the Cassandra-2 draft path (kept exponents as MX-32, [Cassandra]
§3.3): draft decode bit-exact against the oracle and the draft GEMV within
rel-L2 1e-3 of the fp64 product of the oracle's draft weights, on ragged shapes
(K below, at and above the 4096-element tile, several keep fractions, batch 1 to
16) and on the full 4096 x 14336 draft workload."""
import numpy as np
import pytest

import synth
from tests._gate import check
from oracle import bits, cassandra_mx, gemv

pytestmark = pytest.mark.gpu

TOL = 1e-3

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_decode_amd as mbd
    mbd.lib()
    return torch.device("cuda:0")


def _mbd():
    import memory_bound_decode_amd as mbd
    return mbd


def _x_dev(x_bits, dev):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(dev)


def _check(dev, w, norms, keep, batches):
    mbd = _mbd()
    M, K = w.shape
    sec = cassandra_mx.pack_spec(w, norms, *keep)
    expect = cassandra_mx.spec_decode(sec, M, K)
    dw = mbd.to_device(mbd.mbd_pack(mbd.MBD_CASSANDRA_MX, w, norms, *keep), dev)
    out = torch.empty((M, K), dtype=torch.int16, device=dev)
    mbd.mbd_spec_decode(dw, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), expect)
    W = bits.bf16_value(expect)
    for B in batches:
        x = synth.f32_to_bf16_bits(np.random.default_rng(B + K).standard_normal((B, K)).astype(np.float32))
        y = torch.full((B, M), float("nan"), dtype=torch.float32, device=dev)
        mbd.mbd_spec_gemv(dw, _x_dev(x, dev), y)
        torch.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got))
        err, worst = check(got, gemv.gemv(W, x))
        assert err <= TOL, (B, err)


SHAPES = [(1, 128, (3, 10)), (5, 384, (3, 10)), (33, 1152, (3, 10)), (3, 4096 + 128, (3, 10)),
          (17, 8192, (3, 10)), (4, 14336, (3, 10)), (9, 2048, (1, 10)), (6, 1024, (1, 1)), (7, 512, (0, 1))]


@pytest.mark.parametrize("M,K,keep", SHAPES)
def test_mx_draft_ragged(dev, M, K, keep):
    print("case mx draft", M, K, keep, flush=True)
    rng = np.random.default_rng(M * 31 + K)
    w = synth.f32_to_bf16_bits((rng.standard_t(4, (M, K)) * 0.02).astype(np.float32))
    w[0, :6] = [0, 0x8000, 1, 0x8001, 0x3F80, 0xBF80]           # zeros, subnormals, +-1
    norms = rng.lognormal(0, 1, K).astype(np.float32)
    _check(dev, w, norms, keep, [1, 2, 3, 8, 16])


def test_mx_draft_full(dev):
    wl = synth.WORKLOADS["cassandra_spec"]
    w = synth.gen_weights(wl)
    norms = synth.gen_act_norms(wl)
    print("case mx draft full 4096x14336", flush=True)
    _check(dev, w, norms, (3, 10), [1, 2])


def test_mx_draft_rejects_verify_calls(dev):
    mbd = _mbd()
    rng = np.random.default_rng(2)
    w = synth.f32_to_bf16_bits((rng.standard_normal((4, 256)) * 0.02).astype(np.float32))
    dw = mbd.to_device(mbd.mbd_pack(mbd.MBD_CASSANDRA_MX, w, np.ones(256, np.float32)), dev)
    y = torch.empty((1, 4), dtype=torch.float32, device=dev)
    x = _x_dev(synth.f32_to_bf16_bits(np.ones((1, 256), np.float32)), dev)
    with pytest.raises(mbd.MbdError):
        mbd.mbd_gemv(dw, x, y)                           # speculation data only
