"""GPU parity of the device Cassandra encoder ([Cassandra] 3.2-3.3, the online
encoder of 3.5): all eight sections bit-exact against the oracle's packing on
ragged shapes, keep fractions, exact score ties and special values, the full
4096 x 14336 workload the encoder is timed on, a restore of the encoded sections
back to the original bits, and the error path."""
import ctypes

import numpy as np
import pytest

import synth
from oracle import cassandra

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAMES = ["bitmap", "spec_nib", "unary", "codebook", "bitoff", "kprefix", "lo_nib", "pruned"]


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


def _encode(dev, w, norms, keep):
    mbd = _mbd()
    M, K = w.shape
    wd = torch.from_numpy(np.ascontiguousarray(w).view(np.int16)).to(dev)
    nd = torch.from_numpy(np.ascontiguousarray(norms, dtype=np.float32)).to(dev)
    ws = torch.empty(mbd.mbd_encode_workspace_bytes(M), dtype=torch.uint8, device=dev)
    plan = mbd.mbd_encode_plan(wd, nd, keep[0], keep[1], ws)
    secs = [torch.full((int(plan.padded_bytes[i]),), 0xA5, dtype=torch.uint8, device=dev) for i in range(8)]
    mbd.mbd_encode_cassandra(wd, nd, keep[0], keep[1], plan, secs, ws)
    torch.cuda.synchronize()
    return plan, secs


def _check(dev, w, norms, keep):
    M, K = w.shape
    ref = cassandra.pack(w, norms, *keep)
    plan, secs = _encode(dev, w, norms, keep)
    assert plan.n_kept == ref["n_kept"] and plan.n_sym == ref["n_sym"] and plan.unary_bits == ref["unary_bits"]
    for i, name in enumerate(NAMES):
        want = np.asarray(ref[name])
        raw = secs[i].cpu().numpy()
        nbytes = int(plan.bytes[i])
        assert nbytes == want.nbytes, name
        np.testing.assert_array_equal(raw[:nbytes].view(want.dtype), want.reshape(-1), err_msg=name)
        assert not raw[nbytes:].any(), name + " padding"
    return plan, secs


SHAPES = [(3, 1024, (3, 10)), (5, 128, (1, 2)), (33, 1152, (3, 10)), (2, 4096 + 128, (3, 10)), (7, 256, (0, 1)),
          (2, 256, (1, 1)), (17, 8192, (3, 10)), (1, 28672, (3, 10)),
          (2, 40960, (3, 10)), (1, 65536 + 128, (3, 10))]      # wider rows: other thread layouts


@pytest.mark.parametrize("M,K,keep", SHAPES)
def test_encoder_ragged(dev, M, K, keep):
    print("case encoder", M, K, keep, flush=True)
    rng = np.random.default_rng(M * 7 + K)
    w = synth.f32_to_bf16_bits((rng.standard_t(4, (M, K)) * 0.02).astype(np.float32))
    w[0, :6] = [0, 0x8000, 1, 0x8001, 0x3F80, 0xBF80]            # zeros, subnormals, +-1
    norms = rng.lognormal(0, 1, K).astype(np.float32)
    _check(dev, w, norms, keep)


def test_encoder_ties(dev):
    """Many equal scores: the keep rule takes the lower columns first."""
    rng = np.random.default_rng(5)
    M, K = 9, 640
    w = (rng.choice([0x3C00, 0xBC00, 0x3C80, 0], (M, K))).astype(np.uint16)     # few distinct magnitudes
    norms = np.ones(K, np.float32)
    norms[::7] = 2.0
    _check(dev, w, norms, (3, 10))


def test_encoder_workload_rows_and_restore(dev):
    mbd = _mbd()
    wl = synth.WORKLOADS["cassandra_spec"]
    w = synth.gen_weights(wl, 0, 256)
    norms = synth.gen_act_norms(wl)
    print("case encoder 256x14336 + restore", flush=True)
    plan, secs = _check(dev, w, norms, (3, 10))
    M, K = w.shape
    d = mbd.MbdDWeights()
    d.fmt, d.n_sym, d.M, d.K, d.n_kept, d.n_mats = mbd.MBD_CASSANDRA, plan.n_sym, M, K, plan.n_kept, 1
    for i in range(8):
        d.sec[i] = secs[i].data_ptr()
    out = torch.empty((M, K), dtype=torch.int16, device=dev)
    mbd.check(mbd.lib().mbd_verify_restore(ctypes.byref(d), mbd._ptr(out), None), "mbd_verify_restore")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), w)


def test_encoder_full_workload(dev):
    """The whole 4096 x 14336 weight the encoder is timed on: all eight sections
    bit-exact against the oracle's pack (matrix-global codebook ranking, u64 bit
    offsets and kept prefixes of all 14 336 tiles)."""
    wl = synth.WORKLOADS["cassandra_spec"]
    w = synth.gen_weights(wl)
    norms = synth.gen_act_norms(wl)
    print("case encoder full 4096x14336", flush=True)
    plan, _ = _check(dev, w, norms, (3, 10))
    assert plan.n_kept == wl.M * cassandra.keep_count(wl.K) and plan.n_tiles == wl.M * wl.K // cassandra.TILE


def test_encoder_rejects_nonfinite(dev):
    mbd = _mbd()
    w = np.zeros((2, 256), np.uint16)
    w[1, 3] = 0x7F80                                            # +Inf
    wd = torch.from_numpy(w.view(np.int16)).to(dev)
    nd = torch.ones(256, dtype=torch.float32, device=dev)
    ws = torch.empty(mbd.mbd_encode_workspace_bytes(2), dtype=torch.uint8, device=dev)
    with pytest.raises(mbd.MbdError) as e:
        mbd.mbd_encode_plan(wd, nd, 3, 10, ws)
    assert e.value.status == mbd.MBD_ERANGE
    w[1, 3] = 0
    nd[5] = -1.0
    with pytest.raises(mbd.MbdError) as e:
        mbd.mbd_encode_plan(torch.from_numpy(w.view(np.int16)).to(dev), nd, 3, 10, ws)
    assert e.value.status == mbd.MBD_ERANGE
