"""HIP-graph replays of every launch sequence the bench times: each call is
captured once, the graph is replayed several times with eager work and
synchronisations in between, and every replay must equal the eager result bit
for bit (the kernels reduce in a fixed order, so repeated calls agree exactly)."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

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


def _bits(seed, shape, scale=0.02):
    rng = np.random.default_rng(seed)
    return synth.f32_to_bf16_bits((rng.standard_t(4, shape) * scale).astype(np.float32))


def _xd(seed, B, K, dev):
    x = synth.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((B, K)).astype(np.float32))
    return torch.from_numpy(x.view(np.int16)).to(dev)


def _replays_match(call, outs, n=3):
    """call() enqueues the work writing the tensors `outs`; eager result vs n replays."""
    call()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(n):
        for o in outs:
            o.fill_(float("nan") if o.dtype == torch.float32 else 0x5A)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o, w), "replay %d differs from the eager call" % i


@pytest.mark.parametrize("fmt,B", [("int4", 1), ("int4", 4), ("int4", 8), ("ternary", 1), ("ternary", 16),
                                   ("skip", 1), ("skip", 8)])
def test_graph_gemv(dev, fmt, B):
    mbd = _mbd()
    M, K = 300, 4096
    w = _bits(1, (M, K))
    if fmt == "skip":
        w = synth.zero_out_blocks(w, synth.gen_zero_blocks(3, M, K, 0.3))
    f = {"int4": mbd.MBD_INT4_G128, "ternary": mbd.MBD_TERNARY_B128, "skip": mbd.MBD_TERNARY_SKIP}[fmt]
    dw = mbd.to_device(mbd.mbd_pack(f, w), dev)
    x = _xd(2, B, K, dev)
    y = torch.empty((B, M), dtype=torch.float32, device=dev)
    _replays_match(lambda: mbd.mbd_gemv(dw, x, y), [y])


@pytest.mark.parametrize("T", [1, 8])
def test_graph_moe(dev, T):
    mbd = _mbd()
    E, k, M, K = 16, 4, 96, 512
    w = _bits(5, (E * M, K))
    dw = mbd.to_device(mbd.mbd_pack(mbd.MBD_INT4_G128, w, n_mats=E), dev, n_mats=E)
    rng = np.random.default_rng(T)
    route = torch.from_numpy(np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)).to(dev)
    x = _xd(6, T, K, dev)
    y = torch.empty((T, k, M), dtype=torch.float32, device=dev)
    ws = torch.empty(mbd.mbd_moe_workspace_bytes(E, T, k), dtype=torch.uint8, device=dev)
    _replays_match(lambda: mbd.mbd_moe_gemv(dw, route, x, False, y, ws), [y])


def test_graph_cassandra(dev):
    mbd = _mbd()
    M, K = 48, 8192
    w = _bits(7, (M, K))
    norms = np.random.default_rng(8).lognormal(0, 1, K).astype(np.float32)
    cw = mbd.to_device(mbd.mbd_pack(mbd.MBD_CASSANDRA, w, norms), dev)
    x1, x16 = _xd(9, 1, K, dev), _xd(10, 16, K, dev)
    y1 = torch.empty((1, M), dtype=torch.float32, device=dev)
    y16 = torch.empty((16, M), dtype=torch.float32, device=dev)
    out = torch.empty((M, K), dtype=torch.int16, device=dev)

    def call():
        mbd.mbd_spec_gemv(cw, x1, y1)
        mbd.mbd_gemv(cw, x16, y16)
        mbd.mbd_verify_restore(cw, out)
    _replays_match(call, [y1, y16, out])
    mw = mbd.to_device(mbd.mbd_pack(mbd.MBD_CASSANDRA_MX, w, norms), dev)
    _replays_match(lambda: mbd.mbd_spec_gemv(mw, x1, y1), [y1])
    xw = mbd.to_device(mbd.mbd_pack(mbd.MBD_MX32, w), dev)
    _replays_match(lambda: mbd.mbd_gemv(xw, x16, y16), [y16])


def test_graph_encoder(dev):
    mbd = _mbd()
    M, K = 40, 4096
    w = _bits(11, (M, K))
    norms = np.random.default_rng(12).lognormal(0, 1, K).astype(np.float32)
    wd = torch.from_numpy(w.view(np.int16)).to(dev)
    nd = torch.from_numpy(norms).to(dev)
    ws = torch.empty(mbd.mbd_encode_workspace_bytes(M), dtype=torch.uint8, device=dev)
    plan = mbd.mbd_encode_plan(wd, nd, 3, 10, ws)
    secs = [torch.empty(int(plan.padded_bytes[i]), dtype=torch.uint8, device=dev) for i in range(8)]
    _replays_match(lambda: mbd.mbd_encode_cassandra(wd, nd, 3, 10, plan, secs, ws), secs)
