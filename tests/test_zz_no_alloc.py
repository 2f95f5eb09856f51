"""The allocation-free expert GEMV (mbd_moe_gemv_noalloc, the library's static device
scratch in place of a caller workspace) against the workspace entry point
(mbd_moe_gemv) on the same inputs: identical outputs on consecutive calls, the second
with a smaller route, over the grouping paths that use the scratch (the grouping
kernel above 256 pairs, the one-workgroup sort up to 256) and one that does not (one
token).  Both calls run the same kernels, so the outputs must agree bit for bit; the
first call is also held to the oracle."""
import numpy as np
import pytest

import synth
from tests._gate import check
from oracle import bits, gemv, int4, ternary

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import memory_bound_decode_amd as mbd
    mbd.lib()
    return torch.device("cuda:0")


def _x_dev(x_bits, dev):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(dev)


def _setup(kind, E, M, K, dev):
    import memory_bound_decode_amd as mbd
    rng = np.random.default_rng(E * 7 + M)
    mats = [synth.f32_to_bf16_bits((rng.standard_t(4, (M, K)) * 0.02).astype(np.float32)) for _ in range(E)]
    fmt = mbd.MBD_TERNARY_B128 if kind == "ternary" else mbd.MBD_INT4_G128
    dw = mbd.to_device(mbd.mbd_pack(fmt, np.concatenate(mats), n_mats=E), dev, n_mats=E)
    return mats, dw


def _routes(seed, E, T, k):
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("kind", ["ternary", "int4"])
def test_noalloc_matches_workspace_entry(dev, kind):
    import memory_bound_decode_amd as mbd
    E, M, K, k = 24, 48, 512, 8
    print("case noalloc", kind, E, M, K, k, flush=True)
    mats, dw = _setup(kind, E, M, K, dev)
    mod = ternary if kind == "ternary" else int4
    deq = [mod.dequant(*mod.quantize(m)) for m in mats]
    for i, (T, per_pair) in enumerate([(64, False), (20, True), (1, False), (40, True)]):
        routes = _routes(1000 + T, E, T, k)
        xb = synth.f32_to_bf16_bits(np.random.default_rng(T).standard_normal(
            (T * k if per_pair else T, K)).astype(np.float32))
        r, x = torch.from_numpy(routes).to(dev), _x_dev(xb, dev)
        ws = torch.empty(mbd.mbd_moe_workspace_bytes(E, T, k), dtype=torch.uint8, device=dev)
        y_ws = torch.full((T, k, M), float("nan"), dtype=torch.float32, device=dev)
        y_na = torch.full((T, k, M), float("nan"), dtype=torch.float32, device=dev)
        mbd.mbd_moe_gemv(dw, r, x, per_pair, y_ws, ws)
        mbd.mbd_moe_gemv_noalloc(dw, r, x, per_pair, y_na)
        torch.cuda.synchronize()
        a, b = y_ws.cpu().numpy(), y_na.cpu().numpy()
        assert not np.isnan(b).any()
        np.testing.assert_array_equal(b, a, err_msg="call %d (T=%d)" % (i, T))
        if i == 0:
            xv = bits.bf16_value(xb)
            ref = np.stack([[deq[routes[t, j]] @ (xv[t * k + j] if per_pair else xv[t]) for j in range(k)]
                            for t in range(T)])
            err, worst = check(b.astype(np.float64), ref)
            print("noalloc %s T=%d rel_l2=%.3e worst_row=%.3e" % (kind, T, err, worst), flush=True)
            assert err <= 1e-3
