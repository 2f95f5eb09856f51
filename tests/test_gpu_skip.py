"""GPU parity of the block-skipping ternary format (all-zero 128-blocks flagged and
not stored, [Bonsai2] §3.4 / §5.5): the fused GEMV against the fp64 oracle at
rel-L2 <= 1e-3 on ragged shapes, both kernels (batch 1..4 staged, 5..16 the
32-row kernel, and the staged chunks that take very long rows), full size on
sampled rows, and the dense dequant bit-exact."""
import numpy as np
import pytest

import synth
from tests._gate import check
from oracle import gemv, ternary

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


def _sparse_w(seed, M, K, frac):
    w = synth.f32_to_bf16_bits(synth.gen_weight_rows(seed, M, K, "t4", 0.02).astype(np.float32))
    return synth.zero_out_blocks(w, synth.gen_zero_blocks(seed, M, K, frac))


def _x(seed, B, K):
    return synth.f32_to_bf16_bits(np.random.default_rng(seed).standard_normal((B, K)).astype(np.float32))


def _xval(x_bits):
    return (np.asarray(x_bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _run(dw, x_bits, dev):
    mbd = _mbd()
    y = torch.full((x_bits.shape[0], dw.M), float("nan"), dtype=torch.float32, device=dev)
    mbd.mbd_gemv(dw, torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to(dev), y)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def _pack(w, dev):
    mbd = _mbd()
    return mbd.to_device(mbd.mbd_pack(mbd.MBD_TERNARY_SKIP, w), dev)


# (29, 16384): 16-wave blocks of the 32-row kernel (from 5 rows; with one block, 2..4
# rows stay on the few-row kernel, which the full 8192 x 28672 case below does not)
RAGGED = [(1, 128), (3, 384), (100, 1152), (333, 1536), (64, 4096), (17, 8320), (5, 128 * 45), (29, 16384)]


@pytest.mark.parametrize("M,K", RAGGED)
@pytest.mark.parametrize("B", [1, 2, 4, 5, 8, 16])
def test_skip_gemv_ragged(dev, M, K, B):
    print("case skip gemv", M, K, B, flush=True)
    w = _sparse_w(M * 5 + K, M, K, 0.3)
    x = _x(B * 3 + K, B, K)
    q, s = ternary.quantize(w)
    ref = gemv.gemv(ternary.dequant(q, s), x)
    y = _run(_pack(w, dev), x, dev)
    assert np.all(np.isfinite(y))
    check(y, ref)


@pytest.mark.parametrize("frac", [0.0, 0.9, 1.0])
@pytest.mark.parametrize("B", [1, 8])
def test_skip_gemv_extremes(dev, frac, B):
    """No block skipped, nearly all skipped, and all skipped.  With every block
    all-zero the oracle gives y = 0; the kernel's fp32 sum of (code value) x minus
    the per-group constant leaves only rounding.  Its terms are at most 129 |x_k|,
    so each rounding is at most 129 * 2^-24 sum |x| = 7.7e-6 sum |x|; the bound
    1e-5 sum |x| holds while the roundings partly cancel, as they do for random x."""
    print("case skip extremes", frac, B, flush=True)
    M, K = 70, 2048
    w = _sparse_w(17, M, K, frac)
    x = _x(4, B, K)
    y = _run(_pack(w, dev), x, dev)
    if frac == 1.0:
        bound = 1e-5 * np.abs(_xval(x)).sum(axis=1)
        print("all-zero max |y| %.3e, bound %.3e" % (np.abs(y).max(), bound.min()), flush=True)
        assert np.all(np.abs(y) <= bound[:, None])
        return
    q, s = ternary.quantize(w)
    check(y, gemv.gemv(ternary.dequant(q, s), x))


def test_skip_gemv_long_rows_batched(dev):
    """K = 131072: batch 6 runs as staged launches of 4 + 2 rows."""
    print("case skip long rows B=6", flush=True)
    M, K, B = 40, 131072, 6
    w = _sparse_w(23, M, K, 0.2)
    x = _x(6, B, K)
    q, s = ternary.quantize(w)
    check(_run(_pack(w, dev), x, dev), gemv.gemv(ternary.dequant(q, s), x))


@pytest.fixture(scope="module")
def skip_full(dev):
    """8192 x 28672 block-sparse ternary (t(4) * 0.02, 20% of blocks zero), the
    bench's shape."""
    wl = synth.WORKLOADS["ternary_moe"]
    M, K = 8192, 28672
    seed = wl.seed + 1000 * M + K
    w = synth.f32_to_bf16_bits(synth.gen_weight_rows(seed, M, K, wl.dist, wl.scale).astype(np.float32))
    w = synth.zero_out_blocks(w, synth.gen_zero_blocks(seed, M, K))
    return wl, w, _pack(w, dev)


@pytest.mark.parametrize("B", [1, 4, 8, 16])
def test_skip_gemv_full(dev, skip_full, B):
    wl, w, dw = skip_full
    M, K = w.shape
    x = synth.gen_x(wl, B, K)
    print("case skip 8192x28672 full B=%d" % B, flush=True)
    y = _run(dw, x, dev)
    assert np.all(np.isfinite(y))
    rows = np.unique(np.concatenate([np.arange(24), np.arange(M - 8, M),
                                     np.random.default_rng(B).integers(0, M, 40)]))
    q, s = ternary.quantize(w[rows])
    err, worst = check(y[:, rows], gemv.gemv(ternary.dequant(q, s), x))
    print("skip 8192x28672 B=%d rel_l2=%.3e worst_row=%.3e" % (B, err, worst), flush=True)
    assert err <= TOL


def test_skip_dequant_exact(dev):
    mbd = _mbd()
    M, K = 45, 1152
    w = _sparse_w(8, M, K, 0.35)
    dw = _pack(w, dev)
    out = torch.empty((M, K), dtype=torch.float32, device=dev)
    mbd.mbd_dequant(dw, out)
    torch.cuda.synchronize()
    q, s = ternary.quantize(w)
    np.testing.assert_array_equal(out.cpu().numpy().astype(np.float64), ternary.dequant(q, s))


def test_skip_and_dense_formats_on_block_sparse_weights(dev):
    """The same block-sparse weights in the skip and the dense format, each against
    the oracle.  The skip format adds exactly nothing for an all-zero block (scale 0
    in the kernel); the dense format stores such a block as codes q = 0 under the
    scale 1 of the pages' rule, and its offset sums (129 sum x in fp32, once with
    the codes and once as the bias) leave a rounding residue under that scale of 1,
    about 50 times the real blocks' scales: it meets the whole-output gate, and the
    skip format is at least as close to the oracle."""
    mbd = _mbd()
    M, K, B = 256, 4096, 3
    w = _sparse_w(31, M, K, 0.25)
    x = _x(31, B, K)
    q, s = ternary.quantize(w)
    ref = gemv.gemv(ternary.dequant(q, s), x)
    y_skip = _run(_pack(w, dev), x, dev)
    y_dense = _run(mbd.to_device(mbd.mbd_pack(mbd.MBD_TERNARY_B128, w), dev), x, dev)
    rs, ws = check(y_skip, ref)
    rd, wd = gemv.rel_l2(y_dense, ref), gemv.worst_row(y_dense, ref)
    print("block-sparse skip rel_l2=%.3e worst_row=%.3e; dense rel_l2=%.3e worst_row=%.3e" % (rs, ws, rd, wd),
          flush=True)
    assert rd <= TOL
    assert rs <= rd + 1e-7
