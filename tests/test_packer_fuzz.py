"""Property tests of the C++ packer against the oracle on random small shapes and
value mixes (zeros, subnormals, huge and tiny magnitudes, zeroed blocks): every
section bit-exact for every format, and the handle's validation accepts it."""
import numpy as np
import pytest

import synth
from oracle import cassandra, cassandra_mx, int4, mx, ternary, ternary_skip

mbd = pytest.importorskip("memory_bound_decode_amd")
hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _lib():
    try:
        mbd.lib()
    except ImportError as e:                         # pragma: no cover
        pytest.skip(str(e))


def _weights(seed, M, K, kind):
    rng = np.random.default_rng(seed)
    if kind == 0:
        v = rng.standard_t(4, (M, K)) * 0.02
    elif kind == 1:                                  # wide dynamic range
        v = rng.standard_normal((M, K)) * np.exp2(rng.integers(-30, 10, (M, K)))
    else:                                            # few distinct values: ties
        v = rng.choice([-0.5, -0.25, 0.0, 0.25, 0.5, 1e-40], (M, K))
    w = synth.f32_to_bf16_bits(v.astype(np.float32))
    zero = rng.random((M, K // 128)) < 0.2           # some all-zero blocks
    w = w.reshape(M, K // 128, 128)
    w[zero] = 0
    return w.reshape(M, K)


def _check(p, ref, names):
    for k in names:
        got = p.section(k, np.asarray(ref[k]).dtype)
        np.testing.assert_array_equal(got, np.asarray(ref[k]).reshape(-1), err_msg=k)
    p.validate()


shapes = st.tuples(st.integers(1, 40), st.integers(1, 12), st.integers(0, 2), st.integers(0, 10 ** 6))


@settings(max_examples=25, deadline=None)
@given(shapes)
def test_fuzz_block_quant(sh):
    M, kb, kind, seed = sh
    w = _weights(seed, M, 128 * kb, kind)
    _check(mbd.mbd_pack(mbd.MBD_TERNARY_B128, w), ternary.pack(w), ["codes", "scales"])
    _check(mbd.mbd_pack(mbd.MBD_INT4_G128, w), int4.pack(w), ["codes", "scales"])
    _check(mbd.mbd_pack(mbd.MBD_TERNARY_SKIP, w), ternary_skip.pack(w), ["codes", "scales", "slabs", "tile_base"])
    _check(mbd.mbd_pack(mbd.MBD_MX32, w), mx.encode(w), ["mx_exp", "mx_sign", "mx_mag"])


keeps = st.sampled_from([(3, 10), (1, 2), (1, 10), (0, 1), (1, 1), (7, 8)])


@settings(max_examples=20, deadline=None)
@given(shapes, keeps)
def test_fuzz_cassandra(sh, keep):
    M, kb, kind, seed = sh
    K = 128 * kb
    w = _weights(seed, M, K, kind)
    norms = np.random.default_rng(seed + 1).lognormal(0, 1, K).astype(np.float32)
    if kind == 2:
        norms[:] = 1.0                               # exact score ties
    _check(mbd.mbd_pack(mbd.MBD_CASSANDRA, w, norms, *keep), cassandra.pack(w, norms, *keep),
           ["bitmap", "spec_nib", "unary", "codebook", "bitoff", "kprefix", "lo_nib", "pruned"])
    _check(mbd.mbd_pack(mbd.MBD_CASSANDRA_MX, w, norms, *keep), cassandra_mx.pack_spec(w, norms, *keep),
           ["bitmap", "mx_nib", "mx_sign", "mx_exp", "kprefix"])
