"""C++ packer (libmbd, CPU) against the oracle on the full matrices of the benched
workloads: every section bit-exact, so that the matrix-global parts (the Cassandra
codebook ranking over all kept values, the u64 unary bit offsets of the tile table,
the kept prefixes past 2^24) are checked at the size the kernels are timed on, not
only on row subsets.  CPU only; about 1.5 minutes and 15 GB for 8192 x 28672."""
import gc

import numpy as np
import pytest

import synth
from oracle import cassandra, int4

mbd = pytest.importorskip("memory_bound_decode_amd")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    try:
        mbd.lib()
    except ImportError as e:                         # pragma: no cover
        pytest.skip(str(e))


def _check(p, ref, names):
    secs = p.sections()
    for k in names:
        want = np.asarray(ref[k]).reshape(-1)
        raw, nbytes = secs[k]
        assert nbytes == want.nbytes, k
        np.testing.assert_array_equal(raw[:nbytes].view(want.dtype), want, err_msg=k)
        assert not raw[nbytes:].any(), k + " padding"


def test_int4_full_8192x8192():
    w = synth.gen_weights(synth.WORKLOADS["int4_8k"])
    _check(mbd.mbd_pack(mbd.MBD_INT4_G128, w), int4.pack(w), ["codes", "scales"])


@pytest.mark.parametrize("name", ["cassandra_spec", "cassandra_verify"])
def test_cassandra_full(name):
    wl = synth.WORKLOADS[name]
    w = synth.gen_weights(wl)
    norms = synth.gen_act_norms(wl)
    p = mbd.mbd_pack(mbd.MBD_CASSANDRA, w, norms)
    ref = cassandra.pack(w, norms)
    del w
    gc.collect()
    _check(p, ref, ["bitmap", "spec_nib", "unary", "codebook", "bitoff", "kprefix", "lo_nib", "pruned"])
    st = p.stats()
    assert (st.n_kept, st.n_sym, st.unary_bits) == (ref["n_kept"], ref["n_sym"], ref["unary_bits"])
    assert st.n_kept == wl.M * cassandra.keep_count(wl.K)
