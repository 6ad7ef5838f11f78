"""GPU parity of the retrieval configuration: 1536-dimensional unit-norm
embeddings from a 64-component Gaussian mixture, zero-padded to 2048 and
rotated by the sign-flipped Hadamard transform, TurboQuant-prod at b = 2 and
b = 4 (1 and 3 MSE bits + QJL), against the oracle."""
import numpy as np
import pytest

from tests.gpu_util import Setup, compare_encode
from tq_inputs import mixture_database

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _setup(bits, seed=4):
    return Setup(d=1536, d_rot=2048, bits=bits, prod=True, rot="hadamard", seed=seed)


@pytest.mark.parametrize("bits", [2, 4])
def test_encode_2048_prod(bits):
    _log(f"retrieval encode b{bits}: 3000 x 1536 -> 2048")
    db, _ = mixture_database(3000, 1536, seed=4)
    st = _setup(bits)
    planes, scal = st.encode_gpu(db)
    _log(f"  {compare_encode(st, planes, scal, st.encode_oracle(db))}")


def test_encode_2048_chunks_and_slots():
    # more vectors than one residual chunk (32768), records scattered by slot
    _log("retrieval encode across the chunk boundary, scattered slots")
    n = 40000
    db, _ = mixture_database(n, 1536, seed=5)
    st = _setup(2, seed=5)
    slot = np.random.default_rng(5).permutation(n + 100)[:n]
    planes, scal = st.encode_gpu(db, slot=slot, records=n + 100)
    rows = np.r_[0:200, 32668:32868, n - 200:n]
    _log(f"  {compare_encode(st, planes[slot[rows]], scal[slot[rows]], st.encode_oracle(db[rows]))}")
