"""GPU parity of tq_encode_prod / tq_encode_mse against the oracle."""
import numpy as np
import pytest

from tests.gpu_util import Setup, compare_encode, torch, value_indices
from tq_inputs import kv_tensor, tiny_vectors

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def test_tiny_config_prod_b3_fp32():
    # N=4096, d=128, fp32 N(0,1) with 4 outlier channels x20, seed 0; prod at b=3
    _log("encode tiny prod b3 fp32")
    x = tiny_vectors(4096, 128, seed=0)
    st = Setup(bits=3, prod=True, seed=0)
    planes, scal = st.encode_gpu(x)
    stats = compare_encode(st, planes, scal, st.encode_oracle(x))
    _log(f"  {stats}")


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_prod_bits_dtypes_ragged(bits, dtype):
    _log(f"encode prod b{bits} {dtype} ragged")
    x = kv_tensor(1, 1, 1000, 128, seed=1)[0, 0]
    x = x if dtype == "f16" else x.astype(np.float32)
    st = Setup(bits=bits, prod=True, seed=1)
    planes, scal = st.encode_gpu(x)
    compare_encode(st, planes, scal, st.encode_oracle(x))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_mse_bits_dtypes_ragged(bits, dtype):
    _log(f"encode mse b{bits} {dtype} ragged")
    x = kv_tensor(1, 1, 777, 128, seed=2, value=True)[0, 0]
    x = x if dtype == "f16" else x.astype(np.float32)
    st = Setup(bits=bits, prod=False, seed=2, purpose_pi=4)
    planes, scal = st.encode_gpu(x)
    compare_encode(st, value_indices(planes, len(x)), scal, st.encode_oracle(x))


def test_zero_vectors_and_slots():
    _log("encode zero vectors + slots")
    rg = np.random.default_rng(3)
    x = rg.standard_normal((70, 128)).astype(np.float32)
    x[[0, 5, 69]] = 0.0
    slot = rg.permutation(100)[:70]
    st = Setup(bits=3, prod=True, seed=3)
    planes, scal = st.encode_gpu(x, slot=slot, records=100)
    ocode = st.encode_oracle(x)
    compare_encode(st, planes[slot], scal[slot], ocode)
    untouched = np.setdiff1d(np.arange(100), slot)
    assert not planes[untouched].any() and not scal[untouched].view(np.uint16).any()
    assert np.all(scal[slot[[0, 5, 69]], 0] == 0)


def test_strided_rows():
    _log("encode strided rows")
    T = torch()
    x = kv_tensor(1, 1, 300, 128, seed=4)[0, 0]
    big = np.zeros((300, 192), np.float16)
    big[:, :128] = x
    st = Setup(bits=3, prod=True, seed=4)
    xt = T.from_numpy(big).cuda()[:, :128]
    import kv_cache_vector_02_amd as tq
    cache = tq.alloc_cache(st.layout(), 300)
    tq.encode_prod(st.params, xt, cache)
    T.cuda.synchronize()
    planes = cache.planes.cpu().numpy().view(np.uint32)
    compare_encode(st, planes, cache.scalars.cpu().numpy(), st.encode_oracle(x))


def test_qwen_shaped_full_size_sampled():
    # 36 layers x 2 KV heads x 8192 tokens x 128, fp16, prod b=3 keys and mse b=3
    # values at full size in one launch each; the oracle checks a seeded sample
    _log("encode qwen-shaped full size (sampled)")
    T = torch()
    k = kv_tensor(36, 2, 8192, 128, seed=1).reshape(-1, 128)
    v = kv_tensor(36, 2, 8192, 128, seed=1, value=True).reshape(-1, 128)
    rg = np.random.default_rng(0)
    sample = np.sort(rg.choice(k.shape[0], 3000, replace=False))
    sample[-1] = k.shape[0] - 1
    for x, prod in ((k, True), (v, False)):
        st = Setup(bits=3, prod=prod, seed=1, purpose_pi=2 if prod else 4)
        planes, scal = st.encode_gpu(x)
        if not prod:
            planes = value_indices(planes, len(x))
        compare_encode(st, planes[sample], scal[sample], st.encode_oracle(x[sample]))
        del planes, scal
        T.cuda.empty_cache()


@pytest.mark.parametrize("mode", ["aligned_slots", "scattered_slots", "ragged"])
def test_value_block_paths(mode):
    # whole-block stores for aligned groups of 32, per-bit atomics otherwise;
    # the cache is pre-filled so stale bits of re-encoded records must clear
    _log(f"encode values, {mode}")
    rg = np.random.default_rng(8)
    records = 256
    st = Setup(bits=3, prod=False, seed=8, purpose_pi=4)
    old = kv_tensor(1, 1, records, 128, seed=9, value=True)[0, 0]
    cache = st.alloc(records)
    st.encode_gpu(old, cache=cache)
    x = kv_tensor(1, 1, 100 if mode == "ragged" else 96, 128, seed=10, value=True)[0, 0]
    if mode == "aligned_slots":
        slot = np.concatenate([np.arange(64, 128), np.arange(192, 224)])
    elif mode == "scattered_slots":
        slot = rg.permutation(records)[: len(x)]
    else:
        slot = None
    planes, scal = st.encode_gpu(x, slot=slot, cache=cache)
    idx = value_indices(planes, records)
    where = np.arange(len(x)) if slot is None else slot
    compare_encode(st, idx[where], scal[where], st.encode_oracle(x))
    rest = np.setdiff1d(np.arange(records), where)
    compare_encode(st, idx[rest], scal[rest], st.encode_oracle(old[rest]))


def test_value_blocks_shared_across_workgroups():
    # 4096 values whose slots interleave: vector i goes to token i // 128 of
    # block i % 128, so every 32-token block is written bit by bit by 32
    # vectors from 32 different wave tiles spread over many workgroups; the
    # cache is pre-filled, so every bit is either set or cleared concurrently
    _log("encode values, blocks shared by many workgroups")
    st = Setup(bits=3, prod=False, seed=11, purpose_pi=4)
    records = 4096
    old = kv_tensor(1, 1, records, 128, seed=12, value=True)[0, 0]
    cache = st.alloc(records)
    st.encode_gpu(old, cache=cache)
    x = kv_tensor(1, 1, records, 128, seed=13, value=True)[0, 0]
    i = np.arange(records)
    slot = (i % 128) * 32 + i // 128
    planes, scal = st.encode_gpu(x, slot=slot, cache=cache)
    idx = value_indices(planes, records)
    compare_encode(st, idx[slot], scal[slot], st.encode_oracle(x))


@pytest.mark.parametrize("n", [512, 4100])
def test_value_append_one_record_per_block(n):
    # a decode step's append: each vector goes to its own 32-token block of a
    # pre-filled cache (block b gets token b % 32).  Up to 4096 vectors a call
    # finds every block single-written and rewrites whole words; above that it
    # sets the bits with atomics.  Every other record must keep its old bits.
    _log(f"encode values, one record per block, n = {n}")
    st = Setup(bits=3, prod=False, seed=21, purpose_pi=4)
    records = 32 * n
    old = kv_tensor(1, 1, records, 128, seed=22, value=True)[0, 0]
    cache = st.alloc(records)
    st.encode_gpu(old, cache=cache)
    x = kv_tensor(1, 1, n, 128, seed=23, value=True)[0, 0]
    b = np.arange(n)
    slot = b * 32 + b % 32
    planes, scal = st.encode_gpu(x, slot=slot, cache=cache)
    idx = value_indices(planes, records)
    compare_encode(st, idx[slot], scal[slot], st.encode_oracle(x))
    rest = np.setdiff1d(np.arange(records), slot)[::7]
    compare_encode(st, idx[rest], scal[rest], st.encode_oracle(old[rest]))


@pytest.mark.parametrize("prod,bits", [(True, 2), (True, 3), (True, 4), (False, 1), (False, 2), (False, 3),
                                       (False, 4)])
@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_hadamard_rotation(prod, bits, dtype):
    # sign-flipped Hadamard rotation at d = d_rot = 128, ragged count
    _log(f"encode hadamard {'prod' if prod else 'mse'} b{bits} {dtype}")
    x = kv_tensor(1, 1, 900, 128, seed=6, value=not prod)[0, 0]
    x = x if dtype == "f16" else x.astype(np.float32)
    st = Setup(bits=bits, prod=prod, seed=6, rot="hadamard", purpose_eps=5 if prod else 6)
    planes, scal = st.encode_gpu(x)
    if not prod:
        planes = value_indices(planes, len(x))
    _log(f"  {compare_encode(st, planes, scal, st.encode_oracle(x))}")


@pytest.mark.parametrize("kind", ["prod", "mse", "prod_2048"])
def test_slots_outside_the_capacity_are_not_written(kind):
    # the cache descriptor says 64 records; slots 64.., and negative slots,
    # name no record and must leave every byte past the capacity untouched,
    # while the records inside it are encoded as usual
    import kv_cache_vector_02_amd as tq
    _log(f"encode slots outside the capacity ({kind})")
    T = torch()
    rg = np.random.default_rng(31)
    if kind == "prod_2048":
        from tq_inputs import mixture_database
        x, _ = mixture_database(48, 1536, seed=31)
        st = Setup(d=1536, d_rot=2048, bits=2, prod=True, rot="hadamard", seed=31)
    else:
        x = kv_tensor(1, 1, 48, 128, seed=31)[0, 0]
        st = Setup(bits=3, prod=kind == "prod", seed=31, purpose_pi=2 if kind == "prod" else 4)
    slot = rg.permutation(64)[:48].astype(np.int64)
    out_of_range = [3, 17, 40]
    slot[out_of_range] = [64, 100, -1]
    full = st.alloc(128)                                   # room past the stated capacity
    cache = tq.Cache(full.planes, full.scalars[:64], 0)    # capacity: 64 records
    assert cache.records == 64
    xd = T.from_numpy(np.ascontiguousarray(x)).cuda()
    sl = T.from_numpy(slot).cuda()
    if kind == "prod_2048":
        tq.encode_prod(st.params, xd, cache, slot=sl, ws=tq.alloc_workspace(tq.encode_workspace(st.params, 48)))
    else:
        (tq.encode_prod if st.prod else tq.encode_mse)(st.params, xd, cache, slot=sl)
    T.cuda.synchronize()
    planes = full.planes.cpu().numpy().view(np.uint32)
    scal = full.scalars.cpu().numpy()
    keep = np.setdiff1d(np.arange(48), out_of_range)
    assert not scal[64:].view(np.uint16).any(), "scalars past the capacity were written"
    if st.prod:
        assert not planes[64:].any(), "records past the capacity were written"
        compare_encode(st, planes[slot[keep]], scal[slot[keep]], st.encode_oracle(x[keep]))
    else:
        assert not planes[2:].any(), "value blocks past the capacity were written"
        idx = value_indices(planes[:2], 64)
        compare_encode(st, idx[slot[keep]], scal[slot[keep]], st.encode_oracle(x[keep]))
