"""mla_run_noalloc (the entry point that allocates nothing, page table in
device memory) through the C ABI, against mla_plan + mla_run on the same
inputs and against the fp64 oracle: two calls in a row on the same GPU
workspace, the second with a smaller batch; the limits and the device-side
rejection of a bad page table."""

import numpy as np
import pytest

import workloads as W
from gpu_util import assert_close, from_dev_bf16, oracle_of, run_library, to_dev_bf16

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_attention_amd as pm
    pm.library()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _noalloc(w, max_kv_len=None):
    import paged_mla_attention_amd as pm
    mk = int(w.kv_lens().max()) if max_kv_len is None else max_kv_len
    o, lse = pm.run_noalloc(_i32(w.qo_indptr), _i32(w.kv_indptr), _i32(w.kv_indices),
                            _i32(w.kv_last_page_len), to_dev_bf16(w.q_nope), to_dev_bf16(w.q_pe),
                            to_dev_bf16(w.kv_cache), w.page_size, mk, causal=w.causal,
                            sm_scale=w.sm_scale, return_lse=True)
    torch.cuda.synchronize()
    return from_dev_bf16(o), lse.cpu().numpy()


def _check_pair(w):
    o_na, l_na = _noalloc(w)
    o_pl, l_pl = run_library(w)
    # against the existing entry point's result, at the oracle tolerances
    assert_close(o_na, l_na, W_widen(o_pl), l_pl.astype(np.float64), f"{w.name} vs mla_run")
    o_ref, l_ref = oracle_of(w)
    assert_close(o_na, l_na, o_ref, l_ref, f"{w.name} vs oracle")


def W_widen(bits):
    import oracle
    return oracle.widen(bits)


@pytest.mark.parametrize("heads,page_size", [(128, 64), (16, 1), (64, 33)])
def test_noalloc_matches_plan_and_run_twice(heads, page_size):
    """A larger batch, then a smaller one, on the shared workspace."""
    rng = np.random.default_rng(500 + heads + page_size)
    big = W.make_workload("na_big", 0, [700, 33, 1500, 64, 2200, 0, 90],
                          [1, 1, 1, 1, 1, 2, 17], heads, page_size, rng=rng)
    small = W.make_workload("na_small", 0, [50, 300], [1, 4], heads, page_size, rng=rng)
    _check_pair(big)
    _check_pair(small)


def test_noalloc_decode_batch_full():
    """The decode batch of 64 rows, 128 heads (every token split over
    workers), twice in a row."""
    w = W.decode_batch()
    for _ in range(2):
        _check_pair(w)


def test_noalloc_limits_and_bad_table():
    import paged_mla_attention_amd as pm
    from paged_mla_attention_amd import _native
    rng = np.random.default_rng(9)
    w = W.make_workload("na_lim", 0, [100, 40], [1, 1], 128, 16, rng=rng)
    # rows declared longer than the workspace can split at 128 heads
    with pytest.raises(_native.MLAError, match="workspace"):
        _noalloc(w, max_kv_len=1 << 24)
    # a row longer than the declared max_kv_len, and a page id out of range:
    # rejected on the device, every token gets zero output and -inf LSE
    for bad in ("len", "page"):
        idx = w.kv_indices.copy()
        mk = int(w.kv_lens().max())
        if bad == "len":
            mk = 50
        else:
            idx[-1] = w.num_pages + 3
        wb = W.Workload(**{**w.__dict__, "kv_indices": idx})
        o, lse = _noalloc(wb, max_kv_len=mk)
        assert np.all(o == 0) and np.all(np.isneginf(lse)), bad
    # and a good call after them on the same workspace
    o, lse = _noalloc(w)
    o_ref, l_ref = oracle_of(w)
    assert_close(o, lse, o_ref, l_ref, "after rejected tables")
