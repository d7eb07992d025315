"""Seeded random ragged batches through the C ABI against the fp64 oracle:
each case draws the number of rows, their key and query counts (decode rows,
prefill rows, rows without keys, rows with more causal queries than keys),
the head count, the page size and causal or not, and runs it on a bf16 or
an fp8 cache, so that every kernel variant (one, two and four computing
waves, the two-wave fp8 kernel, tiles inside pages or not, host-slot and
device schedules) meets shapes no hand-written case chose."""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_close, from_dev_bf16, oracle_of, run_library, to_dev_bf16

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

HEADS = [1, 5, 16, 32, 48, 64, 96, 128]
PAGES = [1, 3, 16, 32, 64, 128]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_mla_attention_amd as pm
    pm.library()


def _draw(seed):
    rng = np.random.default_rng(7000 + seed)
    heads = int(rng.choice(HEADS))
    page = int(rng.choice(PAGES))
    causal = bool(rng.random() < 0.8)
    rows = int(rng.integers(1, 9))
    kv, qo = [], []
    for _ in range(rows):
        kind = rng.random()
        if kind < 0.45:  # decode
            kv.append(int(rng.integers(1, 3000)))
            qo.append(1)
        elif kind < 0.85:  # prefill
            L = int(rng.integers(1, 1500))
            kv.append(L)
            qo.append(int(rng.integers(1, min(L, 64) + 1)))
        elif kind < 0.93:  # no keys
            kv.append(0)
            qo.append(int(rng.integers(1, 4)))
        else:  # more queries than keys
            L = int(rng.integers(1, 20))
            kv.append(L)
            qo.append(L + int(rng.integers(1, 6)))
    fp8 = bool(rng.random() < 0.35)
    w = W.make_workload(f"rand{seed}", 0, kv, qo, heads, page, causal=causal, rng=rng)
    return w, fp8


@pytest.mark.parametrize("seed", range(24))
def test_random_batch(seed):
    import paged_mla_attention_amd as pm
    w, fp8 = _draw(seed)
    what = f"seed {seed}: H={w.num_heads} P={w.page_size} causal={w.causal} fp8={fp8} " \
           f"kv={w.kv_lens().tolist()} qo={np.diff(w.qo_indptr).tolist()}"
    if not fp8:
        o, lse = run_library(w)
        o_ref, l_ref = oracle_of(w)
    else:
        scale = 0.13
        codes = W.fp8_cache_codes(w.kv_cache, scale)
        plan = pm.MLAPlan(w.num_heads, w.page_size)
        try:
            plan.plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.kv_last_page_len,
                      causal=w.causal, sm_scale=w.sm_scale, num_cache_pages=w.num_pages,
                      kv_dtype="fp8_e4m3")
            kv = torch.from_numpy(np.ascontiguousarray(codes)).cuda()
            out, lse_t = plan.run(to_dev_bf16(w.q_nope), to_dev_bf16(w.q_pe), kv,
                                  return_lse=True, kv_scale=scale)
            torch.cuda.synchronize()
        finally:
            plan.close()
        o, lse = from_dev_bf16(out), lse_t.cpu().numpy()
        o_ref, l_ref = oracle.attention_fp8(w.q_nope, w.q_pe, codes, w.qo_indptr, w.kv_indptr,
                                            w.kv_indices, w.kv_last_page_len, w.page_size,
                                            w.causal, w.sm_scale, scale)
    print(what, flush=True)
    assert_close(o, lse, o_ref, l_ref, what)
