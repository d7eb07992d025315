"""Seeded random ragged batches through the C ABI against the fp64 oracle:
each case draws the number of rows, their key and query counts (decode rows,
prefill rows, rows without keys, rows with more causal queries than keys),
the head count, the page size and causal or not, and runs it on a bf16 or
an fp8 cache, so that every kernel variant (one, two and four computing
waves, the two-wave kernels with a producer wave, 32 or 16 head slots,
tiles inside pages or not, host-slot and device schedules) meets shapes no
hand-written case chose.  A second set draws odd shapes: head counts around
the kernels' 16/32/64 boundaries, page sizes around the 32-key tile and
rows of up to 20,000 keys (large cases compare sampled tokens)."""

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_close, from_dev_bf16, oracle_of, run_library, to_dev_bf16

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

HEADS = [1, 5, 16, 32, 48, 64, 96, 128]
PAGES = [1, 3, 16, 32, 64, 128]
# (odd shapes: head counts around the 16/32/64 kernel boundaries, page sizes
# around the tile size, rows up to 20,000 keys and 200 queries)
ODD_HEADS = [1, 2, 3, 7, 15, 16, 17, 31, 33, 47, 63, 65, 97, 127, 128]
ODD_PAGES = [1, 2, 7, 31, 32, 33, 63, 64, 65, 96, 128, 256]


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


def _draw_odd(seed):
    rng = np.random.default_rng(90000 + seed)
    heads = int(rng.choice(ODD_HEADS))
    page = int(rng.choice(ODD_PAGES))
    causal = bool(rng.random() < 0.7)
    rows = int(rng.integers(1, 12))
    kv, qo = [], []
    for _ in range(rows):
        r = rng.random()
        if r < 0.4:
            kv.append(int(rng.integers(1, 20000)))
            qo.append(1)
        elif r < 0.8:
            L = int(rng.integers(1, 3000))
            kv.append(L)
            qo.append(int(rng.integers(1, min(L, 200) + 1)))
        elif r < 0.9:
            kv.append(0)
            qo.append(int(rng.integers(1, 3)))
        else:
            L = int(rng.integers(1, 40))
            kv.append(L)
            qo.append(L + int(rng.integers(1, 9)))
    fp8 = bool(rng.random() < 0.3)
    w = W.make_workload(f"odd{seed}", 0, kv, qo, heads, page, causal=causal, rng=rng)
    # (large cases: the first, a few random and the last query tokens)
    T = w.num_tokens
    tok = None
    if T * sum(kv) >= 3e6:
        tok = np.unique(np.concatenate([np.arange(min(T, 8)), rng.integers(0, T, 24), [T - 1]]))
        tok = tok.astype(np.int64)
    return w, fp8, tok


def _check(w, fp8, tok, what, scale=0.13):
    import paged_mla_attention_amd as pm
    if not fp8:
        o, lse = run_library(w)
        o_ref, l_ref = oracle_of(w, tokens=tok)
    else:
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
                                            w.causal, w.sm_scale, scale, tokens=tok)
    if tok is not None:
        o, lse = o[tok], lse[tok]
    print(what, flush=True)
    assert_close(o, lse, o_ref, l_ref, what)


@pytest.mark.parametrize("seed", range(16))
def test_random_batch_odd_shapes(seed):
    w, fp8, tok = _draw_odd(seed)
    what = f"odd seed {seed}: H={w.num_heads} P={w.page_size} causal={w.causal} fp8={fp8} " \
           f"kv={w.kv_lens().tolist()} qo={np.diff(w.qo_indptr).tolist()}"
    _check(w, fp8, tok, what)


@pytest.mark.parametrize("seed", range(24))
def test_random_batch(seed):
    w, fp8 = _draw(seed)
    what = f"seed {seed}: H={w.num_heads} P={w.page_size} causal={w.causal} fp8={fp8} " \
           f"kv={w.kv_lens().tolist()} qo={np.diff(w.qo_indptr).tolist()}"
    _check(w, fp8, None, what)
