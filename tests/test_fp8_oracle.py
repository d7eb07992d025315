"""Pins for the oracle's fp8 (OCP E4M3) latent cache: the code table against
PyTorch's float8_e4m3fn type (a library routine) and the format's closed
forms, the rounding against PyTorch on exact ties and near-ties, saturation,
and attention over an fp8 cache against the bf16 oracle on the same values."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = oracle.fp8_e4m3_decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.isnan(ours).sum() == 2  # 0x7F and 0xFF
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_closed_forms():
    d = oracle.fp8_e4m3_decode
    cases = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9,
             0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x40: 2.0, 0x3C: 1.5, 0x30: 0.5}
    for c, v in cases.items():
        assert d(np.uint8(c)) == v, hex(c)
    assert np.signbit(d(np.uint8(0x80))) and d(np.uint8(0x80)) == 0.0


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(oracle.fp8_e4m3_encode(oracle.fp8_e4m3_decode(codes)), codes)
    assert oracle.fp8_e4m3_encode(np.array([-0.0, -1e-9]))[1] == 0x80  # signed zero


def test_encode_ties_and_near_ties_match_torch():
    """Exact midpoints between neighbouring codes (ties to the even
    mantissa) and values one fp32 step either side, all within range."""
    grid = oracle.fp8_e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    near = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    vals = np.concatenate([near, -near, grid, [464.0]]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle.fp8_e4m3_encode(vals.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_encode_random_matches_torch():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 150)])
    vals = np.clip(vals, -448, 448).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.fp8_e4m3_encode(vals.astype(np.float64)), ref)


def test_encode_saturates():
    e = oracle.fp8_e4m3_encode
    assert list(e(np.array([448.0, 449.0, 464.0, 465.0, 1e6]))) == [0x7E] * 5
    assert list(e(np.array([-449.0, -1e30]))) == [0xFE] * 2


def test_quantize_rows_is_fp32_quotient_rounded():
    rng = np.random.default_rng(5)
    x = W.bf16_normals(rng, (4000,))
    xf = oracle.widen(x).astype(np.float32)
    for s in (1.0, 0.0625, 3.0, 0.37):
        q = (torch.from_numpy(xf) / torch.tensor(np.float32(s))).clamp(-448, 448)
        ref = q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(oracle.fp8_quantize_rows(x, s), ref), s


def _fp8_workload(seed, kv, qo, H, P, scale):
    rng = np.random.default_rng(seed)
    w = W.make_workload("fp8", 0, kv, qo, H, P, rng=rng)
    codes = oracle.fp8_quantize_rows(w.kv_cache, scale)
    return w, codes


@pytest.mark.parametrize("scale", [1.0, 0.25, 4.0])
def test_attention_fp8_equals_bf16_oracle_on_the_same_values(scale):
    """With a power-of-two scale every dequantised value is a bf16 value, so
    attention over the fp8 cache must equal, bit for bit, the bf16 oracle
    over a bf16 cache holding those values."""
    w, codes = _fp8_workload(11, [37, 100, 1], [1, 5, 1], 4, 16, scale)
    vals = oracle.fp8_e4m3_decode(codes) * scale
    bf = W.f32_to_bf16_bits(vals.astype(np.float32))
    assert np.array_equal(oracle.widen(bf), vals)  # exact in bf16
    o8, l8 = oracle.attention_fp8(w.q_nope, w.q_pe, codes, w.qo_indptr, w.kv_indptr,
                                  w.kv_indices, w.kv_last_page_len, 16, True, w.sm_scale, scale)
    ob, lb = oracle.attention(w.q_nope, w.q_pe, bf, w.qo_indptr, w.kv_indptr, w.kv_indices,
                              w.kv_last_page_len, 16, True, w.sm_scale)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def test_attention_fp8_close_to_unquantised():
    """Quantising a N(0,1) cache with scale 1/64 changes outputs only by the
    fp8 rounding (3 mantissa bits); a scale left out would change them 64-fold."""
    w, codes = _fp8_workload(12, [300, 64], [1, 7], 8, 16, 1 / 64)
    o8, l8 = oracle.attention_fp8(w.q_nope, w.q_pe, codes, w.qo_indptr, w.kv_indptr,
                                  w.kv_indices, w.kv_last_page_len, 16, True, w.sm_scale, 1 / 64)
    ob, lb = oracle.attention(w.q_nope, w.q_pe, w.kv_cache, w.qo_indptr, w.kv_indptr,
                              w.kv_indices, w.kv_last_page_len, 16, True, w.sm_scale)
    # (a row of 7 causal queries over 64 keys averages few keys: up to 0.1)
    assert np.abs(o8 - ob).max() < 0.2 and np.abs(l8 - lb).max() < 0.1
    assert np.abs(o8 - ob).mean() < 0.02


def test_append_fp8_stores_quantised_rows():
    rng = np.random.default_rng(13)
    w, codes = _fp8_workload(13, [40, 3, 70], [2, 3, 1], 2, 16, 0.5)
    T = w.num_tokens
    ckv, kpe = W.bf16_normals(rng, (T, 512)), W.bf16_normals(rng, (T, 64))
    out = oracle.append_kv_fp8(codes, ckv, kpe, w.qo_indptr, w.kv_indptr, w.kv_indices,
                               w.kv_last_page_len, 16, 0.5)
    lens = w.kv_lens()
    for b in range(w.batch):
        Q = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
        for i in range(Q):
            j = int(lens[b]) - Q + i
            pg = w.kv_indices[w.kv_indptr[b] + j // 16]
            row = out[pg, j % 16]
            t = int(w.qo_indptr[b]) + i
            want = np.concatenate([ckv[t], kpe[t]])
            # each code decodes to the value nearest x / 0.5 (within half a step)
            x = oracle.widen(want) / 0.5
            got = oracle.fp8_e4m3_decode(row)
            step = np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -6))) - 3)
            assert np.all(np.abs(got - x) <= step / 2 + 1e-12)
    untouched = np.ones(out.shape[:2], bool)
    for b in range(w.batch):
        Q = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
        for i in range(Q):
            j = int(lens[b]) - Q + i
            untouched[w.kv_indices[w.kv_indptr[b] + j // 16], j % 16] = False
    assert np.array_equal(out[untouched], codes[untouched])
