"""Mutation check of the oracle's pins: each plausible mistake below is
planted in a temporary copy of the oracle (never in the repository's copy),
and the oracle's pin tests are run against that copy in a subprocess.  Every
mutation must make at least one pin fail; a mutation that survives means the
pins cannot tell that mistake from the method."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["test_oracle.py", "test_append_oracle.py", "test_fp8_oracle.py"]

# (name, exact text in oracle/mla_oracle.py, replacement)
MUTATIONS = [
    ("dropped_q_pe_term", "scores = sm * (qn @ ckv.T + qp @ kpe.T)", "scores = sm * (qn @ ckv.T)"),
    ("causal_off_by_one", "max(0, i + kv_len - q_len + 1)", "max(0, i + kv_len - q_len)"),
    ("page_slot_swap", "[int(kv_indptr[row]) + j // page_size]",
     "[int(kv_indptr[row]) + j % page_size]"),
    ("lse_without_max", "lse[hs] = (m + np.log(z))[..., 0]", "lse[hs] = (np.log(z))[..., 0]"),
    ("scale_of_full_latent", "    sm = float(np.float32(sm_scale))\n    lens",
     "    sm = 576.0 ** -0.5\n    lens"),
    ("row_length_ignores_last_page", "np.where(n > 0, (n - 1) * page_size + last, 0)",
     "np.where(n > 0, n * page_size, 0)"),
    ("merge_weights_swapped", "v = (wa[..., None] * va + wb[..., None] * vb)",
     "v = (wb[..., None] * va + wa[..., None] * vb)"),
    ("append_off_by_one", "            j = L - Q + i\n", "            j = L - Q + i - 1\n"),
    ("projection_head_order", 'np.einsum("thk,hkn->thn", xf, wf)',
     'np.einsum("thk,hkn->thn", xf, wf[::-1])'),
    ("fp8_exponent_bias", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("fp8_subnormal_step", "m / 8.0 * 2.0 ** -6", "m / 8.0 * 2.0 ** -7"),
    ("fp8_ties_away_from_zero", "((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))",
     "((d_hi == d_lo) & (hi != lo))"),
    ("fp8_scale_dropped", "return fp8_e4m3_decode(kv_cache_fp8) * float(np.float32(kv_scale))",
     "return fp8_e4m3_decode(kv_cache_fp8)"),
    ("fp8_quantize_multiplies", "astype(np.float32) / np.float32(kv_scale)",
     "astype(np.float32) * np.float32(kv_scale)"),
]


def _copy_tree(dst):
    """Everything the pin tests import, in a scratch directory."""
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), os.path.join(dst, "tests"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "workloads.py"), dst)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(tmp_path, name, old, new):
    dst = str(tmp_path)
    _copy_tree(dst)
    path = os.path.join(dst, "oracle", "mla_oracle.py")
    src = open(path).read()
    assert src.count(old) == 1, f"{name}: the text to mutate is not unique in the oracle"
    with open(path, "w") as fh:
        fh.write(src.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *[os.path.join("tests", t) for t in PIN_TESTS]],
                       cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"{name}: no pin failed (rc={r.returncode})\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, r.stdout[-2000:]


def test_unmutated_copy_passes(tmp_path):
    """The scratch copy itself passes every pin (so a failure above is the
    mutation's doing)."""
    dst = str(tmp_path)
    _copy_tree(dst)
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        *[os.path.join("tests", t) for t in PIN_TESTS]],
                       cwd=dst, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
