"""Plant plausible mistakes in copies of the oracle and show the pins catch each.

Each mutant edits one expression of the oracle's source (a dropped term, a
flipped sign, an off-by-one, a transposed operand or index), loads the edited
copy as a separate package and runs the pins of ``tests/pins.py`` -- closed
forms, invariants, the hand-worked example, finite differences and autograd,
but NOT the scalar brute-force cross-check, which would catch everything
trivially. A mutant that passes every pin would mean a hole in the pins.
"""
import importlib.util
import os
import shutil
import sys

import pytest

from tests import pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTANTS = [
    # (id, file, original snippet, planted mistake)
    ("silu_is_sigmoid", "attention.py", "return x / (1.0 + np.exp(-x))", "return 1.0 / (1.0 + np.exp(-x))"),
    ("silu_sign", "attention.py", "return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))"),
    ("mask_leaks_next", "attention.py", "(cols[None, :] <= rows[:, None])", "(cols[None, :] <= rows[:, None] + 1)"),
    ("mask_no_self_term", "attention.py", ") | \\\n        (cols[None, :] == rows[:, None])", ")"),
    ("norm_L_plus_1", "attention.py", "P = np.where(m, silu(S), 0.0) / L\n                A[s + rows",
     "P = np.where(m, silu(S), 0.0) / (L + 1)\n                A[s + rows"),
    ("norm_max_len", "attention.py", "P = np.where(m, silu(S), 0.0) / L\n                A[s + rows",
     "P = np.where(m, silu(S), 0.0) / max_len\n                A[s + rows"),
    ("qk_swapped", "attention.py", "S = q[s + rows, h, :] @ k[s:e, h, :].T\n                S += _bias",
     "S = k[s + rows, h, :] @ q[s:e, h, :].T\n                S += _bias"),
    ("time_bias_sign", "attention.py", "bias += rab_time[hr]", "bias -= rab_time[hr]"),
    ("rab_head_ignored", "attention.py", "return 0 if tab is None or tab.shape[0] == 1 else h", "return 0"),
    ("pos_sign", "buckets.py", "rel = cols[None, :] - p[:, None]", "rel = p[:, None] - cols[None, :]"),
    ("candidate_position", "buckets.py", "p = np.minimum(rows, hist)", "p = rows"),
    ("time_off_by_one", "buckets.py", "return np.minimum(bl - 1, n_buckets - 1)",
     "return np.minimum(bl, n_buckets - 1)"),
    ("time_no_plus_one", "buckets.py", "plus1 = absdiff + np.uint64(1)", "plus1 = absdiff"),
    ("dsilu_missing_factor", "attention.py", "dP * sig * (1.0 + S * (1.0 - sig))", "dP * sig"),
    ("dsilu_wrong_sign", "attention.py", "dP * sig * (1.0 + S * (1.0 - sig))", "dP * sig * (1.0 - S * (1.0 - sig))"),
    ("ds_no_norm", "attention.py", "(1.0 - sig)), 0.0) / L", "(1.0 - sig)), 0.0)"),
    ("dv_ungated", "attention.py", "dv[s:e, h, :] += P.T @ dAr", "dv[s:e, h, :] += P.T @ d_o[s + rows, h, :]"),
    ("dk_wrong_operand", "attention.py", "dk[s:e, h, :] += dS.T @ q[s + rows, h, :]",
     "dk[s:e, h, :] += dS.T @ k[s + rows, h, :]"),
    ("dq_wrong_operand", "attention.py", "dq[s + rows, h, :] = dS @ k[s:e, h, :]",
     "dq[s + rows, h, :] = dS @ q[s:e, h, :]"),
    ("d_rab_pos_transposed", "attention.py", "np.bincount(bp[m], weights=dS[m]",
     "np.bincount(bp.T[m], weights=dS[m]"),
    ("du_wrong", "attention.py", "du = d_o * A if", "du = d_o * u if"),
    ("da_ungated", "attention.py", "dA = d_o * u if", "dA = d_o if"),
]

NON_SCALAR_PINS = pins.BUCKET_PINS + pins.FWD_PINS + pins.BWD_PINS


def _load_mutant(tmp_path, name, fname, old, new):
    pkg = tmp_path / name
    shutil.copytree(ORACLE_DIR, pkg, ignore=shutil.ignore_patterns("__pycache__"))
    path = pkg / fname
    src = path.read_text()
    assert old in src, f"snippet for mutant {name} not found in oracle/{fname}"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(name, pkg / "__init__.py",
                                                  submodule_search_locations=[str(pkg)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("mid,fname,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mid, fname, old, new):
    name = f"oracle_mutant_{mid}"
    mod = _load_mutant(tmp_path, name, fname, old, new)
    failed = []
    try:
        for pin in NON_SCALAR_PINS:
            try:
                pin(mod)
            except (AssertionError, FloatingPointError, ValueError, IndexError):
                failed.append(pin.__name__)
    finally:
        for key in [k for k in sys.modules if k == name or k.startswith(name + ".")]:
            del sys.modules[key]
    assert failed, f"mutant {mid} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    mod = _load_mutant(tmp_path, "oracle_unmutated", "attention.py", "import numpy as np",
                       "import numpy as np")
    try:
        for pin in NON_SCALAR_PINS:
            pin(mod)
    finally:
        for key in [k for k in sys.modules if k.startswith("oracle_unmutated")]:
            del sys.modules[key]
