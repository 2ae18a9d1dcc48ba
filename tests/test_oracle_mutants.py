"""The oracle's pins catch plausible mistakes: each case plants one mistake
(a flipped sign, a dropped term, a wrong index or scale, a transposed
operand) in a copy of oracle/model.py, on the CPU, and runs the pin suite
(test_oracle_pins.py) against the copy in a child process, which must fail.
Nothing outside the temporary copy is modified."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (text in oracle/model.py, the mistake that replaces it)
MUTANTS = [
    ("y[..., 1::2] = x0 * s + x1 * c", "y[..., 1::2] = -x0 * s + x1 * c"),                 # rotary sign
    ("theta = base ** (-2.0 * i / Q)", "theta = base ** (-1.0 * i / Q)"),                   # rotary frequencies
    ("return r[..., None] * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))",
     "return r[..., None] * dy"),                                                             # RMSNorm bwd term
    ("S = (qh @ kh.T) / math.sqrt(Q)", "S = (qh @ kh.T)"),                                   # attention scale
    ("np.triu(np.ones((T, T), dtype=bool), 1)", "np.triu(np.ones((T, T), dtype=bool), 2)"),  # causal mask
    ("dk[:, h, :] = (dS.T @ q[:, h, :]) * sc", "dk[:, h, :] = (dS @ q[:, h, :]) * sc"),      # transposed operand
    ('x1 = x + o @ lp["Wo"].T', 'x1 = o @ lp["Wo"].T'),                                      # dropped residual
    ('grads["W1"] += dh.T @ c["m"]', 'grads["W1"] += du.T @ c["m"]'),                        # wrong gradient
    ("return 2.0 * np.maximum(h, 0.0)", "return np.maximum(h, 0.0)"),                        # relu^2 derivative
    ('g = g + rmsnorm_bwd(c["m"], c["r2"], dm)', 'g = rmsnorm_bwd(c["m"], c["r2"], dm)'),    # dropped residual grad
    ("dz[rows, tgt[rows]] -= 1.0", "dz[rows, tgt[rows]] -= 0.5"),                            # CE gradient
    ("(s / (LN2 * nbytes) if nbytes else 0.0)", "(s / nbytes if nbytes else 0.0)"),          # bpb without ln 2
    ("xf, rf = rmsnorm(x, cfg.rms_eps)", "xf, rf = x, np.ones(x.shape[0])"),                 # dropped final norm
    ("dq = rope(dqr, phi, inverse=True)", "dq = rope(dqr, phi)"),                            # wrong inverse rotation
]


def _run_pins_on_copy(tmp_path, old, new):
    src = open(os.path.join(ROOT, "oracle", "model.py")).read()
    assert src.count(old) == 1, "the mutation no longer applies to the oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synthdata"), tmp_path / "synthdata",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    (tmp_path / "oracle" / "model.py").write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        str(tmp_path / "tests" / "test_oracle_pins.py")],
                       cwd=tmp_path, capture_output=True, text=True, timeout=600)
    return r


def test_unmodified_copy_passes(tmp_path):
    """Control: the copy with no mistake passes, so a failing mutant fails
    because of its mistake."""
    r = _run_pins_on_copy(tmp_path, MUTANTS[0][0], MUTANTS[0][0])
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("old,new", MUTANTS, ids=[f"m{i}" for i in range(len(MUTANTS))])
def test_planted_mistake_fails_a_pin(tmp_path, old, new):
    r = _run_pins_on_copy(tmp_path, old, new)
    assert r.returncode == 1, f"mutant survived the pins:\n{r.stdout[-2000:]}"
