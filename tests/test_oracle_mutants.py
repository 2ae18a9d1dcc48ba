"""The oracle's pins catch plausible mistakes: each case plants one mistake
(a flipped sign, a dropped term, a wrong index or scale, a transposed
operand) in a copy of oracle/model.py or oracle/optim.py, on the CPU, and
runs that module's pin suite (test_oracle_pins.py, test_oracle_optim.py)
against the copy in a child process, which must fail.  Nothing outside the
temporary copy is modified."""
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
    ("row_scale = scale if token_weights is None else scale * np.asarray(token_weights[b], dtype=np.float64)",
     "row_scale = scale"),                                                                    # token weights ignored
    ("np.where(valid, w * ce, 0.0)", "np.where(valid, ce, 0.0)"),                            # weighted loss unweighted
    ("np.exp((z - z.max()) / temperature)", "np.exp((z - z.max()) * temperature)"),          # temperature inverted
    ("thr = np.sort(z)[::-1][top_k - 1]", "thr = np.sort(z)[::-1][top_k]"),                  # top-k off by one
    ("keep = z >= thr", "keep = z > thr"),                                                    # ties at the k-th dropped
]

# (text in oracle/optim.py, the mistake that replaces it)
MUTANTS_OPTIM = [
    ("NS_COEFFS = (3.4445, -4.7750, 2.0315)", "NS_COEFFS = (3.4445, 2.0315, -4.7750)"),    # coefficient order
    ("B = b * A + c * (A @ A)", "B = c * A + b * (A @ A)"),                                # powers swapped
    ("X = X / (np.linalg.norm(X) + eps)", "X = X / (np.abs(X).max() + eps)"),              # wrong normalisation
    ("buf = momentum * buf + G", "buf = momentum * buf + (1.0 - momentum) * G"),          # momentum form
    ("u = G + momentum * buf if nesterov else buf", "u = buf"),                            # Nesterov dropped
    ("max(1.0, W.shape[0] / W.shape[1])", "max(1.0, W.shape[1] / W.shape[0])"),            # aspect scale inverted
    ("v_hat = v / (1.0 - beta2 ** step)", "v_hat = v"),                                    # bias correction dropped
    ("p = p * (1.0 - lr * wd)", "p = p * (1.0 - wd)"),                                     # decay not scaled by lr
    ("np.sqrt(v_hat) + eps)", "np.sqrt(v_hat + eps))"),                                    # eps inside the root
    ("(1.0 - progress) / warmdown_ratio", "progress / warmdown_ratio"),                    # schedule direction
    ("(1.0 - frac) * start + frac * end", "frac * start + (1.0 - frac) * end"),            # momentum ramp reversed
    ("(d_model / 768.0) ** -0.5", "(d_model / 768.0) ** 0.5"),                             # width scale inverted
    ('hp["lr_embed"] if name == "E" else hp["lr_unembed"]',
     'hp["lr_unembed"] if name == "E" else hp["lr_embed"]'),                                # rates swapped
    ('.reshape(r, c) * hp["grad_scale"]', '.reshape(r, c)'),                               # grad scale dropped
]


def _run_pins_on_copy(tmp_path, old, new, module="model.py", pins="test_oracle_pins.py"):
    src = open(os.path.join(ROOT, "oracle", module)).read()
    assert src.count(old) == 1, "the mutation no longer applies to the oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synthdata"), tmp_path / "synthdata",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", pins):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    (tmp_path / "oracle" / module).write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        str(tmp_path / "tests" / pins)],
                       cwd=tmp_path, capture_output=True, text=True, timeout=600)
    return r


def test_unmodified_copy_passes(tmp_path):
    """Control: the copy with no mistake passes, so a failing mutant fails
    because of its mistake."""
    r = _run_pins_on_copy(tmp_path, MUTANTS[0][0], MUTANTS[0][0])
    assert r.returncode == 0, r.stdout[-2000:]


def test_unmodified_optim_copy_passes(tmp_path):
    r = _run_pins_on_copy(tmp_path, MUTANTS_OPTIM[0][0], MUTANTS_OPTIM[0][0], "optim.py", "test_oracle_optim.py")
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("old,new", MUTANTS, ids=[f"m{i}" for i in range(len(MUTANTS))])
def test_planted_mistake_fails_a_pin(tmp_path, old, new):
    r = _run_pins_on_copy(tmp_path, old, new)
    assert r.returncode == 1, f"mutant survived the pins:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("old,new", MUTANTS_OPTIM, ids=[f"o{i}" for i in range(len(MUTANTS_OPTIM))])
def test_planted_optimiser_mistake_fails_a_pin(tmp_path, old, new):
    r = _run_pins_on_copy(tmp_path, old, new, "optim.py", "test_oracle_optim.py")
    assert r.returncode == 1, f"mutant survived the pins:\n{r.stdout[-2000:]}"
