"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign, a transposed or
swapped operand, the wrong tie rule or nibble order, a wrong rounding) in a
temporary copy of ``oracle/`` and runs the pin tests against that copy; at
least one pin must fail.  The repository's own files are never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("qlora.py", "Y = X @ W.T + s * (XA @ B.T)", "Y = X @ W.T - s * (XA @ B.T)"),
    ("qlora.py", "dX = dY @ W + s * (T @ A)", "dX = dY @ W + (T @ A)"),
    ("qlora.py", "dB = s * (dY.T @ XA)", "dB = s * (dY.T @ (X @ A[::-1].T))"),
    ("qlora.py", "dA = s * (T.T @ X)", "dA = s * (T.T @ X[::-1])"),
    ("qlora.py", "return sg * (1.0 + g * (1.0 - sg))", "return sg * (1.0 + g * (1.0 + sg))"),
    ("qlora.py", "dG = dH * U * silu_grad(G)", "dG = dH * U * sigmoid(G)"),
    ("qlora.py", "dU = dH * silu(G)", "dU = dH * sigmoid(G)"),
    ("qlora.py", "return float(alpha) / float(r)", "return float(alpha) / float(r + 1)"),
    ("qlora.py", "return W + lora_scale(alpha, A.shape[0]) * (B @ A)", "return W + alpha * (B @ A)"),
    ("qlora.py", "return W + lora_scale(alpha, A.shape[0]) * (B @ A)",
     "return W + lora_scale(alpha, A.shape[0]) * (B @ A[:, ::-1])"),
    ("qlora.py", "q = np.maximum(e - 8, -133)", "q = np.maximum(e - 9, -133)"),
    ("qlora.py", "y = np.ldexp(np.rint(np.ldexp(x, -q)), q)", "y = np.ldexp(np.floor(np.ldexp(x, -q) + 0.5), q)"),
    ("rmsnorm.py", "dX = rstd[:, None] * g - (rstd ** 3 / D * c)[:, None] * X",
     "dX = rstd[:, None] * g + (rstd ** 3 / D * c)[:, None] * X"),
    ("rmsnorm.py", "rstd ** 3 / D", "rstd ** 2 / D"),
    ("rmsnorm.py", "dw = np.sum(dY * X * rstd[:, None], axis=0)", "dw = np.sum(dY * X, axis=0)"),
    ("rmsnorm.py", "ms = np.mean(X * X, axis=1)", "ms = np.sum(X * X, axis=1)"),
    ("linear_ce.py", "lse = zmax + np.log(S)", "lse = np.log(S)"),
    ("linear_ce.py", "G[np.arange(T), tgt] -= 1.0", "G[np.arange(T), tgt] += 1.0"),
    ("linear_ce.py", "loss = float(token_loss.sum() / n) if n > 0 else 0.0",
     "loss = float(token_loss.sum() / T) if n > 0 else 0.0"),
    ("linear_ce.py", "dX = (G @ W) / n if n > 0 else np.zeros_like(X)",
     "dX = (G @ W[::-1]) / n if n > 0 else np.zeros_like(X)"),
    ("linear_ce.py", "G[~valid] = 0.0", "G[~valid] *= 1.0"),
    ("linear_ce.py", "E = np.exp(Z - zmax[:, None])", "E = np.exp(Z - zmax[::-1, None])"),
    ("nf4.py", 'side="left"', 'side="right"'),
    ("nf4.py", "flat[0::2] | (flat[1::2] << np.uint8(4))", "flat[1::2] | (flat[0::2] << np.uint8(4))"),
    ("nf4.py", "np.minimum(np.rint(ratio), 255.0)", "np.minimum(np.floor(ratio), 255.0)"),
    ("nf4.py", "return (cb[:-1] + cb[1:]) / 2.0", "return (cb[:-1] + cb[1:]) / 2.0 + 1e-9"),
    ("nf4.py", "S = np.float32(seg.max()) / np.float32(255.0)",
     "S = np.float32(seg.max()) / np.float32(256.0)"),
    ("nf4.py", "vals = cb[q].reshape(-1, bs) * a[:, None]",
     "vals = cb[q].reshape(-1, bs) * a.mean()"),
]


@pytest.fixture(scope="module")
def sandbox(tmp_path_factory):
    d = tmp_path_factory.mktemp("oracle_mut")
    shutil.copytree(os.path.join(ROOT, "synth"), d / "synth",
                    ignore=shutil.ignore_patterns("*.tmp*", "__pycache__"))
    os.makedirs(d / "tests" / "golden")
    for f in ("conftest.py", "test_oracle_nf4.py", "test_oracle_qlora.py", "test_oracle_rmsnorm.py",
              "test_oracle_linear_ce.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), d / "tests" / f)
    shutil.copy(os.path.join(ROOT, "tests", "golden", "nf4_codebook.txt"),
                d / "tests" / "golden" / "nf4_codebook.txt")
    return d


@pytest.mark.parametrize("fname,old,new", MUTATIONS, ids=[m[2][:40] for m in MUTATIONS])
def test_pins_catch_mutation(sandbox, fname, old, new):
    od = sandbox / "oracle"
    if od.exists():
        shutil.rmtree(od)
    shutil.copytree(os.path.join(ROOT, "oracle"), od, ignore=shutil.ignore_patterns("__pycache__"))
    src = (od / fname).read_text()
    assert old in src
    (od / fname).write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_nf4.py", "tests/test_oracle_qlora.py", "tests/test_oracle_rmsnorm.py",
                        "tests/test_oracle_linear_ce.py"],
                       cwd=str(sandbox), capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, "mutation survived: %s\n%s" % (new, r.stdout[-2000:])
