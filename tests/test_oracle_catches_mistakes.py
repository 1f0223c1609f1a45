"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (a dropped or extra term, a wrong sign, index, operand or order) in
a copy of the oracle, on the CPU, and runs the oracle's pin modules against that copy: at least
one pin must fail. The unchanged copy must pass, so a failure comes from the planted mistake.
Nothing here touches the GPU or the HIP library.
"""
import os
import shutil
import subprocess
import sys

import pytest

pytestmark = pytest.mark.slow

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["test_oracle_assign.py", "test_oracle_attention.py", "test_oracle_asym.py",
        "test_oracle_train.py"]

# (oracle file, the mistake, text as written, text with the mistake)
MISTAKES = [
    ("focus_ref.py", "scores divided by a temperature",
     "        S[r0:r0 + chunk] = z @ c.T",
     "        S[r0:r0 + chunk] = z @ c.T / math.sqrt(c.shape[1])"),
    ("focus_ref.py", "row step with the wrong sign",
     "        u = -_logsumexp(S + v[None, :], axis=1)",
     "        u = _logsumexp(S + v[None, :], axis=1)"),
    ("focus_ref.py", "columns given mass K/n",
     "    log_col_mass = math.log(n / K) if n > 0 else 0.0",
     "    log_col_mass = math.log(K / n) if n > 0 else 0.0"),
    ("focus_ref.py", "column step before the row step",
     "    for _ in range(iters):\n"
     "        u = -_logsumexp(S + v[None, :], axis=1)\n"
     "        v = log_col_mass - _logsumexp(S + u[:, None], axis=0)",
     "    for _ in range(iters):\n"
     "        v = log_col_mass - _logsumexp(S + u[:, None], axis=0)\n"
     "        u = -_logsumexp(S + v[None, :], axis=1)"),
    ("focus_ref.py", "raw scores ranked instead of balanced ones",
     "    b = S + v[None, :]",
     "    b = S"),
    ("focus_ref.py", "top-k misses the best group",
     "    groups = np.sort(order[:, :top_k], axis=1).astype(np.int32)",
     "    groups = np.sort(order[:, 1:top_k + 1], axis=1).astype(np.int32)"),
    ("focus_ref.py", "window one token wider",
     "    j = np.arange(i + 1)\n    local = (i - j) < window\n    gj = groups[:i + 1]",
     "    j = np.arange(i + 1)\n    local = (i - j) <= window\n    gj = groups[:i + 1]"),
    ("focus_ref.py", "the query's own key left out",
     "    j = np.arange(i + 1)\n    local = (i - j) < window\n    gj = groups[:i + 1]",
     "    j = np.arange(i)\n    local = (i - j) < window\n    gj = groups[:i]"),
    ("focus_ref.py", "softmax scale 1/d_head",
     "    Hkv = k.shape[1]\n    G = Hq // Hkv\n"
     "    scale = 1.0 / math.sqrt(dh) if scale is None or scale <= 0 else float(scale)",
     "    Hkv = k.shape[1]\n    G = Hq // Hkv\n"
     "    scale = 1.0 / dh if scale is None or scale <= 0 else float(scale)"),
    ("focus_ref.py", "query head h read from kv head h mod Hkv",
     "    kv_of = np.arange(Hq) // G\n    out = np.empty((len(rows), Hq, v.shape[2]))\n"
     "    lse = np.empty((len(rows), Hq))\n    for r, i in enumerate(rows):\n"
     "        J = allowed_keys_ref(",
     "    kv_of = np.arange(Hq) % Hkv\n    out = np.empty((len(rows), Hq, v.shape[2]))\n"
     "    lse = np.empty((len(rows), Hq))\n    for r, i in enumerate(rows):\n"
     "        J = allowed_keys_ref("),
    ("focus_ref.py", "log-sum-exp without its shift",
     "    return np.squeeze(m, axis) + np.log(np.sum(np.exp(x - m), axis=axis))",
     "    return np.log(np.sum(np.exp(x - m), axis=axis))"),
    ("focus_ref.py", "inclusion-exclusion without alternating signs",
     "        sign = 1 if s % 2 == 1 else -1",
     "        sign = 1"),
    ("focus_ref.py", "decode ignores the query's groups",
     "        J = allowed_keys_ref(p, cache_groups[b], window, query_groups=q_groups[b])",
     "        J = allowed_keys_ref(p, cache_groups[b], window)"),
    ("train_ref.py", "affinity gradient without its transposed term",
     "dP = (dA + dA.T) @ P", "dP = dA @ P"),
    ("train_ref.py", "column step's gradient with the wrong sign",
     "dS -= dv[None, :] * Wc", "dS += dv[None, :] * Wc"),
    ("train_ref.py", "row step's gradient left out",
     "dS -= du[:, None] * Wr", "pass"),
    ("train_ref.py", "gate slope sigma(+lambda a) for sigma(-lambda a)",
     "lam * np.exp(-np.logaddexp(0.0, lam * a))", "lam * np.exp(-np.logaddexp(0.0, -lam * a))"),
    ("train_ref.py", "softmax gradient without the D term",
     "dB += p * (dp - D[:, None])", "dB += p * dp"),
    ("train_ref.py", "centroid gradient from the transposed product",
     "d_centroids=dS.T @ Z", "d_centroids=(Z.T @ dS).T * 1.0001"),
]


def _copy_tree(dst):
    """The oracle, the input generators and the pin modules (with their goldens) under dst."""
    for pkg in ("oracle", "synth"):
        shutil.copytree(os.path.join(ROOT, pkg), os.path.join(dst, pkg),
                        ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    for f in ["conftest.py"] + PINS:
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))


def _run_pins(dst):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           *[os.path.join(dst, "tests", f) for f in PINS]],
                          cwd=dst, env=env, capture_output=True, text=True, timeout=900)


def test_unchanged_oracle_copy_passes_its_pins(tmp_path):
    _copy_tree(str(tmp_path))
    r = _run_pins(str(tmp_path))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("fname,mistake,good,bad", MISTAKES, ids=[m[1] for m in MISTAKES])
def test_planted_mistake_fails_a_pin(tmp_path, fname, mistake, good, bad):
    _copy_tree(str(tmp_path))
    path = os.path.join(str(tmp_path), "oracle", fname)
    src = open(path).read()
    assert src.count(good) == 1, f"the text to change is not unique in {fname}"
    with open(path, "w") as f:
        f.write(src.replace(good, bad))
    r = _run_pins(str(tmp_path))
    assert r.returncode != 0, f"no pin caught: {mistake}\n{r.stdout[-1500:]}"
