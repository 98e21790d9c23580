"""The pins in test_oracle_pins.py must catch plausible mistakes in the oracle.

Each case plants one mistake in a scratch copy of oracle/signmuon_oracle.c (a
dropped or flipped term, a transposed operand, a wrong index, a missing
rounding, a wrong tie rule ...), builds that copy with oracle/build.py and runs
the pin suite against it: the suite must fail. The unmodified copy must pass,
so a failure is the mistake's doing and not the harness's. Everything runs on
the CPU; the GPU path is not involved. (Reading the Gram transposed in the
product is no mistake to plant: the Gram is symmetric entry for entry, so that
change computes the same values.)"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "signmuon_oracle.c")

# (what the mistake is, text in the oracle, the mistaken text)
MUTATIONS = [
    # Newton-Schulz (cubic 1.5 / -0.5, Gram of the smaller side)
    ("sign of the cubic term", "double next = 1.5 * x[t] - 0.5 * p[t];",
     "double next = 1.5 * x[t] + 0.5 * p[t];"),
    ("linear coefficient", "double next = 1.5 * x[t] - 0.5 * p[t];",
     "double next = 1.4 * x[t] - 0.5 * p[t];"),
    ("Gram of the wide orientation with a wrong operand index",
     "acc += x[i * C + k] * x[l * C + k];",
     "acc += x[i * C + k] * x[k * C + l < R*C ? k * C + l : 0];"),
    ("Gram of the tall orientation with a transposed operand",
     "a[i * C + l] += xi * x[k * C + l];", "a[i * C + l] += xi * x[k * C + i];"),
    ("wide product reads the wrong row of X", "p[i * C + j] += ail * x[l * C + j];",
     "p[i * C + j] += ail * x[i * C + j];"),
    ("tall product keeps only the Gram's diagonal", "p[i * C + j] += xil * a[l * C + j];",
     "p[i * C + j] += xil * a[l * C + l];"),
    ("Gram not rounded to the storage type", "a[t] = round_ns(a[t], ns_dt);", "a[t] = a[t];"),
    ("intermediate iterate not rounded", "x[t] = last ? next : round_ns(next, ns_dt);",
     "x[t] = next;"),
    # sign and pack
    ("bit order reversed in the word", "words[i / 64] |= (uint64_t)1 << (i % 64);",
     "words[i / 64] |= (uint64_t)1 << (63 - i % 64);"),
    ("zero maps to -1", "if (load_elem(u, u_dt, i) >= 0.0)", "if (load_elem(u, u_dt, i) > 0.0)"),
    # vote and update
    ("vote tie moves the weight", "int8_t v = sum > 0 ? 1 : (sum < 0 ? -1 : 0);",
     "int8_t v = sum >= 0 ? 1 : -1;"),
    ("update with the wrong sign", "w[i] = w[i] - eta;", "w[i] = w[i] + eta;"),
    # momentum and normalisation
    ("momentum rounded twice instead of one fused multiply-add",
     "store_f32_value(m, m_dt, i, fmaf(beta, mi, gi));",
     "store_f32_value(m, m_dt, i, beta * mi + gi);"),
    ("bf16 rounding: ties not to even", "u += 0x7fffu + keep_lsb;", "u += 0x8000u;"),
    ("scale from the squared norm", "double s = nu > 0.0 ? 1.0 / nu : 0.0;",
     "double s = nu > 0.0 ? 1.0 / ss : 0.0;"),
    ("momentum input not rounded to bf16", "f = orc_bf16_to_f32(orc_bf16_from_f32(f));", "f = f;"),
    # post-vote polar step
    ("vote not normalised before the polar step", "y0[i] = s * (double)vote[i];",
     "y0[i] = (double)vote[i];"),
    # int8 payload
    ("int8 sign: zero maps to -1",
     "s[i] = load_elem(u, u_dt, i) >= 0.0 ? (int8_t)1 : (int8_t)-1;",
     "s[i] = load_elem(u, u_dt, i) > 0.0 ? (int8_t)1 : (int8_t)-1;"),
    ("int8 vote sums signs instead of values", "sum += signs[(int64_t)m * n + i];",
     "sum += signs[(int64_t)m * n + i] > 0 ? 1 : -1;"),
    ("int8 vote drops the worker index", "sum += signs[(int64_t)m * n + i];", "sum += signs[i];"),
    # spectral normalisation
    ("power vector not normalised", "            v[i] = w[i] / lambda;", "            v[i] = w[i];"),
    ("power iteration from a basis vector", "        v[i] = 1.0 / sqrt((double)r);",
     "        v[i] = i == 0 ? 1.0 : 0.0;"),
    ("spectral scale 1/lambda instead of 1/sqrt(lambda)",
     "    double s = lambda > 0.0 ? 1.0 / sqrt(lambda) : 0.0;",
     "    double s = lambda > 0.0 ? 1.0 / lambda : 0.0;"),
    ("first Gram scaled by s instead of s^2", "        a0[t] = round_ns(s2d * a0[t], ns_dt);",
     "        a0[t] = round_ns(sqrt(s2d) * a0[t], ns_dt);"),
    ("given first Gram used at the wrong iteration", "        if (j == 0 && a0)",
     "        if (j == 1 && a0)"),
    # Muon comparison step
    ("Muon update rounded twice", "            w[i] = fmaf(-eta, (float)u[i], w[i]);",
     "            w[i] = w[i] - eta * (float)u[i];"),
    ("Muon update with the wrong sign", "            w[i] = fmaf(-eta, (float)u[i], w[i]);",
     "            w[i] = fmaf(eta, (float)u[i], w[i]);"),
]


def run_pins(source_text):
    """Build the oracle from `source_text` in a scratch tree and run the pins.
    Returns pytest's exit status (0: every pin passed)."""
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        for d in ("oracle", "synthetic"):
            shutil.copytree(os.path.join(ROOT, d), os.path.join(tmp, d),
                            ignore=shutil.ignore_patterns("*.so", "__pycache__"))
        os.makedirs(os.path.join(tmp, "tests"))
        for f in ("conftest.py", "test_oracle_pins.py"):
            shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(tmp, "tests", f))
        shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tmp, "tests", "golden"))
        with open(os.path.join(tmp, "oracle", "signmuon_oracle.c"), "w") as f:
            f.write(source_text)
        env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
        subprocess.run([sys.executable, os.path.join("oracle", "build.py")], cwd=tmp, env=env,
                       check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                            os.path.join("tests", "test_oracle_pins.py")],
                           cwd=tmp, env=env, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL,
                           timeout=600)
        return r.returncode
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_every_planted_mistake_fails_a_pin():
    with open(SRC) as f:
        text = f.read()
    mutants = []
    for what, old, new in MUTATIONS:
        assert text.count(old) >= 1, f"mutation site not found: {what}"
        mutants.append((what, text.replace(old, new, 1)))
    jobs = [("unmodified", text)] + mutants
    with ThreadPoolExecutor(max_workers=4) as pool:
        status = dict(zip([w for w, _ in jobs], pool.map(lambda j: run_pins(j[1]), jobs)))
    assert status["unmodified"] == 0, "the pins fail on the unmodified oracle copy"
    survived = [w for w, _ in mutants if status[w] == 0]
    assert not survived, f"mistakes no pin caught: {survived}"
