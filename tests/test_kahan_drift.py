"""Accuracy of the compensated float32 scores over the 4,000,000-token stream
(Report §4.4 Q1: H2O with position rolling streams 4 million tokens).

A slot's score gains one attention weight per decode step.  The increments are
drawn from the weights the oracle computes on the stream workload itself
(LLaMA-7B shape, k = 1024 + 1024, weights of every cached entry over 1,400 steps
with the cache full), and 4,000,000 of them are summed the way the decode kernel
does (plain float32 adds for the first 1,024 steps after the prefill, then
compensated ones; ``tests/native/kahan_drift.c``) and in float64.  The score the
eviction compares (the running sum s) and the folded score s - c must stay
within 1e-4 relative of the float64 sum at every million steps, and after the
first 1,024 plain adds within their bound 1024 * 2^-24; a plain float32 sum is
shown to drift far past 1e-4."""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import run_unit
from workload import get, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "kahan_drift.c")
OUT = os.path.join(ROOT, "kv_cache_eviction_prefill_amd", "_build", "kahan_drift.so")
STEPS = 4_000_000
EVERY = 1_000_000
PLAIN = 1024  # decode steps after a prefill whose weights are added without compensation


@pytest.fixture(scope="module")
def kahan():
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", SRC, "-o", OUT],
                   check=True)
    lib = ctypes.CDLL(OUT)
    f32p, f64p = ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)
    lib.kahan_drift.argtypes = [f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, f32p, f32p, f32p, f64p]
    lib.kahan_drift.restype = None

    def run(w, every=EVERY):
        w = np.ascontiguousarray(w, np.float32)
        m = len(w) // every
        s, c, p = (np.zeros(m, np.float32) for _ in range(3))
        e = np.zeros(m, np.float64)
        f32 = lambda a: a.ctypes.data_as(f32p)  # noqa: E731
        lib.kahan_drift(f32(w), len(w), PLAIN, every, f32(s), f32(c), f32(p), e.ctypes.data_as(f64p))
        return s, c, p, e
    return run


@pytest.fixture(scope="module")
def measured_weights():
    # the oracle on one head of the stream workload: every attended entry's weight
    # at every step once the cache holds k = 2048 entries
    w = get("llama7b-stream-4m")
    L, T = w.prompt_len, 2048 + 1400 - w.prompt_len + 512
    Q, K, V = synth.unit_qkv(w, 0, 0, 0, 0, L + T)
    res = run_unit(Q, K, V, L, w.heavy_budget, w.recent_budget, keep_weights=True)
    full = [a for (pos, a) in res["weights"] if len(a) == w.k + 1]
    assert len(full) >= 1000
    return np.concatenate(full)


@pytest.mark.parametrize("kind", ["typical", "heavy", "light"])
def test_compensated_scores_over_four_million_steps(kahan, measured_weights, kind):
    g = np.random.default_rng({"typical": 1, "heavy": 2, "light": 3}[kind])
    pool = np.sort(measured_weights)
    if kind == "heavy":   # a heavy hitter: increments from the top 1 % of the weights
        pool = pool[-len(pool) // 100:]
    elif kind == "light":  # a rarely attended token: the bottom 10 %
        pool = pool[:len(pool) // 10]
    inc = g.choice(pool, size=STEPS).astype(np.float32)
    s, c, plain, exact = kahan(inc)
    rel_s = np.abs(s.astype(np.float64) - exact) / exact
    rel_f = np.abs(s.astype(np.float64) - c.astype(np.float64) - exact) / exact
    rel_p = np.abs(plain.astype(np.float64) - exact) / exact
    print(f"{kind}: mean increment {inc.mean():.3g}; relative error at 1M..4M steps: running sum "
          f"{rel_s.tolist()}, folded {rel_f.tolist()}, plain float32 {rel_p.tolist()}")
    assert rel_s.max() <= 1e-4
    assert rel_f.max() <= 1e-4
    assert rel_p.max() > 100 * rel_f.max()  # the compensation is what keeps it there
    # the plain adds alone: a prompt score (the first increment) plus 1,024 weights
    s1, _, _, e1 = kahan(inc[:PLAIN + 1], every=PLAIN + 1)
    assert abs(float(s1[0]) - e1[0]) / e1[0] <= PLAIN * 2.0 ** -24
