"""The oracle's CPU pins catch plausible mistakes in the oracle.

Each mutant in tests/oracle_mutants.py plants one slip in the oracle's source
(a wrong head map, a dropped scale, a reversed gather, a sign error in the
split-K merge, a wrong FP8 exponent bias or tie rule, a wrong slot formula,
the allocator popping the wrong end, a copy in the wrong direction, a dropped
K+V factor, ...). For every mutant the pins run in a fresh pytest process
with the mutant applied, and at least one of them must fail; the unmutated
oracle must pass the same run. All of this runs on the CPU.
"""

import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

import oracle_mutants

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PINS = ["test_oracle_pins.py", "test_oracle_multi_query.py", "test_oracle_cascade.py",
        "test_oracle_swap.py", "test_oracle_prefix_cache.py", "test_fp8_codec.py",
        "test_fp4_codec.py"]


def run_pins(mutant):
    env = dict(os.environ)
    env.pop("ORACLE_MUTANT", None)
    if mutant:
        env["ORACLE_MUTANT"] = mutant
    env["OMP_NUM_THREADS"] = "1"
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           "-m", "not gpu", *[os.path.join(HERE, f) for f in PINS]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return mutant, r.returncode, r.stdout[-2000:] + r.stderr[-2000:]


def test_every_mutant_text_occurs_once():
    for name, (module, old, new) in oracle_mutants.MUTANTS.items():
        _, src = oracle_mutants.source_of(module)
        assert src.count(old) == 1, name
        assert old != new, name


def test_pins_pass_on_the_oracle_and_fail_on_every_mutant():
    names = [None] + sorted(oracle_mutants.MUTANTS)
    workers = min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(run_pins, names))
    clean = results[0]
    assert clean[1] == 0, f"the unmutated oracle fails its pins:\n{clean[2]}"
    survivors = [name for name, rc, _ in results[1:] if rc != 1]
    detail = {name: out for name, rc, out in results[1:] if rc != 1}
    assert not survivors, f"mutants not caught (or errored): {survivors}\n{detail}"
