"""Mutation check of the oracle's pins: each entry below plants one plausible mistake in a
copy of oracle/bsa_oracle.c (a wrong index, a dropped or inverted scale, a flipped rule),
builds it, and runs the whole pin module against it. Every mutant must fail at least one
pin; a mutant that passes would mean a part of the oracle no pin constrains.

CPU only: the mutants are built with gcc into a temporary folder and loaded through the
BSA_ORACLE_LIB override of the oracle package.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in bsa_oracle.c, replacement, which occurrence)
MUTANTS = [
    ("fp8 block scale: the first block's for every token", "T->scale[bh * T->nblk + t / T->block]",
     "T->scale[bh * T->nblk]", 0),
    ("fp8 block scale: head offset missing", "T->scale[bh * T->nblk + t / T->block]", "T->scale[t / T->block]", 0),
    ("fp8 block scale dropped", ": (double)T->scale[bh * T->nblk + t / T->block];", ": 1.0;", 0),
    ("fp8 dequantisation divides by the scale", "return e4m3_table[T->e4m3[off]] * sc;",
     "return e4m3_table[T->e4m3[off]] / sc;", 0),
    ("V channel scale: the first channel's", "T->chan_scale[bh * T->D + d]", "T->chan_scale[bh * T->D]", 0),
    ("V channel scale: head offset missing", "T->chan_scale[bh * T->D + d]", "T->chan_scale[d]", 0),
    ("fp8-QK: K dequantised with Q's scales", "K = {NULL, k8, k_scale, NULL,", "K = {NULL, k8, q_scale, NULL,", 0),
    ("full fp8 operands: V with block scales", "V = {NULL, v8, NULL, v_scale,", "V = {NULL, v8, k_scale, NULL,", 0),
    ("spread term without the weights", "dv[d] += p * e;", "dv[d] += e;", 0),
    ("logit scale 1/sqrt(D) dropped", "logit[a] = dot * inv;", "logit[a] = dot;", 0),
    ("partial block mean divides by the block size", "xbar[r * D + d] = sum / (double)(t1 - t0);",
     "xbar[r * D + d] = sum / (double)block;", 0),
    ("ties go to the higher block index", "return (x->j > y->j) - (x->j < y->j);",
     "return (x->j < y->j) - (x->j > y->j);", 0),
    ("k rounded to nearest", "double k = ceil(keep_ratio * (double)n - 1e-6);",
     "double k = floor(keep_ratio * (double)n + 0.5);", 0),
    ("scores with Q and K means swapped", "dot += qbar[r * D + d] * kbar[(bh * n + j) * D + d];",
     "dot += kbar[r * D + d] * qbar[(bh * n + j) * D + d];", 0),
    ("fp8 quantiser range 240", "float sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;",
     "float sc = (amax > 0.0f) ? amax / 240.0f : 1.0f;", 0),
    ("V read at the query token", "o[d] += p * load(V, bh, key[a], d);", "o[d] += p * load(V, bh, t, d);", 0),
    ("E4M3 ties away from even", "else pick = (lo % 2 == 0) ? lo : hi;", "else pick = hi;", 0),
    ("E4M3 subnormal step 2^-7", "mag = ldexp((double)m / 8.0, -6);", "mag = ldexp((double)m / 8.0, -7);", 0),
]


def mutate(src, old, new, occurrence):
    at = -1
    for _ in range(occurrence + 1):
        at = src.find(old, at + 1)
        assert at >= 0, "mutation target not found: %r" % old
    return src[:at] + new + src[at + len(old):]


def run_pins(lib):
    env = dict(os.environ, BSA_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-400:]


def test_every_mutant_fails_a_pin():
    src = open(oracle_build.SRC).read()
    for name, old, new, occ in MUTANTS:  # each target must be present as written
        mutate(src, old, new, occ)
    with tempfile.TemporaryDirectory() as tmp:
        libs = []
        for i, (name, old, new, occ) in enumerate(MUTANTS):
            path = os.path.join(tmp, "mutant%02d.c" % i)
            with open(path, "w") as f:
                f.write(mutate(src, old, new, occ))
            libs.append(oracle_build.build(src=path, lib=os.path.join(tmp, "mutant%02d.so" % i)))
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(run_pins, libs))
    survivors = [(name, out) for (name, *_), (rc, out) in zip(MUTANTS, results) if rc == 0]
    assert not survivors, "mutants that pass every pin: %s" % survivors


def test_unmutated_copy_passes_the_pins():
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle_build.build(lib=os.path.join(tmp, "copy.so"))
        rc, out = run_pins(lib)
    assert rc == 0, out
