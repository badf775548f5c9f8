"""Pin for the oracle's Philox4x32-10 against rocRAND's implementation.

rocRAND's header-only Philox4x32-10 engine is compiled for the host with g++
and run on the same (key, counter) pairs; its source is not copied.  The
stochastic-rounding bit mapping is checked against its written rule.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROCRAND_INC = "/opt/rocm/include"


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    hdr = os.path.join(ROCRAND_INC, "rocrand", "rocrand_philox4x32_10.h")
    if shutil.which("g++") is None or not os.path.exists(hdr):
        pytest.skip("g++ or rocRAND header not available")
    exe = str(tmp_path_factory.mktemp("philox") / "pin")
    subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", ROCRAND_INC,
                    os.path.join(HERE, "philox_rocrand_pin.cpp"), "-o", exe], check=True)

    def run(triples):
        inp = "".join(f"{s} {q} {o}\n" for s, q, o in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return np.array([[int(w) for w in ln.split()] for ln in out.strip().splitlines()],
                        dtype=np.uint64)
    return run


def test_philox_matches_rocrand(rocrand_philox):
    rng = np.random.default_rng(123)
    triples = [(0, 0, 0), (2**64 - 1, 2**62 - 1, 2**64 - 1), (1, 1, 1)]
    triples += [(int(s), int(q), int(o)) for s, q, o in zip(
        rng.integers(0, 2**63, 200, dtype=np.uint64),
        rng.integers(0, 2**40, 200, dtype=np.uint64),
        rng.integers(0, 2**63, 200, dtype=np.uint64))]
    ref = rocrand_philox(triples)
    for (s, q, o), want in zip(triples, ref):
        got = oracle.philox4x32_10(q & 0xFFFFFFFF, q >> 32, o & 0xFFFFFFFF, o >> 32,
                                   s & 0xFFFFFFFF, s >> 32)
        assert [int(w) for w in got] == [int(w) for w in want], (s, q, o)


def test_sr_bits_mapping_rule(rocrand_philox):
    seed, off = 0x0123456789ABCDEF, 5
    p = np.arange(64, dtype=np.uint64) + np.uint64(8 * 1000)
    bits = oracle.sr_bits16(p, seed, off)
    words = rocrand_philox([(seed, int(pp) >> 3, off) for pp in p])
    for i, pp in enumerate(p):
        pp = int(pp)
        w = int(words[i][(pp >> 1) & 3])
        assert int(bits[i]) == (w >> (16 * (pp & 1))) & 0xFFFF


def test_sr_bits_uniform_statistics():
    p = np.arange(1 << 18, dtype=np.uint64)
    r = oracle.sr_bits16(p, 99, 0).astype(np.float64)
    assert abs(r.mean() / 65535.0 - 0.5) < 0.005
    counts = np.bincount((r.astype(np.int64) >> 12), minlength=16)
    expected = len(r) / 16
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert chi2 < 45          # 15 dof, p ~ 1e-4


def test_sr_bits8_mapping_rule(rocrand_philox):
    """8-bit draws: element p takes byte (p & 3) of word ((p >> 2) & 3) of the
    Philox call p >> 4 (rocRAND's engine, run on the host, supplies the words)."""
    seed, off = 0xFEDCBA9876543210, 7
    p = np.arange(96, dtype=np.uint64) + np.uint64(16 * 777 + 5)
    bits = oracle.sr_bits8(p, seed, off)
    words = rocrand_philox([(seed, int(pp) >> 4, off) for pp in p])
    for i, pp in enumerate(p):
        pp = int(pp)
        w = int(words[i][(pp >> 2) & 3])
        assert int(bits[i]) == (w >> (8 * (pp & 3))) & 0xFF


def test_sr_bits8_uniform_statistics():
    r = oracle.sr_bits8(np.arange(1 << 18, dtype=np.uint64), 99, 0).astype(np.int64)
    counts = np.bincount(r >> 4, minlength=16)
    expected = len(r) / 16
    assert ((counts - expected) ** 2 / expected).sum() < 45
    assert abs(r.mean() / 255.0 - 0.5) < 0.005
