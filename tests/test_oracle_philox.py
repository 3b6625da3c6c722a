"""Exact pins of the oracle's Philox-4x32-10 generator and of the map from a
score position to a generator word, against rocRAND.

rocRAND (ROCm's random-number library) ships its own implementation of
Philox-4x32-10, the generator of Salmon, Moraes, Dror and Shaw, "Parallel
random numbers: as easy as 1, 2, 3" (SC 2011), usable from host code.  The
helper `rocrand_philox_ref.cpp` is compiled here with hipcc (host code only)
and asked for:
  * whole blocks at given 128-bit counters and 64-bit keys -- compared with
    `fa_oracle_philox4x32_10` word for word;
  * the word at stream position n of a stream that starts at counter
    `offset` -- rocRAND's own counter arithmetic (word n mod 4 of counter
    offset + floor(n / 4), carrying from the low counter word into the high
    one), which is the map ruDNN dense_attention.rs `keep_global` describes;
    the oracle's keep decision at that position must flip exactly at
    u = floor(w / 2^8) / 2^24.
The two implementations share no source: a wrong multiplier, Weyl
increment, word order or counter carry on the oracle's side fails here.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import dropout_multiplier, philox4x32_10

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rocrand_philox_ref.cpp")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc or the rocRAND headers are not installed")
    exe = str(tmp_path_factory.mktemp("rocrand") / "philox_ref")
    subprocess.run([hipcc, "-O1", SRC, "-o", exe], check=True, capture_output=True)

    def run(lines):
        out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
        return out.stdout.split("\n")[:len(lines)]

    return run


def _blocks(run, reqs):
    lines = ["B " + " ".join(f"{x:08x}" for x in (*key, *ctr)) for ctr, key in reqs]
    return [[int(w, 16) for w in line.split()] for line in run(lines)]


def test_known_counters_and_keys(rocrand_ref):
    reqs = [((0, 0, 0, 0), (0, 0)),
            ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF)),
            ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0)),
            ((1, 0, 0, 0), (0, 0)),
            ((0, 0, 0, 1), (0, 0)),
            ((0, 0, 0, 0), (0, 1))]
    for (ctr, key), ref in zip(reqs, _blocks(rocrand_ref, reqs)):
        assert philox4x32_10(ctr, key) == ref, (ctr, key)


def test_random_counters_and_keys(rocrand_ref):
    rng = np.random.default_rng(2011)
    reqs = [(tuple(int(x) for x in rng.integers(0, 2 ** 32, 4)), tuple(int(x) for x in rng.integers(0, 2 ** 32, 2)))
            for _ in range(400)]
    got = [philox4x32_10(c, k) for c, k in reqs]
    assert got == _blocks(rocrand_ref, reqs)


@pytest.mark.parametrize("seed,offset", [(0, 0), (0x0123456789ABCDEF, 3),
                                         (99, 0xFFFFFFFF),            # low counter word carries into the high one
                                         (7, 0x00000001FFFFFFFE),
                                         (0xFFFFFFFFFFFFFFFF, 12345)])
def test_position_to_word_and_keep_threshold(rocrand_ref, seed, offset):
    """The oracle keeps position n exactly when u_n >= p, with u_n from the
    rocRAND word at that position: p = u_n keeps, p = u_n + 2^-24 drops."""
    ns = list(range(0, 16)) + [1 << 20, (1 << 20) + 3, (1 << 34) + 5, (1 << 34) + 6]
    lines = [f"W {seed & 0xFFFFFFFF:08x} {seed >> 32:08x} {offset & 0xFFFFFFFF:08x} {offset >> 32:08x} "
             f"{n & 0xFFFFFFFF:08x} {n >> 32:08x}" for n in ns]
    words = [int(x, 16) for x in rocrand_ref(lines)]
    for n, w in zip(ns, words):
        top = w >> 8
        u = top / 2.0 ** 24
        assert np.float32(u) == u  # exact in fp32, as the API's rate is
        if u < 1.0:
            kept = dropout_multiplier(n, u, seed, offset)
            assert kept == pytest.approx(1.0 / (1.0 - float(np.float32(u))), rel=1e-15), (n, hex(w))
        if top + 1 < (1 << 24):
            assert dropout_multiplier(n, (top + 1) / 2.0 ** 24, seed, offset) == 0.0, (n, hex(w))


# ---- the pins have teeth: copies of the oracle with one planted mistake in
# the generator or the position map must disagree with rocRAND ----

PHILOX_MUTANTS = {
    "multipliers_swapped": ("const uint64_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;",
                            "const uint64_t M0 = 0xCD9E8D57u, M1 = 0xD2511F53u;"),
    "weyl_increment_wrong": ("const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;",
                             "const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE86u;"),
    "output_words_swapped": ("out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;",
                             "out[0] = c1; out[1] = c0; out[2] = c2; out[3] = c3;"),
    "nine_rounds": ("for (int round = 0; round < 10; ++round) {", "for (int round = 0; round < 9; ++round) {"),
    "key_words_swapped": ("const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};",
                          "const uint32_t key[2] = {(uint32_t)(seed >> 32), (uint32_t)seed};"),
    "no_carry_into_high_word": ("const uint32_t ctr[4] = {(uint32_t)ctr64, (uint32_t)(ctr64 >> 32), 0u, 0u};",
                                "const uint32_t ctr[4] = {(uint32_t)ctr64, 0u, 0u, 0u};"),
    "word_order_reversed": ("const double u = (double)(w[n % 4] >> 8) / 16777216.0;",
                            "const double u = (double)(w[3 - n % 4] >> 8) / 16777216.0;"),
    "low_bits_used": ("const double u = (double)(w[n % 4] >> 8) / 16777216.0;",
                      "const double u = (double)(w[n % 4] & 0xFFFFFFu) / 16777216.0;"),
}


@pytest.mark.parametrize("name", sorted(PHILOX_MUTANTS))
def test_philox_mutant_is_caught(rocrand_ref, tmp_path, name, monkeypatch):
    import oracle.oracle as orc
    from oracle import OracleLib
    from test_oracle_mutants import _build_mutant

    old, new = PHILOX_MUTANTS[name]
    mut = OracleLib(_build_mutant(str(tmp_path), name, old, new))
    monkeypatch.setattr(orc, "_DEFAULT", mut)
    caught = []
    for t, args in ((test_known_counters_and_keys, ()), (test_random_counters_and_keys, ()),
                    (test_position_to_word_and_keep_threshold, (99, 0xFFFFFFFF)),
                    (test_position_to_word_and_keep_threshold, (0x0123456789ABCDEF, 3))):
        try:
            t(rocrand_ref, *args)
        except AssertionError:
            caught.append(t.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
