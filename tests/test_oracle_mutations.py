"""The oracle's pins catch plausible mistakes.  Each mutation below is
planted in a copy of the oracle source (never in the source itself), compiled
to a temporary library, and the oracle's pin tests are run against it with
PAFP8_ORACLE_LIB: they must fail.  The mutations: a wrong exponent bias or
subnormal scale, rounding half up or ties to odd, no saturation, K and V
layouts off, the GQA head map, a dropped softmax scale or max, the V scale
taken from K, an unnormalised combine, a tag check of the first page only,
multiply for divide, the append position, a page index off by one, INT4
nibble, sign, scale and block-index mistakes, and reallocation mistakes.

Compiling and running the pins 28 times takes several minutes, so the check
runs only with PAFP8_MUTATION=1; that every mutation still applies to the
current source is checked always.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, text in the oracle source, replacement)
MUTATIONS = [
    ('decode bias 8',
     'mag = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 7);',
     'mag = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 8);'),
    ('subnormal scale',
     'mag = (double)m * ldexp(1.0, -9);',
     'mag = (double)m * ldexp(1.0, -10);'),
    ('fast encode floor',
     'q = rint(ldexp(a, 3 - E));',
     'q = floor(ldexp(a, 3 - E) + 0.5);'),
    ('tie odd',
     '(d == best_d && (c & 1) == 0)',
     '(d == best_d && (c & 1) == 1)'),
    ('no saturation at 448 (fast)',
     '    if (a >= 448.0)\n        return (uint8_t)(0x7E | sign);\n    if (a < ldexp(1.0, -6)) {',
     '    if (a >= 464.0)\n        return (uint8_t)(0x7F | sign);\n    if (a < ldexp(1.0, -6)) {'),
    ('k chunk quarter and column swapped',
     '+ ((int64_t)((j * KL + l) * 4 + q) * (4 * NS) + 4 * sub + a) * 16',
     '+ ((int64_t)((j * KL + q) * 4 + l) * (4 * NS) + 4 * sub + a) * 16'),
    ('k token group and lane swapped',
     '+ ((int64_t)((j * KL + l) * 4 + q) * (4 * NS) + 4 * sub + a) * 16',
     '+ ((int64_t)((j * KL + l) * 4 + q) * (4 * NS) + 4 * a + sub) * 16'),
    ('v token-major',
     'return (page * Hkv + g) * (int64_t)P * D + ((int64_t)(slot / SEG) * D + d) * SEG + slot % SEG;',
     'return (page * Hkv + g) * (int64_t)P * D + (int64_t)slot * D + d;'),
    ('v one segment per page',
     'return (page * Hkv + g) * (int64_t)P * D + ((int64_t)(slot / SEG) * D + d) * SEG + slot % SEG;',
     'return (page * Hkv + g) * (int64_t)P * D + (int64_t)d * P + slot;'),
    ('gqa mod',
     'q + bh * D, h / G, sm_scale, 0, L, o, &lse[bh]);',
     'q + bh * D, h % Hkv, sm_scale, 0, L, o, &lse[bh]);'),
    ('no sm_scale',
     's[t] = sm_scale * acc;',
     's[t] = acc;'),
    ('lse without max',
     '*lse = m + log(sum);',
     '*lse = log(sum);'),
    ('v scale from k',
     'kv_value(kv_dtype, 1, v_pool, v_scale,',
     'kv_value(kv_dtype, 1, v_pool, k_scale,'),
    ('combine unnormalised',
     'w = exp((double)pl[s] - LSE);',
     'w = exp((double)pl[s] - M);'),
    ('tag check first page only',
     'int n = (L + P - 1) / P, i;',
     'int n = 1, i;'),
    ('quantize multiply',
     'volatile float q = num / den;',
     'volatile float q = num * den;'),
    ('append position L',
     'int32_t start = context_lens[b] - 1, one = 1;',
     'int32_t start = context_lens[b], one = 1;'),
    ('page index off by one',
     'int64_t pi = t / P;\n    int slot = (int)(t % P);\n    int32_t page;\n    int64_t off;',
     'int64_t pi = (t + 1) / P;\n    int slot = (int)(t % P);\n    int32_t page;\n    int64_t off;'),
    ('int4 nibbles swapped',
     'int nib = high ? (packed[byte] >> 4) & 15 : packed[byte] & 15;',
     'int nib = high ? packed[byte] & 15 : (packed[byte] >> 4) & 15;'),
    ('int4 unsigned',
     'return nib >= 8 ? nib - 16 : nib;',
     'return nib;'),
    ('int4 offset binary',
     'return nib >= 8 ? nib - 16 : nib;',
     'return nib - 8;'),
    ('int4 scale transposed',
     'scales[(int64_t)(k / 128) * N + n]',
     'scales[(int64_t)n * (K / 128) + k / 128]'),
    ('int4 group 64',
     'scales[(int64_t)(k / 128) * N + n]',
     'scales[(int64_t)((k / 64) % (K / 128)) * N + n]'),
    ('int4 j/kq swapped',
     'int j = r / 32, kq = (r % 32) / 8,',
     'int kq = r / 32, j = (r % 32) / 8,'),
    ('realloc no bump',
     'page_tags[page] = page_tags[page] + 1u;',
     'page_tags[page] = page_tags[page];'),
    ('realloc records old tag',
     'expected_tags[(int64_t)b * maxP + i] = page_tags[page];',
     'expected_tags[(int64_t)b * maxP + i] = page_tags[page] - 1u;'),
    ('realloc no table update',
     'page_table[(int64_t)b * maxP + i] = page;',
     '(void)page;'),
    ('realloc ignores pool bound',
     'if (page < 0 || page >= num_pages)\n            continue;\n        page_tags[page] = page_tags[page] + 1u;',
     'if (page < 0 || page >= num_pages + 1)\n            continue;\n        if (page < num_pages) page_tags[page] = page_tags[page] + 1u;'),
]


def _source():
    with open(oracle._SRC) as f:
        return f.read()


def test_every_mutation_applies_to_the_current_source():
    src = _source()
    for name, old, _ in MUTATIONS:
        assert src.count(old) == 1, name


@pytest.mark.skipif(os.environ.get("PAFP8_MUTATION") != "1",
                    reason="several minutes: set PAFP8_MUTATION=1")
@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_the_mutation(name, old, new, tmp_path):
    mutant = tmp_path / "mutant.c"
    mutant.write_text(_source().replace(old, new, 1))
    lib = oracle.build(force=True, src=str(mutant), out=str(tmp_path / "mutant.so"))
    env = dict(os.environ, PAFP8_ORACLE_LIB=lib, PAFP8_MUTATION="0")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", "-k", "(oracle or inputs) and not mutation"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1800)
    # 1: some pin failed.  A negative code: the mutant corrupted the test
    # process's memory (mutated offsets can write past the pool) and it died
    # from a signal, which no correct oracle does.  0 would mean every pin
    # passed; other codes are usage errors.
    assert r.returncode == 1 or r.returncode < 0, (name, r.returncode, r.stdout[-1500:])
