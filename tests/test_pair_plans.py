"""CPU checks of the code-pair plans the affine kernels use (pair_plans.h).

The plans are produced by csrc/gen_pair_plans.py.  Here they are simulated in
exact integer arithmetic: every 64-code group (or, for the piece plans, every
16-byte piece of 128/b codes) is rebuilt from the plan's bf16x2 operands and
compared with the oracle's unpack, and the factored dot product
sum(x' * (128 + 2^p q)) - 128 * sum(x') is checked to equal sum(x * q).  The
generated C++ is checked on the GPU by the bit-exact unpack and one-hot tests.
"""
import functools
import os
import sys
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "affine_quantized_gemv_amd", "csrc")
sys.path.insert(0, CSRC)
import gen_pair_plans  # noqa: E402

MAGIC = 0x43004300


# (bits, stream bits): one group of 64 codes for every width, and one 16-byte
# piece for the widths whose codes never straddle a piece
CASES = [(b, 64 * b) for b in range(2, 9)] + [(b, 128) for b in gen_pair_plans.PIECE_BITS]
IDS = ["group-q%d" % b for b in range(2, 9)] + ["piece-q%d" % b for b in gen_pair_plans.PIECE_BITS]


@functools.lru_cache(maxsize=None)
def plan(bits, nbits):
    return gen_pair_plans.plan(bits, nbits)


def test_committed_header_matches_generator(tmp_path):
    out = tmp_path / "pair_plans.h"
    gen_pair_plans.main(["gen", str(out)])
    assert out.read_text() == open(os.path.join(CSRC, "pair_plans.h")).read()


@pytest.mark.parametrize("bits,nbits", CASES, ids=IDS)
def test_plan_covers_every_code_bit_once(bits, nbits):
    p = plan(bits, nbits)
    ncodes = nbits // bits
    sw = p["sw"]
    cover = {}
    for pr in p["pairs"]:
        for k, g, pos in ((pr["kl"], pr["gl"], pr["pl"]), (pr["kh"], pr["gh"], pr["ph"])):
            assert 0 <= pos and pos + sw <= 7, "field must stay inside the 7-bit mantissa"
            for i in range(sw):
                key = (k, g + i)
                assert key not in cover
                cover[key] = True
    assert set(cover) == {(k, i) for k in range(ncodes) for i in range(bits)}


def _window(stream: int, st: int, nbits: int) -> int:
    full = stream & ((1 << nbits) - 1)
    v = (full << -st) if st < 0 else (full >> st)
    return v & 0xFFFFFFFF


@pytest.mark.parametrize("bits,nbits", CASES, ids=IDS)
def test_plan_simulation_rebuilds_codes_and_dot_products(bits, nbits):
    p = plan(bits, nbits)
    sw = p["sw"]
    ncodes = nbits // bits
    fm = (1 << sw) - 1
    # whole groups from the generator; a piece plan is checked on every piece
    # of them (the oracle unpacks the group, the plan one piece at a time)
    words = synth.random_words((6, 2 * bits), 60, "plan/%d" % bits)
    codes = oracle.unpack(words, bits, 64)
    g = synth.rng(60, "planx/%d/%d" % (bits, nbits))
    nw = nbits // 32
    for row, piece in [(r, q) for r in range(words.shape[0]) for q in range(2 * bits // nw)]:
        stream = sum(int(w) << (32 * i) for i, w in enumerate(words[row, nw * piece:nw * piece + nw]))
        want = [int(c) for c in codes[row, ncodes * piece:ncodes * piece + ncodes]]
        rebuilt = [0] * ncodes
        x = [int(v) for v in g.integers(-9, 10, size=ncodes)]
        dot = Fraction(0)
        xsum = Fraction(0)
        for pr in p["pairs"]:
            wl = _window(stream, pr["sl"], nbits)
            wh = _window(stream, pr["sh"], nbits)
            op = ((wl & pr["ml"]) | (wh & pr["mh"])) | MAGIC
            lo, hi = op & 0xFFFF, op >> 16
            assert lo & 0xFF80 == 0x4300 and hi & 0xFF80 == 0x4300
            ql, qh = (lo >> pr["pl"]) & fm, (hi >> pr["ph"]) & fm
            rebuilt[pr["kl"]] |= ql << pr["gl"]
            rebuilt[pr["kh"]] |= qh << pr["gh"]
            # bf16 values 128 + (field << p) times activations scaled by 2^e
            xl = Fraction(x[pr["kl"]]) * Fraction(2) ** (pr["gl"] - pr["pl"])
            xh = Fraction(x[pr["kh"]]) * Fraction(2) ** (pr["gh"] - pr["ph"])
            dot += xl * (128 + (lo & 0x7F)) + xh * (128 + (hi & 0x7F))
            xsum += xl + xh
        assert rebuilt == want
        assert dot - 128 * xsum == sum(x[k] * want[k] for k in range(ncodes))
