"""The stored format against the figures the pages print (tests/golden/pages_format.txt).

The oracle's double-quantised records are read back field by field, at
d = 128 and R = the pages' default residual size: every 4-bit code is below
16, the mean has one (S, Z) pair per 32 channels and s1 one per block of R
tokens, and N2 stays fp16.  The bits they hold per element then come to the
pages' figure of roughly 0.23 (0.238 here: each group keeps a zero next to its
step), so the effective width is 2.23 / 1.23 bits.  The records are padded to
16 bytes in memory (0.25 bits at R = 64), which the pages' figure does not
count.
"""
import os

import numpy as np
import pytest

import oracle
from kv_cache_bit_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_format.txt")


def _golden() -> dict:
    out = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, rest = line.split("=", 1)
        value, cite = rest.split(";", 1)
        assert cite.strip(), f"{key} has no citation"
        out[key.strip()] = value.strip()
    return out


def test_golden_file_is_cited_and_complete():
    g = _golden()
    for key in ("nsn_overhead_bits", "effective_bits_2bit", "effective_bits_1bit", "dq_code_bits",
                "dq_mean_group", "dq_s1_group", "residual_default"):
        assert key in g


@pytest.mark.parametrize("bits", [2, 1])
def test_dq_records_match_printed_format(oracle_codebooks, bits):
    g = _golden()
    R, D = int(g["residual_default"]), 128  # the s1 group and mean block are the residual size
    group, cbits = int(g["dq_mean_group"]), int(g["dq_code_bits"])
    assert g["dq_s1_group"] == "R"
    L = 4 * R + 3
    x = synth.kv_unit(71 + bits, L, D).numpy()
    enc = oracle.encode(x[None], R, oracle_codebooks[bits], dq=True)
    nb = enc["n_quant"] // R
    sc = enc["scales"][0].reshape(nb, -1)
    mu = enc["mu"][0].reshape(nb, -1)
    # scales record: N2 fp16 per token, then one 4-bit s1 code per token, then
    # a single (S1, Z1) fp16 pair for the block (the s1 group is the block)
    s1 = sc[:, 2 * R:2 * R + R // 2]
    s1_codes = np.stack([s1 & 15, s1 >> 4], -1).reshape(nb, R)
    assert s1_codes.max() < 2 ** cbits
    sz1 = sc[:, 2 * R + R // 2:2 * R + R // 2 + 4].copy().view(np.float16)
    assert np.all(np.isfinite(sz1.astype(np.float64))) and np.all(sc[:, 2 * R + R // 2 + 4:] == 0)
    # mean record: one 4-bit code per channel, then (S, Z) fp16 per group of channels
    codes = np.stack([mu[:, :D // 2] & 15, mu[:, :D // 2] >> 4], -1).reshape(nb, D)
    assert codes.max() < 2 ** cbits
    pairs = mu[:, D // 2:].copy().view(np.float16).reshape(nb, -1, 2)
    assert pairs.shape[1] == D // group
    # the groups really are 32 channels: each group's codes span its own range
    # (some channel at level 0 and one at level 15 in every group of a block
    # whose means are not constant)
    g_codes = codes.reshape(nb, D // group, group)
    assert np.all(g_codes.min(-1) == 0) and np.all(g_codes.max(-1) == 2 ** cbits - 1)
    # bits per element the records hold: N2 (16) and s1 (4) per token, the
    # s1 pair once per block, the mean codes (4) and pairs per block
    held = 16 * R + cbits * R + 32 + cbits * D + 32 * (D // group)
    over = held / (R * D)
    assert over == pytest.approx(float(g["nsn_overhead_bits"]), abs=0.01)
    eff = float(g[f"effective_bits_{bits}bit"])
    assert bits + over == pytest.approx(eff, abs=0.01)
    # and the padded records as stored
    stored = 8 * (sc.shape[1] + mu.shape[1]) / (R * D)
    assert stored == pytest.approx(0.25, abs=1e-12) and stored >= over
