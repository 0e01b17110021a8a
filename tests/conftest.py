import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_codebooks():
    """Small fp16 codebooks fit by the oracle's k-means on seeded randn data
    (n = 2^14 samples, 10 Lloyd iterations): {bits: uint16 bits [256, s]}."""
    import oracle
    from kv_cache_bit_amd import synth
    out = {}
    for bits, s in ((2, 4), (1, 8)):
        x = synth.randn_samples(seed=bits, n=1 << 14, s=s).numpy()
        _, cb, _ = oracle.kmeans(x, 256, 10)
        out[bits] = cb
    return out
