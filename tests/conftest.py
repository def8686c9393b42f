import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly (not skip) when no GPU is present and they were
    # selected explicitly with -m gpu; in a plain CPU run they are skipped.
    markexpr = config.getoption("-m") or ""
    if "gpu" in markexpr and "not gpu" not in markexpr:
        return
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def read_band_fixture(name):
    """Return (num_layers, num_bands, [band per layer]) from a golden file."""
    path = os.path.join(GOLDEN, name)
    bands = []
    num_layers = num_bands = None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("# num_layers="):
                parts = dict(p.split("=") for p in line[2:].split())
                num_layers, num_bands = int(parts["num_layers"]), int(parts["num_bands"])
            elif line and not line.startswith("#"):
                l, b = map(int, line.split())
                assert l == len(bands)
                bands.append(b)
    assert num_layers == len(bands)
    return num_layers, num_bands, bands


BAND_FIXTURES = [
    "band_map_26_g4.txt", "band_map_26_g13.txt", "band_map_60_g6.txt",
    "band_map_4_g2.txt", "band_map_26_g26.txt", "band_map_26_g1.txt",
]
