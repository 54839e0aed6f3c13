import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")
    # A fresh checkout has no built library (built files stay out of the
    # history): build it once, in-tree. An existing build is used as it is.
    from moe_token_dispatch_amd import build as libbuild

    if not os.path.exists(libbuild.LIB_PATH):
        libbuild.build()
