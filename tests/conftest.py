import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload; takes tens of seconds")
    # every feature-gradient call in the tests reads back its status word
    # (a turn wait that gave up raises instead of leaving a wrong dh)
    from group_shared_fixed_amd import binding
    binding.CHECK_DH_STATUS = True
