"""Every helper the GPU tests call on the GPU harness exists (the GPU tests
themselves only run where a GPU is present, so a missing name would
otherwise show first on the GPU)."""
import glob
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))


def test_gpu_tests_use_existing_harness_names():
    import gpu_harness as gh

    used = set()
    for f in glob.glob(os.path.join(HERE, "test_*.py")):
        used |= set(re.findall(r"\bgh\.(\w+)", open(f).read()))
    assert used, "no harness use found"
    missing = sorted(u for u in used if not hasattr(gh, u))
    assert not missing, missing
