"""Run CPU test files against sanitizer builds (used by test_sanitize_cpu.py).

    python sanitize_runner.py oracle <liboracle built with ASan/UBSan> <test files..>
    python sanitize_runner.py abi <libdp built with host ASan/UBSan> <test files..>

The process is started with the sanitizer runtime preloaded; this script
points the oracle or the binding at the instrumented library before anything
loads it, then runs pytest on the named files (CPU tests only).
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
sys.path.insert(0, HERE)

import pytest  # noqa: E402

which, lib, files = sys.argv[1], sys.argv[2], sys.argv[3:]
if which == "oracle":
    import oracle.build as ob
    ob.LIB = lib
else:
    from linear_rnn_sequence_amd import binding
    binding.LIB_PATH = lib
sys.exit(pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *files]))
