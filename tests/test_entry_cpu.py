"""The driver-facing entry module: it must import and expose build() and
smoke() as plain callables taking no arguments."""
import importlib
import inspect
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_graft_entry_exposes_build_and_smoke():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    mod = importlib.import_module("__graft_entry__")
    for name in ("build", "smoke"):
        fn = getattr(mod, name, None)
        assert callable(fn), f"__graft_entry__.{name} missing"
        sig = inspect.signature(fn)
        assert all(p.default is not inspect.Parameter.empty for p in sig.parameters.values()), \
            f"__graft_entry__.{name} must be callable without arguments"


def test_build_lists_every_translation_unit():
    """Every .hip translation unit under csrc/ is compiled by build()."""
    from delta_rule_rnn_amd import build
    hips = sorted(f for f in os.listdir(build.CSRC) if f.endswith(".hip"))
    assert hips and set(hips) <= set(build.SOURCES), set(hips) - set(build.SOURCES)
