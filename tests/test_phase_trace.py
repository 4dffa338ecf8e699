"""The phase-trace probe (tests/probes/phase_trace.py) generates its traced
copy of csrc/pa_decode.hip by text substitution: every anchor it patches must
still occur exactly once in the decode source, and the copy must carry one
stamp per phase boundary and the host's trace switch."""
import importlib.util
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def _probe():
    spec = importlib.util.spec_from_file_location("phase_trace", os.path.join(HERE, "probes", "phase_trace.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_phase_trace_anchors_match_the_decode_source():
    pt = _probe()
    src = pt.patched_source()   # raises if an anchor moved or repeats
    # stamps 0-6, stamp 6 at each of the three ends of the single-token path
    assert src.count("__builtin_amdgcn_s_memrealtime()") == 9
    for i in range(7):
        assert f"* {pt.SLOTS} + {i}] = __builtin_amdgcn_s_memrealtime();" in src
    assert f"* {pt.SLOTS} + 7] = m;" in src
    assert 'extern "C" void pa_debug_set_trace(void* p)' in src
    assert "prm.trace = g_trace;" in src
