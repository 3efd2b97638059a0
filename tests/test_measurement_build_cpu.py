"""The measurement build (-DLORA_PHASE_CLOCK), which bench.py's --phase-budget
and --tile-phase-budget compile on the GPU host, still compiles for gfx950 and
exports its phase-buffer entry point (CPU only: hipcc cross-compiles)."""
import ctypes
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_measurement_build_compiles(tmp_path):
    spec = importlib.util.spec_from_file_location(
        "_lora_hip_build", os.path.join(ROOT, "segmented_gather_rank_amd", "build.py"))
    hb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(hb)
    out = hb.build(out=str(tmp_path / "liblora_mi355x_phase.so"), extra=["-DLORA_PHASE_CLOCK"])
    lib = ctypes.CDLL(out)
    assert hasattr(lib, "lora_debug_phase_clock")
    assert hasattr(lib, "lora_apply") and lib.lora_abi_version() > 0
