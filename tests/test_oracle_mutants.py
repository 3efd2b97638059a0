"""Plant plausible mistakes in copies of the oracle (on the CPU) and require
that at least one pin catches each.  The real oracle source is never changed:
each mutant is a text substitution applied to a temporary copy."""
import os

import pytest

import oracle
import oracle_pins
from oracle import build as obuild

MUTANTS = [
    ("scale dropped", "u[j] = sc * acc;", "u[j] = acc;"),
    ("A indexed transposed", "abase + k * r_max + j", "abase + j * d_in + k"),
    ("B indexed transposed", "acc += u[j] * elem(B[s], dtype, bbase + (int64_t)j * w + n);",
     "acc += u[j] * elem(B[s], dtype, bbase + (int64_t)n * r_max + j);"),
    ("add flag ignored", "const double base = add ? yrow[off + n] : 0.0;\n                yrow[off + n] = base + acc;\n            }\n        }\n    }\n    free(u);",
     "const double base = yrow[off + n];\n                yrow[off + n] = base + acc;\n            }\n        }\n    }\n    free(u);"),
    ("slice offset dropped", "const int64_t w = width[s], off = offset[s];\n            if (slot < 0)",
     "const int64_t w = width[s], off = 0;\n            if (slot < 0)"),
    ("sign of delta", "yrow[off + n] = base + acc;\n            }\n        }\n    }\n    free(u);",
     "yrow[off + n] = base - acc;\n            }\n        }\n    }\n    free(u);"),
    ("slot off by one", "const int64_t abase = a_slot_stride[s] * slot;",
     "const int64_t abase = a_slot_stride[s] * (slot > 0 ? slot - 1 : slot);"),
    ("per-slot scale ignored", "scale * (slot_scale ? (double)slot_scale[slot] : 1.0)", "scale"),
    ("unstable order inside a key",
     "for (int64_t t = 0; t < T; ++t) {\n            if (effective_slot(token_slot[t], S) == key)",
     "for (int64_t t = T - 1; t >= 0; --t) {\n            if (effective_slot(token_slot[t], S) == key)"),
    ("no-adapter key placed with the top slot",
     "if (effective_slot(token_slot[t], S) == key) {",
     "if (effective_slot(token_slot[t], S) == (key == -1 ? S - 1 : (key == S - 1 ? -1 : key))) {"),
    ("start offsets off by one", "seg_start[nseg + 1] = seg_start[nseg] + count;",
     "seg_start[nseg + 1] = seg_start[nseg] + count - 1;"),
    ("no_lora flag wrong", "*no_lora = (with_adapter == 0) ? 1 : 0;", "*no_lora = (with_adapter <= 1) ? 1 : 0;"),
    ("bad ids kept", "return (id >= -1 && id < num_slots) ? id : -1;", "return id < num_slots ? id : -1;"),
    ("padding of unused starts", "seg_start[i] = (int32_t)T;", "seg_start[i] = 0;"),
    ("bf16 widened wrong", "<< 16;\n    float f;", "<< 15;\n    float f;"),
    ("expand alone ignores add", "const double base = add ? yrow[off + n] : 0.0;\n                yrow[off + n] = base + acc;\n            }\n        }\n    }\n    return ORACLE_OK;",
     "const double base = yrow[off + n];\n                yrow[off + n] = base + acc;\n            }\n        }\n    }\n    return ORACLE_OK;"),
    ("expand alone reads the wrong token", "const float *ut = u + ((int64_t)s * ldu + t) * r_max;",
     "const float *ut = u + ((int64_t)s * ldu + (t > 0 ? t - 1 : t)) * r_max;"),
    ("moe key strides slots by all experts", "key = slot * E_local + local;", "key = slot * E_global + local;"),
    ("moe expert map ignored", "local = expert_map[e];", "local = e < E_local ? e : -2;"),
    ("moe remote experts kept", "else if (slot == -1 || local == -1)", "else if (slot == -1)"),
    ("moe reads the wrong choice", "const int32_t e = topk_ids[t * topk + j];", "const int32_t e = topk_ids[t * topk];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib_path = obuild.build(str(mutated), str(tmp_path / "libmutant.so"))
    lib = oracle.load(lib_path)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake '{name}'"
