"""Host-side harness logic of the workloads (no GPU): the sampler's row list
and the structure of the logits workload."""
import numpy as np

import workloads as W


def test_sampler_rows_are_last_rows():
    # requests of lengths 1, 3, 1, 5 occupy rows 0 | 1-3 | 4 | 5-9 of the step
    assert list(W.sampler_rows([1, 3, 1, 5])) == [0, 3, 4, 9]
    assert list(W.sampler_rows([1, 1, 1])) == [0, 1, 2]
    assert W.sampler_rows([]).shape == (0,)


def test_logits_workload_structure():
    c = W.config(6)
    lengths = c.notes["step_lengths"]
    rows = c.notes["sampled_token_rows"]
    assert c.T == lengths.shape[0] == rows.shape[0] == 200
    assert np.all(np.diff(rows) > 0) and rows[-1] == lengths.sum() - 1
    assert int(np.sum(c.token_slot < 0)) == 10
    assert c.widths == [76800] and c.B[0].shape == (8, 16, 76800)
