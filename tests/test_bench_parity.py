"""The benchmark's parity record (its CPU leg compares the timed step's
outputs on a row sample with the oracle): exact outputs give zero errors,
a perturbed output and a changed selection are reported."""
import numpy as np

import bench
import oracle


def test_parity_record_reports_errors_and_selection_changes():
    name, budget = "prefill_2k", 64
    Tq, pos0, _, _ = bench.WORKLOADS[name]
    x = bench.gen_prefill(name)
    Kr = oracle.rope(x.K)
    kb = oracle.compress(x.ki)
    rows = np.array([0, 1, 2, 3, 700, 1500, Tq - 1], dtype=np.int64)
    pos = pos0 + rows
    ref = oracle.qsa_rows_at(oracle.rope(x.Q[rows], pos=pos), Kr, x.V, x.qi[rows], kb, pos,
                             Kbudget=budget)
    gpu = dict(rows=rows, O=ref["O"].astype(np.float32), lse=ref["lse"].astype(np.float32),
               sel=ref["sel"].copy(), nsel=ref["nsel"].copy())
    rec = bench.parity_record(oracle, name, x, Kr, kb, budget, gpu)
    assert rec["rows"] == rows.size and rec["selection_equal_rows"] == rows.size
    a = rec["attention_on_gpu_selection"]
    assert a["O_max_abs"] < 1e-6 and a["lse_max_abs"] < 1e-5 and rec["within_bar"]
    # a perturbed output row passes the bar no longer
    bad = dict(gpu, O=gpu["O"].copy())
    bad["O"][4, 3, 7] += 0.5
    rec = bench.parity_record(oracle, name, x, Kr, kb, budget, bad)
    assert abs(rec["attention_on_gpu_selection"]["O_max_abs"] - 0.5) < 1e-3
    assert not rec["within_bar"]
    # a row whose selection differs leaves the end-to-end set; the attention
    # is still checked on the GPU's own selection
    i = 6   # the last row: a full budget of 64 out of 511 complete blocks
    assert ref["nsel"][i] == budget
    other = dict(gpu, sel=gpu["sel"].copy())
    chosen = set(other["sel"][i, :budget].tolist())
    repl = next(b for b in range(511) if b not in chosen)
    other["sel"][i, budget - 1] = repl
    other["sel"][i, :budget] = np.sort(other["sel"][i, :budget])
    rec = bench.parity_record(oracle, name, x, Kr, kb, budget, other)
    assert rec["selection_equal_rows"] == rows.size - 1
    assert rec["selection_differing_rows"] == 1
    assert not rec["within_bar"]   # the outputs were computed over the oracle's selection
