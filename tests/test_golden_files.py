"""The stored oracle outputs (tests/golden/oracle_*.npz, written by
make_oracle_golden.py) still match the seeded inputs and the live oracle: the
input digests are recomputed, and sampled rows of every stored array are
recomputed with the oracle on the CPU."""
import numpy as np
import pytest

import oracle
import synth
from tests.golden.make_oracle_golden import INT8_LOGIT_ROWS, LOGPROB_ROWS, digest, path_of, \
    row_digests

pytestmark = pytest.mark.slow


def load(name):
    with np.load(path_of(name), allow_pickle=False) as f:
        return {k: f[k] for k in f.files}


@pytest.fixture(scope="module")
def o():
    return oracle.default()


def test_int8_file(o):
    d = synth.make_inputs("int8")
    g = load("int8")
    assert str(g["inputs"]) == digest(d["x"], d["w"], d["scale"], d["target"], d["hidden"])
    assert np.array_equal(g["logit_rows"], INT8_LOGIT_ROWS)
    rows = np.array([0, 255, 511])
    ids, raw, vals, margin = o.greedy_i8(d["x"][rows], d["w"], d["scale"][rows])
    assert np.array_equal(ids, g["ids"][rows]) and np.array_equal(raw, g["raw"][rows])
    assert np.array_equal(vals.view(np.int32), g["vals"][rows].view(np.int32))
    assert np.array_equal(margin.view(np.int32), g["margin"][rows].view(np.int32))
    lp = o.logprob_i8(d["x"][rows], d["w"], d["target"][rows], d["scale"][rows])
    assert np.array_equal(lp, g["logprob"][rows])
    lr = INT8_LOGIT_ROWS[[0, -1]]
    assert list(row_digests(o.logits_i8(d["x"][lr], d["w"]))) == list(g["logit_digests"][[0, -1]])
    q, M, E = o.quantize_rows(d["hidden"][rows])
    assert list(row_digests(q.astype(np.int32))) == list(g["q_digests"][rows])
    assert np.array_equal(M, g["step_m"][rows]) and np.array_equal(E, g["step_e"][rows])
    lq = o.logprob_int(q, d["w"], *d["unit"], M, E, d["target"][rows])
    assert np.array_equal(lq, g["logprob_q"][rows])


def test_logprob_file(o):
    d = synth.make_inputs("logprob")
    g = load("logprob")
    assert str(g["inputs"]) == digest(d["x"], d["w"], d["target"])
    assert np.array_equal(g["rows"], LOGPROB_ROWS)
    pick = [0, len(LOGPROB_ROWS) - 1]
    rows = LOGPROB_ROWS[pick]
    lp = o.logprob_bf16(d["x"][rows], d["w"], d["target"][rows])
    assert np.array_equal(lp, g["logprob"][pick])


def test_neartie_file(o):
    d = synth.make_inputs("neartie")
    g = load("neartie")
    assert str(g["inputs"]) == digest(d["x"], d["w"])
    rows = np.array([0, 2047, 4095])
    for rnd, sfx in ((False, ""), (True, "16")):
        ids, vals, margin = o.greedy_bf16(d["x"][rows], d["w"], round_bf16=rnd)
        assert np.array_equal(ids, g["ids" + sfx][rows])
        assert np.array_equal(vals, g["vals" + sfx][rows])
        assert np.array_equal(margin, g["margin" + sfx][rows])
