"""The generated figure tables of the repository's documents are exactly
what `python bench.py --write-tables` renders from the committed result files
(results/*.json) and the committed counter summary: no table is typed by hand
or left stale ("batch-logprob-gap", "Tables": every reported number comes from
a result file)."""
import importlib.util
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
BLOCK = re.compile(r"<!-- generated:(\w+) -->\n(.*?)\n?<!-- /generated:\1 -->", re.S)


@pytest.fixture(scope="module")
def tables():
    spec = importlib.util.spec_from_file_location("bench_tables", ROOT / "bench.py")
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    t = bench.render_tables(ROOT / "results")
    t.update(bench.render_counter_table(ROOT / "profiles" / "counters_greedy_tinyllama_b512.md"))
    return t


@pytest.fixture(scope="module")
def docs():
    spec = importlib.util.spec_from_file_location("bench_docs", ROOT / "bench.py")
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    return bench.DOCS


@pytest.mark.parametrize("i", [0, 1])
def test_generated_blocks_match_results(tables, docs, i):
    doc = docs[i]
    blocks = BLOCK.findall(doc.read_text())
    assert blocks, f"{doc} has no generated tables"
    for name, body in blocks:
        assert name in tables, f"{doc}: no renderer for table {name!r}"
        assert body.strip() == tables[name].strip(), \
            f"{doc}: table {name!r} differs from the result files (run python bench.py --write-tables)"
