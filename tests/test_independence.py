"""The oracle and the HIP path share nothing; the input generator holds no method code."""

import ast
import os

import numpy as np

from conftest import ROOT
import workloads


def _imports(path):
    names = set()
    for dirpath, _, files in os.walk(path):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(dirpath, f)).read())
            for node in ast.walk(tree):
                if isinstance(node, ast.Import):
                    names.update(a.name.split(".")[0] for a in node.names)
                elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
                    names.add(node.module.split(".")[0])
    return names


def test_oracle_imports_no_product_code():
    used = _imports(os.path.join(ROOT, "oracle"))
    assert "paged_kv_cache_293_amd" not in used
    assert "workloads" not in used
    assert used <= {"numpy", "math", "fractions", "collections"}


def test_product_imports_no_oracle():
    pkg = os.path.join(ROOT, "paged_kv_cache_293_amd")
    if os.path.isdir(pkg):
        used = _imports(pkg)
        assert "oracle" not in used and "workloads" not in used
        for dirpath, _, files in os.walk(pkg):
            for f in files:
                if f.endswith((".hip", ".cpp", ".h", ".hpp")):
                    for line in open(os.path.join(dirpath, f)):
                        if line.lstrip().startswith("#include"):
                            assert "oracle" not in line and "workloads" not in line


def test_generator_imports_neither_side():
    used = _imports(os.path.join(ROOT, "workloads"))
    assert "oracle" not in used and "paged_kv_cache_293_amd" not in used


def test_generator_is_deterministic_and_seeded_per_config():
    a, b = workloads.make("c2s"), workloads.make("c2s")
    for name in ("seq_lens", "block_tables", "q", "k_new", "v_new", "k_pre", "v_pre"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    c = workloads.make("c3s")
    assert a.seed != c.seed


def test_generator_shapes_follow_the_configs():
    c1 = workloads.make("c1")
    assert c1.seq_lens.tolist() == [17, 100, 250, 513] and c1.num_blocks == 128
    assert (c1.num_q_heads, c1.num_kv_heads, c1.head_dim, c1.kv_dtype) == (8, 2, 64, "f32")
    c2 = workloads.make("c2", materialize=False)
    assert c2.batch == 64 and c2.seq_lens.min() >= 512 and c2.seq_lens.max() <= 4096
    assert c2.num_blocks == -(-int(1.25 * 1e6 * c2.info["blocks_used"]) // 1000000)
    c4 = workloads.make("c4", materialize=False)
    assert c4.max_blocks == 8192 and (c4.seq_lens == 131072).all()
    c5 = workloads.make("c5", materialize=False)
    assert c5.k_rows == 5 and c5.batch == 128
    assert (c5.block_tables[:, :128] == c5.block_tables[0, :128]).all()
    suffix = c5.seq_lens - 2048 - 5
    assert suffix.min() >= 64 and suffix.max() <= 1024
    c3 = workloads.make("c3", materialize=False)
    assert ((c3.seq_lens >= 4096).sum(), (c3.seq_lens <= 1024).sum()) == (77, 179)
    # every table is a placement: used entries distinct across sequences
    for w in (c1, c2, c4):
        used = np.concatenate([w.block_tables[s, :-(-int(n) // 16)] for s, n in enumerate(w.seq_lens)])
        assert len(np.unique(used)) == len(used) and used.min() >= 0 and used.max() < w.num_blocks
