"""Driver run by tests/test_planner_sanitized.py in a child process whose
loader preloads the sanitizer runtimes: the binding loads the planner-only
build (address + undefined-behaviour sanitizers, host code only) and the
existing planner, partition and routing comparisons run through it on the
fixed trees of those tests and on seeded random forests.  Any sanitizer
report aborts the process (halt on the first error)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path[:0] = [ROOT, os.path.join(ROOT, "tests")]
os.environ["TA_HOST_ONLY_LIBRARY"] = "1"

import numpy as np  # noqa: E402

import prefix_shared_masked_amd as pkg  # noqa: E402

pkg._LIB_PATH = sys.argv[1]
n_random = int(sys.argv[2])
import workloads as W  # noqa: E402
import test_plan_native as tp  # noqa: E402
import test_partition_native as tpart  # noqa: E402
import test_route_native as troute  # noqa: E402

pkg.load_library()
fixed = [W.six_node_tree(16), W.spine_tree(),
         W.Tree(np.array([-1] + [0] * 64, np.int32), np.array([5] + [3] * 64, np.int32), "star64"),
         W.Tree(np.arange(-1, 199, dtype=np.int32), np.full(200, 7, np.int32), "chain200"),
         W.Tree(np.array([-1, 0, 1, 1, 0], np.int32), np.array([0, 0, 33, 0, 31], np.int32), "zeros")]
for t in fixed:
    tp.compare(t)
    troute.check(t, 4)
print(f"fixed trees ok: {len(fixed)}", flush=True)
for name in ("test_node_lengths_around_tile_edges", "test_cut_key_tiles", "test_star_with_64_children_and_deep_chain",
             "test_determinism", "test_error_codes", "test_zero_token_nodes_only_between"):
    getattr(tp, name)()
for name in ("test_whole_tree_fits_one_partition_per_root", "test_spine_tree_counts", "test_cut_rule_on_small_examples",
             "test_zero_token_partition_has_no_plan", "test_errors", "test_prefix_plan_validation"):
    getattr(tpart, name)()
troute.test_errors()
print("planner, partition and routing tests ok", flush=True)
rng = np.random.default_rng(20261202)
shapes = ["random", "chain", "star"]
for i in range(n_random):
    n = int(rng.integers(1, 17))
    t = W.random_tree(rng, n, max_len=int(rng.integers(1, 48)), p_zero=float(rng.choice([0.0, 0.1, 0.4])),
                      n_roots=int(rng.integers(1, 5)), shape=shapes[i % 3])
    tp.compare(t)
    if i % 10 == 0:
        lens = t.seg_len[t.seg_len > 0]
        cap = int(max(lens.max() if lens.size else 1, rng.integers(1, 200)))
        tpart.check_partition(t, cap)
    if i % 10 == 5:
        troute.check(t, int(rng.integers(1, 9)))
print(f"random forests ok: {n_random}", flush=True)
