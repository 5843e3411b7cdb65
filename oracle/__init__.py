"""CPU oracle for tree attention over a DFS-packed prefix tree.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything here.
The product path (``prefix_shared_masked_amd``) never imports it, and this
package imports nothing from the product path: the two share no code.

Everything is plain Python + NumPy in float64, written from the definitions
on the pages:

* ``plan``      -- DFS serialisation, depth positions, path counts g_t, K, the
                   DFS interval of every node, visible-key sets per query tile
                   (recursive DFS and parent-pointer walks).
* ``attention`` -- the tree-packed result obtained by running every
                   root-to-leaf path as its own causal sequence (and summing
                   the path gradients back), plus a dense-mask brute force.
* ``nll``       -- the g_t/K weighted negative log-likelihood and its gradient.
* ``decode``    -- single-query attention over a KV span list and the
                   (max, numerator, denominator) merge algebra.
* ``lmhead``    -- the output layer h W^T fused with the weighted NLL, in its
                   full form and in the chunk-and-recompute form.
* ``ssm``       -- tree-routed linear recurrence and causal-conv context, by
                   running every root-to-leaf path as its own sequence.

Parity status of each function is stated in its docstring; the pins live in
``tests/test_oracle_*.py``.
"""
from .plan import (oracle_plan, fwd_tile_keys, bwd_tiles, OraclePlan, dense_mask,  # noqa: F401
                   por, speedup_upper)
from .attention import (per_path_attention, dense_mask_attention, rope,  # noqa: F401
                        rope_transpose, rows_attention, rows_attention_grads,
                        causal_sequence_grads)
from .nll import weighted_nll, per_path_loss  # noqa: F401
from .ssm import tree_scan, tree_conv  # noqa: F401
from .lmhead import lmhead_weighted_nll, chunked_lmhead_weighted_nll, lmhead_vocab_rows  # noqa: F401
from .decode import (decode_attention, partial_triple, merge_triples,  # noqa: F401
                     finalize_triple, triple_from_lse, IDENTITY)
