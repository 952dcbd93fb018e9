"""Plain, slow fp64 CPU oracle for the Bi-Level Routing Attention (BRA) forward pass.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it. It shares no code with the HIP path
(``vision_transformer_dynamic_amd``), and neither side imports the other.

Modules
-------
``bra_oracle``  the method, step by step, in float64 numpy (pool, affinity,
                top-k routing, gather, naive softmax attention).
``brute``       independent brute-force formulations used only to pin
                ``bra_oracle`` (pairwise token affinity, dense global
                attention, window attention by reshaping).

Every function in ``bra_oracle`` is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py``; see the header of ``bra_oracle`` for the list.
"""

from .bra_oracle import (  # noqa: F401
    check_config,
    region_size,
    region_token_coords,
    region_mean,
    affinity,
    topk_route,
    route,
    gather_coords,
    softmax_attention,
    attend,
    bra,
    attended_tokens,
)
