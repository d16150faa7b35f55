"""Seeded synthetic inputs for verification attention over a draft tree.

This module only draws numbers and tree shapes. It holds none of the
attention arithmetic, so both the CPU oracle (``oracle/``) and the GPU path
(tests, ``bench.py``) may use it without sharing any of the method's code.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    Workload,
    WorkloadConfig,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_custom,
    make_workload,
    tree_bounded,
    tree_chain,
    tree_depths,
    tree_star,
    tree_uniform,
)
from .accept_gen import AcceptCase, make_accept_case  # noqa: F401,E402
from .draft_gen import WindowCase, make_window_case  # noqa: F401,E402
from .tree_gen import TreeCase, make_tree_case  # noqa: F401,E402
