"""Seeded synthetic inputs for head-aware SegPaged attention.

This package only draws numbers. It holds none of the method's arithmetic (no visibility
rule, no page or segment logic, no softmax): the CPU oracle under ``oracle/`` and the HIP
path both read the same seeded arrays from here, and nothing else is shared between them.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    GLOBAL,
    LOCAL,
    LOCAL_ADAPTIVE,
    RETRIEVAL,
    Case,
    config_case,
    custom_case,
    decode_tokens,
    free_list,
    importance_scores,
)
