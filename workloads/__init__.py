"""Seeded synthetic inputs for paged decode attention.

This package only draws inputs: context lengths, block tables, slot mappings, copy pairs and the random
query / key / value tensors. It holds none of the attention or cache-update arithmetic, so the CPU oracle
and the HIP library can both consume it without sharing any of the method's code.
"""

from .decode import (  # noqa: F401
    CONFIG_NAMES,
    EXTRA_NAMES,
    DecodeStructure,
    build_structure,
    custom_structure,
    live_slot_mask,
    materialize,
    algorithmic_bytes,
    query_rows,
)
from .requests import Request, request_stream  # noqa: F401,E402
