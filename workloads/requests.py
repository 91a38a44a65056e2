"""Seeded synthetic request streams for the multi-step decode loop.

A request is a prompt (token ids) plus the number of tokens to generate. The prompt lengths follow the mixed
workload of the pages' evaluation (page 1 section 2.1: short prompts under 500 tokens and long ones of 1k-4k,
mixed), a fraction of the prompts open with one common system prompt (page 2 section 4.3: shared prefixes such
as system prompts are where sharing saves most), and a few requests ask for two continuations of the same
prompt (parallel sampling: the second one starts as a fork of the first, page 1 section 3.2). Nothing here
computes attention or touches a cache.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class Request:
    prompt: np.ndarray  # int32 token ids
    max_new_tokens: int
    parallel: int  # continuations of this prompt: 1, or 2 for parallel sampling


def request_stream(seed: int, *, system_prompt_len: int = 1024, shared_fraction: float = 0.3,
                   short=(32, 500), long=(1024, 4096), long_fraction: float = 0.3, new_tokens=(32, 256),
                   parallel_fraction: float = 0.05, vocab: int = 32000):
    """Endless generator of requests drawn from numpy's PCG64 with the given seed."""
    rng = np.random.default_rng(seed)
    system = rng.integers(0, vocab, size=system_prompt_len).astype(np.int32)
    while True:
        lo, hi = long if rng.random() < long_fraction else short
        n = int(rng.integers(lo, hi, endpoint=True))
        if rng.random() < shared_fraction and n > system_prompt_len:
            prompt = np.concatenate([system, rng.integers(0, vocab, size=n - system_prompt_len).astype(np.int32)])
        else:
            prompt = rng.integers(0, vocab, size=n).astype(np.int32)
        yield Request(prompt=prompt, max_new_tokens=int(rng.integers(new_tokens[0], new_tokens[1], endpoint=True)),
                      parallel=2 if rng.random() < parallel_fraction else 1)
