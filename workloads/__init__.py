"""Seeded synthetic inputs for the TopK selector.

This package holds only input generation (random draws, bf16 rounding of the
drawn values, the ``-inf`` tail past a row's valid length).  It contains none
of the selection arithmetic, so both the CPU oracle and the GPU path can take
their inputs from it without sharing any of the method.
"""

from .synth import (  # noqa: F401
    ALIASES,
    CONFIGS,
    Config,
    K_DEFAULT,
    Workload,
    bf16_round,
    config,
    gen_row,
    generate,
    lengths_for,
    sha256_of,
)
from .indexer import (  # noqa: F401
    INDEXER_CONFIGS,
    IndexerConfig,
    IndexerWorkload,
    bf16_bits,
    draw,
    generate_indexer,
)
from .attention import (  # noqa: F401
    ATTENTION_CONFIGS,
    AttentionConfig,
    AttentionWorkload,
    draw_attention,
    generate_attention,
)
