"""Seeded synthetic inputs for the paged KV workloads.

This module is shared by the product's tests/bench and by the CPU oracle, so
it holds none of the method's arithmetic: no slots, block tables, allocation,
sharing plans or attention.  It only draws random numbers and lays them out:

* page placement (a permutation handed to the allocator as its free order),
* sequence lengths, token ids and draft-acceptance counts,
* Q/K/V values ~ N(0, 1), drawn in float32 and, for bf16 workloads, rounded
  to bfloat16 with round-to-nearest-even and kept as raw uint16 bit patterns.

Every stream comes from ``numpy.random.default_rng(SeedSequence(seed,
spawn_key=(workload, stream, instance)))`` so each quantity is reproducible on
its own.
"""

from .gen import (  # noqa: F401
    BF16,
    F32,
    DecodeBatch,
    PrefixTraces,
    RewindDocs,
    SpecDecode,
    TinyBatch,
    bf16_bits_to_f32,
    decode_batch,
    f32_to_bf16_bits,
    generator,
    normal_values,
    prefix_traces,
    rewind_docs,
    spec_decode,
    tiny_batch,
    to_f64,
)
