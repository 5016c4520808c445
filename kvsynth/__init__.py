"""Seeded synthetic inputs for the KV-relocation workloads.

Shared by the tests, the benchmark and the smoke check.  This module only
*draws*: shapes, integer parameters (directives, chunk placements, block
tables, pending shifts) and random cache contents.  It contains none of the
relocation arithmetic (no rotation, no splice or gather index maps); those live
in the HIP library and, independently, in the oracle.

Every stream comes from ``numpy.random.default_rng([BASE_SEED, *keys])`` so any
slab can be regenerated from its keys.  Device-sized contents are drawn on the
GPU with torch's seeded generator instead (see ``fill_normal_``).
"""

from .workloads import (  # noqa: F401
    BASE_SEED, rng, bf16_normal, f32_normal, fill_normal_, normal_range_,
    MLA, GQA, SpliceWorkload, GatherWorkload, PatchWorkload, DecodeWorkload, GqaDecodeWorkload,
    KeyingWorkload, single_splice, batched_splice, registry_gather, gqa_patch, rotate_on_read_decode,
    gqa_rotate_on_read_decode, registry_streams, PatchFormationWorkload, patch_formation, deficit_batch_,
)
