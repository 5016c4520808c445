"""Plain, slow CPU oracle for KV-row relocation by closed-form RoPE rotation.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library under ``rope_rotation_splice_amd/`` and imports nothing from it.

Everything is computed in float64 with numpy (mpmath appears only in tests, as
an independent pin).  Each function cites the passage of the source pages that
defines what it computes.  The pages are three technical summaries published on
gist.science; citations use these short names:

* **Leyline** -- "Leyline : Directives de Cache KV pour l'Inférence Agentique"
  (French summary, gist.science/fr/paper/2606.01065; the Portuguese summary at
  gist.science/pt/paper/2606.01065 is a translation with the same sections).
* **Kamera** -- "Kamera : Un KV Cache Multimodal Unifié et Invariant à la
  Position pour la Réutilisation sans Réentraînement"
  (gist.science/fr/paper/2606.23581).
* **Irminsul** -- "Irminsul: Cache Independente de Posição Nativo para MLA para
  Atendimento de LLMs Agentes" (gist.science/pt/paper/2605.05696).

Readings taken where the pages are silent (RoPE pairing and frequencies,
half-open ranges, rounding, patch frame, ...) are stated in each module's
docstring.

Parity status per function (what pins it, in ``tests/test_oracle_*.py``):

* ``rope``      -- pinned: mpmath angles, complex-exponential RoPE, closure,
                   inverse, norm, plane-rotation special case.
* ``bf16``      -- pinned: torch's float32->bfloat16 conversion, all 65536 codes.
* ``splice``    -- pinned: brute-force index maps against list slicing; golden
                   figures of the single-sequence splice workload.
* ``gather``    -- pinned: brute-force paged maps, O(n^2) overlap check.
* ``patch``     -- pinned: textbook GEMM on asymmetric shapes; memory fractions.
* ``lazy``      -- pinned: slot map equal to the eager splice's, block
                   conservation, one-rotation composition; the block-table
                   gather against each entry row's landing slot and owed shift,
                   and against decoding the eagerly relocated rows.
* ``decode``    -- pinned: textbook softmax attention on explicitly rotated keys,
                   needle retrieval, brute-force per-key loop on tiny inputs;
                   the GQA form against torch's scaled_dot_product_attention on
                   independently rotated keys, a needle, and a grouping mutant.
* ``keying``    -- pinned: xxHash64 against the xxhash library and its published
                   empty-input value, the Gear recurrence against its window
                   sum, the cut rule by brute force, content alignment.
* ``svd``       -- pinned: exact recovery of planted rank-m deficits,
                   Eckart-Young, a pure-Python power iteration for the leading
                   triplet, a transposed-factor mutant, the orbit mean.
* FORGET mode   -- status and truncated length only; parity unpinned beyond that
                   (truly forgetting needs a model re-prefill).
* patch frame   -- the patch is added after rotation, in the target frame, as the
                   reuse operator is written; parity unpinned beyond that formula.
"""

from . import bf16, rope, splice, gather, patch, decode, lazy, keying, svd, tolerance  # noqa: F401
