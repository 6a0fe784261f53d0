"""CPU oracle for paged KV storage and paged attention.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
statement of what the paged hot path computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product library (``pagedattention_pkv_store_amd``) never
imports, calls or links anything here, and this package imports nothing from
the product: the two share no kernels, headers, helpers, tables or constants.
The only code both sides use is the seeded input generator in ``synth/``,
which holds none of the method's arithmetic.

Everything is Python + NumPy.  Attention is computed in float64.

Modules
-------
paging      block-table / slot model and the reference page allocator
            (KV cache docs of TileInfer.jl, "Pages and block tables" and
            "Growing, rolling back, releasing"; "KV Cache Management and
            PagedAttention", Figures 1-3 and 6, "Return blocks after a request
            ends"; Quail docs "KV", "Paged KV").
planner     the sorted-adjacent-document prefix-sharing plan (Quail docs "KV",
            "The sharing plan").
attention   softmax attention over a sequence's logical K/V, gathered through
            the block table ("KV Cache Management and PagedAttention",
            "Compute attention over scattered KV", Figure 4).
retention   the KV retention pool: priority = probability_of_reuse *
            recompute_seconds / pages, lowest evicted first (Quail docs "KV",
            "KV retention").
quant       INT8 KV pages: per-vector symmetric codes and fp32 scales, and
            attention over them (TileInfer.jl "KV cache", "INT8 cache").
codec       group-wise Q8/Q4 KV codec: groups of 64, fp16 scales, packed
            payloads (ReKV section 2.2).
accounting  closed forms for KV bytes per position and per layer (TileInfer.jl
            "Sizing" table and "INT8 cache"; ReKV section 2.1 eqs. (1)-(2) and
            section 2.2 eq. (7)).

Pinning status (what each function is checked against, in ``tests/``):
  paging      copy-on-write (fork, reserve_cow, copy_pages): the blog's Figure 6
              walk-through (golden fixture), the full-shared-block rule,
              all-or-nothing, and every forked response reading exactly its
              prompt and its own tokens after random writes and page copies.
  paging      the worked example of "KV Cache Management and PagedAttention"
              (block counts; B in physical blocks 3, 0 and C in 1, 4; growth
              into block 5),
              invariants (truncate-then-reserve returns the same pages,
              all-or-nothing OOM).
  planner     Quail "KV" worked example (order/parent/shared, 1,916 vs 4,300
              tokens);
              brute force on tiny alphabets (maximal sharing, page identity).
              The parent-link chase is pinned only by the page-identity
              invariant: the pages' example never walks a link, so the
              choice among equivalent parents is parity unpinned.
  attention   closed forms, fp64 SDPA library special case, scalar brute force,
              permutation invariance.
  retention   hand-worked priorities and eviction orders from the page's
              formula; ties, per-page value, take-back, shared pages
              surviving, the two-forward-pass limit.
  quant       hand-worked codes from the page's rule (incl. the ties-to-even
              reading), zero vector, peak code +-127, the symmetric error
              bound, placement by slot, brute force of the page's folded-scale
              formulation, page-placement invariance.
  codec       payload size = eq. (7) and the page's 8.25 / 179.75 / 231 MiB
              figures; hand-worked Q8 and Q4 groups (ties, nibble order);
              the error bound; zero groups; pack/unpack and layout inverses.
  accounting  every cell of the TileInfer.jl sizing table and the ReKV byte
              figures.
"""

from . import accounting, attention, codec, paging, planner, quant, retention  # noqa: F401
