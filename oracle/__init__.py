"""CPU oracle for the Spense hybrid sparse-dense linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library (no
kernels, headers, tables or helpers); the two meet only through the seeded
inputs drawn by ``synth``.

Every function here is plain NumPy in float64 (integer work on bit patterns),
written from the definitions on the pages:

  * "SpenseGPT: Practical One-shot Pruning Enabling Sparse and Dense GEMMs for
    LLM Inference" (gist.science explainer), Technical Summary 2.A "The Spense
    Format": each weight matrix is split into a contiguous dense region that
    keeps its weights and a contiguous 2:4 region; the input-split variant runs
    the first part of the input through the sparse GEMM and the second through
    the dense GEMM and accumulates both into one output.
  * same page, Technical Summary 2.B "Dense Index Selection Strategies":
    SpenseGPT keeps the last p% of indices dense; SpenseGPT+ keeps a selected
    index set dense and permutes it into the contiguous dense block.
  * same page, Technical Summary 2.A: the output-split variant splits the
    output rows instead (dense rows, and rows that are 2:4 along K), with no
    accumulation across the parts; the page uses it for the GLU gate and up
    projections (``resolve_dense_rows``, ``pack_rows``, ``linear_rows_ref``).
  * same page, Technical Summary 2.A with 2.B: the GLU block runs gate and up
    output-split and down input-split over one dense set of intermediate
    indices (``glu_block_ref``; SiLU gate, as in the GLU models the page
    evaluates).
  * same page, Technical Summary 2.B "SpenseGPT+": a score per intermediate
    index from |W_ij| * sqrt(H_jj) over gate, up and down, the top-scoring
    indices kept dense (``glu_scores_ref``, ``select_dense_ref``).
  * same page, Technical Summary 4 "Experimental Results" (layers run in
    FP8) with the SlideSparse explainer's Methodology 2.B "Activation
    Lifting" and 2.C (per-token activation quantisation online, the column
    re-ordering folded into it, then the 2:4 GEMM): the W8A8 form
    (``e4m3_round``, ``quantize_tokens_ref``, ``linear_w8a8_ref``) with the
    absmax per-token scale, the reading stated in ``spense.py``.
  * same page, Technical Summary 1 "Problem Statement" (and the SlideSparse
    explainer's Technical summary 1): 2:4 means at most two nonzeros in every
    four consecutive weights.

Parity status: every function is pinned by ``tests/test_oracle.py`` (closed
forms, exhaustive brute force on tiny inputs, library routines for the
special cases).  No function is "parity unpinned".
"""

from .spense import (  # noqa: F401
    DT_BF16,
    DT_F32,
    DT_FP8,
    DenseSetError,
    Packed,
    PackedRows,
    decode_values,
    decompress,
    dense_linear_ref,
    e4m3_round,
    down_ref,
    glu_block_ref,
    glu_scores_ref,
    hessian_diag,
    linear_ref,
    linear_rows_ref,
    linear_w8a8_ref,
    magnitude_key,
    pack,
    pack_rows,
    quantize_tokens_ref,
    resolve_dense_rows,
    resolve_dense_set,
    select_dense_ref,
    silu,
    unpack_bits,
    unpack_rows_bits,
)
