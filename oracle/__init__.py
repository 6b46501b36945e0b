"""CPU oracle (fp64, numpy) for varlen attention and the AttentionUpdate merge.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product library. It shares no
code with the HIP kernels or their host launcher.

Parity status per function (what pins it; see tests/test_oracle_*.py):
  varlen_attention / varlen_attention_rows -- pinned: brute force with
      math.fsum on tiny cases, torch CPU fp64 scaled_dot_product_attention on
      padded per-sequence inputs, closed forms (Q = 0, causal row 0, constant
      V, single key) and invariants (packing, GQA = MHA on repeated K/V,
      key shift, scale folding, lse bounds, sequence permutation). The
      causal_offset option: brute force with offsets, and a key chunk
      computed alone with offset -a equals the chunked partial that keeps
      absolute positions through key_range.
  attn_update -- pinned: hand-worked golden values, chunked + merged equals
      unchunked attention, sp = 1 identity, chunk permutation, -inf chunks.
  chunked_partials -- pinned through the chunked + merged == unchunked check.
  last_token_gather -- pinned: golden indices for the tiny workload.
  paged_gather / paged_attention_rows -- pinned: a hand-worked paged fixture
      (Q = 0, so each row is the mean of the value rows it gathers) and
      scatter-into-shuffled-pages equals the contiguous oracle, with NaN in
      every slot the block table does not name.
  prologue.rms_norm / rotary / qk_norm_rope -- pinned: a hand-worked value
      (tests/golden/qk_norm_rope_handworked.json), torch's fp64 rms_norm,
      the rotation as complex multiplication by exp(i theta), identity at
      position 0, and the pair norms it preserves.
  linear_attention.gated_delta_rule -- pinned: a hand-worked overwrite
      (tests/golden/gated_delta_handworked.json), beta = 0 closed form,
      orthonormal-key associative recall, continuation through the state,
      packed == per sequence, linearity in v, and an independently written
      chunked (WY) formulation. These pin it to the recurrence its docstring
      states; the page that names the operator prints no formula, so that
      recurrence is a reading and its agreement with the page's own operator
      is unpinned.
"""
from .attention import (  # noqa: F401
    varlen_attention,
    varlen_attention_rows,
    attn_update,
    last_token_gather,
    chunked_partials,
    paged_gather,
    paged_attention_rows,
)
from .prologue import (  # noqa: F401
    rms_norm,
    rotate_half,
    rotary,
    qk_norm_rope,
)
from .linear_attention import gated_delta_rule  # noqa: F401
