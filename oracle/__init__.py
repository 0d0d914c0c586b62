"""CPU oracle of OSCAR-style attention-aware INT2 KV caching (test infrastructure).

This package is a plain, slow, obviously-correct statement of what the decode hot path
computes, written from the OSCAR pages:

* "Together AI open-sources OSCAR" (news.chathome.org): the key-logit error identity and
  the query covariance C_Q (section "OSCAR's difference"), the score-weighted value
  covariance C_S, the composed rotations R_K = U_Q.H.P_br and R_V = U_S.H.P_br, and the
  three-region cache layout (section "serving system: mixed-precision cache layout").
* The OSCAR overview page (m.kljzs.com): demote = rotate/clip/quantize/pack of the oldest
  recent token, 4 two-bit codes per byte, INT2 kernel = unpack + scale/zero restore +
  float accumulation, BF16 kernel for sink/recent, online-softmax merge (method paragraph).
* The OSCAR study note (estelledc.github.io): clip constants c_K ~ 0.96, c_V ~ 0.92
  (case 2), the [BF16 sink] | [INT2 history] | [BF16 recent] layout with sink 64 and
  recent 256 (core point 3).
* The TriAxialKV reading note (miraclefarms.github.io): INT2/INT4 dual pool split at an
  address offset (section 4) and bitwidth-homogeneous decode splits.
* The OSCAR overview page, the paragraph that sets OSCAR beside TurboQuant: a Lloyd-Max
  codebook with the attention-aware rotation (``codebook.py``, pinned against textbook
  Lloyd-Max values, brute force and the uniform codec).

Who may use it: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py``. The product package never imports, links or runs anything here, and this
package never imports the product package. The two share no code; only the seeded input
generators in ``synth`` serve both.

Precision: fp64 everywhere, except the quantiser, whose integer decisions are taken in
fp32 op by op (the precision of the kernel, since the pages fix none) so that codes can be
compared bit for bit on the same fp32 rotated inputs.
"""
from .rotation import (hadamard, bitrev_indices, bitrev_matrix, query_covariance,
                       score_weighted_value_covariance, eigenbasis, compose_rotation,
                       rotation_fp32)
from .quant import (bf16_round, bf16_bits, bf16_from_bits, quantize_group, quantize_rows,
                    pack_codes, unpack_codes, dequantize_rows, rotate_rows_fp32)
from .cache import (SINK, RECENT, segments, effective_bits, OracleCache)
from .attention import (softmax_attention, lse_merge, decode_attention, plain_decode_attention,
                        partial_attention)
from .allocate import greedy_bit_allocation, exhaustive_bit_allocation
from .codebook import (UNIFORM_LEVELS, fp16_levels, fp16_patterns, thresholds_fp32, code_of_coordinate,
                       group_coordinates, quantize_rows_codebook, dequantize_rows_codebook, lloyd_max,
                       fit_codebook)

__all__ = [n for n in dir() if not n.startswith("_")]
