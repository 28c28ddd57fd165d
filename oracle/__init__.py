"""CPU oracle for the W4A16 group-quantized linear layer.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The HIP library never does, and
this package never imports the HIP library or anything under
``gemm_w4a16_group_amd``: the two sides share no code.

What it computes (all arithmetic in float64, numpy only):

* ``pack`` / ``unpack``: the packed storage of 4-bit codes, eight codes per
  32-bit word along the reduction axis, lowest nibble first.
* ``dequant``: Wdeq[m, k] = (q[m, k] - z[m, k // 128]) * s[m, k // 128].
* ``reference``: C = Wdeq @ X and the absolute-value bound A = |Wdeq| @ |X|.
* ``check``: the element-wise acceptance rule |C_gpu - C| <= 5e-3 * A + 1e-3.
* ``quantize_rtn``: a round-to-nearest min/max group quantizer (the step
  before the kernel; AWQ's activation-aware scale search is not modelled).

Sources (the PerfXLLM page on Snapdragon 8 Gen2, 3532n.com/d/2322131):

* §3.1 (low-precision quantization): weights only are quantized to int4,
  with a group size of 128 and a scale and a zero per group; the scale and
  zero add roughly one percent of storage.
* §3.3 item 1 (GEMM): C[m, n] = A[m, k] . B[k, n]; here A is the
  dequantized weight matrix and B the activations.
* §3.3 item 2 (GEMV): the n = 1 case of the same product.

Readings where the page is silent (each is listed with its reason in the
repository's design notes):

* the zero is an integer code subtracted before scaling: (q - z) * s;
* a group is 128 consecutive k of one output row m;
* the zero is stored as a 4-bit code, packed like the weights along the
  group axis (8 groups per word, lowest nibble first, padding nibbles 0);
* X is [K, N] and C is [M, N], both row-major (N contiguous);
* codes above 15 contribute their low nibble only.

Every function here is pinned by ``tests/test_oracle_*.py`` against
brute force, closed forms and invariants; none is "parity unpinned".
"""

from .w4a16 import (  # noqa: F401
    GROUP,
    pack_nibbles,
    unpack_nibbles,
    pack,
    unpack,
    dequant,
    reference,
    reference_rows,
    tolerance,
    check,
    quantize_rtn,
    format_bytes,
)
