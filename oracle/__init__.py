"""CPU oracle for rotated, codebook-quantised, paged KV decode attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or run anything in this package.
The product path (``quantized_paged_kv_amd``) never imports it, and this
package imports nothing from the product: the two share no code.  The only
shared module is ``workloads`` (seeded input generators, no method
arithmetic).

It is deliberately slow and plain: numpy in float64, one step per function,
in the order the pages describe the method.  It plays the role of the
"diagnostic route" of the TurboQuant design page: it reconstructs dense K/V
from packed pages and runs attention on them, which the serving route must
never do.

Sources, cited by page title and section:

* [D]  "Design" page of the TurboQuant documentation
       (ginkgoq.github.io/TurboQuant/design): sections "System Invariants",
       "Data Ownership", "Diagnostic Route Design", "Serving Route Design",
       "Format Strategy", "Recipe Strategy", "Error Model".
* [S]  "TurboQuant Inference Server" README: "What it does" table,
       "Architecture notes" (Lloyd-Max codebook caching, calibration).
* [T]  "Tattletale" README, "Highlights": random Hadamard rotations with
       codebooks (EXL3) as prior art for rotate-then-codebook.

Where the pages leave a point open, the function that depends on it
states the reading it takes.

Parity status: every function here is pinned by tests in
``tests/test_oracle_*.py`` against closed forms, published values,
brute force or invariants.  No function is "parity unpinned".  The QJL
stage (``qjl.py``) follows a reading of fields the pages only name; it is
pinned to the published estimator's closed-form mean and variance and to
its identity / permutation special cases, not to anything on the pages.
"""
from .codebook import lloyd_max_gaussian, codebook_f16, thresholds_f64, f64_to_f16_bits
from .rotation import fwht, sylvester_hadamard, rotate, inverse_rotate
from .encode import Format, tree_sum, encode_rows, quantize_rotated, pack_group, unpack_group, row_bytes
from .pages import tile_layout, write_pages, read_rows, reconstruct_sequence
from .attn import attention, split_partials, merge_partials, decode_reference
from .ledger import ledger
from . import qjl

__all__ = [
    "lloyd_max_gaussian", "codebook_f16", "thresholds_f64", "f64_to_f16_bits",
    "fwht", "sylvester_hadamard", "rotate", "inverse_rotate",
    "Format", "tree_sum", "encode_rows", "quantize_rotated", "pack_group", "unpack_group", "row_bytes",
    "tile_layout", "write_pages", "read_rows", "reconstruct_sequence",
    "attention", "split_partials", "merge_partials", "decode_reference",
    "ledger", "qjl",
]
