"""MLA speculative-decoding verify attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library `libmla_verify.so` (C ABI, declared in
include/mla_verify.h); this package is its thin Python binding.  Importing the
package does not load the library; `speculative_decode_mla_amd.api` does, and
raises if the library has not been built.
"""
__all__ = ["api", "inputs"]
