"""SAS (Simple Attention Sparsification) gated block-sparse attention for MI355X.

The compute lives in the HIP library `libsas.so` (C ABI declared in
include/sas.h); `binding` marshals torch tensors into its calls.  Import
`binding` to use it: it raises at import when the library is not built.
"""
