"""MI355X-native Gated DeltaNet layer hot path.

The compute lives in the HIP library libgdn.so (C ABI, declared in
include/gdn.h); `linear_attention_layers_amd.gdn` is the thin ctypes binding
over it and `linear_attention_layers_amd.inputs` draws seeded synthetic
workloads.  Importing this package loads nothing; importing `.gdn` loads the
library and fails loudly if it has not been built.
"""
