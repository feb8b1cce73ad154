"""MI355X-native decode hot path of Prism Attention (proposal-refined token-level sparse attention).

The compute path is the HIP library built from csrc/ (libprism.so, C ABI declared in
include/prism.h); `binding` marshals torch tensors to it.  `workload` generates seeded
synthetic inputs.  Importing the package does not load the HIP library; the first call
through `binding` does, and raises if it is missing.
"""
__all__ = ["binding", "workload"]
