"""MI355X-native ReverseMambaLayer forward (R2LM right-to-left Mamba sidecar).

The compute path is the HIP library ``libr2l.so`` (C ABI, ``include/r2l.h``);
``reverse_selective_scan_amd.binding`` marshals torch tensors into it.
"""
