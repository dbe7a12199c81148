"""MI355X (gfx950) replay-free block verification for a hybrid conv/IIR/attention layer.

Importing the package loads nothing native; ``hybrid_conv_iir_amd.hci``
loads the HIP library (``libhci.so``) and fails loudly if it is missing.
"""
