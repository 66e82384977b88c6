"""MI355X-native importance-weighted GGML IQ encoder and imatrix collector.

The compute path is the HIP library ``libiq.so`` (built from ``csrc/``); this
package only marshals arguments into its C ABI.  Importing the package loads
nothing: the library is loaded on first use by ``ggml_iq_codebook_imatrix_amd.api``
and the call fails loudly if it is missing.
"""
FORMATS = ("IQ2_XXS", "IQ2_XS", "IQ2_S", "IQ1_S", "IQ1_M")

__all__ = ["FORMATS"]
