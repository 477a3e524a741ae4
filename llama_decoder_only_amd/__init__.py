"""SmolLM2-shaped decoder forward on MI355X (gfx950): HIP kernels behind a C ABI.

``llama_decoder_only_amd.binding`` loads ``libsmol.so`` (built in-tree by
``llama_decoder_only_amd/csrc/build.py``) and exposes the C entry points with the
same names. Importing this package loads nothing; the library is opened on the
first call into the binding.
"""

__all__ = ["binding", "synthetic"]
