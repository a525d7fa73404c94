"""SAS gated block-sparse attention on MI355X (gfx950).

The compute path is the C-ABI library ``libsas.so`` built from ``csrc/``; the
Python functions re-exported here only marshal torch tensors into its calls.
Importing this package does not load the library; the first call does, and it
raises if the library has not been built.
"""

_BINDING_NAMES = (
    "sas_block_summaries", "sas_select", "sas_decode_fwd", "sas_decode_step",
    "sas_decode_step_paged", "sas_block_summaries_paged", "sas_prefill_fwd", "sas_bwd",
    "sas_selector_bwd", "sas_workspace_bytes", "SasError",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
