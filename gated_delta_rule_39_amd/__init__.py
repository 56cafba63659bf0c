"""MI355X (gfx950) Kimi Delta Attention forward.

The forward is the C-ABI library ``libkda.so`` (hand-written HIP kernels);
``gated_delta_rule_39_amd.kda`` is its Python binding.  The binding is loaded
on first use (so that ``_build`` can run before the library exists) and fails
loudly if the library has not been built.
"""
_EXPORTS = ("KDAError", "fwd", "workspace_size", "version")


def __getattr__(name):
    if name in _EXPORTS:
        from . import kda
        return getattr(kda, name)
    raise AttributeError(name)
