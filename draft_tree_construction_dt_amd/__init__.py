"""MI355X-native draft-tree construction (DART / DARTree hot path).

The C-ABI library ``libdt.so`` (declared in ``include/dt.h``) does all of the
work on the GPU; ``binding`` marshals torch tensors into it.  Binding names
are loaded lazily so that the input generator (``synth``) can be imported on
machines where the library has not been built yet.
"""

_BINDING_NAMES = {
    "dt_build_tree", "dt_workspace_size", "dt_status_string", "dt_position_topk",
    "DtError", "DeviceProblem", "upload_problem", "alloc_tree_out", "library_path",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
