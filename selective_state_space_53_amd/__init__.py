"""MI355X (gfx950) selective scan: Mamba's input-dependent SSM recurrence as a
C-ABI HIP library (libssmscan.so, include/ssm_scan.h) with a thin ctypes binding.

    from selective_state_space_53_amd import ssm_scan_fwd, ssm_state_update

The binding is loaded lazily so that importing the package works on machines
without the built library; calling an entry point then raises ImportError.
"""

__all__ = ["ssm_scan_fwd", "ssm_state_update", "ssm_scan_workspace_bytes",
           "ssm_status_string", "ssm_last_error", "ssm_abi_version", "binding"]


def __getattr__(name):
    if name in __all__:
        import importlib
        # raises ImportError when libssmscan.so is missing
        binding = importlib.import_module(__name__ + ".binding")
        return binding if name == "binding" else getattr(binding, name)
    raise AttributeError(name)
