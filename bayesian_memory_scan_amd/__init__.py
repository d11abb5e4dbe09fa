"""libkdnscan: precision-tracking associative-memory scans on AMD MI355X (gfx950).

The C-ABI library (include/kdnscan.h) is reached through the ``kdnscan``
submodule, loaded on first use of any ``kdn_*`` name; it raises ImportError
when libkdnscan.so has not been built -- there is no fallback path.
``synth`` (seeded synthetic inputs) needs no library.
"""
from __future__ import annotations

import importlib

_BINDING = {
    "lib", "LIB_PATH", "KDN_OK", "KDN_EINVAL", "KDN_EUNSUPPORTED", "KDN_EWORKSPACE", "KDN_EHIP",
    "KDN_ESCRATCH", "KDN_F32", "KDN_BF16", "KDN_ECHO_WORDS", "KdnError", "ScanOpts", "kdn_diag_scan_fwd",
    "kdn_diag_scan_fwd_noalloc", "kdn_diag_scan_bwd", "kdn_diag_noise_scan_fwd",
    "kdn_diag_scan_varlen_fwd", "kdn_diag_scan_varlen_bwd",
    "kdn_mobius_precision_scan",
    "kdn_decode_step", "kdn_diag_plan", "kdn_diag_varlen_plan", "kdn_status_string",
    "kdn_last_hip_error",
    "header_functions",
}


def __getattr__(name):
    if name in _BINDING:
        return getattr(importlib.import_module(".kdnscan", __name__), name)
    raise AttributeError(name)
