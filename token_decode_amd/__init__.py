"""MI355X-native one-token decode for Llama-family transformers.

The work runs in the HIP library libpn.so (include/pn.h); this package holds
its ctypes binding (`_capi`, same function names as the C ABI) and torch-based
device plumbing (`device`).  Importing it does not need a GPU; calling the
library's compute entry points does.
"""
from . import _capi as capi
from ._capi import (PN_BF16, PN_EHIP, PN_EINVAL, PN_ERANGE, PN_EUNSUPPORTED, PN_F32, PN_I8, PN_OK,
                    PNError, check, lib)

__all__ = ["capi", "lib", "check", "PNError", "PN_F32", "PN_BF16", "PN_I8", "PN_OK", "PN_EINVAL",
           "PN_ERANGE", "PN_EUNSUPPORTED", "PN_EHIP"]
