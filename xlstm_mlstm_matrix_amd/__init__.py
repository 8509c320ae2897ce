"""mLSTM cell forward (xLSTM) on AMD MI355X (gfx950).

The compute path is the HIP library ``libmlstm.so`` behind the C ABI in
``include/mlstm.h``; :mod:`.binding` marshals torch tensors into it.
"""
from .binding import (BF16, F32, MlstmError, fwd_chunkwise, lib, status_string, step,  # noqa: F401
                      workspace_size)

__version__ = "0.1.0"
