"""MI355X (gfx950) Recurrent Looped Transformer decoder step.

The product is the C-ABI library ``librlt.so`` (include/rlt.h); this package holds its HIP
sources (``csrc/``), the build script and a thin ctypes binding with the same call names.
"""
from .binding import (  # noqa: F401
    LIB_PATH, Memory, Model, RLTError, State, bptt_workspace, clock_buffer, grad_buffers,
    load_library,
    make_config, parallel_workspace, rlt_bptt,
    rlt_config, rlt_decoder_step, rlt_decoder_step_ragged, rlt_memproj, rlt_run_parallel,
    rlt_run_parallel_noalloc,
    rlt_run_sequence, rlt_state_export, rlt_state_import, rlt_state_import_ragged,
    upload_weights, Head, upload_head_weights, rlt_encode, rlt_readout, readout_workspace,
)
