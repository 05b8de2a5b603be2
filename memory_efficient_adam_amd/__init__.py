"""MI355X-native compressed-moment Adam/AdamW step.

Thin Python binding over ``libadam_mi355x.so`` (C ABI in
``include/adam_mi355x.h``): the functions below carry the C names and only
marshal arguments (torch tensors -> device pointers, the caller's current
HIP stream).  Every step of the update runs in the library's HIP kernels;
there is no CPU or PyTorch fallback -- if the library is not built, the
first call raises.
"""
from ._binding import (  # noqa: F401
    ADAM_BLOCK_SIZE,
    AdamError,
    AdamState,
    BUFFERS,
    GRAD_DTYPES,
    OPT_AMSGRAD,
    STORAGES,
    adam_last_error,
    adam_state_buffer_bytes,
    adam_state_bytes,
    adam_state_create,
    adam_state_describe,
    adam_state_destroy,
    adam_state_get_draw_index,
    adam_state_load,
    adam_state_read,
    adam_state_save,
    adam_state_serialized_bytes,
    adam_state_set_draw_index,
    adam_state_write,
    adam_step,
    adam_step_noalloc,
    library,
    library_path,
    state_buffer_sizes,
)
