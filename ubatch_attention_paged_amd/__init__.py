"""MI355X-native per-ubatch attention over a cell-granular F16 KV cache.

The work runs in ``libkvattn.so`` (hand-written HIP for gfx950 behind the C
ABI of ``include/kvattn.h`` and ``include/kvsched.h``); this package is its ctypes binding.  Importing
it loads the library and fails loudly when it has not been built -- there is
no CPU fallback.
"""

from .kvattn import (  # noqa: F401
    KVATTN_OK, KVATTN_NO_SLOT, KVATTN_EINVAL, KVATTN_ESTATE, KVATTN_ENOMEM, KVATTN_EHIP, KVATTN_ENODEV,
    KvattnError, Context, Ubatch, SeqIds, kvattn_params, kvattn_batch, kvattn_ubatch, load, LIB_PATH,
    kvattn_workspace_bytes, kvattn_cache_bytes, kvattn_create, kvattn_destroy, kvattn_split,
    kvattn_store, kvattn_attend, kvattn_attend_noalloc, kvattn_n_kv, kvattn_get_mask, kvattn_get_classes, kvattn_get_cells,
    kvattn_seq_rm, kvattn_seq_pos_max, kvattn_plan_stats, kvattn_last_error, kvattn_get_params,
    kvattn_split_batch, Scheduler, kvattn_sched_params, kvattn_sched_iter, kvattn_sched_create,
    kvattn_sched_destroy, kvattn_sched_submit, kvattn_sched_step, kvattn_sched_advance,
    kvattn_sched_request, kvattn_sched_last_error, KVATTN_ADMIT_RESERVE, KVATTN_ADMIT_PAGED,
    KVATTN_REQ_WAITING, KVATTN_REQ_RUNNING, KVATTN_REQ_DONE,
    kvattn_seq_state_size, kvattn_seq_state_save, kvattn_seq_state_load,
    kvattn_time_next_attend, KVATTN_KERNEL_MFMA, KVATTN_KERNEL_VALU, KVATTN_KERNEL_MERGE,
    kvattn_probe_gather, kvattn_probe_mfma, MAX_SEQ, SEQ_WORDS, seqset_int, seqset_members,
)

load()
