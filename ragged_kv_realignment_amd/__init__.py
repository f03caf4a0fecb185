"""MI355X-native verify-and-resynchronize step of batch speculative decoding.

The work is done by libspecdec.so (hand-written HIP kernels for gfx950 behind
the C ABI in include/specdec.h); this package is its Python binding.
"""
from .specdec import (  # noqa: F401
    APPEND_INPLACE, BF16, EQSPEC, EQSPEC_INPLACE, EQSPEC_INPLACE_ZERO_PAD, F16, F32, GATHER, S_CAPACITY, S_DRAFT_RANGE, S_LEN_RANGE, S_PROB, S_ROWS_DUP,
    SeqBuf, SpecDecError, append, gather, group_by_len, lib, realign_eqspec, realign_eqspec_inplace, specdec_group_by_len,
    specdec_realign_kv, specdec_verify_greedy, specdec_verify_greedy_noalloc, specdec_verify_sample, specdec_verify_sample_logits, specdec_version,
    sample_workspace, sample_verify_workspace, verify_greedy, verify_greedy_noalloc, verify_sample, verify_sample_logits, workspace, PagedKV, paged_admit,
    paged_append, paged_gather, paged_retire, Sched, pool_admit, pool_finish)
