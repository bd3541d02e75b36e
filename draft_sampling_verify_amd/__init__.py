"""MI355X-native output side of a speculative-decoding step.

The product is libspec.so (HIP kernels for gfx950 behind the C ABI in
include/spec.h); this package is its thin ctypes binding.  See
``_binding`` for the functions, named after the C entry points.
"""
from ._binding import (  # noqa: F401
    ClusterWorkspace, LIB_PATH, SPEC_BF16, SPEC_DEV_BAD_CLUSTER, SPEC_DEV_BAD_CONFIDENCE, SPEC_DEV_BAD_LENGTH, SPEC_DEV_BAD_TOKEN,
    SPEC_DEV_WAIT_FAILED, SPEC_EDEVICE, SPEC_EDTYPE, SPEC_EINVAL, SPEC_ELAUNCH, SPEC_EUNSUPPORTED,
    SPEC_EWORKSPACE, SPEC_F32, SPEC_OK, SPEC_OP_CONFIDENCE, SPEC_OP_LOSS, SPEC_OP_PROPOSE,
    SPEC_OP_ROUNDS, SPEC_OP_SCHEDULE, SPEC_OP_VERIFY, SpecError, Workspace, lib, spec_cluster_index, spec_cluster_propose,
    spec_cluster_verify, spec_cluster_workspace_bytes, spec_confidence, spec_decode_rounds, spec_draft_loss,
    spec_device_status, spec_markov_propose, spec_markov_propose_noalloc, SPEC_NOALLOC_BYTES,
    spec_pack_w2, spec_pack_w2_rv, spec_packed_w2_bytes, spec_philox_words,
    spec_profile_enable, spec_profile_names, spec_profile_read, spec_profile_reset, spec_schedule,
    spec_schedule_async, spec_verify, spec_workspace_bytes, spec_workspace_init, status_str,
    SPEC_PATH_AUTO, SPEC_PATH_NO_FUSED_PROPOSE, SPEC_PATH_NO_PIPELINED_SWEEP)
from ._binding import status_str as spec_status_str  # noqa: F811
