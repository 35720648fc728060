"""libgdnverify: GDN ReplaySSM ring spec-verify for AMD MI355X (gfx950).

The compute lives in the HIP library ``libgdnverify.so`` (C ABI declared in
``include/gdnverify.h``); ``gdnverify`` is its ctypes binding and ``synth``
the seeded synthetic workload generator.
"""
from .gdnverify import (  # noqa: F401
    GDN_BF16, GDN_EINVAL, GDN_ELAUNCH, GDN_EUNSUPPORTED, GDN_F32, GDN_OK, GdnError, GdnShape,
    gdn_advance_cursors, gdn_exact_fold, gdn_recurrent_verify_snapshot, gdn_reset_cursors,
    gdn_ring_bytes, gdn_snapshot_bytes, gdn_snapshot_commit, gdn_spec_verify_ring,
    gdn_validate_shape, lib, status_str, gdn_spec_verify_dcache, gdn_dring_bytes,
    gdn_kda_spec_verify_ring, gdn_kda_exact_fold, gdn_kda_ring_bytes,
)
