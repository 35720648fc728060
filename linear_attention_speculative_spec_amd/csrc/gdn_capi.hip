// gdn_capi.hip -- the extern "C" boundary of libgdnverify: host-side argument
// validation, then kernel launches on the caller's stream.  No allocation,
// no synchronisation; a rejected call enqueues nothing.
#include <cmath>

#include "gdn_common.h"
#include "gdn_internal.h"

namespace {

using namespace gdn;

bool aligned(const void* p, size_t a)
{
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Non-null and aligned for its widest access.
bool ok_ptr(const void* p, size_t a)
{
    return p != nullptr && aligned(p, a);
}

int check_shape(const gdn_shape* sh)
{
    if (sh == nullptr)
        return GDN_EINVAL;
    const gdn_shape& s = *sh;
    if (s.B < 0 || s.T < 1 || s.H < 1 || s.HV < 1 || s.K < 1 || s.V < 1 || s.L < 2 ||
        s.max_spec_len < 1 || s.num_slots < 1)
        return GDN_EINVAL;
    if (s.HV % s.H != 0)
        return GDN_EINVAL;
    if ((s.L & (s.L - 1)) != 0)                       // ring length: power of two
        return GDN_EINVAL;
    if (s.T > s.max_spec_len || 2 * s.max_spec_len > s.L)   // room for one more window
        return GDN_EINVAL;
    if (s.act != GDN_F32 && s.act != GDN_BF16)
        return GDN_EINVAL;
    if (!std::isfinite(s.scale) || !std::isfinite(s.softplus_threshold) ||
        !std::isfinite(s.l2norm_eps) || s.l2norm_eps < 0.0f)
        return GDN_EINVAL;
    if (s.K != 64 && s.K != 128 && s.K != 256)
        return GDN_EUNSUPPORTED;
    if (s.V % 16 != 0 || s.V > 256)
        return GDN_EUNSUPPORTED;
    if (s.max_spec_len > 16 || s.L > 128)
        return GDN_EUNSUPPORTED;
    if (s.K == 256 && s.L > 64)          // verify staging would exceed the register budget
        return GDN_EUNSUPPORTED;
    if (s.B > 65535 || s.HV > 65535)
        return GDN_EUNSUPPORTED;
    // work items (row, value head, value tile) are counted in 32-bit ints
    if (static_cast<long long>(s.B) * s.HV * (s.V / 16) > 0x7FFFFFFFLL)
        return GDN_EUNSUPPORTED;
    if (verify_lds_bytes(s) > max_lds_bytes())
        return GDN_EUNSUPPORTED;
    return GDN_OK;
}

// Layer count of a multi-layer fold; its work items (row, layer, value head,
// value tile) are counted in 32-bit ints.
int check_layers(const gdn_shape& s, int num_layers)
{
    if (num_layers < 1)
        return GDN_EINVAL;
    if (static_cast<long long>(num_layers) * s.HV > 65535 ||
        static_cast<long long>(s.B) * num_layers * s.HV * (s.V / 16) > 0x7FFFFFFFLL)
        return GDN_EUNSUPPORTED;
    return GDN_OK;
}

// Layer strides of a multi-layer fold (0: back to back), resolved in place.
int resolve_layer_strides(const gdn_shape& sh, int num_layers, int64_t& layer_stride_S,
                          int64_t& layer_stride_ring)
{
    const int64_t layer_S = static_cast<int64_t>(sh.num_slots) * sh.HV * sh.V * sh.K;
    if (layer_stride_S < 0 || layer_stride_ring < 0)
        return GDN_EINVAL;
    if (layer_stride_S == 0)
        layer_stride_S = layer_S;
    if (layer_stride_ring == 0)
        layer_stride_ring = sh.num_slots;
    if (num_layers > 1 &&
        (layer_stride_S < layer_S || layer_stride_ring < sh.num_slots || layer_stride_S % 4 != 0))
        return GDN_EINVAL;
    return GDN_OK;
}

size_t act_bytes(const gdn_shape& s)
{
    return s.act == GDN_BF16 ? 2 : 4;
}

int status_of(hipError_t e)
{
    return e == hipSuccess ? GDN_OK : GDN_ELAUNCH;
}

}  // namespace

extern "C" {

int gdn_validate_shape(const gdn_shape* shape)
{
    return check_shape(shape);
}

const char* gdn_status_str(int status)
{
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_EINVAL: return "invalid argument (shape, null or misaligned pointer)";
    case GDN_EUNSUPPORTED: return "shape outside what the kernels support";
    case GDN_ELAUNCH: return "kernel launch rejected by the HIP runtime";
    default: return "unknown status";
    }
}

size_t gdn_ring_bytes(const gdn_shape* shape)
{
    if (check_shape(shape) != GDN_OK)
        return 0;
    const gdn_shape& s = *shape;
    const size_t eb = act_bytes(s);
    const size_t rec = static_cast<size_t>(s.H) * s.K * eb + static_cast<size_t>(s.HV) * s.V * eb +
                       static_cast<size_t>(s.HV) * 8;
    return static_cast<size_t>(s.num_slots) * s.L * rec;
}

size_t gdn_snapshot_bytes(const gdn_shape* shape)
{
    if (check_shape(shape) != GDN_OK)
        return 0;
    const gdn_shape& s = *shape;
    return static_cast<size_t>(s.B) * s.T * s.HV * s.V * s.K * 4;
}

int gdn_spec_verify_ring(const gdn_shape* shape, const void* q, const void* k, const void* v,
                         const void* a, const void* b, const float* A_log, const float* dt_bias,
                         float* S, const int32_t* slot_idx, const int32_t* write_pos,
                         const int32_t* cache_base, const int32_t* is_flush, void* ring_rawk,
                         void* ring_rawv, float* ring_g, float* ring_beta, int write_ring,
                         int fold_flagged, void* o, void* stream)
{
    int st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    const gdn_shape& sh = *shape;
    const size_t eb = act_bytes(sh);
    if (!ok_ptr(q, 16) || !ok_ptr(k, 16) || !ok_ptr(v, 16) || !ok_ptr(a, eb) || !ok_ptr(b, eb) ||
        !ok_ptr(A_log, 4) || !ok_ptr(dt_bias, 4) || !ok_ptr(S, 16) || !ok_ptr(slot_idx, 4) ||
        !ok_ptr(write_pos, 4) || !ok_ptr(cache_base, 4) || !ok_ptr(is_flush, 4) ||
        !ok_ptr(ring_rawk, 16) || !ok_ptr(ring_rawv, 16) || !ok_ptr(ring_g, 4) ||
        !ok_ptr(ring_beta, 4) || !ok_ptr(o, 16))
        return GDN_EINVAL;
    if (o == q || o == k || o == v || o == S)
        return GDN_EINVAL;
    // bf16 gate inputs are read as aligned words of two activations: the
    // words must be aligned and the last one must not reach past the end
    if (sh.act == GDN_BF16) {
        if (!aligned(a, 4) || !aligned(b, 4))
            return GDN_EINVAL;
        if ((static_cast<long long>(sh.B) * sh.T * sh.HV) % 2 != 0)
            return GDN_EUNSUPPORTED;
    }
    hipStream_t strm = static_cast<hipStream_t>(stream);
    const WindowPtrs w = {q, k, v, a, b, A_log, dt_bias};
    const CursorPtrs c = {write_pos, cache_base, is_flush};
    const RingPtrs r = {ring_rawk, ring_rawv, ring_g, ring_beta};
    if (fold_flagged) {
        // launch 1: rows flagged for flush advance their checkpoint exactly
        st = status_of(launch_fold(sh, 1, 0, 0, S, r, slot_idx, c, 1, strm));
        if (st != GDN_OK)
            return st;
    }
    // launch 2: outputs of every row from checkpoint + history + window
    return status_of(launch_verify(sh, w, S, slot_idx, c, r, write_ring ? 1 : 0, o, strm));
}

int gdn_spec_verify_dcache(const gdn_shape* shape, const void* q, const void* k, const void* v,
                           const void* a, const void* b, const float* A_log,
                           const float* dt_bias, float* S, const int32_t* slot_idx,
                           const int32_t* write_pos, const int32_t* cache_base,
                           const int32_t* is_flush, void* ring_rawk, void* ring_rawv,
                           float* ring_g, float* ring_beta, float* ring_d, int write_ring,
                           int fold_flagged, void* o, void* stream)
{
    int st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    const gdn_shape& sh = *shape;
    if (dcache_lds_bytes(sh) > max_lds_bytes())
        return GDN_EUNSUPPORTED;
    const size_t eb = act_bytes(sh);
    if (!ok_ptr(q, 16) || !ok_ptr(k, 16) || !ok_ptr(v, 16) || !ok_ptr(a, eb) || !ok_ptr(b, eb) ||
        !ok_ptr(A_log, 4) || !ok_ptr(dt_bias, 4) || !ok_ptr(S, 16) || !ok_ptr(slot_idx, 4) ||
        !ok_ptr(write_pos, 4) || !ok_ptr(cache_base, 4) || !ok_ptr(is_flush, 4) ||
        !ok_ptr(ring_rawk, 16) || !ok_ptr(ring_rawv, 16) || !ok_ptr(ring_g, 4) ||
        !ok_ptr(ring_beta, 4) || !ok_ptr(ring_d, 16) || !ok_ptr(o, 16))
        return GDN_EINVAL;
    if (o == q || o == k || o == v || o == S || o == ring_d)
        return GDN_EINVAL;
    hipStream_t strm = static_cast<hipStream_t>(stream);
    const WindowPtrs w = {q, k, v, a, b, A_log, dt_bias};
    const CursorPtrs c = {write_pos, cache_base, is_flush};
    const RingPtrs r = {ring_rawk, ring_rawv, ring_g, ring_beta};
    if (fold_flagged) {
        // launch 1: flagged rows advance their checkpoint exactly (raw records)
        st = status_of(launch_fold(sh, 1, 0, 0, S, r, slot_idx, c, 1, strm));
        if (st != GDN_OK)
            return st;
    }
    // launch 2: outputs through the stored deltas; the window's deltas recorded
    return status_of(launch_dcache_verify(sh, w, S, slot_idx, c, r, ring_d, write_ring ? 1 : 0,
                                          o, strm));
}

size_t gdn_dring_bytes(const gdn_shape* shape)
{
    if (check_shape(shape) != GDN_OK)
        return 0;
    const gdn_shape& s = *shape;
    return static_cast<size_t>(s.num_slots) * s.HV * s.L * s.V * 4;
}

int gdn_exact_fold(const gdn_shape* shape, int num_layers, int64_t layer_stride_S,
                   int64_t layer_stride_ring, float* S, const void* ring_rawk,
                   const void* ring_rawv, const float* ring_g, const float* ring_beta,
                   const int32_t* slot_idx, const int32_t* write_pos, const int32_t* cache_base,
                   const int32_t* is_flush, int only_flagged, void* stream)
{
    int st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    const gdn_shape& sh = *shape;
    st = check_layers(sh, num_layers);
    if (st != GDN_OK)
        return st;
    // per-layer strides: fp32 elements of S, slots of the ring arrays
    st = resolve_layer_strides(sh, num_layers, layer_stride_S, layer_stride_ring);
    if (st != GDN_OK)
        return st;
    if (!ok_ptr(S, 16) || !ok_ptr(ring_rawk, 16) || !ok_ptr(ring_rawv, 16) || !ok_ptr(ring_g, 4) ||
        !ok_ptr(ring_beta, 4) || !ok_ptr(slot_idx, 4) || !ok_ptr(write_pos, 4) ||
        !ok_ptr(cache_base, 4) || (only_flagged && !ok_ptr(is_flush, 4)))
        return GDN_EINVAL;
    const RingPtrs r = {const_cast<void*>(ring_rawk), const_cast<void*>(ring_rawv),
                        const_cast<float*>(ring_g), const_cast<float*>(ring_beta)};
    const CursorPtrs c = {write_pos, cache_base, is_flush};
    return status_of(launch_fold(sh, num_layers, layer_stride_S, layer_stride_ring, S, r, slot_idx,
                                 c, only_flagged ? 1 : 0, static_cast<hipStream_t>(stream)));
}

int gdn_kda_spec_verify_ring(const gdn_shape* shape, const void* q, const void* k, const void* v,
                             const void* a, const void* b, const float* A_log, const float* dt_bias,
                             float* S, const int32_t* slot_idx, const int32_t* write_pos,
                             const int32_t* cache_base, const int32_t* is_flush, void* ring_rawk,
                             void* ring_rawv, float* ring_g, float* ring_beta, int write_ring,
                             int fold_flagged, void* o, void* stream)
{
    int st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    const gdn_shape& sh = *shape;
    if (!kda_shape_supported(sh))
        return GDN_EUNSUPPORTED;
    const size_t eb = act_bytes(sh);
    if (!ok_ptr(q, 16) || !ok_ptr(k, 16) || !ok_ptr(v, 16) || !ok_ptr(a, eb) || !ok_ptr(b, eb) ||
        !ok_ptr(A_log, 4) || !ok_ptr(dt_bias, 4) || !ok_ptr(S, 16) || !ok_ptr(slot_idx, 4) ||
        !ok_ptr(write_pos, 4) || !ok_ptr(cache_base, 4) || !ok_ptr(is_flush, 4) ||
        !ok_ptr(ring_rawk, 16) || !ok_ptr(ring_rawv, 16) || !ok_ptr(ring_g, 16) ||
        !ok_ptr(ring_beta, 4) || !ok_ptr(o, 16))
        return GDN_EINVAL;
    if (o == q || o == k || o == v || o == S)
        return GDN_EINVAL;
    const WindowPtrs w = {q, k, v, a, b, A_log, dt_bias};
    const CursorPtrs c = {write_pos, cache_base, is_flush};
    const RingPtrs r = {ring_rawk, ring_rawv, ring_g, ring_beta};
    // one launch: history replay (stored for flagged rows), then the window
    return status_of(launch_kda_verify(sh, w, S, slot_idx, c, r, write_ring ? 1 : 0,
                                       fold_flagged ? 1 : 0, o, static_cast<hipStream_t>(stream)));
}

int gdn_kda_exact_fold(const gdn_shape* shape, int num_layers, int64_t layer_stride_S,
                       int64_t layer_stride_ring, float* S, const void* ring_rawk,
                       const void* ring_rawv, const float* ring_g, const float* ring_beta,
                       const int32_t* slot_idx, const int32_t* write_pos, const int32_t* cache_base,
                       const int32_t* is_flush, int only_flagged, void* stream)
{
    int st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    const gdn_shape& sh = *shape;
    if (!kda_shape_supported(sh))
        return GDN_EUNSUPPORTED;
    st = check_layers(sh, num_layers);
    if (st != GDN_OK)
        return st;
    st = resolve_layer_strides(sh, num_layers, layer_stride_S, layer_stride_ring);
    if (st != GDN_OK)
        return st;
    if (!ok_ptr(S, 16) || !ok_ptr(ring_rawk, 16) || !ok_ptr(ring_rawv, 16) || !ok_ptr(ring_g, 16) ||
        !ok_ptr(ring_beta, 4) || !ok_ptr(slot_idx, 4) || !ok_ptr(write_pos, 4) ||
        !ok_ptr(cache_base, 4) || (only_flagged && !ok_ptr(is_flush, 4)))
        return GDN_EINVAL;
    const RingPtrs r = {const_cast<void*>(ring_rawk), const_cast<void*>(ring_rawv),
                        const_cast<float*>(ring_g), const_cast<float*>(ring_beta)};
    const CursorPtrs c = {write_pos, cache_base, is_flush};
    return status_of(launch_kda_fold(sh, num_layers, layer_stride_S, layer_stride_ring, S, r,
                                     slot_idx, c, only_flagged ? 1 : 0,
                                     static_cast<hipStream_t>(stream)));
}

size_t gdn_kda_ring_bytes(const gdn_shape* shape)
{
    if (check_shape(shape) != GDN_OK || !kda_shape_supported(*shape))
        return 0;
    const gdn_shape& s = *shape;
    const size_t eb = act_bytes(s);
    const size_t rec = static_cast<size_t>(s.H) * s.K * eb + static_cast<size_t>(s.HV) * s.V * eb +
                       static_cast<size_t>(s.HV) * s.K * 4 + static_cast<size_t>(s.HV) * 4;
    return static_cast<size_t>(s.num_slots) * s.L * rec;
}

int gdn_advance_cursors(const gdn_shape* shape, const int32_t* slot_idx, const int32_t* accept,
                        int32_t* write_pos, int32_t* cache_base, int32_t* is_flush, void* stream)
{
    int st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    if (!ok_ptr(slot_idx, 4) || !ok_ptr(accept, 4) || !ok_ptr(write_pos, 4) ||
        !ok_ptr(cache_base, 4) || !ok_ptr(is_flush, 4))
        return GDN_EINVAL;
    return status_of(launch_advance(*shape, slot_idx, accept, write_pos, cache_base, is_flush,
                                    static_cast<hipStream_t>(stream)));
}

int gdn_reset_cursors(const gdn_shape* shape, const int32_t* slots, int32_t n, int32_t init_flush,
                      int32_t* write_pos, int32_t* cache_base, int32_t* is_flush, void* stream)
{
    int st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    if (n < 0)
        return GDN_EINVAL;
    if (n > 0 && (!ok_ptr(slots, 4) || !ok_ptr(write_pos, 4) || !ok_ptr(cache_base, 4) ||
                  !ok_ptr(is_flush, 4)))
        return GDN_EINVAL;
    return status_of(launch_reset(*shape, slots, n, init_flush, write_pos, cache_base, is_flush,
                                  static_cast<hipStream_t>(stream)));
}

int gdn_recurrent_verify_snapshot(const gdn_shape* shape, const void* q, const void* k,
                                  const void* v, const void* a, const void* b, const float* A_log,
                                  const float* dt_bias, const float* S, const int32_t* slot_idx,
                                  float* snap, void* o, void* ring_rawk, void* ring_rawv,
                                  float* ring_g, float* ring_beta, const int32_t* write_pos,
                                  const int32_t* cache_base, int write_ring, void* stream)
{
    int st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    const gdn_shape& sh = *shape;
    const size_t eb = act_bytes(sh);
    if (!ok_ptr(q, 16) || !ok_ptr(k, 16) || !ok_ptr(v, 16) || !ok_ptr(a, eb) || !ok_ptr(b, eb) ||
        !ok_ptr(A_log, 4) || !ok_ptr(dt_bias, 4) || !ok_ptr(S, 16) || !ok_ptr(slot_idx, 4) ||
        !ok_ptr(snap, 16) || !ok_ptr(o, eb))
        return GDN_EINVAL;
    if (write_ring && (!ok_ptr(ring_rawk, 16) || !ok_ptr(ring_rawv, 16) || !ok_ptr(ring_g, 4) ||
                       !ok_ptr(ring_beta, 4) || !ok_ptr(write_pos, 4) || !ok_ptr(cache_base, 4)))
        return GDN_EINVAL;
    if (static_cast<const void*>(snap) == static_cast<const void*>(S))
        return GDN_EINVAL;
    const WindowPtrs w = {q, k, v, a, b, A_log, dt_bias};
    const RingPtrs r = {ring_rawk, ring_rawv, ring_g, ring_beta};
    return status_of(launch_snapshot(sh, w, S, slot_idx, snap, o, r, write_pos, cache_base,
                                     write_ring ? 1 : 0, static_cast<hipStream_t>(stream)));
}

int gdn_snapshot_commit(const gdn_shape* shape, const float* snap, const int32_t* slot_idx,
                        const int32_t* accept, float* S, void* stream)
{
    int st = check_shape(shape);
    if (st != GDN_OK)
        return st;
    if (!ok_ptr(snap, 16) || !ok_ptr(slot_idx, 4) || !ok_ptr(accept, 4) || !ok_ptr(S, 16))
        return GDN_EINVAL;
    return status_of(launch_snapshot_commit(*shape, snap, slot_idx, accept, S,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
