// gdn_internal.h -- host-side launch interface between the C ABI and kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdnverify.h"

namespace gdn {

// Pointers of one call, untyped for activations (dtype from the shape).
struct RingPtrs {
    void* rawk;
    void* rawv;
    float* g;
    float* beta;
};

struct CursorPtrs {
    const int32_t* write_pos;
    const int32_t* cache_base;
    const int32_t* is_flush;
};

struct WindowPtrs {
    const void* q;
    const void* k;
    const void* v;
    const void* a;
    const void* b;
    const float* A_log;
    const float* dt_bias;
};

// Value columns per verify workgroup and the dynamic LDS it needs.
int verify_tile_cols(const gdn_shape& sh);
size_t verify_lds_bytes(const gdn_shape& sh);
size_t max_lds_bytes();

hipError_t launch_verify(const gdn_shape& sh, const WindowPtrs& w, const float* S,
                         const int32_t* slot_idx, const CursorPtrs& c, const RingPtrs& r,
                         int write_ring, void* o, hipStream_t stream);

// The d-cache verify: history through stored corrected deltas ring_d
// [num_slots, HV, L, V] fp32; records the window's deltas there (write_ring).
size_t dcache_lds_bytes(const gdn_shape& sh);

hipError_t launch_dcache_verify(const gdn_shape& sh, const WindowPtrs& w, const float* S,
                                const int32_t* slot_idx, const CursorPtrs& c, const RingPtrs& r,
                                float* ring_d, int write_ring, void* o, hipStream_t stream);

// Layer l of a multi-layer fold: S + l * layer_stride_S (fp32 elements; 0 for
// back to back), ring arrays l * layer_stride_ring slots past their bases.
hipError_t launch_fold(const gdn_shape& sh, int num_layers, int64_t layer_stride_S,
                       int64_t layer_stride_ring, float* S, const RingPtrs& r,
                       const int32_t* slot_idx, const CursorPtrs& c, int only_flagged,
                       hipStream_t stream);

// The per-channel-gate (KDA) layer: ring g [num_slots, HV, L, K], window a
// [B*T, HV, K], dt_bias [HV, K].  Verify by replay from the checkpoint (a
// flagged row folds when fold_flagged), and the multi-layer exact fold.
bool kda_shape_supported(const gdn_shape& sh);

hipError_t launch_kda_verify(const gdn_shape& sh, const WindowPtrs& w, float* S, const int32_t* slot_idx,
                             const CursorPtrs& c, const RingPtrs& r, int write_ring, int fold_flagged, void* o,
                             hipStream_t stream);

hipError_t launch_kda_fold(const gdn_shape& sh, int num_layers, int64_t layer_stride_S, int64_t layer_stride_ring,
                           float* S, const RingPtrs& r, const int32_t* slot_idx, const CursorPtrs& c,
                           int only_flagged, hipStream_t stream);

hipError_t launch_snapshot(const gdn_shape& sh, const WindowPtrs& w, const float* S,
                           const int32_t* slot_idx, float* snap, void* o, const RingPtrs& r,
                           const int32_t* write_pos, const int32_t* cache_base, int write_ring,
                           hipStream_t stream);

hipError_t launch_snapshot_commit(const gdn_shape& sh, const float* snap,
                                  const int32_t* slot_idx, const int32_t* accept, float* S,
                                  hipStream_t stream);

hipError_t launch_advance(const gdn_shape& sh, const int32_t* slot_idx, const int32_t* accept,
                          int32_t* write_pos, int32_t* cache_base, int32_t* is_flush,
                          hipStream_t stream);

hipError_t launch_reset(const gdn_shape& sh, const int32_t* slots, int32_t n, int32_t init_flush,
                        int32_t* write_pos, int32_t* cache_base, int32_t* is_flush,
                        hipStream_t stream);

}  // namespace gdn
