// gdn_cursors.hip -- ring cursor arithmetic (integer only).
//
// Commit by accept count and the prefill->decode reset of the per-slot
// write_pos / cache_base / is_flush cursors (replayssm(B)SpecDecode §4.2,
// §8.1-8.2, §9.3, App. A.2).  One thread per row: rows of one call have
// distinct slots, so there is no cross-thread dependence.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

__global__ __launch_bounds__(256) void advance_kernel(int B, int T, int L, int max_spec,
                                                      int num_slots, const int32_t* slot_idx,
                                                      const int32_t* accept, int32_t* write_pos,
                                                      int32_t* cache_base, int32_t* is_flush)
{
    const int row = blockIdx.x * blockDim.x + threadIdx.x;
    if (row >= B)
        return;
    const int s = slot_idx[row];
    if (!valid_slot(s, num_slots))
        return;
    const int acc = min(max(accept[row], 0), T);
    int wp = clamp_wp(write_pos[s], L, T);
    if (is_flush[s] != 0) {
        // the history [base, base+wp) was folded by this step's verify:
        // move the head past it; the accepted drafts start the new history
        cache_base[s] = (cache_base[s] + wp) & (L - 1);
        wp = acc;
    } else {
        wp += acc;
    }
    write_pos[s] = wp;
    // early flush: fold before one more window could overflow the ring
    is_flush[s] = (wp + 2 * max_spec > L) ? 1 : 0;
}

__global__ __launch_bounds__(256) void reset_kernel(int n, int num_slots, int32_t init_flush,
                                                    const int32_t* slots, int32_t* write_pos,
                                                    int32_t* cache_base, int32_t* is_flush)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n)
        return;
    const int s = slots[i];
    if (!valid_slot(s, num_slots))
        return;
    write_pos[s] = 0;
    cache_base[s] = 0;
    is_flush[s] = init_flush;
}

hipError_t launch_advance(const gdn_shape& sh, const int32_t* slot_idx, const int32_t* accept,
                          int32_t* write_pos, int32_t* cache_base, int32_t* is_flush,
                          hipStream_t stream)
{
    if (sh.B == 0)
        return hipSuccess;
    const int blocks = (sh.B + 255) / 256;
    hipLaunchKernelGGL(advance_kernel, dim3(blocks), dim3(256), 0, stream, sh.B, sh.T, sh.L,
                       sh.max_spec_len, sh.num_slots, slot_idx, accept, write_pos, cache_base,
                       is_flush);
    return hipGetLastError();
}

hipError_t launch_reset(const gdn_shape& sh, const int32_t* slots, int32_t n, int32_t init_flush,
                        int32_t* write_pos, int32_t* cache_base, int32_t* is_flush,
                        hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    const int blocks = (n + 255) / 256;
    hipLaunchKernelGGL(reset_kernel, dim3(blocks), dim3(256), 0, stream, n, sh.num_slots,
                       init_flush, slots, write_pos, cache_base, is_flush);
    return hipGetLastError();
}

}  // namespace gdn
