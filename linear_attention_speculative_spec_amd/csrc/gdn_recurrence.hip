// gdn_recurrence.hip -- the sequential gated delta rule on fp32 state rows:
//   * exact fold: replay committed ring records into the checkpoint in place
//     (PR #28695 summary: closed-loop exact fold from the raw records;
//      replayssm(B)SpecDecode §12.7: the checkpoint advances by the true,
//      contractive recurrence, never by the chunked closed form);
//   * snapshot verify: the baseline that stores a full state per draft token
//     (PR #36821 summary: a [K,V] fp32 snapshot per head-step);
//   * the snapshot path's commit copy.
//
// Layout: a workgroup of 4 waves owns 16 consecutive rows of one (slot, value
// head) state; each row lives on 16 lanes, lane c holding columns
// 64*m + 4*c + e.  State loads/stores are 256-byte contiguous per row and
// per instruction; the row dot products reduce over 16 lanes with DPP.  Both
// recurrence kernels run the identical per-record arithmetic (rnorm16,
// step_row from gdn_common.h), which is what makes the fold of a recorded
// window bit-identical to the snapshot of the same window.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

struct RecParams {
    int B, T, H, HV, V, L, num_slots;
    float scale, softplus_threshold, eps;
    // fold
    float* S;
    const void* rawk;
    const void* rawv;
    const float* rg;
    const float* rb;
    const int32_t* slot_idx;
    const int32_t* write_pos;
    const int32_t* cache_base;
    const int32_t* is_flush;
    int only_flagged;
    // snapshot
    const void *q, *k, *v, *a, *b;
    const float *A_log, *dt_bias;
    const float* S_in;
    float* snap;
    void* o;
    void* wrawk;
    void* wrawv;
    float* wg;
    float* wbeta;
    int write_ring;
};

template <class Act, int K>
__device__ __forceinline__ void load_cols(const typename Act::storage* row, int c,
                                          float (&x)[K / 16])
{
#pragma unroll
    for (int m = 0; m < K / 64; ++m) {
        const f32x4 t = load4<Act>(row + 64 * m + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            x[4 * m + e] = t[e];
    }
}

// grid (V/16, B, HV * num_layers), block 256
template <class Act, int K>
__global__ __launch_bounds__(256) void fold_kernel(const RecParams p)
{
    using st = typename Act::storage;
    constexpr int EPL = K / 16;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane & 15, grp = lane >> 4;
    const int vrow = blockIdx.x * 16 + w * 4 + grp;
    const int b = blockIdx.y;
    const int layer = blockIdx.z / p.HV, hv = blockIdx.z - layer * p.HV;
    const int h = hv / (p.HV / p.H);
    const int L = p.L;

    const int s = p.slot_idx[b];
    if (!valid_slot(s, p.num_slots))
        return;
    if (p.only_flagged && p.is_flush[s] == 0)
        return;
    const int n = clamp_wp(p.write_pos[s], L, p.T);
    if (n == 0)
        return;
    const int base = p.cache_base[s];

    const size_t ring_slots = static_cast<size_t>(p.num_slots) * L;
    float* Srow = p.S + static_cast<size_t>(layer) * p.num_slots * p.HV * p.V * K +
                  ((static_cast<size_t>(s) * p.HV + hv) * p.V + vrow) * K;
    const st* rk = static_cast<const st*>(p.rawk) + static_cast<size_t>(layer) * ring_slots * p.H * K +
                   (static_cast<size_t>(s) * p.H + h) * L * K;
    const st* rv = static_cast<const st*>(p.rawv) + static_cast<size_t>(layer) * ring_slots * p.HV * p.V +
                   (static_cast<size_t>(s) * p.HV + hv) * L * p.V + vrow;
    const size_t gofs = static_cast<size_t>(layer) * ring_slots * p.HV +
                        (static_cast<size_t>(s) * p.HV + hv) * L;
    const float* rg = p.rg + gofs;
    const float* rb = p.rb + gofs;

    float sv[EPL];
#pragma unroll
    for (int m = 0; m < K / 64; ++m) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(Srow + 64 * m + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            sv[4 * m + e] = t[e];
    }

    // records are independent of the state: fetch one ahead
    float kn[EPL], vn, gn, bn;
    {
        const int ph = base & (L - 1);
        load_cols<Act, K>(rk + static_cast<size_t>(ph) * K, c, kn);
        vn = Act::load(rv + static_cast<size_t>(ph) * p.V);
        gn = rg[ph];
        bn = rb[ph];
    }
    for (int j = 0; j < n; ++j) {
        float kc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            kc[e] = kn[e];
        const float vc = vn, gc = gn, bc = bn;
        if (j + 1 < n) {
            const int ph = (base + j + 1) & (L - 1);
            load_cols<Act, K>(rk + static_cast<size_t>(ph) * K, c, kn);
            vn = Act::load(rv + static_cast<size_t>(ph) * p.V);
            gn = rg[ph];
            bn = rb[ph];
        }
        const float rn = rnorm16<EPL>(kc, p.eps);
        float kh[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            kh[e] = kc[e] * rn;
        step_row<EPL>(sv, kh, vc, expf(gc), bc);
    }

#pragma unroll
    for (int m = 0; m < K / 64; ++m)
        *reinterpret_cast<f32x4*>(Srow + 64 * m + 4 * c) =
            f32x4{sv[4 * m], sv[4 * m + 1], sv[4 * m + 2], sv[4 * m + 3]};
}

// grid (V/16, B, HV), block 256
template <class Act, int K>
__global__ __launch_bounds__(256) void snapshot_kernel(const RecParams p)
{
    using st = typename Act::storage;
    constexpr int EPL = K / 16;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane & 15, grp = lane >> 4;
    const int vrow = blockIdx.x * 16 + w * 4 + grp;
    const int b = blockIdx.y, hv = blockIdx.z;
    const int G = p.HV / p.H, h = hv / G;
    const int T = p.T, L = p.L;

    const int s = p.slot_idx[b];
    if (!valid_slot(s, p.num_slots))
        return;

    const float* Srow = p.S_in + ((static_cast<size_t>(s) * p.HV + hv) * p.V + vrow) * K;
    float sv[EPL];
#pragma unroll
    for (int m = 0; m < K / 64; ++m) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(Srow + 64 * m + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            sv[4 * m + e] = t[e];
    }
    int wpc = 0, base = 0;
    if (p.write_ring) {
        wpc = clamp_wp(p.write_pos[s], L, T);
        base = p.cache_base[s];
    }
    const float A_log = p.A_log[hv], dt_bias = p.dt_bias[hv];

    for (int t = 0; t < T; ++t) {
        const size_t tok = static_cast<size_t>(b) * T + t;
        const st* krow = static_cast<const st*>(p.k) + (tok * p.H + h) * K;
        const st* qrow = static_cast<const st*>(p.q) + (tok * p.H + h) * K;
        const st* vptr = static_cast<const st*>(p.v) + (tok * p.HV + hv) * p.V + vrow;
        float kc[EPL], qc[EPL];
        load_cols<Act, K>(krow, c, kc);
        load_cols<Act, K>(qrow, c, qc);
        const float vc = Act::load(vptr);
        float g, beta;
        gdn_gate(Act::load(static_cast<const st*>(p.a) + tok * p.HV + hv),
                 Act::load(static_cast<const st*>(p.b) + tok * p.HV + hv), A_log, dt_bias,
                 p.softplus_threshold, g, beta);

        const float rn = rnorm16<EPL>(kc, p.eps);
        float kh[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            kh[e] = kc[e] * rn;
        step_row<EPL>(sv, kh, vc, expf(g), beta);

        float* srow = p.snap + (((static_cast<size_t>(b) * T + t) * p.HV + hv) * p.V + vrow) * K;
#pragma unroll
        for (int m = 0; m < K / 64; ++m)
            *reinterpret_cast<f32x4*>(srow + 64 * m + 4 * c) =
                f32x4{sv[4 * m], sv[4 * m + 1], sv[4 * m + 2], sv[4 * m + 3]};

        const float rq = rnorm16<EPL>(qc, p.eps);
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            dot = __builtin_fmaf(sv[e], qc[e] * rq, dot);
        dot = group16_sum(dot);
        if (c == 0)
            static_cast<st*>(p.o)[(tok * p.HV + hv) * p.V + vrow] = Act::from_f32(p.scale * dot);

        if (p.write_ring) {
            const int ph = (base + wpc + t) & (L - 1);
            if (hv % G == 0 && blockIdx.x == 0 && w == 0 && grp == 0) {
                st* dk = static_cast<st*>(p.wrawk) + ((static_cast<size_t>(s) * p.H + h) * L + ph) * K;
#pragma unroll
                for (int m = 0; m < K / 64; ++m)
                    copy4<Act>(dk + 64 * m + 4 * c, krow + 64 * m + 4 * c);
            }
            if (c == 0)
                static_cast<st*>(p.wrawv)[((static_cast<size_t>(s) * p.HV + hv) * L + ph) * p.V + vrow] =
                    *vptr;
            if (blockIdx.x == 0 && threadIdx.x == 0) {
                const size_t gi = (static_cast<size_t>(s) * p.HV + hv) * L + ph;
                p.wg[gi] = g;
                p.wbeta[gi] = beta;
            }
        }
    }
}

// S[slot] = snap[b, a-1] for rows accepting at least one draft.
// grid (ceil(HV*V*K/4 / 256), B), block 256
__global__ __launch_bounds__(256) void snapshot_commit_kernel(int T, int num_slots, size_t n4,
                                                              const f32x4* snap,
                                                              const int32_t* slot_idx,
                                                              const int32_t* accept, f32x4* S)
{
    const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int b = blockIdx.y;
    if (i >= n4)
        return;
    const int s = slot_idx[b];
    if (!valid_slot(s, num_slots))
        return;
    const int acc = min(max(accept[b], 0), T);
    if (acc == 0)
        return;
    S[static_cast<size_t>(s) * n4 + i] = snap[(static_cast<size_t>(b) * T + acc - 1) * n4 + i];
}

template <class Act>
static hipError_t launch_fold_act(const gdn_shape& sh, int num_layers, const RecParams& p,
                                  hipStream_t stream)
{
    const dim3 grid(sh.V / 16, sh.B, sh.HV * num_layers);
    switch (sh.K) {
    case 64: hipLaunchKernelGGL((fold_kernel<Act, 64>), grid, dim3(256), 0, stream, p); break;
    case 128: hipLaunchKernelGGL((fold_kernel<Act, 128>), grid, dim3(256), 0, stream, p); break;
    case 256: hipLaunchKernelGGL((fold_kernel<Act, 256>), grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class Act>
static hipError_t launch_snapshot_act(const gdn_shape& sh, const RecParams& p, hipStream_t stream)
{
    const dim3 grid(sh.V / 16, sh.B, sh.HV);
    switch (sh.K) {
    case 64: hipLaunchKernelGGL((snapshot_kernel<Act, 64>), grid, dim3(256), 0, stream, p); break;
    case 128: hipLaunchKernelGGL((snapshot_kernel<Act, 128>), grid, dim3(256), 0, stream, p); break;
    case 256: hipLaunchKernelGGL((snapshot_kernel<Act, 256>), grid, dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

static RecParams base_params(const gdn_shape& sh)
{
    RecParams p = {};
    p.B = sh.B;
    p.T = sh.T;
    p.H = sh.H;
    p.HV = sh.HV;
    p.V = sh.V;
    p.L = sh.L;
    p.num_slots = sh.num_slots;
    p.scale = sh.scale;
    p.softplus_threshold = sh.softplus_threshold;
    p.eps = sh.l2norm_eps;
    return p;
}

hipError_t launch_fold(const gdn_shape& sh, int num_layers, float* S, const RingPtrs& r,
                       const int32_t* slot_idx, const CursorPtrs& c, int only_flagged,
                       hipStream_t stream)
{
    if (sh.B == 0 || num_layers == 0)
        return hipSuccess;
    RecParams p = base_params(sh);
    p.S = S;
    p.rawk = r.rawk;
    p.rawv = r.rawv;
    p.rg = r.g;
    p.rb = r.beta;
    p.slot_idx = slot_idx;
    p.write_pos = c.write_pos;
    p.cache_base = c.cache_base;
    p.is_flush = c.is_flush;
    p.only_flagged = only_flagged;
    return sh.act == GDN_BF16 ? launch_fold_act<ActBF16>(sh, num_layers, p, stream)
                              : launch_fold_act<ActF32>(sh, num_layers, p, stream);
}

hipError_t launch_snapshot(const gdn_shape& sh, const WindowPtrs& w, const float* S,
                           const int32_t* slot_idx, float* snap, void* o, const RingPtrs& r,
                           const int32_t* write_pos, const int32_t* cache_base, int write_ring,
                           hipStream_t stream)
{
    if (sh.B == 0)
        return hipSuccess;
    RecParams p = base_params(sh);
    p.q = w.q;
    p.k = w.k;
    p.v = w.v;
    p.a = w.a;
    p.b = w.b;
    p.A_log = w.A_log;
    p.dt_bias = w.dt_bias;
    p.S_in = S;
    p.slot_idx = slot_idx;
    p.snap = snap;
    p.o = o;
    p.wrawk = r.rawk;
    p.wrawv = r.rawv;
    p.wg = r.g;
    p.wbeta = r.beta;
    p.write_pos = write_pos;
    p.cache_base = cache_base;
    p.write_ring = write_ring;
    return sh.act == GDN_BF16 ? launch_snapshot_act<ActBF16>(sh, p, stream)
                              : launch_snapshot_act<ActF32>(sh, p, stream);
}

hipError_t launch_snapshot_commit(const gdn_shape& sh, const float* snap,
                                  const int32_t* slot_idx, const int32_t* accept, float* S,
                                  hipStream_t stream)
{
    if (sh.B == 0)
        return hipSuccess;
    const size_t n4 = static_cast<size_t>(sh.HV) * sh.V * sh.K / 4;
    const dim3 grid(static_cast<unsigned>((n4 + 255) / 256), sh.B);
    hipLaunchKernelGGL(snapshot_commit_kernel, grid, dim3(256), 0, stream, sh.T, sh.num_slots, n4,
                       reinterpret_cast<const f32x4*>(snap), slot_idx, accept,
                       reinterpret_cast<f32x4*>(S));
    return hipGetLastError();
}

}  // namespace gdn
