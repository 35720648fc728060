// gdn_recurrence.hip -- the sequential gated delta rule on fp32 state rows:
//   * exact fold: replay committed ring records into the checkpoint in place
//     (PR #28695 summary: closed-loop exact fold from the raw records;
//      replayssm(B)SpecDecode §12.7: the checkpoint advances by the true,
//      contractive recurrence, never by the chunked closed form);
//   * snapshot verify: the baseline that stores a full state per draft token
//     (PR #36821 summary: a [K,V] fp32 snapshot per head-step);
//   * the snapshot path's commit copy.
//
// Layout: a workgroup of 4 waves owns a tile of 16 RPG rows of one (slot,
// value head) state (the snapshot verify: RPG = 1; the fold: RPG = 4 where
// the value rows allow 64-row tiles); each row lives on 16 lanes, lane c
// holding columns 64*m + 4*c + e.  State loads/stores are 256-byte contiguous per row and
// per instruction; the row dot products reduce over 16 lanes with DPP.  Both
// recurrence kernels run the identical per-record arithmetic (rnorm16,
// scale_decay, step_row from gdn_common.h, or step_rows4 where a lane group
// holds four rows and updates them on the matrix units, which gives each row
// step_row's bits: the head's decay is
// carried in a scalar, not applied to every element), which is what makes the
// fold of a recorded window bit-identical to the snapshot of the same window.
#include <type_traits>

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
    long long lsS, lsR;   // layer strides: fp32 elements of S, slots of the ring arrays
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

// Per-record quantities that do not depend on the state: the normalised key
// (columns of this lane) and the decay e^g.  Computed by one 16-lane group
// per record, with the same lane layout and reduction tree everywhere, so the
// fold and the snapshot verify see identical bits.
template <int EPL>
__device__ __forceinline__ void prep_key(const float (&kc)[EPL], float eps, float (&kh)[EPL])
{
    const float rn = rnorm16<EPL>(kc, eps);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        kh[e] = kc[e] * rn;
}

template <int K>
__device__ __forceinline__ void load_cols_f32(const float* row, int c, float (&x)[K / 16])
{
#pragma unroll
    for (int m = 0; m < K / 64; ++m) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(row + 64 * m + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            x[4 * m + e] = t[e];
    }
}

template <int K>
__device__ __forceinline__ void store_cols_f32(float* row, int c, const float (&x)[K / 16])
{
#pragma unroll
    for (int m = 0; m < K / 64; ++m)
        *reinterpret_cast<f32x4*>(row + 64 * m + 4 * c) =
            f32x4{x[4 * m], x[4 * m + 1], x[4 * m + 2], x[4 * m + 3]};
}

// Threads that load a batch's gates and betas (they may also load values).
constexpr int kGateT = 128;


// Records of the fold are staged through LDS in batches of kFoldBatch,
// double-buffered: the loads of batch i+1 are in flight while the sequential
// steps of batch i run from LDS.  Each thread loads the raw key columns it
// normalises itself (record tid / 16 of the batch, columns 64 m + 4 c .. +3),
// so raw keys never pass through LDS.
constexpr int kFoldBatch = 16;

// RPG state rows per 16-lane group: a tile is 16 RPG value rows.  Several
// rows per lane give each wave independent step chains to interleave.
template <class Act, int K, int RPG = 1>
struct FoldStage {
    static constexpr int VU = RPG * 16 * Act::bytes / 16;     // 16-byte units of a record's tile values
    static constexpr int VUB = kFoldBatch * VU;
    typedef typename std::conditional<Act::bytes == 4, uint4, uint2>::type KRaw;   // 4 activations
};

template <class Act, int K, int RPG = 1>
struct FoldShared {
    uint4 vbuf[2][FoldStage<Act, K, RPG>::VUB];     // this tile's values per record
    float gbuf[2][kFoldBatch], bbuf[2][kFoldBatch];  // decay e^g and beta
    float khs[2][kFoldBatch][K];                     // normalised keys
};

// Four raw activations widened to fp32 exactly as load4 widens them.
__device__ __forceinline__ f32x4 widen4(uint4 u)
{
    return f32x4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
}

__device__ __forceinline__ f32x4 widen4(uint2 u)
{
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                 __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
}

// Fold of one work item: the n committed records of slot s into the 16 RPG
// rows (tile) of one layer's value head hv.  Called uniformly by the
// workgroup.
template <class Act, int K, int RPG = 1, class P = const RecParams>
__device__ void fold_item(P& p, FoldShared<Act, K, RPG>& sh, int s, int n, int base,
                          int layer, int hv, int tile)
{
    using st = typename Act::storage;
    using FS = FoldStage<Act, K, RPG>;
    constexpr int TR = 16 * RPG;                   // rows of a tile
    using KRaw = typename FS::KRaw;
    constexpr int EPL = K / 16;
    constexpr int RB = kFoldBatch;
    auto& vbuf = sh.vbuf;
    auto& gbuf = sh.gbuf;
    auto& bbuf = sh.bbuf;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, grp = lane >> 4;
    const int row16 = w * 4 + grp;                 // lane group: rows row16 + 16 j of the tile
    const int vrow = tile * TR + row16;
    const int h = hv / (p.HV / p.H);
    const int L = p.L;

    // layer l: S at l * lsS elements, the ring arrays l * lsR slots in
    const size_t layer_recs = static_cast<size_t>(layer) * static_cast<size_t>(p.lsR) * L;
    float* Srow = p.S + static_cast<size_t>(layer) * static_cast<size_t>(p.lsS) +
                  ((static_cast<size_t>(s) * p.HV + hv) * p.V + vrow) * K;   // + 16 j K for row j
    const st* rk = static_cast<const st*>(p.rawk) + layer_recs * p.H * K +
                   (static_cast<size_t>(s) * p.H + h) * L * K;
    const st* rv = static_cast<const st*>(p.rawv) + layer_recs * p.HV * p.V +
                   (static_cast<size_t>(s) * p.HV + hv) * L * p.V + tile * TR;
    const size_t gofs = layer_recs * p.HV + (static_cast<size_t>(s) * p.HV + hv) * L;
    const float* rg = p.rg + gofs;
    const float* rb = p.rb + gofs;

    // registers of one batch in flight
    KRaw kreg[K / 64];
    uint4 vreg;
    float greg;
    auto issue = [&](int bi) {
        const int jk = bi * RB + row16;
#pragma unroll
        for (int m = 0; m < K / 64; ++m) {
            kreg[m] = KRaw{};
            if (jk < n) {
                const int ph = (base + jk) & (L - 1);
                kreg[m] = *reinterpret_cast<const KRaw*>(rk + static_cast<size_t>(ph) * K + 64 * m + 4 * c);
            }
        }
        vreg = uint4{0u, 0u, 0u, 0u};
        greg = 0.0f;
        if (tid < FS::VUB) {
            const int j = bi * RB + tid / FS::VU;
            if (j < n) {
                const int ph = (base + j) & (L - 1);
                vreg = reinterpret_cast<const uint4*>(rv + static_cast<size_t>(ph) * p.V)[tid % FS::VU];
            }
        }
        if (tid >= kGateT && tid < kGateT + 2 * RB) {
            const int r = tid - kGateT;
            const int j = bi * RB + (r % RB);
            if (j < n) {
                const int ph = (base + j) & (L - 1);
                greg = r < RB ? rg[ph] : rb[ph];
            }
        }
    };
    auto commit = [&](int buf) {
        if (tid < FS::VUB)
            vbuf[buf][tid] = vreg;
        if (tid >= kGateT && tid < kGateT + 2 * RB) {
            const int r = tid - kGateT;
            if (r < RB)
                gbuf[buf][r] = expf(greg);
            else
                bbuf[buf][r - RB] = greg;
        }
    };

    // 16 lane groups normalise the 16 keys of a batch in parallel, from the
    // registers their own loads filled
    auto prep = [&](int buf, int cnt) {
        const int jj = row16;
        float kc[EPL], kh[EPL];
#pragma unroll
        for (int m = 0; m < K / 64; ++m) {
            const f32x4 t = widen4(kreg[m]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                kc[4 * m + e] = t[e];
        }
        if (jj < cnt) {
            prep_key<EPL>(kc, p.eps, kh);
            store_cols_f32<K>(sh.khs[buf][jj], c, kh);
        }
    };

    issue(0);
    float sv[RPG][EPL];
#pragma unroll
    for (int j = 0; j < RPG; ++j)
        load_cols_f32<K>(Srow + static_cast<size_t>(16 * j) * K, c, sv[j]);
    commit(0);
    prep(0, min(RB, n));
    // The state rows' loads complete here (a use of each row register), so
    // the record loop carries no wait for them: placed there, such a wait
    // would also hold up, at the first record of every batch, the prefetch
    // of the next batch issued after the state's loads.
#pragma unroll
    for (int j = 0; j < RPG; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            asm volatile("" ::"v"(sv[j][e]));
    // four rows per lane group: the state per column, in step_rows4's
    // register order (rows 0, 2, 1, 3)
    constexpr bool kRows4 = RPG == 4;
    f32x4 av[kRows4 ? EPL : 1];
    if constexpr (kRows4) {
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            av[e] = f32x4{sv[0][e], sv[2][e], sv[1][e], sv[3][e]};
    }
    __syncthreads();

    float cs = 1.0f;      // the state is cs S' (step_row)
    // step_rows4: the row whose d this lane forms
    const bool odd = (c & 1) != 0, second = (c & 2) != 0;
    const int vofs = 16 * row4_of_lane(c);
    const int nbatch = (n + RB - 1) / RB;
    for (int bi = 0; bi < nbatch; ++bi) {
        const int buf = bi & 1;
        if (bi + 1 < nbatch)
            issue(bi + 1);
        const int cnt = min(RB, n - bi * RB);
        const st* vb = reinterpret_cast<const st*>(vbuf[buf]);
        for (int jj = 0; jj < cnt; ++jj) {
            float kh[EPL];
            load_cols_f32<K>(sh.khs[buf][jj], c, kh);
            const float dec = gbuf[buf][jj], bta = bbuf[buf][jj];
            float f;
            if (scale_decay(cs, dec, f)) {
                if constexpr (kRows4) {
#pragma unroll
                    for (int e = 0; e < EPL; ++e)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            av[e][i] *= f;
                } else {
#pragma unroll
                    for (int j = 0; j < RPG; ++j)
#pragma unroll
                        for (int e = 0; e < EPL; ++e)
                            sv[j][e] *= f;
                }
            }
            const float bc = scaled_beta(bta, cs);
            if constexpr (kRows4) {
                step_rows4<Act, EPL>(av, kh, vb + jj * TR + row16, vofs, odd, second, bc, bta);
            } else {
#pragma unroll
                for (int j = 0; j < RPG; ++j)
                    step_row<EPL>(sv[j], kh, Act::load(vb + jj * TR + 16 * j + row16), bc, bta);
            }
        }
        // buffer buf ^ 1 was last read by the previous batch's steps, which
        // every thread finished before the barrier that ended that batch
        if (bi + 1 < nbatch) {
            commit(buf ^ 1);
            prep(buf ^ 1, min(RB, n - (bi + 1) * RB));
        }
        __syncthreads();
    }

    if constexpr (kRows4) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            sv[0][e] = av[e][0];
            sv[2][e] = av[e][1];
            sv[1][e] = av[e][2];
            sv[3][e] = av[e][3];
        }
    }
#pragma unroll
    for (int j = 0; j < RPG; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            sv[j][e] = cs * sv[j][e];
        store_cols_f32<K>(Srow + static_cast<size_t>(16 * j) * K, c, sv[j]);
    }
}

// Persistent fold: every workgroup compacts the rows to fold (in chunks of
// kFoldRows) into LDS, then strides over the work items (row, layer, value
// head, 16-row tile).  Rows with nothing to fold cost no workgroup.
constexpr int kFoldRows = 512;

template <class Act, int K, int RPG>
__global__ __launch_bounds__(256) void fold_kernel(const RecParams p, int num_layers)
{
    __shared__ FoldShared<Act, K, RPG> sh;
    __shared__ int rows[kFoldRows];
    __shared__ int wcount[4];
    __shared__ int nrows;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int tiles = p.V / (16 * RPG);
    const int per_row = num_layers * p.HV * tiles;
    for (int c0 = 0; c0 < p.B; c0 += kFoldRows) {
        const int cend = min(c0 + kFoldRows, p.B);
        if (tid == 0)
            nrows = 0;
        __syncthreads();
        // Compaction in row order (ballot + prefix counts): every workgroup
        // must build the same list, since work items are indexed into it.
        for (int r0 = c0; r0 < cend; r0 += 256) {
            const int r = r0 + tid;
            bool keep = false;
            if (r < cend) {
                const int s = p.slot_idx[r];
                keep = valid_slot(s, p.num_slots) && (!p.only_flagged || p.is_flush[s] != 0) &&
                       clamp_wp(p.write_pos[s], p.L, p.T) > 0;
            }
            const unsigned long long m = __ballot(keep);
            if (lane == 0)
                wcount[wave] = __popcll(m);
            __syncthreads();
            int pos = nrows + __popcll(m & ((1ull << lane) - 1ull));
            for (int w = 0; w < wave; ++w)
                pos += wcount[w];
            if (keep)
                rows[pos] = r;
            __syncthreads();
            if (tid == 0)
                nrows += wcount[0] + wcount[1] + wcount[2] + wcount[3];
            __syncthreads();
        }
        const int nitems = nrows * per_row;
        for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
            const int row = rows[it / per_row];
            const int rem = it % per_row;
            const int tile = rem % tiles;
            const int lh = rem / tiles;              // layer * HV + hv
            const int s = p.slot_idx[row];
            fold_item<Act, K, RPG>(p, sh, s, clamp_wp(p.write_pos[s], p.L, p.T), p.cache_base[s],
                                   lh / p.HV, lh % p.HV, tile);
        }
        __syncthreads();
    }
}

// Window of the snapshot verify, staged once through LDS (T <= 16 tokens).
constexpr int kMaxT = 16;

// grid (V/16, B, HV), block 256
template <class Act, int K>
__global__ __launch_bounds__(256) void snapshot_kernel(const RecParams p)
{
    using st = typename Act::storage;
    constexpr int EPL = K / 16;
    constexpr int KU = K * Act::bytes / 16;      // 16-byte units per key/query row
    constexpr int VU = 16 * Act::bytes / 16;     // units of the tile's 16 values
    __shared__ uint4 kq[2 * kMaxT * KU];         // raw keys then queries
    __shared__ uint4 vv[kMaxT * VU];
    __shared__ float gs[kMaxT], bs[kMaxT];       // decay e^g and beta
    __shared__ float khs[kMaxT][K], qhs[kMaxT][K];   // normalised keys / queries

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, grp = lane >> 4;
    const int row16 = w * 4 + grp;
    const int vrow = blockIdx.x * 16 + row16;
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
    const size_t tok0 = static_cast<size_t>(b) * T;

    // ---- stage the window: keys, queries, this tile's values, gates
    for (int u = tid; u < 2 * T * KU; u += 256) {
        const int r = u / KU, part = u % KU;          // r < T: key t=r; else query t=r-T
        const st* src = (r < T ? static_cast<const st*>(p.k) : static_cast<const st*>(p.q)) +
                        ((tok0 + (r < T ? r : r - T)) * p.H + h) * K;
        kq[u] = reinterpret_cast<const uint4*>(src)[part];
    }
    for (int u = tid; u < T * VU; u += 256) {
        const st* src = static_cast<const st*>(p.v) + ((tok0 + u / VU) * p.HV + hv) * p.V +
                        blockIdx.x * 16;
        vv[u] = reinterpret_cast<const uint4*>(src)[u % VU];
    }
    if (tid < T) {
        const size_t tok = tok0 + tid;
        float g, beta;
        gdn_gate(Act::load(static_cast<const st*>(p.a) + tok * p.HV + hv),
                 Act::load(static_cast<const st*>(p.b) + tok * p.HV + hv), p.A_log[hv],
                 p.dt_bias[hv], p.softplus_threshold, g, beta);
        gs[tid] = g;
        bs[tid] = beta;
        if (p.write_ring && blockIdx.x == 0) {
            const size_t gi = (static_cast<size_t>(s) * p.HV + hv) * L + ((base + wpc + tid) & (L - 1));
            p.wg[gi] = g;
            p.wbeta[gi] = beta;
        }
    }
    __syncthreads();

    const st* kst = reinterpret_cast<const st*>(kq);
    const st* vst = reinterpret_cast<const st*>(vv);
    // 16 lane groups normalise the window's keys and queries in parallel
    if (row16 < T) {
        const int t = row16;
        float xc[EPL], xh[EPL];
        load_cols<Act, K>(kst + static_cast<size_t>(t) * K, c, xc);
        prep_key<EPL>(xc, p.eps, xh);
        store_cols_f32<K>(khs[t], c, xh);
        load_cols<Act, K>(kst + static_cast<size_t>(T + t) * K, c, xc);
        prep_key<EPL>(xc, p.eps, xh);
        store_cols_f32<K>(qhs[t], c, xh);
        if (c == 0)
            gs[t] = expf(gs[t]);
    }
    __syncthreads();

    float cs = 1.0f;      // the state is cs S' (step_row)
    for (int t = 0; t < T; ++t) {
        const size_t tok = tok0 + t;
        float kh[EPL], qh[EPL];
        load_cols_f32<K>(khs[t], c, kh);
        load_cols_f32<K>(qhs[t], c, qh);
        const float vc = Act::load(vst + t * 16 + row16);
        float f;
        if (scale_decay(cs, gs[t], f)) {
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                sv[e] *= f;
        }
        step_row<EPL>(sv, kh, vc, scaled_beta(bs[t], cs), bs[t]);

        float* srow = p.snap + (((static_cast<size_t>(b) * T + t) * p.HV + hv) * p.V + vrow) * K;
#pragma unroll
        for (int m = 0; m < K / 64; ++m)
            *reinterpret_cast<f32x4*>(srow + 64 * m + 4 * c) =
                f32x4{cs * sv[4 * m], cs * sv[4 * m + 1], cs * sv[4 * m + 2], cs * sv[4 * m + 3]};

        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            dot = __builtin_fmaf(sv[e], qh[e], dot);
        dot = group16_sum(dot);
        if (c == 0)
            static_cast<st*>(p.o)[(tok * p.HV + hv) * p.V + vrow] = Act::from_f32(p.scale * (cs * dot));

        if (p.write_ring) {
            const int ph = (base + wpc + t) & (L - 1);
            if (hv % G == 0 && blockIdx.x == 0 && w == 0 && grp == 0) {
                st* dk = static_cast<st*>(p.wrawk) + ((static_cast<size_t>(s) * p.H + h) * L + ph) * K;
#pragma unroll
                for (int m = 0; m < K / 64; ++m)
                    copy4<Act>(dk + 64 * m + 4 * c, kst + static_cast<size_t>(t) * K + 64 * m + 4 * c);
            }
            if (c == 0)
                static_cast<st*>(p.wrawv)[((static_cast<size_t>(s) * p.HV + hv) * L + ph) * p.V + vrow] =
                    vst[t * 16 + row16];
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

template <class Act, int RPG>
static hipError_t launch_fold_rpg(const gdn_shape& sh, int num_layers, const RecParams& p,
                                  hipStream_t stream)
{
    // persistent grid of 2048 workgroups, never more than items.  That is more
    // than fit at once (7 per compute unit at K = 128): the ones that wait for
    // a slot balance the load.  A grid of exactly the resident workgroups
    // was slower both for a few flagged rows and for folding every row.
    const long long items = static_cast<long long>(sh.B) * num_layers * sh.HV * (sh.V / (16 * RPG));
    const unsigned grid = static_cast<unsigned>(items < 2048 ? items : 2048);
    switch (sh.K) {
    case 64: hipLaunchKernelGGL((fold_kernel<Act, 64, RPG>), dim3(grid), dim3(256), 0, stream, p, num_layers); break;
    case 128: hipLaunchKernelGGL((fold_kernel<Act, 128, RPG>), dim3(grid), dim3(256), 0, stream, p, num_layers); break;
    case 256: hipLaunchKernelGGL((fold_kernel<Act, 256, RPG>), dim3(grid), dim3(256), 0, stream, p, num_layers); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Four state rows per lane group wherever the value rows allow 64-row tiles:
// the same time as one row per group when a few flagged rows are folded
// (56.8 against 56.5 us for 13 rows at the B=256 workload), 20% less when
// every row is (448 against 563 us), and the same bits.
template <class Act>
static hipError_t launch_fold_act(const gdn_shape& sh, int num_layers, const RecParams& p,
                                  hipStream_t stream)
{
    if (sh.V % 64 == 0)
        return launch_fold_rpg<Act, 4>(sh, num_layers, p, stream);
    if (sh.V % 32 == 0)
        return launch_fold_rpg<Act, 2>(sh, num_layers, p, stream);
    return launch_fold_rpg<Act, 1>(sh, num_layers, p, stream);
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

hipError_t launch_fold(const gdn_shape& sh, int num_layers, int64_t layer_stride_S,
                       int64_t layer_stride_ring, float* S, const RingPtrs& r,
                       const int32_t* slot_idx, const CursorPtrs& c, int only_flagged,
                       hipStream_t stream)
{
    if (sh.B == 0 || num_layers == 0)
        return hipSuccess;
    RecParams p = base_params(sh);
    p.lsS = layer_stride_S > 0 ? layer_stride_S
                               : static_cast<long long>(sh.num_slots) * sh.HV * sh.V * sh.K;
    p.lsR = layer_stride_ring > 0 ? layer_stride_ring : sh.num_slots;
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
