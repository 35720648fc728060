// gdn_kda.hip -- the per-channel-gate (KDA) layer on the ReplaySSM ring:
// verify by replaying the committed records from the frozen checkpoint, the
// exact fold, and the ring write.
//
// A KDA layer's gate is a vector over the key channels: the ring keeps K fp32
// gate values per record beside raw k, raw v and a scalar beta (PR #36821
// summary, the KDA spec ring layout checked by _replayssm_ring_ok: g is
// [slots, HV, L, K] fp32; the same ring discipline and verify -> commit ->
// verify lifecycle as the GDN ring).  The step decays state column c by
// e^{g_c}:
//     S[:, c] <- e^{g_c} S[:, c];  u = S k_hat;  S <- S + beta (v - u) k_hat^T
// and o_t = scale S_t q_hat_t.  g_c = -exp(A_log) softplus(a_c + dt_bias_c),
// the GDN gate per channel.
//
// Execution: a persistent grid over items (row, value head, tile of 64
// value rows); a workgroup of 4 waves holds the tile's state rows in
// registers, four rows per 16-lane group (lane c holds columns 64 m + 4 c ..
// +3 of each), and steps them through the records: the committed history,
// staged through LDS in batches of 16 (the next batch's loads in flight
// while the current one is stepped) and stepped two records at a time, then
// the draft window with its outputs.  A row flagged for flush stores the
// state reached after its history (the exact fold) and verifies its window
// from there.  The work is the sequential recurrence: this kernel is bound
// by the fp32 vector ALU, not by HBM.
#include <type_traits>

#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

struct KdaParams {
    int B, T, H, HV, V, L, num_slots;
    float scale, softplus_threshold, eps;
    float* S;
    long long lsS, lsR;          // fold: layer strides (fp32 elements of S, slots of the rings)
    void* rawk;
    void* rawv;
    float* rg;                   // [slots, HV, L, K]
    float* rb;                   // [slots, HV, L]
    const int32_t* slot_idx;
    const int32_t *write_pos, *cache_base, *is_flush;
    const void *q, *k, *v, *a, *b;
    const float *A_log, *dt_bias;
    void* o;
    int write_ring, fold_flagged, only_flagged;
};

constexpr int kKdaThreads = 256;
constexpr int kKdaBatch = 16;   // records per LDS batch (and window tokens at most)
constexpr int kKdaRPG = 4;      // state rows per 16-lane group

// Records are replayed in pairs: two steps j, j+1 from state S are
//     u_j     = S . (d_j * kh_j)
//     u_j+1   = S . (d_j * d_j+1 * kh_j+1) + delta_j c_j,   c_j = kh_j . (d_j+1 * kh_j+1)
//     S      <- S * (d_j * d_j+1) + delta_j (kh_j * d_j+1)^T + delta_j+1 kh_j+1^T
// with d the channel decays e^{g} and delta = beta (v - u): the state takes
// one multiply and two FMAs per element for two records instead of two of
// each, and the two dots are independent.  Only products of decays appear,
// so nothing can overflow.  The five vectors and c_j of a pair are formed
// once per batch, shared by every state row.
template <class Act, int K>
struct KdaShared {
    static constexpr int TR = 16 * kKdaRPG;                 // tile rows
    static constexpr int VU = TR * Act::bytes / 16;         // 16-byte units of a record's tile values
    static constexpr int NP = kKdaBatch / 2;                // record pairs per batch
    uint4 vbuf[kKdaBatch * VU];                             // window: tile values per token
    float bvf[kKdaBatch * TR];                              // replay: beta v per record and tile row
    float bbuf[kKdaBatch];                                  // beta
    float cbuf[NP];                                         // c_j of each pair
    // per pair: d_j kh_j, d_j d_j+1 kh_j+1, d_j d_j+1, kh_j d_j+1, kh_j+1 (rows
    // 5 pp .. 5 pp + 4).  The window reuses the space: 16 rows each of keys,
    // queries and decays.
    float rows[48][K];
    __device__ float* pair_vec(int pp, int i) { return rows[5 * pp + i]; }
    __device__ float* win_key(int t) { return rows[t]; }
    __device__ float* win_query(int t) { return rows[16 + t]; }
    __device__ float* win_decay(int t) { return rows[32 + t]; }
};

template <int EPL>
__device__ __forceinline__ float kda_rnorm16(const float (&x)[EPL], float eps)
{
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        ss = __builtin_fmaf(x[e], x[e], ss);
    ss = group16_sum(ss);
    return 1.0f / sqrtf(ss + eps);
}

// S_row[:, c] <- e^{g_c} S_row[:, c]; u = S_row . k_hat; S_row += beta (v - u) k_hat
template <int EPL>
__device__ __forceinline__ void kda_step_row(float (&s)[EPL], const float (&kh)[EPL], const float (&dec)[EPL],
                                             float v, float beta)
{
    float u = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        s[e] = s[e] * dec[e];
        u = __builtin_fmaf(s[e], kh[e], u);
    }
    u = group16_sum(u);
    const float d = beta * (v - u);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        s[e] = __builtin_fmaf(d, kh[e], s[e]);
}

// Channel gate of the GDN form: -exp(A_log) softplus(a + dt_bias).
__device__ __forceinline__ float kda_gate_c(float a, float dt_bias, float A_log, float threshold)
{
    const float x = a + dt_bias;
    const float sp = x > threshold ? x : log1pf(expf(x));
    return -expf(A_log) * sp;
}

template <int K>
__device__ __forceinline__ void cols_f32(const float* row, int c, float (&x)[K / 16])
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
__device__ __forceinline__ void put_cols_f32(float* row, int c, const float (&x)[K / 16])
{
#pragma unroll
    for (int m = 0; m < K / 64; ++m)
        *reinterpret_cast<f32x4*>(row + 64 * m + 4 * c) =
            f32x4{x[4 * m], x[4 * m + 1], x[4 * m + 2], x[4 * m + 3]};
}

template <class Act, int K>
__device__ __forceinline__ void act_cols(const typename Act::storage* row, int c, float (&x)[K / 16])
{
#pragma unroll
    for (int m = 0; m < K / 64; ++m) {
        const f32x4 t = load4<Act>(row + 64 * m + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            x[4 * m + e] = t[e];
    }
}

// Steps the tile's state rows sv through the n committed records of slot s
// (layer `layer`, value head hv), reading the ring, in batches of 16.  The
// rows are held per column while the records are stepped (register i of av[e]
// is row 0, 2, 1, 3); the two rank-1 updates of a record pair run on 4x4x1
// fp32 matrix products, each rounded once as fmaf rounds.
template <class Act, int K, class P>
__device__ void kda_replay(P& p, KdaShared<Act, K>& sh, int s, int n, int base, int layer,
                           int hv, int tile, float (&sv)[kKdaRPG][K / 16])
{
    using st = typename Act::storage;
    using SH = KdaShared<Act, K>;
    constexpr int EPL = K / 16, RB = kKdaBatch, TR = SH::TR, VU = SH::VU;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, grp = lane >> 4;
    const int row16 = w * 4 + grp;
    static_assert(kKdaRPG == 4, "the record loop reduces four rows per lane group");
    const bool odd = (c & 1) != 0, second = (c & 2) != 0;
    const int vofs = 16 * row4_of_lane(c);     // the row whose d pair this lane forms
    const int h = hv / (p.HV / p.H);
    const int L = p.L;
    const size_t recs = static_cast<size_t>(layer) * static_cast<size_t>(p.lsR) * L;   // ring records before the layer
    const st* rk = static_cast<const st*>(p.rawk) + recs * p.H * K + (static_cast<size_t>(s) * p.H + h) * L * K;
    const st* rv = static_cast<const st*>(p.rawv) + recs * p.HV * p.V +
                   (static_cast<size_t>(s) * p.HV + hv) * L * p.V + tile * TR;
    const float* rg = p.rg + (recs * p.HV + (static_cast<size_t>(s) * p.HV + hv) * L) * K;
    const float* rb = p.rb + recs * p.HV + (static_cast<size_t>(s) * p.HV + hv) * L;

    // one batch in flight: lane c of group row16 holds record row16 of the
    // batch at columns 64 m + 4 c .. +3 (raw key and gate); a chunk of tile
    // values and a beta
    typedef typename std::conditional<Act::bytes == 4, uint4, uint2>::type KRaw;
    KRaw kreg[K / 64];
    f32x4 greg[K / 64];
    uint4 vreg;
    float breg, bvreg;
    auto issue = [&](int bi) {
        const int jk = bi * RB + row16;
        const size_t roff = static_cast<size_t>((base + jk) & (L - 1)) * K + 4 * c;
#pragma unroll
        for (int m = 0; m < K / 64; ++m) {
            kreg[m] = KRaw{};
            greg[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (jk < n) {
                kreg[m] = *reinterpret_cast<const KRaw*>(rk + roff + 64 * m);
                greg[m] = *reinterpret_cast<const f32x4*>(rg + roff + 64 * m);
            }
        }
        vreg = uint4{0u, 0u, 0u, 0u};
        bvreg = 0.0f;
        if (tid < RB * VU) {
            const int j = bi * RB + tid / VU;
            if (j < n) {
                const int ph = (base + j) & (L - 1);
                vreg = reinterpret_cast<const uint4*>(rv + static_cast<size_t>(ph) * p.V)[tid % VU];
                bvreg = rb[ph];                  // the record's beta, for beta v
            }
        }
        breg = 0.0f;
        if (tid < RB) {
            const int j = bi * RB + tid;
            if (j < n)
                breg = rb[(base + j) & (L - 1)];
        }
    };
    // Records past the batch's count act as identity steps: key 0, decay 1,
    // beta 0 and value 0 (so an odd count ends with a half-empty pair).
    auto commit = [&](int cnt) {
        if (tid < RB * VU) {
            // beta v in fp32: the step then forms delta = beta v - beta u in one FMA
            constexpr int EPC = 16 / Act::bytes;
            f32x4 w[EPC / 4];
            if constexpr (Act::bytes == 4) {
                w[0] = f32x4{__uint_as_float(vreg.x), __uint_as_float(vreg.y), __uint_as_float(vreg.z),
                             __uint_as_float(vreg.w)};
            } else {
                w[0] = f32x4{__uint_as_float(vreg.x << 16), __uint_as_float(vreg.x & 0xFFFF0000u),
                             __uint_as_float(vreg.y << 16), __uint_as_float(vreg.y & 0xFFFF0000u)};
                w[1] = f32x4{__uint_as_float(vreg.z << 16), __uint_as_float(vreg.z & 0xFFFF0000u),
                             __uint_as_float(vreg.w << 16), __uint_as_float(vreg.w & 0xFFFF0000u)};
            }
#pragma unroll
            for (int h4 = 0; h4 < EPC / 4; ++h4)
                *reinterpret_cast<f32x4*>(&sh.bvf[(tid / VU) * TR + (tid % VU) * EPC + 4 * h4]) = w[h4] * bvreg;
        }
        if (tid < RB)
            sh.bbuf[tid] = breg;
        float kc[EPL], kh[EPL], dk[EPL];
#pragma unroll
        for (int m = 0; m < K / 64; ++m) {
            f32x4 t;
            if constexpr (Act::bytes == 4)
                t = f32x4{__uint_as_float(kreg[m].x), __uint_as_float(kreg[m].y), __uint_as_float(kreg[m].z),
                          __uint_as_float(kreg[m].w)};
            else
                t = f32x4{__uint_as_float(kreg[m].x << 16), __uint_as_float(kreg[m].x & 0xFFFF0000u),
                          __uint_as_float(kreg[m].y << 16), __uint_as_float(kreg[m].y & 0xFFFF0000u)};
            const f32x4 gv = greg[m];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kc[4 * m + e] = t[e];
                dk[4 * m + e] = expf(gv[e]);     // gate 0 past the count: decay 1
            }
        }
        const bool live = row16 < cnt;
        const float r = kda_rnorm16<EPL>(kc, p.eps);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            kh[e] = live ? kc[e] * r : 0.0f;
        // the partner record (row16 ^ 1) sits in the paired 16-lane row
        float kp[EPL], dp[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            kp[e] = __shfl_xor(kh[e], 16, 64);
            dp[e] = __shfl_xor(dk[e], 16, 64);
        }
        const int pp = row16 >> 1;
        float x0[EPL], x1[EPL], x2[EPL];
        if ((row16 & 1) == 0) {        // record j: d_j kh_j, d_j d_j+1 kh_j+1, d_j d_j+1
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                x2[e] = dk[e] * dp[e];
                x0[e] = dk[e] * kh[e];
                x1[e] = x2[e] * kp[e];
            }
            put_cols_f32<K>(sh.pair_vec(pp, 0), c, x0);
            put_cols_f32<K>(sh.pair_vec(pp, 1), c, x1);
            put_cols_f32<K>(sh.pair_vec(pp, 2), c, x2);
        } else {                       // record j+1: kh_j d_j+1, kh_j+1 and c_j
            float cp = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                x0[e] = kp[e] * dk[e];
                cp = __builtin_fmaf(x0[e], kh[e], cp);
            }
            cp = group16_sum(cp);
            put_cols_f32<K>(sh.pair_vec(pp, 3), c, x0);
            put_cols_f32<K>(sh.pair_vec(pp, 4), c, kh);
            if (c == 0)
                sh.cbuf[pp] = cp;
        }
    };

    const int nbatch = (n + RB - 1) / RB;
    if (nbatch > 0)
        issue(0);
    // The state rows' loads complete here on every path (a use of each row
    // register), so that the record loop below carries no wait for them: a
    // wait placed there would also hold up, at the first record of every
    // batch, the prefetch of the next batch issued after the state's loads.
#pragma unroll
    for (int r = 0; r < kKdaRPG; ++r)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            asm volatile("" ::"v"(sv[r][e]));
    if (nbatch > 0)
        commit(min(RB, n));
    // the state per column for the matrix-unit updates, register i holding
    // row 0, 2, 1, 3 (the row whose d lane i of each quad forms)
    f32x4 av[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        av[e] = f32x4{sv[0][e], sv[2][e], sv[1][e], sv[3][e]};
    __syncthreads();
    // one LDS buffer: the next batch is committed after a barrier that ends
    // every thread's reads of the current one (its loads were in flight
    // meanwhile)
    for (int bi = 0; bi < nbatch; ++bi) {
        if (bi + 1 < nbatch)
            issue(bi + 1);
        const int cnt = min(RB, n - bi * RB);
        for (int pp = 0; pp < (cnt + 1) >> 1; ++pp) {
            float a0[EPL], a1[EPL];
            cols_f32<K>(sh.pair_vec(pp, 0), c, a0);
            cols_f32<K>(sh.pair_vec(pp, 1), c, a1);
            const float cj = sh.cbuf[pp];
            const float b0 = sh.bbuf[2 * pp], b1 = sh.bbuf[2 * pp + 1];
            // the four rows' sums reduced transposed (sum16_rows4: each row
            // gets group16_sum's bits); each lane forms its own row's d pair
            float w0[4], w1[4];   // by register
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w0[i] = 0.0f;
                w1[i] = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    w0[i] = __builtin_fmaf(av[e][i], a0[e], w0[i]);
                    w1[i] = __builtin_fmaf(av[e][i], a1[e], w1[i]);
                }
            }
            const float u0[kKdaRPG] = {w0[0], w0[2], w0[1], w0[3]};
            const float u1[kKdaRPG] = {w1[0], w1[2], w1[1], w1[3]};
            const float z0 = sum16_rows4(u0, odd, second);
            float z1 = sum16_rows4(u1, odd, second);
            const float bv0 = sh.bvf[(2 * pp) * TR + vofs + row16];
            const float bv1 = sh.bvf[(2 * pp + 1) * TR + vofs + row16];
            const float e0 = __builtin_fmaf(-b0, z0, bv0);
            z1 = __builtin_fmaf(e0, cj, z1);
            const float e1 = __builtin_fmaf(-b1, z1, bv1);
            // quads 1 and 3 hold the full sums; quads 0 and 2 take theirs
            const float d0 = quads13(e0), d1 = quads13(e1);
            float dd[EPL], kd[EPL], k1[EPL];
            cols_f32<K>(sh.pair_vec(pp, 2), c, dd);
            cols_f32<K>(sh.pair_vec(pp, 3), c, kd);
            cols_f32<K>(sh.pair_vec(pp, 4), c, k1);
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                f32x4 x;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    x[i] = av[e][i] * dd[e];
                x = __builtin_amdgcn_mfma_f32_4x4x1f32(d0, kd[e], x, 0, 0, 0);
                av[e] = __builtin_amdgcn_mfma_f32_4x4x1f32(d1, k1[e], x, 0, 0, 0);
            }
        }
        if (bi + 1 < nbatch) {
            __syncthreads();
            commit(min(RB, n - (bi + 1) * RB));
        }
        __syncthreads();
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        sv[0][e] = av[e][0];
        sv[2][e] = av[e][1];
        sv[1][e] = av[e][2];
        sv[3][e] = av[e][3];
    }
}

// The draft window of batch row b from the state sv: outputs, and with
// write_ring the window's records (raw k bits once per qk head, raw v bits,
// the K channel gates and beta) at logical positions wpc + t.
template <class Act, int K, class P>
__device__ void kda_window(P& p, KdaShared<Act, K>& sh, int b, int s, int wpc, int base, int hv,
                           int tile, float (&sv)[kKdaRPG][K / 16])
{
    using st = typename Act::storage;
    using SH = KdaShared<Act, K>;
    constexpr int EPL = K / 16, TR = SH::TR;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, grp = lane >> 4;
    const int row16 = w * 4 + grp;
    const int G = p.HV / p.H, h = hv / G;
    const int T = p.T, L = p.L;
    const size_t tok0 = static_cast<size_t>(b) * T;
    const bool ring = p.write_ring != 0;
    st* vb = reinterpret_cast<st*>(sh.vbuf);

    // keys and queries: one token per 16-lane group
    if (row16 < T) {
        const int t = row16;
        const st* kr = static_cast<const st*>(p.k) + ((tok0 + t) * p.H + h) * K;
        const st* qr = static_cast<const st*>(p.q) + ((tok0 + t) * p.H + h) * K;
        float xc[EPL], xh[EPL];
        act_cols<Act, K>(kr, c, xc);
        float r = kda_rnorm16<EPL>(xc, p.eps);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            xh[e] = xc[e] * r;
        put_cols_f32<K>(sh.win_key(t), c, xh);
        act_cols<Act, K>(qr, c, xc);
        r = kda_rnorm16<EPL>(xc, p.eps);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            xh[e] = xc[e] * r;
        put_cols_f32<K>(sh.win_query(t), c, xh);
        if (ring && hv % G == 0 && tile == 0) {
            const int ph = (base + wpc + t) & (L - 1);
            st* dk = static_cast<st*>(p.rawk) + ((static_cast<size_t>(s) * p.H + h) * L + ph) * K;
#pragma unroll
            for (int m = 0; m < K / 64; ++m)
                copy4<Act>(dk + 64 * m + 4 * c, kr + 64 * m + 4 * c);
        }
    }
    // the tile's values of each token
    for (int e = tid; e < T * TR; e += kKdaThreads) {
        const int t = e / TR, r = e % TR;
        const st val = static_cast<const st*>(p.v)[((tok0 + t) * p.HV + hv) * p.V + tile * TR + r];
        vb[t * TR + r] = val;
        if (ring)
            static_cast<st*>(p.rawv)[((static_cast<size_t>(s) * p.HV + hv) * L + ((base + wpc + t) & (L - 1))) * p.V +
                                     tile * TR + r] = val;
    }
    // channel gates and betas of each token
    const float A_log = p.A_log[hv];
    for (int e = tid; e < T * K; e += kKdaThreads) {
        const int t = e / K, ch = e % K;
        const float g = kda_gate_c(Act::load(static_cast<const st*>(p.a) + ((tok0 + t) * p.HV + hv) * K + ch),
                                   p.dt_bias[static_cast<size_t>(hv) * K + ch], A_log, p.softplus_threshold);
        sh.win_decay(t)[ch] = expf(g);
        if (ring && tile == 0)
            p.rg[((static_cast<size_t>(s) * p.HV + hv) * L + ((base + wpc + t) & (L - 1))) * K + ch] = g;
    }
    if (tid < T) {
        const int t = tid;
        const float bv = Act::load(static_cast<const st*>(p.b) + (tok0 + t) * p.HV + hv);
        const float beta = 1.0f / (1.0f + expf(-bv));
        sh.bbuf[t] = beta;
        if (ring && tile == 0)
            p.rb[(static_cast<size_t>(s) * p.HV + hv) * L + ((base + wpc + t) & (L - 1))] = beta;
    }
    __syncthreads();
    for (int t = 0; t < T; ++t) {
        {
            float kh[EPL], dk[EPL];
            cols_f32<K>(sh.win_key(t), c, kh);
            cols_f32<K>(sh.win_decay(t), c, dk);
            const float bta = sh.bbuf[t];
#pragma unroll
            for (int r = 0; r < kKdaRPG; ++r)
                kda_step_row<EPL>(sv[r], kh, dk, Act::load(vb + t * TR + 16 * r + row16), bta);
        }
        float qh[EPL];
        cols_f32<K>(sh.win_query(t), c, qh);
#pragma unroll
        for (int r = 0; r < kKdaRPG; ++r) {
            float dot = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
                dot = __builtin_fmaf(sv[r][e], qh[e], dot);
            dot = group16_sum(dot);
            if (c == 0)
                static_cast<st*>(p.o)[((tok0 + t) * p.HV + hv) * p.V + tile * TR + 16 * r + row16] =
                    Act::from_f32(p.scale * dot);
        }
    }
    __syncthreads();
}

// kVerify: every row replays its history (a flagged row: folds it when
// fold_flagged, else it has none) and verifies its window.  Otherwise: the
// exact fold of every layer's rows (only flagged ones with only_flagged).
// The launch arguments in the kernel-argument segment (constant address
// space), read through a pointer laundered between phases so that no
// argument stays live across the replay and the window (kept live, they
// overflow the scalar registers).
typedef const __attribute__((address_space(4))) KdaParams KKda;

__device__ __forceinline__ KKda* launder_kda(KKda* pk)
{
    asm volatile("" : "+s"(pk));
    return pk;
}

template <class Act, int K, bool kVerify>
__global__ __launch_bounds__(kKdaThreads, K <= 128 ? 4 : 2) void kda_kernel(const KdaParams p_arg, int num_layers)
{
    (void)p_arg;   // read through the argument segment instead
    KKda* pk = launder_kda((KKda*)__builtin_amdgcn_kernarg_segment_ptr());
    __shared__ KdaShared<Act, K> sh;
    constexpr int EPL = K / 16, TR = KdaShared<Act, K>::TR;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, grp = lane >> 4;
    const int row16 = w * 4 + grp;
    const int tiles = pk->V / TR;
    const int per_row = num_layers * pk->HV * tiles;
    const int nitems = pk->B * per_row;
    for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
        pk = launder_kda(pk);
        KKda& p = *pk;
        const int b = it / per_row;
        const int rem = it % per_row;
        const int tile = rem % tiles;
        const int lh = rem / tiles;                  // layer * HV + hv
        const int layer = lh / p.HV, hv = lh % p.HV;
        const int s = p.slot_idx[b];
        if (!valid_slot(s, p.num_slots))
            continue;                                // padding row: nothing read or written
        // the fold reads is_flush only with only_flagged (it may be NULL otherwise)
        const bool flagged = (kVerify || p.only_flagged) && p.is_flush[s] != 0;
        const int wpc = clamp_wp(p.write_pos[s], p.L, p.T);
        const int base = p.cache_base[s];
        int n;
        bool store;
        if constexpr (kVerify) {
            n = flagged ? (p.fold_flagged ? wpc : 0) : wpc;
            store = flagged && p.fold_flagged;
        } else {
            if (p.only_flagged && !flagged)
                continue;
            n = wpc;
            store = true;
        }
        float* Srow = p.S + static_cast<size_t>(layer) * static_cast<size_t>(p.lsS) +
                      ((static_cast<size_t>(s) * p.HV + hv) * p.V + tile * TR + row16) * K;
        float sv[kKdaRPG][EPL];
#pragma unroll
        for (int r = 0; r < kKdaRPG; ++r)
            cols_f32<K>(Srow + static_cast<size_t>(16 * r) * K, c, sv[r]);
        kda_replay<Act, K>(*launder_kda(pk), sh, s, n, base, layer, hv, tile, sv);
        if (store) {
#pragma unroll
            for (int r = 0; r < kKdaRPG; ++r)
                put_cols_f32<K>(Srow + static_cast<size_t>(16 * r) * K, c, sv[r]);
        }
        if constexpr (kVerify)
            kda_window<Act, K>(*launder_kda(pk), sh, b, s, wpc, base, hv, tile, sv);
    }
}

template <class Act, bool kVerify>
hipError_t launch_kda_act(const gdn_shape& sh, int num_layers, const KdaParams& p, hipStream_t stream)
{
    const long long items = static_cast<long long>(sh.B) * num_layers * sh.HV * (sh.V / (16 * kKdaRPG));
    const unsigned grid = static_cast<unsigned>(items < 2048 ? (items > 0 ? items : 1) : 2048);
    switch (sh.K) {
    case 64: hipLaunchKernelGGL((kda_kernel<Act, 64, kVerify>), dim3(grid), dim3(kKdaThreads), 0, stream, p, num_layers); break;
    case 128: hipLaunchKernelGGL((kda_kernel<Act, 128, kVerify>), dim3(grid), dim3(kKdaThreads), 0, stream, p, num_layers); break;
    case 256: hipLaunchKernelGGL((kda_kernel<Act, 256, kVerify>), dim3(grid), dim3(kKdaThreads), 0, stream, p, num_layers); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

KdaParams kda_params(const gdn_shape& sh, float* S, const RingPtrs& r, const int32_t* slot_idx,
                     const CursorPtrs& c)
{
    KdaParams p = {};
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
    p.S = S;
    p.lsS = static_cast<long long>(sh.num_slots) * sh.HV * sh.V * sh.K;
    p.lsR = sh.num_slots;
    p.rawk = r.rawk;
    p.rawv = r.rawv;
    p.rg = r.g;
    p.rb = r.beta;
    p.slot_idx = slot_idx;
    p.write_pos = c.write_pos;
    p.cache_base = c.cache_base;
    p.is_flush = c.is_flush;
    return p;
}

}  // namespace

bool kda_shape_supported(const gdn_shape& sh)
{
    return sh.V % (16 * kKdaRPG) == 0 && sh.T <= kKdaBatch;
}

hipError_t launch_kda_verify(const gdn_shape& sh, const WindowPtrs& w, float* S, const int32_t* slot_idx,
                             const CursorPtrs& c, const RingPtrs& r, int write_ring, int fold_flagged, void* o,
                             hipStream_t stream)
{
    if (sh.B == 0)
        return hipSuccess;
    KdaParams p = kda_params(sh, S, r, slot_idx, c);
    p.q = w.q;
    p.k = w.k;
    p.v = w.v;
    p.a = w.a;
    p.b = w.b;
    p.A_log = w.A_log;
    p.dt_bias = w.dt_bias;
    p.o = o;
    p.write_ring = write_ring;
    p.fold_flagged = fold_flagged;
    return sh.act == GDN_BF16 ? launch_kda_act<ActBF16, true>(sh, 1, p, stream)
                              : launch_kda_act<ActF32, true>(sh, 1, p, stream);
}

hipError_t launch_kda_fold(const gdn_shape& sh, int num_layers, int64_t layer_stride_S, int64_t layer_stride_ring,
                           float* S, const RingPtrs& r, const int32_t* slot_idx, const CursorPtrs& c,
                           int only_flagged, hipStream_t stream)
{
    if (sh.B == 0 || num_layers == 0)
        return hipSuccess;
    KdaParams p = kda_params(sh, S, r, slot_idx, c);
    if (layer_stride_S > 0)
        p.lsS = layer_stride_S;
    if (layer_stride_ring > 0)
        p.lsR = layer_stride_ring;
    p.only_flagged = only_flagged;
    return sh.act == GDN_BF16 ? launch_kda_act<ActBF16, false>(sh, num_layers, p, stream)
                              : launch_kda_act<ActF32, false>(sh, num_layers, p, stream);
}

}  // namespace gdn
