// gdn_dcache.hip -- GDN spec-verify through a ring of corrected deltas.
//
// The first-generation ring of the ReplaySSM walkthrough (replayssm(B)SpecDecode
// §1.1 table: d, k and g are cached per committed token) keeps, beside the raw
// records, each committed token's corrected delta
//     d_j = beta_j (v_j - e^{g_j} S_{j-1} kh_j)        (V values, fp32),
// the rank-1 factor its step adds along kh_j.  With the combined sequence
// (hist committed records, then the T window tokens), prefix gate sums Gam,
// normalised keys kh and queries qh and the frozen checkpoint S0, the state
// after record i is S_i = e^{Gam_i} S0 + sum_{j<=i} e^{Gam_i - Gam_j} d_j kh_j^T
// (the same induction as the raw-replay verify; §12.3).  A committed record's
// delta depends only on its prefix, so the stored d_j are exactly the history
// rows of the closed form's D, and only the window's deltas are unknown:
//     d_i = beta_i (v_i - e^{Gam_i} S0 kh_i) - sum_{j<hist} A_ij d_j
//                                           - sum_{hist<=j<i} A_ij d_j,
//     A_ij = beta_i e^{Gam_i - Gam_j} (kh_i . kh_j),
//     o_t  = scale (e^{Gam_i} S0 qh_t + sum_{j<=i} e^{Gam_i - Gam_j} (kh_j . qh_t) d_j),
// with i = hist + t.  The history's keys meet only the 2T window columns (no
// hist x hist Gram, no solve over the history), the checkpoint meets 2T
// columns (window keys and queries), and the history's values are replaced by
// its stored deltas.  The window's deltas are written to the d ring at
// logical positions write_pos + t beside the raw records, for the verifies
// that follow; the exact fold still replays the raw records.
//
// Execution: one workgroup (8 waves) per item (row, value head, value tile of
// up to 128 rows, 16 per wave):
//   1. the wave's checkpoint rows are issued as 128-bit loads (lane l: row
//      l % 8 (+8), key columns 32 i + 4 (l / 8)); the window's keys and queries
//      are normalised into LDS; the gates of the combined sequence are staged;
//   2. one wave forms the prefix sums of the gates; every thread forms dot
//      products of the history keys with the window columns; each wave forms
//      S0 [kh_w, qh_w] for its rows on MFMA 4x4x1 (sums over the eight key
//      groups by a rotate and lane swaps);
//   3. the dot products become the coupling (A) and output (F) coefficients;
//   4. four thread groups split the history, each value row summing its
//      stored deltas against the coefficients;
//   5. one thread per value row runs the window's T-step recurrence for its
//      deltas and forms the outputs; the others write the raw records.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kDcWaves = 8;
constexpr int kDcThreads = 64 * kDcWaves;
constexpr int kDcRows = 128;          // value rows per workgroup (16 per wave)
constexpr int kDcGroups = kDcThreads / kDcRows;   // thread groups over the history
// LDS arrays indexed by value row are stored column by column, so that the
// lanes of a wave (consecutive value rows) touch consecutive banks.  The
// column stride of SP is padded by 16 floats: its writes put four columns of
// 16 rows in one instruction, on disjoint banks.
constexpr int kSPS = kDcRows + 16;
constexpr int kTMax = 16;             // window tokens at most (max_spec_len <= 16)
constexpr int kDPre = 16;             // stored deltas per thread loaded at the start
constexpr float kLog2eDc = 1.4426950408889634f;

struct DcParams {
    int B, T, TP, H, HV, V, L, num_slots, write_ring, nvt;
    float scale, softplus_threshold, eps;
    const void *q, *k, *v, *a, *b;
    const float *A_log, *dt_bias;
    const float* S;
    const int32_t* slot_idx;
    const int32_t *write_pos, *cache_base, *is_flush;
    void* rawk;
    void* rawv;
    float* rg;
    float* rb;
    float* rd;
    void* o;
    // LDS carve-up, in floats
    int KX;            // row stride of the window columns
    int PC;            // columns per record: TP window keys, then TP queries
    int o_x, o_gam, o_bet, o_wg, o_p, o_sp, o_part;
};

__device__ __forceinline__ float swap16_sum_dc(float x)
{
    const unsigned u = __float_as_uint(x);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned lo = p[0], hi = p[1];
    return __uint_as_float(lo) + __uint_as_float(hi);
}

__device__ __forceinline__ float swap32_sum_dc(float x)
{
    const unsigned u = __float_as_uint(x);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned lo = p[0], hi = p[1];
    return __uint_as_float(lo) + __uint_as_float(hi);
}

// Sum over the eight lanes l + 8 c (c = 0..7) of a wave, delivered to each.
__device__ __forceinline__ float rows8_sum_dc(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    return swap32_sum_dc(swap16_sum_dc(x));
}

// Activation element i of a row as fp32 (exact widening).
template <class Act>
__device__ __forceinline__ float act_at(const void* base, size_t i)
{
    return Act::load(static_cast<const typename Act::storage*>(base) + i);
}

}  // namespace

// TM: window tokens at most for this instantiation (4, 8 or 16): the per-row
// register arrays are sized by it.  Two workgroups per compute unit (128
// VGPRs) up to K = 128; K = 256 holds twice the checkpoint registers and runs
// one.
template <class Act, int K, int TM>
__global__ __launch_bounds__(kDcThreads, K >= 256 ? 2 : 4) void dcache_verify_kernel(const DcParams p)
{
    extern __shared__ __align__(16) float sm[];
    float* Xs = sm + p.o_x;        // [PC][KX] normalised window keys, then queries
    // Element k of a window column sits at xs_col(k): each quarter of the key
    // (K / 4 elements, the share of one lane of a dot-product quad) is
    // followed by 4 unused floats, so the quad's reads fall on distinct banks
    // while each lane still reads (and loads) a contiguous quarter.  A row is
    // K + 16 floats.
    constexpr int KQ = K / 4;
    auto xs_col = [](int k) { return k + 4 * (k / KQ); };
    float* gam = sm + p.o_gam;     // [n] log2(e) * prefix sums of g (raw g until the scan)
    float* bet = sm + p.o_bet;     // [n] beta
    float* wg = sm + p.o_wg;       // [2 kTMax] window g then beta (for the ring)
    float* P = sm + p.o_p;         // [L][PC] dot products, then coefficients
    float* SP = sm + p.o_sp;       // [PC][kSPS] S0 times the window columns (column c, value row r)
    float* part = sm + p.o_part;   // [kDcGroups - 1][2 kTMax][kDcRows] history partial sums

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int item = blockIdx.x;
    const int vt = item % p.nvt;
    const int hv = (item / p.nvt) % p.HV;
    const int b = item / p.nvt / p.HV;
    const int s = p.slot_idx[b];
    if (!valid_slot(s, p.num_slots))
        return;                                    // padding row: nothing read or written
    const int T = p.T, TP = p.TP, PC = p.PC, L = p.L, HV = p.HV, H = p.H, V = p.V;
    const int G = HV / H, h = hv / G;
    const bool flagged = p.is_flush[s] != 0;
    const int wpc = clamp_wp(p.write_pos[s], L, T);
    const int base = p.cache_base[s];
    const int hist = flagged ? 0 : wpc;
    const int n = hist + T;
    const int v0 = vt * kDcRows;
    const int BV = (V - v0) < kDcRows ? (V - v0) : kDcRows;

    // ---- 1. Loads, small ones first: the waits for the gate inputs, window
    // values and window columns then never wait on the checkpoint stream
    // behind them (vector-memory waits count loads in issue order).
    const int grp = tid / kDcRows, vr = tid % kDcRows;   // (wave-uniform grp)
    // gate inputs of the combined sequence (record j = tid < n): history from
    // the ring, window a and b
    float gin_a = 0.0f, gin_b = 0.0f;
    const size_t gbase = (static_cast<size_t>(s) * HV + hv) * L;
    const bool gate_thread = tid < n;
    if (gate_thread) {
        if (tid < hist) {
            const int ph = (base + tid) & (L - 1);
            gin_a = p.rg[gbase + ph];
            gin_b = p.rb[gbase + ph];
        } else {
            const size_t tok = static_cast<size_t>(b) * T + (tid - hist);
            gin_a = act_at<Act>(p.a, tok * HV + hv);
            gin_b = act_at<Act>(p.b, tok * HV + hv);
        }
    }
    // the window values of this thread's value row (used in step 5 by group 0)
    float vwin[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
        vwin[i] = 0.0f;
    if (grp == 0 && vr < BV) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int ic = i < T ? i : T - 1;
            const size_t tok = static_cast<size_t>(b) * T + ic;
            vwin[i] = act_at<Act>(p.v, (tok * HV + hv) * V + v0 + vr);
        }
    }
    // the first window column of this wave (window keys are columns 0..TP-1,
    // queries TP..2TP-1; zero past T)
    auto column_loads = [&](int c, float (&x)[K / 64]) {
        const bool isq = c >= TP;
        const int t = isq ? c - TP : c;
#pragma unroll
        for (int e = 0; e < K / 64; ++e) {
            x[e] = 0.0f;
            if (t < T) {
                const size_t tok = static_cast<size_t>(b) * T + t;
                x[e] = act_at<Act>(isq ? p.q : p.k, (tok * H + h) * K + 64 * e + lane);
            }
        }
    };
    float x0[K / 64];
    column_loads(wave < PC ? wave : 0, x0);
    // checkpoint rows of this wave (in flight while the rest stages)
    const bool has_rows = wave * 16 < BV;
    const int r0 = v0 + (has_rows ? wave * 16 : 0);
    const float* Srow = p.S + ((static_cast<size_t>(s) * HV + hv) * V + r0 + (lane & 7)) * K + 4 * (lane >> 3);
    f32x4 sraw[K / 16];
#pragma unroll
    for (int i = 0; i < K / 16; ++i)
        sraw[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Srow + (i & 1) * 8 * K + (i >> 1) * 32));
    // the stored deltas this thread sums in step 4 (records grp + kDcGroups m,
    // the first kDPre of them); indices past the history are clamped to a
    // valid record and skipped in step 4
    const float* dring = p.rd + (static_cast<size_t>(s) * HV + hv) * L * V + v0 + vr;
    float dpre[kDPre];
#pragma unroll
    for (int m = 0; m < kDPre; ++m)
        dpre[m] = 0.0f;
    if (hist > 0 && vr < BV) {
#pragma unroll
        for (int m = 0; m < kDPre; ++m) {
            const int j = grp + kDcGroups * m;
            const int jc = j < hist ? j : hist - 1;
            dpre[m] = dring[static_cast<size_t>((base + jc) & (L - 1)) * V];
        }
    }

    // window columns normalised into LDS, one wave per column
    for (int c = wave; c < PC; c += kDcWaves) {
        const bool isq = c >= TP;
        const int t = isq ? c - TP : c;
        float x[K / 64];
        if (c == wave) {
#pragma unroll
            for (int e = 0; e < K / 64; ++e)
                x[e] = x0[e];
        } else {
            column_loads(c, x);
        }
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < K / 64; ++e)
            ss = __builtin_fmaf(x[e], x[e], ss);
        ss = group_sum<64>(ss);
        const float rn = t < T ? 1.0f / sqrtf(ss + p.eps) : 0.0f;
#pragma unroll
        for (int e = 0; e < K / 64; ++e)
            Xs[c * p.KX + xs_col(64 * e + lane)] = x[e] * rn;
    }
    // gates of the combined sequence: history as recorded, window computed
    if (gate_thread) {
        const int j = tid;
        float g = gin_a, be = gin_b;
        if (j >= hist) {
            gdn_gate(gin_a, gin_b, p.A_log[hv], p.dt_bias[hv], p.softplus_threshold, g, be);
            wg[j - hist] = g;
            wg[kTMax + j - hist] = be;
        }
        gam[j] = g;
        bet[j] = be;
    }
    __syncthreads();

    // ---- 2a. prefix sums of the gates (wave 0; two records per lane, n <= 128)
    if (wave == 0) {
        const int j0 = 2 * lane;
        const float g0 = j0 < n ? gam[j0] : 0.0f;
        const float g1 = j0 + 1 < n ? gam[j0 + 1] : 0.0f;
        const float pair = g0 + g1;
        float incl = pair;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(incl, d, 64);
            incl += lane >= d ? y : 0.0f;
        }
        const float excl = incl - pair;
        // (all lanes read before any writes: the shuffles above synchronise the wave)
        if (j0 < n)
            gam[j0] = (excl + g0) * kLog2eDc;
        if (j0 + 1 < n)
            gam[j0 + 1] = (excl + g0 + g1) * kLog2eDc;
    }
    // ---- 2b. dot products of every record's key with the window columns:
    // P[j][c] = kh_j . Xs[c] (history keys normalised here, window keys are
    // the normalised columns themselves).  Four lanes share a product, each
    // over a quarter of the key with all its loads issued first, and meet by
    // quad swaps.
    for (int t4 = tid; t4 < n * PC * 4; t4 += kDcThreads) {
        const int sub = t4 & 3, task = t4 >> 2;
        const int j = task / PC, c = task % PC;
        const float* xc = Xs + c * p.KX + xs_col(sub * KQ);
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, ss[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (j < hist) {
            const int ph = (base + j) & (L - 1);
            const typename Act::storage* kr = static_cast<const typename Act::storage*>(p.rawk) +
                                              ((static_cast<size_t>(s) * H + h) * L + ph) * K + sub * KQ;
            f32x4 kv[KQ / 4];
#pragma unroll
            for (int e = 0; e < KQ / 4; ++e)
                kv[e] = load4<Act>(kr + 4 * e);
#pragma unroll
            for (int e = 0; e < KQ / 4; ++e) {
                const f32x4 xv = *reinterpret_cast<const f32x4*>(xc + 4 * e);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    ss[u] = __builtin_fmaf(kv[e][u], kv[e][u], ss[u]);
                    acc[u] = __builtin_fmaf(kv[e][u], xv[u], acc[u]);
                }
            }
        } else {
            const float* xr = Xs + (j - hist) * p.KX + xs_col(sub * KQ);
#pragma unroll
            for (int e = 0; e < KQ / 4; ++e) {
                const f32x4 kv = *reinterpret_cast<const f32x4*>(xr + 4 * e);
                const f32x4 xv = *reinterpret_cast<const f32x4*>(xc + 4 * e);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    acc[u] = __builtin_fmaf(kv[u], xv[u], acc[u]);
            }
        }
        float a4 = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        float s4 = (ss[0] + ss[1]) + (ss[2] + ss[3]);
        a4 += dpp<0xB1>(a4);          // quad_perm [1,0,3,2]
        a4 += dpp<0x4E>(a4);          // quad_perm [2,3,0,1]
        s4 += dpp<0xB1>(s4);
        s4 += dpp<0x4E>(s4);
        if (sub == 0)
            P[j * PC + c] = j < hist ? a4 * (1.0f / sqrtf(s4 + p.eps)) : a4;
    }
    // ---- 2c. S0 [kh_w, qh_w] for this wave's 16 rows, four columns per group
    if (has_rows) {
        for (int cg = 0; cg < PC / 4; ++cg) {
            const float* xrow = Xs + (4 * cg + (lane & 3)) * p.KX;
            f32x4 a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0, b0 = a0, b1 = a0;
#pragma unroll
            for (int i = 0; i < K / 16; ++i) {
                const f32x4 za = *reinterpret_cast<const f32x4*>(xrow + xs_col(4 * (lane >> 3) + 32 * (i >> 1)));
                if (i & 1) {
                    a1 = __builtin_amdgcn_mfma_f32_4x4x1f32(za[0], sraw[i][0], a1, 0, 0, 0);
                    b1 = __builtin_amdgcn_mfma_f32_4x4x1f32(za[1], sraw[i][1], b1, 0, 0, 0);
                    a1 = __builtin_amdgcn_mfma_f32_4x4x1f32(za[2], sraw[i][2], a1, 0, 0, 0);
                    b1 = __builtin_amdgcn_mfma_f32_4x4x1f32(za[3], sraw[i][3], b1, 0, 0, 0);
                } else {
                    a0 = __builtin_amdgcn_mfma_f32_4x4x1f32(za[0], sraw[i][0], a0, 0, 0, 0);
                    b0 = __builtin_amdgcn_mfma_f32_4x4x1f32(za[1], sraw[i][1], b0, 0, 0, 0);
                    a0 = __builtin_amdgcn_mfma_f32_4x4x1f32(za[2], sraw[i][2], a0, 0, 0, 0);
                    b0 = __builtin_amdgcn_mfma_f32_4x4x1f32(za[3], sraw[i][3], b0, 0, 0, 0);
                }
            }
            // lane l, register r: column 4 cg + r of row 8 hh + l % 8 (hh = 0:
            // a0 + b0, 1: a1 + b1), partial over key group l / 8
            const f32x4 lo = a0 + b0, hi = a1 + b1;
            const int c = lane >> 3;
            float val = 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float sl = rows8_sum_dc(lo[r]), sh = rows8_sum_dc(hi[r]);
                val = c == r ? sl : (c == 4 + r ? sh : val);
            }
            const int row = wave * 16 + (lane & 7) + 8 * (c >> 2);
            SP[(4 * cg + (c & 3)) * kSPS + row] = val;
        }
    }
    __syncthreads();

    // ---- 3. coefficients: column i < T of record j couples window token i to
    // j (j < hist + i): beta e^{Gam_{h+i} - Gam_j} kh_i . kh_j; query column t
    // weighs d_j in output t (j <= hist + t): e^{Gam_{h+t} - Gam_j} kh_j . qh_t
    for (int task = tid; task < n * PC; task += kDcThreads) {
        const int j = task / PC, c = task % PC;
        const bool isq = c >= TP;
        const int t = isq ? c - TP : c;
        float coef = 0.0f;
        if (t < T) {
            const int i = hist + t;
            const bool live = isq ? j <= i : j < i;
            if (live) {
                const float w = exp2f(gam[i] - gam[j]);
                coef = (isq ? w : bet[i] * w) * P[task];
            }
        }
        P[task] = coef;
    }
    __syncthreads();

    // ---- 4. history through the stored deltas: each thread group takes
    // every kDcGroups-th record for its value row (the first kDPre from the
    // registers loaded at the start)
    float hA[TM], hF[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        hA[t] = 0.0f;
        hF[t] = 0.0f;
    }
    if (vr < BV) {
#pragma unroll
        for (int m = 0; m < kDPre; ++m) {
            const int j = grp + kDcGroups * m;
            if (j < hist) {                      // wave-uniform
                const float dj = dpre[m];
                const float* cj = P + j * PC;
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    if (t < T) {
                        hA[t] = __builtin_fmaf(cj[t], dj, hA[t]);
                        hF[t] = __builtin_fmaf(cj[TP + t], dj, hF[t]);
                    }
                }
            }
        }
        for (int j = grp + kDcGroups * kDPre; j < hist; j += kDcGroups) {
            const float dj = dring[static_cast<size_t>((base + j) & (L - 1)) * V];
            const float* cj = P + j * PC;
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                if (t < T) {
                    hA[t] = __builtin_fmaf(cj[t], dj, hA[t]);
                    hF[t] = __builtin_fmaf(cj[TP + t], dj, hF[t]);
                }
            }
        }
        if (grp > 0) {
            float* pr = part + (grp - 1) * 2 * kTMax * kDcRows + vr;
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                if (t < T) {
                    pr[t * kDcRows] = hA[t];
                    pr[(kTMax + t) * kDcRows] = hF[t];
                }
            }
        }
    }
    __syncthreads();

    // ---- 5. window deltas and outputs (group 0, one thread per value row);
    // raw records to the ring (other groups)
    const int wp_phys0 = base + wpc;
    if (grp == 0) {
        if (vr < BV) {
#pragma unroll
            for (int gq = 1; gq < kDcGroups; ++gq) {
                const float* pr = part + (gq - 1) * 2 * kTMax * kDcRows + vr;
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    if (t < T) {
                        hA[t] += pr[t * kDcRows];
                        hF[t] += pr[(kTMax + t) * kDcRows];
                    }
                }
            }
            const int v = v0 + vr;
            float dw[TM];
            const float* spr = SP + vr;
            using st = typename Act::storage;
            st* out = static_cast<st*>(p.o);
            float* dout = p.rd + (static_cast<size_t>(s) * HV + hv) * L * V + v;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                dw[i] = 0.0f;
                if (i < T) {
                    const int ii = hist + i;
                    float d = bet[ii] * (vwin[i] - exp2f(gam[ii]) * spr[i * kSPS]) - hA[i];
#pragma unroll
                    for (int i2 = 0; i2 < TM; ++i2)
                        if (i2 < i)
                            d = __builtin_fmaf(-P[(hist + i2) * PC + i], dw[i2], d);
                    dw[i] = d;
                    if (p.write_ring)
                        dout[static_cast<size_t>((wp_phys0 + i) & (L - 1)) * V] = d;
                }
            }
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                if (t < T) {
                    const int it = hist + t;
                    float acc = exp2f(gam[it]) * spr[(TP + t) * kSPS] + hF[t];
#pragma unroll
                    for (int i = 0; i < TM; ++i)
                        if (i <= t)
                            acc = __builtin_fmaf(P[(hist + i) * PC + TP + t], dw[i], acc);
                    const size_t tok = static_cast<size_t>(b) * T + t;
                    out[(tok * HV + hv) * V + v] = Act::from_f32(p.scale * acc);
                }
            }
        }
    } else if (p.write_ring) {
        // pre-mutation raw bits of the window: keys once per qk head (value
        // head hv % G == 0, value tile 0), this tile's values, gates (tile 0)
        using st = typename Act::storage;
        const int rt = tid - kDcRows;                 // 0 .. 3 kDcRows - 1
        const int nrt = kDcThreads - kDcRows;
        const st* kwin = static_cast<const st*>(p.k);
        const st* vwin = static_cast<const st*>(p.v);
        st* rk = static_cast<st*>(p.rawk) + (static_cast<size_t>(s) * H + h) * L * K;
        st* rv = static_cast<st*>(p.rawv) + (static_cast<size_t>(s) * HV + hv) * L * V + v0;
        if (hv % G == 0 && vt == 0) {
            for (int e = rt; e < T * K; e += nrt) {
                const int t = e / K, c = e % K;
                const size_t tok = static_cast<size_t>(b) * T + t;
                rk[static_cast<size_t>((wp_phys0 + t) & (L - 1)) * K + c] = kwin[(tok * H + h) * K + c];
            }
        }
        for (int e = rt; e < T * BV; e += nrt) {
            const int t = e / BV, c = e % BV;
            const size_t tok = static_cast<size_t>(b) * T + t;
            rv[static_cast<size_t>((wp_phys0 + t) & (L - 1)) * V + c] = vwin[(tok * HV + hv) * V + v0 + c];
        }
        if (vt == 0 && rt < T) {
            const int ph = (wp_phys0 + rt) & (L - 1);
            p.rg[gbase + ph] = wg[rt];
            p.rb[gbase + ph] = wg[kTMax + rt];
        }
    }
    // the checkpoint registers of waves without rows count as consumed
    if (!has_rows) {
#pragma unroll
        for (int i = 0; i < K / 16; ++i)
            asm volatile("" ::"v"(sraw[i][0]), "v"(sraw[i][1]), "v"(sraw[i][2]), "v"(sraw[i][3]));
    }
}

// ------------------------------------------------------------------- host

size_t dcache_lds_bytes(const gdn_shape& sh)
{
    const int TP = (sh.T + 3) & ~3;
    const int PC = 2 * TP;
    const int KX = sh.K + 16;
    size_t f = 0;
    f += static_cast<size_t>(PC) * KX;               // Xs
    f += 2 * static_cast<size_t>(sh.L);              // gam, bet
    f += 2 * kTMax;                                  // wg
    f += static_cast<size_t>(sh.L) * PC;             // P
    f += static_cast<size_t>(PC) * kSPS;             // SP
    f += static_cast<size_t>(kDcGroups - 1) * kDcRows * 2 * kTMax;   // part
    return f * 4;
}

template <class Act, int K, int TM>
static hipError_t launch_dc_k(const gdn_shape& sh, const DcParams& p, hipStream_t stream)
{
    auto kern = dcache_verify_kernel<Act, K, TM>;
    const size_t lds = dcache_lds_bytes(sh);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess)
            return e;
    }
    const unsigned grid = static_cast<unsigned>(sh.B) * sh.HV * p.nvt;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kDcThreads), lds, stream, p);
    return hipGetLastError();
}

template <class Act, int K>
static hipError_t launch_dc_t(const gdn_shape& sh, const DcParams& p, hipStream_t stream)
{
    if (sh.T <= 4)
        return launch_dc_k<Act, K, 4>(sh, p, stream);
    if (sh.T <= 8)
        return launch_dc_k<Act, K, 8>(sh, p, stream);
    return launch_dc_k<Act, K, kTMax>(sh, p, stream);
}

template <class Act>
static hipError_t launch_dc_act(const gdn_shape& sh, const DcParams& p, hipStream_t stream)
{
    switch (sh.K) {
    case 64: return launch_dc_t<Act, 64>(sh, p, stream);
    case 128: return launch_dc_t<Act, 128>(sh, p, stream);
    case 256: return launch_dc_t<Act, 256>(sh, p, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dcache_verify(const gdn_shape& sh, const WindowPtrs& w, const float* S,
                                const int32_t* slot_idx, const CursorPtrs& c, const RingPtrs& r,
                                float* ring_d, int write_ring, void* o, hipStream_t stream)
{
    if (sh.B == 0)
        return hipSuccess;
    DcParams p = {};
    p.B = sh.B;
    p.T = sh.T;
    p.TP = (sh.T + 3) & ~3;
    p.H = sh.H;
    p.HV = sh.HV;
    p.V = sh.V;
    p.L = sh.L;
    p.num_slots = sh.num_slots;
    p.write_ring = write_ring;
    p.nvt = (sh.V + kDcRows - 1) / kDcRows;
    p.scale = sh.scale;
    p.softplus_threshold = sh.softplus_threshold;
    p.eps = sh.l2norm_eps;
    p.q = w.q;
    p.k = w.k;
    p.v = w.v;
    p.a = w.a;
    p.b = w.b;
    p.A_log = w.A_log;
    p.dt_bias = w.dt_bias;
    p.S = S;
    p.slot_idx = slot_idx;
    p.write_pos = c.write_pos;
    p.cache_base = c.cache_base;
    p.is_flush = c.is_flush;
    p.rawk = r.rawk;
    p.rawv = r.rawv;
    p.rg = r.g;
    p.rb = r.beta;
    p.rd = ring_d;
    p.o = o;
    p.PC = 2 * p.TP;
    p.KX = sh.K + 16;   // rows read four at a time as 16-byte groups: a 64-byte pad keeps them off each other's banks
    p.o_x = 0;
    p.o_gam = p.o_x + p.PC * p.KX;
    p.o_bet = p.o_gam + sh.L;
    p.o_wg = p.o_bet + sh.L;
    p.o_p = p.o_wg + 2 * kTMax;
    p.o_sp = p.o_p + sh.L * p.PC;
    p.o_part = p.o_sp + p.PC * kSPS;
    return sh.act == GDN_BF16 ? launch_dc_act<ActBF16>(sh, p, stream)
                              : launch_dc_act<ActF32>(sh, p, stream);
}

}  // namespace gdn
