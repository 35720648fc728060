// gdn_verify.hip -- GDN ring spec-verify: outputs of the whole draft window
// from the frozen checkpoint plus the raw ring history, in closed form.
//
// Math (replayssm(B)SpecDecode §1.1 table and §12.3-12.4; the page's formulas
// are stripped, this is the reading that the recurrence determines).  For one
// (row, value head) let the combined sequence i = 0..n-1 be the hist committed
// ring records followed by the T window tokens, Gam_i = sum_{m<=i} g_m, kh/qh
// the l2-normalised raw keys/queries, S0 the checkpoint (V x K).  Then
//     S_i = e^{Gam_i} S0 + sum_{j<=i} e^{Gam_i-Gam_j} d_j kh_j^T,
//     (I + A) D = R,  A_ij = beta_i e^{Gam_i-Gam_j} (kh_i . kh_j)   (j < i),
//                     R_i  = beta_i (v_i - e^{Gam_i} S0 kh_i),
//     o_t = scale (e^{Gam_{h+t}} S0 qh_t + sum_j F_jt d_j),
//     F_jt = e^{Gam_{h+t}-Gam_j} (kh_j . qh_t) [j <= h+t],   h = hist,
// so with M = (I + A)^{-T} F (n x T):   O^T = e^{Gam_win} (S0 Qh^T) + R^T M.
// Only the T columns of M are solved (a unit upper-triangular back
// substitution), never the n x V deltas and never a per-token state.
//
// Work decomposition (grid = (V/BV, B, HV), one workgroup per row, value head
// and BV-wide value tile; BV = 16 * waves):
//   1. each wave issues its 16 checkpoint rows (V index) as 128-bit loads into
//      registers, 64 contiguous bytes per row per instruction;
//   2. the workgroup stages X = [raw history keys; window keys; window
//      queries] in LDS as bf16 (fp32 activations: a bf16 hi + lo pair), with
//      the per-row l2 norms reduced over the lanes that loaded the row, and the
//      value tile of the same records; window records are copied to the ring
//      on the way (pre-mutation raw bits, single writer per qk head);
//   3. gates: ring g/beta for history, fused gating for the window, prefix
//      sums by a wave scan;
//   4. Gram tiles k k^T (strictly lower) and k q^T on MFMA 16x16x32 bf16,
//      exact products of raw bf16 keys, scaled afterwards into A and F;
//   5. back substitution for M, one window column per wave;
//   6. each wave splits its fp32 checkpoint rows into bf16 hi + lo and
//      projects them onto X with MFMA (P = X S0^T, hi and lo accumulated in
//      fp32), turns the key rows into R and accumulates O on MFMA 16x16x4 fp32
//      seeded with the query rows.
// The checkpoint read dominates the bytes; everything else stays on chip.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

struct VerifyParams {
    int B, T, H, HV, V, L, LP, num_slots, BVP, write_ring;
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
    void* o;
};

static inline int round16(int x) { return (x + 15) & ~15; }

// LDS carve-up shared by host and device.
struct VerifyLds {
    size_t x_hi, x_lo, rn, gam, bet, vs, as, fs, total;
};

__host__ __device__ inline VerifyLds verify_lds(int K, int LP, int BVP, int act_bytes)
{
    VerifyLds l;
    const size_t KP = static_cast<size_t>(K) + 8;
    const size_t NXR = static_cast<size_t>(LP) + 16;
    l.x_hi = 0;
    l.x_lo = l.x_hi + NXR * KP * 2;
    l.rn = l.x_lo + (act_bytes == 4 ? NXR * KP * 2 : 0);
    l.gam = l.rn + NXR * 4;
    l.bet = l.gam + static_cast<size_t>(LP) * 4;
    l.vs = l.bet + static_cast<size_t>(LP) * 4;
    l.as = l.vs + static_cast<size_t>(LP) * BVP * act_bytes;
    l.fs = l.as + static_cast<size_t>(LP) * LP * 4;
    l.total = l.fs + static_cast<size_t>(LP) * 16 * 4;
    return l;
}

// 8 consecutive activations: raw storage words and their fp32 values.
template <class Act>
struct Chunk8 {
    uint4 raw[Act::bytes / 2];
    float x[8];
};

template <class Act>
__device__ __forceinline__ void load8(const typename Act::storage* src, Chunk8<Act>& ch)
{
    if constexpr (Act::bytes == 2) {
        ch.raw[0] = *reinterpret_cast<const uint4*>(src);
        const uint32_t w[4] = {ch.raw[0].x, ch.raw[0].y, ch.raw[0].z, ch.raw[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ch.x[2 * i] = __uint_as_float(w[i] << 16);
            ch.x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        ch.raw[0] = *reinterpret_cast<const uint4*>(src);
        ch.raw[1] = *reinterpret_cast<const uint4*>(src + 4);
        const uint32_t w[8] = {ch.raw[0].x, ch.raw[0].y, ch.raw[0].z, ch.raw[0].w,
                               ch.raw[1].x, ch.raw[1].y, ch.raw[1].z, ch.raw[1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ch.x[i] = __uint_as_float(w[i]);
    }
}

template <class Act>
__device__ __forceinline__ void store8(typename Act::storage* dst, const Chunk8<Act>& ch)
{
    *reinterpret_cast<uint4*>(dst) = ch.raw[0];
    if constexpr (Act::bytes == 4)
        *reinterpret_cast<uint4*>(dst + 4) = ch.raw[1];
}

__device__ __forceinline__ float readlane_f(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Position of natural column k (within its 32-wide step) in the MFMA operand
// order: lane group g holds k = 4g..4g+3 and 16+4g..16+4g+3 as its 8 slots.
// Chunk c (8 natural columns, c = 0..3 of the step) splits into two halves.
__device__ __forceinline__ int perm_pos(int kl)
{
    return kl < 16 ? 8 * (kl >> 2) : 8 * ((kl - 16) >> 2) + 4;
}

template <class Act, int K>
__global__ __launch_bounds__(512) void verify_kernel(const VerifyParams p)
{
    using st = typename Act::storage;
    constexpr bool kF32 = Act::bytes == 4;
    constexpr int KS = K / 32;   // MFMA k-steps
    constexpr int CPR = K / 8;   // 8-element chunks per X row
    constexpr int KP = K + 8;    // LDS row stride of X (bf16 elements)

    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NT = blockDim.x, NW = NT >> 6, BV = NW * 16;
    const int col = lane & 15, grp = lane >> 4;
    const int vt = blockIdx.x, b = blockIdx.y, hv = blockIdx.z;
    const int G = p.HV / p.H, h = hv / G;
    const int T = p.T, L = p.L, LP = p.LP;

    const int s = p.slot_idx[b];
    if (!valid_slot(s, p.num_slots))
        return;
    const bool flagged = p.is_flush[s] != 0;
    const int wpc = clamp_wp(p.write_pos[s], L, T);
    const int base = p.cache_base[s];
    const int hist = flagged ? 0 : wpc;
    const int n = hist + T;
    const int NB = (n + 15) >> 4;   // 16-row blocks of keys
    const int NQ0 = NB << 4;        // first query row of X
    const int NXA = NQ0 + 16;       // X rows in use

    const VerifyLds lay = verify_lds(K, LP, p.BVP, Act::bytes);
    uint16_t* Xhi = reinterpret_cast<uint16_t*>(smem + lay.x_hi);
    uint16_t* Xlo = reinterpret_cast<uint16_t*>(smem + lay.x_lo);
    float* rnX = reinterpret_cast<float*>(smem + lay.rn);
    float* gam = reinterpret_cast<float*>(smem + lay.gam);
    float* bet = reinterpret_cast<float*>(smem + lay.bet);
    st* Vs = reinterpret_cast<st*>(smem + lay.vs);
    float* As = reinterpret_cast<float*>(smem + lay.as);
    float* Fs = reinterpret_cast<float*>(smem + lay.fs);

    // ---- 1. checkpoint rows of this wave's 16 value columns -> registers
    const int vcol = vt * BV + wave * 16 + col;
    const float* Srow = p.S + ((static_cast<size_t>(s) * p.HV + hv) * p.V + vcol) * K;
    f32x4 sraw[2 * KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        sraw[2 * ks] = *reinterpret_cast<const f32x4*>(Srow + 32 * ks + 4 * grp);
        sraw[2 * ks + 1] = *reinterpret_cast<const f32x4*>(Srow + 32 * ks + 16 + 4 * grp);
    }

    // ---- 2. X rows: history keys, window keys, window queries (+ norms)
    const st* kwin = static_cast<const st*>(p.k);
    const st* qwin = static_cast<const st*>(p.q);
    st* ringk = static_cast<st*>(p.rawk) + (static_cast<size_t>(s) * p.H + h) * L * K;
    const bool k_writer = p.write_ring && (hv % G == 0) && vt == 0;
    for (int it = 0; it * NT < NXA * CPR; ++it) {
        const int idx = it * NT + tid;
        const int row = idx / CPR, ch = idx % CPR;
        const st* src = nullptr;
        if (row < hist)
            src = ringk + static_cast<size_t>((base + row) & (L - 1)) * K;
        else if (row < n)
            src = kwin + ((static_cast<size_t>(b) * T + (row - hist)) * p.H + h) * K;
        else if (row >= NQ0 && row < NQ0 + T)
            src = qwin + ((static_cast<size_t>(b) * T + (row - NQ0)) * p.H + h) * K;
        Chunk8<Act> c8;
        if (src) {
            load8<Act>(src + 8 * ch, c8);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                c8.x[e] = 0.0f;
        }
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            ss = __builtin_fmaf(c8.x[e], c8.x[e], ss);
        ss = group_sum<CPR>(ss);
        if (row < NXA) {
            if (ch == 0)
                rnX[row] = src ? 1.0f / sqrtf(ss + p.eps) : 0.0f;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int pos = 32 * (ch >> 2) + perm_pos(8 * (ch & 3) + 4 * hh);
                const float* x = c8.x + 4 * hh;
                uint2 hi;
                if constexpr (kF32) {
                    hi.x = pack_bf16x2(x[0], x[1]);
                    hi.y = pack_bf16x2(x[2], x[3]);
                    uint2 lo;
                    lo.x = pack_bf16x2(x[0] - __uint_as_float(hi.x << 16),
                                       x[1] - __uint_as_float(hi.x & 0xFFFF0000u));
                    lo.y = pack_bf16x2(x[2] - __uint_as_float(hi.y << 16),
                                       x[3] - __uint_as_float(hi.y & 0xFFFF0000u));
                    *reinterpret_cast<uint2*>(Xlo + row * KP + pos) = lo;
                } else {
                    hi = hh == 0 ? uint2{c8.raw[0].x, c8.raw[0].y} : uint2{c8.raw[0].z, c8.raw[0].w};
                }
                *reinterpret_cast<uint2*>(Xhi + row * KP + pos) = hi;
            }
            if (k_writer && row >= hist && row < n) {
                const int ph = (base + wpc + (row - hist)) & (L - 1);
                store8<Act>(ringk + static_cast<size_t>(ph) * K + 8 * ch, c8);
            }
        }
    }

    // ---- 2b. value tile of the n records (+ rawv ring write)
    const int CPV = BV / 8;
    const st* vwin = static_cast<const st*>(p.v);
    st* ringv = static_cast<st*>(p.rawv) + (static_cast<size_t>(s) * p.HV + hv) * L * p.V + vt * BV;
    for (int idx = tid; idx < n * CPV; idx += NT) {
        const int row = idx / CPV, ch = idx - row * CPV;
        const st* src = row < hist
                            ? ringv + static_cast<size_t>((base + row) & (L - 1)) * p.V + 8 * ch
                            : vwin + ((static_cast<size_t>(b) * T + (row - hist)) * p.HV + hv) * p.V +
                                  vt * BV + 8 * ch;
        Chunk8<Act> c8;
        load8<Act>(src, c8);
        store8<Act>(Vs + row * p.BVP + 8 * ch, c8);
        if (p.write_ring && row >= hist) {
            const int ph = (base + wpc + (row - hist)) & (L - 1);
            store8<Act>(ringv + static_cast<size_t>(ph) * p.V + 8 * ch, c8);
        }
    }

    // ---- 3. gates, beta and prefix sums of the gates (wave 0; n <= 128)
    if (wave == 0) {
        const size_t gbase = (static_cast<size_t>(s) * p.HV + hv) * L;
        float gl[2], bl[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int i = 2 * lane + r;
            gl[r] = 0.0f;
            bl[r] = 0.0f;
            if (i < hist) {
                const int ph = (base + i) & (L - 1);
                gl[r] = p.rg[gbase + ph];
                bl[r] = p.rb[gbase + ph];
            } else if (i < n) {
                const int t = i - hist;
                const size_t tok = static_cast<size_t>(b) * T + t;
                gdn_gate(Act::load(static_cast<const st*>(p.a) + tok * p.HV + hv),
                         Act::load(static_cast<const st*>(p.b) + tok * p.HV + hv), p.A_log[hv],
                         p.dt_bias[hv], p.softplus_threshold, gl[r], bl[r]);
                if (p.write_ring && vt == 0) {
                    const int ph = (base + wpc + t) & (L - 1);
                    p.rg[gbase + ph] = gl[r];
                    p.rb[gbase + ph] = bl[r];
                }
            }
        }
        const float pair = gl[0] + gl[1];
        float incl = pair;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(incl, off, 64);
            if (lane >= off)
                incl += y;
        }
        float excl = __shfl_up(incl, 1, 64);
        if (lane == 0)
            excl = 0.0f;
        const int i0 = 2 * lane;
        if (i0 < n) {
            gam[i0] = excl + gl[0];
            bet[i0] = bl[0];
        }
        if (i0 + 1 < n) {
            gam[i0 + 1] = (excl + gl[0]) + gl[1];
            bet[i0 + 1] = bl[1];
        }
    }
    __syncthreads();

    // ---- 4. Gram tiles: A (strictly lower, n x n) and F (n x T)
    const int NT1 = NB * (NB + 1) / 2;
    for (int ti = wave; ti < NT1 + NB; ti += NW) {
        int I, rowJ;
        const bool qtile = ti >= NT1;
        if (!qtile) {
            I = 0;
            while ((I + 1) * (I + 2) / 2 <= ti)
                ++I;
            rowJ = 16 * (ti - I * (I + 1) / 2);
        } else {
            I = ti - NT1;
            rowJ = NQ0;
        }
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int off = 32 * ks + 8 * grp;
            const bf16x8 xa = *reinterpret_cast<const bf16x8*>(Xhi + (16 * I + col) * KP + off);
            const bf16x8 xb = *reinterpret_cast<const bf16x8*>(Xhi + (rowJ + col) * KP + off);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, xb, acc, 0, 0, 0);
            if constexpr (kF32) {
                const bf16x8 la = *reinterpret_cast<const bf16x8*>(Xlo + (16 * I + col) * KP + off);
                const bf16x8 lb = *reinterpret_cast<const bf16x8*>(Xlo + (rowJ + col) * KP + off);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, lb, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(la, xb, acc, 0, 0, 0);
            }
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int i = 16 * I + 4 * grp + jj;
            if (!qtile) {
                const int j = rowJ + col;
                float val = 0.0f;
                if (j < i && i < n)
                    val = bet[i] * expf(gam[i] - gam[j]) * rnX[i] * rnX[j] * acc[jj];
                As[i * LP + j] = val;
            } else {
                const int t = col;
                float val = 0.0f;
                if (t < T && i < n && i <= hist + t)
                    val = expf(gam[min(hist + t, n - 1)] - gam[i]) * rnX[i] * rnX[NQ0 + t] * acc[jj];
                Fs[i * 16 + t] = val;
            }
        }
    }
    __syncthreads();

    // ---- 5. M = (I + A)^{-T} F by back substitution, one column per wave
    for (int t = wave; t < T; t += NW) {
        float acc0 = lane < n ? Fs[lane * 16 + t] : 0.0f;
        float acc1 = lane + 64 < n ? Fs[(lane + 64) * 16 + t] : 0.0f;
        for (int i = n - 1; i >= 1; --i) {
            const float Mi = i < 64 ? readlane_f(acc0, i) : readlane_f(acc1, i - 64);
            const float a0 = lane < i ? As[i * LP + lane] : 0.0f;
            acc0 = __builtin_fmaf(-a0, Mi, acc0);
            if (n > 64) {
                const float a1 = lane + 64 < i ? As[i * LP + 64 + lane] : 0.0f;
                acc1 = __builtin_fmaf(-a1, Mi, acc1);
            }
        }
        if (lane < n)
            Fs[lane * 16 + t] = acc0;
        if (lane + 64 < n)
            Fs[(lane + 64) * 16 + t] = acc1;
    }

    // ---- 6a. checkpoint rows -> bf16 hi + lo MFMA operands
    bf16x8 Sh[KS], Sl[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const float x[8] = {sraw[2 * ks][0],     sraw[2 * ks][1],     sraw[2 * ks][2],
                            sraw[2 * ks][3],     sraw[2 * ks + 1][0], sraw[2 * ks + 1][1],
                            sraw[2 * ks + 1][2], sraw[2 * ks + 1][3]};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hi[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
            lo[e] = pack_bf16x2(x[2 * e] - __uint_as_float(hi[e] << 16),
                                x[2 * e + 1] - __uint_as_float(hi[e] & 0xFFFF0000u));
        }
        Sh[ks] = __builtin_bit_cast(bf16x8, uint4{hi[0], hi[1], hi[2], hi[3]});
        Sl[ks] = __builtin_bit_cast(bf16x8, uint4{lo[0], lo[1], lo[2], lo[3]});
    }
    __syncthreads();

    // ---- 6b. projections, residuals, outputs
    auto project = [&](int row0) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int off = (row0 + col) * KP + 32 * ks + 8 * grp;
            const bf16x8 xa = *reinterpret_cast<const bf16x8*>(Xhi + off);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, Sh[ks], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, Sl[ks], acc, 0, 0, 0);
            if constexpr (kF32) {
                const bf16x8 la = *reinterpret_cast<const bf16x8*>(Xlo + off);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(la, Sh[ks], acc, 0, 0, 0);
            }
        }
        return acc;
    };

    // query rows: O seeded with e^{Gam_win} * rn_q * (S0 q)
    f32x4 oacc;
    {
        const f32x4 pq = project(NQ0);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int t = 4 * grp + jj;
            oacc[jj] = t < T ? expf(gam[min(hist + t, n - 1)]) * rnX[NQ0 + t] * pq[jj] : 0.0f;
        }
    }
    // key rows: R = beta (v - e^{Gam} rn (S0 k)), then O += M^T-weighted R
    for (int rb = 0; rb < NB; ++rb) {
        const f32x4 pk = project(16 * rb);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int i = 16 * rb + 4 * grp + jj;
            float r = 0.0f;
            if (i < n)
                r = bet[i] * (Act::load(Vs + i * p.BVP + wave * 16 + col) -
                              expf(gam[i]) * rnX[i] * pk[jj]);
            // A operand: lane (t = col, k-group grp) holds M[i][t] for the same i
            const float m = Fs[i * 16 + col];
            oacc = __builtin_amdgcn_mfma_f32_16x16x4f32(m, r, oacc, 0, 0, 0);
        }
    }
    st* out = static_cast<st*>(p.o);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int t = 4 * grp + jj;
        if (t < T)
            out[((static_cast<size_t>(b) * T + t) * p.HV + hv) * p.V + vcol] =
                Act::from_f32(p.scale * oacc[jj]);
    }
}

// ------------------------------------------------------------------- host

int verify_waves(const gdn_shape& sh)
{
    const int tiles = sh.V / 16;
    for (int w = 8; w >= 1; --w)
        if (tiles % w == 0)
            return w;
    return 1;
}

static int verify_bvp(const gdn_shape& sh)
{
    return verify_waves(sh) * 16 + 8;
}

size_t verify_lds_bytes(const gdn_shape& sh)
{
    const int LP = round16(sh.L);
    return verify_lds(sh.K, LP, verify_bvp(sh), sh.act == GDN_BF16 ? 2 : 4).total;
}

size_t max_lds_bytes()
{
    return 160 * 1024;
}

template <class Act, int K>
static hipError_t launch_verify_k(const gdn_shape& sh, const VerifyParams& p, hipStream_t stream)
{
    const int NW = verify_waves(sh);
    const size_t lds = verify_lds_bytes(sh);
    auto kern = verify_kernel<Act, K>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess)
            return e;
    }
    const dim3 grid(sh.V / (16 * NW), sh.B, sh.HV);
    hipLaunchKernelGGL(kern, grid, dim3(64 * NW), lds, stream, p);
    return hipGetLastError();
}

template <class Act>
static hipError_t launch_verify_act(const gdn_shape& sh, const VerifyParams& p, hipStream_t stream)
{
    switch (sh.K) {
    case 64: return launch_verify_k<Act, 64>(sh, p, stream);
    case 128: return launch_verify_k<Act, 128>(sh, p, stream);
    case 256: return launch_verify_k<Act, 256>(sh, p, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_verify(const gdn_shape& sh, const WindowPtrs& w, const float* S,
                         const int32_t* slot_idx, const CursorPtrs& c, const RingPtrs& r,
                         int write_ring, void* o, hipStream_t stream)
{
    if (sh.B == 0)
        return hipSuccess;
    VerifyParams p = {};
    p.B = sh.B;
    p.T = sh.T;
    p.H = sh.H;
    p.HV = sh.HV;
    p.V = sh.V;
    p.L = sh.L;
    p.LP = round16(sh.L);
    p.num_slots = sh.num_slots;
    p.BVP = verify_bvp(sh);
    p.write_ring = write_ring;
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
    p.o = o;
    return sh.act == GDN_BF16 ? launch_verify_act<ActBF16>(sh, p, stream)
                              : launch_verify_act<ActF32>(sh, p, stream);
}

}  // namespace gdn
