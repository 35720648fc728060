// gdn_verify.hip -- GDN ring spec-verify: outputs of the whole draft window
// from the frozen checkpoint plus the raw ring history, in closed form.
//
// Math (replayssm(B)SpecDecode §1.1 table and §12.3-12.4; the page's formulas
// are stripped, this is the reading that the recurrence determines).  For one
// (row, value head) let the combined sequence i = 0..n-1 be the hist committed
// ring records followed by the T window tokens, Gam_i = sum_{m<=i} g_m, kh/qh
// the l2-normalised raw keys/queries (kh_i = rn_i k_i), S0 the checkpoint
// (V x K).  Then
//     S_i = e^{Gam_i} S0 + sum_{j<=i} e^{Gam_i-Gam_j} d_j kh_j^T,
//     (I + A) D = R,  A_ij = beta_i e^{Gam_i-Gam_j} (kh_i . kh_j)   (j < i),
//                     R_i  = beta_i (v_i - e^{Gam_i} S0 kh_i),
//     o_t = scale (e^{Gam_{h+t}} S0 qh_t + sum_j F_jt d_j),
//     F_jt = e^{Gam_{h+t}-Gam_j} (kh_j . qh_t) [j <= h+t],   h = hist.
// With M = (I + A)^{-T} F (n x T) the outputs regroup as
//     O = S0 Z + V^T U,   U_it = beta_i M_it,
//     Z_t = e^{Gam_{h+t}} qh_t - sum_i beta_i e^{Gam_i} rn_i M_it k_i   (K x T),
// so the checkpoint meets only the T columns of Z: the per-token states and
// the n x V deltas are never formed.
//
// Execution: a persistent grid; each workgroup (8 waves) strides over items
// (row, value head, value tile of BV columns) and pipelines them:
//   * the raw keys/queries (X), the value tile and the gate inputs of the next
//     item are loaded into registers while the current item computes;
//   * staging: X to LDS as bf16 (fp32 activations: bf16 hi + lo) with the row
//     l2 norms reduced over the lanes that hold the row, the value tile, the
//     gates (ring g/beta for history, fused gating for the window) and their
//     prefix sums; the window records are copied to the ring on the way
//     (pre-mutation raw bits, single writer per qk head);
//   * the item's checkpoint rows are then issued as non-temporal 128-bit
//     loads (each instruction: 4 rows x 256 contiguous bytes) and stream in
//     behind the key-side work:
//       - Gram tiles k k^T (strictly lower) and k q^T on MFMA 16x16x32 bf16
//         (exact products of raw bf16 keys), scaled into A and F;
//       - M by a blocked back substitution (one window column per wave:
//         16x16 diagonal blocks sequentially from registers, off-diagonal
//         blocks as batched LDS reads), U and the coefficients of Z;
//       - Z^T = C^T X and U^T V (the value part of O) on MFMA 16x16x4 fp32;
//   * each wave finishes O for its 16 value rows: fp32 dot products of the
//     checkpoint rows with the T columns of Z (VALU, 16-lane DPP
//     reductions), plus the value part, scaled and stored.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

struct VerifyParams {
    int B, T, H, HV, V, L, LP, num_slots, BV, BVP, write_ring;
    int cpv_shift;              // log2(BV / 8)
    int step_vt, step_hv, step_b;  // the persistent grid stride as (vt, hv, b) digits
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
    size_t x_hi, x_lo, rn, gam, bet, vs, us, cs, az, total;
};

__host__ __device__ inline size_t align16(size_t x)
{
    return (x + 15) & ~static_cast<size_t>(15);
}

// az holds the packed strictly-lower A during the solve, then Z^T (fp32,
// 16 x K).
__host__ __device__ inline VerifyLds verify_lds(int K, int LP, int BV, int BVP, int act_bytes)
{
    VerifyLds l;
    const size_t KP = static_cast<size_t>(K) + 8;
    const size_t NXR = static_cast<size_t>(LP) + 16;
    const size_t tri = static_cast<size_t>(LP) * (LP - 1) / 2 * 4;
    const size_t zo = 16 * static_cast<size_t>(K) * 4;
    l.x_hi = 0;
    l.x_lo = l.x_hi + NXR * KP * 2;
    l.rn = l.x_lo + (act_bytes == 4 ? NXR * KP * 2 : 0);
    l.gam = l.rn + NXR * 4;
    l.bet = l.gam + static_cast<size_t>(LP) * 4;
    l.vs = l.bet + static_cast<size_t>(LP) * 4;
    l.us = l.vs + align16(static_cast<size_t>(LP) * BVP * act_bytes);
    l.cs = l.us + static_cast<size_t>(LP + 4) * 16 * 4;
    l.az = l.cs + (NXR + 4) * 16 * 4;
    l.total = l.az + align16(tri > zo ? tri : zo);
    return l;
}

// 8 consecutive activations kept as raw storage words (bit-exact for the
// ring side channel); widened to fp32 on use.
template <class Act>
struct Chunk8 {
    uint4 raw[Act::bytes / 2];
};

template <class Act>
__device__ __forceinline__ void load8(const typename Act::storage* src, Chunk8<Act>& ch)
{
    ch.raw[0] = *reinterpret_cast<const uint4*>(src);
    if constexpr (Act::bytes == 4)
        ch.raw[1] = *reinterpret_cast<const uint4*>(src + 4);
}

// The chunk's 8 elements as fp32 (exact widening).
template <class Act>
__device__ __forceinline__ void widen8(const Chunk8<Act>& ch, float (&x)[8])
{
    if constexpr (Act::bytes == 2) {
        const uint4 w = ch.raw[0];
        x[0] = __uint_as_float(w.x << 16);
        x[1] = __uint_as_float(w.x & 0xFFFF0000u);
        x[2] = __uint_as_float(w.y << 16);
        x[3] = __uint_as_float(w.y & 0xFFFF0000u);
        x[4] = __uint_as_float(w.z << 16);
        x[5] = __uint_as_float(w.z & 0xFFFF0000u);
        x[6] = __uint_as_float(w.w << 16);
        x[7] = __uint_as_float(w.w & 0xFFFF0000u);
    } else {
        x[0] = __uint_as_float(ch.raw[0].x);
        x[1] = __uint_as_float(ch.raw[0].y);
        x[2] = __uint_as_float(ch.raw[0].z);
        x[3] = __uint_as_float(ch.raw[0].w);
        x[4] = __uint_as_float(ch.raw[1].x);
        x[5] = __uint_as_float(ch.raw[1].y);
        x[6] = __uint_as_float(ch.raw[1].z);
        x[7] = __uint_as_float(ch.raw[1].w);
    }
}

template <class Act>
__device__ __forceinline__ void store8(typename Act::storage* dst, const Chunk8<Act>& ch)
{
    *reinterpret_cast<uint4*>(dst) = ch.raw[0];
    if constexpr (Act::bytes == 4)
        *reinterpret_cast<uint4*>(dst + 4) = ch.raw[1];
}

template <class Act>
__device__ __forceinline__ void zero8(Chunk8<Act>& ch)
{
#pragma unroll
    for (int i = 0; i < Act::bytes / 2; ++i)
        ch.raw[i] = uint4{0u, 0u, 0u, 0u};
}

// Row i of a strictly lower-triangular matrix stored row by row (i >= 1).
__host__ __device__ __forceinline__ int tri_index(int i)
{
    return i * (i - 1) / 2;
}

// e^x for the key-side coefficients (outputs only): exp2 of x log2(e) on the
// hardware exp unit.  Relative error ~1e-6 for |x| <= 100; results below the
// fp32 normal range flush to zero.
__device__ __forceinline__ float fast_exp(float x)
{
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

__device__ __forceinline__ float readlane_f(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Fixed workgroup: 8 waves.  Waves whose 16 value rows fall outside the tile
// only stage data and help with the key-side work.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

// Staging chunks per thread, sized for rings of up to LM records.
template <int K, int LM>
struct StageCounts {
    static constexpr int CPR = K / 8;                                   // chunks per X row
    static constexpr int NXR = LM + 16;                                 // X rows at most
    static constexpr int MXC = (NXR * CPR + kThreads - 1) / kThreads;   // X chunks / thread
    static constexpr int MVC = (LM * 16 + kThreads - 1) / kThreads;     // V chunks / thread
};

// Scalars of one work item (row b, value head hv, value tile vt).
struct Item {
    int valid, s, b, hv, vt, hist, n, base, wpc;
};

__device__ __forceinline__ void load_item_cursors(const VerifyParams& p, Item& c)
{
    const int s = p.slot_idx[c.b];
    c.valid = valid_slot(s, p.num_slots);
    c.s = c.valid ? s : 0;            // padding rows address slot 0 but never use it
    const bool flagged = p.is_flush[c.s] != 0;
    c.wpc = clamp_wp(p.write_pos[c.s], p.L, p.T);
    c.base = p.cache_base[c.s];
    c.hist = flagged ? 0 : c.wpc;
    c.n = c.hist + p.T;
}

// The item after c in this workgroup's sequence: add the grid stride digit by
// digit (no integer division per item).  Past the end the item is repeated.
__device__ __forceinline__ Item next_item(const VerifyParams& p, const Item& c, int nvt)
{
    Item d = c;
    int vt = c.vt + p.step_vt, hv = c.hv + p.step_hv, b = c.b + p.step_b;
    if (vt >= nvt) {
        vt -= nvt;
        ++hv;
    }
    if (hv >= p.HV) {
        hv -= p.HV;
        ++b;
    }
    if (b < p.B) {
        d.vt = vt;
        d.hv = hv;
        d.b = b;
        load_item_cursors(p, d);
    }
    return d;
}

// Raw loads of one item's key-side inputs, held in registers until staged.
template <class Act, int K, int LM>
struct Prefetch {
    using SC = StageCounts<K, LM>;
    Chunk8<Act> xc[SC::MXC];
    Chunk8<Act> vc[SC::MVC];
    float rgv[2], rbv[2];
    typename Act::storage rav[2], rbw[2];
};

template <class Act, int K, int LM>
__device__ __forceinline__ void issue_prefetch(const VerifyParams& p, const Item& c, int BV,
                                               int tid, Prefetch<Act, K, LM>& f)
{
    using st = typename Act::storage;
    using SC = StageCounts<K, LM>;
    constexpr int CPR = SC::CPR;
    const int lane = tid & 63;
    const int T = p.T, L = p.L;
    const int h = c.hv / (p.HV / p.H);
    const int NQ0 = ((c.n + 15) >> 4) << 4;
    const st* ringk = static_cast<const st*>(p.rawk) + (static_cast<size_t>(c.s) * p.H + h) * L * K;
    const st* ringv = static_cast<const st*>(p.rawv) + (static_cast<size_t>(c.s) * p.HV + c.hv) * L * p.V +
                      c.vt * BV;
    const st* kwin = static_cast<const st*>(p.k);
    const st* qwin = static_cast<const st*>(p.q);
    const st* vwin = static_cast<const st*>(p.v);
#pragma unroll
    for (int i = 0; i < SC::MXC; ++i) {
        const int idx = i * kThreads + tid;
        const int row = idx / CPR, ch = idx % CPR;
        const st* src = nullptr;
        if (row < c.hist)
            src = ringk + static_cast<size_t>((c.base + row) & (L - 1)) * K;
        else if (row < c.n)
            src = kwin + ((static_cast<size_t>(c.b) * T + (row - c.hist)) * p.H + h) * K;
        else if (row >= NQ0 && row < NQ0 + T)
            src = qwin + ((static_cast<size_t>(c.b) * T + (row - NQ0)) * p.H + h) * K;
        if (src)
            load8<Act>(src + 8 * ch, f.xc[i]);
        else
            zero8<Act>(f.xc[i]);
    }
#pragma unroll
    for (int i = 0; i < SC::MVC; ++i) {
        const int idx = i * kThreads + tid;
        const int row = idx >> p.cpv_shift, ch = idx & ((1 << p.cpv_shift) - 1);
        if (row < c.n) {
            const st* src = row < c.hist
                                ? ringv + static_cast<size_t>((c.base + row) & (L - 1)) * p.V + 8 * ch
                                : vwin + ((static_cast<size_t>(c.b) * T + (row - c.hist)) * p.HV + c.hv) *
                                             p.V + c.vt * BV + 8 * ch;
            load8<Act>(src, f.vc[i]);
        } else {
            zero8<Act>(f.vc[i]);
        }
    }
    // gate inputs, two records per lane (wave 0 uses them); clamped addresses
    const size_t gbase = (static_cast<size_t>(c.s) * p.HV + c.hv) * L;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int i = 2 * lane + r;
        const int ph = (c.base + min(i, max(c.hist - 1, 0))) & (L - 1);
        const size_t tok = static_cast<size_t>(c.b) * T + min(max(i - c.hist, 0), T - 1);
        f.rgv[r] = p.rg[gbase + ph];
        f.rbv[r] = p.rb[gbase + ph];
        f.rav[r] = static_cast<const st*>(p.a)[tok * p.HV + c.hv];
        f.rbw[r] = static_cast<const st*>(p.b)[tok * p.HV + c.hv];
    }
}

// Diagonal 16x16 block of the unit upper-triangular solve (I + A)^T m = f
// for rows i0..i0+15: lane j (row jrow) holds its running value in acc;
// Ms[r] receives the solved m of row i0 + r (zero for rows at or past n).
__device__ __forceinline__ void solve_diag_block(const float* As, int n, int i0, int jrow,
                                                 float& acc, float (&Ms)[16])
{
    float dA[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = i0 + r;
        const bool ok = i < n && jrow >= i0 && jrow < i;
        const float a = As[ok ? tri_index(i) + jrow : 0];
        dA[r] = ok ? a : 0.0f;
    }
    const int src = i0 & 63;
#pragma unroll
    for (int r = 15; r >= 0; --r) {
        Ms[r] = readlane_f(acc, src + r);
        acc = __builtin_fmaf(-dA[r], Ms[r], acc);
    }
}

template <class Act, int K, int LM>
__global__ __launch_bounds__(kThreads, 4) void verify_kernel(const VerifyParams p)
{
    using st = typename Act::storage;
    using SC = StageCounts<K, LM>;
    constexpr bool kF32 = Act::bytes == 4;
    constexpr int KS = K / 32;       // MFMA k-steps of the Gram tiles
    constexpr int CPR = SC::CPR;
    constexpr int KP = K + 8;        // LDS row stride of X (bf16 elements)
    constexpr int NT = kThreads;

    extern __shared__ __align__(16) unsigned char smem[];

    const int BV = p.BV, nvt = p.V / BV;
    const int nitems = p.B * p.HV * nvt;
    const int T = p.T, L = p.L, LP = p.LP;
    const int G = p.HV / p.H;

    const VerifyLds lay = verify_lds(K, LP, BV, p.BVP, Act::bytes);
    uint16_t* Xhi = reinterpret_cast<uint16_t*>(smem + lay.x_hi);
    uint16_t* Xlo = reinterpret_cast<uint16_t*>(smem + lay.x_lo);
    float* rnX = reinterpret_cast<float*>(smem + lay.rn);
    float* gam = reinterpret_cast<float*>(smem + lay.gam);
    float* bet = reinterpret_cast<float*>(smem + lay.bet);
    st* Vs = reinterpret_cast<st*>(smem + lay.vs);
    float* Us = reinterpret_cast<float*>(smem + lay.us);   // F, then U = beta M   [16][UST]
    float* Cs = reinterpret_cast<float*>(smem + lay.cs);   // coefficients of Z    [16][CST]
    const int UST = LP + 4, CST = LP + 16 + 4;
    float* As = reinterpret_cast<float*>(smem + lay.az);   // packed strictly-lower A ...
    float* Zs = reinterpret_cast<float*>(smem + lay.az);   // ... later Z^T [16][K]

    int it = blockIdx.x;
    if (it >= nitems)
        return;
    Item cur;
    cur.vt = it % nvt;
    cur.hv = (it / nvt) % p.HV;
    cur.b = it / nvt / p.HV;
    load_item_cursors(p, cur);
    Prefetch<Act, K, LM> pf;
    issue_prefetch<Act, K, LM>(p, cur, BV, threadIdx.x, pf);

    for (; it < nitems; it += gridDim.x) {
        // Per-lane indices are rederived from an opaque copy of the thread id
        // in every iteration: kept live across the loop they would be spilled,
        // and a spill reload waits behind the in-flight checkpoint loads.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wave = tid >> 6;
        const int col = lane & 15, grp = lane >> 4;
        // scalars of the next item (the last item repeats itself, which keeps
        // the prefetch below unconditional)
        const Item nxt = next_item(p, cur, nvt);
        if (!cur.valid) {                      // padding row: nothing to read or write
            issue_prefetch<Act, K, LM>(p, nxt, BV, tid, pf);
            cur = nxt;
            continue;
        }
        const int s = cur.s, b = cur.b, hv = cur.hv, vt = cur.vt;
        const int h = hv / G;
        const int hist = cur.hist, n = cur.n, base = cur.base, wpc = cur.wpc;
        const int NB = (n + 15) >> 4;   // 16-row blocks of keys
        const int NQ0 = NB << 4;        // first query row of X
        const int NXA = NQ0 + 16;       // X rows in use
        const size_t gbase = (static_cast<size_t>(s) * p.HV + hv) * L;
        st* ringk = static_cast<st*>(p.rawk) + (static_cast<size_t>(s) * p.H + h) * L * K;
        st* ringv = static_cast<st*>(p.rawv) + (static_cast<size_t>(s) * p.HV + hv) * L * p.V + vt * BV;

        // ============ staging from the prefetch registers into LDS (raw copies)
        const bool k_writer = p.write_ring && (hv % G == 0) && vt == 0;
#pragma unroll
        for (int i = 0; i < SC::MXC; ++i) {
            const int idx = i * NT + tid;
            const int row = idx / CPR, ch = idx % CPR;
            if (row < NXA) {
                if constexpr (kF32) {
                    float xf[8];
                    widen8<Act>(pf.xc[i], xf);
                    uint4 hi, lo;
                    uint32_t* hp = reinterpret_cast<uint32_t*>(&hi);
                    uint32_t* lp = reinterpret_cast<uint32_t*>(&lo);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        hp[e] = pack_bf16x2(xf[2 * e], xf[2 * e + 1]);
                        lp[e] = pack_bf16x2(xf[2 * e] - __uint_as_float(hp[e] << 16),
                                            xf[2 * e + 1] - __uint_as_float(hp[e] & 0xFFFF0000u));
                    }
                    *reinterpret_cast<uint4*>(Xhi + row * KP + 8 * ch) = hi;
                    *reinterpret_cast<uint4*>(Xlo + row * KP + 8 * ch) = lo;
                } else {
                    *reinterpret_cast<uint4*>(Xhi + row * KP + 8 * ch) = pf.xc[i].raw[0];
                }
                if (k_writer && row >= hist && row < n) {
                    const int ph = (base + wpc + (row - hist)) & (L - 1);
                    store8<Act>(ringk + static_cast<size_t>(ph) * K + 8 * ch, pf.xc[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < SC::MVC; ++i) {
            const int idx = i * NT + tid;
            const int row = idx >> p.cpv_shift, ch = idx & ((1 << p.cpv_shift) - 1);
            if (row < n) {
                store8<Act>(Vs + row * p.BVP + 8 * ch, pf.vc[i]);
                if (p.write_ring && row >= hist) {
                    const int ph = (base + wpc + (row - hist)) & (L - 1);
                    store8<Act>(ringv + static_cast<size_t>(ph) * p.V + 8 * ch, pf.vc[i]);
                }
            }
        }
        if (wave == 0) {
            float gl[2], bl[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int i = 2 * lane + r;
                gl[r] = 0.0f;
                bl[r] = 0.0f;
                if (i < hist) {
                    gl[r] = pf.rgv[r];
                    bl[r] = pf.rbv[r];
                } else if (i < n) {
                    gdn_gate(Act::load(&pf.rav[r]), Act::load(&pf.rbw[r]), p.A_log[hv],
                             p.dt_bias[hv], p.softplus_threshold, gl[r], bl[r]);
                    if (p.write_ring && vt == 0) {
                        const int ph = (base + wpc + (i - hist)) & (L - 1);
                        p.rg[gbase + ph] = gl[r];
                        p.rb[gbase + ph] = bl[r];
                    }
                }
            }
            // inclusive prefix sums of the gates over the combined sequence
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

        // ============ the checkpoint rows of this wave (non-temporal stream):
        // lane (row col, group grp) holds columns 16 i + 4 grp .. +3 of row
        // r0 + col, the fp32 MFMA operand order (k step 4 i + e).
        const bool has_rows = wave * 16 < BV;
        const int r0 = vt * BV + (has_rows ? wave * 16 : 0);
        const float* Srow = p.S + ((static_cast<size_t>(s) * p.HV + hv) * p.V + r0 + col) * K + 4 * grp;
        f32x4 sraw[K / 16];
#pragma unroll
        for (int i = 0; i < K / 16; ++i)
            sraw[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Srow + 16 * i));
        __syncthreads();

        // ============ l2 norms of the X rows: 16 lanes per row from LDS.  For
        // fp32 activations the row is the staged hi + lo pair.
        for (int row0 = 0; row0 < NXA; row0 += 4 * kWaves) {
            const int row = row0 + 4 * wave + grp;
            float ss = 0.0f;
            if (row < NXA) {
#pragma unroll
                for (int m = 0; m < K / 128; ++m) {
                    const uint4 w = *reinterpret_cast<const uint4*>(Xhi + row * KP + 128 * m + 8 * col);
                    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
                    uint32_t wl[4] = {0u, 0u, 0u, 0u};
                    if constexpr (kF32) {
                        const uint4 l = *reinterpret_cast<const uint4*>(Xlo + row * KP + 128 * m + 8 * col);
                        wl[0] = l.x; wl[1] = l.y; wl[2] = l.z; wl[3] = l.w;
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x0 = __uint_as_float(ww[e] << 16) + __uint_as_float(wl[e] << 16);
                        const float x1 = __uint_as_float(ww[e] & 0xFFFF0000u) +
                                         __uint_as_float(wl[e] & 0xFFFF0000u);
                        ss = __builtin_fmaf(x0, x0, ss);
                        ss = __builtin_fmaf(x1, x1, ss);
                    }
                }
                if constexpr (K == 64) {
                    // 64 columns over 16 lanes: 4 per lane
                    ss = 0.0f;
                    const uint2 w = *reinterpret_cast<const uint2*>(Xhi + row * KP + 4 * col);
                    uint2 l = {0u, 0u};
                    if constexpr (kF32)
                        l = *reinterpret_cast<const uint2*>(Xlo + row * KP + 4 * col);
                    const uint32_t ww[2] = {w.x, w.y}, wl[2] = {l.x, l.y};
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const float x0 = __uint_as_float(ww[e] << 16) + __uint_as_float(wl[e] << 16);
                        const float x1 = __uint_as_float(ww[e] & 0xFFFF0000u) +
                                         __uint_as_float(wl[e] & 0xFFFF0000u);
                        ss = __builtin_fmaf(x0, x0, ss);
                        ss = __builtin_fmaf(x1, x1, ss);
                    }
                }
            }
            ss = group16_sum(ss);
            if (row < NXA && col == 0) {
                const bool real = row < n || (row >= NQ0 && row < NQ0 + T);
                rnX[row] = real ? 1.0f / sqrtf(ss + p.eps) : 0.0f;
            }
        }
        __syncthreads();

        // ============ Gram tiles: A (strictly lower, n x n) and F (n x T)
        const int NT1 = NB * (NB + 1) / 2;
        for (int ti = wave; ti < NT1 + NB; ti += kWaves) {
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
                    if (j < i && i < n)
                        As[tri_index(i) + j] = bet[i] * fast_exp(gam[i] - gam[j]) * rnX[i] * rnX[j] * acc[jj];
                } else {
                    const int t = col;
                    float val = 0.0f;
                    if (t < T && i < n && i <= hist + t)
                        val = fast_exp(gam[min(hist + t, n - 1)] - gam[i]) * rnX[i] * rnX[NQ0 + t] * acc[jj];
                    Us[t * UST + i] = val;
                }
            }
        }
        // coefficient rows of Z that no solve column writes: zero
        for (int idx = tid; idx < NXA * 16; idx += NT) {
            const int t = idx / NXA, row = idx - t * NXA;
            if (row >= n || t >= T)
                Cs[t * CST + row] = 0.0f;
        }
        // the next item's key-side inputs stream in behind the rest of this one
        issue_prefetch<Act, K, LM>(p, nxt, BV, tid, pf);
        __syncthreads();

        // ============ M = (I + A)^{-T} F, one window column per wave.  Lane j
        // holds row j (acc0) and row j+64 (acc1).  Blocks of 16 rows from the
        // last: the diagonal block is solved sequentially from registers, then
        // its solution updates all earlier rows at once.  Rows at or past n
        // carry zero coefficients, so their M stays zero and no step branches.
        for (int t = wave; t < T; t += kWaves) {
            const float f0 = Us[t * UST + lane];                  // F
            const float f1 = LM > 64 ? Us[t * UST + 64 + lane] : 0.0f;
            float acc0 = lane < n ? f0 : 0.0f;
            float acc1 = lane + 64 < n ? f1 : 0.0f;
            for (int I = NB - 1; I >= 0; --I) {
                const int i0 = 16 * I;
                float Ms[16];
                if (LM <= 64 || i0 < 64)
                    solve_diag_block(As, n, i0, lane, acc0, Ms);
                else
                    solve_diag_block(As, n, i0, lane + 64, acc1, Ms);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = i0 + r;
                    const int tri = tri_index(min(i, n - 1));
                    const float a0 = As[tri + min(lane, i0 > 0 ? i0 - 1 : 0)];
                    acc0 = __builtin_fmaf(-((lane < i0 && i < n) ? a0 : 0.0f), Ms[r], acc0);
                    if (LM > 64) {
                        const int j1 = lane + 64;
                        const float a1 = As[tri + min(j1, i0 > 0 ? i0 - 1 : 0)];
                        acc1 = __builtin_fmaf(-((j1 < i0 && i < n) ? a1 : 0.0f), Ms[r], acc1);
                    }
                }
            }
            // U = beta M; Z coefficients: -beta e^{Gam} rn M on keys, e^{Gam_win} rn_q on the query
#pragma unroll
            for (int hh = 0; hh < (LM > 64 ? 2 : 1); ++hh) {
                const int j = lane + 64 * hh;
                const float m = hh ? acc1 : acc0;
                if (j < n) {
                    Us[t * UST + j] = bet[j] * m;
                    Cs[t * CST + j] = -bet[j] * fast_exp(gam[j]) * rnX[j] * m;
                }
            }
            if (lane < 16)
                Cs[t * CST + NQ0 + lane] = lane == t ? fast_exp(gam[hist + t]) * rnX[NQ0 + t] : 0.0f;
        }
        __syncthreads();

        // ============ Z^T = C^T X: 16-wide k tiles over the waves, two
        // interleaved accumulators.
        for (int kt = wave; kt < K / 16; kt += kWaves) {
            f32x4 z0 = {0.0f, 0.0f, 0.0f, 0.0f}, z1 = z0;
            for (int q = 0; q < NXA / 4; q += 2) {
                const int i = 4 * q + grp;
                float x0 = bf16_to_f32(Xhi[i * KP + 16 * kt + col]);
                float x1 = bf16_to_f32(Xhi[(i + 4) * KP + 16 * kt + col]);
                if constexpr (kF32) {
                    x0 += bf16_to_f32(Xlo[i * KP + 16 * kt + col]);
                    x1 += bf16_to_f32(Xlo[(i + 4) * KP + 16 * kt + col]);
                }
                z0 = __builtin_amdgcn_mfma_f32_16x16x4f32(Cs[col * CST + i], x0, z0, 0, 0, 0);
                z1 = __builtin_amdgcn_mfma_f32_16x16x4f32(Cs[col * CST + i + 4], x1, z1, 0, 0, 0);
            }
            // lane (k = 16 kt + col, rows t = 4 grp + jj)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                Zs[(4 * grp + jj) * K + 16 * kt + col] = z0[jj] + z1[jj];
        }
        // the value part U^T V of this wave's 16 rows, in the output layout:
        // lane (row col, window positions t = 4 grp + jj)
        f32x4 o0 = {0.0f, 0.0f, 0.0f, 0.0f}, o1 = o0;
        if (has_rows) {
            for (int q = 0; q < (n + 3) / 4; q += 2) {
                const int i = 4 * q + grp;
                const bool ok0 = i < n, ok1 = i + 4 < n;
                const float v0 = ok0 ? Act::load(Vs + i * p.BVP + wave * 16 + col) : 0.0f;
                const float v1 = ok1 ? Act::load(Vs + (i + 4) * p.BVP + wave * 16 + col) : 0.0f;
                const float u0 = ok0 ? Us[col * UST + i] : 0.0f;
                const float u1 = ok1 ? Us[col * UST + i + 4] : 0.0f;
                o0 = __builtin_amdgcn_mfma_f32_16x16x4f32(u0, v0, o0, 0, 0, 0);
                o1 = __builtin_amdgcn_mfma_f32_16x16x4f32(u1, v1, o1, 0, 0, 0);
            }
        }
        __syncthreads();

        // ============ O = S0 Z + V^T U for this wave's 16 rows on fp32 MFMA:
        // A = Z^T (lane (t col, group grp) reads Z[t][16 i + 4 grp + e]),
        // B = the checkpoint registers, accumulators seeded with the value part.
        if (has_rows) {
#pragma unroll
            for (int i = 0; i < K / 16; ++i) {
                const f32x4 za = *reinterpret_cast<const f32x4*>(Zs + col * K + 16 * i + 4 * grp);
                f32x4& acc = (i & 1) ? o1 : o0;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(za[e], sraw[i][e], acc, 0, 0, 0);
            }
            st* out = static_cast<st*>(p.o);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int t = 4 * grp + jj;
                if (t < T)
                    out[((static_cast<size_t>(b) * T + t) * p.HV + hv) * p.V + r0 + col] =
                        Act::from_f32(p.scale * (o0[jj] + o1[jj]));
            }
        }
        __syncthreads();   // LDS is restaged by the next item
        cur = nxt;
    }
}

// ------------------------------------------------------------------- host

// Value rows per work item: the largest power of two (16..128) that divides V,
// 16 per wave.
int verify_tile_cols(const gdn_shape& sh)
{
    for (int bv = 16 * kWaves; bv >= 16; bv >>= 1)
        if (sh.V % bv == 0)
            return bv;
    return 16;
}

static int verify_bvp(const gdn_shape& sh)
{
    return verify_tile_cols(sh) + 8;
}

size_t verify_lds_bytes(const gdn_shape& sh)
{
    const int LP = round16(sh.L);
    return verify_lds(sh.K, LP, verify_tile_cols(sh), verify_bvp(sh), sh.act == GDN_BF16 ? 2 : 4).total;
}

size_t max_lds_bytes()
{
    return 160 * 1024;
}

// Compute units of the current device (cached per device).
static int compute_units()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <class Act, int K, int LM>
static hipError_t launch_verify_k(const gdn_shape& sh, const VerifyParams& p, hipStream_t stream)
{
    const size_t lds = verify_lds_bytes(sh);
    auto kern = verify_kernel<Act, K, LM>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess)
            return e;
    }
    // persistent grid: two workgroups per compute unit, never more than items
    const int nvt = sh.V / p.BV;
    const long long items = static_cast<long long>(sh.B) * sh.HV * nvt;
    const long long cap = 2LL * compute_units();
    const unsigned grid = static_cast<unsigned>(items < cap ? items : cap);
    VerifyParams q = p;
    q.step_vt = static_cast<int>(grid % nvt);
    q.step_hv = static_cast<int>((grid / nvt) % sh.HV);
    q.step_b = static_cast<int>(grid / nvt / sh.HV);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), lds, stream, q);
    return hipGetLastError();
}

template <class Act, int K>
static hipError_t launch_verify_l(const gdn_shape& sh, const VerifyParams& p, hipStream_t stream)
{
    return sh.L <= 64 ? launch_verify_k<Act, K, 64>(sh, p, stream)
                      : launch_verify_k<Act, K, 128>(sh, p, stream);
}

template <class Act>
static hipError_t launch_verify_act(const gdn_shape& sh, const VerifyParams& p, hipStream_t stream)
{
    switch (sh.K) {
    case 64: return launch_verify_l<Act, 64>(sh, p, stream);
    case 128: return launch_verify_l<Act, 128>(sh, p, stream);
    case 256:
        if (sh.L > 64)
            return hipErrorInvalidValue;
        return launch_verify_k<Act, 256, 64>(sh, p, stream);
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
    p.BV = verify_tile_cols(sh);
    p.cpv_shift = 0;
    while ((8 << p.cpv_shift) < p.BV)
        ++p.cpv_shift;
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
