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
// (row, value head, value tile of BV <= 128 rows, 16 rows per wave):
//   1. the item's checkpoint rows are issued as non-temporal 128-bit loads
//      (lane (row c, group g) holds columns 16 i + 4 g .. +3 of row c), in
//      four groups at the first four phase boundaries (a steady stream);
//   2. the raw keys/queries (X) and the value rows, loaded into registers
//      while the previous item computed, are copied to LDS; the row l2 norms
//      are reduced from the same registers; the window records are copied to
//      the ring on the way (pre-mutation raw bits, single writer per qk head);
//      one wave forms the gates and their prefix sums;
//   3. Gram tiles k k^T and k q^T on MFMA 16x16x32 bf16 (exact products of raw
//      bf16 keys) scaled into the strictly lower A (stored as one dense panel
//      per 16-row block) and F;
//   4. the next item's inputs are issued; M by back substitution, one window
//      column per wave: the block's A values are read up front, then per row
//      one lane broadcast and one FMA; then U and the coefficients of Z;
//   5. Z = C^T X on MFMA 4x4x1 (16 blocks: 64 key columns x 4 window columns
//      per instruction, no padding at T = 4; the query terms are four more
//      coefficient rows) while the other waves form the value part U^T V of
//      their rows on the same instruction;
//   6. S0 Z for each wave's 16 rows on MFMA 4x4x1 straight from the checkpoint
//      registers (4 key-column groups summed by lane-half swaps), plus the
//      value part, scaled and stored.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

struct VerifyParams {
    int B, T, H, HV, V, L, num_slots, write_ring;
    int BV, nvt, vshift;           // value tile rows, tiles per head, log2(16-byte chunks per tile row)
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

// The launch arguments as seen in the kernel-argument segment (constant
// address space).  The kernel reads them through a pointer it re-launders at
// every phase boundary: each phase re-reads the fields it needs with scalar
// loads, so no argument or product of arguments stays live across phases (kept
// live, they overflow the scalar registers and every use becomes a VALU lane
// read).
typedef const __attribute__((address_space(4))) VerifyParams KParams;

__device__ __forceinline__ KParams* launder(KParams* pk)
{
    asm volatile("" : "+s"(pk));
    return pk;
}

// Fixed workgroup: 8 waves.  Waves whose 16 value rows fall outside the tile
// only stage data and help with the key-side work.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

constexpr int ilog2c(int x)
{
    return x <= 1 ? 0 : 1 + ilog2c(x / 2);
}

constexpr size_t align16c(size_t x)
{
    return (x + 15) & ~static_cast<size_t>(15);
}

// Compile-time layout of one instantiation: activation type, key width K,
// ring capacity LM (64 or 128 records), value tile capacity BVM.
template <class Act, int K_, int LM_, int BVM_>
struct VCfg {
    static constexpr int K = K_, LM = LM_, BVM = BVM_;
    static constexpr int eb = Act::bytes;
    static constexpr bool kF32 = eb == 4;
    static constexpr int EPC = 16 / eb;            // activations per 16-byte chunk
    static constexpr int CPR = K / EPC;            // chunks per key row
    static constexpr int CSH = ilog2c(CPR);
    // LDS X row, bf16 elements.  A 32-byte pad: with 16 bytes the Gram tiles'
    // 16-byte operand reads and the staging writes conflicted on the banks
    // (SQ_LDS_BANK_CONFLICT 1.9 M cycles per launch at B=256, K=V=128, T=4);
    // with 32 they read zero.
    static constexpr int KP = K + 16;
    static constexpr int NXR = LM + 16;            // X rows: keys (< LM), 16 query rows at NQ0
    static constexpr int VP = BVM + EPC;           // LDS value row, activations (16-byte pad)
    static constexpr int FST = LM + 20;            // F / U row stride (floats; U is zero past n)
    static constexpr int CST = LM + 20;            // Z coefficient row stride (floats)
    static constexpr int NBM = LM / 16;            // 16-row key blocks
    // A is stored per 16-row block I as a dense panel of 16 rows x 16 (I + 1)
    // columns (row stride 16 I + 20): only the part at or left of the block
    // diagonal exists.
    static constexpr int A_FLOATS = 128 * NBM * (NBM + 1) + 64 * NBM;
    // Z row stride (floats), where A's space allows it.  The output products
    // read four Z rows at eight 16-byte column groups per instruction; of the
    // strides K + 4, K + 16 and K + 32, K + 16 gives the fewest LDS
    // bank-conflict cycles (SQ_LDS_BANK_CONFLICT 5.2 M, 2.1 M and 3.1 M per
    // launch at B=256, K=V=128, T=4).
    static constexpr int ZST = 16 * (K + 16) <= A_FLOATS ? K + 16 : K + 4;
    static constexpr int Z_FLOATS = 16 * ZST;     // up to 16 window columns
    static constexpr int AZ = A_FLOATS > Z_FLOATS ? A_FLOATS : Z_FLOATS;
    static constexpr int VCRM = BVM / EPC;         // chunks per value row at most
    // register chunks per thread
    static constexpr int MH = ((LM - 1) * CPR + kThreads - 1) / kThreads;    // history keys
    static constexpr int MW = (2 * 16 * CPR + kThreads - 1) / kThreads;      // window keys + queries
    static constexpr int MVH = ((LM - 1) * VCRM + kThreads - 1) / kThreads;  // history values
    static constexpr int MVW = (16 * VCRM + kThreads - 1) / kThreads;       // window values
    static constexpr int RPL = LM / 64;                                      // gate records per lane
    // LDS carve-up (bytes)
    static constexpr size_t o_xhi = 0;
    static constexpr size_t o_xlo = o_xhi + static_cast<size_t>(NXR) * KP * 2;
    static constexpr size_t o_v = o_xlo + (kF32 ? static_cast<size_t>(NXR) * KP * 2 : 0);
    static constexpr int NVR = LM + 16;           // value rows: up to LM, then 16 zero rows
    static constexpr size_t o_az = o_v + align16c(static_cast<size_t>(NVR) * VP * eb);
    static constexpr size_t o_fu = o_az + static_cast<size_t>(AZ) * 4;
    static constexpr size_t o_cs = o_fu + static_cast<size_t>(16) * FST * 4;
    static constexpr size_t o_rn = o_cs + static_cast<size_t>(16) * CST * 4;
    static constexpr size_t o_gam = o_rn + static_cast<size_t>(NXR) * 4;
    static constexpr size_t o_bet = o_gam + static_cast<size_t>(LM) * 4;
    static constexpr size_t total = o_bet + static_cast<size_t>(LM) * 4;
    // two workgroups per compute unit when they fit in 160 KB of LDS
    static constexpr int kPerCU = total <= 80 * 1024 ? 2 : 1;
};

// Start of block I's panel and its row stride (floats).
__host__ __device__ constexpr int panel_base(int I)
{
    return 128 * I * (I + 1) + 64 * I;
}

__host__ __device__ constexpr int panel_stride(int I)
{
    return 16 * I + 20;
}

// e^x for the key-side coefficients as exp2 on the hardware unit: the gates'
// prefix sums are kept pre-multiplied by log2(e).  Results below the fp32
// normal range flush to zero.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_hw(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float readlane_f(float x, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// x from the paired 16-lane row (16) or 32-lane half (32), added to x.  The
// swap results are read as plain element values: a bit cast applied to an
// element of the returned vector reads element 0 with this compiler.
__device__ __forceinline__ float swap16_sum(float x)
{
    const unsigned u = __float_as_uint(x);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned lo = p[0], hi = p[1];
    return __uint_as_float(lo) + __uint_as_float(hi);
}

__device__ __forceinline__ float swap32_sum(float x)
{
    const unsigned u = __float_as_uint(x);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned lo = p[0], hi = p[1];
    return __uint_as_float(lo) + __uint_as_float(hi);
}

// Sum of the four 16-lane rows of a wave, delivered to every lane: rows
// (0 + 1) and (2 + 3) by a 16-lane swap, then the two halves by a 32-lane
// swap.  Every lane computes the same sums in the same order.
__device__ __forceinline__ float rows4_sum(float x)
{
    return swap32_sum(swap16_sum(x));
}

// Sum over the eight lanes l + 8 c (c = 0..7) of a wave, delivered to every
// one of them: l ^ 8 inside each 16-lane row by a DPP rotate, then the row
// pairs and the halves by lane swaps.
__device__ __forceinline__ float rows8_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
    return rows4_sum(x);
}

// DPP move of x with row mask RM; lanes without a source (or outside the
// mask) receive 0.
template <int CTRL, int RM>
__device__ __forceinline__ float dpp0(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, RM, 0xF, true));
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then the last lane of row 0 into row 1 (and of row 2 into row
// 3) and the last lane of row 1 into rows 2 and 3.
__device__ __forceinline__ float wave_incl_scan(float x)
{
    x += dpp0<0x111, 0xF>(x);   // row_shr:1
    x += dpp0<0x112, 0xF>(x);   // row_shr:2
    x += dpp0<0x114, 0xF>(x);   // row_shr:4
    x += dpp0<0x118, 0xF>(x);   // row_shr:8
    x += dpp0<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp0<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// Sum over aligned groups of W lanes (W = 8, 16, 32 or 64).
template <int W>
__device__ __forceinline__ float lane_group_sum(float x)
{
    if constexpr (W == 8) {
        x += dpp<0xB1>(x);
        x += dpp<0x4E>(x);
        x += dpp<0x141>(x);
        return x;
    } else if constexpr (W == 16) {
        return group16_sum(x);
    } else if constexpr (W == 32) {
        return swap16_sum(group16_sum(x));
    } else {
        return rows4_sum(group16_sum(x));
    }
}

// Sum of squares of one 16-byte chunk of activations (bf16 pairs on the
// packed dot-product unit: exact products, fp32 sums).
template <class Act>
__device__ __forceinline__ float chunk_sumsq(const uint4& w)
{
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    float ss = 0.0f;
    if constexpr (Act::bytes == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t ue = u[e];
            const bf16x2 x = __builtin_bit_cast(bf16x2, ue);
            ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = __uint_as_float(u[e]);
            ss = __builtin_fmaf(x, x, ss);
        }
    }
    return ss;
}

// 1 / sqrt(ss + eps) on the hardware reciprocal square root (about 1 ulp).
__device__ __forceinline__ float rnorm_hw(float ss, float eps)
{
    return __builtin_amdgcn_rsqf(ss + eps);
}

// One 16-byte chunk of a key/query row into LDS: raw bf16 bits, or for fp32
// activations the bf16 hi part and the bf16 rounding of the remainder.
template <class Act>
__device__ __forceinline__ void stage_x_chunk(uint16_t* hi_row, uint16_t* lo_row, const uint4& w)
{
    if constexpr (Act::bytes == 2) {
        *reinterpret_cast<uint4*>(hi_row) = w;
    } else {
        const float x[4] = {__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                            __uint_as_float(w.w)};
        const uint32_t h0 = pack_bf16x2(x[0], x[1]), h1 = pack_bf16x2(x[2], x[3]);
        const uint32_t l0 = pack_bf16x2(x[0] - __uint_as_float(h0 << 16), x[1] - __uint_as_float(h0 & 0xFFFF0000u));
        const uint32_t l1 = pack_bf16x2(x[2] - __uint_as_float(h1 << 16), x[3] - __uint_as_float(h1 & 0xFFFF0000u));
        *reinterpret_cast<uint2*>(hi_row) = uint2{h0, h1};
        *reinterpret_cast<uint2*>(lo_row) = uint2{l0, l1};
    }
}

// Element (row, column) of X as fp32 (hi + lo for fp32 activations).
template <bool kF32>
__device__ __forceinline__ float x_elem(const uint16_t* Xhi, const uint16_t* Xlo, int idx)
{
    float x = bf16_to_f32(Xhi[idx]);
    if constexpr (kF32)
        x += bf16_to_f32(Xlo[idx]);
    return x;
}

// Activation element idx from the aligned 32-bit word that holds it (exact
// widening).
// LDS reads through 32-bit offsets in the LDS address space (generic
// pointer arithmetic here is 64-bit, and its temporaries serialise reads).
template <class T>
__device__ __forceinline__ T lds_read(const void* base, uint32_t byte_off)
{
    typedef const __attribute__((address_space(3))) T* lptr;
    typedef const __attribute__((address_space(3))) char* lbase;
    return *((lptr)(((lbase)base) + byte_off));
}

template <class Act>
__device__ __forceinline__ float act_from_word(uint32_t w, size_t idx)
{
    if constexpr (Act::bytes == 2)
        return __uint_as_float((idx & 1) ? (w & 0xFFFF0000u) : (w << 16));
    else
        return __uint_as_float(w);
}

// 16-byte load at a uniform base plus a 32-bit per-lane byte offset.
__device__ __forceinline__ uint4 ld16(const void* base, uint32_t off)
{
    return *reinterpret_cast<const uint4*>(static_cast<const char*>(base) + off);
}

__device__ __forceinline__ void st16(void* base, uint32_t off, const uint4& w)
{
    *reinterpret_cast<uint4*>(static_cast<char*>(base) + off) = w;
}

// Read-only, wave-uniform metadata (slot indices, cursors, gate parameters)
// through the constant address space: scalar loads, counted apart from the
// vector loads, so reading them never waits on the checkpoint stream.
template <class T>
__device__ __forceinline__ T ld_uniform(const T* ptr, size_t i)
{
    typedef const __attribute__((address_space(4))) T* cptr;
    return ((cptr)ptr)[i];
}

// Scalars of one work item (row b, value head hv, value tile vt).
struct Item {
    int valid, s, b, hv, vt, hist, n, base, wpc;
};

__device__ __forceinline__ void load_item_cursors(KParams& p, Item& c)
{
    const int s = ld_uniform(p.slot_idx, c.b);
    c.valid = valid_slot(s, p.num_slots);
    c.s = c.valid ? s : 0;            // padding rows address slot 0 but never use it
    const bool flagged = ld_uniform(p.is_flush, c.s) != 0;
    c.wpc = clamp_wp(ld_uniform(p.write_pos, c.s), p.L, p.T);
    c.base = ld_uniform(p.cache_base, c.s);
    c.hist = flagged ? 0 : c.wpc;
    c.n = c.hist + p.T;
}

// The item after c in this workgroup's sequence: add the grid stride digit by
// digit (no integer division per item).  Past the end the item is repeated.
// The waves with extra work (the gates; the Z units) move by two waves in
// the second half of the grid.  Two workgroups share a compute unit, one
// from each half, and the waves of a workgroup go to the SIMDs in order, so
// the two workgroups put that work on different SIMDs.
__device__ __forceinline__ int role_shift()
{
    return 2 * blockIdx.x >= gridDim.x ? 2 : 0;
}

__device__ __forceinline__ Item next_item(KParams& p, const Item& c)
{
    Item d = c;
    int vt = c.vt + p.step_vt, hv = c.hv + p.step_hv, b = c.b + p.step_b;
    if (vt >= p.nvt) {
        vt -= p.nvt;
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

// Raw loads of one item's inputs, held in registers until staged.
template <class Cfg, class Act>
struct Prefetch {
    uint4 xh[Cfg::MH];
    uint4 xw[Cfg::MW];
    float rg[Cfg::RPL], rb[Cfg::RPL];
    uint32_t ra[Cfg::RPL], rbw[Cfg::RPL];   // aligned 32-bit words holding the activations
};

template <class Cfg, class Act>
__device__ __forceinline__ void issue_prefetch(KParams& p, const Item& c, int tid,
                                               Prefetch<Cfg, Act>& f)
{
    using st = typename Act::storage;
    constexpr int K = Cfg::K, CPR = Cfg::CPR, CSH = Cfg::CSH, eb = Cfg::eb;
    const int lane = tid & 63, wave = tid >> 6;
    const int T = p.T, L = p.L, H = p.H, HV = p.HV;
    const int h = c.hv / (HV / H);
    const int hist = c.hist;
    // keys: history from the ring (qk head slab of L records), window k and q
    const char* ringk = static_cast<const char*>(p.rawk) + (static_cast<size_t>(c.s) * H + h) * L * K * eb;
    const char* kwin = static_cast<const char*>(p.k) + (static_cast<size_t>(c.b) * T * H + h) * K * eb;
    const char* qwin = static_cast<const char*>(p.q) + (static_cast<size_t>(c.b) * T * H + h) * K * eb;
#pragma unroll
    for (int m = 0; m < Cfg::MH; ++m) {
        const int cc = tid + kThreads * m;
        const int row = cc >> CSH, ch = cc & (CPR - 1);
        f.xh[m] = uint4{0u, 0u, 0u, 0u};   // lanes without a row: no value flows in from elsewhere
        if (row < hist)
            f.xh[m] = ld16(ringk, static_cast<uint32_t>(((c.base + row) & (L - 1)) * (K * eb) + ch * 16));
    }
#pragma unroll
    for (int m = 0; m < Cfg::MW; ++m) {
        const int cc = tid + kThreads * m;
        f.xw[m] = uint4{0u, 0u, 0u, 0u};
        if (cc < 2 * T * CPR) {
            const bool isq = cc >= T * CPR;
            const int c2 = isq ? cc - T * CPR : cc;
            const uint32_t off = static_cast<uint32_t>((c2 >> CSH) * (H * K * eb) + (c2 & (CPR - 1)) * 16);
            f.xw[m] = ld16(isq ? qwin : kwin, off);
        }
    }
    // gate inputs of records RPL lane + r (the gate wave forms the gates):
    // every lane loads all four, at clamped in-range indices, so no load is
    // conditional (a register written by a load on one path and a copy on
    // the other would have to wait for the load)
    if (wave == kWaves - 1 - role_shift()) {
        const size_t gbase = (static_cast<size_t>(c.s) * HV + c.hv) * L;
        const int hl = hist > 0 ? hist - 1 : 0;
#pragma unroll
        for (int r = 0; r < Cfg::RPL; ++r) {
            const int i = Cfg::RPL * lane + r;
            const int ph = (c.base + (i < hl ? i : hl)) & (L - 1);
            const int tw = i - hist < 0 ? 0 : (i - hist < T ? i - hist : T - 1);
            const size_t idx = (static_cast<size_t>(c.b) * T + tw) * HV + c.hv;
            const size_t w = Act::bytes == 2 ? idx >> 1 : idx;
            f.rg[r] = p.rg[gbase + ph];
            f.rb[r] = p.rb[gbase + ph];
            f.ra[r] = static_cast<const uint32_t*>(p.a)[w];
            f.rbw[r] = static_cast<const uint32_t*>(p.b)[w];
        }
    }
}

// Checkpoint loads of quarter Q (of K / 16 per lane): the item's 64 KB are
// issued in four groups (at the item's start, the Gram tiles, the solve and
// the Z phase), so the memory pipe sees a steady stream instead of one burst
// per item.  Load i of lane l reads row
// 8 (i & 1) + l % 8 of the wave's 16, key columns 32 (i >> 1) + 4 (l / 8) ..
// +3: every load instruction covers whole 128-byte lines (8 rows x 128 B),
// which streams measurably faster than 16 rows x 64 B.  Sl points at the
// lane's first element (row l % 8, column 4 (l / 8)).
template <int K, int Q>
__device__ __forceinline__ void load_ckpt(f32x4 (&sraw)[K / 16], const float* Sl)
{
    constexpr int N = K / 64;
#pragma unroll
    for (int i = Q * N; i < (Q + 1) * N; ++i)
        sraw[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sl + (i & 1) * 8 * K + (i >> 1) * 32));
}

// The item's value rows (ring history and window, this tile's columns),
// loaded at the start of the item and staged to LDS after the Gram tiles: a
// short register live range, well ahead of their first use.
template <class Cfg>
struct ValueRows {
    uint4 vh[Cfg::MVH];
    uint4 vw[Cfg::MVW];
};

template <class Cfg>
__device__ __forceinline__ void load_value_rows(KParams& p, const Item& c, int tid, ValueRows<Cfg>& f)
{
    constexpr int eb = Cfg::eb;
    const int T = p.T, L = p.L, HV = p.HV;
    const int hist = c.hist;
    const int VCR = 1 << p.vshift;
    const size_t vrow = static_cast<size_t>(p.V) * eb;
    const char* ringv = static_cast<const char*>(p.rawv) + (static_cast<size_t>(c.s) * HV + c.hv) * L * vrow +
                        static_cast<size_t>(c.vt) * p.BV * eb;
    const char* vwin = static_cast<const char*>(p.v) + (static_cast<size_t>(c.b) * T * HV + c.hv) * vrow +
                       static_cast<size_t>(c.vt) * p.BV * eb;
#pragma unroll
    for (int m = 0; m < Cfg::MVH; ++m) {
        const int cc = tid + kThreads * m;
        const int row = cc >> p.vshift, ch = cc & (VCR - 1);
        f.vh[m] = uint4{0u, 0u, 0u, 0u};   // lanes without a row: no value flows in from elsewhere
        if (row < hist)
            f.vh[m] = ld16(ringv, static_cast<uint32_t>(((c.base + row) & (L - 1)) * vrow + ch * 16));
    }
#pragma unroll
    for (int m = 0; m < Cfg::MVW; ++m) {
        const int cc = tid + kThreads * m;
        f.vw[m] = uint4{0u, 0u, 0u, 0u};
        if (cc < T * VCR)
            f.vw[m] = ld16(vwin, static_cast<uint32_t>((cc >> p.vshift) * (HV * vrow) + (cc & (VCR - 1)) * 16));
    }
}

// Back substitution through block I of (I + A)^T m = f.  Lane j holds the
// running value of row j (acc0: rows 0..63, acc1: rows 64..127).  Rows of
// the block from the last: its value is final, is broadcast, and is removed
// from every row to its left.  Lanes right of the panel are final already and
// are left alone.
template <int I, int LM>
__device__ __forceinline__ void solve_block(const float* As, int lane, float& acc0, float& acc1)
{
    constexpr int RS = panel_stride(I);
    constexpr int W = 16 * (I + 1);
    const float* pr = As + panel_base(I) + lane;
    // the block's 16 rows of A are read up front; the chain then runs from registers
    if constexpr (W <= 64) {
        if (lane < W) {
            float a[16];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                a[r] = pr[r * RS];
#pragma unroll
            for (int r = 15; r >= 0; --r) {
                const float m = readlane_f(acc0, 16 * I + r);
                acc0 = __builtin_fmaf(-a[r], m, acc0);
            }
        }
    } else {
        const bool upd1 = lane + 64 < W;
        float a0[16], a1[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            a0[r] = pr[r * RS];
            a1[r] = pr[r * RS + 64];
        }
#pragma unroll
        for (int r = 15; r >= 0; --r) {
            const float m = readlane_f(acc1, 16 * I + r - 64);
            acc0 = __builtin_fmaf(-a0[r], m, acc0);
            acc1 = upd1 ? __builtin_fmaf(-a1[r], m, acc1) : acc1;
        }
    }
}

template <int LM>
__device__ __forceinline__ void solve_all(const float* As, int NB, int lane, float& acc0, float& acc1)
{
    switch (NB) {
    case 8:
        if constexpr (LM > 64)
            solve_block<7, LM>(As, lane, acc0, acc1);
        [[fallthrough]];
    case 7:
        if constexpr (LM > 64)
            solve_block<6, LM>(As, lane, acc0, acc1);
        [[fallthrough]];
    case 6:
        if constexpr (LM > 64)
            solve_block<5, LM>(As, lane, acc0, acc1);
        [[fallthrough]];
    case 5:
        if constexpr (LM > 64)
            solve_block<4, LM>(As, lane, acc0, acc1);
        [[fallthrough]];
    case 4: solve_block<3, LM>(As, lane, acc0, acc1); [[fallthrough]];
    case 3: solve_block<2, LM>(As, lane, acc0, acc1); [[fallthrough]];
    case 2: solve_block<1, LM>(As, lane, acc0, acc1); [[fallthrough]];
    case 1: solve_block<0, LM>(As, lane, acc0, acc1); [[fallthrough]];
    default: break;
    }
}

// V^T U for this wave's 16 value rows and window columns 4 tg .. +3, in the
// layout of the output products: MFMA 4x4x1 block b = l / 4 of lane l holds
// value rows vrow0 + 8 h + 4 (b & 1) + (0..3) (h = 0: vp0, h = 1: vp1) and
// sums the records i = 8 m + l / 8; the eight groups l / 8 meet with the
// checkpoint products.  U and the value rows are zero past n, so whole
// groups of eight records are read.
template <class Cfg, class Act>
__device__ __forceinline__ void value_part(const float* FU, const typename Act::storage* Vs, int n, int tg,
                                           int lane, int vrow0, f32x4& vp0, f32x4& vp1)
{
    const int c = lane >> 3;
    const float* urow = FU + (4 * tg + (lane & 3)) * Cfg::FST;
    const int vc = vrow0 + (lane & 7);
    f32x4 a0 = {0.0f, 0.0f, 0.0f, 0.0f}, a1 = a0;
    for (int m0 = 0; 8 * m0 < n; m0 += 2) {
        float u[2], v0[2], v1[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const uint32_t i = static_cast<uint32_t>(8 * (m0 + e) + c);
            u[e] = lds_read<float>(urow, i * 4u);
            if constexpr (Act::bytes == 2) {
                v0[e] = bf16_to_f32(lds_read<uint16_t>(Vs, (i * Cfg::VP + vc) * 2u));
                v1[e] = bf16_to_f32(lds_read<uint16_t>(Vs, (i * Cfg::VP + vc + 8) * 2u));
            } else {
                v0[e] = lds_read<float>(Vs, (i * Cfg::VP + vc) * 4u);
                v1[e] = lds_read<float>(Vs, (i * Cfg::VP + vc + 8) * 4u);
            }
        }
        a0 = __builtin_amdgcn_mfma_f32_4x4x1f32(u[0], v0[0], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_4x4x1f32(u[0], v1[0], a1, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_4x4x1f32(u[1], v0[1], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_4x4x1f32(u[1], v1[1], a1, 0, 0, 0);
    }
    vp0 = a0;
    vp1 = a1;
}

template <class Act, int K, int LM, int BVM, int MINW>
__global__ __launch_bounds__(kThreads, MINW) void verify_kernel(const VerifyParams p_arg)
{
    using Cfg = VCfg<Act, K, LM, BVM>;
    using st = typename Act::storage;
    constexpr bool kF32 = Cfg::kF32;
    constexpr int CPR = Cfg::CPR, CSH = Cfg::CSH, KP = Cfg::KP, EPC = Cfg::EPC;
    constexpr int FST = Cfg::FST, CST = Cfg::CST, VP = Cfg::VP;
    constexpr int KS = K / 32;       // MFMA k-steps of the Gram tiles

    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* Xhi = reinterpret_cast<uint16_t*>(smem + Cfg::o_xhi);
    uint16_t* Xlo = reinterpret_cast<uint16_t*>(smem + Cfg::o_xlo);
    st* Vs = reinterpret_cast<st*>(smem + Cfg::o_v);
    float* As = reinterpret_cast<float*>(smem + Cfg::o_az);   // panels of A ...
    float* Zs = As;                                            // ... later Z [16][K]
    float* FU = reinterpret_cast<float*>(smem + Cfg::o_fu);   // F, then U = beta M  [16][FST]
    float* Cs = reinterpret_cast<float*>(smem + Cfg::o_cs);   // coefficients of Z   [16][CST]
    float* rn = reinterpret_cast<float*>(smem + Cfg::o_rn);   // 1/||x|| per X row (0 on zero rows)
    float* gam = reinterpret_cast<float*>(smem + Cfg::o_gam); // log2(e) * prefix sums of g
    float* bet = reinterpret_cast<float*>(smem + Cfg::o_bet); // beta (0 past n)

    (void)p_arg;   // read through the argument segment instead
    KParams* pk = launder((KParams*)__builtin_amdgcn_kernarg_segment_ptr());
    const int nitems = pk->B * pk->HV * pk->nvt;
    const int T = pk->T, L = pk->L, G = pk->HV / pk->H;
    const int TP = (T + 3) & ~3;

    int it = blockIdx.x;
    if (it >= nitems)
        return;
    Item cur;
    cur.vt = it % pk->nvt;
    cur.hv = (it / pk->nvt) % pk->HV;
    cur.b = it / pk->nvt / pk->HV;
    load_item_cursors(*pk, cur);

    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    // Staging of item c from the prefetch registers into LDS: raw keys and
    // queries (fp32 activations: bf16 hi + lo), their l2 norms reduced from
    // the same registers, zero padding rows, the window's ring records
    // (pre-mutation raw bits, single writer per qk head), and the gates with
    // their prefix sums (gate wave).  It runs while the previous item's
    // outputs are formed: X, the norms and the gates are not read by that
    // phase.
    auto stage_keys = [&](const Item& c, const Prefetch<Cfg, Act>& pf, int tid, int lane, bool ring) {
        KParams* pk2 = launder(pk);
        const int s = c.s, b = c.b, hv = c.hv, vt = c.vt;
        const int h = hv / G;
        const int hist = c.hist, n = c.n, base = c.base, wpc = c.wpc;
        const int NQ0 = ((n + 15) >> 4) << 4;
            const bool write_ring = ring && pk2->write_ring != 0;
            const bool k_writer = write_ring && (hv % G == 0) && vt == 0;
            char* ringk = static_cast<char*>(pk2->rawk) + (static_cast<size_t>(s) * pk2->H + h) * L * K * Cfg::eb;
            // history keys
    #pragma unroll
            for (int m = 0; m < Cfg::MH; ++m) {
                const int cc = tid + kThreads * m;
                const int row = cc >> CSH, ch = cc & (CPR - 1);
                // the sum is formed on every lane (zero chunks on lanes
                // without a row), so every load is consumed on every path
                float ss = chunk_sumsq<Act>(pf.xh[m]);
                if (row < hist)
                    stage_x_chunk<Act>(Xhi + row * KP + ch * EPC, Xlo + row * KP + ch * EPC, pf.xh[m]);
                ss = lane_group_sum<CPR>(ss);
                if (row < hist && ch == 0)
                    rn[row] = rnorm_hw(ss, pk2->eps);
            }
            // window keys (rows hist..n-1) and queries (rows NQ0..NQ0+T-1)
    #pragma unroll
            for (int m = 0; m < Cfg::MW; ++m) {
                const int cc = tid + kThreads * m;
                const bool live = cc < 2 * T * CPR;
                const bool isq = cc >= T * CPR;
                const int c2 = isq ? cc - T * CPR : cc;
                const int t = c2 >> CSH, ch = c2 & (CPR - 1);
                const int row = isq ? NQ0 + t : hist + t;
                float ss = chunk_sumsq<Act>(pf.xw[m]);
                if (live) {
                    stage_x_chunk<Act>(Xhi + row * KP + ch * EPC, Xlo + row * KP + ch * EPC, pf.xw[m]);
                    if (!isq && k_writer)
                        st16(ringk, static_cast<uint32_t>(((base + wpc + t) & (L - 1)) * (K * Cfg::eb) + ch * 16),
                             pf.xw[m]);
                }
                ss = lane_group_sum<CPR>(ss);
                if (live && ch == 0)
                    rn[row] = rnorm_hw(ss, pk2->eps);
            }
            // key rows n..NQ0-1 are zero (they pad the last Gram block), and so
            // are query rows NQ0+T..NQ0+TP-1 (they pad the last group of Z rows)
            const int nz = NQ0 - n;
            for (int cc = tid; cc < (nz + TP - T) * CPR; cc += kThreads) {
                const int zr = cc >> CSH, ch = cc & (CPR - 1);
                const int row = zr < nz ? n + zr : NQ0 + T + (zr - nz);
                const uint4 z = {0u, 0u, 0u, 0u};
                stage_x_chunk<Act>(Xhi + row * KP + ch * EPC, Xlo + row * KP + ch * EPC, z);
                if (ch == 0)
                    rn[row] = 0.0f;
            }
            // gates of the combined sequence and their prefix sums (gate wave)
            if (wave == kWaves - 1 - role_shift()) {
                const size_t gbase = (static_cast<size_t>(s) * pk2->HV + hv) * L;
                float gl[Cfg::RPL], bl[Cfg::RPL];
                float pair = 0.0f;
    #pragma unroll
                for (int r = 0; r < Cfg::RPL; ++r) {
                    const int i = Cfg::RPL * lane + r;
                    gl[r] = 0.0f;
                    bl[r] = 0.0f;
                    if (i < hist) {
                        gl[r] = pf.rg[r];
                        bl[r] = pf.rb[r];
                    } else if (i < n) {
                        const size_t idx = (static_cast<size_t>(b) * T + (i - hist)) * pk2->HV + hv;
                        gdn_gate(act_from_word<Act>(pf.ra[r], idx), act_from_word<Act>(pf.rbw[r], idx), ld_uniform(pk2->A_log, hv),
                                 ld_uniform(pk2->dt_bias, hv), pk2->softplus_threshold, gl[r], bl[r]);
                        if (write_ring && vt == 0) {
                            const int ph = (base + wpc + (i - hist)) & (L - 1);
                            pk2->rg[gbase + ph] = gl[r];
                            pk2->rb[gbase + ph] = bl[r];
                        }
                    }
                    pair += gl[r];
                }
                const float incl = wave_incl_scan(pair);
                float run = dpp0<0x138, 0xF>(incl);   // wave_shr:1: the exclusive prefix
    #pragma unroll
                for (int r = 0; r < Cfg::RPL; ++r) {
                    const int i = Cfg::RPL * lane + r;
                    run += gl[r];
                    gam[i] = run * kLog2e;
                    bet[i] = bl[r];
                }
            }
            // the gate registers count as consumed in every wave (only the
            // gate wave loaded them)
#pragma unroll
            for (int r = 0; r < Cfg::RPL; ++r)
                asm volatile("" ::"v"(pf.rg[r]), "v"(pf.rb[r]), "v"(pf.ra[r]), "v"(pf.rbw[r]));
    };

    // the first item is staged here; every later one is staged before its
    // turn (during the previous item's outputs, or right after a padding row)
    {
        const int tid0 = static_cast<int>(threadIdx.x);
        Prefetch<Cfg, Act> pf0;
        issue_prefetch<Cfg, Act>(*pk, cur, tid0, pf0);
        stage_keys(cur, pf0, tid0, tid0 & 63, cur.valid != 0);
    }
    for (; it < nitems; it += gridDim.x) {
        pk = launder(pk);
        // The lane index is rebuilt in every iteration from an opaque zero
        // (mbcnt cannot be hoisted then): a thread id kept live across the
        // loop would be spilled, and its reload waits behind the in-flight
        // checkpoint loads.
        unsigned zero;
        asm volatile("s_mov_b32 %0, 0" : "=s"(zero));
        const int lane = static_cast<int>(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, zero)));
        const int tid = wave * 64 + lane;
        const int col = lane & 15, grp = lane >> 4;
        // the next item's raw keys, loaded while this one computes (declared
        // per iteration: nothing flows through them from one item to the next)
        Prefetch<Cfg, Act> pf;
        if (!cur.valid) {                      // padding row: nothing to read or write
            // every wave is done staging the padding item before the next
            // one is staged over it (rows are assigned to threads by position
            // in the window, so two items' rows land on different waves)
            __syncthreads();
            cur = next_item(*pk, cur);           // (the last item repeats itself)
            // loads and staging are unconditional (a padding row or a repeated
            // item stages harmlessly, with its ring writes off): a load on
            // one path only would make later waits drain every load in flight
            issue_prefetch<Cfg, Act>(*pk, cur, tid, pf);
            stage_keys(cur, pf, tid, lane, cur.valid && it + static_cast<int>(gridDim.x) < nitems);
            continue;
        }
        const int s = cur.s, b = cur.b, hv = cur.hv, vt = cur.vt;
        const int h = hv / G;
        const int hist = cur.hist, n = cur.n, base = cur.base, wpc = cur.wpc;
        const int NB = (n + 15) >> 4;   // 16-row key blocks
        const int NQ0 = NB << 4;        // first query row of X
        const int BV = pk->BV;

        // ============ 1. checkpoint rows of this wave (non-temporal stream,
        // first quarter; the rest follow at the next phase boundaries)
        const bool has_rows = wave * 16 < BV;
        const int r0 = vt * BV + (has_rows ? wave * 16 : 0);
        const float* Srow = pk->S + ((static_cast<size_t>(s) * pk->HV + hv) * pk->V + r0 + (lane & 7)) * K +
                            4 * (lane >> 3);
        f32x4 sraw[K / 16];
        load_ckpt<K, 0>(sraw, Srow);
        ValueRows<Cfg> vr;
        load_value_rows<Cfg>(*pk, cur, tid, vr);

        // ============ 2. the keys were staged before this item's turn

        __syncthreads();
        pk = launder(pk);

        // ============ 3. Gram tiles.  Block row I holds I + 1 tiles of A
        // (J <= I) and one tile of F (its keys against the queries).
        const int ntiles = NB * (NB + 3) / 2;
        load_ckpt<K, 1>(sraw, Srow);   // (after the value rows: their wait below leaves it in flight)
        for (int ti = wave; ti < ntiles; ti += kWaves) {
            int I = 0;
            while ((I + 1) * (I + 4) / 2 <= ti)
                ++I;
            const int J = ti - I * (I + 3) / 2;
            const bool ftile = J == I + 1;
            const int rowA = 16 * (ftile ? I : J) + col;   // MFMA rows m: keys j
            const int rowB = (ftile ? NQ0 : 16 * I) + col; // MFMA columns n: keys i or queries t
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
            // all operand reads of the tile before the first product
            bf16x8 xa[KS], xb[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint32_t off = 32 * ks + 8 * grp;
                xa[ks] = lds_read<bf16x8>(Xhi, (static_cast<uint32_t>(rowA) * KP + off) * 2u);
                xb[ks] = lds_read<bf16x8>(Xhi, (static_cast<uint32_t>(rowB) * KP + off) * 2u);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[ks], xb[ks], acc, 0, 0, 0);
                if constexpr (kF32) {
                    const uint32_t off = 32 * ks + 8 * grp;
                    const bf16x8 la = lds_read<bf16x8>(Xlo, (static_cast<uint32_t>(rowA) * KP + off) * 2u);
                    const bf16x8 lb = lds_read<bf16x8>(Xlo, (static_cast<uint32_t>(rowB) * KP + off) * 2u);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[ks], lb, acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(la, xb[ks], acc, 0, 0, 0);
                }
            }
            // lane (col, grp) holds rows j = 16 (I or J) + 4 grp + jj of column col
            const int j4 = rowA - col + 4 * grp;
            const f32x4 gj = *reinterpret_cast<const f32x4*>(gam + j4);
            const f32x4 rj = *reinterpret_cast<const f32x4*>(rn + j4);
            f32x4 val;
            if (!ftile) {
                const int i = 16 * I + col;
                const float gi = gam[i], bri = bet[i] * rn[i];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float x = acc[jj] * bri * rj[jj] * exp2_hw(gi - gj[jj]);
                    val[jj] = (J == I && 4 * grp + jj >= col) ? 0.0f : x;
                }
                *reinterpret_cast<f32x4*>(As + panel_base(I) + col * panel_stride(I) + 16 * J + 4 * grp) = val;
            } else {
                const int t = col;
                const int tc = t < T ? t : T - 1;
                const int ht = hist + tc;
                const float gq = gam[ht], rq = rn[NQ0 + tc];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float x = acc[jj] * rq * rj[jj] * exp2_hw(gq - gj[jj]);
                    val[jj] = (t < T && j4 + jj <= ht) ? x : 0.0f;
                }
                *reinterpret_cast<f32x4*>(FU + t * FST + j4) = val;
            }
        }
        // value rows of the tile (loaded at the start of the item)
        {
            const bool write_ring = pk->write_ring != 0;
            const int VCR = 1 << pk->vshift;
            const size_t vrow = static_cast<size_t>(pk->V) * Cfg::eb;
            char* ringv = static_cast<char*>(pk->rawv) + (static_cast<size_t>(s) * pk->HV + hv) * L * vrow +
                          static_cast<size_t>(vt) * BV * Cfg::eb;
#pragma unroll
            for (int m = 0; m < Cfg::MVH; ++m) {
                const int cc = tid + kThreads * m;
                const int row = cc >> pk->vshift, ch = cc & (VCR - 1);
                if (row < hist)
                    *reinterpret_cast<uint4*>(Vs + row * VP + ch * EPC) = vr.vh[m];
            }
#pragma unroll
            for (int m = 0; m < Cfg::MVW; ++m) {
                const int cc = tid + kThreads * m;
                if (cc < T * VCR) {
                    const int t = cc >> pk->vshift, ch = cc & (VCR - 1);
                    *reinterpret_cast<uint4*>(Vs + (hist + t) * VP + ch * EPC) = vr.vw[m];
                    if (write_ring)
                        st16(ringv, static_cast<uint32_t>(((base + wpc + t) & (L - 1)) * vrow + ch * 16), vr.vw[m]);
                }
            }
            // rows n..n+15 are zero: the value part reads whole 4-row groups
            for (int cc = tid; cc < 16 * VCR; cc += kThreads) {
                const int row = n + (cc >> pk->vshift), ch = cc & (VCR - 1);
                *reinterpret_cast<uint4*>(Vs + row * VP + ch * EPC) = uint4{0u, 0u, 0u, 0u};
            }
        }
        // the value-row registers count as consumed on every path
#pragma unroll
        for (int m = 0; m < Cfg::MVH; ++m)
            asm volatile("" ::"v"(vr.vh[m].x), "v"(vr.vh[m].y), "v"(vr.vh[m].z), "v"(vr.vh[m].w));
#pragma unroll
        for (int m = 0; m < Cfg::MVW; ++m)
            asm volatile("" ::"v"(vr.vw[m].x), "v"(vr.vw[m].y), "v"(vr.vw[m].z), "v"(vr.vw[m].w));
        __syncthreads();
        pk = launder(pk);

        // the checkpoint's third quarter, then the next item's inputs, stream
        // in behind the rest of this one
        load_ckpt<K, 2>(sraw, Srow);
        const Item nxt = next_item(*pk, cur);
        issue_prefetch<Cfg, Act>(*pk, nxt, tid, pf);

        // the waves on the critical path of the solve and of Z issue first
        // (the other workgroup on the unit runs its own phases meanwhile)
        if (wave < TP)
            __builtin_amdgcn_s_setprio(2);
        // ============ 4. M = (I + A)^{-T} F, one window column per wave
        for (int t = wave; t < TP; t += kWaves) {
            float acc0 = FU[t * FST + lane];
            float acc1 = LM > 64 ? FU[t * FST + 64 + lane] : 0.0f;
            solve_all<LM>(As, NB, lane, acc0, acc1);
            // U = beta M; Z coefficients -beta e^{Gam} rn M on keys
#pragma unroll
            for (int hh = 0; hh < LM / 64; ++hh) {
                const int j = lane + 64 * hh;
                const float m = hh ? acc1 : acc0;
                const bool ok = j < n;
                const float bj = bet[j];
                const float u = bj * m;
                const float cf = -(bj * rn[j]) * exp2_hw(gam[j]) * m;
                FU[t * FST + j] = ok ? u : 0.0f;
                Cs[t * CST + j] = ok ? cf : 0.0f;
            }
            // U past the ring capacity is zero too (the value part reads
            // whole 4-row groups); the query rows: e^{Gam_{h+t}} rn_q on the diagonal
            if (lane < 16)
                FU[t * FST + LM + lane] = 0.0f;
            if (lane < 16)
                Cs[t * CST + NQ0 + lane] =
                    (lane == t && t < T) ? exp2_hw(gam[hist + t]) * rn[NQ0 + t] : 0.0f;
        }
        __syncthreads();
        pk = launder(pk);

        const int zwave = (wave + kWaves - role_shift()) & (kWaves - 1);
        if (zwave < (TP / 4) * (K / 64))
            __builtin_amdgcn_s_setprio(2);
        else
            __builtin_amdgcn_s_setprio(0);
        load_ckpt<K, 3>(sraw, Srow);

        // ============ 5. Z = C^T X (keys, then the query rows) on MFMA 4x4x1:
        // unit (tg, kset): window columns 4 tg .. +3, key columns 64 kset + lane.
        // Eight key rows per batch: every read is issued before the products.
        constexpr int NKS = K / 64;
        constexpr int ZST = Cfg::ZST;
        const int nk8 = (n + 7) & ~7;          // rows n..nk8-1 are zero rows (< NQ0)
        for (int u = zwave; u < (TP / 4) * NKS; u += kWaves) {
            const int tg = u / NKS, ks = u % NKS;
            const float* crow = Cs + (4 * tg + (lane & 3)) * CST;
            const int kc = 64 * ks + lane;
            f32x4 z0 = {0.0f, 0.0f, 0.0f, 0.0f}, z1 = z0;
            for (int i = 0; i < nk8; i += 8) {
                const f32x4 ca = *reinterpret_cast<const f32x4*>(crow + i);
                const f32x4 cb = *reinterpret_cast<const f32x4*>(crow + i + 4);
                float x[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[e] = x_elem<kF32>(Xhi, Xlo, (i + e) * KP + kc);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    z0 = __builtin_amdgcn_mfma_f32_4x4x1f32(ca[e], x[e], z0, 0, 0, 0);
                    z1 = __builtin_amdgcn_mfma_f32_4x4x1f32(cb[e], x[4 + e], z1, 0, 0, 0);
                }
            }
            for (int i = NQ0; i < NQ0 + TP; i += 4) {   // the query rows
                const f32x4 cq = *reinterpret_cast<const f32x4*>(crow + i);
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[e] = x_elem<kF32>(Xhi, Xlo, (i + e) * KP + kc);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    z0 = __builtin_amdgcn_mfma_f32_4x4x1f32(cq[e], x[e], z0, 0, 0, 0);
            }
            // lane l, register r: Z[4 tg + r][kc]
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Zs[(4 * tg + r) * ZST + kc] = z0[r] + z1[r];
        }
        __builtin_amdgcn_s_setprio(0);
        // the value part of this wave's rows for the first four window columns
        f32x4 vp0 = {0.0f, 0.0f, 0.0f, 0.0f}, vp1 = vp0;
        if (has_rows)
            value_part<Cfg, Act>(FU, Vs, n, 0, lane, wave * 16, vp0, vp1);
        __syncthreads();
        pk = launder(pk);


        // ============ 6. O = S0 Z + V^T U for this wave's 16 rows.  Block
        // b = l / 4 of lane l sums key columns 32 q + 4 (l / 8) + e for rows
        // 8 h + 4 (b & 1) + (0..3) (h = 0 from the even loads, 1 from the odd
        // ones); the eight key groups l / 8 meet by a rotate and lane swaps.
        if (has_rows) {
            st* out = static_cast<st*>(pk->o);
            // window columns 4 tg .. +3 (the first group is peeled off the loop,
            // so its products can start as each checkpoint group lands)
            auto out_group = [&](int tg, f32x4 a0, f32x4 a1) {
                f32x4 b0 = {0.0f, 0.0f, 0.0f, 0.0f}, b1 = b0;
                const float* zrow = Zs + (4 * tg + (lane & 3)) * Cfg::ZST + 4 * (lane >> 3);
                // all of this lane's Z values are read before the first product
                f32x4 zall[K / 32];
#pragma unroll
                for (int q = 0; q < K / 32; ++q)
                    zall[q] = lds_read<f32x4>(zrow, 128u * q);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < K / 16; ++i) {
                    const f32x4 za = zall[i >> 1];
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
                // lane l, register r: window column r of row 8 h + l % 8 (partial
                // over key group l / 8); after the sums lane l stores half
                // (l / 8) / 4, window column (l / 8) % 4
                const f32x4 lo = a0 + b0, hi = a1 + b1;
                const int c = lane >> 3;
                float val = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sl = rows8_sum(lo[r]), sh = rows8_sum(hi[r]);
                    val = c == r ? sl : (c == 4 + r ? sh : val);
                }
                const int t = 4 * tg + (c & 3);
                if (t < T)
                    out[((static_cast<size_t>(b) * T + t) * pk->HV + hv) * pk->V + r0 + (lane & 7) + 8 * (c >> 2)] =
                        Act::from_f32(pk->scale * val);
            };
            out_group(0, vp0, vp1);
            for (int tg = 1; tg < TP / 4; ++tg) {
                f32x4 v0, v1;
                value_part<Cfg, Act>(FU, Vs, n, tg, lane, wave * 16, v0, v1);
                out_group(tg, v0, v1);
            }
        } else {
            // waves without rows load the checkpoint registers too and drop them
#pragma unroll
            for (int i = 0; i < K / 16; ++i)
                asm volatile("" ::"v"(sraw[i][0]), "v"(sraw[i][1]), "v"(sraw[i][2]), "v"(sraw[i][3]));
        }
        pk = launder(pk);
        // the next item's keys go to LDS after the outputs (its ring stores
        // would otherwise sit in front of the checkpoint loads the outputs
        // wait for)
        stage_keys(nxt, pf, tid, lane, nxt.valid && it + static_cast<int>(gridDim.x) < nitems);
        cur = nxt;   // the barrier after the next item's first loads orders the LDS reuse
    }
}

// ------------------------------------------------------------------- host

template <class Act, int K, int LM>
struct VSel;

// Value tile capacity per instantiation: 128 rows, except fp32 activations
// with 128-record rings (32 rows) where LDS would not hold more.
template <class Act, int LM>
constexpr int bvm_of()
{
    return (Act::bytes == 4 && LM > 64) ? 32 : 128;
}

template <class Act, int K, int LM>
using CfgOf = VCfg<Act, K, LM, bvm_of<Act, LM>()>;

template <class Act, int K, int LM>
static size_t lds_of()
{
    return CfgOf<Act, K, LM>::total;
}

static size_t lds_for(const gdn_shape& sh)
{
    const bool bf = sh.act == GDN_BF16;
    const bool big = sh.L > 64;
    switch (sh.K) {
    case 64:
        return bf ? (big ? lds_of<ActBF16, 64, 128>() : lds_of<ActBF16, 64, 64>())
                  : (big ? lds_of<ActF32, 64, 128>() : lds_of<ActF32, 64, 64>());
    case 128:
        return bf ? (big ? lds_of<ActBF16, 128, 128>() : lds_of<ActBF16, 128, 64>())
                  : (big ? lds_of<ActF32, 128, 128>() : lds_of<ActF32, 128, 64>());
    case 256:
        return bf ? lds_of<ActBF16, 256, 64>() : lds_of<ActF32, 256, 64>();
    default: return ~static_cast<size_t>(0);
    }
}

static int bvm_for(const gdn_shape& sh)
{
    return (sh.act == GDN_F32 && sh.L > 64) ? 32 : 128;
}

// Value rows per work item: the largest power of two (16..capacity) that
// divides V, 16 per wave.
int verify_tile_cols(const gdn_shape& sh)
{
    for (int bv = bvm_for(sh); bv >= 16; bv >>= 1)
        if (sh.V % bv == 0)
            return bv;
    return 16;
}

size_t verify_lds_bytes(const gdn_shape& sh)
{
    return lds_for(sh);
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
    using Cfg = CfgOf<Act, K, LM>;
    constexpr int kMinWaves = Cfg::kPerCU == 2 ? 4 : 2;
    const size_t lds = Cfg::total;
    auto kern = verify_kernel<Act, K, LM, Cfg::BVM, kMinWaves>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess)
            return e;
    }
    // persistent grid: as many workgroups as fit at once, never more than items
    const long long items = static_cast<long long>(sh.B) * sh.HV * p.nvt;
    const long long cap = static_cast<long long>(Cfg::kPerCU) * compute_units();
    const unsigned grid = static_cast<unsigned>(items < cap ? items : cap);
    VerifyParams q = p;
    q.step_vt = static_cast<int>(grid % p.nvt);
    q.step_hv = static_cast<int>((grid / p.nvt) % sh.HV);
    q.step_b = static_cast<int>(grid / p.nvt / sh.HV);
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
    p.num_slots = sh.num_slots;
    p.write_ring = write_ring;
    p.BV = verify_tile_cols(sh);
    p.nvt = sh.V / p.BV;
    const int eb = sh.act == GDN_BF16 ? 2 : 4;
    const int vcr = p.BV * eb / 16;      // 16-byte chunks per value-tile row (power of two)
    p.vshift = 0;
    while ((1 << p.vshift) < vcr)
        ++p.vshift;
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
