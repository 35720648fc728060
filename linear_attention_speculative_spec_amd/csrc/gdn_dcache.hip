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
// Execution: one workgroup of four waves per item (row, value head, up to 64
// value rows); wave w owns key tile w (records 16 w .. 16 w + 15, and 16 w +
// 64 .. for 128-record rings) and value tile w (rows 16 w .. 16 w + 15):
//   1. loads, the key side's first: the window keys and queries, once per
//      workgroup (the threads share the live columns' 16-byte chunks), then
//      each wave's key tile (ring history, then window keys; tiles past the
//      last record load nothing) and the gate inputs, then the wave's
//      checkpoint rows: waiting for the key side never waits for these;
//   2. the window columns' norms (reduced over the threads of a column), their
//      raw bits and normalised values to LDS, the window keys to the raw
//      ring; one wave forms the gates and their prefix sums (DPP scan); after
//      a barrier each wave forms the dot products of its key rows with the
//      window columns on MFMA 16x16x32 bf16: raw bf16 keys give exact
//      products summed in fp32 (fp32 activations enter as bf16 high parts
//      plus remainders, three products per step); the stored deltas and the
//      window values are issued;
//   3. (barrier) the coupling and output coefficients, over all threads, with
//      the key and column norms;
//   4. (barrier) each wave: e^{Gam} S0 [kh, qh] for its 16 rows on MFMA 4x4x1
//      straight from the checkpoint registers; the stored deltas against the
//      history's coefficients on MFMA 16x16x4 f32; each lane group runs the
//      T-step window recurrence for the 16 rows and writes every fourth
//      output and delta.
// Workgroups are not persistent: several items per compute unit are in
// different phases at once, so one item's load latency is covered by the
// others' arithmetic.  The items of one qk head (its value heads and value
// parts read the same keys and window columns) get workgroup numbers equal
// modulo 8, which puts them on one die and its L2.
#include <type_traits>

#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kDcWaves = 4;                        // waves per workgroup (one item)
constexpr int kDcThreads = 64 * kDcWaves;
constexpr int kRPI = 16 * kDcWaves;                // value rows per item (a tile of 16 per wave)
constexpr int kTMax = 16;                          // window tokens at most
constexpr int kDPre = 16;                          // stored deltas per lane held in registers
constexpr float kLog2eDc = 1.4426950408889634f;

// Compile-time layout of one instantiation: activation type, key width K,
// window capacity TM (4, 8 or 16 tokens), ring capacity LM (64 or 128).
template <class Act, int K_, int TM_, int LM_>
struct DcCfg {
    static constexpr int K = K_, TM = TM_, LM = LM_;
    static constexpr int eb = Act::bytes;
    static constexpr bool kF32 = eb == 4;
    static constexpr int KS = K / 32;              // matrix steps over the key
    static constexpr int TP = TM;                  // window columns of each kind (keys, queries)
    static constexpr int PC = 2 * TP;              // window columns: keys 0..TP-1, queries TP..
    static constexpr int NCT = (PC + 15) / 16;     // 16-column groups of window columns
    static constexpr int SW = PC + 16 * NCT + 4;   // row stride of a wave's result rows
    static constexpr int CPC = K * eb / 16;        // 16-byte chunks of a key row
    static constexpr int NBL = (2 * TM * CPC + kDcThreads - 1) / kDcThreads;   // window chunks per thread
    static constexpr int BRS = K * eb + 16;        // bytes per raw window column in LDS (16-byte pad: banks)
    static constexpr int RPL = LM / 64;            // gate records per lane
    static constexpr int NTW = LM / 64;            // 16-record key tiles per wave
    // registers: checkpoint tile, deltas, window values, window and key
    // operands (fp32 activations carry a remainder part too)
    static constexpr int kRegs = K / 4 + kDPre + TM + (kF32 ? 2 : 1) * 4 * KS * (NCT + NTW) + 36;
    // waves per SIMD: 6 (six workgroups per compute unit, 80 registers) for
    // bf16 windows of up to 4 tokens on 64-record rings up to K = 128: the
    // window columns take one 16-byte chunk per thread, and the deltas and
    // window values are loaded once the key operands are consumed; else 4
    // where the estimate fits 128 registers, else 2.  More items per compute
    // unit cover more of each item's load latency.
    static constexpr int kMinWaves = (!kF32 && TM == 4 && LM == 64 && K <= 128) ? 6 : (kRegs <= 128 ? 4 : 2);
};

struct DcParams {
    int B, T, H, HV, V, L, num_slots, write_ring, nparts, nunits;
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
    // the workgroup's LDS, in floats: X [PC][KX] normalised window keys
    // (columns 0..TP-1) and queries (TP..PC-1); P [L + 4][PC] raw dot
    // products, then the history's coefficients (rows hist .. hist + 2
    // zero); W [TP][PC] the window records' coefficients; E [PC] the window
    // tokens' decays e^{Gam}; BW [TP] their betas; RNC [PC] window column
    // norms; gam [L], bet [L], RN [L] records' prefix gates (log2), betas,
    // key norms; R [kDcWaves][16][SW] each wave's rows: decayed S0 products
    // (columns 0..PC-1), then the history's sums (PC..); BR [16 NCT] raw
    // window columns (keys 0..T-1, then queries), the dot products' operands
    int KX, o_p, o_w, o_e, o_bw, o_rnc, o_gam, o_bet, o_rn, o_r, o_br;
};

// Read-only, wave-uniform metadata through the constant address space.
template <class T>
__device__ __forceinline__ T ldu(const T* ptr, size_t i)
{
    typedef const __attribute__((address_space(4))) T* cptr;
    return ((cptr)ptr)[i];
}

// x plus its value in the paired 16-lane row (lane l ^ 16) or 32-lane half
// (lane l ^ 32): every lane of the pair receives the same bits.
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

// Sum over the four lanes l % 16 + 16 q (q = 0..3), delivered to each.
__device__ __forceinline__ float quarters_sum_dc(float x)
{
    return swap32_sum_dc(swap16_sum_dc(x));
}

// Sum over aligned groups of N lanes (N = 8, 16, 32 or 64), delivered to
// each lane of the group: DPP within quads, half rows and rows, then lane
// swaps between rows.
template <int N>
__device__ __forceinline__ float group_sum_dc(float x)
{
    static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group of 8, 16, 32 or 64 lanes");
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));   // row_half_mirror
    if constexpr (N >= 16)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));   // row_mirror
    if constexpr (N >= 32)
        x = swap16_sum_dc(x);
    if constexpr (N >= 64)
        x = swap32_sum_dc(x);
    return x;
}

// Two values summed over lane pairs at once: lanes with bit 5 clear (lanes
// 0..31) receive x[l] + x[l ^ 32], the others y[l] + y[l ^ 32].
__device__ __forceinline__ float pair32_sum(float x, float y)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const unsigned a = p[0], b = p[1];
    return __uint_as_float(a) + __uint_as_float(b);
}

// The same over lane bit 4: x[l] + x[l ^ 16] where bit 4 is clear, else
// y[l] + y[l ^ 16].
__device__ __forceinline__ float pair16_sum(float x, float y)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    const unsigned a = p[0], b = p[1];
    return __uint_as_float(a) + __uint_as_float(b);
}

// The same over lane bit 3 (a DPP rotation by 8 within each 16-lane row).
__device__ __forceinline__ float pair8_sum(float x, float y, bool b3)
{
    const float send = b3 ? x : y, keep = b3 ? y : x;
    return keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x128, 0xF, 0xF, false));
}

// DPP move of x; lanes without a source receive 0.
template <int CTRL, int RM>
__device__ __forceinline__ float dpp0_dc(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, RM, 0xF, true));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_scan_dc(float x)
{
    x += dpp0_dc<0x111, 0xF>(x);   // row_shr:1
    x += dpp0_dc<0x112, 0xF>(x);   // row_shr:2
    x += dpp0_dc<0x114, 0xF>(x);   // row_shr:4
    x += dpp0_dc<0x118, 0xF>(x);   // row_shr:8
    x += dpp0_dc<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp0_dc<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// Eight consecutive activations of a key or query row: their raw bits (one
// 16-byte load for bf16, two for fp32), loaded unconditionally (callers pass
// a valid row for dead lanes and drop the values later): a load under a
// branch, or arithmetic on the value right after it, makes the compiler wait
// for it, and with it for every load issued before.
template <class Act>
struct RawChunk {
    uint4 w[Act::bytes == 2 ? 1 : 2];
};

template <class Act>
__device__ __forceinline__ RawChunk<Act> load_raw(const typename Act::storage* row, int e0)
{
    RawChunk<Act> c;
    c.w[0] = *reinterpret_cast<const uint4*>(row + e0);
    if constexpr (Act::bytes == 4)
        c.w[1] = *reinterpret_cast<const uint4*>(row + e0 + 4);
    return c;
}

// The chunk as the operand of a bf16 matrix step: the raw bits themselves
// (bf16), or the bf16 rounding hi and the bf16 rounding of the remainder lo
// (fp32).  Dead lanes carry the values of a valid row; their products are
// never stored.
template <class Act>
struct KeyChunk {
    bf16x8 hi, lo;
};

template <class Act>
__device__ __forceinline__ KeyChunk<Act> to_operand(const RawChunk<Act>& r)
{
    KeyChunk<Act> c;
    if constexpr (Act::bytes == 2) {
        c.hi = __builtin_bit_cast(bf16x8, r.w[0]);
        c.lo = c.hi;
    } else {
        const uint4 w0 = r.w[0], w1 = r.w[1];
        const float x[8] = {__uint_as_float(w0.x), __uint_as_float(w0.y), __uint_as_float(w0.z), __uint_as_float(w0.w),
                            __uint_as_float(w1.x), __uint_as_float(w1.y), __uint_as_float(w1.z), __uint_as_float(w1.w)};
        uint32_t h[4], l[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
            l[e] = pack_bf16x2(x[2 * e] - __uint_as_float(h[e] << 16), x[2 * e + 1] - __uint_as_float(h[e] & 0xFFFF0000u));
        }
        c.hi = __builtin_bit_cast(bf16x8, uint4{h[0], h[1], h[2], h[3]});
        c.lo = __builtin_bit_cast(bf16x8, uint4{l[0], l[1], l[2], l[3]});
    }
    return c;
}

// ss plus the chunk's sum of squares (of the activations as stored).
template <class Act>
__device__ __forceinline__ float raw_sumsq(const RawChunk<Act>& r, float ss)
{
    if constexpr (Act::bytes == 2) {
        const uint4 w = r.w[0];
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bf16x2 x = __builtin_bit_cast(bf16x2, u[e]);
            ss = __builtin_amdgcn_fdot2_f32_bf16(x, x, ss, false);
        }
    } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 w = r.w[h];
            const float x[4] = {__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w)};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ss = __builtin_fmaf(x[e], x[e], ss);
        }
    }
    return ss;
}

template <class Act>
__device__ __forceinline__ f32x4 key_product(const KeyChunk<Act>& a, const KeyChunk<Act>& b, f32x4 acc)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    if constexpr (Act::bytes == 4) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    }
    return acc;
}

// Checkpoint rows r0 .. r0 + 15 of one (slot, value head): load i of lane l
// reads row 8 (i & 1) + l % 8, key columns 32 (i >> 1) + 4 (l / 8) .. +3, so
// every load instruction covers whole 128-byte lines.
template <int K>
__device__ __forceinline__ void load_tile(const float* rows, int lane, f32x4 (&sraw)[K / 16])
{
    const char* base = reinterpret_cast<const char*>(rows);
    const uint32_t off = static_cast<uint32_t>(((lane & 7) * K + 4 * (lane >> 3)) * 4);
#pragma unroll
    for (int i = 0; i < K / 16; ++i)
        sraw[i] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(base + ((i & 1) * 8 * K + (i >> 1) * 32) * 4 + off));
}

// Stored deltas of lane (row l % 16, group l / 16): records grp + 4 m, m <
// kDPre.  Every load is issued (records past the history read the last one,
// or record 0, again; their coefficients are zero): loads under a branch
// would turn the array into one register vector copied by every branch.
// Offsets are 32-bit from the slab's (uniform) address.
__device__ __forceinline__ void load_deltas(const float* slab, int V, int L, int base, int hist, int lane,
                                            float (&d)[kDPre])
{
    const char* sb = reinterpret_cast<const char*>(slab);
    const uint32_t rb = static_cast<uint32_t>(V) * 4u;
    const uint32_t l4 = static_cast<uint32_t>(lane & 15) * 4u;
    const uint32_t wrap = static_cast<uint32_t>(L - 1);
    const int hb = base + (hist > 0 ? hist - 1 : 0);   // the last history record, before the wrap
    const int gb = base + (lane >> 4);
#pragma unroll
    for (int m = 0; m < kDPre; ++m) {
        const int jb = gb + 4 * m;
        const uint32_t ph = static_cast<uint32_t>(jb < hb ? jb : hb) & wrap;
        d[m] = *reinterpret_cast<const float*>(sb + (__umul24(ph, rb) + l4));
    }
}

}  // namespace

template <class Act, int K, int TM, int LM, int MINW>
__global__ __launch_bounds__(kDcThreads, MINW) void dcache_verify_kernel(const DcParams p)
{
    using Cfg = DcCfg<Act, K, TM, LM>;
    using st = typename Act::storage;
    constexpr int KS = Cfg::KS, NCT = Cfg::NCT, NTW = Cfg::NTW;
    extern __shared__ __align__(16) float sm[];
    float* X = sm;
    float* P = sm + p.o_p;
    float* gam = sm + p.o_gam;
    float* bet = sm + p.o_bet;

    // item of this workgroup: blocks of 8 qk-head units x their per items,
    // one unit per die (workgroup number mod 8)
    const int G = p.HV / p.H;
    const int per = G * p.nparts;
    const int gx = static_cast<int>(blockIdx.x) & 7, gq = static_cast<int>(blockIdx.x) >> 3;
    const int u = (gq / per) * 8 + gx, r = gq % per;
    if (u >= p.nunits)
        return;
    const int b = u / p.H, h = u % p.H;
    const int hv = h * G + r / p.nparts, part = r % p.nparts;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int grp = lane >> 4, rl = lane & 15;
    const int T = p.T, H = p.H;
    const st* kin = static_cast<const st*>(p.k);
    const st* qin = static_cast<const st*>(p.q);
    // ---- 1. loads.  The window columns first, once per workgroup: they
    // depend on the row and qk head only, so they are in flight while the
    // slot's cursors are read.  Chunk m of thread tid: live column c = idx /
    // CPC (keys 0..T-1, then queries), bytes 16 (idx % CPC) .. +15, idx = tid
    // + 256 m; threads past the live columns read column 0 again.
    constexpr int CPC = Cfg::CPC, NBL = Cfg::NBL;
    uint4 braw[NBL];
#pragma unroll
    for (int m = 0; m < NBL; ++m) {
        const int idx = tid + kDcThreads * m;
        const int c = idx / CPC, e = idx % CPC;
        const bool live = c < 2 * T;
        const bool isq = live && c >= T;
        const int t = live ? (isq ? c - T : c) : 0;
        const st* row = (isq ? qin : kin) + ((static_cast<size_t>(b) * T + t) * H + h) * K;
        braw[m] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(row) + 16 * e);
    }
    const int s = ldu(p.slot_idx, b);
    if (!valid_slot(s, p.num_slots)) {
        // padding row: nothing written (the window columns in flight count as used)
#pragma unroll
        for (int m = 0; m < NBL; ++m)
            asm volatile("" ::"v"(braw[m].x), "v"(braw[m].y), "v"(braw[m].z), "v"(braw[m].w));
        return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // the wave with extra work (the gates) rotates with the workgroup number,
    // so that no SIMD hosts all of them: the waves of a workgroup go to the
    // SIMDs in order
    const int gwave = static_cast<int>(blockIdx.x >> 3) & 3;
    constexpr int TP = Cfg::TP, PC = Cfg::PC, SW = Cfg::SW;
    const int L = p.L, KX = p.KX, V = p.V, HV = p.HV;
    const bool flagged = ldu(p.is_flush, s) != 0;
    const int wpc = clamp_wp(ldu(p.write_pos, s), L, T);
    const int base = ldu(p.cache_base, s);
    const int hist = flagged ? 0 : wpc;
    const int n = hist + T;
    const int wp0 = base + wpc;
    const int v0 = part * kRPI;
    const int rows = (V - v0) < kRPI ? (V - v0) : kRPI;
    const bool has_tile = 16 * wave < rows;
    const int r0 = v0 + (has_tile ? 16 * wave : 0);
    const bool wr = p.write_ring != 0;
    const size_t head = static_cast<size_t>(s) * HV + hv;
    st* ringk = static_cast<st*>(p.rawk) + (static_cast<size_t>(s) * H + h) * L * K;

    // then this wave's key tiles, gate inputs, window values and deltas
    // (tiles past the last record load nothing: their products are never
    // formed)
    RawChunk<Act> arow_raw[NTW][KS];
#pragma unroll
    for (int tw = 0; tw < NTW; ++tw) {
        if (16 * (wave + kDcWaves * tw) < n) {
            const int j = 16 * (wave + kDcWaves * tw) + rl;
            const bool live = j < n;
            // dead lanes read window key 0 (valid memory; dropped below)
            const st* row = (live && j < hist) ? ringk + static_cast<size_t>((base + j) & (L - 1)) * K
                                               : kin + ((static_cast<size_t>(b) * T + (live ? j - hist : 0)) * H + h) * K;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                arow_raw[tw][ks] = load_raw<Act>(row, 32 * ks + 8 * grp);
        }
    }
    // gate inputs of records RPL lane + q (gate wave): raw bits of the ring's
    // g and beta, or of the window's a and b (widened in step 2)
    constexpr int RPL = Cfg::RPL;
    typedef typename std::conditional<Cfg::eb == 2, uint16_t, uint32_t>::type actraw;
    uint32_t ga[RPL], gb[RPL];
    const size_t gslab = head * L;
    if (wave == gwave) {
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
            const int j = RPL * lane + q;
            const int jc = j < n ? j : 0;
            if (jc < hist) {
                const int ph = (base + jc) & (L - 1);
                ga[q] = reinterpret_cast<const uint32_t*>(p.rg)[gslab + ph];
                gb[q] = reinterpret_cast<const uint32_t*>(p.rb)[gslab + ph];
            } else {
                const size_t idx = (static_cast<size_t>(b) * T + (jc - hist)) * HV + hv;
                ga[q] = reinterpret_cast<const actraw*>(p.a)[idx];
                gb[q] = reinterpret_cast<const actraw*>(p.b)[idx];
            }
        }
    }
    // the checkpoint rows, behind the key side's loads: loads complete in
    // order for the wait counter, so waiting for the key side does not wait
    // for these
    f32x4 sraw[K / 16];
    load_tile<K>(p.S + (head * V + r0) * K, lane, sraw);

    // ---- 2. dot products of this wave's key rows and the window columns;
    // norms; X (one wave); gates and prefix sums (another)
    float* W = sm + p.o_w;
    float* E = sm + p.o_e;
    float* BW = sm + p.o_bw;
    float* RNC = sm + p.o_rnc;
    float* RN = sm + p.o_rn;
    char* BR = reinterpret_cast<char*>(sm + p.o_br);
    {
        // the window columns: raw bits to BR, normalised to X (norms reduced
        // over the CPC threads of a column), the keys to the ring (part 0 of
        // the first value head of the qk head); dead rows of X are zero
        const bool k_writer = wr && (hv % G == 0) && part == 0;
        constexpr int EPC = 16 / Cfg::eb;            // elements per chunk
#pragma unroll
        for (int m = 0; m < NBL; ++m) {
            const int idx = tid + kDcThreads * m;
            const int c = idx / CPC, e = idx % CPC;
            const uint4 w = braw[m];
            float x[EPC];
            if constexpr (Cfg::eb == 2) {
                const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    x[2 * q] = __uint_as_float(u[q] << 16);
                    x[2 * q + 1] = __uint_as_float(u[q] & 0xFFFF0000u);
                }
            } else {
                x[0] = __uint_as_float(w.x);
                x[1] = __uint_as_float(w.y);
                x[2] = __uint_as_float(w.z);
                x[3] = __uint_as_float(w.w);
            }
            float ss = 0.0f;
#pragma unroll
            for (int q = 0; q < EPC; ++q)
                ss = __builtin_fmaf(x[q], x[q], ss);
            ss = group_sum_dc<CPC>(ss);
            if (c < 2 * T) {
                const bool isq = c >= T;
                const int t = isq ? c - T : c;
                const int col = isq ? TP + t : t;
                const float rn = __builtin_amdgcn_rsqf(ss + p.eps);
                *reinterpret_cast<uint4*>(BR + c * Cfg::BRS + 16 * e) = w;
                float* dst = X + col * KX + EPC * e;
#pragma unroll
                for (int q = 0; q < EPC; q += 4)
                    *reinterpret_cast<f32x4*>(dst + q) = f32x4{x[q] * rn, x[q + 1] * rn, x[q + 2] * rn, x[q + 3] * rn};
                if (!isq && k_writer)
                    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(ringk + static_cast<size_t>((wp0 + t) & (L - 1)) * K) + 16 * e) = w;
                if (e == 0)
                    RNC[col] = rn;
            } else if (c < 2 * TP) {
                // window columns T..TP-1 and TP+T..PC-1 are zero (their products are never read)
                const int z = c - 2 * T;
                const int col = z < TP - T ? T + z : TP + T + (z - (TP - T));
                float* dst = X + col * KX + EPC * e;
#pragma unroll
                for (int q = 0; q < EPC; q += 4)
                    *reinterpret_cast<f32x4*>(dst + q) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
    }
    if (wave == gwave) {
        // gates of the combined sequence: history as recorded, window formed
        // here (and recorded in the ring by part 0); prefix sums
        float gl[RPL], bl[RPL];
        float pair = 0.0f;
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
            const int j = RPL * lane + q;
            gl[q] = 0.0f;
            bl[q] = 0.0f;
            if (j < hist) {
                gl[q] = __uint_as_float(ga[q]);
                bl[q] = __uint_as_float(gb[q]);
            } else if (j < n) {
                const float a_in = Cfg::eb == 2 ? __uint_as_float(ga[q] << 16) : __uint_as_float(ga[q]);
                const float b_in = Cfg::eb == 2 ? __uint_as_float(gb[q] << 16) : __uint_as_float(gb[q]);
                gdn_gate(a_in, b_in, ldu(p.A_log, hv), ldu(p.dt_bias, hv), p.softplus_threshold, gl[q], bl[q]);
                if (wr && part == 0) {
                    const int ph = (wp0 + j - hist) & (L - 1);
                    p.rg[gslab + ph] = gl[q];
                    p.rb[gslab + ph] = bl[q];
                }
            }
            pair += gl[q];
        }
        float run = wave_scan_dc(pair) - pair;
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
            const int j = RPL * lane + q;
            run += gl[q];
            if (j < n) {
                gam[j] = run * kLog2eDc;
                bet[j] = bl[q];
            }
        }
    }
    __syncthreads();
    // the window columns as operands of the bf16 matrix steps (column 16 ct +
    // l % 16, key elements 32 ks + 8 (l / 16) .. +7; columns past 2T hold
    // whatever LDS held: their products are never stored)
    KeyChunk<Act> bcol[NCT][KS];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const char* src = BR + (16 * ct + rl) * Cfg::BRS + (32 * ks + 8 * grp) * Cfg::eb;
            RawChunk<Act> rc;
            rc.w[0] = *reinterpret_cast<const uint4*>(src);
            if constexpr (Cfg::eb == 4)
                rc.w[1] = *reinterpret_cast<const uint4*>(src + 16);
            bcol[ct][ks] = to_operand<Act>(rc);
        }
    // this wave's key tiles against the window columns (raw products, the
    // norms enter with the coefficients); lane l, register q: record 16
    // (wave + 4 tw) + 4 (l / 16) + q, column 16 ct + l % 16
#pragma unroll
    for (int tw = 0; tw < NTW; ++tw) {
        const int j0 = 16 * (wave + kDcWaves * tw);
        if (j0 >= n)
            continue;
        KeyChunk<Act> arow[KS];
        float ss = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            arow[ks] = to_operand<Act>(arow_raw[tw][ks]);
            ss = raw_sumsq<Act>(arow_raw[tw][ks], ss);
        }
        ss = quarters_sum_dc(ss);
        if (grp == 0 && j0 + rl < n)
            RN[j0 + rl] = __builtin_amdgcn_rsqf(ss + p.eps);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = key_product<Act>(arow[ks], bcol[ct][ks], acc);
            const int c = 16 * ct + rl;
            if (c < 2 * T) {
                const int col = c < T ? c : TP + (c - T);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int jr = j0 + 4 * grp + q;
                    if (jr < n)
                        P[jr * PC + col] = acc[q];
                }
            }
        }
    }
    // the stored deltas and window values, issued once the key operands'
    // registers are free (they are first read after the checkpoint products)
    float dpre[kDPre];
    load_deltas(p.rd + head * L * V + r0, V, L, base, hist, lane, dpre);
    st vw[TM];
    {
        const st* vb = static_cast<const st*>(p.v) + (static_cast<size_t>(b) * T * HV + hv) * V + r0 + rl;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            vw[i] = vb[static_cast<size_t>(i < T ? i : T - 1) * HV * V];
    }
    __syncthreads();

    // ---- 3. coefficients: column i < T of record j couples window token i to
    // j (j < hist + i): beta e^{Gam_{h+i} - Gam_j} kh_i . kh_j; query column t
    // weighs d_j in output t (j <= hist + t): e^{Gam_{h+t} - Gam_j} kh_j . qh_t.
    // History records' coefficients stay in P, whose rows hist .. hist + 2
    // become zero (the history product reads them for records past the
    // history); the window records' go to W.
    {
        const int nz = hist + (T > 3 ? T : 3);
        for (int task = tid; task < nz * PC; task += kDcThreads) {
            const int j = task / PC, col = task % PC;
            const bool isq = col >= TP;
            const int t = isq ? col - TP : col;
            float coef = 0.0f;
            if (j < n && t < T) {
                const int i = hist + t;
                if (isq ? j <= i : j < i) {
                    const float w = __builtin_amdgcn_exp2f(gam[i] - gam[j]);
                    coef = (isq ? w : bet[i] * w) * (P[task] * (RN[j] * RNC[col]));
                }
            }
            if (j < hist) {
                P[task] = coef;
            } else {
                P[task] = 0.0f;
                if (j < n)
                    W[(j - hist) * PC + col] = coef;
            }
        }
        if (tid < PC) {
            const bool isq = tid >= TP;
            const int t = isq ? tid - TP : tid;
            E[tid] = t < T ? __builtin_amdgcn_exp2f(gam[hist + t]) : 0.0f;
            for (int u = T; u < TP; ++u)
                W[u * PC + tid] = 0.0f;
            if (tid < TP)
                BW[tid] = tid < T ? bet[hist + tid] : 0.0f;
        }
    }
    __syncthreads();

    // ---- 4. this wave's tile
    if (!has_tile) {
#pragma unroll
        for (int i = 0; i < K / 16; ++i)
            asm volatile("" ::"v"(sraw[i][0]), "v"(sraw[i][1]), "v"(sraw[i][2]), "v"(sraw[i][3]));
#pragma unroll
        for (int m = 0; m < kDPre; ++m)
            asm volatile("" ::"v"(dpre[m]));
        return;
    }
    float* Rw = sm + p.o_r + wave * 16 * SW;
    // e^{Gam} S0 [kh, qh] for the tile's rows, eight window columns at a time
    // on MFMA 4x4x1: lane l, register q of acc[e][hh] holds column 8 cp + 4 e
    // + q of row 8 hh + l % 8, partial over key group l / 8.  The 16 partial
    // sums of a lane are reduced over the key groups (lane bits 3..5) while
    // being spread out: afterwards lane l holds column 8 cp + l / 8 of rows
    // l % 8 and 8 + l % 8.
#pragma unroll
    for (int cp = 0; cp < PC / 8; ++cp) {
        f32x4 acc[2][2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
            acc[e][0] = acc[e][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < K / 16; ++i) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const f32x4 za = *reinterpret_cast<const f32x4*>(
                    X + (8 * cp + 4 * e + (lane & 3)) * KX + 4 * (lane >> 3) + 32 * (i >> 1));
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    acc[e][i & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(za[k], sraw[i][k], acc[e][i & 1], 0, 0, 0);
            }
        }
        float v8[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v8[4 * hh + q] = pair32_sum(acc[0][hh][q], acc[1][hh][q]);
        const bool b3 = (lane & 8) != 0;
        const int c = 8 * cp + (lane >> 3);
        const float ec = E[c];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const float x = pair16_sum(v8[4 * hh], v8[4 * hh + 2]);
            const float y = pair16_sum(v8[4 * hh + 1], v8[4 * hh + 3]);
            Rw[(8 * hh + (lane & 7)) * SW + c] = pair8_sum(x, y, b3) * ec;
        }
    }
    // stored deltas against the history's coefficients on MFMA 16x16x4 f32:
    // A (lane l) the delta of record grp + 4 m at row rl, B (lane l) the
    // coefficient of record grp + 4 m in column 16 cb + rl; D (lane l,
    // register r) row 4 grp + r, column 16 cb + rl.  Coefficient rows from
    // hist on are zero, so records past the history weigh nothing (columns
    // past PC read the next row and are never used).
    f32x4 hacc[NCT];
#pragma unroll
    for (int cb = 0; cb < NCT; ++cb)
        hacc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < kDPre; ++m) {
        if (4 * m < hist) {                      // uniform
            const float* cj = P + (grp + 4 * m) * PC + rl;
#pragma unroll
            for (int cb = 0; cb < NCT; ++cb)
                hacc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(dpre[m], cj[16 * cb], hacc[cb], 0, 0, 0);
        }
    }
    if constexpr (LM - 1 > 4 * kDPre) {
        // records past the registers (rings longer than 64 records)
        const float* dslab = p.rd + head * L * V + r0 + rl;
        for (int m = kDPre; 4 * m < hist; ++m) {
            const int j = grp + 4 * m;
            const int jc = j < hist ? j : hist - 1;
            const float dv = dslab[static_cast<size_t>((base + jc) & (L - 1)) * V];
            const float* cj = P + j * PC + rl;
#pragma unroll
            for (int cb = 0; cb < NCT; ++cb)
                hacc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(dv, cj[16 * cb], hacc[cb], 0, 0, 0);
        }
    }
#pragma unroll
    for (int cb = 0; cb < NCT; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            Rw[(4 * grp + r) * SW + PC + 16 * cb + rl] = hacc[cb][r];
    // window deltas of row r0 + rl: every lane forms all T of them (the
    // recurrence); lane group grp then takes tokens t = grp + 4 m with
    // uniform code (per-lane LDS indices and selects over the registers: one
    // branch per token would be issued by every lane group), writing the
    // output, the delta and the raw value
    const float* Rr = Rw + rl * SW;
    float dw[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        dw[i] = 0.0f;
        if (i < T) {
            float vi;
            if constexpr (Act::bytes == 2)
                vi = bf16_to_f32(vw[i]);
            else
                vi = vw[i];
            float d = BW[i] * (vi - Rr[i]) - Rr[PC + i];
#pragma unroll
            for (int i2 = 0; i2 < TM; ++i2)
                if (i2 < i)
                    d = __builtin_fmaf(-W[i2 * PC + i], dw[i2], d);
            dw[i] = d;
        }
    }
    char* obase = reinterpret_cast<char*>(static_cast<st*>(p.o) + (static_cast<size_t>(b) * T * HV + hv) * V + r0);
    char* dbase = reinterpret_cast<char*>(p.rd + gslab * V + r0);
    char* vbase = reinterpret_cast<char*>(static_cast<st*>(p.rawv) + gslab * V + r0);
#pragma unroll
    for (int m = 0; m < TM / 4; ++m) {
        const int t = grp + 4 * m;
        const int tc = t < T ? t : T - 1;          // dead lanes read a valid token
        float dsel = 0.0f;
        st vsel = vw[0];
#pragma unroll
        for (int u = 0; u < TM; ++u) {
            dsel = tc == u ? dw[u] : dsel;
            vsel = tc == u ? vw[u] : vsel;
        }
        float acc = Rr[TP + tc] + Rr[PC + TP + tc];
        const float* wq = W + TP + tc;
#pragma unroll
        for (int u = 0; u < TM; ++u)
            if (u < T)                             // coefficients past token tc are zero
                acc = __builtin_fmaf(wq[u * PC], dw[u], acc);
        if (t < T) {
            const uint32_t oo = static_cast<uint32_t>(t * HV * V + rl) * Cfg::eb;
            *reinterpret_cast<st*>(obase + oo) = Act::from_f32(p.scale * acc);
            if (wr) {
                const uint32_t ri = static_cast<uint32_t>(((wp0 + t) & (L - 1)) * V + rl);
                *reinterpret_cast<float*>(dbase + ri * 4u) = dsel;
                *reinterpret_cast<st*>(vbase + ri * Cfg::eb) = vsel;
            }
        }
    }
}

// ------------------------------------------------------------------- host

namespace {

struct DcLayout {
    int KX, o_p, o_w, o_e, o_bw, o_rnc, o_gam, o_bet, o_rn, o_r, o_br, total;   // floats
};

// Window capacity of the instantiation that serves T tokens.
int dc_tm(int T)
{
    return T <= 4 ? 4 : (T <= 8 ? 8 : kTMax);
}

DcLayout dc_layout(const gdn_shape& sh)
{
    const int TP = dc_tm(sh.T), PC = 2 * TP;
    const int SW = PC + 16 * ((PC + 15) / 16) + 4;
    auto up4 = [](int x) { return (x + 3) & ~3; };
    DcLayout d;
    d.KX = sh.K + 16;   // rows read four at a time as 16-byte groups: a 64-byte pad keeps them off each other's banks
    d.o_p = PC * d.KX;
    d.o_w = d.o_p + (sh.L + 4) * PC;
    d.o_e = d.o_w + TP * PC;
    d.o_bw = d.o_e + PC;
    d.o_rnc = up4(d.o_bw + TP);
    d.o_gam = d.o_rnc + PC;
    d.o_bet = d.o_gam + sh.L;
    d.o_rn = d.o_bet + sh.L;
    d.o_r = up4(d.o_rn + sh.L);
    d.o_br = d.o_r + kDcWaves * 16 * SW;
    const int brs = sh.K * (sh.act == GDN_BF16 ? 2 : 4) + 16;   // bytes per raw window column
    d.total = d.o_br + 16 * ((PC + 15) / 16) * brs / 4;
    return d;
}

}  // namespace

size_t dcache_lds_bytes(const gdn_shape& sh)
{
    return static_cast<size_t>(dc_layout(sh).total) * 4;
}

template <class Act, int K, int TM, int LM>
static hipError_t launch_dc_k(const gdn_shape& sh, const DcParams& p, hipStream_t stream)
{
    using Cfg = DcCfg<Act, K, TM, LM>;
    auto kern = dcache_verify_kernel<Act, K, TM, LM, Cfg::kMinWaves>;
    const size_t lds = dcache_lds_bytes(sh);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess)
            return e;
    }
    // blocks of 8 qk-head units, each unit's items one per row of 8
    const long long per = static_cast<long long>(sh.HV / sh.H) * p.nparts;
    const long long blocks = (static_cast<long long>(p.nunits) + 7) / 8;
    const unsigned grid = static_cast<unsigned>(blocks * 8 * per);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kDcThreads), lds, stream, p);
    return hipGetLastError();
}

template <class Act, int K, int LM>
static hipError_t launch_dc_t(const gdn_shape& sh, const DcParams& p, hipStream_t stream)
{
    if (sh.T <= 4)
        return launch_dc_k<Act, K, 4, LM>(sh, p, stream);
    if (sh.T <= 8)
        return launch_dc_k<Act, K, 8, LM>(sh, p, stream);
    return launch_dc_k<Act, K, kTMax, LM>(sh, p, stream);
}

template <class Act>
static hipError_t launch_dc_act(const gdn_shape& sh, const DcParams& p, hipStream_t stream)
{
    const bool big = sh.L > 64;
    switch (sh.K) {
    case 64: return big ? launch_dc_t<Act, 64, 128>(sh, p, stream) : launch_dc_t<Act, 64, 64>(sh, p, stream);
    case 128: return big ? launch_dc_t<Act, 128, 128>(sh, p, stream) : launch_dc_t<Act, 128, 64>(sh, p, stream);
    case 256:
        if (big)
            return hipErrorInvalidValue;
        return launch_dc_t<Act, 256, 64>(sh, p, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dcache_verify(const gdn_shape& sh, const WindowPtrs& w, const float* S,
                                const int32_t* slot_idx, const CursorPtrs& c, const RingPtrs& r,
                                float* ring_d, int write_ring, void* o, hipStream_t stream)
{
    if (sh.B == 0)
        return hipSuccess;
    const DcLayout lay = dc_layout(sh);
    DcParams p = {};
    p.B = sh.B;
    p.T = sh.T;
    p.H = sh.H;
    p.HV = sh.HV;
    p.V = sh.V;
    p.L = sh.L;
    p.num_slots = sh.num_slots;
    p.write_ring = write_ring;
    p.nparts = (sh.V + kRPI - 1) / kRPI;
    p.nunits = sh.B * sh.H;
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
    p.KX = lay.KX;
    p.o_p = lay.o_p;
    p.o_w = lay.o_w;
    p.o_e = lay.o_e;
    p.o_bw = lay.o_bw;
    p.o_rnc = lay.o_rnc;
    p.o_gam = lay.o_gam;
    p.o_bet = lay.o_bet;
    p.o_rn = lay.o_rn;
    p.o_r = lay.o_r;
    p.o_br = lay.o_br;
    return sh.act == GDN_BF16 ? launch_dc_act<ActBF16>(sh, p, stream)
                              : launch_dc_act<ActF32>(sh, p, stream);
}

}  // namespace gdn
