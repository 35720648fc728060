// gdn_common.h -- device helpers shared by the libgdnverify kernels (gfx950).
//
// Everything numeric that two kernels must reproduce bit for bit lives here
// once: the gating of a window token, the l2 norm and the gated delta step of
// one state row (with the head's decay carried in a scalar).  The ring
// verify and the snapshot verify both call gdn_gate, so the gate/beta they
// record in the ring are the same bits; the exact fold and the snapshot
// verify both call rnorm16/scale_decay/step_row (or step_rows4, which gives
// four rows step_row's bits), so folding a recorded window reproduces the
// snapshot path's state exactly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdnverify.h"

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ bf16 helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t u)
{
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Round-to-nearest-even of two floats into packed bf16 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x)
{
    return static_cast<uint16_t>(pack_bf16x2(x, 0.0f) & 0xFFFFu);
}

// Activation dtype traits: storage type and exact widening to fp32.
struct ActF32 {
    typedef float storage;
    static constexpr int bytes = 4;
    __device__ static float load(const storage* p) { return *p; }
    __device__ static storage from_f32(float x) { return x; }
};

struct ActBF16 {
    typedef uint16_t storage;
    static constexpr int bytes = 2;
    __device__ static float load(const storage* p) { return bf16_to_f32(*p); }
    __device__ static storage from_f32(float x) { return f32_to_bf16(x); }
};

// Four consecutive activations widened to fp32 (8-byte or 16-byte load).
template <class Act>
__device__ __forceinline__ f32x4 load4(const typename Act::storage* p);

template <>
__device__ __forceinline__ f32x4 load4<ActF32>(const float* p)
{
    return *reinterpret_cast<const f32x4*>(p);
}

template <>
__device__ __forceinline__ f32x4 load4<ActBF16>(const uint16_t* p)
{
    uint2 u = *reinterpret_cast<const uint2*>(p);
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                 __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u)};
}

// Raw copy of four activations (the ring's bit-exact side channel).
template <class Act>
__device__ __forceinline__ void copy4(typename Act::storage* dst, const typename Act::storage* src)
{
    if constexpr (Act::bytes == 4)
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
    else
        *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
}

// ------------------------------------------------------------------ gating

// g = -exp(A_log) * softplus(a + dt_bias), beta = sigmoid(b), in fp32
// (fused GDN gating with an fp32 sigmoid; softplus is the identity above the
// threshold).  The one routine every kernel uses for window tokens.
__device__ __forceinline__ void gdn_gate(float a, float b, float A_log, float dt_bias,
                                         float threshold, float& g, float& beta)
{
    const float x = a + dt_bias;
    const float sp = x > threshold ? x : log1pf(expf(x));
    g = -expf(A_log) * sp;
    beta = 1.0f / (1.0f + expf(-b));
}

// -------------------------------------------------------- wave reductions

template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of 16 lanes; every lane of the group receives
// the same bits (each stage adds a pair in both orders of a commutative op).
__device__ __forceinline__ float group16_sum(float x)
{
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);   // row_half_mirror: lanes i <-> 7-i within 8
    x += dpp<0x140>(x);   // row_mirror: lanes i <-> 15-i within 16
    return x;
}

// Sum over aligned groups of W lanes (W a power of two <= 64) by xor shuffles.
template <int W>
__device__ __forceinline__ float group_sum(float x)
{
#pragma unroll
    for (int m = 1; m < W; m <<= 1)
        x += __shfl_xor(x, m, 64);
    return x;
}

// ------------------------------------------------- one state row of a step
//
// A row of S (V x K, K contiguous) is spread over 16 lanes; lane c holds
// columns 64*m + 4*c + e (m < K/64, e < 4), EPL = K/16 values.

template <int EPL>
__device__ __forceinline__ float rnorm16(const float (&x)[EPL], float eps)
{
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        ss = __builtin_fmaf(x[e], x[e], ss);
    ss = group16_sum(ss);
    return 1.0f / sqrtf(ss + eps);
}

// The state of one (slot, value head) is carried as c S': one scalar c
// shared by all its rows, and the rows S'.  A record's decay e^g multiplies c
// only; the rows take the delta-rule step divided through by c, so a step
// costs no per-element decay.  When c would drop below 2^-64 the rows absorb
// it (S' <- c S', c <- 1), which keeps S' within 2^64 of the state.  The
// gates are at most 1 (g <= 0), so c stays in [2^-64, 1].
constexpr float kScaleFloor = 5.421010862427522e-20f;   // 2^-64

// c <- c e^g.  True when the rows must first be multiplied by f (and c is
// then 1).
__device__ __forceinline__ bool scale_decay(float& c, float decay, float& f)
{
    f = c * decay;
    const bool absorb = f < kScaleFloor;
    c = absorb ? 1.0f : f;
    return absorb;
}

// One record on a row held as S' (state c S'): u' = S' . k_hat, then
// S' += (bc v - beta u') k_hat with bc = beta / c, i.e. the delta rule
// S <- S + beta (v - c u') k_hat divided by c.
template <int EPL>
__device__ __forceinline__ void step_row(float (&s)[EPL], const float (&kh)[EPL], float v,
                                         float bc, float beta)
{
    float u = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        u = __builtin_fmaf(s[e], kh[e], u);
    u = group16_sum(u);
    const float d = __builtin_fmaf(-beta, u, bc * v);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        s[e] = __builtin_fmaf(d, kh[e], s[e]);
}

// group16_sum of four values (one per state row of the lane group) reduced
// transposed, with the same bits per row: at every stage a lane adds, for
// fewer rows, exactly the two partial sums that group16_sum adds (quad_perm
// pairs, then the other quad of the octet, then the other octet; fp add is
// commutative, so the operand order per lane does not matter).  After the
// first two stages lane i holds row 2 (i & 1) + ((i >> 1) & 1) (odd = i & 1,
// second = i & 2); the two rotations leave the full sums in quads 1 and 3
// (quads 0 and 2 add the octets in another association).  Row j's sum is
// then on lane 12 + (j >> 1) + 2 (j & 1) of the group: bcast_row<j> reads it.
__device__ __forceinline__ float sum16_rows4(const float (&u)[4], bool odd, bool second)
{
    // lanes i, i^1: even lanes keep rows 0 and 1, odd lanes rows 2 and 3
    const float ka = odd ? u[2] : u[0], kb = odd ? u[3] : u[1];
    const float sa = odd ? u[0] : u[2], sb = odd ? u[1] : u[3];
    const float y0 = ka + dpp<0xB1>(sa), y1 = kb + dpp<0xB1>(sb);
    // lanes i, i^2 (same parity): bit 1 picks the row
    const float k2 = second ? y1 : y0, s2 = second ? y0 : y1;
    float z = k2 + dpp<0x4E>(s2);
    z += dpp<0x124>(z);   // row_ror:4: quad q adds quad q-1
    z += dpp<0x128>(z);   // row_ror:8: quad q adds quad q-2
    return z;
}

// Row j's value of a per-lane quantity laid out as sum16_rows4 leaves it,
// on every lane of the group (row_newbcast from lane 12 + (j >> 1) + 2 (j & 1)).
template <int J>
__device__ __forceinline__ float bcast_row(float x)
{
    return dpp<0x15C + (J >> 1) + 2 * (J & 1)>(x);
}

// Lane-invariant parts of the transposed layout: the lane's row is
// 2 odd + second.
__device__ __forceinline__ int row4_of_lane(int c) { return 2 * (c & 1) + ((c >> 1) & 1); }

// A per-lane value of the sum16_rows4 layout whose quads 1 and 3 are right
// (the full sums), copied into quads 0 and 2: row_ror:4 written to banks 0
// and 2 only, so quad 0 reads quad 3 and quad 2 reads quad 1.  Lane i of
// every quad then holds the value of row row4_of_lane(i).
__device__ __forceinline__ float quads13(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, x), __builtin_bit_cast(int, x), 0x124, 0xF, 0x5, false));
}

// step_row on four rows held by one 16-lane group, with the same bits for
// each row.  The lane's EPL columns of the four rows are held as a[e], one
// 4-vector per column, register i holding row pi(i), pi = (0, 2, 1, 3): the
// row whose d lane i of each quad forms.  The dot products run on the vector
// ALU in step_row's order and are reduced by sum16_rows4; each lane forms its
// own row's d.  Quads 1 and 3 hold the full sums, and quads 0 and 2 take
// theirs by one row rotation written to banks 0 and 2 only.  The update
// a[e] += d kh[e] is then one 4x4x1 fp32 matrix product per column (16 blocks
// of 4 lanes; A from lane i of a block is the d of register i's row, B from
// each lane is its own column's key): one product and one add per element,
// rounded once, so each element gets step_row's fmaf bits.
// vofs = 16 * row4_of_lane(lane & 15); v points at row 0's value (row j's is
// v[16 j]).
template <class Act, int EPL>
__device__ __forceinline__ void step_rows4(f32x4 (&a)[EPL], const float (&kh)[EPL],
                                           const typename Act::storage* v, int vofs, bool odd,
                                           bool second, float bc, float beta)
{
    float ur[4];   // by register
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ur[i] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            ur[i] = __builtin_fmaf(a[e][i], kh[e], ur[i]);
    }
    const float u[4] = {ur[0], ur[2], ur[1], ur[3]};   // by row
    const float z = sum16_rows4(u, odd, second);
    const float d = __builtin_fmaf(-beta, z, bc * Act::load(v + vofs));
    const float dm = quads13(d);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        a[e] = __builtin_amdgcn_mfma_f32_4x4x1f32(dm, kh[e], a[e], 0, 0, 0);
}

// beta / c for step_row
__device__ __forceinline__ float scaled_beta(float beta, float c)
{
    return beta * __builtin_amdgcn_rcpf(c);
}

__device__ __forceinline__ int clamp_wp(int wp, int L, int T)
{
    return wp < 0 ? 0 : (wp > L - T ? L - T : wp);
}

__device__ __forceinline__ bool valid_slot(int s, int num_slots)
{
    return s >= 0 && s < num_slots;
}

}  // namespace gdn
