// gdn2_device.h -- gfx950 building blocks shared by the GDN-2 kernels.
//
// MFMA operand layouts used throughout (wave of 64 lanes, lane l, r = l % 16,
// g = l / 16), checked on gfx950:
//   v_mfma_f32_16x16x32_bf16   A: lane holds A[r][8g + i], i < 8
//                              B: lane holds B[8g + i][r]
//                              D: lane holds D[4g + i][r], i < 4
//   v_mfma_f32_16x16x16_bf16   A: A[r][4g + i], B: B[4g + i][r], D: D[4g + i][r]
// Only the sum over the contraction index matters, so any consistent
// permutation of it between A and B is allowed; the kernels use that to feed a
// D fragment of a transposed product straight back in as an A operand.
//
// Precision: products whose error reaches the output directly use a split
// ("hi + lo") bf16 representation of each fp32 operand, x = hi + lo with
// hi = bf16(x), lo = bf16(x - hi), and three MFMAs (lo*hi + hi*lo + hi*hi),
// which carries about 16 significant bits; accumulation is fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunk = 64;

// Decay range.  The rule puts no floor under alpha (blog on Gated DeltaNet-2, section
// "Independent control on two axes"), so the chunk kernels take any log_alpha <= 0:
//  - a per-token log-decay below kLogDecayFloor is computed as kLogDecayFloor.  A factor
//    exp(-30) = 9.4e-14 on whatever the state held is far below fp32 resolution, and the
//    floor keeps alpha = 0 (log_alpha = -inf) from turning cumulative sums into -inf - -inf;
//  - a chunk in which some key channel's total decay gamma = exp(g_C) is below kGamMin
//    (2^-92, g_C < -63.8) is flagged.  The factorised operands of the chunk form, whose
//    exp(-G) would leave fp32 range there, are then replaced by the exact pairwise decays
//    exp(G_i - G_j) (i >= j, at most 1) in a second, exact pass over the flagged chunks.
// A NaN log-decay passes the floor unchanged, so it propagates.
constexpr float kLogDecayFloor = -30.f;
constexpr float kGamMin = 0x1p-92f;
__device__ __forceinline__ float floor_log_decay(float x) { return x < kLogDecayFloor ? kLogDecayFloor : x; }
constexpr int kThreads = 256;
constexpr int kChunkThreads = 2 * kThreads;   // workgroup of the chunk-parallel backward kernels

// Keep the scheduler from hoisting the LDS fragment loads of later unrolled steps
// above this point (bounds the live registers of a wave).
#define GDN2_SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Phase stamps of the instrumented build (-DGDN2_STAMPS, libgdn2_stamps.so).  GDN2_STAMP_REGS
// declares a wave's eight stamp registers (zero); GDN2_STAMP(buf, idx) reads the shader-clock
// counter (s_memtime) into register idx (a constant); GDN2_STAMP_FLUSH(buf) has lane 0 write all
// eight to buf[0..7] when buf is set.  The flush comes once, after a unit of work's last stamp:
// a store per stamp would queue behind the kernel's own memory traffic and stretch the phases it
// measures.  In the normal build the macros are empty.
#ifdef GDN2_STAMPS
#define GDN2_STAMP_REGS unsigned long long gdn2_stv[8] = {0, 0, 0, 0, 0, 0, 0, 0}
#define GDN2_STAMP(buf, idx)                          \
    do {                                             \
        gdn2_stv[idx] = __builtin_amdgcn_s_memtime(); \
    } while (0)
#define GDN2_STAMP_FLUSH(buf)                                                              \
    do {                                                                                  \
        if ((buf) != nullptr && (threadIdx.x & 63) == 0) {                                \
            _Pragma("unroll") for (int gdn2_i = 0; gdn2_i < 8; ++gdn2_i)(buf)[gdn2_i] =    \
                gdn2_stv[gdn2_i];                                                         \
        }                                                                                 \
    } while (0)
#else
#define GDN2_STAMP_REGS \
    do {                \
    } while (0)
#define GDN2_STAMP(buf, idx) \
    do {                     \
    } while (0)
#define GDN2_STAMP_FLUSH(buf) \
    do {                      \
    } while (0)
#endif

// LDS poison fill of the debug build (-DGDN2_LDS_POISON, libgdn2_poison.so).  At the top of
// every kernel the workgroup fills its whole static LDS allocation, bytes [0,
// __builtin_amdgcn_groupstaticsize()), with all-ones words (a NaN in fp32 and in bf16) and
// waits at a barrier.  A kernel that reads a word of LDS before writing it then sees NaN
// instead of a previous workgroup's leftovers, and its results differ from the normal build's.
// In the normal build the macro is empty.
#ifdef GDN2_LDS_POISON
__device__ __forceinline__ void lds_poison_fill() {
    typedef __attribute__((address_space(3))) unsigned lds_u32;
    // LDS address 0 from a value the compiler cannot fold: a literal null would become the
    // local address space's null value, which is not address 0
    unsigned base = 0;
    asm volatile("" : "+v"(base));
    lds_u32 *p = reinterpret_cast<lds_u32 *>(static_cast<uintptr_t>(base));
    const unsigned n = __builtin_amdgcn_groupstaticsize() / 4u;
    for (unsigned i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0xffffffffu;
    __syncthreads();
}
#define GDN2_POISON_LDS() lds_poison_fill()
#else
#define GDN2_POISON_LDS() \
    do {                  \
    } while (0)
#endif

struct Split8 {
    bf16x8 hi, lo;
};
struct Split4 {
    bf16x4 hi, lo;
};

__device__ __forceinline__ f32x4 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x4 &a, const bf16x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// split-bf16 product: about 16 significant bits per operand
__device__ __forceinline__ f32x4 mfma32x3(const Split8 &a, const Split8 &b, f32x4 c) {
    c = mfma32(a.lo, b.hi, c);
    c = mfma32(a.hi, b.lo, c);
    return mfma32(a.hi, b.hi, c);
}

__device__ __forceinline__ f32x4 mfma16x3(const Split4 &a, const Split4 &b, f32x4 c) {
    c = mfma16(a.lo, b.hi, c);
    c = mfma16(a.hi, b.lo, c);
    return mfma16(a.hi, b.hi, c);
}

__device__ __forceinline__ void split1(float x, __bf16 &hi, __bf16 &lo) {
    hi = (__bf16)x;
    lo = (__bf16)(x - (float)hi);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two values at a time, so each conversion is one packed v_cvt_pk_bf16_f32
__device__ __forceinline__ void split2(float x0, float x1, bf16x2 &hi, bf16x2 &lo) {
    const f32x2 x = {x0, x1};
    hi = __builtin_convertvector(x, bf16x2);
    lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x2), bf16x2);
}

__device__ __forceinline__ Split8 split8(const float *x) {
    bf16x2 h0, h1, h2, h3, l0, l1, l2, l3;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    split2(x[4], x[5], h2, l2);
    split2(x[6], x[7], h3, l3);
    Split8 s;
    s.hi = __builtin_shufflevector(__builtin_shufflevector(h0, h1, 0, 1, 2, 3), __builtin_shufflevector(h2, h3, 0, 1, 2, 3),
                                   0, 1, 2, 3, 4, 5, 6, 7);
    s.lo = __builtin_shufflevector(__builtin_shufflevector(l0, l1, 0, 1, 2, 3), __builtin_shufflevector(l2, l3, 0, 1, 2, 3),
                                   0, 1, 2, 3, 4, 5, 6, 7);
    return s;
}

__device__ __forceinline__ Split4 split4(const f32x4 &x) {
    bf16x2 h0, h1, l0, l1;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    Split4 s;
    s.hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3);
    s.lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3);
    return s;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposing LDS read (ds_read_b64_tr_b16, gfx950).  Within each group of 16
// lanes, lane p receives element (p % 4) of the 4-element bf16 segments that
// lanes 4i + p/4 of the same group address, for i = 0..3.  If lane (p, g)
// addresses row R0 + 4g + p/4, columns C0 + 4(p%4) .. +3 of a row-major bf16
// tile, it receives column C0 + p of rows R0 + 4g + {0,1,2,3}: a 16x16 block
// read transposed, in the MFMA A/B operand order (checked on gfx950).
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16 *p) {
    typedef short s16x4_lds __attribute__((ext_vector_type(4)));
    const s16x4_lds v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_lds *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// value of lane (l - n) inside the same 16-lane row, 0 for the first n lanes of a row
template <int N>
__device__ __forceinline__ float row_shr(float v) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8, "row_shr");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                0x110 + N, 0xf, 0xf, true));
}

// inclusive prefix sum over the 16 lanes of each row
__device__ __forceinline__ float row_scan16(float v) {
    v += row_shr<1>(v);
    v += row_shr<2>(v);
    v += row_shr<4>(v);
    v += row_shr<8>(v);
    return v;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __builtin_bit_cast(float, bits16 << 16);
}

// 8 consecutive elements of a token row, widened to fp32
template <bool BF16>
__device__ __forceinline__ void load8(const void *base, size_t off, bool valid, float *out) {
    if (BF16) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (valid) u = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + off);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            out[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        }
    } else {
        float4 a = make_float4(0, 0, 0, 0), b = make_float4(0, 0, 0, 0);
        if (valid) {
            const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + off);
            a = p[0];
            b = p[1];
        }
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void *base, size_t off, bool valid) {
    if (!valid) return 0.f;
    if (BF16) return bf16_bits_to_float(reinterpret_cast<const uint16_t *>(base)[off]);
    return reinterpret_cast<const float *>(base)[off];
}

// ---- gate inputs: fp32 values, or bf16 logits activated in-kernel ----
// With logits (GL), b = sigmoid(x_b), w = sigmoid(x_w) and log_alpha = log(sigmoid(x_a))
// (the gates are sigmoid outputs of linear projections: blog on Gated DeltaNet-2,
// section "Independent control on two axes"; the decay keeps an fp32 log form).
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.f + exp2_fast(-x * kLog2e)); }

// log(sigmoid(x)) = min(x, 0) - log(1 + exp(-|x|)), in base-2 hardware exp/log
__device__ __forceinline__ float log_sigmoid_f(float x) {
    return fminf(x, 0.f) - __builtin_amdgcn_logf(1.f + exp2_fast(-fabsf(x) * kLog2e)) * kLn2;
}

// one gate element as stored: fp32 value or bf16 logit widened to fp32
template <bool GL>
__device__ __forceinline__ float load_gate1(const void *base, size_t off) {
    if (GL) return bf16_bits_to_float(reinterpret_cast<const uint16_t *>(base)[off]);
    return reinterpret_cast<const float *>(base)[off];
}
// stored decay -> log_alpha, and d log_alpha / d stored
template <bool GL> __device__ __forceinline__ float decay_act(float x) { return GL ? log_sigmoid_f(x) : x; }
template <bool GL> __device__ __forceinline__ float decay_dact(float x) { return GL ? sigmoid_f(-x) : 1.f; }
// stored erase/write gate -> gate value, and d gate / d stored as a function of the gate value
template <bool GL> __device__ __forceinline__ float gate_act(float x) { return GL ? sigmoid_f(x) : x; }
template <bool GL> __device__ __forceinline__ float gate_dact(float v) { return GL ? v * (1.f - v) : 1.f; }

// Map the launch index to a logical work index so that consecutive logical
// indices (the value tiles of one (batch, head)) land on the same XCD and share
// its L2: the hardware deals workgroups to the 8 XCDs round-robin.
__device__ __forceinline__ int xcd_swizzle(int bid, int nb) {
    if (nb % 8 != 0) return bid;
    return (bid % 8) * (nb / 8) + bid / 8;
}

// value of lane (quad base + perm[lane & 3]) for a DPP quad permutation
template <int QPERM>
__device__ __forceinline__ float quad_perm(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), QPERM, 0xf, 0xf, false));
}

// 4x4 transpose inside each quad of lanes (lanes 4q .. 4q + 3).  Before, lane j of the
// quad holds column j of a 4x4 block, x[i] = M[i][j]; after, it holds row j,
// x[i] = M[j][i].  Two exchange rounds (partner j ^ 1, then j ^ 2, as DPP quad
// permutations), each swapping 2x2 sub-blocks.  Used to turn the MFMA D layout (a lane
// holds four rows of one column) into four consecutive columns of one row, for 16-byte
// global loads and stores.
__device__ __forceinline__ void quad_transpose4(float (&x)[4]) {
    const int j = __lane_id() & 3;
    const bool odd = j & 1, hi = j & 2;
    constexpr int kXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);   // quad_perm [1, 0, 3, 2]
    constexpr int kXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);   // quad_perm [2, 3, 0, 1]
    const float t0 = quad_perm<kXor1>(x[0]), t1 = quad_perm<kXor1>(x[1]);
    const float t2 = quad_perm<kXor1>(x[2]), t3 = quad_perm<kXor1>(x[3]);
    const float y0 = odd ? t1 : x[0], y1 = odd ? x[1] : t0, y2 = odd ? t3 : x[2], y3 = odd ? x[3] : t2;
    const float u0 = quad_perm<kXor2>(y0), u1 = quad_perm<kXor2>(y1);
    const float u2 = quad_perm<kXor2>(y2), u3 = quad_perm<kXor2>(y3);
    x[0] = hi ? u2 : y0;
    x[1] = hi ? u3 : y1;
    x[2] = hi ? y2 : u0;
    x[3] = hi ? y3 : u1;
}

}  // namespace gdn2
