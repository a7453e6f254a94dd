// gdn2_chunk.h -- per-chunk building blocks shared by the forward and backward kernels.
//
// A workgroup has 4 waves; wave w owns tokens 16w..16w+15 of a 64-token chunk
// (token = 16w + r, r = lane % 16).  Key-side element work keeps, per lane,
// NE = DK/4 channels of its token.
#pragma once

#ifndef GDN2_SPLIT_PAIRS
#define GDN2_SPLIT_PAIRS 0
#endif
#include "gdn2_device.h"

namespace gdn2 {

// Inclusive cumulative sum of log2-decay over the chunk's tokens, per key
// channel, in fp32 (blog on Gated DeltaNet-2, section "Token path and parallel
// training": the cumulative channel decay is formed in fp32).
// x[e]: this lane's log2-decay values (already multiplied by log2(e));
// on return x[e] = G (inclusive prefix over the chunk), tot[e] = chunk total.
// ch(e) maps element index -> channel.  sTot: 4*DK floats of LDS.
// Contains one workgroup barrier.
template <int NE, int DK, typename ChanFn>
__device__ __forceinline__ void chunk_scan(float (&x)[NE], float (&tot)[NE], float *sTot, int w, int r,
                                           ChanFn ch) {
#pragma unroll
    for (int e = 0; e < NE; ++e) x[e] = row_scan16(x[e]);
    if (r == 15) {
#pragma unroll
        for (int e = 0; e < NE; ++e) sTot[w * DK + ch(e)] = x[e];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int c = ch(e);
        const float t0 = sTot[c], t1 = sTot[DK + c], t2 = sTot[2 * DK + c], t3 = sTot[3 * DK + c];
        const float pre = (w > 0 ? t0 : 0.f) + (w > 1 ? t1 : 0.f) + (w > 2 ? t2 : 0.f);
        x[e] += pre;
        tot[e] = (t0 + t1) + (t2 + t3);
    }
}

// The offsets chunk_scan adds to the in-wave prefixes, from the per-block totals it leaves in
// sTot (the same sums in the same order): pre = sum of the totals of the token blocks before w.
// Thread t < 4 DK writes the offset of block t / DK, channel t % DK, to pre[t].  Call after a
// chunk_scan, before sTot is overwritten.
template <int DK, int NTH>
__device__ __forceinline__ void chunk_scan_offsets(const float *sTot, float *pre, int tid) {
#pragma unroll
    for (int t = tid; t < 4 * DK; t += NTH) {
        const int w = t / DK, c = t % DK;
        const float t0 = sTot[c], t1 = sTot[DK + c], t2 = sTot[2 * DK + c];
        pre[t] = (w > 0 ? t0 : 0.f) + (w > 1 ? t1 : 0.f) + (w > 2 ? t2 : 0.f);
    }
}

// chunk_scan's result without its barrier, given its offsets: x[e] (log2-decay of this lane's
// elements) becomes the inclusive prefix G; pre4[m] holds the offsets of channels ch(4m) ..
// ch(4m + 3) of this lane's token block.
template <int NE>
__device__ __forceinline__ void scan_with_offsets(float (&x)[NE], const f32x4 (&pre4)[NE / 4]) {
#pragma unroll
    for (int e = 0; e < NE; ++e) x[e] = row_scan16(x[e]) + pre4[e / 4][e % 4];
}

// Two chunk_scan's at once (x with totals through sTotX, y through sTotY): one barrier.
template <int NE, int DK, typename ChanFn>
__device__ __forceinline__ void chunk_scan2(float (&x)[NE], float (&xt)[NE], float *sTotX, float (&y)[NE],
                                            float (&yt)[NE], float *sTotY, int w, int r, ChanFn ch) {
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        x[e] = row_scan16(x[e]);
        y[e] = row_scan16(y[e]);
    }
    if (r == 15) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            sTotX[w * DK + ch(e)] = x[e];
            sTotY[w * DK + ch(e)] = y[e];
        }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int c = ch(e);
        const float a0 = sTotX[c], a1 = sTotX[DK + c], a2 = sTotX[2 * DK + c], a3 = sTotX[3 * DK + c];
        const float b0 = sTotY[c], b1 = sTotY[DK + c], b2 = sTotY[2 * DK + c], b3 = sTotY[3 * DK + c];
        x[e] += (w > 0 ? a0 : 0.f) + (w > 1 ? a1 : 0.f) + (w > 2 ? a2 : 0.f);
        y[e] += (w > 0 ? b0 : 0.f) + (w > 1 ? b1 : 0.f) + (w > 2 ? b2 : 0.f);
        xt[e] = (a0 + a1) + (a2 + a3);
        yt[e] = (b0 + b1) + (b2 + b3);
    }
}

// Inverse of one unit-lower 16x16 block, (I + N)^-1 with N strictly lower, so
// N^16 = 0 and (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) exactly.  The
// powers are formed on MFMA in both the row layout (lane holds X[r][4g+i]) and
// the column layout (lane holds X[4g+i][r]): the product of two column-layout
// operands' transposes lands in row layout, so no data leaves the registers.
// nA / nB: N in row / column layout.  Returns (I + N)^-1 in column layout.
__device__ __forceinline__ f32x4 unit_lower_inverse16(const f32x4 &nA, const f32x4 &nB, int r, int g) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 eye;
#pragma unroll
    for (int i = 0; i < 4; ++i) eye[i] = (4 * g + i == r) ? 1.f : 0.f;   // same in both layouts
    const Split4 NA = split4(nA), NB = split4(nB);
    const f32x4 n2B = mfma16x3(NA, NB, zero);        // N^2, column layout
    const f32x4 n2A = mfma16x3(NB, NA, zero);        // (N^T N^T) = (N^2)^T, column layout = N^2 row layout
    const Split4 N2A = split4(n2A), N2B = split4(n2B);
    const f32x4 n4B = mfma16x3(N2A, N2B, zero);
    const f32x4 n4A = mfma16x3(N2B, N2A, zero);
    const Split4 N4A = split4(n4A);
    const f32x4 n8B = mfma16x3(N4A, split4(n4B), zero);
    f32x4 y = n8B + eye;                             // (I + N^8), column layout
    y = mfma16x3(split4(n4A + eye), split4(y), zero);
    y = mfma16x3(split4(n2A + eye), split4(y), zero);
    y = mfma16x3(split4(eye - nA), split4(y), zero);
    return y;
}

// T = (I + A)^-1 for the strictly lower 64x64 A of a chunk (triangular solve
// of the WY form).  sA: A in fp32 [64][PA] (only the strictly lower 16x16
// blocks on or below the diagonal are read); sT: fp32 [64][PA], whose strictly
// upper 16x16 blocks must already be zero.  On return sT holds T.
// Diagonal blocks: unit_lower_inverse16 (wave w inverts block w); off-diagonal
// blocks by block distance: T_IJ = -T_II * sum_{K=J}^{I-1} A_IK T_KJ.  All
// products run on MFMA with split-bf16 operands (about 16 significant bits,
// fp32 accumulation).  Contains 4 workgroup barriers; sA is not written.
template <int PA>
__device__ __forceinline__ void solve_T(const float *sA, float *sT, int w, int r, int g) {
    {
        f32x4 nA = *reinterpret_cast<const f32x4 *>(&sA[(16 * w + r) * PA + 16 * w + 4 * g]);
        f32x4 nB;
#pragma unroll
        for (int i = 0; i < 4; ++i) nB[i] = sA[(16 * w + 4 * g + i) * PA + 16 * w + r];
        // only the strictly lower part of the diagonal block is A
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!(4 * g + i < r)) nA[i] = 0.f;
            if (!(r < 4 * g + i)) nB[i] = 0.f;
        }
        const f32x4 tB = unit_lower_inverse16(nA, nB, r, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[(16 * w + 4 * g + i) * PA + 16 * w + r] = tB[i];
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        if (w >= d) {
            const int I = w, J = w - d;
            f32x4 Y = {0.f, 0.f, 0.f, 0.f};
            for (int K = J; K < I; ++K) {
                const f32x4 av = *reinterpret_cast<const f32x4 *>(&sA[(16 * I + r) * PA + 16 * K + 4 * g]);
                f32x4 tv;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) tv[ii] = sT[(16 * K + 4 * g + ii) * PA + 16 * J + r];
                Y = mfma16x3(split4(av), split4(tv), Y);
            }
            const f32x4 tiv = *reinterpret_cast<const f32x4 *>(&sT[(16 * I + r) * PA + 16 * I + 4 * g]);
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const f32x4 R = mfma16x3(split4(tiv), split4(-Y), zero);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sT[(16 * I + 4 * g + ii) * PA + 16 * J + r] = R[ii];
        }
        __syncthreads();
    }
}

// Same as solve_T, with A and T sharing one fp32 [64][PA] buffer: each wave
// first keeps its own row blocks of A in registers (only wave I ever reads
// row block I of A), then T is written over A.  The strictly upper 16x16
// blocks of the buffer must be zero and stay zero.  4 workgroup barriers,
// which every wave of the workgroup reaches; only waves with `active` set
// (one per row block w) compute.  The others call side(k) before barrier k
// (k = 0 .. 3): work of their own that touches neither A nor T.
struct NoSide {
    __device__ void operator()(int) const {}
};
template <int PA, class Side = NoSide>
__device__ __forceinline__ void solve_T_inplace(float *sAT, int w, int r, int g, bool active = true,
                                                const Side &side = Side()) {
    f32x4 arow[3];
#pragma unroll
    for (int K = 0; K < 3; ++K)
        if (active && K < w) arow[K] = *reinterpret_cast<const f32x4 *>(&sAT[(16 * w + r) * PA + 16 * K + 4 * g]);
    if (active) {
        f32x4 nA = *reinterpret_cast<const f32x4 *>(&sAT[(16 * w + r) * PA + 16 * w + 4 * g]);
        f32x4 nB;
#pragma unroll
        for (int i = 0; i < 4; ++i) nB[i] = sAT[(16 * w + 4 * g + i) * PA + 16 * w + r];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!(4 * g + i < r)) nA[i] = 0.f;
            if (!(r < 4 * g + i)) nB[i] = 0.f;
        }
        const f32x4 tB = unit_lower_inverse16(nA, nB, r, g);
#pragma unroll
        for (int i = 0; i < 4; ++i) sAT[(16 * w + 4 * g + i) * PA + 16 * w + r] = tB[i];
    } else {
        side(0);
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < 4; ++d) {
        if (!active) side(d);
        if (active && w >= d) {
            const int I = w, J = w - d;
            f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int K = 0; K < 3; ++K) {
                if (K >= J && K < I) {
                    f32x4 tv;
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) tv[ii] = sAT[(16 * K + 4 * g + ii) * PA + 16 * J + r];
                    Y = mfma16x3(split4(arow[K]), split4(tv), Y);
                }
            }
            const f32x4 tiv = *reinterpret_cast<const f32x4 *>(&sAT[(16 * I + r) * PA + 16 * I + 4 * g]);
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const f32x4 R = mfma16x3(split4(tiv), split4(-Y), zero);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sAT[(16 * I + 4 * g + ii) * PA + 16 * J + r] = R[ii];
        }
        __syncthreads();
    }
}

// A-operand fragment of X^T for the 16x16x32 MFMA, read transposed from a
// row-major [row][col] bf16 tile (hi and lo planes): lane (r, g) receives
// column c0 + r of rows k0 + 4g + {0..3} (slots 0..3) and k0 + 16 + 4g + {0..3}
// (slots 4..7), the "4-group" contraction order.
template <int P>
__device__ __forceinline__ Split8 frag_tr(const __bf16 *hi, const __bf16 *lo, int k0, int c0, int r, int g) {
    const int o0 = (k0 + 4 * g + (r >> 2)) * P + c0 + 4 * (r & 3);
    const int o1 = o0 + 16 * P;
    Split8 f;
    const bf16x4 a = lds_read_tr(hi + o0), b = lds_read_tr(hi + o1);
    const bf16x4 c = lds_read_tr(lo + o0), d = lds_read_tr(lo + o1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.hi[i] = a[i];
        f.hi[4 + i] = b[i];
        f.lo[i] = c[i];
        f.lo[4 + i] = d[i];
    }
    return f;
}

// Split-bf16 MFMA fragment with the "4-group" contraction order: slots 0..3 are
// taken from p0[0..3] and slots 4..7 from p1[0..3].  SPLIT: the four 8-byte reads are kept apart.
// Left to itself the compiler pairs them into ds_read2_b64, and the pieces of a pair then share
// banks with another lane's (the hi pieces 32 bytes apart: lane r's second with lane r + 2's
// first, at every row pitch); four ds_read_b64 are each conflict-free at rows of 8 mod 16 bf16.
// Offsets the compiler cannot see through keep them apart.
template <int SPLIT = GDN2_SPLIT_PAIRS>
__device__ __forceinline__ Split8 frag_2x4(const __bf16 *hi0, const __bf16 *hi1, const __bf16 *lo0,
                                           const __bf16 *lo1) {
    if constexpr (SPLIT != 0) {
        int z0 = 0, z1 = 0, z2 = 0;
        asm volatile("" : "+s"(z0), "+s"(z1), "+s"(z2));
        hi1 += z0;
        lo0 += z1;
        lo1 += z2;
    }
    Split8 f;
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(hi0);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(hi1);
    const bf16x4 c = *reinterpret_cast<const bf16x4 *>(lo0);
    const bf16x4 d = *reinterpret_cast<const bf16x4 *>(lo1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.hi[i] = a[i];
        f.hi[4 + i] = b[i];
        f.lo[i] = c[i];
        f.lo[4 + i] = d[i];
    }
    return f;
}

__device__ __forceinline__ Split8 frag_8(const __bf16 *hi, const __bf16 *lo) {
    Split8 f;
    f.hi = *reinterpret_cast<const bf16x8 *>(hi);
    f.lo = *reinterpret_cast<const bf16x8 *>(lo);
    return f;
}

__device__ __forceinline__ Split8 join(const Split4 &a, const Split4 &b) {
    Split8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.hi[i] = a.hi[i];
        f.hi[4 + i] = b.hi[i];
        f.lo[i] = a.lo[i];
        f.lo[4 + i] = b.lo[i];
    }
    return f;
}

// 8 fp32 values -> split fragment
__device__ __forceinline__ Split8 split8v(const f32x4 &a, const f32x4 &b) {
    const float t[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return split8(t);
}


// ---------------------------------------------------------------------------
// Key-side element layout of the backward kernels ("4-groups"): lane (w, r, g)
// holds token 16w + r and channels 16m + 4g + i (i < 4); element e = 4m + i.  The
// MFMA fragment of contraction step j is elements 8j..8j+7, i.e. channels
// 32j + 4g + {0..3} and 32j + 16 + 4g + {0..3}.  It equals the D layout of a
// product whose rows are channels, so key-side gradients come out of transposed
// products already in element layout.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int ch4(int e, int g) { return 16 * (e >> 2) + 4 * g + (e & 3); }

// key-side inputs of one token for the 4-group layout; GL: log_alpha and b are bf16 logits;
// SG: log_alpha and/or b may be given per token (broadcast over the channels)
template <int DK, bool BF16, bool GL = false, bool SG = false>
struct KeyRaw4 {
    static constexpr int NM = DK / 16;
    // native vector types: HIP's vector structs keep arrays of them that live across loops in
    // scratch memory
    u32x2 q[NM], k[NM];
    f32x4 qx[NM], kx[NM];
    f32x4 la[NM], bg[NM];           // fp32 gate values
    u32x2 la16[NM], bg16[NM];       // bf16 gate logits
    bool valid;

    // q, k: qkv dtype; rowoff: element offset of channel 0 of the token row; srow: the
    // token's offset in per-token gate tensors; scalar: kScalar* bits (SG only)
    __device__ __forceinline__ void issue(const void *qp, const void *kp, const void *lap, const void *bgp,
                                          size_t rowoff, int g, bool v, size_t srow = 0, int scalar = 0) {
        valid = v;
        float sla = 0.f, sbg = 0.f;
        if (SG) {
            sla = reinterpret_cast<const float *>(lap)[(scalar & 1) ? srow : rowoff];
            sbg = reinterpret_cast<const float *>(bgp)[(scalar & 2) ? srow : rowoff];
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const size_t off = rowoff + 16 * m + 4 * g;
            if (BF16) {
                q[m] = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(qp) + off);
                k[m] = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(kp) + off);
            } else {
                qx[m] = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(qp) + off);
                kx[m] = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(kp) + off);
            }
            if (GL) {
                la16[m] = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(lap) + off);
                bg16[m] = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(bgp) + off);
            } else if (SG) {
                la[m] = (scalar & 1) ? f32x4{sla, sla, sla, sla}
                                     : *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(lap) + off);
                bg[m] = (scalar & 2) ? f32x4{sbg, sbg, sbg, sbg}
                                     : *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(bgp) + off);
            } else {
                la[m] = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(lap) + off);
                bg[m] = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(bgp) + off);
            }
        }
    }

    static __device__ __forceinline__ void bf16x4_to(const u32x2 &u, float *o) {
        o[0] = __builtin_bit_cast(float, u[0] << 16);
        o[1] = __builtin_bit_cast(float, u[0] & 0xffff0000u);
        o[2] = __builtin_bit_cast(float, u[1] << 16);
        o[3] = __builtin_bit_cast(float, u[1] & 0xffff0000u);
    }

    // q and k only (zero for a missing token)
    __device__ __forceinline__ void unpack_qk(float (&qf)[4 * NM], float (&kf)[4 * NM]) const {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (BF16) {
                bf16x4_to(q[m], &qf[4 * m]);
                bf16x4_to(k[m], &kf[4 * m]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qf[4 * m + i] = qx[m][i];
                    kf[4 * m + i] = kx[m][i];
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 4 * NM; ++e) {
            qf[e] = valid ? qf[e] : 0.f;
            kf[e] = valid ? kf[e] : 0.f;
        }
    }

    // q, k, log_alpha and b (activated when the gates are logits); zero for a missing token
    __device__ __forceinline__ void unpack(float (&qf)[4 * NM], float (&kf)[4 * NM], float (&laf)[4 * NM],
                                           float (&bgf)[4 * NM]) const {
        unpack_qk(qf, kf);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (GL) {
                float x[4], y[4];
                bf16x4_to(la16[m], x);
                bf16x4_to(bg16[m], y);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    laf[4 * m + i] = decay_act<GL>(x[i]);
                    bgf[4 * m + i] = gate_act<GL>(y[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    laf[4 * m + i] = la[m][i];
                    bgf[4 * m + i] = bg[m][i];
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 4 * NM; ++e) {
            laf[e] = valid ? floor_log_decay(laf[e]) : 0.f;
            bgf[e] = valid ? bgf[e] : 0.f;
        }
    }

    // d log_alpha / d stored decay input (1 for fp32 values)
    __device__ __forceinline__ void decay_dact_all(float (&d)[4 * NM]) const {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (GL) {
                float x[4];
                bf16x4_to(la16[m], x);
#pragma unroll
                for (int i = 0; i < 4; ++i) d[4 * m + i] = decay_dact<GL>(x[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) d[4 * m + i] = 1.f;
            }
        }
    }
};

// Key-side fragment (4-group contraction order) of row `row` of a [row][channel] tile.
template <int PK, int SPLIT = GDN2_SPLIT_PAIRS>
__device__ __forceinline__ Split8 row_frag4(const __bf16 *hi, const __bf16 *lo, int row, int j, int g) {
    return frag_2x4<SPLIT>(&hi[row * PK + 32 * j + 4 * g], &hi[row * PK + 32 * j + 16 + 4 * g],
                           &lo[row * PK + 32 * j + 4 * g], &lo[row * PK + 32 * j + 16 + 4 * g]);
}

// A = strictly-lower(Et Kt^T) and P = lower(Qt Kt^T) of one chunk, from [token][channel] split-bf16
// rows in LDS (Kt, Et, Qt: hi plane, lo plane RK elements later, pitch PK).  The ten pairs (query
// block qb, key block kb <= qb) come from a queue that every wave of the workgroup draws from
// (*cnt: zero beforehand, and a barrier between); a pair's A and P tiles share the Kt fragment and
// run as two interleaved MFMA chains.  A goes to sAT [64][PA] fp32 (tiles above the diagonal
// blocks are left as they are); P goes to sPf as split-bf16 fragment tiles (tile 4 qb + kb, 16
// bytes per lane: four hi then four lo values of P[16qb + r][16kb + 4g + i]).  No global access.
template <int DK, int PK, int PA>
__device__ __forceinline__ void ap_pair_queue(const __bf16 *sKt, const __bf16 *sEt, const __bf16 *sQt, float *sAT,
                                              char *sPf, int *cnt, int l, int r, int g) {
    constexpr int NKS = DK / 32, RK = kChunk * PK;
    auto grab = [&]() {
        int p = 0;
        if (l == 0) p = atomicAdd(cnt, 1);
        return __builtin_amdgcn_readfirstlane(p);
    };
    for (int p = grab(); p < 10; p = grab()) {
        const int qb = p < 1 ? 0 : (p < 3 ? 1 : (p < 6 ? 2 : 3)), kb = p - qb * (qb + 1) / 2;
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
            const Split8 kf = row_frag4<PK>(sKt, sKt + RK, 16 * kb + r, j, g);
            accA = mfma32x3(kf, row_frag4<PK>(sEt, sEt + RK, 16 * qb + r, j, g), accA);
            accP = mfma32x3(kf, row_frag4<PK>(sQt, sQt + RK, 16 * qb + r, j, g), accP);
        }
        // lane holds A[16qb + r][16kb + 4g + i] (strictly lower) and P[16qb + r][16kb + 4g + i]
        // (key <= query: the query reads the updated state)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!(16 * kb + 4 * g + i < 16 * qb + r)) accA[i] = 0.f;
            if (!(16 * kb + 4 * g + i <= 16 * qb + r)) accP[i] = 0.f;
        }
        *reinterpret_cast<f32x4 *>(&sAT[(16 * qb + r) * PA + 16 * kb + 4 * g]) = accA;
        const Split4 pf = split4(accP);
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[i] = pf.hi[i];
            o[4 + i] = pf.lo[i];
        }
        *reinterpret_cast<bf16x8 *>(sPf + (size_t)((4 * qb + kb) * 64 + l) * 16) = o;
    }
}

// ---- adjoint factor tiles (R and Q2^T of a chunk, MFMA fragment order) ----
constexpr int kFragTile = 64 * 8;   // bf16 per stored 16x16 factor tile

template <int DK>
constexpr size_t factor_elems_per_chunk() {
    return (size_t)((DK / 16) * (DK / 16) + (DK / 16) * 4) * kFragTile;
}

// ---- chunk operand record ----
// The key-side operands of one (batch, head, chunk), formed once by the adjoint-factor
// kernel and read by the forward sweep and the chunk-gradient kernel:
//   Kh, Et, Qt rows    [token][channel] split bf16, hi plane then lo plane, pitch DK
//                      (Kh = k exp(g_C - G), Et = b k exp(G), Qt = q exp(G): factors <= 1)
//   T = (I + A)^-1     [row][col] split bf16, hi then lo, pitch 64
//   P^T fragments      tile (key block w, query block mt) at (4w + mt) * 64 lanes * 8 bf16:
//                      lane (r, g) holds P[16mt + 4g + i][16w + r], hi (i < 4) then lo
//                      (tiles with mt < w are zero and written as such)
//   P fragments        tile (query block w, key block mt) at (4w + mt) * 64 lanes * 8 bf16:
//                      lane (r, g) holds P[16w + r][16mt + 4g + i], hi then lo (zero for mt > w)
//   Every tile is written, so readers load all four of a block row unconditionally (a
//   load under a branch would make the compiler wait for all loads in flight).
//   PRE                [4][DK] fp32: per token block w and key channel, the log2 decay of the
//                      chunk's tokens before the block (the cross-wave part of chunk_scan), so
//                      that a reader forms the decay prefix G from log alpha with one in-wave
//                      scan (scan_with_offsets) and no barrier
//   gamma              [DK] fp32, the chunk's total decay per key channel
template <int DK>
struct ChunkRecord {
    static constexpr int PLANE = kChunk * DK * 2;               // bytes of one [token][channel] bf16 plane
    static constexpr int ROWS = 2 * PLANE;                      // an operand's hi and lo planes
    static constexpr int oKh = 0, oEt = oKh + ROWS, oQt = oEt + ROWS;
    static constexpr int oT = oQt + ROWS, B_T = kChunk * kChunk * 2 * 2;
    static constexpr int B_FR = 16 * 64 * 8 * 2;                // 16 fragment tiles of 64 lanes x 8 bf16
    static constexpr int oPt = oT + B_T, oP = oPt + B_FR;
    static constexpr int oPre = oP + B_FR, B_PRE = 4 * DK * 4;
    static constexpr int oGam = oPre + B_PRE;
    static constexpr int BYTES = (oGam + DK * 4 + 255) / 256 * 256;
};

// A buffer of `items` records is followed by one int per record: 1 if the chunk's decay is
// too strong for the factorised operands (some gamma below kGamMin), else 0.
template <int DK>
__host__ __device__ constexpr size_t record_flags_offset(long items) {
    return (size_t)items * ChunkRecord<DK>::BYTES;
}
__host__ __device__ constexpr size_t record_flags_bytes(long items) { return ((size_t)items * 4 + 255) / 256 * 256; }

// Work list of an exact pass: the flagged items among base, base + stride, ...,
// base + (NTH - 1) stride (one candidate per thread), gathered into sList (NTH ints of LDS);
// returns their number (uniform over the workgroup).  *sCount: one int of LDS.  Two barriers.
template <int NTH>
__device__ __forceinline__ int gather_flagged(const int *flags, long nitems, long base, int stride, int *sList,
                                              int *sCount) {
    if (threadIdx.x == 0) *sCount = 0;
    __syncthreads();
    const long L = base + (long)threadIdx.x * stride;
    if (L < nitems && flags[L] != 0) sList[atomicAdd(sCount, 1)] = (int)L;
    __syncthreads();
    return *sCount;
}

}  // namespace gdn2
