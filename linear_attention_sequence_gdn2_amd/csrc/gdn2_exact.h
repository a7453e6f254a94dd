// gdn2_exact.h -- the exact intra-chunk decay products for chunks with strong decay.
//
// In the chunk form (blog on Gated DeltaNet-2, section "Token path and parallel training":
// cumulative channel decay absorbed into asymmetric erase factors) the intra-chunk products
// carry, per key channel c and token pair j <= i, the decay between the two tokens,
//     exp(G_ic - G_jc) = prod_{t = j+1 .. i} alpha_tc  <= 1,
// with G the inclusive cumulative log-decay of the chunk.  The fast kernels factor it as
// exp(G_i) * exp(-G_j), one factor per operand row, which leaves fp32 range once a channel's
// decay over the chunk passes about exp(-64) (kGamMin).  For such chunks this header forms the
// products with the pairwise factor itself, in fp32:
//     A_ij = sum_c e_ic k_jc x_ijc (j < i),        P_ij = sum_c q_ic k_jc x_ijc (j <= i),
// and, backward, the matching sums over token pairs of dA and dP (gdn2_bwd.hip).
// Everything here works on "channel slices": 16 key channels of each half of the workgroup's
// key-side element layout (gdn2_chunk.h, "4-groups"), staged in LDS as fp32 [channel][token].
// Decays are in log2 units, as in the kernels (G multiplied by log2(e)).
#pragma once

#include "gdn2_chunk.h"

namespace gdn2 {

constexpr int kSlicePitch = kChunk + 4;                     // floats per channel row of a slice array
constexpr int kSliceArrays = 4;                             // e = b k, q, k, G
constexpr int kSliceFloats = 2 * kSliceArrays * 16 * kSlicePitch;

// array a (0: e, 1: q, 2: k, 3: G) of half hf, channel cc (0..15 within the slice), token t
__device__ __forceinline__ int slice_idx(int hf, int a, int cc, int t) {
    return ((hf * kSliceArrays + a) * 16 + cc) * kSlicePitch + t;
}

// Lane (hf, w, r, g) of the 512-thread workgroup holds token 16w + r and, for slice mm, the
// channels 16 mm + 4g + i (i < 4) of half hf: elements e = 4mm + i of its key-side arrays.
template <int NEH>
__device__ __forceinline__ void slice_put(float *sl, int mm, int hf, int w, int r, int g, const float (&ev)[NEH],
                                          const float (&qv)[NEH], const float (&kv)[NEH], const float (&Gv)[NEH]) {
    const int t = 16 * w + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = 4 * mm + i, cc = 4 * g + i;
        sl[slice_idx(hf, 0, cc, t)] = ev[e];
        sl[slice_idx(hf, 1, cc, t)] = qv[e];
        sl[slice_idx(hf, 2, cc, t)] = kv[e];
        sl[slice_idx(hf, 3, cc, t)] = Gv[e];
    }
}

// A (strictly lower) and P (lower, diagonal included) of one chunk with the exact pairwise
// decay.  Every thread of the 512 takes row i = tid / 8 and columns 8 (tid % 8) .. + 7, and
// accumulates over all channels, one slice of both halves at a time.  On return sA[i][j]
// (pitch PA) holds A and sP[i][j] holds P, with zeros above the diagonal; sP may overlay the
// slice scratch sl.  ev, qv, kv, Gv: this lane's key-side elements (e = b k, q, k and the
// log2 decay prefix G); tokens past the end of the sequence hold zeros.  Barriers: 2 per slice
// and one before sA / sP are written, reached by every thread.
template <int NEH, int PA>
__device__ __forceinline__ void exact_AP(float *sl, float *sA, float *sP, int hf, int w, int r, int g,
                                         const float (&ev)[NEH], const float (&qv)[NEH], const float (&kv)[NEH],
                                         const float (&Gv)[NEH]) {
    const int tid = threadIdx.x, i = tid >> 3, c8 = 8 * (tid & 7);
    float A[8], P[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) A[jj] = P[jj] = 0.f;
#pragma unroll
    for (int mm = 0; mm < NEH / 4; ++mm) {
        __syncthreads();   // the previous slice has been read
        slice_put<NEH>(sl, mm, hf, w, r, g, ev, qv, kv, Gv);
        __syncthreads();
        if (c8 <= i) {
            for (int h2 = 0; h2 < 2; ++h2) {
                for (int cc = 0; cc < 16; ++cc) {
                    const float ei = sl[slice_idx(h2, 0, cc, i)], qi = sl[slice_idx(h2, 1, cc, i)];
                    const float gi = sl[slice_idx(h2, 3, cc, i)];
                    const float4 k0 = *reinterpret_cast<const float4 *>(&sl[slice_idx(h2, 2, cc, c8)]);
                    const float4 k1 = *reinterpret_cast<const float4 *>(&sl[slice_idx(h2, 2, cc, c8 + 4)]);
                    const float4 g0 = *reinterpret_cast<const float4 *>(&sl[slice_idx(h2, 3, cc, c8)]);
                    const float4 g1 = *reinterpret_cast<const float4 *>(&sl[slice_idx(h2, 3, cc, c8 + 4)]);
                    const float kj[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
                    const float gj[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        // for j > i the factor may be inf; those entries are replaced by zeros below
                        const float kx = kj[jj] * exp2_fast(gi - gj[jj]);
                        A[jj] = fmaf(ei, kx, A[jj]);
                        P[jj] = fmaf(qi, kx, P[jj]);
                    }
                }
            }
        }
    }
    __syncthreads();   // every slice has been read: sP may overwrite the scratch
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        const int j = c8 + jj;
        sA[i * PA + j] = j < i ? A[jj] : 0.f;
        sP[i * PA + j] = j <= i ? P[jj] : 0.f;
    }
}

}  // namespace gdn2
