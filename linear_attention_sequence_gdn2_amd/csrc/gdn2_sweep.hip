// gdn2_sweep.hip -- forward sweep of the Gated DeltaNet-2 rule from the chunk operand
// records on gfx950.
//
// Chunk form (blog on Gated DeltaNet-2, section "Token path and parallel training":
// cumulative channel decay absorbed into asymmetric erase factors, a triangular solve
// and dense products).  For a chunk with start state S:
//     X = Z - Et S,   U = T X,   O = Qt S + P U,   S' = diag(gamma) (S + Kt^T U),
// with Z = w * v and Et, Kt, Qt, T = (I + A)^-1, P, gamma depending on the key side of
// the chunk only.  The adjoint-factor kernel forms those for every chunk at once and
// keeps them in the chunk operand records; what is left for this sequential sweep are
// the products with the state, which cannot run ahead of the previous chunk.
//
// Work decomposition as in the fused forward (gdn2_fwd.hip): one workgroup of 4 waves
// per (batch, head, value tile of VT columns), wave w owning tokens 16w..16w+15 for the
// rows of X, U and O and NTS tiles of the state; the fp32 state stays in registers (D
// layout) with a split-bf16 copy in LDS as the next chunk's operand.  Per chunk the
// wave loads its A operands (rows of Et, Qt, T and P) straight from the record into
// registers, and the workgroup stages the Kt rows in LDS for the transposed reads of
// the state update.  At VT = 32 a workgroup needs about 71 KB of LDS, so two share a CU.
// Four barriers per chunk: Kt rows and the state copy written; X written; U written;
// every wave done with the chunk's LDS.
#include "gdn2_chunk.h"
#include "gdn2_kernels.h"

namespace gdn2 {

#define GDN2_SWEEP_FENCE() __builtin_amdgcn_sched_barrier(0)

template <int DK, int VT, bool BF16, bool OUT, bool STATES, bool GL, bool SG>
__global__ __launch_bounds__(kThreads, 2) void fwd_sweep_kernel(FwdArgs a) {
    using Rec = ChunkRecord<DK>;
    constexpr int NKS = DK / 32;           // 32-channel contraction steps
    constexpr int NVT = VT / 16;           // 16-column value tiles
    constexpr int NMT = DK / 16;           // 16-row key tiles of S
    constexpr int NTS = NMT * NVT / 4;     // S tiles per wave
    static_assert((NMT * NVT) % 4 == 0, "S tiles must split over 4 waves");
    constexpr bool FAST = BF16;            // X = Z - Et S with the hi part of Et only
    constexpr int PK = DK + 8;             // row pitch of [row][channel] bf16 tiles
    constexpr int PT = kChunk + 8;         // row pitch of [col][token] bf16 tiles
    constexpr int RK = kChunk * PK;        // one [token][channel] plane
    constexpr int NKT = 2 * kChunk * DK / 8 / kThreads;   // 16-byte pieces per thread of the Kt planes
    static_assert(NKT * kThreads * 8 == 2 * kChunk * DK, "Kt planes split evenly over the threads");

    __shared__ __align__(16) __bf16 sK[2 * RK];         // Kt rows [token][channel] (hi, lo)
    __shared__ __align__(16) __bf16 sS[2 * VT * PK];    // S^T [col][channel] (hi, lo)
    __shared__ __align__(16) __bf16 sX[2 * VT * PT];    // X^T [col][token] (hi, lo)
    __shared__ __align__(16) __bf16 sU[2 * VT * PT];    // U^T [col][token] (hi, lo)

    const int tid = threadIdx.x, w = tid >> 6, r = tid & 15, g = (tid >> 4) & 3;
    const int L = xcd_swizzle(blockIdx.x, gridDim.x);
    const int vt = L % a.nvt, bh = L / a.nvt, h = bh % a.H, b = bh / a.H;
    const int T = a.T, H = a.H, DV = a.dv;
    const int j0 = vt * VT;
    const size_t tokV = (size_t)H * DV;
    const size_t baseK = ((size_t)b * T * H + h) * DK;
    const size_t baseV = ((size_t)b * T * H + h) * DV + j0;
    const size_t sbase = ((size_t)b * H + h) * (size_t)DK * DV + j0;
    const int NC = (T + kChunk - 1) / kChunk;
    // records of this (batch, head), after the adjoint factors of all chunks
    const char *recs = reinterpret_cast<const char *>(a.factors) +
                       (size_t)a.B * H * NC * factor_elems_per_chunk<DK>() * 2 + (size_t)bh * NC * Rec::BYTES;

    f32x4 S[NTS];
#pragma unroll
    for (int s = 0; s < NTS; ++s) {
        const int id = w * NTS + s, m = id / NVT, n = id % NVT;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[s][i] = a.S0 ? a.S0[sbase + (size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] : 0.f;
    }
    auto store_state_lds = [&](int w, int r, int g) {
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT, n = id % NVT;
            const Split4 sp = split4(S[s]);
            *reinterpret_cast<bf16x4 *>(&sS[(16 * n + r) * PK + 16 * m + 4 * g]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&sS[VT * PK + (16 * n + r) * PK + 16 * m + 4 * g]) = sp.lo;
        }
    };
    store_state_lds(w, r, g);

    for (int c = 0; c < NC; ++c) {
        // lane indices afresh from an opaque copy of the thread index each chunk
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
        const int nkk = (w >= 2) ? 2 : 1;
        const int t0 = c * kChunk;
        const char *rec = recs + (size_t)c * Rec::BYTES;
        if (STATES) {
            float *dst = a.states + (((size_t)b * H + h) * NC + c) * (size_t)DK * DV + j0;
#pragma unroll
            for (int s = 0; s < NTS; ++s) {
                const int id = w * NTS + s, m = id / NVT, n = id % NVT;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] = S[s][i];
            }
        }

        // ---- loads: Kt rows (for LDS), this wave's A operands, gamma, z = w * v ----
        uint4 kraw[NKT];
#pragma unroll
        for (int it = 0; it < NKT; ++it)
            kraw[it] = *reinterpret_cast<const uint4 *>(rec + Rec::oKt + (size_t)(tid + kThreads * it) * 16);
        // Et, Qt rows 16w + r, channels 32j + 8g .. + 7 (the contraction order of the S reads)
        Split8 Et[NKS], Qt[NKS];
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
            const size_t o = (size_t)((16 * w + r) * DK + 32 * j + 8 * g) * 2;
            Et[j].hi = *reinterpret_cast<const bf16x8 *>(rec + Rec::oEt + o);
            if (!FAST) Et[j].lo = *reinterpret_cast<const bf16x8 *>(rec + Rec::oEt + Rec::PLANE + o);
            if (OUT) {
                Qt[j].hi = *reinterpret_cast<const bf16x8 *>(rec + Rec::oQt + o);
                Qt[j].lo = *reinterpret_cast<const bf16x8 *>(rec + Rec::oQt + Rec::PLANE + o);
            }
        }
        // T row 16w + r, columns 32kk + 8g .. + 7
        Split8 Tf[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const size_t o = (size_t)((16 * w + r) * kChunk + (kk < nkk ? 32 * kk : 0) + 8 * g) * 2;
            Tf[kk].hi = *reinterpret_cast<const bf16x8 *>(rec + Rec::oT + o);
            Tf[kk].lo = *reinterpret_cast<const bf16x8 *>(rec + Rec::oT + kChunk * kChunk * 2 + o);
        }
        // P fragments of query block w (key blocks mt <= w; the rest is zero)
        Split4 Pf[4];
        if (OUT) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const uint4 u = mt <= w ? *reinterpret_cast<const uint4 *>(rec + Rec::oP + (size_t)((4 * w + mt) * 64 + l) * 16)
                                        : make_uint4(0u, 0u, 0u, 0u);
                const bf16x8 o = __builtin_bit_cast(bf16x8, u);
                Pf[mt].hi = __builtin_shufflevector(o, o, 0, 1, 2, 3);
                Pf[mt].lo = __builtin_shufflevector(o, o, 4, 5, 6, 7);
            }
        }
        // gamma of the key rows of this wave's state tiles
        f32x4 gam[NTS];
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT;
            gam[s] = *reinterpret_cast<const f32x4 *>(rec + Rec::oGam + (size_t)(16 * m + 4 * g) * 4);
        }
        float z[NVT][4];
#pragma unroll
        for (int n = 0; n < NVT; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tv = t0 + 16 * w + 4 * g + i;
                const size_t off = baseV + (size_t)(tv < T ? tv : T - 1) * tokV + 16 * n + r;
                const size_t offw = (SG && (a.scalar & kScalarWrite)) ? baseK / DK + (size_t)(tv < T ? tv : T - 1) * H
                                                                       : off;
                const float zz = gate_act<GL>(load_gate1<GL>(a.wg, offw)) * load1<BF16>(a.v, off, true);
                z[n][i] = tv < T ? zz : 0.f;
            }

        // ---- Kt rows into LDS (pitch PK); with the state copy of the previous chunk's end ----
#pragma unroll
        for (int it = 0; it < NKT; ++it) {
            const int idx = tid + kThreads * it, plane = idx / (8 * DK), rem = idx % (8 * DK);
            const int row = rem / (DK / 8), c8 = 8 * (rem % (DK / 8));
            *reinterpret_cast<uint4 *>(&sK[plane * RK + row * PK + c8]) = kraw[it];
        }
        __syncthreads();

        // ---- X = Z - Et S and Qt S for this wave's rows (S from LDS) ----
        f32x4 QS[NVT];
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
            f32x4 accX = {-z[n][0], -z[n][1], -z[n][2], -z[n][3]};
            f32x4 accQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                const Split8 sf = frag_8(&sS[(16 * n + r) * PK + 32 * j + 8 * g],
                                         &sS[VT * PK + (16 * n + r) * PK + 32 * j + 8 * g]);
                if (FAST) accX = mfma32(Et[j].hi, sf.hi, accX);
                else accX = mfma32x3(Et[j], sf, accX);
                if (OUT) accQ = mfma32x3(Qt[j], sf, accQ);
            }
            const Split4 xs = split4(-accX);  // lane holds X[16w + 4g + i][16n + r]
            *reinterpret_cast<bf16x4 *>(&sX[(16 * n + r) * PT + 16 * w + 4 * g]) = xs.hi;
            *reinterpret_cast<bf16x4 *>(&sX[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = xs.lo;
            QS[n] = accQ;
            GDN2_SWEEP_FENCE();
        }
        __syncthreads();

        // ---- U = T X for this wave's rows ----
        f32x4 accU[NVT];
#pragma unroll
        for (int n = 0; n < NVT; ++n) accU[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk < nkk) {
#pragma unroll
                for (int n = 0; n < NVT; ++n)
                    accU[n] = mfma32x3(Tf[kk], frag_8(&sX[(16 * n + r) * PT + 32 * kk + 8 * g],
                                                      &sX[VT * PT + (16 * n + r) * PT + 32 * kk + 8 * g]), accU[n]);
            }
        }
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
            const Split4 us = split4(accU[n]);
            *reinterpret_cast<bf16x4 *>(&sU[(16 * n + r) * PT + 16 * w + 4 * g]) = us.hi;
            *reinterpret_cast<bf16x4 *>(&sU[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = us.lo;
        }
        __syncthreads();

        // ---- O = Qt S + P U (P in the 4-group key order) ----
        if (OUT) {
#pragma unroll
            for (int n = 0; n < NVT; ++n) {
                f32x4 acc = QS[n];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk < nkk) {
                        const __bf16 *uh = &sU[(16 * n + r) * PT + 32 * kk];
                        const __bf16 *ul = &sU[VT * PT + (16 * n + r) * PT + 32 * kk];
                        acc = mfma32x3(join(Pf[2 * kk], Pf[2 * kk + 1]),
                                       frag_2x4(uh + 4 * g, uh + 16 + 4 * g, ul + 4 * g, ul + 16 + 4 * g), acc);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int to = t0 + 16 * w + 4 * g + i;
                    if (to < T) a.o[baseV + (size_t)to * tokV + 16 * n + r] = acc[i];
                }
                GDN2_SWEEP_FENCE();
            }
        }

        // ---- S' = diag(gamma) (S + Kt^T U), this wave's tiles of S ----
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT, n = id % NVT;
            f32x4 acc = S[s];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const Split8 kh = frag_tr<PK>(sK, sK + RK, 32 * kk, 16 * m, r, g);   // Kt^T
                const __bf16 *uh = &sU[(16 * n + r) * PT + 32 * kk];
                const __bf16 *ul = &sU[VT * PT + (16 * n + r) * PT + 32 * kk];
                acc = mfma32x3(kh, frag_2x4(uh + 4 * g, uh + 16 + 4 * g, ul + 4 * g, ul + 16 + 4 * g), acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) S[s][i] = acc[i] * gam[s][i];
            GDN2_SWEEP_FENCE();
        }
        __syncthreads();   // every wave is done with sK, sS, sX and sU of this chunk
        store_state_lds(w, r, g);
    }

    if (a.S_final) {
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT, n = id % NVT;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.S_final[sbase + (size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] = S[s][i];
        }
    }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------

template <int DK, int VT, bool BF16, bool GL, bool SG, int MODE>
static hipError_t sweep_t(const FwdArgs &a, hipStream_t st) {
    constexpr bool OUT = MODE != kFwdStates, STATES = MODE != kFwdOut;
    hipLaunchKernelGGL((fwd_sweep_kernel<DK, VT, BF16, OUT, STATES, GL, SG>), dim3((unsigned)(a.B * a.H * a.nvt)),
                       dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int DK, bool BF16, bool GL, bool SG, int MODE>
static hipError_t sweep_vt(const FwdArgs &a, int vt, hipStream_t st) {
    if constexpr (DK >= 64) {
        if (vt == 16) return sweep_t<DK, 16, BF16, GL, SG, MODE>(a, st);
    }
    if (vt == 32) return sweep_t<DK, 32, BF16, GL, SG, MODE>(a, st);
    if (vt == 64) return sweep_t<DK, 64, BF16, GL, SG, MODE>(a, st);
    return hipErrorInvalidValue;
}

template <bool BF16, bool GL, bool SG, int MODE>
static hipError_t sweep_dk(const FwdArgs &a, int dk, int vt, hipStream_t st) {
    switch (dk) {
        case 32: return sweep_vt<32, BF16, GL, SG, MODE>(a, vt, st);
        case 64: return sweep_vt<64, BF16, GL, SG, MODE>(a, vt, st);
        case 128: return sweep_vt<128, BF16, GL, SG, MODE>(a, vt, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16, bool GL, bool SG>
static hipError_t sweep_mode(const FwdArgs &a, int dk, int vt, FwdMode mode, hipStream_t st) {
    switch (mode) {
        case kFwdOut: return sweep_dk<BF16, GL, SG, kFwdOut>(a, dk, vt, st);
        case kFwdStates: return sweep_dk<BF16, GL, SG, kFwdStates>(a, dk, vt, st);
        case kFwdOutStates: return sweep_dk<BF16, GL, SG, kFwdOutStates>(a, dk, vt, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fwd_sweep(const FwdArgs &a, int dk, int vt, bool bf16, bool gl, bool sg, FwdMode mode,
                            hipStream_t st) {
    if (vt > a.dv || a.dv % vt != 0 || ((dk / 16) * (vt / 16)) % 4 != 0) return hipErrorInvalidValue;
    if (gl && sg) return hipErrorInvalidValue;
    if (gl) return bf16 ? sweep_mode<true, true, false>(a, dk, vt, mode, st) : hipErrorInvalidValue;
    if (sg) return bf16 ? sweep_mode<true, false, true>(a, dk, vt, mode, st) : hipErrorInvalidValue;
    return bf16 ? sweep_mode<true, false, false>(a, dk, vt, mode, st) : sweep_mode<false, false, false>(a, dk, vt, mode, st);
}

}  // namespace gdn2
