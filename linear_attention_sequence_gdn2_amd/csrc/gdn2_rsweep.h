// gdn2_rsweep.h -- the reverse sweep of the gate-aware backward as a device function, so that
// the reverse-sweep kernel and the combined forward/reverse sweep launch share one body.
//
// Per chunk, going backwards, the gradient of the chunk's start state is
//     dS = R dS' + Q2^T dO,   R = diag(gamma) - W^T Kh,   Q2 = Qt - P W,   W = T Et
// (the adjoint of the chunk equations of the blog on Gated DeltaNet-2, section "Token path and
// parallel training"), with R and Q2 read from the factor buffer that bwd_factors_kernel wrote.
#pragma once

#include "gdn2_chunk.h"
#include "gdn2_kernels.h"

namespace gdn2 {

// A operand of contraction step j from the two stored tiles kb = 2j, 2j + 1
__device__ __forceinline__ Split8 frag_from_tiles(const uint4 &t0, const uint4 &t1) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, t0), b = __builtin_bit_cast(bf16x8, t1);
    Split8 f;
    f.hi = __builtin_shufflevector(a, b, 0, 1, 2, 3, 8, 9, 10, 11);
    f.lo = __builtin_shufflevector(a, b, 4, 5, 6, 7, 12, 13, 14, 15);
    return f;
}

// ---------------------------------------------------------------------------
// reverse sweep: dS' of every chunk (dstates) and dS0
// ---------------------------------------------------------------------------
// One workgroup per (batch, head, value tile of VT columns); each wave owns the
// state tiles of one 16-row block.  Per chunk, going backwards: store dS', stage it
// and dO in LDS (double-buffered, so one barrier per chunk), then
// dS = R dS' + Q2^T dO.  The factors are chunk-local, so at VT = 64 (one workgroup
// per CU, registers to spare) the next chunk's fragments are loaded while the
// current chunk's products run; at VT = 32 and 16 two workgroups may share a CU instead.
template <int DK, int VT>
struct ReverseCfg {
    static constexpr int NM = DK / 16, NVT = VT / 16;
    static constexpr int NWAVES = (NM * NVT >= 8) ? 8 : NM * NVT;
    static constexpr int NTH = 64 * NWAVES;
    static constexpr int TPW = NM * NVT / NWAVES;   // state tiles per wave, all in one row block
    static constexpr bool PREFETCH = VT == 64;
    static constexpr int WG_PER_CU = VT == 64 ? 1 : 2;
    static_assert(TPW <= NVT, "a wave's tiles must share one row block");
};

// LDS: dS' tiles as [col][channel] (hi, lo) in sD0 / sD1 (RevLds::D elements each) and dO
// tiles as [col][token] (hi, lo) in sO0 / sO1 (RevLds::O each), double-buffered by chunk
// parity.  L: this workgroup's (batch, head, value tile) index.
template <int DK, int VT>
struct RevLds {
    static constexpr int D = 2 * VT * (DK + 8), O = 2 * VT * (kChunk + 8);
};

template <int DK, int VT>
__device__ __forceinline__ void bwd_reverse_body(const BwdArgs &a, const int L, __bf16 *sD0, __bf16 *sD1,
                                                 __bf16 *sO0, __bf16 *sO1) {
    using Cfg = ReverseCfg<DK, VT>;
    constexpr int NM = DK / 16, NKS = DK / 32, NVT = VT / 16;
    constexpr int NTH = Cfg::NTH, TPW = Cfg::TPW;
    constexpr int PK = DK + 8, PT = kChunk + 8;
    // dO elements per thread per chunk (at least 4: with more threads than that needs, the
    // upper ones load and stage a copy of the lower ones' values)
    constexpr int OPT = VT * kChunk / NTH >= 4 ? VT * kChunk / NTH : 4, OTG = kChunk / OPT;
    static_assert(OPT % 4 == 0 && OTG * OPT == kChunk, "dO staging");
    constexpr size_t FPC = factor_elems_per_chunk<DK>();

    const int tid = threadIdx.x, wv = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
    const int nvt = a.DV / VT;
    const int vt = L % nvt, bh = L / nvt, h = bh % a.H, b = bh / a.H;
    const int T = a.T, H = a.H, DV = a.DV;
    const int NC = (T + kChunk - 1) / kChunk;
    const int j0 = vt * VT;
    const size_t tokV = (size_t)H * DV;
    const size_t baseV = ((size_t)b * T * H + h) * DV + j0;
    const size_t sbase = ((size_t)b * H + h) * (size_t)DK * DV + j0;
    const int m = (wv * TPW) / NVT;                 // row block of this wave's state tiles
    const __bf16 *fbh = reinterpret_cast<const __bf16 *>(a.factors) + (size_t)bh * NC * FPC;
    auto col_block = [&](int s) { return (wv * TPW + s) % NVT; };

    f32x4 DS[TPW];
#pragma unroll
    for (int s = 0; s < TPW; ++s) {
        const int n = col_block(s);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            DS[s][i] = a.dS_final ? a.dS_final[sbase + (size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] : 0.f;
    }
    // dO staging: column tid % VT, tokens OPT * (tid / VT) .. + OPT - 1 of the chunk.  Loaded
    // 16 bytes at a time: for each group of 4 tokens a lane reads token + (tid % 4) at columns
    // 4 ((tid / 4) % (VT / 4)) ..; the 4x4 transpose inside each quad of lanes (at staging) gives
    // the lane its column.
    const int ocol = tid % VT, otg = (tid / VT) % OTG;
    float ox[OPT];
    auto load_dO = [&](int cc) {
#pragma unroll
        for (int q4 = 0; q4 < OPT / 4; ++q4) {
            const int t = cc * kChunk + OPT * otg + 4 * q4 + (tid & 3);
            const float4 f = *reinterpret_cast<const float4 *>(
                a.dO + baseV + (size_t)(t < T ? t : T - 1) * tokV + 4 * ((tid >> 2) % (VT / 4)));
            ox[4 * q4] = f.x, ox[4 * q4 + 1] = f.y, ox[4 * q4 + 2] = f.z, ox[4 * q4 + 3] = f.w;
        }
    };
    // factor fragments of row block m: R tiles (m, kb) and Q2^T tiles (m, kb)
    uint4 fr[NM], fq[4];
    auto load_factors = [&](int cc, uint4 (&xr)[NM], uint4 (&xq)[4]) {
        const __bf16 *fc = fbh + (size_t)cc * FPC;
#pragma unroll
        for (int kb = 0; kb < NM; ++kb)
            xr[kb] = *reinterpret_cast<const uint4 *>(fc + (size_t)(m * NM + kb) * kFragTile + 8 * l);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            xq[kb] = *reinterpret_cast<const uint4 *>(fc + (size_t)(NM * NM + m * 4 + kb) * kFragTile + 8 * l);
    };
    load_dO(NC - 1);
    if (Cfg::PREFETCH) load_factors(NC - 1, fr, fq);

    for (int c = NC - 1; c >= 0; --c) {
        __bf16 *const sDb = (c & 1) ? sD1 : sD0, *const sOb = (c & 1) ? sO1 : sO0;
        if (!Cfg::PREFETCH) load_factors(c, fr, fq);

        // gradient w.r.t. the end state of chunk c
        float *dst = a.dstates + ((size_t)bh * NC + c) * (size_t)DK * DV + j0;
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            const int n = col_block(s);
            {
                // one 16-byte store: the quad transpose gives the lane row 16m + 4g + (r % 4),
                // columns 16n + 4 (r / 4) ..
                float x[4] = {DS[s][0], DS[s][1], DS[s][2], DS[s][3]};
                quad_transpose4(x);
                *reinterpret_cast<float4 *>(&dst[(size_t)(16 * m + 4 * g + (r & 3)) * DV + 16 * n + 4 * (r >> 2)]) =
                    make_float4(x[0], x[1], x[2], x[3]);
            }
            const Split4 sp = split4(DS[s]);
            *reinterpret_cast<bf16x4 *>(&sDb[(16 * n + r) * PK + 16 * m + 4 * g]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&sDb[VT * PK + (16 * n + r) * PK + 16 * m + 4 * g]) = sp.lo;
        }
#pragma unroll
        for (int q4 = 0; q4 < OPT / 4; ++q4) {
            float x[4] = {ox[4 * q4], ox[4 * q4 + 1], ox[4 * q4 + 2], ox[4 * q4 + 3]};
            quad_transpose4(x);
#pragma unroll
            for (int i = 0; i < 4; ++i) ox[4 * q4 + i] = x[i];
        }
#pragma unroll
        for (int q4 = 0; q4 < OPT / 4; ++q4) {
            f32x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = (c * kChunk + OPT * otg + 4 * q4 + i < T) ? ox[4 * q4 + i] : 0.f;
            const Split4 so = split4(ov);
            *reinterpret_cast<bf16x4 *>(&sOb[ocol * PT + OPT * otg + 4 * q4]) = so.hi;
            *reinterpret_cast<bf16x4 *>(&sOb[VT * PT + ocol * PT + OPT * otg + 4 * q4]) = so.lo;
        }
        load_dO(c > 0 ? c - 1 : 0);   // the next chunk's dO is in flight during this chunk's products
        __syncthreads();
        uint4 nr[NM], nq[4];
        if (Cfg::PREFETCH) load_factors(c > 0 ? c - 1 : 0, nr, nq);

        // dS = R dS' + Q2^T dO
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            const int n = col_block(s);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NKS; ++j)
                acc = mfma32x3(frag_from_tiles(fr[2 * j], fr[2 * j + 1]),
                               row_frag4<PK, 1>(sDb, sDb + VT * PK, 16 * n + r, j, g), acc);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const __bf16 *oh = &sOb[(16 * n + r) * PT + 32 * kk], *ol = oh + VT * PT;
                acc = mfma32x3(frag_from_tiles(fq[2 * kk], fq[2 * kk + 1]),
                               frag_2x4<1>(oh + 4 * g, oh + 16 + 4 * g, ol + 4 * g, ol + 16 + 4 * g), acc);
            }
            DS[s] = acc;
        }
        if (Cfg::PREFETCH) {
#pragma unroll
            for (int kb = 0; kb < NM; ++kb) fr[kb] = nr[kb];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) fq[kb] = nq[kb];
        }
    }

    if (a.dS0) {
#pragma unroll
        for (int s = 0; s < TPW; ++s) {
            const int n = col_block(s);
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dS0[sbase + (size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] = DS[s][i];
        }
    }
}

}  // namespace gdn2
