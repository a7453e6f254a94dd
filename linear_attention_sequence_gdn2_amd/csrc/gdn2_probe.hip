// gdn2_probe.hip -- GEMM-phase microkernels of the forward, for the instrumented build only.
//
// The forward's GEMM phases (the record kernel's A and P products and triangular solve; the
// sweep's X / Qt S, U = T X, O and S' products) run here with every operand resident in LDS or
// registers and no global memory access inside the timed windows, each phase repeated `reps`
// times per workgroup, one workgroup of eight waves per CU.  They use the product kernels' own
// helpers (ap_pair_queue and solve_T_inplace are the functions the record kernel calls) and, for
// the sweep, the same tiles, fragments and loop order as fwd_sweep64_body at dk = 128 with
// 64-column tiles.  The operands are small deterministic values: only the time matters.  This
// measures what the GEMM code reaches when it does not wait on memory, the cross-check of the
// per-phase stamps taken inside the product kernels.
//
// Stamps: per (workgroup, wave, repetition) 8 slots of s_memtime (register-buffered, written
// after the repetition): phase 0 (A, P): 0 start, 1 end; phase 1 (solve): 0 start, 1 end;
// phase 2 (sweep stages): 0-1 X and Qt S, 2-3 U = T X, 4-5 O, 5-6 S'.
#ifdef GDN2_STAMPS

#include <hip/hip_runtime.h>

#include "gdn2_chunk.h"
#include "gdn2_kernels.h"

namespace gdn2 {
namespace {

constexpr int kProbeDK = 128, kProbeVT = 64;
constexpr int kPK = kProbeDK + 8, kPT = kChunk + 8, kPA = kChunk + 4, kRK = kChunk * kPK;

// a small value in [-1/16, 1/16) from an index (a multiplicative hash)
__device__ __forceinline__ float probe_val(unsigned i) {
    return ((float)((i * 2654435761u) >> 8) * (1.f / 16777216.f) - 0.5f) * 0.125f;
}

__device__ __forceinline__ void probe_fill_bf16(__bf16 *p, int n, unsigned salt) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = (__bf16)probe_val(salt + (unsigned)i);
}

__device__ __forceinline__ unsigned long long *probe_slot(unsigned long long *st, int reps, int rep) {
    const int wv = threadIdx.x >> 6;
    return st + (((size_t)blockIdx.x * 8 + wv) * reps + rep) * 8;
}

// phase 0: A and P of one chunk from the pair queue (the record kernel's a5 phase)
__global__ __launch_bounds__(kChunkThreads, 1) void probe_ap_kernel(unsigned long long *st, int reps, float *sink) {
    __shared__ __align__(16) __bf16 sKt[2 * kRK], sEt[2 * kRK], sQt[2 * kRK];
    __shared__ __align__(16) float sAT[kChunk * kPA];
    __shared__ __align__(16) char sPf[16 * 64 * 16];
    __shared__ int sCnt;
    probe_fill_bf16(sKt, 2 * kRK, 1u);
    probe_fill_bf16(sEt, 2 * kRK, 7u);
    probe_fill_bf16(sQt, 2 * kRK, 13u);
    const int tid = threadIdx.x, l = tid & 63, r = l & 15, g = l >> 4;
    for (int rep = 0; rep < reps; ++rep) {
        if (tid == 0) sCnt = 0;
        __syncthreads();
        GDN2_STAMP_REGS;
        GDN2_STAMP(st, 0);
        ap_pair_queue<kProbeDK, kPK, kPA>(sKt, sEt, sQt, sAT, sPf, &sCnt, l, r, g);
        __syncthreads();
        GDN2_STAMP(st, 1);
        GDN2_STAMP_FLUSH(probe_slot(st, reps, rep));
    }
    // keep the results live
    const float tot = sAT[(tid * 7) % (kChunk * kPA)] + (float)reinterpret_cast<const __bf16 *>(sPf)[tid * 8];
    if (tot == 12345.f) sink[blockIdx.x] = tot;   // practically never; the compiler cannot tell
}

// phase 1: the triangular solve T = (I + A)^-1 in place (the record kernel's a6 phase); A is
// restored from a copy before every repetition, outside the window
__global__ __launch_bounds__(kChunkThreads, 1) void probe_solve_kernel(unsigned long long *st, int reps, float *sink) {
    __shared__ __align__(16) float sAT[kChunk * kPA], sA0[kChunk * kPA];
    for (int i = threadIdx.x; i < kChunk * kPA; i += blockDim.x) {
        const int row = i / kPA, col = i % kPA;
        sA0[i] = col < row ? probe_val(3u + (unsigned)i) : 0.f;   // strictly lower
    }
    const int tid = threadIdx.x, wv = tid >> 6, hf = wv >> 2, w = wv & 3, l = tid & 63, r = l & 15, g = l >> 4;
    (void)l;
    for (int rep = 0; rep < reps; ++rep) {
        __syncthreads();
        for (int i = tid; i < kChunk * kPA; i += blockDim.x) sAT[i] = sA0[i];
        __syncthreads();
        GDN2_STAMP_REGS;
        GDN2_STAMP(st, 0);
        solve_T_inplace<kPA>(sAT, w, r, g, hf == 0);   // ends with a barrier
        GDN2_STAMP(st, 1);
        GDN2_STAMP_FLUSH(probe_slot(st, reps, rep));
    }
    const float tot = sAT[(tid * 7) % (kChunk * kPA)];
    if (tot == 12345.f) sink[blockIdx.x] = tot;
}

// phase 2: the sweep's products for one chunk (fwd_sweep64_body's stages A, B and C, with o
// written to LDS-free registers only), repeated on the same resident rows
__global__ __launch_bounds__(kChunkThreads, 1) void probe_sweep_kernel(unsigned long long *st, int reps,
                                                                       float *sink) {
    constexpr int DK = kProbeDK, VT = kProbeVT, NTH = kChunkThreads;
    constexpr int NCB = VT / 16, CBW = VT / 32, NKS = DK / 32, NMT = DK / 16, NTS = NMT * NCB / 8;
    constexpr int PK = kPK, PT = kPT, RK = kRK;
    static_assert(NTH == 512 && NTS * 8 == NMT * NCB, "eight waves, whole state tiles");
    __shared__ __align__(16) __bf16 sK[2 * RK], sE[RK], sQ[2 * RK];
    __shared__ __align__(16) __bf16 sS[2 * VT * PK], sX[2 * VT * PT], sU[2 * VT * PT];
    probe_fill_bf16(sK, 2 * RK, 21u);
    probe_fill_bf16(sE, RK, 29u);
    probe_fill_bf16(sQ, 2 * RK, 37u);
    const int tid = threadIdx.x, wv = tid >> 6, w = wv & 3, hf = wv >> 2, l = tid & 63, r = l & 15, g = l >> 4;
    const int nkk = (w >= 2) ? 2 : 1;
    // registers the sweep loads from the record: T (two split 8-wide fragments), P (four tiles),
    // gamma; the state and z
    Split8 Tf[2];
    uint4 pv[4];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            Tf[kk].hi[i] = (__bf16)probe_val(41u + 16u * kk + i + 64u * l);
            Tf[kk].lo[i] = (__bf16)0.f;
        }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (__bf16)(i < 4 ? probe_val(53u + 8u * mt + i + 64u * l) : 0.f);
        pv[mt] = __builtin_bit_cast(uint4, o);
    }
    const f32x4 gam = {0.5f, 0.5f, 0.5f, 0.5f};
    f32x4 S[NTS];
    float z[CBW][4];
#pragma unroll
    for (int s = 0; s < NTS; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[s][i] = probe_val(61u + 4u * s + i + 64u * tid);
#pragma unroll
    for (int n = 0; n < CBW; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) z[n][i] = probe_val(71u + 4u * n + i + 8u * tid);
    auto store_state_lds = [&]() {
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = wv * NTS + s, m = id / NCB, n = id % NCB;
            const Split4 sp = split4(S[s]);
            *reinterpret_cast<bf16x4 *>(&sS[(16 * n + r) * PK + 16 * m + 4 * g]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&sS[VT * PK + (16 * n + r) * PK + 16 * m + 4 * g]) = sp.lo;
        }
    };
    store_state_lds();
    float ssum = 0.f;
    for (int rep = 0; rep < reps; ++rep) {
        __syncthreads();
        GDN2_STAMP_REGS;
        // [A] X = Z - Et S and Qt S
        GDN2_STAMP(st, 0);
        f32x4 QS[CBW];
#pragma unroll
        for (int n = 0; n < CBW; ++n) {
            const int cb = CBW * hf + n;
            f32x4 accX = {-z[n][0], -z[n][1], -z[n][2], -z[n][3]};
            f32x4 accQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                const Split8 sf = frag_8(&sS[(16 * cb + r) * PK + 32 * j + 8 * g],
                                         &sS[VT * PK + (16 * cb + r) * PK + 32 * j + 8 * g]);
                const bf16x8 eh = *reinterpret_cast<const bf16x8 *>(&sE[(16 * w + r) * PK + 32 * j + 8 * g]);
                accX = mfma32(eh, sf.lo, mfma32(eh, sf.hi, accX));
                accQ = mfma32x3(frag_8(&sQ[(16 * w + r) * PK + 32 * j + 8 * g],
                                       &sQ[RK + (16 * w + r) * PK + 32 * j + 8 * g]), sf, accQ);
            }
            const Split4 xs = split4(-accX);
            *reinterpret_cast<bf16x4 *>(&sX[(16 * cb + r) * PT + 16 * w + 4 * g]) = xs.hi;
            *reinterpret_cast<bf16x4 *>(&sX[VT * PT + (16 * cb + r) * PT + 16 * w + 4 * g]) = xs.lo;
            QS[n] = accQ;
        }
        GDN2_STAMP(st, 1);
        __syncthreads();
        // [B] U = T X
        GDN2_STAMP(st, 2);
        {
            f32x4 accU[CBW];
#pragma unroll
            for (int n = 0; n < CBW; ++n) accU[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk < nkk) {
#pragma unroll
                    for (int n = 0; n < CBW; ++n) {
                        const int cb = CBW * hf + n;
                        accU[n] = mfma32x3(Tf[kk], frag_8(&sX[(16 * cb + r) * PT + 32 * kk + 8 * g],
                                                          &sX[VT * PT + (16 * cb + r) * PT + 32 * kk + 8 * g]),
                                           accU[n]);
                    }
                }
            }
#pragma unroll
            for (int n = 0; n < CBW; ++n) {
                const int cb = CBW * hf + n;
                const Split4 us = split4(accU[n]);
                *reinterpret_cast<bf16x4 *>(&sU[(16 * cb + r) * PT + 16 * w + 4 * g]) = us.hi;
                *reinterpret_cast<bf16x4 *>(&sU[VT * PT + (16 * cb + r) * PT + 16 * w + 4 * g]) = us.lo;
            }
        }
        GDN2_STAMP(st, 3);
        __syncthreads();
        // [C] O = Qt S + P U (kept in registers); S' = diag(gamma) S + Kh^T U
        GDN2_STAMP(st, 4);
        {
            Split4 Pf[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8 o = __builtin_bit_cast(bf16x8, pv[mt]);
                Pf[mt].hi = __builtin_shufflevector(o, o, 0, 1, 2, 3);
                Pf[mt].lo = __builtin_shufflevector(o, o, 4, 5, 6, 7);
            }
#pragma unroll
            for (int n = 0; n < CBW; ++n) {
                const int cb = CBW * hf + n;
                f32x4 acc = QS[n];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk < nkk) {
                        const __bf16 *uh = &sU[(16 * cb + r) * PT + 32 * kk];
                        const __bf16 *ul = &sU[VT * PT + (16 * cb + r) * PT + 32 * kk];
                        acc = mfma32x3(join(Pf[2 * kk], Pf[2 * kk + 1]),
                                       frag_2x4(uh + 4 * g, uh + 16 + 4 * g, ul + 4 * g, ul + 16 + 4 * g), acc);
                    }
                }
                float x[4] = {acc[0], acc[1], acc[2], acc[3]};
                quad_transpose4(x);
                ssum += (x[0] + x[1]) + (x[2] + x[3]);
            }
        }
        GDN2_STAMP(st, 5);
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = wv * NTS + s, m = id / NCB, n = id % NCB;
            f32x4 acc = S[s] * gam;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const Split8 kh = frag_tr<PK>(sK, sK + RK, 32 * kk, 16 * m, r, g);
                const __bf16 *uh = &sU[(16 * n + r) * PT + 32 * kk];
                const __bf16 *ul = &sU[VT * PT + (16 * n + r) * PT + 32 * kk];
                acc = mfma32x3(kh, frag_2x4(uh + 4 * g, uh + 16 + 4 * g, ul + 4 * g, ul + 16 + 4 * g), acc);
            }
            S[s] = acc;
        }
        GDN2_STAMP(st, 6);
        store_state_lds();
        GDN2_STAMP_FLUSH(probe_slot(st, reps, rep));
    }
    // keep the results live
    float tot = ssum;
#pragma unroll
    for (int s = 0; s < NTS; ++s) tot += (S[s][0] + S[s][1]) + (S[s][2] + S[s][3]);
    if (tot == 12345.f) sink[blockIdx.x] = tot;   // practically never; the compiler cannot tell
}

}  // namespace

// Runs GEMM-phase microkernel `phase` (0: A and P, 1: solve, 2: sweep stages) with `grid`
// workgroups of 512 threads for `reps` repetitions each, on `stream`.  `stamps`: device buffer of
// grid * 8 * reps * 8 uint64 (see the top of this file); `sink`: one float per workgroup (never
// written in practice; it keeps the results live).  0 on success, 4 on a launch error, 1 on bad
// arguments.
extern "C" int gdn2_probe_gemm_phases(int phase, int grid, int reps, void *stamps, void *sink, void *stream) {
    if (phase < 0 || phase > 2 || grid < 1 || reps < 1 || stamps == nullptr || sink == nullptr) return 1;
    auto *st = static_cast<unsigned long long *>(stamps);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (phase == 0)
        hipLaunchKernelGGL(probe_ap_kernel, dim3((unsigned)grid), dim3(kChunkThreads), 0, s, st, reps,
                           static_cast<float *>(sink));
    else if (phase == 1)
        hipLaunchKernelGGL(probe_solve_kernel, dim3((unsigned)grid), dim3(kChunkThreads), 0, s, st, reps,
                           static_cast<float *>(sink));
    else
        hipLaunchKernelGGL(probe_sweep_kernel, dim3((unsigned)grid), dim3(kChunkThreads), 0, s, st, reps,
                           static_cast<float *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace gdn2

#endif  // GDN2_STAMPS
