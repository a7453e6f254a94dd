// gdn2_sweep.hip -- forward sweep of the Gated DeltaNet-2 rule from the chunk operand
// records on gfx950.
//
// Chunk form (blog on Gated DeltaNet-2, section "Token path and parallel training":
// cumulative channel decay absorbed into asymmetric erase factors, a triangular solve
// and dense products).  For a chunk with start state S:
//     X = Z - Et S,   U = T X,   O = Qt S + P U,   S' = diag(gamma) S + Kh^T U,
// with Z = w * v and Et, Kh, Qt, T = (I + A)^-1, P, gamma depending on the key side of
// the chunk only (Et = b k exp(G), Qt = q exp(G), Kh = k exp(g_C - G): every decay factor
// is at most 1, so these products stay in range whatever the decay).  The adjoint-factor kernel forms those for every chunk at once and
// keeps them in the chunk operand records; what is left for this sequential sweep are
// the products with the state, which cannot run ahead of the previous chunk.
//
// Kernels here:
//   fwd_sweep_kernel      4 waves per (batch, head, value tile of 16/32/64 columns), two per CU
//                         (fp32 q/k/v, dk = 32, dv not a multiple of 64, states-only with few heads)
//   fwd_sweep64_kernel    8 waves per 64-column tile, one per CU (body fwd_sweep64_body); its SEG
//                         modes are the passes of the segmented sweep
//   seg_combine_kernel    the segments' start states from their affine maps
//   fwd_rev_sweep_kernel  the wide forward sweep and the reverse sweep (gdn2_rsweep.h) side by
//                         side in one launch
//
// fwd_sweep_kernel: work decomposition as in the fused forward (gdn2_fwd.hip): one workgroup of 4 waves
// per (batch, head, value tile of VT columns), wave w owning tokens 16w..16w+15 for the
// rows of X, U and O and NTS tiles of the state; the fp32 state stays in registers (D
// layout) with a split-bf16 copy in LDS as the next chunk's operand.  Per chunk the
// wave loads its A operands (rows of Et, Qt, T and P) straight from the record into
// registers, and the workgroup stages the Kh rows in LDS for the transposed reads of
// the state update.  At VT = 32 a workgroup needs about 71 KB of LDS, so two share a CU.
// Four barriers per chunk: Kh rows and the state copy written; X written; U written;
// every wave done with the chunk's LDS.
#include "gdn2_chunk.h"
#include "gdn2_kernels.h"
#include "gdn2_rsweep.h"

namespace gdn2 {

#define GDN2_SWEEP_FENCE() __builtin_amdgcn_sched_barrier(0)

// Reads of a row-sum word of the fused epilogue before a wait counts as run out (each takes a
// load and a short sleep; in a correct run the word is there at the first read or soon after).
constexpr int kXrowSpins = 1 << 16;

#ifdef GDN2_STAMPS
// stamps of the unsegmented wide sweep: 8 per (workgroup, wave, chunk), see fwd_sweep64_body
static __device__ unsigned long long *g_sweep_stamps;
#endif

template <int DK, int VT, bool BF16, bool OUT, bool STATES, bool GL, bool SG>
__global__ __launch_bounds__(kThreads, 2) void fwd_sweep_kernel(FwdArgs a) {
    GDN2_POISON_LDS();
    using Rec = ChunkRecord<DK>;
    constexpr int NKS = DK / 32;           // 32-channel contraction steps
    constexpr int NVT = VT / 16;           // 16-column value tiles
    constexpr int NMT = DK / 16;           // 16-row key tiles of S
    constexpr int NTS = NMT * NVT / 4;     // S tiles per wave
    static_assert((NMT * NVT) % 4 == 0, "S tiles must split over 4 waves");
    constexpr bool FAST = BF16;            // X = Z - Et S with the hi part of Et (and all of S)
    constexpr int PK = DK + 8;             // row pitch of [row][channel] bf16 tiles
    constexpr int PT = kChunk + 8;         // row pitch of [col][token] bf16 tiles
    constexpr int RK = kChunk * PK;        // one [token][channel] plane
    constexpr int NKT = 2 * kChunk * DK / 8 / kThreads;   // 16-byte pieces per thread of the Kh planes
    static_assert(NKT * kThreads * 8 == 2 * kChunk * DK, "Kh planes split evenly over the threads");

    __shared__ __align__(16) __bf16 sK[2 * RK];         // Kh rows [token][channel] (hi, lo)
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
    // records of this (batch, head)
    const char *recs = reinterpret_cast<const char *>(a.records) + (size_t)bh * NC * Rec::BYTES;

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

        // ---- loads: Kh rows (for LDS), this wave's A operands, gamma, z = w * v ----
        uint4 kraw[NKT];
#pragma unroll
        for (int it = 0; it < NKT; ++it)
            kraw[it] = *reinterpret_cast<const uint4 *>(rec + Rec::oKh + (size_t)(tid + kThreads * it) * 16);
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
        // P fragments of query block w (the tiles with mt > w hold zeros)
        Split4 Pf[4];
        if (OUT) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const uint4 u = *reinterpret_cast<const uint4 *>(rec + Rec::oP + (size_t)((4 * w + mt) * 64 + l) * 16);
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

        // ---- Kh rows into LDS (pitch PK); with the state copy of the previous chunk's end ----
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
                if (FAST) accX = mfma32(Et[j].hi, sf.lo, mfma32(Et[j].hi, sf.hi, accX));
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

        // ---- S' = diag(gamma) S + Kh^T U, this wave's tiles of S ----
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT, n = id % NVT;
            f32x4 acc = S[s] * gam[s];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const Split8 kh = frag_tr<PK>(sK, sK + RK, 32 * kk, 16 * m, r, g);   // Kh^T
                const __bf16 *uh = &sU[(16 * n + r) * PT + 32 * kk];
                const __bf16 *ul = &sU[VT * PT + (16 * n + r) * PT + 32 * kk];
                acc = mfma32x3(kh, frag_2x4(uh + 4 * g, uh + 16 + 4 * g, ul + 4 * g, ul + 16 + 4 * g), acc);
            }
            S[s] = acc;
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
// 64-column value tiles: eight waves, one workgroup per CU, next chunk prefetched
// ---------------------------------------------------------------------------
// With 32-column tiles the four workgroups of a (batch, head) each read the whole
// record of every chunk, and every wave its own copy of the Et and Qt rows, right when
// the chunk starts; the sweep then waits on those loads.  Here a workgroup of eight
// waves takes 64 columns (half the record reads per head), stages the Kh, Et and Qt
// rows in LDS once for all waves, and loads each chunk's rows and value inputs while
// the previous chunk is in its products:
//   chunk c start      issue Kh rows, v, w of chunk c + 1
//   [A] X, Qt S        (Et, Qt rows and S from LDS)                 barrier
//   [B] U = T X        issue T of chunk c + 1; with STATES store S (the chunk's start state);
//                      Et, Qt rows of chunk c + 1 into LDS           barrier
//   [C] O; S'          after O, P of chunk c + 1 and the Et, Qt rows of chunk c + 2;
//                      after S', gamma of chunk c + 1; S' into LDS   barrier
//   Kh rows of chunk c + 1 into LDS
// Wave (hf, w) owns tokens 16w..16w+15 and columns 32hf..32hf+31 of X, U and O, and
// the state tiles of one 16-row block (at DK = 128).  bf16 q/k/v only (the X product
// uses the hi part of Et, so one Et plane is staged); about 155 KB of LDS.
// LDS arrays of the wide sweep (bf16 elements): Kh rows [token][channel] (hi, lo), Et rows (hi),
// Qt rows (hi, lo; only when o is written), S^T [col][channel], X^T and U^T [col][token] (hi, lo)
template <int DK, bool OUT, int VT = 64>
struct Sweep64Lds {
    static constexpr int RK = kChunk * (DK + 8);
    static constexpr int K = 2 * RK, E = RK, Q = OUT ? 2 * RK : 8;
    static constexpr int S = 2 * VT * (DK + 8), X = 2 * VT * (kChunk + 8), U = X;
};

// One workgroup's sweep: L is its (batch, head[, segment], value tile) index in launch order.
// VT = 64 value columns per tile, or 32 (no segments) where 64-column tiles would leave CUs idle.
// NV > 0: the output epilogue is fused, and a head has NV value tiles (dv = NV * VT).  Then
// o is never stored: the O tile of chunk c stays in registers until chunk c + 1, when the
// sums of squares of its rows over all dv columns are known, and y is stored instead.  Each
// wave publishes the sums of its 16 rows over its VT / 2 columns as 64-bit words
// {value, c + 1} (one store, so the tag and the value become visible together) with
// device-scope atomic stores; during the next chunk the four lanes of a row read the row's
// 2 NV words between them with device-scope atomic loads and add them with lane shuffles.  A
// word whose tag is not there yet is read again (bounded; a.xerr counts waits that ran out).
// Every wave adds the 2 NV sums in the same order, so the tiles of a row apply the same factor.
template <int DK, bool OUT, bool STATES, bool GL, bool SG, int SEG, int VT = 64, int NV = 0>
__device__ __forceinline__ void fwd_sweep64_body(const FwdArgs &a, const int L, __bf16 *sK, __bf16 *sE,
                                                 __bf16 *sQ, __bf16 *sS, __bf16 *sX, __bf16 *sU,
                                                 float *sW = nullptr) {
    using Rec = ChunkRecord<DK>;
    static_assert(VT == 64 || (VT == 32 && SEG == 0), "64-column tiles, or 32 without segments");
    constexpr bool EPI = NV > 0;
    constexpr int NSRC = 2 * (EPI ? NV : 1);             // row sums per row: both halves of every tile
    static_assert(!EPI || (OUT && !STATES && SEG == 0 && NV <= 4), "the epilogue rides on the plain o sweep");
    constexpr int NTH = kChunkThreads;
    constexpr int NCB = VT / 16, CBW = VT / 32;          // 16-column blocks: per tile, per wave half
    constexpr int NKS = DK / 32, NMT = DK / 16;
    constexpr int NTS = NMT * NCB / 8;                   // state tiles per wave
    static_assert((NMT * NCB) % 8 == 0 && NCB % NTS == 0, "a wave's state tiles share one row block");
    constexpr int PK = DK + 8, PT = kChunk + 8, RK = kChunk * PK;
    constexpr int PL16 = kChunk * DK / 8;                // 16-byte pieces of one row plane
    constexpr int NKP = 2 * PL16 / NTH;                  // Kh pieces per thread
    constexpr int NEQ = 1 + (OUT ? 2 : 0);               // Et hi, Qt hi and lo
    constexpr int NEP = NEQ * PL16 / NTH;                // Et/Qt pieces per thread
    static_assert(NKP * NTH == 2 * PL16 && NEP * NTH == NEQ * PL16, "row planes split evenly");

    // Segments (SEG 1, 2): each (b, h) is split into nseg runs of seg_len chunks.  SEG 1 sweeps a
    // segment from a zero state (value tiles) and, in DK / 64 more tiles, from the identity with
    // z = 0: the end states N and M give the segment's map S -> M S + N.  SEG 2 sweeps a segment
    // from its true start state (the maps composed in order) and writes o.
    const int ntile = SEG == 1 ? a.nvt + DK / 64 : a.nvt;
    const int vt = L % ntile, rest = L / ntile;
    const int seg = SEG ? rest % a.nseg : 0, bh = SEG ? rest / a.nseg : rest;
    const bool ident = SEG == 1 && vt >= a.nvt;         // a tile of the segment's state map
    const int h = bh % a.H, b = bh / a.H;
    const int T = a.T, H = a.H, DV = a.dv;
    const int j0 = (ident ? 0 : vt) * VT;               // identity tiles read column 0's v and w
    const int jI = ident ? (vt - a.nvt) * VT : 0;       // and hold columns jI.. of the DK x DK map
    const size_t tokV = (size_t)H * DV;
    const size_t baseK = ((size_t)b * T * H + h) * DK;
    const size_t baseV = ((size_t)b * T * H + h) * DV + j0;
    const size_t sbase = ((size_t)b * H + h) * (size_t)DK * DV + j0;
    const int NC = (T + kChunk - 1) / kChunk;
    const int c_lo = SEG ? seg * a.seg_len : 0;
    const int c_hi = SEG ? min(c_lo + a.seg_len, NC) : NC;
    const float zon = ident ? 0.f : 1.f;                // z = w * v, zero on identity tiles
    const char *recs = reinterpret_cast<const char *>(a.records) + (size_t)bh * NC * Rec::BYTES;

    // record pieces of the Kh planes and of the Et/Qt planes, and where they go in LDS
    auto kt_piece = [&](int c, int it, int tid) {
        return *reinterpret_cast<const uint4 *>(recs + (size_t)c * Rec::BYTES + Rec::oKh +
                                                 (size_t)(tid + NTH * it) * 16);
    };
    auto kt_store = [&](const uint4 &u, int it, int tid) {
        const int idx = tid + NTH * it, p = idx / PL16, rem = idx % PL16;
        *reinterpret_cast<uint4 *>(&sK[p * RK + (rem / (DK / 8)) * PK + 8 * (rem % (DK / 8))]) = u;
    };
    auto eq_piece = [&](int c, int it, int tid) {
        const int idx = tid + NTH * it, p = idx / PL16, rem = idx % PL16;
        // plane 0: Et hi; planes 1, 2: Qt hi, lo
        const int src = p == 0 ? Rec::oEt : Rec::oQt + (p - 1) * Rec::PLANE;
        return *reinterpret_cast<const uint4 *>(recs + (size_t)c * Rec::BYTES + src + (size_t)rem * 16);
    };
    auto eq_store = [&](const uint4 &u, int it, int tid) {
        const int idx = tid + NTH * it, p = idx / PL16, rem = idx % PL16;
        __bf16 *dst = p == 0 ? sE : sQ + (p - 1) * RK;
        *reinterpret_cast<uint4 *>(&dst[(rem / (DK / 8)) * PK + 8 * (rem % (DK / 8))]) = u;
    };
    // v and w of this wave's X rows: each lane loads four consecutive columns of one token
    // row (token 16w + 4g + (r & 3), columns 32hf + 16n + 4(r >> 2) ..), and a quad
    // transpose turns them into the D layout (token 16w + 4g + i, column 32hf + 16n + r)
    auto load_vw = [&](int c, float (&vv)[CBW][4], float (&ww)[CBW][4], int w, int hf, int r, int g) {
        const int tv = c * kChunk + 16 * w + 4 * g + (r & 3);
        const size_t row = (size_t)(tv < T ? tv : T - 1);
#pragma unroll
        for (int n = 0; n < CBW; ++n) {
            const size_t off = baseV + row * tokV + 16 * CBW * hf + 16 * n + 4 * (r >> 2);
            const uint2 vr = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(a.v) + off);
            vv[n][0] = __builtin_bit_cast(float, vr.x << 16);
            vv[n][1] = __builtin_bit_cast(float, vr.x & 0xffff0000u);
            vv[n][2] = __builtin_bit_cast(float, vr.y << 16);
            vv[n][3] = __builtin_bit_cast(float, vr.y & 0xffff0000u);
            if (SG && (a.scalar & kScalarWrite)) {
                const float wt = reinterpret_cast<const float *>(a.wg)[baseK / DK + row * H];
                ww[n][0] = ww[n][1] = ww[n][2] = ww[n][3] = wt;
            } else if (GL) {
                const uint2 wr = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(a.wg) + off);
                ww[n][0] = __builtin_bit_cast(float, wr.x << 16);
                ww[n][1] = __builtin_bit_cast(float, wr.x & 0xffff0000u);
                ww[n][2] = __builtin_bit_cast(float, wr.y << 16);
                ww[n][3] = __builtin_bit_cast(float, wr.y & 0xffff0000u);
            } else {
                const float4 wr = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.wg) + off);
                ww[n][0] = wr.x; ww[n][1] = wr.y; ww[n][2] = wr.z; ww[n][3] = wr.w;
            }
        }
    };
    auto to_d_layout = [](float (&vv)[CBW][4], float (&ww)[CBW][4]) {
#pragma unroll
        for (int n = 0; n < CBW; ++n) {
            quad_transpose4(vv[n]);
            quad_transpose4(ww[n]);
        }
    };

    int tid = threadIdx.x;
    int wv = tid >> 6, w = wv & 3, hf = wv >> 2, l = tid & 63, r = l & 15, g = l >> 4;
    f32x4 S[NTS];
#pragma unroll
    for (int s = 0; s < NTS; ++s) {
        const int id = wv * NTS + s, m = id / NCB, n = id % NCB;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * m + 4 * g + i, col = 16 * n + r;
            if (SEG == 0) S[s][i] = a.S0 ? a.S0[sbase + (size_t)row * DV + col] : 0.f;
            else if (SEG == 1) S[s][i] = (ident && row == jI + col) ? 1.f : 0.f;
            else S[s][i] = a.S0[(((size_t)bh * a.nseg + seg) * DK + row) * DV + j0 + col];
        }
    }
    auto store_state_lds = [&](int wv, int r, int g) {
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = wv * NTS + s, m = id / NCB, n = id % NCB;
            const Split4 sp = split4(S[s]);
            *reinterpret_cast<bf16x4 *>(&sS[(16 * n + r) * PK + 16 * m + 4 * g]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&sS[VT * PK + (16 * n + r) * PK + 16 * m + 4 * g]) = sp.lo;
        }
    };
    // prologue: chunk 0's rows into LDS, its value inputs, chunk 1's Et/Qt rows in flight
    float vv[CBW][4], ww[CBW][4], z[CBW][4];
    load_vw(c_lo, vv, ww, w, hf, r, g);
    to_d_layout(vv, ww);
#pragma unroll
    for (int n = 0; n < CBW; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            z[n][i] = c_lo * kChunk + 16 * w + 4 * g + i < T ? zon * gate_act<GL>(ww[n][i]) * vv[n][i] : 0.f;
    {
        uint4 kp[NKP], ep[NEP];
#pragma unroll
        for (int it = 0; it < NKP; ++it) kp[it] = kt_piece(c_lo, it, tid);
#pragma unroll
        for (int it = 0; it < NEP; ++it) ep[it] = eq_piece(c_lo, it, tid);
#pragma unroll
        for (int it = 0; it < NKP; ++it) kt_store(kp[it], it, tid);
#pragma unroll
        for (int it = 0; it < NEP; ++it) eq_store(ep[it], it, tid);
    }
    uint4 eqn[NEP];                                      // Et/Qt rows of the next chunk
#pragma unroll
    for (int it = 0; it < NEP; ++it) eqn[it] = eq_piece(c_lo + 1 < c_hi ? c_lo + 1 : c_lo, it, tid);
    store_state_lds(wv, r, g);
    if constexpr (EPI) {
        if (tid < VT) sW[tid] = a.oweight ? a.oweight[j0 + tid] : 1.f;   // this tile's norm weights
    }
    __syncthreads();

    const int nkk = (w >= 2) ? 2 : 1;
    // T, P and gamma of a chunk are loaded during the previous chunk, each right after its last
    // use there, so they are in flight across a whole stage without extra registers
    auto load_T = [&](const char *rc, Split8 (&tf)[2]) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const size_t o = (size_t)((16 * w + r) * kChunk + (kk < nkk ? 32 * kk : 0) + 8 * g) * 2;
            tf[kk].hi = *reinterpret_cast<const bf16x8 *>(rc + Rec::oT + o);
            tf[kk].lo = *reinterpret_cast<const bf16x8 *>(rc + Rec::oT + kChunk * kChunk * 2 + o);
        }
    };
    auto load_P = [&](const char *rc, uint4 (&p)[4]) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)   // the tiles with mt > w hold zeros
            p[mt] = *reinterpret_cast<const uint4 *>(rc + Rec::oP + (size_t)((4 * w + mt) * 64 + l) * 16);
    };
    auto load_gam = [&](const char *rc) {
        return *reinterpret_cast<const f32x4 *>(rc + Rec::oGam + (size_t)(16 * ((wv * NTS) / NCB) + 4 * g) * 4);
    };
    // ---- fused output epilogue (NV > 0) ----
    // eo: the O tile of the pending chunk in the lane layout after the quad transpose (row erow =
    // 16w + 4g + (r & 3), columns 16cb + 4(r >> 2) .. + 3); gr: its output-gate values as loaded
    // (four bf16 in .x, .y, or four fp32).  The 2 NV row sums of a row are read by its four lanes
    // (r >> 2 = 0 .. 3): lane k takes sources k, k + 4, .. (NSRC 2: source k & 1), and two xor
    // shuffles add them, in an order that every wave of every tile repeats.  Words live in a
    // ring of two chunk slots: slot c & 1 of chunk c is written again at chunk c + 2, after every
    // reader of it has published chunk c + 1 (each reads its chunk-c words before that).
    constexpr int XS = NSRC >= 4 ? NSRC / 4 : 1;          // words a lane reads per row and chunk
    float eo[CBW][4];
    unsigned long long xw[XS];
    uint4 gr[CBW];
    const int erow = 16 * w + 4 * g + (r & 3);
    auto xrow_idx = [&](int cc, int src, int row) {
        return ((size_t)(bh * 2 + (cc & 1)) * NSRC + src) * 64 + row;
    };
    auto xsrc = [&](int k) { return NSRC >= 4 ? (r >> 2) + 4 * k : (r >> 2) & 1; };
    // loads for chunk cp: this lane's row-sum words (whatever is there yet) and the gate values
    auto epi_issue = [&](int cp) {
#pragma unroll
        for (int k = 0; k < XS; ++k)
            xw[k] = __hip_atomic_load(a.xrow + xrow_idx(cp, xsrc(k), erow), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        const int t = cp * kChunk + erow;
        const size_t row = (size_t)(t < T ? t : T - 1);
        const unsigned esz = a.og_bf16 ? 2u : 4u;
#pragma unroll
        for (int n = 0; n < CBW; ++n) {
            // both halves loaded whatever the dtype (the bf16 case reads its 8 bytes twice), so that
            // no load sits under a branch
            const char *p = reinterpret_cast<const char *>(a.og) +
                            (baseV + row * tokV + 16 * (CBW * hf + n) + 4 * (r >> 2)) * esz;
            const uint2 lo = *reinterpret_cast<const uint2 *>(p);
            const uint2 hi = *reinterpret_cast<const uint2 *>(p + (a.og_bf16 ? 0 : 8));
            gr[n] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
    };
    // a word whose tag has not arrived: read again, bounded
    auto epi_wait = [&](int cp) {
        const unsigned tag = (unsigned)(cp + 1);
        for (int spin = 0; spin < kXrowSpins; ++spin) {
            __builtin_amdgcn_s_sleep(2);
            bool ok = true;
#pragma unroll
            for (int k = 0; k < XS; ++k) {
                if ((unsigned)(xw[k] >> 32) != tag)
                    xw[k] = __hip_atomic_load(a.xrow + xrow_idx(cp, xsrc(k), erow), __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                ok = ok && (unsigned)(xw[k] >> 32) == tag;
            }
            if (__all(ok)) return;
        }
        if ((threadIdx.x & 63) == 0) atomicAdd(a.xerr, 1);
    };
    // y of chunk cp from eo: the row's sum of squares over all dv columns, then norm, weight and
    // gate
    auto epi_finish = [&](int cp) {
        const unsigned tag = (unsigned)(cp + 1);
        bool ok = true;
#pragma unroll
        for (int k = 0; k < XS; ++k) ok = ok && (unsigned)(xw[k] >> 32) == tag;
        if (!__all(ok)) epi_wait(cp);
        float tot = __uint_as_float((unsigned)xw[0]);
#pragma unroll
        for (int k = 1; k < XS; ++k) tot += __uint_as_float((unsigned)xw[k]);
        tot += __shfl_xor(tot, 4);
        if (NSRC >= 4) tot += __shfl_xor(tot, 8);
        const float rs = __builtin_amdgcn_rsqf(tot * (1.f / (float)(NSRC / 2 * VT)) + a.eps);
        const int t = cp * kChunk + erow;
#pragma unroll
        for (int n = 0; n < CBW; ++n) {
            const int col = 16 * (CBW * hf + n) + 4 * (r >> 2);
            const float4 wt = *reinterpret_cast<const float4 *>(&sW[col]);
            float gv[4];
            if (a.og_bf16) {
                gv[0] = __uint_as_float(gr[n].x << 16), gv[1] = __uint_as_float(gr[n].x & 0xffff0000u);
                gv[2] = __uint_as_float(gr[n].y << 16), gv[3] = __uint_as_float(gr[n].y & 0xffff0000u);
            } else {
                gv[0] = __uint_as_float(gr[n].x), gv[1] = __uint_as_float(gr[n].y);
                gv[2] = __uint_as_float(gr[n].z), gv[3] = __uint_as_float(gr[n].w);
            }
            const f32x4 yv = {eo[n][0] * rs * wt.x * gv[0], eo[n][1] * rs * wt.y * gv[1], eo[n][2] * rs * wt.z * gv[2],
                              eo[n][3] * rs * wt.w * gv[3]};
            if (t < T) {
                const size_t off = baseV + (size_t)t * tokV + col;
                if (a.y_bf16)
                    *reinterpret_cast<bf16x4 *>(reinterpret_cast<__bf16 *>(a.y) + off) =
                        __builtin_convertvector(yv, bf16x4);
                else
                    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.y) + off) = yv;
            }
        }
    };
    (void)xrow_idx;
    (void)epi_issue;
    (void)epi_finish;

    Split8 Tf[2];
    uint4 pv[4];
    load_T(recs + (size_t)c_lo * Rec::BYTES, Tf);
    if (OUT) load_P(recs + (size_t)c_lo * Rec::BYTES, pv);
    f32x4 gam = load_gam(recs + (size_t)c_lo * Rec::BYTES);
    for (int c = c_lo; c < c_hi; ++c) {
        const int t0 = c * kChunk;
        const int cn = c + 1 < c_hi ? c + 1 : c;         // the next chunk (itself at the end)
        const int cn2 = c + 2 < c_hi ? c + 2 : cn;       // the one after
#ifdef GDN2_STAMPS
        // [A] from 0 to 1, [B] 2 to 3, O 4 to 5, S' 5 to 6; 1-2, 3-4 and 6-7 are barriers
        unsigned long long *stp = SEG == 0 && !EPI && g_sweep_stamps
                                      ? g_sweep_stamps + (((size_t)L * 8 + wv) * NC + c) * 8
                                      : nullptr;
#else
        unsigned long long *stp = nullptr;
#endif
        (void)stp;
        GDN2_STAMP_REGS;

        // ---- loads: Kh rows, v, w of the next chunk (T, P and gamma of this one are in flight);
        // with the epilogue after stage A, where they leave room for its registers ----
        uint4 ktn[NKP];
        if constexpr (!EPI) {
#pragma unroll
            for (int it = 0; it < NKP; ++it) ktn[it] = kt_piece(cn, it, tid);
            load_vw(cn, vv, ww, w, hf, r, g);   // z of the next chunk is formed at this chunk's end
        } else {
            // the row sums and gate values of the pending chunk, two stages ahead of their use
            epi_issue(c > c_lo ? c - 1 : c_lo);   // unconditional: at c_lo its values go unused
        }

        // ---- [A] X = Z - Et S and Qt S: tiles (token block w, column blocks 2hf, 2hf + 1) ----
        GDN2_STAMP(stp, 0);
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
                accX = mfma32(eh, sf.lo, mfma32(eh, sf.hi, accX));   // Et (hi part) times S (hi and lo)
                if (OUT)
                    accQ = mfma32x3(frag_8(&sQ[(16 * w + r) * PK + 32 * j + 8 * g],
                                           &sQ[RK + (16 * w + r) * PK + 32 * j + 8 * g]), sf, accQ);
            }
            const Split4 xs = split4(-accX);  // lane holds X[16w + 4g + i][16cb + r]
            *reinterpret_cast<bf16x4 *>(&sX[(16 * cb + r) * PT + 16 * w + 4 * g]) = xs.hi;
            *reinterpret_cast<bf16x4 *>(&sX[VT * PT + (16 * cb + r) * PT + 16 * w + 4 * g]) = xs.lo;
            QS[n] = accQ;
        }
        GDN2_STAMP(stp, 1);
        __syncthreads();
        if constexpr (EPI) {
#pragma unroll
            for (int it = 0; it < NKP; ++it) ktn[it] = kt_piece(cn, it, tid);
            load_vw(cn, vv, ww, w, hf, r, g);
        }

        // ---- [B] U = T X; then the next chunk's Et/Qt rows into LDS ----
        GDN2_STAMP(stp, 2);
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
            load_T(recs + (size_t)cn * Rec::BYTES, Tf);
        if (STATES) {
            // the chunk-start state (S is updated only in S'), here rather than at the chunk's
            // start, where the stores held up the issue of the next chunk's loads.  One 16-byte
            // store per tile: the quad transpose gives the lane row 16m + 4g + (r & 3), columns
            // 16n + 4(r >> 2) ..
            float *dst = a.states + (((size_t)b * H + h) * NC + c) * (size_t)DK * DV + j0;
#pragma unroll
            for (int s = 0; s < NTS; ++s) {
                const int id = wv * NTS + s, m = id / NCB, n = id % NCB;
                float x[4] = {S[s][0], S[s][1], S[s][2], S[s][3]};
                quad_transpose4(x);
                *reinterpret_cast<float4 *>(&dst[(size_t)(16 * m + 4 * g + (r & 3)) * DV + 16 * n + 4 * (r >> 2)]) =
                    make_float4(x[0], x[1], x[2], x[3]);
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
        GDN2_STAMP(stp, 3);
        if (c + 1 < c_hi) {
#pragma unroll
            for (int it = 0; it < NEP; ++it) eq_store(eqn[it], it, tid);
        }
        __syncthreads();
        GDN2_STAMP(stp, 4);

        // ---- [C] O = Qt S + P U; S' = diag(gamma) S + Kh^T U ----
        if constexpr (EPI) {
            if (c > c_lo) epi_finish(c - 1);   // y of the pending chunk; frees eo for this one
        }
        if (OUT) {
            Split4 Pf[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8 o = __builtin_bit_cast(bf16x8, pv[mt]);
                Pf[mt].hi = __builtin_shufflevector(o, o, 0, 1, 2, 3);
                Pf[mt].lo = __builtin_shufflevector(o, o, 4, 5, 6, 7);
            }
            float ss = 0.f;                         // sum of squares of this lane's O elements
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
                quad_transpose4(x);   // row 16w + 4g + (r & 3), columns 16cb + 4(r >> 2) ..
                if constexpr (EPI) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        eo[n][i] = x[i];
                        ss += x[i] * x[i];
                    }
                } else {
                    const int to = t0 + 16 * w + 4 * g + (r & 3);
                    if (to < T)
                        *reinterpret_cast<float4 *>(&a.o[baseV + (size_t)to * tokV + 16 * cb + 4 * (r >> 2)]) =
                            make_float4(x[0], x[1], x[2], x[3]);
                }
            }
            if constexpr (EPI) {
                // the row's sum over this wave's columns: the four lanes r >> 2 = 0 .. 3 of the row
                ss += __shfl_xor(ss, 4);
                ss += __shfl_xor(ss, 8);
                if ((r >> 2) == 0) {
                    const unsigned long long word =
                        ((unsigned long long)(unsigned)(c + 1) << 32) | (unsigned long long)__float_as_uint(ss);
                    __hip_atomic_store(a.xrow + xrow_idx(c, 2 * vt + hf, 16 * w + 4 * g + r), word, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            load_P(recs + (size_t)cn * Rec::BYTES, pv);
        }
        // the Et/Qt rows of chunk c + 2, after O's products (issued before them, they held the
        // products up behind a full memory queue)
#pragma unroll
        for (int it = 0; it < NEP; ++it) eqn[it] = eq_piece(cn2, it, tid);
        GDN2_STAMP(stp, 5);
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = wv * NTS + s, m = id / NCB, n = id % NCB;
            f32x4 acc = S[s] * gam;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const Split8 kh = frag_tr<PK>(sK, sK + RK, 32 * kk, 16 * m, r, g);   // Kh^T
                const __bf16 *uh = &sU[(16 * n + r) * PT + 32 * kk];
                const __bf16 *ul = &sU[VT * PT + (16 * n + r) * PT + 32 * kk];
                acc = mfma32x3(kh, frag_2x4(uh + 4 * g, uh + 16 + 4 * g, ul + 4 * g, ul + 16 + 4 * g), acc);
            }
            S[s] = acc;
        }
        GDN2_STAMP(stp, 6);
        gam = load_gam(recs + (size_t)cn * Rec::BYTES);
        store_state_lds(wv, r, g);     // sS is not read again in this chunk
        __syncthreads();
        GDN2_STAMP(stp, 7);
        GDN2_STAMP_FLUSH(stp);
        // the next chunk's Kh rows (sK is not read again in this chunk) and its z = w * v,
        // from loads issued at this chunk's start
        if (c + 1 < c_hi) {
#pragma unroll
            for (int it = 0; it < NKP; ++it) kt_store(ktn[it], it, tid);
        }
        to_d_layout(vv, ww);
#pragma unroll
        for (int n = 0; n < CBW; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                z[n][i] = (c + 1) * kChunk + 16 * w + 4 * g + i < T ? zon * gate_act<GL>(ww[n][i]) * vv[n][i] : 0.f;
    }

    if constexpr (EPI) {
        if (c_hi > c_lo) {
            epi_issue(c_hi - 1);
            epi_finish(c_hi - 1);
        }
    }

    if (SEG == 1) {
        // the segment's end-state block [N | M], DK x (DV + DK), of this (b, h) and segment
        const int ldE = DV + DK;
        float *e = a.states + ((size_t)bh * a.nseg + seg) * DK * ldE + (ident ? DV + jI : j0);
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = wv * NTS + s, m = id / NCB, n = id % NCB;
#pragma unroll
            for (int i = 0; i < 4; ++i) e[(size_t)(16 * m + 4 * g + i) * ldE + 16 * n + r] = S[s][i];
        }
    } else if (a.S_final && (SEG == 0 || seg == a.nseg - 1)) {
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = wv * NTS + s, m = id / NCB, n = id % NCB;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.S_final[sbase + (size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] = S[s][i];
        }
    }
}

template <int DK, bool OUT, bool STATES, bool GL, bool SG, int SEG, int VT = 64, int NV = 0>
__global__ __launch_bounds__(kChunkThreads, 1) void fwd_sweep64_kernel(FwdArgs a) {
    GDN2_POISON_LDS();
    using Lds = Sweep64Lds<DK, OUT, VT>;
    __shared__ __align__(16) __bf16 sK[Lds::K], sE[Lds::E], sQ[Lds::Q], sS[Lds::S], sX[Lds::X], sU[Lds::U];
    __shared__ __align__(16) float sW[NV > 0 ? VT : 4];
    fwd_sweep64_body<DK, OUT, STATES, GL, SG, SEG, VT, NV>(a, xcd_swizzle(blockIdx.x, gridDim.x), sK, sE, sQ, sS,
                                                           sX, sU, sW);
}

// The training step's two sweeps in one launch: the forward sweep (the state before every chunk,
// and o and S_final when OUT) and the reverse sweep (dS' of every chunk, dS0), both from one factor
// buffer.  Neither reads what the other writes, and with few heads each alone leaves CUs idle.
// The first nfwd workgroups (in the swizzled order) sweep forward, the others backward, both on
// VT-column tiles (64, or 32 when even those leave every workgroup a CU of its own); the reverse
// role keeps its dS' and dO buffers in the forward role's arrays.
template <int DK, bool OUT, bool GL, bool SG, int VT>
__global__ __launch_bounds__(kChunkThreads, 1) void fwd_rev_sweep_kernel(FwdArgs fa, BwdArgs ba, int nfwd) {
    GDN2_POISON_LDS();
    using Lds = Sweep64Lds<DK, OUT, VT>;
    using RL = RevLds<DK, VT>;
    static_assert(RL::D <= Lds::K && RL::D <= Lds::S && RL::O <= Lds::X && RL::O <= Lds::U,
                  "the reverse role's buffers fit the forward role's arrays");
    static_assert(ReverseCfg<DK, VT>::NTH == kChunkThreads, "both roles take the whole workgroup");
    __shared__ __align__(16) __bf16 sK[Lds::K], sE[Lds::E], sQ[Lds::Q], sS[Lds::S], sX[Lds::X], sU[Lds::U];
    const int L = xcd_swizzle(blockIdx.x, gridDim.x);
    if (L < nfwd) fwd_sweep64_body<DK, OUT, true, GL, SG, 0, VT>(fa, L, sK, sE, sQ, sS, sX, sU);
    else bwd_reverse_body<DK, VT>(ba, L - nfwd, sK, sS, sX, sU);
}

// ---------------------------------------------------------------------------
// segment composition: the start state of every segment of a (b, h)
// ---------------------------------------------------------------------------
// The chunk map is affine in the state (S' = M S + N, the form the multi-GPU design splits a
// sequence by), so a segment's is too.  Given each segment's end-state block [N_s | M_s]
// (DK x (DV + DK), from the SEG 1 sweep), the start states follow in order:
//     S_0 = S0 (or zero),   S_{s+1} = M_s S_s + N_s.
// One workgroup per (b, h) and 16 state columns; fp32 FMA, M_s staged in LDS.
template <int DK>
__global__ __launch_bounds__(256) void seg_combine_kernel(const float *E, const float *S0, float *Sin, int DV,
                                                          int nseg) {
    GDN2_POISON_LDS();
    constexpr int NCB = 16;                       // state columns per workgroup
    constexpr int PM = DK + 4;                    // row pitch of M in LDS
    constexpr int RPT = DK / 64;                  // rows per thread: 64 row blocks x 4 column blocks
    __shared__ __align__(16) float sS[DK * NCB];
    __shared__ __align__(16) float sM[DK * PM];
    const int ncb = DV / NCB;
    const int bh = blockIdx.x / ncb, j0 = NCB * (blockIdx.x % ncb);
    const int tid = threadIdx.x, rb = tid >> 2, cb = tid & 3;
    const int ldE = DV + DK;
    for (int idx = tid; idx < DK * NCB; idx += 256) {
        const int row = idx / NCB, col = idx % NCB;
        sS[idx] = S0 ? S0[((size_t)bh * DK + row) * DV + j0 + col] : 0.f;
    }
    __syncthreads();
    for (int s = 0; s < nseg; ++s) {
        const size_t blk = (size_t)bh * nseg + s;
        for (int idx = tid; idx < DK * NCB; idx += 256) {
            const int row = idx / NCB, col = idx % NCB;
            Sin[(blk * DK + row) * DV + j0 + col] = sS[idx];
        }
        if (s + 1 == nseg) break;
        for (int idx = tid; idx < DK * DK / 4; idx += 256) {
            const int row = idx / (DK / 4), k4 = idx % (DK / 4);
            *reinterpret_cast<float4 *>(&sM[row * PM + 4 * k4]) =
                *reinterpret_cast<const float4 *>(&E[(blk * DK + row) * ldE + DV + 4 * k4]);
        }
        __syncthreads();
        float acc[RPT][4];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float4 nv = *reinterpret_cast<const float4 *>(&E[(blk * DK + RPT * rb + i) * ldE + j0 + 4 * cb]);
            acc[i][0] = nv.x, acc[i][1] = nv.y, acc[i][2] = nv.z, acc[i][3] = nv.w;
        }
        for (int kx = 0; kx < DK; ++kx) {
            const float4 sv = *reinterpret_cast<const float4 *>(&sS[kx * NCB + 4 * cb]);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const float mv = sM[(RPT * rb + i) * PM + kx];
                acc[i][0] = fmaf(mv, sv.x, acc[i][0]);
                acc[i][1] = fmaf(mv, sv.y, acc[i][1]);
                acc[i][2] = fmaf(mv, sv.z, acc[i][2]);
                acc[i][3] = fmaf(mv, sv.w, acc[i][3]);
            }
        }
        __syncthreads();   // every thread has read this segment's state and map
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            *reinterpret_cast<float4 *>(&sS[(RPT * rb + i) * NCB + 4 * cb]) =
                make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
#ifdef GDN2_STAMPS
// the instrumented build only: where the unsegmented wide sweep writes its phase stamps
// (8 per workgroup, wave and chunk; nullptr = none)
extern "C" int gdn2_stamps_sweep(void *buf) {
    unsigned long long *p = static_cast<unsigned long long *>(buf);
    return hipMemcpyToSymbol(HIP_SYMBOL(g_sweep_stamps), &p, sizeof(p)) == hipSuccess ? 0 : 4;
}
#endif

// Value-tile width of the four-wave sweep: 32 columns (two workgroups share a CU), 16 where that
// gives too few workgroups (aiming at 512 or more).
int fwd_value_tile(int B, int H, int dk, int dv) {
    auto ok = [&](int vt) { return vt <= dv && dv % vt == 0 && ((dk / 16) * (vt / 16)) % 4 == 0; };
    int vt = dv < 32 ? dv : 32;
    while (vt > 16 && (long)B * H * (dv / vt) < 512 && ok(vt / 2)) vt /= 2;
    return vt;
}

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

template <int DK, bool GL, bool SG, int MODE, int VT>
static hipError_t sweep64_t(const FwdArgs &a, hipStream_t st) {
    constexpr bool OUT = MODE != kFwdStates, STATES = MODE != kFwdOut;
    hipLaunchKernelGGL((fwd_sweep64_kernel<DK, OUT, STATES, GL, SG, 0, VT>), dim3((unsigned)(a.B * a.H * a.nvt)),
                       dim3(kChunkThreads), 0, st, a);
    return hipGetLastError();
}

template <int DK, bool GL, bool SG>
static hipError_t sweep64_dk(const FwdArgs &a, FwdMode mode, hipStream_t st) {
    // 32-column tiles only where o is written (the states-only sweep takes the wide kernel only
    // when 64-column tiles fill every CU)
    const bool vt32 = a.nvt * 32 == a.dv;
    switch (mode) {
        case kFwdOut: return vt32 ? sweep64_t<DK, GL, SG, kFwdOut, 32>(a, st) : sweep64_t<DK, GL, SG, kFwdOut, 64>(a, st);
        case kFwdStates: return vt32 ? hipErrorInvalidValue : sweep64_t<DK, GL, SG, kFwdStates, 64>(a, st);
        case kFwdOutStates:
            return vt32 ? sweep64_t<DK, GL, SG, kFwdOutStates, 32>(a, st) : sweep64_t<DK, GL, SG, kFwdOutStates, 64>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool GL, bool SG>
static hipError_t sweep64_mode(const FwdArgs &a, int dk, FwdMode mode, hipStream_t st) {
    if (dk == 128) return sweep64_dk<128, GL, SG>(a, mode, st);
    if (dk == 64) return sweep64_dk<64, GL, SG>(a, mode, st);
    return hipErrorInvalidValue;
}

// SEG 1: the maps; SEG 2: o (ST false) or the state before every chunk (ST true)
template <int DK, bool GL, bool SG, int SEG, bool ST>
static hipError_t seg_t(const FwdArgs &a, hipStream_t st) {
    const int ntile = SEG == 1 ? a.nvt + DK / 64 : a.nvt;
    hipLaunchKernelGGL((fwd_sweep64_kernel<DK, SEG == 2 && !ST, SEG == 2 && ST, GL, SG, SEG>),
                       dim3((unsigned)(a.B * a.H * a.nseg * ntile)), dim3(kChunkThreads), 0, st, a);
    return hipGetLastError();
}

template <int SEG, bool ST>
static hipError_t seg_dk(const FwdArgs &a, int dk, bool gl, bool sg, hipStream_t st) {
    if (gl && sg) return hipErrorInvalidValue;
    if (dk == 128) return gl ? seg_t<128, true, false, SEG, ST>(a, st) : sg ? seg_t<128, false, true, SEG, ST>(a, st)
                                                                              : seg_t<128, false, false, SEG, ST>(a, st);
    if (dk == 64) return gl ? seg_t<64, true, false, SEG, ST>(a, st) : sg ? seg_t<64, false, true, SEG, ST>(a, st)
                                                                            : seg_t<64, false, false, SEG, ST>(a, st);
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_segments(const FwdArgs &a_in, int dk, bool gl, bool sg, float *E, float *Sin,
                               hipStream_t st) {
    if (a_in.dv % 64 != 0 || a_in.nseg < 1 || a_in.seg_len < 1) return hipErrorInvalidValue;
    if ((a_in.o == nullptr) == (a_in.states == nullptr)) return hipErrorInvalidValue;   // o or states
    FwdArgs a = a_in;
    a.nvt = a.dv / 64;
    // 1: every segment's map from zero and identity starts
    a.S0 = nullptr, a.o = nullptr, a.S_final = nullptr, a.states = E;
    hipError_t e = seg_dk<1, false>(a, dk, gl, sg, st);
    if (e != hipSuccess) return e;
    // 2: the start states, composed in order
    const unsigned ncomb = (unsigned)(a.B * a.H * (a.dv / 16));
    if (dk == 128) hipLaunchKernelGGL((seg_combine_kernel<128>), dim3(ncomb), dim3(256), 0, st, E, a_in.S0, Sin, a.dv, a.nseg);
    else if (dk == 64) hipLaunchKernelGGL((seg_combine_kernel<64>), dim3(ncomb), dim3(256), 0, st, E, a_in.S0, Sin, a.dv, a.nseg);
    else return hipErrorInvalidValue;
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // 3: every segment again from its start state, writing o or the chunk states (and S_final
    // from the last segment)
    a.S0 = Sin, a.o = a_in.o, a.S_final = a_in.S_final, a.states = a_in.states;
    return a_in.states ? seg_dk<2, true>(a, dk, gl, sg, st) : seg_dk<2, false>(a, dk, gl, sg, st);
}

hipError_t launch_fwd_sweep(const FwdArgs &a_in, int dk, int vt, bool bf16, bool gl, bool sg, FwdMode mode,
                            hipStream_t st) {
    if (gl && sg) return hipErrorInvalidValue;
    // 64-column (or 32-column) tiles (eight waves, one workgroup per CU) whenever o is written: a sequential
    // chain is paced by its per-chunk latency, and the eight-wave chunk step is about half that of
    // the four-wave one, which more than pays for leaving CUs idle when there are few heads
    // (B1 T16K H16: 1.56 against 2.33 ms).  The states-only sweep has less per-chunk work and
    // takes the narrower tiles of the four-wave kernel unless the wide ones fill every CU
    // (B1 T16K H16: 0.85 against 1.13 ms).
    const bool wide_fills = (long)a_in.B * a_in.H * (a_in.dv / 64) >= cu_count();
    if (bf16 && (dk == 64 || dk == 128) && a_in.dv % 64 == 0 && (mode != kFwdStates || wide_fills)) {
        FwdArgs a = a_in;
        // 32-column tiles where even they give each workgroup a CU of its own: a chunk step with
        // half the columns is shorter, and the sweep is paced by its depth (B4 T4K H16: the
        // inference forward 0.57 -> 0.50 ms, o and states 0.44 -> 0.33 ms; bit-identical results)
        const bool vt32 = mode != kFwdStates && 2L * a.B * a.H * (a.dv / 64) <= cu_count();
        a.nvt = a.dv / (vt32 ? 32 : 64);
        if (gl) return sweep64_mode<true, false>(a, dk, mode, st);
        if (sg) return sweep64_mode<false, true>(a, dk, mode, st);
        return sweep64_mode<false, false>(a, dk, mode, st);
    }
    const FwdArgs &a = a_in;
    if (vt > a.dv || a.dv % vt != 0 || ((dk / 16) * (vt / 16)) % 4 != 0) return hipErrorInvalidValue;
    if (gl) return bf16 ? sweep_mode<true, true, false>(a, dk, vt, mode, st) : hipErrorInvalidValue;
    if (sg) return bf16 ? sweep_mode<true, false, true>(a, dk, vt, mode, st) : hipErrorInvalidValue;
    return bf16 ? sweep_mode<true, false, false>(a, dk, vt, mode, st) : sweep_mode<false, false, false>(a, dk, vt, mode, st);
}

// ---- the forward sweep with the output epilogue fused ----
// The tile width is the plain o sweep's (32 columns where they still give each workgroup a CU
// of its own); NV = dv / width tiles share a row.  With NV > 1 the tiles of a head wait on each
// other's row sums, so the launch is cooperative: every workgroup is resident at once.
static int out_tile(int B, int H, int dv) { return 2L * B * H * (dv / 64) <= cu_count() ? 32 : 64; }

template <int DK, bool GL, bool SG, int VT, int NV>
static const void *out_kernel() {
    return reinterpret_cast<const void *>(&fwd_sweep64_kernel<DK, true, false, GL, SG, 0, VT, NV>);
}

template <int DK, bool GL, bool SG>
static const void *out_kernel_vt(int vt, int nv) {
    if (vt == 64 && nv == 1) return out_kernel<DK, GL, SG, 64, 1>();
    if (vt == 64 && nv == 2) return out_kernel<DK, GL, SG, 64, 2>();
    if (vt == 32 && nv == 2) return out_kernel<DK, GL, SG, 32, 2>();
    if (vt == 32 && nv == 4) return out_kernel<DK, GL, SG, 32, 4>();
    return nullptr;
}

static const void *out_kernel_for(int dk, bool gl, bool sg, int vt, int nv) {
    if (gl && sg) return nullptr;
    if (dk == 128)
        return gl ? out_kernel_vt<128, true, false>(vt, nv) : sg ? out_kernel_vt<128, false, true>(vt, nv)
                                                                   : out_kernel_vt<128, false, false>(vt, nv);
    if (dk == 64)
        return gl ? out_kernel_vt<64, true, false>(vt, nv) : sg ? out_kernel_vt<64, false, true>(vt, nv)
                                                                  : out_kernel_vt<64, false, false>(vt, nv);
    return nullptr;
}

bool fwd_out_fused(int B, int H, int T, int dk, int dv, bool bf16) {
    (void)T;
    if (!bf16 || (dk != 64 && dk != 128) || dv % 64 != 0) return false;
    const int vt = out_tile(B, H, dv), nv = dv / vt;
    const void *k = out_kernel_for(dk, false, false, vt, nv);
    if (!k) return false;
    if (nv == 1) return true;
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k, kChunkThreads, 0) != hipSuccess || per < 1) return false;
    return (long)B * H * nv <= (long)per * cu_count();
}

size_t fwd_out_exchange_bytes(int B, int H, int T, int dk, int dv) {
    (void)dk;
    const int nv = dv / out_tile(B, H, dv);
    (void)T;
    const size_t words = (size_t)B * H * 2 * (2 * nv) * 64;   // two chunk slots of 2 nv sources x 64 rows
    return words * sizeof(unsigned long long) + 256;          // then the run-out counter (one int, 256-byte slot)
}

hipError_t launch_fwd_sweep_out(const FwdArgs &a_in, int dk, bool gl, bool sg, hipStream_t st) {
    if (!fwd_out_fused(a_in.B, a_in.H, a_in.T, dk, a_in.dv, true)) return hipErrorInvalidValue;
    FwdArgs a = a_in;
    const int vt = out_tile(a.B, a.H, a.dv), nv = a.dv / vt;
    a.nvt = nv;
    a.o = nullptr, a.states = nullptr;
    const void *k = out_kernel_for(dk, gl, sg, vt, nv);
    if (!k) return hipErrorInvalidValue;
    void *args[] = {&a};
    const dim3 grid((unsigned)(a.B * a.H * nv)), block(kChunkThreads);
    if (nv == 1) return hipLaunchKernel(k, grid, block, args, 0, st);
    return hipLaunchCooperativeKernel(k, grid, block, args, 0, st);
}

template <int DK, bool GL, bool SG, int VT>
static hipError_t fwd_rev_vt(const FwdArgs &fa_in, const BwdArgs &ba, hipStream_t st) {
    FwdArgs fa = fa_in;
    fa.nvt = fa.dv / VT;
    const int nfwd = fa.B * fa.H * fa.nvt;
    if (fa.o)
        hipLaunchKernelGGL((fwd_rev_sweep_kernel<DK, true, GL, SG, VT>), dim3((unsigned)(2 * nfwd)), dim3(kChunkThreads),
                           0, st, fa, ba, nfwd);
    else
        hipLaunchKernelGGL((fwd_rev_sweep_kernel<DK, false, GL, SG, VT>), dim3((unsigned)(2 * nfwd)),
                           dim3(kChunkThreads), 0, st, fa, ba, nfwd);
    return hipGetLastError();
}

// 32-column tiles for both roles where they still give every workgroup a CU of its own (the
// chunk steps of both sweeps are shorter at 32 columns), else 64
template <int DK, bool GL, bool SG>
static hipError_t fwd_rev_t(const FwdArgs &fa, const BwdArgs &ba, hipStream_t st) {
    if (4L * fa.B * fa.H * (fa.dv / 64) <= cu_count()) return fwd_rev_vt<DK, GL, SG, 32>(fa, ba, st);
    return fwd_rev_vt<DK, GL, SG, 64>(fa, ba, st);
}

bool fwd_rev_fused(int B, int H, int dk, int dv, bool bf16) {
    return bf16 && (dk == 64 || dk == 128) && dv % 64 == 0 && 2L * B * H * (dv / 64) <= cu_count();
}

hipError_t launch_fwd_rev_sweeps(const FwdArgs &fa_in, const BwdArgs &ba, int dk, bool gl, bool sg, hipStream_t st) {
    if (gl && sg) return hipErrorInvalidValue;
    if (!fwd_rev_fused(fa_in.B, fa_in.H, dk, fa_in.dv, true) || !fa_in.states || !ba.dstates)
        return hipErrorInvalidValue;
    const FwdArgs &fa = fa_in;
    if (dk == 128) return gl ? fwd_rev_t<128, true, false>(fa, ba, st) : sg ? fwd_rev_t<128, false, true>(fa, ba, st)
                                                                           : fwd_rev_t<128, false, false>(fa, ba, st);
    return gl ? fwd_rev_t<64, true, false>(fa, ba, st) : sg ? fwd_rev_t<64, false, true>(fa, ba, st)
                                                             : fwd_rev_t<64, false, false>(fa, ba, st);
}

}  // namespace gdn2
