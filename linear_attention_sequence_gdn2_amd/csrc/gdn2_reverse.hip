// gdn2_reverse.hip -- reverse sweep of the gate-aware backward on gfx950: per-chunk
// adjoint factors (chunk-parallel), then the chunk-to-chunk recurrence of the state
// gradient (sequential over chunks).
//
// Chunk notation of gdn2_fwd.hip (blog on Gated DeltaNet-2, section "Token path and
// parallel training"): start state S, end state S' = diag(gamma)(S + Kt^T U),
// U = T X, X = Z - Et S, O = Qt S + P U.  The adjoint of one chunk gives for the
// gradient of its start state
//     dS = Qt^T dO + diag(gamma) dS' - Et^T dX,   dX = T^T (P^T dO + Kt diag(gamma) dS').
// With W = T Et (the WY factor of the erase keys) this is
//     dS = R dS' + Q2^T dO,   R = (I - W^T Kt) diag(gamma),   Q2 = Qt - P W,
// where R (dk x dk) and Q2 (64 x dk) depend on the key side of the chunk only.
// bwd_factors_kernel forms them for every (batch, head, chunk) at once, and
// bwd_reverse_kernel is left with two dense products per chunk on its critical path.
//
// Factor buffer of one (batch, head, chunk): NM*NM tiles of R, then NM*4 tiles of
// Q2^T (NM = dk/16).  Tile (m, kb) of a matrix X holds X[16m + r'][16kb + c'] for
// r', c' < 16 in MFMA fragment order: 64 lanes x 8 bf16, lane (r, g) storing
// X[16m + r][16kb + 4g + i] split as hi (i < 4) then lo (i < 4).  Two tiles kb = 2j,
// 2j + 1 give a lane its whole A operand of contraction step j in the 4-group order,
// with one 16-byte load each.
#include "gdn2_chunk.h"
#include "gdn2_kernels.h"
#include "gdn2_rsweep.h"

namespace gdn2 {

// 16x16 tile from its D-layout transpose: the lane holds X[16m + r][16kb + 4g + i] (i < 4)
__device__ __forceinline__ void store_frag_tile(__bf16 *tile, int l, const f32x4 &v) {
    const Split4 s = split4(v);
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[i] = s.hi[i];
        o[4 + i] = s.lo[i];
    }
    *reinterpret_cast<bf16x8 *>(tile + 8 * l) = o;
}

// ---------------------------------------------------------------------------
// adjoint factors R and Q2^T of every (batch, head, chunk)
// ---------------------------------------------------------------------------
// Eight waves in two halves, as in bwd_chunk_kernel: wave (hf, w) owns tokens
// 16w..16w+15 and, for the element work, the channels of half hf.
// FWD: forward-only records (a.factors holds just the records): the rows, T, P and gamma
// that the forward sweep reads, without the adjoint factors, P^T, G or the Et lo plane.
template <int DK, bool BF16, bool GL, bool SG, bool FWD>
__global__ __launch_bounds__(kChunkThreads, 1) void bwd_factors_kernel(BwdArgs a) {
    constexpr int NTH = kChunkThreads;
    constexpr int NM = DK / 16, NKS = DK / 32, NMH = DK / 32, NEH = 4 * NMH;
    constexpr int PK = DK + 8, PT = kChunk + 8, PA = kChunk + 4;
    constexpr int RK = kChunk * PK;
    using Rec = ChunkRecord<DK>;
    // LDS (bytes): Kt, Et, Qt rows [token][channel] (hi, lo); the decay totals after the
    // Et rows; W^T [channel][token] (hi, lo) later over the Et rows and the totals;
    // A then T (fp32); gamma per channel.
    constexpr int B_ROWS = 2 * RK * 2, B_WT = 2 * DK * PT * 2, B_TOT = 4 * DK * 4;
    constexpr int oKt = 0, oEt = oKt + B_ROWS, oTot = oEt + B_ROWS;
    constexpr int oQt0 = (oTot + B_TOT > oEt + B_WT) ? oTot + B_TOT : oEt + B_WT;
    constexpr int oQt = (oQt0 + 15) / 16 * 16;
    constexpr int oAT = oQt + B_ROWS, oGam = oAT + kChunk * PA * 4;
    constexpr int SMEM = oGam + DK * 4;
    static_assert(SMEM <= 160 * 1024, "LDS budget of a CU");

    __shared__ __align__(16) char smem[SMEM];
    __bf16 *sKt = reinterpret_cast<__bf16 *>(smem + oKt), *sEt = reinterpret_cast<__bf16 *>(smem + oEt);
    __bf16 *sQt = reinterpret_cast<__bf16 *>(smem + oQt), *sWT = reinterpret_cast<__bf16 *>(smem + oEt);
    float *sTot = reinterpret_cast<float *>(smem + oTot), *sAT = reinterpret_cast<float *>(smem + oAT);
    float *sGam = reinterpret_cast<float *>(smem + oGam);

    const int tid = threadIdx.x, wv = tid >> 6, hf = wv >> 2, w = wv & 3, l = tid & 63, r = l & 15, g = l >> 4;
    const int NC = (a.T + kChunk - 1) / kChunk;
    const int T = a.T, H = a.H;
    const int nitems = a.B * H * NC;                    // item L = (b * H + h) * NC + c
    const size_t tokK = (size_t)H * DK;
    const int nkk = (w >= 2) ? 2 : 1;
    const int chh = hf * (DK / 2);
    auto ch = [&](int e) { return chh + ch4(e, g); };
    // this lane's token row (channel 0 of its half) in item L, and whether the token exists
    auto item_row = [&](int L, bool &valid) {
        const int c = L % NC, bh = L / NC, h = bh % H, b = bh / H;
        const int tk = c * kChunk + 16 * w + r;
        valid = tk < T;
        return ((size_t)b * T * H + h) * DK + (size_t)(valid ? tk : T - 1) * tokK + chh;
    };

    // Persistent: the workgroup walks items blockIdx.x, + gridDim.x, ...; the key-side
    // inputs of the next item are loaded while the current one is in its products.
    KeyRaw4<DK / 2, BF16, GL, SG> raw;
    {
        bool v0;
        const size_t row0 = item_row(blockIdx.x < nitems ? blockIdx.x : 0, v0);
        raw.issue(a.q, a.k, a.la, a.bg, row0, g, v0, (row0 - chh) / DK, a.scalar);
    }
    for (int L = blockIdx.x; L < nitems; L += gridDim.x) {
    const int tid = threadIdx.x;
    const int wv = tid >> 6, hf = wv >> 2, w = wv & 3, l = tid & 63, r = l & 15, g = l >> 4;
    const int nkk = (w >= 2) ? 2 : 1;
    const int chh = hf * (DK / 2);
    auto ch = [&](int e) { return chh + ch4(e, g); };
    auto item_row = [&](int L, bool &valid) {
        const int c = L % NC, bh = L / NC, h = bh % H, b = bh / H;
        const int tk = c * kChunk + 16 * w + r;
        valid = tk < T;
        return ((size_t)b * T * H + h) * DK + (size_t)(valid ? tk : T - 1) * tokK + chh;
    };
    __bf16 *fac = reinterpret_cast<__bf16 *>(a.factors) + (size_t)L * factor_elems_per_chunk<DK>();
    // this item's chunk operand record, after the factors of all items
    char *rec = reinterpret_cast<char *>(a.factors) + (FWD ? 0 : (size_t)nitems * factor_elems_per_chunk<DK>() * 2) +
                (size_t)L * Rec::BYTES;

    for (int idx = tid; idx < kChunk * PA; idx += NTH) sAT[idx] = 0.f;
    {
        float qf[NEH], kf[NEH], G[NEH], bgf[NEH], gC[NEH];
        raw.unpack(qf, kf, G, bgf);
#pragma unroll
        for (int e = 0; e < NEH; ++e) G[e] *= kLog2e;
        chunk_scan<NEH, DK>(G, gC, sTot, w, r, ch);
        if (w == 0 && r == 0) {
#pragma unroll
            for (int e = 0; e < NEH; ++e) {
                const float gm = exp2_fast(gC[e]);
                sGam[ch(e)] = gm;
                reinterpret_cast<float *>(rec + Rec::oGam)[ch(e)] = gm;
            }
        }
        if (!FWD) {
#pragma unroll
            for (int e = 0; e < NEH; e += 4)
                *reinterpret_cast<f32x4 *>(rec + Rec::oG + (size_t)(tid * NEH + e) * 4) =
                    f32x4{G[e], G[e + 1], G[e + 2], G[e + 3]};
        }
#pragma unroll
        for (int mm = 0; mm < NMH; ++mm) {
            f32x4 et, qt, kt;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * mm + i;
                const float eg = exp2_fast(G[e]), eng = exp2_fast(-G[e]);
                et[i] = bgf[e] * kf[e] * eg;
                qt[i] = qf[e] * eg;
                kt[i] = kf[e] * eng;
            }
            const int o = (16 * w + r) * PK + chh + 16 * mm + 4 * g;
            const Split4 se = split4(et), sq = split4(qt), sk = split4(kt);
            *reinterpret_cast<bf16x4 *>(&sEt[o]) = se.hi;
            *reinterpret_cast<bf16x4 *>(&sEt[RK + o]) = se.lo;
            *reinterpret_cast<bf16x4 *>(&sQt[o]) = sq.hi;
            *reinterpret_cast<bf16x4 *>(&sQt[RK + o]) = sq.lo;
            *reinterpret_cast<bf16x4 *>(&sKt[o]) = sk.hi;
            *reinterpret_cast<bf16x4 *>(&sKt[RK + o]) = sk.lo;
        }
    }
    __syncthreads();

    // ---- record: Kt, Et and Qt rows (dense pitch), P^T fragments ----
    static_assert((6 * 8 * DK) % NTH == 0, "row planes split evenly over the threads");
#pragma unroll
    for (int it = 0; it < 6 * 8 * DK / NTH; ++it) {
        const int idx = tid + NTH * it, plane = idx / (8 * DK), rem = idx % (8 * DK);
        const int row = rem / (DK / 8), c8 = 8 * (rem % (DK / 8));
        const __bf16 *src = (plane < 2 ? sKt : plane < 4 ? sEt : sQt) + (plane & 1) * RK + row * PK + c8;
        if (!(FWD && plane == 3))   // the forward sweep reads the hi plane of Et only
            *reinterpret_cast<uint4 *>(rec + Rec::oKt + (size_t)plane * Rec::PLANE + (size_t)(row * DK + c8) * 2) =
                *reinterpret_cast<const uint4 *>(src);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        if (!FWD && (mt & 1) == hf) {   // every tile is written (zero for mt < w): readers load all four
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (mt >= w) {
#pragma unroll
                for (int j = 0; j < NKS; ++j)
                    acc = mfma32x3(row_frag4<PK>(sQt, sQt + RK, 16 * mt + r, j, g),
                                   row_frag4<PK>(sKt, sKt + RK, 16 * w + r, j, g), acc);
                // lane holds P[16mt + 4g + i][16w + r]; the query reads the updated state: key <= query
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (!(16 * w + r <= 16 * mt + 4 * g + i)) acc[i] = 0.f;
            }
            const Split4 sp = split4(acc);
            bf16x8 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[i] = sp.hi[i];
                o[4 + i] = sp.lo[i];
            }
            *reinterpret_cast<bf16x8 *>(rec + Rec::oPt + (size_t)((4 * w + mt) * 64 + l) * 16) = o;
        }
    }

    {
        // the next item's key-side inputs, issued after this item's row stores: issued at the
        // top of the item they would queue behind the previous item's factor stores
        const int Ln = L + (int)gridDim.x < nitems ? L + (int)gridDim.x : L;
        bool vn;
        const size_t rown = item_row(Ln, vn);
        raw.issue(a.q, a.k, a.la, a.bg, rown, g, vn, (rown - chh) / DK, a.scalar);
    }

    // ---- A (shared out between the halves) and the rows of P of query block w ----
    Split4 Pf[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        if (mt <= w && (mt & 1) == hf) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                const Split8 kf = row_frag4<PK>(sKt, sKt + RK, 16 * mt + r, j, g);
                const Split8 ef = row_frag4<PK>(sEt, sEt + RK, 16 * w + r, j, g);
                acc = mfma32x3(kf, ef, acc);
            }
            // lane holds A[16w + r][16mt + 4g + i]
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (!(16 * mt + 4 * g + i < 16 * w + r)) acc[i] = 0.f;
            *reinterpret_cast<f32x4 *>(&sAT[(16 * w + r) * PA + 16 * mt + 4 * g]) = acc;
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (mt <= w) {
#pragma unroll
            for (int j = 0; j < NKS; ++j)
                acc = mfma32x3(row_frag4<PK>(sKt, sKt + RK, 16 * mt + r, j, g),
                               row_frag4<PK>(sQt, sQt + RK, 16 * w + r, j, g), acc);
            // lane holds P[16w + r][16mt + 4g + i]; the query reads the updated state: key <= query
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (!(16 * mt + 4 * g + i <= 16 * w + r)) acc[i] = 0.f;
        }
        Pf[mt] = split4(acc);
        if (hf == 0) {
            // record: P fragment of tile (query block w, key block mt), zero for mt > w
            bf16x8 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o[i] = Pf[mt].hi[i];
                o[4 + i] = Pf[mt].lo[i];
            }
            *reinterpret_cast<bf16x8 *>(rec + Rec::oP + (size_t)((4 * w + mt) * 64 + l) * 16) = o;
        }
    }
    __syncthreads();
    solve_T_inplace<PA>(sAT, w, r, g, hf == 0);   // ends with a barrier
    {
        // record: T as split bf16 [row][col], one thread per 8 elements
        static_assert(NTH == 8 * kChunk, "one thread per 8 elements of T");
        const int row = tid >> 3, c8 = 8 * (tid & 7);
        const Split8 ts = split8v(*reinterpret_cast<const f32x4 *>(&sAT[row * PA + c8]),
                                  *reinterpret_cast<const f32x4 *>(&sAT[row * PA + c8 + 4]));
        *reinterpret_cast<bf16x8 *>(rec + Rec::oT + (size_t)(row * kChunk + c8) * 2) = ts.hi;
        *reinterpret_cast<bf16x8 *>(rec + Rec::oT + (size_t)(kChunk * kChunk + row * kChunk + c8) * 2) = ts.lo;
    }
    if (FWD) {
        __syncthreads();   // the next item overwrites the LDS this one still reads
        continue;
    }

    // ---- W = T Et: tiles (token block w, channel blocks of half hf) ----
    f32x4 Wt[NMH];
#pragma unroll
    for (int aa = 0; aa < NMH; ++aa) {
        const int am = NMH * hf + aa;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk < nkk) {
                const float *trow = &sAT[(16 * w + r) * PA + 32 * kk];
                const Split8 tf = split8v(*reinterpret_cast<const f32x4 *>(trow + 4 * g),
                                          *reinterpret_cast<const f32x4 *>(trow + 16 + 4 * g));
                acc = mfma32x3(tf, frag_tr<PK>(sEt, sEt + RK, 32 * kk, 16 * am, r, g), acc);
            }
        }
        Wt[aa] = acc;   // lane holds W[16w + 4g + i][16am + r]
    }
    __syncthreads();    // the Et rows and the decay totals are dead: W^T goes over them
#pragma unroll
    for (int aa = 0; aa < NMH; ++aa) {
        const int am = NMH * hf + aa;
        const Split4 sw = split4(Wt[aa]);
        *reinterpret_cast<bf16x4 *>(&sWT[(16 * am + r) * PT + 16 * w + 4 * g]) = sw.hi;
        *reinterpret_cast<bf16x4 *>(&sWT[DK * PT + (16 * am + r) * PT + 16 * w + 4 * g]) = sw.lo;
    }
    __syncthreads();

    // ---- Q2 = Qt - P W: tiles (token block w, channel blocks of half hf), stored as Q2^T ----
#pragma unroll
    for (int aa = 0; aa < NMH; ++aa) {
        const int am = NMH * hf + aa;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk < nkk) {
                const __bf16 *wh = &sWT[(16 * am + r) * PT + 32 * kk], *wl = wh + DK * PT;
                acc = mfma32x3(join(Pf[2 * kk], Pf[2 * kk + 1]),
                               frag_2x4(wh + 4 * g, wh + 16 + 4 * g, wl + 4 * g, wl + 16 + 4 * g), acc);
            }
        }
        // lane holds (P W)[16w + 4g + i][16am + r] = (W^T P^T)[16am + r][16w + 4g + i]
        f32x4 q2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int o = (16 * w + 4 * g + i) * PK + 16 * am + r;
            q2[i] = ((float)sQt[o] + (float)sQt[RK + o]) - acc[i];
        }
        store_frag_tile(fac + (size_t)(NM * NM + am * 4 + w) * kFragTile, l, q2);
    }

    // ---- R = (I - W^T Kt) diag(gamma), tile (row block am, column block bm) ----
    for (int t = wv; t < NM * NM; t += NTH / 64) {
        const int bm = t / NM, am = t % NM;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const __bf16 *wh = &sWT[(16 * am + r) * PT + 32 * kk], *wl = wh + DK * PT;
            acc = mfma32x3(frag_tr<PK>(sKt, sKt + RK, 32 * kk, 16 * bm, r, g),
                           frag_2x4(wh + 4 * g, wh + 16 + 4 * g, wl + 4 * g, wl + 16 + 4 * g), acc);
        }
        // lane holds (Kt^T W)[16bm + 4g + i][16am + r] = (W^T Kt)[16am + r][16bm + 4g + i]
        f32x4 rt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = 16 * bm + 4 * g + i, rr = 16 * am + r;
            rt[i] = sGam[cc] * ((cc == rr ? 1.f : 0.f) - acc[i]);
        }
        store_frag_tile(fac + (size_t)(am * NM + bm) * kFragTile, l, rt);
    }
    __syncthreads();   // the next item overwrites the LDS this one still reads
    }
}

// ---------------------------------------------------------------------------
// reverse sweep kernel (body in gdn2_rsweep.h)
// ---------------------------------------------------------------------------
template <int DK, int VT>
__global__ __launch_bounds__((ReverseCfg<DK, VT>::NTH), (ReverseCfg<DK, VT>::WG_PER_CU)) void bwd_reverse_kernel(
    BwdArgs a) {
    using Lds = RevLds<DK, VT>;
    __shared__ __align__(16) __bf16 sD0[Lds::D], sD1[Lds::D], sO0[Lds::O], sO1[Lds::O];
    bwd_reverse_body<DK, VT>(a, xcd_swizzle(blockIdx.x, gridDim.x), sD0, sD1, sO0, sO1);
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
size_t factor_buffer_bytes(long items, int dk) {
    switch (dk) {
        case 32: return (size_t)items * (factor_elems_per_chunk<32>() * 2 + ChunkRecord<32>::BYTES);
        case 64: return (size_t)items * (factor_elems_per_chunk<64>() * 2 + ChunkRecord<64>::BYTES);
        case 128: return (size_t)items * (factor_elems_per_chunk<128>() * 2 + ChunkRecord<128>::BYTES);
        default: return 0;
    }
}

size_t record_buffer_bytes(long items, int dk) {
    switch (dk) {
        case 32: return (size_t)items * ChunkRecord<32>::BYTES;
        case 64: return (size_t)items * ChunkRecord<64>::BYTES;
        case 128: return (size_t)items * ChunkRecord<128>::BYTES;
        default: return 0;
    }
}

template <int DK, bool BF16, bool GL, bool SG, bool FWD>
static hipError_t factors_t(const BwdArgs &a, hipStream_t st) {
    const long items = (long)a.B * a.H * ((a.T + kChunk - 1) / kChunk);
    // one persistent workgroup per CU (the kernel's LDS allows no second one)
    const long grid = items < cu_count() ? items : cu_count();
    hipLaunchKernelGGL((bwd_factors_kernel<DK, BF16, GL, SG, FWD>), dim3((unsigned)grid), dim3(kChunkThreads), 0, st,
                       a);
    return hipGetLastError();
}

template <bool BF16, bool GL, bool SG, bool FWD>
static hipError_t factors_dk(const BwdArgs &a, int dk, hipStream_t st) {
    switch (dk) {
        case 32: return factors_t<32, BF16, GL, SG, FWD>(a, st);
        case 64: return factors_t<64, BF16, GL, SG, FWD>(a, st);
        case 128: return factors_t<128, BF16, GL, SG, FWD>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool FWD>
static hipError_t factors_any(const BwdArgs &a, int dk, bool bf16, bool gl, bool sg, hipStream_t st) {
    if (gl && sg) return hipErrorInvalidValue;
    if (gl) return bf16 ? factors_dk<true, true, false, FWD>(a, dk, st) : hipErrorInvalidValue;
    if (sg) return bf16 ? factors_dk<true, false, true, FWD>(a, dk, st) : hipErrorInvalidValue;
    return bf16 ? factors_dk<true, false, false, FWD>(a, dk, st) : factors_dk<false, false, false, FWD>(a, dk, st);
}

hipError_t launch_bwd_factors(const BwdArgs &a, int dk, bool bf16, bool gl, bool sg, hipStream_t st) {
    return factors_any<false>(a, dk, bf16, gl, sg, st);
}

hipError_t launch_fwd_records(const BwdArgs &a, int dk, bool bf16, bool gl, bool sg, hipStream_t st) {
    return factors_any<true>(a, dk, bf16, gl, sg, st);
}

template <int DK, int VT>
static hipError_t reverse_t(const BwdArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((bwd_reverse_kernel<DK, VT>), dim3((unsigned)(a.B * a.H * (a.DV / VT))),
                       dim3(ReverseCfg<DK, VT>::NTH), 0, st, a);
    return hipGetLastError();
}

// 64-column tiles when they still give every CU a workgroup; else 32 (two workgroups per CU),
// or 16 when even 16-column tiles leave CUs without one.  A sequential chain is paced by its
// per-chunk latency, which narrower tiles shorten: B1 T16K H16 takes about 1.35, 0.78 and
// 0.57 ms at 64, 32 and 16 columns.  At B4 T4K H16 the 32-column tiles beat the 16-column
// ones (0.24 against 0.30 ms); prefetching the next chunk's factors gains nothing at 32 columns.
template <int DK>
static hipError_t reverse_vt(const BwdArgs &a, hipStream_t st) {
    const long bh = (long)a.B * a.H;
    const int cus = cu_count();
    if (a.DV >= 64 && bh * (a.DV / 64) >= cus) return reverse_t<DK, 64>(a, st);
    if (bh * (a.DV / 16) <= cus) return reverse_t<DK, 16>(a, st);
    return reverse_t<DK, 32>(a, st);
}

hipError_t launch_bwd_reverse(const BwdArgs &a, int dk, hipStream_t st) {
    if (a.DV % 32 != 0) return hipErrorInvalidValue;
    switch (dk) {
        case 32: return reverse_vt<32>(a, st);
        case 64: return reverse_vt<64>(a, st);
        case 128: return reverse_vt<128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn2
