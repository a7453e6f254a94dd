// gdn2_reverse.hip -- reverse sweep of the gate-aware backward on gfx950: per-chunk
// adjoint factors (chunk-parallel), then the chunk-to-chunk recurrence of the state
// gradient (sequential over chunks).
//
// Chunk notation of gdn2_sweep.hip (blog on Gated DeltaNet-2, section "Token path and
// parallel training"): start state S, end state S' = diag(gamma) S + Kh^T U,
// U = T X, X = Z - Et S, O = Qt S + P U.  The adjoint of one chunk gives for the
// gradient of its start state
//     dS = Qt^T dO + diag(gamma) dS' - Et^T dX,   dX = T^T (P^T dO + Kh dS').
// With W = T Et (the WY factor of the erase keys) this is
//     dS = R dS' + Q2^T dO,   R = diag(gamma) - W^T Kh,   Q2 = Qt - P W,
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
#include "gdn2_exact.h"
#include "gdn2_kernels.h"
#include "gdn2_rsweep.h"

namespace gdn2 {

#ifdef GDN2_STAMPS
// stamps of the fast pass of the factor kernel: 8 per (item, wave), see bwd_factors_kernel
static __device__ unsigned long long *g_factor_stamps;
#endif

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
// that the forward sweep reads, without the adjoint factors, P^T or the decay offsets (and
// without the Et lo plane for bf16 q/k/v, whose sweep reads the hi plane only).
// EX: the exact pass.  The fast pass (EX false) forms A = Et Kt^T and P = Qt Kt^T from the
// factorised rows Kt = k exp(-G), and flags every chunk in which some channel's decay gamma
// is below kGamMin, where exp(-G) may leave fp32 range; the exact pass then redoes only the
// flagged chunks, with A and P from the pairwise decays (gdn2_exact.h) and R = diag(gamma) -
// W^T Kh.  The record's Kh, Et, Qt rows, gamma and decay offsets are the same in both passes.
template <int DK, bool BF16, bool GL, bool SG, bool FWD, bool EX>
__global__ __launch_bounds__(kChunkThreads, 1) void bwd_factors_kernel(BwdArgs a) {
    GDN2_POISON_LDS();
    constexpr int NTH = kChunkThreads;
    constexpr int NM = DK / 16, NKS = DK / 32, NMH = DK / 32, NEH = 4 * NMH;
    constexpr int PK = DK + 8, PT = kChunk + 8, PA = kChunk + 4;
    constexpr int RK = kChunk * PK;
    using Rec = ChunkRecord<DK>;
    // LDS (bytes): Kt (Kh in the exact pass), Et, Qt rows [token][channel] (hi, lo); the decay
    // totals after the Et rows; W^T [channel][token] (hi, lo) later over the Et rows and the
    // totals; A then T (fp32); gamma per channel; in the exact pass the channel slices (then
    // P, fp32) and the work list.
    constexpr int B_ROWS = 2 * RK * 2, B_WT = 2 * DK * PT * 2, B_TOT = 4 * DK * 4;
    constexpr int oKt = 0, oEt = oKt + B_ROWS, oTot = oEt + B_ROWS;
    constexpr int oQt0 = (oTot + B_TOT > oEt + B_WT) ? oTot + B_TOT : oEt + B_WT;
    constexpr int oQt = (oQt0 + 15) / 16 * 16;
    constexpr int oAT = oQt + B_ROWS, oGam = oAT + kChunk * PA * 4;
    constexpr int oEx = oGam + DK * 4, B_EX = EX ? kSliceFloats * 4 : 0;
    constexpr int oList = oEx + B_EX, B_LIST = EX ? (NTH + 4) * 4 : 0;
    constexpr int oCnt = oList + B_LIST;                // tile-pair queue of the forward records
    constexpr int oPf = oCnt + 16;                      // their P fragment tiles, until stored
    constexpr int SMEM = oPf + (FWD && !EX && BF16 ? Rec::B_FR : 0);
    static_assert(SMEM <= 160 * 1024, "LDS budget of a CU");
    static_assert(kChunk * PA <= kSliceFloats, "P fits over the slices");

    __shared__ __align__(16) char smem[SMEM];
    __bf16 *sKt = reinterpret_cast<__bf16 *>(smem + oKt), *sEt = reinterpret_cast<__bf16 *>(smem + oEt);
    __bf16 *sQt = reinterpret_cast<__bf16 *>(smem + oQt), *sWT = reinterpret_cast<__bf16 *>(smem + oEt);
    float *sTot = reinterpret_cast<float *>(smem + oTot), *sAT = reinterpret_cast<float *>(smem + oAT);
    float *sGam = reinterpret_cast<float *>(smem + oGam);
    float *sEx = reinterpret_cast<float *>(smem + oEx);
    int *sList = reinterpret_cast<int *>(smem + oList);
    int *sCnt = reinterpret_cast<int *>(smem + oCnt);
    char *sPf = smem + oPf;
    // Forward records (FWD, fast pass, bf16 inputs): A and P come from a queue of the ten (query
    // block, key block) pairs that any wave takes, with no global access in that phase; the row
    // planes and the P tiles are stored by the half that the solve leaves idle, during the solve.
    // (With fp32 inputs the next item's inputs take too many registers across the solve for it.)
    constexpr bool QUEUE = FWD && !EX && BF16;

    const int NC = (a.T + kChunk - 1) / kChunk;
    const int T = a.T, H = a.H;
    const int nitems = a.B * H * NC;                    // item L = (b * H + h) * NC + c
    const size_t tokK = (size_t)H * DK;
    char *const recs = reinterpret_cast<char *>(a.factors) + (FWD ? 0 : (size_t)nitems * factor_elems_per_chunk<DK>() * 2);
    int *const flags = reinterpret_cast<int *>(recs + record_flags_offset<DK>(nitems));
    // this lane's token row (channel 0 of its half) in item L, and whether the token exists
    auto item_row = [&](int L, bool &valid) {
        const int tid = threadIdx.x, w = (tid >> 6) & 3, r = tid & 15, chh = (tid >> 8) * (DK / 2);
        const int c = L % NC, bh = L / NC, h = bh % H, b = bh / H;
        const int tk = c * kChunk + 16 * w + r;
        valid = tk < T;
        return ((size_t)b * T * H + h) * DK + (size_t)(valid ? tk : T - 1) * tokK + chh;
    };

    KeyRaw4<DK / 2, BF16, GL, SG> raw;
    auto issue = [&](int L) {
        bool v;
        const size_t row = item_row(L, v);
        raw.issue(a.q, a.k, a.la, a.bg, row, (threadIdx.x >> 4) & 3, v, (row - (threadIdx.x >> 8) * (DK / 2)) / DK,
                  a.scalar);
    };

    // Work list.  Fast pass: persistent, items blockIdx.x, + gridDim.x, ...; the key-side inputs
    // of the next item (Ln) are loaded while the current one is in its products.  Exact pass: the
    // flagged items of the same share, gathered NTH candidates at a time, each loading its
    // inputs at its start.
    const int nmine = blockIdx.x < (unsigned)nitems ? (nitems - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
    if (!EX) issue(blockIdx.x < (unsigned)nitems ? blockIdx.x : 0);
    if (!EX && a.zero) {
        // the area a launch that follows needs cleared (vector stores, grid-stride)
        uint4 *z = reinterpret_cast<uint4 *>(a.zero);
        for (long i = (long)blockIdx.x * NTH + threadIdx.x; i < a.zero16; i += (long)gridDim.x * NTH)
            z[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    for (long base = blockIdx.x; base < (EX ? nitems : (long)blockIdx.x + 1); base += (long)gridDim.x * NTH) {
    const int nwork = EX ? gather_flagged<NTH>(flags, nitems, base, gridDim.x, sList, sList + NTH) : nmine;
    for (int wi = 0; wi < nwork; ++wi) {
    const int L = EX ? sList[wi] : (int)blockIdx.x + wi * (int)gridDim.x;
    const int Ln = EX ? L : (L + (int)gridDim.x < nitems ? L + (int)gridDim.x : L);
    if (EX) issue(L);
    const int tid = threadIdx.x;
    const int wv = tid >> 6, hf = wv >> 2, w = wv & 3, l = tid & 63, r = l & 15, g = l >> 4;
    const int nkk = (w >= 2) ? 2 : 1;
    const int chh = hf * (DK / 2);
    auto ch = [&](int e) { return chh + ch4(e, g); };
#ifdef GDN2_STAMPS
    // element phase 0-1, record rows 1-2, A and P 2-3, the solve 3-4, T 4-5, W, Q2, R 5-6; in
    // the queued forward records, 2-6 issues the next item's loads and 6-3 is A and P
    unsigned long long *stp = !EX && g_factor_stamps ? g_factor_stamps + ((size_t)L * 8 + wv) * 8 : nullptr;
#else
    unsigned long long *stp = nullptr;
#endif
    (void)stp;
    GDN2_STAMP_REGS;
    GDN2_STAMP(stp, 0);
    __bf16 *fac = reinterpret_cast<__bf16 *>(a.factors) + (size_t)L * factor_elems_per_chunk<DK>();
    char *rec = recs + (size_t)L * Rec::BYTES;

    for (int idx = tid; idx < kChunk * PA; idx += NTH) sAT[idx] = 0.f;
    if (QUEUE && tid == 0) *sCnt = 0;
    float qf[NEH], kf[NEH], G[NEH], bgf[NEH], ev[NEH];   // ev (e = b k) and G kept for the exact products
    int unsafe;
    {
        float gC[NEH];
        raw.unpack(qf, kf, G, bgf);
#pragma unroll
        for (int e = 0; e < NEH; ++e) G[e] *= kLog2e;
        chunk_scan<NEH, DK>(G, gC, sTot, w, r, ch);
        bool strong = false;
#pragma unroll
        for (int e = 0; e < NEH; ++e) strong |= exp2_fast(gC[e]) < kGamMin;
        if (w == 0 && r == 0) {
#pragma unroll
            for (int e = 0; e < NEH; ++e) {
                const float gm = exp2_fast(gC[e]);
                sGam[ch(e)] = gm;
                reinterpret_cast<float *>(rec + Rec::oGam)[ch(e)] = gm;
            }
        }
        // the scan's cross-block offsets, from which the chunk-gradient kernel forms G again
        if (!FWD) chunk_scan_offsets<DK, NTH>(sTot, reinterpret_cast<float *>(rec + Rec::oPre), tid);
#pragma unroll
        for (int mm = 0; mm < NMH; ++mm) {
            f32x4 et, qt, kt;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * mm + i;
                const float eg = exp2_fast(G[e]);
                ev[e] = bgf[e] * kf[e];
                et[i] = ev[e] * eg;
                qt[i] = qf[e] * eg;
                // the exact pass stages Kh = k exp(g_C - G) (its Kt may leave fp32 range)
                kt[i] = kf[e] * exp2_fast(EX ? gC[e] - G[e] : -G[e]);
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
        unsafe = __syncthreads_or(strong);
    }
    if (!EX && tid == 0) flags[L] = unsafe ? 1 : 0;
    GDN2_STAMP(stp, 1);

    // ---- record: Kh rows (Kt diag(gamma) from the fast pass's Kt rows; the exact pass's LDS
    // rows are Kh already), one thread per 8 channels of a row (hi and lo) ----
    auto kh_group = [&](int idx) {
        const int row = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
        Split8 kh = frag_8(&sKt[row * PK + c8], &sKt[RK + row * PK + c8]);
        if (!EX) {
            const f32x4 g0 = *reinterpret_cast<const f32x4 *>(&sGam[c8]);
            const f32x4 g1 = *reinterpret_cast<const f32x4 *>(&sGam[c8 + 4]);
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = ((float)kh.hi[i] + (float)kh.lo[i]) * (i < 4 ? g0[i] : g1[i - 4]);
            kh = split8(x);
        }
        const size_t ro = (size_t)(row * DK + c8) * 2;
        *reinterpret_cast<bf16x8 *>(rec + Rec::oKh + ro) = kh.hi;
        *reinterpret_cast<bf16x8 *>(rec + Rec::oKh + Rec::PLANE + ro) = kh.lo;
    };
    // ---- record: Et and Qt rows (dense pitch); plane 2 + k: Et hi, Et lo, Qt hi, Qt lo ----
    auto eq_piece = [&](int plane, int rem) {
        const int row = rem / (DK / 8), c8 = 8 * (rem % (DK / 8));
        const __bf16 *src = (plane < 4 ? sEt : sQt) + (plane & 1) * RK + row * PK + c8;
        *reinterpret_cast<uint4 *>(rec + Rec::oKh + (size_t)plane * Rec::PLANE + (size_t)(row * DK + c8) * 2) =
            *reinterpret_cast<const uint4 *>(src);
    };
    if constexpr (!QUEUE) {
#pragma unroll
        for (int it = 0; it < (8 * DK + NTH - 1) / NTH; ++it) {
            const int idx = tid + NTH * it, row = idx / (DK / 8), c8 = 8 * (idx % (DK / 8));
            if (idx >= 8 * DK) break;
            Split8 kh = frag_8(&sKt[row * PK + c8], &sKt[RK + row * PK + c8]);
            if (!EX) {
                const f32x4 g0 = *reinterpret_cast<const f32x4 *>(&sGam[c8]);
                const f32x4 g1 = *reinterpret_cast<const f32x4 *>(&sGam[c8 + 4]);
                float x[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = ((float)kh.hi[i] + (float)kh.lo[i]) * (i < 4 ? g0[i] : g1[i - 4]);
                kh = split8(x);
            }
            const size_t ro = (size_t)(row * DK + c8) * 2;
            *reinterpret_cast<bf16x8 *>(rec + Rec::oKh + ro) = kh.hi;
            *reinterpret_cast<bf16x8 *>(rec + Rec::oKh + Rec::PLANE + ro) = kh.lo;
        }
        static_assert((4 * 8 * DK) % NTH == 0, "row planes split evenly over the threads");
#pragma unroll
        for (int it = 0; it < 4 * 8 * DK / NTH; ++it) {
            const int idx = tid + NTH * it, plane = 2 + idx / (8 * DK), rem = idx % (8 * DK);
            const int row = rem / (DK / 8), c8 = 8 * (rem % (DK / 8));
            const __bf16 *src = (plane < 4 ? sEt : sQt) + (plane & 1) * RK + row * PK + c8;
            if (!(FWD && BF16 && plane == 3))   // the bf16 forward sweep reads the hi plane of Et only
                *reinterpret_cast<uint4 *>(rec + Rec::oKh + (size_t)plane * Rec::PLANE + (size_t)(row * DK + c8) * 2) =
                    *reinterpret_cast<const uint4 *>(src);
        }
    }
    // The same stores in the forward records, by the waves of half 1 during the solve: part k of
    // four before its barrier k.  Items: the 8 DK Kh groups, the pieces of the Et and Qt planes
    // the sweep reads (the bf16 sweep reads the hi plane of Et only), then the 16 P tiles' lane
    // pieces (zero above the diagonal blocks, the others from LDS).
    auto row_stores = [&](int k) {
        constexpr int NG = 8 * DK, NPL = BF16 ? 3 : 4, NROW = NG * (1 + NPL), NITEM = NROW + 16 * 64;
        constexpr int NH = NTH / 2, PER = (NITEM + 4 * NH - 1) / (4 * NH);
        const int t1 = (int)threadIdx.x - NH;
#pragma unroll
        for (int it = 0; it < PER; ++it) {
            const int idx = (it * 4 + k) * NH + t1;
            if (idx < NG) {
                kh_group(idx);
            } else if (idx < NROW) {
                const int p = idx - NG, kq = p / NG;
                eq_piece(2 + kq + (NPL == 3 && kq >= 1 ? 1 : 0), p % NG);
            } else if (idx < NITEM) {
                const int pc = idx - NROW, tile = pc >> 6;   // tile 4 qb + kb
                const uint4 v = (tile & 3) > (tile >> 2) ? uint4{0u, 0u, 0u, 0u}
                                                         : *reinterpret_cast<const uint4 *>(sPf + (size_t)pc * 16);
                *reinterpret_cast<uint4 *>(rec + Rec::oP + (size_t)pc * 16) = v;
            }
            // one item's registers at a time (the next item's inputs are live across the solve)
            asm volatile("" ::: "memory");
        }
    };

    Split4 Pf[4];
    GDN2_STAMP(stp, 2);
    if constexpr (EX) {
        // ---- A and P with the exact pairwise decays; P fp32 over the slices ----
        float *sP = sEx;
        exact_AP<NEH, PA>(sEx, sAT, sP, hf, w, r, g, ev, qf, kf, G);
        __syncthreads();
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            // lane holds P[16w + r][16mt + 4g + i] (zero for mt > w)
            const f32x4 pv = *reinterpret_cast<const f32x4 *>(&sP[(16 * w + r) * PA + 16 * mt + 4 * g]);
            Pf[mt] = split4(pv);
            if (hf == 0) {
                bf16x8 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = Pf[mt].hi[i];
                    o[4 + i] = Pf[mt].lo[i];
                }
                *reinterpret_cast<bf16x8 *>(rec + Rec::oP + (size_t)((4 * w + mt) * 64 + l) * 16) = o;
            }
            if (!FWD && (mt & 1) == hf) {
                // P^T fragment: lane holds P[16mt + 4g + i][16w + r] (zero for mt < w)
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = sP[(16 * mt + 4 * g + i) * PA + 16 * w + r];
                store_frag_tile(reinterpret_cast<__bf16 *>(rec + Rec::oPt) + (size_t)((4 * w + mt) * 64) * 8, l, acc);
            }
        }
        __syncthreads();
    } else if constexpr (QUEUE) {
        // the next item's key-side inputs first.  Issuing them waits for room in the memory queue
        // (the previous item's row stores are still draining); the waves that get through first
        // take the pairs meanwhile, so the products run under that wait.  (Issued after the
        // products instead, the item took 27.4K cycles against 23.7K.)
        issue(Ln);
        GDN2_STAMP(stp, 6);   // (slot 6 is free in the forward records)
        // ---- A and P from the pair queue: pair p = (query block qb, key block kb <= qb); its
        // A and P tiles share the Kt fragment and run as two interleaved MFMA chains ----
        ap_pair_queue<DK, PK, PA>(sKt, sEt, sQt, sAT, sPf, sCnt, l, r, g);
        __syncthreads();
    } else {
        // ---- record: P^T fragments ----
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
                store_frag_tile(reinterpret_cast<__bf16 *>(rec + Rec::oPt) + (size_t)((4 * w + mt) * 64) * 8, l, acc);
            }
        }

        // the next item's key-side inputs, issued after this item's row stores: issued at the
        // top of the item they would queue behind the previous item's factor stores
        issue(Ln);

        // ---- A (shared out between the halves) and the rows of P of query block w ----
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
    }
    GDN2_STAMP(stp, 3);
    if constexpr (QUEUE)
        solve_T_inplace<PA>(sAT, w, r, g, hf == 0, row_stores);   // ends with a barrier
    else
        solve_T_inplace<PA>(sAT, w, r, g, hf == 0);
    GDN2_STAMP(stp, 4);
    {
        // record: T as split bf16 [row][col], one thread per 8 elements
        static_assert(NTH == 8 * kChunk, "one thread per 8 elements of T");
        const int row = tid >> 3, c8 = 8 * (tid & 7);
        const Split8 ts = split8v(*reinterpret_cast<const f32x4 *>(&sAT[row * PA + c8]),
                                  *reinterpret_cast<const f32x4 *>(&sAT[row * PA + c8 + 4]));
        *reinterpret_cast<bf16x8 *>(rec + Rec::oT + (size_t)(row * kChunk + c8) * 2) = ts.hi;
        *reinterpret_cast<bf16x8 *>(rec + Rec::oT + (size_t)(kChunk * kChunk + row * kChunk + c8) * 2) = ts.lo;
    }
    GDN2_STAMP(stp, 5);
    if (FWD) {
        GDN2_STAMP_FLUSH(stp);
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

    // ---- R = (I - W^T Kt) diag(gamma) = diag(gamma) - W^T Kh, tile (row block am, column block bm) ----
    for (int t = wv; t < NM * NM; t += NTH / 64) {
        const int bm = t / NM, am = t % NM;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const __bf16 *wh = &sWT[(16 * am + r) * PT + 32 * kk], *wl = wh + DK * PT;
            acc = mfma32x3(frag_tr<PK>(sKt, sKt + RK, 32 * kk, 16 * bm, r, g),
                           frag_2x4(wh + 4 * g, wh + 16 + 4 * g, wl + 4 * g, wl + 16 + 4 * g), acc);
        }
        // lane holds (K^T W)[16bm + 4g + i][16am + r] = (W^T K)[16am + r][16bm + 4g + i], K = Kt or Kh
        f32x4 rt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = 16 * bm + 4 * g + i, rr = 16 * am + r;
            rt[i] = EX ? sGam[cc] * (cc == rr ? 1.f : 0.f) - acc[i] : sGam[cc] * ((cc == rr ? 1.f : 0.f) - acc[i]);
        }
        store_frag_tile(fac + (size_t)(am * NM + bm) * kFragTile, l, rt);
    }
    GDN2_STAMP(stp, 6);
    GDN2_STAMP_FLUSH(stp);
    __syncthreads();   // the next item overwrites the LDS this one still reads
    }
    }
}

// ---------------------------------------------------------------------------
// reverse sweep kernel (body in gdn2_rsweep.h)
// ---------------------------------------------------------------------------
template <int DK, int VT>
__global__ __launch_bounds__((ReverseCfg<DK, VT>::NTH), (ReverseCfg<DK, VT>::WG_PER_CU)) void bwd_reverse_kernel(
    BwdArgs a) {
    GDN2_POISON_LDS();
    using Lds = RevLds<DK, VT>;
    __shared__ __align__(16) __bf16 sD0[Lds::D], sD1[Lds::D], sO0[Lds::O], sO1[Lds::O];
    bwd_reverse_body<DK, VT>(a, xcd_swizzle(blockIdx.x, gridDim.x), sD0, sD1, sO0, sO1);
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
#ifdef GDN2_STAMPS
// the instrumented build only: where the factor kernel's fast pass writes its phase stamps
// (8 per item and wave; nullptr = none)
extern "C" int gdn2_stamps_factors(void *buf) {
    unsigned long long *p = static_cast<unsigned long long *>(buf);
    return hipMemcpyToSymbol(HIP_SYMBOL(g_factor_stamps), &p, sizeof(p)) == hipSuccess ? 0 : 4;
}
#endif

size_t record_buffer_bytes(long items, int dk) {
    switch (dk) {
        case 32: return (size_t)items * ChunkRecord<32>::BYTES + record_flags_bytes(items);
        case 64: return (size_t)items * ChunkRecord<64>::BYTES + record_flags_bytes(items);
        case 128: return (size_t)items * ChunkRecord<128>::BYTES + record_flags_bytes(items);
        default: return 0;
    }
}

size_t factor_buffer_bytes(long items, int dk) {
    switch (dk) {
        case 32: return (size_t)items * factor_elems_per_chunk<32>() * 2 + record_buffer_bytes(items, 32);
        case 64: return (size_t)items * factor_elems_per_chunk<64>() * 2 + record_buffer_bytes(items, 64);
        case 128: return (size_t)items * factor_elems_per_chunk<128>() * 2 + record_buffer_bytes(items, 128);
        default: return 0;
    }
}

// The fast pass over every chunk, then the exact pass over the chunks it flagged (a workgroup
// whose share holds no flagged chunk reads its flags and ends).
template <int DK, bool BF16, bool GL, bool SG, bool FWD>
static hipError_t factors_t(const BwdArgs &a, hipStream_t st) {
    const long items = (long)a.B * a.H * ((a.T + kChunk - 1) / kChunk);
    // one persistent workgroup per CU (the kernel's LDS allows no second one)
    const long grid = items < cu_count() ? items : cu_count();
    hipLaunchKernelGGL((bwd_factors_kernel<DK, BF16, GL, SG, FWD, false>), dim3((unsigned)grid), dim3(kChunkThreads),
                       0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_factors_kernel<DK, BF16, GL, SG, FWD, true>), dim3((unsigned)grid), dim3(kChunkThreads),
                       0, st, a);
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
