// gdn2_bwd.hip -- gate-aware backward of the Gated DeltaNet-2 chunkwise-WY operator on gfx950.
//
// Source of the method: blog on Gated DeltaNet-2 (iplexlaw.co.kr), section
// "Token path and parallel training": the backward accumulates gradients with
// the already-gated keys and values (e = b*k, z = w*v) and keeps the
// chunkwise WY structure; the paper abstract (OpenAlex record) calls it the
// gate-aware backward pass.
//
// Per chunk (start state S, end-state gradient dS', notation of gdn2_sweep.hip),
// the adjoint of
//     X = Z - Et S,  U = T X,  O = Qt S + P U,  S' = diag(gamma) S + Kh^T U
// is
//     dU  = P^T dO + Kh dS'               dX = T^T dU            dZ = dX
//     dS  = Qt^T dO + diag(gamma) dS' - Et^T dX        (carried to the previous chunk)
//     dQt = dO S^T + dP Kt                dP = lower(dO U^T)
//     dEt = -dX S^T + dA Kt               dA = -strictly-lower(dX U^T)
//     dKt = dA^T Et + dP^T Qt             dKh = U dS'^T          dgamma = rowsum(dS' * S)
// followed by the element-wise chain through Et = b*k*exp(G), Qt = q*exp(G),
// Kt = k*exp(-G), Kh = k*exp(g_C - G), Z = w*v and the reverse cumulative sum
// of dG into dlog_alpha.  The record holds Kh (decay factors at most 1); the products with
// Kt = Kh diag(1/gamma) are formed as (dP Kh) diag(1/gamma), the channel factor applied to
// the accumulator.  On chunks whose decay the factor kernel flagged (some gamma below
// kGamMin, where exp(-G) leaves fp32 range) the exact pass (EX) forms the three intra-chunk
// products with the pairwise decays instead (gdn2_exact.h):
//     dq_i += sum_{j<=i} dP_ij k_j x_ij,   dE_i += sum_{j<i} dA_ij k_j x_ij,
//     dk_j += sum_{i>=j} (dA_ij e_i + dP_ij q_i) x_ij,    x_ij = exp(G_i - G_j) per channel.
//
// Launches of the backward: the forward state sweep (gdn2_fwd.hip) stores every
// chunk's start state; the reverse sweep (gdn2_reverse.hip) walks the chunks
// backwards per (batch, head, value tile) and stores each chunk's dS'; bwd_chunk_kernel
// (this file) then treats every (batch, head, chunk) independently and writes all token
// gradients.  Value columns are independent in S, dS and dS', so value tiles need no
// exchange; the key-side gradients sum over all value columns inside one
// bwd_chunk_kernel workgroup.
//
#include <type_traits>

#include "gdn2_chunk.h"
#include "gdn2_exact.h"
#include "gdn2_kernels.h"

namespace gdn2 {

#ifdef GDN2_STAMPS
// stamps of the fast pass of the chunk-gradient kernel: 8 per (item, wave), see bwd_chunk_kernel
static __device__ unsigned long long *g_chunk_stamps;
#endif

// ---------------------------------------------------------------------------
// chunk-parallel gradients of every token input
// ---------------------------------------------------------------------------

// Value-tile inputs of the chunk-gradient kernel, loaded one tile ahead into registers.
template <int DK>
struct ChunkTile {
    static constexpr int NSF = (DK * 8 + kChunkThreads - 1) / kChunkThreads;   // float4 of a state tile per thread
    f32x4 s[NSF], d[NSF];    // S and dS' (channel idx/8, columns 4*(idx%8)..+3)
    float o[4];              // dO; after the quad transpose: column tid%32, tokens 4*(tid/32)..+3
    float v[4], wg[4];       // v and w of this wave's X tile; D layout after the quad transpose
};

// Value tile j0 (32 columns) of item L = (b * H + h) * NC + c.  Addresses: a base pointer common
// to the workgroup (the item's chunk and the tile's first column) plus a 32-bit byte offset per
// lane; the offsets stay inside one chunk of one (b, h), so they fit, and the loads take the
// scalar-base + vector-offset form.
template <int DK, bool BF16, bool GL, bool SG>
__device__ __forceinline__ void chunk_load_tile(const BwdArgs &a, int NC, int L, int j0, ChunkTile<DK> &x, int tid) {
    constexpr int NTH = kChunkThreads, NSF = ChunkTile<DK>::NSF;
    constexpr unsigned ES = BF16 ? 2u : 4u, GS = GL ? 2u : 4u;
    const int T = a.T, H = a.H, DV = a.DV;
    const size_t tokV = (size_t)H * DV;
    const int w = (tid >> 6) & 3, n = tid >> 8, r = tid & 15, g = (tid >> 4) & 3;
    const int c = L % NC, bh = L / NC, h = bh % H, b = bh / H, t0 = c * kChunk;
    const size_t stoff = ((size_t)bh * NC + c) * (size_t)DK * DV;
    const size_t baseK = ((size_t)b * T * H + h) * DK;
    const size_t tokBase = ((size_t)b * T * H + h) * DV + (size_t)t0 * tokV;
    const unsigned last = (unsigned)(T - 1 - t0);   // last existing token of the chunk, from t0
    const char *sb = reinterpret_cast<const char *>(a.states + stoff + j0);
    const char *db = reinterpret_cast<const char *>(a.dstates + stoff + j0);
#pragma unroll
    for (int it = 0; it < NSF; ++it) {
        int idx = tid + NTH * it;
        idx = idx < DK * 8 ? idx : 0;
        const unsigned o = (unsigned)((idx >> 3) * DV + 4 * (idx & 7)) * 4u;
        x.s[it] = *reinterpret_cast<const f32x4 *>(sb + o);
        x.d[it] = *reinterpret_cast<const f32x4 *>(db + o);
    }
    // Wide loads: a lane reads 4 consecutive columns of one token; the 4x4 transpose inside
    // each quad of lanes, done at staging, turns that into one column of 4 tokens.
    {
        // dO: token 4 (tid / 32) + (tid % 4), columns 4 ((tid / 4) % 8) ..; after the
        // transpose: column tid % 32, tokens 4 (tid / 32) ..
        const char *ob = reinterpret_cast<const char *>(a.dO + tokBase + j0);
        const unsigned tr = min((unsigned)(4 * (tid >> 5) + (tid & 3)), last);
        const f32x4 o4 = *reinterpret_cast<const f32x4 *>(ob + (tr * (unsigned)tokV + 4u * ((tid >> 2) & 7)) * 4u);
        x.o[0] = o4[0], x.o[1] = o4[1], x.o[2] = o4[2], x.o[3] = o4[3];
    }
    // v and w of the X tile: row 16w + 4g + (r % 4), columns 16n + 4 (r / 4) ..; after the
    // transpose: rows 16w + 4g + i, column 16n + r (the D layout)
    const unsigned vr = min((unsigned)(16 * w + 4 * g + (r & 3)), last);
    const unsigned vo = vr * (unsigned)tokV + (unsigned)(16 * n + 4 * (r >> 2));
    auto load4 = [](const char *p, bool b16, float (&y)[4]) {
        if (b16) {
            typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 u = *reinterpret_cast<const u32x2 *>(p);
            y[0] = __uint_as_float(u[0] << 16), y[1] = __uint_as_float(u[0] & 0xffff0000u);
            y[2] = __uint_as_float(u[1] << 16), y[3] = __uint_as_float(u[1] & 0xffff0000u);
        } else {
            const f32x4 f = *reinterpret_cast<const f32x4 *>(p);
            y[0] = f[0], y[1] = f[1], y[2] = f[2], y[3] = f[3];
        }
    };
    load4(reinterpret_cast<const char *>(a.v) + ((tokBase + j0) + vo) * ES, BF16, x.v);
    if constexpr (SG) {
        // gates per token or per channel (decided at run time): element loads, D layout as loaded
        const bool wtok = a.scalar & kScalarWrite;
        const char *wb = reinterpret_cast<const char *>(a.wg) + (wtok ? baseK / DK + (size_t)t0 * H : tokBase + j0) * GS;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned tr = min((unsigned)(16 * w + 4 * g + i), last);
            const unsigned ow = wtok ? tr * (unsigned)H : tr * (unsigned)tokV + (unsigned)(16 * n + r);
            x.wg[i] = GL ? bf16_bits_to_float(*reinterpret_cast<const uint16_t *>(wb + ow * GS))
                         : *reinterpret_cast<const float *>(wb + ow * GS);
        }
    } else {
        load4(reinterpret_cast<const char *>(a.wg) + ((tokBase + j0) + vo) * GS, GL, x.wg);   // as stored
    }
}

// The pieces of item L's chunk operand record the chunk-gradient kernel keeps (Kh and Et row
// planes, T, P^T fragments, gamma), loaded into registers: the first half of its preparation.
template <int DK>
struct ChunkRecRegs {
    u32x4 rv[DK / 16];   // 16-byte pieces of the four row planes, thread tid + 512 it
    u32x4 th, tl;        // T hi and lo: row tid / 8, columns 8 (tid % 8) ..
    u32x4 pv[4];         // the four P^T tiles of this lane (those with mt < w hold zeros)
    float gm;            // gamma of channel tid (tid < DK)
};

template <int DK>
__device__ __forceinline__ void chunk_load_record(const char *rc, int tid, ChunkRecRegs<DK> &x) {
    using Rec = ChunkRecord<DK>;
    constexpr int NTH = kChunkThreads;
    static_assert(NTH == 8 * kChunk, "one thread per 8 elements of T");
    const int w = (tid >> 6) & 3, l = tid & 63, trow = tid >> 3, tc8 = 8 * (tid & 7);
#pragma unroll
    for (int it = 0; it < DK / 16; ++it)
        x.rv[it] = *reinterpret_cast<const u32x4 *>(rc + Rec::oKh + (size_t)(tid + NTH * it) * 16);   // Kh, Et planes
    x.th = *reinterpret_cast<const u32x4 *>(rc + Rec::oT + (size_t)(trow * kChunk + tc8) * 2);
    x.tl = *reinterpret_cast<const u32x4 *>(rc + Rec::oT + (size_t)(kChunk * kChunk + trow * kChunk + tc8) * 2);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        x.pv[mt] = *reinterpret_cast<const u32x4 *>(rc + Rec::oPt + (size_t)((4 * w + mt) * 64 + l) * 16);
    x.gm = reinterpret_cast<const float *>(rc + Rec::oGam)[tid < DK ? tid : 0];
}
// Eight waves in two halves of four.  Wave (hf, w) owns the 16 tokens 16w..16w+15 in
// both halves; for the key-side element work and the key-side gradients it owns
// channels of its half only (hf * DK/2 .. +DK/2), in the 4-group layout; on the value
// side it computes the 16x16 tiles (token block w, column block hf) of X, U, dU and dX
// of each 32-column value tile.  The operand rows Kh and Et stay in LDS for the whole
// chunk, so one workgroup takes most of a CU's LDS and the two halves give every SIMD
// two waves.
// EX: the exact pass, persistent over the chunks the factor kernel flagged; it redoes
// those chunks whole and writes all their gradients over the fast pass's.

template <int DK, bool BF16, bool GL, bool SG, bool EX>
__global__ __launch_bounds__(kChunkThreads, 1) void bwd_chunk_kernel(BwdArgs a) {
    GDN2_POISON_LDS();
    constexpr int NTH = kChunkThreads;
    constexpr int VT = 32;                       // value columns per tile
    constexpr int NKS = DK / 32;                 // 32-channel contraction steps
    constexpr int NMH = DK / 32;                 // 16-channel key tiles per half
    constexpr int NEH = 4 * NMH;                 // key elements per lane
    constexpr int PK = DK + 8, PT = kChunk + 8, PA = kChunk + 4, PS = VT + 4;   // PS: 18-bank rows, conflict-free transposed reads
    constexpr int RK = kChunk * PK;              // one [token][channel] bf16 plane
    constexpr int NSF = (DK * 8 + NTH - 1) / NTH;   // float4 of a state tile per thread
    constexpr bool FAST = BF16;
    // LDS (byte offsets).  Whole chunk: Kh and Et rows [token][channel] (hi, lo); in the
    // epilogue of the exact pass the channel slices go over them.
    // Value loop: S and dS' tiles as [channel][col]; dO, X then U, dU then -dX as
    // [col][token]; A then T (fp32).  Preparation puts the Qt rows where the value tiles go;
    // the epilogue puts Qt rows, dP^T and dA^T ([key][query]) and scratch over the value
    // tiles and T.
    constexpr int B_ROWS = 2 * RK * 2, B_ST = 2 * DK * PS * 2, B_VT = 2 * VT * PT * 2, B_PT = 2 * kChunk * PT * 2;
    constexpr int oKt = 0, oEt = oKt + B_ROWS, oLoop = oEt + B_ROWS;
    constexpr int oS1 = oLoop, oD1 = oS1 + B_ST, oO1 = oD1 + B_ST, oXU = oO1 + B_VT, odUX = oXU + B_VT;
    // After the solve, T is kept as split bf16 [row][col] over A/T and the (by then dead)
    // decay totals, for the value loop.
    constexpr int B_TS = 2 * kChunk * PT * 2;
    constexpr int oAT = odUX + B_VT, oTot = oAT + kChunk * PA * 4, oTs = oAT;
    constexpr int oGam = (oTot + 4 * DK * 4 > oTs + B_TS) ? oTot + 4 * DK * 4 : oTs + B_TS;
    constexpr int oDG = oGam + DK * 4;
    constexpr int oRed = oDG + DK * 4;           // per-token gate gradients of half 1 (SG)
    constexpr int oList = oRed + (SG ? 3 * kChunk * 4 : 0);   // work list of the exact pass
    // the channel slices of the exact pass go over the Kh and Et rows where they fit (dk >= 64)
    constexpr bool SL_OVER = kSliceFloats * 4 <= 2 * B_ROWS;
    constexpr int oSl = SL_OVER ? oKt : oList + (NTH + 4) * 4;
    constexpr int SMEM = oList + (EX ? (NTH + 4) * 4 + (SL_OVER ? 0 : kSliceFloats * 4) : 0);
    constexpr int oQt = oLoop, odPt = oQt + B_ROWS, odAt = odPt + B_PT;
    constexpr int oScr = odAt + B_PT, oTotA = oScr + 8 * DK * 4, oTotB = oTotA + 4 * DK * 4;
    static_assert(oQt + B_ROWS <= oAT, "Qt rows overlap T during preparation");
    static_assert(oTotB + 4 * DK * 4 <= oTot, "epilogue layout overlaps the decay totals");
    static_assert(SMEM <= 160 * 1024, "LDS budget of a CU");

    __shared__ __align__(16) char smem[SMEM];
    __bf16 *sKt = reinterpret_cast<__bf16 *>(smem + oKt), *sEt = reinterpret_cast<__bf16 *>(smem + oEt);
    __bf16 *sQt = reinterpret_cast<__bf16 *>(smem + oQt);
    __bf16 *S1 = reinterpret_cast<__bf16 *>(smem + oS1), *D1 = reinterpret_cast<__bf16 *>(smem + oD1);
    __bf16 *O1 = reinterpret_cast<__bf16 *>(smem + oO1), *XU = reinterpret_cast<__bf16 *>(smem + oXU);
    __bf16 *dUX = reinterpret_cast<__bf16 *>(smem + odUX);
    __bf16 *dPt = reinterpret_cast<__bf16 *>(smem + odPt), *dAt = reinterpret_cast<__bf16 *>(smem + odAt);
    float *sAT = reinterpret_cast<float *>(smem + oAT), *sTot = reinterpret_cast<float *>(smem + oTot);
    float *sGam = reinterpret_cast<float *>(smem + oGam), *sDG = reinterpret_cast<float *>(smem + oDG);
    float *sScr = reinterpret_cast<float *>(smem + oScr);
    float *sRed = reinterpret_cast<float *>(smem + oRed);
    __bf16 *sTs = reinterpret_cast<__bf16 *>(smem + oTs);
    int *sList = reinterpret_cast<int *>(smem + oList);
    const int NC = (a.T + kChunk - 1) / kChunk;

    // Work list: the fast pass takes its one chunk; the exact pass walks the flagged chunks of
    // its share, gathered NTH candidates at a time.  Chunk L = (b * H + h) * NC + c.
    const long nitems = (long)a.B * a.H * NC;
    const int *flags = reinterpret_cast<const int *>(reinterpret_cast<const char *>(a.factors) +
                                                     (size_t)nitems * factor_elems_per_chunk<DK>() * 2 +
                                                     record_flags_offset<DK>(nitems));
    // Work list.  Fast pass: persistent (one workgroup per CU), items blockIdx.x, + gridDim.x, ...;
    // each item loads the next one's record pieces and first value tile into registers during its
    // scans and stores, where they are free and the loads' latency is hidden.  Exact pass: the
    // flagged chunks of its share, gathered NTH candidates at a time.
    const int nmine = EX ? 0 : (blockIdx.x < (unsigned)nitems ? (int)((nitems - 1 - blockIdx.x) / gridDim.x) + 1 : 0);
    ChunkTile<DK> cur;               // value-tile inputs, one tile ahead (the next item's first in the fast pass)
    ChunkRecRegs<DK> pr;
    if (!EX && nmine > 0) {
        const int L0 = blockIdx.x;
        chunk_load_tile<DK, BF16, GL, SG>(a, NC, L0, 0, cur, threadIdx.x);
        chunk_load_record<DK>(reinterpret_cast<const char *>(a.factors) +
                                  (size_t)a.B * a.H * NC * factor_elems_per_chunk<DK>() * 2 +
                                  (size_t)L0 * ChunkRecord<DK>::BYTES,
                              threadIdx.x, pr);
    }
    for (long base = blockIdx.x; base < (EX ? nitems : (long)blockIdx.x + 1); base += (long)gridDim.x * NTH) {
    const int nwork = EX ? gather_flagged<NTH>(flags, nitems, base, gridDim.x, sList, sList + NTH) : nmine;
    for (int wi = 0; wi < nwork; ++wi) {
    const int L = EX ? sList[wi] : (int)blockIdx.x + wi * (int)gridDim.x;
    const int tid = threadIdx.x, wv = tid >> 6, hf = wv >> 2, w = wv & 3, l = tid & 63, r = l & 15, g = l >> 4;
    const int n = hf;                            // value column block of this wave's tiles
    const int c = L % NC, bh = L / NC, h = bh % a.H, b = bh / a.H;
    const int T = a.T, H = a.H, DV = a.DV;
    const int t0 = c * kChunk;
    const size_t tokK = (size_t)H * DK, tokV = (size_t)H * DV;
    const size_t baseK = ((size_t)b * T * H + h) * DK;
    const size_t baseV0 = ((size_t)b * T * H + h) * DV;
    const size_t tokBase = baseV0 + (size_t)t0 * tokV;
    const int kk_lo = (w >= 2) ? 1 : 0;
    const int nkk = (w >= 2) ? 2 : 1;
    const int tk = t0 + 16 * w + r;
    const bool vk = tk < T;
    const size_t rowK = baseK + (size_t)(vk ? tk : T - 1) * tokK;
    const size_t srowK = baseK / DK + (size_t)(vk ? tk : T - 1) * H;   // per-token gate offset (SG)
    const int chh = hf * (DK / 2);               // first key channel of this half
    auto ch = [&](int e) { return chh + ch4(e, g); };
#ifdef GDN2_STAMPS
    // start 0, record in LDS 1, value tiles 0 and 1 done 2, 3, all tiles 4, epilogue inputs 5,
    // element chain 6, end 7
    unsigned long long *stp = !EX && g_chunk_stamps ? g_chunk_stamps + ((size_t)L * 8 + wv) * 8 : nullptr;
#else
    unsigned long long *stp = nullptr;
#endif
    (void)stp;
    GDN2_STAMP_REGS;
    GDN2_STAMP(stp, 0);

    // ---- preparation: the chunk operand record that the adjoint-factor kernel wrote (Kh and
    // Et rows, T, P^T fragments and gamma), into LDS and registers.  The fast pass loaded it (and
    // the first value tile) during the previous item or before the first; the exact pass loads
    // it here.
    using Rec = ChunkRecord<DK>;
    const char *rec = reinterpret_cast<const char *>(a.factors) +
                      (size_t)a.B * H * NC * factor_elems_per_chunk<DK>() * 2 + (size_t)L * Rec::BYTES;
    if (EX) {
        chunk_load_tile<DK, BF16, GL, SG>(a, NC, L, 0, cur, tid);
        chunk_load_record<DK>(rec, tid, pr);
    }
    Split4 Pt[4];                  // lane holds P[16mt + 4g + i][16w + r] (zero for mt < w)
    {
        const int trow = tid >> 3, tc8 = 8 * (tid & 7);
        if (tid < DK) sGam[tid] = pr.gm;
#pragma unroll
        for (int it = 0; it < DK / 16; ++it) {
            const int idx = tid + NTH * it, plane = idx / (8 * DK), rem = idx % (8 * DK);
            const int row = rem / (DK / 8), c8 = 8 * (rem % (DK / 8));
            *reinterpret_cast<u32x4 *>((plane < 2 ? sKt : sEt) + (plane & 1) * RK + row * PK + c8) = pr.rv[it];
        }
        *reinterpret_cast<u32x4 *>(&sTs[trow * PT + tc8]) = pr.th;
        *reinterpret_cast<u32x4 *>(&sTs[kChunk * PT + trow * PT + tc8]) = pr.tl;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const bf16x8 o = __builtin_bit_cast(bf16x8, pr.pv[mt]);
            Pt[mt].hi = __builtin_shufflevector(o, o, 0, 1, 2, 3);
            Pt[mt].lo = __builtin_shufflevector(o, o, 4, 5, 6, 7);
        }
    }
    __syncthreads();
    GDN2_STAMP(stp, 1);

    // ---- value tiles: X, U, dU, dX and the key-side accumulators ----
    f32x4 aQ[NMH], aE[NMH], aH[NMH], aPA[4];     // aPA: dP (half 0) or dA (half 1)
#pragma unroll
    for (int m = 0; m < NMH; ++m) aQ[m] = aE[m] = aH[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) aPA[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    float pw[4] = {0.f, 0.f, 0.f, 0.f};          // per-token dw partial sums (write gate per token)
    float dgp[NSF];
#pragma unroll
    for (int it = 0; it < NSF; ++it) dgp[it] = 0.f;

    for (int j0 = 0; j0 < DV; j0 += VT) {
        // lane indices afresh from an opaque copy of the thread index: the address
        // arithmetic is redone each tile instead of being held in registers
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int wv = tid >> 6, hf = wv >> 2, w = wv & 3, l = tid & 63, r = l & 15, g = l >> 4;
        const int n = hf;
        const int kk_lo = (w >= 2) ? 1 : 0;
        const int nkk = (w >= 2) ? 2 : 1;
        // stage S, dS' ([channel][col]) and dO ([col][token]); dgamma partial sums
#pragma unroll
        for (int it = 0; it < NSF; ++it) {
            const int idx = tid + NTH * it;
            if (idx < DK * 8) {
                const int chn = idx >> 3, q = idx & 7;
                const f32x4 sv = cur.s[it], dv = cur.d[it];
                dgp[it] += (sv[0] * dv[0] + sv[1] * dv[1]) + (sv[2] * dv[2] + sv[3] * dv[3]);
                const Split4 ss = split4(sv);
                const Split4 ds = split4(dv);
                *reinterpret_cast<bf16x4 *>(&S1[chn * PS + 4 * q]) = ss.hi;
                *reinterpret_cast<bf16x4 *>(&S1[DK * PS + chn * PS + 4 * q]) = ss.lo;
                *reinterpret_cast<bf16x4 *>(&D1[chn * PS + 4 * q]) = ds.hi;
                *reinterpret_cast<bf16x4 *>(&D1[DK * PS + chn * PS + 4 * q]) = ds.lo;
            }
        }
        quad_transpose4(cur.o);
        quad_transpose4(cur.v);
        if constexpr (!SG) quad_transpose4(cur.wg);
        {
            const int col = tid & 31, tg = tid >> 5;
            f32x4 ov;
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = (t0 + 4 * tg + i < T) ? cur.o[i] : 0.f;
            const Split4 so = split4(ov);
            *reinterpret_cast<bf16x4 *>(&O1[col * PT + 4 * tg]) = so.hi;
            *reinterpret_cast<bf16x4 *>(&O1[VT * PT + col * PT + 4 * tg]) = so.lo;
        }
        float vD[4], wD[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = t0 + 16 * w + 4 * g + i < T;
            vD[i] = ok ? cur.v[i] : 0.f;
            wD[i] = ok ? gate_act<GL>(cur.wg[i]) : 0.f;
        }
        __syncthreads();
        // next tile's loads are in flight during this tile's products
        {
            // the next tile of this item, or after the last one the first tile of the next item
            // (fast pass; the exact pass reloads its last tile), chosen by address: no branch
            const bool more = j0 + VT < DV;
            const int Lt = more ? L : (EX ? L : (wi + 1 < nwork ? L + (int)gridDim.x : L));
            chunk_load_tile<DK, BF16, GL, SG>(a, NC, Lt, more ? j0 + VT : (EX ? j0 : 0), cur, tid);
        }

        // X = Z - Et S and dU = P^T dO + Kh dS': tile (token block w, column block n)
        {
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = -(wD[i] * vD[i]);
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                const Split8 ef = row_frag4<PK>(sEt, sEt + RK, 16 * w + r, j, g);
                const Split8 sf = frag_tr<PS>(S1, S1 + DK * PS, 32 * j, 16 * n, r, g);
                if (FAST) acc = mfma32(ef.hi, sf.lo, mfma32(ef.hi, sf.hi, acc));   // Et (hi part) times S
                else acc = mfma32x3(ef, sf, acc);
            }
            const Split4 sx = split4(-acc);    // lane holds X[16w + 4g + i][16n + r]
            *reinterpret_cast<bf16x4 *>(&XU[(16 * n + r) * PT + 16 * w + 4 * g]) = sx.hi;
            *reinterpret_cast<bf16x4 *>(&XU[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = sx.lo;
            f32x4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk >= kk_lo) {
                    const __bf16 *oh = &O1[(16 * n + r) * PT + 32 * kk], *ol = oh + VT * PT;
                    du = mfma32x3(join(Pt[2 * kk], Pt[2 * kk + 1]),
                                  frag_2x4(oh + 4 * g, oh + 16 + 4 * g, ol + 4 * g, ol + 16 + 4 * g), du);
                }
            }
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                du = mfma32x3(row_frag4<PK>(sKt, sKt + RK, 16 * w + r, j, g),
                              frag_tr<PS>(D1, D1 + DK * PS, 32 * j, 16 * n, r, g), du);
            }
            const Split4 sd = split4(du);
            *reinterpret_cast<bf16x4 *>(&dUX[(16 * n + r) * PT + 16 * w + 4 * g]) = sd.hi;
            *reinterpret_cast<bf16x4 *>(&dUX[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = sd.lo;
        }
        __syncthreads();
        // U = T X and dX = T^T dU (registers); dv = dX * w and dw = dX * v
        f32x4 Ur = {0.f, 0.f, 0.f, 0.f}, dXr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk < nkk)
                Ur = mfma32x3(frag_8(&sTs[(16 * w + r) * PT + 32 * kk + 8 * g],
                                     &sTs[kChunk * PT + (16 * w + r) * PT + 32 * kk + 8 * g]),
                              frag_8(&XU[(16 * n + r) * PT + 32 * kk + 8 * g],
                                     &XU[VT * PT + (16 * n + r) * PT + 32 * kk + 8 * g]), Ur);
            if (kk >= kk_lo) {
                const __bf16 *dh = &dUX[(16 * n + r) * PT + 32 * kk], *dl = dh + VT * PT;
                dXr = mfma32x3(frag_tr<PT>(sTs, sTs + kChunk * PT, 32 * kk, 16 * w, r, g),   // T^T rows
                               frag_2x4(dh + 4 * g, dh + 16 + 4 * g, dl + 4 * g, dl + 16 + 4 * g), dXr);
            }
        }
        {
            char *dvb = reinterpret_cast<char *>(a.dv + tokBase + j0);
            char *dwb = reinterpret_cast<char *>(a.dw + tokBase + j0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tr = 16 * w + 4 * g + i;
                if (SG && (a.scalar & kScalarWrite)) pw[i] += dXr[i] * vD[i];
                if (t0 + tr < T) {
                    const unsigned o = ((unsigned)tr * (unsigned)tokV + (unsigned)(16 * n + r)) * 4u;
                    *reinterpret_cast<float *>(dvb + o) = dXr[i] * wD[i];
                    if (!(SG && (a.scalar & kScalarWrite)))
                        *reinterpret_cast<float *>(dwb + o) = dXr[i] * vD[i] * gate_dact<GL>(wD[i]);
                }
            }
        }
        __syncthreads();
        {
            const Split4 su = split4(Ur), sx = split4(-dXr);
            *reinterpret_cast<bf16x4 *>(&XU[(16 * n + r) * PT + 16 * w + 4 * g]) = su.hi;
            *reinterpret_cast<bf16x4 *>(&XU[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = su.lo;
            *reinterpret_cast<bf16x4 *>(&dUX[(16 * n + r) * PT + 16 * w + 4 * g]) = sx.hi;
            *reinterpret_cast<bf16x4 *>(&dUX[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = sx.lo;
        }
        __syncthreads();
        // key-side accumulators, sums over this tile's columns (every operand whose
        // contraction index is the value column is read transposed from its [col][.] tile)
        {
            const Split8 oT = frag_tr<PT>(O1, O1 + VT * PT, 0, 16 * w, r, g);    // dO[token 16w + r][col]
            const Split8 xT = frag_tr<PT>(dUX, dUX + VT * PT, 0, 16 * w, r, g);  // -dX[token][col]
            const Split8 uT = frag_tr<PT>(XU, XU + VT * PT, 0, 16 * w, r, g);    // U[token][col]
#pragma unroll
            for (int mm = 0; mm < NMH; ++mm) {
                const int m = NMH * hf + mm;
                const __bf16 *sh = &S1[(16 * m + r) * PS], *sl = sh + DK * PS;
                const Split8 sa = frag_2x4(sh + 4 * g, sh + 16 + 4 * g, sl + 4 * g, sl + 16 + 4 * g);
                aQ[mm] = mfma32x3(sa, oT, aQ[mm]);   // (dO S^T)^T
                aE[mm] = mfma32x3(sa, xT, aE[mm]);   // (-dX S^T)^T
                const __bf16 *dh = &D1[(16 * m + r) * PS], *dl = dh + DK * PS;
                aH[mm] = mfma32x3(frag_2x4(dh + 4 * g, dh + 16 + 4 * g, dl + 4 * g, dl + 16 + 4 * g), uT,
                                  aH[mm]);           // (U dS'^T)^T = dKh^T
            }
            const Split8 lhs = hf ? xT : oT;         // dO U^T or -dX U^T
#pragma unroll
            for (int nn = 0; nn < 4; ++nn)
                if (nn <= w) {
                    aPA[nn] = mfma32x3(lhs, frag_tr<PT>(XU, XU + VT * PT, 0, 16 * nn, r, g), aPA[nn]);
                }
        }
        __syncthreads();
        if (j0 == 0) GDN2_STAMP(stp, 2);
        if (j0 == VT) GDN2_STAMP(stp, 3);
    }
    GDN2_STAMP(stp, 4);

    // ---- epilogue: dgamma, dP/dA products, element-wise chain ----
    // q, k, log alpha and b are read again, and the decay prefix G is formed from log alpha with
    // the factor kernel's cross-block offsets from the record: only this chain uses it, and
    // leaving it out of the preparation shortens the loads the first value tile waits for.  The lane
    // indices are derived afresh from an opaque copy of the thread index, so that no
    // address arithmetic of the preparation is kept live across the value loop.
  {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wv = tid >> 6, hf = wv >> 2, w = wv & 3, l = tid & 63, r = l & 15, g = l >> 4;
    const int kk_lo = (w >= 2) ? 1 : 0;
    const int nkk = (w >= 2) ? 2 : 1;
    const int tk = t0 + 16 * w + r;
    const bool vk = tk < T;
    const size_t rowK = baseK + (size_t)(vk ? tk : T - 1) * tokK;
    const size_t srowK = baseK / DK + (size_t)(vk ? tk : T - 1) * H;
    const int chh = hf * (DK / 2);
    auto ch = [&](int e) { return chh + ch4(e, g); };
    // a per-token gate's gradient is the sum over its channels: sum this lane's part, then
    // over the lanes of the token (shuffles) and over the two halves (LDS)
    auto lane_sum16 = [](float x) {   // over the 16 lanes of a row
        x += __shfl_xor(x, 1);
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 4);
        x += __shfl_xor(x, 8);
        return x;
    };
    auto group_sum4 = [](float x) {   // over g: lanes r, r + 16, r + 32, r + 48
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        return x;
    };
    if (SG && (a.scalar & kScalarWrite)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = lane_sum16(pw[i]);   // tokens 16w + 4g + i, columns of half hf
        if (hf == 1 && r == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sRed[2 * kChunk + 16 * w + 4 * g + i] = pw[i];
        }
    }
#pragma unroll
    for (int it = 0; it < NSF; ++it) {
        const int idx = tid + NTH * it;
        if (idx < DK * 8) sScr[idx] = dgp[it];
    }
    {
        // dP = lower(dO U^T) (half 0), dA = strictly-lower(-dX U^T) (half 1); lane holds
        // row 16w + 4g + i, key 16nn + r; written as [key][query]
        __bf16 *dM = hf ? dAt : dPt;
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
            f32x4 v4 = aPA[nn];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int qry = 16 * w + 4 * g + i, key = 16 * nn + r;
                if (!(hf ? key < qry : key <= qry)) v4[i] = 0.f;
            }
            const Split4 sp = split4(v4);
            *reinterpret_cast<bf16x4 *>(&dM[(16 * nn + r) * PT + 16 * w + 4 * g]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&dM[kChunk * PT + (16 * nn + r) * PT + 16 * w + 4 * g]) = sp.lo;
        }
    }
    float qf[NEH], kf[NEH], G[NEH], bgf[NEH];
    KeyRaw4<DK / 2, BF16, GL, SG> raw;
    raw.issue(a.q, a.k, a.la, a.bg, rowK + chh, g, vk, srowK, a.scalar);
    f32x4 pre4[NEH / 4];           // decay offsets of this wave's token block, channels ch(4m) ..
#pragma unroll
    for (int m4 = 0; m4 < NEH / 4; ++m4)
        pre4[m4] = *reinterpret_cast<const f32x4 *>(rec + Rec::oPre + (size_t)(w * DK + chh + 16 * m4 + 4 * g) * 4);
    raw.unpack(qf, kf, G, bgf);
    float dact[NEH];               // d log_alpha / d stored decay input
    raw.decay_dact_all(dact);
    // G: the log2 decay prefix, as the factor kernel's chunk_scan forms it
#pragma unroll
    for (int e = 0; e < NEH; ++e) G[e] *= kLog2e;
    scan_with_offsets<NEH>(G, pre4);
    if constexpr (!EX) {
        // Qt rows of this half's channels again
#pragma unroll
        for (int mm = 0; mm < NMH; ++mm) {
            f32x4 qt;
#pragma unroll
            for (int i = 0; i < 4; ++i) qt[i] = qf[4 * mm + i] * exp2_fast(G[4 * mm + i]);
            const Split4 sq = split4(qt);
            const int o = (16 * w + r) * PK + chh + 16 * mm + 4 * g;
            *reinterpret_cast<bf16x4 *>(&sQt[o]) = sq.hi;
            *reinterpret_cast<bf16x4 *>(&sQt[RK + o]) = sq.lo;
        }
    }
    __syncthreads();
    if (SG && (a.scalar & kScalarWrite) && hf == 0 && r == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 16 * w + 4 * g + i;
            if (t < T) a.dw[baseK / DK + (size_t)t * H] = pw[i] + sRed[2 * kChunk + 16 * w + 4 * g + i];
        }
    }
    if (tid < DK) {
        float sacc = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) sacc += sScr[8 * tid + q];
        sDG[tid] = sacc;
    }
    GDN2_STAMP(stp, 5);

    // ---- element-wise chain (token 16w + r, channels ch(e)) ----
    // chain(mm, dq, dE, dK, h) for elements 4mm .. 4mm + 3, in the natural variables: dq, dE (the
    // gradient of e = b k), dK (k's gradient through A and P) and h = exp(g_C - G), so that
    // Kh = k h; writes dq, dk, db and leaves dG (xg) and dKh * Kh (yh) for the decay scan.
    float xg[NEH], yh[NEH];
    float sb = 0.f;                // per-token db partial (erase gate per token)
    auto chain = [&](int mm, const float (&dq)[4], const float (&dE)[4], const float (&dK)[4],
                     const float (&h)[4]) __attribute__((always_inline)) {
        f32x4 vq, vk4, vb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * mm + i;
            const float dKh = aH[mm][i];
            vq[i] = dq[i];
            vb[i] = dE[i] * kf[e] * gate_dact<GL>(bgf[e]);
            vk4[i] = dK[i] + dKh * h[i] + dE[i] * bgf[e];
            yh[e] = dKh * kf[e] * h[i];
            xg[e] = dq[i] * qf[e] + dE[i] * bgf[e] * kf[e] - dK[i] * kf[e] - yh[e];
        }
        if (SG && (a.scalar & kScalarErase)) sb += (vb[0] + vb[1]) + (vb[2] + vb[3]);
        if (vk) {
            const size_t off = rowK + chh + 16 * mm + 4 * g;
            *reinterpret_cast<f32x4 *>(a.dq + off) = vq;
            *reinterpret_cast<f32x4 *>(a.dk + off) = vk4;
            if (!(SG && (a.scalar & kScalarErase))) *reinterpret_cast<f32x4 *>(a.db + off) = vb;
        }
    };
    if constexpr (!EX) {
        // dQt^T = gamma^-1 (gamma dQt_S^T + Kh^T dP^T) and dEt^T likewise with dA (keys up to this
        // wave's queries); dKt^T = Qt^T dP + Et^T dA (queries from this wave's keys on)
#pragma unroll
        for (int mm = 0; mm < NMH; ++mm) {
            const int m = NMH * hf + mm;
            const f32x4 gam = *reinterpret_cast<const f32x4 *>(&sGam[16 * m + 4 * g]);
            aQ[mm] *= gam;
            aE[mm] *= gam;
            f32x4 aK = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk < nkk) {
                    const Split8 kh = frag_tr<PK>(sKt, sKt + RK, 32 * kk, 16 * m, r, g);
                    aQ[mm] = mfma32x3(kh, frag_tr<PT>(dPt, dPt + kChunk * PT, 32 * kk, 16 * w, r, g), aQ[mm]);
                    aE[mm] = mfma32x3(kh, frag_tr<PT>(dAt, dAt + kChunk * PT, 32 * kk, 16 * w, r, g), aE[mm]);
                }
                if (kk >= kk_lo) {
                    const __bf16 *ph = &dPt[(16 * w + r) * PT + 32 * kk], *pl = ph + kChunk * PT;
                    aK = mfma32x3(frag_tr<PK>(sQt, sQt + RK, 32 * kk, 16 * m, r, g),
                                  frag_2x4(ph + 4 * g, ph + 16 + 4 * g, pl + 4 * g, pl + 16 + 4 * g), aK);
                    const __bf16 *ah = &dAt[(16 * w + r) * PT + 32 * kk], *al = ah + kChunk * PT;
                    aK = mfma32x3(frag_tr<PK>(sEt, sEt + RK, 32 * kk, 16 * m, r, g),
                                  frag_2x4(ah + 4 * g, ah + 16 + 4 * g, al + 4 * g, al + 16 + 4 * g), aK);
                }
            }
            float dq[4], dE[4], dK[4], h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * mm + i;
                const float eg = exp2_fast(G[e]), eng = exp2_fast(-G[e]);
                const float rg = eg * __builtin_amdgcn_rcpf(gam[i]);   // exp(G - g_C): finite on unflagged chunks
                dq[i] = aQ[mm][i] * rg;
                dE[i] = aE[mm][i] * rg;
                dK[i] = aK[i] * eng;
                h[i] = gam[i] * eng;
            }
            chain(mm, dq, dE, dK, h);
        }
    } else {
        // exact pairwise decays, one slice of 16 channels per half at a time (over the Kh and
        // Et rows, which this pass no longer reads, where they fit)
        float *slc = reinterpret_cast<float *>(smem + oSl);
        float ev[NEH];
#pragma unroll
        for (int e = 0; e < NEH; ++e) ev[e] = bgf[e] * kf[e];
        const int t = 16 * w + r;
        const int jhi = 16 * w + 16;                  // keys j <= t of this wave's queries: j < jhi
#pragma unroll
        for (int mm = 0; mm < NMH; ++mm) {
            __syncthreads();
            slice_put<NEH>(slc, mm, hf, w, r, g, ev, qf, kf, G);
            __syncthreads();
            float rq[4] = {0.f, 0.f, 0.f, 0.f}, ra[4] = {0.f, 0.f, 0.f, 0.f}, ck[4] = {0.f, 0.f, 0.f, 0.f};
            // row side: dq_t += sum_{j <= t} dP_tj k_j x_tj, dE_t += sum_{j < t} dA_tj k_j x_tj
            for (int j = 0; j < jhi; ++j) {
                const float dp = (float)dPt[j * PT + t] + (float)dPt[kChunk * PT + j * PT + t];
                const float da = (float)dAt[j * PT + t] + (float)dAt[kChunk * PT + j * PT + t];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int cc = 4 * g + i;
                    const float kx = slc[slice_idx(hf, 2, cc, j)] * exp2_fast(G[4 * mm + i] - slc[slice_idx(hf, 3, cc, j)]);
                    const bool on = j <= t;   // beyond it the factor may be inf
                    rq[i] += on ? dp * kx : 0.f;
                    ra[i] += on ? da * kx : 0.f;
                }
            }
            // column side: dk_t += sum_{i >= t} (dA_it e_i + dP_it q_i) x_it
            for (int q = 16 * w; q < kChunk; ++q) {
                const float dp = (float)dPt[t * PT + q] + (float)dPt[kChunk * PT + t * PT + q];
                const float da = (float)dAt[t * PT + q] + (float)dAt[kChunk * PT + t * PT + q];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int cc = 4 * g + i;
                    const float x = exp2_fast(slc[slice_idx(hf, 3, cc, q)] - G[4 * mm + i]);
                    const float y = (da * slc[slice_idx(hf, 0, cc, q)] + dp * slc[slice_idx(hf, 1, cc, q)]) * x;
                    ck[i] += q >= t ? y : 0.f;
                }
            }
            float dq[4], dE[4], h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * mm + i;
                const float eg = exp2_fast(G[e]);
                const float gC = slc[slice_idx(hf, 3, 4 * g + i, kChunk - 1)];
                dq[i] = aQ[mm][i] * eg + rq[i];
                dE[i] = aE[mm][i] * eg + ra[i];
                h[i] = exp2_fast(gC - G[e]);
            }
            chain(mm, dq, dE, ck, h);
        }
    }
    GDN2_STAMP(stp, 6);
    if (!EX) {
        // the next item's record pieces, in flight during the scans and stores below (its first
        // value tile was loaded during the last tile; the last item loads its own again: with a
        // branch around the loads the compiler keeps two copies of these registers live and spills)
        const int Ln = wi + 1 < nwork ? L + (int)gridDim.x : L;
        chunk_load_record<DK>(reinterpret_cast<const char *>(a.factors) +
                                  (size_t)a.B * H * NC * factor_elems_per_chunk<DK>() * 2 + (size_t)Ln * Rec::BYTES,
                              tid, pr);
    }
    // dlog_alpha_t = sum_{s >= t} dG_s + dg_C, with dg_C = sum_s dKh_s Kh_s + dgamma gamma
    float xin[NEH], xtot[NEH], ytot[NEH];
#pragma unroll
    for (int e = 0; e < NEH; ++e) xin[e] = xg[e];
    if (SG && (a.scalar & kScalarErase)) {
        sb = group_sum4(sb);
        if (hf == 1 && g == 0) sRed[16 * w + r] = sb;
    }
    if constexpr (!SG) {
        // both scans behind one barrier (with per-token gates their registers do not fit at once)
        chunk_scan2<NEH, DK>(xin, xtot, reinterpret_cast<float *>(smem + oTotA), yh, ytot,
                             reinterpret_cast<float *>(smem + oTotB), w, r, ch);
    } else {
        chunk_scan<NEH, DK>(xin, xtot, reinterpret_cast<float *>(smem + oTotA), w, r, ch);
        if ((a.scalar & kScalarErase) && hf == 0 && g == 0 && vk) a.db[srowK] = sb + sRed[16 * w + r];
        chunk_scan<NEH, DK>(yh, ytot, reinterpret_cast<float *>(smem + oTotB), w, r, ch);
    }
    float sl = 0.f;                // per-token dlog_alpha partial (decay per token)
#pragma unroll
    for (int mm = 0; mm < NMH; ++mm) {
        f32x4 vl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * mm + i;
            vl[i] = ((xtot[e] - xin[e] + xg[e]) + ytot[e] + sDG[ch(e)] * sGam[ch(e)]) * dact[e];
        }
        if (SG && (a.scalar & kScalarDecay)) sl += (vl[0] + vl[1]) + (vl[2] + vl[3]);
        else if (vk) *reinterpret_cast<f32x4 *>(a.dla + rowK + chh + 16 * mm + 4 * g) = vl;
    }
    if (SG && (a.scalar & kScalarDecay)) {
        sl = group_sum4(sl);
        if (hf == 1 && g == 0) sRed[kChunk + 16 * w + r] = sl;
        __syncthreads();
        if (hf == 0 && g == 0 && vk) a.dla[srowK] = sl + sRed[kChunk + 16 * w + r];
    }
    GDN2_STAMP(stp, 7);
    GDN2_STAMP_FLUSH(stp);
  }
    __syncthreads();   // the next item's preparation overwrites this one's LDS
    }
    }
}

#ifdef GDN2_STAMPS
// the instrumented build only: where the chunk-gradient kernel's fast pass writes its phase
// stamps (8 per item and wave; nullptr = none)
extern "C" int gdn2_stamps_chunk(void *buf) {
    unsigned long long *p = static_cast<unsigned long long *>(buf);
    return hipMemcpyToSymbol(HIP_SYMBOL(g_chunk_stamps), &p, sizeof(p)) == hipSuccess ? 0 : 4;
}
#endif

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
// The fast pass over every chunk, then the exact pass (persistent, one workgroup per CU) over
// the chunks the factor kernel flagged; its workgroups read their share of the flags and end
// when none is set.
template <int DK, bool BF16, bool GL, bool SG>
static hipError_t chunk_t(const BwdArgs &a, hipStream_t st) {
    const int NC = (a.T + kChunk - 1) / kChunk;
    const long items = (long)a.B * a.H * NC;
    // both passes persistent: one workgroup per CU (the kernel's LDS allows no second one)
    const long grid = items < cu_count() ? items : cu_count();
    hipLaunchKernelGGL((bwd_chunk_kernel<DK, BF16, GL, SG, false>), dim3((unsigned)grid), dim3(kChunkThreads), 0, st,
                       a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_chunk_kernel<DK, BF16, GL, SG, true>), dim3((unsigned)grid), dim3(kChunkThreads), 0, st,
                       a);
    return hipGetLastError();
}

template <bool BF16, bool GL, bool SG>
static hipError_t chunk_dk(const BwdArgs &a, int dk, hipStream_t st) {
    switch (dk) {
        case 32: return chunk_t<32, BF16, GL, SG>(a, st);
        case 64: return chunk_t<64, BF16, GL, SG>(a, st);
        case 128: return chunk_t<128, BF16, GL, SG>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_bwd_chunk(const BwdArgs &a, int dk, bool bf16, bool gl, bool sg, hipStream_t st) {
    if (a.DV % 32 != 0) return hipErrorInvalidValue;
    if (gl && sg) return hipErrorInvalidValue;
    if (gl) return bf16 ? chunk_dk<true, true, false>(a, dk, st) : hipErrorInvalidValue;
    if (sg) return bf16 ? chunk_dk<true, false, true>(a, dk, st) : hipErrorInvalidValue;
    return bf16 ? chunk_dk<true, false, false>(a, dk, st) : chunk_dk<false, false, false>(a, dk, st);
}

}  // namespace gdn2
