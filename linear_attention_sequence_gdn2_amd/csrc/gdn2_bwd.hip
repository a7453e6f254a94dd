// gdn2_bwd.hip -- gate-aware backward of the Gated DeltaNet-2 chunkwise-WY operator on gfx950.
//
// Source of the method: blog on Gated DeltaNet-2 (iplexlaw.co.kr), section
// "Token path and parallel training": the backward accumulates gradients with
// the already-gated keys and values (e = b*k, z = w*v) and keeps the
// chunkwise WY structure; the paper abstract (OpenAlex record) calls it the
// gate-aware backward pass.
//
// Per chunk (start state S, end-state gradient dS', notation of gdn2_fwd.hip),
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
// of dG into dlog_alpha.
//
// Three launches: the forward state sweep (gdn2_fwd.hip) stores every chunk's
// start state; bwd_reverse_kernel walks the chunks backwards per (batch, head,
// value tile), storing each chunk's dS' and finally dS0; bwd_chunk_kernel then
// treats every (batch, head, chunk) independently and writes all token
// gradients.  Value columns are independent in S, dS and dS', so value tiles
// need no exchange; the key-side gradients sum over all value columns inside
// one bwd_chunk_kernel workgroup.
//
// Element layout of key-side data in these kernels ("4-groups"): lane (w, r, g)
// holds token 16w + r and channels 16m + 4g + i (m < DK/16, i < 4); element
// e = 4m + i.  The MFMA fragment of contraction step j is elements 8j..8j+7,
// i.e. channels 32j + 4g + {0..3} and 32j + 16 + 4g + {0..3}.  It equals the D
// layout of a product whose rows are channels, so key-side gradients come out
// of transposed products already in element layout.
#include <type_traits>

#include "gdn2_chunk.h"
#include "gdn2_kernels.h"

namespace gdn2 {

__device__ __forceinline__ int ch4(int e, int g) { return 16 * (e >> 2) + 4 * g + (e & 3); }

// key-side inputs of one token for the 4-group layout
template <int DK, bool BF16>
struct KeyRaw4 {
    static constexpr int NM = DK / 16;
    uint2 q[NM], k[NM];
    float4 qx[NM], kx[NM];
    float4 la[NM], bg[NM];
    bool valid;

    __device__ __forceinline__ void issue(const BwdArgs &a, size_t rowoff, int g, bool v) {
        valid = v;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const size_t off = rowoff + 16 * m + 4 * g;
            if (BF16) {
                q[m] = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(a.q) + off);
                k[m] = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(a.k) + off);
            } else {
                qx[m] = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.q) + off);
                kx[m] = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.k) + off);
            }
            la[m] = *reinterpret_cast<const float4 *>(a.la + off);
            bg[m] = *reinterpret_cast<const float4 *>(a.bg + off);
        }
    }

    __device__ __forceinline__ void unpack(float (&qf)[4 * NM], float (&kf)[4 * NM], float (&laf)[4 * NM],
                                           float (&bgf)[4 * NM]) const {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (BF16) {
                qf[4 * m + 0] = __builtin_bit_cast(float, q[m].x << 16);
                qf[4 * m + 1] = __builtin_bit_cast(float, q[m].x & 0xffff0000u);
                qf[4 * m + 2] = __builtin_bit_cast(float, q[m].y << 16);
                qf[4 * m + 3] = __builtin_bit_cast(float, q[m].y & 0xffff0000u);
                kf[4 * m + 0] = __builtin_bit_cast(float, k[m].x << 16);
                kf[4 * m + 1] = __builtin_bit_cast(float, k[m].x & 0xffff0000u);
                kf[4 * m + 2] = __builtin_bit_cast(float, k[m].y << 16);
                kf[4 * m + 3] = __builtin_bit_cast(float, k[m].y & 0xffff0000u);
            } else {
                qf[4 * m + 0] = qx[m].x; qf[4 * m + 1] = qx[m].y; qf[4 * m + 2] = qx[m].z; qf[4 * m + 3] = qx[m].w;
                kf[4 * m + 0] = kx[m].x; kf[4 * m + 1] = kx[m].y; kf[4 * m + 2] = kx[m].z; kf[4 * m + 3] = kx[m].w;
            }
            laf[4 * m + 0] = la[m].x; laf[4 * m + 1] = la[m].y; laf[4 * m + 2] = la[m].z; laf[4 * m + 3] = la[m].w;
            bgf[4 * m + 0] = bg[m].x; bgf[4 * m + 1] = bg[m].y; bgf[4 * m + 2] = bg[m].z; bgf[4 * m + 3] = bg[m].w;
        }
#pragma unroll
        for (int e = 0; e < 4 * NM; ++e) {
            qf[e] = valid ? qf[e] : 0.f;
            kf[e] = valid ? kf[e] : 0.f;
            laf[e] = valid ? laf[e] : 0.f;
            bgf[e] = valid ? bgf[e] : 0.f;
        }
    }
};

// Operand fragments of the key side in the 4-group layout.
template <int NKS>
struct KeyOps {
    Split8 E[NKS], Q[NKS], K[NKS], H[NKS];   // Et, Qt, Kt, Kh
};

template <int NE, bool WE = true, bool WQ = true, bool WK = true, bool WH = true>
__device__ __forceinline__ void key_operands(const float (&qf)[NE], const float (&kf)[NE], const float (&bgf)[NE],
                                             const float (&G)[NE], const float (&gC)[NE], KeyOps<NE / 8> &ops) {
#pragma unroll
    for (int j = 0; j < NE / 8; ++j) {
        float et[8], qt[8], kt[8], kh[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int e = 8 * j + s;
            const float eg = (WE || WQ) ? exp2_fast(G[e]) : 0.f;
            const float eng = WK ? exp2_fast(-G[e]) : 0.f;
            const float ek = WH ? exp2_fast(gC[e] - G[e]) : 0.f;
            et[s] = bgf[e] * kf[e] * eg;
            qt[s] = qf[e] * eg;
            kt[s] = kf[e] * eng;
            kh[s] = kf[e] * ek;
        }
        if (WE) ops.E[j] = split8(et);
        if (WQ) ops.Q[j] = split8(qt);
        if (WK) ops.K[j] = split8(kt);
        if (WH) ops.H[j] = split8(kh);
    }
}

// Write this lane's row (token 16w + r) of an operand as [token][channel] bf16 (hi, lo planes).
template <int NKS, int PK>
__device__ __forceinline__ void store_rows(const Split8 (&f)[NKS], __bf16 *hi, __bf16 *lo, int row, int g) {
#pragma unroll
    for (int j = 0; j < NKS; ++j) {
        bf16x4 h0, h1, l0, l1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h0[i] = f[j].hi[i];
            h1[i] = f[j].hi[4 + i];
            l0[i] = f[j].lo[i];
            l1[i] = f[j].lo[4 + i];
        }
        *reinterpret_cast<bf16x4 *>(&hi[row * PK + 32 * j + 4 * g]) = h0;
        *reinterpret_cast<bf16x4 *>(&hi[row * PK + 32 * j + 16 + 4 * g]) = h1;
        *reinterpret_cast<bf16x4 *>(&lo[row * PK + 32 * j + 4 * g]) = l0;
        *reinterpret_cast<bf16x4 *>(&lo[row * PK + 32 * j + 16 + 4 * g]) = l1;
    }
}

// Write this lane's row as columns of a [channel][token] bf16 tile (optionally negated).
template <int NKS, int PT>
__device__ __forceinline__ void store_cols(const Split8 (&f)[NKS], __bf16 *hi, __bf16 *lo, int tok, int g,
                                           bool neg) {
#pragma unroll
    for (int j = 0; j < NKS; ++j)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int ch = 32 * j + 16 * (s >> 2) + 4 * g + (s & 3);
            const __bf16 h = f[j].hi[s], l = f[j].lo[s];
            hi[ch * PT + tok] = neg ? -h : h;
            lo[ch * PT + tok] = neg ? -l : l;
        }
}

// Key-side fragment (4-group contraction order) of row `row` of a [row][channel] tile.
template <int PK>
__device__ __forceinline__ Split8 row_frag4(const __bf16 *hi, const __bf16 *lo, int row, int j, int g) {
    return frag_2x4(&hi[row * PK + 32 * j + 4 * g], &hi[row * PK + 32 * j + 16 + 4 * g],
                    &lo[row * PK + 32 * j + 4 * g], &lo[row * PK + 32 * j + 16 + 4 * g]);
}

// A^T (rows of this wave's queries against key blocks mt <= w) into sA, and
// P^T rows in registers: Pt[mt] holds P[16mt + 4g + i][16w + r] for mt >= w.
template <int NKS, int PK, int PA, bool FAST>
__device__ __forceinline__ void build_A_Pt(const KeyOps<NKS> &ops, const __bf16 *sKh, const __bf16 *sKl,
                                           const __bf16 *sQh, const __bf16 *sQl, float *sA, Split4 (&Pt)[4],
                                           int w, int r, int g) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        if (mt <= w) {
            f32x4 acc = zero;
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                const Split8 kf = row_frag4<PK>(sKh, sKl, 16 * mt + r, j, g);
                if (FAST) acc = mfma32(kf.hi, ops.E[j].hi, acc);
                else acc = mfma32x3(kf, ops.E[j], acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (!(16 * mt + 4 * g + i < 16 * w + r)) acc[i] = 0.f;
            *reinterpret_cast<f32x4 *>(&sA[(16 * w + r) * PA + 16 * mt + 4 * g]) = acc;
        }
        if (mt >= w) {
            f32x4 acc = zero;
#pragma unroll
            for (int j = 0; j < NKS; ++j) acc = mfma32x3(row_frag4<PK>(sQh, sQl, 16 * mt + r, j, g), ops.K[j], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (!(16 * w + r <= 16 * mt + 4 * g + i)) acc[i] = 0.f;
            Pt[mt] = split4(acc);
        } else {
            Pt[mt] = split4(zero);
        }
    }
}

// ---------------------------------------------------------------------------
// reverse sweep: dS' of every chunk, and dS0
// ---------------------------------------------------------------------------
template <int DK, int VT, bool BF16>
__global__ __launch_bounds__(kThreads, 1) void bwd_reverse_kernel(BwdArgs a) {
    constexpr int NE = DK / 4, NM = DK / 16, NKS = DK / 32, NVT = VT / 16;
    constexpr int NTS = NM * NVT / 4;
    static_assert((NM * NVT) % 4 == 0, "state tiles must split over 4 waves");
    constexpr int PK = DK + 8, PT = kChunk + 8, PA = kChunk + 4;
    constexpr int RQ = kChunk * PK, RT = DK * PT;
    constexpr int RM = RQ > RT ? RQ : RT;
    constexpr int TPT = kChunk * VT / kThreads;  // dO tokens per thread
    constexpr bool FAST = BF16;

    __shared__ __align__(16) __bf16 sR1[4 * RM];       // Kt, Qt rows; later Qt^T, -Et^T
    __shared__ __align__(16) float sA[kChunk * PA];
    __shared__ __align__(16) float sT[kChunk * PA];
    __shared__ __align__(16) __bf16 sD[2 * VT * PK];    // dS' [col][channel]
    __shared__ __align__(16) __bf16 sO[2 * VT * PT];    // dO [col][token]
    __shared__ __align__(16) __bf16 sdU[2 * VT * PT];   // dU [col][token]
    __shared__ __align__(16) __bf16 sdX[2 * VT * PT];   // dX [col][token]
    __shared__ __align__(16) float sTot[4 * DK];
    __shared__ __align__(16) float sGam[DK];

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
    const int L = xcd_swizzle(blockIdx.x, gridDim.x);
    const int vt = L % a.nvt, bh = L / a.nvt, h = bh % a.H, b = bh / a.H;
    const int T = a.T, H = a.H, DV = a.DV;
    const int j0 = vt * VT;
    const size_t tokK = (size_t)H * DK, tokV = (size_t)H * DV;
    const size_t baseK = ((size_t)b * T * H + h) * DK;
    const size_t baseV = ((size_t)b * T * H + h) * DV + j0;
    const size_t sbase = ((size_t)b * H + h) * (size_t)DK * DV + j0;
    const int NC = (T + kChunk - 1) / kChunk;
    const int kk_lo = (w >= 2) ? 1 : 0;

    f32x4 DS[NTS];
#pragma unroll
    for (int s = 0; s < NTS; ++s) {
        const int id = w * NTS + s, m = id / NVT, n = id % NVT;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            DS[s][i] = a.dS_final ? a.dS_final[sbase + (size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] : 0.f;
    }
    for (int idx = tid; idx < kChunk * PA; idx += kThreads) sT[idx] = 0.f;
    auto store_dS_lds = [&]() {
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT, n = id % NVT;
            const Split4 sp = split4(DS[s]);
            *reinterpret_cast<bf16x4 *>(&sD[(16 * n + r) * PK + 16 * m + 4 * g]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&sD[VT * PK + (16 * n + r) * PK + 16 * m + 4 * g]) = sp.lo;
        }
    };
    store_dS_lds();
    __syncthreads();

    for (int c = NC - 1; c >= 0; --c) {
        const int t0 = c * kChunk;
        // gradient w.r.t. this chunk's end state
        {
            float *dst = a.dstates + (((size_t)b * H + h) * NC + c) * (size_t)DK * DV + j0;
#pragma unroll
            for (int s = 0; s < NTS; ++s) {
                const int id = w * NTS + s, m = id / NVT, n = id % NVT;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] = DS[s][i];
            }
        }
        // key side of the chunk
        KeyRaw4<DK, BF16> raw;
        {
            const int tk = t0 + 16 * w + r;
            const bool vk = tk < T;
            raw.issue(a, baseK + (size_t)(vk ? tk : T - 1) * tokK, g, vk);
        }
        // dO tile -> [col][token]
        {
            const int col = tid % VT, tg = tid / VT;
            float x[TPT];
#pragma unroll
            for (int i = 0; i < TPT; ++i) {
                const int t = t0 + tg * TPT + i;
                const float vv = a.dO[baseV + (size_t)(t < T ? t : T - 1) * tokV + col];
                x[i] = t < T ? vv : 0.f;
            }
#pragma unroll
            for (int i = 0; i < TPT; ++i) {
                __bf16 hh, ll;
                split1(x[i], hh, ll);
                sO[col * PT + tg * TPT + i] = hh;
                sO[VT * PT + col * PT + tg * TPT + i] = ll;
            }
        }
        float qf[NE], kf[NE], laf[NE], bgf[NE], G[NE], gC[NE];
        raw.unpack(qf, kf, laf, bgf);
#pragma unroll
        for (int e = 0; e < NE; ++e) G[e] = laf[e] * kLog2e;
        chunk_scan<NE, DK>(G, gC, sTot, w, r, [&](int e) { return ch4(e, g); });
        if (w == 0 && r == 0) {
#pragma unroll
            for (int e = 0; e < NE; ++e) sGam[ch4(e, g)] = exp2_fast(gC[e]);
        }
        KeyOps<NKS> ops;
        key_operands<NE>(qf, kf, bgf, G, gC, ops);
        store_rows<NKS, PK>(ops.K, sR1, sR1 + RQ, 16 * w + r, g);
        store_rows<NKS, PK>(ops.Q, sR1 + 2 * RQ, sR1 + 3 * RQ, 16 * w + r, g);
        __syncthreads();

        Split4 Pt[4];
        build_A_Pt<NKS, PK, PA, FAST>(ops, sR1, sR1 + RQ, sR1 + 2 * RQ, sR1 + 3 * RQ, sA, Pt, w, r, g);
        __syncthreads();
        // Qt^T and -Et^T replace the row tiles
        store_cols<NKS, PT>(ops.Q, sR1, sR1 + RT, 16 * w + r, g, false);
        store_cols<NKS, PT>(ops.E, sR1 + 2 * RT, sR1 + 3 * RT, 16 * w + r, g, true);
        solve_T<PA>(sA, sT, w, r, g);

        // dU = P^T dO + Kh dS'
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk >= kk_lo) {
                    const Split8 of = frag_2x4(&sO[(16 * n + r) * PT + 32 * kk + 4 * g],
                                               &sO[(16 * n + r) * PT + 32 * kk + 16 + 4 * g],
                                               &sO[VT * PT + (16 * n + r) * PT + 32 * kk + 4 * g],
                                               &sO[VT * PT + (16 * n + r) * PT + 32 * kk + 16 + 4 * g]);
                    acc = mfma32x3(join(Pt[2 * kk], Pt[2 * kk + 1]), of, acc);
                }
            }
#pragma unroll
            for (int j = 0; j < NKS; ++j)
                acc = mfma32x3(ops.H[j], row_frag4<PK>(sD, sD + VT * PK, 16 * n + r, j, g), acc);
            const Split4 sp = split4(acc);
            *reinterpret_cast<bf16x4 *>(&sdU[(16 * n + r) * PT + 16 * w + 4 * g]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&sdU[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = sp.lo;
        }
        __syncthreads();
        // dX = T^T dU
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk >= kk_lo) {
                    float tv[8];
#pragma unroll
                    for (int s = 0; s < 8; ++s) tv[s] = sT[(32 * kk + 8 * g + s) * PA + 16 * w + r];
                    acc = mfma32x3(split8(tv), frag_8(&sdU[(16 * n + r) * PT + 32 * kk + 8 * g],
                                                      &sdU[VT * PT + (16 * n + r) * PT + 32 * kk + 8 * g]), acc);
                }
            }
            const Split4 sp = split4(acc);
            *reinterpret_cast<bf16x4 *>(&sdX[(16 * n + r) * PT + 16 * w + 4 * g]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&sdX[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = sp.lo;
        }
        __syncthreads();
        // dS <- diag(gamma) dS' + Qt^T dO - Et^T dX
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT, n = id % NVT;
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = sGam[16 * m + 4 * g + i] * DS[s][i];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                acc = mfma32x3(frag_8(&sR1[(16 * m + r) * PT + 32 * kk + 8 * g], &sR1[RT + (16 * m + r) * PT + 32 * kk + 8 * g]),
                               frag_8(&sO[(16 * n + r) * PT + 32 * kk + 8 * g], &sO[VT * PT + (16 * n + r) * PT + 32 * kk + 8 * g]),
                               acc);
                acc = mfma32x3(frag_8(&sR1[2 * RT + (16 * m + r) * PT + 32 * kk + 8 * g],
                                      &sR1[3 * RT + (16 * m + r) * PT + 32 * kk + 8 * g]),
                               frag_8(&sdX[(16 * n + r) * PT + 32 * kk + 8 * g], &sdX[VT * PT + (16 * n + r) * PT + 32 * kk + 8 * g]),
                               acc);
            }
            DS[s] = acc;
        }
        store_dS_lds();
        __syncthreads();
    }

    if (a.dS0) {
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT, n = id % NVT;
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dS0[sbase + (size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] = DS[s][i];
        }
    }
}

// ---------------------------------------------------------------------------
// chunk-parallel gradients of every token input
// ---------------------------------------------------------------------------
template <int DK, bool BF16>
__global__ __launch_bounds__(kThreads, 1) void bwd_chunk_kernel(BwdArgs a) {
    constexpr int VT = 32, NVT = 2;
    constexpr int NE = DK / 4, NM = DK / 16, NKS = DK / 32;
    constexpr int PK = DK + 8, PT = kChunk + 8, PA = kChunk + 4, PC = VT + 8;
    constexpr int RQ = kChunk * PK, RT = DK * PT;
    constexpr bool FAST = BF16;
    // loop-phase layout (bf16 element offsets), hi plane then lo plane for each
    constexpr int oS1 = 0;                         // S  [col][channel]
    constexpr int oS2 = oS1 + 2 * VT * PK;         // S  [channel][col]
    constexpr int oD1 = oS2 + 2 * DK * PC;         // dS' [col][channel]
    constexpr int oD2 = oD1 + 2 * VT * PK;         // dS' [channel][col]
    constexpr int oO1 = oD2 + 2 * DK * PC;         // dO [col][token]
    constexpr int oO2 = oO1 + 2 * VT * PT;         // dO [token][col]
    constexpr int oX1 = oO2 + 2 * kChunk * PC;     // X  [col][token]
    constexpr int oU2 = oX1 + 2 * VT * PT;         // U  [token][col]
    constexpr int odU1 = oU2 + 2 * kChunk * PC;    // dU [col][token]
    constexpr int odX2 = odU1 + 2 * VT * PT;       // -dX [token][col]
    constexpr int LOOP_END = odX2 + 2 * kChunk * PC;
    constexpr int PREP_END = 4 * RQ + 2 * kChunk * PA;     // Kt, Qt rows + fp32 A
    constexpr int EPI_END = 4 * RT + 4 * kChunk * PT;
    constexpr int ZSIZE = LOOP_END > PREP_END ? (LOOP_END > EPI_END ? LOOP_END : EPI_END)
                                              : (PREP_END > EPI_END ? PREP_END : EPI_END);
    constexpr int CPT = DK / 8;   // columns (or channels) per thread when staging state tiles
    constexpr int TPC = kThreads / DK;

    __shared__ __align__(16) __bf16 sZ[ZSIZE];
    __shared__ __align__(16) float sT[kChunk * PA];
    __shared__ __align__(16) float sTot[4 * DK];
    __shared__ __align__(16) float sTot2[4 * DK];
    __shared__ __align__(16) float sTot3[4 * DK];
    __shared__ __align__(16) float sDG[kThreads];

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
    const int NC = (a.T + kChunk - 1) / kChunk;
    const int L = xcd_swizzle(blockIdx.x, gridDim.x);
    const int c = L % NC, bh = L / NC, h = bh % a.H, b = bh / a.H;
    const int T = a.T, H = a.H, DV = a.DV;
    const int t0 = c * kChunk;
    const size_t tokK = (size_t)H * DK, tokV = (size_t)H * DV;
    const size_t baseK = ((size_t)b * T * H + h) * DK;
    const size_t baseV0 = ((size_t)b * T * H + h) * DV;
    const size_t stoff = (((size_t)b * H + h) * NC + c) * (size_t)DK * DV;
    const int kk_lo = (w >= 2) ? 1 : 0;
    const int nkk = (w >= 2) ? 2 : 1;
    const int tk = t0 + 16 * w + r;
    const bool vk = tk < T;
    const size_t rowK = baseK + (size_t)(vk ? tk : T - 1) * tokK;

    for (int idx = tid; idx < kChunk * PA; idx += kThreads) sT[idx] = 0.f;

    // ---- key side, A, P, T ----
    // Only Et (for X) and Kh (for dU) stay in registers through the value loop;
    // Qt and Kt are formed again in the epilogue from a second read of the inputs.
    Split8 Ekeep[NKS], Hkeep[NKS];
    Split4 Pt[4];
    float *sA = reinterpret_cast<float *>(sZ + 4 * RQ);
    {
        KeyOps<NKS> ops;
        {
            KeyRaw4<DK, BF16> raw;
            raw.issue(a, rowK, g, vk);
            float qf[NE], kf[NE], laf[NE], bgf[NE], G[NE], gC[NE];
            raw.unpack(qf, kf, laf, bgf);
#pragma unroll
            for (int e = 0; e < NE; ++e) G[e] = laf[e] * kLog2e;
            chunk_scan<NE, DK>(G, gC, sTot, w, r, [&](int e) { return ch4(e, g); });
            key_operands<NE>(qf, kf, bgf, G, gC, ops);
        }
        store_rows<NKS, PK>(ops.K, sZ, sZ + RQ, 16 * w + r, g);
        store_rows<NKS, PK>(ops.Q, sZ + 2 * RQ, sZ + 3 * RQ, 16 * w + r, g);
        __syncthreads();
        build_A_Pt<NKS, PK, PA, FAST>(ops, sZ, sZ + RQ, sZ + 2 * RQ, sZ + 3 * RQ, sA, Pt, w, r, g);
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
            Ekeep[j] = ops.E[j];
            Hkeep[j] = ops.H[j];
        }
    }
    __syncthreads();
    solve_T<PA>(sA, sT, w, r, g);

    // ---- value tiles ----
    f32x4 aQ[NM], aE[NM], aH[NM], aP[4], aA[4];
#pragma unroll
    for (int m = 0; m < NM; ++m) aQ[m] = aE[m] = aH[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 4; ++n) aP[n] = aA[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dgp = 0.f;

    __bf16 *S1 = sZ + oS1, *S2 = sZ + oS2, *D1 = sZ + oD1, *D2 = sZ + oD2, *O1 = sZ + oO1, *O2 = sZ + oO2;
    __bf16 *X1 = sZ + oX1, *U2 = sZ + oU2, *dU1 = sZ + odU1, *dX2 = sZ + odX2;

    for (int j0 = 0; j0 < DV; j0 += VT) {
        // S and dS' tiles, both layouts; partial of dgamma = rowsum(dS' * S)
        {
            const int cA = tid / TPC, cb = (tid % TPC) * CPT;
            const float *Sg = a.states + stoff + (size_t)cA * DV + j0 + cb;
            const float *Dg = a.dstates + stoff + (size_t)cA * DV + j0 + cb;
#pragma unroll
            for (int q4 = 0; q4 < CPT / 4; ++q4) {
                const f32x4 sv = *reinterpret_cast<const f32x4 *>(Sg + 4 * q4);
                const f32x4 dv4 = *reinterpret_cast<const f32x4 *>(Dg + 4 * q4);
#pragma unroll
                for (int i = 0; i < 4; ++i) dgp += sv[i] * dv4[i];
                const Split4 ss = split4(sv), ds = split4(dv4);
                *reinterpret_cast<bf16x4 *>(&S2[cA * PC + cb + 4 * q4]) = ss.hi;
                *reinterpret_cast<bf16x4 *>(&S2[DK * PC + cA * PC + cb + 4 * q4]) = ss.lo;
                *reinterpret_cast<bf16x4 *>(&D2[cA * PC + cb + 4 * q4]) = ds.hi;
                *reinterpret_cast<bf16x4 *>(&D2[DK * PC + cA * PC + cb + 4 * q4]) = ds.lo;
            }
            const int cB = tid % VT, chb = (tid / VT) * CPT;
#pragma unroll
            for (int q4 = 0; q4 < CPT / 4; ++q4) {
                f32x4 sv, dv4;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sv[i] = a.states[stoff + (size_t)(chb + 4 * q4 + i) * DV + j0 + cB];
                    dv4[i] = a.dstates[stoff + (size_t)(chb + 4 * q4 + i) * DV + j0 + cB];
                }
                const Split4 ss = split4(sv), ds = split4(dv4);
                *reinterpret_cast<bf16x4 *>(&S1[cB * PK + chb + 4 * q4]) = ss.hi;
                *reinterpret_cast<bf16x4 *>(&S1[VT * PK + cB * PK + chb + 4 * q4]) = ss.lo;
                *reinterpret_cast<bf16x4 *>(&D1[cB * PK + chb + 4 * q4]) = ds.hi;
                *reinterpret_cast<bf16x4 *>(&D1[VT * PK + cB * PK + chb + 4 * q4]) = ds.lo;
            }
        }
        // dO tile, both layouts
        {
            const int col = tid % VT, tg = tid / VT;   // 8 tokens per thread
            f32x4 x0, x1;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = t0 + 8 * tg + i;
                const float vv = a.dO[baseV0 + (size_t)(t < T ? t : T - 1) * tokV + j0 + col];
                if (i < 4) x0[i] = t < T ? vv : 0.f;
                else x1[i - 4] = t < T ? vv : 0.f;
            }
            const Split4 p0 = split4(x0), p1 = split4(x1);
            *reinterpret_cast<bf16x4 *>(&O1[col * PT + 8 * tg]) = p0.hi;
            *reinterpret_cast<bf16x4 *>(&O1[col * PT + 8 * tg + 4]) = p1.hi;
            *reinterpret_cast<bf16x4 *>(&O1[VT * PT + col * PT + 8 * tg]) = p0.lo;
            *reinterpret_cast<bf16x4 *>(&O1[VT * PT + col * PT + 8 * tg + 4]) = p1.lo;
            const int tok = tid / 4, cq = (tid % 4) * 8;
            const int t = t0 + tok;
            const float *src = a.dO + baseV0 + (size_t)(t < T ? t : T - 1) * tokV + j0 + cq;
            f32x4 y0 = *reinterpret_cast<const f32x4 *>(src), y1 = *reinterpret_cast<const f32x4 *>(src + 4);
            if (!(t < T)) y0 = y1 = f32x4{0.f, 0.f, 0.f, 0.f};
            const Split4 q0 = split4(y0), q1 = split4(y1);
            *reinterpret_cast<bf16x4 *>(&O2[tok * PC + cq]) = q0.hi;
            *reinterpret_cast<bf16x4 *>(&O2[tok * PC + cq + 4]) = q1.hi;
            *reinterpret_cast<bf16x4 *>(&O2[kChunk * PC + tok * PC + cq]) = q0.lo;
            *reinterpret_cast<bf16x4 *>(&O2[kChunk * PC + tok * PC + cq + 4]) = q1.lo;
        }
        // v, w of this wave's rows in D layout
        float vD[NVT][4], wD[NVT][4];
#pragma unroll
        for (int n = 0; n < NVT; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * w + 4 * g + i;
                const size_t off = baseV0 + (size_t)(t < T ? t : T - 1) * tokV + j0 + 16 * n + r;
                const float vv = BF16 ? bf16_bits_to_float(reinterpret_cast<const uint16_t *>(a.v)[off])
                                      : reinterpret_cast<const float *>(a.v)[off];
                const float ww = a.wg[off];
                vD[n][i] = t < T ? vv : 0.f;
                wD[n][i] = t < T ? ww : 0.f;
            }
        __syncthreads();

        // X = Z - Et S
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
            f32x4 acc = {-wD[n][0] * vD[n][0], -wD[n][1] * vD[n][1], -wD[n][2] * vD[n][2], -wD[n][3] * vD[n][3]};
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                const Split8 sf = row_frag4<PK>(S1, S1 + VT * PK, 16 * n + r, j, g);
                if (FAST) acc = mfma32(Ekeep[j].hi, sf.hi, acc);
                else acc = mfma32x3(Ekeep[j], sf, acc);
            }
            const Split4 sp = split4(-acc);
            *reinterpret_cast<bf16x4 *>(&X1[(16 * n + r) * PT + 16 * w + 4 * g]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&X1[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = sp.lo;
        }
        __syncthreads();
        // U = T X  -> [token][col];  dU = P^T dO + Kh dS' -> [col][token]
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk < nkk) {
                    const f32x4 ta = *reinterpret_cast<const f32x4 *>(&sT[(16 * w + r) * PA + 32 * kk + 8 * g]);
                    const f32x4 tb = *reinterpret_cast<const f32x4 *>(&sT[(16 * w + r) * PA + 32 * kk + 8 * g + 4]);
                    acc = mfma32x3(split8v(ta, tb), frag_8(&X1[(16 * n + r) * PT + 32 * kk + 8 * g],
                                                          &X1[VT * PT + (16 * n + r) * PT + 32 * kk + 8 * g]), acc);
                }
            }
            const Split4 su = split4(acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                U2[(16 * w + 4 * g + i) * PC + 16 * n + r] = su.hi[i];
                U2[kChunk * PC + (16 * w + 4 * g + i) * PC + 16 * n + r] = su.lo[i];
            }
            f32x4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk >= kk_lo) {
                    const Split8 of = frag_2x4(&O1[(16 * n + r) * PT + 32 * kk + 4 * g],
                                               &O1[(16 * n + r) * PT + 32 * kk + 16 + 4 * g],
                                               &O1[VT * PT + (16 * n + r) * PT + 32 * kk + 4 * g],
                                               &O1[VT * PT + (16 * n + r) * PT + 32 * kk + 16 + 4 * g]);
                    du = mfma32x3(join(Pt[2 * kk], Pt[2 * kk + 1]), of, du);
                }
            }
#pragma unroll
            for (int j = 0; j < NKS; ++j) du = mfma32x3(Hkeep[j], row_frag4<PK>(D1, D1 + VT * PK, 16 * n + r, j, g), du);
            const Split4 sd = split4(du);
            *reinterpret_cast<bf16x4 *>(&dU1[(16 * n + r) * PT + 16 * w + 4 * g]) = sd.hi;
            *reinterpret_cast<bf16x4 *>(&dU1[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = sd.lo;
        }
        __syncthreads();
        // dX = T^T dU; dv, dw; -dX -> [token][col]
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk >= kk_lo) {
                    float tv[8];
#pragma unroll
                    for (int s = 0; s < 8; ++s) tv[s] = sT[(32 * kk + 8 * g + s) * PA + 16 * w + r];
                    acc = mfma32x3(split8(tv), frag_8(&dU1[(16 * n + r) * PT + 32 * kk + 8 * g],
                                                      &dU1[VT * PT + (16 * n + r) * PT + 32 * kk + 8 * g]), acc);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * w + 4 * g + i;
                if (t < T) {
                    const size_t off = baseV0 + (size_t)t * tokV + j0 + 16 * n + r;
                    a.dv[off] = acc[i] * wD[n][i];
                    a.dw[off] = acc[i] * vD[n][i];
                }
            }
            const Split4 sx = split4(-acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dX2[(16 * w + 4 * g + i) * PC + 16 * n + r] = sx.hi[i];
                dX2[kChunk * PC + (16 * w + 4 * g + i) * PC + 16 * n + r] = sx.lo[i];
            }
        }
        __syncthreads();
        // key-side accumulators (sums over this tile's value columns)
        {
            const Split8 oq = frag_8(&O2[(16 * w + r) * PC + 8 * g], &O2[kChunk * PC + (16 * w + r) * PC + 8 * g]);
            const Split8 xq = frag_8(&dX2[(16 * w + r) * PC + 8 * g], &dX2[kChunk * PC + (16 * w + r) * PC + 8 * g]);
            const Split8 uq = frag_8(&U2[(16 * w + r) * PC + 8 * g], &U2[kChunk * PC + (16 * w + r) * PC + 8 * g]);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const Split8 sf = frag_8(&S2[(16 * m + r) * PC + 8 * g], &S2[DK * PC + (16 * m + r) * PC + 8 * g]);
                aQ[m] = mfma32x3(sf, oq, aQ[m]);   // (dO S^T)^T
                aE[m] = mfma32x3(sf, xq, aE[m]);   // (-dX S^T)^T
                const Split8 df = frag_8(&D2[(16 * m + r) * PC + 8 * g], &D2[DK * PC + (16 * m + r) * PC + 8 * g]);
                aH[m] = mfma32x3(df, uq, aH[m]);   // (U dS'^T)^T
            }
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                if (n <= w) {
                    const Split8 uk = frag_8(&U2[(16 * n + r) * PC + 8 * g], &U2[kChunk * PC + (16 * n + r) * PC + 8 * g]);
                    aP[n] = mfma32x3(oq, uk, aP[n]);   // dO U^T
                    aA[n] = mfma32x3(xq, uk, aA[n]);   // -dX U^T
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue: dgamma, masks, the A/P terms ----
    sDG[tid] = dgp;
    // dP = lower(dO U^T), dA = strictly-lower(-dX U^T) rows 16w + 4g + i, key cols 16n + r
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qry = 16 * w + 4 * g + i, key = 16 * n + r;
            if (!(key <= qry)) aP[n][i] = 0.f;
            if (!(key < qry)) aA[n][i] = 0.f;
        }
    // key-side operands again (4-group layout), from a fresh read of the inputs
    auto reload_ops = [&](float *sTotBuf, KeyOps<NKS> &o2, auto want_k) {
        KeyRaw4<DK, BF16> raw;
        raw.issue(a, rowK, g, vk);
        float qf[NE], kf[NE], laf[NE], bgf[NE], G[NE], gC[NE];
        raw.unpack(qf, kf, laf, bgf);
#pragma unroll
        for (int e = 0; e < NE; ++e) G[e] = laf[e] * kLog2e;
        chunk_scan<NE, DK>(G, gC, sTotBuf, w, r, [&](int e) { return ch4(e, g); });
        if constexpr (decltype(want_k)::value) key_operands<NE, false, false, true, false>(qf, kf, bgf, G, gC, o2);
        else key_operands<NE, true, true, false, false>(qf, kf, bgf, G, gC, o2);
    };
    {
        __bf16 *KtT = sZ, *dP1 = sZ + 2 * RT, *dA1 = sZ + 2 * RT + 2 * kChunk * PT;
        {
            KeyOps<NKS> o2;
            reload_ops(sTot, o2, std::true_type{});
            store_cols<NKS, PT>(o2.K, KtT, KtT + RT, 16 * w + r, g, false);
        }
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const Split4 sp = split4(aP[n]), sa = split4(aA[n]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * w + 4 * g + i;
                dP1[row * PT + 16 * n + r] = sp.hi[i];
                dP1[kChunk * PT + row * PT + 16 * n + r] = sp.lo[i];
                dA1[row * PT + 16 * n + r] = sa.hi[i];
                dA1[kChunk * PT + row * PT + 16 * n + r] = sa.lo[i];
            }
        }
        __syncthreads();
        // dQt^T += Kt^T dP^T ;  dEt^T += Kt^T dA^T
#pragma unroll
        for (int m = 0; m < NM; ++m) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk < nkk) {
                    const Split8 kt = frag_8(&KtT[(16 * m + r) * PT + 32 * kk + 8 * g], &KtT[RT + (16 * m + r) * PT + 32 * kk + 8 * g]);
                    aQ[m] = mfma32x3(kt, frag_8(&dP1[(16 * w + r) * PT + 32 * kk + 8 * g],
                                                &dP1[kChunk * PT + (16 * w + r) * PT + 32 * kk + 8 * g]), aQ[m]);
                    aE[m] = mfma32x3(kt, frag_8(&dA1[(16 * w + r) * PT + 32 * kk + 8 * g],
                                                &dA1[kChunk * PT + (16 * w + r) * PT + 32 * kk + 8 * g]), aE[m]);
                }
            }
        }
        __syncthreads();
    }
    f32x4 aK[NM];
    {
        __bf16 *QtT = sZ, *EtT = sZ + 2 * RT, *dPt = sZ + 4 * RT, *dAt = sZ + 4 * RT + 2 * kChunk * PT;
        {
            KeyOps<NKS> o2;
            reload_ops(sTot2, o2, std::false_type{});
            store_cols<NKS, PT>(o2.Q, QtT, QtT + RT, 16 * w + r, g, false);
            store_cols<NKS, PT>(o2.E, EtT, EtT + RT, 16 * w + r, g, false);
        }
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const Split4 sp = split4(aP[n]), sa = split4(aA[n]);
            *reinterpret_cast<bf16x4 *>(&dPt[(16 * n + r) * PT + 16 * w + 4 * g]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&dPt[kChunk * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = sp.lo;
            *reinterpret_cast<bf16x4 *>(&dAt[(16 * n + r) * PT + 16 * w + 4 * g]) = sa.hi;
            *reinterpret_cast<bf16x4 *>(&dAt[kChunk * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = sa.lo;
        }
        __syncthreads();
        // dKt^T = Qt^T dP + Et^T dA   (columns = this wave's keys)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk >= kk_lo) {
                    acc = mfma32x3(frag_8(&QtT[(16 * m + r) * PT + 32 * kk + 8 * g], &QtT[RT + (16 * m + r) * PT + 32 * kk + 8 * g]),
                                   frag_8(&dPt[(16 * w + r) * PT + 32 * kk + 8 * g], &dPt[kChunk * PT + (16 * w + r) * PT + 32 * kk + 8 * g]),
                                   acc);
                    acc = mfma32x3(frag_8(&EtT[(16 * m + r) * PT + 32 * kk + 8 * g], &EtT[RT + (16 * m + r) * PT + 32 * kk + 8 * g]),
                                   frag_8(&dAt[(16 * w + r) * PT + 32 * kk + 8 * g], &dAt[kChunk * PT + (16 * w + r) * PT + 32 * kk + 8 * g]),
                                   acc);
                }
            }
            aK[m] = acc;
        }
    }

    // ---- element-wise chain (4-group layout: token 16w + r, channel ch4(e, g)) ----
    // The four key-side gradient accumulators are parked in LDS (each thread
    // reads back only its own values, so no barrier is needed) to keep the
    // chain's register footprint small.
    __syncthreads();
    float *sAcc = reinterpret_cast<float *>(sZ);   // [4][NE][kThreads]
    static_assert(4 * NE * kThreads * 4 <= ZSIZE * 2, "accumulator park does not fit");
#pragma unroll
    for (int e = 0; e < NE; ++e) {
        const int m = e >> 2, i = e & 3;
        sAcc[(0 * NE + e) * kThreads + tid] = aQ[m][i];
        sAcc[(1 * NE + e) * kThreads + tid] = aE[m][i];
        sAcc[(2 * NE + e) * kThreads + tid] = aK[m][i];
        sAcc[(3 * NE + e) * kThreads + tid] = aH[m][i];
    }
    float qf[NE], kf[NE], laf[NE], bgf[NE], G[NE], gC[NE];
    {
        KeyRaw4<DK, BF16> raw;
        raw.issue(a, rowK, g, vk);
        raw.unpack(qf, kf, laf, bgf);
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) G[e] = laf[e] * kLog2e;
    chunk_scan<NE, DK>(G, gC, sTot, w, r, [&](int e) { return ch4(e, g); });  // barrier orders sDG too
    float xg[NE], yh[NE];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        f32x4 vq, vk4, vb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * m + i;
            const float eg = exp2_fast(G[e]), eng = exp2_fast(-G[e]), ek = exp2_fast(gC[e] - G[e]);
            const float Qt = qf[e] * eg, Et = bgf[e] * kf[e] * eg, Kt = kf[e] * eng, Kh = kf[e] * ek;
            const float dQt = sAcc[(0 * NE + e) * kThreads + tid];
            const float dEt = sAcc[(1 * NE + e) * kThreads + tid];
            const float dKt = sAcc[(2 * NE + e) * kThreads + tid];
            const float dKh = sAcc[(3 * NE + e) * kThreads + tid];
            vq[i] = dQt * eg;
            const float dE = dEt * eg;
            vb[i] = dE * kf[e];
            vk4[i] = dKt * eng + dKh * ek + dE * bgf[e];
            xg[e] = dQt * Qt + dEt * Et - dKt * Kt - dKh * Kh;
            yh[e] = dKh * Kh;
        }
        if (vk) {
            const size_t off = rowK + 16 * m + 4 * g;
            *reinterpret_cast<f32x4 *>(a.dq + off) = vq;
            *reinterpret_cast<f32x4 *>(a.dk + off) = vk4;
            *reinterpret_cast<f32x4 *>(a.db + off) = vb;
        }
    }
    // dlog_alpha_t = sum_{s >= t} dG_s + dg_C, with dg_C = sum_s dKh_s*Kh_s + dgamma*gamma
    float xin[NE], xtot[NE], ytot[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) xin[e] = xg[e];
    chunk_scan<NE, DK>(xin, xtot, sTot2, w, r, [&](int e) { return ch4(e, g); });
    chunk_scan<NE, DK>(yh, ytot, sTot3, w, r, [&](int e) { return ch4(e, g); });
    if (vk) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            f32x4 vl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = 4 * m + i, ch = ch4(e, g);
                float dgam = 0.f;
#pragma unroll
                for (int p = 0; p < TPC; ++p) dgam += sDG[ch * TPC + p];
                vl[i] = (xtot[e] - xin[e] + xg[e]) + ytot[e] + dgam * exp2_fast(gC[e]);
            }
            *reinterpret_cast<f32x4 *>(a.dla + rowK + 16 * m + 4 * g) = vl;
        }
    }
}

// ---------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------
template <int DK, int VT, bool BF16>
static hipError_t rev_t(const BwdArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((bwd_reverse_kernel<DK, VT, BF16>), dim3((unsigned)(a.B * a.H * a.nvt)), dim3(kThreads), 0,
                       st, a);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t rev_dk(const BwdArgs &a, int dk, int vt, hipStream_t st) {
    switch (dk) {
        case 32: return vt == 32 ? rev_t<32, 32, BF16>(a, st) : hipErrorInvalidValue;
        case 64: return vt == 16 ? rev_t<64, 16, BF16>(a, st) : vt == 32 ? rev_t<64, 32, BF16>(a, st) : hipErrorInvalidValue;
        case 128: return vt == 16 ? rev_t<128, 16, BF16>(a, st) : vt == 32 ? rev_t<128, 32, BF16>(a, st) : hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

int bwd_value_tile(int B, int H, int dk, int dv) {
    int vt = dv < 32 ? dv : 32;
    if (vt == 32 && dk >= 64 && (long)B * H * (dv / 32) < 256) vt = 16;
    return vt;
}

hipError_t launch_bwd_reverse(const BwdArgs &a, int dk, int vt, bool bf16, hipStream_t st) {
    return bf16 ? rev_dk<true>(a, dk, vt, st) : rev_dk<false>(a, dk, vt, st);
}

template <int DK, bool BF16>
static hipError_t chunk_t(const BwdArgs &a, hipStream_t st) {
    const int NC = (a.T + kChunk - 1) / kChunk;
    hipLaunchKernelGGL((bwd_chunk_kernel<DK, BF16>), dim3((unsigned)(a.B * a.H * NC)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_bwd_chunk(const BwdArgs &a, int dk, bool bf16, hipStream_t st) {
    if (a.DV % 32 != 0) return hipErrorInvalidValue;
    switch (dk) {
        case 32: return bf16 ? chunk_t<32, true>(a, st) : chunk_t<32, false>(a, st);
        case 64: return bf16 ? chunk_t<64, true>(a, st) : chunk_t<64, false>(a, st);
        case 128: return bf16 ? chunk_t<128, true>(a, st) : chunk_t<128, false>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn2
