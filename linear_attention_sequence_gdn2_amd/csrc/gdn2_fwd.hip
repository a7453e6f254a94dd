// gdn2_fwd.hip -- fused chunkwise-WY forward sweep of the Gated DeltaNet-2 rule on gfx950.
//
// Rule (iplexlaw.co.kr blog on Gated DeltaNet-2, section "Independent control on
// two axes"): e = b*k, z = w*v, Sbar = diag(alpha) S, r = Sbar^T e,
// S = Sbar + k (z - r)^T, o = S^T q with the updated S.
//
// Chunk form used here (64 tokens; same blog, section "Token path and parallel
// training": cumulative channel decay absorbed into asymmetric erase factors,
// a triangular solve and dense products).  For a chunk with start state S and
// G = inclusive cumsum of log_alpha over the chunk's tokens (per key channel),
// g_C = G of the last token, gamma = exp(g_C):
//     Et = (b*k) * exp(G)      Kt = k * exp(-G)      Qt = q * exp(G)
//     Kh = k * exp(g_C - G)
//     A  = strictly-lower(Et Kt^T)      P = lower(Qt Kt^T)   (query reads the
//                                                              updated state)
//     U  = (I + A)^-1 (Z - Et S)        with Z = w * v
//     O  = Qt S + P U
//     S' = diag(gamma) S + Kh^T U
// Unrolling the per-token rule inside a chunk gives exactly these equations.
//
// Work decomposition: one workgroup (4 waves) per (batch, head, value tile of
// VT columns).  Value columns of S evolve independently, so tiles need no
// exchange; the key-side work (cumsum, A, P, the solve) is repeated per tile.
// Wave w owns tokens 16w..16w+15 of the chunk for the key-side element work and
// the rows of A, P, X, U and O; the fp32 state stays in registers (D layout),
// with a split-bf16 copy in LDS as the MFMA operand of the next chunk.
#include "gdn2_chunk.h"
#include "gdn2_kernels.h"

namespace gdn2 {

template <int DK, int VT, bool BF16, bool FAST, bool OUT, bool STATES>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(FwdArgs a) {
    constexpr int NKS = DK / 32;           // 32-channel contraction steps
    constexpr int NVT = VT / 16;           // 16-column value tiles
    constexpr int NMT = DK / 16;           // 16-row key tiles of S
    constexpr int NTS = NMT * NVT / 4;     // S tiles per wave
    static_assert((NMT * NVT) % 4 == 0, "S tiles must split over 4 waves");
    constexpr int PK = DK + 8;             // row pitch of [row][channel] bf16 tiles
    constexpr int PT = kChunk + 8;         // row pitch of [row][token] bf16 tiles
    constexpr int PA = kChunk + 4;         // row pitch of fp32 64x64 tiles
    constexpr int R1 = (DK * PT > kChunk * PK) ? DK * PT : kChunk * PK;

    // R1 holds Kt [token][channel] (hi, lo) until A and P are formed, then
    // Kh^T [channel][token] (hi, lo) for the state update.
    __shared__ __align__(16) __bf16 sR1[2 * R1];
    __shared__ __align__(16) __bf16 sS[2 * VT * PK];   // S^T [col][channel] hi, lo
    __shared__ __align__(16) __bf16 sXU[2 * VT * PT];  // X^T then U^T [col][token] hi, lo
    __shared__ __align__(16) float sA[kChunk * PA];
    __shared__ __align__(16) float sT[kChunk * PA];
    __shared__ __align__(16) float sTot[4 * DK];
    __shared__ __align__(16) float sGC[DK];

    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
    const int L = xcd_swizzle(blockIdx.x, gridDim.x);
    const int vt = L % a.nvt, bh = L / a.nvt, h = bh % a.H, b = bh / a.H;
    const int T = a.T, H = a.H, DV = a.dv;
    const int j0 = vt * VT;
    const size_t tokK = (size_t)H * DK, tokV = (size_t)H * DV;
    const size_t baseK = ((size_t)b * T * H + h) * DK;
    const size_t baseV = ((size_t)b * T * H + h) * DV + j0;
    const size_t sbase = ((size_t)b * H + h) * (size_t)DK * DV + j0;
    const int NC = (T + kChunk - 1) / kChunk;

    // ---- start state ----
    f32x4 S[NTS];
#pragma unroll
    for (int s = 0; s < NTS; ++s) {
        const int id = w * NTS + s, m = id / NVT, n = id % NVT;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[s][i] = a.S0 ? a.S0[sbase + (size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] : 0.f;
    }
    for (int idx = tid; idx < kChunk * PA; idx += kThreads) sT[idx] = 0.f;

    auto store_state_lds = [&]() {
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT, n = id % NVT;
            const Split4 sp = split4(S[s]);
            *reinterpret_cast<bf16x4 *>(&sS[(16 * n + r) * PK + 16 * m + 4 * g]) = sp.hi;
            *reinterpret_cast<bf16x4 *>(&sS[VT * PK + (16 * n + r) * PK + 16 * m + 4 * g]) = sp.lo;
        }
    };
    store_state_lds();
    __syncthreads();

    // Raw inputs of one chunk held in registers: the loads for chunk c + 1 are
    // issued once chunk c's inputs have been consumed, so their latency hides
    // behind the rest of chunk c's work.
    struct Raw {
        uint4 q[NKS], k[NKS];
        float4 la[NKS][2], bg[NKS][2];
        float4 qx[NKS][2], kx[NKS][2];   // fp32 q/k when the inputs are fp32
        float w[NVT][4];
        uint32_t v[NVT][4];               // raw bits (bf16 in the low half, or fp32)
        bool vk;                          // this lane's key-side token exists
        uint32_t vmask;                   // bit (4n+i): value-side token exists

        // Loads are unconditional, from addresses clamped into the tensors, so
        // that no branch (and no early wait) separates them; tokens past the
        // end are zeroed when the registers are unpacked.
        // decay and erase gate (the largest inputs) of the chunk starting at t0
        __device__ __forceinline__ void issue_gates(const FwdArgs &a, int t0, int T, int w_, int r_, int g_,
                                                    size_t baseK, size_t tokK) {
            const int tk = t0 + 16 * w_ + r_;
            vk = tk < T;
            const size_t offk = baseK + (size_t)(vk ? tk : T - 1) * tokK + 8 * g_;
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                const size_t o = offk + 32 * j;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    la[j][hh] = reinterpret_cast<const float4 *>(a.la + o)[hh];
                    bg[j][hh] = reinterpret_cast<const float4 *>(a.bg + o)[hh];
                }
            }
        }

        // q, k (key side) and v, w (value side) of the chunk starting at t0
        __device__ __forceinline__ void issue_qkvw(const FwdArgs &a, int t0, int T, int w_, int r_, int g_,
                                                   size_t baseK, size_t tokK, size_t baseV, size_t tokV) {
            const int tk = t0 + 16 * w_ + r_;
            const bool vkk = tk < T;
            const size_t offk = baseK + (size_t)(vkk ? tk : T - 1) * tokK + 8 * g_;
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                const size_t o = offk + 32 * j;
                if (BF16) {
                    if (OUT) q[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.q) + o);
                    k[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.k) + o);
                } else {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        if (OUT) qx[j][hh] = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.q) + o)[hh];
                        kx[j][hh] = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.k) + o)[hh];
                    }
                }
            }
            vmask = 0;
#pragma unroll
            for (int n = 0; n < NVT; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tv = t0 + 16 * w_ + 4 * g_ + i;
                    const bool vv = tv < T;
                    vmask |= vv ? (1u << (4 * n + i)) : 0u;
                    const size_t off = baseV + (size_t)(vv ? tv : T - 1) * tokV + 16 * n + r_;
                    w[n][i] = a.wg[off];
                    if (BF16) v[n][i] = reinterpret_cast<const uint16_t *>(a.v)[off];
                    else v[n][i] = reinterpret_cast<const uint32_t *>(a.v)[off];
                }
        }

        __device__ __forceinline__ void unpack(float (&qf)[NKS][8], float (&kf)[NKS][8], float (&laf)[NKS][8],
                                               float (&bgf)[NKS][8], float (&z)[NVT][4]) const {
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                if (BF16) {
                    const uint32_t qw[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
                    const uint32_t kw[4] = {k[j].x, k[j].y, k[j].z, k[j].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (OUT) {
                            qf[j][2 * i] = __builtin_bit_cast(float, qw[i] << 16);
                            qf[j][2 * i + 1] = __builtin_bit_cast(float, qw[i] & 0xffff0000u);
                        }
                        kf[j][2 * i] = __builtin_bit_cast(float, kw[i] << 16);
                        kf[j][2 * i + 1] = __builtin_bit_cast(float, kw[i] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        if (OUT) {
                            qf[j][4 * hh + 0] = qx[j][hh].x; qf[j][4 * hh + 1] = qx[j][hh].y;
                            qf[j][4 * hh + 2] = qx[j][hh].z; qf[j][4 * hh + 3] = qx[j][hh].w;
                        }
                        kf[j][4 * hh + 0] = kx[j][hh].x; kf[j][4 * hh + 1] = kx[j][hh].y;
                        kf[j][4 * hh + 2] = kx[j][hh].z; kf[j][4 * hh + 3] = kx[j][hh].w;
                    }
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    laf[j][4 * hh + 0] = la[j][hh].x; laf[j][4 * hh + 1] = la[j][hh].y;
                    laf[j][4 * hh + 2] = la[j][hh].z; laf[j][4 * hh + 3] = la[j][hh].w;
                    bgf[j][4 * hh + 0] = bg[j][hh].x; bgf[j][4 * hh + 1] = bg[j][hh].y;
                    bgf[j][4 * hh + 2] = bg[j][hh].z; bgf[j][4 * hh + 3] = bg[j][hh].w;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (OUT) qf[j][i] = vk ? qf[j][i] : 0.f;
                    kf[j][i] = vk ? kf[j][i] : 0.f;
                    laf[j][i] = vk ? laf[j][i] : 0.f;
                    bgf[j][i] = vk ? bgf[j][i] : 0.f;
                }
            }
#pragma unroll
            for (int n = 0; n < NVT; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float vf = BF16 ? __builtin_bit_cast(float, v[n][i] << 16) : __builtin_bit_cast(float, v[n][i]);
                    z[n][i] = ((vmask >> (4 * n + i)) & 1u) ? w[n][i] * vf : 0.f;
                }
        }
    };
    Raw raw;
    raw.issue_gates(a, 0, T, w, r, g, baseK, tokK);
    raw.issue_qkvw(a, 0, T, w, r, g, baseK, tokK, baseV, tokV);

    for (int c = 0; c < NC; ++c) {
        const int t0 = c * kChunk;
        if (STATES) {
            float *dst = a.states + (((size_t)b * H + h) * NC + c) * (size_t)DK * DV + j0;
#pragma unroll
            for (int s = 0; s < NTS; ++s) {
                const int id = w * NTS + s, m = id / NVT, n = id % NVT;
#pragma unroll
                for (int i = 0; i < 4; ++i) dst[(size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] = S[s][i];
            }
        }

        // ---- this chunk's inputs (loaded during the previous chunk) ----
        float qf[NKS][8], kf[NKS][8], laf[NKS][8], bgf[NKS][8], z[NVT][4];
        raw.unpack(qf, kf, laf, bgf, z);

        // ---- cumulative log2-decay over the chunk (fp32) ----
        float G[NKS][8];
#pragma unroll
        for (int j = 0; j < NKS; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) G[j][i] = row_scan16(laf[j][i] * kLog2e);
        if (r == 15) {
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                *reinterpret_cast<float4 *>(&sTot[w * DK + 32 * j + 8 * g]) =
                    make_float4(G[j][0], G[j][1], G[j][2], G[j][3]);
                *reinterpret_cast<float4 *>(&sTot[w * DK + 32 * j + 8 * g + 4]) =
                    make_float4(G[j][4], G[j][5], G[j][6], G[j][7]);
            }
        }
        __syncthreads();
        float gC[NKS][8];
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
#pragma unroll
            for (int i = 0; i < 8; ++i) gC[j][i] = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const float4 u0 = *reinterpret_cast<const float4 *>(&sTot[w2 * DK + 32 * j + 8 * g]);
                const float4 u1 = *reinterpret_cast<const float4 *>(&sTot[w2 * DK + 32 * j + 8 * g + 4]);
                const float tv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    gC[j][i] += tv[i];
                    if (w2 < w) G[j][i] += tv[i];
                }
            }
            if (w == 0 && r == 0) {
                *reinterpret_cast<float4 *>(&sGC[32 * j + 8 * g]) =
                    make_float4(gC[j][0], gC[j][1], gC[j][2], gC[j][3]);
                *reinterpret_cast<float4 *>(&sGC[32 * j + 8 * g + 4]) =
                    make_float4(gC[j][4], gC[j][5], gC[j][6], gC[j][7]);
            }
        }

        // ---- decay absorption and gating (fp32), split into MFMA operands ----
        Split8 Et[NKS], Qt[NKS], Kh[NKS];
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
            float et[8], qt[8], kt[8], kh[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float eg = exp2_fast(G[j][i]);
                const float eng = exp2_fast(-G[j][i]);
                const float ek = exp2_fast(gC[j][i] - G[j][i]);
                et[i] = bgf[j][i] * kf[j][i] * eg;
                qt[i] = OUT ? qf[j][i] * eg : 0.f;
                kt[i] = kf[j][i] * eng;
                kh[i] = kf[j][i] * ek;
            }
            Et[j] = split8(et);
            if (OUT) Qt[j] = split8(qt);
            Kh[j] = split8(kh);
            const Split8 ks = split8(kt);
            *reinterpret_cast<bf16x8 *>(&sR1[(16 * w + r) * PK + 32 * j + 8 * g]) = ks.hi;
            *reinterpret_cast<bf16x8 *>(&sR1[R1 + (16 * w + r) * PK + 32 * j + 8 * g]) = ks.lo;
        }
        if (c + 1 < NC) raw.issue_gates(a, t0 + kChunk, T, w, r, g, baseK, tokK);
        __syncthreads();

        // ---- A^T and P^T for this wave's query rows (keys from LDS) ----
        Split4 Pf[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (mt <= w) {
                f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < NKS; ++j) {
                    Split8 kt;
                    kt.hi = *reinterpret_cast<const bf16x8 *>(&sR1[(16 * mt + r) * PK + 32 * j + 8 * g]);
                    kt.lo = *reinterpret_cast<const bf16x8 *>(&sR1[R1 + (16 * mt + r) * PK + 32 * j + 8 * g]);
                    if (FAST) accA = mfma32(kt.hi, Et[j].hi, accA);
                    else accA = mfma32x3(kt, Et[j], accA);
                    if (OUT) accP = mfma32x3(kt, Qt[j], accP);
                }
                // lane holds A[16w + r][16mt + 4g + i] and P[16w + r][16mt + 4g + i]
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 16 * mt + 4 * g + i, qry = 16 * w + r;
                    if (!(key < qry)) accA[i] = 0.f;
                    if (!(key <= qry)) accP[i] = 0.f;
                }
                *reinterpret_cast<f32x4 *>(&sA[(16 * w + r) * PA + 16 * mt + 4 * g]) = accA;
                if (OUT) Pf[mt] = split4(accP);
            } else if (OUT) {
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                Pf[mt] = split4(zero);
            }
        }

        // ---- X = Z - Et S and Qt S for this wave's rows (S from LDS) ----
        f32x4 QS[NVT];
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
            f32x4 accX = {-z[n][0], -z[n][1], -z[n][2], -z[n][3]};
            f32x4 accQ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NKS; ++j) {
                Split8 sf;
                sf.hi = *reinterpret_cast<const bf16x8 *>(&sS[(16 * n + r) * PK + 32 * j + 8 * g]);
                sf.lo = *reinterpret_cast<const bf16x8 *>(&sS[VT * PK + (16 * n + r) * PK + 32 * j + 8 * g]);
                if (FAST) accX = mfma32(Et[j].hi, sf.hi, accX);
                else accX = mfma32x3(Et[j], sf, accX);
                if (OUT) accQ = mfma32x3(Qt[j], sf, accQ);
            }
            const f32x4 X = -accX;  // lane holds X[16w + 4g + i][16n + r]
            const Split4 xs = split4(X);
            *reinterpret_cast<bf16x4 *>(&sXU[(16 * n + r) * PT + 16 * w + 4 * g]) = xs.hi;
            *reinterpret_cast<bf16x4 *>(&sXU[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = xs.lo;
            QS[n] = accQ;
        }
        __syncthreads();

        if (c + 1 < NC) raw.issue_qkvw(a, t0 + kChunk, T, w, r, g, baseK, tokK, baseV, tokV);

        // ---- Kh^T into R1 (Kt is no longer read) ----
#pragma unroll
        for (int j = 0; j < NKS; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int ch = 32 * j + 8 * g + i;
                sR1[ch * PT + 16 * w + r] = Kh[j].hi[i];
                sR1[R1 + ch * PT + 16 * w + r] = Kh[j].lo[i];
            }

        // ---- T = (I + A)^-1 ----
        solve_T<PA>(sA, sT, w, r, g);

        // ---- U = T X for this wave's rows ----
        const int nkk = (w >= 2) ? 2 : 1;
        f32x4 accU[NVT];
#pragma unroll
        for (int n = 0; n < NVT; ++n) accU[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk < nkk) {
                const f32x4 t0v = *reinterpret_cast<const f32x4 *>(&sT[(16 * w + r) * PA + 32 * kk + 8 * g]);
                const f32x4 t1v = *reinterpret_cast<const f32x4 *>(&sT[(16 * w + r) * PA + 32 * kk + 8 * g + 4]);
                const float tr[8] = {t0v[0], t0v[1], t0v[2], t0v[3], t1v[0], t1v[1], t1v[2], t1v[3]};
                const Split8 ts = split8(tr);
#pragma unroll
                for (int n = 0; n < NVT; ++n) {
                    Split8 xs;
                    xs.hi = *reinterpret_cast<const bf16x8 *>(&sXU[(16 * n + r) * PT + 32 * kk + 8 * g]);
                    xs.lo = *reinterpret_cast<const bf16x8 *>(&sXU[VT * PT + (16 * n + r) * PT + 32 * kk + 8 * g]);
                    accU[n] = mfma32x3(ts, xs, accU[n]);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < NVT; ++n) {
            const Split4 us = split4(accU[n]);
            *reinterpret_cast<bf16x4 *>(&sXU[(16 * n + r) * PT + 16 * w + 4 * g]) = us.hi;
            *reinterpret_cast<bf16x4 *>(&sXU[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = us.lo;
        }
        __syncthreads();

        // ---- O = Qt S + P U (P from registers, key index permuted to match) ----
        if (OUT) {
#pragma unroll
            for (int n = 0; n < NVT; ++n) {
                f32x4 acc = QS[n];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk < nkk) {
                        Split8 pf, us;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            pf.hi[i] = Pf[2 * kk].hi[i];
                            pf.hi[4 + i] = Pf[2 * kk + 1].hi[i];
                            pf.lo[i] = Pf[2 * kk].lo[i];
                            pf.lo[4 + i] = Pf[2 * kk + 1].lo[i];
                        }
                        const __bf16 *uh = &sXU[(16 * n + r) * PT + 32 * kk];
                        const __bf16 *ul = &sXU[VT * PT + (16 * n + r) * PT + 32 * kk];
                        const bf16x4 h0 = *reinterpret_cast<const bf16x4 *>(uh + 4 * g);
                        const bf16x4 h1 = *reinterpret_cast<const bf16x4 *>(uh + 16 + 4 * g);
                        const bf16x4 l0 = *reinterpret_cast<const bf16x4 *>(ul + 4 * g);
                        const bf16x4 l1 = *reinterpret_cast<const bf16x4 *>(ul + 16 + 4 * g);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            us.hi[i] = h0[i];
                            us.hi[4 + i] = h1[i];
                            us.lo[i] = l0[i];
                            us.lo[4 + i] = l1[i];
                        }
                        acc = mfma32x3(pf, us, acc);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int to = t0 + 16 * w + 4 * g + i;
                    if (to < T) a.o[baseV + (size_t)to * tokV + 16 * n + r] = acc[i];
                }
            }
        }

        // ---- S' = diag(gamma) S + Kh^T U (this wave's tiles of S) ----
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT, n = id % NVT;
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = S[s][i] * exp2_fast(sGC[16 * m + 4 * g + i]);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                Split8 kh, us;
                kh.hi = *reinterpret_cast<const bf16x8 *>(&sR1[(16 * m + r) * PT + 32 * kk + 8 * g]);
                kh.lo = *reinterpret_cast<const bf16x8 *>(&sR1[R1 + (16 * m + r) * PT + 32 * kk + 8 * g]);
                us.hi = *reinterpret_cast<const bf16x8 *>(&sXU[(16 * n + r) * PT + 32 * kk + 8 * g]);
                us.lo = *reinterpret_cast<const bf16x8 *>(&sXU[VT * PT + (16 * n + r) * PT + 32 * kk + 8 * g]);
                acc = mfma32x3(kh, us, acc);
            }
            S[s] = acc;
        }
        store_state_lds();
        // the next chunk's first barrier orders these writes before their reads
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

static bool vt_ok(int dk, int vt, int dv) {
    return vt <= dv && dv % vt == 0 && ((dk / 16) * (vt / 16)) % 4 == 0;
}

int fwd_value_tile(int B, int H, int dk, int dv) {
    int vt = dv < 64 ? dv : 64;
    while (vt > 16 && (long)B * H * (dv / vt) < 256 && vt_ok(dk, vt / 2, dv)) vt /= 2;
    return vt;
}

template <int DK, int VT, bool BF16, int MODE>
static hipError_t launch_t(const FwdArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)(a.B * a.H * a.nvt)), block(kThreads);
    constexpr bool OUT = MODE != kFwdStates, STATES = MODE != kFwdOut;
    hipLaunchKernelGGL((fwd_kernel<DK, VT, BF16, BF16, OUT, STATES>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int DK, bool BF16, int MODE>
static hipError_t launch_vt(const FwdArgs &a, int vt, hipStream_t st) {
    if constexpr (DK >= 64) {
        if (vt == 16) return launch_t<DK, 16, BF16, MODE>(a, st);
    }
    if (vt == 32) return launch_t<DK, 32, BF16, MODE>(a, st);
    if (vt == 64) return launch_t<DK, 64, BF16, MODE>(a, st);
    return hipErrorInvalidValue;
}

template <bool BF16, int MODE>
static hipError_t launch_dk(const FwdArgs &a, int dk, int vt, hipStream_t st) {
    switch (dk) {
        case 32: return launch_vt<32, BF16, MODE>(a, vt, st);
        case 64: return launch_vt<64, BF16, MODE>(a, vt, st);
        case 128: return launch_vt<128, BF16, MODE>(a, vt, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
static hipError_t launch_mode(const FwdArgs &a, int dk, int vt, FwdMode mode, hipStream_t st) {
    switch (mode) {
        case kFwdOut: return launch_dk<BF16, kFwdOut>(a, dk, vt, st);
        case kFwdStates: return launch_dk<BF16, kFwdStates>(a, dk, vt, st);
        case kFwdOutStates: return launch_dk<BF16, kFwdOutStates>(a, dk, vt, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fwd(const FwdArgs &a, int dk, int vt, bool bf16, FwdMode mode, hipStream_t st) {
    if (!vt_ok(dk, vt, a.dv)) return hipErrorInvalidValue;
    return bf16 ? launch_mode<true>(a, dk, vt, mode, st) : launch_mode<false>(a, dk, vt, mode, st);
}

}  // namespace gdn2
