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
//     S' = diag(gamma) S + Kh^T U = diag(gamma) (S + Kt^T U)
// (Kh = diag-scaled Kt row by row, so the last form needs no separate Kh.)
// Unrolling the per-token rule inside a chunk gives exactly these equations.
//
// Work decomposition: one workgroup (4 waves) per (batch, head, value tile of
// VT columns).  Value columns of S evolve independently, so tiles need no
// exchange; the key-side work (cumsum, A, P, the solve) is repeated per tile.
// Wave w owns tokens 16w..16w+15 of the chunk for the key-side element work and
// the rows of A, P, X, U and O; the fp32 state stays in registers (D layout),
// with a split-bf16 copy in LDS as the MFMA operand of the next chunk.
// At VT = 32 a workgroup needs under 80 KB of LDS and 256 registers per lane,
// so two workgroups share a CU and hide each other's load and barrier latency.
#include "gdn2_chunk.h"
#include "gdn2_kernels.h"

namespace gdn2 {

// Keep the scheduler from hoisting the next unrolled step's LDS fragment loads
// above this point (bounds the live registers so two workgroups fit on a CU).
#define GDN2_STEP_FENCE() __builtin_amdgcn_sched_barrier(0)

template <int DK, int VT, bool BF16, bool OUT, bool STATES, bool GL, bool SG>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdArgs a) {
    constexpr int NKS = DK / 32;           // 32-channel contraction steps
    constexpr int NVT = VT / 16;           // 16-column value tiles
    constexpr int NMT = DK / 16;           // 16-row key tiles of S
    constexpr int NTS = NMT * NVT / 4;     // S tiles per wave
    static_assert((NMT * NVT) % 4 == 0, "S tiles must split over 4 waves");
    constexpr int PK = DK + 8;             // row pitch of [row][channel] bf16 tiles
    constexpr int PT = kChunk + 8;         // row pitch of [row][token] bf16 tiles
    constexpr int PA = kChunk + 4;         // row pitch of the fp32 64x64 tile
    constexpr int RK = kChunk * PK;        // one [token][channel] plane
    constexpr int RX = 2 * VT * PT > 8 * DK ? 2 * VT * PT : 8 * DK;

    // sK: Kt rows [token][channel] (hi, lo) until A and P are formed, then Kh rows.
    // sXU: per-wave decay totals at the start of a chunk, then X^T, then U^T [col][token].
    // sAT: A, then T = (I + A)^-1 in place.
    __shared__ __align__(16) __bf16 sK[2 * RK];
    __shared__ __align__(16) __bf16 sS[2 * VT * PK];   // S^T [col][channel] hi, lo
    __shared__ __align__(16) __bf16 sXU[RX];
    __shared__ __align__(16) float sAT[kChunk * PA];
    float *sTot = reinterpret_cast<float *>(sXU);

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
    const int nkk = (w >= 2) ? 2 : 1;

    // ---- start state; the strictly upper blocks of sAT stay zero for good ----
    f32x4 S[NTS];
#pragma unroll
    for (int s = 0; s < NTS; ++s) {
        const int id = w * NTS + s, m = id / NVT, n = id % NVT;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[s][i] = a.S0 ? a.S0[sbase + (size_t)(16 * m + 4 * g + i) * DV + 16 * n + r] : 0.f;
    }
    for (int idx = tid; idx < kChunk * PA; idx += kThreads) sAT[idx] = 0.f;
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
    __syncthreads();

    for (int c = 0; c < NC; ++c) {
        // lane indices afresh from an opaque copy of the thread index: the address
        // arithmetic is redone each chunk instead of being held in registers
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
        const int nkk = (w >= 2) ? 2 : 1;
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

        // ---- inputs: key side in token-row layout (channels 32j + 8g + i), value side in D layout ----
        // Loads are unconditional, from addresses clamped into the tensors (no branch, no early
        // wait between them); tokens past the end are zeroed when the values are unpacked.
        const int tk = t0 + 16 * w + r;
        const bool vk = tk < T;
        const size_t offk = baseK + (size_t)(vk ? tk : T - 1) * tokK + 8 * g;
        const size_t offs = baseK / DK + (size_t)(vk ? tk : T - 1) * H;   // the token's per-token gate (SG)
        uint4 qraw[NKS], kraw[NKS];            // bf16 q, k (8 channels per uint4)
        float4 qx[NKS][2], kx[NKS][2];         // fp32 q, k
        float4 la4[NKS][2], bg4[NKS][2];       // fp32 gate values
        uint4 la8[NKS], bg8[NKS];              // bf16 gate logits (GL)
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
            const size_t o = offk + 32 * j;
            if (BF16) {
                if (OUT) qraw[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.q) + o);
                kraw[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.k) + o);
            } else {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    if (OUT) qx[j][hh] = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.q) + o)[hh];
                    kx[j][hh] = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.k) + o)[hh];
                }
            }
            if (GL) {
                la8[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.la) + o);
                bg8[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(a.bg) + o);
            } else if (SG) {
                // a gate given per token is broadcast over the key channels
                if (a.scalar & kScalarDecay) {
                    const float x = reinterpret_cast<const float *>(a.la)[offs];
                    la4[j][0] = la4[j][1] = make_float4(x, x, x, x);
                } else {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        la4[j][hh] = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.la) + o)[hh];
                }
                if (a.scalar & kScalarErase) {
                    const float x = reinterpret_cast<const float *>(a.bg)[offs];
                    bg4[j][0] = bg4[j][1] = make_float4(x, x, x, x);
                } else {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
                        bg4[j][hh] = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.bg) + o)[hh];
                }
            } else {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    la4[j][hh] = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.la) + o)[hh];
                    bg4[j][hh] = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.bg) + o)[hh];
                }
            }
        }
        // 8 gate elements of block j: fp32 values, or bf16 logits widened (activation applied by the caller)
        auto gate8 = [&](const float4 (&fx)[2], const uint4 &raw, float (&out)[8]) {
            if (GL) {
                const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    out[2 * i] = __builtin_bit_cast(float, u[i] << 16);
                    out[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xffff0000u);
                }
            } else {
                out[0] = fx[0].x; out[1] = fx[0].y; out[2] = fx[0].z; out[3] = fx[0].w;
                out[4] = fx[1].x; out[5] = fx[1].y; out[6] = fx[1].z; out[7] = fx[1].w;
            }
        };
        // element i of block j of a packed input row
        auto unpack8 = [&](const uint4 &raw, const float4 (&fx)[2], float (&out)[8]) {
            if (BF16) {
                const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    out[2 * i] = __builtin_bit_cast(float, u[i] << 16);
                    out[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xffff0000u);
                }
            } else {
                out[0] = fx[0].x; out[1] = fx[0].y; out[2] = fx[0].z; out[3] = fx[0].w;
                out[4] = fx[1].x; out[5] = fx[1].y; out[6] = fx[1].z; out[7] = fx[1].w;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) out[i] = vk ? out[i] : 0.f;
        };

        // ---- cumulative log2-decay over the chunk (fp32) ----
        float G[NKS][8];
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
            float lv[8];
            gate8(la4[j], la8[j], lv);
#pragma unroll
            for (int i = 0; i < 8; ++i) G[j][i] = row_scan16(vk ? decay_act<GL>(lv[i]) * kLog2e : 0.f);
        }
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
        // decay of the chunk, gamma = exp(g_C), for the key rows of this wave's state tiles
        float gam[NTS][4];
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = 16 * m + 4 * g + i;
                gam[s][i] = exp2_fast((sTot[ch] + sTot[DK + ch]) + (sTot[2 * DK + ch] + sTot[3 * DK + ch]));
            }
        }

        // ---- decay absorption and gating (fp32), split into MFMA operands, one 32-channel block at a time ----
        Split8 Et[NKS], Qt[NKS];
#pragma unroll
        for (int j = 0; j < NKS; ++j) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                float4 pre = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
                for (int w2 = 0; w2 < 3; ++w2) {
                    if (w2 < w) {
                        const float4 u = *reinterpret_cast<const float4 *>(&sTot[w2 * DK + 32 * j + 8 * g + 4 * hh]);
                        pre.x += u.x; pre.y += u.y; pre.z += u.z; pre.w += u.w;
                    }
                }
                G[j][4 * hh + 0] += pre.x; G[j][4 * hh + 1] += pre.y; G[j][4 * hh + 2] += pre.z; G[j][4 * hh + 3] += pre.w;
            }
            float qv[8], kv[8];
            unpack8(qraw[j], qx[j], qv);
            unpack8(kraw[j], kx[j], kv);
            float bv[8];
            gate8(bg4[j], bg8[j], bv);
#pragma unroll
            for (int i = 0; i < 8; ++i) bv[i] = gate_act<GL>(bv[i]);
            float et[8], qt[8], kt[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float eg = exp2_fast(G[j][i]);
                const float eng = exp2_fast(-G[j][i]);
                et[i] = bv[i] * kv[i] * eg;       // kv is already zero past the end
                qt[i] = OUT ? qv[i] * eg : 0.f;
                kt[i] = kv[i] * eng;
            }
            Et[j] = split8(et);
            if (OUT) Qt[j] = split8(qt);
            const Split8 ks = split8(kt);
            *reinterpret_cast<bf16x8 *>(&sK[(16 * w + r) * PK + 32 * j + 8 * g]) = ks.hi;
            *reinterpret_cast<bf16x8 *>(&sK[RK + (16 * w + r) * PK + 32 * j + 8 * g]) = ks.lo;
            GDN2_STEP_FENCE();
        }
        __syncthreads();

        // ---- A^T and P^T for this wave's query rows (keys from LDS) ----
        Split4 Pf[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (mt <= w) {
                f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < NKS; ++j) {
                    const Split8 kt = frag_8(&sK[(16 * mt + r) * PK + 32 * j + 8 * g],
                                             &sK[RK + (16 * mt + r) * PK + 32 * j + 8 * g]);
                    accA = mfma32x3(kt, Et[j], accA);
                    if (OUT) accP = mfma32x3(kt, Qt[j], accP);
                }
                // lane holds A[16w + r][16mt + 4g + i] and P[16w + r][16mt + 4g + i]
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = 16 * mt + 4 * g + i, qry = 16 * w + r;
                    if (!(key < qry)) accA[i] = 0.f;
                    if (!(key <= qry)) accP[i] = 0.f;
                }
                *reinterpret_cast<f32x4 *>(&sAT[(16 * w + r) * PA + 16 * mt + 4 * g]) = accA;
                if (OUT) Pf[mt] = split4(accP);
            } else if (OUT) {
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                Pf[mt] = split4(zero);
            }
            GDN2_STEP_FENCE();
        }

        // value-side inputs of this wave's rows, D layout (z = w * v)
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
                accX = mfma32x3(Et[j], sf, accX);
                if (OUT) accQ = mfma32x3(Qt[j], sf, accQ);
            }
            const Split4 xs = split4(-accX);  // lane holds X[16w + 4g + i][16n + r]
            *reinterpret_cast<bf16x4 *>(&sXU[(16 * n + r) * PT + 16 * w + 4 * g]) = xs.hi;
            *reinterpret_cast<bf16x4 *>(&sXU[VT * PT + (16 * n + r) * PT + 16 * w + 4 * g]) = xs.lo;
            QS[n] = accQ;
            GDN2_STEP_FENCE();
        }
        __syncthreads();

        // ---- T = (I + A)^-1 ----
        solve_T_inplace<PA>(sAT, w, r, g);

        // ---- U = T X for this wave's rows ----
        f32x4 accU[NVT];
#pragma unroll
        for (int n = 0; n < NVT; ++n) accU[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            if (kk < nkk) {
                const f32x4 t0v = *reinterpret_cast<const f32x4 *>(&sAT[(16 * w + r) * PA + 32 * kk + 8 * g]);
                const f32x4 t1v = *reinterpret_cast<const f32x4 *>(&sAT[(16 * w + r) * PA + 32 * kk + 8 * g + 4]);
                const Split8 ts = split8v(t0v, t1v);
#pragma unroll
                for (int n = 0; n < NVT; ++n)
                    accU[n] = mfma32x3(ts, frag_8(&sXU[(16 * n + r) * PT + 32 * kk + 8 * g],
                                                  &sXU[VT * PT + (16 * n + r) * PT + 32 * kk + 8 * g]), accU[n]);
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

        // ---- O = Qt S + P U (P from registers, key index in the 4-group order) ----
        if (OUT) {
#pragma unroll
            for (int n = 0; n < NVT; ++n) {
                f32x4 acc = QS[n];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    if (kk < nkk) {
                        const __bf16 *uh = &sXU[(16 * n + r) * PT + 32 * kk];
                        const __bf16 *ul = &sXU[VT * PT + (16 * n + r) * PT + 32 * kk];
                        acc = mfma32x3(join(Pf[2 * kk], Pf[2 * kk + 1]),
                                       frag_2x4(uh + 4 * g, uh + 16 + 4 * g, ul + 4 * g, ul + 16 + 4 * g), acc);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int to = t0 + 16 * w + 4 * g + i;
                    if (to < T) a.o[baseV + (size_t)to * tokV + 16 * n + r] = acc[i];
                }
                GDN2_STEP_FENCE();
            }
        }

        // ---- S' = diag(gamma) S + Kh^T U = diag(gamma) (S + Kt^T U), this wave's tiles of S ----
#pragma unroll
        for (int s = 0; s < NTS; ++s) {
            const int id = w * NTS + s, m = id / NVT, n = id % NVT;
            f32x4 acc = S[s];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const Split8 kh = frag_tr<PK>(sK, sK + RK, 32 * kk, 16 * m, r, g);   // Kt^T
                const __bf16 *uh = &sXU[(16 * n + r) * PT + 32 * kk];
                const __bf16 *ul = &sXU[VT * PT + (16 * n + r) * PT + 32 * kk];
                acc = mfma32x3(kh, frag_2x4(uh + 4 * g, uh + 16 + 4 * g, ul + 4 * g, ul + 16 + 4 * g), acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) S[s][i] = acc[i] * gam[s][i];
            GDN2_STEP_FENCE();
        }
        store_state_lds(w, r, g);
        __syncthreads();
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
    // two workgroups fit on a CU at 32-column tiles; aim for >= 512 workgroups
    int vt = dv < 32 ? dv : 32;
    while (vt > 16 && (long)B * H * (dv / vt) < 512 && vt_ok(dk, vt / 2, dv)) vt /= 2;
    return vt;
}

template <int DK, int VT, bool BF16, bool GL, bool SG, int MODE>
static hipError_t launch_t(const FwdArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)(a.B * a.H * a.nvt)), block(kThreads);
    constexpr bool OUT = MODE != kFwdStates, STATES = MODE != kFwdOut;
    hipLaunchKernelGGL((fwd_kernel<DK, VT, BF16, OUT, STATES, GL, SG>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int DK, bool BF16, bool GL, bool SG, int MODE>
static hipError_t launch_vt(const FwdArgs &a, int vt, hipStream_t st) {
    if constexpr (DK >= 64) {
        if (vt == 16) return launch_t<DK, 16, BF16, GL, SG, MODE>(a, st);
    }
    if (vt == 32) return launch_t<DK, 32, BF16, GL, SG, MODE>(a, st);
    if (vt == 64) return launch_t<DK, 64, BF16, GL, SG, MODE>(a, st);
    return hipErrorInvalidValue;
}

template <bool BF16, bool GL, bool SG, int MODE>
static hipError_t launch_dk(const FwdArgs &a, int dk, int vt, hipStream_t st) {
    switch (dk) {
        case 32: return launch_vt<32, BF16, GL, SG, MODE>(a, vt, st);
        case 64: return launch_vt<64, BF16, GL, SG, MODE>(a, vt, st);
        case 128: return launch_vt<128, BF16, GL, SG, MODE>(a, vt, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16, bool GL, bool SG>
static hipError_t launch_mode(const FwdArgs &a, int dk, int vt, FwdMode mode, hipStream_t st) {
    switch (mode) {
        case kFwdOut: return launch_dk<BF16, GL, SG, kFwdOut>(a, dk, vt, st);
        case kFwdStates: return launch_dk<BF16, GL, SG, kFwdStates>(a, dk, vt, st);
        case kFwdOutStates: return launch_dk<BF16, GL, SG, kFwdOutStates>(a, dk, vt, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fwd(const FwdArgs &a, int dk, int vt, bool bf16, bool gl, bool sg, FwdMode mode, hipStream_t st) {
    if (!vt_ok(dk, vt, a.dv)) return hipErrorInvalidValue;
    if (gl && sg) return hipErrorInvalidValue;
    if (gl) return bf16 ? launch_mode<true, true, false>(a, dk, vt, mode, st) : hipErrorInvalidValue;
    if (sg) return bf16 ? launch_mode<true, false, true>(a, dk, vt, mode, st) : hipErrorInvalidValue;
    return bf16 ? launch_mode<true, false, false>(a, dk, vt, mode, st)
                : launch_mode<false, false, false>(a, dk, vt, mode, st);
}

}  // namespace gdn2
