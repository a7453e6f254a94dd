// gdn2_output.hip -- the output epilogue of the Gated DeltaNet-2 operator on gfx950.
//
// The operator's output of each (batch, token, head) goes through an RMS normalisation,
// then an output gate of its own (not the write gate), then the output projection
// (blog on Gated DeltaNet-2, section "Token path and parallel training").  Here, per
// row o (the dv value channels of one (b, t, h)):
//     r = 1 / sqrt(mean_j o_j^2 + eps),   u = o r,   y = u * weight * g
// and, for the backward of sum(dy * y):
//     dg = dy * u * weight,   dweight = sum over rows of dy * u * g,
//     du = dy * weight * g,   do = r (du - u * mean_j(du_j u_j)).
//
// Both directions are one streaming pass over the rows (HBM-bound, no MFMA): DV/4 lanes
// hold one row as float4 columns, the two row sums are lane shuffles within those lanes,
// and each thread keeps several rows' loads in flight.  The chunked forward splits the
// value channels of a head over workgroups, so the normalisation, which needs the whole
// row, cannot run inside it; it runs here, right after it, reading o once.
//
// dweight is a sum over all B*T*H rows: every workgroup of the backward adds its rows
// into per-lane registers and writes one partial row to the workspace; a second small
// kernel adds the partial rows in a fixed order, so the result is reproducible bit for
// bit.
#include "gdn2_device.h"
#include "gdn2_kernels.h"

namespace gdn2 {

namespace {

constexpr int kOutThreads = 256;
constexpr int kOutUnroll = 4;   // rows in flight per thread

template <int DV>
struct OutCfg {
    static constexpr int LPR = DV / 4;                 // lanes per row (one float4 each)
    static constexpr int RPI = kOutThreads / LPR;      // rows per workgroup and unroll step
    static constexpr int RPB = RPI * kOutUnroll;       // rows per workgroup iteration
};

// four gate elements of a row: fp32, or bf16 widened
template <bool GB>
__device__ __forceinline__ float4 load_gate4(const void *g, size_t off) {
    if (GB) {
        const uint2 u = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint16_t *>(g) + off);
        return make_float4(__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xffff0000u),
                           __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xffff0000u));
    }
    return *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(g) + off);
}

// sum over the LPR lanes of a row (LPR divides 64, rows start at multiples of LPR)
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

__device__ __forceinline__ float dot4(const float4 &a, const float4 &b) {
    return (a.x * b.x + a.y * b.y) + (a.z * b.z + a.w * b.w);
}

}  // namespace

template <int DV, bool GB, bool YB>
__global__ __launch_bounds__(kOutThreads) void out_fwd_kernel(OutArgs a) {
    GDN2_POISON_LDS();
    using C = OutCfg<DV>;
    const int lane = threadIdx.x % C::LPR, rg = threadIdx.x / C::LPR;
    const float4 wt = a.weight ? reinterpret_cast<const float4 *>(a.weight)[lane] : make_float4(1.f, 1.f, 1.f, 1.f);
    const long base = (long)blockIdx.x * C::RPB + rg;
    float4 ov[kOutUnroll], gv[kOutUnroll];
#pragma unroll
    for (int u = 0; u < kOutUnroll; ++u) {
        const long row = base + (long)u * C::RPI;
        const size_t off = (size_t)(row < a.rows ? row : a.rows - 1) * DV + 4 * lane;   // clamped: loads issue together
        ov[u] = *reinterpret_cast<const float4 *>(a.o + off);
        gv[u] = load_gate4<GB>(a.g, off);
    }
#pragma unroll
    for (int u = 0; u < kOutUnroll; ++u) {
        const long row = base + (long)u * C::RPI;
        const float r = __builtin_amdgcn_rsqf(row_sum<C::LPR>(dot4(ov[u], ov[u])) * (1.f / DV) + a.eps);
        const float4 y = make_float4(ov[u].x * r * wt.x * gv[u].x, ov[u].y * r * wt.y * gv[u].y,
                                     ov[u].z * r * wt.z * gv[u].z, ov[u].w * r * wt.w * gv[u].w);
        if (row < a.rows) {
            const size_t off = (size_t)row * DV + 4 * lane;
            if (YB) {
                const f32x4 yv = {y.x, y.y, y.z, y.w};
                *reinterpret_cast<bf16x4 *>(reinterpret_cast<__bf16 *>(a.y) + off) =
                    __builtin_convertvector(yv, bf16x4);
            } else {
                *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.y) + off) = y;
            }
        }
    }
}

template <int DV, bool GB>
__global__ __launch_bounds__(kOutThreads) void out_bwd_kernel(OutArgs a) {
    GDN2_POISON_LDS();
    using C = OutCfg<DV>;
    const int lane = threadIdx.x % C::LPR, rg = threadIdx.x / C::LPR;
    const float4 wt = a.weight ? reinterpret_cast<const float4 *>(a.weight)[lane] : make_float4(1.f, 1.f, 1.f, 1.f);
    const long nrb = (a.rows + C::RPB - 1) / C::RPB;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);   // this lane's columns of the dweight partial
    // rows of row block rb (clamped addresses: every load is issued, none is out of bounds)
    float4 ov[kOutUnroll], gv[kOutUnroll], dy[kOutUnroll];
    auto load_rows = [&](long rb, float4 (&o4)[kOutUnroll], float4 (&g4)[kOutUnroll], float4 (&d4)[kOutUnroll]) {
#pragma unroll
        for (int u = 0; u < kOutUnroll; ++u) {
            const long row = rb * C::RPB + rg + (long)u * C::RPI;
            const size_t off = (size_t)(row < a.rows ? row : a.rows - 1) * DV + 4 * lane;
            o4[u] = *reinterpret_cast<const float4 *>(a.o + off);
            g4[u] = load_gate4<GB>(a.g, off);
            d4[u] = *reinterpret_cast<const float4 *>(a.dy + off);
        }
    };
    load_rows(blockIdx.x, ov, gv, dy);
    for (long rb = blockIdx.x; rb < nrb; rb += gridDim.x) {
        const long base = rb * C::RPB + rg;
        // the next row block's loads are in flight while this one is computed and stored
        float4 on[kOutUnroll], gn[kOutUnroll], dn[kOutUnroll];
        load_rows(rb + gridDim.x < nrb ? rb + gridDim.x : rb, on, gn, dn);
#pragma unroll
        for (int u = 0; u < kOutUnroll; ++u) {
            const long row = base + (long)u * C::RPI;
            const float r = __builtin_amdgcn_rsqf(row_sum<C::LPR>(dot4(ov[u], ov[u])) * (1.f / DV) + a.eps);
            const float4 uu = make_float4(ov[u].x * r, ov[u].y * r, ov[u].z * r, ov[u].w * r);
            const float4 du = make_float4(dy[u].x * wt.x * gv[u].x, dy[u].y * wt.y * gv[u].y,
                                          dy[u].z * wt.z * gv[u].z, dy[u].w * wt.w * gv[u].w);
            const float m = row_sum<C::LPR>(dot4(du, uu)) * (1.f / DV);
            if (row < a.rows) {
                const size_t off = (size_t)row * DV + 4 * lane;
                *reinterpret_cast<float4 *>(a.dO + off) =
                    make_float4(r * (du.x - uu.x * m), r * (du.y - uu.y * m), r * (du.z - uu.z * m),
                                r * (du.w - uu.w * m));
                *reinterpret_cast<float4 *>(a.dg + off) =
                    make_float4(dy[u].x * uu.x * wt.x, dy[u].y * uu.y * wt.y, dy[u].z * uu.z * wt.z,
                                dy[u].w * uu.w * wt.w);
                acc.x += dy[u].x * uu.x * gv[u].x;
                acc.y += dy[u].y * uu.y * gv[u].y;
                acc.z += dy[u].z * uu.z * gv[u].z;
                acc.w += dy[u].w * uu.w * gv[u].w;
            }
        }
#pragma unroll
        for (int u = 0; u < kOutUnroll; ++u) {
            ov[u] = on[u];
            gv[u] = gn[u];
            dy[u] = dn[u];
        }
    }
    if (!a.partial) return;   // uniform over the launch
    // this workgroup's partial dweight row: the RPI row groups added in a fixed order
    __shared__ float4 sAcc[kOutThreads];
    sAcc[threadIdx.x] = acc;
    __syncthreads();
    if (rg == 0) {
        float4 t = sAcc[lane];
#pragma unroll
        for (int j = 1; j < C::RPI; ++j) {
            const float4 s = sAcc[j * C::LPR + lane];
            t.x += s.x; t.y += s.y; t.z += s.z; t.w += s.w;
        }
        reinterpret_cast<float4 *>(a.partial + (size_t)blockIdx.x * DV)[lane] = t;
    }
}

// dweight[c] = sum over the nblk partial rows, in a fixed order: 16 columns per
// workgroup of 1024 threads, 64 strided groups of partial rows (each loads its rows in
// batches of 8 before adding, so the loads overlap), then the groups in order.
constexpr int kRedThreads = 1024, kRedCols = 16, kRedGroups = kRedThreads / kRedCols, kRedBatch = 8;
__global__ __launch_bounds__(kRedThreads) void out_dweight_kernel(const float *partial, int nblk, int dv,
                                                                   float *dweight) {
    GDN2_POISON_LDS();
    __shared__ float sPart[kRedThreads];
    const int col = blockIdx.x * kRedCols + threadIdx.x % kRedCols, grp = threadIdx.x / kRedCols;
    float s = 0.f;
    for (int i0 = grp; i0 < nblk; i0 += kRedGroups * kRedBatch) {
        float x[kRedBatch];
#pragma unroll
        for (int j = 0; j < kRedBatch; ++j) {
            const int i = i0 + j * kRedGroups;
            x[j] = i < nblk ? partial[(size_t)i * dv + col] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kRedBatch; ++j) s += x[j];
    }
    sPart[threadIdx.x] = s;
    __syncthreads();
    if (grp == 0) {
        float t = sPart[threadIdx.x];
        for (int j = 1; j < kRedGroups; ++j) t += sPart[j * kRedCols + threadIdx.x];
        dweight[col] = t;
    }
}

int out_bwd_blocks(long rows, int dv) {
    const long rpb = (long)(kOutThreads / (dv / 4)) * kOutUnroll;
    const long nrb = (rows + rpb - 1) / rpb;
    return (int)(nrb < kOutMaxBlocks ? nrb : kOutMaxBlocks);
}

template <int DV, bool GB, bool YB>
static hipError_t out_fwd_t(const OutArgs &a, hipStream_t st) {
    const long nrb = (a.rows + OutCfg<DV>::RPB - 1) / OutCfg<DV>::RPB;
    hipLaunchKernelGGL((out_fwd_kernel<DV, GB, YB>), dim3((unsigned)nrb), dim3(kOutThreads), 0, st, a);
    return hipGetLastError();
}

template <int DV, bool GB>
static hipError_t out_bwd_t(const OutArgs &a, hipStream_t st) {
    const int nblk = out_bwd_blocks(a.rows, DV);
    hipLaunchKernelGGL((out_bwd_kernel<DV, GB>), dim3((unsigned)nblk), dim3(kOutThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.partial) return e;
    hipLaunchKernelGGL(out_dweight_kernel, dim3((unsigned)(DV / kRedCols)), dim3(kRedThreads), 0, st, a.partial, nblk,
                       DV, a.dweight);
    return hipGetLastError();
}

hipError_t launch_out_fwd(const OutArgs &a, int dv, bool g_bf16, bool y_bf16, hipStream_t st) {
#define GDN2_OUT_FWD(D)                                                                  \
    case D:                                                                              \
        return g_bf16 ? (y_bf16 ? out_fwd_t<D, true, true>(a, st) : out_fwd_t<D, true, false>(a, st)) \
                      : (y_bf16 ? out_fwd_t<D, false, true>(a, st) : out_fwd_t<D, false, false>(a, st));
    switch (dv) {
        GDN2_OUT_FWD(32)
        GDN2_OUT_FWD(64)
        GDN2_OUT_FWD(128)
        default: return hipErrorInvalidValue;
    }
#undef GDN2_OUT_FWD
}

hipError_t launch_out_bwd(const OutArgs &a, int dv, bool g_bf16, hipStream_t st) {
    switch (dv) {
        case 32: return g_bf16 ? out_bwd_t<32, true>(a, st) : out_bwd_t<32, false>(a, st);
        case 64: return g_bf16 ? out_bwd_t<64, true>(a, st) : out_bwd_t<64, false>(a, st);
        case 128: return g_bf16 ? out_bwd_t<128, true>(a, st) : out_bwd_t<128, false>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn2
