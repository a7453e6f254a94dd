// gdn2_step.hip -- one recurrent step (decode) of the Gated DeltaNet-2 rule on gfx950.
//
// Rule (blog on Gated DeltaNet-2, section "Independent control on two axes"), for one
// token of one (batch, head) with state S [dk x dv], key channel = row:
//     Sbar = diag(exp(log_alpha)) S,   r = Sbar^T (b*k),
//     S'   = Sbar + k (w*v - r)^T,     o = S'^T q.
// The step reads and writes the whole state once, so it is bound by HBM bandwidth
// (2 * dk * dv * 4 bytes per head); it uses no MFMA.  Every column j of S is
// independent: r_j and o_j are sums over the key channels.
//
// One workgroup of 256 threads per (batch, head, 32 state columns): thread (slice s,
// column j) holds rows s*DK/8 .. s*DK/8 + DK/8 - 1 of column j in registers.  The
// channel vectors (decay, erase key, key, query) are staged once in LDS, and the two
// column sums go through LDS in a fixed order (bitwise reproducible).  Each thread
// writes exactly the elements it read, so S_out may alias S_in.
#include "gdn2_device.h"
#include "gdn2_kernels.h"

namespace gdn2 {

template <int DK, bool BF16, bool GL, bool SG>
__global__ __launch_bounds__(kThreads) void step_kernel(StepArgs a) {
    GDN2_POISON_LDS();
    constexpr int VT = 32, NS = kThreads / VT, RPS = DK / NS;   // slices, rows per slice
    __shared__ float sAlpha[DK], sE[DK], sK[DK], sQ[DK];
    __shared__ float sRed[NS][VT];

    const int tid = threadIdx.x, j = tid % VT, s = tid / VT;
    const int nvt = a.dv / VT;
    const int vt = blockIdx.x % nvt, bh = blockIdx.x / nvt;
    const size_t kbase = (size_t)bh * DK, vbase = (size_t)bh * a.dv + vt * VT;
    const size_t sbase = (size_t)bh * DK * a.dv + vt * VT;

    // a per-token gate (SG) is one value per (batch, head), broadcast over its channels
    const size_t offa = (SG && (a.scalar & kScalarDecay)) ? (size_t)bh : kbase + tid;
    const size_t offb = (SG && (a.scalar & kScalarErase)) ? (size_t)bh : kbase + tid;
    const size_t offw = (SG && (a.scalar & kScalarWrite)) ? (size_t)bh : vbase + j;
    if (tid < DK) {
        const float kk = load1<BF16>(a.k, kbase + tid, true);
        sAlpha[tid] = exp2_fast(decay_act<GL>(load_gate1<GL>(a.la, offa)) * kLog2e);
        sE[tid] = gate_act<GL>(load_gate1<GL>(a.bg, offb)) * kk;
        sK[tid] = kk;
        sQ[tid] = load1<BF16>(a.q, kbase + tid, true);
    }
    float x[RPS];
#pragma unroll
    for (int i = 0; i < RPS; ++i)
        x[i] = a.S_in ? a.S_in[sbase + (size_t)(s * RPS + i) * a.dv + j] : 0.f;
    const float z = gate_act<GL>(load_gate1<GL>(a.wg, offw)) * load1<BF16>(a.v, vbase + j, true);
    __syncthreads();

    // decay, then the read through the erase key
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < RPS; ++i) {
        x[i] *= sAlpha[s * RPS + i];
        part += x[i] * sE[s * RPS + i];
    }
    sRed[s][j] = part;
    __syncthreads();
    float rj = 0.f;
#pragma unroll
    for (int t = 0; t < NS; ++t) rj += sRed[t][j];
    const float u = z - rj;
    // write along the raw key, then the query reads the updated state
    part = 0.f;
#pragma unroll
    for (int i = 0; i < RPS; ++i) {
        x[i] += sK[s * RPS + i] * u;
        part += x[i] * sQ[s * RPS + i];
    }
    __syncthreads();   // every thread has read r_j before the partial sums are replaced
    sRed[s][j] = part;
#pragma unroll
    for (int i = 0; i < RPS; ++i) a.S_out[sbase + (size_t)(s * RPS + i) * a.dv + j] = x[i];
    __syncthreads();
    if (s == 0) {
        float oj = 0.f;
#pragma unroll
        for (int t = 0; t < NS; ++t) oj += sRed[t][j];
        a.o[vbase + j] = oj;
    }
}

template <int DK, bool BF16, bool GL, bool SG>
static hipError_t step_t(const StepArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((step_kernel<DK, BF16, GL, SG>), dim3((unsigned)(a.BH * (a.dv / 32))), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <bool BF16, bool GL, bool SG>
static hipError_t step_dk(const StepArgs &a, int dk, hipStream_t st) {
    switch (dk) {
        case 32: return step_t<32, BF16, GL, SG>(a, st);
        case 64: return step_t<64, BF16, GL, SG>(a, st);
        case 128: return step_t<128, BF16, GL, SG>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_step(const StepArgs &a, int dk, bool bf16, bool gl, bool sg, hipStream_t st) {
    if (a.dv % 32 != 0) return hipErrorInvalidValue;
    if (gl && sg) return hipErrorInvalidValue;
    if (gl) return bf16 ? step_dk<true, true, false>(a, dk, st) : hipErrorInvalidValue;
    if (sg) return bf16 ? step_dk<true, false, true>(a, dk, st) : hipErrorInvalidValue;
    return bf16 ? step_dk<true, false, false>(a, dk, st) : step_dk<false, false, false>(a, dk, st);
}

}  // namespace gdn2
