// gdn2_kernels.h -- launch interface between the C ABI (gdn2_api.cpp) and the
// HIP kernels.  Internal to libgdn2.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdn2 {

// Gates given as one value per token (broadcast over their channels), a bit each.
constexpr int kScalarDecay = 1, kScalarErase = 2, kScalarWrite = 4;

// Arguments of the chunked forward sweep.  Token tensors are [B,T,H,D]
// contiguous; states [B,H,dk,dv] fp32; chunk states [B,H,NC,dk,dv] fp32.
struct FwdArgs {
    const void *q, *k, *v;          // qkv dtype
    const void *la, *bg, *wg;       // log_alpha, b, w: fp32 values or bf16 logits
    const float *S0;                // may be null (zeros)
    float *o;                       // [B,T,H,dv] (forward) or unused (state sweep)
    float *S_final;                 // may be null
    float *states;                  // chunk-start states (state sweep) or null
    const void *records;            // chunk operand records of (b, h, c) at (b * H + h) * NC + c (sweep)
    int B, T, H, dv;
    int nvt;                        // value tiles per (b, h) = dv / value-tile width
    int scalar;                     // kScalar* bits: gates given per token [B,T,H]
    int nseg, seg_len;              // segmented sweep: segments per (b, h), chunks per segment
    // fused output epilogue (launch_fwd_sweep_out): y = o / sqrt(mean_j o_j^2 + eps) * weight * g
    // per (b, t, h) row of dv channels; o itself is not written
    const void *og;                 // output gate values [B,T,H,dv], fp32 or bf16 (og_bf16)
    const float *oweight;           // [dv] or null (ones)
    void *y;                        // [B,T,H,dv], fp32 or bf16 (y_bf16)
    unsigned long long *xrow;       // row sums of squares exchanged between a head's value tiles
    int *xerr;                      // exchange waits that ran out (0 in a correct run)
    float eps;
    int og_bf16, y_bf16;
};

// Arguments of the backward kernels.
struct BwdArgs {
    const void *q, *k, *v;
    const void *la, *bg, *wg;       // fp32 values or bf16 logits
    const float *dO, *dS_final;     // dS_final may be null
    const float *states;            // [B,H,NC,dk,dv] chunk-start states
    float *dstates;                 // [B,H,NC,dk,dv] gradient w.r.t. chunk-end states
    float *dq, *dk, *dv, *dla, *db, *dw, *dS0;
    void *factors;                  // per-chunk adjoint factors (bf16 tiles), then chunk operand records
    void *zero;                     // forward-only records: zero16 16-byte words the fast pass also clears
    long zero16;                    // (for a launch that follows), or null / 0
    int B, T, H, DV;
    int scalar;                     // kScalar* bits: gates (and their gradients) per token [B,T,H]
};

// Arguments of the recurrent step (one token per (batch, head)); token tensors [BH, D].
struct StepArgs {
    const void *q, *k, *v;
    const void *la, *bg, *wg;       // fp32 values or bf16 logits
    const float *S_in;              // may be null (zeros)
    float *S_out;                   // may equal S_in
    float *o;
    int BH, dv;
    int scalar;                     // kScalar* bits: gates given per (batch, head) [B,H]
};
// sg: some gates are given per token (a.scalar), only with bf16 q/k/v and fp32 gate values
hipError_t launch_step(const StepArgs &a, int dk, bool bf16, bool gl, bool sg, hipStream_t st);

// Compute units of the current device (256 if the runtime cannot tell).
inline int cu_count() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return 256;
    return cus;
}

// Value-tile width the four-wave forward sweep uses for this shape (16 or 32).
int fwd_value_tile(int B, int H, int dk, int dv);

// What a forward sweep produces: o only, chunk states only, or both.
enum FwdMode { kFwdOut = 0, kFwdStates = 1, kFwdOutStates = 2 };
// gl: the gates are bf16 logits (only with bf16 q/k/v); sg: some gates are given per token
// (a.scalar; only with bf16 q/k/v and fp32 gate values).
// The forward sweep with the key-side operands of every chunk taken from chunk operand
// records (a.records); q, k, log_alpha and b are not read.
// The forward sweep over few heads, sequence split into a.nseg segments of a.seg_len chunks
// (bf16 q/k/v, dk 64 or 128, dv a multiple of 64): every segment's state map into E
// [B, H, nseg, dk, dv + dk], the composed start states into Sin [B, H, nseg, dk, dv], then
// either o (a.o; a.states null) or the state before every chunk (a.states; a.o null), and S_final
// if a.S_final is set.  a.records holds the chunk records (forward-only ones or those of the
// factor buffer); a.S0 may be null.
hipError_t launch_fwd_segments(const FwdArgs &a, int dk, bool gl, bool sg, float *E, float *Sin, hipStream_t st);
hipError_t launch_fwd_sweep(const FwdArgs &a, int dk, int vt, bool bf16, bool gl, bool sg, FwdMode mode,
                            hipStream_t st);
// The forward sweep with the output epilogue fused (a.og, a.oweight, a.eps, a.y, a.og_bf16,
// a.y_bf16; a.o unused): the wide sweep without segments, where a head has at most four value
// tiles (dv / tile width) and all of its workgroups can be resident at once.  Each wave
// publishes the sums of squares of its rows over its columns as 64-bit words {value, chunk + 1}
// in a.xrow (a ring of two chunks: B * H * 2 * 2 * tiles * 64 words, zero before the launch;
// see fwd_out_exchange_bytes) and reads the other waves' words of its rows one chunk later.
// fwd_out_fused tells whether a shape takes it; launch_fwd_sweep_out returns
// hipErrorInvalidValue where it does not.
bool fwd_out_fused(int B, int H, int T, int dk, int dv, bool bf16);
size_t fwd_out_exchange_bytes(int B, int H, int T, int dk, int dv);
hipError_t launch_fwd_sweep_out(const FwdArgs &a, int dk, bool gl, bool sg, hipStream_t st);
// Whether the forward sweep (o, S_final, chunk states) and the reverse sweep from one factor
// buffer run as one launch: bf16 q/k/v, dk 64 or 128, dv a multiple of 64, and 64-column tiles of
// both sweeps together at most one workgroup per CU.
bool fwd_rev_fused(int B, int H, int dk, int dv, bool bf16);
// That launch (fa: v, w, S0, o, S_final, states, records of the factor buffer; ba: factors, dO,
// dS_final, dstates, dS0; o may be null: the states only).  hipErrorInvalidValue where
// fwd_rev_fused is false.
hipError_t launch_fwd_rev_sweeps(const FwdArgs &fa, const BwdArgs &ba, int dk, bool gl, bool sg, hipStream_t st);
// Bytes of the factor buffer of `items` chunks: the adjoint factors R, Q2^T of every chunk,
// then the chunk operand record of every chunk (read by the chunk-gradient kernel), then the
// strong-decay flag of every chunk.
size_t factor_buffer_bytes(long items, int dk);
// Bytes of `items` chunk operand records and their flags (the forward-only buffer).
size_t record_buffer_bytes(long items, int dk);
hipError_t launch_bwd_factors(const BwdArgs &a, int dk, bool bf16, bool gl, bool sg, hipStream_t st);
// Forward-only records: a.factors receives just the records the forward sweep reads.
hipError_t launch_fwd_records(const BwdArgs &a, int dk, bool bf16, bool gl, bool sg, hipStream_t st);
hipError_t launch_bwd_reverse(const BwdArgs &a, int dk, hipStream_t st);
hipError_t launch_bwd_chunk(const BwdArgs &a, int dk, bool bf16, bool gl, bool sg, hipStream_t st);

// Arguments of the output epilogue (RMS norm over the dv channels of a row, weight, output
// gate).  Row tensors are [rows, dv] contiguous, rows = B*T*H.
struct OutArgs {
    const float *o;                 // operator output, fp32
    const void *g;                  // output gate values, fp32 or bf16
    const float *weight;            // [dv] or null (ones)
    const float *dy;                // backward: upstream gradient of y, fp32
    void *y;                        // forward: fp32 or bf16
    float *dO, *dg;                 // backward outputs, fp32
    float *partial;                 // backward: [blocks, dv] partial dweight rows, or null (no dweight)
    float *dweight;                 // backward: [dv], written when partial is set
    long rows;
    float eps;
};
// workgroups of the backward epilogue (so the partial-row workspace is blocks * dv floats)
constexpr int kOutMaxBlocks = 1024;
int out_bwd_blocks(long rows, int dv);
hipError_t launch_out_fwd(const OutArgs &a, int dv, bool g_bf16, bool y_bf16, hipStream_t st);
hipError_t launch_out_bwd(const OutArgs &a, int dv, bool g_bf16, hipStream_t st);

}  // namespace gdn2
