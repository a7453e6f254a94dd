// gdn2_api.cpp -- the C ABI of libgdn2.so: argument checks, workspace sizing and
// kernel dispatch.  No allocation, no global mutable state, no exceptions.
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#include <initializer_list>

#include "gdn2.h"
#include "gdn2_kernels.h"

namespace {

bool dim_ok(int d) { return d == 32 || d == 64 || d == 128; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool gate_logits(const gdn2_shape *s) { return s->gate_dtype == GDN2_GATES_BF16_LOGITS; }

static_assert(GDN2_SCALAR_DECAY == gdn2::kScalarDecay && GDN2_SCALAR_ERASE == gdn2::kScalarErase &&
                  GDN2_SCALAR_WRITE == gdn2::kScalarWrite,
              "per-token gate bits of the ABI and the kernels agree");
constexpr int kScalarAll = GDN2_SCALAR_DECAY | GDN2_SCALAR_ERASE | GDN2_SCALAR_WRITE;

bool gate_scalar(const gdn2_shape *s) { return s->gate_scalar != 0; }

int check_shape(const gdn2_shape *s) {
    if (!s) return GDN2_ERR_INVALID_ARG;
    if (s->B < 1 || s->T < 1 || s->H < 1 || s->dk < 1 || s->dv < 1) return GDN2_ERR_INVALID_ARG;
    if (s->chunk != 64) return GDN2_ERR_UNSUPPORTED;
    if (!dim_ok(s->dk) || !dim_ok(s->dv)) return GDN2_ERR_UNSUPPORTED;
    if (s->qkv_dtype != GDN2_F32 && s->qkv_dtype != GDN2_BF16) return GDN2_ERR_UNSUPPORTED;
    if (s->gate_dtype != GDN2_GATES_F32 && s->gate_dtype != GDN2_GATES_BF16_LOGITS) return GDN2_ERR_UNSUPPORTED;
    if (s->gate_dtype == GDN2_GATES_BF16_LOGITS && s->qkv_dtype != GDN2_BF16) return GDN2_ERR_UNSUPPORTED;
    if (s->gate_scalar & ~kScalarAll) return GDN2_ERR_UNSUPPORTED;
    if (s->gate_scalar && (s->qkv_dtype != GDN2_BF16 || s->gate_dtype != GDN2_GATES_F32)) return GDN2_ERR_UNSUPPORTED;
    const int dmax = s->dk > s->dv ? s->dk : s->dv;
    const unsigned long long n = (unsigned long long)s->B * s->T * s->H * dmax;
    if (n >= (1ull << 31)) return GDN2_ERR_UNSUPPORTED;
    // the kernels address a chunk's rows of a token tensor by 32-bit byte offsets from the
    // chunk's first row: 64 tokens of H * dmax fp32 values must span less than 4 GiB
    if ((unsigned long long)s->H * dmax >= (1ull << 24)) return GDN2_ERR_UNSUPPORTED;
    // grid size (workgroups) must fit in 32 bits; chunk-state workspace indexing uses size_t
    if ((unsigned long long)s->B * s->H * s->dv / 16 >= (1ull << 31)) return GDN2_ERR_UNSUPPORTED;
    return GDN2_OK;
}

int nchunks(const gdn2_shape *s) { return (s->T + 63) / 64; }

// The inference forward always takes the record path: the chunk records of every chunk
// (the fast pass of the factor kernel, then its exact pass over chunks with strong decay),
// then a sweep over them.  The wide eight-wave sweep applies with bf16 q/k/v, dk 64 or 128
// and dv a multiple of 64; the four-wave sweep takes every other shape.
bool wide_sweep_shape(const gdn2_shape *s) {
    return s->qkv_dtype == GDN2_BF16 && (s->dk == 64 || s->dk == 128) && s->dv % 64 == 0;
}

// Segments of the record-path forward.  With so few heads that the wide sweep keeps at most
// one CU in four busy, and a long sequence, the sequence is split into segments swept side by
// side: a pass for every segment's state map (its value tiles plus DK / 64 identity tiles), the
// maps composed in order, and a pass from the true start states.  About three sweeps' work at a
// quarter or less of the depth; enough segments to give every CU a workgroup in the last pass
// (more only add passes).  B1 T16K H16: 1.47 -> 0.78 ms; B2 T16K H16: 1.66 -> 1.36 ms; at half
// the CUs busy (B4 T8K H16) two segments are slower, 1.09 -> 1.33 ms.  1 = no segments.
int fwd_segments(const gdn2_shape *s, int *seg_len) {
    *seg_len = nchunks(s);
    if (!wide_sweep_shape(s)) return 1;
    const long wide = (long)s->B * s->H * (s->dv / 64);
    const int nc = nchunks(s), cus = gdn2::cu_count();
    if (wide * 4 > cus || nc < 64) return 1;
    int nseg = (int)(cus / wide);
    if (nseg > nc / 8) nseg = nc / 8;             // at least 8 chunks a segment
    const int len = (nc + nseg - 1) / nseg;
    *seg_len = len;
    return (nc + len - 1) / len;
}

// bytes after the records: every segment's [N | M] block, then the composed start states
size_t fwd_segment_bytes(const gdn2_shape *s, int nseg) {
    if (nseg <= 1) return 0;
    const size_t blocks = (size_t)s->B * s->H * nseg * s->dk;
    return blocks * (s->dv + s->dk) * sizeof(float) + blocks * s->dv * sizeof(float);
}

// The forward with the output epilogue fused into its sweep: the wide sweep without segments,
// where every workgroup of the launch can be resident at once (gdn2::fwd_out_fused).
bool out_fused(const gdn2_shape *s) {
    int seg_len;
    return wide_sweep_shape(s) && fwd_segments(s, &seg_len) == 1 &&
           gdn2::fwd_out_fused(s->B, s->H, s->T, s->dk, s->dv, true);
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// the alignment a gate tensor (or its gradient) needs: 4 bytes when it is per token
bool gate_aligned(const gdn2_shape *s, int bit, const void *p) {
    return !p || ((s->gate_scalar & bit) ? aligned4(p) : aligned16(p));
}

bool gates_aligned(const gdn2_shape *s, const void *la, const void *b, const void *w) {
    return gate_aligned(s, GDN2_SCALAR_DECAY, la) && gate_aligned(s, GDN2_SCALAR_ERASE, b) &&
           gate_aligned(s, GDN2_SCALAR_WRITE, w);
}

}  // namespace

extern "C" {

const char *gdn2_strerror(int status) {
    switch (status) {
        case GDN2_OK: return "success";
        case GDN2_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size or misaligned pointer)";
        case GDN2_ERR_UNSUPPORTED: return "unsupported shape or dtype (chunk must be 64, dk/dv in {32,64,128})";
        case GDN2_ERR_WORKSPACE: return "workspace missing or smaller than the required size";
        case GDN2_ERR_HIP: return "HIP runtime error at kernel launch";
        case GDN2_ERR_SCRATCH: return "request larger than the static scratch of gdn2_chunk_fwd_noalloc";
        default: return "unknown gdn2 status";
    }
}

size_t gdn2_chunk_fwd_workspace_size(const gdn2_shape *shape) {
    if (check_shape(shape) != GDN2_OK) return (size_t)-1;
    int seg_len;
    const int nseg = fwd_segments(shape, &seg_len);
    return gdn2::record_buffer_bytes((long)shape->B * shape->H * nchunks(shape), shape->dk) +
           fwd_segment_bytes(shape, nseg);
}

int gdn2_chunk_fwd(const gdn2_shape *shape, const void *q, const void *k, const void *v,
                   const void *log_alpha, const void *b, const void *w, const float *S0, float *o,
                   float *S_final, void *workspace, size_t workspace_bytes, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN2_OK) return st;
    if (!q || !k || !v || !log_alpha || !b || !w || !o) return GDN2_ERR_INVALID_ARG;
    const void *ptrs[] = {q, k, v, S0, o, S_final, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_INVALID_ARG;
    if (!gates_aligned(shape, log_alpha, b, w)) return GDN2_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < gdn2_chunk_fwd_workspace_size(shape)) return GDN2_ERR_WORKSPACE;
    const bool bf16 = shape->qkv_dtype == GDN2_BF16;
    // forward-only chunk records into the workspace, then the sweep from them
    gdn2::BwdArgs r{};
    r.B = shape->B; r.T = shape->T; r.H = shape->H; r.DV = shape->dv; r.scalar = shape->gate_scalar;
    r.q = q; r.k = k; r.la = log_alpha; r.bg = b; r.factors = workspace;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = gdn2::launch_fwd_records(r, shape->dk, bf16, gate_logits(shape), gate_scalar(shape), hs);
    if (e != hipSuccess) return GDN2_ERR_HIP;
    gdn2::FwdArgs f{};
    f.v = v; f.wg = w; f.S0 = S0; f.o = o; f.S_final = S_final; f.states = nullptr; f.records = workspace;
    f.B = shape->B; f.T = shape->T; f.H = shape->H; f.dv = shape->dv; f.scalar = shape->gate_scalar;
    int seg_len;
    const int nseg = fwd_segments(shape, &seg_len);
    if (nseg > 1) {
        // segments side by side: the maps, their composition, o
        f.nseg = nseg;
        f.seg_len = seg_len;
        char *rest = reinterpret_cast<char *>(workspace) +
                     gdn2::record_buffer_bytes((long)shape->B * shape->H * nchunks(shape), shape->dk);
        float *E = reinterpret_cast<float *>(rest);
        float *Sin = E + (size_t)shape->B * shape->H * nseg * shape->dk * (shape->dv + shape->dk);
        const hipError_t e3 = gdn2::launch_fwd_segments(f, shape->dk, gate_logits(shape), gate_scalar(shape), E,
                                                        Sin, hs);
        return e3 == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
    }
    const int vt = gdn2::fwd_value_tile(shape->B, shape->H, shape->dk, shape->dv);
    f.nvt = shape->dv / vt;
    const hipError_t e2 = gdn2::launch_fwd_sweep(f, shape->dk, vt, bf16, gate_logits(shape), gate_scalar(shape),
                                                 gdn2::kFwdOut, hs);
    return e2 == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

size_t gdn2_chunk_fwd_output_workspace_size(const gdn2_shape *shape) {
    if (check_shape(shape) != GDN2_OK) return (size_t)-1;
    if (out_fused(shape))
        return gdn2::record_buffer_bytes((long)shape->B * shape->H * nchunks(shape), shape->dk) +
               gdn2::fwd_out_exchange_bytes(shape->B, shape->H, shape->T, shape->dk, shape->dv);
    // otherwise gdn2_chunk_fwd's workspace, then o
    return round256(gdn2_chunk_fwd_workspace_size(shape)) + (size_t)shape->B * shape->T * shape->H * shape->dv * 4;
}

int gdn2_chunk_fwd_output(const gdn2_shape *shape, const void *q, const void *k, const void *v,
                          const void *log_alpha, const void *b, const void *w, const float *S0, const void *g,
                          int g_dtype, const float *weight, float eps, void *y, int y_dtype, float *S_final,
                          void *workspace, size_t workspace_bytes, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN2_OK) return st;
    if (!q || !k || !v || !log_alpha || !b || !w || !g || !y || !(eps >= 0.f) || !isfinite(eps))
        return GDN2_ERR_INVALID_ARG;
    if ((g_dtype != GDN2_F32 && g_dtype != GDN2_BF16) || (y_dtype != GDN2_F32 && y_dtype != GDN2_BF16))
        return GDN2_ERR_UNSUPPORTED;
    const void *ptrs[] = {q, k, v, S0, g, weight, y, S_final, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_INVALID_ARG;
    if (!gates_aligned(shape, log_alpha, b, w)) return GDN2_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < gdn2_chunk_fwd_output_workspace_size(shape)) return GDN2_ERR_WORKSPACE;
    if (!out_fused(shape)) {
        // the forward into the workspace's o, then the epilogue
        const size_t fw = round256(gdn2_chunk_fwd_workspace_size(shape));
        float *o = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + fw);
        const int rc = gdn2_chunk_fwd(shape, q, k, v, log_alpha, b, w, S0, o, S_final, workspace, fw, stream);
        if (rc != GDN2_OK) return rc;
        return gdn2_output_fwd(shape, o, g, g_dtype, weight, eps, y, y_dtype, stream);
    }
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const long items = (long)shape->B * shape->H * nchunks(shape);
    gdn2::BwdArgs r{};
    r.B = shape->B; r.T = shape->T; r.H = shape->H; r.DV = shape->dv; r.scalar = shape->gate_scalar;
    r.q = q; r.k = k; r.la = log_alpha; r.bg = b; r.factors = workspace;
    // the records kernel also clears the sweep's row-sum exchange area
    char *xr = reinterpret_cast<char *>(workspace) + gdn2::record_buffer_bytes(items, shape->dk);
    const size_t xbytes = gdn2::fwd_out_exchange_bytes(shape->B, shape->H, shape->T, shape->dk, shape->dv);
    r.zero = xr; r.zero16 = (long)(xbytes / 16);
    if (gdn2::launch_fwd_records(r, shape->dk, true, gate_logits(shape), gate_scalar(shape), hs) != hipSuccess)
        return GDN2_ERR_HIP;
    gdn2::FwdArgs f{};
    f.v = v; f.wg = w; f.S0 = S0; f.S_final = S_final; f.records = workspace;
    f.B = shape->B; f.T = shape->T; f.H = shape->H; f.dv = shape->dv; f.scalar = shape->gate_scalar;
    f.og = g; f.oweight = weight; f.y = y; f.eps = eps;
    f.og_bf16 = g_dtype == GDN2_BF16; f.y_bf16 = y_dtype == GDN2_BF16;
    f.xrow = reinterpret_cast<unsigned long long *>(xr);
    f.xerr = reinterpret_cast<int *>(xr + xbytes - 256);
    return gdn2::launch_fwd_sweep_out(f, shape->dk, gate_logits(shape), gate_scalar(shape), hs) == hipSuccess
               ? GDN2_OK
               : GDN2_ERR_HIP;
}

int gdn2_chunk_fwd_output_fused(const gdn2_shape *shape) {
    return check_shape(shape) == GDN2_OK && out_fused(shape) ? 1 : 0;
}

size_t gdn2_chunk_states_bytes(const gdn2_shape *shape) {
    if (check_shape(shape) != GDN2_OK) return (size_t)-1;
    return (size_t)shape->B * shape->H * nchunks(shape) * (size_t)shape->dk * shape->dv * sizeof(float);
}

size_t gdn2_chunk_factors_bytes(const gdn2_shape *shape) {
    if (check_shape(shape) != GDN2_OK) return (size_t)-1;
    return gdn2::factor_buffer_bytes((long)shape->B * shape->H * nchunks(shape), shape->dk);
}

size_t gdn2_chunk_bwd_workspace_size(const gdn2_shape *shape) {
    if (check_shape(shape) != GDN2_OK) return (size_t)-1;
    int seg_len;
    return 2 * gdn2_chunk_states_bytes(shape) + gdn2_chunk_factors_bytes(shape) +
           fwd_segment_bytes(shape, fwd_segments(shape, &seg_len));
}

}  // extern "C"

namespace {

gdn2::FwdArgs fwd_args(const gdn2_shape *shape, const void *q, const void *k, const void *v,
                       const void *log_alpha, const void *b, const void *w, const float *S0, float *o,
                       float *S_final, float *states, int *vt_out) {
    gdn2::FwdArgs f{};
    f.q = q; f.k = k; f.v = v;
    f.la = log_alpha; f.bg = b; f.wg = w;
    f.S0 = S0; f.o = o; f.S_final = S_final; f.states = states;
    f.B = shape->B; f.T = shape->T; f.H = shape->H; f.dv = shape->dv;
    const int vt = gdn2::fwd_value_tile(shape->B, shape->H, shape->dk, shape->dv);
    f.nvt = shape->dv / vt;
    f.scalar = shape->gate_scalar;
    *vt_out = vt;
    return f;
}

gdn2::BwdArgs bwd_args(const gdn2_shape *shape) {
    gdn2::BwdArgs a{};
    a.B = shape->B; a.T = shape->T; a.H = shape->H; a.DV = shape->dv;
    a.scalar = shape->gate_scalar;
    return a;
}

// Sweep arguments from a factor buffer of gdn2_chunk_bwd_factors: its chunk operand records
// follow the adjoint factors of every chunk.
gdn2::FwdArgs factored_args(const gdn2_shape *shape, const void *factors, const void *v, const void *w,
                            const float *S0, float *o, float *S_final, float *states) {
    int vt;
    gdn2::FwdArgs f = fwd_args(shape, nullptr, nullptr, v, nullptr, nullptr, w, S0, o, S_final, states, &vt);
    const long items = (long)shape->B * shape->H * nchunks(shape);
    f.records = reinterpret_cast<const char *>(factors) +
                (gdn2::factor_buffer_bytes(items, shape->dk) - gdn2::record_buffer_bytes(items, shape->dk));
    return f;
}

// Reverse-sweep arguments: the factor buffer, dO, dS_final and the outputs dS' of every chunk, dS0
gdn2::BwdArgs reverse_args(const gdn2_shape *shape, const void *factors, const float *dO, const float *dS_final,
                           float *dstates, float *dS0) {
    gdn2::BwdArgs a = bwd_args(shape);
    a.factors = const_cast<void *>(factors);
    a.dO = dO; a.dS_final = dS_final; a.dstates = dstates; a.dS0 = dS0;
    return a;
}

bool all_aligned(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return false;
    return true;
}

int launch_status(hipError_t e) { return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP; }

}  // namespace

extern "C" {

int gdn2_chunk_bwd_factors(const gdn2_shape *shape, const void *q, const void *k, const void *log_alpha,
                           const void *b, void *factors, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN2_OK) return st;
    if (!q || !k || !log_alpha || !b || !factors) return GDN2_ERR_INVALID_ARG;
    if (!all_aligned({q, k, factors}) || !gates_aligned(shape, log_alpha, b, nullptr)) return GDN2_ERR_INVALID_ARG;
    gdn2::BwdArgs a = bwd_args(shape);
    a.q = q; a.k = k; a.la = log_alpha; a.bg = b; a.factors = factors;
    return launch_status(gdn2::launch_bwd_factors(a, shape->dk, shape->qkv_dtype == GDN2_BF16, gate_logits(shape),
                                                  gate_scalar(shape), reinterpret_cast<hipStream_t>(stream)));
}

int gdn2_chunk_fwd_factored(const gdn2_shape *shape, const void *factors, const void *v, const void *w,
                            const float *S0, float *o, float *S_final, float *states, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN2_OK) return st;
    if (!factors || !v || !w || (!o && !states)) return GDN2_ERR_INVALID_ARG;
    if (!all_aligned({factors, v, S0, o, S_final, states}) || !gates_aligned(shape, nullptr, nullptr, w))
        return GDN2_ERR_INVALID_ARG;
    const gdn2::FwdArgs f = factored_args(shape, factors, v, w, S0, o, S_final, states);
    const int vt = shape->dv / f.nvt;
    const gdn2::FwdMode mode = !o ? gdn2::kFwdStates : states ? gdn2::kFwdOutStates : gdn2::kFwdOut;
    return launch_status(gdn2::launch_fwd_sweep(f, shape->dk, vt, shape->qkv_dtype == GDN2_BF16, gate_logits(shape),
                                                gate_scalar(shape), mode, reinterpret_cast<hipStream_t>(stream)));
}

int gdn2_chunk_bwd_reverse(const gdn2_shape *shape, const void *factors, const float *dO,
                           const float *dS_final, float *dstates, float *dS0, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN2_OK) return st;
    if (!factors || !dO || !dstates) return GDN2_ERR_INVALID_ARG;
    if (!all_aligned({factors, dO, dS_final, dstates, dS0})) return GDN2_ERR_INVALID_ARG;
    return launch_status(gdn2::launch_bwd_reverse(reverse_args(shape, factors, dO, dS_final, dstates, dS0), shape->dk,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

int gdn2_chunk_sweeps_fused(const gdn2_shape *shape) {
    if (check_shape(shape) != GDN2_OK) return -1;
    return gdn2::fwd_rev_fused(shape->B, shape->H, shape->dk, shape->dv, shape->qkv_dtype == GDN2_BF16) ? 1 : 0;
}

int gdn2_chunk_sweeps(const gdn2_shape *shape, const void *factors, const void *v, const void *w, const float *S0,
                      const float *dO, const float *dS_final, float *o, float *S_final, float *states,
                      float *dstates, float *dS0, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN2_OK) return st;
    if (!factors || !v || !w || !dO || !o || !states || !dstates) return GDN2_ERR_INVALID_ARG;
    if (!all_aligned({factors, v, S0, dO, dS_final, o, S_final, states, dstates, dS0}) ||
        !gates_aligned(shape, nullptr, nullptr, w))
        return GDN2_ERR_INVALID_ARG;
    if (gdn2_chunk_sweeps_fused(shape) != 1) {
        // the two sweeps one after the other
        const int rc = gdn2_chunk_fwd_factored(shape, factors, v, w, S0, o, S_final, states, stream);
        if (rc != GDN2_OK) return rc;
        return gdn2_chunk_bwd_reverse(shape, factors, dO, dS_final, dstates, dS0, stream);
    }
    return launch_status(gdn2::launch_fwd_rev_sweeps(factored_args(shape, factors, v, w, S0, o, S_final, states),
                                                     reverse_args(shape, factors, dO, dS_final, dstates, dS0),
                                                     shape->dk, gate_logits(shape), gate_scalar(shape),
                                                     reinterpret_cast<hipStream_t>(stream)));
}

int gdn2_chunk_bwd_grads(const gdn2_shape *shape, const void *q, const void *k, const void *v,
                         const void *log_alpha, const void *b, const void *w, const float *dO,
                         const float *states, const float *dstates, const void *factors, float *dq, float *dk,
                         float *dv, float *dlog_alpha, float *db, float *dw, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN2_OK) return st;
    if (!q || !k || !v || !log_alpha || !b || !w || !dO || !states || !dstates || !factors || !dq || !dk || !dv ||
        !dlog_alpha || !db || !dw)
        return GDN2_ERR_INVALID_ARG;
    if (!all_aligned({q, k, v, dO, states, dstates, factors, dq, dk, dv}) || !gates_aligned(shape, log_alpha, b, w) ||
        !gates_aligned(shape, dlog_alpha, db, dw))
        return GDN2_ERR_INVALID_ARG;
    gdn2::BwdArgs a = bwd_args(shape);
    a.q = q; a.k = k; a.v = v;
    a.la = log_alpha; a.bg = b; a.wg = w;
    a.dO = dO; a.states = states; a.dstates = const_cast<float *>(dstates);
    a.factors = const_cast<void *>(factors);
    a.dq = dq; a.dk = dk; a.dv = dv; a.dla = dlog_alpha; a.db = db; a.dw = dw;
    return launch_status(gdn2::launch_bwd_chunk(a, shape->dk, shape->qkv_dtype == GDN2_BF16, gate_logits(shape),
                                                gate_scalar(shape), reinterpret_cast<hipStream_t>(stream)));
}

int gdn2_chunk_bwd(const gdn2_shape *shape, const void *q, const void *k, const void *v,
                   const void *log_alpha, const void *b, const void *w, const float *S0,
                   const float *dO, const float *dS_final, float *dq, float *dk, float *dv,
                   float *dlog_alpha, float *db, float *dw, float *dS0, void *workspace,
                   size_t workspace_bytes, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN2_OK) return st;
    if (!q || !k || !v || !log_alpha || !b || !w || !dO || !dq || !dk || !dv || !dlog_alpha || !db || !dw)
        return GDN2_ERR_INVALID_ARG;
    if (!all_aligned({q, k, v, S0, dO, dS_final, dq, dk, dv, dS0, workspace}) ||
        !gates_aligned(shape, log_alpha, b, w) || !gates_aligned(shape, dlog_alpha, db, dw))
        return GDN2_ERR_INVALID_ARG;
    const size_t need = gdn2_chunk_bwd_workspace_size(shape);
    if (!workspace || workspace_bytes < need) return GDN2_ERR_WORKSPACE;
    const size_t sbytes = gdn2_chunk_states_bytes(shape);
    float *states = reinterpret_cast<float *>(workspace);
    float *dstates = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + sbytes);
    void *factors = reinterpret_cast<char *>(workspace) + 2 * sbytes;
    // the key-side chunk operands once; then the state before every chunk and dS' of every chunk
    int rc = gdn2_chunk_bwd_factors(shape, q, k, log_alpha, b, factors, stream);
    if (rc != GDN2_OK) return rc;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    int seg_len;
    const int nseg = fwd_segments(shape, &seg_len);
    if (nseg > 1) {
        // few heads, long sequence: the state sweep in segments side by side (as the forward's),
        // the segment blocks after the factors
        gdn2::FwdArgs f = factored_args(shape, factors, v, w, S0, nullptr, nullptr, states);
        f.nseg = nseg;
        f.seg_len = seg_len;
        float *E = reinterpret_cast<float *>(reinterpret_cast<char *>(factors) + gdn2_chunk_factors_bytes(shape));
        float *Sin = E + (size_t)shape->B * shape->H * nseg * shape->dk * (shape->dv + shape->dk);
        rc = launch_status(gdn2::launch_fwd_segments(f, shape->dk, gate_logits(shape), gate_scalar(shape), E, Sin, hs));
        if (rc == GDN2_OK) rc = gdn2_chunk_bwd_reverse(shape, factors, dO, dS_final, dstates, dS0, stream);
    } else if (gdn2_chunk_sweeps_fused(shape) == 1) {
        // few heads: the state sweep and the reverse sweep side by side in one launch
        rc = launch_status(gdn2::launch_fwd_rev_sweeps(
            factored_args(shape, factors, v, w, S0, nullptr, nullptr, states),
            reverse_args(shape, factors, dO, dS_final, dstates, dS0), shape->dk, gate_logits(shape),
            gate_scalar(shape), hs));
    } else {
        rc = gdn2_chunk_fwd_factored(shape, factors, v, w, S0, nullptr, nullptr, states, stream);
        if (rc == GDN2_OK) rc = gdn2_chunk_bwd_reverse(shape, factors, dO, dS_final, dstates, dS0, stream);
    }
    if (rc != GDN2_OK) return rc;
    return gdn2_chunk_bwd_grads(shape, q, k, v, log_alpha, b, w, dO, states, dstates, factors, dq, dk, dv,
                                dlog_alpha, db, dw, stream);
}

int gdn2_step(const gdn2_shape *shape, const void *q, const void *k, const void *v, const void *log_alpha,
              const void *b, const void *w, const float *S_in, float *S_out, float *o, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN2_OK) return st;
    if (shape->T != 1) return GDN2_ERR_INVALID_ARG;
    if (!q || !k || !v || !log_alpha || !b || !w || !S_out || !o) return GDN2_ERR_INVALID_ARG;
    if (!all_aligned({q, k, v, S_in, S_out, o}) || !gates_aligned(shape, log_alpha, b, w)) return GDN2_ERR_INVALID_ARG;
    gdn2::StepArgs a{};
    a.q = q; a.k = k; a.v = v;
    a.la = log_alpha; a.bg = b; a.wg = w;
    a.S_in = S_in; a.S_out = S_out; a.o = o;
    a.BH = shape->B * shape->H; a.dv = shape->dv;
    a.scalar = shape->gate_scalar;
    return launch_status(gdn2::launch_step(a, shape->dk, shape->qkv_dtype == GDN2_BF16, gate_logits(shape),
                                           gate_scalar(shape), reinterpret_cast<hipStream_t>(stream)));
}

size_t gdn2_output_bwd_workspace_size(const gdn2_shape *shape) {
    if (check_shape(shape) != GDN2_OK) return (size_t)-1;
    const long rows = (long)shape->B * shape->T * shape->H;
    return (size_t)gdn2::out_bwd_blocks(rows, shape->dv) * shape->dv * sizeof(float);
}

int gdn2_output_fwd(const gdn2_shape *shape, const float *o, const void *g, int g_dtype, const float *weight,
                    float eps, void *y, int y_dtype, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN2_OK) return st;
    if (!o || !g || !y || !(eps >= 0.f) || !isfinite(eps)) return GDN2_ERR_INVALID_ARG;
    if ((g_dtype != GDN2_F32 && g_dtype != GDN2_BF16) || (y_dtype != GDN2_F32 && y_dtype != GDN2_BF16))
        return GDN2_ERR_UNSUPPORTED;
    if (!all_aligned({o, g, weight, y})) return GDN2_ERR_INVALID_ARG;
    gdn2::OutArgs a{};
    a.o = o; a.g = g; a.weight = weight; a.y = y;
    a.rows = (long)shape->B * shape->T * shape->H;
    a.eps = eps;
    return launch_status(gdn2::launch_out_fwd(a, shape->dv, g_dtype == GDN2_BF16, y_dtype == GDN2_BF16,
                                              reinterpret_cast<hipStream_t>(stream)));
}

int gdn2_output_bwd(const gdn2_shape *shape, const float *o, const void *g, int g_dtype, const float *weight,
                    float eps, const float *dy, float *dO, float *dg, float *dweight, void *workspace,
                    size_t workspace_bytes, void *stream) {
    const int st = check_shape(shape);
    if (st != GDN2_OK) return st;
    if (!o || !g || !dy || !dO || !dg || !(eps >= 0.f) || !isfinite(eps)) return GDN2_ERR_INVALID_ARG;
    if (g_dtype != GDN2_F32 && g_dtype != GDN2_BF16) return GDN2_ERR_UNSUPPORTED;
    if (!all_aligned({o, g, weight, dy, dO, dg, dweight, workspace})) return GDN2_ERR_INVALID_ARG;
    if (dweight && (!workspace || workspace_bytes < gdn2_output_bwd_workspace_size(shape))) return GDN2_ERR_WORKSPACE;
    gdn2::OutArgs a{};
    a.o = o; a.g = g; a.weight = weight; a.dy = dy; a.dO = dO; a.dg = dg;
    a.partial = dweight ? reinterpret_cast<float *>(workspace) : nullptr;
    a.dweight = dweight;
    a.rows = (long)shape->B * shape->T * shape->H;
    a.eps = eps;
    return launch_status(gdn2::launch_out_bwd(a, shape->dv, g_dtype == GDN2_BF16,
                                              reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
