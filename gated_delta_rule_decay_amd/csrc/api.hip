// api.hip -- the C ABI declared in include/gdn2.h: host-side validation,
// then dispatch to the gfx950 kernels on the caller's stream.
//
// Validation never touches the GPU, so every error path is reachable (and
// tested) on a machine without one.  No allocation, no global mutable state.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn2.h"
#include "kernels.h"

namespace {

using gdn2::ChunkArgs;
using gdn2::StepArgs;

struct Span {
    uintptr_t lo = 0, hi = 0;  // [lo, hi); empty when lo == hi
};

Span span_of(const void *p, int64_t bytes) {
    Span s;
    if (p && bytes > 0) {
        s.lo = reinterpret_cast<uintptr_t>(p);
        s.hi = s.lo + static_cast<uintptr_t>(bytes);
    }
    return s;
}

bool overlap(const Span &a, const Span &b) {
    return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}

// a*b*... with an overflow check against int64 (result in *out).
bool mul_ok(int64_t a, int64_t b, int64_t *out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

gdn2_status check_common(const gdn2_desc *d) {
    if (!d) return GDN2_ERR_NULL;
    if (d->batch < 0 || d->seqlen < 0 || d->heads < 1 || d->dk < 1 || d->dv < 1)
        return GDN2_ERR_SHAPE;
    if (d->qkv_dtype != GDN2_F32 && d->qkv_dtype != GDN2_BF16) return GDN2_ERR_DTYPE;
    if (d->o_dtype != GDN2_F32 && d->o_dtype != GDN2_BF16) return GDN2_ERR_DTYPE;
    auto kind_ok = [](int32_t k) { return k == GDN2_GATE_HEAD || k == GDN2_GATE_KEY; };
    if (!kind_ok(d->decay_kind) || !kind_ok(d->erase_kind) ||
        (!d->tie_write_to_erase && !kind_ok(d->write_kind)))
        return GDN2_ERR_SHAPE;
    if (d->form != GDN2_FORM_KEY && d->form != GDN2_FORM_VALUE_WRITE) return GDN2_ERR_SHAPE;
    if (d->form == GDN2_FORM_VALUE_WRITE && d->tie_write_to_erase) return GDN2_ERR_SHAPE;
    if (d->dk > 128 || d->dv > 128) return GDN2_ERR_UNSUPPORTED;
    // every tensor's byte size must fit in int64
    int64_t x;
    const int64_t dmax = d->dk > d->dv ? d->dk : d->dv;
    if (!mul_ok(d->batch, d->seqlen, &x) || !mul_ok(x, d->heads, &x) || !mul_ok(x, dmax, &x) ||
        !mul_ok(x, 8, &x))
        return GDN2_ERR_SHAPE;
    if (!mul_ok(d->batch, d->heads, &x) || !mul_ok(x, d->dk, &x) || !mul_ok(x, d->dv, &x) ||
        !mul_ok(x, 8, &x))
        return GDN2_ERR_SHAPE;
    return GDN2_OK;
}

struct Sizes {
    int64_t tok;     // B*T*H token-heads
    int64_t qk, v;   // bytes of q (=k) and v
    int64_t la, eb, wr;
    int64_t o, st;   // bytes of o and of one state tensor
};

Sizes sizes_of(const gdn2_desc *d, int64_t T) {
    Sizes s;
    const int64_t esz = d->qkv_dtype == GDN2_BF16 ? 2 : 4;
    s.tok = d->batch * T * d->heads;
    s.qk = s.tok * d->dk * esz;
    s.v = s.tok * d->dv * esz;
    const int64_t gsz = d->gate_logits ? 2 : 4;  // bf16 logits or fp32 gates
    s.la = s.tok * (d->decay_kind == GDN2_GATE_KEY ? d->dk : 1) * gsz;
    s.eb = s.tok * (d->erase_kind == GDN2_GATE_KEY ? d->dk : 1) * gsz;
    const int64_t wch = d->form == GDN2_FORM_VALUE_WRITE ? d->dv : d->dk;  // channels of the write gate
    s.wr = d->tie_write_to_erase ? 0 : s.tok * (d->write_kind == GDN2_GATE_KEY ? wch : 1) * gsz;
    s.o = s.tok * d->dv * (d->o_dtype == GDN2_BF16 ? 2 : 4);
    s.st = d->batch * d->heads * d->dk * d->dv * 4;
    return s;
}

gdn2_status hip_status(hipError_t e) { return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP; }

// Kernel arguments of a validated descriptor.  `tied` decides whether the
// write gate pointer is kept (the kernels read a null write gate as tied).
ChunkArgs args_of(const gdn2_desc *d, const void *q, const void *k, const void *v, const float *la,
                  const float *eb, const float *wr, const float *s0, float *o, float *s_out) {
    ChunkArgs a;
    a.q = q; a.k = k; a.v = v;
    a.la = la; a.eb = eb; a.wr = d->tie_write_to_erase ? nullptr : wr;
    a.s0 = s0; a.o = o; a.s_out = s_out;
    a.B = d->batch; a.T = d->seqlen; a.H = d->heads; a.dk = d->dk; a.dv = d->dv;
    a.C = static_cast<int>(d->chunk);
    a.bf16 = d->qkv_dtype == GDN2_BF16;
    a.la_key = d->decay_kind == GDN2_GATE_KEY;
    a.eb_key = d->erase_kind == GDN2_GATE_KEY;
    a.wr_key = d->tie_write_to_erase ? a.eb_key : d->write_kind == GDN2_GATE_KEY;
    a.q_scale = d->q_scale;
    a.value_write = d->form == GDN2_FORM_VALUE_WRITE;
    a.gate_logits = d->gate_logits != 0;
    a.qk_norm = d->qk_l2norm != 0;
    a.o_bf16 = d->o_dtype == GDN2_BF16;
    return a;
}

// Whether the two-pass matrix-core path covers the request (it then needs a
// workspace of chunk_split_workspace bytes).
bool split_path(const gdn2_desc *d) {
    static const float placeholder = 0.f;  // stands for an untied write gate
    const ChunkArgs a = args_of(d, nullptr, nullptr, nullptr, nullptr, nullptr, &placeholder, nullptr,
                                nullptr, nullptr);
    return d->batch * d->seqlen > 0 && gdn2::chunk_split_supported(a);
}

// Packed sequences: batch = N sequences along one axis of seqlen = T
// tokens.  The token tensors are the B = 1 layouts; the states have N rows.
gdn2_status check_varlen(const gdn2_desc *d, gdn2_desc *one) {
    if (!d) return GDN2_ERR_NULL;
    if (d->batch < 0 || d->seqlen < 0) return GDN2_ERR_SHAPE;
    if (d->seqlen > INT32_MAX || d->batch >= INT32_MAX) return GDN2_ERR_SHAPE;  // int32 offsets
    *one = *d;
    one->batch = 1;
    gdn2_status st = check_common(one);
    if (st != GDN2_OK) return st;
    int64_t x;
    if (!mul_ok(d->batch, d->heads, &x) || !mul_ok(x, d->dk, &x) || !mul_ok(x, d->dv, &x) || !mul_ok(x, 8, &x))
        return GDN2_ERR_SHAPE;
    if (d->chunk != 16 && d->chunk != 32 && d->chunk != 64) return GDN2_ERR_UNSUPPORTED;
    return GDN2_OK;
}

bool split_path_varlen(const gdn2_desc *d) {
    static const float placeholder = 0.f;  // stands for an untied write gate
    static const int32_t cu_placeholder = 0;
    ChunkArgs a = args_of(d, nullptr, nullptr, nullptr, nullptr, nullptr, &placeholder, nullptr, nullptr,
                          nullptr);
    a.cu = &cu_placeholder;
    return d->batch > 0 && d->seqlen > 0 && gdn2::chunk_split_supported(a);
}

}  // namespace

extern "C" {

int gdn2_abi_version(void) { return GDN2_ABI_VERSION; }

const char *gdn2_status_str(int status) {
    switch (status) {
        case GDN2_OK: return "ok";
        case GDN2_ERR_NULL: return "a required pointer is NULL";
        case GDN2_ERR_SHAPE: return "invalid sizes or gate kinds";
        case GDN2_ERR_DTYPE: return "unknown q/k/v or o dtype";
        case GDN2_ERR_UNSUPPORTED: return "valid request that no kernel of the library covers";
        case GDN2_ERR_ALIAS: return "an output overlaps an input";
        case GDN2_ERR_WORKSPACE: return "workspace too small";
        case GDN2_ERR_HIP: return "a HIP launch failed";
        case GDN2_ERR_SCRATCH: return "request too large for the library's static device scratch";
        default: return "unknown status";
    }
}

gdn2_status gdn2_chunk_fwd_workspace(const gdn2_desc *desc, size_t *bytes) {
    if (!bytes) return GDN2_ERR_NULL;
    gdn2_status st = check_common(desc);
    if (st != GDN2_OK) return st;
    if (desc->chunk != 16 && desc->chunk != 32 && desc->chunk != 64) return GDN2_ERR_UNSUPPORTED;
    *bytes = split_path(desc) ? gdn2::chunk_split_workspace(desc->batch, desc->heads, desc->seqlen) : 0;
    return GDN2_OK;
}

gdn2_status gdn2_chunk_fwd(const gdn2_desc *d, const void *q, const void *k, const void *v,
                           const float *log_decay, const float *erase, const float *write,
                           const float *state0, float *o, float *state_out, void *workspace,
                           size_t ws_bytes, void *stream) {
    size_t need = 0;
    gdn2_status st = gdn2_chunk_fwd_workspace(d, &need);
    if (st != GDN2_OK) return st;
    // no workspace: the single-pass kernels; a workspace must be large enough
    // and 256-byte aligned
    const bool use_ws = workspace != nullptr && ws_bytes > 0;
    if (use_ws && (ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0))
        return GDN2_ERR_WORKSPACE;
    const int64_t T = d->seqlen;
    const bool work = d->batch * T > 0;
    if (work && (!q || !k || !v || !log_decay || !erase || !o)) return GDN2_ERR_NULL;
    if (work && !d->tie_write_to_erase && !write) return GDN2_ERR_NULL;
    const Sizes sz = sizes_of(d, T);
    const Span in[] = {span_of(q, sz.qk), span_of(k, sz.qk), span_of(v, sz.v),
                       span_of(log_decay, sz.la), span_of(erase, sz.eb),
                       span_of(d->tie_write_to_erase ? nullptr : write, sz.wr)};
    const Span s_in = span_of(state0, sz.st), s_out = span_of(state_out, sz.st);
    const Span o_sp = span_of(o, sz.o);
    for (const Span &x : in) {
        if (overlap(o_sp, x) || overlap(s_out, x)) return GDN2_ERR_ALIAS;
    }
    if (overlap(o_sp, s_in) || overlap(o_sp, s_out)) return GDN2_ERR_ALIAS;
    if (overlap(s_out, s_in) && s_out.lo != s_in.lo) return GDN2_ERR_ALIAS;
    if (use_ws) {
        const Span ws = span_of(workspace, static_cast<int64_t>(ws_bytes));
        for (const Span &x : in)
            if (overlap(ws, x)) return GDN2_ERR_ALIAS;
        if (overlap(ws, o_sp) || overlap(ws, s_in) || overlap(ws, s_out)) return GDN2_ERR_ALIAS;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {
        // nothing to read but the initial state
        if (state_out && state_out != state0)
            return hip_status(gdn2::launch_state_copy(state0, state_out, sz.st / 4, s));
        return GDN2_OK;
    }
    const ChunkArgs a = args_of(d, q, k, v, log_decay, erase, write, state0, o, state_out);
    if (a.B * a.H > 0x7fffffffLL) return GDN2_ERR_UNSUPPORTED;
    if (use_ws && need > 0) return hip_status(gdn2::launch_chunk_split(a, workspace, s));
    if (gdn2::chunk_mfma_supported(a)) return hip_status(gdn2::launch_chunk_mfma(a, s));
    return hip_status(gdn2::launch_chunk_general(a, s));
}

gdn2_status gdn2_chunk_fwd_static(const gdn2_desc *d, const void *q, const void *k, const void *v,
                                  const float *log_decay, const float *erase, const float *write,
                                  const float *state0, float *o, float *state_out, void *stream) {
    size_t need = 0;
    gdn2_status st = gdn2_chunk_fwd_workspace(d, &need);
    if (st != GDN2_OK) return st;
    const int64_t T = d->seqlen;
    const bool work = d->batch * T > 0;
    if (work && (!q || !k || !v || !log_decay || !erase || !o)) return GDN2_ERR_NULL;
    if (work && !d->tie_write_to_erase && !write) return GDN2_ERR_NULL;
    const Sizes sz = sizes_of(d, T);
    const Span in[] = {span_of(q, sz.qk), span_of(k, sz.qk), span_of(v, sz.v),
                       span_of(log_decay, sz.la), span_of(erase, sz.eb),
                       span_of(d->tie_write_to_erase ? nullptr : write, sz.wr)};
    const Span s_in = span_of(state0, sz.st), s_out = span_of(state_out, sz.st);
    const Span o_sp = span_of(o, sz.o);
    for (const Span &x : in) {
        if (overlap(o_sp, x) || overlap(s_out, x)) return GDN2_ERR_ALIAS;
    }
    if (overlap(o_sp, s_in) || overlap(o_sp, s_out)) return GDN2_ERR_ALIAS;
    if (overlap(s_out, s_in) && s_out.lo != s_in.lo) return GDN2_ERR_ALIAS;
    if (need > 0 && !gdn2::chunk_split_static_fits(d->batch, d->heads, T)) return GDN2_ERR_SCRATCH;

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {
        if (state_out && state_out != state0)
            return hip_status(gdn2::launch_state_copy(state0, state_out, sz.st / 4, s));
        return GDN2_OK;
    }
    const ChunkArgs a = args_of(d, q, k, v, log_decay, erase, write, state0, o, state_out);
    if (a.B * a.H > 0x7fffffffLL) return GDN2_ERR_UNSUPPORTED;
    // the two-pass kernels through the static scratch; every other request
    // runs on kernels that use no scratch at all
    if (need > 0) return hip_status(gdn2::launch_chunk_split_static(a, s));
    if (gdn2::chunk_mfma_supported(a)) return hip_status(gdn2::launch_chunk_mfma(a, s));
    return hip_status(gdn2::launch_chunk_general(a, s));
}

gdn2_status gdn2_chunk_fwd_varlen_workspace(const gdn2_desc *desc, size_t *bytes) {
    if (!bytes) return GDN2_ERR_NULL;
    gdn2_desc one;
    gdn2_status st = check_varlen(desc, &one);
    if (st != GDN2_OK) return st;
    *bytes = split_path_varlen(desc) ? gdn2::chunk_split_workspace_varlen(desc->batch, desc->heads, desc->seqlen) : 0;
    return GDN2_OK;
}

gdn2_status gdn2_chunk_fwd_varlen(const gdn2_desc *d, const int32_t *cu_seqlens, const void *q, const void *k,
                                  const void *v, const float *log_decay, const float *erase, const float *write,
                                  const float *state0, float *o, float *state_out, void *workspace,
                                  size_t ws_bytes, void *stream) {
    size_t need = 0;
    gdn2_status st = gdn2_chunk_fwd_varlen_workspace(d, &need);
    if (st != GDN2_OK) return st;
    const bool use_ws = workspace != nullptr && ws_bytes > 0;
    if (use_ws && (ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0))
        return GDN2_ERR_WORKSPACE;
    const int64_t N = d->batch, T = d->seqlen;
    if (N == 0) return GDN2_OK;  // no sequence: nothing to read or write
    if (!cu_seqlens) return GDN2_ERR_NULL;
    const bool work = T > 0;
    if (work && (!q || !k || !v || !log_decay || !erase || !o)) return GDN2_ERR_NULL;
    if (work && !d->tie_write_to_erase && !write) return GDN2_ERR_NULL;
    gdn2_desc one = *d;
    one.batch = 1;
    const Sizes sz = sizes_of(&one, T);
    const int64_t stb = N * d->heads * d->dk * d->dv * 4;
    const Span in[] = {span_of(q, sz.qk), span_of(k, sz.qk), span_of(v, sz.v),
                       span_of(log_decay, sz.la), span_of(erase, sz.eb),
                       span_of(d->tie_write_to_erase ? nullptr : write, sz.wr),
                       span_of(cu_seqlens, (N + 1) * 4)};
    const Span s_in = span_of(state0, stb), s_out = span_of(state_out, stb);
    const Span o_sp = span_of(o, sz.o);
    for (const Span &x : in) {
        if (overlap(o_sp, x) || overlap(s_out, x)) return GDN2_ERR_ALIAS;
    }
    if (overlap(o_sp, s_in) || overlap(o_sp, s_out)) return GDN2_ERR_ALIAS;
    if (overlap(s_out, s_in) && s_out.lo != s_in.lo) return GDN2_ERR_ALIAS;
    if (use_ws) {
        const Span ws = span_of(workspace, static_cast<int64_t>(ws_bytes));
        for (const Span &x : in)
            if (overlap(ws, x)) return GDN2_ERR_ALIAS;
        if (overlap(ws, o_sp) || overlap(ws, s_in) || overlap(ws, s_out)) return GDN2_ERR_ALIAS;
    }

    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {  // every sequence empty
        if (state_out && state_out != state0)
            return hip_status(gdn2::launch_state_copy(state0, state_out, stb / 4, s));
        return GDN2_OK;
    }
    ChunkArgs a = args_of(d, q, k, v, log_decay, erase, write, state0, o, state_out);
    a.cu = cu_seqlens;
    if (a.B * a.H > 0x7fffffffLL) return GDN2_ERR_UNSUPPORTED;
    if (use_ws && need > 0) return hip_status(gdn2::launch_chunk_split(a, workspace, s));
    return hip_status(gdn2::launch_chunk_general(a, s));
}

gdn2_status gdn2_chunk_bwd_workspace(const gdn2_desc *desc, size_t *bytes) {
    if (!bytes) return GDN2_ERR_NULL;
    gdn2_status st = check_common(desc);
    if (st != GDN2_OK) return st;
    if (desc->chunk != 16 && desc->chunk != 32 && desc->chunk != 64) return GDN2_ERR_UNSUPPORTED;
    if (!gdn2::chunk_bwd_chunk(desc->dk, desc->dv, static_cast<int>(desc->chunk))) return GDN2_ERR_UNSUPPORTED;
    static const float placeholder = 0.f;  // stands for an untied write gate
    const ChunkArgs a = args_of(desc, nullptr, nullptr, nullptr, nullptr, nullptr, &placeholder, nullptr,
                                nullptr, nullptr);
    *bytes = gdn2::chunk_bwd_workspace(a);
    return GDN2_OK;
}

gdn2_status gdn2_chunk_bwd(const gdn2_desc *d, const void *q, const void *k, const void *v,
                           const float *log_decay, const float *erase, const float *write,
                           const float *state0, const float *d_o, const float *d_state_out,
                           float *dq, float *dk, float *dv, float *d_log_decay, float *d_erase,
                           float *d_write, float *d_state0, void *workspace, size_t ws_bytes,
                           void *stream) {
    size_t need = 0;
    gdn2_status st = gdn2_chunk_bwd_workspace(d, &need);
    if (st != GDN2_OK) return st;
    if (need > 0 && (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0))
        return GDN2_ERR_WORKSPACE;
    const int64_t T = d->seqlen;
    const bool work = d->batch * T > 0;
    const bool tied = d->tie_write_to_erase != 0;
    if (work && (!q || !k || !v || !log_decay || !erase || !d_o || !dq || !dk || !dv || !d_log_decay || !d_erase))
        return GDN2_ERR_NULL;
    if (work && !tied && (!write || !d_write)) return GDN2_ERR_NULL;
    const Sizes sz = sizes_of(d, T);
    // d_o is fp32 whatever desc->o_dtype says
    const Span in[] = {span_of(q, sz.qk), span_of(k, sz.qk), span_of(v, sz.v),
                       span_of(log_decay, sz.la), span_of(erase, sz.eb),
                       span_of(tied ? nullptr : write, sz.wr), span_of(state0, sz.st),
                       span_of(d_o, sz.tok * d->dv * 4), span_of(d_state_out, sz.st)};
    // gradients are fp32 and shaped like their inputs (those of bf16 gate
    // logits too)
    const int64_t f32 = d->qkv_dtype == GDN2_BF16 ? 2 : 1;
    gdn2_desc d4 = *d;
    d4.gate_logits = 0;
    const Sizes sg = sizes_of(&d4, T);
    const Span out[] = {span_of(dq, sz.qk * f32), span_of(dk, sz.qk * f32), span_of(dv, sz.v * f32),
                        span_of(d_log_decay, sg.la), span_of(d_erase, sg.eb),
                        span_of(tied ? nullptr : d_write, sg.wr), span_of(d_state0, sz.st),
                        span_of(workspace, need > 0 ? static_cast<int64_t>(ws_bytes) : 0)};
    const int nout = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < nout; ++i) {
        for (const Span &x : in)
            if (overlap(out[i], x)) return GDN2_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j])) return GDN2_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {
        // S_T = S0: the state gradient passes through unchanged
        if (d_state0) return hip_status(gdn2::launch_state_copy(d_state_out, d_state0, sz.st / 4, s));
        return GDN2_OK;
    }
    if (d->batch * d->heads > 0x7fffffffLL) return GDN2_ERR_UNSUPPORTED;
    gdn2::BwdArgs a;
    a.f = args_of(d, q, k, v, log_decay, erase, write, state0, nullptr, nullptr);
    a.d_o = d_o;
    a.d_sT = d_state_out;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.dla = d_log_decay; a.deb = d_erase; a.dwr = tied ? nullptr : d_write;
    a.ds0 = d_state0;
    return hip_status(gdn2::launch_chunk_bwd(a, workspace, s));
}

gdn2_status gdn2_chunk_bwd_varlen_workspace(const gdn2_desc *desc, size_t *bytes) {
    if (!bytes) return GDN2_ERR_NULL;
    gdn2_desc one;
    gdn2_status st = check_varlen(desc, &one);
    if (st != GDN2_OK) return st;
    if (!gdn2::chunk_bwd_chunk(desc->dk, desc->dv, static_cast<int>(desc->chunk))) return GDN2_ERR_UNSUPPORTED;
    static const float placeholder = 0.f;  // stands for an untied write gate
    static const int32_t cu_placeholder = 0;
    ChunkArgs a = args_of(desc, nullptr, nullptr, nullptr, nullptr, nullptr, &placeholder, nullptr, nullptr, nullptr);
    a.cu = &cu_placeholder;
    *bytes = gdn2::chunk_bwd_workspace(a);
    return GDN2_OK;
}

gdn2_status gdn2_chunk_bwd_varlen(const gdn2_desc *d, const int32_t *cu_seqlens, const void *q, const void *k,
                                  const void *v, const float *log_decay, const float *erase, const float *write,
                                  const float *state0, const float *d_o, const float *d_state_out, float *dq,
                                  float *dk, float *dv, float *d_log_decay, float *d_erase, float *d_write,
                                  float *d_state0, void *workspace, size_t ws_bytes, void *stream) {
    size_t need = 0;
    gdn2_status st = gdn2_chunk_bwd_varlen_workspace(d, &need);
    if (st != GDN2_OK) return st;
    const int64_t N = d->batch, T = d->seqlen;
    if (N == 0) return GDN2_OK;  // no sequence: nothing to read or write
    if (!cu_seqlens) return GDN2_ERR_NULL;
    if (need > 0 && (!workspace || ws_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255) != 0))
        return GDN2_ERR_WORKSPACE;
    const bool work = T > 0;
    const bool tied = d->tie_write_to_erase != 0;
    if (work && (!q || !k || !v || !log_decay || !erase || !d_o || !dq || !dk || !dv || !d_log_decay || !d_erase))
        return GDN2_ERR_NULL;
    if (work && !tied && (!write || !d_write)) return GDN2_ERR_NULL;
    gdn2_desc one = *d;
    one.batch = 1;
    const Sizes sz = sizes_of(&one, T);
    const int64_t stb = N * d->heads * d->dk * d->dv * 4;
    const Span in[] = {span_of(q, sz.qk), span_of(k, sz.qk), span_of(v, sz.v),
                       span_of(log_decay, sz.la), span_of(erase, sz.eb),
                       span_of(tied ? nullptr : write, sz.wr), span_of(state0, stb),
                       span_of(d_o, sz.tok * d->dv * 4), span_of(d_state_out, stb),
                       span_of(cu_seqlens, (N + 1) * 4)};
    const int64_t f32 = d->qkv_dtype == GDN2_BF16 ? 2 : 1;
    gdn2_desc d4 = one;
    d4.gate_logits = 0;
    const Sizes sg = sizes_of(&d4, T);
    const Span out[] = {span_of(dq, sz.qk * f32), span_of(dk, sz.qk * f32), span_of(dv, sz.v * f32),
                        span_of(d_log_decay, sg.la), span_of(d_erase, sg.eb),
                        span_of(tied ? nullptr : d_write, sg.wr), span_of(d_state0, stb),
                        span_of(workspace, need > 0 ? static_cast<int64_t>(ws_bytes) : 0)};
    const int nout = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < nout; ++i) {
        for (const Span &x : in)
            if (overlap(out[i], x)) return GDN2_ERR_ALIAS;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i], out[j])) return GDN2_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!work) {  // every sequence empty: the state gradients pass through
        if (d_state0) return hip_status(gdn2::launch_state_copy(d_state_out, d_state0, stb / 4, s));
        return GDN2_OK;
    }
    if (N * d->heads > 0x7fffffffLL) return GDN2_ERR_UNSUPPORTED;
    gdn2::BwdArgs a;
    a.f = args_of(d, q, k, v, log_decay, erase, write, state0, nullptr, nullptr);
    a.f.cu = cu_seqlens;
    a.d_o = d_o;
    a.d_sT = d_state_out;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.dla = d_log_decay; a.deb = d_erase; a.dwr = tied ? nullptr : d_write;
    a.ds0 = d_state0;
    return hip_status(gdn2::launch_chunk_bwd(a, workspace, s));
}

gdn2_status gdn2_recurrent_step(const gdn2_desc *d, const void *q, const void *k, const void *v,
                                const float *log_decay, const float *erase, const float *write,
                                float *state, float *o, void *stream) {
    gdn2_status st = check_common(d);
    if (st != GDN2_OK) return st;
    if (d->seqlen != 1) return GDN2_ERR_SHAPE;
    if (d->batch == 0) return GDN2_OK;
    if (!q || !k || !v || !log_decay || !erase || !state || !o) return GDN2_ERR_NULL;
    if (!d->tie_write_to_erase && !write) return GDN2_ERR_NULL;
    const Sizes sz = sizes_of(d, 1);
    const Span in[] = {span_of(q, sz.qk), span_of(k, sz.qk), span_of(v, sz.v),
                       span_of(log_decay, sz.la), span_of(erase, sz.eb),
                       span_of(d->tie_write_to_erase ? nullptr : write, sz.wr)};
    const Span s_sp = span_of(state, sz.st), o_sp = span_of(o, sz.o);
    for (const Span &x : in) {
        if (overlap(o_sp, x) || overlap(s_sp, x)) return GDN2_ERR_ALIAS;
    }
    if (overlap(o_sp, s_sp)) return GDN2_ERR_ALIAS;
    if (d->batch * d->heads > 0x7fffffffLL) return GDN2_ERR_UNSUPPORTED;
    StepArgs a;
    a.q = q; a.k = k; a.v = v;
    a.la = log_decay; a.eb = erase; a.wr = d->tie_write_to_erase ? nullptr : write;
    a.state = state; a.o = o;
    a.N = d->batch; a.H = d->heads; a.dk = d->dk; a.dv = d->dv;
    a.bf16 = d->qkv_dtype == GDN2_BF16;
    a.la_key = d->decay_kind == GDN2_GATE_KEY;
    a.eb_key = d->erase_kind == GDN2_GATE_KEY;
    a.wr_key = d->tie_write_to_erase ? a.eb_key : d->write_kind == GDN2_GATE_KEY;
    a.q_scale = d->q_scale;
    a.value_write = d->form == GDN2_FORM_VALUE_WRITE;
    a.gate_logits = d->gate_logits != 0;
    a.qk_norm = d->qk_l2norm != 0;
    a.o_bf16 = d->o_dtype == GDN2_BF16;
    return hip_status(gdn2::launch_step(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
