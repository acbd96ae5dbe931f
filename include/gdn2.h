/*
 * gdn2.h -- C ABI of the MI355X (gfx950) gated delta rule-2 library.
 *
 * The operation (per batch b, head h; state S in R^{dk x dv}, key-by-value:
 * rows are key channels, columns value channels), for each token t:
 *
 *     Sbar = Diag(a_t) S                 decay first; a_t = exp(log_decay_t)
 *     m    = Sbar^T k_t                  the key read of the decayed state
 *     S    = Sbar - (b_t .* k_t) m^T + (w_t .* k_t) v_t^T
 *     o_t  = S^T (q_scale * q_t)         the query read of the updated state
 *
 * Sources: the "Gated DeltaNet-2" blog summary ("Core Mechanism": separate
 * channel-wise erase gate b_t and write gate w_t, channel-wise decay, the
 * chunkwise WY training algorithm and O(1)-memory recurrent inference); the
 * "Gated DeltaNet" page ("Decay first, then compute the write error": the
 * read and the subtraction use the decayed state); the course slides
 * ("Worked case -- full trace": decay, read, correct, then read with q).
 * Both gates act on the key axis.  Tying b = w = beta (scalar) gives Gated
 * DeltaNet, per-channel decay with tied scalar beta gives KDA, a = 1 gives
 * the delta rule (gist.science summary, "Technische Samenvatting", sec. 1).
 *
 * desc->form = GDN2_FORM_VALUE_WRITE selects the update as the gist.science
 * summary writes it ("Methodologie", 1. "Gated Delta-regel-2"):
 *
 *     S    = (I - k_t (b_t .* k_t)^T) Sbar + k_t (w_t .* v_t)^T
 *
 * i.e. the erase gate weights the read (m = Sbar^T (b_t .* k_t)), the erase
 * and the write run along k_t, and the write gate has one factor per VALUE
 * channel.  With scalar gates both forms are the same operation.
 *
 * Conventions shared by every call:
 *  - Every data pointer is DEVICE memory (hipMalloc'd or torch CUDA
 *    tensors) owned by the caller; the library allocates nothing and is
 *    safe to call from several host threads.  Its only global state is the
 *    static scratch of gdn2_chunk_fwd_static and that array's per-GPU
 *    address, looked up once.
 *  - All tensors are contiguous, row-major, last index fastest:
 *        q, k           [B, T, H, dk]    bf16 or fp32 (desc->qkv_dtype)
 *        v              [B, T, H, dv]    same dtype as q, k
 *        o              [B, T, H, dv]    fp32, or bf16 (desc->o_dtype)
 *        log_decay      [B, T, H, dk] fp32 if decay_kind == GDN2_GATE_KEY,
 *                       [B, T, H]     fp32 if GDN2_GATE_HEAD
 *        erase, write   same rule with erase_kind / write_kind (the write
 *                       gate of GDN2_FORM_VALUE_WRITE: [B, T, H, dv] per
 *                       channel)
 *        state tensors  [B, H, dk, dv]   fp32
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and the call returns without synchronising.  Device faults surface at
 *    the caller's next synchronisation.
 *  - Host-side validation runs before any HIP call: on any status other
 *    than GDN2_OK nothing has been enqueued and no output was touched
 *    (GDN2_ERR_HIP aside, which reports a failed launch).
 *  - Input preparation may be fused (desc->gate_logits, desc->qk_l2norm):
 *    the gates then arrive as bf16 logits and q, k unnormalised, and the
 *    kernels apply the activations and the normalisation as they load them
 *    (2048 instead of 2816 bytes per token-head for the full GDN-2 forward).
 *  - Preconditions not checked (they would need a device pass): log_decay
 *    finite and <= 0 (decay gate in (0, 1], course slides "Stability"),
 *    erase/write in [0, 1], all values finite.  These hold for every call
 *    and every path.  The matrix-core forward kernels of gdn2_chunk_fwd,
 *    gdn2_chunk_fwd_static and gdn2_chunk_fwd_varlen (bf16 q/k/v, dk = dv =
 *    128) hold derived operands, intermediates and a copy of the state in
 *    fp16; a chunk whose values would leave fp16's range is recomputed as
 *    the exact fp32 token recurrence instead, with the workspace and without
 *    it, so they ask nothing more (tested with |v| and states of 2^15).  The
 *    backward, the decode step and the fp32 kernels compute in fp32.
 */
#ifndef GDN2_H
#define GDN2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN2_ABI_VERSION 6

typedef enum gdn2_status {
    GDN2_OK = 0,
    GDN2_ERR_NULL = 1,        /* a required pointer (or desc) is NULL            */
    GDN2_ERR_SHAPE = 2,       /* negative / zero / overflowing sizes            */
    GDN2_ERR_DTYPE = 3,       /* unknown qkv_dtype or o_dtype                    */
    GDN2_ERR_UNSUPPORTED = 4, /* valid request no kernel of the library covers  */
    GDN2_ERR_ALIAS = 5,       /* an output overlaps an input (see each call)     */
    GDN2_ERR_WORKSPACE = 6,   /* workspace smaller than the query reported      */
    GDN2_ERR_HIP = 7,         /* a HIP launch or copy failed                     */
    GDN2_ERR_SCRATCH = 8      /* too large for the static scratch of
                                 gdn2_chunk_fwd_static                           */
} gdn2_status;

typedef enum gdn2_dtype { GDN2_F32 = 0, GDN2_BF16 = 1 } gdn2_dtype;

typedef enum gdn2_gate_kind {
    GDN2_GATE_HEAD = 0, /* one value per token-head, shared by all key channels */
    GDN2_GATE_KEY = 1   /* one value per key channel                            */
} gdn2_gate_kind;

typedef enum gdn2_form {
    GDN2_FORM_KEY = 0,         /* erase (b.*k)(k^T Sbar), write (w.*k) v^T  */
    GDN2_FORM_VALUE_WRITE = 1  /* erase k((b.*k)^T Sbar), write k (w.*v)^T;
                                  needs an untied write gate               */
} gdn2_form;

/* Problem description.  For gdn2_recurrent_step `batch` is the number of
 * sequences N and `seqlen` must be 1. */
typedef struct gdn2_desc {
    int64_t batch;      /* B >= 0 */
    int64_t seqlen;     /* T >= 0 */
    int64_t heads;      /* H >= 1 */
    int64_t dk;         /* key channels,   1..128 */
    int64_t dv;         /* value channels, 1..128 */
    int64_t chunk;      /* chunk length C of the chunkwise algorithm: 16, 32 or 64 */
    int32_t qkv_dtype;  /* gdn2_dtype of q, k, v */
    int32_t decay_kind; /* gdn2_gate_kind of log_decay */
    int32_t erase_kind; /* gdn2_gate_kind of erase      */
    int32_t write_kind; /* gdn2_gate_kind of write (ignored when tied) */
    int32_t tie_write_to_erase; /* nonzero: w := b and `write` is ignored */
    float q_scale;      /* multiplies q; 1.0 for the plain read */
    int32_t form;       /* gdn2_form; a tied write gate with
                           GDN2_FORM_VALUE_WRITE is GDN2_ERR_SHAPE */
    int32_t gate_logits; /* nonzero: log_decay, erase and write point at bf16
                            LOGITS x (same shapes, 2 bytes per element; the
                            float* parameters are reinterpreted); the kernels
                            use log a = -softplus(x), b = sigmoid(x),
                            w = sigmoid(x) */
    int32_t qk_l2norm;  /* nonzero: q and k are divided by their L2 norm over
                           the dk channels of each token-head inside the
                           kernels (a zero vector stays zero), before q_scale */
    int32_t o_dtype;    /* gdn2_dtype of the output o of gdn2_chunk_fwd,
                           gdn2_chunk_fwd_varlen and gdn2_recurrent_step:
                           GDN2_F32 (0, the default) or GDN2_BF16, the fp32
                           result rounded to nearest even (2 bytes per element;
                           the float* o parameter is reinterpreted).  Anything
                           else is GDN2_ERR_DTYPE.  The backward's d_o is fp32
                           whatever this says. */
} gdn2_desc;

/* GDN2_ABI_VERSION of the loaded library. */
int gdn2_abi_version(void);

/* Static, human-readable name of a status code. */
const char *gdn2_status_str(int status);

/* Device workspace, in bytes, for the two-pass form of gdn2_chunk_fwd on
 * `desc`; 0 when the request has no two-pass kernel (it then always runs in
 * one pass).  The two-pass form covers bf16 q/k/v, dk = dv = 128, chunk 64
 * and gates per key channel or per head (a per-head decay only with
 * per-head erase and write gates; untied, the write gate of the erase
 * gate's kind); it needs B*H*ceil(T/64) records of about
 * 71 KiB, and, when B*H is small against T (long sequences on few chains,
 * scanned in parallel segments), two 64 KiB states per (chain, segment).
 * Same validation as gdn2_chunk_fwd. */
gdn2_status gdn2_chunk_fwd_workspace(const gdn2_desc *desc, size_t *bytes);

/*
 * Chunkwise-parallel forward over whole sequences (training / prefill).
 *
 * The "Gated DeltaNet-2" blog summary ("Core Mechanism") and the
 * gist.science summary ("Technische Samenvatting", section 3) describe the
 * algorithm: the cumulative per-channel decay of each chunk is absorbed
 * into the erase and write factors, a unit-lower-triangular solve gives the
 * chunk's auxiliary matrices, and dense chunk contractions carry the state
 * from chunk to chunk.  The result equals running the recurrence above
 * token by token (up to rounding); the chunk length only changes speed.
 *
 *   q, k, v      inputs, see layouts above.
 *   log_decay    log of the decay gate (<= 0).
 *   erase        erase gate b.
 *   write        write gate w; ignored (may be NULL) when
 *                desc->tie_write_to_erase is set.
 *   state0       initial state [B,H,dk,dv] fp32, or NULL for zeros.
 *   o            output [B,T,H,dv], fp32 or bf16 per desc->o_dtype (must not overlap
 *                any input).
 *   state_out    final state [B,H,dk,dv] fp32, or NULL to skip.  It may be
 *                exactly state0 (updated in place); any other overlap with
 *                an input is GDN2_ERR_ALIAS.
 *   workspace    NULL (or ws_bytes 0): run in one pass, no scratch.
 *                Otherwise device scratch of ws_bytes >=
 *                gdn2_chunk_fwd_workspace(), 256-byte aligned, else
 *                GDN2_ERR_WORKSPACE; it must not overlap any other argument
 *                (GDN2_ERR_ALIAS).  The two-pass form first computes every
 *                chunk's state-independent products in parallel into it,
 *                then scans the chunks; its contents need no initialisation
 *                and are undefined afterwards.  Calls that share one
 *                workspace must not overlap in time.
 * With T == 0 nothing is read but state0, o is untouched and state_out
 * receives state0 (or zeros).
 */
gdn2_status gdn2_chunk_fwd(const gdn2_desc *desc,
                           const void *q, const void *k, const void *v,
                           const float *log_decay, const float *erase, const float *write,
                           const float *state0, float *o, float *state_out,
                           void *workspace, size_t ws_bytes, void *stream);

/*
 * gdn2_chunk_fwd without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, layouts, rules and result as
 * gdn2_chunk_fwd with workspace = NULL, except that requests of the
 * two-pass form keep their per-chunk records in one static device array of
 * the library, 128 MiB per GPU, held from the first such call on a GPU until
 * the process ends.  When the records of all ceil(T/64) chunks of every
 * chain do not fit there, the chunks are processed in consecutive windows
 * that do, the state carried from window to window in the same array
 * (more launches, the same arithmetic).  Each record takes 70.5 KiB and
 * each carried state 64 KiB: a request fits in one window up to
 * B*H*ceil(T/64) = 1859 records, in windows up to B*H = 974 chains; beyond
 * both it returns GDN2_ERR_SCRATCH before anything is enqueued.  Requests without a two-pass
 * kernel run the single-pass kernels, which use no scratch.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and give undefined
 * results; serialise them.  The array needs no initialisation.  The first
 * call on each GPU looks up the array's device address (hipGetSymbolAddress)
 * and keeps it; no call allocates or frees memory.
 */
gdn2_status gdn2_chunk_fwd_static(const gdn2_desc *desc,
                                  const void *q, const void *k, const void *v,
                                  const float *log_decay, const float *erase, const float *write,
                                  const float *state0, float *o, float *state_out, void *stream);

/* Device workspace, in bytes, for the two-pass form of gdn2_chunk_fwd_varlen
 * on `desc` (batch = N sequences, seqlen = T packed tokens); 0 when the
 * request has no two-pass kernel.  It holds records for ceil(T/64) + N
 * chunks per head (every sequence may end in a partial chunk) and the
 * sequence plan.  Same validation as gdn2_chunk_fwd_varlen. */
gdn2_status gdn2_chunk_fwd_varlen_workspace(const gdn2_desc *desc, size_t *bytes);

/*
 * The chunkwise forward over N sequences of different lengths packed along
 * one token axis (training on packed documents, prefill of a batch of
 * prompts).  The sequences are independent recurrences, each from its own
 * initial state: the result for sequence i equals gdn2_chunk_fwd on its
 * tokens alone.  Chunks never straddle two sequences; each sequence's
 * chunks start at its first token ("Gated DeltaNet" page, "What makes the
 * architecture more than a recurrence": chunkwise training over long
 * sequences, each transition an affine map of the state).
 *
 *   desc         batch = N >= 0 sequences, seqlen = T >= 0 packed tokens
 *                (T <= INT32_MAX), other fields as for gdn2_chunk_fwd.
 *   cu_seqlens   DEVICE int32 [N+1]: sequence i covers packed tokens
 *                cu_seqlens[i] .. cu_seqlens[i+1]-1; required
 *                0 = cu_seqlens[0] <= cu_seqlens[1] <= ... <= cu_seqlens[N]
 *                = T.  Not checked (it would need a device pass): other
 *                offsets give unspecified results, but every offset is
 *                clamped into [0, T] and every range made non-negative, so
 *                no access leaves the tensors or the workspace.
 *   q, k, v, gates, o   [T, H, ...]: the [B, T, H, ...] layouts with B = 1.
 *   state0, state_out   [N, H, dk, dv] fp32, one state per sequence
 *                (state0 NULL: zeros; state_out NULL: skipped; in place as
 *                for gdn2_chunk_fwd).
 *   workspace    as for gdn2_chunk_fwd with gdn2_chunk_fwd_varlen_workspace()
 *                bytes; NULL runs the single-kernel path.
 * Outputs must not overlap cu_seqlens, any other input or the workspace
 * (GDN2_ERR_ALIAS).  Rows of o outside every sequence are untouched; an
 * empty sequence passes its initial state through.
 */
gdn2_status gdn2_chunk_fwd_varlen(const gdn2_desc *desc, const int32_t *cu_seqlens,
                                  const void *q, const void *k, const void *v,
                                  const float *log_decay, const float *erase, const float *write,
                                  const float *state0, float *o, float *state_out,
                                  void *workspace, size_t ws_bytes, void *stream);

/* Device workspace, in bytes, for gdn2_chunk_bwd on `desc`: two fp32 state
 * histories, B*H*ceil(T/Cb)*dk*dv*4 bytes each (Cb = 16 for dk = dv = 128,
 * larger for small heads); for dk = dv = 128 a 37 KiB fp32 record per
 * (chain, internal chunk); with fused input preparation an fp32 copy of the
 * prepared inputs (q, k, v and two norms per token-head when qk_l2norm, the
 * activated gates when gate_logits).  Each region 256-byte aligned.  Same
 * validation as gdn2_chunk_fwd; GDN2_ERR_UNSUPPORTED if no internal chunk
 * fits. */
gdn2_status gdn2_chunk_bwd_workspace(const gdn2_desc *desc, size_t *bytes);

/*
 * Backward of gdn2_chunk_fwd: the gradients of
 *     L = <d_o, o> + <d_state_out, S_T>
 * with respect to q, k, v, the three gates and state0.  Training is why the
 * chunk form exists ("Gated DeltaNet-2" blog summary, "Core Mechanism": the
 * chunkwise algorithm and its kernels serve training; gist.science summary,
 * "Technische Samenvatting" section 3).  The result equals reverse-mode
 * differentiation of the token recurrence (up to rounding).  It is computed
 * chunk by chunk in fp32 (on the matrix cores for dk = dv = 128): a forward
 * scan records the state entering every internal chunk, a reverse scan
 * carries the state gradient back through the chunks, then every chunk
 * forms its gradients in parallel from the two records.  Both forms
 * (desc->form) are covered.  With fused input preparation (desc->gate_logits,
 * desc->qk_l2norm) the gradients are those of the raw inputs: of the gate
 * logits (through -softplus and sigmoid) and of unnormalised q, k (through
 * the L2 normalisation; a zero row gets zero).
 *
 *   q .. state0  the forward's inputs (same layouts and rules as
 *                gdn2_chunk_fwd; state0 NULL means zeros).
 *   d_o          gradient of o, [B,T,H,dv] fp32 (required).
 *   d_state_out  gradient of the final state [B,H,dk,dv] fp32, or NULL for
 *                zeros.
 *   dq, dk, dv   fp32, [B,T,H,dk] / [B,T,H,dv] (fp32 whatever qkv_dtype).
 *   d_log_decay, d_erase, d_write   fp32, shaped like their gate (per key
 *                channel or per token-head; the value-write form's write gate
 *                per value channel), also for bf16 logits; d_write ignored
 *                (may be NULL) when tied, and then d_erase holds the gradient
 *                of the one shared gate.
 *   d_state0     gradient of state0 [B,H,dk,dv] fp32, or NULL to skip.
 *   workspace    device scratch of ws_bytes >= gdn2_chunk_bwd_workspace(),
 *                256-byte aligned, else GDN2_ERR_WORKSPACE; contents need no
 *                initialisation and are undefined afterwards.
 * Outputs must not overlap each other, any input or the workspace
 * (GDN2_ERR_ALIAS).  Every output is written in full.  With T == 0,
 * d_state0 receives d_state_out (or zeros) and nothing else is touched.
 */
gdn2_status gdn2_chunk_bwd(const gdn2_desc *desc,
                           const void *q, const void *k, const void *v,
                           const float *log_decay, const float *erase, const float *write,
                           const float *state0, const float *d_o, const float *d_state_out,
                           float *dq, float *dk, float *dv,
                           float *d_log_decay, float *d_erase, float *d_write,
                           float *d_state0, void *workspace, size_t ws_bytes, void *stream);

/* Device workspace, in bytes, for gdn2_chunk_bwd_varlen on `desc` (batch =
 * N sequences, seqlen = T packed tokens): the regions of
 * gdn2_chunk_bwd_workspace sized for ceil(T/Cb) + N internal chunks per head,
 * and the sequence plan.  Same validation as gdn2_chunk_bwd_varlen. */
gdn2_status gdn2_chunk_bwd_varlen_workspace(const gdn2_desc *desc, size_t *bytes);

/*
 * Backward of gdn2_chunk_fwd_varlen: the gradients of
 *     L = <d_o, o> + <d_state_out, S_T(i) for every sequence i>
 * for N sequences packed along one token axis, each its own recurrence
 * (training on packed documents).  The result for sequence i equals
 * gdn2_chunk_bwd on its tokens alone.
 *
 *   desc, cu_seqlens   as for gdn2_chunk_fwd_varlen (offsets unchecked, but
 *                clamped so that no access leaves the buffers).
 *   q .. write, d_o, the gradients of q .. write   [T, H, ...] (the B = 1
 *                layouts), rules as for gdn2_chunk_bwd.
 *   state0, d_state_out, d_state0   [N, H, dk, dv] fp32.
 *   workspace    as for gdn2_chunk_bwd, gdn2_chunk_bwd_varlen_workspace() bytes.
 * Outputs must not overlap each other, cu_seqlens, any other input or the
 * workspace (GDN2_ERR_ALIAS).  Rows outside every sequence are untouched; an
 * empty sequence passes its state gradient through to d_state0.
 */
gdn2_status gdn2_chunk_bwd_varlen(const gdn2_desc *desc, const int32_t *cu_seqlens,
                                  const void *q, const void *k, const void *v,
                                  const float *log_decay, const float *erase, const float *write,
                                  const float *state0, const float *d_o, const float *d_state_out,
                                  float *dq, float *dk, float *dv,
                                  float *d_log_decay, float *d_erase, float *d_write,
                                  float *d_state0, void *workspace, size_t ws_bytes, void *stream);

/*
 * One recurrent decode step for N = desc->batch sequences (desc->seqlen must
 * be 1): the O(1)-memory inference form ("Gated DeltaNet-2" blog summary,
 * "Core Mechanism"; the fixed-size state of the divagr.com explainer, part
 * 5).  The fp32 state [N,H,dk,dv] is read and rewritten in place.
 *
 *   q, k [N,H,dk], v [N,H,dv] (qkv_dtype); gates [N,H,dk] or [N,H] fp32;
 *   write ignored when tied; state in/out; o [N,H,dv] fp32 or bf16 (o_dtype), must not overlap
 *   the state or any input.
 */
gdn2_status gdn2_recurrent_step(const gdn2_desc *desc,
                                const void *q, const void *k, const void *v,
                                const float *log_decay, const float *erase, const float *write,
                                float *state, float *o, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H */
