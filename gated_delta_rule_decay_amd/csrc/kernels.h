// kernels.h -- internal interface between the C-ABI layer (api.hip) and the
// gfx950 kernels.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

// Everything a chunked-forward launch needs; pointers are device memory.
struct ChunkArgs {
    const void *q, *k, *v;          // [B,T,H,dk] / [B,T,H,dv], bf16 or fp32
    const float *la, *eb, *wr;      // gates; wr == nullptr when tied
    const float *s0;                // [B,H,dk,dv] or nullptr (zeros)
    float *o;                       // [B,T,H,dv], fp32 (bf16 when o_bf16)
    float *s_out;                   // [B,H,dk,dv] or nullptr
    int64_t B, T, H, dk, dv;
    int C;                          // chunk length requested
    int bf16;                       // q/k/v element type
    int la_key, eb_key, wr_key;     // 1: per key channel, 0: per token-head
    float q_scale;
    int value_write;                // 1: erase gate on the read, write gate per value
                                    //    channel ([B,T,H,dv] when wr_key)
    int gate_logits;                // 1: gates are bf16 logits (-softplus / sigmoid in-kernel)
    int qk_norm;                    // 1: q, k L2-normalised per token-head in-kernel
    const int32_t *cu = nullptr;    // packed sequences: [B+1] token offsets (device), B sequences
                                    // along T of batch-1 tensors; nullptr: B fixed-length ones
    int o_bf16 = 0;                 // 1: o holds bf16 (the fp32 result rounded to nearest even)
};

struct StepArgs {
    const void *q, *k, *v;          // [N,H,dk] / [N,H,dv]
    const float *la, *eb, *wr;      // [N,H,dk] or [N,H]; wr == nullptr when tied
    float *state;                   // [N,H,dk,dv], in place
    float *o;                       // [N,H,dv], fp32 (bf16 when o_bf16)
    int64_t N, H, dk, dv;
    int bf16;
    int la_key, eb_key, wr_key;
    float q_scale;
    int value_write;                // as in ChunkArgs
    int gate_logits, qk_norm;       // as in ChunkArgs
    int o_bf16 = 0;                 // as in ChunkArgs
};

// General chunked forward: fp32 arithmetic on the vector ALU, any dk, dv in
// 1..128, internal chunk <= C chosen to fit LDS.  Returns a hipError_t.
hipError_t launch_chunk_general(const ChunkArgs &a, hipStream_t s);

// bf16, dk = dv = 128, C = 64: the MFMA path.
bool chunk_mfma_supported(const ChunkArgs &a);
hipError_t launch_chunk_mfma(const ChunkArgs &a, hipStream_t s);

// bf16, dk = dv = 128, C = 64, two passes through a device workspace: the
// chunk-local products of every chunk in parallel, then the scan over chunks.
// Same coverage as the single-pass MFMA path.
bool chunk_split_supported(const ChunkArgs &a);
size_t chunk_split_workspace(int64_t B, int64_t H, int64_t T);
hipError_t launch_chunk_split(const ChunkArgs &a, void *ws, hipStream_t s);
// The same for packed sequences (a.cu set): the workspace bound uses at most
// ceil(T/64) + B chunks per head.
size_t chunk_split_workspace_varlen(int64_t N, int64_t H, int64_t T);

// The two-pass form with its records in the library's static device scratch
// of STATIC_SCRATCH_BYTES per GPU instead of a workspace (no allocation):
// the chunks are processed in windows whose records fit, the state carried
// from window to window in the scratch.  chunk_split_static_fits tells
// whether one chunk per chain fits at all (B sequences of T tokens).
constexpr size_t STATIC_SCRATCH_BYTES = size_t(128) << 20;
bool chunk_split_static_fits(int64_t B, int64_t H, int64_t T);
hipError_t launch_chunk_split_static(const ChunkArgs &a, hipStream_t s);

// Packed sequences: the plan built on the device from the offsets
// (varlen.hip), for chunks of C tokens.
struct VarPlan {
    const int2 *seq;  // [N]    token range [lo, hi) of each sequence
    const int *pfx;   // [N+1]  chunks before each sequence; pfx[N]: all chunks
    const int2 *tab;  // [chunk] first token of each chunk, end of its sequence
};
int64_t varlen_chunk_bound(int64_t N, int64_t T, int C);  // ceil(T/C) + N
size_t varlen_plan_bytes(int64_t N, int64_t T, int C);
hipError_t launch_varlen_plan(const int32_t *cu, int64_t N, int64_t T, int C, void *buf, VarPlan *plan,
                              hipStream_t s);

// The general forward recording the state that enters every chunk of Cg
// tokens, hist[B*H][ceil(T/Cg)][dk][dv] (packed sequences: the plan's chunks,
// hist[chunk][H]); writes neither o nor the final state.
hipError_t launch_chunk_general_hist(const ChunkArgs &a, int Cg, float *hist, const VarPlan &vp, hipStream_t s);

// Backward of the chunked forward: gradients of <d_o, o> + <d_sT, S_T>.
struct BwdArgs {
    ChunkArgs f;            // the forward's inputs (f.o and f.s_out unused)
    const float *d_o;       // [B,T,H,dv]
    const float *d_sT;      // [B,H,dk,dv] or nullptr (zeros)
    float *dq, *dk, *dv;    // [B,T,H,dk] / [B,T,H,dv]
    float *dla, *deb, *dwr; // shaped like the gates; dwr nullptr when tied
    float *ds0;             // [B,H,dk,dv] or nullptr
};
int chunk_bwd_chunk(int64_t dk, int64_t dv, int C);  // internal chunk length (0: none fits)
// workspace of launch_chunk_bwd for these arguments (the state records, and
// the prepared inputs when the preparation is fused)
size_t chunk_bwd_workspace(const ChunkArgs &f);
hipError_t launch_chunk_bwd(const BwdArgs &a, void *ws, hipStream_t s);
// dk = dv = 128 (16-token chunks): the whole backward on the matrix cores
// (state and state-gradient scans, per-chunk gradients), through per-chunk
// records of bwd_record_bytes(B*H*chunks) bytes.
size_t bwd_record_bytes(int64_t chunks);
// Long sequences on few chains: the two scans in bwd_segments(chains, nch)
// segments per chain (1: one pass), through bwd_segment_bytes of segment
// summaries (B sequences of T tokens only).
int bwd_segments(int64_t chains, int nch);
size_t bwd_segment_bytes(int64_t chains, int nseg);
hipError_t launch_bwd_d128(const BwdArgs &a, const VarPlan &vp, float *rec, float *hist, float *dhist, float *segs,
                           int nch, hipStream_t s);
// X[j+1] <- F[j] X[j] + X[j+1] for j = 1 .. nseg - 2, in order, for each of
// `chains` chains of nseg row-major 128 x 128 slots in xs and fs
hipError_t launch_segment_combine(float *xs, const float *fs, int64_t chains, int nseg, hipStream_t s);

// Recurrent decode step.
hipError_t launch_step(const StepArgs &a, hipStream_t s);

// state_out <- state0 (or zeros when state0 is null); n floats.
hipError_t launch_state_copy(const float *src, float *dst, int64_t n, hipStream_t s);

}  // namespace gdn2
