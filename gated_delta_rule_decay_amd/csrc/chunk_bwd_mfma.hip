// chunk_bwd_mfma.hip -- the backward on the matrix cores (fp32 MFMA), for
// dk = dv = 128 and the backward's 16-token chunks.
//
// The backward (chunk_bwd.hip has the general path and the adjoint formulas)
// needs, for every chunk, the state S entering it and the gradient dSo of the
// state leaving it; both come from scans over the chunks of a chain.  In the
// chunk form of the recurrence ("Gated DeltaNet-2" blog summary, "Core
// Mechanism"; gist.science summary, "Technische Samenvatting" section 3),
// with Kbar, Qbar, Etil, Util the decayed key, query, erase and write operands
// of a chunk, Tm = (I + A)^-1 and Bm, R, P its Grams:
//   forward:  X = Kbar S + Bm V,  M = Tm X,  S <- Diag(e^gC) S + Util^T V - Etil^T M
//   reverse:  dM = -Etil dSo - R^T dO,  Y = Tm^T dM,
//             dS = Diag(e^gC) dSo + Qbar^T dO + Kbar^T Y
// Three launches:
//   bwd_record_kernel   every chunk in parallel: the Grams (pairwise decays
//                       formed directly, never above 1), Tm by forward
//                       substitution, the decayed operands -> a record;
//   bwd_scans_kernel    two independent scans side by side, each per (chain,
//                       64 value columns): chunks in order with S in
//                       accumulator registers, recorded on entry to each
//                       chunk; chunks in reverse with dS in registers,
//                       recorded on entry (= each chunk's dSo), then dS0;
//   bwd_grads128_kernel every chunk in parallel: all input gradients from the
//                       record, S and dSo.
// With few chains and long sequences the middle launch becomes three
// (bwd_seg_scans_kernel<1>, the segment combine, bwd_seg_scans_kernel<0>):
// the scans run in segments, summarised, combined and rescanned.
// All arithmetic is fp32 (v_mfma_f32_16x16x4f32, fp32 accumulate), so the
// gradients keep the fp32 tolerance.
//
// Register layout.  A wave owns 16 value columns; its state slice (128 key
// channels x 16 columns, or half of them in the scans, where two waves split
// the channels) sits in accumulator tiles: lane l = 16 kq + n holds
// S[16 it + 4 kq + i][n] in register i of tile it.  The k-sum of a product
// may run in any order, so each product is arranged so that the lane's own
// accumulator registers are its B operand: in Kbar S the k-step (it, i) takes
// key channel 16 it + 4 kq + i for lane group kq; in the token contractions
// (Tm X, Etil^T M, ...) k-step j takes token 4 kq + j, which is where the
// token-row accumulators of X, M, dM, Y hold their values.  Only the A
// operands (the chunk's record, shared by the workgroup) come from LDS.
#include "common.h"
#include "kernels.h"

namespace gdn2 {
namespace {

constexpr int BD = 128;   // dk = dv
constexpr int BC = 16;    // tokens per chunk
constexpr int BNT = 256;  // threads per workgroup (4 waves x 16 value columns)
constexpr int RS = 132;   // LDS row stride of the scans' 16 x 128 operands
// LDS layout of the gradient kernel.  The strides follow the measured gfx950
// LDS banking (32 banks of 4 bytes; a 4-byte access is served per half-wave):
// GS: 16 x 128 operands, whose rows are read 16 bytes per lane (lane (kq, m)
//     at row m, column 4 kq) -- a stride of 8 banks mod 32 serves those
//     without conflict;
// OS: the raw per-(token, channel) operands, read at token 4 s + kq and
//     channel 16 w + m -- the two tokens of a half-wave fall 16 banks apart;
// TP: the record's 16 x 16 matrices, read at row 4 kq + j, column m -- the
//     two rows of a half-wave fall 16 banks apart.
constexpr int GS = 136;
constexpr int OS = 144;
constexpr int TP = 20;
typedef float f4 __attribute__((ext_vector_type(4)));

// record of one (chain, chunk), fp32, in this order
constexpr int R_KB = 0;                 // Kbar = k e^g         [16][128]
constexpr int R_QB = R_KB + BC * BD;    // Qbar = q_scale q e^g [16][128]
constexpr int R_ET = R_QB + BC * BD;    // Etil = e e^(gC-g)    [16][128]
constexpr int R_UT = R_ET + BC * BD;    // Util = u e^(gC-g)    [16][128]
constexpr int R_TM = R_UT + BC * BD;    // Tm                   [16][16]
constexpr int R_BM = R_TM + BC * BC;    // Bm (strictly lower)  [16][16]
constexpr int R_RR = R_BM + BC * BC;    // R (lower)            [16][16]
constexpr int R_PP = R_RR + BC * BC;    // P (lower)            [16][16]
constexpr int R_GM = R_PP + BC * BC;    // e^gC                 [128]
constexpr int REC_BWD = R_GM + BD;

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Where a task (one chunk of one head) sits: head h, first token tok0 on the
// flattened [B*T] token axis, end tlim of its sequence.  B sequences of T
// tokens: task = (b H + h) nch + n; packed sequences (f.cu): chunk-major,
// task = chunk H + h, placed by the plan's chunk table.
struct BTask {
    int64_t h, tok0, tlim;
};

__device__ __forceinline__ BTask btask(const ChunkArgs &f, const VarPlan &vp, int64_t task, int nch) {
    BTask t;
    if (f.cu) {
        const int64_t gc = task / f.H;
        const int2 e = vp.tab[gc];
        t.h = task - gc * f.H;
        t.tok0 = e.x;
        t.tlim = e.y;
    } else {
        const int64_t bh = task / nch, n = task - bh * nch, b = bh / f.H;
        t.h = bh - b * f.H;
        t.tok0 = b * f.T + n * BC;
        t.tlim = b * f.T + f.T;
    }
    return t;
}

// The tasks a chain (one sequence, one head; chain = sequence H + head)
// walks: task0 + n tstr for n < nc, tokens from tbase, sequence end tlim.
struct BChain {
    int64_t h, task0, tstr, tbase, tlim;
    int nc;
};

__device__ __forceinline__ BChain bchain(const ChunkArgs &f, const VarPlan &vp, int64_t chain, int nch) {
    BChain c;
    const int64_t i = chain / f.H;
    c.h = chain - i * f.H;
    if (f.cu) {
        const int p0 = vp.pfx[i];
        const int2 e = vp.seq[i];
        c.nc = vp.pfx[i + 1] - p0;
        c.task0 = static_cast<int64_t>(p0) * f.H + c.h;
        c.tstr = f.H;
        c.tbase = e.x;
        c.tlim = e.y;
    } else {
        c.nc = nch;
        c.task0 = chain * nch;
        c.tstr = 1;
        c.tbase = i * f.T;
        c.tlim = c.tbase + f.T;
    }
    return c;
}

// sum_c A[m][c] B[c][n] over the 128 key channels, A row m from LDS (row
// stride GS) in the channel order of the state registers B; four independent
// accumulation chains (channel 16 it + 4 kq + i goes to chain i), so that the
// matrix unit never waits on its own previous result for long.
__device__ __forceinline__ f4 chan_product(const float *A, const f4 (&B)[8], int m, int kq, f4 init) {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    f4 acc[4] = {init, z, z, z};
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const f4 a4 = *reinterpret_cast<const f4 *>(&A[m * GS + 16 * it + 4 * kq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = mfma4(a4[i], B[it][i], acc[i]);
    }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Tasks of a launch: every chunk of every head (read from the plan for
// packed sequences).
__device__ __forceinline__ int64_t btask_count(const ChunkArgs &f, const VarPlan &vp, int nch) {
    return f.cu ? f.H * vp.pfx[f.B] : f.B * f.H * nch;
}

// Buffer resource over rows tok0 .. tlim-1 (at most one chunk) of head h of
// a [tokens, H, width] tensor with elements of es bytes: the hardware returns
// zero for rows past tlim, so loads through it need no select (and no wait).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void *p, int64_t H, int64_t h, int64_t tok0,
                                                           int64_t tlim, int width, int es) {
    const int64_t n = tlim - tok0 < BC ? (tlim - tok0 > 0 ? tlim - tok0 : 0) : BC;
    const char *base = static_cast<const char *>(p) + (tok0 * H + h) * width * es;
    const int bytes = n > 0 ? static_cast<int>(((n - 1) * H * width + width) * es) : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, bytes, 0x00020000);
}

// ---------------------------------------------------------------------------
// the record pass

constexpr int KS = BD + 1;  // odd row stride: loops that read one channel of different rows
constexpr float LOG2E = 1.4426950408889634f;
constexpr int QP = BC + 1;  // quads per channel-quad column in LDS (one pad: the quad writes hit distinct banks)

// Four consecutive channels c0..c0+3 of a q/k/v row (bf16 or fp32), one load.
__device__ __forceinline__ f4 load_qkv4(const void *p, int64_t i, int bf16) {
    if (bf16) {
        const uint2 u = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
        return f4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                  __uint_as_float(u.y & 0xffff0000u)};
    }
    return *reinterpret_cast<const f4 *>(static_cast<const float *>(p) + i);
}

// The gate of channels c0..c0+3 of token-head `row` (one value per token-head
// broadcast when the gate is not per channel).
__device__ __forceinline__ f4 load_gate4(const float *g, int per_key, int64_t row, int c0) {
    if (per_key) return *reinterpret_cast<const f4 *>(g + row * BD + c0);
    const float x = g[row];
    return f4{x, x, x, x};
}

__device__ __forceinline__ f4 exp2_4(f4 x) {
    return f4{__builtin_amdgcn_exp2f(x[0]), __builtin_amdgcn_exp2f(x[1]), __builtin_amdgcn_exp2f(x[2]),
              __builtin_amdgcn_exp2f(x[3])};
}

// LDS of the record pass: the chunk's operands channel-quad-major,
// [channel / 4][row][4 channels] (row BC is padding), so that a Gram thread
// reads four channels of a row in one 16-byte access; the running log2-decay
// in G.
struct RecLds {
    f4 K[32 * QP], Q[32 * QP], G[32 * QP], E[32 * QP], U[32 * QP];
    float A[BC * BC];
};

// The raw input words of one record task for a thread's two channel quads
// (rows tid / 32 and tid / 32 + 8, channels 4 (tid % 32) .. + 3): q and k as
// bf16 pairs (words 0, 1) or fp32 (words 0..3), the gates as fp32 (element 0
// only for a gate per head).  Loaded through buffer ranges (rows past the
// sequence end read as zero), converted only when the task is staged, so a
// task's loads stay in flight while the previous task computes.
struct RecRaw {
    uint32_t k[2][4], q[2][4];
    f4 la[2], eb[2], wr[2];
};

__device__ __forceinline__ void rec_issue(RecRaw &R, const ChunkArgs &f, const BTask &tp, int tid) {
    const int64_t H = f.H, h = tp.h;
    const int es = f.bf16 ? 2 : 4;
    const auto rk = rows_rsrc(f.k, H, h, tp.tok0, tp.tlim, BD, es);
    const auto rq = rows_rsrc(f.q, H, h, tp.tok0, tp.tlim, BD, es);
    const int lw = f.la_key ? BD : 1, ew = f.eb_key ? BD : 1, ww = f.wr && f.wr_key ? BD : 1;
    const auto rla = rows_rsrc(f.la, H, h, tp.tok0, tp.tlim, lw, 4);
    const auto reb = rows_rsrc(f.eb, H, h, tp.tok0, tp.tlim, ew, 4);
    const auto rwr = rows_rsrc(f.wr ? f.wr : f.eb, H, h, tp.tok0, tp.tlim, f.wr ? ww : ew, 4);
    auto gate = [&](__amdgpu_buffer_rsrc_t rs, int width, int r, int c4) {
        if (width == BD)
            return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>((r * H * BD + 4 * c4) * 4), 0, 0));
        return f4{__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(r * H * 4), 0, 0)), 0.f, 0.f, 0.f};
    };
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int qd = tid + BNT * p, r = qd / 32, c4 = qd % 32;
        const int off = static_cast<int>((r * H * BD + 4 * c4) * es);
        if (f.bf16) {
            const uint2 a = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, off, 0, 0));
            const uint2 b = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, off, 0, 0));
            R.k[p][0] = a.x; R.k[p][1] = a.y; R.k[p][2] = R.k[p][3] = 0;
            R.q[p][0] = b.x; R.q[p][1] = b.y; R.q[p][2] = R.q[p][3] = 0;
        } else {
            const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
            const uint4 b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
            R.k[p][0] = a.x; R.k[p][1] = a.y; R.k[p][2] = a.z; R.k[p][3] = a.w;
            R.q[p][0] = b.x; R.q[p][1] = b.y; R.q[p][2] = b.z; R.q[p][3] = b.w;
        }
        R.la[p] = gate(rla, lw, r, c4);
        R.eb[p] = gate(reb, ew, r, c4);
        R.wr[p] = f.wr ? gate(rwr, ww, r, c4) : R.eb[p];
    }
}

__global__ void __launch_bounds__(BNT) bwd_record_kernel(BwdArgs a, VarPlan vp, float *rec, int nch) {
    __shared__ RecLds L;
    const ChunkArgs &f = a.f;
    const int64_t ntask = btask_count(f, vp, nch);
    const int tid = threadIdx.x;
    RecRaw R;
    if (static_cast<int64_t>(blockIdx.x) < ntask) rec_issue(R, f, btask(f, vp, blockIdx.x, nch), tid);
    for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
        float *out = rec + task * REC_BWD;
        __syncthreads();  // the previous task is done with LDS
        // ---- operands: thread = channel quad c4 of rows r (two quads each)
        auto qkv = [&](const uint32_t (&w)[4]) {
            return f.bf16 ? f4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                               __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)}
                          : f4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                               __uint_as_float(w[3])};
        };
        auto bcast = [](f4 x, int key) { return key ? x : f4{x[0], x[0], x[0], x[0]}; };
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int qd = tid + BNT * p, r = qd / 32, c4 = qd % 32;
            f4 kv = qkv(R.k[p]);
            const f4 qv = f.q_scale * qkv(R.q[p]);
            const f4 la = LOG2E * bcast(R.la[p], f.la_key);
            const f4 bb = bcast(R.eb[p], f.eb_key);
            f4 e, u;
            if (f.value_write) {  // read along b k, erase and write along k
                e = u = kv;
                kv *= bb;
            } else {
                const f4 ww = f.wr ? bcast(R.wr[p], f.wr_key) : bb;
                e = bb * kv;
                u = ww * kv;
            }
            const int li = c4 * QP + r;
            L.K[li] = kv; L.Q[li] = qv; L.G[li] = la; L.E[li] = e; L.U[li] = u;
        }
        // the next task's loads go out now, to arrive while this one computes
        if (task + gridDim.x < ntask) rec_issue(R, f, btask(f, vp, task + gridDim.x, nch), tid);
        __syncthreads();
        if (tid < BD) {  // running log2-decay per channel (padded rows add 0)
            float *g = reinterpret_cast<float *>(L.G) + (tid / 4) * QP * 4 + (tid % 4);
            float run = 0.f;
#pragma unroll
            for (int r = 0; r < BC; ++r) {
                run += g[4 * r];
                g[4 * r] = run;
            }
            out[R_GM + tid] = __builtin_amdgcn_exp2f(run);
        }
        __syncthreads();
        {  // the four Grams, one (r, s) pair per thread, pairwise decays
           // 2^(g_r - g_s) <= 1 formed directly
            const int r = tid / BC, s = tid % BC;
            float sa = 0.f, sb = 0.f, sr = 0.f, sp = 0.f;
            if (s <= r) {
#pragma unroll 4
                for (int c4 = 0; c4 < 32; ++c4) {
                    const int lr = c4 * QP + r, ls = c4 * QP + s;
                    const f4 d = exp2_4(L.G[lr] - L.G[ls]);
                    const f4 kd = L.K[lr] * d, qd = L.Q[lr] * d;
                    const f4 e = L.E[ls], u = L.U[ls];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sa += kd[i] * e[i];
                        sb += kd[i] * u[i];
                        sr += qd[i] * e[i];
                        sp += qd[i] * u[i];
                    }
                }
            }
            L.A[tid] = s < r ? sa : 0.f;
            out[R_BM + tid] = s < r ? sb : 0.f;
            out[R_RR + tid] = sr;
            out[R_PP + tid] = sp;
        }
        __syncthreads();
        if (tid < BC) {
            // Tm = (I + A)^-1 by forward substitution, column j = tid in
            // registers: Tm[r][j] = -sum_{j <= s < r} A[r][s] Tm[s][j]
            const int j = tid;
            float t[BC];
#pragma unroll
            for (int r = 0; r < BC; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < r; ++s2) acc += L.A[r * BC + s2] * t[s2];
                t[r] = r < j ? 0.f : (r == j ? 1.f : -acc);
                out[R_TM + r * BC + j] = t[r];
            }
        }
        // the decays folded into the operands (two quads per thread)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int qd = tid + BNT * p, r = qd / 32, c4 = qd % 32, li = c4 * QP + r;
            const f4 g = L.G[li], gc = L.G[c4 * QP + BC - 1];
            const f4 eg = exp2_4(g), ec = exp2_4(gc - g);
            const int o = r * BD + 4 * c4;
            *reinterpret_cast<f4 *>(out + R_KB + o) = L.K[li] * eg;
            *reinterpret_cast<f4 *>(out + R_QB + o) = L.Q[li] * eg;
            *reinterpret_cast<f4 *>(out + R_ET + o) = L.E[li] * ec;
            *reinterpret_cast<f4 *>(out + R_UT + o) = L.U[li] * ec;
        }
    }
}

// ---------------------------------------------------------------------------
// the two scans

// LDS copy of the record parts a scan reads (row stride RS for the 16 x 128
// operands)
struct ScanLds {
    float m0[BC * RS], m1[BC * RS], m2[BC * RS];
    float t0[BC * BC], t1[BC * BC];
    float gm[BD];
};

// The raw words of lane (kq, n)'s rows 4 kq + j of a chunk at column col of a
// [tokens, H, 128] tensor (bf16 bits in the low half, or fp32 bits), zero
// past tlim; with the value-write form also the write gate of those rows
// (fp32 bits).  Nothing is converted here, so prefetched loads stay in flight
// until raw_rows4 uses them.
struct RawRows {
    uint32_t x[4], w[4];
};

__device__ __forceinline__ void load_rows_raw(uint32_t (&x)[4], const void *p, int bf16, int64_t H, int64_t h,
                                              int64_t tok0, int64_t tlim, int kq, int col) {
    const int es = bf16 ? 2 : 4;
    const auto rs = rows_rsrc(p, H, h, tok0, tlim, BD, es);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int off = static_cast<int>(((4 * kq + j) * H * BD + col) * es);
        x[j] = bf16 ? static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0))
                    : __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
    }
}

__device__ __forceinline__ void load_vals_raw(RawRows &r, int64_t tok0, int64_t tlim, int64_t h, int kq, int col,
                                              const ChunkArgs &f) {
    load_rows_raw(r.x, f.v, f.bf16, f.H, h, tok0, tlim, kq, col);
    if (f.value_write) {
        const int gw = f.wr_key ? BD : 1;
        const auto rs = rows_rsrc(f.wr, f.H, h, tok0, tlim, gw, 4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            r.w[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, static_cast<int>(((4 * kq + j) * f.H * gw + (f.wr_key ? col : 0)) * 4), 0, 0);
    }
}

// The four values of raw rows, times the write gate in the value-write form.
__device__ __forceinline__ void raw_rows4(float (&v)[4], const RawRows &r, int bf16, int vw) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[j] = bf16 ? __uint_as_float(r.x[j] << 16) : __uint_as_float(r.x[j]);
        if (vw) v[j] *= __uint_as_float(r.w[j]);
    }
}


// The state entering every chunk, hist[chain][chunk][128][128].
// The scans run 8 waves per workgroup: waves w and w + 4 share value tile
// w % 4 (16 columns) and split the key channels, tiles 0..3 and 4..7, so two
// waves per SIMD hide each other's latency.  A token-row product over the
// channels (Kbar S, Etil dS) is summed from the two halves through LDS; the
// small token products after it (Tm X, Tm^T dM) run in both waves of a pair.
constexpr int SNT = 512;
constexpr int VMCNT0 = (7 << 4) | (15 << 8);  // s_waitcnt: vector memory count 0, the others untouched

// The record parts a scan reads, staged through registers (512 threads: one
// float4 of each 16 x 128 part, one of the two 16 x 16 parts, one of e^gC).
// Every thread loads (duplicates stay in bounds), so no loaded value passes
// through a select and the loads can stay in flight.
struct Staged8 {
    f4 x[3];
    f4 tt;
    float g;
};

__device__ __forceinline__ void stage_load8(Staged8 &st, const float *r, int o0, int o1, int o2, int oT0, int oT1,
                                            int tid) {
#pragma unroll
    for (int p = 0; p < 3; ++p) st.x[p] = *reinterpret_cast<const f4 *>(r + (p == 0 ? o0 : p == 1 ? o1 : o2) + 4 * tid);
    st.tt = *reinterpret_cast<const f4 *>(r + ((tid & 64) ? oT1 : oT0) + 4 * (tid & 63));
    st.g = r[R_GM + (tid & (BD - 1))];
}

__device__ __forceinline__ void stage_store8(const Staged8 &st, ScanLds &L, int tid) {
    const int row = tid / 32, col = 4 * (tid % 32);
#pragma unroll
    for (int p = 0; p < 3; ++p)
        *reinterpret_cast<f4 *>(&(p == 0 ? L.m0 : p == 1 ? L.m1 : L.m2)[row * RS + col]) = st.x[p];
    if (tid < 128) *reinterpret_cast<f4 *>(&((tid & 64) ? L.t1 : L.t0)[4 * (tid & 63)]) = st.tt;
    else if (tid < 128 + BD) L.gm[tid - 128] = st.g;
}

// sum_c A[m][c] B[c][n] over this wave's 64 key channels (tiles 4 kh + t),
// A row m from LDS, B the state registers; four accumulation chains.
__device__ __forceinline__ f4 chan_half(const float *A, const f4 (&B)[4], int m, int kq, int kh) {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    f4 acc[4] = {z, z, z, z};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const f4 a4 = *reinterpret_cast<const f4 *>(&A[m * RS + 16 * (4 * kh + t) + 4 * kq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = mfma4(a4[i], B[t][i], acc[i]);
    }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// The state records (hist, dhist) are stored tile-major, in the accumulator
// layout that writes and reads them: element (16 it + 4 kq + i, 16 cg + m) of
// a 128 x 128 state sits at ((it * 8 + cg) * 64 + 16 kq + m) * 4 + i, so the
// four rows a lane holds are one 16-byte word and a wave's key tile of its 16
// value columns is 1 KiB of contiguous memory.
__device__ __forceinline__ int64_t tile_off(int it, int cg, int lane) {
    return static_cast<int64_t>((it * 8 + cg) * 64 + lane) * 4;
}

// Store a wave's half state slice (tiles 4 kh + t of its 16 columns, column
// group cg) as a state record.
__device__ __forceinline__ void put_tiles(float *dst, const f4 (&s)[4], int kh, int cg, int lane) {
#pragma unroll
    for (int t = 0; t < 4; ++t) *reinterpret_cast<f4 *>(dst + tile_off(4 * kh + t, cg, lane)) = s[t];
}

// Store a wave's half state slice (tiles 4 kh + t, 64 x 16) transposed into
// a [128][128] matrix (element (row, col) at col * 128 + row).
__device__ __forceinline__ void put_half_t(float *dst, const f4 (&s)[4], int kq, int kh, int col) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
        *reinterpret_cast<f4 *>(&dst[col * BD + 16 * (4 * kh + t) + 4 * kq]) = s[t];
}

// Store a wave's half state slice (tiles 4 kh + t, 64 x 16) into a [128][128] matrix.
__device__ __forceinline__ void put_half(float *dst, const f4 (&s)[4], int kq, int kh, int col) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * (4 * kh + t) + 4 * kq + i) * BD + col] = s[t][i];
}

// Both halves of a token-row product: write mine, wait, add my partner's
// (low half first in both waves, so the pair holds identical sums).
__device__ __forceinline__ f4 pair_sum(f4 *xp, f4 mine, int wv, int lane, int kh) {
    xp[wv * 64 + lane] = mine;
    __syncthreads();
    const f4 other = xp[(wv ^ 4) * 64 + lane];
    return kh ? other + mine : mine + other;
}

// The chain and value half of workgroup G among the `units` workgroups of one
// scan.  Workgroups are spread over the 8 XCDs round robin; when `units` is a
// multiple of 16, the two halves of a chain go to workgroups 8 apart, i.e. to
// one XCD, so the record parts both read come into one L2.
struct ScanUnit {
    int64_t chain;
    int half;
};

__device__ __forceinline__ ScanUnit scan_unit(int64_t G, int64_t units) {
    if (units % 16 == 0) return {(G / 16) * 8 + (G % 8), static_cast<int>((G / 8) & 1)};
    return {G >> 1, static_cast<int>(G & 1)};
}

struct ScanLds8 {
    ScanLds r;
    f4 xp[8 * 64];  // the waves' half products
};

// One scan of a chain's value half: over chunks n0 .. n1 - 1 (n1 < 0: all of
// the chain's chunks), in order for the states, in reverse for their
// gradients.  The matrix carried starts as `init` (row-major [128][128]), or
// as zero, or with `ident` as the identity; `inputs` switches the terms in V
// (states) or d_o (gradients) on, off for a segment's transition.  `recs`
// receives the per-chunk records (tile-major; null: none), `out` the matrix
// leaving the scan (row-major; null: none), `out_t` its transpose (null: none).
struct ScanJob {
    int n0, n1;
    const float *init;
    int ident, inputs;
    float *recs, *out, *out_t;
};

// The matrix a job starts from, in this lane's registers (rows 16 (4 kh + t)
// + 4 kq + i of column col).
__device__ __forceinline__ void scan_init(f4 (&S)[4], const ScanJob &job, int kq, int kh, int col) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * (4 * kh + t) + 4 * kq + i;
            S[t][i] = job.init ? job.init[row * BD + col] : (job.ident && row == col ? 1.f : 0.f);
        }
}

// The states: entering each chunk (recorded), carried forward.
__device__ __forceinline__ void state_scan(const BwdArgs &a, const VarPlan &vp, const float *rec, int nch,
                                           ScanLds8 &LL, const ScanUnit su, const ScanJob &job) {
    ScanLds &L = LL.r;
    const ChunkArgs &f = a.f;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int m = lane & 15, kq = lane >> 4, kh = wv >> 2;
    const int64_t bh = su.chain;
    const BChain ch = bchain(f, vp, bh, nch);
    const int64_t h = ch.h;
    const int col = 64 * su.half + 16 * (wv & 3) + m;  // this lane's value column (as n)
    const int n0 = job.n0, n1 = job.n1 < 0 ? ch.nc : job.n1;
    auto rc = [&](int n) { return rec + (ch.task0 + n * ch.tstr) * static_cast<int64_t>(REC_BWD); };
    auto hs = [&](int n) { return job.recs + (ch.task0 + n * ch.tstr) * static_cast<int64_t>(BD * BD); };

    f4 S[4];  // key channel tiles 4 kh + t
    scan_init(S, job, kq, kh, col);
    // the initial state is complete before the loop: no wait inside the loop
    // has to allow for its loads
    __builtin_amdgcn_s_waitcnt(VMCNT0);

    // m0 = Kbar, m1 = Etil, m2 = Util; t0 = Tm, t1 = Bm
    Staged8 st;
    RawRows vn;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (n0 < n1) {
        stage_load8(st, rc(n0), R_KB, R_ET, R_UT, R_TM, R_BM, tid);
        if (job.inputs) load_vals_raw(vn, ch.tbase + static_cast<int64_t>(n0) * BC, ch.tlim, h, kq, col, f);
        stage_store8(st, L, tid);
        if (job.inputs) raw_rows4(v, vn, f.bf16, f.value_write);
    }
    for (int n = n0; n < n1; ++n) {
        // the next chunk's loads go out before this chunk's state stores, so
        // that waiting for them (after this chunk's products) never waits
        // for the stores
        if (n + 1 < n1) {
            stage_load8(st, rc(n + 1), R_KB, R_ET, R_UT, R_TM, R_BM, tid);
            if (job.inputs) load_vals_raw(vn, ch.tbase + (n + 1) * BC, ch.tlim, h, kq, col, f);
        }
        if (job.recs) put_tiles(hs(n), S, kh, col >> 4, lane);
        __syncthreads();  // chunk n's LDS copy complete
        // X = Kbar S + Bm V (token rows)
        f4 X = pair_sum(LL.xp, chan_half(L.m0, S, m, kq, kh), wv, lane, kh);
        {
            const f4 b4 = *reinterpret_cast<const f4 *>(&L.t1[m * BC + 4 * kq]);
#pragma unroll
            for (int j = 0; j < 4; ++j) X = mfma4(b4[j], v[j], X);
        }
        // M = Tm X
        f4 M = {0.f, 0.f, 0.f, 0.f};
        {
            const f4 t4 = *reinterpret_cast<const f4 *>(&L.t0[m * BC + 4 * kq]);
#pragma unroll
            for (int j = 0; j < 4; ++j) M = mfma4(t4[j], X[j], M);
        }
        // S <- Diag(e^gC) S + Util^T V - Etil^T M
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int it = 4 * kh + t;
            const f4 g4 = *reinterpret_cast<const f4 *>(&L.gm[16 * it + 4 * kq]);
            f4 s = g4 * S[t];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s = mfma4(L.m2[(4 * kq + j) * RS + 16 * it + m], v[j], s);
                s = mfma4(-L.m1[(4 * kq + j) * RS + 16 * it + m], M[j], s);
            }
            S[t] = s;
        }
        __syncthreads();  // every wave done with chunk n's LDS copy
        if (n + 1 < n1) {
            stage_store8(st, L, tid);
            if (job.inputs) raw_rows4(v, vn, f.bf16, f.value_write);
        }
    }
    if (job.out) put_half(job.out, S, kq, kh, col);
    if (job.out_t) put_half_t(job.out_t, S, kq, kh, col);
}

// The state gradients: each chunk's exit gradient dSo recorded on entry to
// its step, carried backwards.
__device__ __forceinline__ void dgrad_scan(const BwdArgs &a, const VarPlan &vp, const float *rec, int nch,
                                           ScanLds8 &LL, const ScanUnit su, const ScanJob &job) {
    ScanLds &L = LL.r;
    const ChunkArgs &f = a.f;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int m = lane & 15, kq = lane >> 4, kh = wv >> 2;
    const int64_t bh = su.chain;
    const BChain ch = bchain(f, vp, bh, nch);
    const int64_t h = ch.h;
    const int col = 64 * su.half + 16 * (wv & 3) + m;
    const int n0 = job.n0, nl = (job.n1 < 0 ? ch.nc : job.n1) - 1;
    auto rc = [&](int n) { return rec + (ch.task0 + n * ch.tstr) * static_cast<int64_t>(REC_BWD); };
    auto hs = [&](int n) { return job.recs + (ch.task0 + n * ch.tstr) * static_cast<int64_t>(BD * BD); };

    f4 dS[4];
    scan_init(dS, job, kq, kh, col);
    __builtin_amdgcn_s_waitcnt(VMCNT0);

    // m0 = Etil, m1 = Qbar, m2 = Kbar; t0 = Tm, t1 = R
    Staged8 st;
    RawRows on;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    if (nl >= n0) {
        stage_load8(st, rc(nl), R_ET, R_QB, R_KB, R_TM, R_RR, tid);
        if (job.inputs)
            load_rows_raw(on.x, a.d_o, 0, f.H, h, ch.tbase + static_cast<int64_t>(nl) * BC, ch.tlim, kq, col);
        stage_store8(st, L, tid);
        if (job.inputs) raw_rows4(o, on, 0, 0);
    }
    for (int n = nl; n >= n0; --n) {
        // loads of the chunk before go out ahead of this chunk's stores
        if (n > n0) {
            stage_load8(st, rc(n - 1), R_ET, R_QB, R_KB, R_TM, R_RR, tid);
            if (job.inputs)
                load_rows_raw(on.x, a.d_o, 0, f.H, h, ch.tbase + static_cast<int64_t>(n - 1) * BC, ch.tlim, kq, col);
        }
        if (job.recs) put_tiles(hs(n), dS, kh, col >> 4, lane);
        __syncthreads();  // chunk n's LDS copy complete
        // dM = -(Etil dSo + R^T dO)  (token rows)
        f4 dM = pair_sum(LL.xp, chan_half(L.m0, dS, m, kq, kh), wv, lane, kh);
#pragma unroll
        for (int j = 0; j < 4; ++j) dM = mfma4(L.t1[(4 * kq + j) * BC + m], o[j], dM);
        dM = -dM;
        // Y = Tm^T dM
        f4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) Y = mfma4(L.t0[(4 * kq + j) * BC + m], dM[j], Y);
        // dS <- Diag(e^gC) dSo + Qbar^T dO + Kbar^T Y
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int it = 4 * kh + t;
            const f4 g4 = *reinterpret_cast<const f4 *>(&L.gm[16 * it + 4 * kq]);
            f4 s = g4 * dS[t];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s = mfma4(L.m1[(4 * kq + j) * RS + 16 * it + m], o[j], s);
                s = mfma4(L.m2[(4 * kq + j) * RS + 16 * it + m], Y[j], s);
            }
            dS[t] = s;
        }
        __syncthreads();  // every wave done with chunk n's LDS copy
        if (n > n0) {
            stage_store8(st, L, tid);
            if (job.inputs) raw_rows4(o, on, 0, 0);
        }
    }
    if (job.out) put_half(job.out, dS, kq, kh, col);
}

// Both scans in one launch: neither reads what the other writes (the reverse
// scan needs the record and d_o only), so the first half of the grid carries
// the states forward while the second half carries their gradients back.  At
// 36 KiB of LDS and 4 waves per SIMD two 8-wave workgroups share a CU, one of
// each kind when the grid is twice the CU count, and each hides the other's
// per-chunk load and barrier latency.  Every workgroup of the second half
// keeps its index mod 8 (the XCD) from the first when the half-grid is a
// multiple of 8.
__global__ void __launch_bounds__(SNT) bwd_scans_kernel(BwdArgs a, VarPlan vp, const float *rec, float *hist,
                                                        float *dhist, int nch) {
    __shared__ __attribute__((aligned(16))) ScanLds8 LL;
    const int64_t units = gridDim.x / 2, G = blockIdx.x;
    if (G < units) {
        const ScanUnit su = scan_unit(G, units);
        const ScanJob job{0, -1, a.f.s0 ? a.f.s0 + su.chain * BD * BD : nullptr, 0, 1, hist, nullptr, nullptr};
        state_scan(a, vp, rec, nch, LL, su, job);
    } else {
        const ScanUnit su = scan_unit(G - units, units);
        const ScanJob job{0, -1, a.d_sT ? a.d_sT + su.chain * BD * BD : nullptr, 0, 1, dhist,
                          a.ds0 ? a.ds0 + su.chain * BD * BD : nullptr, nullptr};
        dgrad_scan(a, vp, rec, nch, LL, su, job);
    }
}

// Long sequences on few chains: both scans in segments of `len` chunks (the
// last may be shorter).  Each step of either scan is affine in the matrix it
// carries (S <- F_n S + G_n forward, dS <- P_n dSo + H_n backward, F_n and P_n
// acting on the key rows), and affine maps compose ("Gated DeltaNet" page,
// "What makes the architecture more than a recurrence"):
//   summaries  every segment is scanned from zero with its inputs (the states'
//              first segment from S0, the gradients' last from d_sT, which
//              makes those results exact already), and the identity through
//              each inner segment without inputs gives its transition; the
//              gradients' step is the adjoint of the states' (P_n = F_n^T, as
//              Diag(e^gC) is symmetric), so a segment's gradient transition
//              is the transpose of its state transition and is not scanned;
//   combine    the exact entry of every segment follows in order;
//   rescan     every segment from its exact entry, recording its chunks.
// Slots: xs, fs hold [2 chains][nseg] row-major 128 x 128 matrices, the
// states' (chains 0 .. C-1) with segment j's end state in slot j + 1 and its
// transition in slot j, the gradients' (chains C .. 2C-1) in reverse segment
// order: segment j's start gradient in slot nseg - j, its transition in slot
// nseg - 1 - j.  Then "X[s+1] <- F[s] X[s] + X[s+1], s = 1 .. nseg - 2"
// combines both, and slot 1 of each is exact from the summaries.
struct BwdSegs {
    int nseg, len;
    float *xs, *fs;
    int64_t us;  // workgroups of the states (the grid's first part; the rest: the gradients)
};

// MODE 1: the summaries, per (chain, value half) 2 nseg - 3 units of the
// states (nseg - 1 from zero, nseg - 2 transitions) and nseg - 1 of the
// gradients; MODE 0: the rescan, nseg units of each.
template <int MODE>
__global__ void __launch_bounds__(SNT) bwd_seg_scans_kernel(BwdArgs a, VarPlan vp, const float *rec, float *hist,
                                                            float *dhist, int nch, BwdSegs sg) {
    __shared__ __attribute__((aligned(16))) ScanLds8 LL;
    const int64_t G = blockIdx.x;
    const bool grad = G >= sg.us;
    const ScanUnit u = grad ? scan_unit(G - sg.us, gridDim.x - sg.us) : scan_unit(G, sg.us);
    const int nseg = sg.nseg, per = MODE ? (grad ? nseg - 1 : 2 * nseg - 3) : nseg;
    const int64_t C = a.f.B * a.f.H, chain = u.chain / per;
    const int k = static_cast<int>(u.chain - chain * per);
    const ScanUnit su{chain, u.half};
    constexpr int64_t DD = BD * BD;
    float *xs = sg.xs + (grad ? C + chain : chain) * nseg * DD;
    float *fs = sg.fs + (grad ? C + chain : chain) * nseg * DD;
    ScanJob job{0, 0, nullptr, 0, 1, nullptr, nullptr, nullptr};
    int j;
    if (MODE) {
        const bool from_zero = k < nseg - 1;  // else a transition
        if (!grad) {
            j = from_zero ? k : 1 + (k - (nseg - 1));
            if (from_zero) {
                job.init = j == 0 && a.f.s0 ? a.f.s0 + chain * DD : nullptr;
                job.out = xs + (j + 1) * DD;
            } else {  // the transition, and transposed the gradients' (their slot nseg - 1 - j)
                job.ident = 1;
                job.inputs = 0;
                job.out = fs + j * DD;
                job.out_t = sg.fs + ((C + chain) * nseg + nseg - 1 - j) * DD;
            }
        } else {
            j = nseg - 1 - k;
            job.init = j == nseg - 1 && a.d_sT ? a.d_sT + chain * DD : nullptr;
            job.out = xs + (nseg - j) * DD;
        }
    } else {
        j = k;
        if (!grad) {
            job.init = j > 0 ? xs + j * DD : (a.f.s0 ? a.f.s0 + chain * DD : nullptr);
            job.recs = hist;
        } else {
            job.init = j < nseg - 1 ? xs + (nseg - 1 - j) * DD : (a.d_sT ? a.d_sT + chain * DD : nullptr);
            job.recs = dhist;
            job.out = j == 0 && a.ds0 ? a.ds0 + chain * DD : nullptr;
        }
    }
    job.n0 = j * sg.len;
    job.n1 = job.n0 + sg.len < nch ? job.n0 + sg.len : nch;
    if (!grad)
        state_scan(a, vp, rec, nch, LL, su, job);
    else
        dgrad_scan(a, vp, rec, nch, LL, su, job);
}

// ---------------------------------------------------------------------------
// the per-chunk gradients
//
// One workgroup of 8 waves per chunk.  Wave w first owns value columns
// 16w..16w+15 (the products whose columns are value columns: X, M, dM, Y,
// dV, Bm V), then key channels 16w..16w+15 (the products whose columns are key
// channels, contracting over the value columns: dW = dM S^T, dQbar = dO S^T,
// dEtil = -M dSo^T, dUtil = V dSo^T, then dKbar = Tm^T dW), and finally the
// gradients of its channels' inputs: the Grams pass dA, dBm, dR, dP to their
// operands with every pairwise decay formed directly.

constexpr int GNT = 512;

// Four consecutive elements (16-byte or 8-byte aligned) of q/k/v, bf16 or fp32.
__device__ __forceinline__ f4 load4_qkv(const void *p, int64_t i, int bf16) {
    if (bf16) {
        const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + i);
        return f4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                  __uint_as_float(w.y & 0xffff0000u)};
    }
    return *reinterpret_cast<const f4 *>(static_cast<const float *>(p) + i);
}

// Gate of token-head `row` at channels c4 .. c4 + 3 (one value per head broadcast).
__device__ __forceinline__ f4 load4_gate(const float *g, int per_key, int64_t row, int c4) {
    if (per_key) return *reinterpret_cast<const f4 *>(g + row * BD + c4);
    const float x = g[row];
    return f4{x, x, x, x};
}

// TRP: the row pitch of the buffer that turns S and dSo from value columns
// into key rows, 64 of the 128 columns at a time: written one element per
// lane (lane (kq, m) at row 4 kq + i, column m -- the two row groups of a
// half-wave fall 16 banks apart), read 16 bytes per lane along rows.
constexpr int TRP = 68;

struct GradLds {
    float kb[BC * GS];                                   // record: Kbar
    float tm[BC * TP], bm[BC * TP], rr[BC * TP], pp[BC * TP];
    float gm[BD];                                        // e^gC, later d gC's exit term
    float k[BC * OS], q[BC * OS], e[BC * OS], u[BC * OS], g[BC * OS];  // raw operands; running log-decay
    float gc[BD];
    float v[BC * GS], o[BC * GS];                        // V, dO
    float mm[BC * GS], dm[BC * GS], y[BC * GS], bv[BC * GS];  // M, dM, Y, Bm V; later the per-(x, c) results
    float dw[BC * GS];
    float wpart[8 * BC];  // value-write form, one write gate per head: per-wave partial sums of dw
    // Etil and Util are last read by the value products, the 16 x 16
    // gradients first written after the channel products: between the two the
    // same bytes hold the transpose buffer (16-byte rows throughout)
    union alignas(16) {
        struct {
            float et[BC * GS], ut[BC * GS];  // record: Etil, Util
            float dt[BC * BC], x1[BC * BC], da[BC * BC], dbm[BC * BC], dr[BC * BC], dp[BC * BC];
            float daT[BC * BC], dbmT[BC * BC], drT[BC * BC], dpT[BC * BC];  // transposes (columns as rows)
        };
        float tr[BD * TRP];  // 64 columns of S or dSo
    };
    int steep;  // some channel decays by more than STEEP within the chunk
};
static_assert(offsetof(GradLds, et) % 16 == 0 && offsetof(GradLds, tr) % 16 == 0 && offsetof(GradLds, da) % 16 == 0,
              "16-byte LDS rows");
static_assert(sizeof(GradLds) <= 160 * 1024, "gradient kernel LDS exceeds the CU's 160 KiB");

// Largest decay (nats) of a channel over one chunk for which the Gram
// gradients take the factored form below: its factors e^(+-(g - g_ref)) then
// stay within fp32's normal range.
constexpr float STEEP = 80.f;

// 16 x 16 product over 128 columns of two [16][GS] LDS matrices, X Z^T
// (lane (kq, n) gets rows 4 kq + r, column n)
__device__ __forceinline__ f4 gram16(const float *X, const float *Z, int m, int kq) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
        const f4 xa = *reinterpret_cast<const f4 *>(&X[m * GS + 16 * jt + 4 * kq]);
        const f4 zb = *reinterpret_cast<const f4 *>(&Z[m * GS + 16 * jt + 4 * kq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = mfma4(xa[i], zb[i], acc);
    }
    return acc;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses,
// not for its global loads (so that prefetches stay in flight across it).
// The waves share data through LDS alone; global memory is read-only input
// or write-only output here.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__global__ void __launch_bounds__(GNT) bwd_grads128_kernel(BwdArgs a, VarPlan vp, const float *rec,
                                                           const float *hist, const float *dhist, int nch) {
    __shared__ __attribute__((aligned(16))) GradLds L;
    const ChunkArgs &f = a.f;
    const int64_t H = f.H;
    const int64_t ntask = btask_count(f, vp, nch);
    const bool la_key = f.la_key, eb_key = f.eb_key, wr_key = f.wr_key, tied = f.wr == nullptr;
    const bool vw = f.value_write;  // read along b k, erase / write along k, values w .* v
    // this wave's value columns of S and dSo, consumed by the value products;
    // the next task's are loaded during this one's second half
    f4 S[8], dS[8];
    auto load_sd = [&](int64_t t) __attribute__((always_inline)) {
        // the state records' tiles of column group (wave) threadIdx.x / 64
        const int cg = threadIdx.x >> 6, ln = threadIdx.x & 63;
        const float *sg = hist + t * (BD * BD), *dsg = dhist + t * (BD * BD);
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            S[it] = *reinterpret_cast<const f4 *>(sg + tile_off(it, cg, ln));
            dS[it] = *reinterpret_cast<const f4 *>(dsg + tile_off(it, cg, ln));
        }
    };
    if (static_cast<int64_t>(blockIdx.x) < ntask) load_sd(blockIdx.x);
    for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
        // lane coordinates, re-derived every task so that the addresses built
        // from them are not hoisted out of the loop (and spilled)
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int m = lane & 15, kq = lane >> 4;
        const BTask tp = btask(f, vp, task, nch);
        const int64_t h = tp.h;
        const float *rc = rec + task * REC_BWD;
        auto row_of = [&](int r) { return (tp.tok0 + r) * H + h; };
        auto live = [&](int r) { return tp.tok0 + r < tp.tlim; };
        const int vcol = 16 * wv + m;

        // ---- the chunk's record, raw operands, V and dO.  Every load is issued
        //      before any is used (rows past the sequence end read as zero
        //      through the buffer range; bf16 / fp32 and per-channel / per-head
        //      operands differ only in offsets), and before the barrier that
        //      waits for the previous task's last LDS reads, then converted
        //      into LDS.
        f4 xr[3], xt;
        float xg;
#pragma unroll
        for (int p = 0; p < 3; ++p)  // Kbar, Etil, Util: quad tid of each
            xr[p] = *reinterpret_cast<const f4 *>(rc + (p == 0 ? R_KB : p == 1 ? R_ET : R_UT) + 4 * tid);
        if (tid < 256)  // Tm, Bm, R, P: consecutive in the record
            xt = *reinterpret_cast<const f4 *>(rc + R_TM + 4 * tid);
        else if (tid < 256 + BD)
            xg = rc[R_GM + tid - 256];
        f4 bb, ww;  // erase / write gates of token tid / 32, channels c4 .. c4 + 3 (for the last phase)
        const int r = tid >> 5, c4 = 4 * (tid & 31);
        {
            const int es = f.bf16 ? 2 : 4;
            // dword j of my four channels: bf16 takes two words, fp32 four
            auto qoff = [&](int j) { return static_cast<int>((r * H * BD + c4) * es + 4 * (f.bf16 ? (j < 1 ? j : 1) : j)); };
            auto goff = [&](int key, int j) { return static_cast<int>(key ? (r * H * BD + c4 + j) * 4 : r * H * 4); };
            const auto rk = rows_rsrc(f.k, H, h, tp.tok0, tp.tlim, BD, es);
            const auto rq = rows_rsrc(f.q, H, h, tp.tok0, tp.tlim, BD, es);
            const auto rv = rows_rsrc(f.v, H, h, tp.tok0, tp.tlim, BD, es);
            const auto ro = rows_rsrc(a.d_o, H, h, tp.tok0, tp.tlim, BD, 4);
            const auto rla = rows_rsrc(f.la, H, h, tp.tok0, tp.tlim, la_key ? BD : 1, 4);
            const auto reb = rows_rsrc(f.eb, H, h, tp.tok0, tp.tlim, eb_key ? BD : 1, 4);
            const auto rwr = rows_rsrc(tied ? f.eb : f.wr, H, h, tp.tok0, tp.tlim, (tied ? eb_key : wr_key) ? BD : 1, 4);
            const int wkey = tied ? eb_key : wr_key;
            uint32_t kw[4], qw[4], vw4[4], lw[4], bw[4], ww4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kw[j] = __builtin_amdgcn_raw_buffer_load_b32(rk, qoff(j), 0, 0);
                qw[j] = __builtin_amdgcn_raw_buffer_load_b32(rq, qoff(j), 0, 0);
                lw[j] = __builtin_amdgcn_raw_buffer_load_b32(rla, goff(la_key, j), 0, 0);
                bw[j] = __builtin_amdgcn_raw_buffer_load_b32(reb, goff(eb_key, j), 0, 0);
                ww4[j] = __builtin_amdgcn_raw_buffer_load_b32(rwr, goff(wkey, j), 0, 0);
                vw4[j] = __builtin_amdgcn_raw_buffer_load_b32(rv, qoff(j), 0, 0);
            }
            const f4 ov = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(ro, (r * H * BD + c4) * 4, 0, 0));
            auto qkv = [&](const uint32_t (&w)[4]) {
                return f.bf16 ? f4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                   __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)}
                              : f4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                                   __uint_as_float(w[3])};
            };
            auto gate = [&](const uint32_t (&w)[4]) {
                return f4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3])};
            };
            lds_barrier();  // the previous task is done with LDS
            if (tid == 0) L.steep = 0;
            // the record parts into LDS
#pragma unroll
            for (int p = 0; p < 3; ++p)
                *reinterpret_cast<f4 *>(&(p == 0 ? L.kb : p == 1 ? L.et : L.ut)[(tid / 32) * GS + 4 * (tid % 32)]) = xr[p];
            if (tid < 256) {
                float *dst = tid < 64 ? L.tm : tid < 128 ? L.bm : tid < 192 ? L.rr : L.pp;
                *reinterpret_cast<f4 *>(&dst[((tid & 63) >> 2) * TP + 4 * (tid & 3)]) = xt;
            } else if (tid < 256 + BD) {
                L.gm[tid - 256] = xg;
            }
            const f4 kv = qkv(kw), qv = f.q_scale * qkv(qw), la = gate(lw);
            f4 vv = qkv(vw4);
            bb = gate(bw);
            ww = gate(ww4);  // value-write: per value column
            {
                const int li = r * OS + c4;
                *reinterpret_cast<f4 *>(&L.q[li]) = qv;
                *reinterpret_cast<f4 *>(&L.g[li]) = la;
                *reinterpret_cast<f4 *>(&L.k[li]) = vw ? bb * kv : kv;
                *reinterpret_cast<f4 *>(&L.e[li]) = vw ? kv : bb * kv;
                *reinterpret_cast<f4 *>(&L.u[li]) = vw ? kv : ww * kv;
            }
            if (vw) {  // the raw values and write gates, for dv and dw after the value products
                *reinterpret_cast<f4 *>(&L.mm[r * GS + c4]) = vv;
                *reinterpret_cast<f4 *>(&L.dm[r * GS + c4]) = ww;
                vv = vv * ww;
            }
            *reinterpret_cast<f4 *>(&L.v[r * GS + c4]) = vv;
            *reinterpret_cast<f4 *>(&L.o[r * GS + c4]) = ov;
        }
        lds_barrier();
        if (tid < BD) {  // running log-decay (read only by the last phase)
            float run = 0.f;
            for (int r = 0; r < BC; ++r) {
                run += L.g[r * OS + tid];
                L.g[r * OS + tid] = run;
            }
            L.gc[tid] = run;
            if (L.g[tid] - run > STEEP) L.steep = 1;
        }

        // ---- value columns 16 wv + m: Bm V, X, M, dM, Y, dV
        f4 sr[8], dr[8];  // rows c = 16 wv + m of S and dSo (from the columns, through LDS)
        {
            const int col = vcol;
            float v4[4], o4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v4[j] = L.v[(4 * kq + j) * GS + col];
                o4[j] = L.o[(4 * kq + j) * GS + col];
            }
            f4 BV = {0.f, 0.f, 0.f, 0.f};
            {
                const f4 b4 = *reinterpret_cast<const f4 *>(&L.bm[m * TP + 4 * kq]);
#pragma unroll
                for (int j = 0; j < 4; ++j) BV = mfma4(b4[j], v4[j], BV);
            }
            f4 X = chan_product(L.kb, S, m, kq, BV);
            f4 M = {0.f, 0.f, 0.f, 0.f};
            {
                const f4 t4 = *reinterpret_cast<const f4 *>(&L.tm[m * TP + 4 * kq]);
#pragma unroll
                for (int j = 0; j < 4; ++j) M = mfma4(t4[j], X[j], M);
            }
            f4 dM = chan_product(L.et, dS, m, kq, f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int j = 0; j < 4; ++j) dM = mfma4(L.rr[(4 * kq + j) * TP + m], o4[j], dM);
            dM = -dM;
            f4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) Y = mfma4(L.tm[(4 * kq + j) * TP + m], dM[j], Y);
            f4 dV = chan_product(L.ut, dS, m, kq, f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dV = mfma4(L.pp[(4 * kq + j) * TP + m], o4[j], dV);
                dV = mfma4(L.bm[(4 * kq + j) * TP + m], Y[j], dV);
            }
            float wsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = 4 * kq + r;
                if (vw) {  // dV is the gradient of w .* v
                    const float vr = L.mm[tok * GS + col], wr = L.dm[tok * GS + col];
                    if (live(tok)) {
                        a.dv[row_of(tok) * BD + col] = dV[r] * wr;
                        if (wr_key) a.dwr[row_of(tok) * BD + col] = dV[r] * vr;
                    }
                    wsum[r] = dV[r] * vr;
                } else if (live(tok)) {
                    a.dv[row_of(tok) * BD + col] = dV[r];
                }
                L.mm[tok * GS + col] = M[r];
                L.dm[tok * GS + col] = dM[r];
                L.y[tok * GS + col] = Y[r];
                L.bv[tok * GS + col] = BV[r];
            }
            if (vw && !wr_key) {  // one write gate per head: partial sums over this wave's 16 columns
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float x = wsum[r];
                    x += __shfl_xor(x, 1);
                    x += __shfl_xor(x, 2);
                    x += __shfl_xor(x, 4);
                    x += __shfl_xor(x, 8);
                    if (m == 0) L.wpart[wv * BC + 4 * kq + r] = x;
                }
            }
        }
        lds_barrier();

        // ---- S and dSo from value columns (registers of the value products)
        //      to key rows (the channel products'), through LDS, 64 columns at
        //      a time (the four waves that own them write, every wave reads
        //      its rows' part): each is read from HBM once
        {
            auto rows_half = [&](const f4 (&cols)[8], f4 (&rows)[8], int half) __attribute__((always_inline)) {
                if ((wv >> 2) == half) {
                    const int cl = 16 * (wv & 3) + m;
#pragma unroll
                    for (int it = 0; it < 8; ++it)
#pragma unroll
                        for (int i = 0; i < 4; ++i) L.tr[(16 * it + 4 * kq + i) * TRP + cl] = cols[it][i];
                }
                lds_barrier();
                const float *src = &L.tr[(16 * wv + m) * TRP + 4 * kq];
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) rows[4 * half + jt] = *reinterpret_cast<const f4 *>(src + 16 * jt);
                lds_barrier();
            };
            rows_half(S, sr, 0);
            rows_half(S, sr, 1);
            rows_half(dS, dr, 0);
            rows_half(dS, dr, 1);
        }

        // ---- key channels c = 16 wv + m: dW, dQbar, dEtil, dUtil (over the
        //      value columns, S and dSo read as rows), the exit decay's term
        const int c = 16 * wv + m;
        f4 dW = {0.f, 0.f, 0.f, 0.f}, dQb = dW, dEt = dW, dUt = dW;
        {
            float dot = 0.f;
#pragma unroll
            for (int jt = 0; jt < 8; ++jt) {
                const f4 s4 = sr[jt], d4 = dr[jt];
                const int lo = m * GS + 16 * jt + 4 * kq;
                const f4 am = *reinterpret_cast<const f4 *>(&L.dm[lo]), ao = *reinterpret_cast<const f4 *>(&L.o[lo]);
                const f4 ax = *reinterpret_cast<const f4 *>(&L.mm[lo]), av = *reinterpret_cast<const f4 *>(&L.v[lo]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dW = mfma4(am[i], s4[i], dW);
                    dQb = mfma4(ao[i], s4[i], dQb);
                    dEt = mfma4(ax[i], d4[i], dEt);
                    dUt = mfma4(av[i], d4[i], dUt);
                    dot += s4[i] * d4[i];
                }
            }
            dEt = -dEt;
            dot += __shfl_xor(dot, 16);
            dot += __shfl_xor(dot, 32);
            const float dgc = L.gm[c] * dot;  // e^gC (dSo . S) for channel c
            __builtin_amdgcn_wave_barrier();
            if (kq == 0) L.gm[c] = dgc;  // only this wave reads channel c's entry
#pragma unroll
            for (int r = 0; r < 4; ++r) L.dw[(4 * kq + r) * GS + c] = dW[r];
        }
        lds_barrier();

        // the next task's state records: requested here, once the rows have
        // gone through LDS, so that they arrive while this task's 16 x 16 and
        // Gram gradients run
        if (task + gridDim.x < ntask) load_sd(task + gridDim.x);
        // ---- dKbar = Tm^T dW (registers); the 16 x 16 gradients
        f4 dKb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) dKb = mfma4(L.tm[(4 * kq + j) * TP + m], dW[j], dKb);
        if (wv < 4) {
            f4 x;
            float *dst, *dstT;
            int strict = 0;
            if (wv == 0) {         // dBm = Y V^T, strictly lower
                x = gram16(L.y, L.v, m, kq);
                dst = L.dbm;
                dstT = L.dbmT;
                strict = 1;
            } else if (wv == 1) {  // dR = -dO M^T
                x = -gram16(L.o, L.mm, m, kq);
                dst = L.dr;
                dstT = L.drT;
            } else if (wv == 2) {  // dP = dO V^T
                x = gram16(L.o, L.v, m, kq);
                dst = L.dp;
                dstT = L.dpT;
            } else {               // dT = dW Kbar^T + dM (Bm V)^T
                x = gram16(L.dw, L.kb, m, kq) + gram16(L.dm, L.bv, m, kq);
                dst = L.dt;
                dstT = L.x1;       // (not read)
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * kq + r;
                const float val = (m < row || (!strict && m == row)) ? x[r] : 0.f;
                dst[row * BC + m] = val;
                dstT[m * BC + row] = val;
            }
        }
        lds_barrier();
        // the channel gradients, for the (token, channel) phase below: lane =
        // channel there (V, dO, Kbar, Etil, Util and dW are no longer read)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int li = (4 * kq + r) * GS + c;
            L.kb[li] = dKb[r];
            L.et[li] = dQb[r];
            L.ut[li] = dEt[r];
            L.v[li] = dUt[r];
        }
        {  // the gates, into the regions of dO and dW (no longer read)
            const int r = tid >> 5, c4 = 4 * (tid & 31);
            *reinterpret_cast<f4 *>(&L.o[r * GS + c4]) = bb;
            *reinterpret_cast<f4 *>(&L.dw[r * GS + c4]) = ww;
        }
        if (wv == 0) {  // X1 = Tm^T dT
            f4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) x = mfma4(L.tm[(4 * kq + j) * TP + m], L.dt[(4 * kq + j) * BC + m], x);
#pragma unroll
            for (int r = 0; r < 4; ++r) L.x1[(4 * kq + r) * BC + m] = x[r];
        }
        lds_barrier();
        if (wv == 0) {  // dA = -X1 Tm^T, strictly lower
            f4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) x = mfma4(L.x1[m * BC + 4 * kq + j], L.tm[m * TP + 4 * kq + j], x);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * kq + r;
                const float val = m < row ? -x[r] : 0.f;
                L.da[row * BC + m] = val;
                L.daT[m * BC + row] = val;
            }
        }
        lds_barrier();

        // ---- per (token x, channel c): the Grams' gradients with x as row and
        //      as column, the decayed operands', then q, k and the gates.  Lane
        //      (kq, m) of wave w takes channel c = 16 w + m and tokens 4 kq .. +3.
        //        glk[x] = sum_y d_xy (dA[x][y] e_y + dBm[x][y] u_y)   (y < x)
        //        glq[x] = sum_y d_xy (dR[x][y] e_y + dP[x][y] u_y)    (y <= x)
        //        gre[x] = sum_y d_xy (dA[y][x] k_y + dR[y][x] q_y)    (y >= x)
        //        gru[x] = sum_y d_xy (dBm[y][x] k_y + dP[y][x] q_y)   (y >= x)
        //      with the pairwise decay d_xy = e^-|g_x - g_y| of channel c.
        {
            float *dgv = L.mm, *shr = L.dm, *dbs = L.y, *dws = L.bv;  // [16][GS] each, free now
            const int cc = 16 * wv + m, x0 = 4 * kq;
            const float gcc = L.gc[cc];
            float glk[4], glq[4], gre[4], gru[4];
            if (!L.steep) {
                // factored around g_ref = g at token 7: d_xy = e^(g_x - g_ref) e^(g_ref - g_y)
                // for y <= x (the other way round for y >= x), so the four sums are
                // 16 x 16 by 16 x 128 products on the matrix cores; every factor is
                // below e^STEEP.  The B operand of lane (kq, m) is token 4 s + kq of
                // channel c, the A operand row m of the 16 x 16 gradients, read as
                // column m of the stored transpose (the half-wave's two tokens
                // then fall 16 banks apart).
                const float gref = L.g[7 * OS + cc];
                const f4 z = {0.f, 0.f, 0.f, 0.f};
                f4 GLK = z, GLQ = z, GRE = z, GRU = z;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int y = 4 * s4 + kq, ly = y * OS + cc, ay = y * BC + m;
                    const float gy = L.g[ly];
                    const float fe = __expf(gref - gy), fk = __expf(gy - gref);
                    const float ey = L.e[ly] * fe, uy = L.u[ly] * fe, ky = L.k[ly] * fk, qy = L.q[ly] * fk;
                    GLK = mfma4(L.daT[ay], ey, GLK);   // dA[m][y]
                    GLQ = mfma4(L.drT[ay], ey, GLQ);   // dR[m][y]
                    GRE = mfma4(L.da[ay], ky, GRE);    // dA[y][m]
                    GRU = mfma4(L.dbm[ay], ky, GRU);   // dBm[y][m]
                    GLK = mfma4(L.dbmT[ay], uy, GLK);  // dBm[m][y]
                    GLQ = mfma4(L.dpT[ay], uy, GLQ);   // dP[m][y]
                    GRE = mfma4(L.dr[ay], qy, GRE);    // dR[y][m]
                    GRU = mfma4(L.dp[ay], qy, GRU);    // dP[y][m]
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float gx = L.g[(x0 + r) * OS + cc];
                    const float fr = __expf(gx - gref), fc = __expf(gref - gx);
                    glk[r] = fr * GLK[r];
                    glq[r] = fr * GLQ[r];
                    gre[r] = fc * GRE[r];
                    gru[r] = fc * GRU[r];
                }
            } else {
                // a steep chunk: every pairwise decay formed directly (never above 1);
                // the operands are read where used (this path is rare)
                for (int r = 0; r < 4; ++r) {
                    const int x = x0 + r;
                    const float gx = L.g[x * OS + cc];
                    float sk = 0.f, sq = 0.f, se = 0.f, su = 0.f;
                    for (int jj = 0; jj < 4; ++jj) {
                        const int o4 = x * BC + 4 * jj;
                        const f4 ra = *reinterpret_cast<const f4 *>(&L.da[o4]), rb = *reinterpret_cast<const f4 *>(&L.dbm[o4]);
                        const f4 rr = *reinterpret_cast<const f4 *>(&L.dr[o4]), rp = *reinterpret_cast<const f4 *>(&L.dp[o4]);
                        const f4 ca = *reinterpret_cast<const f4 *>(&L.daT[o4]), cb = *reinterpret_cast<const f4 *>(&L.dbmT[o4]);
                        const f4 cr = *reinterpret_cast<const f4 *>(&L.drT[o4]), cp = *reinterpret_cast<const f4 *>(&L.dpT[o4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int yy = 4 * jj + e, ly = yy * OS + cc;
                            const float gy = L.g[ly], ey = L.e[ly], uy = L.u[ly], ky = L.k[ly], qy = L.q[ly];
                            const float d = __expf(yy < x ? gx - gy : gy - gx);
                            sk += (ra[e] * ey + rb[e] * uy) * d;
                            sq += (rr[e] * ey + rp[e] * uy) * d;
                            se += (ca[e] * ky + cr[e] * qy) * d;
                            su += (cb[e] * ky + cp[e] * qy) * d;
                        }
                    }
                    glk[r] = sk;
                    glq[r] = sq;
                    gre[r] = se;
                    gru[r] = su;
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int x = x0 + r;
                const float gx = L.g[x * OS + cc];
                const int li = x * OS + cc, lr = x * GS + cc;
                const float kx = L.k[li], qx = L.q[li], ex = L.e[li], ux = L.u[li];
                const float eg = __expf(gx), ec = __expf(gcc - gx);
                const float dkb = L.kb[lr], dqb = L.et[lr], det = L.ut[lr], dut = L.v[lr];
                const float de = gre[r] + det * ec, du = gru[r] + dut * ec;
                const float dg = kx * glk[r] + qx * glq[r] - ex * gre[r] - ux * gru[r] + (dkb * kx + dqb * qx) * eg -
                                 (det * ex + dut * ux) * ec;
                float dkk = glk[r] + dkb * eg, dbv = 0.f, dwv = 0.f;
                if (live(x)) {
                    const int64_t row = row_of(x);
                    const float bx = L.o[lr];
                    if (vw) {  // dkk is the gradient of the read key b k; e = u = k
                        dbv = dkk * ex;
                        dkk = dkk * bx + de + du;
                    } else if (tied) {
                        dkk += (de + du) * bx;
                        dbv = (de + du) * kx;
                    } else {
                        const float wx = L.dw[lr];
                        dkk += de * bx + du * wx;
                        dbv = de * kx;
                        dwv = du * kx;
                    }
                    a.dq[row * BD + cc] = f.q_scale * (glq[r] + dqb * eg);
                    a.dk[row * BD + cc] = dkk;
                    if (eb_key) a.deb[row * BD + cc] = dbv;
                    if (!tied && wr_key && !vw) a.dwr[row * BD + cc] = dwv;
                }
                dgv[lr] = dg;
                shr[lr] = (det * ex + dut * ux) * ec;  // this token's share of d gC
                dbs[lr] = dbv;
                dws[lr] = dwv;
            }
        }
        float *dgv = L.mm, *shr = L.dm, *dbs = L.y, *dws = L.bv;
        lds_barrier();
        // ---- d log a: the reverse running sum of dg, d gC entering at the last row
        if (tid < BD) {
            float run = L.gm[tid];
            for (int x = 0; x < BC; ++x) run += shr[x * GS + tid];
            for (int x = BC - 1; x >= 0; --x) {
                run += dgv[x * GS + tid];
                if (la_key) {
                    if (live(x)) a.dla[row_of(x) * BD + tid] = run;
                } else {
                    dgv[x * GS + tid] = run;
                }
            }
        }
        // ---- gates with one value per token-head sum their channels
        if (!la_key || !eb_key || (!tied && !wr_key)) {
            lds_barrier();
            if (tid < BC && live(tid)) {
                const int x = tid;
                float sl = 0.f, sb = 0.f, sw = 0.f;
                // channel (j + x) mod 128 at step j: the 16 lanes' rows then fall
                // on distinct banks (row stride GS is 8 banks mod 32)
                for (int j = 0; j < BD; ++j) {
                    const int cc = (j + x) & (BD - 1);
                    sl += dgv[x * GS + cc];
                    sb += dbs[x * GS + cc];
                    sw += dws[x * GS + cc];
                }
                const int64_t row = row_of(x);
                if (!la_key) a.dla[row] = sl;
                if (!eb_key) a.deb[row] = sb;
                if (vw && !wr_key) {
                    sw = 0.f;
                    for (int w8 = 0; w8 < 8; ++w8) sw += L.wpart[w8 * BC + x];
                }
                if (!tied && !wr_key) a.dwr[row] = sw;
            }
        }
    }
}

}  // namespace

size_t bwd_record_bytes(int64_t chunks) { return static_cast<size_t>(chunks * REC_BWD * 4); }

// Segments per chain for the scans: as many as keep the summaries' 6 nseg - 8
// workgroups per chain within one round of two per CU, each of at least 64
// chunks; one (a single pass) from 32 chains up.  The summaries and the
// rescan each walk one segment at some 4.5 us per step (two workgroups per
// CU), a single pass the whole chain at 3.2 us (its CUs to itself), so the
// segments pay below about 30 chains.
int bwd_segments(int64_t chains, int nch) {
    constexpr int MIN_LEN = 64;
    if (chains <= 0 || chains >= 32) return 1;
    int64_t n = (512 / chains + 8) / 6;
    if (n > nch / MIN_LEN) n = nch / MIN_LEN;
    if (n < 2) return 1;
    const int64_t len = (nch + n - 1) / n;
    return static_cast<int>((nch + len - 1) / len);  // no empty segment
}

size_t bwd_segment_bytes(int64_t chains, int nseg) {
    return static_cast<size_t>(2 * 2 * chains * nseg) * BD * BD * 4;  // xs, fs; states and gradients
}

hipError_t launch_bwd_d128(const BwdArgs &a, const VarPlan &vp, float *rec, float *hist, float *dhist, float *segs,
                           int nch, hipStream_t s) {
    const ChunkArgs &f = a.f;
    // (packed sequences: the bound on the task count; the kernels read the count)
    const int64_t tasks = f.cu ? f.H * varlen_chunk_bound(f.B, f.T, BC) : f.B * f.H * nch;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    // the record pass loops over tasks: as many workgroups as can be resident
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bwd_record_kernel, BNT, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const int64_t g1 = tasks < int64_t(per_cu) * cus ? tasks : int64_t(per_cu) * cus;
    hipLaunchKernelGGL(bwd_record_kernel, dim3(static_cast<unsigned>(g1)), dim3(BNT), 0, s, a, vp, rec, nch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t chains = f.B * f.H;
    const int nseg = f.cu ? 1 : bwd_segments(chains, nch);
    if (nseg > 1) {
        BwdSegs sg;
        sg.nseg = nseg;
        sg.len = (nch + nseg - 1) / nseg;
        sg.xs = segs;
        sg.fs = segs + 2 * chains * nseg * BD * BD;
        // (chain, value half, summary) x (state, gradient); then the exact
        // entries; then (chain, value half, segment) x (state, gradient)
        sg.us = chains * 2 * (2 * nseg - 3);
        const unsigned g1s = static_cast<unsigned>(sg.us + chains * 2 * (nseg - 1));
        hipLaunchKernelGGL(bwd_seg_scans_kernel<1>, dim3(g1s), dim3(SNT), 0, s, a, vp, static_cast<const float *>(rec),
                           hist, dhist, nch, sg);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_segment_combine(sg.xs, sg.fs, 2 * chains, nseg, s)) != hipSuccess) return e;
        sg.us = chains * 2 * nseg;
        const unsigned g0s = static_cast<unsigned>(2 * sg.us);
        hipLaunchKernelGGL(bwd_seg_scans_kernel<0>, dim3(g0s), dim3(SNT), 0, s, a, vp, static_cast<const float *>(rec),
                           hist, dhist, nch, sg);
    } else {
        const unsigned g2 = static_cast<unsigned>(chains * 4);  // (chain, value half) x (state, gradient)
        hipLaunchKernelGGL(bwd_scans_kernel, dim3(g2), dim3(SNT), 0, s, a, vp, static_cast<const float *>(rec), hist,
                           dhist, nch);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t g3 = tasks < cus ? tasks : cus;  // one 137 KiB workgroup per CU
    hipLaunchKernelGGL(bwd_grads128_kernel, dim3(static_cast<unsigned>(g3)), dim3(GNT), 0, s, a, vp,
                       static_cast<const float *>(rec), static_cast<const float *>(hist),
                       static_cast<const float *>(dhist), nch);
    return hipGetLastError();
}

}  // namespace gdn2
