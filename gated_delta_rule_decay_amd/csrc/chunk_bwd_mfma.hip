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
// Four launches:
//   bwd_record_kernel   every chunk in parallel: the Grams (pairwise decays
//                       formed directly, never above 1), Tm by forward
//                       substitution, the decayed operands -> a record;
//   bwd_state_kernel    per (chain, 64 value columns), chunks in order: S in
//                       accumulator registers, recorded on entry to each chunk;
//   bwd_dgrad_kernel    per (chain, 64 value columns), chunks in reverse: dS in
//                       registers, recorded on entry (= each chunk's dSo), dS0;
//   bwd_grads128_kernel every chunk in parallel: all input gradients from the
//                       record, S and dSo.
// All arithmetic is fp32 (v_mfma_f32_16x16x4f32, fp32 accumulate), so the
// gradients keep the fp32 tolerance.
//
// Register layout.  A wave owns 16 value columns; its state slice (128 key
// channels x 16 columns) sits in 8 accumulator tiles: lane l = 16 kq + n holds
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
constexpr int RS = 132;   // LDS row stride of the 16 x 128 operands (2-way banked for the reads below)
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
// stride RS) in the channel order of the state registers B; four independent
// accumulation chains (channel 16 it + 4 kq + i goes to chain i), so that the
// matrix unit never waits on its own previous result for long.
__device__ __forceinline__ f4 chan_product(const float *A, const f4 (&B)[8], int m, int kq, f4 init) {
    const f4 z = {0.f, 0.f, 0.f, 0.f};
    f4 acc[4] = {init, z, z, z};
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const f4 a4 = *reinterpret_cast<const f4 *>(&A[m * RS + 16 * it + 4 * kq]);
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

// ---------------------------------------------------------------------------
// the record pass

constexpr int KS = BD + 1;  // odd row stride: the Gram loops read one channel of different rows

__global__ void __launch_bounds__(BNT) bwd_record_kernel(BwdArgs a, VarPlan vp, float *rec, int nch) {
    __shared__ float K[BC * KS], Q[BC * KS], G[BC * KS], E[BC * KS], U[BC * KS];
    __shared__ float A[BC * BC], Tm[BC * BC], gC[BD];
    const ChunkArgs &f = a.f;
    const int64_t T = f.T, H = f.H;
    const int64_t ntask = btask_count(f, vp, nch);
    const int tid = threadIdx.x;
    for (int64_t task = blockIdx.x; task < ntask; task += gridDim.x) {
        const BTask tp = btask(f, vp, task, nch);
        const int64_t h = tp.h;
        float *out = rec + task * REC_BWD;
        __syncthreads();  // the previous task is done with LDS
        for (int idx = tid; idx < BC * BD; idx += BNT) {
            const int r = idx / BD, c = idx % BD;
            float kv = 0.f, qv = 0.f, la = 0.f, e = 0.f, u = 0.f;
            if (tp.tok0 + r < tp.tlim) {
                const int64_t row = (tp.tok0 + r) * H + h;
                kv = load_qkv(f.k, row * BD + c, f.bf16);
                qv = f.q_scale * load_qkv(f.q, row * BD + c, f.bf16);
                la = load_gate(f.la, f.la_key, row, BD, c);
                const float bb = load_gate(f.eb, f.eb_key, row, BD, c);
                if (f.value_write) {  // read along b k, erase and write along k
                    e = u = kv;
                    kv *= bb;
                } else {
                    const float ww = f.wr ? load_gate(f.wr, f.wr_key, row, BD, c) : bb;
                    e = bb * kv;
                    u = ww * kv;
                }
            }
            const int li = r * KS + c;
            K[li] = kv; Q[li] = qv; G[li] = la; E[li] = e; U[li] = u;
        }
        __syncthreads();
        if (tid < BD) {  // running log-decay per channel (padded rows add 0)
            float run = 0.f;
            for (int r = 0; r < BC; ++r) {
                run += G[r * KS + tid];
                G[r * KS + tid] = run;
            }
            gC[tid] = run;
            out[R_GM + tid] = expf(run);
        }
        __syncthreads();
        {  // the four Grams, one (r, s) pair per thread, pairwise decays formed directly
            const int r = tid / BC, s = tid % BC;
            float sa = 0.f, sb = 0.f, sr = 0.f, sp = 0.f;
            if (s <= r) {
                for (int c = 0; c < BD; ++c) {
                    const float d = expf(G[r * KS + c] - G[s * KS + c]);
                    const float kd = K[r * KS + c] * d, qd = Q[r * KS + c] * d;
                    const float e = E[s * KS + c], u = U[s * KS + c];
                    sa += kd * e;
                    sb += kd * u;
                    sr += qd * e;
                    sp += qd * u;
                }
            }
            A[tid] = s < r ? sa : 0.f;
            out[R_BM + tid] = s < r ? sb : 0.f;
            out[R_RR + tid] = sr;
            out[R_PP + tid] = sp;
        }
        __syncthreads();
        // Tm = (I + A)^-1 by forward substitution, a column per thread; the
        // others fold the decays into the operands meanwhile
        if (tid < BC) {
            const int j = tid;
            for (int r = 0; r < BC; ++r) {
                float val = r < j ? 0.f : 1.f;
                if (r > j) {
                    float acc = 0.f;
                    for (int s = j; s < r; ++s) acc += A[r * BC + s] * Tm[s * BC + j];
                    val = -acc;
                }
                Tm[r * BC + j] = val;
            }
        }
        for (int idx = tid; idx < BC * BD; idx += BNT) {
            const int r = idx / BD, c = idx % BD, li = r * KS + c;
            const float eg = expf(G[li]), ec = expf(gC[c] - G[li]);
            out[R_KB + idx] = K[li] * eg;
            out[R_QB + idx] = Q[li] * eg;
            out[R_ET + idx] = E[li] * ec;
            out[R_UT + idx] = U[li] * ec;
        }
        __syncthreads();
        out[R_TM + tid] = Tm[tid];
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

// Copy the parts [(src0, m0), (src1, m1), (src2, m2), (srcT0, t0), (srcT1, t1), gm]
// of record `r`: every thread moves 8 + 8 + 8 + 1 + 1 (+ gm) floats as float4s.
struct Staged {
    f4 x[6];
    f4 tt[2];
    float g;
};

__device__ __forceinline__ void stage_load(Staged &st, const float *r, int o0, int o1, int o2, int oT0, int oT1,
                                           int tid) {
#pragma unroll
    for (int p = 0; p < 6; ++p) {
        const int part = p / 2, q = tid + BNT * (p % 2);  // float4 index 0..511 within a 16 x 128 part
        const int off = part == 0 ? o0 : part == 1 ? o1 : o2;
        st.x[p] = *reinterpret_cast<const f4 *>(r + off + 4 * q);
    }
    // the two 16 x 16 parts: 64 float4s each, threads 0..63 and 64..127
    const int q = tid & 63;
    st.tt[0] = *reinterpret_cast<const f4 *>(r + (tid < 64 ? oT0 : oT1) + 4 * q);
    st.g = tid < BD ? r[R_GM + tid] : 0.f;
}

__device__ __forceinline__ void stage_store(const Staged &st, ScanLds &L, int tid) {
#pragma unroll
    for (int p = 0; p < 6; ++p) {
        const int part = p / 2, q = tid + BNT * (p % 2);
        const int row = q / 32, col = 4 * (q % 32);
        float *m = part == 0 ? L.m0 : part == 1 ? L.m1 : L.m2;
        *reinterpret_cast<f4 *>(&m[row * RS + col]) = st.x[p];
    }
    if (tid < 128) *reinterpret_cast<f4 *>(&(tid < 64 ? L.t0 : L.t1)[4 * (tid & 63)]) = st.tt[0];
    if (tid < BD) L.gm[tid] = st.g;
}

// Four values of a [B*T*H, 128] row-major tensor for lane (kq, n): rows
// (tokens) 4 kq + j of the chunk, column col; zero past T.
__device__ __forceinline__ void load_rows4(float (&x)[4], const void *p, int bf16, int64_t h, int64_t tok0,
                                           int64_t tlim, int kq, int col, const ChunkArgs &f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t t = tok0 + 4 * kq + j;
        x[j] = t < tlim ? load_qkv(p, (t * f.H + h) * BD + col, bf16) : 0.f;
    }
}

// The values of lane (kq, n)'s rows, times the write gate in the value-write form.
__device__ __forceinline__ void load_vals4(float (&x)[4], int64_t h, int64_t tok0, int64_t tlim, int kq, int col,
                                           const ChunkArgs &f) {
    load_rows4(x, f.v, f.bf16, h, tok0, tlim, kq, col, f);
    if (f.value_write) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t t = tok0 + 4 * kq + j;
            if (t < tlim) x[j] *= load_gate(f.wr, f.wr_key, t * f.H + h, BD, col);
        }
    }
}

// Store (or read) a wave's 128 x 16 state slice to/from a [128][128] matrix.
__device__ __forceinline__ void put_state(float *dst, const f4 (&s)[8], int kq, int col) {
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * it + 4 * kq + i) * BD + col] = s[it][i];
}

// The state entering every chunk, hist[chain][chunk][128][128].
__global__ void __launch_bounds__(BNT) bwd_state_kernel(BwdArgs a, VarPlan vp, const float *rec, float *hist,
                                                        int nch) {
    __shared__ __attribute__((aligned(16))) ScanLds L;
    const ChunkArgs &f = a.f;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int m = lane & 15, kq = lane >> 4;
    const int64_t bh = blockIdx.x >> 1;
    const BChain ch = bchain(f, vp, bh, nch);
    const int64_t h = ch.h;
    const int col = 64 * (blockIdx.x & 1) + 16 * wv + m;  // this lane's value column (as n)
    auto rc = [&](int n) { return rec + (ch.task0 + n * ch.tstr) * static_cast<int64_t>(REC_BWD); };
    auto hs = [&](int n) { return hist + (ch.task0 + n * ch.tstr) * static_cast<int64_t>(BD * BD); };

    f4 S[8];
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[it][i] = f.s0 ? f.s0[bh * BD * BD + (16 * it + 4 * kq + i) * BD + col] : 0.f;

    // m0 = Kbar, m1 = Etil, m2 = Util; t0 = Tm, t1 = Bm
    Staged st;
    float vn[4];
    if (ch.nc > 0) {
        stage_load(st, rc(0), R_KB, R_ET, R_UT, R_TM, R_BM, tid);
        load_vals4(vn, h, ch.tbase, ch.tlim, kq, col, f);
    }
    for (int n = 0; n < ch.nc; ++n) {
        __syncthreads();  // every wave done with the previous chunk's LDS copy
        stage_store(st, L, tid);
        float v[4] = {vn[0], vn[1], vn[2], vn[3]};
        if (n + 1 < ch.nc) {
            stage_load(st, rc(n + 1), R_KB, R_ET, R_UT, R_TM, R_BM, tid);
            load_vals4(vn, h, ch.tbase + (n + 1) * BC, ch.tlim, kq, col, f);
        }
        put_state(hs(n), S, kq, col);
        __syncthreads();
        // X = Kbar S + Bm V (token rows)
        f4 X = chan_product(L.m0, S, m, kq, f4{0.f, 0.f, 0.f, 0.f});
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
        for (int it = 0; it < 8; ++it) {
            const f4 g4 = *reinterpret_cast<const f4 *>(&L.gm[16 * it + 4 * kq]);
            f4 s = g4 * S[it];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s = mfma4(L.m2[(4 * kq + j) * RS + 16 * it + m], v[j], s);
                s = mfma4(-L.m1[(4 * kq + j) * RS + 16 * it + m], M[j], s);
            }
            S[it] = s;
        }
    }
}

// The gradient of every chunk's exit state, dhist[chain][chunk][128][128],
// carried backwards from d_sT; the gradient of S0 at the end.
__global__ void __launch_bounds__(BNT) bwd_dgrad_kernel(BwdArgs a, VarPlan vp, const float *rec, float *dhist,
                                                        int nch) {
    __shared__ __attribute__((aligned(16))) ScanLds L;
    const ChunkArgs &f = a.f;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int m = lane & 15, kq = lane >> 4;
    const int64_t bh = blockIdx.x >> 1;
    const BChain ch = bchain(f, vp, bh, nch);
    const int64_t h = ch.h;
    const int col = 64 * (blockIdx.x & 1) + 16 * wv + m;
    auto rc = [&](int n) { return rec + (ch.task0 + n * ch.tstr) * static_cast<int64_t>(REC_BWD); };
    auto hs = [&](int n) { return dhist + (ch.task0 + n * ch.tstr) * static_cast<int64_t>(BD * BD); };

    f4 dS[8];
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int i = 0; i < 4; ++i) dS[it][i] = a.d_sT ? a.d_sT[bh * BD * BD + (16 * it + 4 * kq + i) * BD + col] : 0.f;

    // m0 = Etil, m1 = Qbar, m2 = Kbar; t0 = Tm, t1 = R
    Staged st;
    float on[4];
    const int nl = ch.nc - 1;
    if (nl >= 0) {
        stage_load(st, rc(nl), R_ET, R_QB, R_KB, R_TM, R_RR, tid);
        load_rows4(on, a.d_o, 0, h, ch.tbase + static_cast<int64_t>(nl) * BC, ch.tlim, kq, col, f);
    }
    for (int n = nl; n >= 0; --n) {
        __syncthreads();
        stage_store(st, L, tid);
        float o[4] = {on[0], on[1], on[2], on[3]};
        if (n > 0) {
            stage_load(st, rc(n - 1), R_ET, R_QB, R_KB, R_TM, R_RR, tid);
            load_rows4(on, a.d_o, 0, h, ch.tbase + static_cast<int64_t>(n - 1) * BC, ch.tlim, kq, col, f);
        }
        put_state(hs(n), dS, kq, col);
        __syncthreads();
        // dM = -(Etil dSo + R^T dO)  (token rows)
        f4 dM = chan_product(L.m0, dS, m, kq, f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int j = 0; j < 4; ++j) dM = mfma4(L.t1[(4 * kq + j) * BC + m], o[j], dM);
        dM = -dM;
        // Y = Tm^T dM
        f4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) Y = mfma4(L.t0[(4 * kq + j) * BC + m], dM[j], Y);
        // dS <- Diag(e^gC) dSo + Qbar^T dO + Kbar^T Y
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const f4 g4 = *reinterpret_cast<const f4 *>(&L.gm[16 * it + 4 * kq]);
            f4 s = g4 * dS[it];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s = mfma4(L.m1[(4 * kq + j) * RS + 16 * it + m], o[j], s);
                s = mfma4(L.m2[(4 * kq + j) * RS + 16 * it + m], Y[j], s);
            }
            dS[it] = s;
        }
    }
    if (a.ds0) put_state(a.ds0 + bh * BD * BD, dS, kq, col);
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

struct GradLds {
    float kb[BC * RS], et[BC * RS], ut[BC * RS];       // record: Kbar, Etil, Util
    float tm[BC * BC], bm[BC * BC], rr[BC * BC], pp[BC * BC];
    float gm[BD];                                        // e^gC, later d gC's exit term
    float k[BC * KS], q[BC * KS], e[BC * KS], u[BC * KS], g[BC * KS];  // raw operands; running log-decay
    float gc[BD];
    float v[BC * RS], o[BC * RS];                        // V, dO
    float mm[BC * RS], dm[BC * RS], y[BC * RS], bv[BC * RS];  // M, dM, Y, Bm V; later the per-(x, c) results
    float dw[BC * RS];
    float dt[BC * BC], x1[BC * BC], da[BC * BC], dbm[BC * BC], dr[BC * BC], dp[BC * BC];
    float daT[BC * BC], dbmT[BC * BC], drT[BC * BC], dpT[BC * BC];  // transposes (columns as rows)
    float wpart[8 * BC];  // value-write form, one write gate per head: per-wave partial sums of dw
};

// 16 x 16 product over 128 columns of two [16][RS] LDS matrices, X Z^T
// (lane (kq, n) gets rows 4 kq + r, column n)
__device__ __forceinline__ f4 gram16(const float *X, const float *Z, int m, int kq) {
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) {
        const f4 xa = *reinterpret_cast<const f4 *>(&X[m * RS + 16 * jt + 4 * kq]);
        const f4 zb = *reinterpret_cast<const f4 *>(&Z[m * RS + 16 * jt + 4 * kq]);
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
    // the next task's are loaded while this one finishes
    f4 S[8], dS[8];
    auto load_sd = [&](int64_t t) __attribute__((always_inline)) {
        const int vc = 16 * (threadIdx.x >> 6) + (threadIdx.x & 15), kk = (threadIdx.x >> 4) & 3;
        const float *sg = hist + t * (BD * BD), *dsg = dhist + t * (BD * BD);
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                S[it][i] = sg[(16 * it + 4 * kk + i) * BD + vc];
                dS[it][i] = dsg[(16 * it + 4 * kk + i) * BD + vc];
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
        const float *Sg = hist + task * (BD * BD), *dSg = dhist + task * (BD * BD);
        auto row_of = [&](int r) { return (tp.tok0 + r) * H + h; };
        auto live = [&](int r) { return tp.tok0 + r < tp.tlim; };
        lds_barrier();  // the previous task is done with LDS

        const int vcol = 16 * wv + m;

        // ---- the chunk's record, raw operands, V and dO
        for (int qi = tid; qi < 3 * 512; qi += GNT) {
            const int part = qi / 512, qq = qi % 512, row = qq / 32, col = 4 * (qq % 32);
            const f4 x = *reinterpret_cast<const f4 *>(rc + (part == 0 ? R_KB : part == 1 ? R_ET : R_UT) + 4 * qq);
            *reinterpret_cast<f4 *>(&(part == 0 ? L.kb : part == 1 ? L.et : L.ut)[row * RS + col]) = x;
        }
        if (tid < 256) {  // Tm, Bm, R, P: consecutive in the record
            const int part = tid / 64, qq = tid % 64;
            const f4 x = *reinterpret_cast<const f4 *>(rc + R_TM + 256 * part + 4 * qq);
            float *dst = part == 0 ? L.tm : part == 1 ? L.bm : part == 2 ? L.rr : L.pp;
            *reinterpret_cast<f4 *>(&dst[4 * qq]) = x;
        } else if (tid < 256 + BD) {
            L.gm[tid - 256] = rc[R_GM + tid - 256];
        }
        f4 bb, ww;  // erase / write gates of token tid / 32, channels c4 .. c4 + 3 (for the last phase)
        {  // token r = tid / 32, channels c4 .. c4 + 3
            const int r = tid >> 5, c4 = 4 * (tid & 31);
            const f4 z = {0.f, 0.f, 0.f, 0.f};
            f4 kv = z, qv = z, la = z, vv = z, ov = z;
            bb = z;
            ww = z;
            if (live(r)) {
                const int64_t row = row_of(r);
                kv = load4_qkv(f.k, row * BD + c4, f.bf16);
                qv = f.q_scale * load4_qkv(f.q, row * BD + c4, f.bf16);
                la = load4_gate(f.la, la_key, row, c4);
                bb = load4_gate(f.eb, eb_key, row, c4);
                ww = tied ? bb : load4_gate(f.wr, wr_key, row, c4);  // value-write: per value column
                vv = load4_qkv(f.v, row * BD + c4, f.bf16);
                ov = *reinterpret_cast<const f4 *>(a.d_o + row * BD + c4);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int li = r * KS + c4 + i;
                L.q[li] = qv[i]; L.g[li] = la[i];
                L.k[li] = vw ? bb[i] * kv[i] : kv[i];
                L.e[li] = vw ? kv[i] : bb[i] * kv[i];
                L.u[li] = vw ? kv[i] : ww[i] * kv[i];
            }
            if (vw) {  // the raw values and write gates, for dv and dw after the value products
                *reinterpret_cast<f4 *>(&L.mm[r * RS + c4]) = vv;
                *reinterpret_cast<f4 *>(&L.dm[r * RS + c4]) = ww;
                vv = vv * ww;
            }
            *reinterpret_cast<f4 *>(&L.v[r * RS + c4]) = vv;
            *reinterpret_cast<f4 *>(&L.o[r * RS + c4]) = ov;
        }
        lds_barrier();
        if (tid < BD) {  // running log-decay (read only by the last phase)
            float run = 0.f;
            for (int r = 0; r < BC; ++r) {
                run += L.g[r * KS + tid];
                L.g[r * KS + tid] = run;
            }
            L.gc[tid] = run;
        }

        // ---- value columns 16 wv + m: Bm V, X, M, dM, Y, dV
        {
            const int col = vcol;
            float v4[4], o4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v4[j] = L.v[(4 * kq + j) * RS + col];
                o4[j] = L.o[(4 * kq + j) * RS + col];
            }
            f4 BV = {0.f, 0.f, 0.f, 0.f};
            {
                const f4 b4 = *reinterpret_cast<const f4 *>(&L.bm[m * BC + 4 * kq]);
#pragma unroll
                for (int j = 0; j < 4; ++j) BV = mfma4(b4[j], v4[j], BV);
            }
            f4 X = chan_product(L.kb, S, m, kq, BV);
            f4 M = {0.f, 0.f, 0.f, 0.f};
            {
                const f4 t4 = *reinterpret_cast<const f4 *>(&L.tm[m * BC + 4 * kq]);
#pragma unroll
                for (int j = 0; j < 4; ++j) M = mfma4(t4[j], X[j], M);
            }
            f4 dM = chan_product(L.et, dS, m, kq, f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int j = 0; j < 4; ++j) dM = mfma4(L.rr[(4 * kq + j) * BC + m], o4[j], dM);
            dM = -dM;
            f4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) Y = mfma4(L.tm[(4 * kq + j) * BC + m], dM[j], Y);
            f4 dV = chan_product(L.ut, dS, m, kq, f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dV = mfma4(L.pp[(4 * kq + j) * BC + m], o4[j], dV);
                dV = mfma4(L.bm[(4 * kq + j) * BC + m], Y[j], dV);
            }
            float wsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tok = 4 * kq + r;
                if (vw) {  // dV is the gradient of w .* v
                    const float vr = L.mm[tok * RS + col], wr = L.dm[tok * RS + col];
                    if (live(tok)) {
                        a.dv[row_of(tok) * BD + col] = dV[r] * wr;
                        if (wr_key) a.dwr[row_of(tok) * BD + col] = dV[r] * vr;
                    }
                    wsum[r] = dV[r] * vr;
                } else if (live(tok)) {
                    a.dv[row_of(tok) * BD + col] = dV[r];
                }
                L.mm[tok * RS + col] = M[r];
                L.dm[tok * RS + col] = dM[r];
                L.y[tok * RS + col] = Y[r];
                L.bv[tok * RS + col] = BV[r];
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

        // ---- key channels c = 16 wv + m: dW, dQbar, dEtil, dUtil (over the
        //      value columns, S and dSo read as rows), the exit decay's term
        const int c = 16 * wv + m;
        f4 dW = {0.f, 0.f, 0.f, 0.f}, dQb = dW, dEt = dW, dUt = dW;
        {
            const float *srow = Sg + c * BD, *drow = dSg + c * BD;
            float dot = 0.f;
#pragma unroll 2
            for (int jt = 0; jt < 8; ++jt) {
                const f4 s4 = *reinterpret_cast<const f4 *>(srow + 16 * jt + 4 * kq);
                const f4 d4 = *reinterpret_cast<const f4 *>(drow + 16 * jt + 4 * kq);
                const int lo = m * RS + 16 * jt + 4 * kq;
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
            for (int r = 0; r < 4; ++r) L.dw[(4 * kq + r) * RS + c] = dW[r];
        }
        if (task + gridDim.x < ntask) load_sd(task + gridDim.x);  // in flight until the next task
        lds_barrier();

        // ---- dKbar = Tm^T dW (registers); the 16 x 16 gradients
        f4 dKb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) dKb = mfma4(L.tm[(4 * kq + j) * BC + m], dW[j], dKb);
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
            const int li = (4 * kq + r) * RS + c;
            L.kb[li] = dKb[r];
            L.et[li] = dQb[r];
            L.ut[li] = dEt[r];
            L.v[li] = dUt[r];
        }
        {  // the gates, into the regions of dO and dW (no longer read)
            const int r = tid >> 5, c4 = 4 * (tid & 31);
            *reinterpret_cast<f4 *>(&L.o[r * RS + c4]) = bb;
            *reinterpret_cast<f4 *>(&L.dw[r * RS + c4]) = ww;
        }
        if (wv == 0) {  // X1 = Tm^T dT
            f4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) x = mfma4(L.tm[(4 * kq + j) * BC + m], L.dt[(4 * kq + j) * BC + m], x);
#pragma unroll
            for (int r = 0; r < 4; ++r) L.x1[(4 * kq + r) * BC + m] = x[r];
        }
        lds_barrier();
        if (wv == 0) {  // dA = -X1 Tm^T, strictly lower
            f4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) x = mfma4(L.x1[m * BC + 4 * kq + j], L.tm[m * BC + 4 * kq + j], x);
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
        //      as column, the decayed operands', then q, k and the gates.  Wave
        //      w takes tokens 4 (w / 2) .. +3 of channels 64 (w % 2) + lane, so
        //      a token is uniform across the wave and the rows (and, through the
        //      transposes, the columns) of dA, dBm, dR, dP are broadcast reads.
        {
            float *dgv = L.mm, *shr = L.dm, *dbs = L.y, *dws = L.bv;  // [16][RS] each, free now
            const int cc = 64 * (wv & 1) + lane, x0 = 4 * (wv >> 1);
            const float gcc = L.gc[cc];
            float gy[BC], ey[BC], uy[BC], ky[BC], qy[BC];  // channel cc of every token
#pragma unroll
            for (int yy = 0; yy < BC; ++yy) {
                const int ly = yy * KS + cc;
                gy[yy] = L.g[ly]; ey[yy] = L.e[ly]; uy[yy] = L.u[ly]; ky[yy] = L.k[ly]; qy[yy] = L.q[ly];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int x = x0 + r;
                const float gx = L.g[x * KS + cc];
                // x as the row (dA[x][y] ...: zero for y >= x, dR/dP also at y = x)
                // and as the column (dA[y][x] ... via the transposes), with the
                // pairwise decay e^(g_x - g_y) for y before x, e^(g_y - g_x) after
                float glk = 0.f, glq = 0.f, gre = 0.f, gru = 0.f;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int o4 = x * BC + 4 * jj;
                    const f4 ra = *reinterpret_cast<const f4 *>(&L.da[o4]), rb = *reinterpret_cast<const f4 *>(&L.dbm[o4]);
                    const f4 rr = *reinterpret_cast<const f4 *>(&L.dr[o4]), rp = *reinterpret_cast<const f4 *>(&L.dp[o4]);
                    const f4 ca = *reinterpret_cast<const f4 *>(&L.daT[o4]), cb = *reinterpret_cast<const f4 *>(&L.dbmT[o4]);
                    const f4 cr = *reinterpret_cast<const f4 *>(&L.drT[o4]), cp = *reinterpret_cast<const f4 *>(&L.dpT[o4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int yy = 4 * jj + e;
                        const float d = __expf(yy < x ? gx - gy[yy] : gy[yy] - gx);
                        glk += (ra[e] * ey[yy] + rb[e] * uy[yy]) * d;
                        glq += (rr[e] * ey[yy] + rp[e] * uy[yy]) * d;
                        gre += (ca[e] * ky[yy] + cr[e] * qy[yy]) * d;
                        gru += (cb[e] * ky[yy] + cp[e] * qy[yy]) * d;
                    }
                }
                const int li = x * KS + cc, lr = x * RS + cc;
                const float kx = L.k[li], qx = L.q[li], ex = L.e[li], ux = L.u[li];
                const float eg = __expf(gx), ec = __expf(gcc - gx);
                const float dkb = L.kb[lr], dqb = L.et[lr], det = L.ut[lr], dut = L.v[lr];
                const float de = gre + det * ec, du = gru + dut * ec;
                const float dg = kx * glk + qx * glq - ex * gre - ux * gru + (dkb * kx + dqb * qx) * eg -
                                 (det * ex + dut * ux) * ec;
                float dkk = glk + dkb * eg, dbv = 0.f, dwv = 0.f;
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
                    a.dq[row * BD + cc] = f.q_scale * (glq + dqb * eg);
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
            for (int x = 0; x < BC; ++x) run += shr[x * RS + tid];
            for (int x = BC - 1; x >= 0; --x) {
                run += dgv[x * RS + tid];
                if (la_key) {
                    if (live(x)) a.dla[row_of(x) * BD + tid] = run;
                } else {
                    dgv[x * RS + tid] = run;
                }
            }
        }
        // ---- gates with one value per token-head sum their channels
        if (!la_key || !eb_key || (!tied && !wr_key)) {
            lds_barrier();
            if (tid < BC && live(tid)) {
                const int x = tid;
                float sl = 0.f, sb = 0.f, sw = 0.f;
                for (int cc = 0; cc < BD; ++cc) {
                    sl += dgv[x * RS + cc];
                    sb += dbs[x * RS + cc];
                    sw += dws[x * RS + cc];
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

hipError_t launch_bwd_d128(const BwdArgs &a, const VarPlan &vp, float *rec, float *hist, float *dhist, int nch,
                           hipStream_t s) {
    const ChunkArgs &f = a.f;
    // (packed sequences: the bound on the task count; the kernels read the count)
    const int64_t tasks = f.cu ? f.H * varlen_chunk_bound(f.B, f.T, BC) : f.B * f.H * nch;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t g1 = tasks < 8 * cus ? tasks : 8 * cus;
    hipLaunchKernelGGL(bwd_record_kernel, dim3(static_cast<unsigned>(g1)), dim3(BNT), 0, s, a, vp, rec, nch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g2 = static_cast<unsigned>(f.B * f.H * 2);
    hipLaunchKernelGGL(bwd_state_kernel, dim3(g2), dim3(BNT), 0, s, a, vp, static_cast<const float *>(rec), hist, nch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dgrad_kernel, dim3(g2), dim3(BNT), 0, s, a, vp, static_cast<const float *>(rec), dhist,
                       nch);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t g3 = tasks < cus ? tasks : cus;  // one 137 KiB workgroup per CU
    hipLaunchKernelGGL(bwd_grads128_kernel, dim3(static_cast<unsigned>(g3)), dim3(GNT), 0, s, a, vp,
                       static_cast<const float *>(rec), static_cast<const float *>(hist),
                       static_cast<const float *>(dhist), nch);
    return hipGetLastError();
}

}  // namespace gdn2
