// chunk_general.hip -- chunkwise-parallel GDN-2 forward, fp32 on the vector ALU.
//
// The general path: any dk, dv in 1..128, q/k/v in fp32 or bf16, every gate
// kind.  It serves fp32 inputs (whose 1e-5 tolerance rules out 16-bit matrix
// operands) and every shape the MFMA path does not cover.
//
// Algorithm (chunkwise WY/UT form; "Gated DeltaNet-2" blog summary, "Core
// Mechanism"; gist.science summary, "Technische Samenvatting" section 3):
// within a chunk of Cg tokens entering with state S, with g the inclusive
// cumulative log-decay of the chunk (per key channel), e = b*k, u = w*k,
//   A[r,s] = sum_c k_r e_s exp(g_r-g_s) (r>s),  Bm: u for e   (erase / write Grams)
//   R[r,s] = sum_c q_r e_s exp(g_r-g_s) (r>=s), P:  u for e   (query Grams)
//   Tm = (I + A)^-1                                           (unit lower triangular)
//   M = Tm (Kbar S + Bm V),  Kbar = k exp(g)                  (erase reads of the decayed state)
//   O = Qbar S + P V - R M,  Qbar = q exp(g)
//   S <- exp(g_C) S + Util^T V - Etil^T M,  Util = u exp(g_C - g), Etil = e exp(g_C - g)
// Every pairwise decay exp(g_r - g_s) is formed directly (r >= s, so it is
// <= 1 and never overflows).  One workgroup owns one (batch, head) chain and
// a DVT-wide slice of the value channels (value columns evolve independently
// given the chunk's Grams) and walks the chunks in order; the state slice
// stays in LDS for the whole sequence.
//
// The value-write form (erase gate on the read, write gate per value
// channel) is the same algebra with the read key b .* k in place of k,
// erase and write vectors k, and values w .* v.
//
// With `hist` set (the backward's first step), the kernel instead records
// the state entering every chunk, hist[chain][chunk][dk][dv] (packed
// sequences: hist[chunk][head][dk][dv], the chunks of the plan), and writes
// no output.
#include "common.h"
#include "kernels.h"

namespace gdn2 {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsBudget = 64 * 1024;

struct GenLayout {
    int kf, qf, g, eb, uw, vv, xx, mm, A, Bm, R, P, Tm, S, gC, total;
};

// Row stride of the Cg x dk arrays: odd, so that lanes reading one channel
// of different rows (the Gram loops) hit different LDS banks.
__host__ __device__ inline int row_stride(int dk) { return dk | 1; }

__host__ __device__ inline GenLayout gen_layout(int Cg, int DVT, int dk) {
    GenLayout L;
    int off = 0;
    const int KS = row_stride(dk);
    auto take = [&](int n) { int o = off; off += n; return o; };
    L.kf = take(Cg * KS);
    L.qf = take(Cg * KS);
    L.g = take(Cg * KS);
    L.eb = take(Cg * KS);
    L.uw = take(Cg * KS);
    L.vv = take(Cg * DVT);
    L.xx = take(Cg * DVT);
    L.mm = take(Cg * DVT);
    L.A = take(Cg * Cg);
    L.Bm = take(Cg * Cg);
    L.R = take(Cg * Cg);
    L.P = take(Cg * Cg);
    L.Tm = take(Cg * Cg);
    L.S = take(dk * DVT);
    L.gC = take(dk);
    L.total = off;
    return L;
}

__global__ void __launch_bounds__(kThreads) chunk_general_kernel(ChunkArgs a, int Cg, int DVT, float *hist,
                                                                 VarPlan vp) {
    extern __shared__ float lds[];
    const int dk = static_cast<int>(a.dk), dv = static_cast<int>(a.dv);
    const int64_t T = a.T, H = a.H;
    const GenLayout L = gen_layout(Cg, DVT, dk);
    const int KS = row_stride(dk);
    float *Kf = lds + L.kf, *Qf = lds + L.qf, *G = lds + L.g, *Eb = lds + L.eb, *Uw = lds + L.uw;
    float *V = lds + L.vv, *X = lds + L.xx, *M = lds + L.mm;
    float *A = lds + L.A, *Bm = lds + L.Bm, *R = lds + L.R, *P = lds + L.P, *Tm = lds + L.Tm;
    float *S = lds + L.S, *gC = lds + L.gC;

    const int64_t bh = blockIdx.x;
    const int64_t b = bh / H, h = bh % H;
    // tokens [lo, hi) of the flattened [B*T] token axis: sequence b of T
    // tokens, or, packed, offsets cu[b], cu[b+1] clamped into [0, T] and
    // [lo, T] (no access leaves the tensors whatever they hold)
    int64_t lo = b * T, hi = lo + T;
    int64_t nmax = (T + Cg - 1) / Cg;  // chunks this chain walks
    if (a.cu && vp.seq) {               // the plan's ranges and chunk counts (the backward's records)
        const int2 e = vp.seq[b];
        lo = e.x;
        hi = e.y;
        nmax = vp.pfx[b + 1] - vp.pfx[b];
    } else if (a.cu) {
        lo = min(max(static_cast<int64_t>(a.cu[b]), int64_t(0)), T);
        hi = min(max(static_cast<int64_t>(a.cu[b + 1]), lo), T);
        nmax = (hi - lo + Cg - 1) / Cg;
    }
    const int col0 = blockIdx.y * DVT;
    const int ncol = min(DVT, dv - col0);
    const int tid = threadIdx.x;
    const int64_t sbase = (b * H + h) * static_cast<int64_t>(dk) * dv;

    for (int idx = tid; idx < dk * DVT; idx += kThreads) {
        const int c = idx / DVT, j = idx % DVT;
        S[idx] = (a.s0 && j < ncol) ? a.s0[sbase + static_cast<int64_t>(c) * dv + col0 + j] : 0.f;
    }

    const int64_t nch = (T + Cg - 1) / Cg;  // (hist: B sequences of T tokens)
    for (int64_t t0 = lo, n = 0; t0 < hi && n < nmax; t0 += Cg, ++n) {
        __syncthreads();
        if (hist) {
            const int64_t rec_i = a.cu ? (vp.pfx[b] + n) * H + h : (b * H + h) * nch + n;
            float *hs = hist + rec_i * static_cast<int64_t>(dk) * dv;
            for (int idx = tid; idx < dk * DVT; idx += kThreads) {
                const int c = idx / DVT, j = idx % DVT;
                if (j < ncol) hs[static_cast<int64_t>(c) * dv + col0 + j] = S[idx];
            }
        }
        // 1. stage the chunk: keys, queries, raw log-decay, e = b*k, u = w*k, values.
        //    With in-kernel q/k normalisation the raw rows and the gates are
        //    staged first and combined once the row norms are known.
        const bool norm = a.qk_norm;
        for (int idx = tid; idx < Cg * dk; idx += kThreads) {
            const int r = idx / dk, c = idx % dk;
            const int64_t t = t0 + r;
            float kv = 0.f, qv = 0.f, la = 0.f, bb = 0.f, ww = 0.f;
            if (t < hi) {
                const int64_t row = t * H + h;
                kv = load_qkv(a.k, row * dk + c, a.bf16);
                qv = load_qkv(a.q, row * dk + c, a.bf16);
                la = load_gate_x(a.la, a.la_key, row, dk, c, a.gate_logits, 0);
                bb = load_gate_x(a.eb, a.eb_key, row, dk, c, a.gate_logits, 1);
                ww = a.value_write ? 0.f : a.wr ? load_gate_x(a.wr, a.wr_key, row, dk, c, a.gate_logits, 1) : bb;
            }
            const int li = r * KS + c;
            G[li] = la;
            if (norm) {
                Kf[li] = kv;
                Qf[li] = qv;
                Eb[li] = bb;
                Uw[li] = ww;
            } else {
                Qf[li] = a.q_scale * qv;
                if (a.value_write) {  // the read key is b .* k; erase and write run along k
                    Kf[li] = bb * kv;
                    Eb[li] = Uw[li] = kv;
                } else {
                    Kf[li] = kv;
                    Eb[li] = bb * kv;
                    Uw[li] = ww * kv;
                }
            }
        }
        for (int idx = tid; idx < Cg * DVT; idx += kThreads) {
            const int r = idx / DVT, j = idx % DVT;
            const int64_t t = t0 + r;
            float vv = 0.f;
            if (t < hi && j < ncol) {
                const int64_t row = t * H + h;
                vv = load_qkv(a.v, row * dv + col0 + j, a.bf16);
                if (a.value_write) vv *= load_gate_x(a.wr, a.wr_key, row, dv, col0 + j, a.gate_logits, 1);  // w .* v
            }
            V[idx] = vv;
        }
        if (norm) {
            __syncthreads();
            float *inv = A;  // 1 / ||k_r||, then 1 / ||q_r|| (A is written later)
            for (int i = tid; i < 2 * Cg; i += kThreads) {
                const float *x = (i < Cg ? Kf : Qf) + (i % Cg) * KS;
                float ss = 0.f;
                for (int c = 0; c < dk; ++c) ss += x[c] * x[c];
                inv[i] = ss > 0.f ? rsqrtf(ss) : 0.f;
            }
            __syncthreads();
            for (int idx = tid; idx < Cg * dk; idx += kThreads) {
                const int r = idx / dk, li = r * KS + idx % dk;
                const float kv = Kf[li] * inv[r], bb = Eb[li], ww = Uw[li];
                Qf[li] = a.q_scale * Qf[li] * inv[Cg + r];
                if (a.value_write) {
                    Kf[li] = bb * kv;
                    Eb[li] = Uw[li] = kv;
                } else {
                    Kf[li] = kv;
                    Eb[li] = bb * kv;
                    Uw[li] = ww * kv;
                }
            }
        }
        __syncthreads();
        // 2. inclusive cumulative log-decay per key channel (padded rows add 0)
        for (int c = tid; c < dk; c += kThreads) {
            float acc = 0.f;
            for (int r = 0; r < Cg; ++r) {
                acc += G[r * KS + c];
                G[r * KS + c] = acc;
            }
            gC[c] = acc;
        }
        __syncthreads();
        // 3. the four decayed Grams
        for (int idx = tid; idx < Cg * Cg; idx += kThreads) {
            const int r = idx / Cg, s = idx % Cg;
            float sa = 0.f, sb = 0.f, sr = 0.f, sp = 0.f;
            if (s <= r) {
                for (int c = 0; c < dk; ++c) {
                    const float d = expf(G[r * KS + c] - G[s * KS + c]);
                    const float kd = Kf[r * KS + c] * d, qd = Qf[r * KS + c] * d;
                    const float e = Eb[s * KS + c], u = Uw[s * KS + c];
                    sa += kd * e;
                    sb += kd * u;
                    sr += qd * e;
                    sp += qd * u;
                }
            }
            A[idx] = s < r ? sa : 0.f;
            Bm[idx] = s < r ? sb : 0.f;
            R[idx] = sr;
            P[idx] = sp;
        }
        __syncthreads();
        // 4. Tm = (I + A)^-1, one column per thread by forward substitution;
        //    meanwhile everyone folds the decay into the state-side operands.
        if (tid < Cg) {
            const int j = tid;
            for (int r = 0; r < Cg; ++r) {
                float val;
                if (r < j) {
                    val = 0.f;
                } else if (r == j) {
                    val = 1.f;
                } else {
                    float acc = 0.f;
                    for (int s = j; s < r; ++s) acc += A[r * Cg + s] * Tm[s * Cg + j];
                    val = -acc;
                }
                Tm[r * Cg + j] = val;
            }
        }
        for (int idx = tid; idx < Cg * dk; idx += kThreads) {
            const int c = idx % dk, li = (idx / dk) * KS + c;
            const float eg = expf(G[li]);
            const float ec = expf(gC[c] - G[li]);
            Kf[li] *= eg;  // Kbar
            Qf[li] *= eg;  // Qbar
            Eb[li] *= ec;  // Etil
            Uw[li] *= ec;  // Util
        }
        __syncthreads();
        // 5. X = Kbar S + Bm V
        for (int idx = tid; idx < Cg * DVT; idx += kThreads) {
            const int r = idx / DVT, j = idx % DVT;
            float acc = 0.f;
            for (int c = 0; c < dk; ++c) acc += Kf[r * KS + c] * S[c * DVT + j];
            for (int s = 0; s < r; ++s) acc += Bm[r * Cg + s] * V[s * DVT + j];
            X[idx] = acc;
        }
        __syncthreads();
        // 6. M = Tm X
        for (int idx = tid; idx < Cg * DVT; idx += kThreads) {
            const int r = idx / DVT, j = idx % DVT;
            float acc = 0.f;
            for (int s = 0; s <= r; ++s) acc += Tm[r * Cg + s] * X[s * DVT + j];
            M[idx] = acc;
        }
        __syncthreads();
        // 7. O = Qbar S + P V - R M
        for (int idx = tid; idx < (hist ? 0 : Cg * DVT); idx += kThreads) {
            const int r = idx / DVT, j = idx % DVT;
            const int64_t t = t0 + r;
            if (t >= hi || j >= ncol) continue;
            float acc = 0.f;
            for (int c = 0; c < dk; ++c) acc += Qf[r * KS + c] * S[c * DVT + j];
            for (int s = 0; s <= r; ++s) acc += P[r * Cg + s] * V[s * DVT + j] - R[r * Cg + s] * M[s * DVT + j];
            store_out(a.o, (t * H + h) * dv + col0 + j, acc, a.o_bf16);
        }
        __syncthreads();
        // 8. S <- exp(g_C) S + Util^T V - Etil^T M (each thread owns its elements)
        for (int idx = tid; idx < dk * DVT; idx += kThreads) {
            const int c = idx / DVT, j = idx % DVT;
            float acc = expf(gC[c]) * S[idx];
            for (int s = 0; s < Cg; ++s) acc += Uw[s * KS + c] * V[s * DVT + j] - Eb[s * KS + c] * M[s * DVT + j];
            S[idx] = acc;
        }
    }
    __syncthreads();
    if (a.s_out) {
        for (int idx = tid; idx < dk * DVT; idx += kThreads) {
            const int c = idx / DVT, j = idx % DVT;
            if (j < ncol) a.s_out[sbase + static_cast<int64_t>(c) * dv + col0 + j] = S[idx];
        }
    }
}

}  // namespace

hipError_t launch_chunk_general(const ChunkArgs &a, hipStream_t s) {
    const int dk = static_cast<int>(a.dk), dv = static_cast<int>(a.dv);
    int Cg = 0, DVT = 0;
    // Largest chunk first, then the widest value slice that fits LDS.
    for (int c = a.C; c >= 16 && !Cg; c /= 2) {
        for (int w = 32; w >= 8; w /= 2) {
            const int wv = dv < w ? dv : w;
            if (gen_layout(c, wv, dk).total * 4 <= kLdsBudget) {
                Cg = c;
                DVT = wv;
                break;
            }
        }
    }
    if (!Cg) return hipErrorInvalidValue;
    const size_t lds = static_cast<size_t>(gen_layout(Cg, DVT, dk).total) * 4;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(chunk_general_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    dim3 grid(static_cast<unsigned>(a.B * a.H), static_cast<unsigned>((dv + DVT - 1) / DVT));
    hipLaunchKernelGGL(chunk_general_kernel, grid, dim3(kThreads), lds, s, a, Cg, DVT, nullptr, VarPlan{});
    return hipGetLastError();
}

hipError_t launch_chunk_general_hist(const ChunkArgs &a, int Cg, float *hist, const VarPlan &vp, hipStream_t s) {
    const int dk = static_cast<int>(a.dk), dv = static_cast<int>(a.dv);
    int DVT = 0;
    for (int w = 32; w >= 8 && !DVT; w /= 2) {
        const int wv = dv < w ? dv : w;
        if (gen_layout(Cg, wv, dk).total * 4 <= kLdsBudget) DVT = wv;
    }
    if (!DVT) return hipErrorInvalidValue;
    const size_t lds = static_cast<size_t>(gen_layout(Cg, DVT, dk).total) * 4;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(chunk_general_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    dim3 grid(static_cast<unsigned>(a.B * a.H), static_cast<unsigned>((dv + DVT - 1) / DVT));
    hipLaunchKernelGGL(chunk_general_kernel, grid, dim3(kThreads), lds, s, a, Cg, DVT, hist, vp);
    return hipGetLastError();
}

}  // namespace gdn2
