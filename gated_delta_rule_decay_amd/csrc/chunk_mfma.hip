// chunk_mfma.hip -- chunkwise GDN-2 forward on the gfx950 matrix cores.
//
// Covers bf16 q/k/v with dk = dv = 128 and chunk C = 64 (any gate kinds, tied
// or not).  One workgroup of 256 lanes owns one (batch, head) chain and a
// VT-wide slice of the value channels, and walks the chunks of the sequence
// in order; the fp32 state slice (128 x VT) lives in MFMA accumulators for
// the whole sequence.
//
// Per chunk (the WY/UT form named in the gist.science summary, "Technische
// Samenvatting" section 3: cumulative per-channel decay absorbed into erase
// and write factors, a unit-lower-triangular solve for the auxiliary
// matrices), with g the inclusive cumulative log-decay of the chunk, e = b*k,
// u = w*k:
//   Grams   A[r,s] = sum_c k_r e_s exp(g_r-g_s) (r>s), Bm with u   (erase / write)
//           R[r,s] = sum_c q_r e_s exp(g_r-g_s) (r>=s), P with u  (query)
//   solve   Tm = (I + A)^-1
//   state   M = Tm (Kbar S + Bm V)          Kbar = k exp(g)
//           O = Qbar S + P V - R M          Qbar = q exp(g)
//           S <- exp(g_C) S + Util^T V - Etil^T M
//
// Numerics.  Every matrix product runs on v_mfma with fp16 operands and fp32
// accumulation; the state, the solve and all gate arithmetic stay fp32.
// fp16 (11-bit significand) rather than bf16 (8-bit) because one bf16
// rounding of the derived operands alone costs ~2.9e-3 relative error, above
// the 2e-3 budget, while fp16 costs ~3.6e-4.  fp16's narrow exponent range
// is handled by factoring exp(g_r - g_s) around a reference inside each
// 16-token block: the row side carries exp(g_r - gm_i), the column side
// exp(gm_j - g_s), and a cross-block factor exp(gm_i - gm_j) <= 1 is folded
// into the column fragment.  All factors stay within fp16 unless eight
// consecutive tokens decay a channel by more than 2^14; such a chunk is
// detected and run as the exact fp32 token recurrence instead.
#include "common.h"
#include "kernels.h"

namespace gdn2 {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;          // chunk length
constexpr int D = 128;         // dk = dv
constexpr int NTH = 256;       // 4 waves
constexpr int KP = D + 8;      // pitch (halves) of [token][channel] operands
constexpr int SP = C + 8;      // pitch (halves) of [row][token] operands
constexpr int AP = C + 4;      // pitch (floats) of the fp32 C x C matrix
constexpr float LOG2E = 1.4426950408889634f;
constexpr float MAX_EXP2 = 14.f;      // largest |log2 factor| on the fast path
constexpr float MAX_OPERAND = 16384.f;  // largest |fp16 operand| on the fast path

// Lower-triangular 16x16 tiles of a 64x64 chunk matrix, (block row, block col).
__constant__ int kTileI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kTileJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <int VT>
struct Smem {
    _Float16 kh[C * KP];   // row-side Gram operand k*2^(g-gm); later Kbar
    _Float16 qh[C * KP];   // q*2^(g-gm); later Qbar
    _Float16 eh[C * KP];   // column-side e*2^(gm-g)
    _Float16 uh[C * KP];   // u*2^(gm-g)
    _Float16 v16[VT * SP]; // values, [v][s]
    _Float16 s16[VT * KP]; // state, [v][c]
    union {
        float af[C * AP];        // A (strict lower), inverted in place into Tm
        _Float16 xm16[VT * SP];  // X, then -M, [v][s]
    };
    _Float16 t16[C * SP];  // Tm  [r][s]
    _Float16 b16[C * SP];  // Bm
    _Float16 r16[C * SP];  // R
    _Float16 p16[C * SP];  // P
    union {
        float segtot[8][D];      // per 8-row segment log2-decay totals
        float wtmp[3][16][16];   // solve scratch
        float tok[6][D];         // token vectors of the exact fallback
    };
    float gm[4][D];   // block reference: log2 cumulative decay at row 16i+7
    float egm[4][D];  // 2^gm
    float fsc[4][D];  // 2^(g_C - gm)
    float gce[D];     // 2^g_C
    float red[2][4][VT];
    int wide;
};

struct Raw {
    uint2 k[8], q[8];  // 4 bf16 channels of 8 rows
    f4 la[8], eb[8], wr[8];
    uint4 v[2];        // 8 bf16 values per piece
};

__device__ __forceinline__ f4 bf16x4_to_f4(uint2 p) {
    f4 r;
    r[0] = __uint_as_float(p.x << 16);
    r[1] = __uint_as_float(p.x & 0xffff0000u);
    r[2] = __uint_as_float(p.y << 16);
    r[3] = __uint_as_float(p.y & 0xffff0000u);
    return r;
}

__device__ __forceinline__ f4 splat(float x) { return f4{x, x, x, x}; }

__device__ __forceinline__ h4 to_h4(f4 x) {
    return h4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}

__device__ __forceinline__ f4 mfma32(h8 a, h8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma16(h4 a, h4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Raw inputs of one chunk: thread (seg, cq) owns rows 8seg..8seg+7 and key
// channels 4cq..4cq+3; the value slice is split in 16-byte pieces.
template <int VT>
__device__ __forceinline__ void load_raw(Raw &R, const ChunkArgs &a, int64_t b, int64_t h,
                                         int64_t t0, int col0, int seg, int cq, int tid) {
    const uint16_t *kp = static_cast<const uint16_t *>(a.k);
    const uint16_t *qp = static_cast<const uint16_t *>(a.q);
    const uint16_t *vp = static_cast<const uint16_t *>(a.v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t t = t0 + seg * 8 + i;
        if (t < a.T) {
            const int64_t row = (b * a.T + t) * a.H + h;
            R.k[i] = *reinterpret_cast<const uint2 *>(kp + row * D + 4 * cq);
            R.q[i] = *reinterpret_cast<const uint2 *>(qp + row * D + 4 * cq);
            R.la[i] = a.la_key ? *reinterpret_cast<const f4 *>(a.la + row * D + 4 * cq) : splat(a.la[row]);
            R.eb[i] = a.eb_key ? *reinterpret_cast<const f4 *>(a.eb + row * D + 4 * cq) : splat(a.eb[row]);
            if (a.wr)
                R.wr[i] = a.wr_key ? *reinterpret_cast<const f4 *>(a.wr + row * D + 4 * cq) : splat(a.wr[row]);
            else
                R.wr[i] = R.eb[i];
        } else {
            R.k[i] = make_uint2(0, 0);
            R.q[i] = make_uint2(0, 0);
            R.la[i] = splat(0.f);
            R.eb[i] = splat(0.f);
            R.wr[i] = splat(0.f);
        }
    }
    constexpr int PPR = VT / 8;           // pieces per token row
    constexpr int NP = C * PPR;           // pieces per chunk
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int p = tid + NTH * n;
        R.v[n] = make_uint4(0, 0, 0, 0);
        if (p < NP) {
            const int s = p / PPR, piece = p % PPR;
            const int64_t t = t0 + s;
            if (t < a.T)
                R.v[n] = *reinterpret_cast<const uint4 *>(vp + ((b * a.T + t) * a.H + h) * D + col0 + 8 * piece);
        }
    }
}

template <int VT, bool TIED>
__global__ void __launch_bounds__(NTH, 1) chunk_mfma_kernel(ChunkArgs a, int nt, int xcd_map) {
    __shared__ Smem<VT> S;
    constexpr int NCT = VT / 16;  // value column tiles

    // Tiles of one chain share their key/gate reads; keep them on one XCD
    // (workgroups are dealt to the 8 XCDs round-robin).
    const int L = blockIdx.x;
    int chain, tile;
    if (xcd_map) {
        tile = (L / 8) % nt;
        chain = (L / (8 * nt)) * 8 + (L % 8);
    } else {
        tile = L % nt;
        chain = L / nt;
    }
    const int64_t b = chain / a.H, h = chain % a.H;
    const int col0 = tile * VT;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int seg = tid >> 5, cq = tid & 31;
    const int64_t sbase = (b * a.H + h) * static_cast<int64_t>(D) * D;

    // zero the upper blocks of the C x C operands once; they are never written
    for (int idx = tid; idx < C * SP; idx += NTH) {
        S.t16[idx] = (_Float16)0.f;
        S.b16[idx] = (_Float16)0.f;
        S.r16[idx] = (_Float16)0.f;
        S.p16[idx] = (_Float16)0.f;
    }
    if (tid == 0) S.wide = 0;

    // state slice: wave wv owns key rows 32wv..32wv+31
    f4 sacc[2][NCT];
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * (2 * wv + r2) + 4 * lg + e;
                const int v = col0 + 16 * ct + lr;
                sacc[r2][ct][e] = a.s0 ? a.s0[sbase + static_cast<int64_t>(c) * D + v] : 0.f;
            }

    Raw R;
    load_raw<VT>(R, a, b, h, 0, col0, seg, cq, tid);

    for (int64_t t0 = 0; t0 < a.T; t0 += C) {
        __syncthreads();  // (0) previous chunk done with every buffer
        // ---- state (fp16 copy) for this chunk's products ----------------
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                *reinterpret_cast<h4 *>(&S.s16[(16 * ct + lr) * KP + 16 * (2 * wv + r2) + 4 * lg]) =
                    to_h4(sacc[r2][ct]);

        // ---- prep 1: cumulative log2-decay inside my 8-row segment ---------
        f4 g[8];
        {
            f4 run = splat(0.f);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                run += R.la[i] * LOG2E;
                g[i] = run;
            }
            *reinterpret_cast<f4 *>(&S.segtot[seg][4 * cq]) = run;
        }
        // values: bf16 -> fp16, stored transposed [v][s]
        {
            constexpr int PPR = VT / 8, NP = C * PPR;
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int p = tid + NTH * n;
                if (p < NP) {
                    const int s = p / PPR, piece = p % PPR;
                    const uint32_t w4[4] = {R.v[n].x, R.v[n].y, R.v[n].z, R.v[n].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        S.v16[(8 * piece + 2 * e) * SP + s] = (_Float16)__uint_as_float(w4[e] << 16);
                        S.v16[(8 * piece + 2 * e + 1) * SP + s] = (_Float16)__uint_as_float(w4[e] & 0xffff0000u);
                    }
                }
            }
        }
        __syncthreads();  // (1) segment totals visible

        // ---- prep 2: block references, factored operands ------------------
        f4 khf[8], qhf[8];
        {
            f4 base = splat(0.f), gmv = splat(0.f);
            const int blk = seg >> 1;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const f4 st = *reinterpret_cast<const f4 *>(&S.segtot[s][4 * cq]);
                if (s < seg) base += st;
                if (s <= 2 * blk) gmv += st;
            }
            if (tid < D) {
                const int c = tid;
                float cum = 0.f;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    cum += S.segtot[s][c];
                    if ((s & 1) == 0) S.gm[s >> 1][c] = cum;
                }
                S.gce[c] = __builtin_amdgcn_exp2f(cum);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float gmj = 0.f;
                    for (int s = 0; s <= 2 * j; ++s) gmj += S.segtot[s][c];
                    S.egm[j][c] = __builtin_amdgcn_exp2f(gmj);
                    S.fsc[j][c] = __builtin_amdgcn_exp2f(cum - gmj);
                }
            }
            const float qs = a.q_scale;
            bool bad = false;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                g[i] += base;
                const f4 x = g[i] - gmv;
                f4 e1, e2;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bad |= !(fabsf(x[j]) <= MAX_EXP2);
                    e1[j] = __builtin_amdgcn_exp2f(x[j]);
                    e2[j] = __builtin_amdgcn_exp2f(-x[j]);
                }
                const f4 kf = bf16x4_to_f4(R.k[i]);
                const f4 qf = bf16x4_to_f4(R.q[i]) * qs;
                khf[i] = kf * e1;
                qhf[i] = qf * e1;
                const f4 ev = R.eb[i] * kf * e2;
                const f4 uv = R.wr[i] * kf * e2;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float m = fmaxf(fmaxf(fabsf(khf[i][j]), fabsf(qhf[i][j])),
                                          fmaxf(fabsf(ev[j]), fabsf(uv[j])));
                    bad |= !(m <= MAX_OPERAND);
                }
                const int r = 8 * seg + i;
                *reinterpret_cast<h4 *>(&S.kh[r * KP + 4 * cq]) = to_h4(khf[i]);
                *reinterpret_cast<h4 *>(&S.qh[r * KP + 4 * cq]) = to_h4(qhf[i]);
                *reinterpret_cast<h4 *>(&S.eh[r * KP + 4 * cq]) = to_h4(ev);
                if (!TIED) *reinterpret_cast<h4 *>(&S.uh[r * KP + 4 * cq]) = to_h4(uv);
            }
            if (bad) S.wide = 1;
        }
        // prefetch the next chunk while this one is computed
        if (t0 + C < a.T) load_raw<VT>(R, a, b, h, t0 + C, col0, seg, cq, tid);
        __syncthreads();  // (2) operands, tables, wide flag visible

        const bool wide = S.wide != 0;
        if (!wide) {
            // ---- Grams: 10 lower 16x16 tiles, 4 products each ------------
            for (int ti = wv; ti < 10; ti += 4) {
                const int i = kTileI[ti], j = kTileJ[ti];
                f4 aA = splat(0.f), aB = splat(0.f), aR = splat(0.f), aP = splat(0.f);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int cb = 32 * ks + 8 * lg;
                    const h8 xk = *reinterpret_cast<const h8 *>(&S.kh[(16 * i + lr) * KP + cb]);
                    const h8 xq = *reinterpret_cast<const h8 *>(&S.qh[(16 * i + lr) * KP + cb]);
                    h8 ye = *reinterpret_cast<const h8 *>(&S.eh[(16 * j + lr) * KP + cb]);
                    h8 yu = TIED ? ye : *reinterpret_cast<const h8 *>(&S.uh[(16 * j + lr) * KP + cb]);
                    if (i != j) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float dd = __builtin_amdgcn_exp2f(S.gm[i][cb + e] - S.gm[j][cb + e]);
                            ye[e] = (_Float16)((float)ye[e] * dd);
                            if (!TIED) yu[e] = (_Float16)((float)yu[e] * dd);
                        }
                    }
                    aA = mfma32(xk, ye, aA);
                    aR = mfma32(xq, ye, aR);
                    if (!TIED) {
                        aB = mfma32(xk, yu, aB);
                        aP = mfma32(xq, yu, aP);
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * i + 4 * lg + e, s = 16 * j + lr;
                    const bool strict = r > s, incl = r >= s;
                    S.af[r * AP + s] = strict ? aA[e] : 0.f;
                    S.b16[r * SP + s] = (_Float16)(strict ? (TIED ? aA[e] : aB[e]) : 0.f);
                    S.r16[r * SP + s] = (_Float16)(incl ? aR[e] : 0.f);
                    if (!TIED) S.p16[r * SP + s] = (_Float16)(incl ? aP[e] : 0.f);
                }
            }
        }
        __syncthreads();  // (3) Grams done, operands free
        if (tid == 0) S.wide = 0;

        if (!wide) {
            // ---- state-side operands Kbar = k 2^g, Qbar = q 2^g ----------
            {
                const int blk = seg >> 1;
                const f4 eg = *reinterpret_cast<const f4 *>(&S.egm[blk][4 * cq]);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 8 * seg + i;
                    *reinterpret_cast<h4 *>(&S.kh[r * KP + 4 * cq]) = to_h4(khf[i] * eg);
                    *reinterpret_cast<h4 *>(&S.qh[r * KP + 4 * cq]) = to_h4(qhf[i] * eg);
                }
            }
            // ---- solve: diagonal 16x16 blocks of (I + A)^-1, one per wave
            if (lane < 16) {
                const int i = wv, j = lane;
                float col[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) col[r] = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int r = 1; r < 16; ++r) {
                    float t = 0.f;
#pragma unroll
                    for (int s = 0; s < r; ++s) t += S.af[(16 * i + r) * AP + 16 * i + s] * col[s];
                    if (r > j) col[r] = -t;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) S.af[(16 * i + r) * AP + 16 * i + j] = col[r];
            }
            __syncthreads();
            // off-diagonal blocks, block row by block row, in place:
            //   Tm_ij = -Tm_ii * sum_{k=j}^{i-1} A_ik Tm_kj
            for (int i = 1; i < 4; ++i) {
                for (int idx = tid; idx < i * 256; idx += NTH) {
                    const int j = idx >> 8, rr = (idx >> 4) & 15, cc = idx & 15;
                    float acc = 0.f;
                    for (int k = j; k < i; ++k)
#pragma unroll
                        for (int m = 0; m < 16; ++m)
                            acc += S.af[(16 * i + rr) * AP + 16 * k + m] * S.af[(16 * k + m) * AP + 16 * j + cc];
                    S.wtmp[j][rr][cc] = acc;
                }
                __syncthreads();
                for (int idx = tid; idx < i * 256; idx += NTH) {
                    const int j = idx >> 8, rr = (idx >> 4) & 15, cc = idx & 15;
                    float acc = 0.f;
#pragma unroll
                    for (int m = 0; m < 16; ++m) acc += S.af[(16 * i + rr) * AP + 16 * i + m] * S.wtmp[j][m][cc];
                    S.af[(16 * i + rr) * AP + 16 * j + cc] = -acc;
                }
                __syncthreads();
            }
            for (int idx = tid; idx < C * C; idx += NTH) {
                const int r = idx >> 6, s = idx & 63;
                if ((s >> 4) <= (r >> 4)) S.t16[r * SP + s] = (_Float16)S.af[r * AP + s];
            }
            __syncthreads();  // (4) Tm ready; af region free for X / -M

            // ---- X = Kbar S + Bm V   (wave wv: rows 16wv..16wv+15) -------
            f4 acc[NCT];
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f4 x = splat(0.f);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int cb = 32 * ks + 8 * lg;
                    x = mfma32(*reinterpret_cast<const h8 *>(&S.kh[(16 * wv + lr) * KP + cb]),
                               *reinterpret_cast<const h8 *>(&S.s16[(16 * ct + lr) * KP + cb]), x);
                }
                for (int ks = 0; ks <= (wv >> 1); ++ks) {
                    const int sb = 32 * ks + 8 * lg;
                    x = mfma32(*reinterpret_cast<const h8 *>(&S.b16[(16 * wv + lr) * SP + sb]),
                               *reinterpret_cast<const h8 *>(&S.v16[(16 * ct + lr) * SP + sb]), x);
                }
                acc[ct] = x;
            }
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                *reinterpret_cast<h4 *>(&S.xm16[(16 * ct + lr) * SP + 16 * wv + 4 * lg]) = to_h4(acc[ct]);
            __syncthreads();

            // ---- M = Tm X ------------------------------------------------
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f4 x = splat(0.f);
                for (int ks = 0; ks <= (wv >> 1); ++ks) {
                    const int sb = 32 * ks + 8 * lg;
                    x = mfma32(*reinterpret_cast<const h8 *>(&S.t16[(16 * wv + lr) * SP + sb]),
                               *reinterpret_cast<const h8 *>(&S.xm16[(16 * ct + lr) * SP + sb]), x);
                }
                acc[ct] = x;
            }
            __syncthreads();
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
                *reinterpret_cast<h4 *>(&S.xm16[(16 * ct + lr) * SP + 16 * wv + 4 * lg]) = to_h4(-acc[ct]);
            __syncthreads();

            // ---- O = Qbar S + P V + R (-M) -> HBM --------------------------
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f4 x = splat(0.f);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int cb = 32 * ks + 8 * lg;
                    x = mfma32(*reinterpret_cast<const h8 *>(&S.qh[(16 * wv + lr) * KP + cb]),
                               *reinterpret_cast<const h8 *>(&S.s16[(16 * ct + lr) * KP + cb]), x);
                }
                for (int ks = 0; ks <= (wv >> 1); ++ks) {
                    const int sb = 32 * ks + 8 * lg;
                    const _Float16 *pp = TIED ? S.r16 : S.p16;
                    x = mfma32(*reinterpret_cast<const h8 *>(&pp[(16 * wv + lr) * SP + sb]),
                               *reinterpret_cast<const h8 *>(&S.v16[(16 * ct + lr) * SP + sb]), x);
                    x = mfma32(*reinterpret_cast<const h8 *>(&S.r16[(16 * wv + lr) * SP + sb]),
                               *reinterpret_cast<const h8 *>(&S.xm16[(16 * ct + lr) * SP + sb]), x);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * wv + 4 * lg + e;
                    const int64_t t = t0 + r;
                    if (t < a.T) a.o[((b * a.T + t) * a.H + h) * D + col0 + 16 * ct + lr] = x[e];
                }
            }

            // ---- S <- 2^gC S + sum_j 2^(gC-gm_j) (Uh_j^T V_j + Eh_j^T (-M)_j)
            const _Float16 *up = TIED ? S.eh : S.uh;
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int rt = 2 * wv + r2;
                f4 gam;
#pragma unroll
                for (int e = 0; e < 4; ++e) gam[e] = S.gce[16 * rt + 4 * lg + e];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) sacc[r2][ct] *= gam;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    h4 au, ae;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 16 * j + 4 * lg + e;
                        au[e] = up[s * KP + 16 * rt + lr];
                        ae[e] = S.eh[s * KP + 16 * rt + lr];
                    }
                    f4 fs;
#pragma unroll
                    for (int e = 0; e < 4; ++e) fs[e] = S.fsc[j][16 * rt + 4 * lg + e];
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const int vb = (16 * ct + lr) * SP + 16 * j + 4 * lg;
                        f4 y = splat(0.f);
                        y = mfma16(au, *reinterpret_cast<const h4 *>(&S.v16[vb]), y);
                        y = mfma16(ae, *reinterpret_cast<const h4 *>(&S.xm16[vb]), y);
                        sacc[r2][ct] += fs * y;
                    }
                }
            }
        } else {
            // ---- exact fallback: the fp32 token recurrence on this slice ----
            const uint16_t *kp = static_cast<const uint16_t *>(a.k);
            const uint16_t *qp = static_cast<const uint16_t *>(a.q);
            const uint16_t *vp = static_cast<const uint16_t *>(a.v);
            for (int r = 0; r < C && t0 + r < a.T; ++r) {
                const int64_t row = (b * a.T + t0 + r) * a.H + h;
                if (tid < D) {
                    const int c = tid;
                    const float kv = bf16_to_f32(kp[row * D + c]);
                    const float bb = load_gate(a.eb, a.eb_key, row, D, c);
                    const float ww = a.wr ? load_gate(a.wr, a.wr_key, row, D, c) : bb;
                    S.tok[0][c] = expf(load_gate(a.la, a.la_key, row, D, c));
                    S.tok[1][c] = kv;
                    S.tok[2][c] = bb * kv;
                    S.tok[3][c] = ww * kv;
                    S.tok[4][c] = a.q_scale * bf16_to_f32(qp[row * D + c]);
                } else if (tid < D + VT) {
                    S.tok[5][tid - D] = bf16_to_f32(vp[row * D + col0 + tid - D]);
                }
                __syncthreads();
                // decay, then partial key reads over my rows
                float pmv[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) pmv[ct] = 0.f;
#pragma unroll
                for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 16 * (2 * wv + r2) + 4 * lg + e;
                        const float ac = S.tok[0][c], kc = S.tok[1][c];
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) {
                            sacc[r2][ct][e] *= ac;
                            pmv[ct] += kc * sacc[r2][ct][e];
                        }
                    }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    float x = pmv[ct];
                    x += __shfl_xor(x, 16);
                    x += __shfl_xor(x, 32);
                    if (lg == 0) S.red[0][wv][16 * ct + lr] = x;
                }
                __syncthreads();
                float mv[NCT], vv[NCT], pov[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const int v = 16 * ct + lr;
                    mv[ct] = S.red[0][0][v] + S.red[0][1][v] + S.red[0][2][v] + S.red[0][3][v];
                    vv[ct] = S.tok[5][v];
                    pov[ct] = 0.f;
                }
#pragma unroll
                for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 16 * (2 * wv + r2) + 4 * lg + e;
                        const float ec = S.tok[2][c], uc = S.tok[3][c], qc = S.tok[4][c];
#pragma unroll
                        for (int ct = 0; ct < NCT; ++ct) {
                            sacc[r2][ct][e] = sacc[r2][ct][e] - ec * mv[ct] + uc * vv[ct];
                            pov[ct] += qc * sacc[r2][ct][e];
                        }
                    }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    float x = pov[ct];
                    x += __shfl_xor(x, 16);
                    x += __shfl_xor(x, 32);
                    if (lg == 0) S.red[1][wv][16 * ct + lr] = x;
                }
                __syncthreads();
                if (tid < VT) {
                    const int v = tid;
                    a.o[row * D + col0 + v] = S.red[1][0][v] + S.red[1][1][v] + S.red[1][2][v] + S.red[1][3][v];
                }
                __syncthreads();  // tok and red reused by the next token
            }
        }
    }

    if (a.s_out) {
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 16 * (2 * wv + r2) + 4 * lg + e;
                    const int v = col0 + 16 * ct + lr;
                    a.s_out[sbase + static_cast<int64_t>(c) * D + v] = sacc[r2][ct][e];
                }
    }
}

template <int VT, bool TIED>
hipError_t launch_vt(const ChunkArgs &a, hipStream_t s) {
    const int nt = D / VT;
    const int64_t chains = a.B * a.H;
    const int xcd_map = (chains % 8 == 0) ? 1 : 0;
    const dim3 grid(static_cast<unsigned>(chains * nt));
    hipLaunchKernelGGL((chunk_mfma_kernel<VT, TIED>), grid, dim3(NTH), 0, s, a, nt, xcd_map);
    return hipGetLastError();
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs &a) {
    return a.bf16 && a.dk == D && a.dv == D && a.C == C;
}

hipError_t launch_chunk_mfma(const ChunkArgs &a, hipStream_t s) {
    // Value slices per chain: enough workgroups to give every CU one.
    const int64_t chains = a.B * a.H;
    const bool tied = a.wr == nullptr;
    int vt = 64;
    if (chains * 2 < 256) vt = 32;
    if (chains * 4 < 256) vt = 16;
    if (vt == 64) return tied ? launch_vt<64, true>(a, s) : launch_vt<64, false>(a, s);
    if (vt == 32) return tied ? launch_vt<32, true>(a, s) : launch_vt<32, false>(a, s);
    return tied ? launch_vt<16, true>(a, s) : launch_vt<16, false>(a, s);
}

}  // namespace gdn2
