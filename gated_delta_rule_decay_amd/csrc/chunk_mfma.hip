// chunk_mfma.hip -- chunkwise GDN-2 forward on the gfx950 matrix cores.
//
// Covers bf16 q/k/v with dk = dv = 128 and chunk C = 64, every gate of one
// kind (all per key channel or all per head), tied or untied write gate.
// One workgroup of 512 lanes (8 waves, two per SIMD) owns one (batch, head)
// chain and a VT-wide slice of the value channels, and walks the chunks of
// the sequence in order; the fp32 state slice (128 x VT) lives in MFMA
// accumulators for the whole sequence, so the state never leaves the CU.
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
// Numerics.  The matrix products run on v_mfma with fp16 operands and fp32
// accumulation; the state, the solve (fp32 MFMA) and all gate arithmetic
// stay fp32.  fp16 (11-bit significand) rather than bf16 (8-bit) because one
// bf16 rounding of the derived operands alone costs ~2.9e-3 relative error,
// above the 2e-3 budget, while fp16 costs ~3.6e-4.  fp16's narrow exponent
// range is handled by factoring exp(g_r - g_s) around a reference inside each
// 16-token block: the row side carries exp(g_r - gm_i), the column side
// exp(gm_j - g_s), and a cross-block factor exp(gm_i - gm_j) <= 1 is folded
// into the column fragment.  The factors stay within fp16 unless about eight
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
constexpr int NTH = 512;       // 8 waves
constexpr int NW = NTH / 64;
constexpr int NSEG = NTH / 32; // 4-row segments of the chunk (16)
constexpr int RPS = C / NSEG;  // rows per segment (4)
constexpr int KP = D + 4;      // pitch (halves) of [token][channel] operands
constexpr int SP = C + 8;      // pitch (halves) of [row][token] operands
constexpr int AP = C + 4;      // pitch (floats) of the fp32 C x C matrix
constexpr float LOG2E = 1.4426950408889634f;
constexpr float MAX_EXP2 = 14.f;        // largest |log2 factor| on the fast path
constexpr float MAX_OPERAND = 16384.f;  // largest |fp16 operand| on the fast path

// (block row, block col) of the strictly-lower 16x16 tiles of a 64x64 chunk
// matrix, and the index of each such pair in the cross-block factor table.
__constant__ int kOffI[6] = {1, 2, 2, 3, 3, 3};
__constant__ int kOffJ[6] = {0, 0, 1, 0, 1, 2};
__constant__ int kPair[4][4] = {{-1, -1, -1, -1}, {0, -1, -1, -1}, {1, 2, -1, -1}, {3, 4, 5, -1}};

template <int VT>
struct Smem {
    _Float16 kh[C * KP];   // row-side Gram operand k*2^(g-gm); later Kbar
    _Float16 qh[C * KP];   // q*2^(g-gm); later Qbar
    _Float16 eh[C * KP];   // column-side e*2^(gm-g)
    _Float16 uh[C * KP];   // u*2^(gm-g)
    _Float16 v16[VT * SP]; // values, [v][s]
    _Float16 s16[VT * KP]; // state, [v][c]
    union {
        float af[C * AP];         // A (strict lower), then Tm in place (fp32)
        _Float16 xm16[VT * SP];   // X, then -M, [v][s]
        float segtot[NSEG][D];    // per-segment log2-decay totals
        struct {
            float tok[6][D];      // token vectors of the exact fallback
            float red[2][NW][VT]; // its cross-wave reductions
        } fb;
    };
    _Float16 t16[C * SP];  // Tm  [r][s]
    _Float16 b16[C * SP];  // Bm
    _Float16 r16[C * SP];  // R
    _Float16 p16[C * SP];  // P
    union {
        float dtab[6][D];        // 2^(gm_i - gm_j), i > j (Gram phase)
        float scr[8][16 * 16];   // solve scratch (after the Grams)
    };
    float fsc[4][D];         // 2^(g_C - gm_j)
    float gce[D];            // 2^g_C
    int wide;
};

// Raw inputs of one chunk held in registers: thread (seg, cq) owns rows
// RPS*seg.. and key channels 4cq..4cq+3; gates are 4 values per row when
// they are per key channel (KEYG) and one value per row when per head.
template <bool KEYG>
struct GateRow;
template <>
struct GateRow<true> {
    f4 x[RPS];
};
template <>
struct GateRow<false> {
    float x[RPS];
};

template <bool KEYG>
struct Raw {
    uint2 k[RPS], q[RPS];
    GateRow<KEYG> la, eb, wr;
    uint4 v;  // 8 bf16 values
};

__device__ __forceinline__ f4 gate4(const GateRow<true> &g, int i) { return g.x[i]; }
__device__ __forceinline__ f4 gate4(const GateRow<false> &g, int i) {
    return f4{g.x[i], g.x[i], g.x[i], g.x[i]};
}

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

// 16x16x16 product of fp32 blocks held in LDS (row pitches xp, yp), on the
// fp32 matrix unit: acc += X * Y.  Lane l reads X[l%16][4kk + l/16] and
// Y[4kk + l/16][l%16].
__device__ __forceinline__ f4 mfma_f32_block(const float *X, int xp, const float *Y, int yp, f4 acc,
                                             int lr, int lg) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[lr * xp + 4 * kk + lg], Y[(4 * kk + lg) * yp + lr],
                                                  acc, 0, 0, 0);
    return acc;
}

// In-place inverse of a unit-lower-triangular 16x16 block I + N held (N
// strictly lower, zero diagonal) in LDS at `na` with row pitch AP:
// (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) since N^16 = 0.  One wave;
// `sa`, `sb` are two private 16x16 fp32 scratch blocks.  The result is written
// back to `na` (fp32) and to `th` (fp16, row pitch SP).
__device__ __forceinline__ void invert_unit_lower16(float *na, _Float16 *th, float *sa, float *sb, int lr,
                                                    int lg) {
    f4 nn, eye;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        nn[e] = na[(4 * lg + e) * AP + lr];
        eye[e] = (4 * lg + e == lr) ? 1.f : 0.f;
    }
    // a wave's LDS writes are seen by its later reads, so no barrier is needed
    const f4 n2 = mfma_f32_block(na, AP, na, AP, splat(0.f), lr, lg);
#pragma unroll
    for (int e = 0; e < 4; ++e) sa[(4 * lg + e) * 16 + lr] = n2[e];
    const f4 n3 = mfma_f32_block(na, AP, sa, 16, splat(0.f), lr, lg);
    const f4 t1 = eye - nn + n2 - n3;  // (I - N)(I + N^2)
    const f4 n4 = mfma_f32_block(sa, 16, sa, 16, splat(0.f), lr, lg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        sb[(4 * lg + e) * 16 + lr] = t1[e];
        sa[(4 * lg + e) * 16 + lr] = n4[e];
    }
    const f4 t2 = mfma_f32_block(sb, 16, sa, 16, t1, lr, lg);  // T1 (I + N^4)
    const f4 n8 = mfma_f32_block(sa, 16, sa, 16, splat(0.f), lr, lg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        sb[(4 * lg + e) * 16 + lr] = t2[e];
        sa[(4 * lg + e) * 16 + lr] = n8[e];
    }
    const f4 t3 = mfma_f32_block(sb, 16, sa, 16, t2, lr, lg);  // T2 (I + N^8)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        na[(4 * lg + e) * AP + lr] = t3[e];
        th[(4 * lg + e) * SP + lr] = (_Float16)t3[e];
    }
}

// Buffer descriptor over the rows t0..t0+C-1 of one (batch, head) chain of a
// [B,T,H,width] tensor: rows at or past T fall outside num_records, so the
// hardware returns zeros for them and the loads need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chain_rsrc(const void *base, const ChunkArgs &a,
                                                            int64_t b, int64_t h, int64_t t0,
                                                            int width, int esize, int col0) {
    const int64_t nvalid = a.T - t0 < C ? (a.T - t0 > 0 ? a.T - t0 : 0) : C;
    const char *p = static_cast<const char *>(base) +
                    (((b * a.T + t0) * a.H + h) * width + col0) * static_cast<int64_t>(esize);
    const int64_t bytes = nvalid > 0 ? ((nvalid - 1) * a.H * width + width - col0) * esize : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), (short)0, static_cast<int>(bytes),
                                             0x00020000);
}

// Issue every load of one chunk (no waits: the values are first used by the
// next chunk's prep).
template <int VT, bool TIED, bool KEYG>
__device__ __forceinline__ void load_raw(Raw<KEYG> &R, const ChunkArgs &a, int64_t b, int64_t h,
                                         int64_t t0, int col0, int seg, int cq, int tid) {
    const auto rk = chain_rsrc(a.k, a, b, h, t0, D, 2, 0);
    const auto rq = chain_rsrc(a.q, a, b, h, t0, D, 2, 0);
    const auto rv = chain_rsrc(a.v, a, b, h, t0, D, 2, col0);
    const int gw = KEYG ? D : 1;
    const auto rla = chain_rsrc(a.la, a, b, h, t0, gw, 4, 0);
    const auto reb = chain_rsrc(a.eb, a, b, h, t0, gw, 4, 0);
    const auto rwr = chain_rsrc(TIED ? a.eb : a.wr, a, b, h, t0, gw, 4, 0);
    const int rowk = static_cast<int>(a.H) * D;  // elements between consecutive tokens
    const int rowg = static_cast<int>(a.H) * gw;
#pragma unroll
    for (int i = 0; i < RPS; ++i) {
        const int r = seg * RPS + i;
        const int ok = (r * rowk + 4 * cq) * 2;
        R.k[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, ok, 0, 0));
        R.q[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, ok, 0, 0));
        if constexpr (KEYG) {
            const int og = (r * rowg + 4 * cq) * 4;
            R.la.x[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rla, og, 0, 0));
            R.eb.x[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(reb, og, 0, 0));
            if (!TIED) R.wr.x[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rwr, og, 0, 0));
        } else {
            const int og = r * rowg * 4;
            R.la.x[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rla, og, 0, 0));
            R.eb.x[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(reb, og, 0, 0));
            if (!TIED) R.wr.x[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rwr, og, 0, 0));
        }
    }
    constexpr int PPR = VT / 8;  // 16-byte pieces per token row
    if (tid < C * PPR) {
        const int s = tid / PPR, piece = tid % PPR;
        R.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, (s * rowk + 8 * piece) * 2, 0, 0));
    }
}

template <int VT, bool TIED, bool KEYG>
__global__ void __launch_bounds__(NTH) chunk_mfma_kernel(ChunkArgs a, int nt, int xcd_map) {
    __shared__ Smem<VT> S;
    constexpr int NCT = VT / 16;       // value column tiles
    constexpr int NCTW = NCT >= 2 ? NCT / 2 : 1;  // value tiles per wave in X, M, O
    constexpr int PPR = VT / 8;

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
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane0 = tid & 63;
    const int64_t sbase = (b * a.H + h) * static_cast<int64_t>(D) * D;

    // zero the upper blocks of the C x C operands once; they are never written
    for (int idx = tid; idx < C * SP; idx += NTH) {
        S.t16[idx] = (_Float16)0.f;
        S.b16[idx] = (_Float16)0.f;
        S.r16[idx] = (_Float16)0.f;
        S.p16[idx] = (_Float16)0.f;
    }
    if (tid == 0) S.wide = 0;

    // state slice: wave wv owns key rows 16wv..16wv+15, every value tile
    f4 sacc[NCT];
    {
    const int lr = lane0 & 15, lg = lane0 >> 4;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = 16 * wv + 4 * lg + e;
            const int v = col0 + 16 * ct + lr;
            sacc[ct][e] = a.s0 ? a.s0[sbase + static_cast<int64_t>(c) * D + v] : 0.f;
        }
    }

    Raw<KEYG> R;
    load_raw<VT, TIED, KEYG>(R, a, b, h, 0, col0, tid >> 5, tid & 31, tid);

    for (int64_t t0 = 0; t0 < a.T; t0 += C) {
        __syncthreads();  // previous chunk done with every buffer
        // lane coordinates, re-derived every chunk so that the many LDS
        // addresses built from them are not hoisted out of the loop (they
        // would stay live across it and spill)
        int tl = tid;
        asm volatile("" : "+v"(tl));
        const int lane = tl & 63, lr = lane & 15, lg = lane >> 4;
        const int seg = tl >> 5, cq = tl & 31;

        // ---- prep 1: fp16 state copy, values, segment log2-decay totals ----
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
            *reinterpret_cast<h4 *>(&S.s16[(16 * ct + lr) * KP + 16 * wv + 4 * lg]) = to_h4(sacc[ct]);
        if (tid < C * PPR) {
            const int s = tid / PPR, piece = tid % PPR;
            const uint32_t w4[4] = {R.v.x, R.v.y, R.v.z, R.v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S.v16[(8 * piece + 2 * e) * SP + s] = (_Float16)__uint_as_float(w4[e] << 16);
                S.v16[(8 * piece + 2 * e + 1) * SP + s] = (_Float16)__uint_as_float(w4[e] & 0xffff0000u);
            }
        }
        f4 g[RPS];
        {
            f4 run = splat(0.f);
#pragma unroll
            for (int i = 0; i < RPS; ++i) {
                run += gate4(R.la, i) * LOG2E;
                g[i] = run;
            }
            *reinterpret_cast<f4 *>(&S.segtot[seg][4 * cq]) = run;
        }
        __syncthreads();
        // exclusive prefix of the segment totals, in place, one lane per key
        // channel; the same lanes fill the per-chunk factor tables
        if (tid < D) {
            const int c = tid;
            float gmc[4], cum = 0.f;
#pragma unroll
            for (int s = 0; s < NSEG; ++s) {
                const float st = S.segtot[s][c];
                S.segtot[s][c] = cum;
                cum += st;
                if ((s & 3) == 1) gmc[s >> 2] = cum;  // block reference: after row 16j+7
            }
            S.gce[c] = __builtin_amdgcn_exp2f(cum);
#pragma unroll
            for (int j = 0; j < 4; ++j) S.fsc[j][c] = __builtin_amdgcn_exp2f(cum - gmc[j]);
            S.dtab[0][c] = __builtin_amdgcn_exp2f(gmc[1] - gmc[0]);
            S.dtab[1][c] = __builtin_amdgcn_exp2f(gmc[2] - gmc[0]);
            S.dtab[2][c] = __builtin_amdgcn_exp2f(gmc[2] - gmc[1]);
            S.dtab[3][c] = __builtin_amdgcn_exp2f(gmc[3] - gmc[0]);
            S.dtab[4][c] = __builtin_amdgcn_exp2f(gmc[3] - gmc[1]);
            S.dtab[5][c] = __builtin_amdgcn_exp2f(gmc[3] - gmc[2]);
        }
        __syncthreads();

        // ---- prep 2: factored fp16 operands ----------------------------------
        f4 khf[RPS], qhf[RPS], egm;
        {
            const int blk = seg / 4;  // 16-row block of my rows
            const f4 base = *reinterpret_cast<const f4 *>(&S.segtot[seg][4 * cq]);
            const f4 gmv = *reinterpret_cast<const f4 *>(&S.segtot[4 * blk + 2][4 * cq]);
#pragma unroll
            for (int j = 0; j < 4; ++j) egm[j] = __builtin_amdgcn_exp2f(gmv[j]);
            const float qs = a.q_scale;
            bool bad = false;
#pragma unroll
            for (int i = 0; i < RPS; ++i) {
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
                const f4 ev = gate4(R.eb, i) * kf * e2;
                const f4 uv = TIED ? ev : gate4(R.wr, i) * kf * e2;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float m = fmaxf(fmaxf(fabsf(khf[i][j]), fabsf(qhf[i][j])),
                                          fmaxf(fabsf(ev[j]), fabsf(uv[j])));
                    bad |= !(m <= MAX_OPERAND);
                }
                const int r = RPS * seg + i;
                *reinterpret_cast<h4 *>(&S.kh[r * KP + 4 * cq]) = to_h4(khf[i]);
                *reinterpret_cast<h4 *>(&S.qh[r * KP + 4 * cq]) = to_h4(qhf[i]);
                *reinterpret_cast<h4 *>(&S.eh[r * KP + 4 * cq]) = to_h4(ev);
                if (!TIED) *reinterpret_cast<h4 *>(&S.uh[r * KP + 4 * cq]) = to_h4(uv);
            }
            if (bad) S.wide = 1;
        }
        __syncthreads();

        const bool wide = S.wide != 0;
        if (!wide) {
            // ---- Grams: one 16x16 tile per unit, A/Bm/R/P sharing fragments;
            //      waves 0,1 take two diagonal tiles each, waves 2..7 one
            //      off-diagonal tile (those also fold the cross-block factor)
            for (int n = 0; n < 2; ++n) {
                int i, j;
                if (wv < 2) {
                    i = j = 2 * wv + n;
                } else {
                    if (n) break;
                    i = kOffI[wv - 2];
                    j = kOffJ[wv - 2];
                }
                const float *dj = (i != j) ? S.dtab[kPair[i][j]] : nullptr;
                f4 aA = splat(0.f), aB = splat(0.f), aR = splat(0.f), aP = splat(0.f);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int cb = 32 * ks + 8 * lg;
                    const h8 xk = *reinterpret_cast<const h8 *>(&S.kh[(16 * i + lr) * KP + cb]);
                    const h8 xq = *reinterpret_cast<const h8 *>(&S.qh[(16 * i + lr) * KP + cb]);
                    h8 ye = *reinterpret_cast<const h8 *>(&S.eh[(16 * j + lr) * KP + cb]);
                    h8 yu = TIED ? ye : *reinterpret_cast<const h8 *>(&S.uh[(16 * j + lr) * KP + cb]);
                    if (dj) {
                        const f4 d0 = *reinterpret_cast<const f4 *>(&dj[cb]);
                        const f4 d1 = *reinterpret_cast<const f4 *>(&dj[cb + 4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            ye[e] = (_Float16)((float)ye[e] * d0[e]);
                            ye[e + 4] = (_Float16)((float)ye[e + 4] * d1[e]);
                            if (!TIED) {
                                yu[e] = (_Float16)((float)yu[e] * d0[e]);
                                yu[e + 4] = (_Float16)((float)yu[e + 4] * d1[e]);
                            }
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
                // a diagonal tile's wave inverts it right away (overlapping the
                // off-diagonal tiles of the other waves); scratch blocks 4..7
                // do not overlap the cross-block factor table still in use
                if (i == j)
                    invert_unit_lower16(&S.af[(16 * i) * AP + 16 * i], &S.t16[(16 * i) * SP + 16 * i],
                                        S.scr[4 + 2 * wv], S.scr[5 + 2 * wv], lr, lg);
            }
        }
        __syncthreads();
        if (tid == 0) S.wide = 0;

        if (!wide) {
            // ---- state-side operands Kbar = k 2^g, Qbar = q 2^g ----------
#pragma unroll
            for (int i = 0; i < RPS; ++i) {
                const int r = RPS * seg + i;
                *reinterpret_cast<h4 *>(&S.kh[r * KP + 4 * cq]) = to_h4(khf[i] * egm);
                *reinterpret_cast<h4 *>(&S.qh[r * KP + 4 * cq]) = to_h4(qhf[i] * egm);
            }
        }
        // prefetch the next chunk while this one is computed (rows past the
        // end come back as zeros)
        load_raw<VT, TIED, KEYG>(R, a, b, h, t0 + C, col0, seg, cq, tid);

        if (!wide) {
            // ---- solve Tm = (I + A)^-1, all fp32 (diagonal blocks were
            //      inverted in the Gram phase).
            // Off-diagonal blocks from the 2x2 split into 32x32 halves,
            // Tm = [[T_A, 0], [-T_B A_BL T_A, T_B]], on the fp32 matrix unit.
            // Level 1: T_10 = -T_11 A_10 T_00 and T_32 = -T_33 A_32 T_22.
            auto blk = [&](int bi, int bj) { return &S.af[(16 * bi) * AP + 16 * bj]; };
            auto store_t = [&](int bi, int bj, f4 t, bool keep32) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * bi + 4 * lg + e, c = 16 * bj + lr;
                    if (keep32) S.af[r * AP + c] = t[e];
                    S.t16[r * SP + c] = (_Float16)t[e];
                }
            };
            if (wv < 2) {
                const int d = 2 * wv;  // (1,0) from blocks 0,1; (3,2) from blocks 2,3
                float *wt = S.scr[wv];
                const f4 w = mfma_f32_block(blk(d + 1, d), AP, blk(d, d), AP, splat(0.f), lr, lg);
#pragma unroll
                for (int e = 0; e < 4; ++e) wt[(4 * lg + e) * 16 + lr] = w[e];
                // the same wave reads back what it wrote: LDS keeps a wave's order
                const f4 t = -mfma_f32_block(blk(d + 1, d + 1), AP, wt, 16, splat(0.f), lr, lg);
                // A_10 / A_32 are not needed again: overwrite in place
                store_t(d + 1, d, t, true);
            }
            __syncthreads();
            // Level 2: W = A_BL T_A (2x2 blocks), one block per wave 0..3
            if (wv < 4) {
                const int wi = 2 + (wv >> 1), wj = wv & 1;  // W block (row wi of A, col wj of T_A)
                f4 w = mfma_f32_block(blk(wi, 1), AP, blk(1, wj), AP, splat(0.f), lr, lg);  // A_wi1 T_1wj
                if (wj == 0) w = mfma_f32_block(blk(wi, 0), AP, blk(0, 0), AP, w, lr, lg);  // + A_wi0 T_00
                float *wt = S.scr[wv];
#pragma unroll
                for (int e = 0; e < 4; ++e) wt[(4 * lg + e) * 16 + lr] = w[e];
            }
            __syncthreads();
            // Level 3: lower-left quarter = -T_B W, one block per wave 0..3
            if (wv < 4) {
                const int ti = 2 + (wv >> 1), tj = wv & 1;
                // row ti of T_B: T_22 (ti = 2) or [T_32, T_33] (ti = 3); W blocks scr[wj + 2*row]
                f4 t = mfma_f32_block(blk(ti, ti), AP, S.scr[tj + 2 * (ti - 2)], 16, splat(0.f), lr, lg);
                if (ti == 3) t = mfma_f32_block(blk(3, 2), AP, S.scr[tj], 16, t, lr, lg);
                store_t(ti, tj, -t, false);
            }
            __syncthreads();  // Tm ready in fp16; af region free for X / -M

            // Chunk-row outputs (X, M, O: C x VT): wave wv owns row block
            // rb = wv/2 and NCTW value tiles, so its row-side fragment is read
            // once per k-step for all of them.
            const int rb = wv >> 1, ct0 = (wv & 1) * NCTW;
            const bool rows_active = NCT >= 2 || (wv & 1) == 0;

            // ---- X = Kbar S + Bm V -------------------------------------------
            f4 acc[NCTW];
            if (rows_active) {
#pragma unroll
                for (int n = 0; n < NCTW; ++n) acc[n] = splat(0.f);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int cb = 32 * ks + 8 * lg;
                    const h8 xa = *reinterpret_cast<const h8 *>(&S.kh[(16 * rb + lr) * KP + cb]);
#pragma unroll
                    for (int n = 0; n < NCTW; ++n)
                        acc[n] = mfma32(xa, *reinterpret_cast<const h8 *>(&S.s16[(16 * (ct0 + n) + lr) * KP + cb]), acc[n]);
                }
                for (int ks = 0; ks <= (rb >> 1); ++ks) {
                    const int sb = 32 * ks + 8 * lg;
                    const h8 xa = *reinterpret_cast<const h8 *>(&S.b16[(16 * rb + lr) * SP + sb]);
#pragma unroll
                    for (int n = 0; n < NCTW; ++n)
                        acc[n] = mfma32(xa, *reinterpret_cast<const h8 *>(&S.v16[(16 * (ct0 + n) + lr) * SP + sb]), acc[n]);
                }
#pragma unroll
                for (int n = 0; n < NCTW; ++n)
                    *reinterpret_cast<h4 *>(&S.xm16[(16 * (ct0 + n) + lr) * SP + 16 * rb + 4 * lg]) = to_h4(acc[n]);
            }
            __syncthreads();

            // ---- M = Tm X ------------------------------------------------------
            if (rows_active) {
#pragma unroll
                for (int n = 0; n < NCTW; ++n) acc[n] = splat(0.f);
                for (int ks = 0; ks <= (rb >> 1); ++ks) {
                    const int sb = 32 * ks + 8 * lg;
                    const h8 xa = *reinterpret_cast<const h8 *>(&S.t16[(16 * rb + lr) * SP + sb]);
#pragma unroll
                    for (int n = 0; n < NCTW; ++n)
                        acc[n] = mfma32(xa, *reinterpret_cast<const h8 *>(&S.xm16[(16 * (ct0 + n) + lr) * SP + sb]), acc[n]);
                }
            }
            __syncthreads();
            if (rows_active) {
#pragma unroll
                for (int n = 0; n < NCTW; ++n)
                    *reinterpret_cast<h4 *>(&S.xm16[(16 * (ct0 + n) + lr) * SP + 16 * rb + 4 * lg]) = to_h4(-acc[n]);
            }
            __syncthreads();

            // ---- O = Qbar S + P V + R (-M) -> HBM --------------------------------
            if (rows_active) {
                const _Float16 *pp = TIED ? S.r16 : S.p16;
#pragma unroll
                for (int n = 0; n < NCTW; ++n) acc[n] = splat(0.f);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int cb = 32 * ks + 8 * lg;
                    const h8 xa = *reinterpret_cast<const h8 *>(&S.qh[(16 * rb + lr) * KP + cb]);
#pragma unroll
                    for (int n = 0; n < NCTW; ++n)
                        acc[n] = mfma32(xa, *reinterpret_cast<const h8 *>(&S.s16[(16 * (ct0 + n) + lr) * KP + cb]), acc[n]);
                }
                for (int ks = 0; ks <= (rb >> 1); ++ks) {
                    const int sb = 32 * ks + 8 * lg;
                    const h8 xp = *reinterpret_cast<const h8 *>(&pp[(16 * rb + lr) * SP + sb]);
                    const h8 xr = *reinterpret_cast<const h8 *>(&S.r16[(16 * rb + lr) * SP + sb]);
#pragma unroll
                    for (int n = 0; n < NCTW; ++n) {
                        acc[n] = mfma32(xp, *reinterpret_cast<const h8 *>(&S.v16[(16 * (ct0 + n) + lr) * SP + sb]), acc[n]);
                        acc[n] = mfma32(xr, *reinterpret_cast<const h8 *>(&S.xm16[(16 * (ct0 + n) + lr) * SP + sb]), acc[n]);
                    }
                }
#pragma unroll
                for (int n = 0; n < NCTW; ++n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t t = t0 + 16 * rb + 4 * lg + e;
                        if (t < a.T) a.o[((b * a.T + t) * a.H + h) * D + col0 + 16 * (ct0 + n) + lr] = acc[n][e];
                    }
            }

            // ---- S <- 2^gC S + sum_j 2^(gC-gm_j) (Uh_j^T V_j + Eh_j^T (-M)_j) --
            const _Float16 *up = TIED ? S.eh : S.uh;
            {
                const int rt = wv;
                f4 gam;
#pragma unroll
                for (int e = 0; e < 4; ++e) gam[e] = S.gce[16 * rt + 4 * lg + e];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) sacc[ct] *= gam;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    h4 au, ae;
                    f4 fs;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 16 * j + 4 * lg + e;
                        au[e] = up[s * KP + 16 * rt + lr];
                        ae[e] = S.eh[s * KP + 16 * rt + lr];
                        fs[e] = S.fsc[j][16 * rt + 4 * lg + e];
                    }
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const int vb = (16 * ct + lr) * SP + 16 * j + 4 * lg;
                        f4 y = splat(0.f);
                        y = mfma16(au, *reinterpret_cast<const h4 *>(&S.v16[vb]), y);
                        y = mfma16(ae, *reinterpret_cast<const h4 *>(&S.xm16[vb]), y);
                        sacc[ct] += fs * y;
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
                    S.fb.tok[0][c] = expf(load_gate(a.la, a.la_key, row, D, c));
                    S.fb.tok[1][c] = kv;
                    S.fb.tok[2][c] = bb * kv;
                    S.fb.tok[3][c] = ww * kv;
                    S.fb.tok[4][c] = a.q_scale * bf16_to_f32(qp[row * D + c]);
                } else if (tid < D + VT) {
                    S.fb.tok[5][tid - D] = bf16_to_f32(vp[row * D + col0 + tid - D]);
                }
                __syncthreads();
                float pmv[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) pmv[ct] = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 16 * wv + 4 * lg + e;
                    const float ac = S.fb.tok[0][c], kc = S.fb.tok[1][c];
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        sacc[ct][e] *= ac;
                        pmv[ct] += kc * sacc[ct][e];
                    }
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    float x = pmv[ct];
                    x += __shfl_xor(x, 16);
                    x += __shfl_xor(x, 32);
                    if (lg == 0) S.fb.red[0][wv][16 * ct + lr] = x;
                }
                __syncthreads();
                float mv[NCT], vv[NCT], pov[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const int v = 16 * ct + lr;
                    float m = 0.f;
#pragma unroll
                    for (int w = 0; w < NW; ++w) m += S.fb.red[0][w][v];
                    mv[ct] = m;
                    vv[ct] = S.fb.tok[5][v];
                    pov[ct] = 0.f;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 16 * wv + 4 * lg + e;
                    const float ec = S.fb.tok[2][c], uc = S.fb.tok[3][c], qc = S.fb.tok[4][c];
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        sacc[ct][e] = sacc[ct][e] - ec * mv[ct] + uc * vv[ct];
                        pov[ct] += qc * sacc[ct][e];
                    }
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    float x = pov[ct];
                    x += __shfl_xor(x, 16);
                    x += __shfl_xor(x, 32);
                    if (lg == 0) S.fb.red[1][wv][16 * ct + lr] = x;
                }
                __syncthreads();
                if (tid < VT) {
                    float o = 0.f;
#pragma unroll
                    for (int w = 0; w < NW; ++w) o += S.fb.red[1][w][tid];
                    a.o[row * D + col0 + tid] = o;
                }
                __syncthreads();  // tok and red reused by the next token
            }
        }
    }

    if (a.s_out) {
        const int lr = lane0 & 15, lg = lane0 >> 4;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * wv + 4 * lg + e;
                const int v = col0 + 16 * ct + lr;
                a.s_out[sbase + static_cast<int64_t>(c) * D + v] = sacc[ct][e];
            }
    }
}

template <int VT, bool TIED, bool KEYG>
hipError_t launch_vt(const ChunkArgs &a, hipStream_t s) {
    const int nt = D / VT;
    const int64_t chains = a.B * a.H;
    const int xcd_map = (chains % 8 == 0) ? 1 : 0;
    const dim3 grid(static_cast<unsigned>(chains * nt));
    hipLaunchKernelGGL((chunk_mfma_kernel<VT, TIED, KEYG>), grid, dim3(NTH), 0, s, a, nt, xcd_map);
    return hipGetLastError();
}

template <int VT>
hipError_t launch_kind(const ChunkArgs &a, hipStream_t s) {
    const bool tied = a.wr == nullptr, keyg = a.la_key != 0;
    if (tied) return keyg ? launch_vt<VT, true, true>(a, s) : launch_vt<VT, true, false>(a, s);
    return keyg ? launch_vt<VT, false, true>(a, s) : launch_vt<VT, false, false>(a, s);
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs &a) {
    // every present gate of one kind (all per key channel or all per head)
    const bool tied = a.wr == nullptr;
    const bool same = a.la_key == a.eb_key && (tied || a.wr_key == a.eb_key);
    return a.bf16 && a.dk == D && a.dv == D && a.C == C && same &&
           a.H * D * 4 * C < (int64_t(1) << 31);
}

hipError_t launch_chunk_mfma(const ChunkArgs &a, hipStream_t s) {
    // Value slices per chain: enough workgroups to give every CU one.
    const int64_t chains = a.B * a.H;
    if (chains * 2 >= 256) return launch_kind<64>(a, s);
    if (chains * 4 >= 256) return launch_kind<32>(a, s);
    return launch_kind<16>(a, s);
}

}  // namespace gdn2
