// chunk_common.h -- pieces shared by the matrix-core chunk kernels
// (bf16 q/k/v, dk = dv = 128, chunk C = 64): fragment helpers, the per-chunk
// gate tables, the factored fp16 Gram operands, the four Grams and the
// unit-lower-triangular inverse.
//
// Notation (the WY/UT chunk form of the gist.science summary, "Technische
// Samenvatting" section 3): g is the inclusive cumulative log-decay inside
// the chunk, e = b*k and u = w*k;
//   A[r,s] = sum_c k_r e_s exp(g_r-g_s) (r>s), Bm the same with u,
//   R[r,s] = sum_c q_r e_s exp(g_r-g_s) (r>=s), P the same with u,
//   Tm = (I + A)^-1.
//
// fp16 operands.  exp(g_r - g_s) is factored around a reference gm inside
// each 16-token block: the row side carries 2^(g_r - gm_i), the column side
// 2^(gm_j - g_s), and the cross-block factor 2^(gm_i - gm_j) <= 1 is folded
// into the column fragment.  A chunk whose factors or operands leave the
// fast range (|log2 factor| > 14, |operand| > 16384) is flagged `wide` and
// the caller computes it exactly instead.
#pragma once

#include "common.h"
#include "kernels.h"

namespace gdn2 {
namespace mfma {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;          // chunk length
constexpr int D = 128;         // dk = dv
constexpr int NTH = 512;       // 8 waves
constexpr int NW = NTH / 64;
constexpr int NSEG = NTH / 32; // 4-row segments of the chunk (16)
constexpr int RPS = C / NSEG;  // rows per segment (4)
// LDS pitches.  Every row of an fp16 or fp32 array starts on a 16-byte
// boundary (so 8- and 16-byte accesses can be single ds_read/ds_write
// instructions), and the pitches keep the wide row reads of the MFMA
// operand fragments free of bank conflicts or nearly so (measured on gfx950:
// rows 272 bytes apart cost 4 extra cycles per 16-byte read, 264 bytes 12).
constexpr int KP = D + 8;      // pitch (halves) of [token][channel] operands
constexpr int SP = C + 8;      // pitch (halves) of [row][token] operands
constexpr int AP = C + 4;      // pitch (floats) of the fp32 C x C matrix
constexpr int IP = 18;         // pitch (floats) of the 16x16 inverse scratch
constexpr int GP = D + 4;      // pitch (floats) of the segment totals (a quad's four rows: 2-way banked)
                               // (read along its rows by the matrix unit)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float MAX_EXP2 = 14.f;        // largest |log2 factor| on the fast path
constexpr float MAX_OPERAND = 16384.f;  // largest |fp16 operand| on the fast path
constexpr float MAX_RESULT = 30000.f;   // largest |fp16 product| kept on the fast path
constexpr float MAX_STATE = 16384.f;    // largest |state| whose fp16 copy feeds a product

// (block row, block col) of the strictly-lower 16x16 tiles of a 64x64 chunk
// matrix, and the index of each such pair in the cross-block factor table.
// (one private copy per translation unit)
namespace {
__constant__ int kOffI[6] = {1, 2, 2, 3, 3, 3};
__constant__ int kOffJ[6] = {0, 0, 1, 0, 1, 2};
__constant__ int kPair[4][4] = {{-1, -1, -1, -1}, {0, -1, -1, -1}, {1, 2, -1, -1}, {3, 4, 5, -1}};
}  // namespace

// Gate kinds of a request, one compile-time code GK: 0 every gate one value
// per token-head; 1 every gate per key channel; 2 the decay per key channel
// and the erase / write rates per token-head (KDA's gates: per-channel decay,
// one rate per head).
constexpr bool decay_key(int GK) { return GK != 0; }
constexpr bool rate_key(int GK) { return GK == 1; }

// Raw gate rows held in registers: 4 key channels per row when a gate is
// per key channel, one value per row when per head.
template <bool KEYG>
struct GateRow;
template <>
struct GateRow<true> {
    static constexpr bool key = true;
    f4 x[RPS];
};
template <>
struct GateRow<false> {
    static constexpr bool key = false;
    float x[RPS];
};

// Raw inputs of one chunk held in registers: thread (seg, cq) owns rows
// RPS*seg.. and key channels 4cq..4cq+3; NV 16-byte pieces of values.
template <int GK, int NV>
struct Raw {
    uint2 k[RPS], q[RPS];
    GateRow<decay_key(GK)> la;
    GateRow<rate_key(GK)> eb, wr;
    uint4 v[NV];
};

__device__ __forceinline__ f4 gate4(const GateRow<true> &g, int i) { return g.x[i]; }
__device__ __forceinline__ f4 gate4(const GateRow<false> &g, int i) {
    return f4{g.x[i], g.x[i], g.x[i], g.x[i]};
}


// With bf16 gate logits, a gate row holds the raw bits (per channel: four
// logits in the first two words; per head: the logit in the low half) and
// is activated where it is used (act 0: -softplus, the log-decay; act 1:
// sigmoid).
__device__ __forceinline__ float act_gate(float x, int act) { return act == 0 ? neg_softplus(x) : sigmoid_gate(x); }
__device__ __forceinline__ f4 gate4a(const GateRow<true> &g, int i, int logits, int act) {
    if (!logits) return g.x[i];
    const uint32_t lo = __float_as_uint(g.x[i][0]), hi = __float_as_uint(g.x[i][1]);
    return f4{act_gate(__uint_as_float(lo << 16), act), act_gate(__uint_as_float(lo & 0xffff0000u), act),
              act_gate(__uint_as_float(hi << 16), act), act_gate(__uint_as_float(hi & 0xffff0000u), act)};
}
__device__ __forceinline__ f4 gate4a(const GateRow<false> &g, int i, int logits, int act) {
    if (!logits) return gate4(g, i);
    const float x = act_gate(__uint_as_float(__float_as_uint(g.x[i]) << 16), act);
    return f4{x, x, x, x};
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

// Vector LDS accesses at the alignment the layouts guarantee (each use's
// offset is a multiple of the vector's size), so that they compile to single
// wide ds_read / ds_write instructions rather than pairs of 4-byte accesses.
template <typename V, typename T>
__device__ __forceinline__ V lds_ld(const T *p) {
    return *reinterpret_cast<const V *>(__builtin_assume_aligned(p, sizeof(V)));
}
template <typename V, typename T>
__device__ __forceinline__ void lds_st(T *p, V x) {
    *reinterpret_cast<V *>(__builtin_assume_aligned(p, sizeof(V))) = x;
}

// Whether a product about to be rounded to fp16 leaves the fast range (or is
// not finite).
__device__ __forceinline__ bool out_of_range(f4 x) {
    return !(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))) <= MAX_RESULT);
}

__device__ __forceinline__ h4 to_h4(f4 x) {
    return h4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}
__device__ __forceinline__ f4 to_f4(h4 x) { return f4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]}; }

// Two 4-element halves -> one 8-element fragment.
__device__ __forceinline__ h8 join(h4 lo, h4 hi) {
    return h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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
// `sa`, `sb` are two private 16x16 fp32 scratch blocks of row pitch IP.  The result is written
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
    for (int e = 0; e < 4; ++e) sa[(4 * lg + e) * IP + lr] = n2[e];
    const f4 n3 = mfma_f32_block(na, AP, sa, IP, splat(0.f), lr, lg);
    const f4 t1 = eye - nn + n2 - n3;  // (I - N)(I + N^2)
    const f4 n4 = mfma_f32_block(sa, IP, sa, IP, splat(0.f), lr, lg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        sb[(4 * lg + e) * IP + lr] = t1[e];
        sa[(4 * lg + e) * IP + lr] = n4[e];
    }
    const f4 t2 = mfma_f32_block(sb, IP, sa, IP, t1, lr, lg);  // T1 (I + N^4)
    const f4 n8 = mfma_f32_block(sa, IP, sa, IP, splat(0.f), lr, lg);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        sb[(4 * lg + e) * IP + lr] = t2[e];
        sa[(4 * lg + e) * IP + lr] = n8[e];
    }
    const f4 t3 = mfma_f32_block(sb, IP, sa, IP, t2, lr, lg);  // T2 (I + N^8)
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
                                                            int width, int esize, int col0,
                                                            int64_t tlim = -1) {
    // rows at or past tlim (default: the sequence length T) read as zero
    const int64_t lim = tlim < 0 ? a.T : tlim;
    const int64_t nvalid = lim - t0 < C ? (lim - t0 > 0 ? lim - t0 : 0) : C;
    const char *p = static_cast<const char *>(base) +
                    (((b * a.T + t0) * a.H + h) * width + col0) * static_cast<int64_t>(esize);
    const int64_t bytes = nvalid > 0 ? ((nvalid - 1) * a.H * width + width - col0) * esize : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), (short)0, static_cast<int>(bytes),
                                             0x00020000);
}

// Issue the key, query and gate loads of one chunk (no waits).
// Row i of my segment of one fp32 gate (per key channel or per head) into
// `x`, from the buffer resource `rs` over the chunk's rows (no wait).
template <bool KEY>
__device__ __forceinline__ void load_gate_row(GateRow<KEY> &x, __amdgpu_buffer_rsrc_t rs, int row_elems,
                                              int seg, int cq) {
#pragma unroll
    for (int i = 0; i < RPS; ++i) {
        const int r = seg * RPS + i;
        if constexpr (KEY)
            x.x[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rs, (r * row_elems + 4 * cq) * 4, 0, 0));
        else
            x.x[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, r * row_elems * 4, 0, 0));
    }
}

template <bool TIED, int GK, int NV>
__device__ __forceinline__ void load_kqg(Raw<GK, NV> &R, const ChunkArgs &a, int64_t b, int64_t h,
                                         int64_t t0, int seg, int cq) {
    const auto rk = chain_rsrc(a.k, a, b, h, t0, D, 2, 0);
    const auto rq = chain_rsrc(a.q, a, b, h, t0, D, 2, 0);
    const int ga = decay_key(GK) ? D : 1, gr = rate_key(GK) ? D : 1;
    const int rowk = static_cast<int>(a.H) * D;  // elements between consecutive tokens
#pragma unroll
    for (int i = 0; i < RPS; ++i) {
        const int ok = ((seg * RPS + i) * rowk + 4 * cq) * 2;
        R.k[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, ok, 0, 0));
        R.q[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, ok, 0, 0));
    }
    load_gate_row(R.la, chain_rsrc(a.la, a, b, h, t0, ga, 4, 0), static_cast<int>(a.H) * ga, seg, cq);
    load_gate_row(R.eb, chain_rsrc(a.eb, a, b, h, t0, gr, 4, 0), static_cast<int>(a.H) * gr, seg, cq);
    if (!TIED) load_gate_row(R.wr, chain_rsrc(a.wr, a, b, h, t0, gr, 4, 0), static_cast<int>(a.H) * gr, seg, cq);
}

// Running log2-decay of my RPS rows (relative to the start of my segment);
// the segment total goes to segtot[seg].
// With logits, rows past the end of the sequence (which load as zero
// logits, i.e. a real decay of 1/2) are given no decay: nvalid = T - t0.
template <typename SM, int GK, int NV>
__device__ __forceinline__ void segment_cumsum(SM &S, const Raw<GK, NV> &R, f4 (&g)[RPS], int seg,
                                               int cq, int logits = 0, int64_t nvalid = C) {
    f4 run = splat(0.f);
#pragma unroll
    for (int i = 0; i < RPS; ++i) {
        const f4 x = gate4a(R.la, i, logits, 0) * LOG2E;
        run += (!logits || seg * RPS + i < nvalid) ? x : splat(0.f);  // a select, not a branch
        g[i] = run;
    }
    lds_st<f4>(&S.segtot[seg][4 * cq], run);
}

// x moved across lanes by the DPP control CTRL (all rows and banks).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Exclusive prefix of the segment totals, in place, and the per-chunk factor
// tables, four lanes per key channel (every thread of the workgroup: channel
// c = tid / 4, lane j = tid % 4 of its quad takes segments 4j .. 4j+3, whose
// second row ends block j's reference):
//   gce[c] = 2^g_C, fsc[j][c] = 2^(g_C - gm_j), dtab = 2^(gm_i - gm_j), i > j.
// The prefix is summed in segment order, as one lane would (three rounds pass
// each quad lane's running total to the next lane), so the tables do not
// depend on how the work is split.
template <typename SM>
__device__ __forceinline__ void chunk_tables(SM &S, int tid) {
    const int c = tid >> 2, j = tid & 3;
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = S.segtot[4 * j + k][c];
    float base = 0.f, tot = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        tot = base;
#pragma unroll
        for (int k = 0; k < 4; ++k) tot += v[k];
        if (r < 3) {
            const float prev = dpp_f32<0x90>(tot);  // quad_perm [0, 0, 1, 2]: lane j - 1's total
            base = j ? prev : 0.f;
        }
    }
    float run = base, gm = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        S.segtot[4 * j + k][c] = run;
        run += v[k];
        if (k == 1) gm = run;  // block reference: after row 16j+7
    }
    const float cum = dpp_f32<0xFF>(tot);  // quad_perm [3, 3, 3, 3]: the chunk total
    const float g0 = dpp_f32<0x00>(gm), g1 = dpp_f32<0x55>(gm), g2 = dpp_f32<0xAA>(gm);
    if (j == 0) S.gce[c] = __builtin_amdgcn_exp2f(cum);
    S.fsc[j][c] = __builtin_amdgcn_exp2f(cum - gm);
    if (j == 1) {
        S.dtab[0][c] = __builtin_amdgcn_exp2f(gm - g0);
    } else if (j == 2) {
        S.dtab[1][c] = __builtin_amdgcn_exp2f(gm - g0);
        S.dtab[2][c] = __builtin_amdgcn_exp2f(gm - g1);
    } else if (j == 3) {
        S.dtab[3][c] = __builtin_amdgcn_exp2f(gm - g0);
        S.dtab[4][c] = __builtin_amdgcn_exp2f(gm - g1);
        S.dtab[5][c] = __builtin_amdgcn_exp2f(gm - g2);
    }
}

// Sum over each half-wave's 32 lanes (the 32 lanes that hold one token row),
// the same total in every lane: within rows of 16 lanes the quad swaps
// (lane ^ 1, lane ^ 2), then the half-row and row mirrors (lane i with 7 - i,
// then with 15 - i), each pairing a lane with one from the other group; last
// a swizzle that swaps the two rows of the half-wave (lane ^ 16).
__device__ __forceinline__ float half_wave_sum(float x) {
    x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp_f32<0x141>(x);  // row_half_mirror
    x += dpp_f32<0x140>(x);  // row_mirror
    return x + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));  // xor 16 in 32
}

// Factored fp16 Gram operands of my rows: kh = k 2^(g-gm), qh = q 2^(g-gm),
// eh = e 2^(gm-g), uh = u 2^(gm-g); keeps k 2^(g-gm), q 2^(g-gm) (fp32) and
// 2^gm for the later Kbar/Qbar rewrite.  Raises S.wide when a factor or
// operand leaves the fast range.
// With VW (the value-write form: erase gate on the read, erase and write
// along k; TIED holds) the row operand is b k and the column operand k.
// With `logits` the gates are activated here; with `qknorm` every row of k
// and q is divided by its L2 norm (the 32 lanes of a segment hold a row).
template <typename SM, bool TIED, int GK, int NV, bool VW = false>
__device__ __forceinline__ void factored_operands(SM &S, const Raw<GK, NV> &R, f4 (&g)[RPS],
                                                  f4 (&khf)[RPS], f4 (&qhf)[RPS], f4 &egm, int seg,
                                                  int cq, float qs, int logits = 0, int qknorm = 0) {
    static_assert(!VW || TIED, "the value-write form erases and writes along the same vector");
    const int blk = seg / 4;  // 16-row block of my rows
    const f4 base = lds_ld<f4>(&S.segtot[seg][4 * cq]);
    const f4 gmv = lds_ld<f4>(&S.segtot[4 * blk + 2][4 * cq]);
#pragma unroll
    for (int j = 0; j < 4; ++j) egm[j] = __builtin_amdgcn_exp2f(gmv[j]);
    bool bad = false;
#pragma unroll
    for (int i = 0; i < RPS; ++i) {
        g[i] += base;
        const f4 x = g[i] - gmv;
        f4 e1, e2;
        if constexpr (!decay_key(GK)) {
            // one decay per token-head: the running sums, and so the four
            // channels' factors, are equal (the same values, summed alike)
            bad |= !(fabsf(x[0]) <= MAX_EXP2);
            e1 = splat(__builtin_amdgcn_exp2f(x[0]));
            e2 = splat(__builtin_amdgcn_exp2f(-x[0]));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bad |= !(fabsf(x[j]) <= MAX_EXP2);
                e1[j] = __builtin_amdgcn_exp2f(x[j]);
                e2[j] = __builtin_amdgcn_exp2f(-x[j]);
            }
        }
        f4 kraw = bf16x4_to_f4(R.k[i]);
        f4 qraw = bf16x4_to_f4(R.q[i]);
        if (qknorm) {
            const float sk = half_wave_sum(kraw[0] * kraw[0] + kraw[1] * kraw[1] + kraw[2] * kraw[2] + kraw[3] * kraw[3]);
            const float sq = half_wave_sum(qraw[0] * qraw[0] + qraw[1] * qraw[1] + qraw[2] * qraw[2] + qraw[3] * qraw[3]);
            kraw = kraw * (sk > 0.f ? rsqrtf(sk) : 0.f);
            qraw = qraw * (sq > 0.f ? rsqrtf(sq) : 0.f);
        }
        const f4 eb = gate4a(R.eb, i, logits, 1);
        const f4 kf = VW ? eb * kraw : kraw;  // the read key
        const f4 qf = qraw * qs;
        khf[i] = kf * e1;
        qhf[i] = qf * e1;
        const f4 ev = VW ? kraw * e2 : eb * kraw * e2;
        const f4 uv = TIED ? ev : gate4a(R.wr, i, logits, 1) * kf * e2;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float m = fmaxf(fmaxf(fabsf(khf[i][j]), fabsf(qhf[i][j])), fmaxf(fabsf(ev[j]), fabsf(uv[j])));
            bad |= !(m <= MAX_OPERAND);
        }
        const int r = RPS * seg + i;
        lds_st<h4>(&S.kh[r * KP + 4 * cq], to_h4(khf[i]));
        lds_st<h4>(&S.qh[r * KP + 4 * cq], to_h4(qhf[i]));
        lds_st<h4>(&S.eh[r * KP + 4 * cq], to_h4(ev));
        if (!TIED) lds_st<h4>(&S.uh[r * KP + 4 * cq], to_h4(uv));
    }
    if (bad) S.wide = 1;
}

// One 16x16 tile (block row i, block column j <= i) of the four Grams, A/Bm/R/P
// sharing fragments; an off-diagonal tile folds the cross-block factor into
// its column fragment.  Writes af (A, fp32), b16, r16 and p16, and returns
// whether an entry stored in fp16 (Bm, R, P) left the fast range.  PARTS
// selects a share of the tile, so that two waves can split one: bit 0 the
// Grams on the erase column operand (A and R), bit 1 those on the write
// column operand (Bm and P); with tied gates (Bm = A, P = R) bit 0 is A, bit 1
// is R.  Each Gram is accumulated in the same order whatever the share.
// With BT the write Gram Bm is also stored transposed (S.ut.bt, [s][r]).
template <typename SM, bool TIED, int PARTS = 3, bool BT = false>
__device__ __forceinline__ bool gram_tile(SM &S, int i, int j, int lr, int lg) {
    constexpr bool doA = PARTS & 1, doR = TIED ? (PARTS & 2) != 0 : (PARTS & 1) != 0;
    constexpr bool doB = !TIED && (PARTS & 2), doP = !TIED && (PARTS & 2);
    constexpr bool useE = doA || doR, useU = doB || doP;
    constexpr bool useK = doA || doB, useQ = doR || doP;
    const float *dj = (i != j) ? S.dtab[kPair[i][j]] : nullptr;
    f4 aA = splat(0.f), aB = splat(0.f), aR = splat(0.f), aP = splat(0.f);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int cb = 32 * ks + 8 * lg;
        h8 xk{}, xq{}, ye{}, yu{};
        if (useK) xk = lds_ld<h8>(&S.kh[(16 * i + lr) * KP + cb]);
        if (useQ) xq = lds_ld<h8>(&S.qh[(16 * i + lr) * KP + cb]);
        if (useE) ye = lds_ld<h8>(&S.eh[(16 * j + lr) * KP + cb]);
        if (useU) yu = lds_ld<h8>(&S.uh[(16 * j + lr) * KP + cb]);
        if (dj) {
            const f4 d0 = lds_ld<f4>(&dj[cb]);
            const f4 d1 = lds_ld<f4>(&dj[cb + 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (useE) {
                    ye[e] = (_Float16)((float)ye[e] * d0[e]);
                    ye[e + 4] = (_Float16)((float)ye[e + 4] * d1[e]);
                }
                if (useU) {
                    yu[e] = (_Float16)((float)yu[e] * d0[e]);
                    yu[e + 4] = (_Float16)((float)yu[e + 4] * d1[e]);
                }
            }
        }
        if (doA) aA = mfma32(xk, ye, aA);
        if (doR) aR = mfma32(xq, ye, aR);
        if (doB) aB = mfma32(xk, yu, aB);
        if (doP) aP = mfma32(xq, yu, aP);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 16 * i + 4 * lg + e, s = 16 * j + lr;
        const bool strict = r > s, incl = r >= s;
        if (doA) S.af[r * AP + s] = strict ? aA[e] : 0.f;
        if (TIED ? doA : doB) S.b16[r * SP + s] = (_Float16)(strict ? (TIED ? aA[e] : aB[e]) : 0.f);
        if (doR) S.r16[r * SP + s] = (_Float16)(incl ? aR[e] : 0.f);
        if (doP) S.p16[r * SP + s] = (_Float16)(incl ? aP[e] : 0.f);
    }
    if constexpr (BT && doB) {
        // Bm^T: lane (lr, lg) holds rows 16i+4lg..+3 of column 16j+lr, one row of the transpose
        h4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (_Float16)((16 * i + 4 * lg + e > 16 * j + lr) ? aB[e] : 0.f);
        lds_st<h4>(&S.ut.bt[(16 * j + lr) * SP + 16 * i + 4 * lg], t);
    }
    return (doR && out_of_range(aR)) || (doB && out_of_range(aB)) || (doP && out_of_range(aP));
}

// The four Grams with 8 waves: waves 0,1 take two diagonal tiles each (and
// invert them right away), waves 2..7 one off-diagonal tile each.  Writes
// af (A, fp32, diagonal blocks then inverted), b16, r16, p16 and the
// diagonal blocks of t16; returns whether a Gram entry held in fp16 left the
// fast range (A and Tm are checked through the products they enter).
template <typename SM, bool TIED>
__device__ __forceinline__ bool gram_tiles(SM &S, int wv, int lr, int lg) {
    bool big = false;
    for (int n = 0; n < 2; ++n) {
        int i, j;
        if (wv < 2) {
            i = j = 2 * wv + n;
        } else {
            if (n) break;
            i = kOffI[wv - 2];
            j = kOffJ[wv - 2];
        }
        big |= gram_tile<SM, TIED>(S, i, j, lr, lg);
        // scratch blocks 4..7 do not overlap the cross-block factor table
        // that the off-diagonal waves are still reading
        if (i == j)
            invert_unit_lower16(&S.af[(16 * i) * AP + 16 * i], &S.t16[(16 * i) * SP + 16 * i],
                                S.scr[4 + 2 * wv], S.scr[5 + 2 * wv], lr, lg);
    }
    return big;
}

// Off-diagonal blocks of Tm = (I + A)^-1 (diagonal blocks already inverted),
// from the 2x2 split into 32x32 halves, Tm = [[T_A, 0], [-T_B A_BL T_A, T_B]],
// on the fp32 matrix unit.  Every thread of the workgroup calls it; it holds
// three barriers and leaves Tm complete in t16 (fp16).
template <typename SM>
__device__ __forceinline__ void solve_offdiag(SM &S, int wv, int lr, int lg) {
    auto blk = [&](int bi, int bj) { return &S.af[(16 * bi) * AP + 16 * bj]; };
    auto store_t = [&](int bi, int bj, f4 t, bool keep32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * bi + 4 * lg + e, c = 16 * bj + lr;
            if (keep32) S.af[r * AP + c] = t[e];
            S.t16[r * SP + c] = (_Float16)t[e];
        }
    };
    // Level 1: T_10 = -T_11 A_10 T_00 and T_32 = -T_33 A_32 T_22.
    if (wv < 2) {
        const int d = 2 * wv;
        float *wt = S.scr[wv];
        const f4 w = mfma_f32_block(blk(d + 1, d), AP, blk(d, d), AP, splat(0.f), lr, lg);
#pragma unroll
        for (int e = 0; e < 4; ++e) wt[(4 * lg + e) * 16 + lr] = w[e];
        // the same wave reads back what it wrote: LDS keeps a wave's order
        const f4 t = -mfma_f32_block(blk(d + 1, d + 1), AP, wt, 16, splat(0.f), lr, lg);
        store_t(d + 1, d, t, true);  // A_10 / A_32 are not needed again
    }
    __syncthreads();
    // Level 2: W = A_BL T_A (2x2 blocks), one block per wave 0..3
    if (wv < 4) {
        const int wi = 2 + (wv >> 1), wj = wv & 1;
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
        f4 t = mfma_f32_block(blk(ti, ti), AP, S.scr[tj + 2 * (ti - 2)], 16, splat(0.f), lr, lg);
        if (ti == 3) t = mfma_f32_block(blk(3, 2), AP, S.scr[tj], 16, t, lr, lg);
        store_t(ti, tj, -t, false);
    }
    __syncthreads();
}

}  // namespace mfma
}  // namespace gdn2
