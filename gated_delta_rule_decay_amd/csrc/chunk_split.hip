// chunk_split.hip -- two-pass chunkwise GDN-2 forward on the gfx950 matrix
// cores (bf16 q/k/v, dk = dv = 128, chunk C = 64, every gate of one kind).
//
// The chunk form (gist.science summary, "Technische Samenvatting" section 3:
// cumulative decay absorbed into the erase and write factors, a
// unit-lower-triangular solve for the auxiliary matrices) splits each chunk
// into work that needs the incoming state S and work that does not.  With
// Tm = (I + A)^-1, Kbar = k e^g, Qbar = q e^g, Util = u e^(gC-g),
// Etil = e e^(gC-g):
//   W  = Tm Kbar           U  = Tm Bm V          (the pseudo-value solve)
//   Qe = Qbar - R W        Oe = P V - R U
//   G  = Util^T V - Etil^T U
// depend on the chunk alone, and then
//   O = Qe S + Oe,   S <- Diag(e^gC) S + G - Etil^T (W S)
// is all that the sequential scan over chunks has to do (M = W S + U is the
// erase read of the token form).
//
// Pass 1 (chunk_prep_kernel) runs every (chain, chunk) in parallel -- one
// 512-lane workgroup per task, persistent, with the next task's inputs
// prefetched into registers -- and writes W, Qe, Etil^T, G and Oe as fp16
// fragments in exactly the register order the scan's MFMA operands take,
// plus e^gC and a flag.  Pass 2 (chunk_scan_kernel) gives each wave one
// chain and 16*NB value columns; the fp32 state slice (128 x 16*NB) stays in
// MFMA accumulators, every operand is one coalesced 16-byte load per lane,
// and waves never synchronise, so a chain's value columns proceed on as
// many CUs as there are waves.
//
// A chunk whose fp16 factors, operands or results would leave the fast
// range is flagged by pass 1; pass 2 runs it as the exact fp32 token
// recurrence on the raw inputs instead (so does a chunk whose state or erase
// read would overflow fp16).
#include "chunk_common.h"

namespace gdn2 {
namespace {

using namespace mfma;

// fp16 record of one (chain, chunk), offsets in halves.  Fragment orders (the
// scan's 16x16x32 operands; "slot" = contraction index inside a 32-block,
// slot 8m+e <-> index 4m+e and slot 8m+4+e <-> index 16+4m+e, so that two
// accumulator tiles form one operand without any data exchange):
//   W, Qe  [rt 4][kb 4][lane 64][8]  lane i+16m: token 16rt+i, key channels
//                                    of block kb in slots 8m..8m+7
//   EtT    [it 8][kb 2][lane 64][8]  lane i+16m: key channel 16it+i, tokens
//                                    of block kb in slots 8m..8m+7
//   G      [ct 8][it 8][lane 64][4]  accumulator tile: lane j+16m holds
//                                    G[16it+4m+e][16ct+j]
//   Oe     [ct 8][rt 4][lane 64][4]  lane j+16m holds Oe[16rt+4m+e][16ct+j]
constexpr int64_t OFF_W = 0;
constexpr int64_t OFF_Q = 8192;
constexpr int64_t OFF_E = 16384;
constexpr int64_t OFF_G = 24576;
constexpr int64_t OFF_O = 40960;
constexpr int64_t REC = 49152;
constexpr float MAX_RESULT = 30000.f;  // largest |fp16 value| a record may hold

struct SplitWs {
    _Float16 *frag;  // [task][REC]
    float *gam;      // [task][D]   e^gC per key channel
    int *flag;       // [task]      1: run the chunk exactly
};

struct PrepSmem {
    _Float16 kh[C * KP];   // Gram row operand k 2^(g-gm); later Kbar
    _Float16 qh[C * KP];   // q 2^(g-gm); later Qbar
    _Float16 eh[C * KP];   // Gram column operand e 2^(gm-g)
    _Float16 uh[C * KP];   // u 2^(gm-g)
    _Float16 v16[D * SP];  // values, [j][s]
    union {
        float af[C * AP];       // A (strict lower), then Tm in place (fp32)
        _Float16 u16[D * SP];   // U, [j][s]
        float segtot[NSEG][D];  // per-segment log2-decay totals
    };
    _Float16 t16[C * SP];  // Tm  [r][s]
    _Float16 b16[C * SP];  // Bm
    _Float16 r16[C * SP];  // R
    _Float16 p16[C * SP];  // P
    union {
        float dtab[6][D];        // 2^(gm_i - gm_j), i > j (Gram phase)
        float scr[8][16 * 16];   // solve scratch (after the Grams)
    };
    float fsc[4][D];  // 2^(g_C - gm_j)
    float gce[D];     // 2^g_C
    float iscr[4][2][16 * 16];  // private scratch of the four diagonal inverses
    int wide;
};

__device__ __forceinline__ bool out_of_range(f4 x) {
    return !(fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))) <= MAX_RESULT);
}

// Loads of task `task` in four parts (no waits), so that a task's requests
// are spread over the previous task instead of arriving at HBM in one burst:
// part 0 the decay, 1 the erase gate, 2 the write gate and the values
// (thread = token pair tid%32, 8-column piece tid/32), 3 keys and queries.
struct TaskPos {
    int64_t b, h, t0;
};

// (batch, head, first token) of task `task` = chain * nc + chunk; 32-bit
// division (the task count is checked to fit on the host).
__device__ __forceinline__ TaskPos task_pos(int64_t task, int nc, int H) {
    const uint32_t t = static_cast<uint32_t>(task), chain = t / static_cast<uint32_t>(nc);
    TaskPos p;
    p.b = chain / static_cast<uint32_t>(H);
    p.h = chain % static_cast<uint32_t>(H);
    p.t0 = static_cast<int64_t>(t - chain * static_cast<uint32_t>(nc)) * C;
    return p;
}

template <int PART, bool TIED, bool KEYG>
__device__ __forceinline__ void load_part(Raw<KEYG, 2> &R, const ChunkArgs &a, const TaskPos &tp0, int tid) {
    const int64_t b = tp0.b, h = tp0.h, t0 = tp0.t0;
    const int seg = tid >> 5, cq = tid & 31;
    const int gw = KEYG ? D : 1;
    const int rowk = static_cast<int>(a.H) * D, rowg = static_cast<int>(a.H) * gw;
    auto gates = [&](GateRow<KEYG> &x, const float *src) {
        const auto rs = chain_rsrc(src, a, b, h, t0, gw, 4, 0);
#pragma unroll
        for (int i = 0; i < RPS; ++i) {
            const int r = seg * RPS + i;
            if constexpr (KEYG)
                x.x[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(rs, (r * rowg + 4 * cq) * 4, 0, 0));
            else
                x.x[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, r * rowg * 4, 0, 0));
        }
    };
    if constexpr (PART == 0) gates(R.la, a.la);
    if constexpr (PART == 1) gates(R.eb, a.eb);
    if constexpr (PART == 2) {
        if (!TIED) gates(R.wr, a.wr);
        const auto rv = chain_rsrc(a.v, a, b, h, t0, D, 2, 0);
        const int tp = tid & 31, piece = tid >> 5;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            R.v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, ((2 * tp + i) * rowk + 8 * piece) * 2, 0, 0));
    }
    if constexpr (PART == 3) {
        const auto rk = chain_rsrc(a.k, a, b, h, t0, D, 2, 0);
        const auto rq = chain_rsrc(a.q, a, b, h, t0, D, 2, 0);
#pragma unroll
        for (int i = 0; i < RPS; ++i) {
            const int ok = ((seg * RPS + i) * rowk + 4 * cq) * 2;
            R.k[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rk, ok, 0, 0));
            R.q[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rq, ok, 0, 0));
        }
    }
}

// Row block rt of a C x C fp16 matrix (pitch SP) as a 16x16x32 A operand
// over token block ks, token slots permuted as in the record (so that it
// pairs with a B operand built from two accumulator tiles).
__device__ __forceinline__ h8 perm_frag(const _Float16 *m, int rt, int ks, int lr, int lg) {
    const _Float16 *p = &m[(16 * rt + lr) * SP + 32 * ks + 4 * lg];
    return join(*reinterpret_cast<const h4 *>(p), *reinterpret_cast<const h4 *>(p + 16));
}

// W^T and Qe^T = Qbar^T - W^T R^T for key channel tiles 2kb, 2kb+1 and token
// tiles 2RH, 2RH+1, written to the record; W = Tm Kbar comes first as tiles
// (tokens x channels) whose registers are the A operand of W^T R^T.
// Returns whether a result left the fp16 range.
template <int RH>
__device__ __forceinline__ bool wq_tiles(const PrepSmem &S, _Float16 *rec, int kb, int lane, int lr, int lg) {
    constexpr int NST = 2 * RH + 2;  // token tiles of W needed
    h8 kbf[2][RH + 1];               // Kbar[:, tile 2kb+cc] per 32-token block, natural order
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int ks = 0; ks <= RH; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) kbf[cc][ks][e] = S.kh[(32 * ks + 8 * lg + e) * KP + 16 * (2 * kb + cc) + lr];
    h8 tn[4][RH + 1];  // Tm rows, natural token order
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int ks = 0; ks <= RH; ++ks)
            tn[st][ks] = *reinterpret_cast<const h8 *>(&S.t16[(16 * st + lr) * SP + 32 * ks + 8 * lg]);
    f4 wt[4][2];
#pragma unroll
    for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            wt[st][cc] = mfma32(tn[st][0], kbf[cc][0], splat(0.f));
            if (st >= 2) wt[st][cc] = mfma32(tn[st][1], kbf[cc][RH], wt[st][cc]);
        }
    bool big = false;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int rt = 2 * RH + rr;
        f4 wT[2], qT[2];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            wT[cc] = mfma32(kbf[cc][0], tn[rt][0], splat(0.f));
            if (RH) wT[cc] = mfma32(kbf[cc][RH], tn[rt][RH], wT[cc]);
            qT[cc] = to_f4(*reinterpret_cast<const h4 *>(&S.qh[(16 * rt + lr) * KP + 16 * (2 * kb + cc) + 4 * lg]));
#pragma unroll
            for (int ks = 0; ks <= RH; ++ks) {
                const h8 wa = join(to_h4(wt[2 * ks][cc]), to_h4(wt[2 * ks + 1][cc]));
                qT[cc] = mfma32(-wa, perm_frag(S.r16, rt, ks, lr, lg), qT[cc]);
            }
            big |= out_of_range(wT[cc]) || out_of_range(qT[cc]);
        }
        const int64_t o = ((rt * 4 + kb) * 64 + lane) * 8;
        *reinterpret_cast<h8 *>(rec + OFF_W + o) = join(to_h4(wT[0]), to_h4(wT[1]));
        *reinterpret_cast<h8 *>(rec + OFF_Q + o) = join(to_h4(qT[0]), to_h4(qT[1]));
    }
    return big;
}

template <bool TIED, bool KEYG>
__global__ void __launch_bounds__(NTH) chunk_prep_kernel(ChunkArgs a, SplitWs w, int nc) {
    __shared__ PrepSmem S;
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t ntask = a.B * a.H * nc;

    // zero the upper blocks of the C x C operands once; they are never written
    for (int idx = tid; idx < C * SP; idx += NTH) {
        S.t16[idx] = (_Float16)0.f;
        S.b16[idx] = (_Float16)0.f;
        S.r16[idx] = (_Float16)0.f;
        S.p16[idx] = (_Float16)0.f;
    }
    if (tid == 0) S.wide = 0;

    Raw<KEYG, 2> R;
    int64_t task = blockIdx.x;
    if (task < ntask) {
        const TaskPos p0 = task_pos(task, nc, static_cast<int>(a.H));
        load_part<0, TIED>(R, a, p0, tid);
        load_part<1, TIED>(R, a, p0, tid);
        load_part<2, TIED>(R, a, p0, tid);
        load_part<3, TIED>(R, a, p0, tid);
    }

    for (; task < ntask; task += gridDim.x) {
        __syncthreads();  // previous task done with every buffer
        // lane coordinates, re-derived every task so that the LDS addresses
        // built from them are not hoisted out of the loop (and spilled)
        int tl = tid;
        asm volatile("" : "+v"(tl));
        const int lane = tl & 63, lr = lane & 15, lg = lane >> 4;
        const int seg = tl >> 5, cq = tl & 31;

        // ---- values [j][s]: each thread packs its two tokens of one column
        //      into a 32-bit word (a wave's writes then hit 64 distinct banks);
        //      segment log2-decay totals
        {
            const int tp = tl & 31, piece = tl >> 5;
            const uint32_t r0[4] = {R.v[0].x, R.v[0].y, R.v[0].z, R.v[0].w};
            const uint32_t r1[4] = {R.v[1].x, R.v[1].y, R.v[1].z, R.v[1].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const _Float16 a0 = (_Float16)__uint_as_float(r0[e] << 16), a1 = (_Float16)__uint_as_float(r1[e] << 16);
                const _Float16 b0 = (_Float16)__uint_as_float(r0[e] & 0xffff0000u);
                const _Float16 b1 = (_Float16)__uint_as_float(r1[e] & 0xffff0000u);
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                *reinterpret_cast<h2 *>(&S.v16[(8 * piece + 2 * e) * SP + 2 * tp]) = h2{a0, a1};
                *reinterpret_cast<h2 *>(&S.v16[(8 * piece + 2 * e + 1) * SP + 2 * tp]) = h2{b0, b1};
            }
        }
        f4 g[RPS];
        segment_cumsum(S, R, g, seg, cq);
        __syncthreads();
        if (tid < D) chunk_tables(S, tid);
        __syncthreads();

        // ---- factored fp16 Gram operands -------------------------------------
        f4 khf[RPS], qhf[RPS], egm;
        factored_operands<PrepSmem, TIED>(S, R, g, khf, qhf, egm, seg, cq, a.q_scale);
        const int64_t next = task + gridDim.x;  // prefetched in four parts below
        const TaskPos pn = task_pos(next < ntask ? next : task, nc, static_cast<int>(a.H));
        if (next < ntask) load_part<0, TIED>(R, a, pn, tid);
        __syncthreads();

        const bool wide = S.wide != 0;  // read by all before any later write
        if (!wide) {
            // ---- Grams: waves 0..3 one diagonal tile each, inverted at once;
            //      waves 4..7 the six off-diagonal tiles
            if (wv < 4) {
                gram_tile<PrepSmem, TIED>(S, wv, wv, lr, lg);
                invert_unit_lower16(&S.af[(16 * wv) * AP + 16 * wv], &S.t16[(16 * wv) * SP + 16 * wv],
                                    S.iscr[wv][0], S.iscr[wv][1], lr, lg);
            } else {
                const int u = wv - 4;  // off-diagonal tiles u and u + 4 (< 6)
                gram_tile<PrepSmem, TIED>(S, kOffI[u], kOffJ[u], lr, lg);
                if (u < 2) gram_tile<PrepSmem, TIED>(S, kOffI[u + 4], kOffJ[u + 4], lr, lg);
            }
        }
        __syncthreads();

        if (!wide) {
            // ---- Kbar = k 2^g, Qbar = q 2^g, in place of the row operands
#pragma unroll
            for (int i = 0; i < RPS; ++i) {
                const int r = RPS * seg + i;
                *reinterpret_cast<h4 *>(&S.kh[r * KP + 4 * cq]) = to_h4(khf[i] * egm);
                *reinterpret_cast<h4 *>(&S.qh[r * KP + 4 * cq]) = to_h4(qhf[i] * egm);
            }
        }
        if (next < ntask) load_part<1, TIED>(R, a, pn, tid);

        _Float16 *rec = w.frag + task * REC;
        if (!wide) {
            // ---- Tm = (I + A)^-1 (diagonal blocks were inverted with the Grams)
            solve_offdiag(S, wv, lr, lg);
            // Only the products below are range-checked: an fp16 Gram or Tm
            // entry that overflowed is inf and turns every product it enters
            // into inf or NaN.  All LDS reads of this phase come before its
            // LDS writes, so the compiler may issue them early.
            bool big = false;

            // ---- (1) value tile ct = wv: Y = Bm V, U = Tm Y ------------------
            const int ct = wv;
            h8 vb[2];  // V[:, ct] as a B operand, natural token order
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) vb[ks] = *reinterpret_cast<const h8 *>(&S.v16[(16 * ct + lr) * SP + 32 * ks + 8 * lg]);
            f4 y[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                y[rt] = splat(0.f);
#pragma unroll
                for (int ks = 0; ks <= (rt >> 1); ++ks)
                    y[rt] = mfma32(*reinterpret_cast<const h8 *>(&S.b16[(16 * rt + lr) * SP + 32 * ks + 8 * lg]), vb[ks], y[rt]);
                big |= out_of_range(y[rt]);
            }
            f4 uacc[4];
            {
                const h8 yb0 = join(to_h4(y[0]), to_h4(y[1])), yb1 = join(to_h4(y[2]), to_h4(y[3]));
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    uacc[rt] = mfma32(perm_frag(S.t16, rt, 0, lr, lg), yb0, splat(0.f));
                    if (rt >= 2) uacc[rt] = mfma32(perm_frag(S.t16, rt, 1, lr, lg), yb1, uacc[rt]);
                    big |= out_of_range(uacc[rt]);
                }
            }

            // ---- (2) key channel tiles 2kb, 2kb+1: W^T and Qe^T -> HBM -------
            if (wv >= 4)
                big |= wq_tiles<1>(S, rec, wv & 3, lane, lr, lg);
            else
                big |= wq_tiles<0>(S, rec, wv & 3, lane, lr, lg);

            // ---- (3) key channel tile it = wv: Etil^T, Util^T fragments
            //      (chunk-end reference: column operand times 2^(gC - gm_j))
            const int it = wv;
            h8 ef[2], uf[2];
            {
                const int c = 16 * it + lr;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const float f0 = S.fsc[2 * kb][c], f1 = S.fsc[2 * kb + 1][c];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s0 = 32 * kb + 4 * lg + e, s1 = s0 + 16;
                        ef[kb][e] = (_Float16)((float)S.eh[s0 * KP + c] * f0);
                        ef[kb][e + 4] = (_Float16)((float)S.eh[s1 * KP + c] * f1);
                        if (!TIED) {
                            uf[kb][e] = (_Float16)((float)S.uh[s0 * KP + c] * f0);
                            uf[kb][e + 4] = (_Float16)((float)S.uh[s1 * KP + c] * f1);
                        }
                    }
                    if (TIED) uf[kb] = ef[kb];
                    *reinterpret_cast<h8 *>(rec + OFF_E + ((it * 2 + kb) * 64 + lane) * 8) = ef[kb];
                }
            }
            // U -> u16 [j][s] for the value-column products of every wave
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                *reinterpret_cast<h4 *>(&S.u16[(16 * ct + lr) * SP + 16 * rt + 4 * lg]) = to_h4(uacc[rt]);
            if (big) S.wide = 1;
            __syncthreads();  // U complete in u16
            if (next < ntask) load_part<2, TIED>(R, a, pn, tid);

            // ---- (4) Oe[:, ct] = P V - R U -> HBM ----------------------------
            {
                const _Float16 *pp = TIED ? S.r16 : S.p16;
                const h8 ub0 = join(to_h4(uacc[0]), to_h4(uacc[1])), ub1 = join(to_h4(uacc[2]), to_h4(uacc[3]));
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    f4 acc = splat(0.f);
#pragma unroll
                    for (int ks = 0; ks <= (rt >> 1); ++ks) {
                        acc = mfma32(*reinterpret_cast<const h8 *>(&pp[(16 * rt + lr) * SP + 32 * ks + 8 * lg]), vb[ks], acc);
                        acc = mfma32(perm_frag(S.r16, rt, ks, lr, lg), ks ? -ub1 : -ub0, acc);
                    }
                    big |= out_of_range(acc);
                    *reinterpret_cast<h4 *>(rec + OFF_O + ((ct * 4 + rt) * 64 + lane) * 4) = to_h4(acc);
                }
            }
            // ---- (5) G[it, :] = Util^T V - Etil^T U -> HBM -------------------
            {
                const h8 ne0 = -ef[0], ne1 = -ef[1];
#pragma unroll
                for (int c2 = 0; c2 < 8; ++c2) {
                    f4 acc = splat(0.f);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) {
                        const _Float16 *pv = &S.v16[(16 * c2 + lr) * SP + 32 * kb + 4 * lg];
                        const _Float16 *pu = &S.u16[(16 * c2 + lr) * SP + 32 * kb + 4 * lg];
                        const h8 vp = join(*reinterpret_cast<const h4 *>(pv), *reinterpret_cast<const h4 *>(pv + 16));
                        const h8 up = join(*reinterpret_cast<const h4 *>(pu), *reinterpret_cast<const h4 *>(pu + 16));
                        acc = mfma32(uf[kb], vp, acc);
                        acc = mfma32(kb ? ne1 : ne0, up, acc);
                    }
                    big |= out_of_range(acc);
                    *reinterpret_cast<h4 *>(rec + OFF_G + ((c2 * 8 + it) * 64 + lane) * 4) = to_h4(acc);
                }
            }
            if (big) S.wide = 1;
            if (tid < D) w.gam[task * D + tid] = S.gce[tid];
        } else if (next < ntask) {
            load_part<2, TIED>(R, a, pn, tid);
        }
        if (next < ntask) load_part<3, TIED>(R, a, pn, tid);
        __syncthreads();
        if (tid == 0) {
            w.flag[task] = (wide || S.wide) ? 1 : 0;
            S.wide = 0;
        }
    }
}

// ----------------------------------------------------------------------------
// Pass 2: the scan over chunks.  One wave = one chain x NB value tiles.
// The per-chunk operands a wave of NB value tiles needs besides W, Qe, EtT.
template <int NB>
struct ScanSmall {
    h4 g[NB][8], o[NB][4];
    f4 gam[8];
    int flag;
};

__device__ __forceinline__ void load_wq(h8 (&x)[4][4], const _Float16 *p, int lane) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) x[rt][kb] = *reinterpret_cast<const h8 *>(p + ((rt * 4 + kb) * 64 + lane) * 8);
}
__device__ __forceinline__ void load_e(h8 (&x)[8][2], const _Float16 *p, int lane) {
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) x[it][kb] = *reinterpret_cast<const h8 *>(p + ((it * 2 + kb) * 64 + lane) * 8);
}

template <int NB, bool TIED, bool KEYG>
__global__ void __launch_bounds__(64) chunk_scan_kernel(ChunkArgs a, SplitWs w, int nc, int ngrp, int xcd_map) {
    const int L = blockIdx.x;
    int chain, grp;
    if (xcd_map) {  // a chain's waves on one XCD, so its records are read into one L2
        grp = (L / 8) % ngrp;
        chain = (L / (8 * ngrp)) * 8 + (L % 8);
    } else {
        grp = L % ngrp;
        chain = L / ngrp;
    }
    const int64_t b = chain / a.H, h = chain % a.H;
    const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;
    const int ct0 = grp * NB;
    const int64_t sbase = (b * a.H + h) * static_cast<int64_t>(D) * D;

    // state slice: tile (n, it) holds S[16it+4lg+e][16(ct0+n)+lr]
    f4 sacc[NB][8];
#pragma unroll
    for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t c = 16 * it + 4 * lg + e, v = 16 * (ct0 + n) + lr;
                sacc[n][it][e] = a.s0 ? a.s0[sbase + c * D + v] : 0.f;
            }

    // Every operand of chunk n+1 is requested while chunk n is computed (each
    // right after its last use in chunk n), so the scan waits on memory only
    // when a chunk's compute is shorter than the load latency.
    const int64_t task0 = static_cast<int64_t>(chain) * nc;
    h8 wf[4][4], qf[4][4], ef[8][2];
    ScanSmall<NB> cur, nx;
    auto load_small = [&](ScanSmall<NB> &x, int64_t task) {
        const _Float16 *rec = w.frag + task * REC;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
#pragma unroll
            for (int it = 0; it < 8; ++it)
                x.g[j][it] = *reinterpret_cast<const h4 *>(rec + OFF_G + (((ct0 + j) * 8 + it) * 64 + lane) * 4);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                x.o[j][rt] = *reinterpret_cast<const h4 *>(rec + OFF_O + (((ct0 + j) * 4 + rt) * 64 + lane) * 4);
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) x.gam[it] = *reinterpret_cast<const f4 *>(&w.gam[task * D + 16 * it + 4 * lg]);
        x.flag = w.flag[task];
    };
    load_wq(wf, w.frag + task0 * REC + OFF_W, lane);
    load_wq(qf, w.frag + task0 * REC + OFF_Q, lane);
    load_e(ef, w.frag + task0 * REC + OFF_E, lane);
    load_small(cur, task0);

    for (int n = 0; n < nc; ++n) {
        const int64_t t0 = static_cast<int64_t>(n) * C;
        const int64_t nxt = task0 + (n + 1 < nc ? n + 1 : n);
        load_small(nx, nxt);

        // the fp16 copies of the state and of the erase read must stay finite
        bool big = false;
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int it = 0; it < 8; ++it) big |= !(fmaxf(fmaxf(fabsf(sacc[j][it][0]), fabsf(sacc[j][it][1])),
                                                          fmaxf(fabsf(sacc[j][it][2]), fabsf(sacc[j][it][3]))) <= 16384.f);
        bool bad = cur.flag != 0 || __ballot(big) != 0;
        f4 p1[NB][4], oacc[NB][4];
        big = false;
        if (!bad) {
            // P1 = W S and O = Qe S + Oe; the state tiles 2kb, 2kb+1 form the
            // B operand of key block kb in the permuted slot order
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                h8 sb[4];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) sb[kb] = join(to_h4(sacc[j][2 * kb]), to_h4(sacc[j][2 * kb + 1]));
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    f4 p = splat(0.f), o = to_f4(cur.o[j][rt]);
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) {
                        p = mfma32(wf[rt][kb], sb[kb], p);
                        o = mfma32(qf[rt][kb], sb[kb], o);
                    }
                    p1[j][rt] = p;
                    oacc[j][rt] = o;
                    big |= out_of_range(p);
                }
            }
        }
        // W and Qe of this chunk are consumed: fetch the next chunk's
        load_wq(wf, w.frag + nxt * REC + OFF_W, lane);
        load_wq(qf, w.frag + nxt * REC + OFF_Q, lane);

        bad = bad || __ballot(big) != 0;
        if (!bad) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int64_t col = 16 * (ct0 + j) + lr;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t t = t0 + 16 * rt + 4 * lg + e;
                        if (t < a.T) a.o[((b * a.T + t) * a.H + h) * D + col] = oacc[j][rt][e];
                    }
                // S <- Diag(e^gC) S + G - Etil^T P1, tokens in permuted slots
                const h8 pb0 = join(to_h4(-p1[j][0]), to_h4(-p1[j][1]));
                const h8 pb1 = join(to_h4(-p1[j][2]), to_h4(-p1[j][3]));
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    f4 s = cur.gam[it] * sacc[j][it] + to_f4(cur.g[j][it]);
                    s = mfma32(ef[it][0], pb0, s);
                    s = mfma32(ef[it][1], pb1, s);
                    sacc[j][it] = s;
                }
            }
        } else {
            // exact fp32 token recurrence on the raw inputs of this chunk
            const uint16_t *kp = static_cast<const uint16_t *>(a.k);
            const uint16_t *qp = static_cast<const uint16_t *>(a.q);
            const uint16_t *vp = static_cast<const uint16_t *>(a.v);
            const int gw = KEYG ? D : 1;
            for (int r = 0; r < C && t0 + r < a.T; ++r) {
                const int64_t row = (b * a.T + t0 + r) * a.H + h;
                // gates of key channel c of this token (per channel or per head)
                auto gate = [&](const float *g, int c) { return g[row * gw + (KEYG ? c : 0)]; };
                float m[NB], o[NB];
#pragma unroll
                for (int j = 0; j < NB; ++j) m[j] = o[j] = 0.f;
                // decay, then the erase read m = k^T S_bar
#pragma unroll
                for (int it = 0; it < 8; ++it)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 16 * it + 4 * lg + e;
                        const float ac = expf(gate(a.la, c)), kc = bf16_to_f32(kp[row * D + c]);
#pragma unroll
                        for (int j = 0; j < NB; ++j) {
                            sacc[j][it][e] *= ac;
                            m[j] += kc * sacc[j][it][e];
                        }
                    }
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    m[j] += __shfl_xor(m[j], 16);
                    m[j] += __shfl_xor(m[j], 32);
                }
                float vv[NB];
#pragma unroll
                for (int j = 0; j < NB; ++j) vv[j] = bf16_to_f32(vp[row * D + 16 * (ct0 + j) + lr]);
                // erase and write, then the read o = S^T q
#pragma unroll
                for (int it = 0; it < 8; ++it)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 16 * it + 4 * lg + e;
                        const float kc = bf16_to_f32(kp[row * D + c]);
                        const float bb = gate(a.eb, c);
                        const float ec = bb * kc, uc = (TIED ? bb : gate(a.wr, c)) * kc;
                        const float qc = a.q_scale * bf16_to_f32(qp[row * D + c]);
#pragma unroll
                        for (int j = 0; j < NB; ++j) {
                            sacc[j][it][e] = sacc[j][it][e] - ec * m[j] + uc * vv[j];
                            o[j] += qc * sacc[j][it][e];
                        }
                    }
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    o[j] += __shfl_xor(o[j], 16);
                    o[j] += __shfl_xor(o[j], 32);
                    if (lg == 0) a.o[row * D + 16 * (ct0 + j) + lr] = o[j];
                }
            }
        }
        load_e(ef, w.frag + nxt * REC + OFF_E, lane);
        cur = nx;
    }

    if (a.s_out) {
#pragma unroll
        for (int n = 0; n < NB; ++n)
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t c = 16 * it + 4 * lg + e, v = 16 * (ct0 + n) + lr;
                    a.s_out[sbase + c * D + v] = sacc[n][it][e];
                }
    }
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

SplitWs carve(const ChunkArgs &a, void *ws) {
    const int64_t ntask = a.B * a.H * ((a.T + C - 1) / C);
    char *p = static_cast<char *>(ws);
    SplitWs w;
    w.frag = reinterpret_cast<_Float16 *>(p);
    p += align256(ntask * REC * 2);
    w.gam = reinterpret_cast<float *>(p);
    p += align256(ntask * D * 4);
    w.flag = reinterpret_cast<int *>(p);
    return w;
}

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

template <bool TIED, bool KEYG>
hipError_t launch_kinds(const ChunkArgs &a, void *ws, hipStream_t s) {
    const int nc = static_cast<int>((a.T + C - 1) / C);
    const int64_t chains = a.B * a.H, ntask = chains * nc;
    const SplitWs w = carve(a, ws);
    const int64_t g1 = ntask < cu_count() ? ntask : cu_count();
    hipLaunchKernelGGL((chunk_prep_kernel<TIED, KEYG>), dim3(static_cast<unsigned>(g1)), dim3(NTH), 0, s, a, w, nc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int xcd_map = (chains % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((chunk_scan_kernel<1, TIED, KEYG>), dim3(static_cast<unsigned>(chains * 8)), dim3(64), 0, s,
                       a, w, nc, 8, xcd_map);
    return hipGetLastError();
}

}  // namespace

bool chunk_split_supported(const ChunkArgs &a) {
    // the kernels index tasks (chain * chunks + chunk) with 32-bit arithmetic
    const int64_t ntask = a.B * a.H * ((a.T + C - 1) / C);
    return chunk_mfma_supported(a) && ntask > 0 && ntask < (int64_t(1) << 31);
}

size_t chunk_split_workspace(int64_t B, int64_t H, int64_t T) {
    const int64_t ntask = B * H * ((T + C - 1) / C);
    return static_cast<size_t>(align256(ntask * REC * 2) + align256(ntask * D * 4) + align256(ntask * 4));
}

hipError_t launch_chunk_split(const ChunkArgs &a, void *ws, hipStream_t s) {
    const bool tied = a.wr == nullptr, keyg = a.la_key != 0;
    if (tied) return keyg ? launch_kinds<true, true>(a, ws, s) : launch_kinds<true, false>(a, ws, s);
    return keyg ? launch_kinds<false, true>(a, ws, s) : launch_kinds<false, false>(a, ws, s);
}

}  // namespace gdn2
