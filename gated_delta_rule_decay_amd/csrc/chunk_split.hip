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
// plus e^gC (which also carries the exact-path mark).  Pass 2 (chunk_scan_kernel) gives each wave one
// chain and 16*NB value columns; the fp32 state slice (128 x 16*NB) stays in
// MFMA accumulators, every operand is one coalesced 16-byte load per lane,
// and waves never synchronise, so a chain's value columns proceed on as
// many CUs as there are waves.
//
// A chunk whose fp16 factors, operands or results would leave the fast
// range is flagged by pass 1; pass 2 runs it as the exact fp32 token
// recurrence on the raw inputs instead (so does a chunk whose state or erase
// read would overflow fp16).
#include <utility>

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
//   G      [ct 8][ip 4][lane 64][8]  accumulator tiles it = 2ip, 2ip+1: lane
//                                    j+16m holds G[16it+4m+e][16ct+j] in
//                                    elements 4(it&1)+e
//   OeT    [ct 8][rp 2][lane 64][8]  transposed tiles rt = 2rp, 2rp+1: lane
//                                    t+16m holds Oe[16rt+t][16ct+4m+e] in
//                                    elements 4(rt&1)+e (four adjacent value
//                                    columns of one token)
constexpr int64_t OFF_W = 0;
constexpr int64_t OFF_Q = 8192;
constexpr int64_t OFF_E = 16384;
constexpr int64_t OFF_G = 24576;
constexpr int64_t OFF_O = 40960;
constexpr int64_t REC = 49152;
constexpr float MAX_RESULT = 30000.f;  // largest |fp16 value| a record may hold

struct SplitWs {
    _Float16 *frag;  // [task][REC]
    float *gam;      // [task][D]   e^gC per key channel; -1 in channel 0 marks
                     //             a chunk to be run as the exact recurrence
    // packed sequences only (built on the device from the offsets):
    const int2 *vseq;  // [N]    token range [lo, hi) of each sequence
    const int *vpfx;   // [N+1]  chunks before each sequence; vpfx[N]: all chunks
    const int2 *vtab;  // [chunk] first token of each chunk, end of its sequence
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
// Token positions count over the flattened [B*T] token axis.
struct TaskPos {
    int64_t h, t0, tlim;  // head, first token, end of the chunk's sequence
};

// Position of task `task`: chain * nc + chunk for B sequences of T tokens;
// for packed sequences chunk-major (task = chunk * H + head, chunks of all
// sequences in order), placed by the chunk table.  32-bit division (the task
// count is checked to fit on the host).
__device__ __forceinline__ TaskPos task_pos(const ChunkArgs &a, const SplitWs &w, int64_t task, int nc) {
    const uint32_t t = static_cast<uint32_t>(task), H = static_cast<uint32_t>(a.H);
    TaskPos p;
    if (a.cu) {
        const uint32_t gc = t / H;
        const int2 e = w.vtab[gc];
        p.h = t - gc * H;
        p.t0 = e.x;
        p.tlim = e.y;
    } else {
        const uint32_t chain = t / static_cast<uint32_t>(nc), b = chain / H;
        p.h = chain - b * H;
        p.t0 = static_cast<int64_t>(b) * a.T + static_cast<int64_t>(t - chain * static_cast<uint32_t>(nc)) * C;
        p.tlim = static_cast<int64_t>(b) * a.T + a.T;
    }
    return p;
}

template <int PART, bool TIED, bool KEYG, bool VW = false, bool RAW = false>
__device__ __forceinline__ void load_part(Raw<KEYG, 2> &R, const ChunkArgs &a, const TaskPos &tp0, int tid) {
    const bool logits = RAW && a.gate_logits;  // bf16 gate logits (fused input preparation)
    const int64_t b = 0, h = tp0.h, t0 = tp0.t0, tl = tp0.tlim;
    const int seg = tid >> 5, cq = tid & 31;
    const int gw = KEYG ? D : 1;
    const int rowk = static_cast<int>(a.H) * D, rowg = static_cast<int>(a.H) * gw;
    auto gates = [&](GateRow<KEYG> &x, const float *src) {
        if (logits) {  // bf16 logits: raw bits, activated where used
            const auto rs = chain_rsrc(src, a, b, h, t0, gw, 2, 0, tl);
#pragma unroll
            for (int i = 0; i < RPS; ++i) {
                const int r = seg * RPS + i;
                if constexpr (KEYG) {
                    const uint2 u = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, (r * rowg + 4 * cq) * 2, 0, 0));
                    x.x[i] = f4{__uint_as_float(u.x), __uint_as_float(u.y), 0.f, 0.f};
                } else {
                    x.x[i] = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rs, r * rowg * 2, 0, 0)));
                }
            }
            return;
        }
        const auto rs = chain_rsrc(src, a, b, h, t0, gw, 4, 0, tl);
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
        const auto rv = chain_rsrc(a.v, a, b, h, t0, D, 2, 0, tl);
        const int tp = tid & 31, piece = tid >> 5;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            R.v[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, ((2 * tp + i) * rowk + 8 * piece) * 2, 0, 0));
        if constexpr (VW) {
            // write gate of my two tokens' 8 value columns (per channel) or
            // of my two tokens (per head), into the unused wr registers
            // (bf16 logits: the 8 columns of token i in wr.x[2i])
            const int es = logits ? 2 : 4;
            const auto rw = chain_rsrc(a.wr, a, b, h, t0, gw, es, 0, tl);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if constexpr (KEYG) {
                    if (logits) {
                        R.wr.x[2 * i] = __builtin_bit_cast(
                            f4, __builtin_amdgcn_raw_buffer_load_b128(rw, ((2 * tp + i) * rowg + 8 * piece) * 2, 0, 0));
                    } else {
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh)
                            R.wr.x[2 * i + hh] = __builtin_bit_cast(
                                f4, __builtin_amdgcn_raw_buffer_load_b128(rw, ((2 * tp + i) * rowg + 8 * piece + 4 * hh) * 4, 0, 0));
                    }
                } else if (logits) {
                    R.wr.x[i] = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rw, (2 * tp + i) * rowg * 2, 0, 0)));
                } else {
                    R.wr.x[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rw, (2 * tp + i) * rowg * 4, 0, 0));
                }
            }
        }
    }
    if constexpr (PART == 3) {
        const auto rk = chain_rsrc(a.k, a, b, h, t0, D, 2, 0, tl);
        const auto rq = chain_rsrc(a.q, a, b, h, t0, D, 2, 0, tl);
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
            if (st >= 2) wt[st][cc] = mfma32(tn[st][RH], kbf[cc][RH], wt[st][cc]);
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

template <bool TIED, bool KEYG, bool VW, bool RAW>
__global__ void __launch_bounds__(NTH) chunk_prep_kernel(ChunkArgs a, SplitWs w, int nc) {
    // RAW: fused input preparation (bf16 gate logits and / or q, k normalised here)
    const int logits = RAW ? a.gate_logits : 0, qknorm = RAW ? a.qk_norm : 0;
    __shared__ PrepSmem S;
    const int tid = threadIdx.x;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t ntask = a.cu ? a.H * w.vpfx[a.B] : a.B * a.H * nc;

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
    TaskPos cur{0, 0, 0};
    if (task < ntask) {
        const TaskPos p0 = task_pos(a, w, task, nc);
        cur = p0;
        load_part<0, TIED, KEYG, VW, RAW>(R, a, p0, tid);
        load_part<1, TIED, KEYG, VW, RAW>(R, a, p0, tid);
        load_part<2, TIED, KEYG, VW, RAW>(R, a, p0, tid);
        load_part<3, TIED, KEYG, VW, RAW>(R, a, p0, tid);
    }

    for (; task < ntask; task += gridDim.x) {
        __syncthreads();  // previous task done with every buffer (and with S.wide)
        if (tid == 0) S.wide = 0;
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
            // the value-write form writes w .* v: gate of token i, column 2e + s
            auto wg = [&](int i, int e, int s) -> float {
                if constexpr (!VW) {
                    return 1.f;
                } else if constexpr (KEYG) {
                    if (logits) {  // column 2e+s of token i: half s of word e
                        const uint32_t u = __float_as_uint(R.wr.x[2 * i][e]);
                        return sigmoid_gate(__uint_as_float(s ? (u & 0xffff0000u) : (u << 16)));
                    }
                    return R.wr.x[2 * i + (2 * e + s) / 4][(2 * e + s) % 4];
                } else {
                    return logits ? sigmoid_gate(__uint_as_float(__float_as_uint(R.wr.x[i]) << 16)) : R.wr.x[i];
                }
            };
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const _Float16 a0 = (_Float16)(__uint_as_float(r0[e] << 16) * wg(0, e, 0));
                const _Float16 a1 = (_Float16)(__uint_as_float(r1[e] << 16) * wg(1, e, 0));
                const _Float16 b0 = (_Float16)(__uint_as_float(r0[e] & 0xffff0000u) * wg(0, e, 1));
                const _Float16 b1 = (_Float16)(__uint_as_float(r1[e] & 0xffff0000u) * wg(1, e, 1));
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                *reinterpret_cast<h2 *>(&S.v16[(8 * piece + 2 * e) * SP + 2 * tp]) = h2{a0, a1};
                *reinterpret_cast<h2 *>(&S.v16[(8 * piece + 2 * e + 1) * SP + 2 * tp]) = h2{b0, b1};
            }
        }
        f4 g[RPS];
        segment_cumsum(S, R, g, seg, cq, logits, RAW ? cur.tlim - cur.t0 : C);
        __syncthreads();
        if (tid < D) chunk_tables(S, tid);
        __syncthreads();

        // ---- factored fp16 Gram operands -------------------------------------
        f4 khf[RPS], qhf[RPS], egm;
        factored_operands<PrepSmem, TIED, KEYG, 2, VW>(S, R, g, khf, qhf, egm, seg, cq, a.q_scale, logits, qknorm);
        const int64_t next = task + gridDim.x;  // prefetched in four parts below
        TaskPos pn = task_pos(a, w, next < ntask ? next : task, nc);
        // Without a next task the loads still issue, over an empty range (they
        // read zeros and touch no memory): every path through the loop then
        // has the same memory operations in flight, so the waits before the
        // first use of each part count only what was issued after it.
        if (next >= ntask) pn.tlim = pn.t0;
        load_part<0, TIED, KEYG, VW, RAW>(R, a, pn, tid);
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
        load_part<1, TIED, KEYG, VW, RAW>(R, a, pn, tid);

        _Float16 *rec = w.frag + task * REC;
        bool big = false;
        const int ct = wv, it = wv;  // value tile, key channel tile of this wave
        h8 vb[2], ef[2], uf[2];
        f4 uacc[4];
        if (!wide) {
            // ---- Tm = (I + A)^-1 (diagonal blocks were inverted with the Grams)
            solve_offdiag(S, wv, lr, lg);
            // Only the products below are range-checked: an fp16 Gram or Tm
            // entry that overflowed is inf and turns every product it enters
            // into inf or NaN.  All LDS reads of this phase come before its
            // LDS writes, so the compiler may issue them early.

            // ---- (1) value tile ct = wv: Y = Bm V, U = Tm Y ------------------
            // vb: V[:, ct] as a B operand, natural token order
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
        }
        __syncthreads();  // U complete in u16
        load_part<2, TIED, KEYG, VW, RAW>(R, a, pn, tid);
        if (!wide) {
            // ---- (4) Oe^T[ct, :] = V^T P^T - U^T R^T -> HBM (transposed, so
            //      the scan's output tiles hold adjacent columns per lane)
            {
                const _Float16 *pp = TIED ? S.r16 : S.p16;
                const h8 ub0 = join(to_h4(uacc[0]), to_h4(uacc[1])), ub1 = join(to_h4(uacc[2]), to_h4(uacc[3]));
                f4 acc[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    acc[rt] = splat(0.f);
#pragma unroll
                    for (int ks = 0; ks <= (rt >> 1); ++ks) {
                        acc[rt] = mfma32(vb[ks], *reinterpret_cast<const h8 *>(&pp[(16 * rt + lr) * SP + 32 * ks + 8 * lg]), acc[rt]);
                        acc[rt] = mfma32(ks ? -ub1 : -ub0, perm_frag(S.r16, rt, ks, lr, lg), acc[rt]);
                    }
                    big |= out_of_range(acc[rt]);
                }
#pragma unroll
                for (int rp = 0; rp < 2; ++rp)
                    *reinterpret_cast<h8 *>(rec + OFF_O + ((ct * 2 + rp) * 64 + lane) * 8) =
                        join(to_h4(acc[2 * rp]), to_h4(acc[2 * rp + 1]));
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
                    *reinterpret_cast<h4 *>(rec + OFF_G + ((c2 * 4 + (it >> 1)) * 64 + lane) * 8 + 4 * (it & 1)) = to_h4(acc);
                }
            }
            if (big) S.wide = 1;
        }
        load_part<3, TIED, KEYG, VW, RAW>(R, a, pn, tid);
        __syncthreads();
        // e^gC per key channel; a chunk to be run exactly is marked by -1 in
        // channel 0 (e^gC is never negative)
        const bool exact = wide || S.wide;  // reset after the next task's first barrier
        if (tid < D) w.gam[task * D + tid] = (tid == 0 && exact) ? -1.f : S.gce[tid];
        cur = pn;
    }
}

// ----------------------------------------------------------------------------
// Pass 2: the scan over chunks.  A workgroup of SCAN_W compute waves owns one
// chain (or one segment of it, below) and SCAN_W value tiles (16 columns
// each, one per wave); each wave keeps its 128 x 16 fp32 state slice in
// accumulators.  Everything a chunk needs -- W, Qe, EtT (48 KiB, shared by
// the waves), the workgroup's slices of G and Oe and e^gC -- is copied by the
// memory unit straight into LDS (global_load_lds) one chunk ahead, into one
// of two slots, by SCAN_P copy waves of the same workgroup, so the compute
// waves never wait behind memory instructions; one barrier per chunk hands a
// slot over.
//
// Long sequences on few chains use the affine view of a chunk (the Gated
// DeltaNet page, "What makes the architecture more than a recurrence": each
// gated transition is still affine, S -> F S + G, and such maps compose): a
// chain's chunks are cut into segments, and
//   A (MODE 1)  every segment j but the last is scanned from S = 0, giving
//               its end state X[j+1], and its columns are also scanned from
//               S = I without the write terms, giving its transition F[j];
//               segment 0 starts from the chain's initial state instead (and
//               copies it to X[0]), so X[1] is already the state entering
//               segment 1;
//   B           X[j+1] <- F[j] X[j] + X[j+1] for j = 1, 2, ... in order
//               (segment_combine_kernel), so X[j] becomes the state entering
//               segment j;
//   C (MODE 0)  every segment j is scanned from X[j], writing O, and the
//               last one the final state.
// With one segment only C runs, as the plain scan, from the initial state.
// (Phase C never reads the initial state, so the final state may overwrite
// it in place.)
constexpr int SCAN_W = 4;                 // compute waves per value half (one tile each)
constexpr int SCAN_P = 4;                 // copy waves
constexpr int SLOT_F = 3 * 8192;          // halves of W | Qe | EtT
constexpr int SLOT_G = SCAN_W * 4 * 512;  // halves of G for my tiles (4 pair rows of 512)
constexpr int SLOT_O = SCAN_W * 2 * 512;  // halves of Oe^T for my tiles
constexpr int SLOT_H = SLOT_F + SLOT_G + SLOT_O;  // MODE 0 slot
constexpr int SLOT_A = 2 * 8192 + SLOT_G;         // MODE 1 slot: W | EtT | G
static_assert(SLOT_H * 2 % (1024 * SCAN_P) == 0 && SLOT_A * 2 % (1024 * SCAN_P) == 0,
              "slot copies must tile the copy waves");
constexpr int SEG_MIN = 16;   // fewest chunks per segment
constexpr int SEG_WG = 256;   // scan workgroups aimed at when chains are few

constexpr int scan_threads(int mode) { return 64 * (SCAN_P + (mode ? 2 : 1) * SCAN_W); }

// The exact fp32 token recurrence of one chunk on one wave's 16 state
// columns, from the raw inputs (the fallback when a chunk leaves the fp16
// range; the columns of F drop the write term).  Kept out of line: its
// registers do not burden the scan's fast path.
template <bool TIED, bool KEYG, bool VW, bool WITH_O>
__device__ __noinline__ void exact_chunk(ChunkArgs a, f4 *sacc, int64_t h, int64_t t0, int64_t tlim, int ct,
                                         int lr, int lg, bool frun) {
    const uint16_t *kp = static_cast<const uint16_t *>(a.k);
    const uint16_t *qp = static_cast<const uint16_t *>(a.q);
    const uint16_t *vp = static_cast<const uint16_t *>(a.v);
    for (int r = 0; r < C && t0 + r < tlim; ++r) {
        const int64_t row = (t0 + r) * a.H + h;
        // gates of channel c of this token (per channel or per head;
        // bf16 logits activated here)
        auto gate = [&](const float *g, int c, int act) {
            return load_gate_x(g, KEYG, row, D, c, a.gate_logits, act);
        };
        // 1 / ||k||, 1 / ||q|| of this token when normalised in the kernel
        float ik = 1.f, iq = 1.f;
        if (a.qk_norm) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 16 * it + 4 * lg + e;
                    const float kc = bf16_to_f32(kp[row * D + c]), qc = bf16_to_f32(qp[row * D + c]);
                    sk += kc * kc;
                    sq += qc * qc;
                }
            sk += __shfl_xor(sk, 16);
            sk += __shfl_xor(sk, 32);
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
            ik = sk > 0.f ? rsqrtf(sk) : 0.f;
            iq = sq > 0.f ? rsqrtf(sq) : 0.f;
        }
        float m = 0.f, o = 0.f;
        // decay, then the erase read m = k^T S_bar (the value-write
        // form reads along b .* k)
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * it + 4 * lg + e;
                sacc[it][e] *= expf(gate(a.la, c, 0));
                const float kc = ik * bf16_to_f32(kp[row * D + c]);
                m += (VW ? gate(a.eb, c, 1) * kc : kc) * sacc[it][e];
            }
        m += __shfl_xor(m, 16);
        m += __shfl_xor(m, 32);
        float vv = frun ? 0.f : bf16_to_f32(vp[row * D + 16 * ct + lr]);
        if (VW) vv *= gate(a.wr, 16 * ct + lr, 1);
        // erase and write, then the read o = S^T q
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * it + 4 * lg + e;
                const float kc = ik * bf16_to_f32(kp[row * D + c]);
                const float bb = gate(a.eb, c, 1);
                const float ec = VW ? kc : bb * kc;
                const float uc = VW ? kc : (TIED ? bb : gate(a.wr, c, 1)) * kc;
                sacc[it][e] = sacc[it][e] - ec * m + uc * vv;
                if (WITH_O) o += a.q_scale * iq * bf16_to_f32(qp[row * D + c]) * sacc[it][e];
            }
        if (WITH_O) {
            o += __shfl_xor(o, 16);
            o += __shfl_xor(o, 32);
            if (lg == 0) store_out(a.o, row * D + 16 * ct + lr, o, a.o_bf16);
        }
    }
}

// The workgroup barrier that hands a slot over.  The empty asm statements
// keep the compiler from moving LDS accesses across it (the barrier
// intrinsic alone does not order memory), without the waits a fence adds.
__device__ __forceinline__ void slot_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (other counters untouched)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

struct ScanPlan {
    int nseg;     // segments per chain (1: plain scan); packed: unused
    int seg_len;  // chunks per segment; the last one may be shorter
    float *xs;    // [chain][nseg][D][D] segment entry states X (packed: [slot][H][D][D])
    float *fs;    // [chain][nseg][D][D] segment transitions F (0 and nseg-1 unused)
    // packed sequences, [N+1] exclusive prefix counts over the sequences of:
    const int *qs;  // segments (the units of the scan proper)
    const int *q1;  // segments but each sequence's last (the units of the summaries)
    const int *zs;  // X / F slots (the segments of sequences cut in two or more)
    const int *c2;  // sequences cut in three or more (the units of the combine)
};

// Packed sequences: the last sequence i in [0, n) with pre[i] <= q (for q
// below pre[n], the one whose range of units holds q).
__device__ __forceinline__ int seq_of(const int *pre, int n, int q) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= q) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// MODE 0: the scan proper (O and, for the last segment, the final state).
// MODE 1: segment summaries; SCAN_W more compute waves carry the columns of
// F (the first SCAN_W carry the state), no Qe / Oe / O.
template <bool TIED, bool KEYG, bool VW, int MODE>
__global__ void __launch_bounds__(scan_threads(MODE))
chunk_scan_kernel(ChunkArgs a, SplitWs w, int nc, ScanPlan sp, int xcd_map) {
    constexpr bool WITH_O = MODE == 0;
    constexpr int NCOMP = (MODE ? 2 : 1) * SCAN_W;
    constexpr int SH = MODE ? SLOT_A : SLOT_H;
    constexpr int S_Q = 8192, S_E = MODE ? 8192 : 16384, S_G = MODE ? 16384 : SLOT_F, S_O = SLOT_F + SLOT_G;
    constexpr int PIECES = SH * 2 / 1024 / SCAN_P;  // 1 KiB copies per copy wave
    // two distinct slots (distinct objects, so the compiler can tell the slot
    // being filled from the one being read)
    __shared__ __attribute__((aligned(16))) _Float16 fr0[SH], fr1[SH];
    __shared__ __attribute__((aligned(16))) float gm0[2 * D], gm1[2 * D];
    const int G = blockIdx.x;
    int unit, half;
    if (xcd_map) {  // a unit's two workgroups on one XCD, so its records are read into one L2
        half = (G / 8) & 1;
        unit = (G / 16) * 8 + (G % 8);
    } else {
        half = G & 1;
        unit = G / 2;
    }
    // chunks [n0, n1) of this unit; chunk n is task task0 + n * tstr and
    // starts at token tbase + n * C of the flattened token axis; the
    // sequence ends at tlim.  The chain has nsegc segments; its segment slots
    // (X, F) are xbase + j xstep.
    int chain, seg, nsegc, n0, n1;
    int64_t h, task0, tstr, tbase, tlim, xbase, xstep;
    if (a.cu) {  // packed sequences: units are (segment, head), segment-major
        const int H = static_cast<int>(a.H), N = static_cast<int>(a.B);
        const int q = unit / H;
        const int *pre = MODE ? sp.q1 : sp.qs;  // the summaries skip each sequence's last segment
        if (q >= pre[N]) return;                 // launched for the bound (the whole workgroup)
        const int i = seq_of(pre, N, q), p0 = w.vpfx[i], nci = w.vpfx[i + 1] - p0;
        const int2 e = w.vseq[i];
        h = unit - q * H;
        seg = q - pre[i];
        nsegc = sp.qs[i + 1] - sp.qs[i];
        chain = i * H + static_cast<int>(h);
        n0 = seg * sp.seg_len;
        n1 = nsegc == 1 ? nci : min(nci, n0 + sp.seg_len);
        task0 = static_cast<int64_t>(p0) * a.H + h;
        tstr = a.H;
        tbase = e.x;
        tlim = e.y;
        xbase = ((static_cast<int64_t>(sp.zs[i]) + seg) * a.H + h) * D * D;
        xstep = a.H * D * D;
    } else {
        const int nsl = MODE ? sp.nseg - 1 : sp.nseg;  // segments per chain in this launch
        chain = unit / nsl;
        seg = unit % nsl;
        nsegc = sp.nseg;
        const int64_t b = chain / a.H;
        h = chain % a.H;
        n0 = seg * sp.seg_len;
        n1 = min(nc, n0 + sp.seg_len);
        task0 = static_cast<int64_t>(chain) * nc;
        tstr = 1;
        tbase = b * a.T;
        tlim = tbase + a.T;
        xbase = (static_cast<int64_t>(chain) * sp.nseg + seg) * D * D;  // slot seg
        xstep = D * D;
    }
    const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool copier = wv >= NCOMP;
    const bool frun = MODE && !copier && wv >= SCAN_W;  // this wave carries columns of F
    const bool idle = frun && seg == 0;                 // the first segment's F is never used
    const int wt = wv % SCAN_W;                          // my tile within the slot's slices
    const int ct = SCAN_W * half + (copier ? 0 : wt);   // my value (or key) tile
    const int64_t sbase = static_cast<int64_t>(chain) * D * D;

    f4 sacc[8];  // state slice (compute waves): tile it holds S[16it+4lg+e][16ct+lr]

    // Chunks travel memory -> copy-wave registers -> LDS slot.  While the
    // compute waves work on chunk n (one slot), the copy waves write chunk
    // n+1 from their registers into the other slot and issue the loads of
    // chunk n+2 into their registers, so two chunks' memory latency is always
    // in flight.  A slot holds W | Qe | EtT (MODE 1: W | EtT), then my
    // workgroup's G and Oe^T tiles (contiguous in the record), then e^gC.
    // Each wave moves 1 KiB per instruction (lane l -> bytes 16l..16l+15).
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    u4v cr[PIECES];
    float cgam = 0.f;
    auto load_regs = [&](int64_t task, int pw) __attribute__((always_inline)) {
        // one buffer resource per record: every piece is the same lane offset
        // plus a uniform byte offset, so no per-piece address registers
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(w.frag + task * REC, (short)0, static_cast<int>(REC * 2),
                                                          0x00020000);
        const int og = 2 * (static_cast<int>(OFF_G) + SCAN_W * half * 4 * 512);
        const int oo = 2 * (static_cast<int>(OFF_O) + SCAN_W * half * 2 * 512);
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
            const int byte = 1024 * (SCAN_P * i + pw);  // my 1 KiB block of the slot
            int src;
            if (MODE == 0)
                src = byte < 2 * SLOT_F ? byte
                    : byte < 2 * (SLOT_F + SLOT_G) ? og + (byte - 2 * SLOT_F)
                                                   : oo + (byte - 2 * (SLOT_F + SLOT_G));
            else
                src = byte < 2 * 8192 ? byte
                    : byte < 4 * 8192 ? 2 * static_cast<int>(OFF_E) + (byte - 2 * 8192)
                                      : og + (byte - 4 * 8192);
            cr[i] = __builtin_bit_cast(u4v, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, src, 0));
        }
        // e^gC: copy waves 0,1 bring channels 0..127
        if (pw < 2) cgam = w.gam[task * D + 64 * pw + lane];
    };
    auto store_regs = [&](_Float16 *fr, float *gm, int pw) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < PIECES; ++i)
            *reinterpret_cast<u4v *>(reinterpret_cast<char *>(fr) + 1024 * (SCAN_P * i + pw) + 16 * lane) = cr[i];
        if (pw < 2) gm[64 * pw + lane] = cgam;
    };

    // One chunk n on this wave, from slot (fr, gm).
    auto compute = [&](int n, const _Float16 *fr, const float *gm) __attribute__((always_inline)) {
        // lane coordinates re-derived per chunk, so that the LDS addresses
        // built from them are not hoisted out of the loop (and spilled)
        int lane_ = lane;
        asm volatile("" : "+v"(lane_));
        const int lane = lane_, lr = lane & 15, lg = lane >> 4;
        const _Float16 *fg = fr + S_G + wt * 4 * 512;  // my G pairs
        const _Float16 *fo = fr + S_O + wt * 2 * 512;  // my Oe^T pairs (MODE 0)
        const int64_t t0 = tbase + static_cast<int64_t>(n) * C;
        // the fp16 copies of the state and of the erase read must stay finite
        bool big = false;
#pragma unroll
        for (int it = 0; it < 8; ++it)
            big |= !(fmaxf(fmaxf(fabsf(sacc[it][0]), fabsf(sacc[it][1])), fmaxf(fabsf(sacc[it][2]), fabsf(sacc[it][3]))) <= 16384.f);
        bool bad = gm[0] < 0.f || __ballot(big) != 0;  // chunk marked for the exact path
        f4 p1[4], oacc[4];
        h8 ef[8][2];
        big = false;
        if (!bad) {
            // Fragments are read from LDS ahead of use (W/Qe of the next row
            // tile while the current one is multiplied, EtT at the start),
            // each group fenced so the scheduler keeps reads early.
            auto read_wq = [&](h8 (&x)[2][4], int rt) __attribute__((always_inline)) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const int off = ((rt * 4 + kb) * 64 + lane) * 8;
                    x[0][kb] = *reinterpret_cast<const h8 *>(fr + OFF_W + off);
                    if (WITH_O) x[1][kb] = *reinterpret_cast<const h8 *>(fr + S_Q + off);
                }
            };
            h8 wq[2][2][4];
            read_wq(wq[0], 0);
            if (MODE == 0) {  // MODE 1 reads EtT where it is used (register budget of 12 waves)
#pragma unroll
                for (int it = 0; it < 8; ++it)
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) ef[it][k2] = *reinterpret_cast<const h8 *>(fr + S_E + ((it * 2 + k2) * 64 + lane) * 8);
            }
            // P1 = W S and O^T = S^T Qe^T + Oe^T.  State tiles 2kb, 2kb+1 in
            // the record's permuted slot order are both the B operand of key
            // block kb (for W S) and the A operand of S^T (for O^T).
            h8 sb[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sb[kb] = join(to_h4(sacc[2 * kb]), to_h4(sacc[2 * kb + 1]));
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if (rt < 3) read_wq(wq[(rt + 1) & 1], rt + 1);
                h8 oe;
                if (WITH_O) oe = *reinterpret_cast<const h8 *>(fo + ((rt >> 1) * 64 + lane) * 8);
                __builtin_amdgcn_sched_barrier(0);
                f4 p = splat(0.f);
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) p = mfma32(wq[rt & 1][0][kb], sb[kb], p);
                if (WITH_O) {
                    f4 o = (rt & 1) ? f4{(float)oe[4], (float)oe[5], (float)oe[6], (float)oe[7]}
                                    : f4{(float)oe[0], (float)oe[1], (float)oe[2], (float)oe[3]};
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) o = mfma32(sb[kb], wq[rt & 1][1][kb], o);
                    oacc[rt] = o;
                }
                p1[rt] = p;
                big |= out_of_range(p);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        bad = bad || __ballot(big) != 0;
        if (!bad) {
            f4 gam[8];
            h8 gp[4];
            if (MODE == 0) {
#pragma unroll
                for (int it = 0; it < 8; ++it) gam[it] = *reinterpret_cast<const f4 *>(&gm[16 * it + 4 * lg]);
#pragma unroll
                for (int ip = 0; ip < 4; ++ip) gp[ip] = *reinterpret_cast<const h8 *>(fg + (ip * 64 + lane) * 8);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (WITH_O) {
                // O^T tile: lane t+16m holds token 16rt+t, value columns
                // 16ct+4m..+3 -> one 16-byte store per lane and tile
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int64_t t = t0 + 16 * rt + lr;
                    if (t < tlim)
                        store_out4(a.o, (t * a.H + h) * D + 16 * ct + 4 * lg, oacc[rt][0], oacc[rt][1], oacc[rt][2],
                                   oacc[rt][3], a.o_bf16);
                }
            }
            // S <- Diag(e^gC) S + G - Etil^T P1, tokens in permuted slots
            // (the columns of F take no G)
            const h8 pb0 = join(to_h4(-p1[0]), to_h4(-p1[1]));
            const h8 pb1 = join(to_h4(-p1[2]), to_h4(-p1[3]));
            const float gsel = frun ? 0.f : 1.f;
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                if (MODE) {
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) ef[it][k2] = *reinterpret_cast<const h8 *>(fr + S_E + ((it * 2 + k2) * 64 + lane) * 8);
                    gam[it] = *reinterpret_cast<const f4 *>(&gm[16 * it + 4 * lg]);
                    if ((it & 1) == 0) gp[it >> 1] = *reinterpret_cast<const h8 *>(fg + ((it >> 1) * 64 + lane) * 8);
                }
                const h8 g2 = gp[it >> 1];
                const f4 gv = (it & 1) ? f4{(float)g2[4], (float)g2[5], (float)g2[6], (float)g2[7]}
                                       : f4{(float)g2[0], (float)g2[1], (float)g2[2], (float)g2[3]};
                f4 sv = gam[it] * sacc[it] + (MODE ? gsel * gv : gv);
                sv = mfma32(ef[it][0], pb0, sv);
                sv = mfma32(ef[it][1], pb1, sv);
                sacc[it] = sv;
            }
        } else {
            // exact fp32 token recurrence on the raw inputs of this chunk
            // (a separate function: its registers do not burden the fast path)
            f4 st[8];
#pragma unroll
            for (int it = 0; it < 8; ++it) st[it] = sacc[it];
            exact_chunk<TIED, KEYG, VW, WITH_O>(a, st, h, t0, tlim, ct, lr, lg, frun);
#pragma unroll
            for (int it = 0; it < 8; ++it) sacc[it] = st[it];
            // leave nothing of this (rare) path outstanding, so that the fast
            // path's precise waits for the prefetched slices survive the merge
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
    };

    // Chunk n: the barrier finds slot n & 1 complete (its copy waves waited
    // for their LDS writes before arriving) and every compute wave past chunk
    // n-1; then the copy waves write chunk n+1 into the other slot (last read
    // in chunk n-1) and start the loads of chunk n+2, while the compute waves
    // compute chunk n.  The two roles run separate loops with one barrier per
    // chunk each (so the copy registers and the compute registers are never
    // live at once), unrolled by two so both slots are named statically.
    constexpr int LGKM0 = 15 | (7 << 4) | (3 << 14);  // s_waitcnt lgkmcnt(0), other counters untouched
    if (copier) {
        const int pw = wv - NCOMP;
        if (n0 < n1) {
            load_regs(task0 + n0 * tstr, pw);
            store_regs(fr0, gm0, pw);
        }
        if (n0 + 1 < n1) load_regs(task0 + (n0 + 1) * tstr, pw);
        __builtin_amdgcn_s_waitcnt(LGKM0);
#define GDN2_COPY_STEP(N, FRN, GMN)                                                \
        do {                                                                      \
            slot_barrier();                                                       \
            if ((N) + 1 < n1) store_regs(FRN, GMN, pw);                           \
            if ((N) + 2 < n1) load_regs(task0 + ((N) + 2) * tstr, pw);            \
            __builtin_amdgcn_s_waitcnt(LGKM0);                                    \
        } while (0)
        int n = n0;
        for (; n + 1 < n1; n += 2) {
            GDN2_COPY_STEP(n, fr1, gm1);
            GDN2_COPY_STEP(n + 1, fr0, gm0);
        }
        if (n < n1) GDN2_COPY_STEP(n, fr1, gm1);
#undef GDN2_COPY_STEP
    } else {
        const float *init = nullptr;
        if (MODE == 0) init = nsegc == 1 ? (a.s0 ? a.s0 + sbase : nullptr) : sp.xs + xbase;
        else if (!frun && seg == 0 && a.s0) init = a.s0 + sbase;
#pragma unroll
        for (int it = 0; it < 8; ++it)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * it + 4 * lg + e, v = 16 * ct + lr;
                sacc[it][e] = init ? init[c * D + v] : (frun && c == v) ? 1.f : 0.f;
                if (MODE == 1 && !frun && seg == 0) sp.xs[xbase + c * D + v] = sacc[it][e];
            }
        int n = n0;
        for (; n + 1 < n1; n += 2) {
            slot_barrier();
            if (!idle) compute(n, fr0, gm0);
            slot_barrier();
            if (!idle) compute(n + 1, fr1, gm1);
        }
        if (n < n1) {
            slot_barrier();
            if (!idle) compute(n, fr0, gm0);
        }
        float *dst = nullptr;
        if (idle) dst = nullptr;
        else if (MODE == 0) dst = (seg == nsegc - 1 && a.s_out) ? a.s_out + sbase : nullptr;
        else dst = frun ? sp.fs + xbase : sp.xs + xbase + xstep;  // F[seg], X[seg+1]
        if (dst) {
#pragma unroll
            for (int it = 0; it < 8; ++it)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 16 * it + 4 * lg + e, v = 16 * ct + lr;
                    dst[c * D + v] = sacc[it][e];
                }
        }
    }
}

// Phase B of the segmented scan: X[j+1] <- F[j] X[j] + X[j+1] for j = 1 ..
// nseg-2, in order.  One workgroup per (chain, 16 columns); lane l owns row
// l % 128 and 8 of the 16 columns.  F[j+1] is fetched into registers while
// step j runs.
constexpr int CMB_NTH = 256;
constexpr int CMB_COLS = 16;
constexpr int CMB_FST = D + 1;  // odd row stride: lanes on distinct rows hit distinct banks

__global__ void __launch_bounds__(CMB_NTH) segment_combine_kernel(float *xs, const float *fs, int nseg, ScanPlan sp,
                                                                  int N, int H) {
    __shared__ float fl[D * CMB_FST];
    __shared__ float sx[D * CMB_COLS];
    const int chain = blockIdx.x / (D / CMB_COLS), cb = (blockIdx.x % (D / CMB_COLS)) * CMB_COLS;
    const int tid = threadIdx.x, i = tid % D, c0 = 8 * (tid / D);
    // slot j of this chain at base + j step: [chain][nseg] for B sequences of
    // T tokens; packed, the chains cut in three or more, slots (zs[s] + j) H + h
    int64_t base = static_cast<int64_t>(chain) * nseg * D * D, step = static_cast<int64_t>(D) * D;
    if (sp.qs) {
        const int k = chain / H, h = chain - k * H;
        if (k >= sp.c2[N]) return;  // launched for the bound
        const int sq = seq_of(sp.c2, N, k);
        nseg = sp.qs[sq + 1] - sp.qs[sq];
        base = (static_cast<int64_t>(sp.zs[sq]) * H + h) * D * D;
        step = static_cast<int64_t>(H) * D * D;
    }
    for (int e = tid; e < D * CMB_COLS; e += CMB_NTH) sx[e] = xs[base + step + (e / CMB_COLS) * D + cb + e % CMB_COLS];
    f4 pf[16];
    auto load_f = [&](int j) __attribute__((always_inline)) {
        const f4 *src = reinterpret_cast<const f4 *>(fs + base + static_cast<int64_t>(j) * step);
#pragma unroll
        for (int q = 0; q < 16; ++q) pf[q] = src[tid + CMB_NTH * q];
    };
    if (nseg > 2) load_f(1);
    for (int j = 1; j <= nseg - 2; ++j) {
        __syncthreads();  // step j-1 is done with fl and has written sx
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int f = 4 * (tid + CMB_NTH * q), r = f / D, c = f % D;
#pragma unroll
            for (int e = 0; e < 4; ++e) fl[r * CMB_FST + c + e] = pf[q][e];
        }
        __syncthreads();
        if (j + 1 <= nseg - 2) load_f(j + 1);
        float *xj = xs + base + static_cast<int64_t>(j + 1) * step + static_cast<int64_t>(i) * D + cb + c0;
        f4 acc0 = *reinterpret_cast<const f4 *>(xj), acc1 = *reinterpret_cast<const f4 *>(xj + 4);
        for (int k = 0; k < D; ++k) {
            const float f = fl[i * CMB_FST + k];
            const f4 s0 = *reinterpret_cast<const f4 *>(&sx[k * CMB_COLS + c0]);
            const f4 s1 = *reinterpret_cast<const f4 *>(&sx[k * CMB_COLS + c0 + 4]);
            acc0 += f * s0;
            acc1 += f * s1;
        }
        __syncthreads();  // every lane has read sx
        *reinterpret_cast<f4 *>(&sx[i * CMB_COLS + c0]) = acc0;
        *reinterpret_cast<f4 *>(&sx[i * CMB_COLS + c0 + 4]) = acc1;
        *reinterpret_cast<f4 *>(xj) = acc0;
        *reinterpret_cast<f4 *>(xj + 4) = acc1;
    }
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Segments per chain: one, unless the chains cannot fill SEG_WG scan
// workgroups; then as many as fill them, each of at least SEG_MIN chunks.
int scan_segments(int64_t chains, int64_t nc) {
    if (chains * 2 * 2 > SEG_WG) return 1;
    int64_t n = SEG_WG / (2 * chains);
    if (n > nc / SEG_MIN) n = nc / SEG_MIN;
    if (n < 2) return 1;
    const int64_t len = (nc + n - 1) / n;
    return static_cast<int>((nc + len - 1) / len);  // no empty segment
}

// Packed sequences: the segments of the two-level scan.  Sequence i of nc_i
// chunks is cut into ceil(nc_i / L) segments when nc_i > 2 L, else scanned in
// one: the summaries of all but the last segment run before the scan proper,
// so two segments would cost as many sequential steps as none, three or more
// cut the chain's sequential length to 2 L.  The host sizes the units and slots for valid offsets (bounds that
// depend on T alone); a sequence that would exceed one is scanned in one
// segment instead (which only offsets that break the contract can cause), so
// every count stays within its bound and every result is still exact.
constexpr int SP_NTH = 1024;

__device__ __forceinline__ void block_scan4(int4 *part, int tid) {
    for (int off = 1; off < SP_NTH; off <<= 1) {
        const int4 x = tid >= off ? part[tid - off] : make_int4(0, 0, 0, 0);
        __syncthreads();
        part[tid].x += x.x;
        part[tid].y += x.y;
        part[tid].z += x.z;
        part[tid].w += x.w;
        __syncthreads();
    }
}

__global__ void __launch_bounds__(SP_NTH) varlen_segment_kernel(const int *pfx, int n, int L, int q1b, int zb, int c2b,
                                                                int *qs, int *q1, int *zs, int *c2) {
    __shared__ int4 part[SP_NTH];
    const int tid = threadIdx.x;
    int4 c_orig = make_int4(0, 0, 0, 0), c_fin = make_int4(0, 0, 0, 0);  // carries
    auto counts = [](int ns) { return make_int4(ns, ns - 1, ns > 1 ? ns : 0, ns > 2 ? 1 : 0); };
    for (int base = 0; base < n; base += SP_NTH) {
        const int i = base + tid;
        int ns = 0;
        if (i < n) {
            const int nc = pfx[i + 1] - pfx[i];
            ns = nc > 2 * L ? (nc + L - 1) / L : 1;
        }
        // the requested cuts' prefix decides which sequences stay cut
        const int4 want = i < n ? counts(ns) : make_int4(0, 0, 0, 0);
        part[tid] = want;
        __syncthreads();
        block_scan4(part, tid);
        const int4 incl = part[tid];
        const int4 tot = part[SP_NTH - 1];
        if (i < n && ns > 1 &&
            (c_orig.y + incl.y > q1b || c_orig.z + incl.z > zb || c_orig.w + incl.w > c2b))
            ns = 1;
        c_orig.x += tot.x; c_orig.y += tot.y; c_orig.z += tot.z; c_orig.w += tot.w;
        __syncthreads();
        // the final counts' prefix
        const int4 have = i < n ? counts(ns) : make_int4(0, 0, 0, 0);
        part[tid] = have;
        __syncthreads();
        block_scan4(part, tid);
        const int4 in2 = part[tid], tot2 = part[SP_NTH - 1];
        if (i < n) {
            qs[i] = c_fin.x + in2.x - have.x;
            q1[i] = c_fin.y + in2.y - have.y;
            zs[i] = c_fin.z + in2.z - have.z;
            c2[i] = c_fin.w + in2.w - have.w;
        }
        c_fin.x += tot2.x; c_fin.y += tot2.y; c_fin.z += tot2.z; c_fin.w += tot2.w;
        __syncthreads();
    }
    if (tid == 0) {
        qs[n] = c_fin.x;
        q1[n] = c_fin.y;
        zs[n] = c_fin.z;
        c2[n] = c_fin.w;
    }
}

struct Layout {
    int64_t nc, chains, ntask, nseg, seg_len;
    int64_t off_gam, off_xs, off_fs, bytes;
    // packed sequences: the plan (varlen.hip), the segment prefix counts, and
    // the bounds on the summary units, slots and combined sequences
    int64_t off_plan, off_seg, q1b, zb, c2b;
};

Layout layout(int64_t B, int64_t H, int64_t T) {
    Layout l;
    l.nc = (T + C - 1) / C;
    l.chains = B * H;
    l.ntask = l.chains * l.nc;
    l.nseg = scan_segments(l.chains, l.nc);
    l.seg_len = (l.nc + l.nseg - 1) / l.nseg;
    const int64_t sts = l.nseg > 1 ? align256(l.chains * l.nseg * D * D * 4) : 0;
    l.off_gam = align256(l.ntask * REC * 2);
    l.off_xs = l.off_gam + align256(l.ntask * D * 4);
    l.off_fs = l.off_xs + sts;
    l.bytes = l.off_fs + sts;
    return l;
}

// Packed sequences: N sequences, T tokens in all, at most ceil(T/C) + N
// chunks per head (each sequence's last chunk the only partial one).
// Packed sequences: segments of L chunks, L chosen (from T and H, the host
// knows no lengths) so that the longest chain is cut to about as many chunks
// as SEG_WG / 2 scan units share evenly.  A sequence cut has more than 2 L
// chunks, so more than 64 L tokens: at most long_max = ceil(T / 64 L) are cut,
// and the units and slots are bounded by T alone (not by the sequence count).
Layout layout_varlen(int64_t N, int64_t H, int64_t T) {
    Layout l;
    const int64_t ct = (T + C - 1) / C;
    l.nc = ct + N;  // chunk bound per head
    l.chains = N * H;
    l.ntask = l.nc * H;
    l.nseg = 1;
    const int64_t want = (H * ct + SEG_WG / 2 - 1) / (SEG_WG / 2);
    l.seg_len = want > SEG_MIN ? want : SEG_MIN;
    const int64_t long_max = (T + C * l.seg_len - 1) / (C * l.seg_len);
    l.q1b = (ct + long_max) / l.seg_len + 1;  // > sum over sequences of (segments - 1)
    l.zb = l.q1b + long_max;                   // >= segments of the sequences cut
    l.c2b = long_max;                          // >= sequences cut in three or more
    l.off_gam = align256(l.ntask * REC * 2);
    l.off_plan = l.off_gam + align256(l.ntask * D * 4);
    l.off_seg = l.off_plan + static_cast<int64_t>(varlen_plan_bytes(N, T, C));
    l.off_xs = l.off_seg + 4 * align256((N + 1) * 4);
    l.off_fs = l.off_xs + align256(l.zb * H * D * D * 4);
    l.bytes = l.off_fs + align256(l.zb * H * D * D * 4);
    return l;
}

int cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

template <bool TIED, bool KEYG, bool VW = false>
hipError_t launch_kinds(const ChunkArgs &a, void *ws, hipStream_t s) {
    const Layout l = a.cu ? layout_varlen(a.B, a.H, a.T) : layout(a.B, a.H, a.T);
    char *p = static_cast<char *>(ws);
    SplitWs w;
    w.frag = reinterpret_cast<_Float16 *>(p);
    w.gam = reinterpret_cast<float *>(p + l.off_gam);
    w.vseq = nullptr;
    w.vpfx = nullptr;
    w.vtab = nullptr;
    ScanPlan sp;
    sp.nseg = static_cast<int>(l.nseg);
    sp.seg_len = static_cast<int>(l.seg_len);
    sp.xs = l.nseg > 1 ? reinterpret_cast<float *>(p + l.off_xs) : nullptr;
    sp.fs = l.nseg > 1 ? reinterpret_cast<float *>(p + l.off_fs) : nullptr;
    sp.qs = sp.q1 = sp.zs = sp.c2 = nullptr;
    if (a.cu) {
        VarPlan vp;
        hipError_t e = launch_varlen_plan(a.cu, a.B, a.T, C, p + l.off_plan, &vp, s);
        if (e != hipSuccess) return e;
        w.vseq = vp.seq;
        w.vpfx = vp.pfx;
        w.vtab = vp.tab;
        const int64_t stride = align256((a.B + 1) * 4);
        int *qs = reinterpret_cast<int *>(p + l.off_seg), *q1 = reinterpret_cast<int *>(p + l.off_seg + stride);
        int *zs = reinterpret_cast<int *>(p + l.off_seg + 2 * stride), *c2 = reinterpret_cast<int *>(p + l.off_seg + 3 * stride);
        hipLaunchKernelGGL(varlen_segment_kernel, dim3(1), dim3(SP_NTH), 0, s, vp.pfx, static_cast<int>(a.B),
                           static_cast<int>(l.seg_len), static_cast<int>(l.q1b), static_cast<int>(l.zb),
                           static_cast<int>(l.c2b), qs, q1, zs, c2);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        sp.qs = qs;
        sp.q1 = q1;
        sp.zs = zs;
        sp.c2 = c2;
        sp.xs = reinterpret_cast<float *>(p + l.off_xs);
        sp.fs = reinterpret_cast<float *>(p + l.off_fs);
    }
    const int nc = static_cast<int>(l.nc);
    const int64_t g1 = l.ntask < cu_count() ? l.ntask : cu_count();
    if (a.gate_logits || a.qk_norm)
        hipLaunchKernelGGL((chunk_prep_kernel<TIED, KEYG, VW, true>), dim3(static_cast<unsigned>(g1)), dim3(NTH), 0, s, a, w, nc);
    else
        hipLaunchKernelGGL((chunk_prep_kernel<TIED, KEYG, VW, false>), dim3(static_cast<unsigned>(g1)), dim3(NTH), 0, s, a, w, nc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.cu) {  // packed: the units are bounded on the host, counted on the device
        const int64_t u1 = a.H * l.q1b, uc = a.H * l.c2b, u0 = a.H * (a.B + l.q1b);
        hipLaunchKernelGGL((chunk_scan_kernel<TIED, KEYG, VW, 1>), dim3(static_cast<unsigned>(u1 * 2)),
                           dim3(scan_threads(1)), 0, s, a, w, nc, sp, u1 % 8 == 0 ? 1 : 0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (uc > 0) {
            hipLaunchKernelGGL(segment_combine_kernel, dim3(static_cast<unsigned>(uc * (D / CMB_COLS))), dim3(CMB_NTH), 0,
                               s, sp.xs, sp.fs, 0, sp, static_cast<int>(a.B), static_cast<int>(a.H));
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        hipLaunchKernelGGL((chunk_scan_kernel<TIED, KEYG, VW, 0>), dim3(static_cast<unsigned>(u0 * 2)),
                           dim3(scan_threads(0)), 0, s, a, w, nc, sp, u0 % 8 == 0 ? 1 : 0);
        return hipGetLastError();
    }
    if (l.nseg > 1) {
        const int64_t units = l.chains * (l.nseg - 1);
        hipLaunchKernelGGL((chunk_scan_kernel<TIED, KEYG, VW, 1>), dim3(static_cast<unsigned>(units * 2)),
                           dim3(scan_threads(1)), 0, s, a, w, nc, sp, units % 8 == 0 ? 1 : 0);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (l.nseg > 2) {
            hipLaunchKernelGGL(segment_combine_kernel, dim3(static_cast<unsigned>(l.chains * (D / CMB_COLS))),
                               dim3(CMB_NTH), 0, s, sp.xs, sp.fs, sp.nseg, sp, 0, static_cast<int>(a.H));
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    const int64_t units = l.chains * l.nseg;
    hipLaunchKernelGGL((chunk_scan_kernel<TIED, KEYG, VW, 0>), dim3(static_cast<unsigned>(units * 2)),
                       dim3(scan_threads(0)), 0, s, a, w, nc, sp, units % 8 == 0 ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

bool chunk_split_supported(const ChunkArgs &a) {
    // every present gate of one kind (all per channel or all per head); the
    // kernels index tasks (chain * chunks + chunk) with 32-bit arithmetic
    const bool tied = a.wr == nullptr;
    const bool same = a.la_key == a.eb_key && (tied || a.wr_key == a.eb_key);
    const int64_t ntask = a.cu ? a.H * ((a.T + C - 1) / C + a.B) : a.B * a.H * ((a.T + C - 1) / C);
    return a.bf16 && a.dk == D && a.dv == D && a.C == C && same && (!a.value_write || !tied) &&
           a.H * D * 4 * C < (int64_t(1) << 31) && ntask > 0 && ntask < (int64_t(1) << 31);
}

size_t chunk_split_workspace(int64_t B, int64_t H, int64_t T) { return static_cast<size_t>(layout(B, H, T).bytes); }

size_t chunk_split_workspace_varlen(int64_t N, int64_t H, int64_t T) {
    return static_cast<size_t>(layout_varlen(N, H, T).bytes);
}

hipError_t launch_chunk_split(const ChunkArgs &a, void *ws, hipStream_t s) {
    const bool tied = a.wr == nullptr, keyg = a.la_key != 0;
    if (a.value_write) return keyg ? launch_kinds<true, true, true>(a, ws, s) : launch_kinds<true, false, true>(a, ws, s);
    if (tied) return keyg ? launch_kinds<true, true>(a, ws, s) : launch_kinds<true, false>(a, ws, s);
    return keyg ? launch_kinds<false, true>(a, ws, s) : launch_kinds<false, false>(a, ws, s);
}

}  // namespace gdn2
