// chunk_mfma.hip -- chunkwise GDN-2 forward on the gfx950 matrix cores.
//
// Covers bf16 q/k/v with dk = dv = 128 and chunk C = 64, the gates all per
// key channel, all per head, or the decay per key channel with per-head
// erase / write rates (KDA's gates), tied or untied write gate.
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
// consecutive tokens decay a channel by more than 2^14.  The fp16 copies
// of the state, the Grams and the intermediates X and M are range-checked
// before anything of the chunk is stored (|state| <= 16384, products <=
// 30000, all finite); a chunk that fails any check is run as the exact fp32
// token recurrence instead.
#include "chunk_common.h"

namespace gdn2 {
namespace {

using namespace mfma;

template <int VT>
struct alignas(16) Smem {
    _Float16 kh[C * KP];   // row-side Gram operand k*2^(g-gm); later Kbar
    _Float16 qh[C * KP];   // q*2^(g-gm); later Qbar
    _Float16 eh[C * KP];   // column-side e*2^(gm-g)
    _Float16 uh[C * KP];   // u*2^(gm-g)
    _Float16 v16[VT * SP]; // values, [v][s]
    _Float16 s16[VT * KP]; // state, [v][c]
    union {
        float af[C * AP];         // A (strict lower), then Tm in place (fp32)
        _Float16 xm16[VT * SP];   // X, then -M, [v][s]
        float segtot[NSEG][GP];    // per-segment log2-decay totals
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
        float scr[8][16 * IP];   // solve scratch (after the Grams); blocks
                                 // 4..7 serve the diagonal inverses (pitch IP)
    };
    float fsc[4][D];         // 2^(g_C - gm_j)
    float gce[D];            // 2^g_C
    int wide;    // the chunk's factors or operands leave the fast range
    int wide2;   // its state copy, Grams, X or M do
};

// Issue every load of one chunk (no waits: the values are first used by the
// next chunk's prep).
template <int VT, bool TIED, int GK>
__device__ __forceinline__ void load_raw(Raw<GK, 1> &R, const ChunkArgs &a, int64_t b, int64_t h,
                                         int64_t t0, int col0, int seg, int cq, int tid) {
    load_kqg<TIED>(R, a, b, h, t0, seg, cq);
    const auto rv = chain_rsrc(a.v, a, b, h, t0, D, 2, col0);
    const int rowk = static_cast<int>(a.H) * D;
    constexpr int PPR = VT / 8;  // 16-byte pieces per token row
    if (tid < C * PPR) {
        const int s = tid / PPR, piece = tid % PPR;
        R.v[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, (s * rowk + 8 * piece) * 2, 0, 0));
    }
}

template <int VT, bool TIED, int GK>
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
    if (tid == 0) {
        S.wide = 0;
        S.wide2 = 0;
    }

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

    Raw<GK, 1> R;
    load_raw<VT, TIED, GK>(R, a, b, h, 0, col0, tid >> 5, tid & 31, tid);

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
        if (tid == 0) S.wide2 = 0;  // last read before this chunk's first barrier
        bool sbig = false;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            sbig |= !(fmaxf(fmaxf(fabsf(sacc[ct][0]), fabsf(sacc[ct][1])), fmaxf(fabsf(sacc[ct][2]), fabsf(sacc[ct][3]))) <= MAX_STATE);
            lds_st<h4>(&S.s16[(16 * ct + lr) * KP + 16 * wv + 4 * lg], to_h4(sacc[ct]));
        }
        if (__ballot(sbig) != 0 && lane == 0) S.wide = 1;
        if (tid < C * PPR) {
            const int s = tid / PPR, piece = tid % PPR;
            const uint32_t w4[4] = {R.v[0].x, R.v[0].y, R.v[0].z, R.v[0].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S.v16[(8 * piece + 2 * e) * SP + s] = (_Float16)__uint_as_float(w4[e] << 16);
                S.v16[(8 * piece + 2 * e + 1) * SP + s] = (_Float16)__uint_as_float(w4[e] & 0xffff0000u);
            }
        }
        f4 g[RPS];
        segment_cumsum(S, R, g, seg, cq);
        __syncthreads();
        chunk_tables(S, tid);
        __syncthreads();

        // ---- prep 2: factored fp16 operands ----------------------------------
        f4 khf[RPS], qhf[RPS], egm;
        factored_operands<Smem<VT>, TIED>(S, R, g, khf, qhf, egm, seg, cq, a.q_scale);
        __syncthreads();

        const bool wide = S.wide != 0;
        if (!wide && gram_tiles<Smem<VT>, TIED>(S, wv, lr, lg)) S.wide2 = 1;
        __syncthreads();
        if (tid == 0) S.wide = 0;

        if (!wide) {
            // ---- state-side operands Kbar = k 2^g, Qbar = q 2^g ----------
#pragma unroll
            for (int i = 0; i < RPS; ++i) {
                const int r = RPS * seg + i;
                lds_st<h4>(&S.kh[r * KP + 4 * cq], to_h4(khf[i] * egm));
                lds_st<h4>(&S.qh[r * KP + 4 * cq], to_h4(qhf[i] * egm));
            }
        }
        // prefetch the next chunk while this one is computed (rows past the
        // end come back as zeros)
        load_raw<VT, TIED, GK>(R, a, b, h, t0 + C, col0, seg, cq, tid);

        // Chunk-row outputs (X, M, O: C x VT): wave wv owns row block
        // rb = wv/2 and NCTW value tiles, so its row-side fragment is read
        // once per k-step for all of them.
        const int rb = wv >> 1, ct0 = (wv & 1) * NCTW;
        const bool rows_active = NCT >= 2 || (wv & 1) == 0;
        f4 acc[NCTW];
        // Nothing of the chunk is stored (o, the state) before X and M have
        // passed their range checks, so a chunk that fails one can still
        // take the exact path from the unchanged state.
        bool fast = !wide;
        if (fast) {
            // ---- Tm = (I + A)^-1 (diagonal blocks were inverted with the Grams)
            solve_offdiag(S, wv, lr, lg);  // Tm ready in fp16; af region free for X / -M

            // ---- X = Kbar S + Bm V -------------------------------------------
            if (rows_active) {
#pragma unroll
                for (int n = 0; n < NCTW; ++n) acc[n] = splat(0.f);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int cb = 32 * ks + 8 * lg;
                    const h8 xa = lds_ld<h8>(&S.kh[(16 * rb + lr) * KP + cb]);
#pragma unroll
                    for (int n = 0; n < NCTW; ++n)
                        acc[n] = mfma32(xa, lds_ld<h8>(&S.s16[(16 * (ct0 + n) + lr) * KP + cb]), acc[n]);
                }
                for (int ks = 0; ks <= (rb >> 1); ++ks) {
                    const int sb = 32 * ks + 8 * lg;
                    const h8 xa = lds_ld<h8>(&S.b16[(16 * rb + lr) * SP + sb]);
#pragma unroll
                    for (int n = 0; n < NCTW; ++n)
                        acc[n] = mfma32(xa, lds_ld<h8>(&S.v16[(16 * (ct0 + n) + lr) * SP + sb]), acc[n]);
                }
                bool big = false;
#pragma unroll
                for (int n = 0; n < NCTW; ++n) {
                    big |= out_of_range(acc[n]);
                    lds_st<h4>(&S.xm16[(16 * (ct0 + n) + lr) * SP + 16 * rb + 4 * lg], to_h4(acc[n]));
                }
                if (__ballot(big) != 0 && lane == 0) S.wide2 = 1;
            }
        }
        __syncthreads();  // X complete; the flags of the Grams and of X visible
        fast = fast && S.wide2 == 0;
        if (fast) {
            // ---- M = Tm X ------------------------------------------------------
            if (rows_active) {
#pragma unroll
                for (int n = 0; n < NCTW; ++n) acc[n] = splat(0.f);
                for (int ks = 0; ks <= (rb >> 1); ++ks) {
                    const int sb = 32 * ks + 8 * lg;
                    const h8 xa = lds_ld<h8>(&S.t16[(16 * rb + lr) * SP + sb]);
#pragma unroll
                    for (int n = 0; n < NCTW; ++n)
                        acc[n] = mfma32(xa, lds_ld<h8>(&S.xm16[(16 * (ct0 + n) + lr) * SP + sb]), acc[n]);
                }
                bool big = false;
#pragma unroll
                for (int n = 0; n < NCTW; ++n) big |= out_of_range(acc[n]);
                if (__ballot(big) != 0 && lane == 0) S.wide2 = 1;
            }
        }
        __syncthreads();  // every wave has read X; the flag of M visible
        fast = fast && S.wide2 == 0;
        if (fast) {
            if (rows_active) {
#pragma unroll
                for (int n = 0; n < NCTW; ++n)
                    lds_st<h4>(&S.xm16[(16 * (ct0 + n) + lr) * SP + 16 * rb + 4 * lg], to_h4(-acc[n]));
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
                    const h8 xa = lds_ld<h8>(&S.qh[(16 * rb + lr) * KP + cb]);
#pragma unroll
                    for (int n = 0; n < NCTW; ++n)
                        acc[n] = mfma32(xa, lds_ld<h8>(&S.s16[(16 * (ct0 + n) + lr) * KP + cb]), acc[n]);
                }
                for (int ks = 0; ks <= (rb >> 1); ++ks) {
                    const int sb = 32 * ks + 8 * lg;
                    const h8 xp = lds_ld<h8>(&pp[(16 * rb + lr) * SP + sb]);
                    const h8 xr = lds_ld<h8>(&S.r16[(16 * rb + lr) * SP + sb]);
#pragma unroll
                    for (int n = 0; n < NCTW; ++n) {
                        acc[n] = mfma32(xp, lds_ld<h8>(&S.v16[(16 * (ct0 + n) + lr) * SP + sb]), acc[n]);
                        acc[n] = mfma32(xr, lds_ld<h8>(&S.xm16[(16 * (ct0 + n) + lr) * SP + sb]), acc[n]);
                    }
                }
#pragma unroll
                for (int n = 0; n < NCTW; ++n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int64_t t = t0 + 16 * rb + 4 * lg + e;
                        if (t < a.T)
                            store_out(a.o, ((b * a.T + t) * a.H + h) * D + col0 + 16 * (ct0 + n) + lr, acc[n][e],
                                      a.o_bf16);
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
                        y = mfma16(au, lds_ld<h4>(&S.v16[vb]), y);
                        y = mfma16(ae, lds_ld<h4>(&S.xm16[vb]), y);
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
                    store_out(a.o, row * D + col0 + tid, o, a.o_bf16);
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

template <int VT, bool TIED, int GK>
hipError_t launch_vt(const ChunkArgs &a, hipStream_t s) {
    const int nt = D / VT;
    const int64_t chains = a.B * a.H;
    const int xcd_map = (chains % 8 == 0) ? 1 : 0;
    const dim3 grid(static_cast<unsigned>(chains * nt));
    hipLaunchKernelGGL((chunk_mfma_kernel<VT, TIED, GK>), grid, dim3(NTH), 0, s, a, nt, xcd_map);
    return hipGetLastError();
}

template <int VT, bool TIED>
hipError_t launch_tied(const ChunkArgs &a, hipStream_t s) {
    const int gk = !a.la_key ? 0 : a.eb_key ? 1 : 2;
    return gk == 1 ? launch_vt<VT, TIED, 1>(a, s) : gk == 2 ? launch_vt<VT, TIED, 2>(a, s) : launch_vt<VT, TIED, 0>(a, s);
}

template <int VT>
hipError_t launch_kind(const ChunkArgs &a, hipStream_t s) {
    return a.wr == nullptr ? launch_tied<VT, true>(a, s) : launch_tied<VT, false>(a, s);
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs &a) {
    // the erase and write gates of one kind, the decay of that kind or per
    // key channel (gate kinds 0, 1, 2)
    const bool tied = a.wr == nullptr;
    const bool same = (a.la_key || !a.eb_key) && (tied || a.wr_key == a.eb_key);
    return a.bf16 && a.dk == D && a.dv == D && a.C == C && same && !a.value_write && !a.gate_logits && !a.qk_norm &&
           !a.cu &&
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
