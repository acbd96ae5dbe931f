// decode.hip -- one recurrent GDN-2 step per (sequence, head), state in place.
//
// The O(1)-memory inference form ("Gated DeltaNet-2" blog summary, "Core
// Mechanism"): for each head, with the fp32 state S (dk x dv) in HBM,
//   Sbar = Diag(a) S,  m = Sbar^T k,  S = Sbar - (b*k) m^T + (w*k) v^T,  o = S^T q
// (value-write form: m = Sbar^T (b*k), S = Sbar - k m^T + k (w*v)^T).
// Decay comes first and the read sees the decayed state ("Gated DeltaNet"
// page, "Decay first, then compute the write error").
//
// The step is bound by HBM: every head streams its 64 KiB state in and out
// once (9 d^2 flops against 8 d^2 bytes).  The d = 128 kernel gives one
// workgroup of 256 lanes to a head; lane (rg, cg) holds value columns
// 4cg..4cg+3 of key rows rg, rg+8, ..., rg+120 in registers (16 float4), so
// the state is read once with 16-byte coalesced loads, both reductions over
// the key rows run in registers plus one cross-wave exchange in LDS, and
// the state is written once.
#include "common.h"
#include "kernels.h"

namespace gdn2 {
namespace {

constexpr int kD = 128;
constexpr int kRowsPerLane = 16;

__global__ void __launch_bounds__(256) step128_kernel(StepArgs a) {
    __shared__ float s_k[kD], s_q[kD], s_a[kD], s_e[kD], s_u[kD];
    __shared__ float4 s_red[2][4][32];

    const int64_t head = blockIdx.x;  // n * H + h
    const int tid = threadIdx.x;
    const int cg = tid & 31, rg = tid >> 5, wave = tid >> 6;
    float *state = a.state + head * (kD * kD);

    // Issue the 16 state loads first; the gate vectors are staged meanwhile.
    float4 S[kRowsPerLane];
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i)
        S[i] = *reinterpret_cast<const float4 *>(state + (rg + 8 * i) * kD + 4 * cg);

    float kv = 0.f, qv = 0.f, bb = 0.f, ww = 0.f;
    if (tid < kD) {
        const int c = tid;
        kv = load_qkv(a.k, head * kD + c, a.bf16);
        qv = load_qkv(a.q, head * kD + c, a.bf16);
        s_a[c] = __expf(load_gate_x(a.la, a.la_key, head, kD, c, a.gate_logits, 0));
        bb = load_gate_x(a.eb, a.eb_key, head, kD, c, a.gate_logits, 1);
        ww = a.value_write ? 0.f : a.wr ? load_gate_x(a.wr, a.wr_key, head, kD, c, a.gate_logits, 1) : bb;
    }
    float4 v;
    v.x = load_qkv(a.v, head * kD + 4 * cg + 0, a.bf16);
    v.y = load_qkv(a.v, head * kD + 4 * cg + 1, a.bf16);
    v.z = load_qkv(a.v, head * kD + 4 * cg + 2, a.bf16);
    v.w = load_qkv(a.v, head * kD + 4 * cg + 3, a.bf16);
    if (a.value_write) {  // w .* v, one factor per value channel (or per head)
        v.x *= load_gate_x(a.wr, a.wr_key, head, kD, 4 * cg + 0, a.gate_logits, 1);
        v.y *= load_gate_x(a.wr, a.wr_key, head, kD, 4 * cg + 1, a.gate_logits, 1);
        v.z *= load_gate_x(a.wr, a.wr_key, head, kD, 4 * cg + 2, a.gate_logits, 1);
        v.w *= load_gate_x(a.wr, a.wr_key, head, kD, 4 * cg + 3, a.gate_logits, 1);
    }
    if (a.qk_norm) {
        // waves 0 and 1 hold the 128 channels: squared norms of k and q
        float sk = kv * kv, sq = qv * qv;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            sk += __shfl_xor(sk, o);
            sq += __shfl_xor(sq, o);
        }
        if (tid < kD && (tid & 63) == 0) {
            s_red[0][wave][0].x = sk;
            s_red[0][wave][0].y = sq;
        }
        __syncthreads();
        const float nk = s_red[0][0][0].x + s_red[0][1][0].x, nq = s_red[0][0][0].y + s_red[0][1][0].y;
        kv *= nk > 0.f ? rsqrtf(nk) : 0.f;
        qv *= nq > 0.f ? rsqrtf(nq) : 0.f;
        __syncthreads();  // s_red is reused below
    }
    if (tid < kD) {
        const int c = tid;
        s_q[c] = a.q_scale * qv;
        if (a.value_write) {  // read along b .* k, erase and write along k
            s_k[c] = bb * kv;
            s_e[c] = kv;
            s_u[c] = kv;
        } else {
            s_k[c] = kv;
            s_e[c] = bb * kv;
            s_u[c] = ww * kv;
        }
    }
    __syncthreads();

    // decay, then the key read of the decayed state
    float4 mp = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
        const int r = rg + 8 * i;
        const float ar = s_a[r], kr = s_k[r];
        S[i].x *= ar; S[i].y *= ar; S[i].z *= ar; S[i].w *= ar;
        mp.x += kr * S[i].x; mp.y += kr * S[i].y; mp.z += kr * S[i].z; mp.w += kr * S[i].w;
    }
    mp.x += __shfl_xor(mp.x, 32);
    mp.y += __shfl_xor(mp.y, 32);
    mp.z += __shfl_xor(mp.z, 32);
    mp.w += __shfl_xor(mp.w, 32);
    if ((tid & 32) == 0) s_red[0][wave][cg] = mp;
    __syncthreads();
    float4 m = s_red[0][0][cg];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        const float4 p = s_red[0][w][cg];
        m.x += p.x; m.y += p.y; m.z += p.z; m.w += p.w;
    }

    // erase along the key, write the value, then the query read
    float4 op = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
        const int r = rg + 8 * i;
        const float er = s_e[r], ur = s_u[r], qr = s_q[r];
        S[i].x = S[i].x - er * m.x + ur * v.x;
        S[i].y = S[i].y - er * m.y + ur * v.y;
        S[i].z = S[i].z - er * m.z + ur * v.z;
        S[i].w = S[i].w - er * m.w + ur * v.w;
        op.x += qr * S[i].x; op.y += qr * S[i].y; op.z += qr * S[i].z; op.w += qr * S[i].w;
        *reinterpret_cast<float4 *>(state + r * kD + 4 * cg) = S[i];
    }
    op.x += __shfl_xor(op.x, 32);
    op.y += __shfl_xor(op.y, 32);
    op.z += __shfl_xor(op.z, 32);
    op.w += __shfl_xor(op.w, 32);
    if ((tid & 32) == 0) s_red[1][wave][cg] = op;
    __syncthreads();
    if (tid < 32) {
        float4 o = s_red[1][0][cg];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            const float4 p = s_red[1][w][cg];
            o.x += p.x; o.y += p.y; o.z += p.z; o.w += p.w;
        }
        store_out4(a.o, head * kD + 4 * cg, o.x, o.y, o.z, o.w, a.o_bf16);
    }
}

// Any dk, dv <= 128: one lane per value column walks the key rows twice.
__global__ void __launch_bounds__(128) step_general_kernel(StepArgs a) {
    __shared__ float s_k[128], s_q[128], s_a[128], s_e[128], s_u[128];
    const int64_t head = blockIdx.x;
    const int dk = static_cast<int>(a.dk), dv = static_cast<int>(a.dv);
    const int j = threadIdx.x;
    float kv = 0.f, qv = 0.f, bb = 0.f, ww = 0.f;
    if (j < dk) {
        kv = load_qkv(a.k, head * dk + j, a.bf16);
        qv = load_qkv(a.q, head * dk + j, a.bf16);
        bb = load_gate_x(a.eb, a.eb_key, head, dk, j, a.gate_logits, 1);
        ww = a.value_write ? 0.f : a.wr ? load_gate_x(a.wr, a.wr_key, head, dk, j, a.gate_logits, 1) : bb;
        s_a[j] = expf(load_gate_x(a.la, a.la_key, head, dk, j, a.gate_logits, 0));
    }
    if (a.qk_norm) {  // squared norms over the dk channels (lanes past dk hold 0)
        s_k[j] = kv * kv;
        s_q[j] = qv * qv;
        __syncthreads();
        float nk = 0.f, nq = 0.f;
        for (int c = 0; c < dk; ++c) {
            nk += s_k[c];
            nq += s_q[c];
        }
        kv *= nk > 0.f ? rsqrtf(nk) : 0.f;
        qv *= nq > 0.f ? rsqrtf(nq) : 0.f;
        __syncthreads();
    }
    if (j < dk) {
        s_q[j] = a.q_scale * qv;
        if (a.value_write) {
            s_k[j] = bb * kv;
            s_e[j] = kv;
            s_u[j] = kv;
        } else {
            s_k[j] = kv;
            s_e[j] = bb * kv;
            s_u[j] = ww * kv;
        }
    }
    __syncthreads();
    if (j >= dv) return;
    float *col = a.state + head * static_cast<int64_t>(dk) * dv + j;
    float m = 0.f;
    for (int c = 0; c < dk; ++c) m += s_k[c] * (s_a[c] * col[static_cast<int64_t>(c) * dv]);
    float vj = load_qkv(a.v, head * dv + j, a.bf16);
    if (a.value_write) vj *= load_gate_x(a.wr, a.wr_key, head, dv, j, a.gate_logits, 1);
    float o = 0.f;
    for (int c = 0; c < dk; ++c) {
        const float sn = s_a[c] * col[static_cast<int64_t>(c) * dv] - s_e[c] * m + s_u[c] * vj;
        col[static_cast<int64_t>(c) * dv] = sn;
        o += s_q[c] * sn;
    }
    store_out(a.o, head * dv + j, o, a.o_bf16);
}

__global__ void state_copy_kernel(const float *src, float *dst, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.f;
}

}  // namespace

hipError_t launch_step(const StepArgs &a, hipStream_t s) {
    const int64_t heads = a.N * a.H;
    if (a.dk == kD && a.dv == kD) {
        hipLaunchKernelGGL(step128_kernel, dim3(static_cast<unsigned>(heads)), dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL(step_general_kernel, dim3(static_cast<unsigned>(heads)), dim3(128), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_state_copy(const float *src, float *dst, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(state_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace gdn2
