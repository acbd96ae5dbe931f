// varlen.hip -- the plan of N sequences packed along one token axis.
//
// Sequence i covers tokens [lo_i, hi_i) of the flattened token axis, lo_i =
// cu[i] and hi_i = cu[i+1] clamped into [0, T] and [lo_i, T]; its chunks of C
// tokens start at lo_i, lo_i + C, ... (the last one ragged), and a chunk never
// straddles two sequences: each sequence is its own recurrence.  The plan
// lives in device memory, built from the device offsets, so the host never
// reads them.  Chunk counts are capped at the bound the workspaces are sized
// for, ceil(T/C) + N chunks in all: offsets that break 0 = cu[0] <= ... <=
// cu[N] = T give unspecified results but never an access outside the tensors
// or a workspace.
#include "common.h"
#include "kernels.h"

namespace gdn2 {
namespace {

constexpr int PLAN_NTH = 1024;

// Ranges and chunk prefix counts (one workgroup, blocks of PLAN_NTH
// sequences, an LDS scan per block).
__global__ void __launch_bounds__(PLAN_NTH) varlen_plan_kernel(const int32_t *cu, int n, int64_t T, int C,
                                                               int cap, int2 *seq, int *pfx) {
    __shared__ int64_t part[PLAN_NTH];  // 64-bit: overlapping ranges may sum past 2^31 chunks
    const int tid = threadIdx.x;
    int64_t carry = 0;
    for (int base = 0; base < n; base += PLAN_NTH) {
        const int i = base + tid;
        int64_t cnt = 0;
        if (i < n) {
            const int64_t lo = min(max(static_cast<int64_t>(cu[i]), int64_t(0)), T);
            const int64_t hi = min(max(static_cast<int64_t>(cu[i + 1]), lo), T);
            seq[i] = make_int2(static_cast<int>(lo), static_cast<int>(hi));
            cnt = (hi - lo + C - 1) / C;
        }
        part[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < PLAN_NTH; off <<= 1) {
            const int64_t x = tid >= off ? part[tid - off] : 0;
            __syncthreads();
            part[tid] += x;
            __syncthreads();
        }
        if (i < n) pfx[i] = static_cast<int>(min(carry + part[tid] - cnt, static_cast<int64_t>(cap)));
        const int64_t tot = part[PLAN_NTH - 1];
        __syncthreads();  // every read of this block's scan before the next block's writes
        carry = min(carry + tot, static_cast<int64_t>(cap));
    }
    if (tid == 0) pfx[n] = static_cast<int>(carry);
}

// The chunk table: first token of each chunk and the end of its sequence.
__global__ void __launch_bounds__(256) varlen_table_kernel(const int2 *seq, const int *pfx, int n, int C,
                                                          int2 *tab) {
    const int total = pfx[n];
    for (int gc = blockIdx.x * 256 + threadIdx.x; gc < total; gc += gridDim.x * 256) {
        int lo = 0, hi = n - 1;  // the last sequence that starts at or before chunk gc
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pfx[mid] <= gc) lo = mid;
            else hi = mid - 1;
        }
        const int2 e = seq[lo];
        tab[gc] = make_int2(e.x + C * (gc - pfx[lo]), e.y);
    }
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

}  // namespace

int64_t varlen_chunk_bound(int64_t N, int64_t T, int C) { return (T + C - 1) / C + N; }

size_t varlen_plan_bytes(int64_t N, int64_t T, int C) {
    return static_cast<size_t>(align256(N * 8) + align256((N + 1) * 4) + align256(varlen_chunk_bound(N, T, C) * 8));
}

hipError_t launch_varlen_plan(const int32_t *cu, int64_t N, int64_t T, int C, void *buf, VarPlan *plan,
                              hipStream_t s) {
    char *p = static_cast<char *>(buf);
    int2 *seq = reinterpret_cast<int2 *>(p);
    int *pfx = reinterpret_cast<int *>(p + align256(N * 8));
    int2 *tab = reinterpret_cast<int2 *>(p + align256(N * 8) + align256((N + 1) * 4));
    const int64_t cap = varlen_chunk_bound(N, T, C);
    hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(PLAN_NTH), 0, s, cu, static_cast<int>(N), T, C,
                       static_cast<int>(cap), seq, pfx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t tb = (cap + 255) / 256;
    hipLaunchKernelGGL(varlen_table_kernel, dim3(static_cast<unsigned>(tb < 1024 ? tb : 1024)), dim3(256), 0, s, seq,
                       pfx, static_cast<int>(N), C, tab);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    plan->seq = seq;
    plan->pfx = pfx;
    plan->tab = tab;
    return hipSuccess;
}

}  // namespace gdn2
