// KV append: the newest tokens' keys and values into their paged-cache slots.
//
// The cache write that precedes attention over a paged KV cache (the
// KV-cache writer of the RoseLLM README, "Systems highlights", "Inference
// and serving"; the mapped KV store of the microLLM-rocm README, "Why this
// project exists").  k_new / v_new [B, Hkv, Tn, d] hold the last Tn tokens
// of each sequence, whose length after the append is seq_lens[b]: token t
// goes to position seq_lens[b] - Tn + t, slot position % 16 of page
// block_table[b][position / 16], for every kv head.  A pure copy, bound by
// HBM bandwidth: each 16-byte chunk of a d-row is one lane's load and store,
// so a wave moves four 256-byte rows (d = 128) per instruction, reading
// k_new / v_new sequentially and writing whole rows of the 4 KiB
// (page, kv head) slices.
#include "device_common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kPage = 16;      // tokens per page
constexpr int kThreads = 256;  // threads per workgroup

template <int D>
__global__ __launch_bounds__(kThreads) void kv_append_kernel(const u32x4* __restrict__ k_new,
                                                             const u32x4* __restrict__ v_new,
                                                             u32x4* __restrict__ k_pages, u32x4* __restrict__ v_pages,
                                                             const int* __restrict__ block_table,
                                                             const int* __restrict__ seq_lens, int Hkv, int Tn, int W,
                                                             int rows) {
    constexpr int CPR = D * 2 / 16;       // 16-byte chunks per row
    constexpr int RPB = kThreads / CPR;   // rows per workgroup per step
    const int ch = threadIdx.x % CPR;
    for (int r = blockIdx.x * RPB + threadIdx.x / CPR; r < rows; r += gridDim.x * RPB) {
        const int t = r % Tn;
        const int bk = r / Tn;
        const int kvh = bk % Hkv;
        const int b = bk / Hkv;
        const int pos = seq_lens[b] - Tn + t;
        const size_t page = (size_t)block_table[(size_t)b * W + pos / kPage];
        const size_t dst = ((page * Hkv + kvh) * kPage + pos % kPage) * CPR + ch;
        const size_t src = (size_t)r * CPR + ch;
        const u32x4 kv = k_new[src];
        const u32x4 vv = v_new[src];
        k_pages[dst] = kv;
        v_pages[dst] = vv;
    }
}

template <int D>
hipError_t launch_d(const KvAppendArgs& a, hipStream_t stream) {
    constexpr int RPB = kThreads / (D * 2 / 16);
    const int rows = a.B * a.Hkv * a.Tn;
    const int grid = (rows + RPB - 1) / RPB < 65536 ? (rows + RPB - 1) / RPB : 65536;
    hipLaunchKernelGGL((kv_append_kernel<D>), dim3(grid), dim3(kThreads), 0, stream, (const u32x4*)a.k_new,
                       (const u32x4*)a.v_new, (u32x4*)a.k_pages, (u32x4*)a.v_pages, a.block_table, a.seq_lens, a.Hkv,
                       a.Tn, a.W, rows);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append_bf16(const KvAppendArgs& a, hipStream_t stream) {
    return a.d == 128 ? launch_d<128>(a, stream) : launch_d<64>(a, stream);
}

}  // namespace attn
