// Read-bandwidth probe: the practical ceiling against which the paged
// decode's HBM rate is read.  Not part of the attention library: it is built
// into a library of its own and used only by the benchmark.
//
// probe_read_slices reads `n` slices of `slice_bytes` bytes from `base`,
// slice i starting at byte offs[i] (or at i * slice_bytes when offs is
// null), and does nothing with the data but fold it into one register, so
// the time is that of the reads alone.  One workgroup of slice_bytes / 16
// lanes reads a whole slice with 16-byte loads, eight slices per round
// (eight loads in flight per lane); workgroups stride over the slices.  The
// loads are ordinary or non-temporal (nt), the policy the decode's K and V
// loads use.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kUnroll = 8;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool kNT>
__global__ __launch_bounds__(256) void probe_read_slices_kernel(const char* __restrict__ base,
                                                                 const long long* __restrict__ offs, long long n,
                                                                 int slice_bytes, unsigned* __restrict__ sink) {
    const long long lane_off = (long long)threadIdx.x * 16;
    unsigned acc = 0;
    for (long long i0 = (long long)blockIdx.x * kUnroll; i0 < n; i0 += (long long)gridDim.x * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const long long i = i0 + u;
            v[u] = u32x4{0, 0, 0, 0};
            if (i < n) {
                const long long o = offs ? offs[i] : i * (long long)slice_bytes;
                const u32x4* p = reinterpret_cast<const u32x4*>(base + o + lane_off);
                if constexpr (kNT) v[u] = __builtin_nontemporal_load(p);
                else v[u] = *p;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // Keeps the loads: a store that (practically) never happens.
    if (acc == 0x9e3779b9u) sink[blockIdx.x & 255] = acc;
}

}  // namespace

extern "C" {

// Returns 0, or a HIP error code.  slice_bytes must be a multiple of 16 and
// at most 4096; base + offs[i] must be 16-byte aligned and the slice inside
// the buffer (the caller's contract; nothing is checked on the device).
// sink: 256 unsigned words of device memory.  blocks: workgroups to launch.
// nt: 0 ordinary loads, 1 non-temporal loads.
int probe_read_slices(const void* base, const long long* offs, long long n, int slice_bytes, unsigned* sink,
                      int blocks, int nt, hipStream_t stream) {
    if (!base || !sink || n < 0 || slice_bytes < 16 || slice_bytes > 4096 || slice_bytes % 16 || blocks < 1 ||
        (nt != 0 && nt != 1))
        return (int)hipErrorInvalidValue;
    if (n == 0) return 0;
    const dim3 grid((unsigned)blocks), block((unsigned)(slice_bytes / 16));
    const char* b = static_cast<const char*>(base);
    if (nt)
        hipLaunchKernelGGL(probe_read_slices_kernel<true>, grid, block, 0, stream, b, offs, n, slice_bytes, sink);
    else
        hipLaunchKernelGGL(probe_read_slices_kernel<false>, grid, block, 0, stream, b, offs, n, slice_bytes, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
