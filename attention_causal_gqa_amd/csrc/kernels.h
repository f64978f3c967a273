// Internal launch interface between the C-ABI host layer (attn_api.cpp) and
// the HIP kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct PrefillArgs {
    const void* q;   // [B, Hq, T, d]
    const void* k;   // [B, Hkv, T, d]
    const void* v;   // [B, Hkv, T, d]
    void* out;       // [B, Hq, T, d]
    float* lse;      // [B, Hq, T] or nullptr
    int B, Hq, Hkv, T, d;
    float scale;
};

// Most one-wave workgroups the streaming decode kernel launches; the
// workspace has B * Hkv + kMaxStreamWaves piece slots.
constexpr int kMaxStreamWaves = 4096;

struct DecodeArgs {
    const void* q;            // [B, Hq, d]
    const void* k_pages;      // [num_pages, Hkv, page_size, d]
    const void* v_pages;      // [num_pages, Hkv, page_size, d]
    const int32_t* block_table;  // [B, W]
    const int32_t* seq_lens;     // [B]
    void* out;                // [B, Hq, d]
    float* lse;               // [B, Hq] or nullptr
    float* o_part;            // workspace [slots, Hq / Hkv, d], slots = B * Hkv + kMaxStreamWaves
    float* lse_part;          // workspace [slots, Hq / Hkv]
    int* run_info;            // workspace [B * Hkv, 4]: each run's first slot, piece count, offset, share size
    int B, Hq, Hkv, d, page_size, W;
    int pages_per_split;
    float scale;
};

struct KvAppendArgs {
    const void* k_new;           // [B, Hkv, Tn, d]
    const void* v_new;           // [B, Hkv, Tn, d]
    void* k_pages;               // [num_pages, Hkv, 16, d]
    void* v_pages;               // [num_pages, Hkv, 16, d]
    const int32_t* block_table;  // [B, W]
    const int32_t* seq_lens;     // [B], lengths after the append
    int B, Hkv, Tn, d, W;
};

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
// Chunked prefill over a paged cache: a.k / a.v are the page pools
// [num_pages, Hkv, 16, d], a.T is the chunk length; block_table [B, W].
hipError_t launch_prefill_paged_bf16(const PrefillArgs& a, const int32_t* block_table, const int32_t* seq_lens, int W,
                                     hipStream_t stream);
// The chunked prefill with the chunk's own keys and values in k_new / v_new
// [B, Hkv, T, d] (not yet in the pools a.k / a.v); the launch also writes
// them into the pools through k_pages / v_pages (the same pools, writable).
hipError_t launch_prefill_paged_append_bf16(const PrefillArgs& a, const void* k_new, const void* v_new, void* k_pages,
                                            void* v_pages, const int32_t* block_table, const int32_t* seq_lens, int W,
                                            hipStream_t stream);
// Ragged batch packed along the token axis: a.q / a.out [N, Hq, d], a.k / a.v
// [N, Hkv, d], a.lse [N, Hq]; a.B sequences, cu_seqlens [B+1]; a.T is the
// longest sequence.
// total_tokens = N.  The grid is Hkv * varlen_items_bound(...) workgroups.
hipError_t launch_prefill_varlen_bf16(const PrefillArgs& a, const int32_t* cu_seqlens, int total_tokens,
                                      hipStream_t stream);
// Bound on the query blocks of BMt tokens over all S sequences of a packed
// batch of N tokens, the longest Tmax: sum_s ceil(T_s / BMt) is at most
// floor(N / BMt) + S and at most S * ceil(Tmax / BMt).
inline int64_t varlen_items_bound(int64_t N, int64_t S, int64_t Tmax, int64_t BMt) {
    const int64_t a = N / BMt + S, b = S * ((Tmax + BMt - 1) / BMt);
    return a < b ? a : b;
}
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
// The same decode with the newest token of each sequence (position
// seq_lens[b] - 1) given as k_new / v_new [B, Hkv, d] rather than in the
// pools; the launch also writes it into its slot of a.k_pages / a.v_pages.
hipError_t launch_decode_append_bf16(const DecodeArgs& a, const void* k_new, const void* v_new, hipStream_t stream);
// FP8 E4M3 page pools (one byte per value) with per-tensor scales.
hipError_t launch_decode_fp8(const DecodeArgs& a, float kscale, float vscale, hipStream_t stream);
hipError_t launch_kv_append_bf16(const KvAppendArgs& a, hipStream_t stream);

// Size of the decode scratch array (the workspace of the no-allocation
// decode entry point), and its device address on the device that owns
// `stream` (looked up once per device; no allocation).
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
hipError_t decode_scratch(hipStream_t stream, void** ptr);

}  // namespace attn
