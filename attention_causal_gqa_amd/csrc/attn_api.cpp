// C-ABI host layer: argument validation, split planning, workspace sizing and
// dispatch to the HIP kernels.  Every check runs before any HIP call, so a
// rejected call has no device side effect and can be tested without a GPU.
// Unsupported-but-valid requests are reported as such, never served by a
// fallback (the microLLM-rocm README, "Why this project exists", keeps
// unsupported rows explicit; "The design keeps three implementations":
// an optimised path honours the same shape and error contracts).
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "attn.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ATTN_OK;
    return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kPageSize = 16;
constexpr int kMaxDecodeGroup = 16;
constexpr int kMaxPrefillGroup = 128;
constexpr int64_t kMaxGrid = 0x7fffffff;
constexpr int kMaxChunkTablePages = 8192;  // block-table entries the chunked prefill stages in LDS

// ---- decode split plan ------------------------------------------------------
struct Plan {
    int splits;
    int pages_per_split;
};

// A split is an item: pages_per_split (pps) consecutive pages of one
// (sequence, kv head), starting at a multiple of pps.  The streaming kernel
// hands each wave an equal share of all pages, cut only at item starts, so
// a wave's share is off by at most pps - 1 pages; a sequence is cut into at
// most `splits` pieces.
//
// Automatic plan: pps about 1/32 of the page count per wave when every
// sequence is full (B * Hkv * W pages over 2048 waves, 8 per CU on 256
// CUs), clamped to [1, 64].  The share imbalance then stays near 3%, and
// the slot count ceil(W / pps) stays near 65536 / (B * Hkv), bounding the
// workspace.
Plan make_plan(int B, int Hkv, int W, int num_splits) {
    Plan p{};
    if (num_splits > 0) {
        const int s = num_splits < W ? num_splits : W;
        p.pages_per_split = (W + s - 1) / s;
    } else {
        const int64_t per_wave = ((int64_t)B * Hkv * W + 2047) / 2048;
        const int64_t pps = per_wave / 32;
        p.pages_per_split = (int)(pps < 1 ? 1 : pps > 64 ? 64 : pps);
    }
    p.splits = (W + p.pages_per_split - 1) / p.pages_per_split;
    return p;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Decode workspace: the streaming kernel stores the piece of run r (sequence
// b, kv head j: r = b * Hkv + j) met by wave w in slot r + w, so there are
// fewer than B * Hkv + kMaxStreamWaves slots, each holding G = Hq / Hkv
// partial rows of d fp32 values and G fp32 log-sum-exps; after them, one
// record of four int32 per run (first slot, piece count, and where the
// pieces lie: the run's offset in its first wave's share and the share size).  The size does not depend on the
// sequence lengths or the split plan.
struct WorkspaceLayout {
    size_t o_part, lse_part, run_info, bytes;  // byte offsets, total
};

WorkspaceLayout workspace_layout(int B, int Hq, int Hkv, int d) {
    const size_t runs = (size_t)B * Hkv;
    const size_t rows = (runs + attn::kMaxStreamWaves) * (size_t)(Hq / Hkv);
    WorkspaceLayout w{};
    w.o_part = 0;
    w.lse_part = round256(rows * d * sizeof(float));
    w.run_info = w.lse_part + round256(rows * sizeof(float));
    w.bytes = w.run_info + round256(runs * 4 * sizeof(int));
    return w;
}

int check_decode_sizes(int B, int Hq, int Hkv, int d, int page_size, int W, int num_splits) {
    if (B < 0) return fail(ATTN_ERR_INVALID_ARG, "B=%d must be >= 0", B);
    if (Hq < 1 || Hkv < 1) return fail(ATTN_ERR_INVALID_ARG, "Hq=%d, Hkv=%d must be >= 1", Hq, Hkv);
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (d < 1) return fail(ATTN_ERR_INVALID_ARG, "d=%d must be >= 1", d);
    if (page_size < 1) return fail(ATTN_ERR_INVALID_ARG, "page_size=%d must be >= 1", page_size);
    if (W < 1) return fail(ATTN_ERR_INVALID_ARG, "max_pages_per_seq=%d must be >= 1", W);
    if (num_splits < 0) return fail(ATTN_ERR_INVALID_ARG, "num_splits=%d must be >= 0", num_splits);
    if ((int64_t)W * page_size > 0x7fffffff) return fail(ATTN_ERR_INVALID_ARG, "max_pages_per_seq * page_size overflows int");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "decode supports d = 64 or 128, not %d", d);
    if (page_size != kPageSize) return fail(ATTN_ERR_UNSUPPORTED, "decode supports page_size = 16, not %d", page_size);
    if (Hq / Hkv > kMaxDecodeGroup)
        return fail(ATTN_ERR_UNSUPPORTED, "decode supports Hq/Hkv <= %d, not %d", kMaxDecodeGroup, Hq / Hkv);
    // The kernels index the flattened (sequence, kv head, page) stream and the
    // run records with 32-bit offsets.
    if ((int64_t)B * Hkv * W > 0x7fffffff)
        return fail(ATTN_ERR_UNSUPPORTED, "decode supports B * Hkv * max_pages_per_seq < 2^31, not %lld",
                    (long long)B * Hkv * W);
    return ATTN_OK;
}

// The launch arguments of a validated decode call: the split plan and the
// workspace carved into its three regions.
int decode_args(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                const int32_t* seq_lens, void* out, float* lse, int B, int Hq, int Hkv, int d, int page_size, int W,
                float scale, int num_splits, void* workspace, size_t workspace_bytes, attn::DecodeArgs* a) {
    if ((int64_t)B * Hq > kMaxGrid) return fail(ATTN_ERR_INVALID_ARG, "problem too large");
    const WorkspaceLayout lay = workspace_layout(B, Hq, Hkv, d);
    if (!workspace || workspace_bytes < lay.bytes)
        return fail(ATTN_ERR_WORKSPACE, "workspace %zu bytes given, %zu needed", workspace ? workspace_bytes : 0,
                    lay.bytes);
    if (!aligned(workspace, 16)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    char* ws = static_cast<char*>(workspace);
    const Plan plan = make_plan(B, Hkv, W, num_splits);
    *a = attn::DecodeArgs{q,
                          k_pages,
                          v_pages,
                          block_table,
                          seq_lens,
                          out,
                          lse,
                          reinterpret_cast<float*>(ws + lay.o_part),
                          reinterpret_cast<float*>(ws + lay.lse_part),
                          reinterpret_cast<int*>(ws + lay.run_info),
                          B,
                          Hq,
                          Hkv,
                          d,
                          page_size,
                          W,
                          plan.pages_per_split,
                          scale};
    return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument";
        case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: valid request with no kernel in this build";
        case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace missing or too small";
        case ATTN_ERR_HIP: return "ATTN_ERR_HIP: HIP runtime error";
        default: return "unknown attn status";
    }
}

const char* attn_last_error_message(void) { return g_last_error.c_str(); }

int attn_prefill(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int T,
                 int d, float scale, int dtype, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (B < 0 || T < 0) return fail(ATTN_ERR_INVALID_ARG, "B=%d, T=%d must be >= 0", B, T);
    if (Hq < 1 || Hkv < 1) return fail(ATTN_ERR_INVALID_ARG, "Hq=%d, Hkv=%d must be >= 1", Hq, Hkv);
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (d < 1) return fail(ATTN_ERR_INVALID_ARG, "d=%d must be >= 1", d);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "prefill supports d = 64 or 128, not %d", d);
    if (dtype == ATTN_BF16 && Hq / Hkv > kMaxPrefillGroup)
        return fail(ATTN_ERR_UNSUPPORTED, "bf16 prefill supports Hq/Hkv <= %d", kMaxPrefillGroup);
    if (B == 0 || T == 0) return ATTN_OK;
    if (!q || !k || !v || !out) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and out must be non-null");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    // The launch grid must fit the kernels' int index arithmetic: the fp32
    // kernel takes 64 rows of one head per workgroup, the bf16 kernel 256
    // (token, head) rows of one kv group.
    const int64_t rows_per_block = dtype == ATTN_F32 ? 64 : (256 / (Hq / Hkv));
    const int64_t nqb = (T + rows_per_block - 1) / rows_per_block;
    const int64_t blocks = nqb * B * (dtype == ATTN_F32 ? Hq : Hkv);
    if (blocks > kMaxGrid) return fail(ATTN_ERR_INVALID_ARG, "problem too large: %lld workgroups", (long long)blocks);

    attn::PrefillArgs a{q, k, v, out, lse, B, Hq, Hkv, T, d, scale};
    hipError_t e = dtype == ATTN_F32 ? attn::launch_prefill_f32(a, stream) : attn::launch_prefill_bf16(a, stream);
    return from_hip(e, "attn_prefill launch");
}

int attn_prefill_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                       const int32_t* seq_lens, void* out, float* lse, int B, int Hq, int Hkv, int Tq, int d,
                       int page_size, int num_pages, int max_pages_per_seq, float scale, int dtype,
                       hipStream_t stream) {
    g_last_error.clear();
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (B < 0 || Tq < 0) return fail(ATTN_ERR_INVALID_ARG, "B=%d, Tq=%d must be >= 0", B, Tq);
    if (Hq < 1 || Hkv < 1) return fail(ATTN_ERR_INVALID_ARG, "Hq=%d, Hkv=%d must be >= 1", Hq, Hkv);
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (d < 1) return fail(ATTN_ERR_INVALID_ARG, "d=%d must be >= 1", d);
    if (page_size < 1) return fail(ATTN_ERR_INVALID_ARG, "page_size=%d must be >= 1", page_size);
    if (max_pages_per_seq < 1) return fail(ATTN_ERR_INVALID_ARG, "max_pages_per_seq=%d must be >= 1", max_pages_per_seq);
    if (num_pages < 0) return fail(ATTN_ERR_INVALID_ARG, "num_pages=%d must be >= 0", num_pages);
    if ((int64_t)max_pages_per_seq * page_size > 0x7fffffff)
        return fail(ATTN_ERR_INVALID_ARG, "max_pages_per_seq * page_size overflows int");
    if ((int64_t)Tq > (int64_t)max_pages_per_seq * page_size)
        return fail(ATTN_ERR_INVALID_ARG, "Tq=%d exceeds the cache capacity max_pages_per_seq * page_size", Tq);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "chunked prefill supports ATTN_BF16 only");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "chunked prefill supports d = 64 or 128, not %d", d);
    if (page_size != kPageSize)
        return fail(ATTN_ERR_UNSUPPORTED, "chunked prefill supports page_size = 16, not %d", page_size);
    if (Hq / Hkv > kMaxPrefillGroup)
        return fail(ATTN_ERR_UNSUPPORTED, "chunked prefill supports Hq/Hkv <= %d", kMaxPrefillGroup);
    if (max_pages_per_seq > kMaxChunkTablePages)
        return fail(ATTN_ERR_UNSUPPORTED, "chunked prefill supports max_pages_per_seq <= %d", kMaxChunkTablePages);
    if (B == 0 || Tq == 0) return ATTN_OK;
    if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out)
        return fail(ATTN_ERR_INVALID_ARG, "q, k_pages, v_pages, block_table, seq_lens and out must be non-null");
    if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k_pages, v_pages and out must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
        return fail(ATTN_ERR_INVALID_ARG, "block_table, seq_lens and lse must be 4-byte aligned");
    const int64_t rows_per_block = 256 / (Hq / Hkv);
    const int64_t blocks = (Tq + rows_per_block - 1) / rows_per_block * B * Hkv;
    if (blocks > kMaxGrid) return fail(ATTN_ERR_INVALID_ARG, "problem too large: %lld workgroups", (long long)blocks);

    attn::PrefillArgs a{q, k_pages, v_pages, out, lse, B, Hq, Hkv, Tq, d, scale};
    return from_hip(attn::launch_prefill_paged_bf16(a, block_table, seq_lens, max_pages_per_seq, stream),
                    "attn_prefill_paged launch");
}

int attn_prefill_paged_append(const void* q, const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                              const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse, int B, int Hq,
                              int Hkv, int Tq, int d, int page_size, int num_pages, int max_pages_per_seq, float scale,
                              int dtype, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (B < 0 || Tq < 0) return fail(ATTN_ERR_INVALID_ARG, "B=%d, Tq=%d must be >= 0", B, Tq);
    if (Hq < 1 || Hkv < 1) return fail(ATTN_ERR_INVALID_ARG, "Hq=%d, Hkv=%d must be >= 1", Hq, Hkv);
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (d < 1) return fail(ATTN_ERR_INVALID_ARG, "d=%d must be >= 1", d);
    if (page_size < 1) return fail(ATTN_ERR_INVALID_ARG, "page_size=%d must be >= 1", page_size);
    if (max_pages_per_seq < 1) return fail(ATTN_ERR_INVALID_ARG, "max_pages_per_seq=%d must be >= 1", max_pages_per_seq);
    if (num_pages < 0) return fail(ATTN_ERR_INVALID_ARG, "num_pages=%d must be >= 0", num_pages);
    if ((int64_t)max_pages_per_seq * page_size > 0x7fffffff)
        return fail(ATTN_ERR_INVALID_ARG, "max_pages_per_seq * page_size overflows int");
    if ((int64_t)Tq > (int64_t)max_pages_per_seq * page_size)
        return fail(ATTN_ERR_INVALID_ARG, "Tq=%d exceeds the cache capacity max_pages_per_seq * page_size", Tq);
    if ((int64_t)B * Hkv * Tq > 0x7fffffff) return fail(ATTN_ERR_INVALID_ARG, "B * Hkv * Tq overflows int");
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "fused append + chunked prefill supports ATTN_BF16 only");
    if (d != 64 && d != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "fused append + chunked prefill supports d = 64 or 128, not %d", d);
    if (page_size != kPageSize)
        return fail(ATTN_ERR_UNSUPPORTED, "fused append + chunked prefill supports page_size = 16, not %d", page_size);
    if (Hq / Hkv > kMaxPrefillGroup)
        return fail(ATTN_ERR_UNSUPPORTED, "fused append + chunked prefill supports Hq/Hkv <= %d", kMaxPrefillGroup);
    if (max_pages_per_seq > kMaxChunkTablePages)
        return fail(ATTN_ERR_UNSUPPORTED, "fused append + chunked prefill supports max_pages_per_seq <= %d",
                    kMaxChunkTablePages);
    if (B == 0 || Tq == 0) return ATTN_OK;
    if (!q || !k_new || !v_new || !k_pages || !v_pages || !block_table || !seq_lens || !out)
        return fail(ATTN_ERR_INVALID_ARG,
                    "q, k_new, v_new, k_pages, v_pages, block_table, seq_lens and out must be non-null");
    if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pages, 16) ||
        !aligned(v_pages, 16) || !aligned(out, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k_new, v_new, k_pages, v_pages and out must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
        return fail(ATTN_ERR_INVALID_ARG, "block_table, seq_lens and lse must be 4-byte aligned");
    const int64_t rows_per_block = 256 / (Hq / Hkv);
    const int64_t blocks = (Tq + rows_per_block - 1) / rows_per_block * B * Hkv;
    if (blocks > kMaxGrid) return fail(ATTN_ERR_INVALID_ARG, "problem too large: %lld workgroups", (long long)blocks);

    attn::PrefillArgs a{q, k_pages, v_pages, out, lse, B, Hq, Hkv, Tq, d, scale};
    return from_hip(attn::launch_prefill_paged_append_bf16(a, k_new, v_new, k_pages, v_pages, block_table, seq_lens,
                                                           max_pages_per_seq, stream),
                    "attn_prefill_paged_append launch");
}

int attn_prefill_varlen(const void* q, const void* k, const void* v, void* out, float* lse, const int32_t* cu_seqlens,
                        int num_seqs, int total_tokens, int max_seqlen, int Hq, int Hkv, int d, float scale,
                        int dtype, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0)
        return fail(ATTN_ERR_INVALID_ARG, "num_seqs=%d, total_tokens=%d, max_seqlen=%d must be >= 0", num_seqs,
                    total_tokens, max_seqlen);
    if (Hq < 1 || Hkv < 1) return fail(ATTN_ERR_INVALID_ARG, "Hq=%d, Hkv=%d must be >= 1", Hq, Hkv);
    if (Hq % Hkv != 0) return fail(ATTN_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (d < 1) return fail(ATTN_ERR_INVALID_ARG, "d=%d must be >= 1", d);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "ragged prefill supports ATTN_BF16 only");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "ragged prefill supports d = 64 or 128, not %d", d);
    if (Hq / Hkv > kMaxPrefillGroup)
        return fail(ATTN_ERR_UNSUPPORTED, "ragged prefill supports Hq/Hkv <= %d", kMaxPrefillGroup);
    if (num_seqs == 0 || total_tokens == 0 || max_seqlen == 0) return ATTN_OK;
    if (!q || !k || !v || !out || !cu_seqlens)
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v, out and cu_seqlens must be non-null");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
    if (!aligned(cu_seqlens, 4) || (lse && !aligned(lse, 4)))
        return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens and lse must be 4-byte aligned");
    const int64_t rows_per_block = 256 / (Hq / Hkv);
    const int64_t blocks = attn::varlen_items_bound(total_tokens, num_seqs, max_seqlen, rows_per_block) * Hkv;
    if (blocks > kMaxGrid) return fail(ATTN_ERR_INVALID_ARG, "problem too large: %lld workgroups", (long long)blocks);

    attn::PrefillArgs a{q, k, v, out, lse, num_seqs, Hq, Hkv, max_seqlen, d, scale};
    return from_hip(attn::launch_prefill_varlen_bf16(a, cu_seqlens, total_tokens, stream),
                    "attn_prefill_varlen launch");
}

int attn_validate_varlen_metadata(const int32_t* cu_seqlens_host, int num_seqs, int total_tokens, int max_seqlen) {
    g_last_error.clear();
    if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0)
        return fail(ATTN_ERR_INVALID_ARG, "bad sizes: num_seqs=%d total_tokens=%d max_seqlen=%d", num_seqs,
                    total_tokens, max_seqlen);
    if (!cu_seqlens_host) return fail(ATTN_ERR_INVALID_ARG, "null cu_seqlens");
    if (cu_seqlens_host[0] != 0) return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens[0]=%d must be 0", cu_seqlens_host[0]);
    for (int s = 0; s < num_seqs; ++s) {
        const int64_t n = (int64_t)cu_seqlens_host[s + 1] - cu_seqlens_host[s];
        if (n < 0 || n > max_seqlen)
            return fail(ATTN_ERR_INVALID_ARG, "sequence %d has %lld tokens, outside [0, max_seqlen=%d]", s, (long long)n,
                        max_seqlen);
    }
    if (cu_seqlens_host[num_seqs] != total_tokens)
        return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens[%d]=%d must equal total_tokens=%d", num_seqs,
                    cu_seqlens_host[num_seqs], total_tokens);
    return ATTN_OK;
}

int attn_kv_append(const void* k_new, const void* v_new, void* k_pages, void* v_pages, const int32_t* block_table,
                   const int32_t* seq_lens, int B, int Hkv, int Tn, int d, int page_size, int num_pages,
                   int max_pages_per_seq, int dtype, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (B < 0 || Tn < 0) return fail(ATTN_ERR_INVALID_ARG, "B=%d, Tn=%d must be >= 0", B, Tn);
    if (Hkv < 1) return fail(ATTN_ERR_INVALID_ARG, "Hkv=%d must be >= 1", Hkv);
    if (d < 1) return fail(ATTN_ERR_INVALID_ARG, "d=%d must be >= 1", d);
    if (page_size < 1) return fail(ATTN_ERR_INVALID_ARG, "page_size=%d must be >= 1", page_size);
    if (max_pages_per_seq < 1) return fail(ATTN_ERR_INVALID_ARG, "max_pages_per_seq=%d must be >= 1", max_pages_per_seq);
    if (num_pages < 0) return fail(ATTN_ERR_INVALID_ARG, "num_pages=%d must be >= 0", num_pages);
    if ((int64_t)Tn > (int64_t)max_pages_per_seq * page_size)
        return fail(ATTN_ERR_INVALID_ARG, "Tn=%d exceeds the cache capacity max_pages_per_seq * page_size", Tn);
    if ((int64_t)B * Hkv * Tn > 0x7fffffff) return fail(ATTN_ERR_INVALID_ARG, "B * Hkv * Tn overflows int");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "KV append supports ATTN_BF16 only");
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "KV append supports d = 64 or 128, not %d", d);
    if (page_size != kPageSize) return fail(ATTN_ERR_UNSUPPORTED, "KV append supports page_size = 16, not %d", page_size);
    if (B == 0 || Tn == 0) return ATTN_OK;
    if (!k_new || !v_new || !k_pages || !v_pages || !block_table || !seq_lens)
        return fail(ATTN_ERR_INVALID_ARG, "k_new, v_new, k_pages, v_pages, block_table and seq_lens must be non-null");
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16))
        return fail(ATTN_ERR_INVALID_ARG, "k_new, v_new, k_pages and v_pages must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4))
        return fail(ATTN_ERR_INVALID_ARG, "block_table and seq_lens must be 4-byte aligned");
    attn::KvAppendArgs a{k_new, v_new, k_pages, v_pages, block_table, seq_lens, B, Hkv, Tn, d, max_pages_per_seq};
    return from_hip(attn::launch_kv_append_bf16(a, stream), "attn_kv_append launch");
}

int attn_decode_num_splits(int B, int Hq, int Hkv, int d, int page_size, int max_pages_per_seq, int num_splits) {
    g_last_error.clear();
    int st = check_decode_sizes(B, Hq, Hkv, d, page_size, max_pages_per_seq, num_splits);
    if (st != ATTN_OK) return st;
    return make_plan(B, Hkv, max_pages_per_seq, num_splits).splits;
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int page_size, int max_pages_per_seq,
                                   int num_splits) {
    g_last_error.clear();
    if (check_decode_sizes(B, Hq, Hkv, d, page_size, max_pages_per_seq, num_splits) != ATTN_OK) return 0;
    return workspace_layout(B, Hq, Hkv, d).bytes;
}

int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                      const int32_t* seq_lens, void* out, float* lse, int B, int Hq, int Hkv, int d, int page_size,
                      int num_pages, int max_pages_per_seq, float scale, int dtype, int num_splits,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    int st = check_decode_sizes(B, Hq, Hkv, d, page_size, max_pages_per_seq, num_splits);
    if (st != ATTN_OK) return st;
    if (num_pages < 0) return fail(ATTN_ERR_INVALID_ARG, "num_pages=%d must be >= 0", num_pages);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "decode supports ATTN_BF16 only");
    if (B == 0) return ATTN_OK;
    if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out)
        return fail(ATTN_ERR_INVALID_ARG, "q, k_pages, v_pages, block_table, seq_lens and out must be non-null");
    if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k_pages, v_pages and out must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
        return fail(ATTN_ERR_INVALID_ARG, "block_table, seq_lens and lse must be 4-byte aligned");

    attn::DecodeArgs a{};
    st = decode_args(q, k_pages, v_pages, block_table, seq_lens, out, lse, B, Hq, Hkv, d, page_size,
                     max_pages_per_seq, scale, num_splits, workspace, workspace_bytes, &a);
    if (st != ATTN_OK) return st;
    return from_hip(attn::launch_decode_bf16(a, stream), "attn_decode_paged launch");
}

int attn_decode_paged_append(const void* q, const void* k_new, const void* v_new, void* k_pages, void* v_pages,
                             const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse, int B, int Hq,
                             int Hkv, int d, int page_size, int num_pages, int max_pages_per_seq, float scale,
                             int dtype, int num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    int st = check_decode_sizes(B, Hq, Hkv, d, page_size, max_pages_per_seq, num_splits);
    if (st != ATTN_OK) return st;
    if (num_pages < 0) return fail(ATTN_ERR_INVALID_ARG, "num_pages=%d must be >= 0", num_pages);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "decode with append supports ATTN_BF16 only");
    if (B == 0) return ATTN_OK;
    if (!q || !k_new || !v_new || !k_pages || !v_pages || !block_table || !seq_lens || !out)
        return fail(ATTN_ERR_INVALID_ARG,
                    "q, k_new, v_new, k_pages, v_pages, block_table, seq_lens and out must be non-null");
    if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pages, 16) ||
        !aligned(v_pages, 16) || !aligned(out, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k_new, v_new, k_pages, v_pages and out must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
        return fail(ATTN_ERR_INVALID_ARG, "block_table, seq_lens and lse must be 4-byte aligned");

    attn::DecodeArgs a{};
    st = decode_args(q, k_pages, v_pages, block_table, seq_lens, out, lse, B, Hq, Hkv, d, page_size,
                     max_pages_per_seq, scale, num_splits, workspace, workspace_bytes, &a);
    if (st != ATTN_OK) return st;
    return from_hip(attn::launch_decode_append_bf16(a, k_new, v_new, stream), "attn_decode_paged_append launch");
}

int attn_decode_paged_noalloc(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                              const int32_t* seq_lens, void* out, float* lse, int B, int Hq, int Hkv, int d,
                              int page_size, int num_pages, int max_pages_per_seq, float scale, int dtype,
                              int num_splits, hipStream_t stream) {
    g_last_error.clear();
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    int st = check_decode_sizes(B, Hq, Hkv, d, page_size, max_pages_per_seq, num_splits);
    if (st != ATTN_OK) return st;
    if (num_pages < 0) return fail(ATTN_ERR_INVALID_ARG, "num_pages=%d must be >= 0", num_pages);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "decode supports ATTN_BF16 only");
    if (B == 0) return ATTN_OK;
    if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out)
        return fail(ATTN_ERR_INVALID_ARG, "q, k_pages, v_pages, block_table, seq_lens and out must be non-null");
    if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k_pages, v_pages and out must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
        return fail(ATTN_ERR_INVALID_ARG, "block_table, seq_lens and lse must be 4-byte aligned");
    const size_t need = workspace_layout(B, Hq, Hkv, d).bytes;
    if (need > attn::kDecodeScratchBytes)
        return fail(ATTN_ERR_WORKSPACE,
                    "this shape needs %zu bytes of workspace; the static scratch of attn_decode_paged_noalloc "
                    "holds %zu (use attn_decode_paged with a caller workspace)",
                    need, attn::kDecodeScratchBytes);
    void* scratch = nullptr;
    const int e = from_hip(attn::decode_scratch(stream, &scratch), "attn_decode_paged_noalloc scratch lookup");
    if (e != ATTN_OK) return e;
    attn::DecodeArgs a{};
    st = decode_args(q, k_pages, v_pages, block_table, seq_lens, out, lse, B, Hq, Hkv, d, page_size,
                     max_pages_per_seq, scale, num_splits, scratch, attn::kDecodeScratchBytes, &a);
    if (st != ATTN_OK) return st;
    return from_hip(attn::launch_decode_bf16(a, stream), "attn_decode_paged_noalloc launch");
}

int attn_decode_paged_fp8(const void* q, const void* k_pages, const void* v_pages, float k_scale, float v_scale,
                          const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse, int B, int Hq,
                          int Hkv, int d, int page_size, int num_pages, int max_pages_per_seq, float scale,
                          int num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_last_error.clear();
    int st = check_decode_sizes(B, Hq, Hkv, d, page_size, max_pages_per_seq, num_splits);
    if (st != ATTN_OK) return st;
    if (num_pages < 0) return fail(ATTN_ERR_INVALID_ARG, "num_pages=%d must be >= 0", num_pages);
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
    if (!std::isfinite(k_scale) || !std::isfinite(v_scale))
        return fail(ATTN_ERR_INVALID_ARG, "k_scale and v_scale must be finite");
    if (B == 0) return ATTN_OK;
    if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out)
        return fail(ATTN_ERR_INVALID_ARG, "q, k_pages, v_pages, block_table, seq_lens and out must be non-null");
    if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16))
        return fail(ATTN_ERR_INVALID_ARG, "q, k_pages, v_pages and out must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || (lse && !aligned(lse, 4)))
        return fail(ATTN_ERR_INVALID_ARG, "block_table, seq_lens and lse must be 4-byte aligned");
    attn::DecodeArgs a{};
    st = decode_args(q, k_pages, v_pages, block_table, seq_lens, out, lse, B, Hq, Hkv, d, page_size,
                     max_pages_per_seq, scale, num_splits, workspace, workspace_bytes, &a);
    if (st != ATTN_OK) return st;
    return from_hip(attn::launch_decode_fp8(a, k_scale, v_scale, stream), "attn_decode_paged_fp8 launch");
}

int attn_validate_chunk_metadata(const int32_t* block_table_host, const int32_t* seq_lens_host, int B,
                                 int max_pages_per_seq, int page_size, int num_pages, int chunk_len) {
    g_last_error.clear();
    if (chunk_len < 0) return fail(ATTN_ERR_INVALID_ARG, "chunk_len=%d must be >= 0", chunk_len);
    const int st = attn_validate_paged_metadata(block_table_host, seq_lens_host, B, max_pages_per_seq, page_size,
                                                num_pages);
    if (st != ATTN_OK) return st;
    for (int b = 0; b < B; ++b)
        if (seq_lens_host[b] < chunk_len)
            return fail(ATTN_ERR_INVALID_ARG, "seq_lens[%d]=%d is shorter than the chunk (%d)", b, seq_lens_host[b],
                        chunk_len);
    return ATTN_OK;
}

int attn_validate_paged_metadata(const int32_t* block_table_host, const int32_t* seq_lens_host, int B,
                                 int max_pages_per_seq, int page_size, int num_pages) {
    g_last_error.clear();
    if (B < 0 || max_pages_per_seq < 1 || page_size < 1 || num_pages < 0)
        return fail(ATTN_ERR_INVALID_ARG, "bad sizes: B=%d W=%d page_size=%d num_pages=%d", B, max_pages_per_seq,
                    page_size, num_pages);
    if (B == 0) return ATTN_OK;
    if (!block_table_host || !seq_lens_host) return fail(ATTN_ERR_INVALID_ARG, "null metadata pointer");
    const int64_t cap = (int64_t)max_pages_per_seq * page_size;
    for (int b = 0; b < B; ++b) {
        const int L = seq_lens_host[b];
        if (L < 0 || L > cap) return fail(ATTN_ERR_INVALID_ARG, "seq_lens[%d]=%d outside [0, %lld]", b, L, (long long)cap);
        const int used = (L + page_size - 1) / page_size;
        for (int j = 0; j < used; ++j) {
            const int pid = block_table_host[(size_t)b * max_pages_per_seq + j];
            if (pid < 0 || pid >= num_pages)
                return fail(ATTN_ERR_INVALID_ARG, "block_table[%d][%d]=%d outside [0, %d)", b, j, pid, num_pages);
        }
    }
    return ATTN_OK;
}

}  // extern "C"
