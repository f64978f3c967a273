// Causal GQA prefill, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// Method: blockwise online softmax (llm-from-scratch "Project Overview",
// "Performance Layer: kernel/ and parallel/"): scores are produced one key
// tile at a time and folded into running row statistics, so the T x T score
// matrix is never stored.  Causal MHA/GQA with BF16 data and FP32
// accumulation as named in the microLLM-rocm README ("Why this project
// exists").
//
// Work decomposition (one workgroup = 8 waves = 512 threads, one per CU):
//   * A workgroup owns 256 query rows of one (batch, kv head).  The rows are
//     (token, head) pairs: BMt = floor(256 / G) consecutive tokens times the
//     G query heads that share the kv head, so every K/V tile staged in LDS
//     serves all G heads (GQA packing).  Wave w owns rows 32w .. 32w+31.
//   * Keys are visited in tiles of 64, from key 0 up to the workgroup's last
//     token; only the tiles that reach past the first token need the causal
//     mask, applied per element behind a wave-uniform branch.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in registers):
//     in the 32x32 accumulator layout each lane then holds 16 keys of one
//     query column and lane l ^ 32 holds the other 16, so a row max or sum
//     is in-lane max3 / add operations plus one v_permlane32_swap.
//   * The same accumulator registers, rounded to bf16, are exactly the B
//     operand of O^T += V^T P^T (the contraction index is relabelled to the
//     key order the accumulator layout gives).  V stays row-major in LDS; the
//     A operand (V^T) comes from transposing ds_read_b64_tr_b16 reads.
//   * K and V tiles are stored unpadded with an XOR swizzle of 16-byte
//     chunks, so both operand read patterns are free of bank conflicts.
//   * One row sum, over the fp32 probabilities, normalises out and gives
//     the log-sum-exp.  The PV product takes the probabilities rounded to
//     bf16, so the weights applied to V sum to 1 within 2^-9 relative (a
//     second sum over the rounded values would make that exact, at 20 more
//     VALU instructions per tile on the critical softmax phase).
//   * The running max is only moved when a tile's max exceeds it by more
//     than 8 (a factor 256 in base 2): rescaling O is then rare, and
//     probabilities stay below 256, well inside fp32 and bf16 range.  The
//     exponentials are computed against the old max before the decision and
//     recomputed only on the rare tiles that move it.
//   * K/V tiles go from HBM straight into LDS (global_load_lds_dwordx4, no
//     staging registers), double-buffered.  The 8 waves form two groups of 4
//     that run in ping-pong (see below): on each SIMD one wave multiplies
//     while the other computes its softmax, and the LDS operand reads of the
//     next MFMAs are interleaved with the current ones by the scheduler.
//   * Workgroups are launched heaviest first (last query blocks have the
//     most keys); consecutive workgroup ids cycle over (batch, kv head) so a
//     kv head's blocks fall on the same XCD and share its L2.
#include "device_common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kRows = 256;  // query rows (token, head pairs) per workgroup
constexpr int kBN = 64;     // keys per tile
constexpr int kPage = 16;   // tokens per page of a paged cache
constexpr int kMaxTablePages = 8192;  // block-table entries staged in LDS (contexts up to 131072 tokens)

// Forms of the prefill kernel: dense [B, H, T, d] tensors; chunked prefill
// over a paged cache; a ragged batch packed along the token axis; chunked
// prefill that also appends the chunk's keys and values to the paged cache.
enum PrefillMode { kDense = 0, kPagedMode = 1, kVarlenMode = 2, kAppendMode = 3 };

// XOR swizzle of 16-byte chunks within an LDS row of CPR chunks: chunk c of
// row r is stored at position c ^ swz(r).  With CPR = 16 (256-byte rows),
// swz(r) = 4(r%4) + (r/4)%4: 16 consecutive rows read at one chunk (the K
// operand reads, 16 lanes x 16 bytes) hit 16 distinct positions, and 4
// consecutive rows read over 64 aligned bytes (the transposing V reads,
// 32 lanes x 8 bytes) land in 4 distinct 64-byte blocks, so neither pattern
// has LDS bank conflicts.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    if constexpr (CPR == 16) {
        return ((r & 3) << 2) | ((r >> 2) & 3);
    } else {
        return ((r & 3) << 1) | ((r >> 2) & 1);
    }
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j points at row
// j/4, columns 4(j%4)..+3 of a 4 x 16 block of 16-bit values; lane i
// receives column i of the block's 4 rows.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
    v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// 16 bytes per lane from global memory straight into LDS (global_load_lds
// dwordx4): lane l's data lands at lds_base + 16 l; lds_base must be the
// same for the whole wave (it goes in M0).  Issued from inline assembly: an
// LDS DMA the compiler can see is counted as touching both global memory
// and LDS, and while one is in flight the compiler makes every LDS read
// wait for all earlier ones, which serialises the operand reads of the
// MFMA phase.  Completion is awaited explicitly (s_waitcnt) before the
// barrier that publishes the tile.
__device__ __forceinline__ void dma16(const void* g, char* lds_base) {
    const uint32_t m = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_base;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m) : "memory", "m0");
}

// Ping-pong schedule.  A workgroup is 8 waves = two groups of 4 (one wave
// of each group per SIMD), 256 query rows, sharing every K/V tile.  Each
// iteration t has an MFMA phase (O += P(t-1) V(t-1), then S(t) = K(t) Q^T)
// and a VALU phase (softmax of S(t) into P(t)), each ended by a workgroup
// barrier.  Group B passes one extra barrier first, so it runs one phase
// behind group A: on every SIMD one wave is in its MFMA phase while the
// other is in its VALU phase, and the barriers keep them that way.
//
// Barrier slots (slot s ends with the s-th barrier): group A runs phase 1 of
// iteration t in slot 2t and phase 2 in slot 2t+1; group B one slot later.
// K(t) and V(t-1) are read in slots 2t (A) and 2t+1 (B).  The DMA of K(t+1)
// and V(t) is issued in slot 2t by group A alone, at the end of its phase 1
// of t (its MFMAs are shorter than group B's softmax, so the address unit
// drains while A would otherwise wait at the barrier), into the buffers last
// read in slots 2t-2 and 2t-1; A waits for it before the barrier that ends
// slot 2t+1.
//
// kMode == kVarlenMode: a ragged batch packed along the token axis
// (q, out [N, Hq, d], k, v [N, Hkv, d], lse [N, Hq]); sequence b holds
// tokens cu[b] .. cu[b+1]-1 (cu is passed as seq_lens) and T is the longest
// sequence.  A workgroup whose query block lies past its sequence's end
// exits before touching memory; rows and keys are read with the token-major
// strides Hq*d and Hkv*d.
//
// kMode == kPagedMode: chunked prefill over a paged cache.  k and v are then page pools
// [num_pages, Hkv, 16, D]; the T queries of sequence b are its last T
// tokens, so query t stands at position pos0 + t with pos0 = seq_lens[b] - T
// and sees keys 0 .. pos0 + t (the causal mask aligned to the bottom-right
// corner).  The block-table entries the workgroup needs are staged in LDS
// once; each DMA row then finds its page there.  With pos0 = 0 and dense
// K/V this is the plain prefill.
//
// kMode == kAppendMode: the chunked prefill whose chunk keys and values
// (positions pos0 .. pos0 + T - 1) arrive as dense tensors kn, vn [B, Hkv,
// T, D] and are not yet in the cache.  Tiles take keys below pos0 from the
// pages and the chunk's keys from kn / vn, so no workgroup waits for
// another's writes; at its end each workgroup copies its own query block's
// rows of kn / vn (its kv head) into their page slots through kw / vw, the
// writable views of the pools.  Every chunk row is written once, by the
// workgroup whose query block holds it, and read from the pools by no
// workgroup of this launch.
template <int D, bool kPosScale, int kMode>
__global__ __launch_bounds__(512, 1) void prefill_bf16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                              const bf16* __restrict__ v, bf16* __restrict__ out,
                                                              float* __restrict__ lse, int B, int Hq, int Hkv, int T,
                                                              int G, int BMt, int nqb, float c1,
                                                              const int* __restrict__ block_table,
                                                              const int* __restrict__ seq_lens, int W,
                                                              const bf16* __restrict__ kn, const bf16* __restrict__ vn,
                                                              bf16* kw, bf16* vw) {
    constexpr int CPR = D / 8;            // 16-byte chunks per key row
    constexpr int ROWB = D * 2;           // bytes per key row (no padding: rows are swizzled)
    constexpr int TILEB = kBN * ROWB;     // bytes per K or V tile
    constexpr int RPI = 64 / CPR;         // rows one 1 KiB wave-wide DMA covers
    constexpr int NIW = kBN / (8 * RPI);  // DMAs per wave per tile per tensor
    constexpr int NKK = D / 16;           // k-steps of QK^T
    constexpr int NMB = D / 32;           // 32-row blocks of O^T
    // Four distinct arrays (not one indexed array) so that the compiler can
    // tell the asynchronous DMA into one buffer from the reads of another and
    // does not make LDS reads wait for it.
    __shared__ __attribute__((aligned(1024))) char Ks0[TILEB];
    __shared__ __attribute__((aligned(1024))) char Ks1[TILEB];
    __shared__ __attribute__((aligned(1024))) char Vs0[TILEB];
    __shared__ __attribute__((aligned(1024))) char Vs1[TILEB];

    // Materialise every pointer argument now.  A scalar load still in flight
    // (the lse pointer is otherwise first used after the key loop) makes the
    // compiler wait for all LDS reads at every LDS wait inside the loop,
    // because scalar loads can complete out of order.
    __asm__ volatile("" ::"s"(q), "s"(k), "s"(v), "s"(out), "s"(lse), "s"(block_table), "s"(seq_lens));
    if constexpr (kMode == kAppendMode) __asm__ volatile("" ::"s"(kn), "s"(vn), "s"(kw), "s"(vw));
    constexpr bool kAppend = kMode == kAppendMode;
    constexpr bool kPaged = kMode == kPagedMode || kAppend;
    constexpr bool kVarlen = kMode == kVarlenMode;
    __shared__ int bt_lds[kPaged ? kMaxTablePages : 1];  // the sequence's block table (paged form)

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index 0..7, in an SGPR
    const int grp = w >> 2;                                  // 0: group A, 1: group B
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // Workgroup -> (sequence b, kv head kvh, query block qb).  Workgroup i
    // runs on XCD i % 8 (the dispatcher deals workgroups to the 8 XCDs in
    // turn, each XCD with its own L2).  The dense form takes the query blocks
    // of every (sequence, kv head) pair level by level, last block first.
    // The paged and packed forms, whose pairs read K/V slices larger than an
    // L2, give each XCD its own pairs (when their count allows) and take a
    // pair's query blocks one after another, last first, so that the
    // workgroups reading one slice run close together on one L2.
    const int bid = (int)blockIdx.x;
    int b, kvh, qb;
    if constexpr (kVarlen) {
        // Item c of kv head kvh: query blocks of sequence 0 (last first), then
        // of sequence 1, ...; sequence s has ceil(T_s / BMt) of them.  nqb is
        // a bound on the items per kv head (the grid is Hkv * nqb).
        int c;
        if ((Hkv & 7) == 0) {
            const int j = bid >> 3, hpx = Hkv >> 3;
            kvh = (bid & 7) + 8 * (j % hpx);
            c = j / hpx;
        } else {
            kvh = bid % Hkv;
            c = bid / Hkv;
        }
        // Find the sequence whose items hold c: a scan of the item counts,
        // 64 sequences at a time (every wave does the same, uniformly).
        const int ln = threadIdx.x & 63;
        int found = -1, first = 0, count = 0, base = 0;
        for (int s0 = 0; s0 < B; s0 += 64) {
            const int sq = s0 + ln;
            const int n = sq < B ? (seq_lens[sq + 1] - seq_lens[sq] + BMt - 1) / BMt : 0;
            int inc = n;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(inc, o);
                if (ln >= o) inc += y;
            }
            const int ex = base + inc - n;
            const unsigned long long hit = __ballot(n > 0 && c >= ex && c < ex + n);
            if (hit) {
                const int l = __ffsll((long long)hit) - 1;
                found = s0 + l;
                first = __shfl(ex, l);
                count = __shfl(n, l);
                break;
            }
            base += __shfl(inc, 63);
        }
        if (found < 0) return;  // past the last item: the whole workgroup, before any barrier
        b = __builtin_amdgcn_readfirstlane(found);
        qb = __builtin_amdgcn_readfirstlane(count - 1 - (c - first));
    } else {
        const int pairs = B * Hkv;
        int pair;
        if (kPaged && (pairs & 7) == 0) {
            const int j = bid >> 3;
            pair = (bid & 7) + 8 * (j / nqb);
            qb = nqb - 1 - j % nqb;
        } else {
            pair = bid % pairs;
            qb = nqb - 1 - bid / pairs;
        }
        b = pair / Hkv;
        kvh = pair % Hkv;
    }
    const int t0 = qb * BMt;
    // Queries of this sequence (Tb), the position of query 0 (pos0), and in
    // the packed form the sequence's first token (tok0).
    int Tb = T, pos0 = 0;
    size_t tok0 = 0;
    if constexpr (kPaged) pos0 = seq_lens[b] - T;
    if constexpr (kVarlen) {
        tok0 = (size_t)seq_lens[b];
        Tb = seq_lens[b + 1] - seq_lens[b];
        if (t0 >= Tb) return;  // never taken (qb < ceil(Tb / BMt)); before any barrier
    }
    const int kend = pos0 + min(t0 + BMt, Tb);  // keys 0..kend-1 are visible to some row

    // This lane's query column: row r of the workgroup (256 rows).
    const int r = 32 * w + l32;
    const int tt = r / G;
    const int head = kvh * G + (r % G);
    const int token = t0 + tt;
    const bool row_ok = tt < BMt && token < Tb;
    const int token_ld = row_ok ? token : t0;  // dead rows compute on a valid row, never stored

    // Q^T as the B operand: lane holds Q[row][16kk + 8hi .. +7].
    bf16x8 qreg[NKK];
    {
        const bf16* qrow = (kVarlen ? q + ((tok0 + token_ld) * Hq + head) * D
                                    : q + ((size_t)(b * Hq + head) * T + token_ld) * D) + 8 * hi;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qreg[kk] = *reinterpret_cast<const bf16x8*>(qrow + 16 * kk);
    }

    // Tile DMA: wave-wide DMA n (0 .. 8*NIW-1) fills LDS bytes [1024n, 1024n + 1024),
    // i.e. rows RPI*n .. RPI*n + RPI-1; lane l lands at row RPI*n + l / CPR,
    // swizzled position l % CPR, so it fetches logical chunk (l % CPR) ^ swz(row).
    // Wave w owns DMAs w*NIW .. w*NIW + NIW-1 of every tile.
    const bf16* kbase = kPaged    ? k + (size_t)kvh * kPage * D
                        : kVarlen ? k + (tok0 * Hkv + kvh) * D
                                  : k + (size_t)(b * Hkv + kvh) * T * D;
    const bf16* vbase = kPaged    ? v + (size_t)kvh * kPage * D
                        : kVarlen ? v + (tok0 * Hkv + kvh) * D
                                  : v + (size_t)(b * Hkv + kvh) * T * D;
    const uint32_t krs = kVarlen ? (uint32_t)(Hkv * ROWB) : (uint32_t)ROWB;  // bytes between consecutive keys
    // Group A (waves 0-3) issues every DMA: wave w takes the DMAs of wave
    // slots w and w + 4, i.e. DMAs w*NIW .. and (w+4)*NIW .. of every tile.
    constexpr int NDW = 2 * NIW;
    int drow[NDW];
    uint32_t doff[NDW];  // byte offset of the lane's chunk within a tile of rows
    uint32_t poff[NDW];  // paged form: byte offset of the lane's chunk within its (page, kv head) slice
    int dslot[NDW];      // wave-wide DMA index within the tile
    static_assert(kPage % RPI == 0, "a wave-wide DMA's rows must lie in one page");
#pragma unroll
    for (int j = 0; j < NDW; ++j) {
        dslot[j] = ((w & 3) + 4 * (j / NIW)) * NIW + j % NIW;
        drow[j] = RPI * dslot[j] + lane / CPR;
        doff[j] = (uint32_t)(drow[j] * krs + 16 * ((lane % CPR) ^ swz<CPR>(drow[j])));
        poff[j] = (uint32_t)((drow[j] % kPage) * ROWB + 16 * ((lane % CPR) ^ swz<CPR>(drow[j])));
    }
    // Keys at or past kend (the paged form) or Tb (the dense and packed
    // forms) are read as the last one before it: they are masked for every
    // row of the workgroup (their positions are below kend), and V is
    // finite, so they add exact zeros.  The paged form must not go past
    // kend - 1: only the block-table entries of keys 0..kend-1 are staged.
    // Append form: this (sequence, kv head)'s rows of the chunk's dense keys
    // and values, and whether key `key` comes from them (key >= pos0) or
    // from the pages.
    const bf16* knb = kAppend ? kn + (size_t)(b * Hkv + kvh) * T * D : nullptr;
    const bf16* vnb = kAppend ? vn + (size_t)(b * Hkv + kvh) * T * D : nullptr;
    auto dma_tile = [&](const bf16* base, const bf16* dense, char* dst, int k0) __attribute__((always_inline)) {
        if constexpr (kPaged) {
            // (page, kv head) slices are kPage rows of ROWB bytes, Hkv slices
            // per page; poff[j] holds the lane's row within the slice.
            const char* bb = reinterpret_cast<const char*>(base);
            const char* db = reinterpret_cast<const char*>(dense);
            if (k0 + kBN <= kend) {
                // A whole tile: the RPI rows of one wave-wide DMA lie in one
                // page, so its page id is wave-uniform and the slice address
                // is scalar work; each lane adds its fixed offset poff[j].
                // The page ids of all the wave's DMAs are read from LDS
                // before the first DMA is issued (the DMAs are asm with a
                // memory clobber, so a read placed after one waits alone).
                int pg[NDW];
#pragma unroll
                for (int j = 0; j < NDW; ++j) pg[j] = bt_lds[(k0 + RPI * dslot[j]) / kPage];
                auto pool_src = [&](int j) __attribute__((always_inline)) {
                    return bb + (size_t)__builtin_amdgcn_readfirstlane(pg[j]) * (size_t)(Hkv * kPage * ROWB);
                };
                if (!kAppend || k0 + kBN <= pos0) {
#pragma unroll
                    for (int j = 0; j < NDW; ++j) dma16(pool_src(j) + poff[j], dst + 1024 * dslot[j]);
                } else {
                    // Append form, a tile that reaches pos0 (the chunk's own
                    // keys): rows of the chunk are contiguous in the dense
                    // tensor and poff[j] offsets them the same way from a
                    // scalar base.  In the one tile that straddles pos0 each
                    // lane picks its base.
                    auto dense_src = [&](int j) __attribute__((always_inline)) {
                        const int r0 = k0 + RPI * dslot[j];  // the DMA's first row (key)
                        return db + (ptrdiff_t)(r0 - pos0 - r0 % kPage) * ROWB;
                    };
                    if (k0 >= pos0) {
#pragma unroll
                        for (int j = 0; j < NDW; ++j) dma16(dense_src(j) + poff[j], dst + 1024 * dslot[j]);
                    } else {
#pragma unroll
                        for (int j = 0; j < NDW; ++j) {
                            const int r0 = k0 + RPI * dslot[j];
                            const char* src = lane / CPR >= pos0 - r0 ? dense_src(j) : pool_src(j);
                            dma16(src + poff[j], dst + 1024 * dslot[j]);
                        }
                    }
                }
            } else {
                // The last tile: keys at or past kend read key kend - 1;
                // each lane finds its own page.
#pragma unroll
                for (int j = 0; j < NDW; ++j) {
                    const int key = min(k0 + drow[j], kend - 1);
                    const uint32_t chunk = poff[j] - (uint32_t)((drow[j] % kPage) * ROWB);
                    const char* src;
                    if (kAppend && key >= pos0)
                        src = db + (size_t)(key - pos0) * ROWB + chunk;
                    else
                        src = bb + ((size_t)bt_lds[key / kPage] * Hkv * kPage + key % kPage) * ROWB + chunk;
                    dma16(src, dst + 1024 * dslot[j]);
                }
            }
        } else if (k0 + kBN <= Tb) {
            const char* tb = reinterpret_cast<const char*>(base) + (size_t)k0 * krs;
#pragma unroll
            for (int j = 0; j < NDW; ++j) dma16(tb + doff[j], dst + 1024 * dslot[j]);
        } else {
            const char* bb = reinterpret_cast<const char*>(base);
#pragma unroll
            for (int j = 0; j < NDW; ++j) {
                const int key = min(k0 + drow[j], Tb - 1);
                dma16(bb + (size_t)key * krs + (doff[j] - (uint32_t)drow[j] * krs), dst + 1024 * dslot[j]);
            }
        }
    };

    // K operand reads (A of S^T): row 32kb + l32, chunk 2kk + hi.  The row's
    // swizzle does not depend on kb, so the offset is kread ^ (kk << 5) plus
    // the row block 32kb * ROWB.
    const int kread = l32 * ROWB + ((hi ^ swz<CPR>(l32)) << 4);
    // V operand reads (A of O^T, transposing): lane i = lane % 16 of group
    // g = lane / 16 reads row 32kb + 16kc + 8h + rl, rl = 4hi + i/4, 8 bytes
    // at column 32mb + 16(g%2) + 4(i%4).
    const int vi = lane & 15;
    const int vgd = (lane >> 4) & 1;
    const int vrl = 4 * hi + (vi >> 2);
    const int vx = 2 * vgd + ((vi & 3) >> 1);  // chunk within the 64-byte column block
    int vbase_off;
    if constexpr (CPR == 16) {
        // Row R0 + vrl (R0 = 32kb + 16kc + 8h) has swz = 4(vi/4) + 2h + hi, so
        // chunk 4mb + vx sits at 4(mb ^ vi/4) + (vx ^ hi ^ 2h).
        vbase_off = vrl * ROWB + 64 * (vi >> 2) + 16 * (vx ^ hi) + 8 * (vi & 1);
    } else {
        vbase_off = vrl * ROWB + ((vx ^ swz<CPR>(vrl)) << 4) + 8 * (vi & 1);
    }
    auto vread_off = [&](int mb, int kb, int kc, int h) __attribute__((always_inline)) {
        const int R0 = 32 * kb + 16 * kc + 8 * h;
        if constexpr (CPR == 16) {
            return R0 * ROWB + (vbase_off ^ (64 * mb + 32 * h));
        } else {
            // swz(R0 + rl) = swz(rl) (R0 is a multiple of 8); chunk 4mb + vx
            return R0 * ROWB + (vbase_off ^ ((4 * mb) << 4));
        }
    };

    f32x16 oacc[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[mb][i] = 0.f;
    f32x16 sacc[2];           // S^T of the current tile (64 keys x 32 query columns)
    uint32_t pb[2][2][4];     // P^T of the previous tile in bf16 (B operand of PV)
    float m_run = -INFINITY;  // running max, base-2 scaled domain
    float l_run = 0.f;        // this lane's share of the row sum of p (fp32)

    const float cc = kPosScale ? c1 : 1.f;
    const int ntiles = (kend + kBN - 1) / kBN;
    const int first_diag = (pos0 + t0 + 1) / kBN;  // tiles from here on reach past row t0's position

    // MFMA phase: O^T += V^T(t-1) P^T(t-1), then S^T(t) = K(t) Q^T.
    auto mfma_phase = [&](bool do_pv, const char* Vp, bool do_qk, const char* Kc) __attribute__((always_inline)) {
        if (do_pv) {
            // B element j of (kb, kc) is key 32kb + 16kc + 8(j/4) + 4hi + j%4;
            // the two transposing reads give V^T at exactly those keys.
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc) {
                    const u32x4 bv = {pb[kb][kc][0], pb[kb][kc][1], pb[kb][kc][2], pb[kb][kc][3]};
#pragma unroll
                    for (int mb = 0; mb < NMB; ++mb) {
                        const u32x2 lo = lds_read_tr16(Vp + vread_off(mb, kb, kc, 0));
                        const u32x2 hv = lds_read_tr16(Vp + vread_off(mb, kb, kc, 1));
                        const u32x4 av = {lo.x, lo.y, hv.x, hv.y};
                        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), oacc[mb], 0, 0, 0);
                    }
                }
            // Schedule: 8 LDS reads ahead, then one MFMA per two new reads, so
            // the LDS latency hides behind the MFMAs of this same wave.
            constexpr int NPV = 4 * NMB;  // MFMAs (2 reads each)
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
            for (int i = 0; i < NPV - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        if (do_qk) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const int off = kread ^ (kk << 5);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kc + kb * 32 * ROWB + off);
                    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[kk], sacc[kb], 0, 0, 0);
                }
            }
            // Schedule: 4 K reads ahead, then one MFMA per new read.
            constexpr int NQK = 2 * NKK;
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
            for (int i = 0; i < NQK - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
        }
    };

    // VALU phase: softmax of tile t (scores in sacc) into pb, row sums, and
    // (rarely) the rescale of O.
    auto softmax_phase = [&](int t) __attribute__((always_inline)) {
        const int k0 = t * kBN;
        if constexpr (!kPosScale) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[kb][i] *= c1;
        }
        // Causal mask on tiles that reach past the position of the
        // workgroup's first row.  Element i of block kb is key k0 + 32kb +
        // 8(i/4) + 4hi + i%4: masked when 32kb + 8(i/4) + i%4 > pos0 + token
        // - k0 - 4hi.
        if (t >= first_diag) {
            // A real (wave-uniform) branch: the empty volatile asm keeps the
            // compiler from turning the mask into selects run on every tile.
            __asm__ volatile("" ::: "memory");
            const int thr = pos0 + token - k0 - 4 * hi;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kb + 8 * (i >> 2) + (i & 3) > thr) sacc[kb][i] = -INFINITY;
        }
        // Probabilities against the current running max, started before the
        // row max is known (they only depend on m_run); the max decides below
        // whether they must be recomputed, which happens only when a tile's
        // max exceeds m_run by more than 8 (base 2).  In tile 0 m_run = -inf,
        // so every lane takes that path.
        float pf[2][16];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) pf[kb][i] = fast_exp2(fmaf(sacc[kb][i], cc, -m_run));
        // Row max: a tree of 3-input maxima, then lane l ^ 32.
        float m3[11];
#pragma unroll
        for (int i = 0; i < 10; ++i) {
            const int a = 3 * i, b2 = 3 * i + 1, c2 = 3 * i + 2;
            m3[i] = fmaxf(fmaxf(sacc[a >> 4][a & 15], sacc[b2 >> 4][b2 & 15]), sacc[c2 >> 4][c2 & 15]);
        }
        m3[10] = fmaxf(sacc[1][14], sacc[1][15]);
        const float m4a = fmaxf(fmaxf(m3[0], m3[1]), m3[2]);
        const float m4b = fmaxf(fmaxf(m3[3], m3[4]), m3[5]);
        const float m4c = fmaxf(fmaxf(m3[6], m3[7]), m3[8]);
        const float m4d = fmaxf(m3[9], m3[10]);
        float mx = fmaxf(fmaxf(m4a, m4b), fmaxf(m4c, m4d));
        mx = pair_max(mx);
        const float mt = mx * cc;  // tile max in the base-2 domain
        // Key 0 lies in tile 0 and is visible to every row, so after tile 0
        // m_run is finite.  The branch is taken by the whole wave, but a lane
        // that does not need it keeps its max (alpha = 1, exact) and its
        // probabilities, so a row's result never depends on the other rows of
        // its wave.  O holds tiles < t here (PV of t-1 is done).
        const bool grow = mt > m_run + 8.f;
        if (__any(grow)) {
            const float mn = grow ? mt : m_run;
            const float alpha = fast_exp2(m_run - mn);
            l_run *= alpha;
#pragma unroll
            for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[mb][i] *= alpha;
            m_run = mn;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) pf[kb][i] = fast_exp2(fmaf(sacc[kb][i], cc, -m_run));
        }
        // P^T in bf16: B operand of the PV product; the row sum over the
        // fp32 values.
        float lsum[4];  // started from the first pair: no additions of zero
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float p0 = pf[kb][8 * kc + 2 * jj];
                    const float p1 = pf[kb][8 * kc + 2 * jj + 1];
                    pb[kb][kc][jj] = pack_bf16x2(p0, p1);
                    lsum[jj] = kb == 0 && kc == 0 ? p0 + p1 : lsum[jj] + (p0 + p1);
                }
        l_run += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    };

    // Prologue: the block table (paged form), K(0) from group A; then group
    // B takes its offset barrier.
    if constexpr (kPaged) {
        const int need = (kend + kPage - 1) / kPage;
        const int* row = block_table + (size_t)b * W;
        for (int i = tid; i < need; i += 512) bt_lds[i] = row[i];
        __syncthreads();
    }
    if (grp == 0) dma_tile(kbase, knb, Ks0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (grp == 1) __syncthreads();

    // Iteration t (t = 0 .. ntiles): phase 1 = PV(t-1) + QK(t), phase 2 =
    // softmax(t).  Buffers: K(t) in Ks[t%2], V(t) in Vs[t%2].
    auto iteration = [&](int t, const char* Kc, char* Knext, const char* Vprev, char* Vcur)
                         __attribute__((always_inline)) {
        // ---- phase 1
        mfma_phase(t > 0, Vprev, t < ntiles, Kc);
        if (grp == 0) {  // the whole tile pair, while group B finishes its softmax
            if (t + 1 < ntiles) dma_tile(kbase, knb, Knext, (t + 1) * kBN);
            if (t < ntiles) dma_tile(vbase, vnb, Vcur, t * kBN);
        }
        __syncthreads();
        // ---- phase 2
        if (t < ntiles) softmax_phase(t);
        if (grp == 0) __builtin_amdgcn_s_waitcnt(0);  // group A's DMA of (K(t+1), V(t))
        __syncthreads();
    };
    for (int t = 0; t <= ntiles; t += 2) {
        // t even: K(t) in Ks0, K(t+1) -> Ks1, V(t-1) in Vs1, V(t) -> Vs0
        iteration(t, Ks0, Ks1, Vs1, Vs0);
        if (t + 1 > ntiles) break;
        iteration(t + 1, Ks1, Ks0, Vs0, Vs1);
    }
    if (grp == 0) __syncthreads();  // matches group B's offset barrier

    // Epilogue: lanes l and l^32 hold halves of the row sum.
    const float lt = pair_sum(l_run);
    if (row_ok) {
        const float inv = 1.f / lt;
        bf16* orow = (kVarlen ? out + ((tok0 + token) * Hq + head) * D
                              : out + ((size_t)(b * Hq + head) * T + token) * D) + 4 * hi;
        // O^T element i of block mb is d = 32mb + 8(i/4) + 4hi + i%4.
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const u32x2 wv = {pack_bf16x2(oacc[mb][4 * g4] * inv, oacc[mb][4 * g4 + 1] * inv),
                                  pack_bf16x2(oacc[mb][4 * g4 + 2] * inv, oacc[mb][4 * g4 + 3] * inv)};
                *reinterpret_cast<u32x2*>(orow + 32 * mb + 8 * g4) = wv;
            }
        if (lse != nullptr && hi == 0)
            lse[kVarlen ? (tok0 + token) * Hq + head : (size_t)(b * Hq + head) * T + token] = (m_run + log2f(lt)) * kLn2;
    }

    // Append form: this query block's chunk rows of kv head kvh go to their
    // page slots (positions pos0 + t0 .. kend - 1, whose block-table entries
    // are staged).  Four 16-byte chunks per lane per round, loads first.
    // (Reading the rows back from the last two LDS tiles instead, where they
    // still are when a block has at most kBN rows, measured no faster.)
    if constexpr (kAppend) {
        const int first = pos0 + t0;         // position of the block's first row
        const int n = (kend - first) * CPR;  // 16-byte chunks per tensor
        auto copy_rows = [&](const bf16* src, bf16* dst) __attribute__((always_inline)) {
            for (int i0 = 0; i0 < n; i0 += 4 * 512) {
                bf16x8 val[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = i0 + 512 * u + tid;
                    if (i < n) val[u] = *reinterpret_cast<const bf16x8*>(src + (size_t)(t0 + i / CPR) * D + 8 * (i % CPR));
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = i0 + 512 * u + tid;
                    if (i < n) {
                        const int pos = first + i / CPR;
                        const size_t slot = ((size_t)bt_lds[pos / kPage] * Hkv + kvh) * kPage + pos % kPage;
                        *reinterpret_cast<bf16x8*>(dst + slot * D + 8 * (i % CPR)) = val[u];
                    }
                }
            }
        };
        copy_rows(knb, kw);
        copy_rows(vnb, vw);
    }
}

template <int D, int kMode>
hipError_t launch_d(const PrefillArgs& a, const int* block_table, const int* seq_lens, int W, hipStream_t stream,
                    int total_tokens = 0, const bf16* kn = nullptr, const bf16* vn = nullptr, bf16* kw = nullptr,
                    bf16* vw = nullptr) {
    const int G = a.Hq / a.Hkv;
    const int BMt = kRows / G;
    // Query blocks per (sequence, kv head) pair; in the packed form, a bound
    // on the blocks of all sequences: sum ceil(T_s / BMt) <= N / BMt + S.
    const int nqb = kMode == kVarlenMode ? (int)varlen_items_bound(total_tokens, a.B, a.T, BMt)
                                         : (a.T + BMt - 1) / BMt;
    const dim3 grid(kMode == kVarlenMode ? (unsigned)nqb * a.Hkv : (unsigned)nqb * a.B * a.Hkv);
    const float c1 = (float)((double)a.scale * 1.4426950408889634);
    if (c1 > 0.f) {
        hipLaunchKernelGGL((prefill_bf16_kernel<D, true, kMode>), grid, dim3(512), 0, stream, (const bf16*)a.q,
                           (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.out, a.lse, a.B, a.Hq, a.Hkv, a.T, G, BMt,
                           nqb, c1, block_table, seq_lens, W, kn, vn, kw, vw);
    } else {
        hipLaunchKernelGGL((prefill_bf16_kernel<D, false, kMode>), grid, dim3(512), 0, stream, (const bf16*)a.q,
                           (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.out, a.lse, a.B, a.Hq, a.Hkv, a.T, G, BMt,
                           nqb, c1, block_table, seq_lens, W, kn, vn, kw, vw);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    return a.d == 128 ? launch_d<128, kDense>(a, nullptr, nullptr, 0, stream)
                      : launch_d<64, kDense>(a, nullptr, nullptr, 0, stream);
}

hipError_t launch_prefill_paged_bf16(const PrefillArgs& a, const int32_t* block_table, const int32_t* seq_lens, int W,
                                     hipStream_t stream) {
    return a.d == 128 ? launch_d<128, kPagedMode>(a, block_table, seq_lens, W, stream)
                      : launch_d<64, kPagedMode>(a, block_table, seq_lens, W, stream);
}

hipError_t launch_prefill_varlen_bf16(const PrefillArgs& a, const int32_t* cu_seqlens, int total_tokens,
                                      hipStream_t stream) {
    return a.d == 128 ? launch_d<128, kVarlenMode>(a, nullptr, cu_seqlens, 0, stream, total_tokens)
                      : launch_d<64, kVarlenMode>(a, nullptr, cu_seqlens, 0, stream, total_tokens);
}

hipError_t launch_prefill_paged_append_bf16(const PrefillArgs& a, const void* k_new, const void* v_new, void* k_pages,
                                            void* v_pages, const int32_t* block_table, const int32_t* seq_lens, int W,
                                            hipStream_t stream) {
    const bf16* kn = static_cast<const bf16*>(k_new);
    const bf16* vn = static_cast<const bf16*>(v_new);
    bf16* kw = static_cast<bf16*>(k_pages);
    bf16* vw = static_cast<bf16*>(v_pages);
    return a.d == 128 ? launch_d<128, kAppendMode>(a, block_table, seq_lens, W, stream, 0, kn, vn, kw, vw)
                      : launch_d<64, kAppendMode>(a, block_table, seq_lens, W, stream, 0, kn, vn, kw, vw);
}

}  // namespace attn
