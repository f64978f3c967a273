// Single-token decode over a paged KV cache: split-KV kernel + LSE combine.
//
// The cache is a pool of pages of 16 tokens; the (page, kv head) slice of K
// or V is a contiguous 16 x d block.  Token j of sequence b lives in page
// block_table[b][j / 16], slot j % 16 (the paged KV cache of the RoseLLM
// README, "What is inside" / "Systems highlights"; the mapped KV store and
// KV-cache decode with BF16 storage and FP32 accumulation of the
// microLLM-rocm README, "Why this project exists").
//
// Streaming split kernel: as many one-wave workgroups as fit on the chip at
// once, each taking an equal share of the flattened stream of all
// (sequence, kv head, page) triples, so that sequences of any mix of lengths
// keep every CU busy without a workgroup per split.  All G query heads of a
// kv group are handled together (16x16 MFMA tiles, G columns used), so each
// K/V byte is read once for the whole group.  Each run of pages of one
// (sequence, kv head) that a wave meets is one piece; its normalised partial
// output and log-sum-exp go to a workspace slot of its own, or, when the
// piece is the whole run, straight to the output.
//
// FP8 form (kFp8): the pools hold FP8 E4M3 codes with one scale per tensor
// (the FP8 KV cache of the microLLM-rocm README, "Why this project exists";
// gfx950's OCP FP8 formats).  A page slice is half as many bytes; K arrives
// 8 bytes per lane and is widened to bf16 in registers
// (v_cvt_scalef32_pk_bf16_fp8, exact: every E4M3 value is a bf16 value),
// V is DMA'd to LDS as FP8 and widened into the bf16 slice layout the
// transposing reads use.  The key scale is folded into the score factor,
// the value scale into the normalisation at the flush.
//
// Combine kernel: per (sequence, query head), the pieces' partial results are
// merged with log-sum-exp weights (block-wise softmax statistics,
// llm-from-scratch "Project Overview", "Performance Layer: kernel/ and
// parallel/").
#include <atomic>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kPage = 16;
constexpr int kMaxDevices = 64;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Max / sum over lanes l and l ^ 16 (v_permlane16_swap exchanges 16-lane
// rows 0<->1 and 2<->3; between them the two results hold both values).
__device__ __forceinline__ float row_pair_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// The page loop's global loads are issued from inline assembly, so the
// compiler's wait-count insertion does not see them; left to it, it drains
// every outstanding load (including the next page's) before the first MFMA
// of each page.  Their completion is awaited explicitly with wait_loads.
//
// Every K/V byte is read once per launch, so the 16-byte loads and the V
// DMA carry the non-temporal (nt) cache policy: a plain 2 GiB streaming read
// on MI355X moved 6.2-6.3 TB/s with ordinary 16-byte loads and 7.0-7.1 TB/s
// with nt ones.  The FP8 form's 8-byte K loads stay ordinary: with nt they
// made that decode about 20% slower.
__device__ __forceinline__ u32x4 gload16(const void* p) {
    u32x4 r;
    asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(r) : "v"(p) : "memory");
    return r;
}
__device__ __forceinline__ u32x2 gload8(const void* p) {
    u32x2 r;
    asm volatile("global_load_dwordx2 %0, %1, off" : "=v"(r) : "v"(p) : "memory");
    return r;
}
// Four FP8 E4M3 codes -> four bf16 (exact), as two packed dwords.
__device__ __forceinline__ u32x2 fp8x4_to_bf16(uint32_t c) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, false);
    const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, true);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}
// 16 bytes per lane, HBM -> LDS: lane l's bytes land at lds + 16 l (lds is
// wave-uniform, passed in M0), non-temporal.
__device__ __forceinline__ void dma16(const void* g, const char* lds) {
    const uint32_t m = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(m) : "memory", "m0");
}
// Wait until at most N of this wave's vector-memory operations are in
// flight (loads complete in issue order).  The memory clobber keeps LDS
// reads below it; the empty statements that follow, one per register set,
// keep the loaded registers' consumers below it.
template <int N>
__device__ __forceinline__ void wait_loads() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <typename T>
__device__ __forceinline__ void after_wait(T& r) {
    asm volatile("" : "+v"(r));
}

// XOR swizzle of the 16-byte chunks of a V page row in LDS: chunk c of row
// r sits at position c ^ vswz(r), so the 32 lanes of a transposing read
// (8 rows x 32 bytes) hit distinct bank groups.
template <int D>
__device__ __forceinline__ int vswz(int r) {
    if constexpr (D == 128) return 2 * (r & 7);
    else return 2 * ((r >> 1) & 3);
}

// Position in a wave's stream of (sequence b, kv head, page j) triples, in
// flattened order: sequence-major, then kv head, then page.  x is the
// flattened offset; n and L are sequence b's page and token counts.
struct Cursor {
    int b, kvh, j, n, L;
    long long x;
};

__device__ __forceinline__ int pages_of(int L) { return (L + kPage - 1) / kPage; }

__device__ __forceinline__ long long readlane64(long long v, int src) {
    const int lo = __builtin_amdgcn_readlane((int)(unsigned long long)v, src);
    const int hi = __builtin_amdgcn_readlane((int)((unsigned long long)v >> 32), src);
    return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ long long wave_incl_scan(long long v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const long long t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

// Streaming split kernel: one wave per workgroup, as many workgroups as fit
// on the chip at once (at most kMaxStreamWaves).  The work is the flattened
// stream of all (sequence, kv head, page) triples (Hkv * sum_b ceil(L_b /
// 16) pages); wave w takes the pages from snap(w C) up to snap((w + 1) C),
// C = ceil(total / waves), where snap moves an offset up to the next item
// start.  An item is a run of pps pages of one (sequence, kv head) beginning
// at a multiple of pps, so every wave gets C pages give or take pps,
// whatever the mix of lengths, and a sequence's keys are cut only at item
// starts.  An item starting at offset e belongs to wave floor(e / C).
//
// A wave keeps one online softmax per (sequence, kv head) run it meets (a
// piece).  The pieces of run r (r = b * Hkv + kv head) belong to consecutive
// waves w_first .. w_last, and the piece of wave w is stored in workspace
// slot r + w: along the stream either r or w grows from one piece to the
// next, so slots are distinct, and there are fewer than B * Hkv + waves of
// them.  The wave that meets a run's first page records (first slot, piece
// count) for the combine kernel; a run that lies inside one wave is
// normalised and written to out / lse directly (piece count recorded as 0).
// Per page (16 tokens) and wave:
//   S^T = K Q^T   (16 tokens x 16 head columns; v_mfma_f32_16x16x32_bf16,
//                  K read from HBM straight into the A-operand layout, the G
//                  query heads of the kv group in the B columns, zero-padded)
//   online softmax over the page, per head column
//   O  += P V     (16 head rows x d; v_mfma_f32_16x16x16bf16_1k: the S^T
//                  accumulator layout is exactly the P A-operand layout, V
//                  comes HBM -> LDS by DMA and is read transposed)
// The next page's K and V loads are in flight while a page is computed, and
// the block-table entry of the page after that is loaded a step earlier.
//
// Append form (kAppend): the newest token of each sequence (position L - 1)
// is not yet in the pools; its key and value rows arrive in kn, vn
// [B, Hkv, d].  On a run's last page the lanes that would load row
// (L - 1) % 16 load it from there instead (same number of loads), so no
// wave reads the slot; the combine kernel, which runs after this one,
// writes it.
template <int D, bool kFp8, bool kAppend>
__global__ __launch_bounds__(64) void decode_stream_kernel(const bf16* __restrict__ q, const char* __restrict__ kp,
                                                            const char* __restrict__ vp,
                                                            const int32_t* __restrict__ block_table,
                                                            const int32_t* __restrict__ seq_lens,
                                                            bf16* __restrict__ out, float* __restrict__ lse,
                                                            float* __restrict__ o_part, float* __restrict__ lse_part,
                                                            int* __restrict__ run_info, int B, int Hq, int Hkv, int G,
                                                            int W, int pps, float c1, float vscale,
                                                            const bf16* __restrict__ kn, const bf16* __restrict__ vn) {
    static_assert(!(kFp8 && kAppend), "the append form reads bf16 pools");
    constexpr int NKK = D / 32;        // k-steps of QK^T (16x16x32)
    constexpr int NB = D / 16;         // 16-column blocks of O (16x16x16)
    constexpr int ROWB = D * 2;        // bytes per token row in bf16 (the LDS layout of V)
    constexpr int SLICEB = kPage * ROWB;  // bytes per bf16 (page, kv head) slice
    constexpr int CPR = D / 8;            // 16-byte bf16 chunks per row
    constexpr int KROWB = kFp8 ? D : ROWB;           // bytes per token row in the pools
    constexpr int KSLICEB = kPage * KROWB;           // bytes per pool slice
    constexpr int NDMA = KSLICEB / 1024;             // wave-wide 1 KiB DMAs per slice
    constexpr int RPD = 1024 / KROWB;                // rows per DMA
    constexpr int KCPR = KROWB / 16;                 // 16-byte chunks per pool row
    // Two slices of V as it arrives (double buffer); the FP8 form widens the
    // current one into Vw, read by the PV MFMAs.
    __shared__ __attribute__((aligned(1024))) char Vb0[KSLICEB];
    __shared__ __attribute__((aligned(1024))) char Vb1[KSLICEB];
    __shared__ __attribute__((aligned(1024))) char Vw[kFp8 ? SLICEB : 16];

    const int lane = threadIdx.x;
    const int hd = lane & 15;  // head column (S^T, P) / d within a 16-block (O)
    const int g = lane >> 4;   // 16-lane row: tokens 4g..4g+3 (S^T, P) / head rows 4g..4g+3 (O)
    const int wv = blockIdx.x;

    // ---- this wave's share of the page stream
    // Lane l sums the pages of the contiguous block of sequences
    // [l per, (l + 1) per), per = ceil(B / 64); a scan over the lanes gives
    // each block's first offset.  All of a lane's loads are independent, so
    // the whole pass is one round trip to memory, whatever B is.
    const int per = (B + 63) >> 6;
    const int blk0 = min(B, lane * per);
    const int blk1 = min(B, blk0 + per);
    int Lself = 0;  // per == 1: this lane's own sequence length
    long long sblk = 0;
    if (per == 1) {
        Lself = blk0 < blk1 ? seq_lens[blk0] : 0;
        sblk = pages_of(Lself);
    } else {
        for (int i = blk0; i < blk1; i += 4) {
            int lv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) lv[u] = i + u < blk1 ? seq_lens[i + u] : 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) sblk += pages_of(lv[u]);
        }
    }
    const long long iblk = wave_incl_scan(sblk, lane);
    const long long total = readlane64(iblk, 63) * Hkv;
    const long long C = (total + gridDim.x - 1) / gridDim.x;
    const long long xa = (long long)wv * C;
    if (xa >= total) return;
    const long long xb = xa + C < total ? xa + C : total;

    // Cursor at snap(x), x < total; c.j may equal c.n (then the item start
    // is the next run's first page, see normalize).
    auto locate = [&](long long x, Cursor& c) __attribute__((always_inline)) {
        // the lane block holding x, then the sequence within it
        const unsigned long long hit = __ballot(sblk > 0 && (iblk - sblk) * Hkv <= x && x < iblk * Hkv);
        const int src = __builtin_ctzll(hit);
        long long base = readlane64(iblk - sblk, src);  // pages of the sequences before the block
        if (per == 1) {
            c.b = src;
            c.L = __builtin_amdgcn_readlane(Lself, src);
            c.n = pages_of(c.L);
        } else {
            const int e1 = min(B, src * per + per);
            for (int c0 = src * per; c0 < e1; c0 += 64) {
                const int bb = c0 + lane;
                const int Lb = bb < e1 ? seq_lens[bb] : 0;
                const int n = pages_of(Lb);
                const long long inc = wave_incl_scan((long long)n, lane);
                const long long e = (base + inc - n) * Hkv;
                const unsigned long long h2 = __ballot(n > 0 && e <= x && x < e + (long long)n * Hkv);
                if (h2) {
                    const int s2 = __builtin_ctzll(h2);
                    c.b = c0 + s2;
                    c.n = __builtin_amdgcn_readlane(n, s2);
                    c.L = __builtin_amdgcn_readlane(Lb, s2);
                    base += readlane64(inc, s2) - c.n;
                    break;
                }
                base += readlane64(inc, 63);
            }
        }
        const long long eb = base * Hkv;  // flattened offset of sequence c.b
        const int r = (int)(x - eb);
        c.kvh = r / c.n;
        const int jr = (r % c.n + pps - 1) / pps * pps;
        c.j = jr < c.n ? jr : c.n;
        c.x = eb + (long long)c.kvh * c.n + c.j;
    };
    // Move a cursor with j == n to the next run's first page.  Only called
    // when c.x < total, so a non-empty sequence follows.
    auto normalize = [&](Cursor& c) __attribute__((always_inline)) {
        if (c.j < c.n) return;
        c.j = 0;
        if (++c.kvh < Hkv) return;
        c.kvh = 0;
        do {
            ++c.b;
            c.L = seq_lens[c.b];
            c.n = pages_of(c.L);
        } while (c.n == 0);
    };

    Cursor cc;  // page being computed
    locate(xa, cc);
    long long xe = total;
    if (xb < total) {
        Cursor ce;
        locate(xb, ce);
        xe = ce.x;
    }
    const long long xs = cc.x;
    if (xs >= xe) return;  // no item starts in this wave's range
    normalize(cc);

    auto advance = [&](Cursor& c) __attribute__((always_inline)) {
        ++c.x;
        ++c.j;
        if (c.x < xe) normalize(c);
    };
    auto page_id = [&](const Cursor& c) __attribute__((always_inline)) {
        return block_table[(size_t)c.b * W + c.j];
    };

    // Q^T as the B operand of S^T: lane holds Q[head hd][32kk + 8g .. +7].
    // Columns hd >= G repeat head G - 1; their results are never stored.
    bf16x8 qb[NKK];
    typedef std::conditional_t<kFp8, u32x2, u32x4> KReg;  // a lane's K A-operand as it arrives
    auto load_q = [&](int b, int kvh) __attribute__((always_inline)) {
        const int hh = hd < G ? hd : G - 1;
        const bf16* qrow = q + ((size_t)b * Hq + (size_t)kvh * G + hh) * D + 8 * g;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qb[kk] = __builtin_bit_cast(bf16x8, gload16(qrow + 32 * kk));
    };

    // K A-operand: lane holds K[token hd][32kk + 8g .. +7].
    const uint32_t koff = (uint32_t)(hd * KROWB + (kFp8 ? 8 : 16) * g);
    // V DMA: DMA n fills slice bytes [1024n, +1024) = rows RPD*n + lane/KCPR,
    // position lane % KCPR.  bf16: logical chunk (lane % CPR) ^ vswz(row),
    // the swizzled layout the transposing reads expect; FP8: in order (the
    // widening pass swizzles).
    uint32_t voff[NDMA];
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
        const int row = RPD * n + lane / KCPR;
        voff[n] = (uint32_t)(row * KROWB + 16 * (kFp8 ? lane % KCPR : (lane % CPR) ^ vswz<D>(row)));
    }
    // V B-operand (transposing read): lane i of 16-lane row g points at token
    // row 4g + i/4, columns 16nb + 4(i%4); chunk 2nb + (i%4)/2 of that row.
    const int vi = hd;
    const int vrow = 4 * g + (vi >> 2);
    const int vread = vrow * ROWB + 8 * (vi & 1) + ((((vi & 3) >> 1) ^ vswz<D>(vrow)) << 4);

    auto issue_page = [&](int pid, const Cursor& c, char* vdst, KReg(&ka)[NKK]) __attribute__((always_inline)) {
        const int kvh = c.kvh;
        const size_t slice = ((size_t)pid * Hkv + kvh) * KSLICEB;
        const char* kb = kp + slice;
        if constexpr (kAppend) {
            // Wave-uniform (the cursor is), made explicit so that the branch
            // is a scalar one: under a vector branch the compiler would run
            // both paths under exec masks, one after the other.
            if (__builtin_amdgcn_readfirstlane(c.j == c.n - 1)) {
                // The run's last page: row nrow is the new token, read from
                // kn / vn (rows of ROWB bytes, the same chunk offsets).
                const int nrow = __builtin_amdgcn_readfirstlane((c.L - 1) % kPage);
                const size_t nr = ((size_t)c.b * Hkv + kvh) * ROWB;
                const char* kr = reinterpret_cast<const char*>(kn) + nr;
                const char* vr = reinterpret_cast<const char*>(vn) + nr;
                const char* kl = hd == nrow ? kr + (koff - (uint32_t)(hd * KROWB)) : kb + koff;
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) ka[kk] = gload16(kl + 64 * kk);
                const char* vb = vp + slice;
#pragma unroll
                for (int n = 0; n < NDMA; ++n) {
                    const int row = RPD * n + lane / KCPR;
                    dma16(row == nrow ? vr + (voff[n] - (uint32_t)(row * KROWB)) : vb + voff[n], vdst + 1024 * n);
                }
                return;
            }
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if constexpr (kFp8) ka[kk] = gload8(kb + koff + 32 * kk);
            else ka[kk] = gload16(kb + koff + 64 * kk);
        }
        const char* vb = vp + slice;
#pragma unroll
        for (int n = 0; n < NDMA; ++n) dma16(vb + voff[n], vdst + 1024 * n);
    };

    f32x4 oacc[NB];
    float m_run, l_run, l_lse;  // running max (base-2 scaled), sum(bf16(p)), sum(p)
    auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run = -INFINITY;
        l_run = 0.f;
        l_lse = 0.f;
    };
    constexpr uint32_t kOnes = 0x3F803F80u;

    auto compute_page = [&](const Cursor& c, const KReg(&kcur)[NKK], char* vslot) __attribute__((always_inline)) {
        const int nvalid = c.L - c.j * kPage;
        char* vbuf = vslot;
        if constexpr (kFp8) {
            // Widen V into the bf16 layout: (row r, 8-value chunk cc) for
            // chunk index lane + 64 i; rows past L become zeros (the pool may
            // hold NaN codes there, and 0 * NaN would reach O).
            constexpr int NCH = kPage * CPR / 64;
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int n = lane + 64 * i;
                const int r = n / CPR, cc = n % CPR;
                u32x4 wv4 = {0u, 0u, 0u, 0u};
                if (r < nvalid) {
                    const u32x2 f = *reinterpret_cast<const u32x2*>(vslot + r * KROWB + 8 * cc);
                    const u32x2 a = fp8x4_to_bf16(f.x), b2 = fp8x4_to_bf16(f.y);
                    wv4 = u32x4{a.x, a.y, b2.x, b2.y};
                }
                *reinterpret_cast<u32x4*>(Vw + r * ROWB + 16 * (cc ^ vswz<D>(r))) = wv4;
            }
            vbuf = Vw;
        } else if (nvalid < kPage) {
            // Tokens past L in the last page: zero their V rows (the pool may
            // hold NaN there, and 0 * NaN would reach O).
#pragma unroll
            for (int n = 0; n < NDMA; ++n) {
                const int row = RPD * n + lane / CPR;
                if (row >= nvalid)
                    *reinterpret_cast<u32x4*>(vbuf + 1024 * n + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
            }
        }
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            u32x4 kop;
            if constexpr (kFp8) {
                const u32x2 a = fp8x4_to_bf16(kcur[kk].x), b2 = fp8x4_to_bf16(kcur[kk].y);
                kop = u32x4{a.x, a.y, b2.x, b2.y};
            } else {
                kop = kcur[kk];
            }
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop), qb[kk], sacc, 0, 0, 0);
        }
        // lane holds S^T[token 4g + i][head hd]
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (4 * g + i < nvalid) ? sacc[i] * c1 : -INFINITY;
        float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = row_pair_max(mx);
        mx = pair_max(mx);  // page max of head column hd, in all 4 rows
        // Move the running max only when the page max exceeds it by more
        // than 8 (base 2): probabilities stay below 256 and O is rescaled
        // rarely.  A piece's first page always moves it (m_run = -inf); a
        // page always has a valid token, so mx is finite.
        const bool grow = mx > m_run + 8.f;
        if (__any(grow)) {
            const float mn = grow ? mx : m_run;
            const float alpha = fast_exp2(m_run - mn);  // this lane's head column
            l_run *= alpha;
            l_lse *= alpha;
            // O rows are heads 4g + i: fetch their alphas from those columns.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * g + i);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) oacc[nb][i] *= ai;
            }
            m_run = mn;
        }
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(x[i] - m_run);
        const uint32_t p01 = pack_bf16x2(pr[0], pr[1]);
        const uint32_t p23 = pack_bf16x2(pr[2], pr[3]);
        l_run = dot2_bf16(p23, kOnes, dot2_bf16(p01, kOnes, l_run));
        l_lse += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        const u32x2 pa = {p01, p23};  // A operand: P[head hd][tokens 4g .. 4g+3]
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const u32x2 vb = lds_read_tr16(vbuf + (vread ^ (nb << 5)));
            oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, pa),
                                                                 __builtin_bit_cast(s16x4, vb), oacc[nb], 0, 0, 0);
        }
    };

    // Current piece: its (sequence, kv head), and whether it is its run's
    // only piece (then it is the final result).
    int pb = 0, pkvh = 0;
    bool psingle = false;
    auto flush = [&]() __attribute__((always_inline)) {
        // Row sums: add the four 16-lane rows (tokens 4g..4g+3).
        const float lr = pair_sum(row_pair_sum(l_run));
        const float ll = pair_sum(row_pair_sum(l_lse));
        const float inv = vscale / lr;
        const float lse_v = (m_run + log2f(ll)) * kLn2;
        const size_t bh0 = (size_t)pb * Hq + (size_t)pkvh * G;
        const size_t slot = (size_t)pb * Hkv + pkvh + wv;
        // lane holds O[head 4g + i][16nb + hd]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int head = 4 * g + i;
            const float ih = __shfl(inv, head);
            if (head < G) {
                if (psingle) {
                    bf16* dst = out + (bh0 + head) * D + hd;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) dst[16 * nb] = (bf16)(oacc[nb][i] * ih);
                } else {
                    float* dst = o_part + (slot * G + head) * D + hd;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) dst[16 * nb] = oacc[nb][i] * ih;
                }
            }
        }
        if (g == 0 && hd < G) {
            if (!psingle) lse_part[slot * G + hd] = lse_v;
            else if (lse != nullptr) lse[bh0 + hd] = lse_v;
        }
    };

    // Page loop, unrolled by two over two (K registers, V buffer) sets: the
    // next page's loads go into the other set while this page is computed.
    // The V buffers are distinct arrays, so the compiler does not make LDS
    // reads wait for the other buffer's DMA.
    KReg ka0[NKK], ka1[NKK];
    issue_page(page_id(cc), cc, Vb0, ka0);
    Cursor cf = cc;  // page whose loads go out next
    advance(cf);
    int pid_f = cf.x < xe ? page_id(cf) : 0;

    auto step = [&](KReg(&kx)[NKK], char* bx, KReg(&ky)[NKK], char* by) __attribute__((always_inline)) {
        const bool first_of_run = cc.j == 0 || cc.x == xs;
        if (first_of_run) load_q(cc.b, cc.kvh);
        const bool more = cf.x < xe;
        Cursor cn = cf;
        int pid_n = 0;
        if (more) {
            issue_page(pid_f, cf, by, ky);
            advance(cn);
            if (cn.x < xe) pid_n = page_id(cn);
            wait_loads<NKK + NDMA>();  // all but the next page's loads
        } else {
            wait_loads<0>();
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            after_wait(kx[kk]);
            after_wait(qb[kk]);
        }
        if (first_of_run) {
            if (cc.x != xs) flush();
            reset();
            pb = cc.b;
            pkvh = cc.kvh;
            if (cc.j == 0) {
                // The run starts here, at x = cc.x (its first item belongs to
                // this wave).  Its K items start at x + k pps and belong to
                // waves floor((x + k pps) / C): with pps < C these are every
                // wave from wv to that of the last item, with pps >= C one
                // wave per item.  One store, so the loads in flight stay
                // countable.
                const int K = (cc.n + pps - 1) / pps;
                const long long e_last = cc.x + (long long)(K - 1) * pps;
                const int npieces = pps >= C ? K : (int)(e_last / C) - wv + 1;
                psingle = npieces == 1;
                if (lane == 0) {
                    const int r = cc.b * Hkv + cc.kvh;
                    *reinterpret_cast<int4*>(run_info + 4 * (size_t)r) =
                        int4{r + wv, psingle ? 0 : npieces, (int)(cc.x - (long long)wv * C), (int)C};
                }
            } else {
                psingle = false;
            }
        }
        compute_page(cc, kx, bx);
        cc = cf;
        cf = cn;
        pid_f = pid_n;
        return more;
    };
    for (;;) {
        if (!step(ka0, Vb0, ka1, Vb1)) break;
        if (!step(ka1, Vb1, ka0, Vb0)) break;
    }
    flush();
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Combine kernel: one wave per (sequence, query head).  The split kernel
// records, per run, its first slot, its piece count (0: the run was one
// piece, already written to out / lse), the offset o of the run's first item
// within its wave's share, and the share size C.  Piece i is in slot
// first + i when items are shorter than a share (pps < C), else in slot
// first + floor((o + i pps) / C) (one wave per item).  Pieces are merged
// with weights exp(lse_i - max lse) (block-wise softmax statistics,
// llm-from-scratch "Project Overview", "Performance Layer: kernel/ and
// parallel/").  The first BATCH partial rows are loaded together with the
// pieces' lse values, so a run of up to BATCH pieces costs one round trip
// after the run record.
//
// Append form (kAppend): the wave of each kv group's first head also writes
// the sequence's newest token (position L - 1) from kn / vn [B, Hkv, d] into
// its slot of the pools kw / vw.  The split kernel has finished by then, and
// it read that token from kn / vn, not from the slot.
template <int D, bool kAppend>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ o_part,
                                                            const float* __restrict__ lse_part,
                                                            const int* __restrict__ run_info,
                                                            const int32_t* __restrict__ seq_lens,
                                                            bf16* __restrict__ out, float* __restrict__ lse, int Hq,
                                                            int Hkv, int G, int pps, const bf16* __restrict__ kn,
                                                            const bf16* __restrict__ vn, bf16* __restrict__ kw,
                                                            bf16* __restrict__ vw,
                                                            const int32_t* __restrict__ block_table, int W) {
    constexpr int NDW = D / 64;  // d values per lane
    constexpr int BATCH = 8;
    const int bh = blockIdx.x;
    const int b = bh / Hq;
    const int h = bh % Hq;
    const int r = b * Hkv + h / G;
    const int hh = h % G;
    const int lane = threadIdx.x;
    const int L = seq_lens[b];
    const int4 info = *reinterpret_cast<const int4*>(run_info + 4 * (size_t)r);
    bf16* orow = out + (size_t)bh * D;
    if constexpr (kAppend) {
        constexpr int CPR = D / 8;  // 16-byte chunks per row
        if (hh == 0 && L > 0 && lane < 2 * CPR) {
            const int pos = L - 1;
            const int kvh = h / G;
            const int c = lane % CPR;
            const bool isv = lane >= CPR;
            const size_t page = (size_t)block_table[(size_t)b * W + pos / kPage];
            const u32x4 val =
                *reinterpret_cast<const u32x4*>((isv ? vn : kn) + ((size_t)b * Hkv + kvh) * D + 8 * c);
            *reinterpret_cast<u32x4*>((isv ? vw : kw) + ((page * Hkv + kvh) * kPage + pos % kPage) * D + 8 * c) = val;
        }
    }
    if (L == 0) {
#pragma unroll
        for (int k = 0; k < NDW; ++k) orow[64 * k + lane] = (bf16)0.f;
        if (lse != nullptr && lane == 0) lse[bh] = -INFINITY;
        return;
    }
    const int first = info.x, count = info.y;
    if (count == 0) return;  // a single piece: the split kernel wrote the result
    const unsigned o = (unsigned)info.z, Cs = (unsigned)info.w;
    const bool itemwise = (unsigned)pps >= Cs;
    // slot of piece i (i < count); o + i pps < 2^31 + 2^27 fits 32 bits
    auto slot = [&](int i) __attribute__((always_inline)) {
        return first + (itemwise ? (int)((o + (unsigned)i * (unsigned)pps) / Cs) : i);
    };
    // slot s holds head hh's partial row at (s G + hh)
    const float* lp = lse_part + hh;
    const float* op = o_part + (size_t)hh * D + lane;
    const size_t rstride = (size_t)G * D;
    const float l0 = lane < count ? lp[(size_t)slot(lane) * G] : -INFINITY;
    float v[BATCH][NDW];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
        const size_t row = (size_t)slot(min(u, count - 1));
#pragma unroll
        for (int k = 0; k < NDW; ++k) v[u][k] = op[row * rstride + 64 * k];
    }
    float M = l0;
    for (int c0 = 64; c0 < count; c0 += 64)
        M = fmaxf(M, c0 + lane < count ? lp[(size_t)slot(c0 + lane) * G] : -INFINITY);
    M = wave_max(M);  // finite: every piece holds at least one token
    float acc[NDW];
#pragma unroll
    for (int k = 0; k < NDW; ++k) acc[k] = 0.f;
    float wsum = 0.f;
    for (int c0 = 0; c0 < count; c0 += 64) {
        const int n = min(64, count - c0);
        const float l = c0 == 0 ? l0 : (lane < n ? lp[(size_t)slot(c0 + lane) * G] : -INFINITY);
        const float wt = fast_exp2((l - M) * kLog2e);  // 0 past the last piece
        wsum += wt;
        for (int u0 = 0; u0 < n; u0 += BATCH) {
            if (c0 + u0 != 0) {
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                    const size_t row = (size_t)slot(c0 + min(u0 + u, n - 1));
#pragma unroll
                    for (int k = 0; k < NDW; ++k) v[u][k] = op[row * rstride + 64 * k];
                }
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const float ws = u0 + u < n ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), u0 + u))
                                            : 0.f;
#pragma unroll
                for (int k = 0; k < NDW; ++k) acc[k] = fmaf(ws, v[u][k], acc[k]);
            }
        }
    }
    wsum = wave_sum(wsum);
    const float inv = 1.f / wsum;
#pragma unroll
    for (int k = 0; k < NDW; ++k) orow[64 * k + lane] = (bf16)(acc[k] * inv);
    if (lse != nullptr && lane == 0) lse[bh] = M + logf(wsum);
}

// Workgroups of the streaming kernel that are resident at once on `dev`
// (compute units x occupancy, at most kMaxStreamWaves), found once per device.
template <int D, bool kFp8, bool kAppend>
hipError_t stream_waves(int dev, int* nw) {
    static std::atomic<int> cache[kMaxDevices];
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0, per = 0;
        hipError_t e;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        // The occupancy query reads the current device's properties: run it
        // with `dev` current.
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, decode_stream_kernel<D, kFp8, kAppend>, 64, 0);
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        v = cus * (per > 0 ? per : 1);
        if (v > kMaxStreamWaves) v = kMaxStreamWaves;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    *nw = v;
    return hipSuccess;
}

template <int D, bool kFp8, bool kAppend>
hipError_t launch_split(const DecodeArgs& a, int dev, hipStream_t stream, float c1, float vscale, const bf16* kn,
                        const bf16* vn) {
    int nw = 0;
    const hipError_t e = stream_waves<D, kFp8, kAppend>(dev, &nw);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_stream_kernel<D, kFp8, kAppend>), dim3((unsigned)nw), dim3(64), 0, stream,
                       (const bf16*)a.q, (const char*)a.k_pages, (const char*)a.v_pages, a.block_table, a.seq_lens,
                       (bf16*)a.out, a.lse, a.o_part, a.lse_part, a.run_info, a.B, a.Hq, a.Hkv, a.Hq / a.Hkv, a.W,
                       a.pages_per_split, c1, vscale, kn, vn);
    return hipGetLastError();
}

template <int D, bool kAppend>
hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream, const bf16* kn, const bf16* vn) {
    hipLaunchKernelGGL((decode_combine_kernel<D, kAppend>), dim3((unsigned)a.B * a.Hq), dim3(64), 0, stream, a.o_part,
                       a.lse_part, a.run_info, a.seq_lens, (bf16*)a.out, a.lse, a.Hq, a.Hkv, a.Hq / a.Hkv,
                       a.pages_per_split, kn, vn, (bf16*)a.k_pages, (bf16*)a.v_pages, a.block_table, a.W);
    return hipGetLastError();
}

// kn / vn: the newest token's key and value rows [B, Hkv, d] (append form),
// or null.
template <bool kFp8, bool kAppend>
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, float kscale, float vscale,
                         const bf16* kn = nullptr, const bf16* vn = nullptr) {
    const float c1 = (float)((double)a.scale * (double)kscale * 1.4426950408889634);
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    e = a.d == 128 ? launch_split<128, kFp8, kAppend>(a, dev, stream, c1, vscale, kn, vn)
                   : launch_split<64, kFp8, kAppend>(a, dev, stream, c1, vscale, kn, vn);
    if (e != hipSuccess) return e;
    return a.d == 128 ? launch_combine<128, kAppend>(a, stream, kn, vn) : launch_combine<64, kAppend>(a, stream, kn, vn);
}

// Workspace of attn_decode_paged_noalloc, for callers that cannot allocate:
// device memory that each GPU the library runs on holds from the library's
// load until the process ends.  Its host-side name is not a device address;
// host code uses the address hipGetSymbolAddress returns for the device.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

}  // namespace

hipError_t decode_scratch(hipStream_t stream, void** ptr) {
    static std::mutex mu;
    static void* addr[kMaxDevices];
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        // Looked up once per device, with that device current: every GPU
        // holds its own copy of the array at its own address.
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    return launch_decode<false, false>(a, stream, 1.0f, 1.0f);
}

hipError_t launch_decode_append_bf16(const DecodeArgs& a, const void* k_new, const void* v_new, hipStream_t stream) {
    return launch_decode<false, true>(a, stream, 1.0f, 1.0f, static_cast<const bf16*>(k_new),
                                      static_cast<const bf16*>(v_new));
}

hipError_t launch_decode_fp8(const DecodeArgs& a, float kscale, float vscale, hipStream_t stream) {
    return launch_decode<true, false>(a, stream, kscale, vscale);
}

}  // namespace attn
