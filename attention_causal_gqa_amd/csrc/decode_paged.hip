// Single-token decode over a paged KV cache: split-KV kernel + LSE combine.
//
// The cache is a pool of pages of 16 tokens; the (page, kv head) slice of K
// or V is a contiguous 16 x d block.  Token j of sequence b lives in page
// block_table[b][j / 16], slot j % 16 (the paged KV cache of the RoseLLM
// README, "What is inside" / "Systems highlights"; the mapped KV store and
// KV-cache decode with BF16 storage and FP32 accumulation of the
// microLLM-rocm README, "Why this project exists").
//
// Split kernel: one workgroup (4 waves) per (sequence, kv head, split); a
// split is a fixed run of pages_per_split pages of the sequence's page list,
// and splits past the sequence's last page exit at once.  Wave w takes pages
// w, w+4, ... of the split.  Each lane holds one 16-byte chunk (8 values of
// d) of TPL tokens per page, so every K/V load is a coalesced 16-byte vector
// load and a token row is read by CPR = d/8 consecutive lanes.  All G query
// heads of the kv group are handled together, so each K/V byte is read once
// for the whole group.  q.k partial sums use v_dot2 on bf16 pairs and a DPP
// row reduction.  Every group of CPR lanes runs its own online softmax over
// its tokens (no cross-lane max per page); the streams are merged once at
// the end (shuffles within the wave, LDS across waves) into a normalised
// partial output and its log-sum-exp, written to the workspace.
//
// Combine kernel: per (sequence, query head), partial results of the
// sequence's non-empty splits are merged with log-sum-exp weights
// (block-wise softmax statistics, llm-from-scratch "Project Overview",
// "Performance Layer: kernel/ and parallel/").
#include "device_common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kPage = 16;

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

__device__ __forceinline__ void dma16(const void* g, char* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (s_waitcnt vmcnt(N), other counters untouched; gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// XOR swizzle of the 16-byte chunks of a V page row in LDS: chunk c of row
// r sits at position c ^ vswz(r), so the 32 lanes of a transposing read
// (8 rows x 32 bytes) hit distinct bank groups.
template <int D>
__device__ __forceinline__ int vswz(int r) {
    if constexpr (D == 128) return 2 * (r & 7);
    else return 2 * ((r >> 1) & 3);
}

// Split kernel.  Workgroup = 4 waves per (sequence, kv head, split); wave w
// takes pages w, w+4, ... of the split.  Per page (16 tokens) and wave:
//   S^T = K Q^T   (16 tokens x 16 head columns; v_mfma_f32_16x16x32_bf16,
//                  K read from HBM straight into the A-operand layout, the G
//                  query heads of the kv group in the B columns, zero-padded)
//   online softmax over the page, per head column
//   O  += P V     (16 head rows x d; v_mfma_f32_16x16x16bf16_1k: the S^T
//                  accumulator layout is exactly the P A-operand layout, V
//                  comes HBM -> LDS by DMA and is read transposed)
// The next page's K and V loads are in flight while a page is computed.
template <int D>
__global__ __launch_bounds__(256) void decode_split_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kp,
                                                           const bf16* __restrict__ vp,
                                                           const int32_t* __restrict__ block_table,
                                                           const int32_t* __restrict__ seq_lens,
                                                           float* __restrict__ o_part, float* __restrict__ lse_part,
                                                           int Hq, int Hkv, int G, int W, int S, int pps, float c1) {
    constexpr int NKK = D / 32;        // k-steps of QK^T (16x16x32)
    constexpr int NB = D / 16;         // 16-column blocks of O (16x16x16)
    constexpr int ROWB = D * 2;        // bytes per token row
    constexpr int SLICEB = kPage * ROWB;  // bytes per (page, kv head) slice
    constexpr int NDMA = SLICEB / 1024;   // wave-wide 1 KiB DMAs per slice
    constexpr int RPD = 1024 / ROWB;      // rows per DMA
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    // Per wave: two V slices (double buffer).  After the page loop a wave's
    // region holds its partial O (16 head rows x D fp32 = 2 slices).
    __shared__ __attribute__((aligned(1024))) char Vb0[4][SLICEB];
    __shared__ __attribute__((aligned(1024))) char Vb1[4][SLICEB];
    __shared__ float sM[4][16];
    __shared__ float sL[4][16];
    __shared__ float sLL[4][16];

    const int s = blockIdx.x % S;
    const int bk = blockIdx.x / S;
    const int kvh = bk % Hkv;
    const int b = bk / Hkv;

    const int L = seq_lens[b];
    const int npages = (L + kPage - 1) / kPage;
    const int p0 = s * pps;
    const int p1 = min(p0 + pps, npages);
    if (p0 >= p1) return;  // empty split: the combine kernel never reads it

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int hd = lane & 15;  // head column (S^T, P) / d within a 16-block (O)
    const int g = lane >> 4;   // 16-lane row: tokens 4g..4g+3 (S^T, P) / head rows 4g..4g+3 (O)

    // Q^T as the B operand of S^T: lane holds Q[head hd][32kk + 8g .. +7]; heads >= G are zero.
    bf16x8 qb[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        if (hd < G) {
            qb[kk] = *reinterpret_cast<const bf16x8*>(q + ((size_t)b * Hq + kvh * G + hd) * D + 32 * kk + 8 * g);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) qb[kk][j] = (bf16)0.f;
        }
    }

    // Page ids of the split, 64 at a time, one per lane; a wave visits its
    // pages in increasing order, so each chunk is loaded once.
    const int32_t* bt_row = block_table + (size_t)b * W + p0;
    int pid_chunk = -1;
    int my_pid = 0;
    auto page_id = [&](int p) __attribute__((always_inline)) {
        const int j = p - p0;  // wave-uniform
        if ((j >> 6) != pid_chunk) {
            pid_chunk = j >> 6;
            const int jj = (pid_chunk << 6) + lane;
            my_pid = (jj < p1 - p0) ? bt_row[jj] : 0;
        }
        return __builtin_amdgcn_readlane(my_pid, j & 63);
    };

    // K A-operand: lane holds K[token hd][32kk + 8g .. +7].
    const uint32_t koff = (uint32_t)(hd * ROWB + 16 * g);
    // V DMA: DMA n fills slice bytes [1024n, +1024) = rows RPD*n + lane/CPR,
    // position lane % CPR, i.e. logical chunk (lane % CPR) ^ vswz(row).
    uint32_t voff[NDMA];
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
        const int row = RPD * n + lane / CPR;
        voff[n] = (uint32_t)(row * ROWB + 16 * ((lane % CPR) ^ vswz<D>(row)));
    }
    // V B-operand (transposing read): lane i of 16-lane row g points at token
    // row 4g + i/4, columns 16nb + 4(i%4); chunk 2nb + (i%4)/2 of that row.
    const int vi = hd;
    const int vrow = 4 * g + (vi >> 2);
    const int vread = vrow * ROWB + 8 * (vi & 1) + ((((vi & 3) >> 1) ^ vswz<D>(vrow)) << 4);

    auto issue_page = [&](int p, char* vdst, u32x4 (&ka)[NKK]) __attribute__((always_inline)) {
        const int pid = page_id(p);
        const size_t slice = ((size_t)pid * Hkv + kvh) * (kPage * D);
        const char* kb = reinterpret_cast<const char*>(kp + slice);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) ka[kk] = *reinterpret_cast<const u32x4*>(kb + koff + 64 * kk);
        const char* vb = reinterpret_cast<const char*>(vp + slice);
#pragma unroll
        for (int n = 0; n < NDMA; ++n) dma16(vb + voff[n], vdst + 1024 * n);
    };

    f32x4 oacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max of head column hd, base-2 scaled
    float l_run = 0.f;        // this lane's share of sum(bf16(p)) (its tokens)
    float l_lse = 0.f;        // the same over fp32 p
    constexpr uint32_t kOnes = 0x3F803F80u;

    auto compute_page = [&](int p, const u32x4 (&kcur)[NKK], char* vbuf) __attribute__((always_inline)) {
        // Tokens past L in the last page: zero their V rows (the pool may
        // hold NaN there, and 0 * NaN would reach O).
        const int nvalid = L - p * kPage;
        if (nvalid < kPage) {
#pragma unroll
            for (int n = 0; n < NDMA; ++n) {
                const int row = RPD * n + lane / CPR;
                if (row >= nvalid)
                    *reinterpret_cast<u32x4*>(vbuf + 1024 * n + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
            }
        }
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kcur[kk]), qb[kk], sacc, 0, 0, 0);
        // lane holds S^T[token 4g + i][head hd]
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (4 * g + i < nvalid) ? sacc[i] * c1 : -INFINITY;
        float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = row_pair_max(mx);
        mx = pair_max(mx);  // page max of head column hd, in all 4 rows
        // Move the running max only when the page max exceeds it by more
        // than 8 (base 2): probabilities stay below 256 and O is rescaled
        // rarely.  The first page always moves it (m_run = -inf); a page
        // always has a valid token, so mx is finite.
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
        // V must have landed (this page's DMA is older than the next page's).
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const u32x2 vb = lds_read_tr16(vbuf + (vread ^ (nb << 5)));
            oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, pa),
                                                                 __builtin_bit_cast(s16x4, vb), oacc[nb], 0, 0, 0);
        }
    };

    // Page loop, unrolled by two over two (K registers, V buffer) sets: the
    // next page's loads go into the other set while this page is computed.
    // The V buffers are distinct arrays, so the compiler does not make LDS
    // reads wait for the other buffer's DMA.
    char* vbuf0 = Vb0[w];
    char* vbuf1 = Vb1[w];
    u32x4 ka0[NKK], ka1[NKK];
    int p = p0 + w;
    if (p < p1) issue_page(p, vbuf0, ka0);
    while (p < p1) {
        if (p + 4 < p1) {
            issue_page(p + 4, vbuf1, ka1);
            wait_vmcnt<NKK + NDMA>();
        } else {
            wait_vmcnt<0>();
        }
        compute_page(p, ka0, vbuf0);
        p += 4;
        if (p >= p1) break;
        if (p + 4 < p1) {
            issue_page(p + 4, vbuf0, ka0);
            wait_vmcnt<NKK + NDMA>();
        } else {
            wait_vmcnt<0>();
        }
        compute_page(p, ka1, vbuf1);
        p += 4;
    }

    // Row sums of this wave: add the four 16-lane rows (tokens 4g..4g+3).
    l_run = pair_sum(row_pair_sum(l_run));
    l_lse = pair_sum(row_pair_sum(l_lse));
    if (g == 0) {
        sM[w][hd] = m_run;
        sL[w][hd] = l_run;
        sLL[w][hd] = l_lse;
    }
    // Partial O into this wave's own LDS region (its V buffers, no longer read):
    // lane holds O[head 4g + i][16nb + hd].
    float* sO = reinterpret_cast<float*>(Vb0[w]);  // 16 x D floats span Vb0[w] and Vb1[w]
    static_assert(sizeof(Vb0[0]) * 2 >= 16 * D * sizeof(float), "partial O must fit the wave's V buffers");
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = (4 * g + i) * D + 16 * nb + hd;
            float* dst = idx < SLICEB / 4 ? sO + idx : reinterpret_cast<float*>(Vb1[w]) + (idx - SLICEB / 4);
            *dst = oacc[nb][i];
        }
    __syncthreads();

    // Merge the 4 waves (a wave with no page has m = -inf, l = 0); write
    // the normalised partial output and its LSE.
    for (int idx = tid; idx < G * D; idx += 256) {
        const int h = idx / D;
        const int d = idx % D;
        float M = sM[0][h];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, sM[ww][h]);
        float lsum = 0.f, llse = 0.f, osum = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float f = (sM[ww][h] == -INFINITY) ? 0.f : fast_exp2(sM[ww][h] - M);
            const int oi = h * D + d;
            const float ov = oi < SLICEB / 4 ? reinterpret_cast<const float*>(Vb0[ww])[oi]
                                             : reinterpret_cast<const float*>(Vb1[ww])[oi - SLICEB / 4];
            lsum = fmaf(f, sL[ww][h], lsum);
            llse = fmaf(f, sLL[ww][h], llse);
            osum = fmaf(f, ov, osum);
        }
        const size_t bh = (size_t)b * Hq + kvh * G + h;
        o_part[(bh * S + s) * D + d] = osum / lsum;
        if (d == 0) lse_part[bh * S + s] = (M + log2f(llse)) * kLn2;
    }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float* __restrict__ o_part,
                                                           const float* __restrict__ lse_part,
                                                           const int32_t* __restrict__ seq_lens, bf16* __restrict__ out,
                                                           float* __restrict__ lse, int Hq, int S, int pps) {
    const int bh = blockIdx.x;
    const int b = bh / Hq;
    const int d = threadIdx.x;
    const int L = seq_lens[b];
    if (L == 0) {
        out[(size_t)bh * D + d] = (bf16)0.f;
        if (lse != nullptr && d == 0) lse[bh] = -INFINITY;
        return;
    }
    const int ns = ((L + kPage - 1) / kPage + pps - 1) / pps;
    const float* lp = lse_part + (size_t)bh * S;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, lp[s]);
    float wsum = 0.f, acc = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float wgt = fast_exp2((lp[s] - M) * kLog2e);
        wsum += wgt;
        acc = fmaf(wgt, o_part[((size_t)bh * S + s) * D + d], acc);
    }
    out[(size_t)bh * D + d] = (bf16)(acc / wsum);
    if (lse != nullptr && d == 0) lse[bh] = M + logf(wsum);
}

template <int D>
void launch_split(const DecodeArgs& a, hipStream_t stream, float c1) {
    const dim3 grid((unsigned)a.num_splits * a.Hkv * a.B);
    hipLaunchKernelGGL((decode_split_kernel<D>), grid, dim3(256), 0, stream, (const bf16*)a.q, (const bf16*)a.k_pages,
                       (const bf16*)a.v_pages, a.block_table, a.seq_lens, a.o_part, a.lse_part, a.Hq, a.Hkv,
                       a.Hq / a.Hkv, a.W, a.num_splits, a.pages_per_split, c1);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    const float c1 = (float)((double)a.scale * 1.4426950408889634);
    if (a.d == 128) {
        launch_split<128>(a, stream, c1);
    } else {
        launch_split<64>(a, stream, c1);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.d == 128) {
        hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((unsigned)a.B * a.Hq), dim3(128), 0, stream, a.o_part,
                           a.lse_part, a.seq_lens, (bf16*)a.out, a.lse, a.Hq, a.num_splits, a.pages_per_split);
    } else {
        hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((unsigned)a.B * a.Hq), dim3(64), 0, stream, a.o_part,
                           a.lse_part, a.seq_lens, (bf16*)a.out, a.lse, a.Hq, a.num_splits, a.pages_per_split);
    }
    return hipGetLastError();
}

}  // namespace attn
