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

template <int D>
__device__ __forceinline__ float chunk_row_sum(float x) {
    if constexpr (D == 128) {
        return dpp_row_sum16<float>(x);
    } else {
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
        x += __shfl_xor(x, 4);
        return x;
    }
}

template <int D, int G>
__global__ __launch_bounds__(256) void decode_split_kernel(const bf16* __restrict__ q, const bf16* __restrict__ kp,
                                                           const bf16* __restrict__ vp,
                                                           const int32_t* __restrict__ block_table,
                                                           const int32_t* __restrict__ seq_lens,
                                                           float* __restrict__ o_part, float* __restrict__ lse_part,
                                                           int Hq, int Hkv, int W, int S, int pps, float c1) {
    constexpr int CPR = D / 8;        // lanes per token row
    constexpr int TPI = 64 / CPR;     // tokens per wave-wide load
    constexpr int TPL = kPage / TPI;  // tokens per lane per page
    __shared__ float sM[4][G];
    __shared__ float sL[4][G];
    __shared__ __attribute__((aligned(16))) float sO[4][G][D];

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
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int c = lane % CPR;
    const int r = lane / CPR;

    // Page ids of the split, 64 at a time, one per lane; a wave visits its
    // pages in increasing order, so each chunk is loaded once.
    const int32_t* bt_row = block_table + (size_t)b * W + p0;
    int pid_chunk = -1;
    int my_pid = 0;

    u32x4 qv[G];
#pragma unroll
    for (int h = 0; h < G; ++h)
        qv[h] = *reinterpret_cast<const u32x4*>(q + ((size_t)b * Hq + kvh * G + h) * D + 8 * c);

    float m[G], l[G], o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
    }

    const size_t slice = (size_t)kPage * D;  // elements per (page, kv head)
    u32x4 kr[TPL], vr[TPL];
    auto load_page = [&](int p) {
        const int j = p - p0;  // wave-uniform
        if ((j >> 6) != pid_chunk) {
            pid_chunk = j >> 6;
            const int jj = (pid_chunk << 6) + lane;
            my_pid = (jj < p1 - p0) ? bt_row[jj] : 0;
        }
        const int pid = __builtin_amdgcn_readlane(my_pid, j & 63);
        const size_t base = ((size_t)pid * Hkv + kvh) * slice + (size_t)r * D + 8 * c;
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            kr[i] = *reinterpret_cast<const u32x4*>(kp + base + (size_t)i * TPI * D);
            vr[i] = *reinterpret_cast<const u32x4*>(vp + base + (size_t)i * TPI * D);
        }
    };

    int p = p0 + w;
    if (p < p1) load_page(p);
    while (p < p1) {
        u32x4 kc[TPL], vc[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            kc[i] = kr[i];
            vc[i] = vr[i];
        }
        const int pn = p + 4;
        if (pn < p1) load_page(pn);

        float x[TPL][G];
        bool valid[TPL];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            valid[i] = p * kPage + r + i * TPI < L;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float acc = dot2_bf16(kc[i].x, qv[h].x, 0.f);
                acc = dot2_bf16(kc[i].y, qv[h].y, acc);
                acc = dot2_bf16(kc[i].z, qv[h].z, acc);
                acc = dot2_bf16(kc[i].w, qv[h].w, acc);
                acc = chunk_row_sum<D>(acc);
                x[i][h] = valid[i] ? acc * c1 : -INFINITY;
            }
            if (!valid[i]) vc[i] = u32x4{0u, 0u, 0u, 0u};  // unused slots may hold NaN
        }
        float vf[TPL][8];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
            vf[i][0] = bf16_lo(vc[i].x); vf[i][1] = bf16_hi(vc[i].x);
            vf[i][2] = bf16_lo(vc[i].y); vf[i][3] = bf16_hi(vc[i].y);
            vf[i][4] = bf16_lo(vc[i].z); vf[i][5] = bf16_hi(vc[i].z);
            vf[i][6] = bf16_lo(vc[i].w); vf[i][7] = bf16_hi(vc[i].w);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mt = x[0][h];
#pragma unroll
            for (int i = 1; i < TPL; ++i) mt = fmaxf(mt, x[i][h]);
            const float mn = fmaxf(m[h], mt);
            const float mu = (mn == -INFINITY) ? 0.f : mn;  // no valid token seen yet
            const float alpha = fast_exp2(m[h] - mu);
            float pr[TPL];
            float ls = 0.f;
#pragma unroll
            for (int i = 0; i < TPL; ++i) {
                pr[i] = fast_exp2(x[i][h] - mu);
                ls += pr[i];
            }
            l[h] = fmaf(l[h], alpha, ls);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = o[h][e] * alpha;
#pragma unroll
                for (int i = 0; i < TPL; ++i) acc = fmaf(pr[i], vf[i][e], acc);
                o[h][e] = acc;
            }
            m[h] = mn;
        }
        p = pn;
    }

    // Merge the 64/CPR token streams of this wave (lanes c, c+CPR, ...).
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float M = m[h];
#pragma unroll
        for (int off = CPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
        const float f = (m[h] == -INFINITY) ? 0.f : fast_exp2(m[h] - M);
        float lw = l[h] * f;
        float ow[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ow[e] = o[h][e] * f;
#pragma unroll
        for (int off = CPR; off < 64; off <<= 1) {
            lw += __shfl_xor(lw, off);
#pragma unroll
            for (int e = 0; e < 8; ++e) ow[e] += __shfl_xor(ow[e], off);
        }
        if (r == 0) {
            if (c == 0) {
                sM[w][h] = M;
                sL[w][h] = lw;
            }
            *reinterpret_cast<float4*>(&sO[w][h][8 * c]) = make_float4(ow[0], ow[1], ow[2], ow[3]);
            *reinterpret_cast<float4*>(&sO[w][h][8 * c + 4]) = make_float4(ow[4], ow[5], ow[6], ow[7]);
        }
    }
    __syncthreads();

    // Merge the 4 waves; write the normalised partial output and its LSE.
    for (int idx = tid; idx < G * D; idx += 256) {
        const int h = idx / D;
        const int d = idx % D;
        float M = sM[0][h];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, sM[ww][h]);
        float lsum = 0.f, osum = 0.f;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
            const float f = (sM[ww][h] == -INFINITY) ? 0.f : fast_exp2(sM[ww][h] - M);
            lsum = fmaf(f, sL[ww][h], lsum);
            osum = fmaf(f, sO[ww][h][d], osum);
        }
        const size_t bh = (size_t)b * Hq + kvh * G + h;
        o_part[(bh * S + s) * D + d] = osum / lsum;
        if (d == 0) lse_part[bh * S + s] = (M + log2f(lsum)) * kLn2;
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

template <int D, int G>
void launch_split(const DecodeArgs& a, hipStream_t stream, float c1) {
    const dim3 grid((unsigned)a.num_splits * a.Hkv * a.B);
    hipLaunchKernelGGL((decode_split_kernel<D, G>), grid, dim3(256), 0, stream, (const bf16*)a.q,
                       (const bf16*)a.k_pages, (const bf16*)a.v_pages, a.block_table, a.seq_lens, a.o_part,
                       a.lse_part, a.Hq, a.Hkv, a.W, a.num_splits, a.pages_per_split, c1);
}

template <int D>
void launch_split_g(const DecodeArgs& a, hipStream_t stream, float c1) {
    switch (a.Hq / a.Hkv) {
        case 1: launch_split<D, 1>(a, stream, c1); break;
        case 2: launch_split<D, 2>(a, stream, c1); break;
        case 3: launch_split<D, 3>(a, stream, c1); break;
        case 4: launch_split<D, 4>(a, stream, c1); break;
        case 5: launch_split<D, 5>(a, stream, c1); break;
        case 6: launch_split<D, 6>(a, stream, c1); break;
        case 7: launch_split<D, 7>(a, stream, c1); break;
        default: launch_split<D, 8>(a, stream, c1); break;
    }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    const float c1 = (float)((double)a.scale * 1.4426950408889634);
    if (a.d == 128) {
        launch_split_g<128>(a, stream, c1);
    } else {
        launch_split_g<64>(a, stream, c1);
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
