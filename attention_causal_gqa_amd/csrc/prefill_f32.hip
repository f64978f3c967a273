// Causal prefill in fp32 (vector ALU): the readable kernel of the path.
//
// Blockwise online softmax (llm-from-scratch "Project Overview", "Performance
// Layer: kernel/ and parallel/": softmax statistics kept per block instead of
// a materialised score matrix).  One workgroup of 256 threads owns 64 query
// rows of one (batch, head); four threads share a row, each holding a quarter
// of q and of the output accumulator.  K and V tiles of 64 keys go through
// LDS; the causal mask is applied per element.  Scores are kept in the base-2
// domain (scale * log2(e) folded into one multiplier) so that v_exp_f32 does
// the exponentials.
#include "device_common.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kBM = 64;  // query rows per workgroup
constexpr int kBN = 64;  // keys per tile

template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                          const float* __restrict__ v, float* __restrict__ out,
                                                          float* __restrict__ lse, int B, int Hq, int Hkv, int T,
                                                          int nqb, float c1) {
    constexpr int kVec = D / 16;    // float4 chunks per thread
    constexpr int kLdsW = D + 4;    // floats per LDS row (pad keeps rows off one bank)
    __shared__ float Ks[kBN * kLdsW];
    __shared__ float Vs[kBN * kLdsW];

    const int tid = threadIdx.x;
    const int row = tid >> 2;
    const int part = tid & 3;
    // Heaviest query blocks (most keys) first.
    const int bid = blockIdx.x;
    const int qb = nqb - 1 - bid / (B * Hq);
    const int bh = bid % (B * Hq);
    const int b = bh / Hq;
    const int h = bh % Hq;
    const int kvh = h / (Hq / Hkv);

    const int t0 = qb * kBM;
    const int i = t0 + row;
    const bool valid = i < T;

    // This thread's d values: 16*e + 4*part + c, c = 0..3.
    float4 qr[kVec], o[kVec];
    const float* qrow = q + ((size_t)(b * Hq + h) * T + (valid ? i : T - 1)) * D;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
        qr[e] = *reinterpret_cast<const float4*>(qrow + 16 * e + 4 * part);
        o[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float m = -INFINITY, l = 0.f;

    const float* kb = k + (size_t)(b * Hkv + kvh) * T * D;
    const float* vb = v + (size_t)(b * Hkv + kvh) * T * D;
    const int kend = min(t0 + kBM, T);

    for (int k0 = 0; k0 < kend; k0 += kBN) {
        __syncthreads();
        for (int idx = tid; idx < kBN * D / 4; idx += 256) {
            const int r = idx / (D / 4);
            const int cc = idx % (D / 4);
            const int key = k0 + r;
            float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
            if (key < T) {
                kk = *reinterpret_cast<const float4*>(kb + (size_t)key * D + 4 * cc);
                vv = *reinterpret_cast<const float4*>(vb + (size_t)key * D + 4 * cc);
            }
            *reinterpret_cast<float4*>(&Ks[r * kLdsW + 4 * cc]) = kk;
            *reinterpret_cast<float4*>(&Vs[r * kLdsW + 4 * cc]) = vv;
        }
        __syncthreads();

        float s[kBN];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < kBN; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const float4 kk = *reinterpret_cast<const float4*>(&Ks[j * kLdsW + 16 * e + 4 * part]);
                acc = fmaf(qr[e].x, kk.x, acc);
                acc = fmaf(qr[e].y, kk.y, acc);
                acc = fmaf(qr[e].z, kk.z, acc);
                acc = fmaf(qr[e].w, kk.w, acc);
            }
            acc += __shfl_xor(acc, 1);
            acc += __shfl_xor(acc, 2);
            s[j] = (k0 + j <= i) ? acc * c1 : -INFINITY;
            mt = fmaxf(mt, s[j]);
        }
        // Key 0 is visible to every row and sits in the first tile, so mn is finite.
        const float mn = fmaxf(m, mt);
        const float alpha = fast_exp2(m - mn);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            o[e].x *= alpha; o[e].y *= alpha; o[e].z *= alpha; o[e].w *= alpha;
        }
#pragma unroll
        for (int j = 0; j < kBN; ++j) {
            const float p = fast_exp2(s[j] - mn);
            l += p;
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const float4 vv = *reinterpret_cast<const float4*>(&Vs[j * kLdsW + 16 * e + 4 * part]);
                o[e].x = fmaf(p, vv.x, o[e].x);
                o[e].y = fmaf(p, vv.y, o[e].y);
                o[e].z = fmaf(p, vv.z, o[e].z);
                o[e].w = fmaf(p, vv.w, o[e].w);
            }
        }
        m = mn;
    }

    if (valid) {
        const float inv = 1.f / l;
        float* orow = out + ((size_t)(b * Hq + h) * T + i) * D;
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            *reinterpret_cast<float4*>(orow + 16 * e + 4 * part) =
                make_float4(o[e].x * inv, o[e].y * inv, o[e].z * inv, o[e].w * inv);
        }
        if (lse != nullptr && part == 0) lse[(size_t)(b * Hq + h) * T + i] = (m + log2f(l)) * kLn2;
    }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
    const int nqb = (a.T + kBM - 1) / kBM;
    const dim3 grid((unsigned)nqb * a.B * a.Hq);
    const float c1 = (float)((double)a.scale * 1.4426950408889634);
    if (a.d == 128) {
        hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(256), 0, stream, (const float*)a.q, (const float*)a.k,
                           (const float*)a.v, (float*)a.out, a.lse, a.B, a.Hq, a.Hkv, a.T, nqb, c1);
    } else {
        hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(256), 0, stream, (const float*)a.q, (const float*)a.k,
                           (const float*)a.v, (float*)a.out, a.lse, a.B, a.Hq, a.Hkv, a.T, nqb, c1);
    }
    return hipGetLastError();
}

}  // namespace attn
