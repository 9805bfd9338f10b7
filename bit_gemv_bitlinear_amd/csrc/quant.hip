// quant.hip -- per-token absmax int8 activation quantisation.
//
// Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
// (blog.gitcode.com), §六 item 3: per token, s = 127 / max|x|, then round and
// clamp to [-128, 127] into int8.  Readings: round half to even; max|x| is
// floored at 1e-5 (as the page's weight quantiser floors its mean); fp32
// throughout, with IEEE division and multiplication.
//
// One workgroup per row.  Pass 1 reads the row in 8-element chunks and
// reduces max|x| (order-independent, so the result does not depend on the
// schedule); pass 2 re-reads the row (L2-resident) and writes 8 int8 per chunk.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kQuantThreads = 256;

template <bool BF16>
__device__ __forceinline__ void load8(const void* x, size_t idx8, float (&v)[8]) {
    if (BF16) {
        const uint4 u = reinterpret_cast<const uint4*>(x)[idx8];
        const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(d[j] << 16);
            v[2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
        }
    } else {
        const float4 a = reinterpret_cast<const float4*>(x)[2 * idx8];
        const float4 b = reinterpret_cast<const float4*>(x)[2 * idx8 + 1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

template <bool BF16>
__global__ __launch_bounds__(kQuantThreads) void quant_kernel(const void* __restrict__ x,
                                                             int8_t* __restrict__ q,
                                                             float* __restrict__ s, int K) {
    __shared__ float wave_amax[kQuantThreads / 64];
    const int m = blockIdx.x;
    const int chunks = K >> 3;
    const size_t row8 = static_cast<size_t>(m) * chunks;

    float amax = 0.0f;
    for (int c = threadIdx.x; c < chunks; c += kQuantThreads) {
        float v[8];
        load8<BF16>(x, row8 + c, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) wave_amax[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = wave_amax[0];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; ++w) amax = fmaxf(amax, wave_amax[w]);
    const float sm = 127.0f / fmaxf(amax, 1e-5f);

    uint2* qrow = reinterpret_cast<uint2*>(q + static_cast<size_t>(m) * K);
    for (int c = threadIdx.x; c < chunks; c += kQuantThreads) {
        float v[8];
        load8<BF16>(x, row8 + c, v);
        uint2 o;
        o.x = quant4(v[0], v[1], v[2], v[3], sm);
        o.y = quant4(v[4], v[5], v[6], v[7], sm);
        qrow[c] = o;
    }
    if (threadIdx.x == 0) s[m] = sm;
}

}  // namespace

hipError_t launch_quant(const void* x, int x_is_bf16, int8_t* q, float* s, int M, int K,
                        hipStream_t stream) {
    if (x_is_bf16)
        quant_kernel<true><<<M, kQuantThreads, 0, stream>>>(x, q, s, K);
    else
        quant_kernel<false><<<M, kQuantThreads, 0, stream>>>(x, q, s, K);
    return hipGetLastError();
}

}  // namespace bl
