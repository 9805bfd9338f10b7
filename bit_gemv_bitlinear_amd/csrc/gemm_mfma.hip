// gemm_mfma.hip -- the batched (M >= 2) W2A8 ternary layer on gfx950 int8 MFMA.
//
// Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
// (blog.gitcode.com), cited as [W2A8].  The page's kernel handles M == 1
// only (§一, §八); the batched path is the same arithmetic -- int8
// activations times ternary weights into int32, then the §5.3 epilogue per
// row m with its own activation scale s[m] -- run on the matrix cores, since
// for M >= 16 the layer is a dense contraction.
//
// Mapping (this library's design):
//   * workgroup (column, mchunk): four 16-row bands = 64 output rows n x up
//     to 64 rows m, 4 wavefronts that split the K steps (64 K each) between
//     them;
//   * per K step a wavefront reads, for each of the four bands t, one word per
//     lane: lane (j = lane%16, g = lane/16) takes the word of row j for the
//     16-wide K chunk g of this step -- byte 256*(j/4) + 64*(step%4) + 16*g +
//     4*(j%4) of the band's 1 KiB tile -- which is exactly the B operand of
//     v_mfma_i32_16x16x64_i8 for that band (16 K of one column);
//     v_perm_b32 turns the 2-bit codes into signed int8 weights (code 0, the
//     padding, becomes 0) after each shift-and-mask of [W2A8] §5.2;
//   * the A operand (16 rows m x 64 K) is read straight from the int8
//     activations, 16 bytes per lane, zero outside M and K;
//   * the four wavefronts' int32 tiles are added with LDS atomics (exact in
//     any order), then the fp64 epilogue writes bf16 (and optionally int32).
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kMfmaWaves = 4;
constexpr int kMfmaThreads = kMfmaWaves * 64;

__device__ __forceinline__ v4i decode_b(uint32_t w) {
    v4i b;
    b.x = static_cast<int>(__builtin_amdgcn_perm(0u, kCodeToInt8, w & 0x03030303u));
    b.y = static_cast<int>(__builtin_amdgcn_perm(0u, kCodeToInt8, (w >> 2) & 0x03030303u));
    b.z = static_cast<int>(__builtin_amdgcn_perm(0u, kCodeToInt8, (w >> 4) & 0x03030303u));
    b.w = static_cast<int>(__builtin_amdgcn_perm(0u, kCodeToInt8, (w >> 6) & 0x03030303u));
    return b;
}

// MT = number of 16-row m tiles this workgroup covers (1..4).
template <int MT>
__global__ __launch_bounds__(kMfmaThreads) void gemm_mfma_kernel(
    const int8_t* __restrict__ xq, const uint8_t* __restrict__ packed, const float* __restrict__ s,
    const uint16_t* __restrict__ ws, int ws_num, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out, int M, int N, int K) {
    __shared__ int red[MT * 16][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = blockIdx.x;                      // 64 output rows = 4 bands
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const int m0 = blockIdx.y * 64;
    const int S256 = (K + kTileK - 1) / kTileK;      // 1 KiB tiles per band
    const int S = (K + 63) / 64;                     // 64-K MFMA steps
    const int s0 = (S * wave) / kMfmaWaves;
    const int s1 = (S * (wave + 1)) / kMfmaWaves;
    const int j = lane & 15;
    const int g = lane >> 4;

    for (int i = threadIdx.x; i < MT * 16 * 64; i += kMfmaThreads) (&red[0][0])[i] = 0;

    v4i c[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) c[mt][t] = v4i{0, 0, 0, 0};

    const uint32_t* words = reinterpret_cast<const uint32_t*>(packed);
    size_t band_base[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        band_base[t] = static_cast<size_t>(min(4 * col + t, nbands - 1)) * S256 * (kTileBytes / 4);
    const int lane_word = 64 * (j >> 2) + 4 * g + (j & 3);
    for (int st = s0; st < s1; ++st) {
        const size_t step_word = static_cast<size_t>(st >> 2) * (kTileBytes / 4) + 16 * (st & 3) + lane_word;
        uint32_t bw[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) bw[t] = __builtin_nontemporal_load(words + band_base[t] + step_word);
        v4i a[MT];
        const int k = st * 64 + 16 * g;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = m0 + 16 * mt + j;
            a[mt] = v4i{0, 0, 0, 0};
            if (m < M && k < K)
                a[mt] = *reinterpret_cast<const v4i*>(xq + static_cast<size_t>(m) * K + k);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const v4i b = decode_b(bw[t]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                c[mt][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[mt], b, c[mt][t], 0, 0, 0);
        }
    }
    __syncthreads();   // red[] zeroed by every thread before any atomics
    // D layout of a 16x16 tile: lane (j, g), register v -> row 4g + v, column j.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            atomicAdd(&red[16 * mt + 4 * g + 0][16 * t + j], c[mt][t].x);
            atomicAdd(&red[16 * mt + 4 * g + 1][16 * t + j], c[mt][t].y);
            atomicAdd(&red[16 * mt + 4 * g + 2][16 * t + j], c[mt][t].z);
            atomicAdd(&red[16 * mt + 4 * g + 3][16 * t + j], c[mt][t].w);
        }
    __syncthreads();
    const int seg = N / ws_num;
    for (int i = threadIdx.x; i < MT * 16 * 64; i += kMfmaThreads) {
        const int ml = i >> 6;
        const int nl = i & 63;
        const int m = m0 + ml;
        const int n = col * 64 + nl;
        if (m < M && n < N) {
            const int32_t total = red[ml][nl];
            const size_t o = static_cast<size_t>(m) * N + n;
            y[o] = epilogue_bf16(total, bf16_to_float(ws[n / seg]), s[m]);
            if (acc_out) acc_out[o] = total;
        }
    }
}

template <int MT>
hipError_t launch_mt(const int8_t* xq, const uint8_t* packed, const float* s, const uint16_t* ws,
                     int ws_num, uint16_t* y, int32_t* acc, int M, int N, int K,
                     hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((N + 63) / 64), static_cast<unsigned>((M + 63) / 64));
    gemm_mfma_kernel<MT><<<grid, kMfmaThreads, 0, stream>>>(xq, packed, s, ws, ws_num, y, acc, M,
                                                             N, K);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma(const int8_t* xq, const uint8_t* packed, const float* s,
                            const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int M,
                            int N, int K, hipStream_t stream) {
    // m tiles needed by the widest workgroup column (all columns but the last
    // are full 64-row chunks).
    const int mt = (M >= 64) ? 4 : (M + 15) / 16;
    switch (mt) {
        case 1: return launch_mt<1>(xq, packed, s, ws, ws_num, y, acc, M, N, K, stream);
        case 2: return launch_mt<2>(xq, packed, s, ws, ws_num, y, acc, M, N, K, stream);
        case 3: return launch_mt<3>(xq, packed, s, ws, ws_num, y, acc, M, N, K, stream);
        default: return launch_mt<4>(xq, packed, s, ws, ws_num, y, acc, M, N, K, stream);
    }
}

}  // namespace bl
