// pack.hip -- packing of ternary weights into the 16x256-tile layout.
//
// Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
// (blog.gitcode.com), §5.2: each weight w in {-1, 0, 1} becomes the code
// w + 2, and the 16 codes of a 32-bit word are interleaved so that element e
// sits at bit 8*(e%4) + 2*(e/4).  The tiling around the words (16 rows x 256 K
// per 1 KiB tile, one 16-byte slot per wavefront lane) is this library's
// own (a 16-byte slot holds four rows of one 16-wide K chunk, so a lane's
// 16-byte load needs a single 16-byte run of activations); it is spelled out
// bit by bit in include/bitlinear.h.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

size_t packed_bytes(int N, int K) {
    if (N <= 0 || K <= 0) return 0;
    const size_t bands = (static_cast<size_t>(N) + kTileRows - 1) / kTileRows;
    const size_t steps = (static_cast<size_t>(K) + kTileK - 1) / kTileK;
    return bands * steps * kTileBytes;
}

__host__ __device__ inline uint32_t ternary_code(int w) {
    return (w == -1) ? 1u : (w == 0) ? 2u : (w == 1) ? 3u : 0u;
}

__host__ __device__ inline int bit_of(int e) { return 8 * (e & 3) + 2 * (e >> 2); }

// One thread per packed 32-bit word.  Word u of tile t is word i = u % 4 of
// slot q = u / 4; it holds k = 256*(t % S) + 16*(q % 16) + e for e = 0..15
// of row n = 16*(t / S) + 4*(q / 16) + i.  VEC: the 16 source bytes are read
// as one 16-byte load (w 16-byte aligned, K % 16 == 0).
template <bool VEC>
__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ w,
                                                   uint32_t* __restrict__ packed, int N, int K,
                                                   int S, size_t n_words,
                                                   int32_t* __restrict__ n_invalid) {
    const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n_words) return;
    const size_t t = blockIdx.x;   // 256 threads per workgroup: the tile is i >> 8
    const int u = static_cast<int>(threadIdx.x);
    const int q = u >> 2;
    const int n = static_cast<int>(t / S) * kTileRows + 4 * (q >> 4) + (u & 3);
    const int k0 = static_cast<int>(t % S) * kTileK + 16 * (q & 15);
    uint32_t word = 0;
    int bad = 0;
    if (n < N && k0 < K) {
        const int8_t* row = w + static_cast<size_t>(n) * K;
        if (VEC) {
            const uint4 v = *reinterpret_cast<const uint4*>(row + k0);
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
            // Four weights at a time: element 4j + b is byte b of d[j] and
            // goes to bits 8b + 2j; for w in {-1, 0, 1} its code w + 2 is
            // (w & 3) ^ 2.  A byte outside {-1, 0, 1} is counted by a byte-
            // parallel test: its low seven bits, flipped when negative, must be
            // 0 (negative: -1) or at most 1 (positive); a nonzero remainder
            // sets bit 7 when 0x7F is added (no carries: every byte <= 0x7F).
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                word |= ((d[j] & 0x03030303u) ^ 0x02020202u) << (2 * j);
                const uint32_t neg = (d[j] & 0x80808080u) >> 7;
                const uint32_t rest = ((d[j] & 0x7F7F7F7Fu) ^ (neg * 0x7Fu)) & (0x7E7E7E7Eu | neg);
                bad += __popc((rest + 0x7F7F7F7Fu) & 0x80808080u);
            }
            if (bad) {   // rare: the per-weight codes, 0 for such a weight, as the host twin makes them
                word = 0;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int wv = static_cast<int8_t>((d[e >> 2] >> (8 * (e & 3))) & 0xFF);
                    word |= ternary_code(wv) << bit_of(e);
                }
            }
        } else {
            for (int e = 0; e < 16; ++e) {
                if (k0 + e >= K) break;
                const uint32_t c = ternary_code(row[k0 + e]);
                bad += (c == 0);
                word |= c << bit_of(e);
            }
        }
    }
    packed[i] = word;
    if (n_invalid && bad) atomicAdd(n_invalid, bad);
}

hipError_t launch_pack(const int8_t* w, uint8_t* packed, int N, int K, int32_t* n_invalid,
                       hipStream_t stream) {
    const int S = (K + kTileK - 1) / kTileK;
    const size_t n_words = packed_bytes(N, K) / 4;
    const unsigned blocks = static_cast<unsigned>((n_words + 255) / 256);
    const bool vec = (K % 16 == 0) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0);
    if (vec)
        pack_kernel<true><<<blocks, 256, 0, stream>>>(w, reinterpret_cast<uint32_t*>(packed), N,
                                                      K, S, n_words, n_invalid);
    else
        pack_kernel<false><<<blocks, 256, 0, stream>>>(w, reinterpret_cast<uint32_t*>(packed), N,
                                                       K, S, n_words, n_invalid);
    return hipGetLastError();
}

// Host twin: the same word-by-word construction on the CPU.
int64_t pack_host(const int8_t* w, uint8_t* packed, int N, int K) {
    const int S = (K + kTileK - 1) / kTileK;
    const size_t n_words = packed_bytes(N, K) / 4;
    uint32_t* out = reinterpret_cast<uint32_t*>(packed);
    int64_t bad = 0;
    for (size_t i = 0; i < n_words; ++i) {
        const size_t t = i >> 8;
        const int u = static_cast<int>(i & 255);
        const int q = u >> 2;
        const int n = static_cast<int>(t / S) * kTileRows + 4 * (q >> 4) + (u & 3);
        const int k0 = static_cast<int>(t % S) * kTileK + 16 * (q & 15);
        uint32_t word = 0;
        if (n < N) {
            for (int e = 0; e < 16 && k0 + e < K; ++e) {
                const uint32_t c = ternary_code(w[static_cast<size_t>(n) * K + k0 + e]);
                bad += (c == 0);
                word |= c << bit_of(e);
            }
        }
        out[i] = word;   // little-endian host: byte j of the word is bits 8j..8j+7
    }
    return bad;
}

}  // namespace bl
