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
//     to 64 rows m (MT tiles of 16), 4 or 8 wavefronts that split the 64-K
//     steps between them, PS consecutive steps per wavefront and chunk;
//   * per K step a wavefront reads, for each of the four bands t, one word per
//     lane: lane (j = lane%16, g = lane/16) takes the word of row j for the
//     16-wide K chunk g of this step -- byte 256*(j/4) + 64*(step%4) + 16*g +
//     4*(j%4) of the band's 1 KiB tile -- which is exactly the B operand of
//     v_mfma_i32_16x16x64_i8 for that band (16 K of one column);
//     v_perm_b32 turns the 2-bit codes into signed int8 weights (code 0, the
//     padding, becomes 0) after each shift-and-mask of [W2A8] §5.2;
//   * all PS x 4 weight words of a chunk are loaded up front (PS is a
//     template argument, so the loads are unconditional: steps past the end
//     re-read the last step and add zero), and so are the
//     chunk's PS x MT A operands (16 rows m x 64 K, 16 bytes per lane from
//     the int8 activations, loaded four lanes to a row and moved into the
//     operand layout through LDS): both come from far enough away that only
//     loads issued together hide their latency (PS * MT <= 20 bounds the
//     registers);
//   * the wavefronts' int32 tiles are added with LDS atomics (exact in any
//     order), then the epilogue writes bf16 four outputs at a time through
//     epilogue4 (fp64 product, fp32, packed bf16; the division only where
//     an fp32 value is a bf16 midpoint), and optionally int32.
#include <algorithm>
#include <array>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kMfmaMaxWaves = 8;
constexpr int kMfmaMaxSteps = 16;   // 64-K steps per wavefront and chunk
constexpr int kMfmaMaxAFrags = 20;  // PS * MT: A operands held per wavefront
// Row pitch of the LDS reduction tile: 64 columns + 4, so that the four lane
// groups adding the same column of a 16x16 tile land in different banks.
constexpr int kRedPitch = 68;

__device__ __forceinline__ v4i decode_b(uint32_t w) {
    v4i b;
    b.x = static_cast<int>(__builtin_amdgcn_perm(0u, kCodeToInt8, w & 0x03030303u));
    b.y = static_cast<int>(__builtin_amdgcn_perm(0u, kCodeToInt8, (w >> 2) & 0x03030303u));
    b.z = static_cast<int>(__builtin_amdgcn_perm(0u, kCodeToInt8, (w >> 4) & 0x03030303u));
    b.w = static_cast<int>(__builtin_amdgcn_perm(0u, kCodeToInt8, (w >> 6) & 0x03030303u));
    return b;
}

// Two words at once: one 64-bit shift per field serves both (what it moves
// from one word into the other falls outside the mask), 19 VALU for two
// words instead of 22.  Used with one m tile only: same box, M = 16 on
// 2560 x 6912 and 13824 x 5120 9.16 / 7.70 -> 9.09 / 7.61 us, but M = 64
// (four m tiles) 17.93 / 15.77 -> 18.15 / 15.83 us.
__device__ __forceinline__ void decode_b2(uint32_t w0, uint32_t w1, v4i& a, v4i& b) {
    const uint64_t p = (static_cast<uint64_t>(w1) << 32) | w0;
    constexpr uint64_t m = 0x0303030303030303ull;
    const uint64_t f0 = p & m, f1 = (p >> 2) & m, f2 = (p >> 4) & m, f3 = (p >> 6) & m;
    auto cv = [](uint64_t f) {
        return static_cast<int>(__builtin_amdgcn_perm(0u, kCodeToInt8, static_cast<uint32_t>(f)));
    };
    a = v4i{cv(f0), cv(f1), cv(f2), cv(f3)};
    b = v4i{cv(f0 >> 32), cv(f1 >> 32), cv(f2 >> 32), cv(f3 >> 32)};
}

// A operands of one 64-K step for MT m tiles, as loaded: 16 bytes of each m
// tile's row (this lane's row) at K offset 64*st + 16*chunk, from clamped
// addresses so that the loads are unconditional.
// Nothing needs zeroing: a row m >= M (read as row M - 1) only reaches its
// own outputs, which are not written; K positions >= K in the last step
// meet padding codes, which decode to 0; whole steps past the end are
// zeroed where they are used.
template <int MT>
__device__ __forceinline__ void load_a(const int8_t* const (&row)[MT], int st, int chunk, int K,
                                       v4i (&a)[MT]) {
    const int kc = min(st * 64 + 16 * chunk, K - 16);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a[mt] = *reinterpret_cast<const v4i*>(row[mt] + kc);
}

// MT = number of 16-row m tiles this workgroup covers (1..4); PS = 64-K steps
// per wavefront and chunk.  blockDim.x = 64 * (4 or 8).
template <int MT, int PS>
__global__ __launch_bounds__(kMfmaMaxWaves * 64) void gemm_mfma_kernel(
    const int8_t* __restrict__ xq, const uint32_t* __restrict__ words,
    const float* __restrict__ s, const uint16_t* __restrict__ ws, uint32_t seg_mul,
    int seg_shift, uint16_t* __restrict__ y, int32_t* __restrict__ acc_out, int M, int N, int K) {
    __shared__ __align__(16) int red[MT * 16][kRedPitch];
    __shared__ double inv_s_sh[MT * 16];
    __shared__ float s_sh[MT * 16];
    __shared__ __align__(16) v4i stage_sh[kMfmaMaxWaves][MT * 64];
    const int nthreads = blockDim.x;
    const int nwaves = nthreads >> 6;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = blockIdx.x;                      // 64 output rows = 4 bands
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const int m0 = blockIdx.y * 64;
    const int S256 = (K + kTileK - 1) / kTileK;      // 1 KiB tiles per band
    const int S64 = (K + 63) / 64;                   // 64-K MFMA steps
    const int j = lane & 15;
    const int g = lane >> 4;

    for (int i = tid; i < MT * 16 * kRedPitch / 4; i += nthreads)
        reinterpret_cast<int4*>(&red[0][0])[i] = int4{0, 0, 0, 0};
    // the activation scale of m row tid (if any) is loaded now and inverted
    // after the main loop, so that neither waits in front of the weight loads
    const float s_row = s[min(m0 + min(tid, MT * 16 - 1), M - 1)];
    // The epilogue's weight scales: this thread writes columns n0 .. n0 + 3
    // of its rows (fixed per thread, the row stride being a multiple of 16),
    // loaded now so that no load is left to wait on after the main loop.
    const int c4 = (tid & 15) * 4;
    const int n0 = col * 64 + c4;
    uint16_t wsb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        wsb[e] = ws[(static_cast<uint64_t>(min(n0 + e, N - 1)) * seg_mul) >> seg_shift];

    // A operands are loaded four lanes to a row -- lane 4q + i takes row q
    // of each m tile, 16-byte chunk (i + q/2) % 4 of the step, so that a quad
    // reads 64 contiguous bytes of one line (loaded in the operand layout,
    // four lanes of a quad would touch four rows, which costs the memory
    // pipeline several times as much) -- and moved into the operand layout
    // (lane (j, g): row j, chunk g) through the wavefront's LDS slots; the
    // skew makes those LDS reads free of bank conflicts.
    const int a_row = lane >> 2;
    const int a_chunk = ((lane & 3) + (lane >> 3)) & 3;
    const int rd_slot = 4 * j + ((g - (j >> 1)) & 3);   // where lane (j, g)'s operand lands
    v4i* const stage = stage_sh[wave];
    const int8_t* row[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        row[mt] = xq + static_cast<size_t>(min(m0 + 16 * mt + a_row, M - 1)) * K;
    size_t band_base[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        band_base[t] = static_cast<size_t>(min(4 * col + t, nbands - 1)) * S256 * (kTileBytes / 4);
    const int lane_word = 64 * (j >> 2) + 4 * g + (j & 3);

    v4i c[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t) c[mt][t] = v4i{0, 0, 0, 0};

    for (int base = wave * PS; base < S64; base += nwaves * PS) {
        // Waits count loads in issue order.  With the A operands first, step
        // p waits for its own weight words only, so the MFMAs run while the
        // weights stream in; but for MT >= 3 the A operands (each workgroup
        // reads all of A) outweigh the weights several times over, and
        // issued first they hold the weight stream back, so there the
        // weights go first.
        constexpr bool kAFirst = MT <= 2;
        v4i a[PS][MT];
        if constexpr (kAFirst) {
#pragma unroll
            for (int p = 0; p < PS; ++p) load_a<MT>(row, base + p, a_chunk, K, a[p]);
        }
        uint32_t bw[PS][4];
#pragma unroll
        for (int p = 0; p < PS; ++p) {
            const int st = min(base + p, S64 - 1);
            const size_t step_word =
                static_cast<size_t>(st >> 2) * (kTileBytes / 4) + 16 * (st & 3) + lane_word;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                bw[p][t] = __builtin_nontemporal_load(words + band_base[t] + step_word);
        }
        if constexpr (!kAFirst) {
#pragma unroll
            for (int p = 0; p < PS; ++p) load_a<MT>(row, base + p, a_chunk, K, a[p]);
        }
        // Nothing may be scheduled above this point: the first wait for an
        // operand would otherwise hold back the remaining loads.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < PS; ++p) {
            // a step past the end (a re-read of the last one) must add nothing
            const bool live = base + p < S64;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) stage[mt * 64 + lane] = a[p][mt];
            // LDS operations of one wavefront complete in order; the fences
            // keep the compiler from moving the reads above the writes (or
            // the next step's writes above these reads).
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            v4i ap[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) ap[mt] = live ? stage[mt * 64 + rd_slot] : v4i{0, 0, 0, 0};
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if constexpr (MT == 1) {
#pragma unroll
                for (int t = 0; t < 4; t += 2) {
                    v4i b0, b1;
                    decode_b2(bw[p][t], bw[p][t + 1], b0, b1);
                    c[0][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ap[0], b0, c[0][t], 0, 0, 0);
                    c[0][t + 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ap[0], b1, c[0][t + 1], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const v4i b = decode_b(bw[p][t]);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        c[mt][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ap[mt], b, c[mt][t], 0, 0, 0);
                }
            }
        }
    }
    if (tid < MT * 16) {
        inv_s_sh[tid] = 1.0 / static_cast<double>(s_row);
        s_sh[tid] = s_row;
    }
    __syncthreads();   // red[] zeroed and inv_s_sh[] written before use
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
    // Each thread writes four consecutive outputs of one row m, columns
    // n0 .. n0 + 3, with 8-byte (bf16) and 16-byte (int32) stores where the
    // row is aligned for them.
    float wsf[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) wsf[e] = bf16_to_float(wsb[e]);
    // (MT * 256 and the block size are multiples of 64, so every lane of a
    // wavefront makes the same trips: epilogue4's branch stays uniform)
    for (int i = tid; i < MT * 16 * 16; i += nthreads) {
        const int ml = i >> 4;
        const int m = m0 + ml;
        const int4 t = *reinterpret_cast<const int4*>(&red[ml][c4]);
        const double inv = inv_s_sh[ml];
        const float sm = s_sh[ml];
        const int tv[4] = {t.x, t.y, t.z, t.w};
        double cs[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[e] = static_cast<double>(wsf[e]) * inv;
        const uint2 ob = epilogue4(tv, wsf, cs, sm);
        const uint32_t o0 = ob.x & 0xFFFFu, o1 = ob.x >> 16, o2 = ob.y & 0xFFFFu, o3 = ob.y >> 16;
        if (m < M && n0 < N) {
            const size_t o = static_cast<size_t>(m) * N + n0;
            uint16_t* yo = y + o;
            const bool full = n0 + 4 <= N;
            if (full && (reinterpret_cast<uintptr_t>(yo) & 7) == 0) {
                *reinterpret_cast<uint2*>(yo) = ob;
            } else {
                yo[0] = static_cast<uint16_t>(o0);
                if (n0 + 1 < N) yo[1] = static_cast<uint16_t>(o1);
                if (n0 + 2 < N) yo[2] = static_cast<uint16_t>(o2);
                if (n0 + 3 < N) yo[3] = static_cast<uint16_t>(o3);
            }
            if (acc_out) {
                int32_t* ao = acc_out + o;
                if (full && (reinterpret_cast<uintptr_t>(ao) & 15) == 0) {
                    *reinterpret_cast<int4*>(ao) = t;
                } else {
                    ao[0] = t.x;
                    if (n0 + 1 < N) ao[1] = t.y;
                    if (n0 + 2 < N) ao[2] = t.z;
                    if (n0 + 3 < N) ao[3] = t.w;
                }
            }
        }
    }
}

using MfmaFn = void (*)(const int8_t*, const uint32_t*, const float*, const uint16_t*, uint32_t,
                        int, uint16_t*, int32_t*, int, int, int);

// Entries past the A-operand budget (PS * MT > kMfmaMaxAFrags) are never
// selected; they repeat the largest allowed PS so that no such kernel exists.
template <int MT, int... Ps>
constexpr std::array<MfmaFn, sizeof...(Ps)> mfma_table(std::integer_sequence<int, Ps...>) {
    return {{&gemm_mfma_kernel<MT, std::min(Ps + 1, kMfmaMaxAFrags / MT)>...}};
}

const std::array<std::array<MfmaFn, kMfmaMaxSteps>, 4> kMfmaKernels = {{
    mfma_table<1>(std::make_integer_sequence<int, kMfmaMaxSteps>{}),
    mfma_table<2>(std::make_integer_sequence<int, kMfmaMaxSteps>{}),
    mfma_table<3>(std::make_integer_sequence<int, kMfmaMaxSteps>{}),
    mfma_table<4>(std::make_integer_sequence<int, kMfmaMaxSteps>{}),
}};

constexpr int kMfmaMinGroups = 128;   // fewer workgroups than this: 8 wavefronts each

}  // namespace

hipError_t launch_gemm_mfma(const int8_t* xq, const uint8_t* packed, const float* s,
                            const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int M,
                            int N, int K, hipStream_t stream) {
    // m tiles needed by the widest workgroup (all but the last are full 64-row chunks)
    const int mt = (M >= 64) ? 4 : (M + 15) / 16;
    const dim3 grid(static_cast<unsigned>((N + 63) / 64), static_cast<unsigned>((M + 63) / 64));
    const int S64 = (K + 63) / 64;
    const int max_ps = std::min(kMfmaMaxSteps, kMfmaMaxAFrags / mt);
    // 8 wavefronts when the grid is small or 4 would need a second chunk
    const int waves =
        (grid.x * grid.y < kMfmaMinGroups || (S64 + 3) / 4 > max_ps) ? 8 : 4;
    const int per_wave = (S64 + waves - 1) / waves;
    const int chunks = (per_wave + max_ps - 1) / max_ps;
    const int ps = (S64 + waves * chunks - 1) / (waves * chunks);
    uint32_t seg_mul;
    int seg_shift;
    seg_divisor(N / ws_num, seg_mul, seg_shift);
    const MfmaFn fn = kMfmaKernels[mt - 1][ps - 1];
    fn<<<grid, waves * 64, 0, stream>>>(xq, reinterpret_cast<const uint32_t*>(packed), s, ws,
                                        seg_mul, seg_shift, y, acc, M, N, K);
    return hipGetLastError();
}

}  // namespace bl
