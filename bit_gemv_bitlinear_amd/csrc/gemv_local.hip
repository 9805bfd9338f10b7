// gemv_local.hip -- the M = 1 layer with bf16 activations, quantised wave by
// wave, on gfx950.  Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit
// 大模型 CUDA GEMV 内核" (blog.gitcode.com), cited as [W2A8]: §5.3 (int8 dot
// products into an int32 accumulator, out = acc * scales), §六 item 3
// (per-token activation quantisation, fused here).
//
// A translation unit of its own because gemv.hip is compiled with its
// leading kernel arguments preloaded into SGPRs, and this kernel measured
// slower that way (2.72 -> 2.80 us at 3840 x 2560, same box).
#include <algorithm>
#include <array>
#include <utility>

#include "gemv_core.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

// The bf16-input layer with the activations kept wave-local (no staged row).
// Lane (rg = l/16, kc = l%16) of a wavefront covers, at step u, the 16-wide K
// chunk kc of tile s0 + u for the four rows of its slot.  It loads the 4 bf16
// values 4*rg .. +3 of that chunk, so the wavefront's 64 lanes cover its K
// range once; the absmax is exchanged across the workgroup (one barrier),
// each lane quantises its 4 values into one int8x4 word and writes it to a
// wavefront-private LDS slot, and reads back the chunk's 16 bytes (the words
// of lanes rg = 0..3) -- within a wavefront no barrier is needed.  The code
// offset -2 * sum(x) is taken per lane over its chunks and folded into its
// four rows before the row reduction.  Workgroup 0's first band writes
// q_out / s_out when given.
//
// Against the staged kernel this saves a barrier and the row copy, but every
// band of a workgroup loads its own copy of the row.  Measured same-box over
// bf16 shapes, it is faster (by about 0.3 us) only with one band per
// workgroup, at most 4 wavefronts and at most 256 workgroups -- 1024, 2560
// and 3840 rows at K = 2560 -- and slower elsewhere (5120 x 2560, 6912 x 2560,
// K >= 5120, 13824 x 2560); the GEMV launcher (gemv.hip) uses it only there.
template <int P>
__global__ __launch_bounds__(kMaxWaves * 64) void gemv_local_kernel(
    const void* __restrict__ xin, const v4u* __restrict__ packed, const float* __restrict__ s_in,
    const uint16_t* __restrict__ ws, uint32_t seg_mul, int seg_shift, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc, int8_t* __restrict__ q_out, float* __restrict__ s_out, int N,
    int K, int B, int lw) {
    extern __shared__ uint32_t actw[];   // W * P * 64 quantised words
    __shared__ int part_sh[kMaxWaves][64];
    __shared__ float amax_sh[kMaxWaves];
    const int Wb = 1 << lw;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const int band = min(static_cast<int>(blockIdx.x) * B + (wave >> lw), nbands - 1);
    const int S = (K + kTileK - 1) / kTileK;
    const int s0 = (wave & (Wb - 1)) * P;
    const int kc = lane & 15;
    const int rg = lane >> 4;

    const int n_out = static_cast<int>(blockIdx.x) * B * kTileRows + tid;   // tid < 16*B writes
    const uint32_t n_ws = static_cast<uint32_t>(min(n_out, N - 1));
    const uint16_t wsb = ws[(static_cast<uint64_t>(n_ws) * seg_mul) >> seg_shift];
    // this lane's 4 activations per step, from clamped addresses (unconditional loads)
    uint2 xb[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int kk = min((s0 + u) * kTileK + 16 * kc + 4 * rg, K - 4);
        xb[u] = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(xin) + kk);
    }
    const v4u* tiles = packed + static_cast<size_t>(band) * S * 64 + lane;
    v4u w[P];
    load_steps<P>(tiles, s0, S - 1, w);
    __builtin_amdgcn_sched_barrier(0);

    int4 xq[P];
    float sm;
    {
        float amax = 0.0f;
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const bool live = (s0 + u) * kTileK + 16 * kc < K;
            const uint32_t lo = live ? xb[u].x : 0u;
            const uint32_t hi = live ? xb[u].y : 0u;
            xb[u] = uint2{lo, hi};
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(__uint_as_float(lo << 16)),
                                           fabsf(__uint_as_float(lo & 0xFFFF0000u))),
                                     fmaxf(fabsf(__uint_as_float(hi << 16)),
                                           fabsf(__uint_as_float(hi & 0xFFFF0000u)))));
        }
        amax = wave_max(amax);
        if (lane == 0) amax_sh[wave] = amax;
        __syncthreads();
        // the Wb wavefronts of this band cover the whole row
        const int first = (wave >> lw) << lw;
        amax = amax_sh[first];
        for (int j = 1; j < Wb; ++j) amax = fmaxf(amax, amax_sh[first + j]);
        sm = 127.0f / fmaxf(amax, 1e-5f);
        uint32_t* mine = actw + static_cast<size_t>(wave) * P * 64;
        const bool write_q = q_out != nullptr && blockIdx.x == 0 && (wave >> lw) == 0;
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const uint32_t word = quant4(__uint_as_float(xb[u].x << 16),
                                         __uint_as_float(xb[u].x & 0xFFFF0000u),
                                         __uint_as_float(xb[u].y << 16),
                                         __uint_as_float(xb[u].y & 0xFFFF0000u), sm);
            mine[u * 64 + 4 * kc + rg] = word;   // word rg of chunk kc
            const int k = (s0 + u) * kTileK + 16 * kc + 4 * rg;
            if (write_q && k < K) *reinterpret_cast<uint32_t*>(q_out + k) = word;
        }
        // Within one wavefront LDS operations complete in order; the fence
        // keeps the compiler from moving the reads above the writes.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int u = 0; u < P; ++u) xq[u] = *reinterpret_cast<const int4*>(mine + u * 64 + 4 * kc);
        if (s_out != nullptr && blockIdx.x == 0 && tid == 0) s_out[0] = sm;
    }
    double cs = 0.0;
    if (wave == 0) {
        cs = static_cast<double>(bf16_to_float(wsb)) * (1.0 / static_cast<double>(sm));
        asm volatile("" : "+v"(cs));
    }

    RowAcc r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a1[i] = r.a4[i] = r.a16[i] = 0;
    int xs = 0;
#pragma unroll
    for (int u = 0; u < P; ++u) {
        dot_slot(w[u], xq[u], r);
        xs = sum_i8x4(xq[u].x, sum_i8x4(xq[u].y, sum_i8x4(xq[u].z, sum_i8x4(xq[u].w, xs))));
    }
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r.a1[i] + (r.a4[i] >> 2) + (r.a16[i] >> 4) - 2 * xs;
    part_sh[wave][lane] = row_group_reduce(v, lane);
    __syncthreads();

    if (wave == 0) {
        const int bw = lane >> 4;
        const int rw = lane & 15;
        const int slot = 16 * (rw >> 2) + (rw & 3);
        const int first = min(bw, B - 1) << lw;
        int total = 0;
        for (int j = 0; j < Wb; ++j) total += part_sh[first + j][slot];
        if (bw < B && n_out < N) {
            y[n_out] = epilogue_bf16_scaled(total, cs, bf16_to_float(wsb), sm);
            if (acc) acc[n_out] = total;
        }
    }
}

using LocalFn = void (*)(const void*, const v4u*, const float*, const uint16_t*, uint32_t, int,
                         uint16_t*, int32_t*, int8_t*, float*, int, int, int, int);

template <int... Ps>
constexpr std::array<LocalFn, sizeof...(Ps)> local_table(std::integer_sequence<int, Ps...>) {
    return {{&gemv_local_kernel<Ps + 1>...}};
}

// P = 1 .. kLocalMaxSteps (beyond that its registers, 8 per step, would not
// fit a 16-wavefront workgroup).
const std::array<LocalFn, kLocalMaxSteps> kLocalKernels =
    local_table(std::make_integer_sequence<int, kLocalMaxSteps>{});

}  // namespace

hipError_t launch_gemv_local(const uint16_t* x, const uint8_t* packed, const uint16_t* ws,
                             uint32_t seg_mul, int seg_shift, uint16_t* y, int32_t* acc,
                             int8_t* q_out, float* s_out, int N, int K, unsigned groups,
                             int waves, int steps, int lw, hipStream_t stream) {
    const size_t lds = static_cast<size_t>(waves) * steps * 64 * 4;
    kLocalKernels[steps - 1]<<<groups, waves * 64, lds, stream>>>(
        x, reinterpret_cast<const v4u*>(packed), nullptr, ws, seg_mul, seg_shift, y, acc, q_out,
        s_out, N, K, 1, lw);
    return hipGetLastError();
}

}  // namespace bl
