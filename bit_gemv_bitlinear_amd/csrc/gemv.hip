// gemv.hip -- the M = 1 decode GEMV of the W2A8 ternary linear layer on gfx950.
//
// Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
// (blog.gitcode.com), cited as [W2A8]: §5.2 (codes w + 2, interleaved 32-bit
// words decoded by shift and mask), §5.3 (int8 dot products into an int32
// accumulator, then out = acc * scales with ws[n / (N / ws_num)]), §六 item 3
// (per-token activation quantisation, fused here for bf16 input).
//
// Mapping (this library's design; the page's sm_80 kernel is prior art):
//   * one workgroup per band of 64 output rows; its W wavefronts split the
//     band's S K-steps (64 K = one 1 KiB tile each), P consecutive steps per
//     wavefront, W and P picked per shape so that W*P covers S with the least
//     waste and the steps spread evenly over the 4 SIMDs;
//   * a wavefront's load of a tile is one coalesced 16-byte-per-lane load of
//     1 KiB; lane l's slot holds rows 4*(l/4) .. +3 of K chunk l%4, so each
//     lane needs one 16-byte run of activations per step;
//   * every weight load of the wavefront is issued up front (P is a template
//     argument, so the loads are unconditional and the compiler counts them
//     exactly), before the activations are staged;
//   * the activation row is staged once per workgroup in LDS (zero-padded to
//     W*P steps; steps past the band's end re-read its last tile and meet zero
//     activations), read back as one 16-byte LDS load per step;
//   * decoding keeps the unsigned codes c = w + 2 and never shifts them into
//     place: field i of a word is masked in place (factor 4^i, i < 3) and
//     dotted with activation word i into one of three accumulators; field 3
//     is shifted down once.  acc = a1 + a4/4 + a16/16 - 2 * sum(x), the last
//     term removing the +2 offset (padding code 0 contributes nothing);
//   * the 4 lanes sharing a K step exchange partial sums with DPP so that
//     lane r ends with row r; the W wavefronts' sums are added through LDS;
//     the epilogue multiplies by a precomputed fp64 1/s and rounds once to
//     bf16, dividing only when the product lies next to a rounding boundary
//     (so the result is that of the exact fp64 division).
#include <array>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kMaxWaves = 16;
constexpr int kCached = 2;   // 16-byte activation chunks per thread kept in registers

struct RowAcc {
    int a1[4], a4[4], a16[4];
};

// Dot of one packed word (16 K of one row) with its four activation words.
__device__ __forceinline__ void dot_word(uint32_t w, const int4& x, int& a1, int& a4, int& a16) {
    a1 = dot4(static_cast<int>(w & 0x03030303u), x.x, a1);
    a4 = dot4(static_cast<int>(w & 0x0C0C0C0Cu), x.y, a4);
    a16 = dot4(static_cast<int>(w & 0x30303030u), x.z, a16);
    a1 = dot4(static_cast<int>((w >> 6) & 0x03030303u), x.w, a1);
}

// One K step of a lane: the four words of its slot are four rows of the same
// 16-wide K chunk, all dotted with the same 16 activation bytes.
__device__ __forceinline__ void dot_slot(const v4u& wv, const int4& x, RowAcc& r) {
    dot_word(wv.x, x, r.a1[0], r.a4[0], r.a16[0]);
    dot_word(wv.y, x, r.a1[1], r.a4[1], r.a16[1]);
    dot_word(wv.z, x, r.a1[2], r.a4[2], r.a16[2]);
    dot_word(wv.w, x, r.a1[3], r.a4[3], r.a16[3]);
}

template <int P>
__device__ __forceinline__ void load_steps(const v4u* __restrict__ tiles, int s0, int s_last,
                                           v4u (&w)[P]) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int st = min(s0 + u, s_last);
        w[u] = __builtin_nontemporal_load(tiles + static_cast<size_t>(st) * 64);
    }
}

// DPP lane exchange inside groups of 4 lanes.
template <int CTRL>
__device__ __forceinline__ int quad_swap(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm(1, 0, 3, 2)
constexpr int kQuadXor2 = 0x4E;   // quad_perm(2, 3, 0, 1)

// Lanes 4g..4g+3 each hold partial sums of rows 4g..4g+3 (over their own K
// chunks); afterwards lane 4g + c holds the full sum of row 4g + c.
__device__ __forceinline__ int quad_reduce_scatter(const int (&v)[4], int lane) {
    const bool b = (lane >> 1) & 1;
    const int send0 = b ? v[0] : v[2];
    const int send1 = b ? v[1] : v[3];
    int keep0 = b ? v[2] : v[0];
    int keep1 = b ? v[3] : v[1];
    keep0 += quad_swap<kQuadXor2>(send0);
    keep1 += quad_swap<kQuadXor2>(send1);
    const bool a = lane & 1;
    const int send = a ? keep0 : keep1;
    int keep = a ? keep1 : keep0;
    keep += quad_swap<kQuadXor1>(send);
    return keep;
}

__device__ __forceinline__ float absmax8_bf16(const uint4& v, float m) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(d[j] << 16)),
                           fabsf(__uint_as_float(d[j] & 0xFFFF0000u))));
    return m;
}

__device__ __forceinline__ uint2 quant8_bf16(const uint4& v, float sm) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint2 o;
    o.x = pack4_i8(quant_one(__uint_as_float(d[0] << 16), sm),
                   quant_one(__uint_as_float(d[0] & 0xFFFF0000u), sm),
                   quant_one(__uint_as_float(d[1] << 16), sm),
                   quant_one(__uint_as_float(d[1] & 0xFFFF0000u), sm));
    o.y = pack4_i8(quant_one(__uint_as_float(d[2] << 16), sm),
                   quant_one(__uint_as_float(d[2] & 0xFFFF0000u), sm),
                   quant_one(__uint_as_float(d[3] << 16), sm),
                   quant_one(__uint_as_float(d[3] & 0xFFFF0000u), sm));
    return o;
}

__device__ __forceinline__ int sum_i8x4(uint32_t d, int acc) {
    return dot4(static_cast<int>(d), 0x01010101, acc);
}

// seg = N / ws_num: rows per weight scale.
// FUSED = false: xin is int8 activations with scale s_in[0].
// FUSED = true:  xin is bf16; the workgroup quantises it (per-token absmax,
//                [W2A8] §六 item 3); workgroup 0 writes q_out / s_out if given.
template <int P, bool FUSED>
__global__ __launch_bounds__(kMaxWaves * 64) void gemv_kernel(
    const void* __restrict__ xin, const v4u* __restrict__ packed, const float* __restrict__ s_in,
    const uint16_t* __restrict__ ws, int seg, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc, int8_t* __restrict__ q_out, float* __restrict__ s_out, int N,
    int K) {
    extern __shared__ int4 act[];   // W*P*4 16-byte chunks: the int8 row, zero-padded
    __shared__ int part_sh[kMaxWaves][64];
    __shared__ int xsum_sh[kMaxWaves];
    __shared__ float amax_sh[kMaxWaves];
    const int nthreads = blockDim.x;
    const int W = nthreads >> 6;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int band = blockIdx.x;
    const int S = (K + kTileK - 1) / kTileK;
    const int s0 = wave * P;
    const int n16 = K >> 4;        // 16-byte chunks of int8 activations
    const int padded16 = W * P * 4;

    // 1. The activation row and this lane's weight scale first (so that
    //    waiting for them does not wait for the weights), then every weight
    //    load of this wavefront.
    const int n = band * 64 + lane;
    const uint16_t wsb = ws[min(n, N - 1) / seg];   // unconditional: no branch, no early wait
    uint4 xv[kCached];
    const int n_in = FUSED ? (K >> 3) : n16;   // 16-byte input chunks
    const uint4* x16 = reinterpret_cast<const uint4*>(xin);
#pragma unroll
    for (int c = 0; c < kCached; ++c) {
        const int idx = tid + c * nthreads;
        xv[c] = make_uint4(0, 0, 0, 0);
        if (idx < n_in) xv[c] = x16[idx];
    }
    const v4u* tiles = packed + static_cast<size_t>(band) * S * 64 + lane;
    v4u w[P];
    load_steps<P>(tiles, s0, S - 1, w);

    // 2. Stage the int8 row in LDS and sum it (for the +2 code offset).
    int xs = 0;
    float sm = 0.0f;
    if (!FUSED) {
        sm = s_in[0];
#pragma unroll
        for (int c = 0; c < kCached; ++c) {
            const int idx = tid + c * nthreads;
            if (idx < n_in) {
                act[idx] = make_int4(xv[c].x, xv[c].y, xv[c].z, xv[c].w);
                xs = sum_i8x4(xv[c].x, sum_i8x4(xv[c].y, sum_i8x4(xv[c].z, sum_i8x4(xv[c].w, xs))));
            }
        }
        for (int idx = tid + kCached * nthreads; idx < n_in; idx += nthreads) {
            const uint4 v = x16[idx];
            act[idx] = make_int4(v.x, v.y, v.z, v.w);
            xs = sum_i8x4(v.x, sum_i8x4(v.y, sum_i8x4(v.z, sum_i8x4(v.w, xs))));
        }
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int c = 0; c < kCached; ++c) amax = absmax8_bf16(xv[c], amax);
        for (int idx = tid + kCached * nthreads; idx < n_in; idx += nthreads)
            amax = absmax8_bf16(x16[idx], amax);
        amax = wave_max(amax);
        if (lane == 0) amax_sh[wave] = amax;
        __syncthreads();
        amax = amax_sh[0];
        for (int i = 1; i < W; ++i) amax = fmaxf(amax, amax_sh[i]);
        sm = 127.0f / fmaxf(amax, 1e-5f);
        uint2* act8 = reinterpret_cast<uint2*>(act);
        const bool write_q = (band == 0) && (q_out != nullptr);
#pragma unroll
        for (int c = 0; c < kCached; ++c) {
            const int idx = tid + c * nthreads;
            if (idx < n_in) {
                const uint2 o = quant8_bf16(xv[c], sm);
                act8[idx] = o;
                xs = sum_i8x4(o.x, sum_i8x4(o.y, xs));
                if (write_q) reinterpret_cast<uint2*>(q_out)[idx] = o;
            }
        }
        for (int idx = tid + kCached * nthreads; idx < n_in; idx += nthreads) {
            const uint2 o = quant8_bf16(x16[idx], sm);
            act8[idx] = o;
            xs = sum_i8x4(o.x, sum_i8x4(o.y, xs));
            if (write_q) reinterpret_cast<uint2*>(q_out)[idx] = o;
        }
        if (band == 0 && s_out != nullptr && tid == 0) s_out[0] = sm;
    }
    for (int i = n16 + tid; i < padded16; i += nthreads) act[i] = make_int4(0, 0, 0, 0);
    // 1/s for the epilogue, computed here while the weights are in flight;
    // the empty asm statement keeps the compiler from sinking the division
    // past the barriers to its use.
    double inv_s = 1.0 / static_cast<double>(sm);
    asm volatile("" : "+v"(inv_s));
    xs = wave_sum(xs);
    if (lane == 0) xsum_sh[wave] = xs;
    __syncthreads();

    // 3. P steps of 4 rows x 16 K per lane.
    RowAcc r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a1[i] = r.a4[i] = r.a16[i] = 0;
    const int kc = lane & 3;
#pragma unroll
    for (int u = 0; u < P; ++u) dot_slot(w[u], act[(s0 + u) * 4 + kc], r);
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r.a1[i] + (r.a4[i] >> 2) + (r.a16[i] >> 4);   // exact
    part_sh[wave][lane] = quad_reduce_scatter(v, lane);
    __syncthreads();

    // 4. Wavefront 0: add the W partial sums of row `lane`, remove the code
    //    offset, epilogue.
    if (wave == 0) {
        int total = 0, xsum = 0;
        for (int i = 0; i < W; ++i) {
            total += part_sh[i][lane];
            xsum += xsum_sh[i];
        }
        total -= 2 * xsum;
        if (n < N) {
            y[n] = epilogue_bf16_fast(total, bf16_to_float(wsb), sm, inv_s);
            if (acc) acc[n] = total;
        }
    }
}

constexpr int kMaxSteps = 20;

using GemvFn = void (*)(const void*, const v4u*, const float*, const uint16_t*, int, uint16_t*,
                        int32_t*, int8_t*, float*, int, int);

template <bool FUSED, int... Ps>
constexpr std::array<GemvFn, sizeof...(Ps)> kernel_table(std::integer_sequence<int, Ps...>) {
    return {{&gemv_kernel<Ps + 1, FUSED>...}};
}

const std::array<GemvFn, kMaxSteps> kI8Kernels =
    kernel_table<false>(std::make_integer_sequence<int, kMaxSteps>{});
const std::array<GemvFn, kMaxSteps> kBf16Kernels =
    kernel_table<true>(std::make_integer_sequence<int, kMaxSteps>{});

hipError_t launch(bool fused, const void* x, const uint8_t* packed, const float* s,
                  const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int8_t* q_out,
                  float* s_out, int N, int K, hipStream_t stream) {
    const GemvShape g = gemv_shape(K);
    if (g.waves == 0) return hipErrorInvalidValue;
    const unsigned bands = static_cast<unsigned>((N + kTileRows - 1) / kTileRows);
    const size_t lds = static_cast<size_t>(g.waves) * g.steps * kTileK;
    const GemvFn fn = fused ? kBf16Kernels[g.steps - 1] : kI8Kernels[g.steps - 1];
    fn<<<bands, g.waves * 64, lds, stream>>>(x, reinterpret_cast<const v4u*>(packed), s, ws,
                                            N / ws_num, y, acc, q_out, s_out, N, K);
    return hipGetLastError();
}

}  // namespace

GemvShape gemv_shape(int K) {
    // W wavefronts x P steps covering S steps: minimise the busiest SIMD's
    // step count (ceil(W/4) * P), then the wasted steps, then prefer more
    // wavefronts.
    const int S = (K + kTileK - 1) / kTileK;
    GemvShape best{0, 0};
    int best_load = 1 << 30, best_waste = 1 << 30;
    for (int W = kMaxWaves; W >= 1; --W) {
        const int P = (S + W - 1) / W;
        if (P > kMaxSteps) continue;
        const int load = ((W + 3) / 4) * P;
        const int waste = W * P - S;
        if (load < best_load || (load == best_load && waste < best_waste)) {
            best = GemvShape{W, P};
            best_load = load;
            best_waste = waste;
        }
    }
    return best;
}

hipError_t launch_gemv_i8(const int8_t* xq, const uint8_t* packed, const float* s,
                          const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int N, int K,
                          hipStream_t stream) {
    return launch(false, xq, packed, s, ws, ws_num, y, acc, nullptr, nullptr, N, K, stream);
}

hipError_t launch_gemv_bf16_fused(const uint16_t* x, const uint8_t* packed, const uint16_t* ws,
                                  int ws_num, uint16_t* y, int8_t* q_out, float* s_out,
                                  int32_t* acc, int N, int K, hipStream_t stream) {
    return launch(true, x, packed, nullptr, ws, ws_num, y, acc, q_out, s_out, N, K, stream);
}

}  // namespace bl
