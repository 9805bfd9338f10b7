// gemv_group.hip -- many independent M = 1 GEMVs with bf16 activations in
// one launch: the decode step replayed as a graph ([W2A8] §六 item 1) whose
// projections do not depend on one another runs them as a single grouped
// kernel instead of one launch each.
//
// Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
// (blog.gitcode.com), cited as [W2A8]: §5.2 (codes w + 2, interleaved 32-bit
// words), §5.3 (int8 dot products into int32, out = acc * scales with
// ws[n / (N / ws_num)]), §六 item 3 (per-token activation quantisation), §六
// item 1 (the decode step captured once and replayed).
//
// Mapping (this library's design):
//   * the host writes one 64-byte work record per workgroup (the node's
//     pointers, N, K, weight-scale segment constants and the workgroup's
//     index within its node); a workgroup reads its record with one scalar
//     load and needs nothing else from the kernel arguments;
//   * every workgroup is 4 wavefronts over 4 consecutive 16-row bands of its
//     node, one wavefront per band, whatever N and K: grouped together the
//     nodes give tens of thousands of bands, so the narrow matrices need no
//     splitting of K across wavefronts, and each staging of the activation
//     row serves 64 output rows;
//   * the workgroup quantises its node's bf16 row into LDS (per-token absmax,
//     as the fused single GEMV does), zero-padded to whole chunks;
//   * a wavefront streams its band in chunks of P = 10 tiles (16-byte
//     non-temporal loads, 1 KiB per wavefront instruction), double-buffered:
//     the first two chunks are issued before the activation row is even
//     quantised, and chunk c + 2 is issued as soon as chunk c has been
//     dotted, so a K = 6912 row (27 tiles: chunks of 10, 10 and 7) keeps
//     two chunks in flight; the last chunk's steps past the row re-read its
//     last tile and meet zero activations.  The chunk count (1 to 4, so
//     K <= 10240) is a template argument of the body, chosen per workgroup
//     by a uniform branch, so that the compiler counts every chunk's loads
//     exactly in its waits;
//   * dot products (v_dot8 on the row staged split into nibbles), row
//     reduction and epilogue are those of the single GEMV (gemv_core.hpp,
//     common.hpp); each wavefront writes its own 16 rows.
#include <algorithm>
#include <vector>

#include "gemv_core.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kGroupWaves = 4;          // wavefronts (= bands) per workgroup
constexpr int kGroupChunk = 10;         // tiles per chunk of a wavefront's band
constexpr int kGroupCached = 2;         // 16-element chunks (32 bytes of bf16) per thread in registers

__device__ __forceinline__ uint4 as_uint4(v4u v) { return make_uint4(v.x, v.y, v.z, v.w); }

// One workgroup's 4 bands; NCH chunks of P tiles per band (a compile-time
// count, so that every wait for a chunk counts its loads exactly).
template <int P, int C, int NCH>
__device__ __forceinline__ void group_body(const GroupWork& g, int4* __restrict__ act,
                                           int* __restrict__ xsum_sh, float* __restrict__ amax_sh) {
    const int N = g.N;
    const int K = g.K;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const int band_lin = g.group * kGroupWaves + wave;
    const int band = min(band_lin, nbands - 1);
    const int S = (K + kTileK - 1) / kTileK;

    // 1. This lane's weight scale and its share of the bf16 row, then the
    //    first two chunks of weights.
    const int n_out = band_lin * kTileRows + 4 * (lane >> 4) + (lane & 3);
    const uint32_t n_ws = static_cast<uint32_t>(min(n_out, N - 1));
    const uint16_t wsb = global(g.ws)[(static_cast<uint64_t>(n_ws) * g.seg_mul) >> g.seg_shift];
    const int n16 = K >> 4;             // 16-element chunks of the row (32 bytes of bf16)
    const global_ptr<const v4u> x16 = global(reinterpret_cast<const v4u*>(g.x));
    uint4 xv[2 * C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int q = tid + c * (kGroupWaves * 64);
        xv[2 * c] = xv[2 * c + 1] = make_uint4(0, 0, 0, 0);
        if (q < n16) {
            xv[2 * c] = as_uint4(x16[2 * q]);
            xv[2 * c + 1] = as_uint4(x16[2 * q + 1]);
        }
    }
    // Every wavefront's row loads go out before any wavefront's weight loads
    // (a barrier without a wait: the loads are issued, not complete), so
    // that no row queues behind another wavefront's weights.  The decode
    // step, six pairs of runs on one box: 85.2 -> 82.7 us on average.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const global_ptr<const v4u> tiles =
        global(reinterpret_cast<const v4u*>(g.packed)) + static_cast<size_t>(band) * S * 64 + lane;
    v4u w[2][P];
    load_steps<P>(tiles, 0, S - 1, w[0]);
    if constexpr (NCH > 1) load_steps<P>(tiles, P, S - 1, w[1]);
    // Nothing above this point: a wait for the row must not hold back a weight load.
    __builtin_amdgcn_sched_barrier(0);

    // 2. Quantise the row into LDS ([W2A8] §六 item 3), whole 16-element
    //    chunks staged split into nibbles for v_dot8, and sum it (for the +2
    //    code offset).
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c)
        if (tid + c * (kGroupWaves * 64) < n16)
            amax = absmax8_bf16(xv[2 * c], absmax8_bf16(xv[2 * c + 1], amax));
    for (int q = tid + C * (kGroupWaves * 64); q < n16; q += kGroupWaves * 64)
        amax = absmax8_bf16(as_uint4(x16[2 * q]), absmax8_bf16(as_uint4(x16[2 * q + 1]), amax));
    amax = wave_max(amax);
    if (lane == 0) amax_sh[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(amax_sh[0], amax_sh[1]), fmaxf(amax_sh[2], amax_sh[3]));
    const float sm = 127.0f / fmaxf(amax, 1e-5f);
    int xs = 0;
    auto put = [&](int q, const uint4& lo, const uint4& hi) {
        const uint2 o0 = quant8_bf16(lo, sm), o1 = quant8_bf16(hi, sm);
        act[q] = nibble_split(make_int4(o0.x, o0.y, o1.x, o1.y));
        xs = sum_i8x4(o0.x, sum_i8x4(o0.y, sum_i8x4(o1.x, sum_i8x4(o1.y, xs))));
    };
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int q = tid + c * (kGroupWaves * 64);
        if (q < n16) put(q, xv[2 * c], xv[2 * c + 1]);
    }
    for (int q = tid + C * (kGroupWaves * 64); q < n16; q += kGroupWaves * 64)
        put(q, as_uint4(x16[2 * q]), as_uint4(x16[2 * q + 1]));
    for (int i = n16 + tid; i < NCH * P * 16; i += kGroupWaves * 64) act[i] = make_int4(0, 0, 0, 0);
    xs = wave_sum(xs);
    if (lane == 0) xsum_sh[wave] = xs;
    __syncthreads();
    const double cs = static_cast<double>(bf16_to_float(wsb)) * (1.0 / static_cast<double>(sm));
    const int offset = -2 * (xsum_sh[0] + xsum_sh[1] + xsum_sh[2] + xsum_sh[3]);

    // 3. NCH chunks of P steps of 4 rows x 16 K per lane; chunk c + 2 goes
    //    out as soon as chunk c is dotted, so two chunks stay in flight.
    NibAcc r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.lo[i] = 0, r.hi[i] = 0;
    const int kc = lane & 15;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int u = 0; u < P; ++u) dot_slot_nib(w[c & 1][u], act[(c * P + u) * 16 + kc], r);
        if (c + 2 < NCH) {
            // not above the dot products: the chunk's registers would then
            // need a third buffer (252 instead of ~130 VGPRs at three chunks)
            __builtin_amdgcn_sched_barrier(0);
            load_steps<P>(tiles, (c + 2) * P, S - 1, w[c & 1]);
        }
    }
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = static_cast<int>(r.lo[i]) + 16 * r.hi[i];   // exact
    const int rsum = row_group_reduce(v, lane);

    // 4. Lane l with (l / 4) % 4 == 0 holds row 4 * (l / 16) + l % 4 of the band.
    if (((lane >> 2) & 3) == 0 && n_out < N) {
        const int total = rsum + offset;
        global(g.y)[n_out] = epilogue_bf16_scaled(total, cs, bf16_to_float(wsb), sm);
        if (g.acc) global(g.acc)[n_out] = total;
    }
}

// One workgroup per work record; the record's K fixes the chunk count (a
// uniform branch).
template <int P, int C>
__global__ __launch_bounds__(kGroupWaves * 64) void gemv_group_kernel(
    const GroupWork* __restrict__ work) {
    extern __shared__ int4 act[];       // the int8 row, zero-padded to whole chunks
    __shared__ int xsum_sh[kGroupWaves];
    __shared__ float amax_sh[kGroupWaves];
    const GroupWork& g = work[blockIdx.x];
    const int S = (g.K + kTileK - 1) / kTileK;
    const int nchunk = (S + P - 1) / P;
    if (nchunk <= 1)
        group_body<P, C, 1>(g, act, xsum_sh, amax_sh);
    else if (nchunk == 2)
        group_body<P, C, 2>(g, act, xsum_sh, amax_sh);
    else if (nchunk == 3)
        group_body<P, C, 3>(g, act, xsum_sh, amax_sh);
    else
        group_body<P, C, 4>(g, act, xsum_sh, amax_sh);
}

}  // namespace

int group_workgroups(int N) {
    const int nbands = (N + kTileRows - 1) / kTileRows;
    return (nbands + kGroupWaves - 1) / kGroupWaves;
}

size_t group_lds_bytes(int K) {
    const int S = (K + kTileK - 1) / kTileK;
    const int nchunk = (S + kGroupChunk - 1) / kGroupChunk;
    return static_cast<size_t>(nchunk) * kGroupChunk * kTileK;
}

bool group_supported(int K) { return K <= kGroupMaxK; }

void group_work_records(const GroupNode& node, std::vector<GroupWork>& out) {
    uint32_t seg_mul;
    int seg_shift;
    seg_divisor(node.N / node.ws_num, seg_mul, seg_shift);
    const int groups = group_workgroups(node.N);
    for (int gi = 0; gi < groups; ++gi) {
        GroupWork w{};
        w.packed = node.packed;
        w.x = node.x;
        w.ws = node.ws;
        w.y = node.y;
        w.acc = node.acc;
        w.N = node.N;
        w.K = node.K;
        w.seg_mul = seg_mul;
        w.seg_shift = seg_shift;
        w.group = gi;
        out.push_back(w);
    }
}

hipError_t launch_gemv_group(const GroupWork* work, int n_work, size_t lds, hipStream_t stream) {
    gemv_group_kernel<kGroupChunk, kGroupCached>
        <<<static_cast<unsigned>(n_work), kGroupWaves * 64, lds, stream>>>(work);
    return hipGetLastError();
}

}  // namespace bl
