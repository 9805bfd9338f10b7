// gemm_band.hip -- the batched W2A8 ternary layer for a few rows of
// activations (2 <= M <= 64, K <= 2560) on gfx950 int8 MFMA, one wavefront
// per one or two 16-row bands of weights.
//
// Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
// (blog.gitcode.com), cited as [W2A8]: §5.2 (codes w + 2, interleaved words),
// §5.3 (int8 products into int32, then out = acc * scales per row).  The
// page's kernel is M == 1 only; here the same arithmetic runs row-wise on
// v_mfma_i32_16x16x64_i8, since with 16 or more rows the layer is a dense
// contraction.
//
// Mapping (this library's design):
//   * a workgroup is 4 wavefronts over 4 BW consecutive 16-row bands (64 BW
//     output rows n) and a group of up to 16 MT rows of activations (MT
//     tiles of 16); each wavefront owns BW bands over the whole of K, so no
//     partial sums cross wavefronts and the epilogue runs from the MFMA
//     accumulators.  BW = 1 with one group of all M <= 32 rows; BW = 2 with
//     groups of 32 rows for M = 33 .. 64, where all rows of K = 2560 would
//     not fit the LDS: a wavefront then reads each staged operand once for
//     two bands' MFMAs, so a CU reads no more LDS per tile than at M = 32,
//     and the row groups of one band group run on one XCD (workgroup ids 8
//     apart), which reads those weights through one L2;
//   * the wavefront's P weight tiles (1 KiB each) are loaded exactly as the
//     GEMV loads them -- one coalesced 16-byte load per lane per tile, all
//     issued up front -- after the activations the workgroup stages;
//   * the activations (16 MT rows x K, int8) are staged once per workgroup
//     in LDS, rows padded by 16 bytes so that the operand reads of a row
//     group fall in different banks; one m tile is loaded as 16-byte chunks
//     (16 threads per row) and stored as 4-byte groups, two as "quads" of
//     four chunks that each thread turns into whole 16-byte operands in
//     registers (measured: M = 16 staging 640 ns vs 755 ns as quads; M = 32
//     1090 ns as quads vs 1490 ns as chunks);
//   * a tile reaches the MFMA B layout through a wavefront-private 1 KiB LDS
//     slot per band: lane l (rows 4 (l / 16) .. +3 of K chunk l % 16) stores
//     its 16 bytes at 64 (l % 16) + 16 (l / 16), so that lane (j, g) finds
//     the word of row j, K chunk 4v + g at 256 v + 64 g + 4 j -- 64
//     consecutive dwords per read, free of bank conflicts (two slots used in
//     turn, so that the next tile's round trip overlaps this tile's MFMAs,
//     measured slower at M = 16 / 32, where the loop runs at the pace the
//     weights arrive, and no faster at M = 64);
//   * the codes stay unsigned (c = w + 2) and each 2-bit field is masked in
//     place: MFMA f takes field f of the lane's four words (chunks g, g + 4,
//     g + 8, g + 12), so all of its bytes carry the factor 4^f (field 3 is
//     shifted down: factor 1), and adds into the accumulator of that factor;
//     the activations are staged so that the matching operand of lane (i, g)
//     is 16 contiguous bytes, and the +2 offset goes with the rows' sums;
//   * epilogue per output: y = bf16(acc * ws[n] / s[m]) through the fp64
//     product and fp32 (as epilogue_bf16_scaled), the exact division only for
//     an output whose fp32 value is a bf16 midpoint.
#include <algorithm>
#include <array>
#include <utility>

#include "gemv_core.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kWaves = 4;                 // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kRowPad = 16;               // bytes past each staged activation row
constexpr int kRawBufferFlags = 0x00020000;   // word 3 of a buffer descriptor: 32-bit data format
constexpr int kOutOfRange = 0x7FFFFFF0;       // a buffer offset past any record: reads as zero

__device__ __forceinline__ void wave_lds_fence() {
    // LDS operations of one wavefront complete in order; the fences keep
    // the compiler from moving reads above writes or writes above reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Field f of a packed word masked in place: the codes of elements 4f .. 4f + 3
// as bytes, times 4^f for f < 3; field 3 is shifted down (factor 1).
template <int F>
__device__ __forceinline__ int field(uint32_t w) {
    if constexpr (F == 3) return static_cast<int>((w >> 6) & 0x03030303u);
    return static_cast<int>(w & (0x03030303u << (2 * F)));
}
// Field f of a tile's four words as the MFMA operand.  Field 3 shifts two
// words at a time (one 64-bit shift per pair; what it moves from one word
// into the other falls outside the mask): 2 VALU fewer per band and tile.
// Same box, 13824 x 2560: M = 16 / 32 / 64 4.23 / 5.80 / 8.85 -> 4.21 /
// 5.76 / 8.84 us.
template <int F>
__device__ __forceinline__ v4i fields(const uint32_t (&w)[4]) {
    if constexpr (F == 3) {
        constexpr uint64_t m = 0x0303030303030303ull;
        const uint64_t lo = (((static_cast<uint64_t>(w[1]) << 32) | w[0]) >> 6) & m;
        const uint64_t hi = (((static_cast<uint64_t>(w[3]) << 32) | w[2]) >> 6) & m;
        return v4i{static_cast<int>(lo), static_cast<int>(lo >> 32), static_cast<int>(hi),
                   static_cast<int>(hi >> 32)};
    }
    return v4i{field<F>(w[0]), field<F>(w[1]), field<F>(w[2]), field<F>(w[3])};
}

// Workgroup id -> (band group bg, row group mg), H row groups.  The GPU hands
// workgroups to its eight XCDs in turn (id mod 8); the H row groups of a band
// group get ids 8 apart, on one XCD, so that they read its weights through
// one L2.  With H = 1 the id is the band group.
template <int H>
__device__ __forceinline__ void split_group_id(int id, int groups, int& bg, int& mg) {
    static_assert(H == 1 || H == 2, "one or two row groups");
    if constexpr (H == 1) {
        bg = id;
        mg = 0;
    } else {
        const int full = groups >> 3;              // runs of 8 band groups
        const int run = id >> 4;
        if (run < full) {
            mg = (id >> 3) & 1;
            bg = 8 * run + (id & 7);
        } else {
            const int r = id - 16 * full;
            const int rest = groups - 8 * full;    // 1 .. 7 band groups left
            mg = r >= rest ? 1 : 0;
            bg = 8 * full + r - mg * rest;
        }
    }
}

// MT = m tiles of 16 rows per row group; P = 256-K tiles per band (= ceil(K / 256));
// BW = bands per wavefront.  BW = 1: one row group (M <= 16 MT); BW = 2: two
// row groups of 16 MT rows (M = 33 .. 64 with MT = 2).
// (Two wavefronts per band, each dotting half the tiles and handing its sums
// to the other through LDS, measured slower at 13824 x 2560: M = 16 4.76 ->
// 5.07 us, M = 32 5.91 -> 6.46 us with an earlier decode, and M = 32 / 64
// 5.81 / 8.98 -> 6.75 / 9.08 us with this one.  Four more wavefronts that
// only stage the activations, so that the bands' weight loads go out at
// once, measured slower still -- M = 16 4.44 -> 5.37 us: a CU returns its
// loads in the order they were issued, so the rows then arrive behind the
// weights.)
template <int MT, int P, int BW>
__global__ __launch_bounds__(kThreads) void gemm_band_kernel(
    const int8_t* __restrict__ xq, const v4u* __restrict__ packed, const float* __restrict__ s,
    const uint16_t* __restrict__ ws, uint32_t seg_mul, int seg_shift, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out, int M, int N, int K) {
    extern __shared__ __align__(16) uint8_t lds[];   // staged rows, then the tile slots
    __shared__ double inv_s_sh[16 * MT];
    __shared__ float s_sh[16 * MT];
    __shared__ int rowsum_sh[16 * MT];
    constexpr int kRows = 16 * MT;
    constexpr int kPitch = P * kTileK + kRowPad;
    constexpr int kGroupBands = kWaves * BW;
    constexpr int H = BW;                             // row groups
    // MT = 1: thread t stages chunks t % 16 + 16 i of row t / 16 (one per tile);
    // MT = 2: thread t stages quads t, t + 256, ... (see below).
    constexpr int kQuadsAll = kRows * 4 * P;                       // a multiple of 64
    constexpr int kIters = MT == 1 ? P : (kQuadsAll + kThreads - 1) / kThreads;
    constexpr int kALoads = MT == 1 ? P : 4 * kIters;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nbands = (N + kTileRows - 1) / kTileRows;
    int bg, mg;
    split_group_id<H>(static_cast<int>(blockIdx.x), (nbands + kGroupBands - 1) / kGroupBands, bg,
                      mg);
    const int m0 = mg * kRows;                        // first activation row of the group
    const int j = lane & 15;
    const int g = lane >> 4;
    // band b of this wavefront: 16 rows from band_lin[b]; n[b] = this lane's output column
    int band_lin[BW], n[BW];
#pragma unroll
    for (int b = 0; b < BW; ++b) {
        band_lin[b] = bg * kGroupBands + wave * BW + b;
        n[b] = band_lin[b] * kTileRows + j;
    }

    // 1. The row scale and this lane's weight scales, this thread's share of
    //    the activation rows, then every weight tile.  Chunks past K and rows
    //    past M are read at an offset beyond the buffer, which the hardware
    //    returns as zeros without a memory access; there is no branch around
    //    a load (a merge would copy its registers, waiting for it), and the
    //    offsets are 24-bit products (a 32-bit multiply-add is selected as the
    //    64-bit one with an undefined high half, which the compiler may take
    //    from a register still being loaded, and wait for it).
    // Buffer loads for the rows and scales: the compiler keeps them where
    // they stand, ahead of the weight loads (plain loads of read-only data it
    // would move to their first use, behind the weights).
    const __amdgpu_buffer_rsrc_t xb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(xq), 0, M * K, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t sb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(s), 0, 4 * M, kRawBufferFlags);
    const int srow = tid & (kRows - 1);            // kRows is 16 or 32
    const float s_row = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(sb, 4 * min(m0 + srow, M - 1), 0, 0));
    // (the index as a 32-bit unsigned: a signed one made the compiler read an
    // undefined high half from a register still being loaded, waiting for it)
    uint16_t wsb[BW];
#pragma unroll
    for (int b = 0; b < BW; ++b) {
        const uint32_t n_ws = static_cast<uint32_t>(min(n[b], N - 1));
        wsb[b] = ws[(static_cast<uint64_t>(n_ws) * seg_mul) >> seg_shift];
    }
    const int nck = K >> 4;                        // real 16-byte chunks per row
    v4u a[kALoads];
    if constexpr (MT == 1) {
        // 16 threads per row, one chunk per tile: a wavefront instruction
        // reads 256-byte runs of four rows
        const int r = tid >> 4;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int c = (tid & 15) + 16 * i;
            a[i] = __builtin_amdgcn_raw_buffer_load_b128(
                xb, c < nck && m0 + r < M ? __mul24(m0 + r, K) + 16 * c : kOutOfRange, 0, 0);
        }
    } else {
        // Quad (u, g) of a row is its 16-wide K chunks g, g + 4, g + 8,
        // g + 12 of tile u; the 4P quads of each row are numbered row-major
        // (g fastest) and thread t takes numbers t, t + 256, ...: a wavefront
        // instruction reads 64-byte runs, and the last round is uniform per
        // wavefront (numbers past the last are read out of range too).
#pragma unroll
        for (int i = 0; i < kIters; ++i) {
            const int q = tid + i * kThreads;
            const int r = q / (4 * P);
            const int jq = q - r * (4 * P);
            const int ck = 16 * (jq >> 2) + (jq & 3);   // chunk of v = 0
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const bool real =
                    (i + 1 < kIters || q < kQuadsAll) && ck + 4 * v < nck && m0 + r < M;
                a[4 * i + v] = __builtin_amdgcn_raw_buffer_load_b128(
                    xb, real ? __mul24(m0 + r, K) + 16 * (ck + 4 * v) : kOutOfRange, 0, 0);
            }
        }
    }
    // The activation loads go out first, so that a wait for them leaves the
    // weight loads in flight, and those of every wavefront before any
    // wavefront's weights (a barrier without a wait: the loads are issued,
    // not complete), so that no row queues behind another wavefront's
    // weights.  Same box: M = 16 / 64 4.28 / 8.97 -> 4.23 / 8.94 us.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // Tile u of every band goes out before tile u + 1 of any, in the order
    // the loop below waits for them.
    const v4u* tiles[BW];
#pragma unroll
    for (int b = 0; b < BW; ++b)
        tiles[b] = packed + static_cast<size_t>(min(band_lin[b], nbands - 1)) * P * 64 + lane;
    v4u wt[BW][P];
#pragma unroll
    for (int u = 0; u < P; ++u)
#pragma unroll
        for (int b = 0; b < BW; ++b) {
            wt[b][u] = __builtin_nontemporal_load(tiles[b] + u * 64);
            __builtin_amdgcn_sched_barrier(0);
        }
    // No load may sink below this point (the compiler would otherwise move the
    // activation loads to their first use, behind a wait that counts every
    // weight load too), and nothing may be scheduled above it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // 2. Stage the rows (waits for the activation loads only), their sums
    //    and the scales.  Group f (bytes 4f .. 4f + 3) of chunk cc of tile u
    //    goes to byte 4 (cc / 4) of slot 4 (f ^ (u % 4)) + cc % 4 of the
    //    row's tile (16 slots of 16 bytes): the operand of MFMA f for lanes
    //    (i, g) -- group f of chunks g, g + 4, g + 8, g + 12 -- is one slot.
    if constexpr (MT == 1) {
        const int r = tid >> 4;
        const int cc = tid & 15;
        int xs = 0;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            uint8_t* tile = lds + r * kPitch + i * kTileK + 16 * (cc & 3) + 4 * (cc >> 2);
#pragma unroll
            for (int f = 0; f < 4; ++f) *reinterpret_cast<uint32_t*>(tile + 64 * (f ^ (i & 3))) = a[i][f];
            xs = sum_i8x4(a[i].x, sum_i8x4(a[i].y, sum_i8x4(a[i].z, sum_i8x4(a[i].w, xs))));
        }
        // the row's 16 threads are a DPP row
        xs += dpp_row<kDppQuadXor1>(xs);
        xs += dpp_row<kDppQuadXor2>(xs);
        xs += dpp_row<kDppRowRor4>(xs);
        xs += dpp_row<kDppRowRor8>(xs);
        if (cc == 0) rowsum_sh[r] = xs;
    } else {
        // A quad's four chunks make whole slots: one 16-byte store per group
        // f, and the stores of 16 consecutive threads (quads of four tiles)
        // hit 16 different slots.  A quad's sum is reduced over its 4 lanes
        // and added into its row's.
        if (tid < kRows) rowsum_sh[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kIters; ++i) {
            const int q = tid + i * kThreads;
            const int r = q / (4 * P);
            const int jq = q - r * (4 * P);
            const int u = jq >> 2;
            if (i + 1 < kIters || q < kQuadsAll) {
                uint8_t* tile = lds + r * kPitch + u * kTileK + 16 * (jq & 3);
                int xs = 0;
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    *reinterpret_cast<v4u*>(tile + 64 * (f ^ (u & 3))) =
                        v4u{a[4 * i][f], a[4 * i + 1][f], a[4 * i + 2][f], a[4 * i + 3][f]};
#pragma unroll
                    for (int v = 0; v < 4; ++v) xs = sum_i8x4(a[4 * i + v][f], xs);
                }
                xs += dpp_row<kDppQuadXor1>(xs);
                xs += dpp_row<kDppQuadXor2>(xs);
                if ((jq & 3) == 0) atomicAdd(&rowsum_sh[r], xs);
            }
        }
    }
    // every thread stores its row's scale (threads tid and tid + kRows store
    // the same value): a store under a branch would let the compiler sink
    // the scale's load into it, behind the weight loads
    s_sh[srow] = s_row;
    inv_s_sh[srow] = 1.0 / static_cast<double>(s_row);
    __syncthreads();

    // 3. Per tile: through the wavefront's slots, lane (j, g) takes the words
    //    of row j of each band for chunks g, g + 4, g + 8, g + 12; MFMA f
    //    multiplies field f of the four (unsigned codes c = w + 2, masked in
    //    place) into the accumulator of its factor: 1 (fields 0 and 3), 4
    //    (field 1), 16 (field 2).  An activation operand read from LDS serves
    //    the MFMAs of all BW bands.
    // This lane's rows' constants for the epilogue, read now so that their
    // LDS latency passes under the main loop: the code offset -2 sum(x), the
    // fp64 scale ws / s of each band and s itself, for rows m0 + 16 mt + 4 g + v.
    float wsf[BW];
#pragma unroll
    for (int b = 0; b < BW; ++b) wsf[b] = bf16_to_float(wsb[b]);
    int offset[MT][4];
    double cs[BW][MT][4];
    float sm[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int r = 16 * mt + 4 * g + v;
            offset[mt][v] = -2 * rowsum_sh[r];
#pragma unroll
            for (int b = 0; b < BW; ++b) cs[b][mt][v] = static_cast<double>(wsf[b]) * inv_s_sh[r];
            sm[mt][v] = s_sh[r];
        }
    uint8_t* slot = lds + kRows * kPitch + wave * BW * kTileBytes;
    v4i acc[3][BW][MT];
#pragma unroll
    for (int k = 0; k < 3; ++k)
#pragma unroll
        for (int b = 0; b < BW; ++b)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[k][b][mt] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < P; ++u) {
#pragma unroll
        for (int b = 0; b < BW; ++b)
            *reinterpret_cast<v4u*>(slot + b * kTileBytes + 64 * (lane & 15) + 16 * (lane >> 4)) =
                wt[b][u];
        wave_lds_fence();
        uint32_t bw[BW][4];
#pragma unroll
        for (int b = 0; b < BW; ++b)
#pragma unroll
            for (int w = 0; w < 4; ++w)
                bw[b][w] = *reinterpret_cast<const uint32_t*>(slot + b * kTileBytes + 256 * w + 4 * lane);
        wave_lds_fence();
        const uint8_t* arow_u = lds + j * kPitch + u * kTileK + 16 * g;
#define BAND_STEP(F, ACC)                                                                         \
        {                                                                                         \
            v4i bop[BW];                                                                          \
            _Pragma("unroll") for (int b = 0; b < BW; ++b)                                        \
                bop[b] = fields<F>(bw[b]);                                                        \
            _Pragma("unroll") for (int mt = 0; mt < MT; ++mt) {                                   \
                const v4i av = *reinterpret_cast<const v4i*>(arow_u + 16 * mt * kPitch +          \
                                                             64 * ((F) ^ (u & 3)));               \
                _Pragma("unroll") for (int b = 0; b < BW; ++b)                                    \
                    acc[ACC][b][mt] =                                                             \
                        __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bop[b], acc[ACC][b][mt], 0, 0, 0); \
            }                                                                                     \
        }
        BAND_STEP(0, 0)
        BAND_STEP(1, 1)
        BAND_STEP(2, 2)
        BAND_STEP(3, 0)
#undef BAND_STEP
    }

    // 4. Epilogue: lane (j, g), register v of m tile mt of band b -> row
    //    m = m0 + 16 mt + 4 g + v, column n[b]; acc = a1 + a4 / 4 + a16 / 16
    //    - 2 sum(x) (exact), then bf16(acc * ws / s) by epilogue_bf16_scaled's
    //    argument, for all the lane's outputs at once: one ballot for the
    //    midpoints, then the stores.
    int total[BW][MT][4];
    float fv[BW][MT][4];
    bool mid[BW][MT][4];
    bool redo = false;
#pragma unroll
    for (int b = 0; b < BW; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const v4i* c = acc[0][b] + mt;
            const v4i* c4 = acc[1][b] + mt;
            const v4i* c16 = acc[2][b] + mt;
            const int t[4] = {c->x + (c4->x >> 2) + (c16->x >> 4), c->y + (c4->y >> 2) + (c16->y >> 4),
                              c->z + (c4->z >> 2) + (c16->z >> 4), c->w + (c4->w >> 2) + (c16->w >> 4)};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                total[b][mt][v] = t[v] + offset[mt][v];
                fv[b][mt][v] = static_cast<float>(static_cast<double>(total[b][mt][v]) * cs[b][mt][v]);
                mid[b][mt][v] = ((__float_as_uint(fv[b][mt][v]) & 0xFFFFu) == 0x8000u) ||
                                __builtin_isnan(fv[b][mt][v]);
                redo |= mid[b][mt][v];
            }
        }
    uint16_t out[BW][MT][4];
#pragma unroll
    for (int b = 0; b < BW; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                out[b][mt][v] = static_cast<uint16_t>(cvt_pk_bf16(fv[b][mt][v], 0.0f));
    // Only the outputs that a lane needs are redone, each under its own
    // ballot: a wavefront that meets a midpoint (about one in 64 at 16
    // outputs a lane) runs one exact division, not one per output.  Redoing
    // all 16 took 5.2 us against 1.3 us for the epilogue (M = 64, 13824 x
    // 2560), and those wavefronts ended the launch.
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(redo) != 0, 0)) {
        asm volatile("");   // kept a branch: if-converted it would cost every output its division
#pragma unroll
        for (int b = 0; b < BW; ++b)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (__builtin_amdgcn_ballot_w64(mid[b][mt][v]) != 0) {
                        asm volatile("");
                        out[b][mt][v] = epilogue_bf16(total[b][mt][v], wsf[b], sm[mt][v]);
                    }
    }
    // y is written through the L2 (device-scope buffer stores): the launch
    // then ends without its dirty output lines to write back.  The stores
    // themselves, and their completion at the end of the launch, cost 0.4 /
    // 0.5 / 0.7 us at M = 16 / 32 / 64 (a copy without them); written
    // through, M = 64 8.98-9.00 -> 8.88-8.89 us, M = 16 / 32 unchanged, same
    // box.  (Every byte offset 2 (m N + n) < 2^31: M <= 64, N <= 2^24.)
    constexpr int kStoreDeviceScope = 16;   // the sc1 bit of the store's cache policy
    // (the record count is an unsigned 32-bit field: 2 M N up to 2^31 bytes)
    const __amdgpu_buffer_rsrc_t yb = __builtin_amdgcn_make_buffer_rsrc(
        y, 0, static_cast<int>(2u * static_cast<uint32_t>(M * N)), kRawBufferFlags);
#pragma unroll
    for (int b = 0; b < BW; ++b) {
        if (n[b] < N) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int m = m0 + 16 * mt + 4 * g + v;
                    if (m < M) {
                        const int o = m * N + n[b];
                        __builtin_amdgcn_raw_buffer_store_b16(out[b][mt][v], yb, 2 * o, 0,
                                                              kStoreDeviceScope);
                        if (acc_out) acc_out[o] = total[b][mt][v];
                    }
                }
        }
    }
}

using BandFn = void (*)(const int8_t*, const v4u*, const float*, const uint16_t*, uint32_t, int,
                        uint16_t*, int32_t*, int, int, int);

template <int MT, int BW, int... Ps>
constexpr std::array<BandFn, sizeof...(Ps)> band_table(std::integer_sequence<int, Ps...>) {
    return {{&gemm_band_kernel<MT, Ps + 1, BW>...}};
}

constexpr int kBandMaxSteps = kBandMaxK / kTileK;

// The instances: m tiles per row group and bands per wavefront.
struct BandShape {
    int mt, bw;
};
constexpr std::array<BandShape, 3> kBandShapes = {{{1, 1}, {2, 1}, {2, 2}}};

// [shape][P - 1]
const std::array<std::array<BandFn, kBandMaxSteps>, 3> kBandKernels = {{
    band_table<1, 1>(std::make_integer_sequence<int, kBandMaxSteps>{}),
    band_table<2, 1>(std::make_integer_sequence<int, kBandMaxSteps>{}),
    band_table<2, 2>(std::make_integer_sequence<int, kBandMaxSteps>{}),
}};

// M <= 16: one m tile; M <= 32: two; M = 33 .. 64: row groups of 32 rows with
// two bands per wavefront (all 64 rows of K = 2560 would need 165 KB of LDS).
int band_shape_of(int M) { return M <= 16 ? 0 : M <= 32 ? 1 : 2; }

size_t band_lds_bytes(const BandShape& sh, int P) {
    return static_cast<size_t>(16 * sh.mt) * (P * kTileK + kRowPad) +
           static_cast<size_t>(kWaves * sh.bw) * kTileBytes;
}

}  // namespace

hipError_t launch_gemm_band(const int8_t* xq, const uint8_t* packed, const float* s,
                            const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int M,
                            int N, int K, hipStream_t stream) {
    if (M < 2 || M > kBandMaxM || K > kBandMaxK) return hipErrorInvalidValue;
    const int shape = band_shape_of(M);
    const BandShape& sh = kBandShapes[shape];
    const int P = (K + kTileK - 1) / kTileK;
    const BandFn fn = kBandKernels[shape][P - 1];
    const size_t lds = band_lds_bytes(sh, P);
    // Staged rows beyond 64 KiB of LDS (more than 16 rows at K = 2560) need
    // the kernel's dynamic-LDS limit raised, once per kernel and device.
    if (lds > 65536) {
        const hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(fn), static_cast<int>(lds));
        if (e != hipSuccess) return e;
    }
    uint32_t seg_mul;
    int seg_shift;
    seg_divisor(N / ws_num, seg_mul, seg_shift);
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const int groups = (nbands + kWaves * sh.bw - 1) / (kWaves * sh.bw);
    const int H = sh.bw;                                  // row groups, as the kernel takes them
    if (M > 16 * sh.mt * H) return hipErrorInvalidValue;
    fn<<<static_cast<unsigned>(groups * H), kThreads, lds, stream>>>(
        xq, reinterpret_cast<const v4u*>(packed), s, ws, seg_mul, seg_shift, y, acc, M, N, K);
    return hipGetLastError();
}

}  // namespace bl
