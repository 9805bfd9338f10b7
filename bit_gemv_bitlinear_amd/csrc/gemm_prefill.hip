// gemm_prefill.hip -- the W2A8 ternary layer for many activation rows
// (prompt processing) on gfx950 int8 MFMA.
//
// Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
// (blog.gitcode.com), cited as [W2A8].  The page runs prompt processing
// through a separate bf16 path (§一); here the same packed bytes serve it:
// int8 activations times ternary weights into int32, then the §5.3
// epilogue per row m with its own activation scale s[m].  For a few hundred
// rows m the layer is a dense contraction with enough reuse to be bound by
// the matrix cores rather than by HBM.
//
// Mapping (this library's design):
//   * workgroup = BN weight rows (BN/16 bands) x BM activation rows, all of
//     K, walked one 256-K tile (one packed tile per band) at a time; the
//     activation tile (BM x 256 bytes) and the BN/16 weight tiles of the
//     next K tile are loaded (16 bytes per lane, contiguous) into registers
//     while the current one is multiplied out of LDS, then stored to the
//     other LDS buffer: one barrier per K tile;
//   * wavefront (wn, wm) owns 64 weight rows (4 bands) x 16 * MTW activation
//     rows: per 64-K step it reads one weight word per band (lane (j, g):
//     row j, 16-K chunk g, [W2A8] §5.2's layout) and turns it into the
//     v_mfma_i32_16x16x64_i8 A operand, reads MTW activation operands
//     (lane (j, g): row m = j, chunk g) as the B operand, and accumulates
//     4 x MTW 16x16 int32 tiles in registers for all of K -- no reduction
//     across wavefronts; the A operand is the unsigned codes w + 2, and the
//     epilogue takes 2 * sum(x) of each activation row off its outputs;
//   * with the weights as the A operand, a lane's result is four
//     consecutive output columns n of one row m: the epilogue multiplies
//     them in fp64 by ws / s, converts to fp32 and packs them to bf16 (the
//     exact division only where an fp32 value is a bf16 midpoint), and
//     stores 8 bytes.
#include <algorithm>
#include <array>

#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

constexpr int kRawBufferFlags = 0x00020000;   // word 3 of a buffer descriptor: 32-bit data format

// LDS pitches.  Activation rows of 256 bytes at a pitch of 272: the operand
// reads (lanes j = 0..7 of a chunk read rows j at the same column) then hit
// eight distinct 16-byte bank groups.  Weight tiles as four 256-byte row
// groups at a pitch of 288: the word reads of one step (lane (j, g): row
// group j/4, word 16 * step + 4 * g + j % 4) hit 32 distinct banks in each
// half-wavefront.
constexpr int kAPitch = 272;
constexpr int kWRowGroupWords = 72;
constexpr int kWTileWords = 4 * kWRowGroupWords;
// The unsigned codes c = w + 2 of two packed words as two A operands of the
// MFMA, K order restored by shifting each 2-bit field down (padding stays 0):
// the MFMA then sums c * x, and the epilogue takes 2 * sum(x) off each row.
// One 64-bit shift serves both words (the bits it moves from one word into
// the other fall outside the mask): 11 VALU for two words instead of 14.
// Same box, 13824 x 2560: M = 256 15.78 -> 15.47 us, M = 512 24.37 -> 24.22.
__device__ __forceinline__ void decode_w2(uint32_t w0, uint32_t w1, v4i& a, v4i& b) {
    const uint64_t p = (static_cast<uint64_t>(w1) << 32) | w0;
    constexpr uint64_t m = 0x0303030303030303ull;
    const uint64_t f0 = p & m, f1 = (p >> 2) & m, f2 = (p >> 4) & m, f3 = (p >> 6) & m;
    a = v4i{static_cast<int>(f0), static_cast<int>(f1), static_cast<int>(f2), static_cast<int>(f3)};
    b = v4i{static_cast<int>(f0 >> 32), static_cast<int>(f1 >> 32), static_cast<int>(f2 >> 32),
            static_cast<int>(f3 >> 32)};
}

// WN x WMW wavefronts; wavefront tile 64 weight rows x 16 * MTW activation rows.
template <int WN, int WMW, int MTW>
__global__ __launch_bounds__(WN * WMW * 64) void gemm_prefill_kernel(
    const int8_t* __restrict__ xq, const v4u* __restrict__ tiles, const float* __restrict__ s,
    const uint16_t* __restrict__ ws, uint32_t seg_mul, int seg_shift, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out, int M, int N, int K) {
    constexpr int kWaves = WN * WMW;
    constexpr int kThreads = kWaves * 64;
    constexpr int BN = 64 * WN;                    // weight rows per workgroup
    constexpr int BM = 16 * MTW * WMW;             // activation rows per workgroup
    constexpr int kBands = BN / 16;
    constexpr int kAChunks = BM * 16 / kThreads;   // 16-byte activation chunks per thread and K tile
    constexpr int kWTiles = (kBands + kWaves - 1) / kWaves;   // weight tiles per wavefront and K tile
    static_assert(BM * 16 % kThreads == 0, "activation tile must split evenly");

    __shared__ __align__(16) int8_t a_lds[2][BM * kAPitch];
    __shared__ __align__(16) uint32_t w_lds[2][kBands * kWTileWords];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % WN;
    const int wm = wave / WN;
    const int j = lane & 15;
    const int g = lane >> 4;
    const int nbands = (N + kTileRows - 1) / kTileRows;
    const int S256 = (K + kTileK - 1) / kTileK;
    // Workgroups are dispatched to the eight XCDs in turn (id % 8).  The
    // blocks of activation rows that share a block of weight rows get ids
    // of one residue mod 8, so they run on one XCD and read those weight
    // tiles through one L2; the grid is padded to a multiple of 8 weight
    // blocks, and padding workgroups leave at once.
    const int gx = (N + BN - 1) / BN;
    const int gy = (M + BM - 1) / BM;
    const int slot = static_cast<int>(blockIdx.x) >> 3;
    const int nblk = static_cast<int>(blockIdx.x & 7) + 8 * (slot / gy);
    const int mblk = slot % gy;
    if (nblk >= gx) return;
    const int n_base = nblk * BN;
    const int m_base = mblk * BM;

    // Epilogue operands, loaded now so that nothing waits after the main
    // loop: the weight scales of this lane's 16 columns n (4 bands x 4
    // consecutive rows) and the activation scales of its MTW rows m.
    float wsf[4][4];
#pragma unroll
    for (int tw = 0; tw < 4; ++tw)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int n = min(n_base + 64 * wn + 16 * tw + 4 * g + v, N - 1);
            wsf[tw][v] = bf16_to_float(ws[(static_cast<uint64_t>(n) * seg_mul) >> seg_shift]);
        }
    float sm[MTW];
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) sm[mt] = s[min(m_base + 16 * (MTW * wm + mt) + j, M - 1)];

    // Global sources of this thread's share of a K tile.  Activation chunk
    // q = tid + kThreads * i is row q / 16, bytes 16 * (q % 16) of the tile
    // (sixteen lanes per 256-byte row); rows past M re-read row M - 1 and K
    // positions past K re-read the last chunk -- they meet rows that are not
    // written and padding codes.  Weight tile q = wave + kWaves * i of the
    // workgroup's bands (bands past the end re-read the last band).
    // Chunk i of this thread is row r0 + (kThreads / 16) * i; rows are
    // addressed from one base per workgroup with 32-bit offsets (BM rows of
    // at most 2^20 bytes).
    const int8_t* const a_blk = xq + static_cast<size_t>(m_base) * K;
    const int a_col = 16 * (tid & 15);   // the same for every chunk of this thread
    const int r0 = tid >> 4;
    const int r_last = M - 1 - m_base;
    const v4u* w_src[kWTiles];
    int w_dst[kWTiles];
    bool w_has[kWTiles];
#pragma unroll
    for (int i = 0; i < kWTiles; ++i) {
        const int bb = wave + kWaves * i;
        w_has[i] = bb < kBands;   // uniform per wavefront
        const int band = min(nblk * kBands + min(bb, kBands - 1), nbands - 1);
        w_src[i] = tiles + static_cast<size_t>(band) * S256 * 64 + lane;
        w_dst[i] = min(bb, kBands - 1) * kWTileWords + kWRowGroupWords * (lane >> 4) + 4 * (lane & 15);
    }

    // One register set carries the next K tile from global memory to LDS
    // while the current one is multiplied out of the other LDS buffer (a
    // second set, loading two tiles ahead, measured no faster).
    v4i ra[kAChunks];
    v4u rw[kWTiles];
    // sum of this thread's activation bytes per chunk row, over real K only
    // (a chunk past K re-reads the last one and must not count)
    int xsum[kAChunks];
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) xsum[i] = 0;
    auto load_tile = [&](int kt) {
        const uint32_t kc = min(kt * kTileK + a_col, K - 16);
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            const uint32_t row = min(r0 + (kThreads / 16) * i, r_last);
            ra[i] = *reinterpret_cast<const v4i*>(a_blk + (row * static_cast<uint32_t>(K) + kc));
        }
#pragma unroll
        for (int i = 0; i < kWTiles; ++i)
            rw[i] = __builtin_nontemporal_load(w_src[i] + static_cast<size_t>(kt) * 64);
    };
    auto store_tile = [&](int buf, int kt) {
        const bool real = kt * kTileK + a_col < K;
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            *reinterpret_cast<v4i*>(&a_lds[buf][(r0 + (kThreads / 16) * i) * kAPitch + a_col]) = ra[i];
            if (real)
                xsum[i] = dot4(ra[i].x, 0x01010101, dot4(ra[i].y, 0x01010101,
                               dot4(ra[i].z, 0x01010101, dot4(ra[i].w, 0x01010101, xsum[i]))));
        }
#pragma unroll
        for (int i = 0; i < kWTiles; ++i)
            if (w_has[i]) *reinterpret_cast<v4u*>(&w_lds[buf][w_dst[i]]) = rw[i];
    };

    v4i c[4][MTW];
#pragma unroll
    for (int tw = 0; tw < 4; ++tw)
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt) c[tw][mt] = v4i{0, 0, 0, 0};

    // operand read offsets within a buffer
    const int w_rd = (4 * wn) * kWTileWords + kWRowGroupWords * (j >> 2) + 4 * g + (j & 3);
    const int a_rd = (16 * MTW * wm + j) * kAPitch + 16 * g;
    // A step's operand reads and weight decode run at a raised wavefront
    // priority, its MFMAs at the normal one: of the two wavefronts on a
    // SIMD, the one still fetching and decoding is issued first, so its
    // MFMAs are ready while the other's run.  Same box, 13824 x 2560:
    // M = 256 17.1 -> 16.15 us, M = 512 25.5 -> 25.0 us (the MFMAs at the
    // raised priority instead: 16.15 / 25.2 us; raised in half of the
    // wavefronts only: 16.85 / 26.4 us).
    auto compute_tile = [&](int buf) {
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            v4i wa[4];
#pragma unroll
            for (int tw = 0; tw < 4; tw += 2)
                decode_w2(w_lds[buf][w_rd + tw * kWTileWords + 16 * st],
                          w_lds[buf][w_rd + (tw + 1) * kWTileWords + 16 * st], wa[tw], wa[tw + 1]);
            v4i xb[MTW];
#pragma unroll
            for (int mt = 0; mt < MTW; ++mt)
                xb[mt] = *reinterpret_cast<const v4i*>(&a_lds[buf][a_rd + 16 * mt * kAPitch + 64 * st]);
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int tw = 0; tw < 4; ++tw)
#pragma unroll
                for (int mt = 0; mt < MTW; ++mt)
                    c[tw][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa[tw], xb[mt], c[tw][mt], 0, 0, 0);
            __builtin_amdgcn_s_setprio(1);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    load_tile(0);
    store_tile(0, 0);
    __syncthreads();
    for (int kt = 0; kt < S256; ++kt) {
        if (kt + 1 < S256) load_tile(kt + 1);
        compute_tile(kt & 1);
        if (kt + 1 < S256) store_tile((kt + 1) & 1, kt + 1);
        __syncthreads();
    }
    // 2 * sum(x) of each activation row: the 16 threads of a row (lanes
    // 16q .. 16q + 15) add their sums with DPP inside the row of lanes; one
    // writes it to the first row of the (now idle) activation buffer
    int* twice_sum = reinterpret_cast<int*>(&a_lds[0][0]);
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
        int v = xsum[i];
        v += dpp_row<kDppQuadXor1>(v);
        v += dpp_row<kDppQuadXor2>(v);
        v += dpp_row<kDppRowRor4>(v);
        v += dpp_row<kDppRowRor8>(v);
        if ((tid & 15) == 0) twice_sum[r0 + (kThreads / 16) * i] = 2 * v;
    }
    __syncthreads();

    // Epilogue.  D layout with the weights as the A operand: lane (j, g),
    // register v -> weight row 4g + v of the band, activation row j of the
    // m tile: four consecutive outputs of one row, one 8-byte store.
    double wsd[4][4];
#pragma unroll
    for (int tw = 0; tw < 4; ++tw)
#pragma unroll
        for (int v = 0; v < 4; ++v) wsd[tw][v] = static_cast<double>(wsf[tw][v]);
    // 8-byte stores wherever four outputs fit: every group of a row when N is
    // a multiple of 4 and y is 8-byte aligned.  They write through the L2
    // (device-scope buffer stores, one descriptor per m tile, whose rows give
    // byte offsets below 2^29): the launch then ends without dirty output
    // lines to write back.  Same box: M = 256 16.19-16.23 -> 15.82-15.86 us,
    // M = 512 25.06-25.14 -> 24.47-24.52 us.
    constexpr int kStoreDeviceScope = 16;   // the sc1 bit of the store's cache policy
    const bool y_vec = (N % 4) == 0 && (reinterpret_cast<uintptr_t>(y) & 7) == 0;
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) {
        const int m_tile = m_base + 16 * (MTW * wm + mt);
        const int m = m_tile + j;
        const int tile_rows = max(0, min(16, M - m_tile));
        const __amdgpu_buffer_rsrc_t yt = __builtin_amdgcn_make_buffer_rsrc(
            y + static_cast<size_t>(min(m_tile, M)) * N, 0, tile_rows * N * 2, kRawBufferFlags);
        const double rs = 1.0 / static_cast<double>(sm[mt]);
#pragma unroll
        for (int tw = 0; tw < 4; ++tw) {
            const int n = n_base + 64 * wn + 16 * tw + 4 * g;
            const int off2 = twice_sum[16 * (MTW * wm + mt) + j];
            const int acc[4] = {c[tw][mt].x - off2, c[tw][mt].y - off2, c[tw][mt].z - off2,
                                c[tw][mt].w - off2};
            double cs[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) cs[v] = wsd[tw][v] * rs;
            // every lane takes part (the exact branch is wave-uniform); only
            // rows and columns inside the layer are stored
            const uint2 o = epilogue4(acc, wsf[tw], cs, sm[mt]);
            if (m >= M || n >= N) continue;
            const size_t off = static_cast<size_t>(m) * N + n;
            uint16_t* yo = y + off;
            if (y_vec && n + 4 <= N) {
                __builtin_amdgcn_raw_buffer_store_b64(v2u{o.x, o.y}, yt, 2 * (j * N + n), 0,
                                                      kStoreDeviceScope);
            } else {
                const uint32_t ov[4] = {o.x & 0xFFFFu, o.x >> 16, o.y & 0xFFFFu, o.y >> 16};
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (n + v < N) yo[v] = static_cast<uint16_t>(ov[v]);
            }
            if (acc_out) {
                int32_t* ao = acc_out + off;
                if (n + 4 <= N && (reinterpret_cast<uintptr_t>(ao) & 15) == 0) {
                    *reinterpret_cast<int4*>(ao) = int4{acc[0], acc[1], acc[2], acc[3]};
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        if (n + v < N) ao[v] = acc[v];
                }
            }
        }
    }
}

using PrefillFn = void (*)(const int8_t*, const v4u*, const float*, const uint16_t*, uint32_t, int,
                           uint16_t*, int32_t*, int, int, int);

struct PrefillShape {
    PrefillFn fn;
    int bn, bm, threads;
};

template <int WN, int WMW, int MTW>
constexpr PrefillShape prefill_shape() {
    return {&gemm_prefill_kernel<WN, WMW, MTW>, 64 * WN, 16 * MTW * WMW, 64 * WN * WMW};
}

// Largest tile first; the launch takes the first that still gives
// kPrefillMinGroups workgroups, else the last.
const std::array<PrefillShape, 4> kPrefillShapes = {{
    prefill_shape<4, 2, 4>(),   // 256 x 128
    prefill_shape<4, 2, 2>(),   // 256 x 64
    prefill_shape<2, 4, 1>(),   // 128 x 64
    prefill_shape<1, 4, 1>(),   //  64 x 64
}};
constexpr long kPrefillMinGroups = 200;

}  // namespace

hipError_t launch_gemm_prefill(const int8_t* xq, const uint8_t* packed, const float* s,
                               const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int M,
                               int N, int K, hipStream_t stream) {
    const PrefillShape* pick = &kPrefillShapes.back();
    for (const PrefillShape& p : kPrefillShapes) {
        const long groups = static_cast<long>((N + p.bn - 1) / p.bn) * ((M + p.bm - 1) / p.bm);
        if (groups >= kPrefillMinGroups) {
            pick = &p;
            break;
        }
    }
    const int gx = (N + pick->bn - 1) / pick->bn;
    const int gy = (M + pick->bm - 1) / pick->bm;
    const dim3 grid(static_cast<unsigned>((gx + 7) / 8 * 8 * gy));
    uint32_t seg_mul;
    int seg_shift;
    seg_divisor(N / ws_num, seg_mul, seg_shift);
    pick->fn<<<grid, pick->threads, 0, stream>>>(xq, reinterpret_cast<const v4u*>(packed), s, ws,
                                                 seg_mul, seg_shift, y, acc, M, N, K);
    return hipGetLastError();
}

}  // namespace bl
