// gemv_norm.hip -- one projection of a decode step with the glue before it,
// in one kernel on gfx950.  Source page: "BitNet GPU 推理框架：从零构建 W2A8 的
// 2-bit 大模型 CUDA GEMV 内核" (blog.gitcode.com), cited as [W2A8].
#include <algorithm>
#include <array>
#include <utility>

#include "gemv_core.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

// ---------------------------------------------------------------------------
// The projection of a decode step with its glue ([W2A8] §4.1 names the
// model's norms attention_norm / ffn_norm / attn_sub_norm / ffn_sub_norm and
// its fused projections wqkv / wo / w13 / w2; the formulas are readings):
//   m  = x, or bf16(max(x, 0)^2 * x_up) for the MLP's down projection
//        (x = the gate half and x_up = the up half of w13's output);
//   xn = bf16( fl64(m * gamma) * fl64(1 / sqrt(sum(m^2) / K + eps)) );
//   per-token absmax int8 quantisation of xn, the ternary layer, and
//   y = bf16(acc * ws / s), or bf16(residual + that) when a residual is given.
// The glue runs in the prologue of every workgroup (the row is at most a few
// thousand elements, read from L2 by each): no kernel of its own, so a chained
// decode step launches one kernel per projection.  In a graph, the MLP's
// activation and the two statistics of down's RMSNorm (the sum of m^2 and the
// largest |m * gamma|) are instead computed once, in the epilogue of the
// gate+up kernel whose output they come from, and handed to down as a row and
// per-workgroup partials (NormLink; MODE kNormLinked on the consumer's side).
// Everything else is the staged GEMV of gemv.hip (its pieces in
// gemv_core.hpp): the weight loads are all issued before the first wait.
// ---------------------------------------------------------------------------

constexpr int kDppRowBcast15 = 0x142;   // each lane of row r <- lane 15 of row r - 1 (r >= 1)

// Sum of a double over the 64 lanes: the two 32-bit halves move together
// through the DPP steps of wave_sum (pairs, quads, rotations by 4 and 8 inside
// each row of 16), then the four row totals are read out and added.  The
// result is the same in every lane.
template <int CTRL>
__device__ __forceinline__ double dpp_row_f64(double v) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
}
// The sum over each row of 16 lanes, in every lane of the row.
__device__ __forceinline__ double row_sum_f64(double v) {
    v += dpp_row_f64<kDppQuadXor1>(v);
    v += dpp_row_f64<kDppQuadXor2>(v);
    v += dpp_row_f64<kDppRowRor4>(v);
    v += dpp_row_f64<kDppRowRor8>(v);
    return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
    v = row_sum_f64(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Unsigned maximum over the 64 lanes, by the same steps.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_row_u32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
    v = max(v, dpp_row_u32<kDppQuadXor1>(v));
    v = max(v, dpp_row_u32<kDppQuadXor2>(v));
    v = max(v, dpp_row_u32<kDppRowRor4>(v));
    v = max(v, dpp_row_u32<kDppRowRor8>(v));
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = row_max_u32(v);
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ uint32_t bf16_lo(uint32_t w) { return w & 0xFFFFu; }
__device__ __forceinline__ uint32_t bf16_hi(uint32_t w) { return w >> 16; }
__device__ __forceinline__ double bf16_f64(uint32_t b) {
    return static_cast<double>(__uint_as_float(b << 16));
}

// Eight fp64 values to bf16 (nearest, ties to even) by way of fp32: one
// conversion to fp32, one to bf16.  Every bf16 midpoint is an fp32 number,
// so the first rounding can land on one but never step across one: the two
// roundings differ from one direct rounding only where the fp32 value is a
// bf16 midpoint (low 16 bits 0x8000).  Such chunks, and NaN, are rounded
// again by bf16_rne_f64.
__device__ __forceinline__ uint4 bf16x8_from_f64(const double (&d)[8]) {
    uint32_t o[4];
    uint64_t redo = 0;   // lanes that need it, one ballot per compare
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float f0 = static_cast<float>(d[2 * j]), f1 = static_cast<float>(d[2 * j + 1]);
        redo |= __builtin_amdgcn_ballot_w64((__float_as_uint(f0) & 0xFFFFu) == 0x8000u);
        redo |= __builtin_amdgcn_ballot_w64((__float_as_uint(f1) & 0xFFFFu) == 0x8000u);
        redo |= __builtin_amdgcn_ballot_w64(__builtin_isunordered(f0, f1));
        o[j] = cvt_pk_bf16(f0, f1);
    }
    // a wave-uniform branch, taken by a wavefront when any of its lanes needs
    // it (rarely); the empty volatile statement keeps the compiler from
    // if-converting it, which would pay its work on every chunk
    if (__builtin_expect(redo != 0, 0)) {
        asm volatile("");
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = bf16_rne_f64(d[2 * j]) | (bf16_rne_f64(d[2 * j + 1]) << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Chunk of 8 bf16: relu2-GLU, exact in fp64 (at most 24 significant bits),
// rounded once, into m.
__device__ __forceinline__ uint4 glu8(const uint4& g, const uint4& u) {
    const uint32_t gd[4] = {g.x, g.y, g.z, g.w};
    const uint32_t ud[4] = {u.x, u.y, u.z, u.w};
    double m[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float a0 = __uint_as_float(gd[j] << 16), a1 = __uint_as_float(gd[j] & 0xFFFF0000u);
        const double g0 = a0 > 0.0f ? static_cast<double>(a0) : 0.0;
        const double g1 = a1 > 0.0f ? static_cast<double>(a1) : 0.0;
        m[2 * j] = g0 * g0 * bf16_f64(bf16_lo(ud[j]));
        m[2 * j + 1] = g1 * g1 * bf16_f64(bf16_hi(ud[j]));
    }
    return bf16x8_from_f64(m);
}

// p = m * gamma (exact in fp64) for a chunk of 8, with the running sum of
// m^2 and the running maximum of |p| as the high word of its encoding: p has
// at most 16 significant bits, all in that word (the low word is zero), so
// comparing high words of magnitudes as integers compares the magnitudes.
__device__ __forceinline__ void products8(const uint4& m, const uint4& g, double (&p)[8],
                                          double& ssq, uint32_t& pm) {
    const uint32_t md[4] = {m.x, m.y, m.z, m.w};
    const uint32_t gd[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const double a = bf16_f64(bf16_lo(md[j])), b = bf16_f64(bf16_hi(md[j]));
        p[2 * j] = a * bf16_f64(bf16_lo(gd[j]));
        p[2 * j + 1] = b * bf16_f64(bf16_hi(gd[j]));
        ssq += a * a;
        ssq += b * b;
        pm = max(pm, max(static_cast<uint32_t>(__double2hiint(p[2 * j])) & 0x7FFFFFFFu,
                         static_cast<uint32_t>(__double2hiint(p[2 * j + 1])) & 0x7FFFFFFFu));
    }
}

// xn = bf16(p * inv) for a chunk of 8 (NaN where inv is infinite and p zero:
// a zero row with eps = 0).
__device__ __forceinline__ uint4 norm8(const double (&p)[8], double inv) {
    double v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = p[e] * inv;
    return bf16x8_from_f64(v);
}

__device__ __forceinline__ uint4 to_uint4(v4u v) { return make_uint4(v.x, v.y, v.z, v.w); }

// A row of K bf16 values as a raw buffer (16-byte loads by chunk index).
using RowBuf = __amdgpu_buffer_rsrc_t;
constexpr int kRawBufferFlags = 0x00020000;   // word 3 of the descriptor: 32-bit data format
__device__ __forceinline__ RowBuf row_buffer(const uint16_t* p, int K) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, 2 * K, kRawBufferFlags);
}
__device__ __forceinline__ uint4 row_load(RowBuf r, int chunk) {
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, chunk * 16, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// At most kNormMaxWaves wavefronts per workgroup: the registers that hold
// the row's exact products (two per value) need the larger per-wavefront
// budget.
constexpr int kNormMaxWaves = 8;

// What the prologue starts from: the row x itself, the relu2-GLU of x and
// x_up, or a row m handed off by the previous projection with its
// statistics (NormLink).
enum : int { kNormPlain = 0, kNormGlu = 1, kNormLinked = 2 };

// One workgroup's bands of one projection: the body of the single-call kernel
// (group = its block index) and of the grouped kernel (group = the index in
// its work record).  The pointers are cast to the global address space: the
// grouped kernel reads them from memory, not from its kernel arguments.
template <int P, int C, int MODE>
__device__ __forceinline__ void norm_body(const NormArgs& a, const NormLink& l, int group) {
    constexpr bool GLU = MODE == kNormGlu;
    constexpr bool LINKED = MODE == kNormLinked;
    extern __shared__ int4 act[];   // Wb*P*16 16-byte chunks: the int8 row, zero-padded
    __shared__ int part_sh[kNormMaxWaves][64];
    __shared__ int xsum_sh[kNormMaxWaves];
    __shared__ double ssq_sh[kNormMaxWaves];
    __shared__ uint32_t pm_sh[kNormMaxWaves];
    const int N = a.N;
    const int K = a.K;
    const int B = a.B;
    const int lw = a.lw;
    const int Wb = 1 << lw;
    const int W = B << lw;
    const int nthreads = W * 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nbands = (N + kTileRows - 1) / kTileRows;
    // The workgroup's j-th band: the next B bands, or, for a projection that
    // hands the GLU off, B / 2 gate bands and the up bands of the same rows.
    // Arithmetic, not branches: a branch here splits the reads of the kernel
    // arguments into rounds, each waiting for the last, before any load
    // (the chained step: 461.5 -> 456.0 us).
    const int hb = l.half >> 4;   // the first up band (0: no hand-off)
    const int hB = B >> 1;
    const int pair = hb != 0;
    const int per_half = pair ? hB : B;
    auto band_at = [&](int j) { return group * per_half + j + (pair & (j >= hB)) * (hb - hB); };
    const int band = min(band_at(wave >> lw), nbands - 1);
    const int S = (K + kTileK - 1) / kTileK;
    const int s0 = (wave & (Wb - 1)) * P;
    const int n16 = K >> 4;
    const int padded16 = Wb * P * 16;
    const int n_in = K >> 3;        // 16-byte chunks of bf16

    // 1. The inputs of this thread's output row (weight scale, residual),
    //    the cached chunks of the row (x, x_up, gamma), then every weight load.
    const int n_out = band_at(min(tid >> 4, B - 1)) * kTileRows + (tid & 15);   // tid < 16*B writes
    const uint32_t n_c = static_cast<uint32_t>(min(n_out, N - 1));
    const uint16_t wsb = global(a.ws)[(static_cast<uint64_t>(n_c) * a.seg_mul) >> a.seg_shift];
    // unconditional (a branch would end in a wait for this load); the weight
    // scales stand in as a source when there is no residual, and when there
    // is no hand-off for the next projection's gamma at this lane's gate row
    const uint16_t resb = global(a.residual ? a.residual : a.ws)[a.residual ? n_c : 0u];
    const uint16_t gnb = global(l.m_out ? l.gamma_next : a.ws)[
        l.m_out ? static_cast<uint32_t>(min(n_out, l.half - 1)) : 0u];
    // The hand-off's partials (a consumer): four 16-byte loads per lane, the
    // ones past n_part reading as zeros (the buffer's range check).
    v4u part[LINKED ? kNormMaxParts / 64 : 1];
    if constexpr (LINKED) {
        const RowBuf rp = __builtin_amdgcn_make_buffer_rsrc(const_cast<NormPart*>(l.part_in), 0,
                                                            16 * l.n_part, kRawBufferFlags);
#pragma unroll
        for (int k = 0; k < kNormMaxParts / 64; ++k)
            part[k] = __builtin_amdgcn_raw_buffer_load_b128(rp, (lane + 64 * k) * 16, 0, 0);
    }
    const global_ptr<const v4u> x16 = global(reinterpret_cast<const v4u*>(a.x));
    const global_ptr<const v4u> u16 = global(reinterpret_cast<const v4u*>(a.x_up));
    const global_ptr<const v4u> g16 = global(reinterpret_cast<const v4u*>(a.gamma));
    // The cached chunks come through buffer loads: the compiler treats plain
    // loads of these read-only rows as free to sink to their first use,
    // past the weight loads, and a wait there would wait for every one.
    const RowBuf rx = row_buffer(a.x, K), ru = row_buffer(a.x_up, K), rg = row_buffer(a.gamma, K);
    // A chunk past the row's end reads as zeros (the buffer's range check),
    // which add nothing to the sum of squares or the maximum.
    uint4 xv[C], uv[GLU ? C : 1], gv[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int idx = tid + c * nthreads;
        xv[c] = row_load(rx, idx);
        if constexpr (GLU) uv[c] = row_load(ru, idx);
        gv[c] = row_load(rg, idx);
    }
    // Every wavefront's row loads go out before any wavefront's weight loads
    // (a barrier without a wait: the loads are issued, not complete): the
    // glue needs the rows first, and the weights only for the dot products
    // after it.  Same box, the chained step: 492.8 -> 487.1 us.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const global_ptr<const v4u> tiles =
        global(reinterpret_cast<const v4u*>(a.packed)) + static_cast<size_t>(band) * S * 64 + lane;
    v4u w[P];
    load_steps<P>(tiles, s0, S - 1, w);
    // No load may move below this point (a row load sunk past the weight
    // loads would wait for all of them: the waits count loads in issue
    // order), and nothing may be scheduled above it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // 2. m (GLU); p = m * gamma, exact in fp64 and kept for step 4; the sum
    //    of m^2 and the largest |p|.  Chunks beyond the C cached ones (rows
    //    longer than C x 8 x threads) are re-read from L2, here and in step 4.
    auto m_chunk = [&](int c, int idx) -> uint4 {
        if (c < C) {
            if constexpr (GLU) return glu8(xv[c], uv[c]);
            return xv[c];
        }
        if constexpr (GLU) return glu8(to_uint4(x16[idx]), to_uint4(u16[idx]));
        return to_uint4(x16[idx]);
    };
    double ssq = 0.0;
    uint32_t pm = 0;   // high word of the largest |p|
    double pv[C][8];
#pragma unroll
    for (int c = 0; c < C; ++c) products8(m_chunk(c, tid + c * nthreads), gv[c], pv[c], ssq, pm);

    // 3. The inverse RMS and the activation scale.  Rounding is monotone and
    //    inv > 0, so the largest |xn| is the bf16 rounding of pmax * inv: the
    //    absmax needs no pass over xn.
    double total_sq = 0.0;
    if constexpr (LINKED) {
        // From the producer's partials, added in the same order by every
        // wavefront (each lane's four in turn, then across the lanes): no
        // barrier and no pass over the row.
        double sp = 0.0;
        uint32_t up = 0;
#pragma unroll
        for (int k = 0; k < kNormMaxParts / 64; ++k) {
            sp += __hiloint2double(static_cast<int>(part[k].y), static_cast<int>(part[k].x));
            up = max(up, part[k].z);
        }
        total_sq = wave_sum_f64(sp);
        pm = wave_max_u32(up);
    } else {
        for (int idx = tid + C * nthreads; idx < n_in; idx += nthreads) {
            double pt[8];
            products8(m_chunk(C, idx), to_uint4(g16[idx]), pt, ssq, pm);
        }
        ssq = wave_sum_f64(ssq);
        pm = wave_max_u32(pm);
        if (lane == 0) {
            ssq_sh[wave] = ssq;
            pm_sh[wave] = pm;
        }
        __syncthreads();
        // The wavefronts' partial sums are added in wave order; all eight
        // slots are read at once and the unused ones dropped.
        pm = 0;
#pragma unroll
        for (int i = 0; i < kNormMaxWaves; ++i) {
            const double v = ssq_sh[i];
            const uint32_t u = pm_sh[i];
            total_sq += i < W ? v : 0.0;
            pm = max(pm, i < W ? u : 0u);
        }
    }
    const double inv = 1.0 / sqrt(total_sq / static_cast<double>(K) + a.eps);
    const double pmax = __hiloint2double(static_cast<int>(pm), 0);
    const float amax = __uint_as_float(bf16_rne_f64(pmax * inv) << 16);
    const float sm = 127.0f / fmaxf(amax, 1e-5f);

    // 4. Quantise xn into LDS (workgroup 0 also writes xn, q and s when asked).
    uint2* act8 = reinterpret_cast<uint2*>(act);
    const bool first = group == 0;
    int xs = 0;
    auto put = [&](int idx, const uint4& v) {
        const uint2 o = quant8_bf16(v, sm);
        act8[idx] = o;
        xs = sum_i8x4(o.x, sum_i8x4(o.y, xs));
        if (first && a.q_out) global(reinterpret_cast<v2u*>(a.q_out))[idx] = v2u{o.x, o.y};
        if (first && a.xn_out) global(reinterpret_cast<v4u*>(a.xn_out))[idx] = v4u{v.x, v.y, v.z, v.w};
    };
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int idx = tid + c * nthreads;
        if (idx < n_in) put(idx, norm8(pv[c], inv));
    }
    for (int idx = tid + C * nthreads; idx < n_in; idx += nthreads) {
        double pt[8];
        products8(m_chunk(C, idx), to_uint4(g16[idx]), pt, ssq, pm);
        put(idx, norm8(pt, inv));
    }
    if (first && a.s_out != nullptr && tid == 0) global(a.s_out)[0] = sm;
    for (int i = n16 + tid; i < padded16; i += nthreads) act[i] = make_int4(0, 0, 0, 0);
    xs = wave_sum(xs);
    if (lane == 0) xsum_sh[wave] = xs;
    __syncthreads();
    double cs = 0.0;
    int offset = 0;
    if (wave == 0) {
        cs = static_cast<double>(bf16_to_float(wsb)) * (1.0 / static_cast<double>(sm));
        for (int i = 0; i < W; ++i) offset -= 2 * xsum_sh[i];
        asm volatile("" : "+v"(cs), "+v"(offset));
    }

    // 5. P steps of 4 rows x 16 K per lane, reduction, epilogue (+ residual).
    RowAcc r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.a1[i] = r.a4[i] = r.a16[i] = 0;
    const int kc = lane & 15;
#pragma unroll
    for (int u = 0; u < P; ++u) dot_slot(w[u], act[(s0 + u) * 16 + kc], r);
    int v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = r.a1[i] + (r.a4[i] >> 2) + (r.a16[i] >> 4);
    part_sh[wave][lane] = row_group_reduce(v, lane);
    __syncthreads();
    if (wave == 0) {
        const int bw = lane >> 4;
        const int rw = lane & 15;
        const int slot = 16 * (rw >> 2) + (rw & 3);
        const int firstw = min(bw, B - 1) << lw;
        int total = offset;
        for (int j = 0; j < Wb; ++j) total += part_sh[firstw + j][slot];
        uint32_t o = 0;
        if (bw < B && n_out < N) {
            o = epilogue_bf16_scaled(total, cs, bf16_to_float(wsb), sm);
            if (a.residual)   // the fp64 sum of two bf16 values rounds to bf16 as the exact sum does
                o = bf16_rne_f64(static_cast<double>(bf16_to_float(static_cast<uint16_t>(resb))) +
                                 static_cast<double>(bf16_to_float(static_cast<uint16_t>(o))));
            global(a.y)[n_out] = static_cast<uint16_t>(o);
            if (a.acc) global(a.acc)[n_out] = total;
        }
        if (l.m_out != nullptr) {
            // The hand-off: lanes 0 .. 8B-1 hold gate rows, lanes 8B .. 16B-1
            // the up rows of the same index.  m = bf16(max(gate, 0)^2 * up),
            // exact in fp64 before the rounding; then the workgroup's sum of
            // m^2 and largest |m * gamma_next| (both exact per value in fp64),
            // as the consumer's prologue would have computed them.  This is
            // the end of the kernel's critical path, so it stays in vector
            // registers: the up values come over by a lane swap (the upper
            // half of the wavefront for B = 4, the odd rows for B = 2), and
            // the totals by row reductions, row 0's added into row 1 for
            // B = 4, stored by a lane that holds them.  Same box, the chained
            // step: 454.0-454.6 -> 452.6-454.4 us.
            const int hl = 8 * B;
            const uint32_t ub =
                hl == 32 ? __builtin_amdgcn_permlane32_swap(o, o, false, false)[1]
                         : __builtin_amdgcn_permlane16_swap(o, o, false, false)[1];
            double sq = 0.0;
            uint32_t pmv = 0;
            if (lane < hl) {
                const double g = bf16_f64(o);
                const double gr = g > 0.0 ? g : 0.0;
                const uint32_t mb = bf16_rne_f64(gr * gr * bf16_f64(ub));
                global(l.m_out)[n_out] = static_cast<uint16_t>(mb);
                const double m = bf16_f64(mb);
                sq = m * m;
                pmv = static_cast<uint32_t>(__double2hiint(m * bf16_f64(gnb))) & 0x7FFFFFFFu;
            }
            sq = row_sum_f64(sq);
            pmv = row_max_u32(pmv);
            if (hl == 32) {
                sq += dpp_row_f64<kDppRowBcast15>(sq);
                pmv = max(pmv, dpp_row_u32<kDppRowBcast15>(pmv));
            }
            if (lane == hl - 16)
                global(reinterpret_cast<v4u*>(l.part_out))[group] =
                    v4u{static_cast<uint32_t>(__double2loint(sq)),
                        static_cast<uint32_t>(__double2hiint(sq)), pmv, 0u};
        }
    }
}

template <int P, int C, int MODE>
__global__ __launch_bounds__(kNormMaxWaves * 64) void gemv_norm_kernel(NormArgs a, NormLink l) {
    // (the arguments' loads go out together, as in the grouped kernel below)
    const NormArgs ac = a;
    const NormLink lc = l;
    __builtin_amdgcn_sched_barrier(0);
    norm_body<P, C, MODE>(ac, lc, static_cast<int>(blockIdx.x));
}

// Several projections of one kernel instance in one launch: workgroup i runs
// the bands of work record i (its projection's arguments and its group).
// No hand-off here.
template <int P, int C, int MODE>
__global__ __launch_bounds__(kNormMaxWaves * 64) void gemv_norm_group_kernel(
    const NormWork* __restrict__ work) {
    // The record's fields are read before anything else is scheduled, so
    // that their loads go out together (the scheduler could otherwise leave
    // some behind a wait for the others, and every row and weight load
    // would then wait for both rounds).
    const NormWork& w = work[blockIdx.x];
    const NormArgs a = w.a;
    const int group = w.group;
    __builtin_amdgcn_sched_barrier(0);
    norm_body<P, C, MODE>(a, NormLink{}, group);
}

using GemvNormFn = void (*)(NormArgs, NormLink);
using GemvNormGroupFn = void (*)(const NormWork*);
template <int C, int MODE, int... Ps>
constexpr std::array<GemvNormFn, sizeof...(Ps)> norm_table(std::integer_sequence<int, Ps...>) {
    return {{&gemv_norm_kernel<Ps + 1, C, MODE>...}};
}
template <int C, int MODE, int... Ps>
constexpr std::array<GemvNormGroupFn, sizeof...(Ps)> norm_group_table(
    std::integer_sequence<int, Ps...>) {
    return {{&gemv_norm_group_kernel<Ps + 1, C, MODE>...}};
}
// P = 1 .. kNormMaxSteps (rows up to kNormMaxK over at most kNormMaxWaves
// wavefronts per band) and C = 1 or 2 cached chunks per thread; the loop over
// uncached chunks serves longer rows.
constexpr int kNormMaxSteps = 16;
using NormRow = std::array<GemvNormFn, kNormMaxSteps>;
using NormGroupRow = std::array<GemvNormGroupFn, kNormMaxSteps>;
template <int MODE>
constexpr std::array<NormRow, 2> norm_rows() {
    return {{norm_table<1, MODE>(std::make_integer_sequence<int, kNormMaxSteps>{}),
             norm_table<2, MODE>(std::make_integer_sequence<int, kNormMaxSteps>{})}};
}
template <int MODE>
constexpr std::array<NormGroupRow, 2> norm_group_rows() {
    return {{norm_group_table<1, MODE>(std::make_integer_sequence<int, kNormMaxSteps>{}),
             norm_group_table<2, MODE>(std::make_integer_sequence<int, kNormMaxSteps>{})}};
}
// [mode][C - 1][P - 1]
const std::array<std::array<NormRow, 2>, 3> kNormKernels = {
    {norm_rows<kNormPlain>(), norm_rows<kNormGlu>(), norm_rows<kNormLinked>()}};
const std::array<std::array<NormGroupRow, 2>, 2> kNormGroupKernels = {
    {norm_group_rows<kNormPlain>(), norm_group_rows<kNormGlu>()}};

// The geometry of gemv_shape with at most kNormMaxWaves wavefronts per
// workgroup, and its own two constants, measured on the chained decode step.
// Every workgroup redoes the glue over the whole row, so fewer, wider
// workgroups share it:
//  - runs of up to 5 steps per wavefront, whatever the width (the GEMV:
//    10, or 4 below 400 bands).  gate+up takes two wavefronts per band
//    (457.2-457.9 -> 453.2-454.8 us per step, same box; with 3 steps, 432
//    workgroups: 538 us, and too many workgroups for the hand-off to down),
//    qkv and o two per band instead of four (424.3-425.8 -> 420.6-421.4 us;
//    down keeps eight: with four, two bands per workgroup, 447 us);
//  - bands per workgroup kept down to 80 workgroups (the GEMV: 200).  qkv
//    and o take two bands per workgroup, 120 + 80 workgroups instead of
//    240 + 160 (452.1-453.8 -> 423.1-424.5 us; four bands, 60 + 40
//    workgroups of eight wavefronts, 430 us).
constexpr int kNormTargetSteps = 5;
constexpr int kNormMinGroups = 80;

GemvShape norm_shape(int N, int K) {
    const int S = (K + kTileK - 1) / kTileK;
    const int nbands = (N + kTileRows - 1) / kTileRows;
    int Wb = 1;
    while (Wb < kNormMaxWaves && (S + Wb - 1) / Wb > kNormTargetSteps) Wb <<= 1;
    const int P = (S + Wb - 1) / Wb;
    if (P > kNormMaxSteps) return GemvShape{0, 0, 0};
    int B = 4;
    while (B > 1 && (nbands / B < kNormMinGroups || B * Wb > kNormMaxWaves)) B >>= 1;
    return GemvShape{B * Wb, P, B};
}

}  // namespace

NormPlan norm_plan(const uint16_t* x, const uint16_t* x_up, const uint16_t* gamma, float eps,
                   const uint8_t* packed, const uint16_t* ws, int ws_num,
                   const uint16_t* residual, uint16_t* y, uint16_t* xn_out, int8_t* q_out,
                   float* s_out, int32_t* acc, int N, int K) {
    NormPlan p{};
    const GemvShape g = norm_shape(N, K);
    if (g.waves == 0 || K > kNormMaxK) return p;
    const int nbands = (N + kTileRows - 1) / kTileRows;
    p.groups = (nbands + g.bands - 1) / g.bands;
    const int wb = g.waves / g.bands;
    int lw = 0;
    while ((1 << lw) < wb) ++lw;
    p.lds = static_cast<size_t>(wb) * g.steps * kTileK;
    p.threads = g.waves * 64;
    const int need = (K / 8 + p.threads - 1) / p.threads;
    p.glu = x_up != nullptr;
    p.cached = need <= 1 ? 1 : 2;
    p.steps = g.steps;
    uint32_t seg_mul;
    int seg_shift;
    seg_divisor(N / ws_num, seg_mul, seg_shift);
    p.args = NormArgs{x, x_up, gamma, reinterpret_cast<const v4u*>(packed), ws, residual, y, acc,
                      q_out, s_out, xn_out, static_cast<double>(eps), seg_mul, seg_shift, N, K,
                      g.bands, lw};
    return p;
}

bool norm_link_supported(const NormPlan& p, int half) {
    // whole bands in each half, the same number of gate bands per workgroup
    // in both, and at most kNormMaxParts workgroups
    const int B = p.args.B;
    return p.groups > 0 && p.groups <= kNormMaxParts && half > 0 && p.args.N == 2 * half &&
           half % kTileRows == 0 && B % 2 == 0 && (half / kTileRows) % (B / 2) == 0;
}

hipError_t launch_gemv_norm_plan(const NormPlan& p, const NormLink& link, hipStream_t stream) {
    if (p.groups == 0) return hipErrorInvalidValue;
    if (link.m_out && !norm_link_supported(p, link.half)) return hipErrorInvalidValue;
    if (link.part_in && (p.glu || link.n_part < 1 || link.n_part > kNormMaxParts))
        return hipErrorInvalidValue;
    const int mode = link.part_in ? kNormLinked : p.glu ? kNormGlu : kNormPlain;
    const GemvNormFn fn = kNormKernels[mode][p.cached - 1][p.steps - 1];
    fn<<<static_cast<unsigned>(p.groups), p.threads, p.lds, stream>>>(p.args, link);
    return hipGetLastError();
}

hipError_t launch_gemv_norm(const uint16_t* x, const uint16_t* x_up, const uint16_t* gamma,
                            float eps, const uint8_t* packed, const uint16_t* ws, int ws_num,
                            const uint16_t* residual, uint16_t* y, uint16_t* xn_out,
                            int8_t* q_out, float* s_out, int32_t* acc, int N, int K,
                            hipStream_t stream) {
    const NormPlan p = norm_plan(x, x_up, gamma, eps, packed, ws, ws_num, residual, y, xn_out,
                                 q_out, s_out, acc, N, K);
    return launch_gemv_norm_plan(p, NormLink{}, stream);
}

hipError_t launch_gemv_norm_group(const NormPlan& key, const NormWork* work, int n_work,
                                  size_t lds, hipStream_t stream) {
    const GemvNormGroupFn fn =
        kNormGroupKernels[key.glu ? kNormGlu : kNormPlain][key.cached - 1][key.steps - 1];
    fn<<<static_cast<unsigned>(n_work), key.threads, lds, stream>>>(work);
    return hipGetLastError();
}

}  // namespace bl
