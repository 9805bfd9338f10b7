// ternarize.hip -- ternarisation of a bf16 weight matrix by its mean absolute
// value, fused with packing into the 16x256-tile layout.
//
// Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
// (blog.gitcode.com), cited as [W2A8].  §4.2 quantises each projection matrix
// on its own: s = 1 / max(mean|W|, 1e-5), Wt = clamp(round(W * s), -1, 1),
// ws = 1 / s, as torch operations on bf16 tensors -- each computed in fp32 and
// rounded to bf16 (nearest, ties to even), which is the arithmetic here.
// mean|W| is the exact mean of the bf16 magnitudes, rounded once to bf16 (an
// fp32 running sum would depend on the order of the additions).  §5.2 then
// packs Wt as codes w + 2.
//
// Mapping:
//   * a bf16 magnitude is m * 2^(E' - 134) with E' = max(E, 1) and
//     m = f + 128 [E >= 1] (E the exponent field, f the fraction): a whole
//     number of units of 2^-133, so the sum of all magnitudes is an integer
//     number of such units -- computed exactly, hence the same in any order;
//   * absmean_hist_kernel accumulates that sum, exactly, as integer bins
//     H[p] of its bit positions (T = sum_p H[p] * 2^p in units of 2^-133):
//     per thread in fp64 when that is exact, else per weight; per workgroup
//     in LDS; then into 256 uint64 bins in the caller's workspace with
//     integer atomics (order-free);
//   * absmean_finalize_kernel assembles T as 32-bit limbs, divides it by
//     N*K 16 bits at a time, rounds the quotient once to bf16, and forms s
//     and ws;
//   * ternarize_pack_kernel: one thread per packed 32-bit word reads its 16
//     bf16 weights and writes the word, like the int8 packer.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace bl {

namespace {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kBins = 256;    // bit positions p of the magnitude sum T = sum_p H[p] * 2^p
constexpr int kLimbs = 12;    // 32-bit limbs of T (< 2^61 * 2^255 < 2^316)

// bf16 of a finite fp32 value, nearest, ties to even.
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ void zero_hist_kernel(unsigned long long* __restrict__ hist) {
    if (threadIdx.x < kBins) hist[threadIdx.x] = 0;
}

// All sums are in units of 2^-133, the spacing of the smallest bf16 values:
// a magnitude with exponent field E and fraction f is m * 2^(E' - 1) units,
// E' = max(E, 1), m = f + 128 [E >= 1].
//
// Each thread adds its n = 8 PER magnitudes (PER 16-byte chunks) in fp64.
// Each is a multiple of 2^(E'min - 1) units below 2^(E'max + 7), so in units
// of 2^(E'min - 1) the sum is below n * 2^(E'max - E'min + 8): the fp64 sum
// is exact when E'max - E'min <= 53 - 8 - ceil(log2 n) (38 for n = 128, 37
// for n = 192); the thread then adds its 53-bit mantissa, as three 18-bit
// pieces, into the bins of its bit positions.  A thread whose magnitudes span
// more binades adds them one by one (bin E' - 1).  Workgroup bins stay below
// 2^32 (256 threads * 2^18, or 48 Ki magnitudes * 255).  With finite
// magnitudes (below 2^128) a thread's sum is below 2^136, i.e. 2^269 units,
// so its pieces land in bins 0 .. 253.
constexpr int ceil_log2(int n) { return n <= 1 ? 0 : 1 + ceil_log2((n + 1) / 2); }
template <int PER>
__global__ __launch_bounds__(256) void absmean_hist_kernel(const uint4* __restrict__ w, size_t n8,
                                                           unsigned long long* __restrict__ hist) {
    constexpr int kPerThread = PER;
    constexpr size_t kHistItems = 256 * kPerThread;     // chunks per workgroup
    constexpr uint32_t kExactSpan = 53 - 8 - ceil_log2(8 * PER);
    static_assert(kExactSpan >= 1 && 256ull * 8 * PER * 255 < (1ull << 32), "bins and spans");
    __shared__ uint32_t h[kBins];
    h[threadIdx.x] = 0;
    __syncthreads();
    const size_t base = static_cast<size_t>(blockIdx.x) * kHistItems + threadIdx.x;
    // All loads first (clamped addresses; chunks past the end count as zero).
    uint4 v[kPerThread];
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
        v[j] = w[min(base + static_cast<size_t>(j) * 256, n8 - 1)];
    __builtin_amdgcn_sched_barrier(0);   // every load issued before the first use
    // Four partial sums, each at most the total: exact under the same bound.
    // The two magnitudes of a 32-bit word are handled as a pair of 16-bit
    // lanes: |w| for both, clamped to the largest finite bf16 (the weights
    // must be finite; this only keeps every sum finite), and the smallest
    // nonzero and the largest magnitude tracked with packed minima and
    // maxima -- the exponent bounds follow from them, since max(b >> 7, 1)
    // grows with b.  (b - 1, wrapping, takes a zero out of the minimum.)
    // The kernel went from 2321 to 1221 instructions; the ternariser (all
    // four kernels, 13824 x 2560) from 46.7 to 44.0-44.2 us, same box.
    double part[4] = {0.0, 0.0, 0.0, 0.0};
    us2 bmin1 = us2{0xFFFFu, 0xFFFFu};   // min of (b - 1) over the weights, per lane
    us2 bmax = us2{0u, 0u};
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const bool live = base + static_cast<size_t>(j) * 256 < n8;
        const uint32_t d[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t a = live ? (d[k] & 0x7FFF7FFFu) : 0u;
            const us2 b = __builtin_elementwise_min(__builtin_bit_cast(us2, a), us2{0x7F7Fu, 0x7F7Fu});
            bmin1 = __builtin_elementwise_min(bmin1, static_cast<us2>(b - us2{1u, 1u}));
            bmax = __builtin_elementwise_max(bmax, b);
            const uint32_t bb = __builtin_bit_cast(uint32_t, b);
            part[(2 * k) & 3] += static_cast<double>(__uint_as_float(bb << 16));
            part[(2 * k + 1) & 3] += static_cast<double>(__uint_as_float(bb & 0xFFFF0000u));
        }
    }
    const uint32_t bhi = max(static_cast<uint32_t>(bmax.x), static_cast<uint32_t>(bmax.y));
    const uint32_t blo = min(static_cast<uint32_t>(bmin1.x), static_cast<uint32_t>(bmin1.y)) + 1u;
    const uint32_t emin = bhi != 0 ? max(blo >> 7, 1u) : 255u;   // blo is then a nonzero magnitude
    const uint32_t emax = bhi != 0 ? max(bhi >> 7, 1u) : 0u;
    const double sum = (part[0] + part[1]) + (part[2] + part[3]);
    if (emax != 0 && emax - emin <= kExactSpan) {
        // sum = mant * 2^(ef - 1075); in units of 2^-133: mant * 2^(ef - 942)
        const unsigned long long bits = static_cast<unsigned long long>(__double_as_longlong(sum));
        unsigned long long mant = (bits & 0xFFFFFFFFFFFFFull) | (1ull << 52);
        int q = static_cast<int>(bits >> 52) - 942;
        if (q < 0) {            // the bits shifted out are zero: the sum is a whole number of units
            mant >>= -q;
            q = 0;
        }
        atomicAdd(&h[q], static_cast<uint32_t>(mant & 0x3FFFFu));
        atomicAdd(&h[q + 18], static_cast<uint32_t>((mant >> 18) & 0x3FFFFu));
        atomicAdd(&h[q + 36], static_cast<uint32_t>(mant >> 36));
    } else if (emax != 0) {
        for (int j = 0; j < kPerThread; ++j) {
            const size_t i = base + static_cast<size_t>(j) * 256;
            if (i >= n8) break;
            const uint4 v = w[i];
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t b = (d[k >> 1] >> (16 * (k & 1))) & 0x7FFFu;
                if (b != 0u && b < 0x7F80u) {
                    const uint32_t e = b >> 7;
                    atomicAdd(&h[max(e, 1u) - 1], (b & 0x7Fu) | (e ? 0x80u : 0u));
                }
            }
        }
    }
    __syncthreads();
    const uint32_t mine = h[threadIdx.x];
    if (mine) atomicAdd(&hist[threadIdx.x], static_cast<unsigned long long>(mine));
}

// Bits [lo, lo + 64) of the limbs Q (bits past the top read as 0); lo >= 0.
__device__ __forceinline__ unsigned long long bits_at(const uint32_t (&Q)[kLimbs], int lo) {
    unsigned long long out = 0;
#pragma unroll
    for (int k = 0; k < kLimbs; ++k) {
        const int off = 32 * k - lo;   // position of limb k's bit 0 in the result
        if (off >= 0 && off < 64)
            out |= static_cast<unsigned long long>(Q[k]) << off;
        else if (off < 0 && off > -32)
            out |= static_cast<unsigned long long>(Q[k] >> (-off));
    }
    return out;
}

// Whether any of bits [0, n) of Q is set.
__device__ __forceinline__ bool any_below(const uint32_t (&Q)[kLimbs], int n) {
    bool any = false;
#pragma unroll
    for (int k = 0; k < kLimbs; ++k) {
        const int keep = n - 32 * k;   // bits of limb k below n
        if (keep >= 32)
            any |= Q[k] != 0u;
        else if (keep > 0)
            any |= (Q[k] & ((1u << keep) - 1u)) != 0u;
    }
    return any;
}

// floor(R / count) for a quotient below 2^16 (R < 2^16 count, count < 2^45),
// exactly: the fp64 estimate R * fl(1/count) is within 2^-34 of the true
// quotient (relative error at most 3 * 2^-53 on a value below 2^16), so its
// truncation is off by at most one, which one integer step in each
// direction corrects.  About a quarter of the instructions of a 64-bit
// integer division, on the finalise's serial path.
__device__ __forceinline__ unsigned long long div_quot16(unsigned long long R,
                                                         unsigned long long count,
                                                         double inv_count) {
    unsigned long long q = static_cast<unsigned long long>(static_cast<double>(R) * inv_count);
    if (q * count > R) --q;
    if ((q + 1) * count <= R) ++q;
    return q;
}

// scales[0] = ws, scales[1] = s, scales[2] = mean|W| (bf16, before the 1e-5 floor).
__global__ __launch_bounds__(256) void absmean_finalize_kernel(
    const unsigned long long* __restrict__ hist, unsigned long long count,
    uint16_t* __restrict__ scales) {
    // T = sum_p hist[p] * 2^p as 64-bit sums of 32-bit pieces per limb
    // (at most 3 * 256 pieces per limb: no overflow).
    __shared__ unsigned long long acc[kLimbs];
    if (threadIdx.x < kLimbs) acc[threadIdx.x] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < kBins; p += blockDim.x) {
        const unsigned long long v = hist[p];   // < 2^61
        if (!v) continue;
        const int wi = p >> 5;
        const int b = p & 31;
        const unsigned long long lo = (v & 0xFFFFFFFFull) << b;   // < 2^63
        const unsigned long long hi = (v >> 32) << b;             // < 2^60
        atomicAdd(&acc[wi], lo & 0xFFFFFFFFull);
        atomicAdd(&acc[wi + 1], (lo >> 32) + (hi & 0xFFFFFFFFull));
        atomicAdd(&acc[wi + 2], hi >> 32);
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    uint32_t L[kLimbs];
    unsigned long long carry = 0;
#pragma unroll
    for (int k = 0; k < kLimbs; ++k) {
        const unsigned long long t = acc[k] + carry;
        L[k] = static_cast<uint32_t>(t);
        carry = t >> 32;
    }
    // Q = floor(T / count), R = T mod count, 16 bits at a time (R < count < 2^45).
    uint32_t Q[kLimbs];
    unsigned long long R = 0;
    const double inv_count = 1.0 / static_cast<double>(count);
#pragma unroll
    for (int k = kLimbs - 1; k >= 0; --k) {
        R = (R << 16) | (L[k] >> 16);
        const unsigned long long qh = div_quot16(R, count, inv_count);
        R -= qh * count;
        R = (R << 16) | (L[k] & 0xFFFFu);
        const unsigned long long ql = div_quot16(R, count, inv_count);
        R -= ql * count;
        Q[k] = static_cast<uint32_t>((qh << 16) | ql);
    }
    int p = -1;   // leading bit of Q
#pragma unroll
    for (int k = kLimbs - 1; k >= 0; --k)
        if (p < 0 && Q[k] != 0u) p = 32 * k + 31 - __clz(Q[k]);
    // mean = (Q + R/count) * 2^-133, leading bit 2^(p - 133): round to the
    // bf16 spacing 2^u, u = E - 7 for E >= -126, else -133.
    const int E = p - 133;
    const int u = (p >= 0 && E >= -126) ? E - 7 : -133;
    const int shift = u + 133;   // >= 0
    uint32_t r = static_cast<uint32_t>(bits_at(Q, shift) & 0x1FFu);
    bool up;
    if (shift == 0) {
        up = (2 * R > count) || (2 * R == count && (r & 1u));
    } else {
        const bool half = bits_at(Q, shift - 1) & 1u;
        const bool sticky = R != 0 || any_below(Q, shift - 1);
        up = half && (sticky || (r & 1u));
    }
    r += up ? 1u : 0u;
    uint32_t mean_bits = (static_cast<uint32_t>(shift) << 7) + r;
    if (mean_bits > 0x7F80u) mean_bits = 0x7F80u;
    float mean = __uint_as_float(mean_bits << 16);
    if (mean < 1e-5f) mean = __uint_as_float(bf16_bits_rne(1e-5f) << 16);
    const uint32_t s_bits = bf16_bits_rne(1.0f / mean);
    const uint32_t ws_bits = bf16_bits_rne(1.0f / __uint_as_float(s_bits << 16));
    scales[0] = static_cast<uint16_t>(ws_bits);
    scales[1] = static_cast<uint16_t>(s_bits);
    scales[2] = static_cast<uint16_t>(mean_bits);
}

// Code of one weight: clamp(round(bf16(w * s)), -1, 1) + 2.  |bf16(w * s)|
// above 0.5 rounds to a magnitude >= 1 (0.5 itself rounds to even 0).
__device__ __forceinline__ uint32_t ternary_code_bf16(uint32_t wbits, float s) {
    // fl32(w * s): exact (8 x 8 significant bits) unless it falls below the
    // normal range, where it is the IEEE product with denormals kept
    const float prod = __uint_as_float(wbits << 16) * s;
    const uint32_t t = bf16_bits_rne(prod) & 0x7FFFu;
    if (t <= 0x3F00u) return 2u;
    return (wbits & 0x8000u) ? 1u : 3u;
}

__device__ __forceinline__ int bit_of(int e) { return 8 * (e & 3) + 2 * (e >> 2); }

// One thread per packed word (the int8 packer's mapping): word u of tile t
// holds k = 256*(t % S) + 16*(q % 16) + e, e = 0..15, of row
// n = 16*(t / S) + 4*(q / 16) + u % 4, q = u / 4.  Rows and K past the
// matrix are padding (code 0).
__global__ __launch_bounds__(256) void ternarize_pack_kernel(const uint16_t* __restrict__ w,
                                                             uint32_t* __restrict__ packed,
                                                             const uint16_t* __restrict__ scales,
                                                             int N, int K, int S, size_t n_words) {
    const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n_words) return;
    const float s = __uint_as_float(static_cast<uint32_t>(scales[1]) << 16);
    const size_t t = i >> 8;
    const int u = static_cast<int>(i & 255);
    const int q = u >> 2;
    const int n = static_cast<int>(t / S) * kTileRows + 4 * (q >> 4) + (u & 3);
    const int k0 = static_cast<int>(t % S) * kTileK + 16 * (q & 15);
    uint32_t word = 0;
    if (n < N && k0 < K) {   // K % 16 == 0: all 16 weights are real
        const uint4* src = reinterpret_cast<const uint4*>(w + static_cast<size_t>(n) * K + k0);
        const uint4 a = src[0];
        const uint4 b = src[1];
        const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t wb = (d[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            word |= ternary_code_bf16(wb, s) << bit_of(e);
        }
    }
    packed[i] = word;
}

}  // namespace

hipError_t launch_ternarize(const uint16_t* w, uint8_t* packed, uint16_t* scales,
                            void* workspace, int N, int K, hipStream_t stream) {
    unsigned long long* hist = static_cast<unsigned long long*>(workspace);
    const size_t count = static_cast<size_t>(N) * K;
    const size_t n8 = count / 8;   // K % 16 == 0
    zero_hist_kernel<<<1, kBins, 0, stream>>>(hist);
    // 24 chunks per thread for large matrices (fewer workgroups, so fewer of
    // their bin additions contend on the same global bins: 13824 x 2560 44.2
    // -> 40.4 us, same box; 28, 32 and 40 chunks 41.7 / 41.5 / 45.3 us), 16
    // otherwise, so that small matrices still spread over the CUs.
    const uint4* w4 = reinterpret_cast<const uint4*>(w);
    constexpr size_t kLarge = 24 * 256;
    if (n8 >= kLarge * 512) {
        absmean_hist_kernel<24><<<static_cast<unsigned>((n8 + kLarge - 1) / kLarge), 256, 0, stream>>>(
            w4, n8, hist);
    } else {
        constexpr size_t kSmall = 16 * 256;
        absmean_hist_kernel<16><<<static_cast<unsigned>((n8 + kSmall - 1) / kSmall), 256, 0, stream>>>(
            w4, n8, hist);
    }
    absmean_finalize_kernel<<<1, 256, 0, stream>>>(hist, count, scales);
    const int S = (K + kTileK - 1) / kTileK;
    const size_t n_words = packed_bytes(N, K) / 4;
    ternarize_pack_kernel<<<static_cast<unsigned>((n_words + 255) / 256), 256, 0, stream>>>(
        w, reinterpret_cast<uint32_t*>(packed), scales, N, K, S, n_words);
    return hipGetLastError();
}

// The histogram of the allocation-free entry point, for callers that cannot
// allocate: one 2 KiB array per GPU, held by the library until the process
// ends.  Its 256 bins serve a matrix of any size.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): the address comes from hipGetSymbolAddress, once per device.
// Every call on a GPU shares that GPU's array; the first kernel of a call
// clears it, and calls that overlap on one GPU race.
static __device__ __align__(256) unsigned long long scratch[kBins];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_addr[kMaxDevices];
hipError_t scratch_status[kMaxDevices];

}  // namespace

hipError_t ternarize_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    // with device `dev` current: each GPU holds its own copy of the array
    std::call_once(scratch_once[dev], [dev] {
        void* p = nullptr;
        scratch_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        scratch_addr[dev] = p;
    });
    if (scratch_status[dev] != hipSuccess) return scratch_status[dev];
    if (scratch_addr[dev] == nullptr) return hipErrorInvalidSymbol;
    *out = scratch_addr[dev];
    return hipSuccess;
}

}  // namespace bl
