// stream_floor.hip -- measurement aid for the benchmark, not part of the layer.
//
// Two kernels with the launch shape of the M = 1 GEMV (workgroups of B
// 16-row bands, Wb wavefronts per band, P 16-byte loads per lane), doing none
// of its work:
//   stream_floor_empty  launches the grid and exits: the fixed cost of a launch;
//   stream_floor_read   reads the same packed bytes with the same per-lane
//                       non-temporal 16-byte loads and folds them into one
//                       value per lane (written only if it equals a sentinel,
//                       so the loads cannot be dropped): the floor a streaming
//                       kernel of this size and shape reaches on the machine.
// Built into libstream_floor.so, separate from libbitlinear.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

namespace {

__global__ void empty_kernel(uint32_t* out) {
    if (threadIdx.x == 0xFFFFFFFFu) out[0] = 0;   // never true; keeps the argument
}

template <int P>
__global__ __launch_bounds__(1024) void read_kernel(const v4u* __restrict__ tiles_base, int nbands,
                                                    int S, int B, uint32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int Wb = (blockDim.x >> 6) / B;
    const int band = min(static_cast<int>(blockIdx.x) * B + wave / Wb, nbands - 1);
    const v4u* tiles = tiles_base + static_cast<size_t>(band) * S * 64 + lane;
    v4u acc = {0, 0, 0, 0};
    v4u w[P];
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int st = min((wave % Wb) * P + u, S - 1);
        w[u] = __builtin_nontemporal_load(tiles + static_cast<size_t>(st) * 64);
    }
#pragma unroll
    for (int u = 0; u < P; ++u) acc ^= w[u];
    const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (r == 0x9E3779B9u) out[blockIdx.x] = r;
}

template <int P>
hipError_t launch_read(const void* packed, int nbands, int S, int B, int waves, uint32_t* out,
                       hipStream_t stream) {
    const int groups = (nbands + B - 1) / B;
    read_kernel<P><<<groups, waves * 64, 0, stream>>>(static_cast<const v4u*>(packed), nbands, S,
                                                      B, out);
    return hipGetLastError();
}

}  // namespace

extern "C" {

// out: device, >= 1 uint32 (never written in practice).
int stream_floor_empty(int groups, int waves, uint32_t* out, hipStream_t stream) {
    if (groups < 1 || waves < 1 || waves > 16 || !out) return -1;
    empty_kernel<<<groups, waves * 64, 0, stream>>>(out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// packed: device, nbands * S * 1024 bytes; out: device, >= ceil(nbands / B) uint32.
// B bands per workgroup, waves = B * Wb, steps = P per wavefront with Wb * P >= S;
// P in {1..10, 12, 14, 16, 18, 20}.
int stream_floor_read(const void* packed, int nbands, int S, int B, int waves, int steps,
                      uint32_t* out, hipStream_t stream) {
    if (!packed || !out || nbands < 1 || S < 1 || B < 1 || waves < B || waves > 16 ||
        waves % B != 0 || (waves / B) * steps < S)
        return -1;
    hipError_t e;
    switch (steps) {
        case 1: e = launch_read<1>(packed, nbands, S, B, waves, out, stream); break;
        case 2: e = launch_read<2>(packed, nbands, S, B, waves, out, stream); break;
        case 3: e = launch_read<3>(packed, nbands, S, B, waves, out, stream); break;
        case 4: e = launch_read<4>(packed, nbands, S, B, waves, out, stream); break;
        case 5: e = launch_read<5>(packed, nbands, S, B, waves, out, stream); break;
        case 6: e = launch_read<6>(packed, nbands, S, B, waves, out, stream); break;
        case 7: e = launch_read<7>(packed, nbands, S, B, waves, out, stream); break;
        case 8: e = launch_read<8>(packed, nbands, S, B, waves, out, stream); break;
        case 9: e = launch_read<9>(packed, nbands, S, B, waves, out, stream); break;
        case 10: e = launch_read<10>(packed, nbands, S, B, waves, out, stream); break;
        case 12: e = launch_read<12>(packed, nbands, S, B, waves, out, stream); break;
        case 14: e = launch_read<14>(packed, nbands, S, B, waves, out, stream); break;
        case 16: e = launch_read<16>(packed, nbands, S, B, waves, out, stream); break;
        case 18: e = launch_read<18>(packed, nbands, S, B, waves, out, stream); break;
        case 20: e = launch_read<20>(packed, nbands, S, B, waves, out, stream); break;
        default: return -1;
    }
    return e == hipSuccess ? 0 : -4;
}

}  // extern "C"
