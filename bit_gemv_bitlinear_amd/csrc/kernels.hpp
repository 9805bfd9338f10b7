// kernels.hpp -- internal host-side launchers of the gfx950 kernels.  The
// launchers assume validated arguments (the C ABI in abi.hip validates) and
// return the status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace bl {

size_t packed_bytes(int N, int K);

hipError_t launch_pack(const int8_t* w, uint8_t* packed, int N, int K, int32_t* n_invalid,
                       hipStream_t stream);
int64_t pack_host(const int8_t* w, uint8_t* packed, int N, int K);

hipError_t launch_quant(const void* x, int x_is_bf16, int8_t* q, float* s, int M, int K,
                        hipStream_t stream);

// Row n's weight-scale index n / d (d = N / ws_num) as (n * mul) >> shift,
// exact for every 0 <= n < 2^24.
void seg_divisor(int d, uint32_t& mul, int& shift);

// Raise kernel fn's dynamic-LDS limit to `bytes` on the current device, once
// per kernel and device (kernels whose LDS exceeds the default 64 KiB); the
// status of that one call, every time.
hipError_t raise_lds_limit(const void* fn, int bytes);

// M == 1 GEMV geometry: `waves` wavefronts per workgroup covering `bands`
// 16-row bands, `steps` K steps (256 K each) per wavefront; waves == 0 when
// K is beyond the GEMV kernels (K > kGemvMaxK), which then leave M == 1 to
// the MFMA kernel.
struct GemvShape {
    int waves;
    int steps;
    int bands;
};
constexpr int kGemvMaxK = 61440;   // LDS copy of the row <= 60 KiB
constexpr int kNormMaxK = 32768;   // the projection with its glue (launch_gemv_norm)
constexpr int kLutMaxK = 8192;     // the table-lookup GEMV: tables of the row in LDS (K * 17 B)
GemvShape gemv_shape(int N, int K);

// M == 1, int8 activations; K <= kGemvMaxK.
hipError_t launch_gemv_i8(const int8_t* xq, const uint8_t* packed, const float* s,
                          const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int N, int K,
                          hipStream_t stream);

// M == 1, bf16 activations quantised inside the kernel; K <= kGemvMaxK.
hipError_t launch_gemv_bf16_fused(const uint16_t* x, const uint8_t* packed, const uint16_t* ws,
                                  int ws_num, uint16_t* y, int8_t* q_out, float* s_out,
                                  int32_t* acc, int N, int K, hipStream_t stream);

// The wave-local variant of the bf16 GEMV: one band per workgroup, `waves`
// (<= 4) wavefronts of `steps` (<= kLocalMaxSteps) K steps, 2^lw = waves;
// seg_mul / seg_shift from seg_divisor(N / ws_num).
constexpr int kLocalMaxSteps = 12;
hipError_t launch_gemv_local(const uint16_t* x, const uint8_t* packed, const uint16_t* ws,
                             uint32_t seg_mul, int seg_shift, uint16_t* y, int32_t* acc,
                             int8_t* q_out, float* s_out, int N, int K, unsigned groups,
                             int waves, int steps, int lw, hipStream_t stream);

// Grouped GEMV: many independent M == 1 bf16 calls in one launch, one
// 64-byte work record per workgroup (4 bands of one node).  K <= kGroupMaxK.
struct GroupNode {
    const uint16_t* x;
    const uint8_t* packed;
    const uint16_t* ws;
    int ws_num;
    uint16_t* y;
    int32_t* acc;
    int N;
    int K;
};
struct alignas(64) GroupWork {
    const void* packed;        // the node's packed weights
    const uint16_t* x;         // its bf16 activation row
    const uint16_t* ws;        // its weight scales
    uint16_t* y;               // its output row
    int32_t* acc;              // or null
    int N;
    int K;
    uint32_t seg_mul;          // weight-scale segment of row n: (n * seg_mul) >> seg_shift
    int seg_shift;
    int group;                 // the workgroup's index within its node
    int pad;
};
static_assert(sizeof(GroupWork) == 64, "one 64-byte record per workgroup");
constexpr int kGroupMaxK = 10240;  // four chunks of ten 256-K tiles
bool group_supported(int K);
int group_workgroups(int N);
size_t group_lds_bytes(int K);
void group_work_records(const GroupNode& node, std::vector<GroupWork>& out);
hipError_t launch_gemv_group(const GroupWork* work, int n_work, size_t lds, hipStream_t stream);

// M == 1, int8 activations, by table lookup (a cross-check of the dot-product
// GEMV); K <= kLutMaxK.
hipError_t launch_gemv_lut(const int8_t* xq, const uint8_t* packed, const float* s,
                           const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int N, int K,
                           hipStream_t stream);

// M == 1 projection with its glue: [relu2-GLU of (x, x_up)] -> RMSNorm(gamma,
// eps) -> per-token int8 quantisation -> ternary layer -> [+ residual];
// K <= kNormMaxK.  xn_out / q_out / s_out / acc may be null.
hipError_t launch_gemv_norm(const uint16_t* x, const uint16_t* x_up, const uint16_t* gamma,
                            float eps, const uint8_t* packed, const uint16_t* ws, int ws_num,
                            const uint16_t* residual, uint16_t* y, uint16_t* xn_out,
                            int8_t* q_out, float* s_out, int32_t* acc, int N, int K,
                            hipStream_t stream);

// The projection with its glue as a plan: its kernel instance (P = steps,
// C = cached chunks, GLU), its launch shape and its arguments.  Projections
// of one instance (same steps, chunks, GLU and threads) can share a grouped
// launch: one 128-byte work record per workgroup.
struct NormArgs {
    const uint16_t* x;
    const uint16_t* x_up;
    const uint16_t* gamma;
    const void* packed;
    const uint16_t* ws;
    const uint16_t* residual;
    uint16_t* y;
    int32_t* acc;
    int8_t* q_out;
    float* s_out;
    uint16_t* xn_out;
    double eps;
    uint32_t seg_mul;
    int seg_shift;
    int N;
    int K;
    int B;        // bands per workgroup
    int lw;       // log2 of the wavefronts per band
};
struct alignas(128) NormWork {
    NormArgs a;
    int group;    // the workgroup's index within its projection
};
static_assert(sizeof(NormWork) == 128, "one 128-byte record per workgroup");
struct NormPlan {
    NormArgs args;
    int groups;   // workgroups (0: shape not supported)
    int threads;
    size_t lds;
    int steps;
    int cached;
    bool glu;
};
NormPlan norm_plan(const uint16_t* x, const uint16_t* x_up, const uint16_t* gamma, float eps,
                   const uint8_t* packed, const uint16_t* ws, int ws_num,
                   const uint16_t* residual, uint16_t* y, uint16_t* xn_out, int8_t* q_out,
                   float* s_out, int32_t* acc, int N, int K);
hipError_t launch_gemv_norm_group(const NormPlan& key, const NormWork* work, int n_work,
                                  size_t lds, hipStream_t stream);

// A hand-off between two projections of a chain: the one whose output holds
// the gate half [0, half) and the up half [half, 2 half) of the MLP computes,
// in its epilogue, the activation m of the next projection and, per
// workgroup, the two statistics the next projection's RMSNorm needs (the sum
// of m^2 and the largest |m * gamma| as the high word of its fp64 encoding).
// The next projection then reads m as its row and the partials instead of
// recomputing them in every workgroup.
struct alignas(16) NormPart {
    double ssq;
    uint32_t pm;
    uint32_t pad;
};
constexpr int kNormMaxParts = 256;   // partials one consumer reads (4 per lane)
struct NormLink {
    // producer (m_out null: none); each of its half / 16 / (B / 2)
    // workgroups takes B / 2 gate bands and the up bands of the same rows
    uint16_t* m_out;
    const uint16_t* gamma_next;
    NormPart* part_out;
    int half;
    // consumer (part_in null: none): the row is m, its statistics the
    // producer's n_part partials
    int n_part;
    const NormPart* part_in;
};
// Whether a projection of plan p can produce the GLU hand-off for rows of
// `half` values (its output is the two halves).
bool norm_link_supported(const NormPlan& p, int half);
hipError_t launch_gemv_norm_plan(const NormPlan& p, const NormLink& link, hipStream_t stream);

// Ternarise a bf16 N x K matrix by its mean |w| and pack it; scales[0..2] =
// ws, s, mean (bf16); workspace: 256 uint64 (the exponent histogram).
hipError_t launch_ternarize(const uint16_t* w, uint8_t* packed, uint16_t* scales,
                            void* workspace, int N, int K, hipStream_t stream);
// Device address, on the current device, of the ternariser's library-held
// histogram (kTernarizeScratchBytes), for the allocation-free entry point.
constexpr size_t kTernarizeScratchBytes = 2048;
hipError_t ternarize_scratch(void** out);

// Many activation rows (prompt processing), int8 activations, int8 MFMA
// with LDS-tiled reuse of both operands.
hipError_t launch_gemm_prefill(const int8_t* xq, const uint8_t* packed, const float* s,
                               const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int M,
                               int N, int K, hipStream_t stream);

// 2 <= M <= kBandMaxM and K <= kBandMaxK: int8 MFMA with one wavefront per
// one or two 16-row bands over all of K and the activation rows (or a group
// of 32 of them) staged in LDS.
constexpr int kBandMaxM = 64;
constexpr int kBandMaxK = 2560;
hipError_t launch_gemm_band(const int8_t* xq, const uint8_t* packed, const float* s,
                            const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int M,
                            int N, int K, hipStream_t stream);

// M >= 2, int8 activations, int8 MFMA.
hipError_t launch_gemm_mfma(const int8_t* xq, const uint8_t* packed, const float* s,
                            const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int M,
                            int N, int K, hipStream_t stream);

}  // namespace bl
