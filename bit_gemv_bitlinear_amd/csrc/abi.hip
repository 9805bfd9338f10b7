// abi.hip -- the C ABI declared in include/bitlinear.h: host-side argument
// checks, kernel selection, and the decode-step graph.
//
// Source page: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
// (blog.gitcode.com), cited as [W2A8]: §二 2.2 (one exported C entry taking
// int8 activations, packed weights, bf16 output, scales, M, N, K and a
// stream), §六 item 1 (each decode step replayed as a captured graph).  The
// page's library selects a kernel by exact (M, N, K) and prints when none
// matches; this one accepts any shape in range and returns a status code.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <iterator>
#include <map>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "bitlinear.h"
#include "kernels.hpp"

namespace bl {

hipError_t raise_lds_limit(const void* fn, int bytes) {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, hipError_t> raised;   // (kernel, device) -> status
    const std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(fn, dev);
    auto it = raised.find(key);
    if (it == raised.end())
        it = raised.emplace(key, hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     bytes)).first;
    return it->second;
}

}  // namespace bl

namespace {

constexpr int kMaxK = 1 << 20;
constexpr int kMaxN = 1 << 24;
// Rows of activations: the MFMA kernels' grids (N/64 x M/64 workgroups, or
// one dimension of at most M*N/2^15 workgroups of 512 threads) stay far
// inside the launch limits, as does the quantiser's one workgroup per row.
constexpr int kMaxM = 1 << 20;
constexpr long long kMaxOutputs = 1LL << 36;   // M * N
constexpr int kMaxWsNum = 64;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_mnk(int M, int N, int K) {
    if (M < 1 || N < 1 || K < 16 || (K % 16) != 0 || K > kMaxK || N > kMaxN || M > kMaxM)
        return BL_ERR_SHAPE;
    if (static_cast<long long>(M) * N > kMaxOutputs) return BL_ERR_SHAPE;
    return BL_OK;
}

int check_ws(int ws_num, int N) {
    if (ws_num < 1 || ws_num > kMaxWsNum || (N % ws_num) != 0) return BL_ERR_ARG;
    return BL_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_HIP; }

int check_layer_i8(const int8_t* xq, const uint8_t* packed, const float* s, const uint16_t* ws,
                   int ws_num, const uint16_t* y, const int32_t* acc, int M, int N, int K) {
    if (!xq || !packed || !s || !ws || !y) return BL_ERR_NULL;
    int rc = check_mnk(M, N, K);
    if (rc) return rc;
    if ((rc = check_ws(ws_num, N))) return rc;
    if (!aligned(xq, 16) || !aligned(packed, 16) || !aligned(s, 4) || !aligned(ws, 2) ||
        !aligned(y, 2) || (acc && !aligned(acc, 4)))
        return BL_ERR_ALIGN;
    return BL_OK;
}

int check_layer_bf16(const uint16_t* x, const uint8_t* packed, const uint16_t* ws, int ws_num,
                     const uint16_t* y, const int8_t* q_out, const float* s_out,
                     const int32_t* acc, int M, int N, int K) {
    if (!x || !packed || !ws || !y) return BL_ERR_NULL;
    int rc = check_mnk(M, N, K);
    if (rc) return rc;
    if ((rc = check_ws(ws_num, N))) return rc;
    const bool staged = (M > 1) || (K > bl::kGemvMaxK);
    if (staged && (!q_out || !s_out)) return BL_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(ws, 2) || !aligned(y, 2) ||
        (q_out && !aligned(q_out, 16)) || (s_out && !aligned(s_out, 4)) ||
        (acc && !aligned(acc, 4)))
        return BL_ERR_ALIGN;
    return BL_OK;
}

// The LDS-tiled kernel (both operands reused across a workgroup) beats the
// one that streams the weights per 64-row chunk as soon as that one needs a
// second chunk, M > 64, for wide layers (13824 x 2560, same box: 13.6 against
// 16.0 us at M = 65, 13.5 against 16.4 at M = 96, 28 against 55 at M = 512);
// up to M = 64 it is slower (12.7 against 10.1 us at M = 64), and for narrow
// layers (N <= 3840) it is slower at every M measured (11.8 against 9.2 us at
// 3840 x 2560, 24.2 against 16.3 at 2560 x 6912, M = 96), too few of its
// larger tiles to fill the chip.
constexpr int kPrefillMinM = 65;
constexpr int kPrefillMinN = 8192;

int check_norm(const uint16_t* x, const uint16_t* x_up, const uint16_t* gamma, float eps,
               const uint8_t* packed, const uint16_t* ws, int ws_num, const uint16_t* residual,
               const uint16_t* y, const uint16_t* xn_out, const int8_t* q_out,
               const float* s_out, const int32_t* acc, int N, int K) {
    if (!x || !gamma || !packed || !ws || !y) return BL_ERR_NULL;
    int rc = check_mnk(1, N, K);
    if (rc) return rc;
    if (K > bl::kNormMaxK) return BL_ERR_SHAPE;
    if ((rc = check_ws(ws_num, N))) return rc;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return BL_ERR_ARG;
    if (!aligned(x, 16) || (x_up && !aligned(x_up, 16)) || !aligned(gamma, 16) ||
        !aligned(packed, 16) || !aligned(ws, 2) || (residual && !aligned(residual, 2)) ||
        !aligned(y, 2) || (xn_out && !aligned(xn_out, 16)) || (q_out && !aligned(q_out, 8)) ||
        (s_out && !aligned(s_out, 4)) || (acc && !aligned(acc, 4)))
        return BL_ERR_ALIGN;
    return BL_OK;
}

int run_layer_i8(const int8_t* xq, const uint8_t* packed, const float* s, const uint16_t* ws,
                 int ws_num, uint16_t* y, int32_t* acc, int M, int N, int K, hipStream_t stream) {
    if (M == 1 && K <= bl::kGemvMaxK)
        return status_of(bl::launch_gemv_i8(xq, packed, s, ws, ws_num, y, acc, N, K, stream));
    if (M >= 2 && M <= bl::kBandMaxM && K <= bl::kBandMaxK)
        return status_of(bl::launch_gemm_band(xq, packed, s, ws, ws_num, y, acc, M, N, K, stream));
    if (M >= kPrefillMinM && N >= kPrefillMinN)
        return status_of(bl::launch_gemm_prefill(xq, packed, s, ws, ws_num, y, acc, M, N, K, stream));
    return status_of(bl::launch_gemm_mfma(xq, packed, s, ws, ws_num, y, acc, M, N, K, stream));
}

int run_layer_bf16(const uint16_t* x, const uint8_t* packed, const uint16_t* ws, int ws_num,
                   uint16_t* y, int8_t* q_out, float* s_out, int32_t* acc, int M, int N, int K,
                   hipStream_t stream) {
    if (M == 1 && K <= bl::kGemvMaxK)
        return status_of(bl::launch_gemv_bf16_fused(x, packed, ws, ws_num, y, q_out, s_out, acc,
                                                    N, K, stream));
    int rc = status_of(bl::launch_quant(x, 1, q_out, s_out, M, K, stream));
    if (rc) return rc;
    return run_layer_i8(q_out, packed, s_out, ws, ws_num, y, acc, M, N, K, stream);
}

}  // namespace

struct bl_graph {
    hipGraphExec_t exec;
    int n;                          // calls the graph holds
    int kernels;                    // kernel launches per replay
    std::vector<void*> tables;      // device memory it owns: work tables, hand-off buffers
    int linked = 0;                 // calls that take a hand-off from the call before
};

namespace {

void free_tables(std::vector<void*>& tables) {
    for (void* p : tables) (void)hipFree(p);
    tables.clear();
}

// Capture n_launch enqueue(i, stream) calls on an internal stream and
// instantiate them into a bl_graph that also owns `tables`.
template <class Enqueue>
int capture_graph(int n_calls, int n_launch, std::vector<void*>& tables, bl_graph** out,
                  Enqueue enqueue) {
    (void)hipGetLastError();
    hipStream_t cs = nullptr;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) {
        free_tables(tables);
        return BL_ERR_HIP;
    }
    int rc = BL_OK;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        rc = BL_ERR_HIP;
    } else {
        for (int i = 0; i < n_launch && rc == BL_OK; ++i) rc = enqueue(i, cs);
        const hipError_t e = hipStreamEndCapture(cs, &graph);
        if (rc == BL_OK && e != hipSuccess) rc = BL_ERR_HIP;
    }
    if (rc == BL_OK && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess)
        rc = BL_ERR_HIP;
    if (graph) (void)hipGraphDestroy(graph);
    (void)hipStreamDestroy(cs);
    if (rc != BL_OK) {
        if (exec) (void)hipGraphExecDestroy(exec);
        free_tables(tables);
        return rc;
    }
    bl_graph* g = new (std::nothrow) bl_graph{exec, n_calls, n_launch, {}, 0};
    if (!g) {
        (void)hipGraphExecDestroy(exec);
        free_tables(tables);
        return BL_ERR_ARG;
    }
    g->tables.swap(tables);
    *out = g;
    return BL_OK;
}

// Byte ranges [lo, hi) of device memory, merged as they are added: the union
// of what a run of calls reads, or of what it writes.
class RangeUnion {
  public:
    bool overlaps(uintptr_t lo, uintptr_t hi) const {
        if (lo >= hi) return false;
        auto it = r_.upper_bound(lo);            // first range starting above lo
        if (it != r_.begin() && std::prev(it)->second > lo) return true;
        return it != r_.end() && it->first < hi;
    }
    void add(uintptr_t lo, uintptr_t hi) {
        if (lo >= hi) return;
        auto it = r_.upper_bound(lo);
        if (it != r_.begin() && std::prev(it)->second >= lo) --it;
        while (it != r_.end() && it->first <= hi) {
            lo = std::min(lo, it->first);
            hi = std::max(hi, it->second);
            it = r_.erase(it);
        }
        r_.emplace(lo, hi);
    }
    void clear() { r_.clear(); }

  private:
    std::map<uintptr_t, uintptr_t> r_;
};

uintptr_t addr(const void* p) { return reinterpret_cast<uintptr_t>(p); }

// The memory one call of the decode step reads and writes.
struct CallRanges {
    uintptr_t in[3][2];
    uintptr_t out[2][2];
};

CallRanges ranges_of(const bl_gemv_desc& d) {
    CallRanges r{};
    r.in[0][0] = addr(d.x);
    r.in[0][1] = addr(d.x) + 2u * static_cast<uintptr_t>(d.K);
    r.in[1][0] = addr(d.packed);
    r.in[1][1] = addr(d.packed) + bl::packed_bytes(d.N, d.K);
    r.in[2][0] = addr(d.ws);
    r.in[2][1] = addr(d.ws) + 2u * static_cast<uintptr_t>(d.ws_num);
    r.out[0][0] = addr(d.y);
    r.out[0][1] = addr(d.y) + 2u * static_cast<uintptr_t>(d.N);
    r.out[1][0] = d.acc ? addr(d.acc) : 0;
    r.out[1][1] = d.acc ? addr(d.acc) + 4u * static_cast<uintptr_t>(d.N) : 0;
    return r;
}

bool any_overlap(const RangeUnion& u, const uintptr_t (*r)[2], int n) {
    for (int i = 0; i < n; ++i)
        if (u.overlaps(r[i][0], r[i][1])) return true;
    return false;
}

// One launch of the decode-step graph: either one call on its own (the
// single GEMV kernel) or a run of independent calls as one grouped launch.
struct Launch {
    int first, count;               // calls [first, first + count)
    const bl::GroupWork* table;     // device work table of a grouped launch
    int n_work;
    size_t lds;
};

}  // namespace

extern "C" {

const char* bl_status_string(int status) {
    switch (status) {
        case BL_OK: return "ok";
        case BL_ERR_NULL: return "a required pointer is NULL";
        case BL_ERR_SHAPE: return "M, N or K outside the supported range";
        case BL_ERR_ALIGN: return "a pointer is not aligned as required";
        case BL_ERR_HIP: return "the HIP runtime reported an error";
        case BL_ERR_ARG: return "bad argument";
        default: return "unknown status";
    }
}

int bl_abi_version(void) { return 1; }

size_t bl_packed_bytes(int N, int K) { return bl::packed_bytes(N, K); }

int pack_ternary_weights(const int8_t* w, uint8_t* packed, int N, int K, int32_t* n_invalid,
                         hipStream_t stream) {
    if (!w || !packed) return BL_ERR_NULL;
    if (N < 1 || K < 1 || N > kMaxN || K > kMaxK) return BL_ERR_SHAPE;
    if (!aligned(packed, 16) || (n_invalid && !aligned(n_invalid, 4))) return BL_ERR_ALIGN;
    (void)hipGetLastError();
    return status_of(bl::launch_pack(w, packed, N, K, n_invalid, stream));
}

int64_t bl_pack_ternary_host(const int8_t* w_host, uint8_t* packed_host, int N, int K) {
    if (!w_host || !packed_host) return BL_ERR_NULL;
    if (N < 1 || K < 1 || N > kMaxN || K > kMaxK) return BL_ERR_SHAPE;
    if (!aligned(packed_host, 4)) return BL_ERR_ALIGN;
    return bl::pack_host(w_host, packed_host, N, K);
}

int ternarize_weights_absmean(const uint16_t* w, uint8_t* packed, uint16_t* scales,
                              void* workspace, int N, int K, hipStream_t stream) {
    if (!w || !packed || !scales || !workspace) return BL_ERR_NULL;
    const int rc = check_mnk(1, N, K);
    if (rc) return rc;
    if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(workspace, 8))
        return BL_ERR_ALIGN;
    (void)hipGetLastError();
    return status_of(bl::launch_ternarize(w, packed, scales, workspace, N, K, stream));
}

int ternarize_weights_absmean_noalloc(const uint16_t* w, uint8_t* packed, uint16_t* scales,
                                      int N, int K, hipStream_t stream) {
    if (!w || !packed || !scales) return BL_ERR_NULL;
    const int rc = check_mnk(1, N, K);
    if (rc) return rc;
    if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(scales, 2)) return BL_ERR_ALIGN;
    static_assert(BL_TERNARIZE_WORKSPACE_BYTES <= bl::kTernarizeScratchBytes,
                  "the library-held histogram holds the workspace of any matrix");
    (void)hipGetLastError();
    void* hist = nullptr;
    if (bl::ternarize_scratch(&hist) != hipSuccess) return BL_ERR_HIP;
    return status_of(bl::launch_ternarize(w, packed, scales, hist, N, K, stream));
}

int quantize_act_absmax_i8(const void* x, int x_dtype, int8_t* q, float* s, int M, int K,
                           hipStream_t stream) {
    if (!x || !q || !s) return BL_ERR_NULL;
    if (x_dtype != 0 && x_dtype != 1) return BL_ERR_ARG;
    if (M < 1 || M > kMaxM || K < 16 || (K % 16) != 0 || K > kMaxK) return BL_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return BL_ERR_ALIGN;
    (void)hipGetLastError();
    return status_of(bl::launch_quant(x, x_dtype, q, s, M, K, stream));
}

int bitlinear_i8xi2(const int8_t* xq, const uint8_t* packed, const float* s, const uint16_t* ws,
                    int ws_num, uint16_t* y, int32_t* acc, int M, int N, int K,
                    hipStream_t stream) {
    const int rc = check_layer_i8(xq, packed, s, ws, ws_num, y, acc, M, N, K);
    if (rc) return rc;
    (void)hipGetLastError();
    return run_layer_i8(xq, packed, s, ws, ws_num, y, acc, M, N, K, stream);
}

int bitlinear_bf16_i8xi2(const uint16_t* x, const uint8_t* packed, const uint16_t* ws,
                         int ws_num, uint16_t* y, int8_t* q_out, float* s_out, int32_t* acc,
                         int M, int N, int K, hipStream_t stream) {
    const int rc = check_layer_bf16(x, packed, ws, ws_num, y, q_out, s_out, acc, M, N, K);
    if (rc) return rc;
    (void)hipGetLastError();
    return run_layer_bf16(x, packed, ws, ws_num, y, q_out, s_out, acc, M, N, K, stream);
}

int bitlinear_lut_i8xi2(const int8_t* xq, const uint8_t* packed, const float* s,
                        const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int N, int K,
                        hipStream_t stream) {
    const int rc = check_layer_i8(xq, packed, s, ws, ws_num, y, acc, 1, N, K);
    if (rc) return rc;
    if (K > bl::kLutMaxK) return BL_ERR_SHAPE;
    (void)hipGetLastError();
    return status_of(bl::launch_gemv_lut(xq, packed, s, ws, ws_num, y, acc, N, K, stream));
}

int bitlinear_rmsnorm_i8xi2(const uint16_t* x, const uint16_t* x_up, const uint16_t* gamma,
                            float eps, const uint8_t* packed, const uint16_t* ws, int ws_num,
                            const uint16_t* residual, uint16_t* y, uint16_t* xn_out,
                            int8_t* q_out, float* s_out, int32_t* acc, int N, int K,
                            hipStream_t stream) {
    const int rc = check_norm(x, x_up, gamma, eps, packed, ws, ws_num, residual, y, xn_out, q_out,
                              s_out, acc, N, K);
    if (rc) return rc;
    (void)hipGetLastError();
    return status_of(bl::launch_gemv_norm(x, x_up, gamma, eps, packed, ws, ws_num, residual, y,
                                          xn_out, q_out, s_out, acc, N, K, stream));
}

int bl_graph_create(const bl_gemv_desc* descs, int n, bl_graph** out) {
    if (!out) return BL_ERR_NULL;
    *out = nullptr;
    if (!descs) return BL_ERR_NULL;
    if (n < 1 || n > 65536) return BL_ERR_ARG;
    std::vector<CallRanges> rng(n);
    for (int i = 0; i < n; ++i) {
        const bl_gemv_desc& d = descs[i];
        const int rc = check_layer_bf16(d.x, d.packed, d.ws, d.ws_num, d.y, nullptr, nullptr,
                                        d.acc, 1, d.N, d.K);
        if (rc) return rc;
        rng[i] = ranges_of(d);
        // a call's outputs may not overlap its own inputs or each other:
        // other workgroups of the same call still read them
        RangeUnion own;
        for (auto& r : rng[i].in) own.add(r[0], r[1]);
        if (any_overlap(own, rng[i].out, 2)) return BL_ERR_ARG;
        RangeUnion y;
        y.add(rng[i].out[0][0], rng[i].out[0][1]);
        if (any_overlap(y, rng[i].out + 1, 1)) return BL_ERR_ARG;
    }
    // Runs of consecutive calls that neither read nor write what another call
    // of the run writes run as one grouped launch, in any order; a call that
    // conflicts with its run starts the next run, so the stream order keeps
    // every dependence.
    std::vector<Launch> launches;
    {
        RangeUnion reads, writes;
        int first = 0;
        for (int i = 0; i <= n; ++i) {
            const bool end = (i == n) || !bl::group_supported(descs[i].K) ||
                             (i > first && !bl::group_supported(descs[first].K)) ||
                             any_overlap(writes, rng[i].in, 3) ||
                             any_overlap(writes, rng[i].out, 2) ||
                             any_overlap(reads, rng[i].out, 2);
            if (end && i > first) {
                launches.push_back(Launch{first, i - first, nullptr, 0, 0});
                reads.clear();
                writes.clear();
                first = i;
            }
            if (i == n) break;
            for (auto& r : rng[i].in) reads.add(r[0], r[1]);
            for (auto& r : rng[i].out) writes.add(r[0], r[1]);
        }
    }
    // Work tables of the grouped launches, written once here.
    std::vector<void*> tables;
    for (Launch& L : launches) {
        if (L.count < 2) continue;
        std::vector<bl::GroupWork> work;
        for (int i = L.first; i < L.first + L.count; ++i) {
            const bl_gemv_desc& d = descs[i];
            bl::group_work_records(bl::GroupNode{d.x, d.packed, d.ws, d.ws_num, d.y, d.acc, d.N, d.K},
                                   work);
            L.lds = std::max(L.lds, bl::group_lds_bytes(d.K));
        }
        // Longest rows first: the workgroups of long-row calls (three or four
        // chunks of tiles) would otherwise be among the last to start, and
        // finish with most CUs idle.  (The decode step: 88.8 -> 87.4 and
        // 90.3 -> 88.7 us, same box.)
        std::stable_sort(work.begin(), work.end(),
                         [](const bl::GroupWork& a, const bl::GroupWork& b) { return a.K > b.K; });
        void* p = nullptr;
        const size_t bytes = work.size() * sizeof(bl::GroupWork);
        if (hipMalloc(&p, bytes) != hipSuccess) {
            free_tables(tables);
            return BL_ERR_HIP;
        }
        tables.push_back(p);
        if (hipMemcpy(p, work.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
            free_tables(tables);
            return BL_ERR_HIP;
        }
        L.table = static_cast<const bl::GroupWork*>(p);
        L.n_work = static_cast<int>(work.size());
    }
    return capture_graph(n, static_cast<int>(launches.size()), tables, out,
                         [&](int li, hipStream_t cs) {
        const Launch& L = launches[li];
        if (L.table) return status_of(bl::launch_gemv_group(L.table, L.n_work, L.lds, cs));
        const bl_gemv_desc& d = descs[L.first];
        return run_layer_bf16(d.x, d.packed, d.ws, d.ws_num, d.y, nullptr, nullptr, d.acc, 1, d.N,
                              d.K, cs);
    });
}

int bl_graph_create_norm(const bl_norm_desc* descs, int n, bl_graph** out) {
    if (!out) return BL_ERR_NULL;
    *out = nullptr;
    if (!descs) return BL_ERR_NULL;
    if (n < 1 || n > 65536) return BL_ERR_ARG;
    // What each call reads (x, x_up, gamma, packed, ws, residual) and writes (y).
    struct NormRanges {
        uintptr_t in[6][2];
        uintptr_t out[1][2];
    };
    std::vector<NormRanges> rng(n);
    for (int i = 0; i < n; ++i) {
        const bl_norm_desc& d = descs[i];
        const int rc = check_norm(d.x, d.x_up, d.gamma, d.eps, d.packed, d.ws, d.ws_num,
                                  d.residual, d.y, nullptr, nullptr, nullptr, nullptr, d.N, d.K);
        if (rc) return rc;
        const uintptr_t K2 = 2u * static_cast<uintptr_t>(d.K), N2 = 2u * static_cast<uintptr_t>(d.N);
        NormRanges& r = rng[i];
        r.in[0][0] = addr(d.x), r.in[0][1] = addr(d.x) + K2;
        r.in[1][0] = d.x_up ? addr(d.x_up) : 0, r.in[1][1] = d.x_up ? addr(d.x_up) + K2 : 0;
        r.in[2][0] = addr(d.gamma), r.in[2][1] = addr(d.gamma) + K2;
        r.in[3][0] = addr(d.packed), r.in[3][1] = addr(d.packed) + bl::packed_bytes(d.N, d.K);
        r.in[4][0] = addr(d.ws), r.in[4][1] = addr(d.ws) + 2u * static_cast<uintptr_t>(d.ws_num);
        r.in[5][0] = d.residual ? addr(d.residual) : 0;
        r.in[5][1] = d.residual ? addr(d.residual) + N2 : 0;
        r.out[0][0] = addr(d.y), r.out[0][1] = addr(d.y) + N2;
        // y may be the residual itself (each output reads only its own
        // residual) but may overlap no other input of its call
        RangeUnion own;
        for (int k = 0; k < 5; ++k) own.add(r.in[k][0], r.in[k][1]);
        if (any_overlap(own, r.out, 1)) return BL_ERR_ARG;
        if (d.residual && d.residual != d.y) {
            RangeUnion res;
            res.add(r.in[5][0], r.in[5][1]);
            if (any_overlap(res, r.out, 1)) return BL_ERR_ARG;
        }
    }
    // Runs of independent calls (as in bl_graph_create); inside a run, the
    // calls of one kernel instance share a grouped launch.
    struct NormLaunch {
        std::vector<int> calls;
        bl::NormPlan key;
        const bl::NormWork* table;
        int n_work;
        size_t lds;
    };
    std::vector<NormLaunch> launches;
    auto same_instance = [](const bl::NormPlan& a, const bl::NormPlan& b) {
        return a.glu == b.glu && a.cached == b.cached && a.steps == b.steps && a.threads == b.threads;
    };
    std::vector<bl::NormPlan> plans(n);
    for (int i = 0; i < n; ++i) {
        const bl_norm_desc& d = descs[i];
        plans[i] = bl::norm_plan(d.x, d.x_up, d.gamma, d.eps, d.packed, d.ws, d.ws_num, d.residual,
                                 d.y, nullptr, nullptr, nullptr, nullptr, d.N, d.K);
        if (plans[i].groups == 0) return BL_ERR_SHAPE;
    }
    {
        RangeUnion reads, writes;
        int first = 0;
        for (int i = 0; i <= n; ++i) {
            const bool end = (i == n) || any_overlap(writes, rng[i].in, 6) ||
                             any_overlap(writes, rng[i].out, 1) || any_overlap(reads, rng[i].out, 1);
            if (end && i > first) {
                std::vector<NormLaunch> run;
                for (int j = first; j < i; ++j) {
                    auto it = std::find_if(run.begin(), run.end(), [&](const NormLaunch& L) {
                        return same_instance(L.key, plans[j]);
                    });
                    if (it == run.end()) run.push_back(NormLaunch{{j}, plans[j], nullptr, 0, 0});
                    else it->calls.push_back(j);
                }
                for (auto& L : run) launches.push_back(std::move(L));
                reads.clear();
                writes.clear();
                first = i;
            }
            if (i == n) break;
            for (auto& r : rng[i].in) reads.add(r[0], r[1]);
            writes.add(rng[i].out[0][0], rng[i].out[0][1]);
        }
    }
    std::vector<void*> tables;
    auto device_alloc = [&](size_t bytes) -> void* {
        void* p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess) return nullptr;
        tables.push_back(p);
        return p;
    };
    // Hand-offs: a GLU call whose x and x_up are the two halves of the y of
    // the call just before it, both launched on their own, takes its row m
    // and its statistics from that call's epilogue (buffers the graph owns).
    std::vector<bl::NormLink> links(launches.size(), bl::NormLink{});
    int linked = 0;
    for (size_t li = 1; li < launches.size(); ++li) {
        const NormLaunch& L = launches[li];
        const NormLaunch& Lp = launches[li - 1];
        if (L.calls.size() != 1 || Lp.calls.size() != 1) continue;
        const int c = L.calls[0], pc = Lp.calls[0];
        const bl_norm_desc& d = descs[c];
        const bl_norm_desc& dp = descs[pc];
        if (!d.x_up || d.x != dp.y || d.x_up != dp.y + d.K) continue;
        if (!bl::norm_link_supported(plans[pc], d.K)) continue;
        uint16_t* m = static_cast<uint16_t*>(device_alloc(2u * static_cast<size_t>(d.K)));
        bl::NormPart* parts = static_cast<bl::NormPart*>(
            m ? device_alloc(sizeof(bl::NormPart) * plans[pc].groups) : nullptr);
        if (!parts) {
            free_tables(tables);
            return BL_ERR_HIP;
        }
        links[li - 1].m_out = m;
        links[li - 1].gamma_next = d.gamma;
        links[li - 1].part_out = parts;
        links[li - 1].half = d.K;
        links[li].n_part = plans[pc].groups;
        links[li].part_in = parts;
        plans[c] = bl::norm_plan(m, nullptr, d.gamma, d.eps, d.packed, d.ws, d.ws_num, d.residual,
                                 d.y, nullptr, nullptr, nullptr, nullptr, d.N, d.K);
        ++linked;
    }
    for (NormLaunch& L : launches) {
        if (L.calls.size() < 2) continue;
        std::vector<bl::NormWork> work;
        for (int j : L.calls) {
            for (int g = 0; g < plans[j].groups; ++g) {
                bl::NormWork w{};
                w.a = plans[j].args;
                w.group = g;
                work.push_back(w);
            }
            L.lds = std::max(L.lds, plans[j].lds);
        }
        void* p = nullptr;
        const size_t bytes = work.size() * sizeof(bl::NormWork);
        if (hipMalloc(&p, bytes) != hipSuccess) {
            free_tables(tables);
            return BL_ERR_HIP;
        }
        tables.push_back(p);
        if (hipMemcpy(p, work.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
            free_tables(tables);
            return BL_ERR_HIP;
        }
        L.table = static_cast<const bl::NormWork*>(p);
        L.n_work = static_cast<int>(work.size());
    }
    const int rc = capture_graph(n, static_cast<int>(launches.size()), tables, out,
                                 [&](int li, hipStream_t cs) {
        const NormLaunch& L = launches[li];
        if (L.table)
            return status_of(bl::launch_gemv_norm_group(L.key, L.table, L.n_work, L.lds, cs));
        return status_of(bl::launch_gemv_norm_plan(plans[L.calls[0]], links[li], cs));
    });
    if (rc == BL_OK) (*out)->linked = linked;
    return rc;
}

int bl_graph_launch(bl_graph* graph, hipStream_t stream) {
    if (!graph) return BL_ERR_NULL;
    return status_of(hipGraphLaunch(graph->exec, stream));
}

int bl_graph_size(const bl_graph* graph) { return graph ? graph->n : BL_ERR_NULL; }

int bl_graph_kernels(const bl_graph* graph) { return graph ? graph->kernels : BL_ERR_NULL; }

int bl_graph_linked(const bl_graph* graph) { return graph ? graph->linked : BL_ERR_NULL; }

int bl_graph_destroy(bl_graph* graph) {
    if (!graph) return BL_OK;
    const hipError_t e = hipGraphExecDestroy(graph->exec);
    free_tables(graph->tables);
    delete graph;
    return status_of(e);
}

}  // extern "C"
