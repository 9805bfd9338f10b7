/*
 * bitlinear.h -- C ABI of the BitNet b1.58 W2A8 ternary linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer: ternary weights {-1, 0, +1} packed four to a byte, per-token
 * absmax int8 activations, exact int32 dot products, rescaled by the weight
 * and activation scales to bf16.  Source page: "BitNet GPU 推理框架：从零构建
 * W2A8 的 2-bit 大模型 CUDA GEMV 内核" (blog.gitcode.com), cited as [W2A8]:
 *   §二 2.2   the single exported entry of the page's library (int8
 *             activations, packed weights, bf16 output, activation scale,
 *             weight scales, M, N, K, stream);
 *   §四 4.2   ternary weights and one bf16 scale per matrix (or per fused
 *             sub-matrix);
 *   §5.1-5.3  packing, decoding, int8 dot products, the epilogue
 *             out = acc * scales, with weight scale ws[n / (N / ws_num)];
 *   §六 item 3 per-token activation quantisation s = 127 / max|x|, round,
 *             clamp to [-128, 127];
 *   §六 item 1 the decode step captured as a graph and replayed.
 *
 * Conventions shared by every call
 *   - Pointers are device pointers unless the name ends in _host.
 *   - bf16 values travel as uint16_t bit patterns.
 *   - Every call checks its arguments on the host first and returns a
 *     negative BL_ERR_* code without touching the device if one is wrong;
 *     otherwise it enqueues work on `stream` and returns BL_OK without
 *     synchronising.  A launch failure reported by the runtime returns
 *     BL_ERR_HIP.  Nothing is printed.
 *   - The caller owns every buffer and keeps it alive until the work on
 *     `stream` (or the graph that captured it) has completed.
 *   - No call allocates or frees device memory except bl_graph_create /
 *     bl_graph_destroy (graph objects and their work tables), so calls on
 *     different streams may run concurrently when their outputs do not
 *     overlap.  The only state the library keeps: which kernels have had
 *     their dynamic-LDS limit raised on which device (those staging more
 *     than 64 KiB: the batched kernel above 16 rows, the table-lookup GEMV
 *     above K = 3840), and the allocation-free ternariser's histogram.
 *   - Alignment: xq, x, packed and q_out 16 bytes; s, s_out, acc 4 bytes;
 *     ws, y 2 bytes.  Otherwise BL_ERR_ALIGN.
 *   - Shapes: 1 <= M <= 1048576, N >= 1, K >= 16 with K % 16 == 0,
 *     K <= 1048576, N <= 16777216, M * N <= 2^36.  Otherwise BL_ERR_SHAPE.
 *   - Activation inputs must be finite; scales must be finite and > 0.
 *     These are not checked on the device; other values give undefined
 *     results (never out-of-bounds accesses).
 *
 * Packed weight layout ("16x256 tiles")
 *   The weight w[n][k] of an N x K matrix (row n produces output n) is the
 *   2-bit code w + 2 ({-1,0,1} -> {1,2,3}, [W2A8] §5.2).  Code 0 marks
 *   padding.  With S = ceil(K/256) steps and ceil(N/16) bands:
 *     tile  t = (n / 16) * S + k / 256                   1024 bytes per tile
 *     slot  q = 16 * ((n % 16) / 4) + (k % 256) / 16     16 bytes per slot
 *     byte  t*1024 + 16*q + 4*(n % 4) + (k % 16) % 4
 *     bits  2*((k % 16) / 4) and the next one
 *   i.e. a tile is 16 rows x 256 K; slot q holds four 32-bit words, rows
 *   4*(q/16) .. +3 of the 16-wide K chunk q%16; inside a word element e sits
 *   at bit 8*(e%4) + 2*(e/4): the page's interleave 0,4,8,12,1,5,... ([W2A8]
 *   §5.2), so (word >> 2i) & 0x03030303 holds elements 4i..4i+3 as bytes.
 *   Lane l of a 64-wide wavefront reads slot l with one 16-byte load (a
 *   wavefront's load of a tile is 1 KiB contiguous) and needs one 16-byte
 *   run of activations for it.  Rows n >= N and columns k >= K of the last
 *   tiles are code 0.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define BL_OK 0
#define BL_ERR_NULL (-1)   /* a required pointer is NULL */
#define BL_ERR_SHAPE (-2)  /* M, N, K outside the supported range */
#define BL_ERR_ALIGN (-3)  /* a pointer is not aligned as required */
#define BL_ERR_HIP (-4)    /* the HIP runtime reported an error */
#define BL_ERR_ARG (-5)    /* any other bad argument (ws_num, dtype, n) */

/* Static description of a status code (never NULL). */
const char* bl_status_string(int status);

/* Version of this ABI; bumped on any incompatible change. */
int bl_abi_version(void);

/*
 * Size in bytes of the packed buffer for an N x K matrix:
 * ceil(N/16) * ceil(K/256) * 1024 (exactly N*K/4 when 16 divides N and 256
 * divides K).
 * Returns 0 for N < 1 or K < 1.
 */
size_t bl_packed_bytes(int N, int K);

/*
 * pack_ternary_weights -- pack a ternary matrix into the 16x256-tile layout
 * ([W2A8] §5.1-5.2: code w + 2, four codes per byte, interleaved words).
 *   w          device, int8, N x K row-major (row n = output n)
 *   packed     device, bl_packed_bytes(N, K) bytes, written in full
 *              (padding included)
 *   n_invalid  device int32 counter or NULL; when given, the number of
 *              entries of w outside {-1, 0, 1} is ADDED to it (those entries
 *              are packed as code 0, which the layer reads as weight -2 for
 *              M = 1 and 0 for M > 1: an invalid matrix gives undefined
 *              results)
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE (K % 16 != 0 is allowed here: any
 * N, K >= 1), BL_ERR_ALIGN (packed not 16-byte aligned), BL_ERR_HIP.
 */
int pack_ternary_weights(const int8_t* w, uint8_t* packed, int N, int K,
                         int32_t* n_invalid, hipStream_t stream);

/*
 * Host twin of pack_ternary_weights, bit-identical, for tooling and tests
 * (no device needed).  Returns the number of invalid entries (>= 0) or a
 * negative BL_ERR_* code.
 */
int64_t bl_pack_ternary_host(const int8_t* w_host, uint8_t* packed_host, int N, int K);

/* Bytes of device workspace ternarize_weights_absmean needs (8-byte aligned). */
#define BL_TERNARIZE_WORKSPACE_BYTES 2048

/*
 * ternarize_weights_absmean -- ternarise a bf16 weight matrix by its mean
 * absolute value and pack it ([W2A8] §4.2, then §5.1-5.2):
 *   mean = bf16(exact mean of |w| over all N*K entries)
 *   s    = bf16(fl32(1 / max(mean, 1e-5)))      (below 1e-5: bf16(1e-5f))
 *   Wt   = clamp(round_half_even(bf16(fl32(w * s))), -1, 1)
 *   ws   = bf16(fl32(1 / s))                    the matrix's weight scale
 * i.e. the page's converter in torch bf16 arithmetic (each operation in fp32,
 * rounded to bf16, ties to even), with the mean taken exactly rather than in
 * an order-dependent fp32 sum.  Wt is written packed, as pack_ternary_weights
 * would pack it.
 *   w          device, bf16, N x K row-major, finite values, 16-byte aligned
 *   packed     device, bl_packed_bytes(N, K) bytes, written in full
 *   scales     device, bf16[3]: scales[0] = ws, scales[1] = s, scales[2] =
 *              mean (before the floor); ws is what bitlinear_* take
 *   workspace  device, BL_TERNARIZE_WORKSPACE_BYTES, 8-byte aligned, owned by
 *              the caller; its contents need no initialisation; calls that
 *              share one workspace must not overlap
 * N and K as for the layer (K % 16 == 0, K <= 2^20, N <= 2^24).  Several
 * matrices meant to share one packed buffer (e.g. w1 and w3 of a fused
 * gate+up with ws_num = 2) are ternarised one by one; when the first has a
 * multiple of 16 rows, their packed buffers concatenate to the packing of the
 * stacked matrix.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP.
 */
int ternarize_weights_absmean(const uint16_t* w, uint8_t* packed, uint16_t* scales,
                              void* workspace, int N, int K, hipStream_t stream);

/*
 * ternarize_weights_absmean_noalloc -- ternarize_weights_absmean without the
 * workspace argument, for callers that cannot allocate device memory (code
 * under graph capture, serving loops that forbid allocation).  The same
 * kernels and bits; the histogram lives in a 2 KiB array the library holds
 * on each GPU it runs on until the process ends (its address is looked up
 * once per device, on the first call with that device current).  The array
 * serves a matrix of any size the layer accepts, so no shape exceeds it;
 * shapes outside the layer's limits return BL_ERR_SHAPE.  The call itself
 * allocates nothing.  Every call on a GPU shares that GPU's array: the call
 * clears it first, and calls that overlap on one GPU (several streams, or
 * replays in flight together) race and give undefined results.
 *   w, packed, scales, N, K as ternarize_weights_absmean.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP.
 */
int ternarize_weights_absmean_noalloc(const uint16_t* w, uint8_t* packed, uint16_t* scales,
                                      int N, int K, hipStream_t stream);

/*
 * quantize_act_absmax_i8 -- per-token (per-row) absmax int8 quantisation
 * ([W2A8] §六 item 3):
 *   s[m]    = 127 / max(max_k |x[m][k]|, 1e-5)          fp32, IEEE division
 *   q[m][k] = clamp(round_half_even(x[m][k] * s[m]), -128, 127)
 *   x        device, M x K, fp32 (x_dtype = 0) or bf16 (x_dtype = 1)
 *   q        device, int8, M x K
 *   s        device, fp32, M
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_ARG (x_dtype),
 * BL_ERR_HIP.
 */
int quantize_act_absmax_i8(const void* x, int x_dtype, int8_t* q, float* s, int M, int K,
                           hipStream_t stream);

/*
 * bitlinear_i8xi2 -- the layer on int8 activations ([W2A8] §二 2.2, §5.3):
 *   acc[m][n] = sum_k xq[m][k] * w[n][k]                       exact int32
 *   y[m][n]   = bf16_rne( (double)acc[m][n] * ws[n / (N / ws_num)] / s[m] )
 *   xq       device, int8, M x K row-major
 *   packed   device, bl_packed_bytes(N, K) bytes, 16x256-tile layout
 *   s        device, fp32, M activation scales (127 / amax of each row)
 *   ws       device, bf16, ws_num weight scales, one per equal N-segment
 *   ws_num   1 <= ws_num <= 64 and N % ws_num == 0
 *   y        device, bf16, M x N row-major
 *   acc      device, int32, M x N row-major, or NULL (not written)
 * The activation scale divides: s = 127/amax quantised the activations, so
 * y approximates x . w^T * ws.
 * M == 1 with K <= 61440 runs the GEMV kernel (workgroups of 1, 2 or 4
 * 16-row bands, v_dot8 on masked codes and nibble-split activations).
 * 2 <= M <= 64 with K <= 2560 (a few sequences decoded together) runs the
 * band kernel: int8 MFMA
 * (v_mfma_i32_16x16x64_i8), one wavefront per 16 weight rows over all of K
 * (two per wavefront, with the rows in two workgroups of 32, for M > 32),
 * the activation rows staged once per workgroup in LDS.  M >= 65 with
 * N >= 8192 (prompt processing on wide layers, the prompt lengths of
 * [W2A8] §7.2) runs the LDS-tiled int8 MFMA kernel (workgroup tiles of up
 * to 256 weight rows x 128 activation rows reuse both operands); any other
 * M >= 2, or K > 61440, runs the int8 MFMA kernel that streams the weights
 * once per 64 rows of M.  All four give the same bits.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_ARG, BL_ERR_HIP.
 */
int bitlinear_i8xi2(const int8_t* xq, const uint8_t* packed, const float* s, const uint16_t* ws,
                    int ws_num, uint16_t* y, int32_t* acc, int M, int N, int K,
                    hipStream_t stream);

/*
 * bitlinear_bf16_i8xi2 -- quantise bf16 activations per token, then the
 * layer, as one call ([W2A8] §六 item 3 followed by §5.3).  The result is
 * bit-identical to quantize_act_absmax_i8 (bf16) followed by
 * bitlinear_i8xi2.
 *   x        device, bf16, M x K
 *   q_out    device, int8, M x K, or NULL: the quantised activations
 *   s_out    device, fp32, M, or NULL: the activation scales
 *   acc      device, int32, M x N, or NULL
 * M == 1 and K <= 61440: one fused kernel (each workgroup quantises the row
 * into LDS).  M >= 2 or K > 61440: q_out and s_out are required (they are
 * the staging buffers of a quantise kernel followed by the layer kernel);
 * BL_ERR_NULL otherwise.
 * Errors: as bitlinear_i8xi2.
 */
int bitlinear_bf16_i8xi2(const uint16_t* x, const uint8_t* packed, const uint16_t* ws,
                         int ws_num, uint16_t* y, int8_t* q_out, float* s_out, int32_t* acc,
                         int M, int N, int K, hipStream_t stream);

/*
 * bitlinear_lut_i8xi2 -- the M = 1 layer on int8 activations by table lookup,
 * a second algorithm for the same result as bitlinear_i8xi2 (same arguments
 * with M = 1; the same acc and y bits).  After the LUT kernels of the CPU
 * page "BitNet на микроконтроллерах: как устроен запуск 1.58-битной LLM на
 * кластере ESP32-S3" (sarnas.ru; its sections on the LUT compilation of the
 * weights and on the qgemm_lut kernel): every pair of activations (elements
 * e and e + 4 of a 16-wide K chunk, e in 0..3 and 8..11) gets a table of its
 * 16 sums (c0 - 2) x0 + (c1 - 2) x1 over 2-bit codes c0, c1, and each 4-bit
 * nibble of a packed word -- the codes of such a pair -- selects one entry.
 * The tables of the whole row live in LDS (17 K bytes).  It is a cross-check
 * of the dot-product kernel, not a faster path on this GPU.
 *   16 <= K <= 8192, K % 16 == 0; other arguments as bitlinear_i8xi2.
 * Errors: as bitlinear_i8xi2 (BL_ERR_SHAPE for K > 8192).
 */
int bitlinear_lut_i8xi2(const int8_t* xq, const uint8_t* packed, const float* s,
                        const uint16_t* ws, int ws_num, uint16_t* y, int32_t* acc, int N, int K,
                        hipStream_t stream);

/*
 * bitlinear_rmsnorm_i8xi2 -- one projection of a decode step with the glue
 * that joins it to the previous one.  [W2A8] §4.1 names the converted
 * model's norms (attention_norm and ffn_norm before the attention and MLP
 * inputs, BitNet b1.58's attn_sub_norm and ffn_sub_norm) and its fused
 * projections (wqkv, wo, w13 = gate_proj then up_proj, w2) but states
 * neither the norm's formula nor the MLP activation; this library reads
 * them as RMSNorm and relu(gate)^2 * up:
 *   m    = x                              (x_up == NULL)
 *        = bf16(max(x, 0)^2 * x_up)       (x_up != NULL: x and x_up are the
 *                                          gate and up halves of w13's output)
 *   xn   = bf16( fl64(m * gamma) * fl64(1 / sqrt(sum(m^2) / K + eps)) )
 *   q, s = per-token absmax int8 quantisation of xn, as quantize_act_absmax_i8
 *   y    = bf16(acc * ws / s), or bf16(residual + bf16(acc * ws / s))
 *   x, x_up, gamma  device, bf16, K, 16-byte aligned (x_up may be NULL)
 *   eps       finite, >= 0 (the model's: 1e-5)
 *   packed, ws, ws_num   as bitlinear_i8xi2
 *   residual  device, bf16, N, or NULL
 *   y         device, bf16, N
 *   xn_out    device, bf16, K, 16-byte aligned, or NULL: the normalised row
 *   q_out     device, int8, K, 8-byte aligned, or NULL
 *   s_out     device, fp32, 1, or NULL
 *   acc       device, int32, N, or NULL
 * One row (M = 1), 16 <= K <= 32768 with K % 16 == 0.  One kernel: every
 * workgroup forms the glue for its copy of the row, then runs the GEMV.
 * y must not overlap x, x_up or gamma (other workgroups still read them);
 * it may be residual itself (each output reads only its own residual).
 * xn matches the fp64 definition except, possibly, when that value lies
 * within about 2^-50 (relative) of a bf16 rounding midpoint (the sum of
 * squares is taken in another order), where it may be the other neighbour.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_ARG (eps or
 * ws_num), BL_ERR_HIP.
 */
int bitlinear_rmsnorm_i8xi2(const uint16_t* x, const uint16_t* x_up, const uint16_t* gamma,
                            float eps, const uint8_t* packed, const uint16_t* ws, int ws_num,
                            const uint16_t* residual, uint16_t* y, uint16_t* xn_out,
                            int8_t* q_out, float* s_out, int32_t* acc, int N, int K,
                            hipStream_t stream);

/*
 * Decode-step graph ([W2A8] §六 item 1: each decode step is a graph
 * replay).  A bl_gemv_desc is one M = 1 call of bitlinear_bf16_i8xi2; the
 * graph runs n of them with the results of running them in array order, and
 * is replayed with one launch.  Consecutive calls that do not touch what
 * another of them writes (no call reads or writes another's y or acc) form
 * a run, and a run of two or more calls with K <= 10240 is one grouped
 * kernel launch: each of its workgroups takes four 16-row bands of one call.
 * A call that reads or overwrites an earlier call's output starts a new
 * run, so it sees that output.  The results are bit-identical to the calls
 * one by one.
 */
typedef struct bl_gemv_desc {
    const uint16_t* x;       /* device, bf16, K */
    const uint8_t* packed;   /* device, bl_packed_bytes(N, K) */
    const uint16_t* ws;      /* device, bf16, ws_num */
    int ws_num;
    uint16_t* y;             /* device, bf16, N */
    int32_t* acc;            /* device, int32, N, or NULL */
    int N;
    int K;
} bl_gemv_desc;

typedef struct bl_graph bl_graph;

/*
 * Capture the n calls (1 <= n <= 65536; every descriptor K <= 61440) on an
 * internal stream of its own (this call takes no stream) and instantiate
 * them.  The descriptors are validated first; the pointers they hold are
 * baked into the graph and must stay valid while it exists.  The work
 * tables of the grouped launches (64 bytes per workgroup) are allocated in
 * device memory here, filled by a synchronous copy, and freed by
 * bl_graph_destroy.  *out receives the graph (NULL on error).
 * Errors: BL_ERR_NULL, BL_ERR_ARG (n; a call whose y or acc overlaps its own
 * x, packed or ws, or whose y and acc overlap), any error of
 * bitlinear_bf16_i8xi2 for an invalid descriptor, BL_ERR_HIP.
 */
int bl_graph_create(const bl_gemv_desc* descs, int n, bl_graph** out);

/*
 * A decode step chained through its glue: each bl_norm_desc is one call of
 * bitlinear_rmsnorm_i8xi2 (without the optional outputs); the graph gives
 * the results of running them in array order, so a call may read what an
 * earlier one wrote (its x, x_up or residual may be an earlier y).  As in
 * bl_graph_create, consecutive calls that do not touch another's y form a
 * run; inside a run, the calls that take the same kernel instance (the same
 * row length class and launch shape, e.g. the qkv and o projections of a
 * layer) share one grouped launch.  A call's y may be its own residual but
 * may overlap none of its other inputs (BL_ERR_ARG).  Same rules and errors
 * as bl_graph_create otherwise, with bitlinear_rmsnorm_i8xi2's checks per
 * descriptor.
 * Hand-off ([W2A8] §4.1: w13 feeds the activation before ffn_sub_norm and
 * w2): when a call with x_up reads as x and x_up the two halves of the y of
 * the call just before it (that call's N = 2K, each half whole 16-row
 * bands, the two calls launched on their own, and the earlier one's launch
 * shape -- chosen from N and K alone -- an even number of bands per
 * workgroup, at most 256 workgroups, and a whole number of workgroups in
 * each half; the model's w13, 13824 x 2560, takes four bands in each of 216
 * workgroups), the earlier call's kernel also computes, in its epilogue,
 * m = bf16(max(gate, 0)^2 * up) and, per workgroup, the sum of m^2 and the
 * largest |m * gamma| of the later call; the later call reads m and those
 * partials instead of redoing the activation and the reductions in each of
 * its workgroups.  The results are the same bits (the sum of squares is
 * added in another order, as the kernel's own order already differs from
 * left to right).  The graph allocates 2K bytes and 16 bytes per producing
 * workgroup of device memory for each hand-off here and frees them in
 * bl_graph_destroy; replays of one graph must not overlap (they share these
 * buffers, as they share the calls' outputs).
 */
typedef struct bl_norm_desc {
    const uint16_t* x;        /* device, bf16, K */
    const uint16_t* x_up;     /* device, bf16, K, or NULL */
    const uint16_t* gamma;    /* device, bf16, K */
    float eps;
    const uint8_t* packed;    /* device, bl_packed_bytes(N, K) */
    const uint16_t* ws;       /* device, bf16, ws_num */
    int ws_num;
    const uint16_t* residual; /* device, bf16, N, or NULL */
    uint16_t* y;              /* device, bf16, N */
    int N;
    int K;
} bl_norm_desc;

int bl_graph_create_norm(const bl_norm_desc* descs, int n, bl_graph** out);

/* Enqueue one replay of the graph on `stream`.  Errors: BL_ERR_NULL, BL_ERR_HIP. */
int bl_graph_launch(bl_graph* graph, hipStream_t stream);

/* Number of calls the graph holds, or BL_ERR_NULL. */
int bl_graph_size(const bl_graph* graph);

/* Number of kernel launches one replay of the graph makes, or BL_ERR_NULL. */
int bl_graph_kernels(const bl_graph* graph);

/* Number of calls of a bl_graph_create_norm graph that take the hand-off from
 * the call before them (0 for bl_graph_create graphs), or BL_ERR_NULL. */
int bl_graph_linked(const bl_graph* graph);

/* Destroy the graph (NULL is allowed).  The caller ensures no replay is in flight. */
int bl_graph_destroy(bl_graph* graph);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
