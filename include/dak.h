/*
 * dak.h -- C ABI of libdak: direct-access split operators over two memory tiers
 * (pinned host memory and HBM) on one AMD Instinct MI355X (gfx950).
 *
 * What the library computes follows the DAK paper ("DAK: Direct-Access-Enabled
 * GPU Memory Offloading with Optimal Efficiency for LLM Inference", Lin, Guo and
 * Lin) and its walkthrough (pinghaoyang.com.cn, "DAK 完全拆解").  The kernels
 * are written for CDNA4; the paper's Hopper TMA/multicast design is not used.
 *
 * Conventions shared by every entry point
 *   - Status codes: DAK_OK (0) on success, a negative dak_status otherwise.  On
 *     error nothing has been launched and no output has been written;
 *     dak_last_error() gives a message (thread-local).
 *   - Ownership: the caller allocates and owns every buffer (device memory,
 *     pinned host memory, workspaces).  The library never allocates on the
 *     compute entry points.
 *   - Streams: `stream` is a hipStream_t passed as void*; NULL means the null
 *     stream.  Compute calls are asynchronous and stream-ordered: outputs are
 *     valid once the stream has completed.  Probes synchronize to time.
 *   - Pointers to device memory must be device allocations on the current
 *     device; pointers to host memory must lie inside a pinned (page-locked)
 *     allocation made with hipHostMalloc / torch pin_memory.  Both are checked
 *     with hipPointerGetAttributes before any launch (DAK_EINVAL otherwise).
 *   - bf16 means IEEE bfloat16 stored as 16-bit words; fp32 is IEEE binary32.
 *   - Deterministic: no atomics in the compute path; for fixed shapes the
 *     result bits do not depend on the host/HBM split, the host CU count or the
 *     in-flight window.
 */
#ifndef DAK_H
#define DAK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dak_status;
enum {
  DAK_OK = 0,
  DAK_EINVAL = -1,        /* bad argument (shape, pointer, alignment, range) */
  DAK_EINFEASIBLE = -2,   /* the host budget exceeds what the ops hold */
  DAK_EHIP = -3,          /* a HIP runtime call failed; see dak_last_hip_error() */
  DAK_EUNSUPPORTED = -4   /* a valid request the library does not implement */
};

/* Message describing the last error on the calling thread ("" if none). */
const char* dak_last_error(void);
/* hipError_t of the last DAK_EHIP on the calling thread (0 if none). */
int32_t dak_last_hip_error(void);
/* ABI version of this header (bumped on any incompatible change). */
int32_t dak_abi_version(void);
#define DAK_ABI_VERSION 3

/* ------------------------------------------------------------------------ */
/* Capacity and planning (pure CPU, deterministic)                            */
/* ------------------------------------------------------------------------ */

/* One operation for the planner.  DAK paper §4.2.2 "Optimal Greedy Offload".
 *   units      n_i: tile-rows of a weight matrix, or requests of a KV cache
 *   unit_bytes u_i: bytes per unit (C_i = n_i * u_i)
 *   t_comp_s   T_comp,i: compute time of the op in seconds (>= 0), e.g. its
 *              flops divided by the measured compute rate                      */
typedef struct {
  uint64_t units;
  uint64_t unit_bytes;
  double t_comp_s;
} dak_op_desc;

/* Lower bound on the global offload ratio for a footprint of M bytes (weights
 * plus KV) and H bytes of usable HBM: max(0, (M - H) / M).  Walkthrough,
 * capacity section (the x_global constraint; runtime workspace ignored).
 * Returns 0 when M == 0. */
double dak_min_offload_ratio(uint64_t footprint_bytes, uint64_t hbm_bytes);

/* Greedy per-operation host-unit counts for a global ratio x_global.
 * DAK paper §4.2.1 (cost model), §4.2.2 (three phases), App. A eq. (1).
 *   T_i(h) = max(T_comp,i, (n_i - h) u_i / b_hbm, h u_i / b_host), byte counts
 *            converted to double before dividing;
 *   a_i, b_i = first and last h in [0, n_i] minimising T_i;
 *   op i is memory-bound iff T_i(0) > T_comp,i;
 *   W = ceil(x_global * sum_i C_i) (one double multiply, then ceil);
 *   phase 1: memory-bound ops raised toward a_i; phase 2: all ops toward b_i;
 *   phase 3: all ops toward n_i; ops visited in index order, each taking only
 *   ceil((W - S) / u_i) more units; allocation stops once S >= W.
 * Arguments
 *   ops[n_ops]          caller-owned, n_ops >= 1, every units >= 1 and
 *                       unit_bytes >= 1, sum C_i <= 2^53
 *   b_hbm, b_host       bytes per second, > 0 and finite (measured)
 *   x_global            in [0, 1]; the caller ensures it is at least
 *                       dak_min_offload_ratio(M, H) (only it knows H)
 *   host_units_out      caller-owned array of n_ops; receives h_i
 *   modeled_time_s_out  nullable; receives sum_i T_i(h_i) (op order)
 * Errors: DAK_EINVAL on bad arguments, DAK_EINFEASIBLE if S < W after phase 3
 * (cannot happen for x_global <= 1).  Outputs are untouched on error. */
dak_status dak_plan_offload(const dak_op_desc* ops, size_t n_ops, double b_hbm, double b_host,
                            double x_global, uint64_t* host_units_out,
                            double* modeled_time_s_out);

/* The planner's modelled time of one op with h of its units on the host.
 * DAK paper §4.2.1 (the offload cost model; walkthrough, the offload-ratio
 * model): T_i(h) = max(T_comp,i, (n_i - h) u_i / b_hbm, h u_i / b_host), byte
 * counts converted to double before dividing, exactly as dak_plan_offload
 * evaluates it.
 *   op       as for dak_plan_offload; 0 <= h <= op->units
 *   t_out    receives T_i(h) in seconds
 * Errors: DAK_EINVAL on bad arguments (t_out untouched). */
dak_status dak_op_time(const dak_op_desc* op, uint64_t h, double b_hbm, double b_host, double* t_out);

/* The uniform policy the greedy planner is measured against (DAK paper
 * §4.2.1, "The Suboptimality of Uniform Offloading"): every op offloads the
 * same ratio x, h_i = min(n_i, ceil(x * n_i)) with x * n_i one double
 * multiply (the rounding rule of dak_plan_offload's budget W), and the
 * modelled time sum_i T_i(h_i) accumulated in op order.
 * Arguments and errors as for dak_plan_offload, with x in [0, 1] in place of
 * x_global (the uniform plan never fails once the arguments are valid). */
dak_status dak_plan_uniform(const dak_op_desc* ops, size_t n_ops, double b_hbm, double b_host, double x,
                            uint64_t* host_units_out, double* modeled_time_s_out);

/* The per-op quantities the planner uses: a_i, b_i (as above) and whether the
 * op is memory-bound.  Any output pointer may be NULL. */
dak_status dak_op_turning_points(const dak_op_desc* op, double b_hbm, double b_host,
                                 uint64_t* a_out, uint64_t* b_out, int32_t* memory_bound_out);

/* Host work-group count for `items` host work items under a cap of `cap`
 * host work-groups: the G in [1, min(cap, items)] with the fewest waves
 * ceil(items / G), and the smallest such G.  DAK paper §4.1 (wave alignment,
 * congestion cap); walkthrough (waves = ceil(tiles / SMs)).  0 if items <= 0
 * (whatever the cap); otherwise -1 if cap <= 0. */
int64_t dak_host_workgroups(int64_t items, int32_t cap);

/* ------------------------------------------------------------------------ */
/* Launch configuration (congestion control)                                  */
/* ------------------------------------------------------------------------ */

/* DAK paper §4.3.1 "Congestion Control over Local/Remote Access": the number
 * of compute units reading the host and the requests each keeps in flight are
 * capped; both come from an offline sweep.
 *   host_cus       cap on work-groups (one per CU) that read host memory;
 *                  0 = per-operator default from the library's host-role
 *                  sweep on MI355X (the fewest that reach the full link rate;
 *                  tuning_defaults.hpp, generated from the sweep table): split
 *                  GEMM N <= 4 (and FP8 at N = 1) and 64 < N <= 256, and
 *                  split attention, one swept cap each; split GEMM
 *                  4 < N <= 64 (bf16) and 2 <= N <= 64 (FP8): the
 *                  fewest whose staged chunks in flight cover about 256 KiB,
 *                  within the sweep's bounds; N > 256: no cap, the
 *                  launch picks its group count from a time model of the
 *                  link and of both roles' rounds.  For N > 256 host
 *                  work-groups come in groups of ceil(N/256), one per
 *                  256-column tile of a 256-row block, placed on one XCD so
 *                  that its L2 serves their repeated reads of the block (the
 *                  link carries each host byte once); a cap is rounded down
 *                  to whole groups, at least one
 *   window         host in-flight window: loop steps whose loads a host-role
 *                  wave issues before consuming the first; one of 1, 2, 4, 8.
 *                  0 = sized so that all host work-groups together keep about
 *                  256 KiB in flight (the link's bandwidth-delay product).  A
 *                  step is 512 k of the wave's 4 rows (GEMM, N <= 4; FP8 at
 *                  N = 1: 1024 k), a 256-k
 *                  chunk of its 16 rows (GEMM, 64 < N <= 256, at most 2
 *                  chunks) or 16 tokens of K and V (attention; clamped to what
 *                  registers allow).  The split GEMM for 4 < N <= 64 and for
 *                  N > 256 stages its tiles through LDS rings whose depth is
 *                  fixed by the kernel; there the window is accepted and
 *                  ignored (its host bytes in flight follow from host_cus)
 *   flags          bit-or of DAK_FLAG_*
 *   byte_counters  device pointer to 2 uint64 (host bytes, HBM bytes), used
 *                  only with DAK_FLAG_COUNT_BYTES: the kernels add the bytes
 *                  of A (or of K and V) they load from each tier.  The caller
 *                  zeroes them.  With DAK_FLAG_RECORD_XCC, 2 + 256 uint64 (see
 *                  there).
 * A NULL dak_launch_cfg* means all defaults. */
typedef struct {
  int32_t host_cus;
  int32_t window;
  int32_t flags;
  int32_t reserved;
  uint64_t* byte_counters;
} dak_launch_cfg;

#define DAK_FLAG_COUNT_BYTES 1
/* The host part of the operand (dak_split_matrix.host, dak_split_matrix_fp8.host,
 * or dak_split_kv.k_host and v_host) is not in pinned host memory: it is a
 * device-memory copy of the host units, staged in HBM by a copy-based
 * prefetcher ahead of the call (the baseline DAK paper §2.3 and Fig. 2
 * compare against: the host bytes are copied over the link into an HBM
 * staging buffer, then read from HBM).  Every work-group then reads device
 * memory: the call runs as if h were 0, with the first h units taken from the
 * staged buffer, and its result is bit-identical to the direct split.  Split
 * GEMM with N <= 256 and dense split attention only (DAK_EUNSUPPORTED for
 * N > 256 and for paged attention); the byte counters count every byte as
 * HBM. */
#define DAK_FLAG_STAGED_HOST 2
/* Split GEMM with N > 256 only (ignored elsewhere): byte_counters then holds
 * 2 + 256 uint64 (the caller zeroes them), and entry 2 + q receives the
 * bitwise OR of 1 << (XCD id) over the work-groups of host group q, read from
 * the hardware's XCC id register.  A mask with one bit shows that the group's
 * work-groups, which request the same host row block, shared one XCD's L2
 * (DAK paper §4.3.2: a host tile must cross the link once; on CDNA4 that L2,
 * not a multicast, serves the repeats).  A debugging aid for the placement
 * the tiled schedule assumes. */
#define DAK_FLAG_RECORD_XCC 4

/* ------------------------------------------------------------------------ */
/* Split GEMM: y = x . A^T with A split by tile-rows across the two tiers      */
/* ------------------------------------------------------------------------ */

/* A weight matrix A (M x K, bf16, row-major, leading dimension K) cut along M
 * into tile-rows of m rows; tile-rows [0, h) are in pinned host memory and
 * [h, M/m) in HBM.  DAK paper §4.1 "Data Partition", Fig. 5a.
 *   host  rows [0, h*m) of A, contiguous, in pinned host memory (may be NULL
 *         when h == 0)
 *   hbm   rows [h*m, M) of A, contiguous, in device memory (may be NULL when
 *         h*m == M)
 *   M, K  M >= 1 a multiple of m; K >= 8 a multiple of 8
 *   m     tile-row height, a positive multiple of 16
 *   h     host tile-rows, 0 <= h <= M/m
 * Both pointers 16-byte aligned. */
typedef struct {
  const void* host;
  const void* hbm;
  int64_t M;
  int64_t K;
  int32_t m;
  int32_t reserved;
  int64_t h;
} dak_split_matrix;

/* y[n, r] = sum_k A[r, k] * x[n, k] for n < N, r < M (fp32 accumulation).
 * DAK paper §4.1 "Kernel over Partitioned Memory": disjoint work-groups compute
 * disjoint output rows; each work-group reads only one tier; a host tile-row
 * is never split along N, so every host byte crosses the link once.
 *   A   the split matrix (see dak_split_matrix)
 *   x   bf16 [N, K] row-major in device memory, 16-byte aligned
 *   N   1 <= N <= 2048.  N <= 64 is the memory-bound (decode) regime; N > 256
 *       the compute-bound one (DAK paper §4.2.1), served by a 256 x 256 tiled
 *       MFMA kernel with one work-group per CU, whose host groups share each
 *       host row block through one XCD's L2
 *   y   fp32 [N, M] row-major in device memory, 16-byte aligned; fully written
 *   cfg nullable launch configuration
 * The result depends on (M, K, m, N) and the inputs only: it is bit-identical
 * for every h, host_cus and window.
 * Errors: DAK_EINVAL for shapes/pointers outside the above; DAK_EUNSUPPORTED
 * for N > 2048 (or, on a device with fewer than 32 CUs per XCD, an N > 256
 * whose host group does not fit one XCD); DAK_EHIP if the launch fails. */
dak_status dak_splitk_gemm(const dak_split_matrix* A, const void* x, int64_t N, float* y,
                           const dak_launch_cfg* cfg, void* stream);

/* Bytes of workspace that dak_splitk_gemm_ws uses for an M x K weight and N
 * activation rows; 0 when the shape is not split.  Shapes of the tiled kernel
 * (N > 256) whose 256 x 256 output tiles would leave most CUs of a round idle
 * (small M: QKV, O or down at a prefill-sized N) split K into 2, 4 or 8
 * segments, chosen from (M, K, N) alone; the workspace holds one fp32 [N, M]
 * partial output per segment. */
uint64_t dak_splitk_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N);

/* dak_splitk_gemm with a workspace.  ws: device memory, 16-byte aligned, of
 * at least dak_splitk_gemm_workspace_bytes(M, K, N) bytes, owned by the
 * caller and not read after the call's work completes on `stream`; NULL runs
 * the shape unsplit (as dak_splitk_gemm does).  Split, each output is the
 * sum, in segment order, of one fp32 MFMA chain per K segment, added by a
 * second kernel on the same stream: a different rounding order from the
 * unsplit launch, still bit-identical for every h, host_cus and window.
 * Errors: those of dak_splitk_gemm, and DAK_EINVAL for a non-NULL workspace
 * that is too small, misaligned or not device memory.  Calls that share one
 * workspace must not overlap. */
dak_status dak_splitk_gemm_ws(const dak_split_matrix* A, const void* x, int64_t N, float* y, void* ws,
                              uint64_t ws_bytes, const dak_launch_cfg* cfg, void* stream);

/* A weight matrix of FP8 codes, cut along M like dak_split_matrix.  Each
 * weight is an OCP FP8 E4M3 code (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits; no infinities; 0x7F and 0xFF are NaN) and each row r carries
 * one fp32 scale: the logical weight is row_scale[r] * e4m3(A[r, k]).  The
 * pages run their models in FP8 (BOOST §5, Models), which halves the bytes of
 * every weight tile-row; they do not fix the scaling, so this is the plainest
 * per-output-channel reading.
 *   host, hbm   uint8 codes, rows [0, h*m) pinned host / rows [h*m, M) device,
 *               row-major with leading dimension K (bytes)
 *   M, K, m, h  as in dak_split_matrix; K a multiple of 16
 *   row_scale   fp32 [M] in device memory
 * All pointers 16-byte aligned. */
typedef struct {
  const void* host;
  const void* hbm;
  int64_t M;
  int64_t K;
  int32_t m;
  int32_t reserved;
  int64_t h;
  const float* row_scale;
} dak_split_matrix_fp8;

/* y[n, r] = row_scale[r] * sum_k e4m3(A[r, k]) * x[n, k] for n < N, r < M.
 * Each product of an e4m3 weight and a bf16 activation is exact in fp32; the
 * sums accumulate in fp32 in an order fixed by the shape, and the scale is
 * applied once to the finished sum, so the result bits do not depend on h,
 * the host CU cap or the window.  Same split rule as dak_splitk_gemm (DAK
 * §4.1): disjoint work-groups own disjoint output rows, each reads one tier,
 * and every host byte crosses the link once.
 *   A     the FP8 split matrix
 *   x     bf16 [N, K] in device memory
 *   N     1 .. 2048: N = 1 takes plain fp32 FMAs (codes widened to fp32
 *         exactly), 2 <= N <= 64 the memory-bound LDS-ring kernel on the
 *         matrix cores; wider activations (DAK §4.2.1's compute-bound regime, where halving
 *         the bytes of a tile-row doubles the turning point's host share)
 *         take the tiled kernel of dak_splitk_gemm with FP8 A tiles, the
 *         codes widened to bf16 (exact) before the same bf16 MFMA
 *   y     fp32 [N, M] in device memory; fully written
 *   cfg   nullable launch configuration (the window applies at N = 1 as in
 *         dak_splitk_gemm's FMA path; the other kernels stage fixed-depth
 *         rings; for N > 64 host_cus caps the host groups as in
 *         dak_splitk_gemm)
 * Errors: DAK_EINVAL for shapes/pointers outside the above, DAK_EUNSUPPORTED
 * for N > 2048 and for a staged host part (DAK_FLAG_STAGED_HOST) with
 * N > 64.  A NaN code gives NaN in its row. */
dak_status dak_splitk_gemm_fp8(const dak_split_matrix_fp8* A, const void* x, int64_t N, float* y,
                               const dak_launch_cfg* cfg, void* stream);

/* The FP8 counterparts of dak_splitk_gemm_workspace_bytes and
 * dak_splitk_gemm_ws (the tiled kernel, and so a split, starts at N > 64);
 * split, the row scale multiplies the sum of the segments' partial sums. */
uint64_t dak_splitk_gemm_fp8_workspace_bytes(int64_t M, int64_t K, int64_t N);
dak_status dak_splitk_gemm_fp8_ws(const dak_split_matrix_fp8* A, const void* x, int64_t N, float* y, void* ws,
                                  uint64_t ws_bytes, const dak_launch_cfg* cfg, void* stream);

/* ------------------------------------------------------------------------ */
/* Split decode attention: KV cache split along the batch                      */
/* ------------------------------------------------------------------------ */

/* KV caches of `batch` requests, split between pinned host memory and HBM.
 * DAK paper §5 "Supporting FlashAttention": the split runs along the batch,
 * each request attending entirely within one tier.  The host share is the
 * first h units in (request, KV head) order: whole requests (unit ==
 * DAK_KV_UNIT_REQUEST, the pages' split), or single KV heads of requests
 * (DAK_KV_UNIT_HEAD: unit u = b * n_kv_heads + g), a finer step for a small
 * batch, where one request is a coarse share of the cache.  Either way every
 * (request, KV head) attends within one tier.
 *   k_host, v_host  bf16, the host units' [ctx, head_dim] blocks in unit order
 *                   ([h, n_kv_heads, ctx, head_dim] for request units), row-major
 *                   (NULL if there are no host units)
 *   k_hbm,  v_hbm   bf16, the remaining units' blocks in unit order (NULL if none)
 *   batch, h        requests; host units (0 <= h <= batch for request units,
 *                   0 <= h <= batch * n_kv_heads for head units)
 *   head_dim        128
 *   ctx             tokens stored per request
 *   unit            DAK_KV_UNIT_REQUEST or DAK_KV_UNIT_HEAD
 *   ctx_lens        nullable device array of `batch` int32: the valid tokens
 *                   of each request, its first ctx_lens[b] positions (1..ctx;
 *                   values outside [0, ctx] are clamped to it, and a request
 *                   with no valid token gets NaN rows); NULL: all ctx valid
 * All pointers 16-byte aligned, ctx_lens included. */
#define DAK_KV_UNIT_REQUEST 0
#define DAK_KV_UNIT_HEAD 1
typedef struct {
  const void* k_host;
  const void* v_host;
  const void* k_hbm;
  const void* v_hbm;
  int64_t batch;
  int64_t h;
  int32_t n_kv_heads;
  int32_t head_dim;
  int64_t ctx;
  int32_t unit;
  int32_t reserved;
  const int32_t* ctx_lens;
} dak_split_kv;

/* Bytes of device workspace dak_splitk_decode_attn needs for these shapes
 * (0 on invalid shapes): one record of head_dim + 2 floats per (request,
 * query head, chunk), chunks of 4096 tokens where kv has no ctx_lens array
 * and the (request, KV head) units times ceil(ctx / 4096) reach 1024 work
 * items, else of 2048. */
size_t dak_decode_attn_workspace_bytes(const dak_split_kv* kv, int32_t n_q_heads);

/* out[b, j, :] = sum_t softmax_t(scale * q[b, j] . K[b, g, t]) V[b, g, t, :]
 * with g = j / (n_q_heads / n_kv_heads) (grouped-query attention), one query
 * token per request, fp32 accumulation, exact softmax; t runs over the
 * request's valid tokens.
 *   q        bf16 [batch, n_q_heads, head_dim] in device memory
 *   kv       the split KV cache
 *   n_q_heads a multiple of n_kv_heads, group size 1, 2, 4 or 8
 *   scale    finite softmax scale (e.g. 1/sqrt(head_dim))
 *   out      fp32 [batch, n_q_heads, head_dim] in device memory; fully written
 *   ws       device workspace of at least dak_decode_attn_workspace_bytes()
 *   cfg      nullable launch configuration
 * Errors: DAK_EINVAL for shapes/pointers outside the above, DAK_EUNSUPPORTED
 * for head_dim != 128 or a group size other than 1, 2, 4, 8. */
dak_status dak_splitk_decode_attn(const void* q, const dak_split_kv* kv, int32_t n_q_heads,
                                  float scale, float* out, void* ws, size_t ws_bytes,
                                  const dak_launch_cfg* cfg, void* stream);

/* dak_splitk_decode_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, hosts that forbid hipMalloc):
 * the same kernels, with the workspace taken from a fixed array the library
 * holds on every device it runs on (dak_decode_attn_scratch_max_bytes()
 * bytes, 16 MiB, kept until the process ends).  Nothing is allocated or
 * freed by the call.  Arguments, results, determinism and errors are those of
 * dak_splitk_decode_attn without ws/ws_bytes; in addition DAK_EINVAL when
 * dak_decode_attn_workspace_bytes(kv, n_q_heads) exceeds the array (more
 * than 32263 records of 520 bytes).
 * Every call on a device shares that device's array: calls that overlap in
 * time on one device (different streams, or different host threads without
 * ordering between their streams) race on it and their outputs are then
 * unspecified; calls ordered on one stream are safe.  No part of the array
 * needs clearing between calls (each call writes every record it reads). */
dak_status dak_splitk_decode_attn_noalloc(const void* q, const dak_split_kv* kv, int32_t n_q_heads, float scale,
                                          float* out, const dak_launch_cfg* cfg, void* stream);
/* Size in bytes of the per-device array dak_splitk_decode_attn_noalloc uses. */
size_t dak_decode_attn_scratch_max_bytes(void);

/* A paged KV cache split between two page pools.  Paged attention keeps each
 * request's cache in fixed-size pages drawn from a free pool; BOOST §3.3 and
 * §4.3 ("Block-level KV Head Chunk Partitioning", "Wave-aware Block
 * Fulfillment") reorder the pages head-major so one KV head's pages can live
 * in the host tier while the request's other heads stay in HBM.  Here the
 * units are (request, KV head) pairs u = b * n_kv_heads + g, each with its own
 * row of the page table, and every unit lies wholly in one tier (DAK §4.1:
 * one data path per work-group).  Which units are host units changes as
 * requests come and go, so it is given on the device: the first n_host_units
 * entries of unit_order name them.
 *   k_host, v_host   bf16 host pool [host_pages, page, head_dim], pinned
 *                    (NULL when host_pages == 0)
 *   k_hbm,  v_hbm    bf16 HBM pool [hbm_pages, page, head_dim], device memory
 *                    (NULL when hbm_pages == 0)
 *   host_pages, hbm_pages  pages in each pool
 *   batch, n_kv_heads, head_dim (128)
 *   page             tokens per page: a power of two, 16 .. 2^20
 *   max_pages        columns of page_table (pages per unit at most)
 *   page_table       device int32 [batch * n_kv_heads, max_pages]: entry
 *                    [u, i] is the index, in u's tier's pool, of the page
 *                    holding u's tokens [i * page, (i + 1) * page)
 *   ctx_lens         device int32 [batch]: valid tokens of each request,
 *                    clamped to [0, max_pages * page]; entries of page_table
 *                    past a unit's last valid page are never read
 *   unit_order       device int32 [batch * n_kv_heads]: a permutation of the
 *                    units; entries [0, n_host_units) are the host units
 *   n_host_units     0 .. batch * n_kv_heads
 * Contents of the device arrays are checked by the kernel, which never reads
 * outside a pool: a unit with a page index outside its pool gets NaN rows;
 * an entry of unit_order outside [0, units) is skipped.  If unit_order is not
 * a permutation, the units it misses get NaN rows (every chunk record of the
 * call is marked unwritten before the partial kernel runs), and a unit it
 * lists twice is computed twice into the same records with the same bits.
 * All pointers 16-byte aligned. */
typedef struct {
  const void* k_host;
  const void* v_host;
  const void* k_hbm;
  const void* v_hbm;
  int64_t host_pages;
  int64_t hbm_pages;
  int64_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t page;
  int32_t max_pages;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  const int32_t* unit_order;
  int64_t n_host_units;
} dak_paged_kv;

/* Bytes of device workspace dak_paged_decode_attn needs (0 on invalid
 * shapes). */
size_t dak_paged_decode_attn_workspace_bytes(const dak_paged_kv* kv, int32_t n_q_heads);

/* dak_splitk_decode_attn over a paged KV cache: out[b, j, :] is the softmax
 * over request b's first ctx_lens[b] tokens of KV head g = j / (n_q_heads /
 * n_kv_heads).  Same arguments, workspace rule, determinism (the result bits
 * do not depend on which units are host units, nor on the pages' pool
 * indices) and errors as dak_splitk_decode_attn.  A request with no valid
 * token gets NaN rows. */
dak_status dak_paged_decode_attn(const void* q, const dak_paged_kv* kv, int32_t n_q_heads, float scale,
                                 float* out, void* ws, size_t ws_bytes, const dak_launch_cfg* cfg,
                                 void* stream);

/* ------------------------------------------------------------------------ */
/* Streaming-read probes (roofline bandwidths and the congestion sweep)        */
/* ------------------------------------------------------------------------ */

/* Streams `bytes` (a multiple of 16, >= 16) from `buf` (device memory or
 * pinned host memory) with `workgroups` work-groups of 256 lanes, each lane
 * keeping `window` 16-byte loads in flight (1, 2, 4, 8 or 16).  Runs one
 * warm-up and `reps` (>= 1) timed launches on `stream`, synchronizing, and
 * writes the median duration in milliseconds to *ms_out.
 * DAK paper §4.3.1 (Fig. 7 microbenchmark). */
dak_status dak_probe_read(const void* buf, size_t bytes, int32_t workgroups, int32_t window,
                          int32_t reps, void* stream, float* ms_out);

/* One launch in which `host_wgs` work-groups stream `host_bytes` of pinned
 * host memory while `hbm_wgs` work-groups stream `hbm_bytes` of device memory
 * (each role with its own window).  Per-role durations come from device
 * timestamps (first start to last end of that role's work-groups), in ms.
 * DAK paper §4.3.1, Fig. 7: host readers can slow down HBM readers. */
dak_status dak_probe_read_concurrent(const void* hbm, size_t hbm_bytes, int32_t hbm_wgs,
                                     int32_t hbm_window, const void* host, size_t host_bytes,
                                     int32_t host_wgs, int32_t host_window, void* stream,
                                     float* ms_total, float* ms_hbm, float* ms_host);

/* What a copy-based prefetcher's background copy costs the kernels it runs
 * beside (DAK paper §2.3 "Limitation of Copy-Based Offloading" and Fig. 2:
 * host-to-HBM copies write the HBM that compute kernels read; the pages
 * measure up to about 10 % less local bandwidth on GH200 and 4-7 % on a PCIe
 * GPU).  The streaming read of dak_probe_read over `hbm_bytes` of the device
 * buffer `hbm` (`workgroups`, `window` as there) runs `reps` times alone on
 * `stream`; then hipMemcpyAsync copies `copy_bytes` from pinned `host_src` to
 * device `dev_dst` on `copy_stream` (a different stream, of the same
 * priority) while the read runs `reps` more times on `stream`.  One untimed
 * copy and one untimed read come first.  Synchronizes both streams.
 * Outputs: *ms_alone, the median read alone; *ms_with_copy, the median over
 * the reads that started after the copy started and ended before it ended
 * (0 if none did); *copy_ms, the copy's own duration; *n_overlapped, how many
 * reads the second median covers.  Choose copy_bytes so that the copy
 * outlasts several reads (e.g. 1 GiB against a 4 GiB read).
 * Errors: DAK_EINVAL for NULL outputs, sizes or counts outside the limits,
 * pointers outside their tiers, or copy_stream == stream. */
dak_status dak_probe_copy_interference(const void* hbm, size_t hbm_bytes, int32_t workgroups, int32_t window,
                                       const void* host_src, void* dev_dst, size_t copy_bytes, int32_t reps,
                                       void* stream, void* copy_stream, float* ms_alone, float* ms_with_copy,
                                       float* copy_ms, int32_t* n_overlapped);

/* Matrix-core peak probe, the compute roof of the compute-bound split GEMM
 * (DAK paper §4.2.1 prices such ops by T_comp): `workgroups` work-groups of 4
 * waves each run 8 independent chains of `iters` v_mfma_f32_16x16x32_bf16 on
 * register operands.  Median of `reps` event-timed launches in *ms_out; the
 * bf16 dense rate it implies in *tflops_out (nullable), at whatever clock the
 * chip holds under that load.  Synchronizes the stream.  DAK_EINVAL for
 * workgroups outside [1, 65536], iters outside [1, 2^24], reps outside
 * [1, 1000] or a NULL ms_out. */
dak_status dak_probe_mfma(int32_t workgroups, int64_t iters, int32_t reps, void* stream, float* ms_out,
                          double* tflops_out);

#ifdef __cplusplus
}
#endif

#endif /* DAK_H */
